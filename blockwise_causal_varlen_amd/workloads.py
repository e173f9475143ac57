"""Device-side set-up of the five workloads and their exact work counts.

Each workload places the seeded inputs (blockwise_causal_varlen_amd.inputs) on
the GPU, lays them out the way the virtual ranks hold them (the zig-zag shard
runs in the library's kernel), and exposes `forward()` / `backward()` steps
that call only the C ABI. The counting helpers give the algorithmic work the
roofline figures are priced on: visible (query, key) pairs per q head, from
closed forms and integer position arithmetic (no attention math).
"""

from __future__ import annotations

import numpy as np
import torch

from . import inputs as I
from . import lib as L


# ----------------------------------------------------------------------------
# exact counts
# ----------------------------------------------------------------------------
def zigzag_rank_pairs(doc_lens, cp):
    """Visible pairs per q head of ONE zig-zag rank over all cp steps (equal
    for every rank). Per document with chunk c = L / (2 cp): the causal block
    over the rank's 2c rows has c (2c + 1) pairs and each of the cp - 1 other
    steps (front keys or back queries) has 2 c^2."""
    tot = 0
    for L_ in doc_lens:
        c = L_ // (2 * cp)
        tot += c * (2 * c + 1) + (cp - 1) * 2 * c * c
    return tot


def zigzag_step_pairs(doc_lens, cp, step):
    tot = 0
    for L_ in doc_lens:
        c = L_ // (2 * cp)
        tot += c * (2 * c + 1) if step == 0 else 2 * c * c
    return tot


def kvp_rank_pairs(s_q, global_q_offset, n_local, R, r, block_size, window):
    """Visible pairs per q head of KV-parallel rank r (round-robin keys)."""
    qpos = global_q_offset + np.arange(s_q, dtype=np.int64)

    def count_le(p):  # local keys with position <= p
        p = np.asarray(p, dtype=np.int64)
        blk, off = p // block_size, p % block_size
        nb = n_local // block_size
        # local blocks b with b*R + r < blk are fully <= p; block b*R + r == blk partly
        full = np.clip((blk - r + R - 1) // R, 0, nb)  # count of b with b*R + r < blk
        part = np.where(((blk - r) % R == 0) & (blk >= r) & ((blk - r) // R < nb), off + 1, 0)
        return np.minimum(full * block_size + part, n_local)

    hi = count_le(qpos)
    lo = count_le(qpos - window) if window > 0 else np.zeros_like(hi)
    return int(np.sum(np.maximum(hi - lo, 0)))


def decode_bytes(k_lens, hq, hkv, d):
    """Algorithmic HBM bytes of one decode pass: K and V once per kv head,
    q and out (bf16), lse (f32), cu_seqlens (int32)."""
    nseq = len(k_lens)
    kv = int(np.sum(np.asarray(k_lens, dtype=np.int64))) * hkv * d * 2 * 2
    return kv + nseq * hq * d * 2 * 2 + nseq * hq * 4 + (2 * nseq + 2) * 4


# ----------------------------------------------------------------------------
# zig-zag
# ----------------------------------------------------------------------------
class ZigzagWorkload:
    """cp virtual zig-zag ranks; `ranks` are the ones that run (all by default)."""

    def __init__(self, case: I.ZigzagCase, ranks=None, device="cuda", with_bwd=False, out_dtype=None):
        self.case, self.cp = case, case.cp
        cp = case.cp
        self.ranks = list(range(cp)) if ranks is None else list(ranks)
        self.device = device
        cu = case.cu
        self.doc_lens = (cu[1:] - cu[:-1]).tolist()
        self.max_len = int(max(self.doc_lens))
        self.max_local = self.max_len // cp
        self.cu_global = cu.to(device)
        self.cu_local = (cu // cp).to(torch.int32).to(device)
        k, v = case.k.to(device), case.v.to(device)
        self.k_loc = [L.zigzag_shard(k, self.cu_global, cp, r, self.max_len) for r in range(cp)]
        self.v_loc = [L.zigzag_shard(v, self.cu_global, cp, r, self.max_len) for r in range(cp)]
        del k, v
        self.q_loc, self.dout_loc, self.runners = {}, {}, {}
        for r in self.ranks:
            if case.q_rank is not None:
                if r != case.q_rank:
                    raise ValueError("this case holds q for one rank only")
                q = case.q.to(device)
                do = case.dout.to(device) if (with_bwd and case.dout is not None) else None
            else:
                q = L.zigzag_shard(case.q.to(device), self.cu_global, cp, r, self.max_len)
                do = (L.zigzag_shard(case.dout.to(device), self.cu_global, cp, r, self.max_len)
                      if (with_bwd and case.dout is not None) else None)
            self.q_loc[r], self.dout_loc[r] = q, do
            self.runners[r] = L.RingRunner("zigzag", cp, r, q, self.k_loc, self.v_loc, self.cu_local,
                                           self.max_local, case.scale, dout=do, out_dtype=out_dtype)
        # Several virtual ranks run at once, each on its own stream (default
        # priority), as they would on their own GPUs: their inputs are shared
        # read-only and each writes only its own outputs and workspace.
        self.streams = ({r: torch.cuda.Stream(device=device) for r in self.ranks}
                        if len(self.ranks) > 1 else None)

    def forward_batched(self):
        """All listed ranks' forwards through attn_zigzag_fwd_ranks: each ring
        step's blocks of every rank in one launch (on the current stream)."""
        if getattr(self, "_batched", None) is None:
            self._batched = L.ZigzagRanksForward([self.runners[r] for r in self.ranks])
        self._batched.forward()

    def _each_rank(self, fn):
        if self.streams is None:
            for r in self.ranks:
                fn(r, None)
            return
        cur = torch.cuda.current_stream()
        for r in self.ranks:
            self.streams[r].wait_stream(cur)
        for r in self.ranks:
            with torch.cuda.stream(self.streams[r]):
                fn(r, self.streams[r])
        for r in self.ranks:
            cur.wait_stream(self.streams[r])

    def forward(self):
        self._each_rank(lambda r, s: self.runners[r].forward(stream=s))

    def backward(self):
        # the drivers store the gradients (no zeroing pass needed first)
        self._each_rank(lambda r, s: self.runners[r].backward(stream=s, set_grads=True))

    def pairs_per_rank(self):
        return zigzag_rank_pairs(self.doc_lens, self.cp)

    def fwd_flops(self):
        hq, d = self.case.q.shape[1], self.case.q.shape[2]
        return 4 * d * hq * self.pairs_per_rank() * len(self.ranks)

    def bwd_flops(self):
        hq, d = self.case.q.shape[1], self.case.q.shape[2]
        return 10 * d * hq * self.pairs_per_rank() * len(self.ranks)


# ----------------------------------------------------------------------------
# EAGLE-3 mixed attention (zig-zag block 0 + TTT diagonal blocks)
# ----------------------------------------------------------------------------
class EagleWorkload:
    """Per virtual rank: cache block 0 runs the zig-zag ring (f32 merged state),
    then each TTT block's per-position diagonal is merged (the last merge writes
    the output in q's dtype). The backward feeds the final merged out and lse to
    the block-0 ring backward and to each diagonal's closed-form backward."""

    def __init__(self, case: I.EagleCase, ranks=None, device="cuda", with_bwd=False):
        base = case.base
        self.case, self.cp, self.n_ttt = case, base.cp, len(case.ttt_k)
        if self.n_ttt < 1:
            raise ValueError("at least one TTT block")
        self.zz = ZigzagWorkload(base, ranks=ranks, device=device, with_bwd=with_bwd, out_dtype=torch.float32)
        self.ranks = self.zz.ranks
        self.tk, self.tv, self.final, self.dtk, self.dtv, self.delta = {}, {}, {}, {}, {}, {}
        for r in self.ranks:
            if base.q_rank is not None:
                tk = [t.to(device) for t in case.ttt_k]
                tv = [t.to(device) for t in case.ttt_v]
            else:
                tk = [L.zigzag_shard(t.to(device), self.zz.cu_global, self.cp, r, self.zz.max_len) for t in case.ttt_k]
                tv = [L.zigzag_shard(t.to(device), self.zz.cu_global, self.cp, r, self.zz.max_len) for t in case.ttt_v]
            self.tk[r], self.tv[r] = tk, tv
            q = self.zz.q_loc[r]
            self.final[r] = torch.empty(q.shape, dtype=q.dtype, device=device)
            run = self.zz.runners[r]
            run.bwd_od = L.desc(self.final[r])  # the backward reads the final merged output
            if with_bwd:
                self.dtk[r] = [torch.zeros(t.shape, dtype=torch.float32, device=device) for t in tk]
                self.dtv[r] = [torch.zeros(t.shape, dtype=torch.float32, device=device) for t in tv]
                self.delta[r] = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=device)

    def forward(self):
        sc = self.case.base.scale
        for r in self.ranks:
            run = self.zz.runners[r]
            run.forward()  # block 0: run.out (f32) and run.lse hold the merged ring
            for i in range(self.n_ttt):
                L.merge_diag(self.zz.q_loc[r], self.tk[r][i], self.tv[r][i], sc, run.out, run.lse,
                             final_out=self.final[r] if i == self.n_ttt - 1 else None)

    def backward(self):
        sc = self.case.base.scale
        for r in self.ranks:
            run = self.zz.runners[r]
            run.backward(set_grads=True)  # block 0 with the final merged out and lse
            L.bwd_delta(self.zz.dout_loc[r], self.final[r], delta=self.delta[r])
            for i in range(self.n_ttt):
                self.dtk[r][i].zero_()
                self.dtv[r][i].zero_()
                L.diag_bwd(self.zz.dout_loc[r], self.zz.q_loc[r], self.tk[r][i], self.tv[r][i], run.lse,
                           self.delta[r], sc, run.dq, self.dtk[r][i], self.dtv[r][i])

    def diag_bytes(self):
        """HBM bytes of the diagonal kernels per rank (algorithmic): merge = q, k,
        v reads + f32 out read/write + lse read/write per (row, head); the last
        merge also writes the output in q's dtype. Backward = q, dout, k, v reads +
        dq f32 read/write per (row, head) + dk, dv f32 read/write per (row, kv head)
        + lse, delta reads."""
        q = self.zz.q_loc[self.ranks[0]]
        n, hq, d = q.shape
        hkv = self.case.ttt_k[0].shape[1]
        e = q.element_size()
        merge = n * hq * (e * d + 8 * d + 8) + 2 * n * hkv * e * d
        merge_last = merge + n * hq * e * d
        bwd = n * hq * (2 * e * d + 8 * d + 8) + n * hkv * (2 * e * d + 16 * d)
        return merge, merge_last, bwd


# ----------------------------------------------------------------------------
# Ulysses (all-to-all) EAGLE-3 mixed attention
# ----------------------------------------------------------------------------
class UlyssesWorkload:
    """uly virtual ranks, each holding a contiguous sequence shard (rows r S/uly ..)
    of q, the block-0 K/V and the TTT blocks. Forward: the all-to-all reshard
    gives each rank the FULL sequence for H/uly heads; block 0 is one varlen
    causal block per rank over the full sequence with the GLOBAL cu_seqlens; the
    inverse reshard brings (out, lse) back to the sequence shards, where the TTT
    diagonals merge shard-locally. Backward: the merged output, dout and lse go
    to head shards, block 0's backward runs on the merged state, its grads come
    back by the inverse reshard, and the diagonals add their closed-form grads."""

    def __init__(self, case: I.EagleCase, uly, device="cuda", with_bwd=False):
        base = case.base
        if base.q_rank is not None:
            raise ValueError("Ulysses needs the whole sequence's q")
        self.case, self.uly, self.n_ttt = case, uly, len(case.ttt_k)
        S, hq, d = base.q.shape
        hkv = base.k.shape[1]
        if S % uly or hq % uly or hkv % uly:
            raise ValueError("rows and heads must divide by uly")
        self.S, self.sl, self.hq, self.hkv, self.d = S, S // uly, hq, hkv, d
        dt = base.q.dtype
        self.cu = base.cu.to(torch.int32).to(device)
        self.max_len = int((base.cu[1:] - base.cu[:-1]).max())
        sl = self.sl

        def shards(x):
            x = x.to(device)
            return [x[r * sl:(r + 1) * sl] for r in range(uly)]

        self.q_loc, self.k_loc, self.v_loc = shards(base.q), shards(base.k), shards(base.v)
        self.tk = [shards(t) for t in case.ttt_k]   # [block][rank]
        self.tv = [shards(t) for t in case.ttt_v]
        emp = lambda *shape, dtype=dt: [torch.empty(*shape, dtype=dtype, device=device) for _ in range(uly)]
        self.qh, self.kh, self.vh = emp(S, hq // uly, d), emp(S, hkv // uly, d), emp(S, hkv // uly, d)
        self.oh = emp(S, hq // uly, d, dtype=torch.float32)
        self.lh = emp(hq // uly, S, dtype=torch.float32)
        self.out_loc = emp(sl, hq, d, dtype=torch.float32)
        self.lse_loc = emp(hq, sl, dtype=torch.float32)
        self.final = emp(sl, hq, d)
        self.mask = L.mask(causal=True)
        self.with_bwd = with_bwd
        if with_bwd:
            self.dout_loc = shards(base.dout)
            self.dh, self.fh = emp(S, hq // uly, d), emp(S, hq // uly, d)
            self.lse_h = emp(hq // uly, S, dtype=torch.float32)
            self.dqh = emp(S, hq // uly, d, dtype=torch.float32)
            self.dkh, self.dvh = emp(S, hkv // uly, d, dtype=torch.float32), emp(S, hkv // uly, d, dtype=torch.float32)
            self.dq, self.dk, self.dv = (emp(sl, hq, d, dtype=torch.float32), emp(sl, hkv, d, dtype=torch.float32),
                                         emp(sl, hkv, d, dtype=torch.float32))
            self.delta = emp(hq, sl, dtype=torch.float32)
            self.dtk = [emp(sl, hkv, d, dtype=torch.float32) for _ in range(self.n_ttt)]
            self.dtv = [emp(sl, hkv, d, dtype=torch.float32) for _ in range(self.n_ttt)]

    def forward(self):
        sc, uly = self.case.base.scale, self.uly
        L.ulysses_reshard(self.q_loc, self.qh, True)
        L.ulysses_reshard(self.k_loc, self.kh, True)
        L.ulysses_reshard(self.v_loc, self.vh, True)
        for r in range(uly):
            L.block_fwd(self.qh[r], self.kh[r], self.vh[r], self.cu, self.cu, self.max_len, self.max_len, sc,
                        self.mask, out=self.oh[r], lse=self.lh[r])
        L.ulysses_reshard(self.oh, self.out_loc, False)
        L.ulysses_reshard_lse(self.lh, self.lse_loc, False, self.sl, self.hq)
        for r in range(uly):
            for i in range(self.n_ttt):
                L.merge_diag(self.q_loc[r], self.tk[i][r], self.tv[i][r], sc, self.out_loc[r], self.lse_loc[r],
                             final_out=self.final[r] if i == self.n_ttt - 1 else None)

    def backward(self):
        sc, uly = self.case.base.scale, self.uly
        for r in range(uly):
            L.bwd_delta(self.dout_loc[r], self.final[r], delta=self.delta[r])
        L.ulysses_reshard(self.final, self.fh, True)
        L.ulysses_reshard(self.dout_loc, self.dh, True)
        L.ulysses_reshard_lse(self.lse_loc, self.lse_h, True, self.sl, self.hq)
        for r in range(uly):
            for t in (self.dqh[r], self.dkh[r], self.dvh[r]):
                t.zero_()
            L.block_bwd(self.dh[r], self.qh[r], self.kh[r], self.vh[r], self.fh[r], self.lse_h[r], self.cu, self.cu,
                        self.max_len, self.max_len, sc, self.mask, dq=self.dqh[r], dk=self.dkh[r], dv=self.dvh[r])
        L.ulysses_reshard(self.dqh, self.dq, False)
        L.ulysses_reshard(self.dkh, self.dk, False)
        L.ulysses_reshard(self.dvh, self.dv, False)
        for r in range(uly):
            for i in range(self.n_ttt):
                self.dtk[i][r].zero_()
                self.dtv[i][r].zero_()
                L.diag_bwd(self.dout_loc[r], self.q_loc[r], self.tk[i][r], self.tv[i][r], self.lse_loc[r],
                           self.delta[r], sc, self.dq[r], self.dtk[i][r], self.dtv[i][r])

    def reshard_bytes(self):
        """Bytes the reshards move per step (each element read once and written
        once): forward q, k, v (q dtype), out (f32), lse; backward final out and
        dout (q dtype), lse, dq, dk, dv (f32)."""
        e = self.case.base.q.element_size()
        S, hq, hkv, d = self.S, self.hq, self.hkv, self.d
        fwd = S * d * (hq + 2 * hkv) * e + S * hq * d * 4 + S * hq * 4
        bwd = 2 * S * hq * d * e + S * hq * 4 + S * d * (hq + 2 * hkv) * 4
        return 2 * (fwd + (bwd if self.with_bwd else 0))

    def block0_pairs(self):
        """Visible pairs per q head of block 0 (causal per document, all ranks)."""
        lens = (self.case.base.cu[1:] - self.case.base.cu[:-1]).tolist()
        return sum(L_ * (L_ + 1) // 2 for L_ in lens)


# ----------------------------------------------------------------------------
# KV-parallel
# ----------------------------------------------------------------------------
class KvpWorkload:
    def __init__(self, case: I.KvpCase, device="cuda"):
        self.case = case
        self.q = case.q.to(device)                      # [H, S, D]
        self.q_shd = self.q.transpose(0, 1)             # [S, H, D] view
        self.kc = [c.to(device) for c in case.k_caches]
        self.vc = [c.to(device) for c in case.v_caches]
        self.tabs = [t.reshape(-1).to(device) for t in case.tables]
        hq, s_q, d = case.q.shape
        self.s_q, self.hq, self.d = s_q, hq, d
        self.n_blocks = case.tables[0].numel()
        self.n_local = self.n_blocks * case.block_size
        self.cu_q = torch.tensor([0, s_q], dtype=torch.int32, device=device)
        self.cu_k = torch.tensor([0, self.n_local], dtype=torch.int32, device=device)
        self.mask = L.mask(causal=True, window=case.window, q_pos_offset=case.global_q_offset,
                           kv_interleave=case.R, block_size=case.block_size, max_blocks=self.n_blocks,
                           page_stride=self.kc[0].stride(0), seg_size=case.seg_size,
                           block_table=self.tabs[0])
        self.out = torch.empty(s_q, hq, d, dtype=case.q.dtype, device=device)
        self.lse = torch.empty(hq, s_q, dtype=torch.float32, device=device)

    def forward(self):
        return L.kvp_fwd(self.q_shd, self.kc, self.vc, self.tabs, self.cu_q, self.cu_k, self.s_q, self.n_local,
                         self.case.scale, self.mask, out=self.out, lse=self.lse)

    def pairs(self):
        c = self.case
        return sum(kvp_rank_pairs(self.s_q, c.global_q_offset, self.n_local, c.R, r, c.block_size, c.window)
                   for r in range(c.R))

    def fwd_flops(self):
        return 4 * self.d * self.hq * self.pairs()


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
class DecodeWorkload:
    def __init__(self, case: I.DecodeCase, device="cuda"):
        self.case = case
        nseq, hq, d = case.q.shape
        self.nseq, self.hq, self.d, self.hkv = nseq, hq, d, case.k.shape[1]
        self.q = case.q.to(device)
        self.k, self.v = case.k.to(device), case.v.to(device)
        self.cu_q = torch.arange(nseq + 1, dtype=torch.int32, device=device)
        self.cu_k = case.cu_k.to(device)
        self.max_k = int(case.k_lens.max())
        self.out = torch.empty(nseq, hq, d, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(hq, nseq, dtype=torch.float32, device=device)

    def forward(self):
        return L.block_fwd(self.q, self.k, self.v, self.cu_q, self.cu_k, 1, self.max_k, self.case.scale, None,
                           out=self.out, lse=self.lse)

    def bytes(self):
        return decode_bytes(self.case.k_lens.numpy(), self.hq, self.hkv, self.d)
