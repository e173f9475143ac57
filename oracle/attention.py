"""Plain fp64 reference of blockwise causal varlen attention (CPU, numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the library.

Sources (web pages, cited by title and section):
  [ZZ]  NeMo AutoModel API docs, "nemo_automodel.components.speculative.eagle.
        zigzag_ring_attention" -- module docstring (zig-zag chunk ownership),
        `get_half_index` / `get_half_lse`, `_block_forward`,
        `update_out_and_lse`, `zigzag_ring_flash_attn_varlen_backward`.
  [RING] NeMo AutoModel API docs, "nemo_automodel.components.speculative.eagle.
        ring_attention" -- `_CachedRingAttention` (single-key lse form),
        `_update_out_and_lse` (sigmoid form), `ring_flash_attn_forward`
        (step <= rank rule, causal only at step 0), `_fa_forward` layouts.
  [ULY] NeMo AutoModel API docs, "...eagle.ulysses_attention" --
        `cached_ulysses_attention` (scale = head_dim ** -0.5).
  [KVP] AWS Neuron NKI library, "Attention KV-Parallel Segmented CTE Kernel API
        Reference" -- Background, parameters `kvp_q_offset`, `kvp_group_size`,
        `seg_size`, `sliding_window`, `block_tables`.
  [DEC] recipes "qsa_fa_fallback.py" (SM121 fallback varlen attention) --
        module docstring (one query row per sequence, GQA) and the
        normalisation guard of its kernel (a query with no keys gives 0).

Conventions (one layout everywhere):
  q, out        [n_q, HQ, D]   packed varlen rows (documents by cu_seqlens)
  k, v          [n_k, HKV, D]
  lse           [HQ, n_q]      natural log of the sum of exp(scaled scores);
                               -inf for a row that sees no key
  cu_seqlens    int, length num_docs + 1; document d of q pairs with
                document d of k.
  q head h reads kv head h // (HQ // HKV)                         ([DEC] GQA)

Nothing here is blocked, fused or reordered beyond what the definitions say:
each function evaluates the defining sums directly (per document, per head, in
row chunks only to bound memory; the chunking does not change any sum).
"""

from __future__ import annotations

import numpy as np

ALL, FRONT, BACK = "all", "front", "back"
NEG_INF = -np.inf

__all__ = [
    "ALL", "FRONT", "BACK", "as_f64", "doc_bounds", "view_range",
    "key_position", "visibility", "block_forward", "block_backward",
    "merge", "full_attention", "attention_grads", "eagle_forward", "eagle_grads",
    "ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_lse_seq_to_head", "ulysses_lse_head_to_seq",
    "zigzag_shard", "zigzag_unshard", "zigzag_global_positions",
    "zigzag_step", "zigzag_block_args", "zigzag_forward", "zigzag_backward",
    "ring_shard", "ring_forward", "ring_backward",
    "kvp_gather_pages", "kvp_global_kv", "kvp_rank_partial", "kvp_forward",
    "decode_forward", "count_visible_pairs",
]


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def as_f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor: .double() widens bf16, f16, f32 exactly and keeps f64
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def doc_bounds(cu):
    cu = [int(c) for c in np.asarray(cu).reshape(-1)]
    return list(zip(cu[:-1], cu[1:]))


def view_range(start: int, end: int, view: str):
    """Rows of one document that a view selects.

    [ZZ] `get_half_index`: the front (early) or back (late) half of EACH varlen
    document. FRONT = first n//2 rows, BACK = the remaining rows, ALL = all.
    """
    n = end - start
    h = n // 2
    if view == ALL:
        return start, end
    if view == FRONT:
        return start, start + h
    if view == BACK:
        return start + h, end
    raise ValueError(f"unknown view {view!r}")


def key_position(t, k_pos_offset=0, kv_interleave=0, kv_rank=0, block_size=0):
    """Position of the key at index t of a document's (logical) key buffer.

    [KVP] `kvp_group_size`: with round-robin distribution over R ranks, rank r
    holds global KV blocks r, r+R, r+2R, ...; so its local block b is global
    block b*R + r, and the token at offset o of that block sits at global
    position (b*R + r)*block_size + o. Contiguous distribution is the identity
    plus an offset (rank r's shard starts at r * local_kv_len).
    """
    t = np.asarray(t, dtype=np.int64)
    if kv_interleave:
        b, o = t // block_size, t % block_size
        return k_pos_offset + (b * kv_interleave + kv_rank) * block_size + o
    return k_pos_offset + t


def visibility(qpos, kpos, causal: bool, window: int):
    """vis[i, j] for one document: the causal and sliding-window predicate.

    Causal: a query at position p sees keys at positions <= p.
    Sliding window W (0 = off): the query also needs key position > p - W,
    i.e. W counts the visible keys including the query's own position. The
    NKI page names the parameter but not its boundary; this is the reading
    used throughout (parity unpinned by the pages).
    """
    qpos = np.asarray(qpos, dtype=np.int64)[:, None]
    kpos = np.asarray(kpos, dtype=np.int64)[None, :]
    vis = np.ones((qpos.shape[0], kpos.shape[1]), dtype=bool)
    if causal:
        vis &= kpos <= qpos
    if window:
        vis &= kpos > qpos - window
    return vis


def _doc_rows(cu_q, cu_k, d, q_view, k_view, rows, k_range):
    (qs, qe), (ks, ke) = doc_bounds(cu_q)[d], doc_bounds(cu_k)[d]
    qa, qb = view_range(qs, qe, q_view)
    ka, kb = view_range(ks, ke, k_view)
    if k_range is not None:  # restrict to doc-local key indices [a, b)
        ka, kb = max(ka, ks + k_range[0]), min(kb, ks + k_range[1])
    qi = np.arange(qa, qb, dtype=np.int64)
    if rows is not None:
        qi = qi[np.isin(qi, rows)]
    kj = np.arange(ka, max(ka, kb), dtype=np.int64)
    return qs, ks, qi, kj


def _positions(qs, ks, qi, kj, m):
    qpos = m.get("q_pos_offset", 0) + (qi - qs)
    kpos = key_position(kj - ks, m.get("k_pos_offset", 0), m.get("kv_interleave", 0),
                        m.get("kv_rank", 0), m.get("block_size", 0))
    return qpos, kpos


_MASK_KEYS = ("causal", "q_view", "k_view", "window", "q_pos_offset",
              "k_pos_offset", "kv_interleave", "kv_rank", "block_size", "k_range")


def _mask_args(kw):
    bad = set(kw) - set(_MASK_KEYS)
    if bad:
        raise TypeError(f"unknown mask arguments {sorted(bad)}")
    m = dict(kw)
    m.setdefault("causal", False)
    m.setdefault("q_view", ALL)
    m.setdefault("k_view", ALL)
    m.setdefault("window", 0)
    return m


# ----------------------------------------------------------------------------
# block forward, merge, backward
# ----------------------------------------------------------------------------
def block_forward(q, k, v, cu_q, cu_k, scale, rows=None, chunk=1024, **mask):
    """One attention block -> (out, lse), by the definition.

    [ZZ] `_block_forward` / [RING] `_fa_forward`: a flash varlen forward over a
    block returns the block's normalised output and its log-sum-exp. Here:
        s_ij  = scale * <q_{i,h}, k_{j,g(h)}>,   g(h) = h // (HQ/HKV)
        lse_i = ln sum_{visible j} exp(s_ij)        (-inf if none visible)
        out_i = sum_{visible j} exp(s_ij - lse_i) v_j   (0 if none visible,
                as the normalisation guard of [DEC] gives)
    The lse is the natural log of SCALED scores: [RING] `_CachedRingAttention`
    gives a one-key block's lse as (Q_t . K_t) * scale.

    Mask keywords: causal, q_view/k_view (ALL/FRONT/BACK per document),
    window, q_pos_offset, k_pos_offset, kv_interleave, kv_rank, block_size
    (key position map, see key_position), k_range (doc-local key index range,
    a KV segment). Rows outside the q view (or not in ``rows``) come back as
    out = 0, lse = -inf.
    """
    m = _mask_args(mask)
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    nq, hq, dim = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    out = np.zeros((nq, hq, dim))
    lse = np.full((hq, nq), NEG_INF)
    ndoc = len(doc_bounds(cu_q))
    for d in range(ndoc):
        qs, ks, qi, kj = _doc_rows(cu_q, cu_k, d, m["q_view"], m["k_view"], rows, m.get("k_range"))
        if len(qi) == 0 or len(kj) == 0:
            continue
        qpos, kpos = _positions(qs, ks, qi, kj, m)
        for c0 in range(0, len(qi), chunk):
            ci = qi[c0:c0 + chunk]
            vis = visibility(qpos[c0:c0 + chunk], kpos, m["causal"], m["window"])
            has = vis.any(axis=1)
            for h in range(hq):
                g = h // grp
                s = scale * (q[ci, h, :] @ k[kj, g, :].T)
                s = np.where(vis, s, NEG_INF)
                mx = np.where(has, s.max(axis=1), 0.0)
                e = np.exp(s - mx[:, None])  # exp(-inf) = 0 on masked pairs
                l = e.sum(axis=1)
                safe = np.where(has, l, 1.0)
                lse[h, ci] = np.where(has, mx + np.log(safe), NEG_INF)
                out[ci, h, :] = np.where(has[:, None], (e @ v[kj, g, :]) / safe[:, None], 0.0)
    return out, lse


def merge(out_a, lse_a, out_b, lse_b):
    """Merge two partials of one softmax -> (out, lse, sigma).

    [ZZ] `update_out_and_lse` / [RING] `_update_out_and_lse`: the online-softmax
    log-sum-exp identity. For disjoint key sets A and B of the same queries,
        lse   = ln(e^{lse_a} + e^{lse_b})
        out   = e^{lse_a - lse} out_a + e^{lse_b - lse} out_b
        sigma = e^{lse_b - lse} = sigmoid(lse_b - lse_a)
    (the pages' "sigmoid form" writes out = out_a - sigma (out_a - out_b); the
    weight they return for the backward is this sigma.) A -inf lse is the
    identity (a block with no visible key); both -inf gives out 0, lse -inf.
    """
    out_a, out_b = as_f64(out_a), as_f64(out_b)
    lse_a, lse_b = as_f64(lse_a), as_f64(lse_b)
    lse = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(lse)
    with np.errstate(invalid="ignore"):
        wa = np.where(fin, np.exp(lse_a - np.where(fin, lse, 0.0)), 0.0)
        wb = np.where(fin, np.exp(lse_b - np.where(fin, lse, 0.0)), 0.0)
    out = wa.T[:, :, None] * out_a + wb.T[:, :, None] * out_b
    return out, lse, wb


def block_backward(dout, q, k, v, out, lse, cu_q, cu_k, scale, chunk=1024, rows=None, krows=None, **mask):
    """Gradient contribution of one block, given the MERGED out and lse.

    [ZZ] `zigzag_ring_flash_attn_varlen_backward`: every block's backward is fed
    the final merged out/lse, which yields the joint-softmax gradient with no
    separate merge backward. For the block's visible pairs:
        delta_i = <dout_i, out_i>            (merged out)
        P_ij    = exp(s_ij - lse_i)          (merged lse)
        dP_ij   = <dout_i, v_j>
        dS_ij   = P_ij (dP_ij - delta_i)
        dq_i   += scale sum_j dS_ij k_j
        dk_j   += scale sum_{i, h in group} dS_ij q_i
        dv_j   += sum_{i, h in group} P_ij dout_i
    Returns (dq [n_q,HQ,D], dk [n_k,HKV,D], dv [n_k,HKV,D]).
    ``rows`` / ``krows`` evaluate the same sums for a sample: only the listed
    query rows (exact dq for them) or only the listed key rows (exact dk/dv
    for them) take part; the other outputs are then partial.
    """
    m = _mask_args(mask)
    dout, q, k, v, out = (as_f64(t) for t in (dout, q, k, v, out))
    lse = as_f64(lse)
    nq, hq, dim = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    delta = np.einsum("ihd,ihd->hi", dout, out)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for d in range(len(doc_bounds(cu_q))):
        qs, ks, qi, kj = _doc_rows(cu_q, cu_k, d, m["q_view"], m["k_view"], rows, m.get("k_range"))
        if krows is not None:
            kj = kj[np.isin(kj, krows)]
        if len(qi) == 0 or len(kj) == 0:
            continue
        qpos, kpos = _positions(qs, ks, qi, kj, m)
        for c0 in range(0, len(qi), chunk):
            ci = qi[c0:c0 + chunk]
            vis = visibility(qpos[c0:c0 + chunk], kpos, m["causal"], m["window"])
            for h in range(hq):
                g = h // grp
                l_i = lse[h, ci]
                ok = vis & np.isfinite(l_i)[:, None]
                s = scale * (q[ci, h, :] @ k[kj, g, :].T)
                p = np.where(ok, np.exp(np.where(ok, s - np.where(np.isfinite(l_i), l_i, 0.0)[:, None], 0.0)), 0.0)
                dp = dout[ci, h, :] @ v[kj, g, :].T
                ds = p * (dp - delta[h, ci][:, None])
                dq[ci, h, :] += scale * (ds @ k[kj, g, :])
                dk[kj, g, :] += scale * (ds.T @ q[ci, h, :])
                dv[kj, g, :] += p.T @ dout[ci, h, :]
    return dq, dk, dv


def full_attention(q, k, v, cu, scale, rows=None):
    """Target of every schedule: causal attention within each document."""
    return block_forward(q, k, v, cu, cu, scale, rows=rows, causal=True)


def attention_grads(dout, q, k, v, cu, scale):
    """Gradients of full causal per-document attention (block bwd over one block)."""
    out, lse = full_attention(q, k, v, cu, scale)
    return block_backward(dout, q, k, v, out, lse, cu, cu, scale, causal=True)


# ----------------------------------------------------------------------------
# EAGLE-3 mixed attention: block 0 causal over the sequence, TTT diagonals
# ----------------------------------------------------------------------------
def eagle_forward(q, ks, vs, cu, scale):
    """Joint softmax of EAGLE-3 mixed attention -> (out, lse), by the definition.

    [RING] `_CachedRingAttention` / [ZZ] `_CachedZigZagRingAttention`: cache
    block 0 (ks[0], vs[0]) is the sequence, seen causally within each
    document; every later block i >= 1 is a test-time-training step that gives
    query t exactly one more key, ks[i][t], with value vs[i][t] (same
    position). All keys enter one softmax:
        s_tj   = scale <q_{t,h}, ks[0]_{j,g(h)}>      (causal keys j of t's doc)
        d_it   = scale <q_{t,h}, ks[i]_{t,g(h)}>      (i = 1 .. n-1)
        lse_t  = ln( sum_j e^{s_tj} + sum_i e^{d_it} )
        out_t  = ( sum_j e^{s_tj} v0_j + sum_i e^{d_it} vi_t ) / e^{lse_t}
    Global (unsharded) layout: q [n, HQ, D], ks/vs lists of [n, HKV, D].
    """
    q = as_f64(q)
    ks = [as_f64(k) for k in ks]
    vs = [as_f64(v) for v in vs]
    n, hq, dim = q.shape
    grp = hq // ks[0].shape[1]
    out = np.zeros((n, hq, dim))
    lse = np.full((hq, n), NEG_INF)
    for qs, qe in doc_bounds(cu):
        L = qe - qs
        if L == 0:
            continue
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(hq):
            g = h // grp
            qd = q[qs:qe, h, :]
            s = np.where(causal, scale * (qd @ ks[0][qs:qe, g, :].T), NEG_INF)
            diag = [scale * np.sum(qd * k[qs:qe, g, :], axis=1) for k in ks[1:]]
            allsc = np.concatenate([s] + [d_[:, None] for d_ in diag], axis=1)
            mx = allsc.max(axis=1)
            e = np.exp(allsc - mx[:, None])
            tot = e.sum(axis=1)
            lse[h, qs:qe] = mx + np.log(tot)
            acc = e[:, :L] @ vs[0][qs:qe, g, :]
            for i, v in enumerate(vs[1:]):
                acc = acc + e[:, L + i][:, None] * v[qs:qe, g, :]
            out[qs:qe, h, :] = acc / tot[:, None]
    return out, lse


def eagle_grads(dout, q, ks, vs, cu, scale, out=None, lse=None):
    """Gradients of the joint softmax of eagle_forward, by the definition.

    The softmax over the augmented key set of each query (block-0 causal keys
    plus one diagonal key per later block) has the usual gradient:
        delta_t = <dout_t, out_t>,  P = e^{score - lse_t},  dP = <dout_t, value>,
        dS = P (dP - delta_t);  dq_t += scale dS key;  dkey += scale dS q_t;
        dvalue += P dout_t   (dk, dv summed over the q heads of a kv head)
    For a diagonal key these sums have the single term of its own position,
    the closed form [RING] `_CachedRingAttention` adds beside the block-0
    backward. ``out`` / ``lse`` (the merged state) default to eagle_forward's;
    given, delta and P are taken from them, as a schedule's backward does.
    Returns (dq, dks list, dvs list).
    """
    q, dout = as_f64(q), as_f64(dout)
    ks = [as_f64(k) for k in ks]
    vs = [as_f64(v) for v in vs]
    if out is None or lse is None:
        out, lse = eagle_forward(q, ks, vs, cu, scale)
    out, lse = as_f64(out), as_f64(lse)
    n, hq, dim = q.shape
    grp = hq // ks[0].shape[1]
    dq = np.zeros_like(q)
    dks = [np.zeros_like(k) for k in ks]
    dvs = [np.zeros_like(v) for v in vs]
    for qs, qe in doc_bounds(cu):
        L = qe - qs
        if L == 0:
            continue
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(hq):
            g = h // grp
            qd, od, dd = q[qs:qe, h, :], out[qs:qe, h, :], dout[qs:qe, h, :]
            l_t = lse[h, qs:qe]
            delta = np.sum(dd * od, axis=1)
            p = np.where(causal, np.exp(np.where(causal, scale * (qd @ ks[0][qs:qe, g, :].T), 0.0) - l_t[:, None]), 0.0)
            dp = dd @ vs[0][qs:qe, g, :].T
            ds = p * (dp - delta[:, None])
            dq[qs:qe, h, :] += scale * (ds @ ks[0][qs:qe, g, :])
            dks[0][qs:qe, g, :] += scale * (ds.T @ qd)
            dvs[0][qs:qe, g, :] += p.T @ dd
            for i in range(1, len(ks)):
                kd, vd = ks[i][qs:qe, g, :], vs[i][qs:qe, g, :]
                pi = np.exp(scale * np.sum(qd * kd, axis=1) - l_t)
                dsi = pi * (np.sum(dd * vd, axis=1) - delta)
                dq[qs:qe, h, :] += scale * dsi[:, None] * kd
                dks[i][qs:qe, g, :] += scale * dsi[:, None] * qd
                dvs[i][qs:qe, g, :] += pi[:, None] * dd
    return dq, dks, dvs


# ----------------------------------------------------------------------------
# Ulysses all-to-all reshard (virtual ranks)
# ----------------------------------------------------------------------------
def ulysses_seq_to_head(locals_, uly):
    """[ULY] `_gather_seq_scatter_heads`: uly sequence shards [S/uly, H, D]
    (rank r holds rows r*S/uly ..) become uly head shards [S, H/uly, D] (rank r
    holds heads r*H/uly ..): out[r][t, j] = locals_[t // (S/uly)][t % (S/uly), r*H/uly + j]."""
    xs = [as_f64(x) for x in locals_]
    full = np.concatenate(xs, axis=0)
    hl = full.shape[1] // uly
    return [full[:, r * hl:(r + 1) * hl] for r in range(uly)]


def ulysses_head_to_seq(heads_, uly):
    """[ULY] `_scatter_seq_gather_heads`, the inverse: uly head shards
    [S, H/uly, D] become uly sequence shards [S/uly, H, D]."""
    xs = [as_f64(x) for x in heads_]
    full = np.concatenate(xs, axis=1)
    sl = full.shape[0] // uly
    return [full[r * sl:(r + 1) * sl] for r in range(uly)]


def ulysses_lse_seq_to_head(lses, uly):
    """[ULY] `_gather_lse`: [H, S/uly] per rank -> [H/uly, S] per rank (contiguous)."""
    full = np.concatenate([as_f64(x) for x in lses], axis=1)
    hl = full.shape[0] // uly
    return [np.ascontiguousarray(full[r * hl:(r + 1) * hl]) for r in range(uly)]


def ulysses_lse_head_to_seq(lses, uly):
    """[ULY] `_scatter_lse`: [H/uly, S] per rank -> [H, S/uly] per rank."""
    full = np.concatenate([as_f64(x) for x in lses], axis=0)
    sl = full.shape[1] // uly
    return [np.ascontiguousarray(full[:, r * sl:(r + 1) * sl]) for r in range(uly)]


# ----------------------------------------------------------------------------
# zig-zag ring (virtual ranks)
# ----------------------------------------------------------------------------
def _zz_chunks(length, cp, r):
    if length % (2 * cp):
        raise ValueError(f"document length {length} not divisible by 2*cp={2 * cp}")
    c = length // (2 * cp)
    return [(r * c, (r + 1) * c), ((2 * cp - 1 - r) * c, (2 * cp - r) * c)]


def zigzag_shard(x, cu, cp, r):
    """Rank r's zig-zag local rows and local cu_seqlens.

    [ZZ] module docstring: the sequence is cut into 2*cp chunks and rank r owns
    chunk r (early) and chunk 2*cp-1-r (late); with varlen this is done per
    document ([ZZ] `get_half_index` works per varlen document), so each local
    document is [chunk r | chunk 2cp-1-r] and local cu_seqlens = global / cp.
    """
    x = as_f64(x)
    parts = []
    for s, e in doc_bounds(cu):
        for a, b in _zz_chunks(e - s, cp, r):
            parts.append(x[s + a:s + b])
    local = np.concatenate(parts, axis=0)
    return local, np.asarray(cu, dtype=np.int64) // cp


def zigzag_unshard(locals_, cu, cp):
    """Inverse of zigzag_shard over all ranks: global packed rows."""
    n = int(np.asarray(cu)[-1])
    out = np.zeros((n,) + np.asarray(locals_[0]).shape[1:], dtype=np.asarray(locals_[0]).dtype)
    for r in range(cp):
        pos = 0
        for s, e in doc_bounds(cu):
            for a, b in _zz_chunks(e - s, cp, r):
                out[s + a:s + b] = locals_[r][pos:pos + (b - a)]
                pos += b - a
    return out


def zigzag_global_positions(cu, cp, r):
    """(doc index, global position in doc) of each of rank r's local rows."""
    docs, pos = [], []
    for d, (s, e) in enumerate(doc_bounds(cu)):
        for a, b in _zz_chunks(e - s, cp, r):
            docs.extend([d] * (b - a))
            pos.extend(range(a, b))
    return np.asarray(docs), np.asarray(pos)


def zigzag_step(r, s, cp):
    """(src, kind) of rank r's block at ring step s.

    K/V move one rank forward per step ([ZZ] `RingComm`: send to rank+1,
    receive from rank-1), so at step s rank r holds the K/V of src = (r-s) mod
    cp. The block kind follows from causality on the chunk order:
      s == 0            -> "diag": own chunks, causal on local order;
      src < r  (1<=s<=r)-> "kv_front": src's early chunk precedes both of r's
                           chunks and its late chunk follows both -> all q rows
                           see exactly src's front half, unmasked;
      src > r  (s > r)  -> "q_back": r's early chunk precedes both of src's
                           chunks and r's late chunk follows both -> only r's
                           back half sees all of src's rows, unmasked.
    The pages state ownership, not this table; zigzag_forward checks it against
    the global-position causal mask on every call (check=True).
    """
    src = (r - s) % cp
    if s == 0:
        return src, "diag"
    return src, ("kv_front" if s <= r else "q_back")


def zigzag_block_args(kind):
    if kind == "diag":
        return dict(causal=True)
    if kind == "kv_front":
        return dict(k_view=FRONT)
    if kind == "q_back":
        return dict(q_view=BACK)
    raise ValueError(kind)


def _check_zigzag_rule(cu_global, cp, r, src, kind):
    cu_l = np.asarray(cu_global, dtype=np.int64) // cp
    qd, qp = zigzag_global_positions(cu_global, cp, r)
    kd, kp = zigzag_global_positions(cu_global, cp, src)
    want = (qd[:, None] == kd[None, :]) & (kp[None, :] <= qp[:, None])
    a = zigzag_block_args(kind)
    got = np.zeros_like(want)
    for d, ((qs, qe), (ks, ke)) in enumerate(zip(doc_bounds(cu_l), doc_bounds(cu_l))):
        qa, qb = view_range(qs, qe, a.get("q_view", ALL))
        ka, kb = view_range(ks, ke, a.get("k_view", ALL))
        blk = np.ones((qb - qa, kb - ka), dtype=bool)
        if a.get("causal"):
            blk = visibility(np.arange(qa - qs, qb - qs), np.arange(ka - ks, kb - ks), True, 0)
        got[qa:qb, ka:kb] = blk
    if not np.array_equal(got, want):
        raise AssertionError(f"zig-zag rule disagrees with global causal mask (r={r}, src={src}, {kind})")


def zigzag_forward(q_loc, k_loc, v_loc, cu_global, cp, r, scale, check=True):
    """Rank r's merged (out, lse) over all cp ring steps, in ring order.

    [ZZ] `zigzag_ring_flash_attn_varlen_forward`: rotate K/V, one flash block per
    step, online-softmax merge. The first block initialises the running state
    ([RING] `_init_out_and_lse`), later ones merge in step order s = 1..cp-1.
    q_loc[r], k_loc[src], v_loc[src] are the ranks' local buffers.
    """
    cu_l = np.asarray(cu_global, dtype=np.int64) // cp
    out = lse = None
    for s in range(cp):
        src, kind = zigzag_step(r, s, cp)
        if check:
            _check_zigzag_rule(cu_global, cp, r, src, kind)
        bo, bl = block_forward(q_loc[r], k_loc[src], v_loc[src], cu_l, cu_l, scale, **zigzag_block_args(kind))
        if out is None:
            out, lse = bo, bl
        else:
            out, lse, _ = merge(out, lse, bo, bl)
    return out, lse


def zigzag_backward(dout_r, q_loc, k_loc, v_loc, out_r, lse_r, cu_global, cp, r, scale):
    """Rank r's dq and its contributions to every owner's dk/dv.

    [ZZ] `zigzag_ring_flash_attn_varlen_backward` (merged-lse trick) and [RING]
    `ring_flash_attn_backward` (K/V grads travel back to their owners): the
    block at step s adds its dk/dv to rank src's buffers.
    Returns (dq_r, dk_by_owner[list of cp], dv_by_owner[list of cp]).
    """
    cu_l = np.asarray(cu_global, dtype=np.int64) // cp
    dq = np.zeros(as_f64(q_loc[r]).shape)
    dk = [np.zeros(as_f64(k_loc[i]).shape) for i in range(cp)]
    dv = [np.zeros(as_f64(v_loc[i]).shape) for i in range(cp)]
    for s in range(cp):
        src, kind = zigzag_step(r, s, cp)
        gq, gk, gv = block_backward(dout_r, q_loc[r], k_loc[src], v_loc[src], out_r, lse_r,
                                    cu_l, cu_l, scale, **zigzag_block_args(kind))
        dq += gq
        dk[src] += gk
        dv[src] += gv
    return dq, dk, dv


# ----------------------------------------------------------------------------
# contiguous ring (virtual ranks)
# ----------------------------------------------------------------------------
def ring_shard(x, cu, cp, r):
    """Rank r's contiguous shard of every sequence: rows [r*S/cp, (r+1)*S/cp)
    of each one ([RING] module docstring: each rank holds a contiguous S/cp)."""
    x = as_f64(x)
    parts = []
    for s, e in doc_bounds(cu):
        if (e - s) % cp:
            raise ValueError("sequence length not divisible by cp")
        n = (e - s) // cp
        parts.append(x[s + r * n:s + (r + 1) * n])
    return np.concatenate(parts, axis=0), np.asarray(cu, dtype=np.int64) // cp


def ring_forward(q_loc, k_loc, v_loc, cu_global, cp, r, scale):
    """[RING] `ring_flash_attn_forward`, causal: rank r only attends the K/V of
    steps s <= r (src = r - s), with the causal mask only at step 0."""
    cu_l = np.asarray(cu_global, dtype=np.int64) // cp
    out = lse = None
    for s in range(r + 1):
        src = r - s
        bo, bl = block_forward(q_loc[r], k_loc[src], v_loc[src], cu_l, cu_l, scale, causal=(s == 0))
        if out is None:
            out, lse = bo, bl
        else:
            out, lse, _ = merge(out, lse, bo, bl)
    return out, lse


def ring_backward(dout_r, q_loc, k_loc, v_loc, out_r, lse_r, cu_global, cp, r, scale):
    cu_l = np.asarray(cu_global, dtype=np.int64) // cp
    dq = np.zeros(as_f64(q_loc[r]).shape)
    dk = [np.zeros(as_f64(k_loc[i]).shape) for i in range(cp)]
    dv = [np.zeros(as_f64(v_loc[i]).shape) for i in range(cp)]
    for s in range(r + 1):
        src = r - s
        gq, gk, gv = block_backward(dout_r, q_loc[r], k_loc[src], v_loc[src], out_r, lse_r,
                                    cu_l, cu_l, scale, causal=(s == 0))
        dq += gq
        dk[src] += gk
        dv[src] += gv
    return dq, dk, dv


# ----------------------------------------------------------------------------
# KV-parallel segmented prefill (virtual ranks)
# ----------------------------------------------------------------------------
def kvp_gather_pages(cache, block_table, n_blocks):
    """Logical local K (or V) of one rank: [KVP] `block_tables` maps logical
    block b to physical cache block block_table[b]; the cache is
    [num_blocks, HKV, block_size, D]. Returns [n_blocks*block_size, HKV, D]."""
    cache = as_f64(cache)
    bt = np.asarray(block_table, dtype=np.int64).reshape(-1)[:n_blocks]
    g = cache[bt]  # [n_blocks, HKV, bs, D]
    return g.transpose(0, 2, 1, 3).reshape(-1, cache.shape[1], cache.shape[3])


def kvp_global_kv(caches, tables, n_blocks, interleave=True):
    """Global K (or V) in position order rebuilt from R ranks' paged caches."""
    R = len(caches)
    loc = [kvp_gather_pages(c, t, n_blocks) for c, t in zip(caches, tables)]
    if not interleave:
        return np.concatenate(loc, axis=0)
    bs = caches[0].shape[2]
    blocks = []
    for b in range(n_blocks):
        for r in range(R):
            blocks.append(loc[r][b * bs:(b + 1) * bs])
    return np.concatenate(blocks, axis=0)


def kvp_rank_partial(q, k_cache, v_cache, block_table, n_blocks, R, r, seg_size, global_q_offset,
                     window, scale, interleave=True, causal=True, rows=None):
    """One rank's partial (out, lse) over its local KV, segment by segment.

    [KVP] Background: each rank attends its local KV shard in segments of
    `seg_size` tokens with online softmax. Query token t sits at global
    position global_q_offset + t. Key positions: round-robin (local block b is
    global block b*R + r) or contiguous (offset r * local_kv_len, which is what
    `kvp_q_offset = -rank*local_kv_len + global_q_offset` expresses when the
    offset is moved to the query side). Segments are merged in order.
    """
    q = as_f64(q)
    k = kvp_gather_pages(k_cache, block_table, n_blocks)
    v = kvp_gather_pages(v_cache, block_table, n_blocks)
    nq, nk = q.shape[0], k.shape[0]
    bs = k_cache.shape[2]
    cu_q, cu_k = [0, nq], [0, nk]
    pos = (dict(kv_interleave=R, kv_rank=r, block_size=bs) if interleave
           else dict(k_pos_offset=r * nk))
    seg = seg_size if seg_size else nk
    out = lse = None
    for a in range(0, nk, seg):
        bo, bl = block_forward(q, k, v, cu_q, cu_k, scale, rows=rows, causal=causal, window=window,
                               q_pos_offset=global_q_offset, k_range=(a, a + seg), **pos)
        if out is None:
            out, lse = bo, bl
        else:
            out, lse, _ = merge(out, lse, bo, bl)
    return out, lse


def kvp_forward(q, k_caches, v_caches, tables, n_blocks, seg_size, global_q_offset, window, scale,
                interleave=True, rows=None, causal=True):
    """[KVP] merged output: the R ranks' partials merged by online softmax
    (rank order 0..R-1). Returns (out, lse, partials). q is [S, HQ, D]."""
    R = len(k_caches)
    parts = [kvp_rank_partial(q, k_caches[r], v_caches[r], tables[r], n_blocks, R, r, seg_size,
                              global_q_offset, window, scale, interleave, causal=causal, rows=rows)
             for r in range(R)]
    out, lse = parts[0]
    for r in range(1, R):
        out, lse, _ = merge(out, lse, *parts[r])
    return out, lse, parts


# ----------------------------------------------------------------------------
# one-query decode
# ----------------------------------------------------------------------------
def decode_forward(q, k, v, cu_k, scale, seqs=None):
    """[DEC] one query row per sequence (cu_seqlens_q = arange), a variable
    number of gathered key rows each, GQA, no mask. ``seqs`` selects a sample
    of sequences; other rows come back as out 0, lse -inf."""
    nq = q.shape[0]
    cu_q = np.arange(nq + 1)
    if seqs is None:
        return block_forward(q, k, v, cu_q, cu_k, scale)
    return block_forward(q, k, v, cu_q, cu_k, scale, rows=np.asarray(seqs))


def count_visible_pairs(cu_q, cu_k, **mask):
    """Number of visible (query, key) pairs of a block, per q head."""
    m = _mask_args(mask)
    total = 0
    for d in range(len(doc_bounds(cu_q))):
        qs, ks, qi, kj = _doc_rows(cu_q, cu_k, d, m["q_view"], m["k_view"], None, m.get("k_range"))
        if len(qi) == 0 or len(kj) == 0:
            continue
        qpos, kpos = _positions(qs, ks, qi, kj, m)
        for c0 in range(0, len(qi), 2048):
            total += int(visibility(qpos[c0:c0 + 2048], kpos, m["causal"], m["window"]).sum())
    return total
