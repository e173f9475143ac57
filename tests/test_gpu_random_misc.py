"""Seeded random sweeps of the KV-parallel prefill and the one-query decode
against the fp64 oracle, every element.

KV-parallel: R = 1, 2 or 4 ranks, pages of 16 or 32 tokens in random block
tables, 1..200 query rows whose global positions sit at, before or past the
end of the keys, windows from 1 key to beyond the keys, segments or none,
round-robin or contiguous key positions, GQA layouts and D. Decode: group
sizes on both sides of the decode kernel's limit (16 q heads per kv head),
short and empty-to-long key lengths, and a few long sequences (the split-KV
regime where (sequence, kv head) pairs alone cannot fill the chip).
"""

import numpy as np
import pytest
import torch

import oracle as O
from blockwise_causal_varlen_amd import inputs, workloads as W

pytestmark = pytest.mark.gpu
OUT_TOL, LSE_TOL = 2e-2, 1e-3


def say(*a):
    print(*a, flush=True)


def check(out, lse, ro, rl, what, tol=OUT_TOL, lse_tol=LSE_TOL):
    go, gl = O.as_f64(out.cpu()), O.as_f64(lse.cpu())
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: -inf pattern of lse differs"
    e_o = float(np.max(np.abs(go - ro), initial=0.0))
    e_l = float(np.max(np.abs(gl[fin] - rl[fin]), initial=0.0))
    say(f"  {what}: out {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= tol and e_l <= lse_tol, (what, e_o, e_l)


@pytest.mark.parametrize("i", range(40))
def test_random_kvp(gpu_lib, i):
    rng = np.random.default_rng(5000 + i)
    R = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([16, 32]))
    nb = int(rng.choice([8, 24, 40]))
    s_q = int(rng.choice([1, 63, 200]))
    hq, hkv = [(8, 1), (4, 2), (2, 2)][int(rng.integers(3))]
    d = int(rng.choice([64, 128]))
    window = int(rng.choice([0, 0, 1, 17, 300, 5000]))
    seg = int(rng.choice([0, 64, 96, 512]))
    n_glob = nb * bs * R
    off = int(rng.integers(max(0, n_glob - s_q - 200), n_glob + 50))
    interleave = bool(rng.random() < 0.6)
    say(f"case {i}: R={R} pages {nb}x{bs} s_q={s_q} heads {hq}/{hkv} D={d} window={window} seg={seg} "
        f"offset={off} interleave={interleave}")
    case = inputs.cfg4(window=window, s_q=s_q, hq=hq, hkv=hkv, d=d, num_blocks=nb, block_size=bs, R=R,
                       seg_size=seg, global_q_offset=off, seed=6000 + i)
    wl = W.KvpWorkload(case)
    if not interleave:
        wl.mask.kv_interleave = 0
    out, lse = wl.forward()
    torch.cuda.synchronize()
    ro, rl, _ = O.kvp_forward(case.q.transpose(0, 1), case.k_caches, case.v_caches, case.tables, nb, seg, off,
                              window, case.scale, interleave=interleave)
    check(out, lse, ro, rl, f"kvp {i}")


@pytest.mark.parametrize("i", range(32))
def test_random_decode(gpu_lib, i):
    L = gpu_lib
    rng = np.random.default_rng(7000 + i)
    hq, hkv = [(32, 4), (16, 1), (32, 1), (4, 4), (8, 2)][int(rng.integers(5))]
    d = int(rng.choice([64, 128]))
    if rng.random() < 0.3:  # a few long sequences: split-KV regime
        lens = [int(x) for x in rng.integers(1, 20000, int(rng.integers(1, 4)))]
        case = inputs.long_decode(lens, hq=hq, hkv=hkv, d=d, seed=8000 + i)
    else:
        nseq, max_len = int(rng.choice([1, 5, 300])), int(rng.choice([1, 33, 600]))
        case = inputs.cfg5(device="cpu", nseq=nseq, max_len=max_len, hq=hq, hkv=hkv, d=d, seed=8000 + i)
    nseq = case.q.shape[0]
    say(f"case {i}: {nseq} sequences, k lengths up to {int(case.k_lens.max())}, heads {hq}/{hkv} D={d}")
    cu_q = torch.arange(nseq + 1, dtype=torch.int32)
    out, lse = L.block_fwd(case.q.cuda(), case.k.cuda(), case.v.cuda(), cu_q, case.cu_k, 1, int(case.k_lens.max()),
                           case.scale, None)
    torch.cuda.synchronize()
    ro, rl = O.decode_forward(case.q, case.k, case.v, case.cu_k, case.scale)
    check(out, lse, ro, rl, f"decode {i}")


@pytest.mark.parametrize("R,dtype", [(10, torch.bfloat16), (3, torch.float32)])
def test_kvp_rank_batches(gpu_lib, R, dtype):
    """The ranks' forwards run batched up to 8 to a launch: 10 ranks take two
    launches; f32 inputs take one launch per rank."""
    say(f"kvp R={R} {dtype}")
    case = inputs.cfg4(window=300, s_q=130, hq=4, hkv=2, d=64, num_blocks=12, block_size=16, R=R, seg_size=96,
                       global_q_offset=R * 12 * 16 - 100, seed=9300 + R, dtype=dtype)
    wl = W.KvpWorkload(case)
    out, lse = wl.forward()
    torch.cuda.synchronize()
    ro, rl, _ = O.kvp_forward(case.q.transpose(0, 1), case.k_caches, case.v_caches, case.tables, 12, 96,
                              R * 12 * 16 - 100, 300, case.scale, interleave=True)
    f32 = dtype == torch.float32
    check(out, lse, ro, rl, f"kvp R={R}", *((1e-4, 1e-5) if f32 else (OUT_TOL, LSE_TOL)))


def test_kvp_one_query_unmasked_contiguous(gpu_lib):
    """A single query row, no causal mask, no window, contiguous shards and no
    block_table in the mask: the driver pages through block_tables and runs
    the tiled forward for every rank (not the one-query decode kernel)."""
    case = inputs.cfg4(window=0, s_q=1, hq=4, hkv=2, d=128, num_blocks=20, block_size=16, R=3, seg_size=0,
                       global_q_offset=700, seed=9400)
    wl = W.KvpWorkload(case)
    wl.mask.causal = 0
    wl.mask.kv_interleave = 0
    wl.mask.block_table = None
    out, lse = wl.forward()
    torch.cuda.synchronize()
    ro, rl, _ = O.kvp_forward(case.q.transpose(0, 1), case.k_caches, case.v_caches, case.tables, 20, 0, 700, 0,
                              case.scale, interleave=False, causal=False)
    check(out, lse, ro, rl, "kvp one query")
