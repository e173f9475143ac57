"""GPU parity of Ulysses EAGLE-3 mixed attention (all-to-all reshard between
virtual ranks, full-sequence varlen causal block 0 with the global
cu_seqlens, shard-local TTT diagonals) against the fp64 oracle: the reshard is
bit-exact, (out, lse) and every gradient within the bf16 bounds (2e-2 / 1e-3).
The backward reference is the oracle's gradient at the GPU's merged state."""

import numpy as np
import pytest
import torch

import oracle as O
from blockwise_causal_varlen_amd import inputs, workloads as W

pytestmark = pytest.mark.gpu
OUT_TOL, LSE_TOL = 2e-2, 1e-3


def say(*a):
    print(*a, flush=True)


def f64(t):
    return O.as_f64(t)


def check(name, got, ref, tol=OUT_TOL):
    e = float(np.max(np.abs(f64(got) - ref), initial=0.0))
    say(f"  {name}: max abs err {e:.3e}")
    assert e <= tol, (name, e)


@pytest.mark.parametrize("which", ["uly2_gqa_d128", "uly4_d64"])
def test_ulysses_eagle(gpu_lib, which):
    if which == "uly2_gqa_d128":
        base = inputs.small_zigzag(1024, 16, 300, 8, 2, 128, torch.bfloat16, 2, seed=5)
        uly, n_ttt = 2, 2
    else:
        base = inputs.small_zigzag(1024, 8, 260, 8, 4, 64, torch.bfloat16, 4, seed=6)
        uly, n_ttt = 4, 1
    case = inputs.eagle_case(base, n_ttt)
    cu = base.cu
    say(f"ulysses {which}: docs {(cu[1:] - cu[:-1]).tolist()} uly={uly} ttt={n_ttt}")
    wl = W.UlyssesWorkload(case, uly, with_bwd=True)
    wl.forward()
    torch.cuda.synchronize()
    # the all-to-all reshard is a copy: bit-exact
    ref_qh = O.ulysses_seq_to_head([f64(x.cpu()) for x in wl.q_loc], uly)
    for r in range(uly):
        assert np.array_equal(f64(wl.qh[r].cpu()), ref_qh[r])
    wl.backward()
    torch.cuda.synchronize()
    sl = wl.sl
    ks = [base.k] + list(case.ttt_k)
    vs = [base.v] + list(case.ttt_v)
    ro, rl = O.eagle_forward(base.q, ks, vs, cu, base.scale)
    for r in range(uly):
        say(f" rank {r}")
        check("out", wl.final[r].cpu(), ro[r * sl:(r + 1) * sl])
        check("lse", wl.lse_loc[r].cpu(), rl[:, r * sl:(r + 1) * sl], LSE_TOL)
    dq, dks, dvs = O.eagle_grads(base.dout, base.q, ks, vs, cu, base.scale)
    for r in range(uly):
        rs = slice(r * sl, (r + 1) * sl)
        say(f" rank {r} grads")
        check("dq", wl.dq[r].cpu(), dq[rs])
        check("dk block0", wl.dk[r].cpu(), dks[0][rs])
        check("dv block0", wl.dv[r].cpu(), dvs[0][rs])
        for i in range(n_ttt):
            check(f"dk ttt{i + 1}", wl.dtk[i][r].cpu(), dks[i + 1][rs])
            check(f"dv ttt{i + 1}", wl.dtv[i][r].cpu(), dvs[i + 1][rs])
