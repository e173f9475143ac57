"""GPU parity of EAGLE-3 mixed attention (zig-zag cache block 0 + per-position
test-time-training diagonal blocks) against the fp64 oracle's joint softmax,
all virtual ranks, forward and backward.

Tolerances as for the schedules: out / dq / dk / dv max abs 2e-2 and lse max
abs 1e-3 (bf16 inputs); the fp32 case asserts the same bounds.
The backward reference is the oracle's gradient at the GPU's merged state (its
final output in q's dtype and its lse), which is what the backward is given.
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


def f64(t):
    return O.as_f64(t)


def check(name, got, ref, tol=OUT_TOL):
    e = float(np.max(np.abs(f64(got) - ref), initial=0.0))
    say(f"  {name}: max abs err {e:.3e}")
    assert e <= tol, (name, e)


def shard(x, cu, cp, r):
    return O.zigzag_shard(x, cu, cp, r)[0]


@pytest.mark.parametrize("which", ["small_bf16", "gqa_d64_bf16", "cfg1_f32"])
def test_eagle_zigzag_all_ranks(gpu_lib, which):
    if which == "small_bf16":
        base = inputs.small_zigzag(1024, 16, 300, 8, 2, 128, torch.bfloat16, 2, seed=3)
        n_ttt = 3
    elif which == "gqa_d64_bf16":
        base = inputs.small_zigzag(768, 8, 200, 4, 1, 64, torch.bfloat16, 4, seed=4)
        n_ttt = 2
    else:
        base = inputs.cfg1()
        n_ttt = 1
    case = inputs.eagle_case(base, n_ttt)
    cp, cu = base.cp, base.cu
    say(f"eagle {which}: docs {(cu[1:] - cu[:-1]).tolist()} cp={cp} ttt={n_ttt}")
    wl = W.EagleWorkload(case, with_bwd=True)
    wl.forward()
    wl.backward()
    torch.cuda.synchronize()
    ks = [base.k] + list(case.ttt_k)
    vs = [base.v] + list(case.ttt_v)
    ro, rl = O.eagle_forward(base.q, ks, vs, cu, base.scale)
    for r in range(cp):
        run = wl.zz.runners[r]
        say(f" rank {r}")
        check("out", wl.final[r].cpu(), shard(ro, cu, cp, r))
        check("lse", run.lse.cpu(), shard(rl.T, cu, cp, r).T, LSE_TOL)
    # end to end: the oracle's gradients of its own joint softmax
    dq, dks, dvs = O.eagle_grads(base.dout, base.q, ks, vs, cu, base.scale)
    dk0 = [torch.zeros_like(wl.zz.runners[0].dk[s]) for s in range(cp)]
    dv0 = [torch.zeros_like(wl.zz.runners[0].dv[s]) for s in range(cp)]
    for r in range(cp):
        run = wl.zz.runners[r]
        say(f" rank {r} grads")
        check("dq", run.dq.cpu(), shard(dq, cu, cp, r))
        for i in range(n_ttt):
            check(f"dk ttt{i + 1}", wl.dtk[r][i].cpu(), shard(dks[i + 1], cu, cp, r))
            check(f"dv ttt{i + 1}", wl.dtv[r][i].cpu(), shard(dvs[i + 1], cu, cp, r))
        for s in range(cp):
            dk0[s] += run.dk[s]
            dv0[s] += run.dv[s]
    for s in range(cp):
        check(f"dk block0 owner {s}", dk0[s].cpu(), shard(dks[0], cu, cp, s))
        check(f"dv block0 owner {s}", dv0[s].cpu(), shard(dvs[0], cu, cp, s))
