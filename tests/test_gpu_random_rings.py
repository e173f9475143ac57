"""Seeded random sweep of the zig-zag ring drivers (forward with the merge in
the epilogue, backward with the merged state) against the fp64 oracle: every
virtual rank of rings of cp = 1, 2, 4 or 8, random document mixes (uniform or
log-uniform lengths, multiples of 2 cp), GQA layouts, D = 64 or 128, bf16 or
f32. Per rank out and lse; per owner the dK / dV summed over the ranks; the
oracle's backward runs at the oracle's own merged (out, lse). The
contiguous causal ring drivers get the same treatment over random documents
(multiples of cp).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from blockwise_causal_varlen_amd import inputs, workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 44


def say(*a):
    print(*a, flush=True)


def draw(i):
    rng = np.random.default_rng(3000 + i)
    cp = int(rng.choice([1, 2, 4, 8]))
    total = int(rng.choice([512, 1024, 2048]))
    lo = 2 * cp * int(rng.integers(1, 8))
    hi = lo + 2 * cp * int(rng.integers(1, 40))
    hq, hkv = [(4, 1), (4, 2), (2, 2), (8, 2)][int(rng.integers(4))]
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    return cp, total, lo, hi, hq, hkv, d, dtype, bool(rng.random() < 0.5)


def err(a, b):
    return float(np.max(np.abs(O.as_f64(a) - b), initial=0.0))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_zigzag(gpu_lib, i):
    cp, total, lo, hi, hq, hkv, d, dtype, logu = draw(i)
    case = inputs.small_zigzag(total, lo, hi, hq, hkv, d, dtype, cp, seed=4000 + i, loguniform=logu)
    cu = case.cu
    say(f"case {i}: cp={cp} docs {(cu[1:] - cu[:-1]).tolist()} heads {hq}/{hkv} D={d} {dtype}")
    tol, lse_tol = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-4, 1e-5)
    wl = W.ZigzagWorkload(case, with_bwd=True)
    wl.forward()
    wl.backward()
    torch.cuda.synchronize()
    oq = [O.zigzag_shard(case.q, cu, cp, r)[0] for r in range(cp)]
    ok = [O.zigzag_shard(case.k, cu, cp, r)[0] for r in range(cp)]
    ov = [O.zigzag_shard(case.v, cu, cp, r)[0] for r in range(cp)]
    odo = [O.zigzag_shard(case.dout, cu, cp, r)[0] for r in range(cp)]
    dk_ref = [np.zeros(np.asarray(x).shape) for x in ok]
    dv_ref = [np.zeros(np.asarray(x).shape) for x in ov]
    dk_got = [np.zeros(np.asarray(x).shape) for x in ok]
    dv_got = [np.zeros(np.asarray(x).shape) for x in ov]
    for r in range(cp):
        run = wl.runners[r]
        ro, rl = O.zigzag_forward(oq, ok, ov, cu, cp, r, case.scale)
        gl = O.as_f64(run.lse.cpu())
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin), f"rank {r}: -inf pattern of lse differs"
        e_out, e_lse = err(run.out.cpu(), ro), float(np.max(np.abs(gl[fin] - rl[fin]), initial=0.0))
        dq, dk, dv = O.zigzag_backward(odo[r], oq, ok, ov, ro, rl, cu, cp, r, case.scale)
        e_dq = err(run.dq.cpu(), dq)
        say(f"  rank {r}: out {e_out:.2e} lse {e_lse:.2e} dq {e_dq:.2e}")
        assert e_out <= tol and e_lse <= lse_tol and e_dq <= tol, (r, e_out, e_lse, e_dq)
        for s in range(cp):
            dk_ref[s] += dk[s]
            dv_ref[s] += dv[s]
            dk_got[s] += O.as_f64(run.dk[s].cpu())
            dv_got[s] += O.as_f64(run.dv[s].cpu())
    for s in range(cp):
        e_dk = float(np.max(np.abs(dk_got[s] - dk_ref[s]), initial=0.0))
        e_dv = float(np.max(np.abs(dv_got[s] - dv_ref[s]), initial=0.0))
        say(f"  owner {s}: dk {e_dk:.2e} dv {e_dv:.2e}")
        assert e_dk <= tol and e_dv <= tol, (s, e_dk, e_dv)


def ring_local(x, cu, cp, r):
    """Rank r's contiguous chunk of every document, packed (torch, on the GPU)."""
    b = cu.tolist()
    return torch.cat([x[s + r * ((e - s) // cp):s + (r + 1) * ((e - s) // cp)] for s, e in zip(b[:-1], b[1:])]).cuda()


@pytest.mark.parametrize("i", range(26))
def test_random_ring(gpu_lib, i):
    """Contiguous causal ring drivers: every rank of cp = 1, 2, 4 or 8 over
    random documents (multiples of cp), stored gradients, against the oracle;
    dK / dV per owner summed over the ranks."""
    L = gpu_lib
    rng = np.random.default_rng(3500 + i)
    cp = int(rng.choice([1, 2, 4, 8]))
    lens = [cp * int(x) for x in rng.integers(1, 300 // cp + 2, int(rng.integers(1, 5)))]
    hq, hkv = [(4, 1), (4, 2), (2, 2), (8, 2)][int(rng.integers(4))]
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    tol, lse_tol = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-4, 1e-5)
    say(f"case {i}: cp={cp} docs {lens} heads {hq}/{hkv} D={d} {dtype}")
    g = torch.Generator().manual_seed(3600 + i)
    cu = inputs.cu_from_lengths(lens)
    n = int(cu[-1])
    q, do = (inputs.normal((n, hq, d), dtype, g) for _ in range(2))
    k, v = (inputs.normal((n, hkv, d), dtype, g) for _ in range(2))
    oq, ok, ov, odo = ([O.ring_shard(x, cu, cp, r)[0] for r in range(cp)] for x in (q, k, v, do))
    tk = [ring_local(k, cu, cp, r) for r in range(cp)]
    tv = [ring_local(v, cu, cp, r) for r in range(cp)]
    cu_l = (cu // cp).cuda()
    max_local = max(lens) // cp
    dk_ref = [np.zeros(np.asarray(x).shape) for x in ok]
    dv_ref = [np.zeros(np.asarray(x).shape) for x in ov]
    dk_got = [np.zeros(np.asarray(x).shape) for x in ok]
    dv_got = [np.zeros(np.asarray(x).shape) for x in ov]
    for r in range(cp):
        run = L.RingRunner("ring", cp, r, ring_local(q, cu, cp, r), tk, tv, cu_l, max_local, 1 / math.sqrt(d),
                           dout=ring_local(do, cu, cp, r))
        run.forward()
        run.backward(set_grads=True)
        torch.cuda.synchronize()
        ro, rl = O.ring_forward(oq, ok, ov, cu, cp, r, 1 / math.sqrt(d))
        gl = O.as_f64(run.lse.cpu())
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin), f"rank {r}: -inf pattern of lse differs"
        e_out, e_lse = err(run.out.cpu(), ro), float(np.max(np.abs(gl[fin] - rl[fin]), initial=0.0))
        dq, dk, dv = O.ring_backward(odo[r], oq, ok, ov, ro, rl, cu, cp, r, 1 / math.sqrt(d))
        e_dq = err(run.dq.cpu(), dq)
        say(f"  rank {r}: out {e_out:.2e} lse {e_lse:.2e} dq {e_dq:.2e}")
        assert e_out <= tol and e_lse <= lse_tol and e_dq <= tol, (r, e_out, e_lse, e_dq)
        for s in range(cp):
            dk_ref[s] += dk[s]
            dv_ref[s] += dv[s]
            dk_got[s] += O.as_f64(run.dk[s].cpu())
            dv_got[s] += O.as_f64(run.dv[s].cpu())
    for s in range(cp):
        e_dk = float(np.max(np.abs(dk_got[s] - dk_ref[s]), initial=0.0))
        e_dv = float(np.max(np.abs(dv_got[s] - dv_ref[s]), initial=0.0))
        say(f"  owner {s}: dk {e_dk:.2e} dv {e_dv:.2e}")
        assert e_dk <= tol and e_dv <= tol, (s, e_dk, e_dv)
