"""ATTN_BWD_SET: the zig-zag and ring backward drivers storing the gradients
into buffers full of NaN must give exactly what adding them into zeroed
buffers gives, rows outside every document and key shards no step visits
included (those come out zero)."""

import math

import numpy as np
import pytest
import torch

from blockwise_causal_varlen_amd import inputs, workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def both_modes(run):
    """(set-mode, add-mode) gradients of one runner."""
    grads = lambda: [run.dq] + run.dk + run.dv
    for t in grads():
        t.fill_(float("nan"))
    run.backward(set_grads=True)
    torch.cuda.synchronize()
    got = [t.clone() for t in grads()]
    run.zero_grads()
    run.backward()
    torch.cuda.synchronize()
    return got, [t.clone() for t in grads()]


def same(got, ref, what):
    for i, (a, b) in enumerate(zip(got, ref)):
        assert not torch.isnan(a).any(), f"{what}: tensor {i} kept a NaN"
        assert torch.equal(a, b), f"{what}: tensor {i} differs ({(a - b).abs().max().item():.3e})"


@pytest.mark.parametrize("cp,seed", [(1, 0), (2, 1), (4, 2), (8, 3)])
def test_zigzag_set_equals_add(gpu_lib, cp, seed):
    case = inputs.small_zigzag(1024, 2 * cp, 2 * cp * 30, 8, 2, 128, torch.bfloat16, cp, seed=9100 + seed,
                               loguniform=True)
    say(f"zig-zag cp={cp} docs {(case.cu[1:] - case.cu[:-1]).tolist()}")
    wl = W.ZigzagWorkload(case, with_bwd=True)
    wl.forward()
    for r in range(cp):
        got, ref = both_modes(wl.runners[r])
        same(got, ref, f"rank {r}")


def test_ring_set_with_padding(gpu_lib):
    """Contiguous ring, cp=4, two documents and 24 padding rows after them on
    every shard; ranks below cp - 1 never visit the later shards."""
    L = gpu_lib
    cp, S, pad, hq, hkv, d = 4, 256, 24, 4, 2, 64
    n = 2 * S // cp
    g = torch.Generator().manual_seed(9200)
    q = [inputs.normal((n + pad, hq, d), torch.bfloat16, g).cuda() for _ in range(cp)]
    k = [inputs.normal((n + pad, hkv, d), torch.bfloat16, g).cuda() for _ in range(cp)]
    v = [inputs.normal((n + pad, hkv, d), torch.bfloat16, g).cuda() for _ in range(cp)]
    do = [inputs.normal((n + pad, hq, d), torch.bfloat16, g).cuda() for _ in range(cp)]
    cu_l = (inputs.cu_from_lengths([S, S]) // cp).cuda()
    for r in range(cp):
        say(f"ring rank {r}")
        run = L.RingRunner("ring", cp, r, q[r], k, v, cu_l, S // cp, 1 / math.sqrt(d), dout=do[r])
        run.forward()
        got, ref = both_modes(run)
        same(got, ref, f"rank {r}")
        assert torch.count_nonzero(got[0][n:]) == 0, "padding rows of dq not zero"
        for c in range(r + 1, cp):  # sources this rank never sees
            assert torch.count_nonzero(got[1 + c]) == 0 and torch.count_nonzero(got[1 + cp + c]) == 0
