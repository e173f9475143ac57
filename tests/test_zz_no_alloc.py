"""attn_block_fwd_noalloc (the forward entry point that allocates nothing; its
workspace is the library's own device array) against attn_block_fwd with a
caller workspace: two calls in a row, the second smaller, each compared with
the workspace entry point's output on the same inputs (bit-exact where both
make the same plan, and within the forward bars 2e-2 / 1e-3 in any case), and
a call too large for the array refused before anything runs."""

import math

import numpy as np
import pytest
import torch

from blockwise_causal_varlen_amd import inputs, lib as L

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_pair(lens, klens, hq, hkv, d, mk, seed):
    g = torch.Generator().manual_seed(seed)
    cu_q, cu_k = inputs.cu_from_lengths(lens), inputs.cu_from_lengths(klens)
    q = inputs.normal((int(cu_q[-1]), hq, d), torch.bfloat16, g).cuda()
    k = inputs.normal((int(cu_k[-1]), hkv, d), torch.bfloat16, g).cuda()
    v = inputs.normal((int(cu_k[-1]), hkv, d), torch.bfloat16, g).cuda()
    scale = 1.0 / math.sqrt(d)
    m = L.mask(**mk)
    ref_o, ref_l = L.block_fwd(q, k, v, cu_q, cu_k, max(lens), max(klens), scale, m)
    out = torch.zeros_like(ref_o)
    lse = torch.full_like(ref_l, float("-inf"))
    L.block_fwd_noalloc(q, k, v, cu_q.cuda(), cu_k.cuda(), max(lens), max(klens), scale, m, out, lse)
    torch.cuda.synchronize()
    e_o = float((out.float() - ref_o.float()).abs().max()) if out.numel() else 0.0
    fin = torch.isfinite(ref_l)
    assert torch.equal(torch.isfinite(lse), fin)
    e_l = float((lse[fin] - ref_l[fin]).abs().max()) if fin.any() else 0.0
    same = torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    say(f"  lens {lens} heads {hq}/{hkv} D={d} {mk}: out {e_o:.2e} lse {e_l:.2e} bit-exact {same}")
    assert e_o <= 2e-2 and e_l <= 1e-3
    return same


def test_noalloc_forward_two_calls(gpu_lib):
    say("first call (larger)")
    # a grid large enough that neither entry point splits the keys: same plan, same bits
    assert run_pair([3000, 1100, 2048], [3000, 1100, 2048], 16, 4, 128, dict(causal=True), seed=21)
    say("second call (smaller, left-over array contents from the first)")
    run_pair([129, 64, 7], [300, 64, 7], 4, 1, 64, dict(causal=True, window=100, q_pos_offset=171), seed=22)


def test_noalloc_refuses_what_does_not_fit(gpu_lib):
    """Paged keys of 2 x 40 MB gathered rows need more workspace than the
    array holds: ATTN_ERR_WORKSPACE, nothing launched, outputs untouched."""
    pages, bs, hkv, d = 2560, 64, 2, 128
    cache = torch.zeros(pages, hkv, bs, d, dtype=torch.bfloat16, device="cuda")
    kd, pstride = L.paged_desc(cache)
    q = torch.zeros(16, 4, d, dtype=torch.bfloat16, device="cuda")
    table = torch.arange(pages, dtype=torch.int32, device="cuda")
    m = L.mask(causal=False, block_size=bs, max_blocks=pages, page_stride=pstride, block_table=table)
    out = torch.full((16, 4, d), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((4, 16), 5.0, dtype=torch.float32, device="cuda")
    cu_q = torch.tensor([0, 16], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, pages * bs], dtype=torch.int32, device="cuda")
    with pytest.raises(L.AttnError) as e:
        L.block_fwd_noalloc(q, None, None, cu_q, cu_k, 16, pages * bs, 0.1, m, out, lse, k_desc=kd, v_desc=kd)
    say(f"  refused: {e.value}")
    assert e.value.status == 8 and "at most" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 5.0).all())
