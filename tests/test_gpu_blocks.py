"""GPU parity of the single-block entry points against the fp64 oracle.

attn_block_fwd, attn_merge_out_lse, attn_merge_n, attn_bwd_delta and
attn_block_bwd are called through the C ABI on seeded inputs, at sizes that
span several tiles and leave ragged tails, and compared element by element
with the oracle. Tolerances: out / dq / dk / dv max abs 2e-2 and lse max abs
1e-3 (bf16 inputs; the same bounds are applied to fp32 inputs, where the
observed errors are far smaller); merges of fp32 inputs 1e-5 relative.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from blockwise_causal_varlen_amd import inputs

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL, MERGE_REL = 2e-2, 1e-3, 1e-5


def say(*a):
    print(*a, flush=True)


def f64(t):
    return O.as_f64(t)


def assert_close_rows(got_out, got_lse, ref_out, ref_lse, rows=None, out_tol=OUT_TOL, lse_tol=LSE_TOL, what=""):
    go, gl = f64(got_out), f64(got_lse)
    if rows is not None:
        go, gl, ref_out, ref_lse = go[rows], gl[:, rows], ref_out[rows], ref_lse[:, rows]
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: -inf pattern of lse differs"
    e_lse = float(np.max(np.abs(gl[fin] - ref_lse[fin]), initial=0.0))
    e_out = float(np.max(np.abs(go - ref_out), initial=0.0))
    say(f"  {what}: max|dout|={e_out:.3e} max|dlse|={e_lse:.3e}")
    assert e_out <= out_tol, f"{what}: out error {e_out}"
    assert e_lse <= lse_tol, f"{what}: lse error {e_lse}"


def rand_case(lens, hq, hkv, d, dtype, seed, k_lens=None):
    g = torch.Generator().manual_seed(seed)
    cu_q = inputs.cu_from_lengths(lens)
    cu_k = inputs.cu_from_lengths(k_lens if k_lens is not None else lens)
    q = inputs.normal((int(cu_q[-1]), hq, d), dtype, g)
    k = inputs.normal((int(cu_k[-1]), hkv, d), dtype, g)
    v = inputs.normal((int(cu_k[-1]), hkv, d), dtype, g)
    return cu_q, cu_k, q, k, v


MASKS = {
    "causal": dict(causal=True),
    "full": dict(),
    "kv_front": dict(k_view="front"),
    "q_back": dict(q_view="back"),
    "window": dict(causal=True, window=77),
    "offsets": dict(causal=True, q_pos_offset=300, k_pos_offset=40),
    "roundrobin": dict(causal=True, q_pos_offset=1000, kv_interleave=4, kv_rank=2, block_size=16),
    "rr_window": dict(causal=True, q_pos_offset=1000, kv_interleave=4, kv_rank=1, block_size=16, window=200),
}


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64),
                                     (torch.float32, 128)])
@pytest.mark.parametrize("mname", list(MASKS))
def test_block_fwd_matches_oracle(gpu_lib, dtype, d, mname):
    L = gpu_lib
    lens = [300, 0, 1, 129, 64, 522]           # empty doc, one-token doc, ragged tails
    klens = lens if "offset" not in mname and "round" not in mname and "rr" not in mname else [310, 0, 5, 140, 64, 530]
    hq, hkv = (8, 2) if d == 128 else (4, 4)
    cu_q, cu_k, q, k, v = rand_case(lens, hq, hkv, d, dtype, seed=7, k_lens=klens)
    mk = MASKS[mname]
    scale = 1.0 / math.sqrt(d)
    say(f"block_fwd {mname} {dtype} D={d} HQ={hq} HKV={hkv}")
    ref_o, ref_l = O.block_forward(q, k, v, cu_q, cu_k, scale, **mk)
    dev = "cuda"
    for out_dtype in (dtype, torch.float32):
        out, lse = L.block_fwd(q.to(dev), k.to(dev), v.to(dev), cu_q, cu_k, max(lens), max(klens), scale,
                               L.mask(**mk), out_dtype=out_dtype)
        torch.cuda.synchronize()
        tol = OUT_TOL if dtype == torch.bfloat16 else 1e-4
        assert_close_rows(out.cpu(), lse.cpu(), ref_o, ref_l, out_tol=tol,
                          lse_tol=LSE_TOL if dtype == torch.bfloat16 else 1e-4, what=f"out {out_dtype}")


def test_block_fwd_untouched_rows_stay(gpu_lib):
    """Rows outside the q view are not written."""
    L = gpu_lib
    cu_q, cu_k, q, k, v = rand_case([64, 200], 4, 4, 64, torch.bfloat16, seed=3)
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((4, q.shape[0]), 9.0, dtype=torch.float32, device="cuda")
    L.block_fwd(q.cuda(), k.cuda(), v.cuda(), cu_q, cu_k, 200, 200, 0.125, L.mask(q_view="back"), out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = out.cpu(), lse.cpu()
    front = list(range(0, 32)) + list(range(64, 164))
    assert torch.all(o[front] == 7.0) and torch.all(l[:, front] == 9.0)
    assert torch.all(o[32:64] != 7.0)


SPLIT_MASKS = {
    "causal_end": dict(causal=True, q_pos_offset=2900),   # query rows at the end of the keys
    "window": dict(causal=True, q_pos_offset=4000, window=700),
    "full": dict(),
    "q_back": dict(q_view="back"),
    "roundrobin": dict(causal=True, q_pos_offset=9000, kv_interleave=4, kv_rank=3, block_size=16),
}


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("mname", list(SPLIT_MASKS))
def test_block_fwd_split_keys(gpu_lib, dtype, d, mname):
    """Few query tiles against thousands of keys: the forward cuts each query
    tile's visible keys into parts (workspace grows by the partials) and
    merges them; every element against the oracle, untouched rows kept."""
    L = gpu_lib
    lens, klens = [96, 200], [3000, 5000]
    hq, hkv = 4, 1
    cu_q, cu_k, q, k, v = rand_case(lens, hq, hkv, d, dtype, seed=41, k_lens=klens)
    mk = SPLIT_MASKS[mname]
    scale = 1.0 / math.sqrt(d)
    say(f"block_fwd split {mname} {dtype} D={d}")
    ws = L.attn_workspace_size(L.OP_BLOCK_FWD, L.desc(q), L.desc(k), len(lens), max(lens), max(klens), L.mask(**mk))
    assert ws >= 2 * q.shape[0] * hq * d * 4, ws   # at least two key parts
    ref_o, ref_l = O.block_forward(q, k, v, cu_q, cu_k, scale, **mk)
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((hq, q.shape[0]), 9.0, dtype=torch.float32, device="cuda")
    L.block_fwd(q.cuda(), k.cuda(), v.cuda(), cu_q, cu_k, max(lens), max(klens), scale, L.mask(**mk),
                out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = out.cpu(), lse.cpu()
    rows = np.arange(q.shape[0])
    if mname == "q_back":
        front = np.r_[0:48, 96:196]
        assert torch.all(o[front] == 7.0) and torch.all(l[:, front] == 9.0)
        rows = np.r_[48:96, 196:296]
    tol = OUT_TOL if dtype == torch.bfloat16 else 1e-4
    assert_close_rows(o, l, ref_o, ref_l, rows=rows, out_tol=tol,
                      lse_tol=LSE_TOL if dtype == torch.bfloat16 else 1e-4, what=mname)


@pytest.mark.parametrize("bdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("view", ["all", "back", "front"])
def test_merge_matches_oracle(gpu_lib, bdtype, view):
    L = gpu_lib
    g = torch.Generator().manual_seed(11)
    lens = [10, 0, 33, 100]
    cu = inputs.cu_from_lengths(lens)
    n, h, d = int(cu[-1]), 3, 128
    out = torch.randn(n, h, d, generator=g)
    lse = torch.randn(h, n, generator=g) * 4
    bout = torch.randn(n, h, d, generator=g).to(bdtype)
    blse = torch.randn(h, n, generator=g) * 4
    lse[0, 5] = float("-inf")
    blse[1, 6] = float("-inf")
    lse[2, 7] = blse[2, 7] = float("-inf")
    ro, rl, rs = O.merge(out, lse, bout, blse)
    # rows outside the view keep the old state
    inview = np.zeros(n, dtype=bool)
    for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()):
        s, e = O.view_range(a, b, view)
        inview[s:e] = True
    ro = np.where(inview[:, None, None], ro, f64(out))
    rl = np.where(inview[None, :], rl, f64(lse))
    go, gl = out.cuda(), lse.cuda()
    w = torch.zeros(h, n, device="cuda")
    fin = torch.zeros(n, h, d, dtype=torch.bfloat16, device="cuda")
    L.merge(go, gl, bout.cuda(), blse.cuda(), cu=cu, q_view=view, weight=w)
    torch.cuda.synchronize()
    err_o = np.max(np.abs(f64(go.cpu()) - ro)) / max(1.0, np.max(np.abs(ro)))
    gl_c = f64(gl.cpu())
    finm = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl_c), finm)
    err_l = np.max(np.abs(gl_c[finm] - rl[finm]) / np.maximum(1.0, np.abs(rl[finm])))
    say(f"merge {bdtype} {view}: rel out {err_o:.2e} rel lse {err_l:.2e}")
    assert err_o <= MERGE_REL and err_l <= MERGE_REL
    ws = f64(w.cpu())[:, inview]
    assert np.max(np.abs(ws - rs[:, inview])) <= MERGE_REL
    # final cast covers every row
    go2, gl2 = out.cuda(), lse.cuda()
    L.merge(go2, gl2, bout.cuda(), blse.cuda(), cu=cu, q_view=view, final_out=fin)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(fin.cpu()) - ro)) <= 1e-2 * max(1.0, np.max(np.abs(ro)))
    assert torch.equal(go2.cpu(), out)  # running out untouched when final_out is given


def test_merge_init_and_merge_n(gpu_lib):
    L = gpu_lib
    g = torch.Generator().manual_seed(5)
    n, h, d = 257, 4, 64
    parts = [torch.randn(n, h, d, generator=g) for _ in range(5)]
    plse = [torch.randn(h, n, generator=g) * 3 for _ in range(5)]
    plse[2][:, 10] = float("-inf")
    for p in plse:
        p[:, 11] = float("-inf")
    ro, rl = f64(parts[0]), f64(plse[0])
    for i in range(1, 5):
        ro, rl, _ = O.merge(ro, rl, parts[i], plse[i])
    out = torch.empty(n, h, d, device="cuda")
    lse = torch.empty(h, n, device="cuda")
    L.merge_n([p.cuda() for p in parts], [p.cuda() for p in plse], out, lse)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(out.cpu()) - ro)) <= MERGE_REL * max(1, np.abs(ro).max())
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(f64(lse.cpu())), fin)
    assert np.max(np.abs(f64(lse.cpu())[fin] - rl[fin])) <= MERGE_REL * max(1, np.abs(rl[fin]).max())
    # init: the state becomes the block, whatever it held
    acc = torch.full((n, h, d), float("nan"), device="cuda")
    al = torch.full((h, n), float("nan"), device="cuda")
    L.merge(acc, al, parts[1].cuda(), plse[1].cuda(), init=True)
    torch.cuda.synchronize()
    assert torch.equal(acc.cpu(), parts[1]) and torch.equal(al.cpu(), plse[1])


def test_delta(gpu_lib):
    L = gpu_lib
    g = torch.Generator().manual_seed(9)
    do = torch.randn(300, 6, 128, generator=g).to(torch.bfloat16)
    o = torch.randn(300, 6, 128, generator=g).to(torch.bfloat16)
    ref = np.einsum("ihd,ihd->hi", f64(do), f64(o))
    got = L.bwd_delta(do.cuda(), o.cuda())
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(got.cpu()) - ref)) < 1e-3


BWD_MASKS = ["causal", "full", "kv_front", "q_back", "window", "offsets", "roundrobin"]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
@pytest.mark.parametrize("mname", BWD_MASKS)
def test_block_bwd_matches_oracle(gpu_lib, dtype, d, mname):
    """Block backward with a merged (here: the block's own, then a foreign)
    out/lse against the oracle's block_backward."""
    L = gpu_lib
    lens = [300, 0, 1, 129, 64, 200]
    klens = lens if mname not in ("offsets", "roundrobin") else [310, 0, 5, 140, 64, 230]
    hq, hkv = (8, 2) if d == 128 else (4, 1)
    cu_q, cu_k, q, k, v = rand_case(lens, hq, hkv, d, dtype, seed=21, k_lens=klens)
    g = torch.Generator().manual_seed(22)
    dout = inputs.normal(q.shape, dtype, g)
    mk = MASKS[mname]
    scale = 1.0 / math.sqrt(d)
    say(f"block_bwd {mname} {dtype} D={d}")
    # merged state = this block plus a synthetic second partial, so lse != block lse
    bo, bl = O.block_forward(q, k, v, cu_q, cu_k, scale, **mk)
    extra_o = np.random.default_rng(3).standard_normal(bo.shape)
    extra_l = np.random.default_rng(4).standard_normal(bl.shape)
    mo, ml, _ = O.merge(bo, bl, extra_o, extra_l)
    out_t = torch.from_numpy(mo).to(dtype)
    lse_t = torch.from_numpy(ml).float()
    rdq, rdk, rdv = O.block_backward(dout, q, k, v, out_t, lse_t, cu_q, cu_k, scale, **mk)
    dq, dk, dv = L.block_bwd(dout.cuda(), q.cuda(), k.cuda(), v.cuda(), out_t.cuda(), lse_t.cuda(), cu_q, cu_k,
                             max(lens), max(klens), scale, L.mask(**mk))
    torch.cuda.synchronize()
    tol = OUT_TOL if dtype == torch.bfloat16 else 1e-4
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e = float(np.max(np.abs(f64(got.cpu()) - ref)))
        say(f"  {name}: {e:.3e} (max |ref| {np.max(np.abs(ref)):.2f})")
        assert e <= tol, (name, e)


def test_block_bwd_accumulates_and_is_deterministic(gpu_lib):
    L = gpu_lib
    cu_q, cu_k, q, k, v = rand_case([500, 77], 8, 2, 128, torch.bfloat16, seed=31)
    dout = inputs.normal(q.shape, torch.bfloat16, torch.Generator().manual_seed(32))
    out, lse = L.block_fwd(q.cuda(), k.cuda(), v.cuda(), cu_q, cu_k, 500, 500, 0.088, L.mask(causal=True))
    args = (dout.cuda(), q.cuda(), k.cuda(), v.cuda(), out, lse, cu_q, cu_k, 500, 500, 0.088, L.mask(causal=True))
    a = L.block_bwd(*args)
    b = L.block_bwd(*args)
    c = L.block_bwd(*args, dq=a[0].clone(), dk=a[1].clone(), dv=a[2].clone())
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y)                     # bitwise repeatable
        assert torch.allclose(z, 2 * x, rtol=1e-6, atol=1e-6)  # += semantics
