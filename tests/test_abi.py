"""CPU tests of the C-ABI library: it loads, exports every entry point the
header declares, and rejects bad arguments with the documented status codes
before touching a GPU (validation never launches anything)."""

import ctypes as C
import os
import re

import pytest
import torch

from blockwise_causal_varlen_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    return L.load()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound(so):
    names = declared()
    assert "attn_block_fwd" in names and "attn_merge_out_lse" in names and "attn_block_bwd" in names
    for n in names:
        assert hasattr(so, n), n
    assert set(names) == set(L.EXPORTS)


def test_version_and_strings(so):
    assert L.attn_abi_version() == 1
    assert L.attn_status_string(0) == "ok"
    assert L.attn_status_string(8) == "workspace too small"


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def T(n=64, h=4, d=128, dtype=L.BF16, st=None, sh=None, data=FAKE):
    return L.AttnTensor(data, dtype, 0, n, h, d, st if st is not None else h * d, sh if sh is not None else d)


def fwd(q, k, v, m=None, out=None, lse=FAKE, ws=FAKE, wsb=1 << 30, num_seqs=1, cu=FAKE, scale=0.1):
    out = out or T(q.n_tok, q.n_head, q.head_dim)
    return L.load().attn_block_fwd(C.byref(q), C.byref(k), C.byref(v), cu, cu, num_seqs, 64, 64,
                                   None if m is None else C.byref(m), scale, C.byref(out), lse, ws, wsb, None)


def test_fwd_error_codes(so):
    q = T()
    assert fwd(q, T(dtype=L.F32), T()) == 2                        # dtype mismatch
    assert fwd(T(dtype=5), T(dtype=5), T(dtype=5)) == 2            # unsupported dtype
    assert fwd(q, T(d=64), T(d=64)) == 3                           # head_dim mismatch
    assert fwd(T(d=96), T(d=96), T(d=96)) == 7                     # D not 64/128
    assert fwd(T(h=6), T(h=4), T(h=4)) == 4                        # GQA
    assert fwd(q, T(), T(), lse=None) == 1                         # null lse
    assert fwd(q, T(), T(), cu=None) == 1                          # null cu_seqlens
    assert fwd(q, T(), T(), num_seqs=-1) == 5
    assert fwd(q, T(st=100), T()) == 6                             # misaligned stride
    assert fwd(q, T(data=FAKE + 2), T()) == 6                      # misaligned pointer
    assert fwd(q, T(), T(), scale=0.0) == 11
    assert fwd(q, T(), T(), ws=None, wsb=0) == 8                   # workspace missing
    assert fwd(q, T(), T(), wsb=16) == 8                           # workspace too small
    assert "workspace" in L.attn_last_error()
    assert fwd(q, T(), T(), out=T(n=63)) == 3                      # out shape


def test_mask_struct_version_and_values(so):
    q = T()
    m = L.mask(causal=True)
    assert C.sizeof(L.AttnMask) == 80
    m.struct_size = 72
    assert fwd(q, T(), T(), m) == 10                               # version mismatch
    assert fwd(q, T(), T(), L.mask(q_view=3)) == 11
    assert fwd(q, T(), T(), L.mask(window=-1)) == 11
    assert fwd(q, T(), T(), L.mask(kv_interleave=4, kv_rank=4, block_size=16)) == 11
    bt = torch.zeros(4, dtype=torch.int32)
    assert fwd(q, T(), T(), L.mask(block_table=bt)) == 11          # paged without sizes
    assert fwd(q, T(), T(), L.mask(seg_size=64, q_view="back")) == 7


def test_workspace_size_is_host_only(so):
    q, k = T(n=1000, h=8), T(n=1000, h=2)
    a = L.attn_workspace_size(L.OP_BLOCK_FWD, q, k, 3, 500, 500, L.mask(causal=True))
    b = L.attn_workspace_size(L.OP_BLOCK_FWD, q, k, 3, 500, 500, L.mask(causal=True, seg_size=128))
    assert 0 < a < b                                               # segments need partial buffers
    assert b - a >= 4 * 1000 * 8 * 128 * 4
    dec = L.attn_workspace_size(L.OP_BLOCK_FWD, T(n=10, h=8), k, 10, 1, 500, None)
    assert dec == 0                                                # one-query decode needs none
    assert L.attn_workspace_size(L.OP_BLOCK_BWD, q, k, 3, 500, 500, None) > 0


def test_workspace_bytes_alias_and_kvp_paging(so):
    """attn_workspace_bytes answers as attn_workspace_size; the KV-parallel
    workspace is planned for paged keys whether or not the mask carries a
    block_table (the tables come in their own argument), and a mask without
    page sizes is refused."""
    lib = L.load()
    q, k = T(n=1000, h=8), T(n=1000, h=2)
    for m in (L.mask(causal=True), L.mask(causal=True, seg_size=128), None):
        a, b = C.c_size_t(0), C.c_size_t(0)
        ref = None if m is None else C.byref(m)
        assert lib.attn_workspace_size(0, C.byref(q), C.byref(k), 3, 500, 500, ref, C.byref(a)) == 0
        assert lib.attn_workspace_bytes(0, C.byref(q), C.byref(k), 3, 500, 500, ref, C.byref(b)) == 0
        assert a.value == b.value > 0
    assert lib.attn_workspace_bytes(5, C.byref(q), C.byref(k), 3, 500, 500, None, C.byref(a)) == 11
    qk, kc = T(n=1, h=4), T(n=320, h=2)
    sizes = []
    for bt in (None, torch.zeros(20, dtype=torch.int32)):
        m = L.mask(block_size=16, max_blocks=20, page_stride=2 * 16 * 128, block_table=bt)
        n = C.c_size_t(0)
        assert lib.attn_kvp_workspace_size(3, C.byref(qk), C.byref(kc), 1, 1, 320, C.byref(m), C.byref(n)) == 0
        sizes.append(n.value)
    assert sizes[0] == sizes[1] >= 3 * 2 * 320 * 2 * 128 * 2      # the three ranks' gathered K and V
    n = C.c_size_t(0)
    m = L.mask(causal=True)
    assert lib.attn_kvp_workspace_size(3, C.byref(qk), C.byref(kc), 1, 1, 320, C.byref(m), C.byref(n)) == 11
    assert lib.attn_kvp_workspace_size(3, C.byref(qk), C.byref(kc), 1, 1, 320, None, C.byref(n)) == 1


def test_merge_and_bwd_error_codes(so):
    lib = L.load()
    o = T(dtype=L.F32)
    assert lib.attn_merge_out_lse(C.byref(T()), FAKE, C.byref(T()), FAKE, None, 0, 0, None, None, 0, None) == 2
    assert lib.attn_merge_out_lse(C.byref(o), FAKE, C.byref(T(n=3)), FAKE, None, 0, 0, None, None, 0, None) == 3
    assert lib.attn_merge_out_lse(C.byref(o), FAKE, C.byref(T()), FAKE, None, 0, 1, None, None, 0, None) == 1
    assert lib.attn_merge_n(0, None, None, C.byref(o), FAKE, None) == 11
    g = T(dtype=L.F32)
    args = [C.byref(T()), C.byref(T()), C.byref(T()), C.byref(T()), C.byref(T()), FAKE, FAKE, FAKE, FAKE, 1, 64, 64,
            None, 0.1, C.byref(g), C.byref(g), C.byref(g), FAKE, 1 << 30, None]
    a = list(args)
    a[14] = C.byref(T())                                           # dq must be f32
    assert lib.attn_block_bwd(*a) == 2
    a = list(args)
    a[12] = C.byref(L.mask(block_table=torch.zeros(2, dtype=torch.int32), block_size=16, max_blocks=2, page_stride=1))
    assert lib.attn_block_bwd(*a) == 7                             # paged backward unsupported
    a = list(args)
    a[18] = 8
    assert lib.attn_block_bwd(*a) == 8


def test_schedule_arg_errors(so):
    lib = L.load()
    arr = (L.AttnTensor * 2)(T(), T())
    o = T(dtype=L.F32)
    assert lib.attn_zigzag_fwd(2, 2, C.byref(T()), arr, arr, FAKE, 1, 64, 0.1, C.byref(o), C.byref(T()), FAKE, FAKE,
                               1 << 30, None) == 11                # rank >= cp
    assert lib.attn_zigzag_fwd(2, 0, C.byref(T()), arr, arr, FAKE, 1, 64, 0.1, C.byref(T()), C.byref(T()), FAKE, FAKE,
                               1 << 30, None) == 2                 # out_acc must be f32
    assert lib.attn_zigzag_shard(C.byref(T(n=64)), FAKE, 1, 64, 2, 0, C.byref(T(n=31)), None) == 3
    assert lib.attn_kvp_fwd(0, C.byref(T()), arr, arr, None, FAKE, FAKE, 1, 64, 64, None, 0.1, C.byref(T()), FAKE,
                            FAKE, 1 << 30, None) == 11


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.load()


def test_backward_driver_flags(so):
    """attn_*_bwd_ex: unknown flag bits, the cp limit of ATTN_BWD_SET and a bad
    gradient shape are refused before anything is launched (no GPU here, so a
    launch would have reported ATTN_ERR_HIP instead)."""
    lib = L.load()

    def call(fn, cp, flags, dk_bad=False):
        kv = (L.AttnTensor * cp)(*[T(h=2) for _ in range(cp)])
        gs = [T(h=2, dtype=L.F32) for _ in range(cp)]
        if dk_bad:
            gs[0] = T(n=63, h=2, dtype=L.F32)  # rank 0 uses source 0 in both rings
        g = (L.AttnTensor * cp)(*gs)
        gv = (L.AttnTensor * cp)(*[T(h=2, dtype=L.F32) for _ in range(cp)])
        return getattr(lib, fn)(cp, 0, C.byref(T()), C.byref(T()), kv, kv, C.byref(T()), FAKE, FAKE, 1, 64, 0.1,
                                C.byref(T(dtype=L.F32)), g, gv, FAKE, 1 << 30, None, flags)

    for fn in ("attn_zigzag_bwd_ex", "attn_ring_bwd_ex"):
        assert call(fn, 2, 2) == 11                                # unknown flag bit
        assert call(fn, 2, 1 | 4) == 11
        assert call(fn, 2, L.BWD_SET, dk_bad=True) == 3            # dk of one owner misshaped
        assert call(fn, 2, 0, dk_bad=True) == 3
    # ring rank 0 uses only source 0, but stored mode zeroes source 1's buffers too
    kv = (L.AttnTensor * 2)(T(h=2), T(h=2))
    for bad, code in ((T(h=2), 2), (T(n=65, h=2, dtype=L.F32), 3)):
        g = (L.AttnTensor * 2)(T(h=2, dtype=L.F32), bad)
        gv = (L.AttnTensor * 2)(T(h=2, dtype=L.F32), T(h=2, dtype=L.F32))
        assert lib.attn_ring_bwd_ex(2, 0, C.byref(T()), C.byref(T()), kv, kv, C.byref(T()), FAKE, FAKE, 1, 64, 0.1,
                                    C.byref(T(dtype=L.F32)), g, gv, FAKE, 1 << 30, None, L.BWD_SET) == code
    assert call("attn_zigzag_bwd_ex", 20, L.BWD_SET) == 7          # 2 cp + 1 buffers beyond the zeroing launch
    assert "ATTN_BWD_SET" in L.attn_last_error()
