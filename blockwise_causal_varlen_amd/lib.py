"""ctypes binding of the C ABI in include/attn.h.

Argument marshalling only: every function here builds descriptors, allocates
outputs and workspaces with torch (device memory and streams are all torch is
used for) and calls the HIP library; all arithmetic runs in the library's
kernels. The library is loaded on first use; a missing build raises.

Low-level names mirror the C ABI (``attn_block_fwd``, ``attn_merge_out_lse``,
``attn_block_bwd``, ...) and take ``AttnTensor`` / ``AttnMask`` structures.
The helpers ``block_fwd``, ``merge``, ``block_bwd``, ``zigzag_fwd`` etc. take
torch tensors.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

BF16, F32 = 0, 1
VIEW_ALL, VIEW_FRONT, VIEW_BACK = 0, 1, 2
OP_BLOCK_FWD, OP_BLOCK_BWD = 0, 1
BWD_SET = 1  # ATTN_BWD_SET: the backward drivers set the gradients instead of adding to them
_VIEWS = {"all": VIEW_ALL, "front": VIEW_FRONT, "back": VIEW_BACK}
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_DTYPE", 3: "ATTN_ERR_SHAPE", 4: "ATTN_ERR_GQA",
          5: "ATTN_ERR_CU_SEQLENS", 6: "ATTN_ERR_LAYOUT", 7: "ATTN_ERR_UNSUPPORTED", 8: "ATTN_ERR_WORKSPACE",
          9: "ATTN_ERR_HIP", 10: "ATTN_ERR_VERSION", 11: "ATTN_ERR_INVALID", 12: "ATTN_ERR_CONTENT"}


class AttnTensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("reserved", C.c_int32),
                ("n_tok", C.c_int64), ("n_head", C.c_int64), ("head_dim", C.c_int64),
                ("stride_tok", C.c_int64), ("stride_head", C.c_int64)]


class AttnMask(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("causal", C.c_uint32), ("q_view", C.c_uint32),
                ("k_view", C.c_uint32), ("window", C.c_int64), ("q_pos_offset", C.c_int64),
                ("k_pos_offset", C.c_int64), ("kv_interleave", C.c_int32), ("kv_rank", C.c_int32),
                ("block_size", C.c_int32), ("max_blocks", C.c_int32), ("block_table", C.c_void_p),
                ("page_stride", C.c_int64), ("seg_size", C.c_int32), ("reserved", C.c_int32)]


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
P = C.c_void_p
T = C.POINTER(AttnTensor)
M = C.POINTER(AttnMask)
I32, I64, U32, F = C.c_int32, C.c_int64, C.c_uint32, C.c_float
SZ = C.c_size_t

_SIGS = {
    "attn_abi_version": (C.c_int, []),
    "attn_status_string": (C.c_char_p, [C.c_int]),
    "attn_last_error": (C.c_char_p, []),
    "attn_workspace_size": (C.c_int, [C.c_int, T, T, I32, I32, I32, M, C.POINTER(SZ)]),
    "attn_workspace_bytes": (C.c_int, [C.c_int, T, T, I32, I32, I32, M, C.POINTER(SZ)]),
    "attn_block_fwd": (C.c_int, [T, T, T, P, P, I32, I32, I32, M, F, T, P, P, SZ, P]),
    "attn_block_fwd_noalloc": (C.c_int, [T, T, T, P, P, I32, I32, I32, M, F, T, P, P]),
    "attn_merge_out_lse": (C.c_int, [T, P, T, P, P, I32, U32, P, T, I32, P]),
    "attn_merge_n": (C.c_int, [I32, T, C.POINTER(P), T, P, P]),
    "attn_bwd_delta": (C.c_int, [T, T, P, P]),
    "attn_merge_diag": (C.c_int, [T, T, T, F, T, P, T, P]),
    "attn_ulysses_reshard": (C.c_int, [I32, I32, T, T, P]),
    "attn_out_transpose": (C.c_int, [T, P, P]),
    "attn_ulysses_reshard_lse": (C.c_int, [I32, I32, P, P, I64, I64, P]),
    "attn_diag_bwd": (C.c_int, [T, T, T, T, P, P, F, T, T, T, P]),
    "attn_block_bwd": (C.c_int, [T, T, T, T, T, P, P, P, P, I32, I32, I32, M, F, T, T, T, P, SZ, P]),
    "attn_zigzag_shard": (C.c_int, [T, P, I32, I32, I32, I32, T, P]),
    "attn_zigzag_workspace_size": (C.c_int, [I32, T, T, I32, I32, C.POINTER(SZ)]),
    "attn_zigzag_fwd": (C.c_int, [I32, I32, T, T, T, P, I32, I32, F, T, T, P, P, SZ, P]),
    "attn_zigzag_fwd_ranks": (C.c_int, [I32, I32, P, T, T, T, P, I32, I32, F, T, T, C.POINTER(P), P, SZ, P]),
    "attn_zigzag_bwd": (C.c_int, [I32, I32, T, T, T, T, T, P, P, I32, I32, F, T, T, T, P, SZ, P]),
    "attn_zigzag_bwd_ex": (C.c_int, [I32, I32, T, T, T, T, T, P, P, I32, I32, F, T, T, T, P, SZ, P, C.c_uint32]),
    "attn_ring_fwd": (C.c_int, [I32, I32, T, T, T, P, I32, I32, F, T, T, P, P, SZ, P]),
    "attn_ring_bwd": (C.c_int, [I32, I32, T, T, T, T, T, P, P, I32, I32, F, T, T, T, P, SZ, P]),
    "attn_ring_bwd_ex": (C.c_int, [I32, I32, T, T, T, T, T, P, P, I32, I32, F, T, T, T, P, SZ, P, C.c_uint32]),
    "attn_kvp_workspace_size": (C.c_int, [I32, T, T, I32, I32, I32, M, C.POINTER(SZ)]),
    "attn_kvp_fwd": (C.c_int, [I32, T, T, T, C.POINTER(P), P, P, I32, I32, I32, M, F, T, P, P, SZ, P]),
    "attn_validate_inputs": (C.c_int, [T, T, P, P, I32, I32, I32, M, I32, I32, P]),
    "attn_timing_enable": (C.c_int, [I32]),
    "attn_timing_report": (C.c_int, [C.c_char_p, SZ, C.POINTER(SZ)]),
}
EXPORTS = tuple(_SIGS)


def load():
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m blockwise_causal_varlen_amd.build`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != 0:
        raise AttnError(st, load().attn_last_error().decode())
    return st


# ----------------------------------------------------------------------------
# descriptors
# ----------------------------------------------------------------------------
def dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {dt}")


def desc(t: torch.Tensor | None) -> AttnTensor | None:
    """Descriptor of a [n_tok, n_head, head_dim] tensor (last dim contiguous)."""
    if t is None:
        return None
    if t.dim() != 3:
        raise ValueError(f"expected [tokens, heads, head_dim], got {tuple(t.shape)}")
    if t.stride(2) != 1:
        raise ValueError("the last dimension must be contiguous")
    return AttnTensor(t.data_ptr(), dtype_code(t.dtype), 0, t.shape[0], t.shape[1], t.shape[2],
                      t.stride(0), t.stride(1))


def paged_desc(cache: torch.Tensor) -> tuple[AttnTensor, int]:
    """Descriptor of a paged cache [pages, HKV, block_size, D] and its page stride."""
    pages, hkv, bs, d = cache.shape
    if cache.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    t = AttnTensor(cache.data_ptr(), dtype_code(cache.dtype), 0, pages * bs, hkv, d, cache.stride(2), cache.stride(1))
    return t, cache.stride(0)


def mask(causal=False, q_view="all", k_view="all", window=0, q_pos_offset=0, k_pos_offset=0, kv_interleave=0,
         kv_rank=0, block_size=0, max_blocks=0, block_table=None, page_stride=0, seg_size=0) -> AttnMask:
    m = AttnMask()
    m.struct_size = C.sizeof(AttnMask)
    m.causal = int(bool(causal))
    m.q_view = _VIEWS[q_view] if isinstance(q_view, str) else int(q_view)
    m.k_view = _VIEWS[k_view] if isinstance(k_view, str) else int(k_view)
    m.window = int(window)
    m.q_pos_offset = int(q_pos_offset)
    m.k_pos_offset = int(k_pos_offset)
    m.kv_interleave = int(kv_interleave)
    m.kv_rank = int(kv_rank)
    m.block_size = int(block_size)
    m.max_blocks = int(max_blocks)
    m.block_table = None if block_table is None else block_table.data_ptr()
    m.page_stride = int(page_stride)
    m.seg_size = int(seg_size)
    return m


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ref(x):
    return None if x is None else C.byref(x)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _aligned(ws):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


def _cu(cu, device):
    if cu.dtype != torch.int32:
        cu = cu.to(torch.int32)
    return cu.to(device).contiguous()


# ----------------------------------------------------------------------------
# low-level names (C ABI)
# ----------------------------------------------------------------------------
def attn_abi_version() -> int:
    return load().attn_abi_version()


def attn_status_string(s) -> str:
    return load().attn_status_string(int(s)).decode()


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_workspace_size(op, q, k, num_seqs, max_q, max_k, m=None) -> int:
    n = SZ(0)
    _call("attn_workspace_size", op, C.byref(q), C.byref(k), num_seqs, max_q, max_k, _ref(m), C.byref(n))
    return n.value


# ----------------------------------------------------------------------------
# torch-level helpers
# ----------------------------------------------------------------------------
def block_fwd(q, k, v, cu_q, cu_k, max_q, max_k, scale, m: AttnMask | None = None, out=None, lse=None,
              out_dtype=None, stream=None, k_desc=None, v_desc=None):
    """attn_block_fwd on torch tensors -> (out, lse). Rows outside the q view
    keep the contents of `out` / `lse` (new outputs start at 0 / -inf)."""
    dev = q.device
    nq, hq, d = q.shape
    if out is None:
        out = torch.zeros(nq, hq, d, dtype=out_dtype or q.dtype, device=dev)
    if lse is None:
        lse = torch.full((hq, nq), float("-inf"), dtype=torch.float32, device=dev)
    qd, kd, vd = desc(q), k_desc or desc(k), v_desc or desc(v)
    cq, ck = _cu(cu_q, dev), _cu(cu_k, dev)
    ns = cq.numel() - 1
    nbytes = attn_workspace_size(OP_BLOCK_FWD, qd, kd, ns, max_q, max_k, m)
    ws = _workspace(nbytes, dev)
    wp, wn = _aligned(ws)
    _call("attn_block_fwd", C.byref(qd), C.byref(kd), C.byref(vd), cq.data_ptr(), ck.data_ptr(), ns, max_q, max_k,
          _ref(m), scale, C.byref(desc(out)), lse.data_ptr(), wp, wn, _stream(stream))
    return out, lse


def block_fwd_noalloc(q, k, v, cu_q, cu_k, max_q, max_k, scale, m: AttnMask | None, out, lse, stream=None,
                      k_desc=None, v_desc=None):
    """attn_block_fwd_noalloc on torch tensors: the caller provides out and lse
    and device cu_seqlens; the library uses its own device array as workspace."""
    qd, kd, vd = desc(q), k_desc or desc(k), v_desc or desc(v)
    ns = cu_q.numel() - 1
    _call("attn_block_fwd_noalloc", C.byref(qd), C.byref(kd), C.byref(vd), cu_q.data_ptr(), cu_k.data_ptr(), ns, max_q,
          max_k, _ref(m), scale, C.byref(desc(out)), lse.data_ptr(), _stream(stream))
    return out, lse


def merge(out, lse, block_out, block_lse, cu=None, q_view="all", weight=None, final_out=None, init=False,
          stream=None):
    """attn_merge_out_lse in place on (out f32, lse)."""
    cu_p = None
    ns = 0
    if cu is not None:
        cu = _cu(cu, out.device)
        cu_p, ns = cu.data_ptr(), cu.numel() - 1
    fd = desc(final_out)
    _call("attn_merge_out_lse", C.byref(desc(out)), lse.data_ptr(), C.byref(desc(block_out)), block_lse.data_ptr(),
          cu_p, ns, _VIEWS[q_view] if isinstance(q_view, str) else q_view, _ptr(weight), _ref(fd), int(init),
          _stream(stream))
    return out, lse


def merge_n(parts_out, parts_lse, out, lse, stream=None):
    n = len(parts_out)
    arr = (AttnTensor * n)(*[desc(p) for p in parts_out])
    lp = (P * n)(*[p.data_ptr() for p in parts_lse])
    _call("attn_merge_n", n, arr, lp, C.byref(desc(out)), lse.data_ptr(), _stream(stream))
    return out, lse


def bwd_delta(dout, out, delta=None, stream=None):
    n, h, _ = out.shape
    if delta is None:
        delta = torch.empty(h, n, dtype=torch.float32, device=out.device)
    _call("attn_bwd_delta", C.byref(desc(dout)), C.byref(desc(out)), delta.data_ptr(), _stream(stream))
    return delta


def merge_diag(q, k, v, scale, out, lse, final_out=None, stream=None):
    """attn_merge_diag: merge one per-position diagonal block (k, v rows = q rows)
    into the f32 running `out` and `lse` (in place); optionally write `final_out`."""
    _call("attn_merge_diag", C.byref(desc(q)), C.byref(desc(k)), C.byref(desc(v)), float(scale), C.byref(desc(out)),
          lse.data_ptr(), C.byref(desc(final_out)) if final_out is not None else None, _stream(stream))
    return out, lse


def out_transpose(src, dst=None, stream=None):
    """attn_out_transpose: [n, H, D] -> contiguous [H, D, n]."""
    n, h, d = src.shape
    if dst is None:
        dst = torch.empty(h, d, n, dtype=src.dtype, device=src.device)
    _call("attn_out_transpose", C.byref(desc(src)), dst.data_ptr(), _stream(stream))
    return dst


def ulysses_reshard(srcs, dsts, to_heads, stream=None):
    """attn_ulysses_reshard over uly = len(srcs) virtual ranks (writes dsts)."""
    uly = len(srcs)
    sa = (AttnTensor * uly)(*[desc(t) for t in srcs])
    da = (AttnTensor * uly)(*[desc(t) for t in dsts])
    _call("attn_ulysses_reshard", uly, int(bool(to_heads)), sa, da, _stream(stream))
    return dsts


def ulysses_reshard_lse(srcs, dsts, to_heads, n_local, n_head, stream=None):
    """attn_ulysses_reshard_lse: [H, S_l] per sequence shard <-> [H_l, S] per head shard."""
    uly = len(srcs)
    sp = (P * uly)(*[t.data_ptr() for t in srcs])
    dp = (P * uly)(*[t.data_ptr() for t in dsts])
    _call("attn_ulysses_reshard_lse", uly, int(bool(to_heads)), sp, dp, n_local, n_head, _stream(stream))
    return dsts


def diag_bwd(dout, q, k, v, lse, delta, scale, dq, dk, dv, stream=None):
    """attn_diag_bwd: ACCUMULATES the diagonal block's grads into dq, dk, dv (f32)."""
    _call("attn_diag_bwd", C.byref(desc(dout)), C.byref(desc(q)), C.byref(desc(k)), C.byref(desc(v)),
          lse.data_ptr(), delta.data_ptr(), float(scale), C.byref(desc(dq)), C.byref(desc(dk)), C.byref(desc(dv)),
          _stream(stream))
    return dq, dk, dv


def block_bwd(dout, q, k, v, out, lse, cu_q, cu_k, max_q, max_k, scale, m: AttnMask | None = None, delta=None,
              dq=None, dk=None, dv=None, stream=None):
    """attn_block_bwd: ACCUMULATES into dq/dk/dv (f32; zero-initialised when not given)."""
    dev = q.device
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.zeros(k.shape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.zeros(v.shape, dtype=torch.float32, device=dev) if dv is None else dv
    cq, ck = _cu(cu_q, dev), _cu(cu_k, dev)
    ns = cq.numel() - 1
    nbytes = attn_workspace_size(OP_BLOCK_BWD, desc(q), desc(k), ns, max_q, max_k, m)
    ws = _workspace(nbytes, dev)
    wp, wn = _aligned(ws)
    _call("attn_block_bwd", C.byref(desc(dout)), C.byref(desc(q)), C.byref(desc(k)), C.byref(desc(v)),
          _ref(desc(out)), lse.data_ptr(), _ptr(delta), cq.data_ptr(), ck.data_ptr(), ns, max_q, max_k, _ref(m),
          scale, C.byref(desc(dq)), C.byref(desc(dk)), C.byref(desc(dv)), wp, wn, _stream(stream))
    return dq, dk, dv


def zigzag_shard(x, cu_global, cp, rank, max_seqlen, out=None, stream=None):
    """Rank `rank`'s zig-zag local rows of a global packed [S, H, D] tensor."""
    if out is None:
        out = torch.empty((x.shape[0] // cp,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    cu = _cu(cu_global, x.device)
    _call("attn_zigzag_shard", C.byref(desc(x)), cu.data_ptr(), cu.numel() - 1, max_seqlen, cp, rank,
          C.byref(desc(out)), _stream(stream))
    return out


class RingRunner:
    """Holds the descriptors and workspace of one rank's ring/zig-zag schedule
    so that repeated steps (the benchmark's loop) marshal nothing new."""

    def __init__(self, kind, cp, rank, q, k_loc, v_loc, cu_local, max_local, scale, dout=None, out_dtype=None):
        self.kind, self.cp, self.rank, self.scale = kind, cp, rank, scale
        dev = q.device
        self.q, self.k_loc, self.v_loc = q, list(k_loc), list(v_loc)
        self.cu = _cu(cu_local, dev)
        self.ns = self.cu.numel() - 1
        self.max_local = max_local
        nq, hq, d = q.shape
        self.out_acc = torch.empty(nq, hq, d, dtype=torch.float32, device=dev)
        self.out = torch.empty(nq, hq, d, dtype=out_dtype or q.dtype, device=dev)
        self.lse = torch.empty(hq, nq, dtype=torch.float32, device=dev)
        self.qd, self.od, self.oad = desc(q), desc(self.out), desc(self.out_acc)
        self.bwd_od = None  # the merged output the backward reads (default: self.out)
        self.kd = (AttnTensor * cp)(*[desc(t) for t in self.k_loc])
        self.vd = (AttnTensor * cp)(*[desc(t) for t in self.v_loc])
        n = SZ(0)
        _call("attn_zigzag_workspace_size", cp, C.byref(self.qd), C.byref(self.kd[0]), self.ns, max_local, C.byref(n))
        self.ws = _workspace(n.value, dev)
        self.wp, self.wn = _aligned(self.ws)
        self.dout = dout
        if dout is not None:
            self.dq = torch.zeros(nq, hq, d, dtype=torch.float32, device=dev)
            self.dk = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in self.k_loc]
            self.dv = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in self.v_loc]
            self.dod, self.dqd = desc(dout), desc(self.dq)
            self.dkd = (AttnTensor * cp)(*[desc(t) for t in self.dk])
            self.dvd = (AttnTensor * cp)(*[desc(t) for t in self.dv])

    def forward(self, stream=None):
        name = "attn_zigzag_fwd" if self.kind == "zigzag" else "attn_ring_fwd"
        _call(name, self.cp, self.rank, C.byref(self.qd), self.kd, self.vd, self.cu.data_ptr(), self.ns,
              self.max_local, self.scale, C.byref(self.oad), C.byref(self.od), self.lse.data_ptr(), self.wp, self.wn,
              _stream(stream))
        return self.out, self.lse

    def zero_grads(self):
        self.dq.zero_()
        for t in self.dk + self.dv:
            t.zero_()

    def backward(self, stream=None, set_grads=False):
        """Gradients into dq / dk / dv: added to them, or (set_grads) set, with
        no zeroing needed first (ATTN_BWD_SET)."""
        name = "attn_zigzag_bwd_ex" if self.kind == "zigzag" else "attn_ring_bwd_ex"
        _call(name, self.cp, self.rank, C.byref(self.dod), C.byref(self.qd), self.kd, self.vd,
              C.byref(self.bwd_od if self.bwd_od is not None else self.od),
              self.lse.data_ptr(), self.cu.data_ptr(), self.ns, self.max_local, self.scale, C.byref(self.dqd),
              self.dkd, self.dvd, self.wp, self.wn, _stream(stream), BWD_SET if set_grads else 0)
        return self.dq, self.dk, self.dv


class ZigzagRanksForward:
    """attn_zigzag_fwd_ranks over the RingRunners of several ranks of one ring
    (their q, out_acc, out and lse): each step's blocks in one launch."""

    def __init__(self, runners):
        r0 = runners[0]
        self.cp, self.n = r0.cp, len(runners)
        self.ranks = (I32 * self.n)(*[r.rank for r in runners])
        self.qd = (AttnTensor * self.n)(*[r.qd for r in runners])
        self.oad = (AttnTensor * self.n)(*[r.oad for r in runners])
        self.od = (AttnTensor * self.n)(*[r.od for r in runners])
        self.lse = (P * self.n)(*[r.lse.data_ptr() for r in runners])
        self.r0 = r0
        slice_ = (r0.wn + 255) // 256 * 256
        self.ws = _workspace(slice_ * self.n, r0.q.device)
        self.wp, self.wn = _aligned(self.ws)

    def forward(self, stream=None):
        r0 = self.r0
        _call("attn_zigzag_fwd_ranks", self.cp, self.n, self.ranks, self.qd, r0.kd, r0.vd, r0.cu.data_ptr(), r0.ns,
              r0.max_local, r0.scale, self.oad, self.od, self.lse, self.wp, self.wn, _stream(stream))


def kvp_fwd(q_shd, k_caches, v_caches, tables, cu_q, cu_k, max_q, max_k, scale, m: AttnMask, out=None, lse=None,
            stream=None):
    """attn_kvp_fwd: q as [S, H, D] (any strides), R paged caches [pages, HKV, bs, D]."""
    R = len(k_caches)
    dev = q_shd.device
    nq, hq, d = q_shd.shape
    if out is None:
        out = torch.empty(nq, hq, d, dtype=q_shd.dtype, device=dev)
    if lse is None:
        lse = torch.empty(hq, nq, dtype=torch.float32, device=dev)
    kd = [paged_desc(c)[0] for c in k_caches]
    vd = [paged_desc(c)[0] for c in v_caches]
    karr = (AttnTensor * R)(*kd)
    varr = (AttnTensor * R)(*vd)
    tp = (P * R)(*[t.data_ptr() for t in tables])
    cq, ck = _cu(cu_q, dev), _cu(cu_k, dev)
    ns = cq.numel() - 1
    qd = desc(q_shd)
    n = SZ(0)
    _call("attn_kvp_workspace_size", R, C.byref(qd), C.byref(karr[0]), ns, max_q, max_k, C.byref(m), C.byref(n))
    ws = _workspace(n.value, dev)
    wp, wn = _aligned(ws)
    _call("attn_kvp_fwd", R, C.byref(qd), karr, varr, tp, cq.data_ptr(), ck.data_ptr(), ns, max_q, max_k, C.byref(m),
          scale, C.byref(desc(out)), lse.data_ptr(), wp, wn, _stream(stream))
    return out, lse


def validate_inputs(q, k, cu_q, cu_k, max_q, max_k, m=None, zigzag_cp=0, one_query=0, k_desc=None, stream=None):
    cq, ck = _cu(cu_q, q.device), _cu(cu_k, q.device)
    kd = k_desc or desc(k)
    _call("attn_validate_inputs", C.byref(desc(q)), C.byref(kd), cq.data_ptr(), ck.data_ptr(), cq.numel() - 1, max_q,
          max_k, _ref(m), zigzag_cp, one_query, _stream(stream))


def attn_timing_enable(on: bool):
    _call("attn_timing_enable", int(bool(on)))


def attn_timing_report() -> dict:
    """{kernel name: (launches, total ms)} since the last report (waits for the events)."""
    n = SZ(0)
    _call("attn_timing_report", None, 0, C.byref(n))
    buf = C.create_string_buffer(n.value + 1)
    _call("attn_timing_report", buf, n.value + 1, C.byref(n))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out
