"""Seeded synthetic inputs for the five workloads (and smaller variants).

This module holds no attention arithmetic: it only draws document lengths,
normal tensors, page tables and sequence lengths from a seeded generator, so
that the library's tests and benchmark and the fp64 oracle see exactly the same
inputs. Recipe (all seeds 0, one torch CPU generator per workload, draws in the
order lengths -> q -> k -> v -> dout -> block tables):

  * tensors: N(0, 1) drawn in float32, then rounded to bfloat16 (round to
    nearest even) where the workload is bf16;
  * scale = 1/sqrt(D) as a float32 value;
  * packed-varlen lengths: a length is drawn, rounded DOWN to a multiple of
    `multiple` (2*cp, so every document splits into 2*cp zig-zag chunks); draws
    stop when the next document would reach or pass the total, and the last
    document takes the remainder (itself a multiple of `multiple`);
  * the decode workload's K/V (~137 GB) are drawn on the GPU with a CUDA
    generator seeded 0, k then v, each in chunks of 2^20 rows of fp32 draws
    rounded to bf16.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


def _gen(seed: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, dtype, gen, device="cpu") -> torch.Tensor:
    """N(0,1) in float32, then cast (RNE for bf16)."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    return x if dtype == torch.float32 else x.to(dtype)


def normal_chunked(shape, gen, device, rows_per_chunk=1 << 20):
    """bf16 N(0,1) drawn on the device in row chunks of fp32 draws (bounded
    temporary memory for the ~137 GB decode K/V)."""
    out = torch.empty(*shape, dtype=torch.bfloat16, device=device)
    for a in range(0, shape[0], rows_per_chunk):
        b = min(shape[0], a + rows_per_chunk)
        out[a:b] = torch.randn((b - a,) + tuple(shape[1:]), generator=gen, dtype=torch.float32,
                               device=device).to(torch.bfloat16)
    return out


def _finish(lengths, total):
    """Last document absorbs the remainder."""
    out, acc = [], 0
    for L in lengths:
        if acc + L >= total:
            break
        out.append(L)
        acc += L
    out.append(total - acc)
    return out


def lengths_uniform_even(total, lo, hi, multiple, gen):
    """Even L ~ U{lo..hi}, rounded down to a multiple of `multiple`."""
    lens, acc = [], 0
    while acc < total:
        L = 2 * int(torch.randint(lo // 2, hi // 2 + 1, (1,), generator=gen))
        L -= L % multiple
        lens.append(L)
        acc += L
    return _finish(lens, total)


def lengths_loguniform(total, lo, hi, multiple, gen):
    """L = round(exp(U[ln lo, ln hi])), rounded down to a multiple of `multiple`."""
    lens, acc = [], 0
    while acc < total:
        u = float(torch.rand(1, generator=gen, dtype=torch.float64))
        L = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        L -= L % multiple
        lens.append(L)
        acc += L
    return _finish(lens, total)


def cu_from_lengths(lens):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


@dataclass
class ZigzagCase:
    """A packed varlen causal problem to be run as cp zig-zag virtual ranks."""
    name: str
    cu: torch.Tensor            # global cu_seqlens, int32 [ndoc+1]
    q: torch.Tensor             # [S, HQ, D] global, or [S/cp, HQ, D] for `q_rank` only
    k: torch.Tensor             # [S, HKV, D] global
    v: torch.Tensor
    dout: torch.Tensor | None   # same shape as q
    cp: int
    scale: float
    q_rank: int | None = None   # q/dout hold only this rank's local rows
    meta: dict = field(default_factory=dict)


def zigzag_case(name, lens, hq, hkv, d, dtype, cp, seed=0, with_dout=True, q_rank=None, gen=None):
    g = gen if gen is not None else _gen(seed)
    cu = cu_from_lengths(lens)
    S = int(cu[-1])
    nq = S // cp if q_rank is not None else S
    q = normal((nq, hq, d), dtype, g)
    k = normal((S, hkv, d), dtype, g)
    v = normal((S, hkv, d), dtype, g)
    dout = normal((nq, hq, d), dtype, g) if with_dout else None
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    return ZigzagCase(name, cu, q, k, v, dout, cp, scale, q_rank)


def cfg1():
    """Tiny zig-zag: one document S=256, H=2, D=64, fp32, cp=2."""
    return zigzag_case("tiny-zigzag S=256 H=2 D=64 fp32 cp=2", [256], 2, 2, 64, torch.float32, 2)


def cfg2(with_dout=False):
    """Packed varlen forward: 8192 tokens, even L~U[128,2048] (multiple of 8), H=16, D=128, bf16, cp=4."""
    g = _gen(0)
    lens = lengths_uniform_even(8192, 128, 2048, 8, g)
    return zigzag_case("packed-varlen 8192 tok H=16 D=128 bf16 cp=4", lens, 16, 16, 128,
                       torch.bfloat16, 4, gen=g, with_dout=with_dout)


def cfg3(rank=3):
    """One zig-zag rank of 131072 tokens, cp=8, HQ=32, HKV=8, D=128, bf16,
    log-uniform L in [1024, 32768] (multiple of 16). q and dout are drawn for
    the chosen rank's 16384 local rows only; K/V for all 131072 tokens."""
    g = _gen(0)
    lens = lengths_loguniform(131072, 1024, 32768, 16, g)
    return zigzag_case(f"zigzag-rank{rank} 131072 tok cp=8 HQ=32 HKV=8 D=128 bf16", lens, 32, 8, 128,
                       torch.bfloat16, 8, gen=g, q_rank=rank)


def small_zigzag(total, lo, hi, hq, hkv, d, dtype, cp, seed=0, loguniform=False):
    """Reduced packed-varlen case with the same recipe (for parity tests)."""
    g = _gen(seed)
    mult = 2 * cp
    if loguniform:
        lens = lengths_loguniform(total, lo, hi, mult, g)
    else:
        lens = lengths_uniform_even(total, lo, hi, mult, g)
    return zigzag_case(f"small zigzag {total} tok", lens, hq, hkv, d, dtype, cp, gen=g)


@dataclass
class EagleCase:
    """EAGLE-3 mixed attention: a zig-zag sequence problem (cache block 0) plus
    n_ttt test-time-training blocks that hold one key/value per q row."""
    base: ZigzagCase
    ttt_k: list                 # n_ttt x [rows of q, HKV, D] (global rows, or q_rank's local rows)
    ttt_v: list


def eagle_case(base: ZigzagCase, n_ttt: int, seed=0):
    """TTT blocks for `base`, drawn from their own seeded stream (k then v per block)."""
    g = _gen(seed + 1000)
    rows, hkv, d = base.q.shape[0], base.k.shape[1], base.k.shape[2]
    ks, vs = [], []
    for _ in range(n_ttt):
        ks.append(normal((rows, hkv, d), base.k.dtype, g))
        vs.append(normal((rows, hkv, d), base.k.dtype, g))
    return EagleCase(base, ks, vs)


@dataclass
class KvpCase:
    """KV-parallel segmented prefill over R round-robin paged shards."""
    q: torch.Tensor              # [HQ, S, D] (NKI layout)
    k_caches: list               # R x [num_blocks, HKV, block_size, D]
    v_caches: list
    tables: list                 # R x int32 [1, num_blocks]
    block_size: int
    seg_size: int
    global_q_offset: int
    window: int
    scale: float
    R: int


def cfg4(window=0, s_q=2048, hq=8, hkv=1, d=128, num_blocks=2048, block_size=16, R=4,
         seg_size=2048, global_q_offset=98304, seed=0, dtype=torch.bfloat16):
    """KV-parallel prefill: q [8, 2048, 128] bf16, 4 round-robin shards of 2048
    paged blocks of 16 tokens (random block tables), seg_size=2048,
    global_q_offset=98304, sliding window 0 or 4096 (other sizes and dtypes for
    the parity tests)."""
    g = _gen(seed)
    q = normal((hq, s_q, d), dtype, g)
    kc = [normal((num_blocks, hkv, block_size, d), dtype, g) for _ in range(R)]
    vc = [normal((num_blocks, hkv, block_size, d), dtype, g) for _ in range(R)]
    tabs = [torch.randperm(num_blocks, generator=g).to(torch.int32).reshape(1, -1) for _ in range(R)]
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    return KvpCase(q, kc, vc, tabs, block_size, seg_size, global_q_offset, window, scale, R)


@dataclass
class DecodeCase:
    q: torch.Tensor          # [nseq, HQ, D]
    k: torch.Tensor          # [sum k_len, HKV, D]
    v: torch.Tensor
    cu_k: torch.Tensor       # int32 [nseq+1]
    k_lens: torch.Tensor     # int64 [nseq]
    scale: float


def decode_lengths(nseq=65536, max_len=2048, seed=0):
    g = _gen(seed)
    return torch.randint(1, max_len + 1, (nseq,), generator=g), g


def cfg5(device="cpu", nseq=65536, max_len=2048, hq=32, hkv=4, d=128, seed=0):
    """One-query decode: 65536 sequences, k_len ~ U{1..2048}, HQ=32, HKV=4,
    D=128, bf16. Lengths and q come from the CPU generator; K/V are drawn on
    `device` (a CUDA generator when it is a GPU)."""
    lens, g = decode_lengths(nseq, max_len, seed)
    cu = torch.zeros(nseq + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    q = normal((nseq, hq, d), torch.bfloat16, g)
    total = int(cu[-1])
    if str(device).startswith("cuda"):
        gd = torch.Generator(device=device)
        gd.manual_seed(seed)
        k = normal_chunked((total, hkv, d), gd, device)
        v = normal_chunked((total, hkv, d), gd, device)
    else:
        k = normal((total, hkv, d), torch.bfloat16, g)
        v = normal((total, hkv, d), torch.bfloat16, g)
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    return DecodeCase(q.to(device), k, v, cu.to(torch.int32), lens, scale)


def long_decode(lens, hq=32, hkv=4, d=128, seed=0, device="cpu"):
    """One-query decode with given (long) key lengths: the split-KV regime where
    the (sequence, kv head) pairs alone cannot fill the chip."""
    g = _gen(seed)
    lens = torch.tensor(lens, dtype=torch.int64)
    nseq = lens.numel()
    cu = torch.zeros(nseq + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    q = normal((nseq, hq, d), torch.bfloat16, g)
    total = int(cu[-1])
    if str(device).startswith("cuda"):
        gd = torch.Generator(device=device)
        gd.manual_seed(seed)
        k = normal_chunked((total, hkv, d), gd, device)
        v = normal_chunked((total, hkv, d), gd, device)
    else:
        k = normal((total, hkv, d), torch.bfloat16, g)
        v = normal((total, hkv, d), torch.bfloat16, g)
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    return DecodeCase(q.to(device), k, v, cu.to(torch.int32), lens, scale)
