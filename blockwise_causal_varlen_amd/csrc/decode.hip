// One-query-per-sequence varlen decode (gfx950).
//
// Each sequence has exactly one query row and a variable number of gathered
// key rows (recipes "qsa_fa_fallback.py", module docstring: cu_seqlens_q =
// arange, cu_seqlens_k prefix sums, GQA; its kernel runs one program per
// (query row, q head) and re-reads the kv head's rows once per q head).
//
// Here one wave serves ALL q heads of one kv head, so every K/V byte is read
// from HBM exactly once. A workgroup = 4 waves = 4 consecutive kv heads of one
// sequence (their key rows are adjacent in memory). Per 32-key chunk a wave:
//   * loads K straight from global memory into the A-operand layout of the
//     16x16x32 bf16 MFMA (lane l: key l % 16 of a 16-key tile; the 4 lane
//     groups l / 16 each own a contiguous quarter of the head dimension);
//   * computes S^T = K Q^T (16 keys x 16 query columns, the group's q heads
//     in columns 0..G-1) with fp32 accumulation;
//   * runs the online softmax per column (the 4 lane groups exchange with
//     xor 16 / xor 32);
//   * stages the V chunk in a wave-private LDS slice and reads V^T operands
//     with the LDS transpose read, then O^T += V^T P^T.
// The next chunk's K and V loads are issued before the current chunk is
// computed, so each wave keeps 16 KB of loads in flight; at <= 256 registers
// two workgroups share a CU (32 KB a SIMD in flight).
#include "internal.h"

namespace attn {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct DecParams {
  const bf16 *q, *k, *v;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  const int32_t *cu_q, *cu_k;
  int32_t hq, hkv, group, num_seqs;
  float scale_log2;
  void *out; int64_t o_st, o_sh;
  float *lse; int64_t lse_n;
  int64_t n_q, n_k;
  // split KV: grid.z splits of split_len keys each; with n_split > 1 each
  // wave writes a partial (out f32 [split][n_q][HQ][D], lse [split][HQ][n_q])
  int32_t n_split, split_len;
  float *part_out, *part_lse;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, typename OutT>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecParams p) {
  constexpr int QD = D / 4;            // head-dim quarter owned by a lane group
  constexpr int NST = QD / 8;          // MFMA k-steps per 16-key tile (4 for D=128)
  constexpr int VP = D + 16;           // LDS pitch of V rows (transpose reads conflict free)
  constexpr int NDT = D / 16;          // 16-row d tiles of O^T
  constexpr int VCH = 32 * D / 8 / 64; // 16-byte V chunks per lane per 32-key chunk
  __shared__ __attribute__((aligned(16))) bf16 sV[4][32 * VP];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, u = lane & 15;
  const int seq = blockIdx.x;
  const int hk = blockIdx.y * 4 + w;
  if (hk >= p.hkv) return;
  int64_t q0 = p.cu_q[seq];
  const int64_t q1 = p.cu_q[seq + 1];
  if (q1 <= q0 || q0 < 0 || q0 >= p.n_q) return;
  int64_t k0 = p.cu_k[seq], k1 = p.cu_k[seq + 1];
  k0 = k0 < 0 ? 0 : (k0 > p.n_k ? p.n_k : k0);
  k1 = k1 < k0 ? k0 : (k1 > p.n_k ? p.n_k : k1);
  // this wave's split of the sequence's keys
  const int64_t ks = k0 + (int64_t)blockIdx.z * p.split_len;
  const int64_t ke = k1 < ks + p.split_len ? k1 : ks + p.split_len;
  const int64_t nk = ke > ks ? ke - ks : 0;
  k0 = ks;

  // Q^T fragments: column u = q head hk*G + u (zero beyond the group).
  const bool col_ok = u < p.group;
  const int hq_col = hk * p.group + u;
  bf16x8 qf[NST];
  {
    const bf16 *qr = p.q + q0 * p.q_st + (int64_t)hq_col * p.q_sh + g * QD;
#pragma unroll
    for (int s = 0; s < NST; ++s)
      qf[s] = col_ok ? __builtin_bit_cast(bf16x8, ld16(qr + s * 8)) : bf16x8{};
  }

  bf16 *myV = sV[w];

  // K and V of this wave's keys through buffer resources based at its first
  // key: per-lane byte offsets are fixed, the chunk's offset is a scalar, and
  // rows past the end read as zero (the host keeps the bytes below 2^31)
  const int kst = (int)p.k_st, vst = (int)p.v_st;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.k + k0 * p.k_st + (int64_t)hk * p.k_sh), (short)0,
                                                     nk > 0 ? (int)(((nk - 1) * p.k_st + D) * 2) : 0, kBufFlags);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.v + k0 * p.v_st + (int64_t)hk * p.v_sh), (short)0,
                                                     nk > 0 ? (int)(((nk - 1) * p.v_st + D) * 2) : 0, kBufFlags);
  int koff[2][NST], voff[VCH];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < NST; ++s) koff[t][s] = ((t * 16 + u) * kst + g * QD + s * 8) * 2;
#pragma unroll
  for (int c = 0; c < VCH; ++c) {
    const int ci = lane + 64 * c;
    voff[c] = ((ci / (D / 8)) * vst + (ci % (D / 8)) * 8) * 2;
  }
  auto load_k = [&](int64_t c0, i32x4 (&kr)[2][NST]) {
    const int so = (int)c0 * kst * 2;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NST; ++s) kr[t][s] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff[t][s], so, 0);
  };
  auto load_v = [&](int64_t c0, i32x4 (&vr)[VCH]) {
    const int so = (int)c0 * vst * 2;
#pragma unroll
    for (int c = 0; c < VCH; ++c) vr[c] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[c], so, 0);
  };

  f32x4 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4{};
  float mrow = neg_inf(), lsum = 0.f;

  i32x4 kcur[2][NST], vcur[VCH];
  if (nk > 0) { load_k(0, kcur); load_v(0, vcur); }
  for (int64_t c0 = 0; c0 < nk; c0 += 32) {
    i32x4 knext[2][NST], vnext[VCH];
    const bool more = c0 + 32 < nk;
    if (more) { load_k(c0 + 32, knext); load_v(c0 + 32, vnext); }

    // stage V chunk (wave-private LDS; LDS ops of one wave execute in order)
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int ci = lane + 64 * c;
      const int kr = ci / (D / 8), col = (ci % (D / 8)) * 8;
      st16(&myV[kr * VP + col], vcur[c]);
    }
    // S^T for keys c0 + [0,16) and c0 + [16,32)
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int s = 0; s < NST; ++s) acc = mfma16(__builtin_bit_cast(bf16x8, kcur[t][s]), qf[s], acc);
      sc[t] = acc;
    }
    // mask keys past the end (lane holds keys t*16 + 4g + r)
    if (c0 + 32 > nk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c0 + t * 16 + 4 * g + r >= nk) sc[t][r] = neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrow, mx * p.scale_log2);
    const float muse = mnew == neg_inf() ? 0.f : mnew;
    const float alpha = fast_exp2(mrow - muse);
    mrow = mnew;
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(__builtin_fmaf(sc[t][r], p.scale_log2, -muse));
        ps += e;
        pf[t * 4 + r] = (bf16)e;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] *= alpha;
    // O^T += V^T P^T: A = V^T rows d = dt*16 + u, slots = keys {4g..4g+3, 16+4g..16+4g+3}
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int col = dt * 16 + 4 * (u & 3);
      const int ra = 4 * g + (u >> 2);
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&myV[ra * VP + col]));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&myV[(ra + 16) * VP + col]));
      bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
      bf16x8 va;
      va[0] = l4[0]; va[1] = l4[1]; va[2] = l4[2]; va[3] = l4[3];
      va[4] = h4[0]; va[5] = h4[1]; va[6] = h4[2]; va[7] = h4[3];
      o[dt] = mfma16(va, pf, o[dt]);
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < NST; ++s) kcur[t][s] = knext[t][s];
#pragma unroll
      for (int c = 0; c < VCH; ++c) vcur[c] = vnext[c];
    }
  }
  float lt = lsum + __shfl_xor(lsum, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (!col_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (mrow + fast_log2(lt)) * kLn2 : neg_inf();
  if (p.n_split > 1) {  // partial of this split (an empty split: out 0, lse -inf)
    float *po = p.part_out + ((int64_t)blockIdx.z * p.n_q + q0) * ((int64_t)p.hq * D) + (int64_t)hq_col * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = dt * 16 + 4 * g;
      float4 v4 = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
      *reinterpret_cast<float4 *>(po + d0) = v4;
    }
    if (g == 0) p.part_lse[((int64_t)blockIdx.z * p.hq + hq_col) * p.n_q + q0] = lse_v;
    return;
  }
  OutT *orow = (OutT *)p.out + q0 * p.o_st + (int64_t)hq_col * p.o_sh;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int d0 = dt * 16 + 4 * g;
    if constexpr (sizeof(OutT) == 4) {
      float4 v4 = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
      *reinterpret_cast<float4 *>(orow + d0) = v4;
    } else {
      bf16x4 v4;
      v4[0] = (bf16)(o[dt][0] * inv); v4[1] = (bf16)(o[dt][1] * inv);
      v4[2] = (bf16)(o[dt][2] * inv); v4[3] = (bf16)(o[dt][3] * inv);
      *reinterpret_cast<bf16x4 *>(orow + d0) = v4;
    }
  }
  if (g == 0) p.lse[(int64_t)hq_col * p.lse_n + q0] = lse_v;
}

// Split-KV merge: per (sequence, q head) the n_split partials of its one row
// combine by online softmax (lse = m + log sum exp(lse_i - m), out = sum
// exp(lse_i - lse) out_i). Rows of no sequence stay untouched. D/4 lanes per
// (sequence, head), 4 elements each.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void decode_split_merge_kernel(DecParams p) {
  constexpr int G = D / 4;
  const int sub = threadIdx.x % G;
  const int64_t total = (int64_t)p.num_seqs * p.hq;
  const int64_t per_blk = 256 / G;
  for (int64_t pr = blockIdx.x * per_blk + threadIdx.x / G; pr < total; pr += (int64_t)gridDim.x * per_blk) {
    const int32_t seq = (int32_t)(pr / p.hq);
    const int32_t h = (int32_t)(pr - (int64_t)seq * p.hq);
    const int64_t q0 = p.cu_q[seq], q1 = p.cu_q[seq + 1];
    if (q1 <= q0 || q0 < 0 || q0 >= p.n_q) continue;
    float m = neg_inf();
    for (int z = 0; z < p.n_split; ++z) m = fmaxf(m, p.part_lse[((int64_t)z * p.hq + h) * p.n_q + q0]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    if (m != neg_inf()) {
      for (int z = 0; z < p.n_split; ++z) {
        const float lz = p.part_lse[((int64_t)z * p.hq + h) * p.n_q + q0];
        const float wz = expf(lz - m);  // 0 for an empty split
        if (wz > 0.f) {
          const f32x4 oz = *reinterpret_cast<const f32x4 *>(
              p.part_out + ((int64_t)z * p.n_q + q0) * ((int64_t)p.hq * D) + (int64_t)h * D + 4 * sub);
          acc += wz * oz;
          l += wz;
        }
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    OutT *orow = (OutT *)p.out + q0 * p.o_st + (int64_t)h * p.o_sh + 4 * sub;
    if constexpr (sizeof(OutT) == 4) {
      *reinterpret_cast<f32x4 *>(orow) = acc * inv;
    } else {
      bf16x4 b;
      b[0] = (bf16)(acc[0] * inv); b[1] = (bf16)(acc[1] * inv); b[2] = (bf16)(acc[2] * inv); b[3] = (bf16)(acc[3] * inv);
      *reinterpret_cast<bf16x4 *>(orow) = b;
    }
    if (sub == 0) p.lse[(int64_t)h * p.lse_n + q0] = l > 0.f ? m + logf(l) : neg_inf();
  }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  DecParams p;
  p.q = (const bf16 *)a.q.data; p.k = (const bf16 *)a.k.data; p.v = (const bf16 *)a.v.data;
  p.q_st = a.q.st; p.q_sh = a.q.sh; p.k_st = a.k.st; p.k_sh = a.k.sh; p.v_st = a.v.st; p.v_sh = a.v.sh;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.hq = a.hq; p.hkv = a.hkv; p.group = a.hq / a.hkv; p.num_seqs = a.num_seqs;
  p.scale_log2 = a.scale * kLog2e;
  p.out = a.out; p.o_st = a.o_st; p.o_sh = a.o_sh;
  p.lse = a.lse; p.lse_n = a.lse_n;
  p.n_q = a.lse_n;
  p.n_k = a.n_k;
  p.n_split = a.n_split > 1 ? a.n_split : 1;
  p.split_len = a.n_split > 1 ? a.split_len : 0x7fffffff;
  p.part_out = a.part_out; p.part_lse = a.part_lse;
  dim3 grid((unsigned)a.num_seqs, (unsigned)((a.hkv + 3) / 4), (unsigned)p.n_split);
  if (a.num_seqs <= 0) return hipSuccess;
  if (a.head_dim == 128) {
    if (a.out_dtype == 0) hipLaunchKernelGGL((decode_kernel<128, bf16>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<128, float>), grid, dim3(256), 0, s, p);
  } else {
    if (a.out_dtype == 0) hipLaunchKernelGGL((decode_kernel<64, bf16>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<64, float>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode_split_merge(const DecodeArgs &a, hipStream_t s) {
  DecParams p{};
  p.cu_q = a.cu_q; p.hq = a.hq; p.num_seqs = a.num_seqs;
  p.out = a.out; p.o_st = a.o_st; p.o_sh = a.o_sh;
  p.lse = a.lse; p.lse_n = a.lse_n; p.n_q = a.lse_n;
  p.n_split = a.n_split; p.part_out = a.part_out; p.part_lse = a.part_lse;
  if (a.num_seqs <= 0) return hipSuccess;
  const int G = a.head_dim / 4;
  int64_t blocks = ((int64_t)a.num_seqs * a.hq + 256 / G - 1) / (256 / G);
  if (blocks > 8192) blocks = 8192;
  if (a.head_dim == 128) {
    if (a.out_dtype == 0) hipLaunchKernelGGL((decode_split_merge_kernel<128, bf16>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_split_merge_kernel<128, float>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  } else {
    if (a.out_dtype == 0) hipLaunchKernelGGL((decode_split_merge_kernel<64, bf16>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_split_merge_kernel<64, float>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace attn
