// Block backward with the merged (out, lse) (gfx950).
//
// NeMo AutoModel zigzag_ring_attention, `zigzag_ring_flash_attn_varlen_backward`:
// every block's backward receives the FINAL merged out and lse, so with
//     P  = exp(scale q.k - lse),   dP = dout . v,   dS = P (dP - delta),
//     delta = <dout, out>  (merged out, computed once by attn_bwd_delta)
// the block's share of the joint-softmax gradient is
//     dq += scale dS k,   dk += scale dS^T q,   dv += P^T dout.
//
// Two kernels, no floating-point atomics (deterministic):
//   * dK/dV: a workgroup owns 128 keys of one kv head (wave w: keys 32w..),
//     keeps K and V of its keys in registers and loops over the q heads of the
//     kv group and the 64-row query tiles that can see its keys. Scores are
//     computed as S = Q K^T with the 32x32 MFMA, so a lane owns one key
//     (column) and 16 query rows; P and dS are then already the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS, whose A operands are read from the
//     query / dout tiles in LDS with the transpose read.
//   * dQ: a workgroup owns 128 query rows of one q head (like the forward),
//     keeps Q and dO in registers, stages K/V tiles, computes S^T = K Q^T and
//     dP^T = V dO^T, and accumulates dQ^T += K^T dS^T (K^T by transpose read).
#include <type_traits>

#include "internal.h"


namespace attn {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS pitch (elements) of tiles read both row-wise (16-byte reads of 16 rows)
// and with the 4-row transpose read: bf16 D + 40 keeps the row reads conflict
// free and the transpose reads at most 2-way; f32 tiles use an odd pitch.
template <typename T, int D> struct Pitch;
template <int D> struct Pitch<bf16, D> { static constexpr int both = D + 40, rows = D + 8; };
template <int D> struct Pitch<float, D> { static constexpr int both = D + 1, rows = D + 1; };

struct BwdParams {
  const void *q, *k, *v, *dout;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, do_st, do_sh;
  int32_t hq, group;
  float scale, scale_log2;
  MaskDev m;
  const float *lse, *delta;
  const float *lse2;  // lse * log2(e), +inf where lse = -inf (rows that see nothing)
  int64_t n_q;
  float *dq; int64_t dq_st, dq_sh;
  float *dk; int64_t dk_st, dk_sh;
  float *dv; int64_t dv_st, dv_sh;
  const WorkItem *items; const int32_t *order; const int32_t *count;
  int32_t set_q, set_kv;  // store dq / dk, dv instead of adding to them
  // half-precision copies of q and dout ([n_q, HQ, D] contiguous) for the
  // dK/dV kernel, and their flag (nonzero: a value did not fit f16); NULL: none
  const void *q16, *do16;
  const int32_t *h16_flag;
};

// Row-operand fragment of a 32x32 MFMA from a tile in LDS: lane row `r`, k-step s.
template <typename T>
__device__ __forceinline__ typename Mfma32<T>::Frag lds_row_frag(const T *base, int pitch, int r, int s, int g) {
  constexpr int KV = Mfma32<T>::KV;
  if constexpr (sizeof(T) == 2) return *reinterpret_cast<const bf16x8 *>(base + r * pitch + s * 2 * KV + g * KV);
  else return base[r * pitch + s * 2 + g];
}

// Row-operand fragment straight from global memory (zero when !ok).
template <typename T>
__device__ __forceinline__ typename Mfma32<T>::Frag glob_row_frag(const T *row, int s, int g, bool ok) {
  constexpr int KV = Mfma32<T>::KV;
  if constexpr (sizeof(T) == 2) {
    i32x4 v = ok ? ld16(row + s * 2 * KV + g * KV) : i32x4{0, 0, 0, 0};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return ok ? row[s * 2 + g] : 0.f;
  }
}

// acc += X^T(d rows dt*32.., k = 32 tile rows starting at r0) * B, where B is
// held in C layout (register j <-> tile row c_row(j)) in `pv` (16 values).
template <typename T>
__device__ __forceinline__ f32x16 acc_transposed(f32x16 acc, const T *base, int pitch, int r0, int dt,
                                                 const float (&pv)[16], int lane) {
  const int g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int u = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = (bf16)pv[t * 8 + e];
      const int ra = r0 + t * 16 + 4 * g + (u >> 2);
      const int col = dt * 32 + dh * 16 + 4 * (u & 3);
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + ra * pitch + col));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + (ra + 8) * pitch + col));
      bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
      bf16x8 a;
      a[0] = l4[0]; a[1] = l4[1]; a[2] = l4[2]; a[3] = l4[3];
      a[4] = h4[0]; a[5] = h4[1]; a[6] = h4[2]; a[7] = h4[3];
      acc = Mfma32<bf16>::mma(a, b, acc);
    }
  } else {
    const int l32 = lane & 31;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc = Mfma32<float>::mma(base[(r0 + c_row(j, lane)) * pitch + dt * 32 + l32], pv[j], acc);
  }
  return acc;
}

// bf16 form over all ND d-tiles: acc[dt] += X^T(d rows dt*32.., k = 32 tile
// rows from r0) * B, B in C layout in `pv`. Per 16-row half t the ND
// MFMAs go back to back on independent accumulators.
template <int ND>
__device__ __forceinline__ void acc_transposed_all(f32x16 (&acc)[ND], const bf16 *base, int pitch, int r0,
                                                   const float (&pv)[16], int lane) {
  const int g = lane >> 5, u = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)pv[t * 8 + e];
    bf16x8 a[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int ra = r0 + t * 16 + 4 * g + (u >> 2);
      const int col = dt * 32 + dh * 16 + 4 * (u & 3);
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + ra * pitch + col));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + (ra + 8) * pitch + col));
      bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
      a[dt][0] = l4[0]; a[dt][1] = l4[1]; a[dt][2] = l4[2]; a[dt][3] = l4[3];
      a[dt][4] = h4[0]; a[dt][5] = h4[1]; a[dt][6] = h4[2]; a[dt][7] = h4[3];
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] = Mfma32<bf16>::mma(a[dt], b, acc[dt]);
  }
}

// The ND transposed A fragments (d rows dt*32.., k = the 16 tile rows from
// blk) of a SwzTile128 (offsets from swz_tr_offsets).
template <int ND>
__device__ __forceinline__ void swz_tr_frags(bf16x8 (&a)[ND], const bf16 *blk, const int (&lo)[ND],
                                             const int (&hi)[ND]) {
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    i16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(blk + lo[dt]));
    i16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(blk + hi[dt]));
    bf16x4 l4 = __builtin_bit_cast(bf16x4, l), h4 = __builtin_bit_cast(bf16x4, h);
    a[dt][0] = l4[0]; a[dt][1] = l4[1]; a[dt][2] = l4[2]; a[dt][3] = l4[3];
    a[dt][4] = h4[0]; a[dt][5] = h4[1]; a[dt][6] = h4[2]; a[dt][7] = h4[3];
  }
}

// acc_transposed_all on a SwzTile128 (offsets from swz_tr_offsets; r0 a
// multiple of 16).
template <int ND>
__device__ __forceinline__ void acc_transposed_swz(f32x16 (&acc)[ND], const bf16 *base, int r0, const int (&lo)[ND],
                                                   const int (&hi)[ND], const float (&pv)[16]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)pv[t * 8 + e];
    bf16x8 a[ND];
    swz_tr_frags<ND>(a, base + (r0 + t * 16) * 128, lo, hi);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] = Mfma32<bf16>::mma(a[dt], b, acc[dt]);
  }
}

// Stage rows [r0, r0 + nrows) (< lim valid) of a [tok, head, D] tensor into LDS.
template <typename T, int D, int NROWS>
__device__ __forceinline__ void stage_rows(T *dst, int pitch, const T *src, int64_t st, int64_t sh, int head,
                                           int64_t r0, int64_t lim, int tid) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int NCH = NROWS * D / CH / 256;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ci = tid + 256 * c;
    const int r = ci / (D / CH);
    const int col = (ci % (D / CH)) * CH;
    const int64_t row = r0 + r;
    i32x4 v = row < lim ? ld16(src + row * st + (int64_t)head * sh + col) : i32x4{0, 0, 0, 0};
    if constexpr (sizeof(T) == 2) {
      st16(dst + r * pitch + col, v);
    } else {
      float4 f = __builtin_bit_cast(float4, v);
      dst[r * pitch + col] = f.x; dst[r * pitch + col + 1] = f.y;
      dst[r * pitch + col + 2] = f.z; dst[r * pitch + col + 3] = f.w;
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdParams p) {
  using M = Mfma32<T>;
  constexpr int NS = D / (2 * M::KV);
  constexpr int ND = D / 32;
  constexpr int QB = kBwdBQ;  // query rows per staged tile
  constexpr int PB = Pitch<T, D>::both;
  __shared__ __attribute__((aligned(16))) T sQ[QB * PB];
  __shared__ __attribute__((aligned(16))) T sO[QB * PB];
  __shared__ float sL[QB], sDl[QB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int hkv_count = p.hq / p.group;
  const int rank = blockIdx.x / hkv_count;
  const int hk = blockIdx.x - rank * hkv_count;
  if (rank >= *p.count) return;
  const WorkItem it = p.items[p.order[rank]];
  const MaskDev &m = p.m;

  const int64_t kr0 = it.k0 + 32 * w;          // first key of this wave
  const int64_t key = kr0 + l32;
  const bool key_ok = key < it.k1;
  const bool wave_on = kr0 < it.k1;
  const int64_t kp_lane = m.pm.kpos(key - it.kdoc0);
  const int64_t wk_lo = m.pm.kpos(kr0 - it.kdoc0);
  const int64_t wk_hi = m.pm.kpos((kr0 + 31 < it.k1 ? kr0 + 31 : it.k1 - 1) - it.kdoc0);

  typename M::Frag kf[NS], vf[NS];
  {
    const T *krow = (const T *)p.k + key * p.k_st + (int64_t)hk * p.k_sh;
    const T *vrow = (const T *)p.v + key * p.v_st + (int64_t)hk * p.v_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = glob_row_frag<T>(krow, s, g, key_ok);
      vf[s] = glob_row_frag<T>(vrow, s, g, key_ok);
    }
  }
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    for (int64_t qt = it.q0; qt < it.q1; qt += QB) {
      __syncthreads();
      stage_rows<T, D, QB>(sQ, PB, (const T *)p.q, p.q_st, p.q_sh, h, qt, it.q1, tid);
      stage_rows<T, D, QB>(sO, PB, (const T *)p.dout, p.do_st, p.do_sh, h, qt, it.q1, tid);
      if (tid < QB) {
        const int64_t row = qt + tid;
        const bool ok = row < it.q1;
        const float l = ok ? p.lse[(int64_t)h * p.n_q + row] : neg_inf();
        // rows without a finite lse (none visible, or padding) contribute nothing
        sL[tid] = (l == neg_inf()) ? __builtin_inff() : l * kLog2e;
        sDl[tid] = ok ? p.delta[(int64_t)h * p.n_q + row] : 0.f;
      }
      __syncthreads();
      if (!wave_on) continue;
#pragma unroll
      for (int sub = 0; sub < QB / 32; ++sub) {
        const int64_t qs0 = qt + sub * 32;
        if (qs0 >= it.q1) break;
        const int64_t qlast = (qs0 + 31 < it.q1 ? qs0 + 31 : it.q1 - 1);
        const int64_t qp_lo = m.q_pos_offset + (qs0 - it.qdoc0);
        const int64_t qp_hi = m.q_pos_offset + (qlast - it.qdoc0);
        if (m.causal && wk_lo > qp_hi) continue;
        if (m.window > 0 && wk_hi <= qp_lo - m.window) continue;
        const bool full = (!m.causal || wk_hi <= qp_lo) && (m.window <= 0 || wk_lo > qp_hi - m.window);
        // S = Q K^T and dP = dO V^T: lane column = its key, rows = 16 query rows
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = M::mma(lds_row_frag<T>(sQ, PB, sub * 32 + l32, st, g), kf[st], s);
          dp = M::mma(lds_row_frag<T>(sO, PB, sub * 32 + l32, st, g), vf[st], dp);
        }
        float pv[16], ds[16];
        const int64_t qp0 = m.q_pos_offset + (qt - it.qdoc0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int qi = sub * 32 + c_row(j, lane);
          const bool vis = full | visible(qp0 + qi, kp_lane, m.causal, m.window);
          const float e = fast_exp2(__builtin_fmaf(s[j], p.scale_log2, -sL[qi]));
          pv[j] = vis ? e : 0.f;
          ds[j] = pv[j] * (dp[j] - sDl[qi]);
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          dv[dt] = acc_transposed<T>(dv[dt], sO, PB, sub * 32, dt, pv, lane);
          dk[dt] = acc_transposed<T>(dk[dt], sQ, PB, sub * 32, dt, ds, lane);
        }
      }
    }
  }
  if (!key_ok) return;
  // dK^T / dV^T in C layout: lane column = its key, rows d = dt*32 + c_row(j)
  float *dkr = p.dk + key * p.dk_st + (int64_t)hk * p.dk_sh;
  float *dvr = p.dv + key * p.dv_st + (int64_t)hk * p.dv_sh;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (!p.set_kv) {
        a = *reinterpret_cast<float4 *>(dkr + d0);
        b = *reinterpret_cast<float4 *>(dvr + d0);
      }
      a.x += p.scale * dk[dt][4 * j4]; a.y += p.scale * dk[dt][4 * j4 + 1];
      a.z += p.scale * dk[dt][4 * j4 + 2]; a.w += p.scale * dk[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dkr + d0) = a;
      b.x += dv[dt][4 * j4]; b.y += dv[dt][4 * j4 + 1]; b.z += dv[dt][4 * j4 + 2]; b.w += dv[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dvr + d0) = b;
    }
}

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdParams p) {
  using M = Mfma32<T>;
  constexpr int NS = D / (2 * M::KV);
  constexpr int ND = D / 32;
  constexpr int KB = kFwdBN;  // keys per staged tile
  constexpr int PK = Pitch<T, D>::both;
  constexpr int PV = Pitch<T, D>::rows;
  __shared__ __attribute__((aligned(16))) T sK[KB * PK];
  __shared__ __attribute__((aligned(16))) T sV[KB * PV];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int rank = blockIdx.x / p.hq;
  const int h = blockIdx.x - rank * p.hq;
  if (rank >= *p.count) return;
  const WorkItem it = p.items[p.order[rank]];
  const int hk = h / p.group;
  const MaskDev &m = p.m;

  const int64_t r0 = it.q0 + 32 * w;
  const int64_t row = r0 + l32;
  const bool row_ok = row < it.q1;
  const bool wave_on = r0 < it.q1;
  const int64_t qpos = m.q_pos_offset + (row - it.qdoc0);
  const int64_t wq_lo = m.q_pos_offset + (r0 - it.qdoc0);
  const int64_t wq_hi = m.q_pos_offset + ((r0 + 31 < it.q1 ? r0 + 31 : it.q1 - 1) - it.qdoc0);

  typename M::Frag qf[NS], of[NS];
  {
    const T *qrow = (const T *)p.q + row * p.q_st + (int64_t)h * p.q_sh;
    const T *orow = (const T *)p.dout + row * p.do_st + (int64_t)h * p.do_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = glob_row_frag<T>(qrow, s, g, row_ok);
      of[s] = glob_row_frag<T>(orow, s, g, row_ok);
    }
  }
  float lrow = row_ok ? p.lse[(int64_t)h * p.n_q + row] : neg_inf();
  lrow = lrow == neg_inf() ? __builtin_inff() : lrow * kLog2e;
  const float drow = row_ok ? p.delta[(int64_t)h * p.n_q + row] : 0.f;

  f32x16 dq[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dq[i] = f32x16{};

  for (int64_t kt = it.k0; kt < it.k1; kt += KB) {
    __syncthreads();
    stage_rows<T, D, KB>(sK, PK, (const T *)p.k, p.k_st, p.k_sh, hk, kt, it.k1, tid);
    stage_rows<T, D, KB>(sV, PV, (const T *)p.v, p.v_st, p.v_sh, hk, kt, it.k1, tid);
    __syncthreads();
    if (!wave_on) continue;
    const int64_t klast = (kt + KB <= it.k1 ? kt + KB : it.k1) - 1;
    const int64_t kp_lo = m.pm.kpos(kt - it.kdoc0);
    const int64_t kp_hi = m.pm.kpos(klast - it.kdoc0);
    if (m.causal && kp_lo > wq_hi) continue;
    if (m.window > 0 && kp_hi <= wq_lo - m.window) continue;
    const bool full = (kt + KB <= it.k1) && (!m.causal || kp_hi <= wq_lo) &&
                      (m.window <= 0 || kp_lo > wq_hi - m.window);
#pragma unroll
    for (int sb = 0; sb < KB / 32; ++sb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = M::mma(lds_row_frag<T>(sK, PK, sb * 32 + l32, st, g), qf[st], s);
        dp = M::mma(lds_row_frag<T>(sV, PV, sb * 32 + l32, st, g), of[st], dp);
      }
      float ds[16];
      const int32_t t0 = (int32_t)(kt - it.kdoc0);
      const int32_t nvalid = (int32_t)(it.k1 - kt);
#pragma unroll
      for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(__builtin_fmaf(s[j], p.scale_log2, -lrow)) * (dp[j] - drow);
      if (!full) {  // wave-uniform
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int32_t kk = sb * 32 + c_row(j, lane);
          const bool vis = (kk < nvalid) & visible(qpos, m.pm.kpos32(t0 + kk), m.causal, m.window);
          ds[j] = vis ? ds[j] : 0.f;
        }
      }
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) dq[dt] = acc_transposed<T>(dq[dt], sK, PK, sb * 32, dt, ds, lane);
    }
  }
  if (!row_ok) return;
  float *dqr = p.dq + row * p.dq_st + (int64_t)h * p.dq_sh;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      float4 a = {0.f, 0.f, 0.f, 0.f};
      if (!p.set_q) a = *reinterpret_cast<float4 *>(dqr + d0);
      a.x += p.scale * dq[dt][4 * j4]; a.y += p.scale * dq[dt][4 * j4 + 1];
      a.z += p.scale * dq[dt][4 * j4 + 2]; a.w += p.scale * dq[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dqr + d0) = a;
    }
}

// ---------------------------------------------------------------------------
// bf16 kernels with asynchronous double-buffered staging (global->LDS copies
// through buffer resources; rows past the end of a tile read as zeros, which
// contribute nothing: zero q/dout rows give dS = 0 and P^T dout = 0).
// ---------------------------------------------------------------------------
__global__ void lse2_kernel(const float *lse, float *lse2, int64_t n, int32_t *h16_flag) {
  if (h16_flag && blockIdx.x == 0 && threadIdx.x == 0) *h16_flag = 0;  // before half_copy_kernel sets it
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float l = lse[i];
    lse2[i] = l == neg_inf() ? __builtin_inff() : l * kLog2e;
  }
}

// Half-precision copies of q and dout for the dK/dV kernel: every bf16 value
// converts to f16 exactly when |x| <= 65504 (f16 keeps 11 significant bits to
// bf16's 8; below 2^-14 the copy is subnormal, off by at most 2^-25). A value
// beyond that range sets *flag, and the dK/dV kernel then keeps bf16.
// Grid-stride over 8-element pieces; q and dout have the same [n, H, D] shape.
__global__ __launch_bounds__(256) void half_copy_kernel(const bf16 *q, int64_t q_st, int64_t q_sh, const bf16 *dout,
                                                        int64_t do_st, int64_t do_sh, f16 *q16, f16 *do16, int64_t n,
                                                        int32_t h, int32_t d, int32_t *flag) {
  const int32_t per_row = h * (d / 8);
  const int64_t total = n * per_row;
  bool bad = false;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row;
    const int32_t r = (int32_t)(i - row * per_row), hh = r / (d / 8), c = (r - hh * (d / 8)) * 8;
    const int64_t o16 = (row * h + hh) * d + c;
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(q + row * q_st + hh * q_sh + c));
    const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(dout + row * do_st + hh * do_sh + c));
    f16x8 qa, ob;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (float)a[e], y = (float)b[e];
      bad |= !(fabsf(x) <= 65504.f) | !(fabsf(y) <= 65504.f);
      qa[e] = (f16)x;
      ob[e] = (f16)y;
    }
    st16(q16 + o16, __builtin_bit_cast(i32x4, qa));
    st16(do16 + o16, __builtin_bit_cast(i32x4, ob));
  }
  if (bad) *flag = 1;
}

// MASK = false: launches without a causal or window mask (every visible tile is
// full), whose softmax step then carries no select.
// E: the element type of the MFMA operands. f16 (q, dout from their f16
// copies, k and v converted in registers; P and dS rounded to f16) unless a
// value does not fit f16, then bf16 (the inputs as given; P and dS rounded to
// bf16). Returns false, having written nothing, when E = f16 and this
// workgroup's k or v does not fit f16, or one of its dS values did not.
template <int D, bool MASK, typename E>
__device__ __forceinline__ bool dkdv_run(const BwdParams &p, E *sQ0, E *sO0, E *sQ1, E *sO1, float *sL0, float *sD0,
                                         float *sL1, float *sD1) {
  using M = Mfma32<E>;
  using Frag = typename M::Frag;
  typedef E E4 __attribute__((ext_vector_type(4)));
  constexpr bool kHalf = sizeof(E) == 2 && !std::is_same<E, bf16>::value;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int QB = kBwdBQ;
  static_assert(QB == 64, "tiles are 64 rows");
  // row reads and transpose reads: swizzled (D = 128) or padded (at most 2-way)
  using QT = std::conditional_t<D == 128, SwzTile128, PadTile<D, D / 8 + 5>>;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < 4);  // 4 waves: lets the copy loops drop their range tests
  const int hkv_count = p.hq / p.group;
  // logical index = (kv head, item): the items of one kv head are neighbours
  const int lb = xcd_block();
  const int cap = gridDim.x / hkv_count;
  const int rank = lb % cap;
  const int hk = lb / cap;
  const WorkItem it = p.items[p.order[rank]];
  // every position and index fits in 32 bits (checked on the host)
  const int32_t q0 = it.q0, q1 = it.q1, qd0 = it.qdoc0, k1 = it.k1, kd0 = it.kdoc0;
  const int32_t causal = MASK ? p.m.causal : 0;  // compile-time 0 without a mask
  const int32_t W = MASK ? (int32_t)p.m.window : 0;
  const int32_t qoff = (int32_t)p.m.q_pos_offset;
  const int32_t koff = (int32_t)p.m.pm.k_pos_offset;
  const int32_t RR = p.m.pm.interleave, rr = p.m.pm.rank, SH = p.m.pm.shift;
  auto kpos_rr = [&](int32_t t) -> int32_t {  // round robin: block t >> SH sits at block R (t >> SH) + r
    return koff + ((((t >> SH) * RR) + rr) << SH) + (t & ((1 << SH) - 1));
  };
  auto kpos = [&](int32_t t) -> int32_t {  // key position of doc-local key t
    return RR == 0 ? koff + t : kpos_rr(t);
  };

  const int32_t kr0 = it.k0 + 32 * w;
  const int32_t key = kr0 + l32;
  const bool key_ok = key < k1;
  const bool wave_on = kr0 < k1;
  const int32_t kp_lane = kpos(key - kd0);
  const int32_t wk_lo = kpos(kr0 - kd0);
  const int32_t wk_hi = kpos((kr0 + 31 < k1 ? kr0 + 31 : k1 - 1) - kd0);

  Frag kf[NS], vf[NS];
  {
    const bf16 *krow = (const bf16 *)p.k + (int64_t)key * p.k_st + (int64_t)hk * p.k_sh;
    const bf16 *vrow = (const bf16 *)p.v + (int64_t)key * p.v_st + (int64_t)hk * p.v_sh;
    bool bad = false;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 kb = glob_row_frag<bf16>(krow, s, g, key_ok);
      const bf16x8 vb = glob_row_frag<bf16>(vrow, s, g, key_ok);
      if constexpr (kHalf) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)kb[e], y = (float)vb[e];
          bad |= !(fabsf(x) <= 65504.f) | !(fabsf(y) <= 65504.f);
          kf[s][e] = (f16)x;
          vf[s][e] = (f16)y;
        }
      } else {
        kf[s] = kb;
        vf[s] = vb;
      }
    }
    // every wave of the workgroup takes the same path
    if constexpr (kHalf)
      if (__syncthreads_or(bad)) return false;
  }
  // (f16 operands) the largest |dS| rounded to f16: dS = P (dP - delta) can
  // leave the f16 range although every input fits it; the workgroup then runs
  // again on bf16 operands
  float ds_max = 0.f;
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  // the q / dout rows: the f16 copies ([n_q, HQ, D] contiguous) or the inputs
  const int64_t q_st = kHalf ? (int64_t)p.hq * D : p.q_st, q_sh = kHalf ? (int64_t)D : p.q_sh;
  const int64_t do_st = kHalf ? (int64_t)p.hq * D : p.do_st, do_sh = kHalf ? (int64_t)D : p.do_sh;
  int qoffs[QT::NJ], ooffs[QT::NJ];
  tile_voffsets<QT>(qoffs, q_st, w, lane);
  tile_voffsets<QT>(ooffs, do_st, w, lane);
  int ro[NS], trl[ND], trh[ND];  // swizzled tiles: per-lane read offsets
  if constexpr (QT::kSwz) {
    swz_row_offsets<NS>(ro, lane);
    swz_tr_offsets<ND>(trl, trh, lane);
  }
  const int32_t qst = (int32_t)q_st, ost = (int32_t)do_st;
  const int32_t nqt = (q1 - q0 + QB - 1) / QB;
  const int32_t total = p.group * nqt;
  const int32_t h0 = hk * p.group;
  const bf16 *qb = (const bf16 *)(kHalf ? p.q16 : p.q);
  const bf16 *ob = (const bf16 *)(kHalf ? p.do16 : p.dout);

  // (q head, tile start) of the next tile to stage and of the next to compute
  int32_t sh = h0, sqt = q0, ch = h0, cqt = q0;
  auto advance = [&](int32_t &h, int32_t &qt) {
    qt += QB;
    if (qt >= q1) { qt = q0; ++h; }
  };

  auto stage = [&](E *sq, E *so, float *sl, float *sd) {
    const int32_t nvalid = q1 - sqt < QB ? q1 - sqt : QB;
    dma_tile_buf<QT>((bf16 *)sq, qb + (int64_t)sqt * q_st + (int64_t)sh * q_sh, ((nvalid - 1) * qst + D) * 2, qoffs,
                     w);
    dma_tile_buf<QT>((bf16 *)so, ob + (int64_t)sqt * do_st + (int64_t)sh * do_sh, ((nvalid - 1) * ost + D) * 2,
                     ooffs, w);
    if (w < 2) {
      const float *src = (w == 0 ? p.lse2 : p.delta) + (int64_t)sh * p.n_q + sqt;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nvalid * 4, kBufFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(w == 0 ? sl : sd), 4, lane * 4, 0, 0, 0);
    }
    advance(sh, sqt);
  };

  // A operand: rows sub*32 + l32 of a Q / dO tile, k-step st (d columns)
  auto afrag = [&](const E *t, int sub, int st) -> Frag {
    const int off = QT::kSwz ? sub * 32 * 128 + ro[st] : (sub * 32 + l32) * QT::PITCH + st * 16 + g * 8;
    return *reinterpret_cast<const Frag *>(t + off);
  };
  // transposed A operand: d rows dt*32.. of a tile, k = its rows r0 + 16 tt +
  // c_row order (the lane's rows 4g + u/4 and 8 more)
  const int u = lane & 15, dh = (lane >> 4) & 1;
  auto trfrag = [&](const E *t, int r0, int tt, int dt) -> Frag {
    const E *lo_p, *hi_p;
    if constexpr (QT::kSwz) {
      const E *blk = t + (r0 + tt * 16) * 128;
      lo_p = blk + trl[dt];
      hi_p = blk + trh[dt];
    } else {
      const int ra = r0 + tt * 16 + 4 * g + (u >> 2);
      const int col = dt * 32 + dh * 16 + 4 * (u & 3);
      lo_p = t + ra * QT::PITCH + col;
      hi_p = t + (ra + 8) * QT::PITCH + col;
    }
    const E4 l4 = __builtin_bit_cast(E4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)lo_p));
    const E4 h4 = __builtin_bit_cast(E4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)hi_p));
    Frag r;
    r[0] = l4[0]; r[1] = l4[1]; r[2] = l4[2]; r[3] = l4[3];
    r[4] = h4[0]; r[5] = h4[1]; r[6] = h4[2]; r[7] = h4[3];
    return r;
  };

  // One 64-row query tile against the wave's 32 keys as one straight-line
  // block of steps, each two MFMAs plus the reads and VALU work placed beside
  // them (the order is pinned by scheduling fences):
  //   score steps k = 0..2NS-1: S = Q K^T and dP = dO V^T of row half k / NS,
  //     d-chunk k % NS; the A fragments are read PFA steps ahead; during the
  //     second half's steps the first half's probabilities are formed;
  //   gradient steps k = 0..4ND-1: dV^T += dO^T P and dK^T += Q^T dS of row
  //     half k / 2ND, 16-row part (k / ND) % 2, d-tile k % ND, transpose reads
  //     PFT steps ahead; during the first half's steps the second half's
  //     probabilities are formed.
  // The mask is branch free (a branch between a masked and an unmasked copy
  // measured slower: the copies' register assignments differ and the joins
  // cost moves): the lane's key is visible from row offset c iff
  // mlo <= c < mlo + mspan (full tiles: every c). Rows past the end of the
  // range hold zeros in Q and dO (and in lse2 / delta), so they add nothing.
  auto body = [&](const E *sq, const E *so, const float *sl, const float *sd, int32_t mlo, uint32_t mspan) {
    constexpr int KS = 2 * NS;      // score steps
    constexpr int KG = 4 * ND;      // gradient steps
    constexpr int PFA = 3, PFT = 3;  // read-ahead distances (steps)
    constexpr int JS = 16 / NS;     // probabilities formed per step (both phases)
    static_assert(16 % NS == 0 && 16 / (2 * ND) == JS, "two probability slots per step");
    const float sl2 = p.scale_log2;
    f32x16 sc[2] = {f32x16{}, f32x16{}}, dpv[2] = {f32x16{}, f32x16{}};
    Frag pb[2][2], db[2][2];  // [half][16-row part]: P and dS as B operands
    f32x4 l4[2], d4[2];         // row terms of the current 4-row group, by half
    // one probability (row c_row(j) of half sub): exp2(S scale log2e - lse2),
    // masked; dS = P (dP - delta)
    auto prob = [&](int sub, int j) {
      if ((j & 3) == 0) {
        const int q4 = sub * 32 + 8 * (j >> 2) + 4 * g;
        l4[sub] = *reinterpret_cast<const f32x4 *>(sl + q4);
        d4[sub] = *reinterpret_cast<const f32x4 *>(sd + q4);
      }
      const int e = j & 3;
      const int c = sub * 32 + 8 * (j >> 2) + e;  // row offset from the lane's first row
      float ex = fast_exp2(__builtin_fmaf(sc[sub][j], sl2, -l4[sub][e]));
      if constexpr (MASK) ex = (uint32_t)(c - mlo) < mspan ? ex : 0.f;
      pb[sub][j >> 3][j & 7] = (E)ex;
      const float dsv = ex * (dpv[sub][j] - d4[sub][e]);
      db[sub][j >> 3][j & 7] = (E)dsv;
      if constexpr (kHalf) ds_max = fmaxf(ds_max, fabsf(dsv));
    };
    Frag fq[KS], fo[KS];  // A fragments by score step (each live for PFA steps)
    auto load_a = [&](int k) {
      fq[k] = afrag(sq, k / NS, k % NS);
      fo[k] = afrag(so, k / NS, k % NS);
    };
    Frag tq[KG], to[KG];  // transposed A fragments by gradient step
    auto load_t = [&](int k) {
      const int sub = k / (2 * ND), tt = (k / ND) % 2, dt = k % ND;
      to[k] = trfrag(so, sub * 32, tt, dt);
      tq[k] = trfrag(sq, sub * 32, tt, dt);
    };
#pragma unroll
    for (int k = 0; k < PFA; ++k) load_a(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (k + PFA < KS) load_a(k + PFA);
      else load_t(k + PFA - KS);  // the first gradient steps' operands
      const int sub = k / NS, st = k % NS;
      sc[sub] = M::mma(fq[k], kf[st], sc[sub]);
      dpv[sub] = M::mma(fo[k], vf[st], dpv[sub]);
      if (sub == 1) {
#pragma unroll
        for (int i = 0; i < JS; ++i) prob(0, st * JS + i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      if (k + PFT < KG) load_t(k + PFT);
      const int sub = k / (2 * ND), tt = (k / ND) % 2, dt = k % ND;
      if (sub == 0) {
#pragma unroll
        for (int i = 0; i < JS; ++i) prob(1, k * JS + i);
      }
      dv[dt] = M::mma(to[k], pb[sub][tt], dv[dt]);
      dk[dt] = M::mma(tq[k], db[sub][tt], dk[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto compute = [&](const E *sq, const E *so, const float *sl, const float *sd) {
    const int32_t qt = cqt;
    advance(ch, cqt);
    if (!wave_on) return;
    const int32_t qlast = (qt + QB <= q1 ? qt + QB : q1) - 1;
    const int32_t qp_lo = qoff + (qt - qd0), qp_hi = qoff + (qlast - qd0);
    if (causal && wk_lo > qp_hi) return;
    if (W > 0 && wk_hi <= qp_lo - W) return;
    const bool full = (!causal || wk_hi <= qp_lo) && (W <= 0 || wk_lo > qp_hi - W);
    // visible row offsets c (from the lane's first row qp_lo + 4g):
    // causal: kp <= qp_lo + 4g + c; window: kp > qp_lo + 4g + c - W
    const int32_t dk0 = kp_lane - (qp_lo + 4 * g);
    const int32_t lo = (full || !causal) ? -(1 << 30) : dk0;
    const int32_t hi = (full || W <= 0) ? (1 << 30) : dk0 + W;
    body(sq, so, sl, sd, lo, (uint32_t)hi - (uint32_t)lo);
  };

  if (total > 0) stage(sQ0, sO0, sL0, sD0);
  __syncthreads();
  for (int32_t i = 0; i < total; i += 2) {
    if (i + 1 < total) stage(sQ1, sO1, sL1, sD1);
    compute(sQ0, sO0, sL0, sD0);
    __syncthreads();
    if (i + 1 >= total) break;
    if (i + 2 < total) stage(sQ0, sO0, sL0, sD0);
    compute(sQ1, sO1, sL1, sD1);
    __syncthreads();
  }
  if constexpr (kHalf)
    if (__syncthreads_or(!(ds_max <= 65504.f))) return false;  // nothing written yet
  if (!key_ok) return true;
  float *dkr = p.dk + (int64_t)key * p.dk_st + (int64_t)hk * p.dk_sh;
  float *dvr = p.dv + (int64_t)key * p.dv_st + (int64_t)hk * p.dv_sh;
  // every load of the key's rows before any store (interleaved, the loads
  // would wait for memory one by one)
  float4 pk[ND][4], pv[ND][4];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      pk[dt][j4] = p.set_kv ? float4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const float4 *>(dkr + d0);
      pv[dt][j4] = p.set_kv ? float4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const float4 *>(dvr + d0);
    }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      float4 a = pk[dt][j4], b = pv[dt][j4];
      a.x += p.scale * dk[dt][4 * j4]; a.y += p.scale * dk[dt][4 * j4 + 1];
      a.z += p.scale * dk[dt][4 * j4 + 2]; a.w += p.scale * dk[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dkr + d0) = a;
      b.x += dv[dt][4 * j4]; b.y += dv[dt][4 * j4 + 1]; b.z += dv[dt][4 * j4 + 2]; b.w += dv[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dvr + d0) = b;
    }
  return true;
}

template <int D, bool MASK>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dkdv_bf16_kernel(BwdParams p) {
  using QT = std::conditional_t<D == 128, SwzTile128, PadTile<D, D / 8 + 5>>;
  constexpr int QB = kBwdBQ;
  __shared__ __attribute__((aligned(1024))) bf16 sQ0[QT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sO0[QT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sQ1[QT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sO1[QT::ELEMS];
  __shared__ __attribute__((aligned(16))) float sL0[QB];
  __shared__ __attribute__((aligned(16))) float sD0[QB];
  __shared__ __attribute__((aligned(16))) float sL1[QB];
  __shared__ __attribute__((aligned(16))) float sD1[QB];
  const int hkv_count = p.hq / p.group;
  const int cap = gridDim.x / hkv_count;
  if (xcd_block() % cap >= *p.count) return;
  if (p.q16 && *p.h16_flag == 0 &&
      dkdv_run<D, MASK, f16>(p, (f16 *)sQ0, (f16 *)sO0, (f16 *)sQ1, (f16 *)sO1, sL0, sD0, sL1, sD1))
    return;
  dkdv_run<D, MASK, bf16>(p, sQ0, sO0, sQ1, sO1, sL0, sD0, sL1, sD1);
}

// MASK = false: launches without a causal or window mask; only the keys past
// the end of a ragged last tile are masked.
template <int D, bool MASK>
__global__ __launch_bounds__(256, 2) void dq_bf16_kernel(BwdParams p) {
  using M = Mfma32<bf16>;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int KB = kFwdBN;
  static_assert(KB == 64, "tiles are 64 rows");
  // row reads and transpose reads: swizzled (D = 128) or padded (at most 2-way)
  using KT = std::conditional_t<D == 128, SwzTile128, PadTile<D, D / 8 + 5>>;
  using VT = PadTile<D, D / 8 + 1>;  // row reads
  __shared__ __attribute__((aligned(1024))) bf16 sK0[KT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[VT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[KT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[VT::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < 4);  // 4 waves: lets the copy loops drop their range tests
  // logical index = (kv head, item, head in group), as in the forward
  const int lb = xcd_block();
  const int cap = gridDim.x / p.hq;
  const int hg = lb % p.group, li = lb / p.group;
  const int rank = li % cap;
  const int hk = li / cap;
  const int h = hk * p.group + hg;
  if (rank >= *p.count) return;
  const WorkItem it = p.items[p.order[rank]];
  // every position and index fits in 32 bits (checked on the host)
  const int32_t q1 = it.q1, k1 = it.k1, kd0 = it.kdoc0;
  const int32_t causal = MASK ? p.m.causal : 0;  // compile-time 0 without a mask
  const int32_t W = MASK ? (int32_t)p.m.window : 0;
  const int32_t qoff = (int32_t)p.m.q_pos_offset;
  const int32_t koff = (int32_t)p.m.pm.k_pos_offset;
  const int32_t RR = p.m.pm.interleave, rr = p.m.pm.rank, SH = p.m.pm.shift;
  auto kpos_rr = [&](int32_t t) -> int32_t {  // round robin: block t >> SH sits at block R (t >> SH) + r
    return koff + ((((t >> SH) * RR) + rr) << SH) + (t & ((1 << SH) - 1));
  };
  auto kpos = [&](int32_t t) -> int32_t {  // key position of doc-local key t
    return RR == 0 ? koff + t : kpos_rr(t);
  };

  const int32_t r0 = it.q0 + 32 * w;
  const int32_t row = r0 + l32;
  const bool row_ok = row < q1;
  const bool wave_on = r0 < q1;
  const int32_t qpos = qoff + (row - it.qdoc0);
  const int32_t wq_lo = qoff + (r0 - it.qdoc0);
  const int32_t wq_hi = qoff + ((r0 + 31 < q1 ? r0 + 31 : q1 - 1) - it.qdoc0);

  bf16x8 qf[NS], of[NS];
  {
    const bf16 *qrow = (const bf16 *)p.q + (int64_t)row * p.q_st + (int64_t)h * p.q_sh;
    const bf16 *orow = (const bf16 *)p.dout + (int64_t)row * p.do_st + (int64_t)h * p.do_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = glob_row_frag<bf16>(qrow, s, g, row_ok);
      of[s] = glob_row_frag<bf16>(orow, s, g, row_ok);
    }
  }
  const float lrow = row_ok ? p.lse2[(int64_t)h * p.n_q + row] : __builtin_inff();
  const float drow = row_ok ? p.delta[(int64_t)h * p.n_q + row] : 0.f;
  const float sl2 = p.scale_log2;
  f32x16 dq[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dq[i] = f32x16{};

  const int32_t kst = (int32_t)p.k_st, vst = (int32_t)p.v_st;
  int koffs[KT::NJ], voffs[VT::NJ];
  tile_voffsets<KT>(koffs, kst, w, lane);
  tile_voffsets<VT>(voffs, vst, w, lane);
  int ro[NS], trl[ND], trh[ND];  // swizzled K tile: per-lane read offsets
  if constexpr (KT::kSwz) {
    swz_row_offsets<NS>(ro, lane);
    swz_tr_offsets<ND>(trl, trh, lane);
  }
  // tile base pointers, advanced by one tile per stage
  const bf16 *kp = (const bf16 *)p.k + (int64_t)it.k0 * p.k_st + (int64_t)hk * p.k_sh;
  const bf16 *vp = (const bf16 *)p.v + (int64_t)it.k0 * p.v_st + (int64_t)hk * p.v_sh;
  auto stage = [&](bf16 *sk, bf16 *sv, int32_t kt) {
    const int32_t nvalid = k1 - kt < KB ? k1 - kt : KB;
    dma_tile_buf<KT>(sk, kp, ((nvalid - 1) * kst + D) * 2, koffs, w);
    dma_tile_buf<VT>(sv, vp, ((nvalid - 1) * vst + D) * 2, voffs, w);
    kp += KB * (int64_t)kst;
    vp += KB * (int64_t)vst;
  };
  // One 64-key tile against the wave's 32 query rows. Keys past the end of the
  // range hold zeros in K and V; the unmasked path only runs on whole tiles.
  auto compute = [&](const bf16 *sk, const bf16 *sv, int32_t kt) {
    if (!wave_on) return;
    const int32_t nvalid = k1 - kt;
    const int32_t kp_lo = kpos(kt - kd0);
    const int32_t kp_hi = kpos((nvalid < KB ? k1 : kt + KB) - 1 - kd0);
    if (causal && kp_lo > wq_hi) return;
    if (W > 0 && kp_hi <= wq_lo - W) return;
    const bool full = (nvalid >= KB) && (!causal || kp_hi <= wq_lo) && (W <= 0 || kp_lo > wq_hi - W);
    // One 32-key half at a time: its S and dP, dS, and its dQ MFMAs, so that
    // only one half's S and dP are live; the registers this frees hold the K
    // and V fragments kRA k-steps ahead of their MFMAs (the compiler would
    // otherwise read each one just before its MFMA). attn_dq 432-434 -> 419-420
    // us a launch on the zig-zag cp=8 rank-3 step (two alternating runs on one
    // box); the halves alone gave about a third of that.
    constexpr int kRA = 3;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 s1 = f32x16{}, dp1 = f32x16{};
      bf16x8 kfr[NS], vfr[NS];
      auto rd = [&](int st) {
        const int koff_ = KT::kSwz ? sb * 32 * 128 + ro[st] : (sb * 32 + l32) * KT::PITCH + st * 16 + g * 8;
        kfr[st] = *reinterpret_cast<const bf16x8 *>(sk + koff_);
        vfr[st] = *reinterpret_cast<const bf16x8 *>(sv + (sb * 32 + l32) * VT::PITCH + st * 16 + g * 8);
      };
#pragma unroll
      for (int st = 0; st < kRA; ++st) rd(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (st + kRA < NS) rd(st + kRA);
        s1 = M::mma(kfr[st], qf[st], s1);
        dp1 = M::mma(vfr[st], of[st], dp1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the K^T fragments of the half's first 16 keys, read before dS is
      // formed so that their latency hides under it: 417-419 -> 414-415 us
      bf16x8 ta[ND];
      if constexpr (KT::kSwz) {
        swz_tr_frags<ND>(ta, sk + sb * 32 * 128, trl, trh);
        __builtin_amdgcn_sched_barrier(0);
      }
      float ds1[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ds1[j] = fast_exp2(__builtin_fmaf(s1[j], sl2, -lrow)) * (dp1[j] - drow);
      if (!full) {  // wave-uniform
        // element j holds key kt + 4g + c, c = 32 sb + 8 (j / 4) + j % 4
        const int32_t lim = nvalid - 4 * g;
        const int32_t t0 = kt - kd0 + 4 * g;
        if constexpr (!MASK) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            ds1[j] = c < lim ? ds1[j] : 0.f;
          }
        } else if (RR == 0) {
          const int32_t d = qpos - (koff + t0), dw = d - W;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            const bool vis = (c < lim) & ((causal == 0) | (c <= d)) & ((W <= 0) | (c > dw));
            ds1[j] = vis ? ds1[j] : 0.f;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            const int32_t kpj = kpos_rr(t0 + c);
            const bool vis = (c < lim) & ((causal == 0) | (kpj <= qpos)) & ((W <= 0) | (kpj > qpos - W));
            ds1[j] = vis ? ds1[j] : 0.f;
          }
        }
      }
      if constexpr (KT::kSwz) {
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (bf16)ds1[e];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dq[dt] = M::mma(ta[dt], b, dq[dt]);
        bf16x8 tb[ND];
        swz_tr_frags<ND>(tb, sk + (sb * 32 + 16) * 128, trl, trh);
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (bf16)ds1[8 + e];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dq[dt] = M::mma(tb[dt], b, dq[dt]);
      } else {
        acc_transposed_all<ND>(dq, sk, KT::PITCH, sb * 32, ds1, lane);
      }
    }
  };

  if (it.k0 < k1) stage(sK0, sV0, it.k0);
  __syncthreads();
  for (int32_t kt = it.k0; kt < k1; kt += 2 * KB) {
    if (kt + KB < k1) stage(sK1, sV1, kt + KB);
    compute(sK0, sV0, kt);
    __syncthreads();
    if (kt + KB >= k1) break;
    if (kt + 2 * KB < k1) stage(sK0, sV0, kt + 2 * KB);
    compute(sK1, sV1, kt + KB);
    __syncthreads();
  }
  if (!row_ok) return;
  float *dqr = p.dq + (int64_t)row * p.dq_st + (int64_t)h * p.dq_sh;
  // every load of the row before any store: the compiler keeps a load after
  // an earlier store of the same row, so interleaved they would wait for
  // memory one by one
  float4 prev[ND][4];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
      prev[dt][j4] = p.set_q ? float4{0.f, 0.f, 0.f, 0.f}
                             : *reinterpret_cast<const float4 *>(dqr + dt * 32 + 8 * j4 + 4 * g);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float4 a = prev[dt][j4];
      a.x += p.scale * dq[dt][4 * j4]; a.y += p.scale * dq[dt][4 * j4 + 1];
      a.z += p.scale * dq[dt][4 * j4 + 2]; a.w += p.scale * dq[dt][4 * j4 + 3];
      *reinterpret_cast<float4 *>(dqr + dt * 32 + 8 * j4 + 4 * g) = a;
    }
}

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdParams &base, const BwdArgs &a, int which, hipStream_t s) {
  BwdParams pp = base;
  constexpr bool kBf16 = sizeof(T) == 2;
  if (which == 0) {
    pp.items = a.ksched.items; pp.order = a.ksched.order; pp.count = a.ksched.count;
    const int64_t gk = a.k_items * a.hkv;
    if (gk > 0) {
      if constexpr (kBf16) {
        if (pp.m.causal || pp.m.window > 0)
          hipLaunchKernelGGL((dkdv_bf16_kernel<D, true>), dim3((unsigned)gk), dim3(256), 0, s, pp);
        else
          hipLaunchKernelGGL((dkdv_bf16_kernel<D, false>), dim3((unsigned)gk), dim3(256), 0, s, pp);
      }
      else hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3((unsigned)gk), dim3(256), 0, s, pp);
    }
  } else {
    pp.items = a.qsched.items; pp.order = a.qsched.order; pp.count = a.qsched.count;
    const int64_t gq = a.q_items * a.hq;
    if (gq > 0) {
      if constexpr (kBf16) {
        if (pp.m.causal || pp.m.window > 0)
          hipLaunchKernelGGL((dq_bf16_kernel<D, true>), dim3((unsigned)gq), dim3(256), 0, s, pp);
        else
          hipLaunchKernelGGL((dq_bf16_kernel<D, false>), dim3((unsigned)gq), dim3(256), 0, s, pp);
      }
      else hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)gq), dim3(256), 0, s, pp);
    }
  }
  return hipGetLastError();
}

// which = 0: the dK/dV kernel, 1: the dQ kernel.
hipError_t launch_bwd(const BwdArgs &a, int which, hipStream_t s) {
  BwdParams p;
  p.q = a.q.data; p.k = a.k.data; p.v = a.v.data; p.dout = a.dout.data;
  p.q_st = a.q.st; p.q_sh = a.q.sh; p.k_st = a.k.st; p.k_sh = a.k.sh;
  p.v_st = a.v.st; p.v_sh = a.v.sh; p.do_st = a.dout.st; p.do_sh = a.dout.sh;
  p.hq = a.hq; p.group = a.hq / a.hkv;
  p.scale = a.scale; p.scale_log2 = a.scale * kLog2e;
  p.m = a.mask;
  p.lse = a.lse; p.delta = a.delta; p.lse2 = a.lse2; p.n_q = a.n_q;
  p.dq = a.dq; p.dq_st = a.dq_st; p.dq_sh = a.dq_sh;
  p.dk = a.dk; p.dk_st = a.dk_st; p.dk_sh = a.dk_sh;
  p.dv = a.dv; p.dv_st = a.dv_st; p.dv_sh = a.dv_sh;
  p.set_q = a.set_q ? 1 : 0;
  p.set_kv = a.set_kv ? 1 : 0;
  p.q16 = a.q16; p.do16 = a.do16; p.h16_flag = a.h16_flag;
  if (a.dtype == 0) {
    if (a.head_dim == 128) return launch_bwd_t<bf16, 128>(p, a, which, s);
    return launch_bwd_t<bf16, 64>(p, a, which, s);
  }
  if (a.head_dim == 128) return launch_bwd_t<float, 128>(p, a, which, s);
  return launch_bwd_t<float, 64>(p, a, which, s);
}

hipError_t launch_lse2(const float *lse, float *lse2, int64_t n, hipStream_t s, int32_t *h16_flag) {
  if (n <= 0) return hipSuccess;
  int64_t b = (n + 255) / 256;
  if (b > 8192) b = 8192;
  hipLaunchKernelGGL(lse2_kernel, dim3((unsigned)b), dim3(256), 0, s, lse, lse2, n, h16_flag);
  return hipGetLastError();
}

hipError_t launch_half_copy(const HalfCopyArgs &a, hipStream_t s) {
  const int64_t pieces = a.n * a.h * (a.d / 8);
  if (pieces <= 0) return hipSuccess;
  int64_t b = (pieces + 255) / 256;
  if (b > 256 * 16) b = 256 * 16;
  hipLaunchKernelGGL(half_copy_kernel, dim3((unsigned)b), dim3(256), 0, s, (const bf16 *)a.q, a.q_st, a.q_sh,
                     (const bf16 *)a.dout, a.do_st, a.do_sh, (f16 *)a.q16, (f16 *)a.do16, a.n, a.h, a.d, a.flag);
  return hipGetLastError();
}

}  // namespace attn
