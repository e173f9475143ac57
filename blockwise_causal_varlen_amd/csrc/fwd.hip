// Tile scheduler and block-forward kernel (gfx950).
//
// Block forward of one attention block over packed varlen documents, as the
// flash varlen forward the pages call per ring step (NeMo AutoModel
// zigzag_ring_attention, `_block_forward`; ring_attention, `_fa_forward`):
// returns the block's normalised output and its log-sum-exp of scaled scores.
// Masks: causal and sliding window on explicit positions, per-document
// front/back half views and a round-robin key position map (AWS NKI
// "Attention KV-Parallel Segmented CTE": kvp_group_size, sliding_window,
// seg_size). Paged keys (its block_tables) are gathered into contiguous rows
// before the forward runs.
//
// Kernel shape. A workgroup = 4 waves = 128 query rows of one q head; wave w
// owns rows [32w, 32w+32). Scores are computed transposed, S^T = K Q^T, with
// the 32x32 MFMA so that a lane owns one query row (lane % 32) and 16 keys of
// every 32-key sub-tile: the row max needs one exchange with lane ^ 32, the
// exponentiated scores are already in the register layout of the B operand of
// O^T += V^T P^T, and the output rescale is a per-lane scalar. K and V tiles
// (32 keys in the bf16 kernel, 64 in the f32 one) are staged through LDS; V^T
// operands are read with the gfx950 LDS transpose read (ds_read_b64_tr_b16), K
// with 16-byte reads on a padded pitch.
#include "internal.h"

namespace attn {

// ---------------------------------------------------------------------------
// Scheduler: one workgroup builds the work list (one item per (q tile,
// segment)), then orders it by decreasing cost (counting sort on the number of
// visible key tiles) so that long tiles start first.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kCostBins = 2048;

size_t sched_bytes(int64_t capacity) {
  size_t b = (size_t)capacity * sizeof(WorkItem);
  b = (b + 255) & ~(size_t)255;
  b += ((size_t)capacity * sizeof(int32_t) + 255) & ~(size_t)255;
  b += 256;
  return b;
}

SchedBufs sched_carve(void *ws, int64_t capacity) {
  char *p = (char *)ws;
  SchedBufs sb;
  sb.items = (WorkItem *)p;
  p += ((size_t)capacity * sizeof(WorkItem) + 255) & ~(size_t)255;
  sb.order = (int32_t *)p;
  p += ((size_t)capacity * sizeof(int32_t) + 255) & ~(size_t)255;
  sb.count = (int32_t *)p;
  sb.capacity = (int32_t)capacity;
  return sb;
}

int64_t sched_capacity(int64_t n_rows, int32_t num_seqs, int32_t tile, int64_t n_seg) {
  return (n_rows / tile + num_seqs + 1) * (n_seg > 0 ? n_seg : 1);
}

using SchedParams = SchedJob;

__device__ __forceinline__ void view_range(int64_t s, int64_t e, int view, int64_t &a, int64_t &b) {
  int64_t h = (e - s) / 2;
  a = s; b = e;
  if (view == 1) b = s + h;
  else if (view == 2) a = s + h;
}

__device__ __forceinline__ int64_t clampi(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Block-wide inclusive scan of one int per thread (kSchedThreads threads).
__device__ __forceinline__ int32_t block_scan(int32_t v, int32_t *buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int32_t x = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += x;
    __syncthreads();
  }
  const int32_t r = buf[tid];
  __syncthreads();
  return r;
}

__device__ void make_item(const SchedParams &p, int64_t qs, int64_t qe, int64_t ks, int64_t ke, int64_t t,
                          int64_t sg, WorkItem &it) {
  const MaskDev &m = p.m;
  int64_t qa, qb, ka, kb;
  view_range(qs, qe, m.q_view, qa, qb);
  view_range(ks, ke, m.k_view, ka, kb);
  const int64_t nk_doc = ke - ks;
  it.qdoc0 = (int32_t)qs;
  it.qmid = (int32_t)(qs + (qe - qs) / 2);
  it.kdoc0 = (int32_t)ks;
  it.seg = (int32_t)sg;
  if (p.by_keys) {
    // a tile of keys and the query rows that can see any of them
    const int64_t k0 = ka + t * p.tile;
    const int64_t k1 = k0 + p.tile < kb ? k0 + p.tile : kb;
    int64_t lo = qa, hi = qb;
    if (m.causal) {  // qpos >= kpos(first key)
      const int64_t c = qs + (m.pm.kpos(k0 - ks) - m.q_pos_offset);
      if (c > lo) lo = c;
    }
    if (m.window > 0) {  // qpos < kpos(last key) + window
      const int64_t c = qs + (m.pm.kpos(k1 - 1 - ks) + m.window - m.q_pos_offset);
      if (c < hi) hi = c;
    }
    if (hi < lo) hi = lo;
    it.q0 = (int32_t)lo; it.q1 = (int32_t)hi;
    it.k0 = (int32_t)k0; it.k1 = (int32_t)k1;
    it.cost = (int32_t)((hi - lo + p.key_tile - 1) / p.key_tile + 1);
    return;
  }
  const int64_t q0 = qa + t * p.tile;
  const int64_t q1 = q0 + p.tile < qb ? q0 + p.tile : qb;
  // keys any row of the tile can see
  int64_t lo = ka, hi = kb;
  if (m.causal) {
    const int64_t c = ks + m.pm.count_le(m.q_pos_offset + (q1 - 1 - qs), nk_doc);
    if (c < hi) hi = c;
  }
  if (m.window > 0) {
    const int64_t c = ks + m.pm.count_le(m.q_pos_offset + (q0 - qs) - m.window, nk_doc);
    if (c > lo) lo = c;
  }
  if (p.nsplit > 1 && hi > lo) {
    // part sg of the visible keys, in whole key tiles
    int64_t chunk = (hi - lo + p.nsplit - 1) / p.nsplit;
    chunk = (chunk + p.key_tile - 1) / p.key_tile * p.key_tile;
    const int64_t a = lo + sg * chunk;
    const int64_t b = a + chunk < hi ? a + chunk : hi;
    lo = a < hi ? a : hi;
    hi = b;
  }
  if (hi < lo) hi = lo;
  it.q0 = (int32_t)q0; it.q1 = (int32_t)q1;
  it.k0 = (int32_t)lo; it.k1 = (int32_t)hi;
  it.cost = (int32_t)((hi - lo + p.key_tile - 1) / p.key_tile + 1);
}

__device__ void sched_run(const SchedParams &p) {
  __shared__ int32_t s_buf[kSchedThreads];
  __shared__ int32_t s_base[kSchedThreads + 1];  // first item of each doc in the chunk
  __shared__ int32_t s_nseg[kSchedThreads];
  __shared__ int32_t s_hist[kCostBins];
  const int tid = threadIdx.x;
  const MaskDev &m = p.m;
  int64_t running = 0;
  for (int c0 = 0; c0 < p.num_seqs; c0 += kSchedThreads) {
    const int d = c0 + tid;
    int64_t ntile = 0, nseg = 1;
    if (d < p.num_seqs) {
      const int64_t qs = clampi(p.cu_q[d], 0, p.n_q), qe = clampi(p.cu_q[d + 1], qs, p.n_q);
      const int64_t ks = clampi(p.cu_k[d], 0, p.n_k), ke = clampi(p.cu_k[d + 1], ks, p.n_k);
      int64_t qa, qb, ka, kb;
      view_range(qs, qe, m.q_view, qa, qb);
      view_range(ks, ke, m.k_view, ka, kb);
      ntile = p.by_keys ? (kb - ka + p.tile - 1) / p.tile : (qb - qa + p.tile - 1) / p.tile;
      if (p.nsplit > 1 && !p.by_keys) nseg = p.nsplit;
      if (nseg > p.max_seg) nseg = p.max_seg;
      if (nseg < 1) nseg = 1;
    }
    const int32_t mine = (int32_t)(ntile * nseg);
    const int32_t incl = block_scan(mine, s_buf);
    s_base[tid] = incl - mine;
    s_nseg[tid] = (int32_t)nseg;
    if (tid == kSchedThreads - 1) s_base[kSchedThreads] = incl;
    __syncthreads();
    const int32_t chunk_total = s_base[kSchedThreads];
    // one thread per item: find its document by binary search over s_base
    for (int32_t i = tid; i < chunk_total; i += kSchedThreads) {
      int lo = 0, hi = kSchedThreads;  // s_base[lo] <= i < s_base[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_base[mid] <= i) lo = mid; else hi = mid;
      }
      const int64_t idx = running + i;
      if (idx >= p.sb.capacity) continue;
      const int dd = c0 + lo;
      const int32_t local = i - s_base[lo];
      const int32_t ns = s_nseg[lo];
      const int64_t qs = clampi(p.cu_q[dd], 0, p.n_q), qe = clampi(p.cu_q[dd + 1], qs, p.n_q);
      const int64_t ks = clampi(p.cu_k[dd], 0, p.n_k), ke = clampi(p.cu_k[dd + 1], ks, p.n_k);
      WorkItem it;
      make_item(p, qs, qe, ks, ke, local / ns, local % ns, it);
      p.sb.items[idx] = it;
    }
    running += chunk_total;
    __syncthreads();
  }
  const int32_t count = (int32_t)(running < p.sb.capacity ? running : p.sb.capacity);
  // counting sort by decreasing cost (bin kCostBins-1-cost)
  for (int i = tid; i < kCostBins; i += kSchedThreads) s_hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < count; i += kSchedThreads) {
    int c = p.sb.items[i].cost;
    c = c >= kCostBins ? kCostBins - 1 : c;
    atomicAdd(&s_hist[kCostBins - 1 - c], 1);
  }
  __syncthreads();
  constexpr int BPT = kCostBins / kSchedThreads;  // bins per thread
  int32_t loc[BPT], sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) { loc[j] = s_hist[tid * BPT + j]; sum += loc[j]; }
  const int32_t incl = block_scan(sum, s_buf);
  int32_t acc = incl - sum;
#pragma unroll
  for (int j = 0; j < BPT; ++j) { s_hist[tid * BPT + j] = acc; acc += loc[j]; }
  __syncthreads();
  for (int i = tid; i < count; i += kSchedThreads) {
    int c = p.sb.items[i].cost;
    c = c >= kCostBins ? kCostBins - 1 : c;
    const int pos = atomicAdd(&s_hist[kCostBins - 1 - c], 1);
    p.sb.order[pos] = i;
  }
  if (tid == 0) *p.sb.count = count;
}

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(SchedParams p) { sched_run(p); }

// several independent schedules, one workgroup each
struct SchedBatch {
  SchedParams p[kMaxSchedJobs];
};
__global__ __launch_bounds__(kSchedThreads) void sched_batch_kernel(SchedBatch b) { sched_run(b.p[blockIdx.x]); }

hipError_t launch_schedule(const int32_t *cu_q, const int32_t *cu_k, int32_t num_seqs, int64_t n_q,
                           int64_t n_k, const MaskDev &m, int32_t tile, int32_t key_tile,
                           int32_t by_keys, int32_t max_seg, SchedBufs sb, hipStream_t s, int32_t nsplit) {
  SchedParams p{cu_q, cu_k, num_seqs, n_q, n_k, m, tile, key_tile, by_keys, max_seg < 1 ? 1 : max_seg, sb, nsplit};
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_schedules(const SchedJob *jobs, int n, hipStream_t s) {
  if (n < 1 || n > kMaxSchedJobs) return hipErrorInvalidValue;
  SchedBatch b{};
  for (int i = 0; i < n; ++i) {
    b.p[i] = jobs[i];
    if (b.p[i].max_seg < 1) b.p[i].max_seg = 1;
  }
  hipLaunchKernelGGL(sched_batch_kernel, dim3((unsigned)n), dim3(kSchedThreads), 0, s, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
struct FwdParams {
  const void *q, *k, *v;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  int32_t hq, group;
  float scale_log2;
  MaskDev m;
  void *out; int64_t o_st, o_sh;
  float *lse; int64_t lse_n;
  int32_t segmented;
  float *part_out, *part_lse;
  int64_t n_q;
  const WorkItem *items; const int32_t *order; const int32_t *count;
  // running state (acc, lse) when acc is set: see FwdArgs
  float *acc; int64_t a_st, a_sh;
  int32_t merge, final_view;
};

template <typename T> struct Tile;  // LDS pitches (elements)
template <> struct Tile<bf16> {
  template <int D> static constexpr int kpitch() { return D + 8; }   // 16-row b128 reads conflict free
  template <int D> static constexpr int vpitch() { return D + 32; }  // 4-row transpose reads conflict free
};
template <> struct Tile<float> {
  template <int D> static constexpr int kpitch() { return D + 1; }
  template <int D> static constexpr int vpitch() { return D + 4; }
};

template <typename T, int D, typename OutT>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  using M = Mfma32<T>;
  constexpr int KV = M::KV;
  constexpr int KSTEP = 2 * KV;
  constexpr int NS = D / KSTEP;
  constexpr int KP = Tile<T>::template kpitch<D>();
  constexpr int VP = Tile<T>::template vpitch<D>();
  constexpr int CH = 16 / sizeof(T);                 // elements per 16-byte chunk
  constexpr int NCH = kFwdBN * D / CH / 256;          // chunks per thread per tensor
  constexpr int ND = D / 32;
  constexpr bool kBf16 = sizeof(T) == 2;

  __shared__ __attribute__((aligned(16))) T sK[kFwdBN * KP];
  __shared__ __attribute__((aligned(16))) T sV[kFwdBN * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
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

  // Q fragments (B operand of S^T = K Q^T): lane holds row `row`, k-slots of group g.
  typename M::Frag qf[NS];
  {
    const T *qrow = (const T *)p.q + row * p.q_st + h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (kBf16) {
        i32x4 v = row_ok ? ld16(qrow + s * KSTEP + g * KV) : i32x4{0, 0, 0, 0};
        qf[s] = __builtin_bit_cast(bf16x8, v);
      } else {
        qf[s] = row_ok ? qrow[s * KSTEP + g] : 0.f;
      }
    }
  }

  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = f32x16{};
  float mrow = neg_inf();  // running max of scaled scores, log2 units
  float lsum = 0.f;        // this lane's share of the running sum

  const T *kb = (const T *)p.k;
  const T *vb = (const T *)p.v;

  for (int64_t kt = it.k0; kt < it.k1; kt += kFwdBN) {
    __syncthreads();
    // ---- stage K and V rows [kt, kt + 64) into LDS
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ci = tid + 256 * c;
      const int kr = ci / (D / CH);
      const int col = (ci % (D / CH)) * CH;
      const int64_t j = kt + kr;
      i32x4 kv4 = {0, 0, 0, 0}, vv4 = {0, 0, 0, 0};
      if (j < it.k1) {
        kv4 = ld16(kb + j * p.k_st + (int64_t)hk * p.k_sh + col);
        vv4 = ld16(vb + j * p.v_st + (int64_t)hk * p.v_sh + col);
      }
      if constexpr (kBf16) {
        st16(&sK[kr * KP + col], kv4);
      } else {
        float4 f = __builtin_bit_cast(float4, kv4);
        sK[kr * KP + col + 0] = f.x; sK[kr * KP + col + 1] = f.y;
        sK[kr * KP + col + 2] = f.z; sK[kr * KP + col + 3] = f.w;
      }
      st16(&sV[kr * VP + col], vv4);
    }
    __syncthreads();
    if (!wave_on) continue;

    // ---- per-wave skip / mask decision (wave-uniform)
    const int64_t klast = (kt + kFwdBN <= it.k1 ? kt + kFwdBN : it.k1) - 1;
    const int64_t kp_lo = m.pm.kpos(kt - it.kdoc0);
    const int64_t kp_hi = m.pm.kpos(klast - it.kdoc0);
    if (m.causal && kp_lo > wq_hi) continue;
    if (m.window > 0 && kp_hi <= wq_lo - m.window) continue;
    const bool full = (kt + kFwdBN <= it.k1) && (!m.causal || kp_hi <= wq_lo) &&
                      (m.window <= 0 || kp_lo > wq_hi - m.window);

    // ---- S^T = K Q^T for two 32-key sub-tiles
    f32x16 sc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 acc = f32x16{};
      const T *krow = &sK[(sb * 32 + l32) * KP + g * KV];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        typename M::Frag a;
        if constexpr (kBf16) a = *reinterpret_cast<const bf16x8 *>(krow + s * KSTEP);
        else a = krow[s * KSTEP];
        acc = M::mma(a, qf[s], acc);
      }
      sc[sb] = acc;
    }
    if (!full) {
      const int32_t t0 = (int32_t)(kt - it.kdoc0);
      const int32_t nvalid = (int32_t)(it.k1 - kt);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int32_t kk = sb * 32 + c_row(j, lane);
          const bool vis = (kk < nvalid) & visible(qpos, m.pm.kpos32(t0 + kk), m.causal, m.window);
          sc[sb][j] = vis ? sc[sb][j] : neg_inf();
        }
      }
    }
    // ---- online softmax (log2 domain)
    float mx = neg_inf();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[sb][j]);
    mx = pair32_max(mx);
    const float mnew = fmaxf(mrow, mx * p.scale_log2);
    const float muse = mnew == neg_inf() ? 0.f : mnew;
    const float alpha = fast_exp2(mrow - muse);
    mrow = mnew;
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(__builtin_fmaf(sc[sb][j], p.scale_log2, -muse));
        sc[sb][j] = e;
        ps += e;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (kBf16) {
      bf16x8 pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[t][e] = (bf16)sc[t >> 1][(t & 1) * 8 + e];
      const int u = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rowa = t * 16 + 4 * g + (u >> 2);
          const int col = dt * 32 + dh * 16 + 4 * (u & 3);
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sV[rowa * VP + col]));
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sV[(rowa + 8) * VP + col]));
          bf16x8 va;
          bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
          va[0] = l4[0]; va[1] = l4[1]; va[2] = l4[2]; va[3] = l4[3];
          va[4] = h4[0]; va[5] = h4[1]; va[6] = h4[2]; va[7] = h4[3];
          o[dt] = M::mma(va, pf[t], o[dt]);
        }
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float a = sV[(sb * 32 + c_row(j, lane)) * VP + dt * 32 + l32];
            o[dt] = M::mma(a, sc[sb][j], o[dt]);
          }
        }
      }
    }
  }
  if (!wave_on) return;

  // ---- epilogue: normalise, store out and lse
  const float lt = pair32_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (mrow + fast_log2(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (p.segmented) {
    // a row that sees no key of this part writes only its lse (-inf): the
    // merge of the parts gives the part weight 0 and never reads its out
    if (lt > 0.f) {
      float *po = p.part_out + ((int64_t)it.seg * p.n_q + row) * ((int64_t)p.hq * D) + (int64_t)h * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = dt * 32 + 8 * j4 + 4 * g;
          float4 v4 = {o[dt][4 * j4] * inv, o[dt][4 * j4 + 1] * inv, o[dt][4 * j4 + 2] * inv,
                       o[dt][4 * j4 + 3] * inv};
          *reinterpret_cast<float4 *>(po + d0) = v4;
        }
    }
    if (g == 0) p.part_lse[((int64_t)it.seg * p.hq + h) * p.n_q + row] = lse_v;
    return;
  }
  OutT *orow = (OutT *)p.out + row * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      if constexpr (sizeof(OutT) == 4) {
        float4 v4 = {o[dt][4 * j4] * inv, o[dt][4 * j4 + 1] * inv, o[dt][4 * j4 + 2] * inv, o[dt][4 * j4 + 3] * inv};
        *reinterpret_cast<float4 *>(orow + d0) = v4;
      } else {
        bf16x4 v4;
        v4[0] = (bf16)(o[dt][4 * j4] * inv); v4[1] = (bf16)(o[dt][4 * j4 + 1] * inv);
        v4[2] = (bf16)(o[dt][4 * j4 + 2] * inv); v4[3] = (bf16)(o[dt][4 * j4 + 3] * inv);
        *reinterpret_cast<bf16x4 *>(orow + d0) = v4;
      }
    }
  if (g == 0) p.lse[(int64_t)h * p.lse_n + row] = lse_v;
}

// ---------------------------------------------------------------------------
// several forwards of one shape in one launch (grid.y = which), e.g. the
// KV-parallel ranks, each too small to fill the chip alone
struct FwdBatch {
  FwdParams p[kMaxFwdBatch];
};
static_assert(sizeof(FwdBatch) <= 4096, "kernel arguments");
__device__ __forceinline__ const FwdParams &fwd_pick(const FwdParams &p) { return p; }
__device__ __forceinline__ const FwdParams &fwd_pick(const FwdBatch &b) { return b.p[blockIdx.y]; }

// bf16 forward: K/V tiles arrive by asynchronous global->LDS copies into two
// padded buffers, so tile t+1 is in flight while tile t is computed; one
// barrier per tile. The loop is unrolled by two so that every LDS read names
// a fixed buffer (the compiler then only waits for the copy at the barrier).
// ---------------------------------------------------------------------------
// MASK = false: launches without a causal or window mask; only the keys past
// the end of a ragged last tile are masked.
// PT: FwdParams (one forward) or FwdBatch (grid.y picks the forward)
// BN: keys per tile; 32 (38 KB of LDS, at most 168 registers) lets three
// workgroups share a CU, 64 fits two.
template <int D, typename OutT, bool MASK, typename PT, int BN>
__global__ __launch_bounds__(256, BN == 32 ? 3 : 2) void fwd_bf16_kernel(PT args) {
  const FwdParams &p = fwd_pick(args);
  using M = Mfma32<bf16>;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int NSB = BN / 32;  // 32-key sub-tiles of a tile
  using KT = PadTile<D, D / 8 + 1, BN>;  // row reads
  using VT = PadTile<D, D / 8 + 4, BN>;  // transpose reads
  static_assert(BN == 32 || BN == 64, "tiles are 32 or 64 keys");
  // A row's reference max may trail its true max: the final lse = max +
  // log2(sum) is exact for any reference, and f32 and bf16 keep the same
  // relative precision at any magnitude. Once every row of a wave has a
  // reference, a tile's probabilities are formed against it without the
  // tile's max; they are kept unless some lane's share of a row's tile sum
  // passes 2^32 (the row's max outgrew the reference by at least 32 - log2(16)
  // log2 units). Otherwise, or while a row has no reference, the tile's max is
  // taken, and the output rescaled when it passes the reference by more than
  // kRescaleSlack.
  constexpr float kRescaleSlack = 8.f;
  constexpr float kTileSumMax = 4294967296.f;  // 2^32
  __shared__ __attribute__((aligned(1024))) bf16 sK0[KT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[VT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[KT::ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[VT::ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31, u = lane & 15, dh = (lane >> 4) & 1;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < 4);  // 4 waves: lets the copy loops drop their range tests
  // logical index = (kv head, item, head in group): the heads that share a kv
  // head, and the items of one kv head, are neighbours
  const int lb = xcd_block();
  const int cap = gridDim.x / p.hq;
  const int hg = lb % p.group, li = lb / p.group;
  const int rank = li % cap;
  const int hk = li / cap;
  const int h = hk * p.group + hg;
  if (rank >= *p.count) return;
  const WorkItem it = p.items[p.order[rank]];
  // every position and index fits in 32 bits (checked on the host)
  const int32_t k1 = it.k1, kd0 = it.kdoc0, q1 = it.q1;
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

  bf16x8 qf[NS];
  {
    const bf16 *qrow = (const bf16 *)p.q + (int64_t)row * p.q_st + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i32x4 v = row_ok ? ld16(qrow + s * 16 + g * 8) : i32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = f32x16{};
  float mrow = neg_inf(), lsum = 0.f;
  const float sl2 = p.scale_log2;

  const bf16 *kb = (const bf16 *)p.k;
  const bf16 *vb = (const bf16 *)p.v;
  const int32_t kst = (int32_t)p.k_st, vst = (int32_t)p.v_st;
  int koffs[KT::NJ], voffs[VT::NJ];
  tile_voffsets<KT>(koffs, kst, w, lane);
  tile_voffsets<VT>(voffs, vst, w, lane);
  // tile base pointers, advanced by one tile per stage
  const bf16 *kp = kb + (int64_t)it.k0 * p.k_st + (int64_t)hk * p.k_sh;
  const bf16 *vp = vb + (int64_t)it.k0 * p.v_st + (int64_t)hk * p.v_sh;
  auto stage = [&](bf16 *sk, bf16 *sv, int32_t kt) {
    const int32_t nvalid = k1 - kt < BN ? k1 - kt : BN;
    dma_tile_buf<KT>(sk, kp, ((nvalid - 1) * kst + D) * 2, koffs, w);
    dma_tile_buf<VT>(sv, vp, ((nvalid - 1) * vst + D) * 2, voffs, w);
    kp += BN * (int64_t)kst;
    vp += BN * (int64_t)vst;
  };

  auto compute = [&](const bf16 *sk, const bf16 *sv, int32_t kt) {
    if (!wave_on) return;
    const int32_t nvalid = k1 - kt;
    const int32_t kp_lo = kpos(kt - kd0);
    const int32_t kp_hi = kpos((nvalid < BN ? k1 : kt + BN) - 1 - kd0);
    if (causal && kp_lo > wq_hi) return;
    if (W > 0 && kp_hi <= wq_lo - W) return;
    const bool full = (nvalid >= BN) && (!causal || kp_hi <= wq_lo) && (W <= 0 || kp_lo > wq_hi - W);
    // with 64-key tiles the two 32-key sub-tiles' MFMAs alternate, so
    // consecutive MFMAs never wait on each other's accumulator; a 32-key tile
    // is one chain, whose waits the SIMD's other waves fill
    f32x16 sc[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) sc[sb] = f32x16{};
    {
      bf16x8 kfr[NSB][NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
          kfr[sb][s] = *reinterpret_cast<const bf16x8 *>(sk + (sb * 32 + l32) * KT::PITCH + s * 16 + g * 8);
      // every K read is issued before the first MFMA (left alone, the
      // compiler issues them two at a time, each pair waited for just before
      // its MFMAs): 304 -> 302 us a launch on the headline step
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) sc[sb] = M::mma(kfr[sb][s], qf[s], sc[sb]);
    }
    if (!full) {  // wave-uniform
      // element (sb, j) holds key kt + 4g + c, c = 32 sb + 8 (j / 4) + j % 4
      // (a compile-time constant): compare c with per-lane bounds
      const int32_t lim = nvalid - 4 * g;
      const int32_t t0 = kt - kd0 + 4 * g;
      if constexpr (!MASK) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            sc[sb][j] = c < lim ? sc[sb][j] : neg_inf();
          }
      } else if (RR == 0) {
        const int32_t d = qpos - (koff + t0), dw = d - W;  // causal: c <= d; window: c > d - W
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            const bool vis = (c < lim) & ((causal == 0) | (c <= d)) & ((W <= 0) | (c > dw));
            sc[sb][j] = vis ? sc[sb][j] : neg_inf();
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = sb * 32 + 8 * (j >> 2) + (j & 3);
            const int32_t kpj = kpos_rr(t0 + c);
            const bool vis = (c < lim) & ((causal == 0) | (kpj <= qpos)) & ((W <= 0) | (kpj > qpos - W));
            sc[sb][j] = vis ? sc[sb][j] : neg_inf();
          }
      }
    }
    bf16x8 pf[BN / 16];
    float ts = 0.f;  // this lane's share of the tile's row sum
    auto probs = [&](float ref) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = fast_exp2(__builtin_fmaf(sc[sb][j], sl2, -ref));
          ts = (sb | j) ? ts + e : e;
          pf[sb * 2 + (j >> 3)][j & 7] = (bf16)e;
        }
    };
    // wave-uniform: a NaN or infinite share fails the test as well
    bool kept = false;
    if (__all(mrow != neg_inf())) {
      probs(mrow);
      kept = __all(ts <= kTileSumMax);
    }
    if (!kept) {
      float mx = neg_inf();
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[sb][j]);
      mx = pair32_max(mx);
      const float mt = mx * sl2;
      if (!__all(mt <= mrow + kRescaleSlack)) {  // some row outgrew its reference
        const float mnew = fmaxf(mrow, mt);
        const float alpha = fast_exp2(mrow - (mnew == neg_inf() ? 0.f : mnew));
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i) o[i] *= alpha;
        mrow = mnew;
      }
      probs(mrow == neg_inf() ? 0.f : mrow);
    }
    lsum += ts;
    // per 16-key chunk t: the ND d-tiles' transpose reads, then their MFMAs
    // (independent accumulators back to back)
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      bf16x8 va[ND];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int ra = t * 16 + 4 * g;
        const int col = dt * 32 + dh * 16;
        const bf16x4 lo = tile_tr4(sv, VT::PITCH, ra, col, u);
        const bf16x4 hi = tile_tr4(sv, VT::PITCH, ra + 8, col, u);
        va[dt][0] = lo[0]; va[dt][1] = lo[1]; va[dt][2] = lo[2]; va[dt][3] = lo[3];
        va[dt][4] = hi[0]; va[dt][5] = hi[1]; va[dt][6] = hi[2]; va[dt][7] = hi[3];
      }
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[dt] = M::mma(va[dt], pf[t], o[dt]);
    }
  };

  if (it.k0 < k1) stage(sK0, sV0, it.k0);
  __syncthreads();
  for (int32_t kt = it.k0; kt < k1; kt += 2 * BN) {
    if (kt + BN < k1) stage(sK1, sV1, kt + BN);
    compute(sK0, sV0, kt);
    __syncthreads();
    if (kt + BN >= k1) break;
    if (kt + 2 * BN < k1) stage(sK0, sV0, kt + 2 * BN);
    compute(sK1, sV1, kt + BN);
    __syncthreads();
  }
  if (!wave_on) return;

  const float lt = pair32_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (mrow + fast_log2(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (p.segmented) {
    // a row that sees no key of this part writes only its lse (-inf): the
    // merge of the parts gives the part weight 0 and never reads its out
    if (lt > 0.f) {
      float *po = p.part_out + ((int64_t)it.seg * p.n_q + row) * ((int64_t)p.hq * D) + (int64_t)h * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = dt * 32 + 8 * j4 + 4 * g;
          float4 v4 = {o[dt][4 * j4] * inv, o[dt][4 * j4 + 1] * inv, o[dt][4 * j4 + 2] * inv,
                       o[dt][4 * j4 + 3] * inv};
          *reinterpret_cast<float4 *>(po + d0) = v4;
        }
    }
    if (g == 0) p.part_lse[((int64_t)it.seg * p.hq + h) * p.n_q + row] = lse_v;
    return;
  }
  OutT *orow = (OutT *)p.out + (int64_t)row * p.o_st + (int64_t)h * p.o_sh;
  float wa = 0.f, wb = inv;  // output = wa * acc + wb * (unnormalised o)
  float *arow = p.acc + (int64_t)row * p.a_st + (int64_t)h * p.a_sh;
  const int64_t lidx = (int64_t)h * p.lse_n + row;
  float ln = lse_v;
  float4 acc4[ND][4];
  if (p.merge) {
    // The running out rows load beside the running lse, not after it: every
    // row a merging launch touches had its acc written by the schedule's
    // first block, and a row whose lse is still -inf takes weight 0 below by
    // a select, so what its acc holds never enters the result.
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        acc4[dt][j4] = *reinterpret_cast<const float4 *>(arow + dt * 32 + 8 * j4 + 4 * g);
    // online-softmax merge with the running state of this (row, head), in the
    // sigmoid form: lse' = max + log1p(exp(-|la - lb|)), sig = exp(lb - lse'),
    // out' = acc - sig (acc - block_out); an empty side has weight 0
    const float la = p.lse[lidx], lb = lse_v;
    if (fmaxf(la, lb) == neg_inf()) {
      ln = neg_inf(); wb = 0.f;
    } else if (la == neg_inf()) {
      ln = lb;
    } else if (lb == neg_inf()) {
      ln = la; wa = 1.f; wb = 0.f;
    } else {
      ln = fmaxf(la, lb) + log1pf(expf(-fabsf(la - lb)));
      const float sig = expf(lb - ln);
      wa = 1.f - sig; wb = sig * inv;
    }
  }
  if (g == 0) p.lse[lidx] = ln;  // after every lane's read: ln depends on it
  // rows whose result is final go to out, the others to the running acc
  const bool fin = p.acc == nullptr || ((row < it.qmid ? 1 : 2) & p.final_view);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = dt * 32 + 8 * j4 + 4 * g;
      float4 v4 = {o[dt][4 * j4] * wb, o[dt][4 * j4 + 1] * wb, o[dt][4 * j4 + 2] * wb, o[dt][4 * j4 + 3] * wb};
      if (p.merge) {
        const float4 a4 = acc4[dt][j4];
        const bool use = wa != 0.f;
        v4.x = use ? v4.x + wa * a4.x : v4.x;
        v4.y = use ? v4.y + wa * a4.y : v4.y;
        v4.z = use ? v4.z + wa * a4.z : v4.z;
        v4.w = use ? v4.w + wa * a4.w : v4.w;
      }
      if (!fin) {
        *reinterpret_cast<float4 *>(arow + d0) = v4;
      } else if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<float4 *>(orow + d0) = v4;
      } else {
        bf16x4 b4;
        b4[0] = (bf16)v4.x; b4[1] = (bf16)v4.y; b4[2] = (bf16)v4.z; b4[3] = (bf16)v4.w;
        *reinterpret_cast<bf16x4 *>(orow + d0) = b4;
      }
    }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams &fp, int out_dtype, int64_t grid, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    const bool mask = fp.m.causal || fp.m.window > 0;
    if (out_dtype == 0) {
      if (mask) hipLaunchKernelGGL((fwd_bf16_kernel<D, bf16, true, FwdParams, kFwdBf16BN>), dim3((unsigned)grid), dim3(256), 0, s, fp);
      else hipLaunchKernelGGL((fwd_bf16_kernel<D, bf16, false, FwdParams, kFwdBf16BN>), dim3((unsigned)grid), dim3(256), 0, s, fp);
    } else {
      if (mask) hipLaunchKernelGGL((fwd_bf16_kernel<D, float, true, FwdParams, kFwdBf16BN>), dim3((unsigned)grid), dim3(256), 0, s, fp);
      else hipLaunchKernelGGL((fwd_bf16_kernel<D, float, false, FwdParams, kFwdBf16BN>), dim3((unsigned)grid), dim3(256), 0, s, fp);
    }
  } else {
    if (out_dtype == 0)
      hipLaunchKernelGGL((fwd_kernel<T, D, bf16>), dim3((unsigned)grid), dim3(256), 0, s, fp);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, float>), dim3((unsigned)grid), dim3(256), 0, s, fp);
  }
  return hipGetLastError();
}

static FwdParams fwd_params(const FwdArgs &a) {
  FwdParams fp;
  fp.q = a.q.data; fp.k = a.k.data; fp.v = a.v.data;
  fp.q_st = a.q.st; fp.q_sh = a.q.sh; fp.k_st = a.k.st; fp.k_sh = a.k.sh; fp.v_st = a.v.st; fp.v_sh = a.v.sh;
  fp.hq = a.hq; fp.group = a.hq / a.hkv;
  fp.scale_log2 = a.scale * kLog2e;
  fp.m = a.mask;
  fp.out = a.out; fp.o_st = a.o_st; fp.o_sh = a.o_sh;
  fp.lse = a.lse; fp.lse_n = a.lse_n;
  fp.segmented = a.part_out != nullptr;
  fp.part_out = a.part_out; fp.part_lse = a.part_lse;
  fp.n_q = a.n_q;
  fp.items = a.sched.items; fp.order = a.sched.order; fp.count = a.sched.count;
  fp.acc = a.acc; fp.a_st = a.a_st; fp.a_sh = a.a_sh;
  fp.merge = a.acc != nullptr && a.merge; fp.final_view = a.final_view;
  return fp;
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t s) {
  const FwdParams fp = fwd_params(a);
  const int64_t grid = a.grid_items * a.hq;
  if (grid <= 0) return hipSuccess;
  if (a.dtype == 0) {
    if (a.head_dim == 128) return launch_fwd_t<bf16, 128>(fp, a.out_dtype, grid, s);
    return launch_fwd_t<bf16, 64>(fp, a.out_dtype, grid, s);
  }
  if (a.head_dim == 128) return launch_fwd_t<float, 128>(fp, a.out_dtype, grid, s);
  return launch_fwd_t<float, 64>(fp, a.out_dtype, grid, s);
}

template <int D>
static hipError_t launch_fwd_batch_t(const FwdBatch &b, bool mask, int out_dtype, int64_t grid, int n, hipStream_t s) {
  const dim3 g((unsigned)grid, (unsigned)n);
  if (out_dtype == 0) {
    if (mask) hipLaunchKernelGGL((fwd_bf16_kernel<D, bf16, true, FwdBatch, kFwdBf16BN>), g, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((fwd_bf16_kernel<D, bf16, false, FwdBatch, kFwdBf16BN>), g, dim3(256), 0, s, b);
  } else {
    if (mask) hipLaunchKernelGGL((fwd_bf16_kernel<D, float, true, FwdBatch, kFwdBf16BN>), g, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((fwd_bf16_kernel<D, float, false, FwdBatch, kFwdBf16BN>), g, dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

bool fwd_batchable(const FwdArgs *a, int n) {
  if (n < 1 || n > kMaxFwdBatch || a[0].dtype != 0) return false;
  const bool mask0 = a[0].mask.causal || a[0].mask.window > 0;
  for (int i = 0; i < n; ++i) {
    const bool mask = a[i].mask.causal || a[i].mask.window > 0;
    if (a[i].dtype != 0 || a[i].head_dim != a[0].head_dim || a[i].out_dtype != a[0].out_dtype ||
        a[i].hq != a[0].hq || a[i].grid_items != a[0].grid_items || mask != mask0)
      return false;
  }
  return true;
}

hipError_t launch_fwd_batch(const FwdArgs *a, int n, hipStream_t s) {
  if (!fwd_batchable(a, n)) return hipErrorInvalidValue;
  FwdBatch b{};
  for (int i = 0; i < n; ++i) b.p[i] = fwd_params(a[i]);
  const int64_t grid = a[0].grid_items * a[0].hq;
  if (grid <= 0) return hipSuccess;
  const bool mask = a[0].mask.causal || a[0].mask.window > 0;
  if (a[0].head_dim == 128) return launch_fwd_batch_t<128>(b, mask, a[0].out_dtype, grid, n, s);
  return launch_fwd_batch_t<64>(b, mask, a[0].out_dtype, grid, n, s);
}

}  // namespace attn
