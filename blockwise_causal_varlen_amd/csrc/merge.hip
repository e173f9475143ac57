// Streaming kernels (HBM bound): online-softmax merges, the backward row term
// delta, a float fill, and the zig-zag shard gather.
//
// Merge (NeMo AutoModel zigzag_ring_attention, `update_out_and_lse`;
// ring_attention, `_update_out_and_lse` in its sigmoid form): for every
// (row, head) of the running state
//     lse' = max + log1p(exp(-|lse - block_lse|))
//     sigma = exp(block_lse - lse')          (= sigmoid(block_lse - lse))
//     out' = out - sigma * (out - block_out)
// A group of D/4 lanes owns one (row, head): each lane moves 16 bytes of the
// f32 running output, so a wave streams two or four contiguous 512-byte rows.
#include "internal.h"

namespace attn {

template <typename T> __device__ __forceinline__ f32x4 ld4(const T *p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 ld4<bf16>(const bf16 *p) {
  bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <typename T> __device__ __forceinline__ void st4(T *p, f32x4 v);
template <> __device__ __forceinline__ void st4<float>(float *p, f32x4 v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ __forceinline__ void st4<bf16>(bf16 *p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4 *>(p) = b;
}
// Streaming forms: nontemporal loads and stores for data a kernel touches
// once (measured on MI355X: a 677 MB merge 4.5 -> 5.6 TB/s, a plain copy
// 5.0 -> 5.7 TB/s).
template <typename T> __device__ __forceinline__ f32x4 ld4s(const T *p);
template <> __device__ __forceinline__ f32x4 ld4s<float>(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
template <> __device__ __forceinline__ f32x4 ld4s<bf16>(const bf16 *p) {
  const bf16x4 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(p));
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <typename T> __device__ __forceinline__ void st4s(T *p, f32x4 v);
template <> __device__ __forceinline__ void st4s<float>(float *p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}
template <> __device__ __forceinline__ void st4s<bf16>(bf16 *p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  __builtin_nontemporal_store(b, reinterpret_cast<bf16x4 *>(p));
}

// Is `row` inside the view of its document? (binary search over cu)
__device__ __forceinline__ bool row_in_view(const int32_t *cu, int32_t num_seqs, int view, int64_t row) {
  if (view == 0) return true;
  int lo = 0, hi = num_seqs;  // find d with cu[d] <= row < cu[d+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  const int64_t s = cu[lo], e = cu[lo + 1];
  if (row < s || row >= e) return false;
  const int64_t h = (e - s) / 2;
  return view == 1 ? row < s + h : row >= s + h;
}

// One workgroup streams one row (all heads) at a time; the view test is one
// (uniform) binary search per row. Per pass a group of D/4 lanes owns one
// head (16 bytes a lane); the NB passes' loads (streaming, nontemporal) are
// all issued before any is used: their head index is clamped to the last
// head instead of guarded, so no branch sits between them (a guarded form
// measured 1.6x slower at NB = 4). INIT: the block initialises the state;
// FINAL: every row goes to the final output (the last merge of a schedule).
template <int D, typename BT, typename FT, bool INIT, bool FINAL>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int G = D / 4;      // lanes per (row, head)
  constexpr int HP = 256 / G;   // heads per pass
  constexpr int NB = 4;         // passes in flight (32 heads of D = 128 at once)
  const int sub = threadIdx.x % G, hl = threadIdx.x / G;
  const int H = (int)a.h;
  for (int64_t row = blockIdx.x; row < a.n; row += gridDim.x) {
    const bool in_view = row_in_view(a.cu, a.num_seqs, a.view, row);
    const float *orow = a.out + row * a.o_st + 4 * sub;
    if (!in_view) {
      // rows outside the view keep their state; a final cast still covers them
      if constexpr (FINAL) {
        FT *frow = (FT *)a.fout + row * a.f_st + 4 * sub;
        for (int hb = 0; hb < H; hb += NB * HP) {
          f32x4 v[NB];
#pragma unroll
          for (int k = 0; k < NB; ++k) {
            const int h = min(hb + k * HP + hl, H - 1);
            v[k] = ld4s<float>(orow + h * a.o_sh);
          }
#pragma unroll
          for (int k = 0; k < NB; ++k) {
            const int h = hb + k * HP + hl;
            if (h < H) st4s<FT>(frow + h * a.f_sh, v[k]);
          }
        }
      }
      continue;
    }
    const BT *brow = (const BT *)a.bout + row * a.b_st + 4 * sub;
    for (int hb = 0; hb < H; hb += NB * HP) {
      f32x4 oa[NB], bo[NB];
      float la[NB], lb[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int h = min(hb + k * HP + hl, H - 1);
        const int64_t li = (int64_t)h * a.n + row;
        lb[k] = a.blse[li];
        bo[k] = ld4s<BT>(brow + h * a.b_sh);
        if constexpr (!INIT) {
          la[k] = a.lse[li];
          oa[k] = ld4s<float>(orow + h * a.o_sh);
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int h = hb + k * HP + hl;
        float ln, sig;
        f32x4 res;
        if constexpr (INIT) {
          ln = lb[k]; sig = 1.f; res = bo[k];
        } else {
          const float mx = fmaxf(la[k], lb[k]);
          // an empty partial (lse = -inf) has weight 0, whatever its out holds
          if (mx == neg_inf()) {
            ln = neg_inf(); sig = 0.f; res = f32x4{};
          } else if (la[k] == neg_inf()) {
            ln = lb[k]; sig = 1.f; res = bo[k];
          } else if (lb[k] == neg_inf()) {
            ln = la[k]; sig = 0.f; res = oa[k];
          } else {
            ln = mx + log1pf(expf(-fabsf(la[k] - lb[k])));
            sig = expf(lb[k] - ln);
            res = oa[k] - sig * (oa[k] - bo[k]);
          }
        }
        if (h < H) {
          if constexpr (FINAL) st4s<FT>((FT *)a.fout + row * a.f_st + h * a.f_sh + 4 * sub, res);
          else st4s<float>(a.out + row * a.o_st + h * a.o_sh + 4 * sub, res);
          if (sub == 0) {
            const int64_t li = (int64_t)h * a.n + row;
            a.lse[li] = ln;
            if (a.weight) a.weight[li] = sig;
          }
        }
      }
    }
  }
}

// workgroups of a row-streaming kernel: one per row up to 64 per CU
static unsigned row_grid(int64_t rows) {
  const int64_t cap = 256 * 64;
  return (unsigned)(rows < 1 ? 1 : (rows > cap ? cap : rows));
}

static unsigned stream_grid(int64_t pairs, int per_blk) {
  int64_t b = (pairs + per_blk - 1) / per_blk;
  const int64_t cap = 256 * 32;  // enough waves to saturate HBM, grid-stride beyond
  if (b > cap) b = cap;
  return (unsigned)(b < 1 ? 1 : b);
}

template <int D, typename BT>
static void launch_merge_b(const MergeArgs &a, hipStream_t s, unsigned grid) {
  const dim3 g(grid), b(256);
  if (a.fout) {
    if (a.fout_dtype == 0) {
      if (a.init) hipLaunchKernelGGL((merge_kernel<D, BT, bf16, true, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((merge_kernel<D, BT, bf16, false, true>), g, b, 0, s, a);
    } else {
      if (a.init) hipLaunchKernelGGL((merge_kernel<D, BT, float, true, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((merge_kernel<D, BT, float, false, true>), g, b, 0, s, a);
    }
  } else {
    if (a.init) hipLaunchKernelGGL((merge_kernel<D, BT, float, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<D, BT, float, false, false>), g, b, 0, s, a);
  }
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
  if (a.n * a.h == 0) return hipSuccess;
  const unsigned grid = row_grid(a.n);
  if (a.d == 128) {
    if (a.bout_dtype == 0) launch_merge_b<128, bf16>(a, s, grid);
    else launch_merge_b<128, float>(a, s, grid);
  } else {
    if (a.bout_dtype == 0) launch_merge_b<64, bf16>(a, s, grid);
    else launch_merge_b<64, float>(a, s, grid);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// EAGLE-3 test-time-training diagonal blocks (NeMo AutoModel ring_attention,
// `_CachedRingAttention`, `_merge_diag`): row t of q head h sees exactly one
// key of such a block, k[t, g] (g = h / group), whose value is v[t, g]. The
// block's partial is (block_out = v[t, g], block_lse = scale <q[t, h], k[t, g]>)
// and merges into the running (out, lse) like any block. Its backward is the
// one-key case of the joint-softmax gradient (given the merged lse, delta):
//   p = exp(scale <q, k> - lse),  ds = p (<dout, v> - delta)
//   dq[t, h] += scale ds k,  dk[t, g] += scale sum_h ds q,  dv[t, g] += sum_h p dout
// A group of D/4 lanes owns one (row, head) (forward) or (row, kv head)
// (backward, looping over the group's q heads: no atomics); each lane holds 4
// elements and the dot products reduce across the group's lanes.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, G);
  return x;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

template <int D, typename T, typename FT>
__global__ __launch_bounds__(256) void diag_merge_kernel(DiagArgs a) {
  constexpr int G = D / 4;
  const int32_t total = a.n * a.hq;
  const int sub = threadIdx.x % G;
  const int32_t per_blk = 256 / G;
  for (int32_t pr = blockIdx.x * per_blk + threadIdx.x / G; pr < total; pr += gridDim.x * per_blk) {
    const int32_t row = pr / a.hq;
    const int32_t h = pr - row * a.hq;
    const int32_t g = h / a.group;
    const f32x4 q4 = ld4<T>((const T *)a.q + row * a.q_st + h * a.q_sh + 4 * sub);
    const f32x4 k4 = ld4<T>((const T *)a.k + row * a.k_st + g * a.k_sh + 4 * sub);
    const f32x4 v4 = ld4<T>((const T *)a.v + row * a.v_st + g * a.v_sh + 4 * sub);
    const float lb = a.scale * group_sum<G>(dot4(q4, k4));
    const int64_t li = (int64_t)h * a.n + row;
    const float la = a.lse[li];
    float* orow = a.out + row * a.o_st + h * a.o_sh + 4 * sub;
    f32x4 res;
    float ln;
    if (la == neg_inf()) {  // nothing merged yet for this row: the diagonal alone
      res = v4;
      ln = lb;
    } else {
      const f32x4 oa = ld4<float>(orow);
      ln = fmaxf(la, lb) + log1pf(expf(-fabsf(la - lb)));
      const float sig = expf(lb - ln);
      res = oa - sig * (oa - v4);
    }
    st4<float>(orow, res);
    if (a.fout) st4<FT>((FT *)a.fout + row * a.f_st + h * a.f_sh + 4 * sub, res);
    if (sub == 0) a.lse[li] = ln;
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void diag_bwd_kernel(DiagArgs a) {
  constexpr int G = D / 4;
  const int32_t hkv = a.hq / a.group;
  const int32_t total = a.n * hkv;
  const int sub = threadIdx.x % G;
  const int32_t per_blk = 256 / G;
  for (int32_t pr = blockIdx.x * per_blk + threadIdx.x / G; pr < total; pr += gridDim.x * per_blk) {
    const int32_t row = pr / hkv;
    const int32_t g = pr - row * hkv;
    const f32x4 k4 = ld4<T>((const T *)a.k + row * a.k_st + g * a.k_sh + 4 * sub);
    const f32x4 v4 = ld4<T>((const T *)a.v + row * a.v_st + g * a.v_sh + 4 * sub);
    f32x4 dka = {0.f, 0.f, 0.f, 0.f}, dva = {0.f, 0.f, 0.f, 0.f};
    for (int32_t hh = 0; hh < a.group; ++hh) {
      const int32_t h = g * a.group + hh;
      const f32x4 q4 = ld4<T>((const T *)a.q + row * a.q_st + h * a.q_sh + 4 * sub);
      const f32x4 o4 = ld4<T>((const T *)a.dout + row * a.do_st + h * a.do_sh + 4 * sub);
      const float s = a.scale * group_sum<G>(dot4(q4, k4));
      const float dp = group_sum<G>(dot4(o4, v4));
      const int64_t li = (int64_t)h * a.n + row;
      const float l = a.lse[li];
      const float pr_ = l == neg_inf() ? 0.f : expf(s - l);
      const float ds = pr_ * (dp - a.delta[li]);
      float *dqr = a.dq + row * a.dq_st + h * a.dq_sh + 4 * sub;
      st4<float>(dqr, ld4<float>(dqr) + (a.scale * ds) * k4);
      dka += ds * q4;
      dva += pr_ * o4;
    }
    float *dkr = a.dk + row * a.dk_st + g * a.dk_sh + 4 * sub;
    float *dvr = a.dv + row * a.dv_st + g * a.dv_sh + 4 * sub;
    st4<float>(dkr, ld4<float>(dkr) + a.scale * dka);
    st4<float>(dvr, ld4<float>(dvr) + dva);
  }
}

template <int D>
static hipError_t launch_diag_merge_d(const DiagArgs &a, hipStream_t s) {
  const unsigned grid = stream_grid((int64_t)a.n * a.hq, 256 / (D / 4));
  const bool fb = a.fout && a.fout_dtype == 0;
  if (a.dtype == 0) {
    if (fb) hipLaunchKernelGGL((diag_merge_kernel<D, bf16, bf16>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((diag_merge_kernel<D, bf16, float>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (fb) hipLaunchKernelGGL((diag_merge_kernel<D, float, bf16>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((diag_merge_kernel<D, float, float>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_diag_merge(const DiagArgs &a, hipStream_t s) {
  if ((int64_t)a.n * a.hq == 0) return hipSuccess;
  return a.d == 128 ? launch_diag_merge_d<128>(a, s) : launch_diag_merge_d<64>(a, s);
}

template <int D>
static hipError_t launch_diag_bwd_d(const DiagArgs &a, hipStream_t s) {
  const unsigned grid = stream_grid((int64_t)a.n * (a.hq / a.group), 256 / (D / 4));
  if (a.dtype == 0) hipLaunchKernelGGL((diag_bwd_kernel<D, bf16>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((diag_bwd_kernel<D, float>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_diag_bwd(const DiagArgs &a, hipStream_t s) {
  if ((int64_t)a.n * a.hq == 0) return hipSuccess;
  return a.d == 128 ? launch_diag_bwd_d<128>(a, s) : launch_diag_bwd_d<64>(a, s);
}

// ---------------------------------------------------------------------------
// Ulysses all-to-all between virtual ranks (NeMo AutoModel ulysses_attention,
// `_gather_seq_scatter_heads` / `_scatter_seq_gather_heads`, `_gather_lse` /
// `_scatter_lse`). With S_l = S / uly rows and H_l = H / uly heads per rank:
//   to heads:  head shard r [S, H_l]:   row t, head j  <- sequence shard t / S_l,
//              row t % S_l, head r H_l + j
//   to rows:   the inverse.
// Work-group (x, y = source rank, z = destination rank) copies the rows that go
// from y to z, 16 bytes per lane; source and destination ranks are uniform, so
// the per-rank pointers are read from the kernel arguments by scalar loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reshard_kernel(ReshardArgs a) {
  const int sr = blockIdx.y, dr = blockIdx.z;
  const int chunks = a.row_bytes / 16;
  const int32_t per_row = a.h_local * chunks;
  const int64_t total = (int64_t)a.n_local * per_row;
  const char *src = a.src[sr];
  char *dst = a.dst[dr];
  const int64_t s_st = a.s_st[sr], s_sh = a.s_sh[sr], d_st = a.d_st[dr], d_sh = a.d_sh[dr];
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int32_t tl = (int32_t)(e / per_row);
    const int32_t rem = (int32_t)(e - (int64_t)tl * per_row);
    const int32_t j = rem / chunks, c = rem - j * chunks;
    int64_t so, dof;
    if (a.to_heads) {  // source: sequence shard sr; destination: head shard dr
      so = tl * s_st + (int64_t)(dr * a.h_local + j) * s_sh;
      dof = ((int64_t)sr * a.n_local + tl) * d_st + j * d_sh;
    } else {           // source: head shard sr; destination: sequence shard dr
      so = ((int64_t)dr * a.n_local + tl) * s_st + j * s_sh;
      dof = tl * d_st + (int64_t)(sr * a.h_local + j) * d_sh;
    }
    st16(dst + dof + 16 * c, ld16(src + so + 16 * c));
  }
}

__global__ __launch_bounds__(256) void lse_reshard_kernel(LseReshardArgs a) {
  const int sr = blockIdx.y, dr = blockIdx.z;
  const int64_t total = (int64_t)a.n_local * a.h_local;
  const float *src = a.src[sr];
  float *dst = a.dst[dr];
  const int64_t n_full = (int64_t)a.n_local * a.uly;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int32_t j = (int32_t)(e / a.n_local);
    const int32_t tl = (int32_t)(e - (int64_t)j * a.n_local);
    if (a.to_heads)  // [H, S_l] of sequence shard sr -> [H_l, S] of head shard dr
      dst[j * n_full + (int64_t)sr * a.n_local + tl] = src[(int64_t)(dr * a.h_local + j) * a.n_local + tl];
    else             // [H_l, S] of head shard sr -> [H, S_l] of sequence shard dr
      dst[(int64_t)(sr * a.h_local + j) * a.n_local + tl] = src[j * n_full + (int64_t)dr * a.n_local + tl];
  }
}

hipError_t launch_reshard(const ReshardArgs &a, hipStream_t s) {
  const int64_t per = (int64_t)a.n_local * a.h_local * (a.row_bytes / 16);
  if (per == 0) return hipSuccess;
  int64_t bx = (per + 255) / 256;
  if (bx > 256) bx = 256;
  hipLaunchKernelGGL(reshard_kernel, dim3((unsigned)bx, a.uly, a.uly), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lse_reshard(const LseReshardArgs &a, hipStream_t s) {
  const int64_t per = (int64_t)a.n_local * a.h_local;
  if (per == 0) return hipSuccess;
  int64_t bx = (per + 255) / 256;
  if (bx > 64) bx = 64;
  hipLaunchKernelGGL(lse_reshard_kernel, dim3((unsigned)bx, a.uly, a.uly), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Transposed output (AWS NKI "Attention KV-Parallel Segmented CTE", parameter
// `tp_out`: the output as [heads, D, S]): dst[h, d, t] = src[t, h, d]. A
// work-group moves a 64-token x 64-column tile of one head through LDS, so
// both the reads (along d) and the writes (along t) are contiguous.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void out_transpose_kernel(TransposeArgs a) {
  __shared__ T tile[64][64 + 1];
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, h = blockIdx.z;
  const T *src = (const T *)a.src;
  T *dst = (T *)a.dst;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // read rows t0 + ty + 4i, columns d0 + tx
    const int t = t0 + ty + 4 * i, d = d0 + tx;
    if (t < a.n && d < a.d) tile[ty + 4 * i][tx] = src[(int64_t)t * a.s_st + (int64_t)h * a.s_sh + d];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // write rows d0 + ty + 4i of head h, columns t0 + tx
    const int d = d0 + ty + 4 * i, t = t0 + tx;
    if (t < a.n && d < a.d) dst[((int64_t)h * a.d + d) * a.n + t] = tile[tx][ty + 4 * i];
  }
}

hipError_t launch_out_transpose(const TransposeArgs &a, hipStream_t s) {
  if (a.n == 0 || a.h == 0) return hipSuccess;
  dim3 grid((unsigned)((a.n + 63) / 64), (unsigned)((a.d + 63) / 64), (unsigned)a.h);
  if (a.esize == 2) hipLaunchKernelGGL(out_transpose_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(out_transpose_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// R-way merge (AWS NKI "Attention KV-Parallel Segmented CTE", Background:
// the partials of the ranks are combined by online softmax):
//   lse = m + log(sum_i exp(lse_i - m)),  out = sum_i exp(lse_i - lse) out_i
// ---------------------------------------------------------------------------
// One workgroup streams one row (all heads) at a time; with a.cu set, rows of
// no document, or outside the view, are left as they are.
template <int D, typename OT>
__global__ __launch_bounds__(256) void merge_n_kernel(MergeNArgs a) {
  constexpr int G = D / 4;     // lanes per (row, head)
  constexpr int HP = 256 / G;  // heads per pass
  const int sub = threadIdx.x % G, hl = threadIdx.x / G;
  const int H = (int)a.h;
  for (int64_t row = blockIdx.x; row < a.n; row += gridDim.x) {
    if (a.cu) {
      if (a.num_seqs <= 0 || row < a.cu[0] || row >= a.cu[a.num_seqs]) continue;
      if (!row_in_view(a.cu, a.num_seqs, a.view, row)) continue;
    }
    for (int h = hl; h < H; h += HP) {
      const int64_t li = (int64_t)h * a.n + row;
      // part i: explicit pointers, or (strided) part 0 advanced by i strides
      auto plse = [&](int i) -> float {
        return a.strided ? a.plse[0][li + i * a.lse_stride] : a.plse[i][li];
      };
      // the G lanes of (row, head) share the parts: lane `sub` reads the lse
      // of parts sub, sub + G, ...; max and sum are reduced over the group
      float mx = neg_inf();
      for (int i = sub; i < a.n_parts; i += G) mx = fmaxf(mx, plse(i));
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, G));
      f32x4 acc = f32x4{};
      float ln = neg_inf();
      if (mx != neg_inf()) {
        float z = 0.f;
        for (int i = sub; i < a.n_parts; i += G) z += expf(plse(i) - mx);
#pragma unroll
        for (int o = G / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, G);
        ln = mx + logf(z);
        const int base = threadIdx.x & 63 & ~(G - 1);  // the group's first lane in the wave
        for (int i0 = 0; i0 < a.n_parts; i0 += G) {
          const float mine = i0 + sub < a.n_parts ? expf(plse(i0 + sub) - ln) : 0.f;
          // parts of weight 0 are not read: a forward part that saw no key
          // leaves its out unwritten
          uint64_t nz = (__ballot(mine != 0.f) >> base) & (G == 64 ? ~0ull : ((1ull << G) - 1));
          while (nz) {
            const int b = __builtin_ctzll(nz);
            nz &= nz - 1;
            const float wgt = __shfl(mine, b, G);
            const int i = i0 + b;
            const int pi = a.strided ? 0 : i;
            const int64_t off = a.strided ? i * a.out_stride : 0;
            f32x4 v = a.pdtype[pi] == 0
                          ? ld4<bf16>((const bf16 *)a.pout[pi] + off + row * a.p_st[pi] + h * a.p_sh[pi] + 4 * sub)
                          : ld4<float>((const float *)a.pout[pi] + off + row * a.p_st[pi] + h * a.p_sh[pi] + 4 * sub);
            acc += wgt * v;
          }
        }
      }
      st4<OT>((OT *)a.out + row * a.o_st + h * a.o_sh + 4 * sub, acc);
      if (sub == 0) a.lse[li] = ln;
    }
  }
}

hipError_t launch_merge_n(const MergeNArgs &a, hipStream_t s) {
  if (a.n * a.h == 0) return hipSuccess;
  const unsigned grid = row_grid(a.n);
  if (a.d == 128) {
    if (a.out_dtype == 0) hipLaunchKernelGGL((merge_n_kernel<128, bf16>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge_n_kernel<128, float>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (a.out_dtype == 0) hipLaunchKernelGGL((merge_n_kernel<64, bf16>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge_n_kernel<64, float>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// delta[h, i] = sum_d dout[i,h,d] * out[i,h,d] with the merged out (NeMo
// AutoModel zigzag_ring_attention, `zigzag_ring_flash_attn_varlen_backward`:
// every block's backward sees the final merged out, so this row term is the
// same for all blocks and is computed once).
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void ld8(const T *p, float (&v)[8]);
template <> __device__ __forceinline__ void ld8<bf16>(const bf16 *p, float (&v)[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}
template <> __device__ __forceinline__ void ld8<float>(const float *p, float (&v)[8]) {
  const f32x4 x = *reinterpret_cast<const f32x4 *>(p), y = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = x[i]; v[4 + i] = y[i]; }
}
template <typename T> __device__ __forceinline__ void ld8s(const T *p, float (&v)[8]);  // streaming
template <> __device__ __forceinline__ void ld8s<bf16>(const bf16 *p, float (&v)[8]) {
  const bf16x8 x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}
template <> __device__ __forceinline__ void ld8s<float>(const float *p, float (&v)[8]) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = x[i]; v[4 + i] = y[i]; }
}
// 8 values to f16 (one 16-byte streaming store); false when one does not fit f16
__device__ __forceinline__ bool st8_f16(f16 *p, const float (&v)[8]) {
  f16x8 h;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ok &= fabsf(v[i]) <= 65504.f;
    h[i] = (f16)v[i];
  }
  __builtin_nontemporal_store(__builtin_bit_cast(i32x4, h), reinterpret_cast<i32x4 *>(p));
  return ok;
}

// One workgroup streams one row (all heads) at a time; a group of D/8 lanes
// owns one head (8 elements a lane), NB passes' loads in flight.
// H16: also the f16 copies of q and dout for the dK/dV kernel (bf16 inputs),
// in the same pass over dout.
template <int D, typename T1, typename T2, bool H16>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int G = D / 8;
  constexpr int HP = 256 / G;
  constexpr int NB = 2;
  const int sub = threadIdx.x % G, hl = threadIdx.x / G;
  const int H = (int)a.h;
  bool fits = true;
  for (int64_t row = blockIdx.x; row < a.n; row += gridDim.x) {
    const T1 *xr = (const T1 *)a.dout + row * a.do_st + 8 * sub;
    const T2 *yr = (const T2 *)a.out + row * a.o_st + 8 * sub;
    for (int hb = 0; hb < H; hb += NB * HP) {
      float x[NB][8], y[NB][8], z[NB][8];
#pragma unroll
      for (int k = 0; k < NB; ++k) {  // clamped, unguarded: every pass's loads in flight at once
        const int h = min(hb + k * HP + hl, H - 1);
        ld8s<T1>(xr + h * a.do_sh, x[k]);
        ld8s<T2>(yr + h * a.o_sh, y[k]);
        if constexpr (H16) ld8s<bf16>((const bf16 *)a.q + row * a.q_st + h * a.q_sh + 8 * sub, z[k]);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int h = hb + k * HP + hl;
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v = __builtin_fmaf(x[k][i], y[k][i], v);
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (h < H && sub == 0) a.delta[(int64_t)h * a.n + row] = v;
        if constexpr (H16) {
          if (h < H) {
            const int64_t o16 = (row * H + h) * D + 8 * sub;
            fits &= st8_f16((f16 *)a.do16 + o16, x[k]);
            fits &= st8_f16((f16 *)a.q16 + o16, z[k]);
          }
        }
      }
    }
  }
  if constexpr (H16)
    if (!fits) *a.h16_flag = 1;
}

template <int D>
static void launch_delta_d(const DeltaArgs &a, hipStream_t s, unsigned grid) {
  const bool h16 = a.q16 != nullptr;  // bf16 q and dout only (checked by the caller)
  if (a.dtype_do == 0 && a.dtype_o == 0) {
    if (h16) hipLaunchKernelGGL((delta_kernel<D, bf16, bf16, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<D, bf16, bf16, false>), dim3(grid), dim3(256), 0, s, a);
  } else if (a.dtype_do == 0) {
    if (h16) hipLaunchKernelGGL((delta_kernel<D, bf16, float, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((delta_kernel<D, bf16, float, false>), dim3(grid), dim3(256), 0, s, a);
  } else if (a.dtype_o == 0) {
    hipLaunchKernelGGL((delta_kernel<D, float, bf16, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((delta_kernel<D, float, float, false>), dim3(grid), dim3(256), 0, s, a);
  }
}

hipError_t launch_delta(const DeltaArgs &a, hipStream_t s) {
  if (a.n * a.h == 0) return hipSuccess;
  const unsigned grid = row_grid(a.n);
  if (a.d == 128) launch_delta_d<128>(a, s, grid);
  else launch_delta_d<64>(a, s, grid);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Zig-zag shard (NeMo AutoModel zigzag_ring_attention, module docstring and
// `get_half_index`): per document of L rows and chunk c = L / (2 cp), local
// row t of rank r is global row  start + r*c + t            (t <  c)
//                                start + (2cp-1-r)*c + t - c  (t >= c).
// One wave copies one local row (all heads) in 16-byte pieces.
// ---------------------------------------------------------------------------
struct ShardParams {
  const char *src; int64_t s_st, s_sh;
  char *dst; int64_t d_st, d_sh;
  int32_t eb; int64_t heads, row_bytes;
  const int32_t *cu; int32_t cp, rank;
  int64_t n_src, n_dst;
};

__global__ __launch_bounds__(256) void zigzag_shard_kernel(ShardParams p) {
  const int doc = blockIdx.y;
  const int64_t gs = p.cu[doc], ge = p.cu[doc + 1];
  const int64_t L = ge - gs;
  const int64_t c = L / (2 * p.cp);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= 2 * c) return;
  const int64_t grow = t < c ? gs + p.rank * c + t : gs + (2 * p.cp - 1 - p.rank) * c + (t - c);
  const int64_t lrow = gs / p.cp + t;
  if (grow < 0 || grow >= p.n_src || lrow < 0 || lrow >= p.n_dst) return;
  const int lane = threadIdx.x & 63;
  const int64_t per_head = p.row_bytes / p.heads;  // bytes of one head (D * eb)
  for (int64_t off = lane * 16; off < p.row_bytes; off += 64 * 16) {
    const int64_t hh = off / per_head, dd = off - hh * per_head;
    const char *s = p.src + (grow * p.s_st + hh * p.s_sh) * p.eb + dd;
    char *d = p.dst + (lrow * p.d_st + hh * p.d_sh) * p.eb + dd;
    st16(d, ld16(s));
  }
}

hipError_t launch_zigzag_shard(const void *src, int64_t s_st, int64_t s_sh, int64_t n_src, void *dst,
                               int64_t d_st, int64_t d_sh, int64_t n_dst, int32_t elem_bytes,
                               int64_t heads, int64_t head_dim, const int32_t *cu, int32_t num_seqs,
                               int32_t max_seqlen, int32_t cp, int32_t rank, hipStream_t s) {
  if (num_seqs <= 0) return hipSuccess;
  ShardParams p{(const char *)src, s_st, s_sh, (char *)dst, d_st, d_sh, elem_bytes, heads,
                heads * head_dim * elem_bytes, cu, cp, rank, n_src, n_dst};
  const int64_t max_local = max_seqlen / cp;  // 2c for the longest document
  const unsigned gx = (unsigned)((max_local + 3) / 4);
  if (gx == 0) return hipSuccess;
  hipLaunchKernelGGL(zigzag_shard_kernel, dim3(gx, (unsigned)num_seqs), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Paged-cache gather (NKI KV-parallel prefill's block_table, Parameters): the
// logical key row t of a paged cache sits at page table[t >> shift], row
// t & (2^shift - 1) of it. One wave copies one logical row (all heads, K and V)
// into contiguous [rows, H, D] buffers; rows of an invalid page read as zero.
// With a visible range (a.cu set) only the rows some query can see are copied.
// ---------------------------------------------------------------------------
__device__ void page_gather_run(const PageGatherArgs &a) {
  const int lane = threadIdx.x & 63;
  const int64_t per_head = (int64_t)a.d * a.eb;
  const int64_t row_bytes = per_head * a.h;
  // a row is row_bytes / 16 pieces of 16 bytes; short rows share a wave
  const int chunks = (int)(row_bytes / 16);
  int lpr = 64;  // lanes per row
  while (lpr > 1 && lpr / 2 >= chunks) lpr >>= 1;
  const int rpw = 64 / lpr;  // rows per wave
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * 4 * rpw;
  for (int64_t t = wave * rpw + lane / lpr; t < a.n_rows; t += step) {
    if (a.cu) {  // rows no query of the call sees are left alone (nothing reads them)
      if (a.num_seqs <= 0 || t < a.cu[0] || t >= a.cu[a.num_seqs]) continue;
      int lo = 0, hi = a.num_seqs;  // cu[lo] <= t < cu[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= t) lo = mid; else hi = mid;
      }
      const int64_t tl = t - a.cu[lo];
      if (tl < a.t_lo || tl >= a.t_hi) continue;
    }
    const int64_t b = t >> a.shift;
    const int64_t pg = b < a.max_blocks ? a.table[b] : -1;
    const bool ok = pg >= 0 && pg < a.n_pages;
    const int64_t prow = t & ((1 << a.shift) - 1);
    for (int c = lane % lpr; c < chunks; c += lpr) {
      const int64_t off = (int64_t)c * 16;
      const int64_t hh = off / per_head, dd = off - hh * per_head;
      const int64_t so = (pg * a.page_stride + hh * a.sh + prow * a.st) * a.eb + dd;
      const int64_t dof = t * row_bytes + off;
      i32x4 vk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (ok) {
        vk = ld16((const char *)a.src_k + so);
        vv = ld16((const char *)a.src_v + so);
      }
      st16((char *)a.dst_k + dof, vk);
      st16((char *)a.dst_v + dof, vv);
    }
  }
}

__global__ __launch_bounds__(256) void page_gather_kernel(PageGatherArgs a) { page_gather_run(a); }

// several gathers (the ranks of a KV-parallel call), grid.y = gather
struct PageGatherBatch {
  PageGatherArgs a[kMaxGatherBatch];
};
__global__ __launch_bounds__(256) void page_gather_batch_kernel(PageGatherBatch b) { page_gather_run(b.a[blockIdx.y]); }

// ---------------------------------------------------------------------------
// Zero the gradient rows a backward that stores (instead of adding) does not
// write. grid.y = tensor; a workgroup takes 64 rows at a time, 16-byte stores.
struct ZeroRowsBatch {
  ZeroRows a[kMaxZeroRows];
  const int32_t *cu;
  int32_t num_seqs;
};

// row is written by a block with this view: inside a document, in the view
__device__ __forceinline__ bool row_covered(const int32_t *cu, int32_t num_seqs, int view, int64_t row) {
  if (view == 3 || num_seqs <= 0 || row < cu[0] || row >= cu[num_seqs]) return false;
  return view == 0 || row_in_view(cu, num_seqs, view, row);
}

constexpr int kZeroRowsChunk = 64;  // rows a workgroup decides at once (one per lane of wave 0)

__global__ __launch_bounds__(256) void zero_rows_kernel(ZeroRowsBatch b) {
  const ZeroRows &a = b.a[blockIdx.y];
  const int per_row = a.h * a.d / 4;  // float4 pieces
  __shared__ int32_t s_zero[kZeroRowsChunk];
  __shared__ int32_t s_any;
  for (int64_t r0 = (int64_t)blockIdx.x * kZeroRowsChunk; r0 < a.n; r0 += (int64_t)gridDim.x * kZeroRowsChunk) {
    // the lanes of wave 0 search their rows' documents side by side
    if (threadIdx.x < kZeroRowsChunk) {
      const int64_t row = r0 + threadIdx.x;
      const bool z = row < a.n && !row_covered(b.cu, b.num_seqs, a.view, row);
      s_zero[threadIdx.x] = z ? 1 : 0;
      const unsigned long long any = __ballot(z);
      if (threadIdx.x == 0) s_any = any != 0ull ? 1 : 0;
    }
    __syncthreads();
    if (s_any) {
      for (int j = threadIdx.x; j < kZeroRowsChunk * per_row; j += 256) {
        const int rr = j / per_row, pc = j - rr * per_row;
        if (!s_zero[rr]) continue;
        const int hh = (4 * pc) / a.d, dd = 4 * pc - hh * a.d;
        *reinterpret_cast<float4 *>(a.t + (r0 + rr) * a.st + hh * a.sh + dd) = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    __syncthreads();
  }
}

hipError_t launch_zero_rows(const ZeroRows *a, int n, const int32_t *cu, int32_t num_seqs, hipStream_t s) {
  if (n < 1 || n > kMaxZeroRows) return hipErrorInvalidValue;
  ZeroRowsBatch zb{};
  int64_t rows = 0;
  for (int i = 0; i < n; ++i) {
    zb.a[i] = a[i];
    if (a[i].n > rows) rows = a[i].n;
  }
  zb.cu = cu;
  zb.num_seqs = num_seqs;
  if (rows <= 0) return hipSuccess;
  int64_t g = (rows + kZeroRowsChunk - 1) / kZeroRowsChunk;
  if (g > 2048) g = 2048;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)g, (unsigned)n), dim3(256), 0, s, zb);
  return hipGetLastError();
}

// workgroups for a gather: 4 waves of rows_per_wave rows each (as page_gather_run)
static int64_t gather_blocks(const PageGatherArgs &a) {
  const int chunks = (int)((int64_t)a.d * a.eb * a.h / 16);
  int lpr = 64;
  while (lpr > 1 && lpr / 2 >= chunks) lpr >>= 1;
  const int64_t rows = 4 * (64 / lpr);
  return (a.n_rows + rows - 1) / rows;
}

hipError_t launch_page_gather(const PageGatherArgs &a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  int64_t b = gather_blocks(a);
  if (b > 256 * 16) b = 256 * 16;
  hipLaunchKernelGGL(page_gather_kernel, dim3((unsigned)b), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_page_gathers(const PageGatherArgs *a, int n, hipStream_t s) {
  if (n < 1 || n > kMaxGatherBatch) return hipErrorInvalidValue;
  PageGatherBatch pb{};
  for (int i = 0; i < n; ++i) pb.a[i] = a[i];
  if (a[0].n_rows <= 0) return hipSuccess;
  int64_t b = gather_blocks(a[0]);
  if (b * n > 256 * 16) b = (256 * 16 + n - 1) / n;
  hipLaunchKernelGGL(page_gather_batch_kernel, dim3((unsigned)b, (unsigned)n), dim3(256), 0, s, pb);
  return hipGetLastError();
}

}  // namespace attn
