// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, lane-layout helpers and the key-position map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// 32x32 MFMA with f32 accumulation. Lane l supplies row (l % 32) of A and
// column (l % 32) of B; the lane group l / 32 supplies its own KV consecutive
// k-slots. The result C[m][n] is held by lane n + 32 * ((m / 4) % 2) in
// register (m / 8) * 4 + m % 4. (Checked on gfx950 against a CPU product.)
// ---------------------------------------------------------------------------
template <typename T> struct Mfma32;

template <> struct Mfma32<bf16> {
  static constexpr int KV = 8;  // elements per lane per instruction (k = 16)
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma32<f16> {
  static constexpr int KV = 8;  // elements per lane per instruction (k = 16)
  typedef f16x8 Frag;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma32<float> {
  static constexpr int KV = 1;  // k = 2
  typedef float Frag;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Key (row) index within a 32x32 result tile held in register j of lane l.
__device__ __forceinline__ int c_row(int j, int lane) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of a value and the one held by lane l ^ 32, in both lanes: one
// v_permlane32_swap hands each half of the wave the other half's values (no
// LDS round trip). Both lanes add in the same order, so they agree exactly.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ i32x4 ld16(const void *p) { return *reinterpret_cast<const i32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, i32x4 v) { *reinterpret_cast<i32x4 *>(p) = v; }

// ---------------------------------------------------------------------------
// Key position map (the visibility rule of the C ABI):
//   kpos = k_pos_offset + t                                   (contiguous)
//   kpos = k_pos_offset + ((t / B) * R + r) * B + t % B       (round robin)
// t is the index of the key inside its document's key buffer. The map is
// strictly increasing in t, which the tile bounds rely on.
// ---------------------------------------------------------------------------
// Logical work-group index. Work-groups go to the chip's 8 XCDs round-robin;
// this gives each XCD one contiguous range of logical indices, so work-groups
// that read the same key/value rows run on one XCD and share its L2.
__device__ __forceinline__ int xcd_block() {
  const int b = blockIdx.x, n = gridDim.x;
  if (n % 8) return b;
  return (b % 8) * (n / 8) + b / 8;
}

struct PosMap {
  int64_t k_pos_offset;
  int32_t interleave;  // R (0 = contiguous)
  int32_t rank;
  int32_t block;       // B
  int32_t shift;       // log2(B) (B is a power of two when R > 0)
  __host__ __device__ __forceinline__ int64_t kpos(int64_t t) const {
    if (interleave == 0) return k_pos_offset + t;
    int64_t b = t / block, o = t - b * block;
    return k_pos_offset + (b * interleave + rank) * block + o;
  }
  // Branch-free 32-bit form for per-element masks (t, positions < 2^31 within
  // one document's window of interest; the offset is applied in 64 bits).
  __device__ __forceinline__ int64_t kpos32(int32_t t) const {
    if (interleave == 0) return k_pos_offset + t;  // uniform branch
    const int32_t b = t / block;
    return k_pos_offset + ((b * interleave + rank) * block + (t - b * block));
  }
  // Number of keys t in [0, n) with kpos(t) <= p (monotone inverse).
  __host__ __device__ __forceinline__ int64_t count_le(int64_t p, int64_t n) const {
    int64_t lo = 0, hi = n;  // answer in [lo, hi]
    while (lo < hi) {
      int64_t mid = (lo + hi) >> 1;
      if (kpos(mid) <= p) lo = mid + 1; else hi = mid;
    }
    return lo;
  }
};

// ---------------------------------------------------------------------------
// Padded bf16 LDS tiles of 64 rows filled by direct global->LDS copies.
// A row is PCH 16-byte chunks: D/8 data chunks + padding. The pitches used:
//   D/8 + 1 chunks: 16-byte row reads of 16 rows hit 16 distinct bank groups;
//   D/8 + 4 chunks: 4-row transpose reads of 64 bytes hit distinct banks;
//   D/8 + 5 chunks: both patterns, the transpose reads at most 2-way.
// A copy instruction moves 64 consecutive 16-byte slots (lane l -> slot
// base + l), so slot s is (row s / PCH, chunk s % PCH); pad slots are given an
// offset past the buffer range and read as zeros.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// ROWS = 64 or 32. The copies write whole 1 KB blocks, so a tile of 32 rows
// whose slots do not fill its last block is given room for all of it.
template <int D, int PCH, int ROWS = 64> struct PadTile {
  static constexpr int CPR = D / 8;                     // data chunks per row
  static constexpr int SPR = PCH;                       // slots per row
  static constexpr int NROWS = ROWS;
  static constexpr int NBLK = (ROWS * PCH + 63) / 64;   // 1 KB blocks
  static constexpr int NJ = (NBLK + 3) / 4;             // blocks per wave (4 waves)
  static constexpr int PITCH = PCH * 8;                 // elements per row
  static constexpr int ELEMS = NBLK * 512;              // elements of the buffer
  static constexpr bool kSwz = false;
};

// Swizzled tile of 64 rows x 128 bf16 (16 chunks a row, no padding): row r
// keeps its logical chunk c in physical chunk c ^ swz128(r), with
// swz128(r) = 4 (r mod 4) + (r / 4 mod 4). With 64 banks of 4 bytes a row is
// one pass over all banks, and a physical chunk is 4 banks. A b128 read pass
// (16 lanes: 16 consecutive rows, one chunk) then sees 16 distinct swizzles,
// and a transpose read pass (32 lanes: 4 aligned rows x 4 aligned chunks)
// puts each row in its own quarter of the chunks: both are conflict free,
// where a padded pitch can serve only one of the two patterns.
struct SwzTile128 {
  static constexpr int CPR = 16, SPR = 16, NROWS = 64, NBLK = 16, NJ = 4, PITCH = 128, ELEMS = 64 * PITCH;
  static constexpr bool kSwz = true;
};
__device__ __forceinline__ int swz128(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Per-lane element offsets into a SwzTile128. Row reads: row l32 (+ a
// multiple of 16 rows, added by the caller), logical chunk 2 st + g.
template <int NS>
__device__ __forceinline__ void swz_row_offsets(int (&ro)[NS], int lane) {
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int st = 0; st < NS; ++st) ro[st] = l32 * 128 + (((2 * st + g) ^ swz128(l32)) << 3);
}
// Transpose reads of d-tile dt: the lane's 16-lane group u = lane % 16 names
// row 4 g + u / 4 (lo; + 8 for hi) of a 16-row block and columns
// 32 dt + 16 dh + 4 (u % 4).. (dh = lane / 16 % 2).
template <int ND>
__device__ __forceinline__ void swz_tr_offsets(int (&lo)[ND], int (&hi)[ND], int lane) {
  const int g = lane >> 5, u = lane & 15, dh = (lane >> 4) & 1;
  const int sl = 4 * (u >> 2) + g, sh = sl ^ 2;  // swizzles of the lo and hi rows
  const int rl = (4 * g + (u >> 2)) * 128;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    const int c = dt * 4 + dh * 2 + ((u & 3) >> 1);
    lo[dt] = rl + ((c ^ sl) << 3) + 4 * (u & 1);
    hi[dt] = rl + 8 * 128 + ((c ^ sh) << 3) + 4 * (u & 1);
  }
}

constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kPastEnd = 0x40000000;   // a byte offset beyond any tile resource

// Bytes of a tile resource covering its valid rows (rows past the end read 0).
__device__ __forceinline__ int tile_bytes(int64_t st, int nvalid, int d) {
  return nvalid > 0 ? (int)(((int64_t)(nvalid - 1) * st + d) * 2) : 0;
}

// Per-lane byte offsets (inside a tile, row stride st elements) of this
// wave's copy instructions.
template <class TT>
__device__ __forceinline__ void tile_voffsets(int *voff, int64_t st, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < TT::NJ; ++j) {
    const int blk = wave + 4 * j;
    const int s = blk * 64 + lane;
    const int r = s / TT::SPR, c = s % TT::SPR;
    const int cl = TT::kSwz ? (c ^ swz128(r)) : c;  // the logical chunk this slot holds
    voff[j] = (blk < TT::NBLK && r < TT::NROWS && c < TT::CPR) ? (int)(r * st * 2) + cl * 16 : kPastEnd;
  }
}

// Asynchronous tile copy through a buffer resource; completion is awaited by
// the next __syncthreads().
template <class TT>
__device__ __forceinline__ void dma_tile_buf(bf16 *lds, const bf16 *tile_row0, int bytes, const int *voff, int wave) {
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)tile_row0, (short)0, bytes, kBufFlags);
#pragma unroll
  for (int j = 0; j < TT::NJ; ++j) {
    const int blk = wave + 4 * j;
    if (blk < TT::NBLK)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(reinterpret_cast<char *>(lds) + blk * 1024), 16,
                                               voff[j], 0, 0, 0);
  }
}

// Transpose read of a padded tile (pitch in elements): the lane's 16-lane
// group u = lane % 16 supplies row r0 + u/4, columns col0 + 4*(u%4)..+3, and
// receives rows r0..r0+3 of column col0 + u.
__device__ __forceinline__ bf16x4 tile_tr4(const bf16 *t, int pitch, int r0, int col0, int u) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
  const bf16 *a = t + (r0 + (u >> 2)) * pitch + col0 + 4 * (u & 3);
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)a);
  return __builtin_bit_cast(bf16x4, v);
}

// Visibility of (query position qp, key position kp) under causal / window,
// written with bitwise ops so it compiles to selects, not branches.
__device__ __forceinline__ bool visible(int64_t qp, int64_t kp, int32_t causal, int64_t window) {
  const bool c = (causal == 0) | (kp <= qp);
  const bool w = (window <= 0) | (kp > qp - window);
  return c & w;
}

}  // namespace attn
