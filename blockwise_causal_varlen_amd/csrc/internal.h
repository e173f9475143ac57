// Declarations shared between the host library and the kernel translation
// units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace attn {

// One unit of forward/backward work: a tile of query rows of one document
// against the keys [k0, k1) it can see (already intersected with the key
// view, the segment and the causal/window bounds).
struct WorkItem {
  int32_t q0, q1;      // absolute query rows [q0, q1)
  int32_t k0, k1;      // absolute (logical) key rows [k0, k1)
  int32_t qdoc0;       // first query row of the document
  int32_t kdoc0;       // first key row of the document
  int32_t seg;         // segment index (0 when not segmented)
  int32_t cost;        // key tiles + 1, the sort key
  int32_t qmid;        // first row of the document's back half
};

// Device view of the visibility rule.
struct MaskDev {
  int32_t causal;
  int32_t q_view, k_view;
  int32_t seg_size;
  int64_t window;
  int64_t q_pos_offset;
  PosMap pm;
};

struct TensorDev {
  const void *data;
  int64_t st, sh;  // token / head strides in elements
};

// Tile-scheduler output layout inside a workspace.
struct SchedBufs {
  WorkItem *items;
  int32_t *order;
  int32_t *count;
  int32_t capacity;
};

constexpr int kFwdBM = 128;   // query rows per forward workgroup (4 waves x 32)
constexpr int kFwdBN = 64;    // keys per staged tile of the f32 forward and the dQ kernels; the
                              // schedule's unit of key parts and costs
// keys per staged tile of the bf16 forward: 32 lets three workgroups share a
// CU (LDS 38 KB each)
constexpr int kFwdBf16BN = 32;
constexpr int kBwdBQ = 64;    // query rows per staged tile of the dK/dV kernel
constexpr int kBwdTile = 128; // query rows per dQ workgroup / key rows per dK-dV workgroup

size_t sched_bytes(int64_t capacity);
SchedBufs sched_carve(void *ws, int64_t capacity);
int64_t sched_capacity(int64_t n_rows_view_bound, int32_t num_seqs, int32_t tile, int64_t n_seg);

// One schedule: the work items of a (cu_q, cu_k, mask) problem, sorted by cost.
struct SchedJob {
  const int32_t *cu_q, *cu_k;
  int32_t num_seqs;
  int64_t n_q, n_k;
  MaskDev m;
  int32_t tile, key_tile;
  int32_t by_keys;  // 0: tiles of query rows; 1: tiles of key rows (dK/dV)
  int32_t max_seg;  // parts the partial buffers hold per query tile
  SchedBufs sb;
  int32_t nsplit = 0;  // > 1 (query tiles, no segments): cut each tile's visible keys in nsplit parts
};
constexpr int kMaxSchedJobs = 8;
// n (<= kMaxSchedJobs) independent schedules in one launch
hipError_t launch_schedules(const SchedJob *jobs, int n, hipStream_t s);

hipError_t launch_schedule(const int32_t *cu_q, const int32_t *cu_k, int32_t num_seqs,
                           int64_t n_q, int64_t n_k, const MaskDev &m, int32_t tile,
                           int32_t key_tile, int32_t by_keys, int32_t max_seg, SchedBufs sb, hipStream_t s,
                           int32_t nsplit = 0);

struct FwdArgs {
  TensorDev q, k, v;
  int32_t dtype;         // 0 bf16, 1 f32 (q/k/v)
  int32_t head_dim;
  int32_t hq, hkv;
  float scale;
  MaskDev mask;
  // outputs: either final (out/lse) or segment partials (part_*)
  void *out; int32_t out_dtype; int64_t o_st, o_sh;
  float *lse; int64_t lse_n;    // lse[h * lse_n + row]
  float *part_out;              // [n_seg][n_q][HQ][D] f32 when segmented
  float *part_lse;              // [n_seg][HQ][n_q]
  int64_t n_q;
  SchedBufs sched;
  int64_t grid_items;           // scheduler capacity (grid bound)
  // Running-state mode (bf16 tiled forward only), when acc is set: `lse` is
  // the running lse; merge: combine the block with (acc, lse) first (else the
  // block initialises them); rows of the halves in final_view (bit 0 front,
  // bit 1 back) go to `out`, the others to acc (f32)
  float *acc = nullptr; int64_t a_st = 0, a_sh = 0;
  int32_t merge = 0, final_view = 0;
};
hipError_t launch_fwd(const FwdArgs &a, hipStream_t s);
// up to kMaxFwdBatch bf16 forwards of one shape (head_dim, hq, out dtype,
// masked or not, schedule capacity) in one launch
constexpr int kMaxFwdBatch = 8;
bool fwd_batchable(const FwdArgs *a, int n);
hipError_t launch_fwd_batch(const FwdArgs *a, int n, hipStream_t s);

struct DecodeArgs {
  TensorDev q, k, v;
  int32_t head_dim, hq, hkv, num_seqs;
  float scale;
  const int32_t *cu_q, *cu_k;
  void *out; int32_t out_dtype; int64_t o_st, o_sh;
  float *lse; int64_t lse_n;
  int64_t n_k;
  int32_t n_split = 1, split_len = 0;      // split KV (flash-decoding) when n_split > 1
  float *part_out = nullptr, *part_lse = nullptr;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_split_merge(const DecodeArgs &a, hipStream_t s);

struct MergeArgs {
  float *out; int64_t o_st, o_sh;          // running f32 state
  float *lse;
  const void *bout; int32_t bout_dtype; int64_t b_st, b_sh;
  const float *blse;
  float *weight;                            // nullable
  void *fout; int32_t fout_dtype; int64_t f_st, f_sh;  // nullable
  const int32_t *cu; int32_t num_seqs; int32_t view;
  int64_t n, h, d;
  int32_t init;
};
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);

struct MergeNArgs {
  int32_t n_parts;
  int32_t strided;                 // parts = part 0 + i * (out_stride, lse_stride)
  int64_t out_stride, lse_stride;  // elements
  const void *pout[16]; int32_t pdtype[16]; int64_t p_st[16], p_sh[16];
  const float *plse[16];
  void *out; int32_t out_dtype; int64_t o_st, o_sh;
  float *lse;
  int64_t n, h, d;
  // non-null cu: only rows of the documents (in `view` of each) are written
  const int32_t *cu = nullptr; int32_t num_seqs = 0, view = 0;
};
hipError_t launch_merge_n(const MergeNArgs &a, hipStream_t s);

// Copy of the logical rows [0, n_rows) of paged K and V caches into
// contiguous [n_rows, h, d] buffers (strides in elements, eb bytes an element).
struct PageGatherArgs {
  const void *src_k, *src_v;
  int64_t page_stride, st, sh;
  const int32_t *table;
  int64_t max_blocks, n_pages;
  int32_t shift;
  void *dst_k, *dst_v;
  int64_t n_rows;
  int32_t h, d, eb;
  // when cu is set, only the rows whose document-local index lies in
  // [t_lo, t_hi) are copied (cu: the documents' first logical key rows)
  const int32_t *cu;
  int32_t num_seqs;
  int64_t t_lo, t_hi;
};
hipError_t launch_page_gather(const PageGatherArgs &a, hipStream_t s);
constexpr int kMaxGatherBatch = 16;
// n (<= kMaxGatherBatch) gathers of equal row counts in one launch
hipError_t launch_page_gathers(const PageGatherArgs *a, int n, hipStream_t s);

struct DeltaArgs {
  const void *dout; int32_t dtype_do; int64_t do_st, do_sh;
  const void *out; int32_t dtype_o; int64_t o_st, o_sh;
  float *delta;
  int64_t n, h, d;
  // optional, bf16 q and dout only: also write their f16 copies ([n, h, d]
  // contiguous) and set *h16_flag where a value does not fit f16 (the flag is
  // zeroed before, by launch_lse2)
  const void *q = nullptr; int64_t q_st = 0, q_sh = 0;
  void *q16 = nullptr, *do16 = nullptr;
  int32_t *h16_flag = nullptr;
};
hipError_t launch_delta(const DeltaArgs &a, hipStream_t s);

// EAGLE-3 test-time-training diagonal blocks: row t of q head h sees the one
// key k[t, h / group] of the block (forward merge and closed-form backward).
struct DiagArgs {
  const void *q, *k, *v;
  int32_t dtype;  // of q, k, v (and dout)
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  float *out; int64_t o_st, o_sh;  // f32 running output (forward)
  float *lse;                      // [HQ, n]
  void *fout; int32_t fout_dtype; int64_t f_st, f_sh;
  const void *dout; int64_t do_st, do_sh;
  const float *delta;
  float *dq; int64_t dq_st, dq_sh;
  float *dk; int64_t dk_st, dk_sh;
  float *dv; int64_t dv_st, dv_sh;
  int32_t n, hq, group, d;
  float scale;
};
hipError_t launch_diag_merge(const DiagArgs &a, hipStream_t s);

// Ulysses all-to-all between virtual ranks: sequence shards <-> head shards.
constexpr int kMaxUly = 16;
struct ReshardArgs {
  const char *src[kMaxUly]; int64_t s_st[kMaxUly], s_sh[kMaxUly];  // strides in bytes
  char *dst[kMaxUly]; int64_t d_st[kMaxUly], d_sh[kMaxUly];
  int32_t uly, to_heads, row_bytes, n_local, h_local;
};
hipError_t launch_reshard(const ReshardArgs &a, hipStream_t s);
struct LseReshardArgs {
  const float *src[kMaxUly];
  float *dst[kMaxUly];
  int32_t uly, to_heads, n_local, h_local;
};
hipError_t launch_lse_reshard(const LseReshardArgs &a, hipStream_t s);

// [KVP] `tp_out`: dst[h, d, t] = src[t, h, d] (contiguous [H, D, n] destination).
struct TransposeArgs {
  const void *src; int64_t s_st, s_sh;  // elements
  void *dst;
  int32_t esize, n, h, d;
};
hipError_t launch_out_transpose(const TransposeArgs &a, hipStream_t s);
hipError_t launch_diag_bwd(const DiagArgs &a, hipStream_t s);

struct BwdArgs {
  TensorDev q, k, v, dout;
  int32_t dtype;
  int32_t head_dim, hq, hkv;
  float scale;
  MaskDev mask;
  const float *lse, *delta;
  const float *lse2;  // lse * log2(e), +inf for -inf (launch_lse2)
  int64_t n_q, n_k;
  float *dq; int64_t dq_st, dq_sh;
  float *dk; int64_t dk_st, dk_sh;
  float *dv; int64_t dv_st, dv_sh;
  SchedBufs qsched;   // tiles of query rows (dQ kernel)
  SchedBufs ksched;   // tiles of key rows (dK/dV kernel)
  int64_t q_items, k_items;
  bool set_q = false, set_kv = false;  // store the gradients instead of adding to them
  // f16 copies of q and dout (launch_half_copy) and their range flag; NULL:
  // the dK/dV kernel runs on the bf16 inputs
  const void *q16 = nullptr, *do16 = nullptr;
  const int32_t *h16_flag = nullptr;
};
hipError_t launch_bwd(const BwdArgs &a, int which, hipStream_t s);  // 0: dK/dV, 1: dQ
// lse2 = lse * log2(e) (+inf where lse = -inf); also zeroes *h16_flag when given
hipError_t launch_lse2(const float *lse, float *lse2, int64_t n, hipStream_t s, int32_t *h16_flag = nullptr);
// f16 copies of bf16 q and dout [n, h, d] into contiguous buffers; sets *flag
// when a value does not fit f16 (the flag is zeroed by launch_lse2 first)
struct HalfCopyArgs {
  const void *q, *dout;
  int64_t q_st, q_sh, do_st, do_sh;
  void *q16, *do16;
  int64_t n;
  int32_t h, d;
  int32_t *flag;
};
hipError_t launch_half_copy(const HalfCopyArgs &a, hipStream_t s);

// Zero the rows of an f32 [n, h, d] tensor that a block with this view does
// not write: rows outside every document, and (view 1 / 2) the back / front
// half of each document; view 3: every row.
struct ZeroRows {
  float *t;
  int64_t st, sh, n;
  int32_t h, d, view;
};
constexpr int kMaxZeroRows = 40;
hipError_t launch_zero_rows(const ZeroRows *a, int n, const int32_t *cu, int32_t num_seqs, hipStream_t s);

hipError_t launch_zigzag_shard(const void *src, int64_t s_st, int64_t s_sh, int64_t n_src, void *dst,
                               int64_t d_st, int64_t d_sh, int64_t n_dst, int32_t elem_bytes,
                               int64_t heads, int64_t head_dim, const int32_t *cu, int32_t num_seqs,
                               int32_t max_seqlen, int32_t cp, int32_t rank, hipStream_t s);


}  // namespace attn
