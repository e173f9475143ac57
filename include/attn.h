/*
 * attn.h -- C ABI of the blockwise causal varlen attention library (gfx950).
 *
 * The library computes softmax attention over packed variable-length
 * documents block by block: every block returns a partial (out, lse) pair,
 * partials are merged with the online-softmax log-sum-exp identity, and the
 * backward of every block is run against the MERGED (out, lse). Context-
 * parallel schedules (zig-zag ring, contiguous ring, KV-parallel prefill) run
 * as virtual ranks on one GPU: the blocks are produced in ring order with no
 * collectives.
 *
 * Sources (web pages, cited by title and section):
 *   [ZZ]   NeMo AutoModel API docs, "...speculative.eagle.zigzag_ring_attention"
 *   [RING] NeMo AutoModel API docs, "...speculative.eagle.ring_attention"
 *   [ULY]  NeMo AutoModel API docs, "...speculative.eagle.ulysses_attention"
 *   [KVP]  AWS Neuron NKI library, "Attention KV-Parallel Segmented CTE Kernel
 *          API Reference"
 *   [DEC]  recipes "qsa_fa_fallback.py" (SM121 fallback varlen attention)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are described by attn_tensor: a device pointer, a dtype, three
 *    sizes [n_tok, n_head, head_dim] and two strides in ELEMENTS (token and
 *    head); the last dimension must be contiguous. [ZZ]'s varlen tensors are
 *    [total, H, D] (the unit batch dimension dropped, `squeeze_batch`); the
 *    NKI query [H, S, D] ([KVP] parameter q) is the same tensor with
 *    stride_tok = D and stride_head = S*D.
 *  - lse is float32 [H, n_tok] contiguous (one layout everywhere; element
 *    (h, i) at lse[h * n_tok + i]), natural log of the sum of exp of the
 *    SCALED scores ([RING] `_CachedRingAttention`: a one-key block has
 *    lse = (Q.K) * scale). A row that sees no key has lse = -inf and out = 0
 *    ([DEC] normalisation guard).
 *  - cu_seqlens_* are DEVICE int32 arrays of num_seqs + 1 prefix sums; document
 *    d of q pairs with document d of k. max_seqlen_* are host ints: upper
 *    bounds on the per-document lengths, used only to size grids ([ZZ]
 *    `_block_forward` takes max_seqlen the same way). Device contents are not
 *    read on the host: no entry point synchronises, so all of them can be
 *    captured in a hipGraph ([DEC] module docstring: cu_seqlens read on device
 *    keep the kernel graph-replay safe). attn_validate_inputs is the one
 *    exception, and says so.
 *  - q head h reads kv head h / (HQ / HKV) ([DEC] kernel: GQA mapping).
 *  - Ownership: the caller allocates every tensor and the workspace; the
 *    library keeps no device memory between calls and never allocates or
 *    frees device memory. Calls are asynchronous on the given stream
 *    (a hipStream_t passed as void*; NULL = the null stream).
 *  - Errors: every entry point returns an attn_status and never aborts. On a
 *    non-OK status nothing was launched, except ATTN_ERR_HIP (a launch
 *    failed). attn_last_error() returns a per-thread message for the last
 *    failure.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_DTYPE = 2,       /* q/k/v dtypes differ or are unsupported */
  ATTN_ERR_SHAPE = 3,       /* head_dim or head count mismatch, bad sizes */
  ATTN_ERR_GQA = 4,         /* HQ is not a multiple of HKV */
  ATTN_ERR_CU_SEQLENS = 5,  /* num_seqs / max_seqlen inconsistent */
  ATTN_ERR_LAYOUT = 6,      /* last dim not contiguous, negative stride */
  ATTN_ERR_UNSUPPORTED = 7, /* valid but not implemented (e.g. D not 64/128) */
  ATTN_ERR_WORKSPACE = 8,   /* workspace missing or too small */
  ATTN_ERR_HIP = 9,         /* a HIP launch failed */
  ATTN_ERR_VERSION = 10,    /* struct_size does not match this library */
  ATTN_ERR_INVALID = 11,    /* other invalid argument (cp, rank, view, ...) */
  ATTN_ERR_CONTENT = 12     /* attn_validate_inputs found bad device data */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;

/* Row selection per document ([ZZ] `get_half_index`: the front (early) or
 * back (late) half of EACH varlen document). FRONT = first n/2 rows of a
 * document of n rows, BACK = the remaining rows. */
typedef enum { ATTN_VIEW_ALL = 0, ATTN_VIEW_FRONT = 1, ATTN_VIEW_BACK = 2 } attn_view;

typedef struct {
  void *data;          /* device pointer */
  int32_t dtype;       /* attn_dtype */
  int32_t reserved;
  int64_t n_tok;       /* rows (tokens); for a paged cache: pages*block_size */
  int64_t n_head;
  int64_t head_dim;
  int64_t stride_tok;  /* elements between consecutive tokens */
  int64_t stride_head; /* elements between consecutive heads */
} attn_tensor;

/*
 * Visibility of key j to query i (same document d):
 *     qpos(i) = q_pos_offset + (i - cu_seqlens_q[d])
 *     t       = j - cu_seqlens_k[d]       (index in the document's key buffer)
 *     kpos(j) = k_pos_offset + t                         if kv_interleave == 0
 *             = k_pos_offset + ((t / B) * R + kv_rank) * B + t % B   otherwise
 *               (B = block_size, R = kv_interleave: [KVP] `kvp_group_size`,
 *                rank r holds global blocks r, r+R, r+2R, ...)
 *     visible iff i in q_view, j in k_view,
 *                 (!causal or kpos <= qpos) and
 *                 (window == 0 or kpos > qpos - window)
 * The window counts visible keys including the query's own position ([KVP]
 * `sliding_window`, 0 = off; the pages do not fix the boundary, this is the
 * reading used). [KVP] `kvp_q_offset` for contiguous shards is
 * q_pos_offset - k_pos_offset here.
 *
 * Paged KV ([KVP] `k_cache`/`v_cache` [num_blocks, HKV, block_size, D] and
 * `block_tables`): when block_table != NULL the key buffer is logical; its
 * token t (t counted from the start of the k tensor, i.e. cu_seqlens_k
 * indexes logical tokens) lives in physical page block_table[t / block_size]
 * at row t % block_size. The k/v attn_tensor then describes the cache:
 * stride_tok = elements between rows of a page, stride_head = elements
 * between heads of a page, and page_stride = elements between pages.
 *
 * Segments ([KVP] `seg_size`): seg_size > 0 bounds the keys one partial
 * covers. Each 128-row query tile's visible keys are cut into n parts of
 * whole 64-key tiles, n = ceil(keys a tile can see / seg_size) (the keys a
 * tile can see: max_seqlen_k, or fewer under a window); every part is computed
 * as its own partial (out, lse) in the workspace and the partials are merged
 * before attn_block_fwd returns. The cut follows each tile's visible range
 * rather than fixed segment boundaries; the merged result is the same up to
 * rounding for any partition.
 */
typedef struct {
  uint32_t struct_size;   /* must equal sizeof(attn_mask) */
  uint32_t causal;
  uint32_t q_view;        /* attn_view */
  uint32_t k_view;        /* attn_view */
  int64_t window;         /* 0 = off */
  int64_t q_pos_offset;
  int64_t k_pos_offset;
  int32_t kv_interleave;  /* R > 0: round-robin key positions; 0: contiguous */
  int32_t kv_rank;        /* r in [0, R) */
  int32_t block_size;     /* page / round-robin block size in tokens (a power of
                             two when kv_interleave > 0 or block_table is set) */
  int32_t max_blocks;     /* entries in block_table */
  const int32_t *block_table; /* device; NULL = not paged */
  int64_t page_stride;    /* elements between pages (paged only; a multiple
                             of 16 bytes, else ATTN_ERR_LAYOUT) */
  int32_t seg_size;       /* 0 = no split */
  int32_t reserved;
} attn_mask;

/* Operation ids for attn_workspace_size. */
typedef enum { ATTN_OP_BLOCK_FWD = 0, ATTN_OP_BLOCK_BWD = 1 } attn_op;

int attn_abi_version(void);
const char *attn_status_string(attn_status s);
/* Message of the calling thread's last failure ("" if none). */
const char *attn_last_error(void);

/* Bytes of workspace attn_block_fwd / attn_block_bwd need for these sizes
 * (same arguments as the call). Host-only; never touches the device. */
attn_status attn_workspace_size(attn_op op, const attn_tensor *q, const attn_tensor *k,
                                int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const attn_mask *mask, size_t *bytes);
/* attn_workspace_bytes -- the same query under a second name (identical
 * arguments, result and errors as attn_workspace_size). */
attn_status attn_workspace_bytes(attn_op op, const attn_tensor *q, const attn_tensor *k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 const attn_mask *mask, size_t *bytes);

/*
 * attn_block_fwd -- one attention block -> (out, lse).
 * [ZZ] `_block_forward` (a flash varlen forward over one block, front/back
 * halves by per-document views), [RING] `_fa_forward` (returns out and lse),
 * [KVP] (paged, round-robin, windowed, segmented local attention), [DEC]
 * (one query row per sequence: max_seqlen_q == 1 with a full mask runs the
 * decode kernel).
 *   q   [n_q, HQ, D]   bf16 or f32
 *   k,v [n_k, HKV, D]  same dtype as q (paged: the cache, see attn_mask)
 *   out [n_q, HQ, D]   bf16 or f32; only rows in the q view are written
 *   lse [HQ, n_q] f32; only rows in the q view are written (NULL allowed
 *       when n_q == 0; the same holds for every lse / delta argument below)
 *   scale: multiplies q.k before the softmax (callers pass 1/sqrt(D) for the
 *          pages' default, [ULY] `cached_ulysses_attention` scale)
 * D must be 64 or 128. mask == NULL means full (no causal, all rows).
 * Workspace: attn_workspace_size(ATTN_OP_BLOCK_FWD, ...) bytes. It holds,
 * besides the tile schedule: the max_blocks * block_size logical rows of paged
 * K and V (gathered into contiguous rows before the forward; rows of pages
 * outside [0, n_tok / block_size) read as zero); and the partials of each
 * query tile's visible keys cut into n parts: the parts seg_size asks for,
 * and, when few 128-row query tiles face many keys (fewer than 512 tile x
 * head workgroups and max_seqlen_k >= 1024), up to 16 parts of >= 512 keys
 * of max_seqlen_k each (the larger count wins; one part needs no partials).
 * Rows outside the q view stay untouched in every case.
 */
attn_status attn_block_fwd(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                           int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const attn_mask *mask, float scale,
                           const attn_tensor *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_block_fwd_noalloc -- attn_block_fwd for callers that cannot allocate
 * device memory: code under hipGraph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments and results as attn_block_fwd,
 * without the workspace: the library keeps one device array of
 * ATTN_NOALLOC_SCRATCH_BYTES per GPU (its address looked up on the first call
 * on that GPU, held until the process ends) and never allocates or frees.
 * A call whose plan needs more workspace than the array holds (paged keys
 * with many pages, segment partials of large calls) fails with
 * ATTN_ERR_WORKSPACE before launching anything; when only the automatic key
 * split of small grids does not fit, the call runs without it (same result up
 * to rounding). Every call on one GPU uses the same array and nothing in it
 * needs to start at zero; calls that overlap in time on one GPU (on different
 * streams or threads) race on it and must not be issued; calls on one stream
 * are ordered by it.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
attn_status attn_block_fwd_noalloc(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                   const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                   int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   const attn_mask *mask, float scale,
                                   const attn_tensor *out, float *lse, void *stream);

/*
 * attn_merge_out_lse -- merge one block's partial into the running state.
 * [ZZ] `update_out_and_lse` / [RING] `_update_out_and_lse`, `_init_out_and_lse`:
 *     lse' = ln(e^lse + e^block_lse)
 *     out' = out + sigma * (block_out - out),  sigma = e^(block_lse - lse')
 *          = sigmoid(block_lse - lse)  (the weight [ZZ] returns for backward)
 * Rows: those of the q view (q_view over cu_seqlens, num_seqs documents);
 * other rows are untouched.
 *   out        [n, H, D] f32, read and written (not read when init != 0)
 *   lse        [H, n] f32, read and written (not read when init != 0)
 *   block_out  [n, H, D] bf16 or f32;  block_lse [H, n] f32
 *   block_weight  nullable [H, n] f32: receives sigma
 *   final_out  nullable [n, H, D] bf16 or f32: receives the merged state of
 *              EVERY row (view rows merged, other rows as they stand) cast
 *              to its dtype (round to nearest even); when given, `out` is
 *              NOT written (the last merge of a schedule)
 *   init != 0: the block initialises the state (out' = block_out,
 *              lse' = block_lse), [RING] `_init_out_and_lse`.
 * cu_seqlens may be NULL when q_view == ATTN_VIEW_ALL.
 */
attn_status attn_merge_out_lse(const attn_tensor *out, float *lse,
                               const attn_tensor *block_out, const float *block_lse,
                               const int32_t *cu_seqlens, int32_t num_seqs, uint32_t q_view,
                               float *block_weight, const attn_tensor *final_out,
                               int32_t init, void *stream);

/*
 * attn_merge_n -- merge n_parts partials of the same rows in one pass
 * ([KVP] Background: partial results of the ranks merged by online softmax).
 *   parts_out  host array of n_parts descriptors, each [n, H, D] bf16/f32
 *   parts_lse  host array of n_parts device pointers, each [H, n] f32
 *   out        [n, H, D] bf16 or f32 (written);  lse [H, n] f32 (written)
 * 1 <= n_parts <= 16.
 */
attn_status attn_merge_n(int32_t n_parts, const attn_tensor *parts_out,
                         const float *const *parts_lse, const attn_tensor *out, float *lse,
                         void *stream);

/*
 * attn_merge_diag -- merge one EAGLE-3 test-time-training diagonal block into
 * the running (out, lse). [RING] `_CachedRingAttention` and `_merge_diag`
 * (and [ZZ] `_CachedZigZagRingAttention`): cache block i >= 1 gives query row
 * t exactly one key, k[t, g(h)], with value v[t, g(h)] (same position, any
 * sharding), so its partial is
 *     block_out[t, h] = v[t, g(h)],  block_lse[h, t] = scale <q[t,h], k[t,g(h)]>
 * and it merges by the online-softmax identity (as attn_merge_out_lse).
 *   q [n, HQ, D]; k, v [n, HKV, D]: all bf16 or all f32 (same rows as q)
 *   out [n, HQ, D] f32 running output (read and written); lse [HQ, n] f32
 *     (read and written; a row at -inf takes the diagonal alone)
 *   final_out  NULL, or [n, HQ, D] bf16/f32 written with the merged output
 *              (the cast of the last merge)
 * Every row is merged. Errors: ATTN_ERR_SHAPE when k/v rows differ from q's.
 */
attn_status attn_merge_diag(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, float scale,
                            const attn_tensor *out, float *lse, const attn_tensor *final_out, void *stream);

/*
 * attn_diag_bwd -- gradient of one diagonal block with the MERGED lse and
 * delta ([RING] `_CachedRingAttention`: the diagonal grads are added in closed
 * form beside the block-0 backward). Per row t and q head h, g = g(h):
 *     p = exp(scale <q,k> - lse),  ds = p (<dout, v> - delta)
 *     dq[t,h] += scale ds k[t,g];  dk[t,g] += scale sum_h ds q[t,h];
 *     dv[t,g] += sum_h p dout[t,h]
 *   dout, q [n, HQ, D]; k, v [n, HKV, D]: all bf16 or all f32
 *   lse, delta [HQ, n] f32 (merged; delta from attn_bwd_delta on the merged out)
 *   dq [n, HQ, D], dk, dv [n, HKV, D] f32, ACCUMULATED (+=); deterministic.
 */
attn_status attn_diag_bwd(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                          const float *lse, const float *delta, float scale, const attn_tensor *dq,
                          const attn_tensor *dk, const attn_tensor *dv, void *stream);

/*
 * attn_ulysses_reshard -- the Ulysses all-to-all between uly virtual ranks
 * ([ULY] `_gather_seq_scatter_heads` / `_scatter_seq_gather_heads`). With
 * S_l rows and H heads per sequence shard and H_l = H / uly:
 *   to_heads != 0:  src[r] [S_l, H, D] (rank r's rows r S_l ..)  ->
 *                   dst[r] [uly S_l, H_l, D] (all rows, heads r H_l ..)
 *   to_heads == 0:  the inverse, src[r] [uly S_l, H_l, D] -> dst[r] [S_l, H, D]
 *   src, dst  host arrays of uly descriptors (bf16 or f32, one shape each side)
 * 1 <= uly <= 16. Errors: ATTN_ERR_SHAPE when heads / rows do not divide.
 */
attn_status attn_ulysses_reshard(int32_t uly, int32_t to_heads, const attn_tensor *src, const attn_tensor *dst,
                                 void *stream);

/*
 * attn_ulysses_reshard_lse -- the same for the log-sum-exp ([ULY]
 * `_gather_lse` / `_scatter_lse`): [H, S_l] per sequence shard <-> [H_l, uly S_l]
 * per head shard, both contiguous f32 (the head-shard result is contiguous, as
 * a backward that reads lse without strides needs).
 *   src, dst  host arrays of uly device pointers; n_local = S_l; n_head = H
 */
attn_status attn_ulysses_reshard_lse(int32_t uly, int32_t to_heads, const float *const *src, float *const *dst,
                                     int64_t n_local, int64_t n_head, void *stream);

/*
 * attn_out_transpose -- the transposed output of [KVP] (`tp_out`: [heads, D, S]
 * instead of [heads, S, D]): dst[h, d, t] = src[t, h, d].
 *   src  [n, H, D] bf16 or f32 (any token / head strides, last dim contiguous)
 *   dst  device pointer to a contiguous [H, D, n] array of src's dtype
 * A pure copy (bit-exact).
 */
attn_status attn_out_transpose(const attn_tensor *src, void *dst, void *stream);

/*
 * attn_bwd_delta -- delta[h, i] = sum_d dout[i,h,d] * out[i,h,d] (f32), the
 * row term of the softmax backward, computed from the MERGED out; it is the
 * same for every block of a schedule, so a schedule computes it once.
 *   dout, out [n, H, D] bf16/f32;  delta [H, n] f32 (written)
 */
attn_status attn_bwd_delta(const attn_tensor *dout, const attn_tensor *out, float *delta,
                           void *stream);

/*
 * attn_block_bwd -- gradient of one block with the MERGED out and lse.
 * [ZZ] `_block_backward` and `zigzag_ring_flash_attn_varlen_backward` (each
 * block's backward is fed the final merged out/lse, which gives the joint
 * softmax gradient without a merge backward); [ULY] `_block0_backward`.
 * For every visible pair of the block (same mask as attn_block_fwd):
 *     P = exp(scale q.k - lse),  dS = P (dout.v - delta)
 *     dq += scale dS k,  dk += scale dS q,  dv += P dout  (dk/dv summed over
 *     the q heads of a kv group)
 *   dout, q, out [n_q, HQ, D]; k, v [n_k, HKV, D]; all bf16 or all f32
 *   lse [HQ, n_q] f32 (merged);  delta nullable [HQ, n_q] f32 from
 *   attn_bwd_delta (computed into the workspace when NULL)
 *   dq [n_q, HQ, D] f32, dk/dv [n_k, HKV, D] f32: ACCUMULATED (+=), the caller
 *   zeroes them; passing another rank's buffers accumulates into that owner
 *   ([RING] `ring_flash_attn_backward`: K/V grads go back to their owners).
 * Deterministic: no floating-point atomics ([ZZ] `deterministic` is implied).
 * Paged K/V and segments are not supported in the backward.
 */
attn_status attn_block_bwd(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k,
                           const attn_tensor *v, const attn_tensor *out, const float *lse,
                           const float *delta, const int32_t *cu_seqlens_q,
                           const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                           int32_t max_seqlen_k, const attn_mask *mask, float scale,
                           const attn_tensor *dq, const attn_tensor *dk, const attn_tensor *dv,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_zigzag_shard -- gather rank `rank`'s zig-zag rows from a global packed
 * tensor ([ZZ] module docstring: 2*cp chunks per document, rank r owns chunk r
 * and chunk 2*cp-1-r; per varlen document as in `get_half_index`).
 *   src [S, H, D] global rows, cu_seqlens_global device [num_seqs+1]
 *   dst [S/cp, H, D] local rows: per document [chunk r | chunk 2cp-1-r]
 * Every document length must be a multiple of 2*cp (not checked on device;
 * attn_validate_inputs checks it). max_seqlen = longest global document.
 */
attn_status attn_zigzag_shard(const attn_tensor *src, const int32_t *cu_seqlens_global,
                              int32_t num_seqs, int32_t max_seqlen, int32_t cp, int32_t rank,
                              const attn_tensor *dst, void *stream);

/*
 * attn_zigzag_fwd -- rank `rank`'s whole zig-zag ring forward as virtual
 * ranks ([ZZ] `zigzag_ring_flash_attn_varlen_forward`): at step s the rank
 * holds the K/V of src = (rank - s) mod cp and runs
 *     s == 0:        causal block over its own rows ("diag"),
 *     1 <= s <= rank: all q rows x src's FRONT halves, unmasked,
 *     s > rank:      q BACK halves x all of src's rows, unmasked,
 * merging every block into the running f32 state in step order.
 *   q          [n_loc, HQ, D] this rank's local rows
 *   k_loc,v_loc host arrays of cp descriptors (every rank's local K/V)
 *   cu_local   device local cu_seqlens (= global / cp)
 *   out_acc    [n_loc, HQ, D] f32 running output (scratch of the caller)
 *   out        [n_loc, HQ, D] final output (q dtype or f32)
 *   lse        [HQ, n_loc] f32 merged lse
 * Workspace: attn_zigzag_workspace_size bytes.
 */
attn_status attn_zigzag_workspace_size(int32_t cp, const attn_tensor *q, const attn_tensor *k,
                                       int32_t num_seqs, int32_t max_seqlen_local, size_t *bytes);
attn_status attn_zigzag_fwd(int32_t cp, int32_t rank, const attn_tensor *q,
                            const attn_tensor *k_loc, const attn_tensor *v_loc,
                            const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                            float scale, const attn_tensor *out_acc, const attn_tensor *out,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_zigzag_fwd_ranks -- attn_zigzag_fwd of n_ranks virtual ranks of one
 * ring together: at each step the ranks' blocks (each independent of the
 * others given the K/V it holds, [ZZ] `zigzag_ring_flash_attn_varlen_forward`)
 * run in one launch, which fills the chip when one rank's block alone cannot
 * (small local shards). Results are those of attn_zigzag_fwd per rank.
 *   ranks      host array of n_ranks distinct ranks in [0, cp) (NULL: 0 .. n_ranks-1)
 *   q, out_acc, out  host arrays of n_ranks descriptors, one per listed rank
 *              (every q shaped alike)
 *   lse        host array of n_ranks device pointers
 *   k_loc, v_loc, cu_local, num_seqs, max_seqlen_local, scale: as for attn_zigzag_fwd
 * Workspace: n_ranks slices of attn_zigzag_workspace_size (each rounded up
 * to 256 bytes), one per listed rank. bf16 inputs run batched (up to 8 ranks a
 * launch); f32 inputs run the ranks one after another. 1 <= n_ranks <= cp.
 */
attn_status attn_zigzag_fwd_ranks(int32_t cp, int32_t n_ranks, const int32_t *ranks, const attn_tensor *q,
                                  const attn_tensor *k_loc, const attn_tensor *v_loc, const int32_t *cu_local,
                                  int32_t num_seqs, int32_t max_seqlen_local, float scale,
                                  const attn_tensor *out_acc, const attn_tensor *out, float *const *lse,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_zigzag_bwd -- rank `rank`'s zig-zag backward with the merged out/lse
 * ([ZZ] `zigzag_ring_flash_attn_varlen_backward`): delta once, then the cp
 * blocks of attn_zigzag_fwd in the same order, dq into `dq`, dk/dv of the
 * block at step s into dk_loc[src]/dv_loc[src] (f32, accumulated).
 */
attn_status attn_zigzag_bwd(int32_t cp, int32_t rank, const attn_tensor *dout,
                            const attn_tensor *q, const attn_tensor *k_loc,
                            const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                            const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                            float scale, const attn_tensor *dq, const attn_tensor *dk_loc,
                            const attn_tensor *dv_loc, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Backward driver flags (attn_zigzag_bwd_ex, attn_ring_bwd_ex; 0 = the
 * accumulating attn_zigzag_bwd / attn_ring_bwd).
 *   ATTN_BWD_SET: the call SETS dq and every dk_loc[c] / dv_loc[c] instead of
 *   adding to them, so the caller need not zero them first ([RING]
 *   `ring_flash_attn_backward` starts its gradient buffers at zero on every
 *   call; this gives the same result without a separate zeroing pass). Each step's source
 *   is a different rank, so each block stores its dk/dv into its owner's
 *   buffers; step 0 (the diagonal block, every row of every document) stores
 *   dq and later steps add; rows no block writes (the other half of a
 *   half-view source, sources no step uses, rows outside every document) are
 *   written as zeros. Results equal the accumulating call on zeroed buffers
 *   exactly. cp <= 19 with this flag (ATTN_ERR_UNSUPPORTED beyond). Every
 *   dk_loc[c] / dv_loc[c], also of a source the rank never uses, is written,
 *   so each must be f32 and shaped like k_loc[c] (ATTN_ERR_DTYPE /
 *   ATTN_ERR_SHAPE), checked before anything is launched.
 * Unknown flag bits: ATTN_ERR_INVALID.
 */
#define ATTN_BWD_SET 1u
attn_status attn_zigzag_bwd_ex(int32_t cp, int32_t rank, const attn_tensor *dout,
                               const attn_tensor *q, const attn_tensor *k_loc,
                               const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                               const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                               float scale, const attn_tensor *dq, const attn_tensor *dk_loc,
                               const attn_tensor *dv_loc, void *workspace, size_t workspace_bytes,
                               void *stream, uint32_t flags);

/*
 * attn_ring_fwd / attn_ring_bwd -- contiguous ring, causal ([RING]
 * `ring_flash_attn_forward` / `ring_flash_attn_backward`): rank r attends the
 * K/V of steps s <= r (src = r - s), causal only at s == 0. Arguments as for
 * the zig-zag entries; cu_local holds each sequence's local shard.
 */
attn_status attn_ring_fwd(int32_t cp, int32_t rank, const attn_tensor *q,
                          const attn_tensor *k_loc, const attn_tensor *v_loc,
                          const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                          float scale, const attn_tensor *out_acc, const attn_tensor *out,
                          float *lse, void *workspace, size_t workspace_bytes, void *stream);
attn_status attn_ring_bwd(int32_t cp, int32_t rank, const attn_tensor *dout,
                          const attn_tensor *q, const attn_tensor *k_loc,
                          const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                          const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                          float scale, const attn_tensor *dq, const attn_tensor *dk_loc,
                          const attn_tensor *dv_loc, void *workspace, size_t workspace_bytes,
                          void *stream);
attn_status attn_ring_bwd_ex(int32_t cp, int32_t rank, const attn_tensor *dout,
                             const attn_tensor *q, const attn_tensor *k_loc,
                             const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                             const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                             float scale, const attn_tensor *dq, const attn_tensor *dk_loc,
                             const attn_tensor *dv_loc, void *workspace, size_t workspace_bytes,
                             void *stream, uint32_t flags);

/*
 * attn_kvp_fwd -- KV-parallel segmented prefill over R virtual ranks ([KVP]
 * Background: each rank attends its local KV shard in segments with online
 * softmax, then the ranks' partials are merged by online softmax). Rank r
 * runs attn_block_fwd on its own paged cache with `mask` (causal, window,
 * q_pos_offset = the global position of query token 0, block_size,
 * max_blocks, page_stride, seg_size) and its own block table, with key
 * positions
 *     round robin  (mask->kv_interleave == R): local block b -> global b*R + r
 *     contiguous   (mask->kv_interleave == 0): k_pos_offset = r * max_seqlen_k
 * ([KVP] `kvp_q_offset` = -r * local_kv_len + global_q_offset is the same
 * mask with the offset moved to the query side). The ranks' key-part
 * partials (f32, in the workspace) are merged by online softmax into out /
 * lse in one pass when all of them fit 1 GiB; otherwise each rank merges its
 * parts and the R rank partials are merged in rank order (same result up to
 * rounding). Rows outside the q view stay untouched.
 *   k_caches, v_caches  host arrays of R cache descriptors
 *   block_tables        host array of R device pointers (each max_blocks int32)
 *   cu_seqlens_k        logical local key counts per document
 *   mask                required; block_size, max_blocks and page_stride must
 *                       be > 0 (ATTN_ERR_INVALID otherwise). The keys are
 *                       always paged through block_tables: mask->block_table
 *                       is ignored by both entries. The per-rank forwards are
 *                       always tiled (max_seqlen_q == 1 does not select the
 *                       decode kernel here).
 * 1 <= R <= 16. Workspace: attn_kvp_workspace_size bytes.
 */
attn_status attn_kvp_workspace_size(int32_t R, const attn_tensor *q, const attn_tensor *k,
                                    int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    const attn_mask *mask, size_t *bytes);
attn_status attn_kvp_fwd(int32_t R, const attn_tensor *q, const attn_tensor *k_caches,
                         const attn_tensor *v_caches, const int32_t *const *block_tables,
                         const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                         int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         const attn_mask *mask, float scale, const attn_tensor *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_validate_inputs -- checks DEVICE contents that the launch paths never
 * read on the host: cu_seqlens non-decreasing, starting at 0, per-document
 * lengths <= max_seqlen_*, totals within n_tok; with a block table every
 * entry used lies in [0, pages); when `zigzag_cp` > 0 every q document length
 * is a multiple of 2*zigzag_cp; when `one_query` != 0 every q length is 1
 * ([DEC] `triton_varlen_attn_func` checks the same before capture).
 * SYNCHRONISES the stream; not for use under graph capture.
 */
attn_status attn_validate_inputs(const attn_tensor *q, const attn_tensor *k,
                                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 const attn_mask *mask, int32_t zigzag_cp, int32_t one_query,
                                 void *stream);

/*
 * Kernel timing (tracing). With timing enabled, every kernel the library
 * launches is bracketed by two hipEvents recorded on the launch stream (the
 * events come from a pool the library keeps for the process; no device
 * memory is allocated). attn_timing_report waits for the recorded events and
 * writes one line per kernel, "name launches total_ms\n", into buf (len bytes
 * including the terminating 0; *written = bytes needed without it), then
 * clears the record; with buf == NULL (a size query) or a buffer that is too
 * small the record is kept. Not for use under graph capture. Process-wide
 * and thread-safe; spans of concurrent callers are merged.
 */
attn_status attn_timing_enable(int32_t on);
attn_status attn_timing_report(char *buf, size_t len, size_t *written);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H_ */
