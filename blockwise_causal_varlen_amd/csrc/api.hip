// Host side of the C ABI declared in include/attn.h: argument validation,
// workspace sizing, kernel selection by shape, and the virtual-rank schedule
// drivers (zig-zag ring, contiguous ring, KV-parallel). No entry point reads
// device memory on the host or synchronises, except attn_validate_inputs.
#include <math.h>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "internal.h"

using namespace attn;

namespace {

thread_local std::string g_err;

attn_status fail(attn_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

attn_status ok() { return ATTN_OK; }

attn_status hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TRY(x)                        \
  do {                                \
    attn_status _s = (x);             \
    if (_s != ATTN_OK) return _s;     \
  } while (0)

// ---------------------------------------------------------------------------
// Kernel timing: when enabled, each launch is bracketed by two hipEvents on
// its stream; attn_timing_report reads and clears them.
// ---------------------------------------------------------------------------
struct Span {
  const char *name;
  hipEvent_t a, b;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<Span> spans;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<long, double>> agg;  // read but not yet delivered
};
Timing &timing() {
  static Timing t;
  return t;
}
hipEvent_t pooled_event() {
  Timing &t = timing();
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  // timestamps only: no system-scope fence around each launch (the report
  // reads them after hipEventSynchronize)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
hipError_t timed(const char *name, hipStream_t s, F &&launch) {
  Timing &t = timing();
  if (!t.on) return launch();
  std::lock_guard<std::mutex> lk(t.mu);
  Span sp{name, pooled_event(), pooled_event()};
  if (sp.a) hipEventRecord(sp.a, s);
  hipError_t e = launch();
  if (sp.b) hipEventRecord(sp.b, s);
  if (sp.a && sp.b) t.spans.push_back(sp);
  return e;
}

int esize(int32_t dt) { return dt == ATTN_BF16 ? 2 : 4; }

// A tensor descriptor with [n_tok, n_head, head_dim], 16-byte aligned rows.
attn_status check_tensor(const attn_tensor *t, const char *name, bool allow_f32 = true) {
  if (!t) return fail(ATTN_ERR_NULL, "%s: descriptor is NULL", name);
  if (!t->data && t->n_tok > 0) return fail(ATTN_ERR_NULL, "%s: data is NULL", name);
  if (t->dtype != ATTN_BF16 && !(allow_f32 && t->dtype == ATTN_F32))
    return fail(ATTN_ERR_DTYPE, "%s: unsupported dtype %d", name, t->dtype);
  if (t->n_tok < 0 || t->n_head <= 0 || t->head_dim <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: bad sizes [%lld, %lld, %lld]", name, (long long)t->n_tok,
                (long long)t->n_head, (long long)t->head_dim);
  if (t->stride_tok <= 0 || t->stride_head <= 0)
    return fail(ATTN_ERR_LAYOUT, "%s: strides must be positive", name);
  const int64_t eb = esize(t->dtype);
  if (((uintptr_t)t->data) % 16 || (t->stride_tok * eb) % 16 || (t->stride_head * eb) % 16)
    return fail(ATTN_ERR_LAYOUT, "%s: data and row strides must be 16-byte aligned", name);
  if (t->stride_head < t->head_dim && t->n_head > 1 && t->stride_tok < t->head_dim)
    return fail(ATTN_ERR_LAYOUT, "%s: rows overlap", name);
  return ok();
}

attn_status check_hd(int64_t d) {
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  return ok();
}

attn_status check_mask(const attn_mask *m) {
  if (!m) return ok();
  if (m->struct_size != sizeof(attn_mask))
    return fail(ATTN_ERR_VERSION, "attn_mask.struct_size %u != %zu (header/library mismatch)", m->struct_size,
                sizeof(attn_mask));
  if (m->q_view > 2 || m->k_view > 2) return fail(ATTN_ERR_INVALID, "bad view %u/%u", m->q_view, m->k_view);
  if (m->window < 0) return fail(ATTN_ERR_INVALID, "window must be >= 0");
  if (m->kv_interleave < 0) return fail(ATTN_ERR_INVALID, "kv_interleave must be >= 0");
  if (m->kv_interleave > 0 && (m->block_size <= 0 || m->kv_rank < 0 || m->kv_rank >= m->kv_interleave))
    return fail(ATTN_ERR_INVALID, "round robin needs block_size > 0 and 0 <= kv_rank < kv_interleave");
  if (m->kv_interleave > 0 && (m->block_size & (m->block_size - 1)))
    return fail(ATTN_ERR_UNSUPPORTED, "round robin needs a power-of-two block_size");
  if (m->block_table && (m->block_size <= 0 || m->max_blocks <= 0 || m->page_stride <= 0))
    return fail(ATTN_ERR_INVALID, "paged keys need block_size, max_blocks and page_stride > 0");
  if (m->block_table && (m->block_size & (m->block_size - 1)))
    return fail(ATTN_ERR_UNSUPPORTED, "paged keys need a power-of-two block_size");
  if (m->seg_size < 0) return fail(ATTN_ERR_INVALID, "seg_size must be >= 0");
  if (m->seg_size > 0 && m->q_view != ATTN_VIEW_ALL)
    return fail(ATTN_ERR_UNSUPPORTED, "segments with a q view are not supported");
  return ok();
}

MaskDev mask_dev(const attn_mask *m) {
  MaskDev d{};
  if (!m) return d;
  d.causal = m->causal ? 1 : 0;
  d.q_view = (int32_t)m->q_view;
  d.k_view = (int32_t)m->k_view;
  d.seg_size = m->seg_size;
  d.window = m->window;
  d.q_pos_offset = m->q_pos_offset;
  d.pm.k_pos_offset = m->k_pos_offset;
  d.pm.interleave = m->kv_interleave;
  d.pm.rank = m->kv_rank;
  d.pm.block = m->block_size;
  d.pm.shift = m->block_size > 0 ? __builtin_ctz((unsigned)m->block_size) : 0;
  return d;
}

TensorDev tdev(const attn_tensor *t) { return TensorDev{t->data, t->stride_tok, t->stride_head}; }

// Document-local key rows [lo, hi) that some query of a call can see: every
// query position lies in [q_pos_offset, q_pos_offset + max_q), so causality
// ends the range and a window starts it. The scheduler's per-item key ranges
// (and so every tile the forward reads) lie inside it, so a paged gather
// copies only these rows.
static void visible_key_rows(const attn_mask *m, int64_t max_q, int64_t max_k, int64_t &lo, int64_t &hi) {
  const MaskDev md = mask_dev(m);
  lo = 0;
  hi = max_k;
  if (md.causal) hi = md.pm.count_le(md.q_pos_offset + max_q - 1, max_k);
  if (md.window > 0) lo = md.pm.count_le(md.q_pos_offset - md.window, max_k);
}



// The kernels index rows, positions and in-tile offsets in 32 bits.
static attn_status check_ranges(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                const attn_mask *m, int64_t n_k_logical) {
  const int64_t lim = (int64_t)1 << 30;
  const int64_t R = (m && m->kv_interleave > 0) ? m->kv_interleave : 1;
  if (q->n_tok >= lim || n_k_logical >= lim || k->n_tok >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "2^30 rows or more");
  if (m && (llabs(m->q_pos_offset) + q->n_tok >= lim || llabs(m->k_pos_offset) + n_k_logical * R >= lim ||
            m->window >= lim))
    return fail(ATTN_ERR_UNSUPPORTED, "positions reach 2^30");
  if (q->stride_tok >= (1 << 22) || k->stride_tok >= (1 << 22) || v->stride_tok >= (1 << 22))
    return fail(ATTN_ERR_UNSUPPORTED, "a row stride of 2^22 elements or more");
  return ok();
}

struct Problem {
  int64_t n_q, n_k_logical, hq, hkv, d;
  int64_t nseg;
  bool decode;
  bool paged;
  int32_t dsplit = 1, dsplit_len = 0;  // decode: split KV over dsplit waves per (sequence, kv head)
  int32_t nsplit = 0;                   // tiled forward: > 1 = each query tile's keys cut in nsplit parts
  bool gather = false;                  // paged keys copied to contiguous buffers first
  int64_t gather_row_bytes = 0;         // bytes of one gathered logical row (all heads) of K or V
};

attn_status check_qkv(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v) {
  TRY(check_tensor(q, "q"));
  TRY(check_tensor(k, "k"));
  TRY(check_tensor(v, "v"));
  if (k->dtype != q->dtype || v->dtype != q->dtype)
    return fail(ATTN_ERR_DTYPE, "q/k/v dtypes differ (%d/%d/%d)", q->dtype, k->dtype, v->dtype);
  if (k->head_dim != q->head_dim || v->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "head_dim mismatch");
  TRY(check_hd(q->head_dim));
  if (k->n_head != v->n_head || k->n_tok != v->n_tok) return fail(ATTN_ERR_SHAPE, "k/v shapes differ");
  if (q->n_head % k->n_head) return fail(ATTN_ERR_GQA, "GQA mismatch: %lld q heads vs %lld kv heads",
                                         (long long)q->n_head, (long long)k->n_head);
  return ok();
}

attn_status plan_fwd(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, int32_t num_seqs,
                     int32_t max_q, int32_t max_k, const attn_mask *m, Problem &P, bool allow_split = true,
                     bool allow_decode = true) {
  TRY(check_qkv(q, k, v));
  TRY(check_mask(m));
  if (num_seqs < 0 || max_q < 0 || max_k < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative num_seqs or max_seqlen");
  P.n_q = q->n_tok;
  P.hq = q->n_head;
  P.hkv = k->n_head;
  P.d = q->head_dim;
  P.paged = m && m->block_table;
  P.n_k_logical = P.paged ? (int64_t)m->max_blocks * m->block_size : k->n_tok;
  P.nseg = 0;
  const bool plain = !m || (!m->causal && m->q_view == 0 && m->k_view == 0 && m->window == 0 &&
                            m->kv_interleave == 0 && !m->block_table && m->seg_size == 0);
  // (the decode kernel addresses one sequence's K / V bytes with 32-bit offsets)
  P.decode = allow_decode && max_q == 1 && plain && q->dtype == ATTN_BF16 && (P.hq / P.hkv) <= 16 &&
             (int64_t)max_k * (k->stride_tok > v->stride_tok ? k->stride_tok : v->stride_tok) * 2 <
                 ((int64_t)1 << 31);
  P.dsplit = 1; P.dsplit_len = 0;
  if (P.decode) {
    // flash-decoding split: when the (sequence, kv head) waves cannot fill the
    // chip (two workgroups of 4 waves a CU), each one's keys are split (>= 256
    // keys a split, at most 32 splits) and the partials merged, as segments are
    const int64_t waves = (int64_t)num_seqs * P.hkv;
    int64_t n = waves > 0 ? (2048 + waves - 1) / waves : 1;
    if (n > 32) n = 32;
    if (n > max_k / 256) n = max_k / 256;
    if (n > 1) {
      int64_t len = (max_k + n - 1) / n;
      len = (len + 31) / 32 * 32;
      P.dsplit = (int32_t)((max_k + len - 1) / len);
      P.dsplit_len = (int32_t)len;
    }
  }
  // paged keys: a streaming gather of the logical rows into contiguous
  // workspace buffers, then the contiguous forward (page lookups inside the
  // forward's tile loop measured 1.5x slower than gather + contiguous)
  P.gather = P.paged;
  if (P.paged) {
    P.gather_row_bytes = k->n_head * k->head_dim * (int64_t)esize(k->dtype);
    if ((m->page_stride * esize(k->dtype)) % 16)
      return fail(ATTN_ERR_LAYOUT, "page_stride must be a multiple of 16 bytes");
  }
  // Parts: each query tile's visible keys are cut into n parts of whole key
  // tiles, computed as partials and merged. Segments ask for at least as many
  // parts as max_seqlen_k has segments (so no part is much longer than
  // seg_size); the cut follows each tile's visible range rather than fixed
  // segment boundaries, so a window does not leave most parts empty and a few
  // long (the partition is internal: any one gives the same merged result). A
  // small grid (the chip holds 512 query-tile workgroups) asks for up to 16
  // parts of >= 512 keys of max_seqlen_k each.
  P.nsplit = 0;
  if (!P.decode) {
    int64_t n = 1;
    if (m && m->seg_size > 0) {
      int64_t span = max_k;  // keys one query tile can see
      if (m->window > 0) {
        const int64_t w = m->window + kFwdBM;
        const int64_t R = m->kv_interleave;
        const int64_t vis = R > 0 ? (w + R - 1) / R + 2 * (int64_t)m->block_size : w;
        if (vis < span) span = vis;
      }
      n = (span + m->seg_size - 1) / m->seg_size;
    }
    if (allow_split && max_k >= 1024) {
      const int64_t wgs = ((int64_t)P.n_q / kFwdBM + num_seqs) * P.hq;
      if (wgs > 0 && wgs < 512) {
        int64_t a = (1024 + wgs - 1) / wgs;
        if (a > 16) a = 16;
        if (a > max_k / 512) a = max_k / 512;
        if (a > n) n = a;
      }
    }
    if (n > 1) {
      P.nsplit = (int32_t)n;
      P.nseg = n;
    }
  }
  return check_ranges(q, k, v, m, P.n_k_logical);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// own_parts = false: the caller provides the key-part partials (block_fwd_impl's PartsOut).
size_t fwd_ws_bytes(const Problem &P, int32_t num_seqs, bool own_parts = true) {
  if (P.decode)
    return P.dsplit > 1 ? align256((size_t)P.dsplit * P.n_q * P.hq * P.d * 4) + align256((size_t)P.dsplit * P.hq * P.n_q * 4)
                        : 0;
  const int64_t cap = sched_capacity(P.n_q, num_seqs, kFwdBM, P.nseg);
  size_t b = align256(sched_bytes(cap));
  if (P.nseg > 0 && own_parts) {
    b += align256((size_t)P.nseg * P.n_q * P.hq * P.d * 4);
    b += align256((size_t)P.nseg * P.hq * P.n_q * 4);
  }
  if (P.gather) b += 2 * align256((size_t)P.n_k_logical * P.gather_row_bytes);  // gathered K, V (last)
  return b;
}

// f16 copies of q and dout for the dK/dV kernel (bf16 inputs) and their flag
size_t half_copy_bytes(int64_t n_q, int64_t hq, int64_t d, int32_t dtype) {
  return dtype == ATTN_BF16 ? 2 * align256((size_t)n_q * hq * d * 2) + 256 : 0;
}

size_t bwd_ws_bytes(int64_t n_q, int64_t n_k, int64_t hq, int64_t d, int32_t dtype, int32_t num_seqs,
                    bool need_delta) {
  size_t b = align256(sched_bytes(sched_capacity(n_q, num_seqs, kBwdTile, 1)));
  b += align256(sched_bytes(sched_capacity(n_k, num_seqs, kBwdTile, 1)));
  b += align256((size_t)hq * n_q * 4);  // lse in log2 units
  if (need_delta) b += align256((size_t)hq * n_q * 4);
  return b + half_copy_bytes(n_q, hq, d, dtype);
}

// Carve the f16 copies (q16, do16, flag) at w; their launch follows lse2's,
// which zeroes the flag.
struct HalfCopies {
  void *q16 = nullptr, *do16 = nullptr;
  int32_t *flag = nullptr;
};
HalfCopies half_carve(char *w, int64_t n_q, int64_t hq, int64_t d) {
  HalfCopies h;
  const size_t b = align256((size_t)n_q * hq * d * 2);
  h.q16 = w;
  h.do16 = w + b;
  h.flag = (int32_t *)(w + 2 * b);
  return h;
}
hipError_t launch_half_copies(const HalfCopies &h, const attn_tensor *q, const attn_tensor *dout, hipStream_t s) {
  HalfCopyArgs a;
  a.q = q->data; a.q_st = q->stride_tok; a.q_sh = q->stride_head;
  a.dout = dout->data; a.do_st = dout->stride_tok; a.do_sh = dout->stride_head;
  a.q16 = h.q16; a.do16 = h.do16; a.flag = h.flag;
  a.n = q->n_tok; a.h = (int32_t)q->n_head; a.d = (int32_t)q->head_dim;
  return launch_half_copy(a, s);
}

attn_status check_out(const attn_tensor *out, const Problem &P, const char *name) {
  TRY(check_tensor(out, name));
  if (out->n_tok != P.n_q || out->n_head != P.hq || out->head_dim != P.d)
    return fail(ATTN_ERR_SHAPE, "%s must be [n_q, HQ, D]", name);
  return ok();
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char *attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_DTYPE: return "unsupported or mismatched dtype";
    case ATTN_ERR_SHAPE: return "shape mismatch";
    case ATTN_ERR_GQA: return "q heads not a multiple of kv heads";
    case ATTN_ERR_CU_SEQLENS: return "bad cu_seqlens / max_seqlen";
    case ATTN_ERR_LAYOUT: return "bad layout";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP error";
    case ATTN_ERR_VERSION: return "struct version mismatch";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_CONTENT: return "invalid device data";
  }
  return "unknown status";
}

const char *attn_last_error(void) { return g_err.c_str(); }

attn_status attn_workspace_size(attn_op op, const attn_tensor *q, const attn_tensor *k, int32_t num_seqs,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask,
                                size_t *bytes) {
  if (!bytes) return fail(ATTN_ERR_NULL, "bytes is NULL");
  TRY(check_tensor(q, "q"));
  TRY(check_tensor(k, "k"));
  TRY(check_mask(mask));
  if (op == ATTN_OP_BLOCK_FWD) {
    Problem P;
    TRY(plan_fwd(q, k, k, num_seqs, max_seqlen_q, max_seqlen_k, mask, P));
    *bytes = fwd_ws_bytes(P, num_seqs);
    return ok();
  }
  if (op == ATTN_OP_BLOCK_BWD) {
    *bytes = bwd_ws_bytes(q->n_tok, k->n_tok, q->n_head, q->head_dim, q->dtype, num_seqs, true);
    return ok();
  }
  return fail(ATTN_ERR_INVALID, "unknown op %d", (int)op);
}

attn_status attn_workspace_bytes(attn_op op, const attn_tensor *q, const attn_tensor *k, int32_t num_seqs,
                                 int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask,
                                 size_t *bytes) {
  return attn_workspace_size(op, q, k, num_seqs, max_seqlen_q, max_seqlen_k, mask, bytes);
}

}  // extern "C"

namespace {

// A block forward that works on a running state (acc f32 with the lse given
// to block_fwd_impl), in the forward kernel's epilogue: merge (else the block
// initialises the state); rows of the document halves in final_view (bit 0
// front, bit 1 back) have their last update here and go to the out tensor.
struct FusedMerge {
  const attn_tensor *acc;
  bool merge;
  int32_t final_view;
};

// Caller-owned partials: the forward writes its key parts there ([nparts]
// slices of [n_q, H, D] f32 and [H, n_q] f32; one part when the plan needs
// none) and leaves the merge to the caller.
struct PartsOut {
  float *out, *lse;
  int64_t nparts;
};

bool can_fuse_merge(const attn_tensor *q, int32_t max_seqlen_q, const attn_mask *m) {
  return q->dtype == ATTN_BF16 && max_seqlen_q != 1 && !(m && (m->seg_size > 0 || m->block_table));
}

attn_status block_fwd_impl(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask, float scale,
                           const attn_tensor *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream, const FusedMerge *fm, const SchedBufs *pre = nullptr,
                           bool allow_split = true, const PartsOut *po = nullptr, FwdArgs *defer = nullptr) {
  Problem P;
  // caller-owned parts always take the tiled forward (never the decode kernel)
  TRY(plan_fwd(q, k, v, num_seqs, max_seqlen_q, max_seqlen_k, mask, P, allow_split && !fm, po == nullptr));
  TRY(check_out(out, P, "out"));
  if (po) {
    if (P.decode || fm) return fail(ATTN_ERR_INVALID, "internal: caller-owned parts need the tiled forward");
    // the caller's partition of each query tile's keys (its schedule was made with it)
    if (po->nparts < 1) return fail(ATTN_ERR_INVALID, "internal: no parts");
    P.nseg = po->nparts;
    P.nsplit = po->nparts > 1 ? po->nparts : 0;
  }
  if (!lse && P.n_q > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  if (num_seqs > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(ATTN_ERR_INVALID, "scale must be positive and finite");
  const size_t need = fwd_ws_bytes(P, num_seqs, po == nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (((uintptr_t)workspace) % 256) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (num_seqs == 0 || P.n_q == 0) return ok();

  if (fm) {
    if (P.decode || P.nseg > 0 || P.paged || q->dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, "a fused merge needs the bf16 tiled forward");
    TRY(check_out(fm->acc, P, "acc"));
    if (fm->acc->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "running out must be f32");
  }

  if (P.decode) {
    DecodeArgs a;
    a.q = tdev(q); a.k = tdev(k); a.v = tdev(v);
    a.head_dim = (int32_t)P.d; a.hq = (int32_t)P.hq; a.hkv = (int32_t)P.hkv; a.num_seqs = num_seqs;
    a.scale = scale; a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.out = out->data; a.out_dtype = out->dtype; a.o_st = out->stride_tok; a.o_sh = out->stride_head;
    a.lse = lse; a.lse_n = P.n_q; a.n_k = k->n_tok;
    if (P.dsplit <= 1)
      return hip_check(timed("attn_decode", s, [&] { return launch_decode(a, s); }), "decode kernel");
    char *w = (char *)workspace;
    a.n_split = P.dsplit; a.split_len = P.dsplit_len;
    a.part_out = (float *)w;
    a.part_lse = (float *)(w + align256((size_t)P.dsplit * P.n_q * P.hq * P.d * 4));
    TRY(hip_check(timed("attn_decode", s, [&] { return launch_decode(a, s); }), "decode kernel"));
    return hip_check(timed("attn_decode_merge", s, [&] { return launch_decode_split_merge(a, s); }),
                     "split-KV merge");
  }

  attn_tensor kg, vg;
  attn_mask mg;
  if (P.gather) {
    // logical rows of the paged caches -> contiguous K, V at the workspace's end
    const size_t gb = align256((size_t)P.n_k_logical * P.gather_row_bytes);
    char *gk = (char *)workspace + need - 2 * gb;
    PageGatherArgs ga;
    ga.src_k = k->data; ga.src_v = v->data;
    ga.page_stride = mask->page_stride; ga.st = k->stride_tok; ga.sh = k->stride_head;
    if (v->stride_tok != k->stride_tok || v->stride_head != k->stride_head)
      return fail(ATTN_ERR_LAYOUT, "paged k and v caches must share their strides");
    ga.table = mask->block_table; ga.max_blocks = mask->max_blocks; ga.n_pages = k->n_tok / mask->block_size;
    ga.shift = __builtin_ctz((unsigned)mask->block_size);
    ga.dst_k = gk; ga.dst_v = gk + gb;
    ga.n_rows = P.n_k_logical; ga.h = (int32_t)P.hkv; ga.d = (int32_t)P.d; ga.eb = esize(k->dtype);
    ga.cu = cu_seqlens_k; ga.num_seqs = num_seqs;
    visible_key_rows(mask, max_seqlen_q, max_seqlen_k, ga.t_lo, ga.t_hi);
    TRY(hip_check(timed("attn_gather", s, [&] { return launch_page_gather(ga, s); }), "page gather"));
    kg = *k;
    kg.data = gk; kg.n_tok = P.n_k_logical; kg.stride_head = P.d; kg.stride_tok = P.hkv * P.d;
    vg = kg;
    vg.data = gk + gb;
    mg = *mask;
    mg.block_table = nullptr; mg.max_blocks = 0; mg.page_stride = 0;
    k = &kg; v = &vg; mask = &mg;
    P.paged = false;
  }
  const int64_t cap = sched_capacity(P.n_q, num_seqs, kFwdBM, P.nseg);
  char *w = (char *)workspace;
  SchedBufs sb = sched_carve(w, cap);
  w += align256(sched_bytes(cap));
  MaskDev md = mask_dev(mask);
  md.seg_size = 0;  // segments are served by parts of each tile's visible keys (plan_fwd)
  if (pre) {
    if (pre->capacity != cap) return fail(ATTN_ERR_INVALID, "internal: schedule capacity differs");
    sb = *pre;
  } else {
    TRY(hip_check(timed("attn_sched", s, [&] {
                    return launch_schedule(cu_seqlens_q, cu_seqlens_k, num_seqs, P.n_q, P.n_k_logical, md, kFwdBM,
                                           kFwdBN, 0, (int32_t)P.nseg, sb, s, P.nsplit);
                  }), "scheduler"));
  }
  FwdArgs a;
  a.q = tdev(q); a.k = tdev(k); a.v = tdev(v);
  a.dtype = q->dtype; a.head_dim = (int32_t)P.d; a.hq = (int32_t)P.hq; a.hkv = (int32_t)P.hkv;
  a.scale = scale; a.mask = md;
  a.out = out->data; a.out_dtype = out->dtype; a.o_st = out->stride_tok; a.o_sh = out->stride_head;
  a.lse = lse; a.lse_n = P.n_q;
  a.part_out = nullptr; a.part_lse = nullptr;
  a.n_q = P.n_q;
  a.sched = sb;
  a.grid_items = cap;
  if (fm) {
    a.acc = (float *)fm->acc->data; a.a_st = fm->acc->stride_tok; a.a_sh = fm->acc->stride_head;
    a.merge = fm->merge ? 1 : 0;
    a.final_view = fm->final_view;
  }
  if (po) {
    a.part_out = po->out;
    a.part_lse = po->lse;
  } else if (P.nseg > 0) {
    a.part_out = (float *)w;
    w += align256((size_t)P.nseg * P.n_q * P.hq * P.d * 4);
    a.part_lse = (float *)w;
    // no fill: every query tile has one item per part, and a part that sees
    // no key still writes lse = -inf for its rows; rows of no tile are not merged
  }
  if (defer) {  // the caller launches it with others (writes to the given parts / its own rows only)
    if (!po && !fm) return fail(ATTN_ERR_INVALID, "internal: a deferred forward needs its parts buffer");
    *defer = a;
    return ok();
  }
  TRY(hip_check(timed("attn_fwd", s, [&] { return launch_fwd(a, s); }), "forward kernel"));
  if (P.nseg > 0 && !po) {
    MergeNArgs mn{};
    mn.n_parts = (int32_t)P.nseg;
    mn.strided = 1;
    mn.out_stride = P.n_q * P.hq * P.d;
    mn.lse_stride = P.hq * P.n_q;
    mn.pout[0] = a.part_out; mn.pdtype[0] = ATTN_F32; mn.p_st[0] = P.hq * P.d; mn.p_sh[0] = P.d;
    mn.plse[0] = a.part_lse;
    mn.out = out->data; mn.out_dtype = out->dtype; mn.o_st = out->stride_tok; mn.o_sh = out->stride_head;
    mn.lse = lse; mn.n = P.n_q; mn.h = P.hq; mn.d = P.d;
    // rows no tile reaches (outside the query view or of no document) stay untouched
    mn.cu = cu_seqlens_q; mn.num_seqs = num_seqs; mn.view = mask ? (int32_t)mask->q_view : 0;
    TRY(hip_check(timed("attn_merge_n", s, [&] { return launch_merge_n(mn, s); }), "segment merge"));
  }
  return ok();
}

}  // namespace

extern "C" {

attn_status attn_block_fwd(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask, float scale,
                           const attn_tensor *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream) {
  return block_fwd_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, mask, scale, out,
                        lse, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The no-allocation forward's workspace: a file-scope device array, one copy
// per GPU. In host code `scratch` names a host-side stand-in, not the device
// copy: kernels get the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device ordinal -> that device's copy of scratch

attn_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p || ((uintptr_t)p) % 256) return fail(ATTN_ERR_HIP, "scratch array address not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

attn_status attn_block_fwd_noalloc(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                   const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask, float scale,
                                   const attn_tensor *out, float *lse, void *stream) {
  constexpr size_t kMax = ATTN_NOALLOC_SCRATCH_BYTES;
  // the plan attn_block_fwd would make; without the automatic key split of
  // small grids when its partials do not fit the array
  Problem P;
  TRY(plan_fwd(q, k, v, num_seqs, max_seqlen_q, max_seqlen_k, mask, P, true));
  bool split = true;
  size_t need = fwd_ws_bytes(P, num_seqs);
  if (need > kMax && P.nsplit > 0 && !(mask && mask->seg_size > 0)) {
    TRY(plan_fwd(q, k, v, num_seqs, max_seqlen_q, max_seqlen_k, mask, P, false));
    split = false;
    need = fwd_ws_bytes(P, num_seqs);
  }
  if (need > kMax)
    return fail(ATTN_ERR_WORKSPACE,
                "attn_block_fwd_noalloc: this call needs %zu bytes of workspace; its array holds at most %zu "
                "(use attn_block_fwd with a caller workspace)", need, kMax);
  void *ws = nullptr;
  TRY(scratch_of_current_device(&ws));
  return block_fwd_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, mask, scale, out,
                        lse, ws, kMax, stream, nullptr, nullptr, split);
}

attn_status attn_merge_out_lse(const attn_tensor *out, float *lse, const attn_tensor *block_out,
                               const float *block_lse, const int32_t *cu_seqlens, int32_t num_seqs,
                               uint32_t q_view, float *block_weight, const attn_tensor *final_out, int32_t init,
                               void *stream) {
  TRY(check_tensor(out, "out"));
  if (out->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "running out must be f32");
  TRY(check_tensor(block_out, "block_out"));
  TRY(check_hd(out->head_dim));
  if (block_out->n_tok != out->n_tok || block_out->n_head != out->n_head || block_out->head_dim != out->head_dim)
    return fail(ATTN_ERR_SHAPE, "block_out shape differs from out");
  if (final_out) {
    TRY(check_tensor(final_out, "final_out"));
    if (final_out->n_tok != out->n_tok || final_out->n_head != out->n_head || final_out->head_dim != out->head_dim)
      return fail(ATTN_ERR_SHAPE, "final_out shape differs from out");
  }
  if ((!lse || !block_lse) && out->n_tok > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  if (q_view > 2) return fail(ATTN_ERR_INVALID, "bad view %u", q_view);
  if (q_view != 0 && (!cu_seqlens || num_seqs <= 0)) return fail(ATTN_ERR_NULL, "a view needs cu_seqlens");
  MergeArgs a;
  a.out = (float *)out->data; a.o_st = out->stride_tok; a.o_sh = out->stride_head;
  a.lse = lse;
  a.bout = block_out->data; a.bout_dtype = block_out->dtype; a.b_st = block_out->stride_tok; a.b_sh = block_out->stride_head;
  a.blse = block_lse; a.weight = block_weight;
  a.fout = final_out ? final_out->data : nullptr;
  a.fout_dtype = final_out ? final_out->dtype : ATTN_F32;
  a.f_st = final_out ? final_out->stride_tok : 0; a.f_sh = final_out ? final_out->stride_head : 0;
  a.cu = cu_seqlens; a.num_seqs = num_seqs; a.view = (int32_t)q_view;
  a.n = out->n_tok; a.h = out->n_head; a.d = out->head_dim; a.init = init ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_merge", s, [&] { return launch_merge(a, s); }), "merge kernel");
}

attn_status attn_merge_n(int32_t n_parts, const attn_tensor *parts_out, const float *const *parts_lse,
                         const attn_tensor *out, float *lse, void *stream) {
  if (n_parts < 1 || n_parts > 16) return fail(ATTN_ERR_INVALID, "n_parts must be in [1, 16]");
  if (!parts_out || !parts_lse || !lse) return fail(ATTN_ERR_NULL, "NULL argument");
  TRY(check_tensor(out, "out"));
  TRY(check_hd(out->head_dim));
  MergeNArgs a{};
  a.n_parts = n_parts;
  for (int i = 0; i < n_parts; ++i) {
    TRY(check_tensor(&parts_out[i], "parts_out[i]"));
    if (parts_out[i].n_tok != out->n_tok || parts_out[i].n_head != out->n_head || parts_out[i].head_dim != out->head_dim)
      return fail(ATTN_ERR_SHAPE, "parts_out[%d] shape differs from out", i);
    if (!parts_lse[i]) return fail(ATTN_ERR_NULL, "parts_lse[%d] is NULL", i);
    a.pout[i] = parts_out[i].data; a.pdtype[i] = parts_out[i].dtype;
    a.p_st[i] = parts_out[i].stride_tok; a.p_sh[i] = parts_out[i].stride_head;
    a.plse[i] = parts_lse[i];
  }
  a.out = out->data; a.out_dtype = out->dtype; a.o_st = out->stride_tok; a.o_sh = out->stride_head;
  a.lse = lse; a.n = out->n_tok; a.h = out->n_head; a.d = out->head_dim;
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_merge_n", s, [&] { return launch_merge_n(a, s); }), "merge_n kernel");
}

static attn_status diag_common(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, DiagArgs &a) {
  TRY(check_qkv(q, k, v));
  if (k->n_tok != q->n_tok) return fail(ATTN_ERR_SHAPE, "a diagonal block needs k/v rows = q rows");
  if (q->n_tok * q->n_head >= ((int64_t)1 << 31)) return fail(ATTN_ERR_UNSUPPORTED, "rows x heads reach 2^31");
  a = DiagArgs{};
  a.q = q->data; a.k = k->data; a.v = v->data; a.dtype = q->dtype;
  a.q_st = q->stride_tok; a.q_sh = q->stride_head; a.k_st = k->stride_tok; a.k_sh = k->stride_head;
  a.v_st = v->stride_tok; a.v_sh = v->stride_head;
  a.n = (int32_t)q->n_tok; a.hq = (int32_t)q->n_head; a.group = (int32_t)(q->n_head / k->n_head);
  a.d = (int32_t)q->head_dim;
  return ok();
}

attn_status attn_merge_diag(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, float scale,
                            const attn_tensor *out, float *lse, const attn_tensor *final_out, void *stream) {
  DiagArgs a;
  TRY(diag_common(q, k, v, a));
  TRY(check_tensor(out, "out"));
  if (out->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "running out must be f32");
  if (out->n_tok != q->n_tok || out->n_head != q->n_head || out->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "out must be shaped like q");
  if (final_out) {
    TRY(check_tensor(final_out, "final_out"));
    if (final_out->n_tok != q->n_tok || final_out->n_head != q->n_head || final_out->head_dim != q->head_dim)
      return fail(ATTN_ERR_SHAPE, "final_out must be shaped like q");
  }
  if (!lse && q->n_tok > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(ATTN_ERR_INVALID, "scale must be positive and finite");
  a.out = (float *)out->data; a.o_st = out->stride_tok; a.o_sh = out->stride_head; a.lse = lse;
  a.fout = final_out ? final_out->data : nullptr;
  a.fout_dtype = final_out ? final_out->dtype : ATTN_F32;
  a.f_st = final_out ? final_out->stride_tok : 0; a.f_sh = final_out ? final_out->stride_head : 0;
  a.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_merge_diag", s, [&] { return launch_diag_merge(a, s); }), "diagonal merge kernel");
}

attn_status attn_diag_bwd(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                          const float *lse, const float *delta, float scale, const attn_tensor *dq,
                          const attn_tensor *dk, const attn_tensor *dv, void *stream) {
  DiagArgs a;
  TRY(diag_common(q, k, v, a));
  TRY(check_tensor(dout, "dout"));
  if (dout->dtype != q->dtype) return fail(ATTN_ERR_DTYPE, "dout dtype differs from q");
  if (dout->n_tok != q->n_tok || dout->n_head != q->n_head || dout->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "dout must be shaped like q");
  if ((!lse || !delta) && q->n_tok > 0) return fail(ATTN_ERR_NULL, "lse / delta is NULL");
  const attn_tensor *gr[3] = {dq, dk, dv};
  const char *gn[3] = {"dq", "dk", "dv"};
  for (int i = 0; i < 3; ++i) {
    TRY(check_tensor(gr[i], gn[i]));
    if (gr[i]->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "%s must be f32", gn[i]);
  }
  if (dq->n_tok != q->n_tok || dq->n_head != q->n_head || dq->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "dq must be shaped like q");
  for (int i = 1; i < 3; ++i)
    if (gr[i]->n_tok != k->n_tok || gr[i]->n_head != k->n_head || gr[i]->head_dim != k->head_dim)
      return fail(ATTN_ERR_SHAPE, "%s must be shaped like k", gn[i]);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(ATTN_ERR_INVALID, "scale must be positive and finite");
  a.dout = dout->data; a.do_st = dout->stride_tok; a.do_sh = dout->stride_head;
  a.lse = (float *)lse; a.delta = delta;
  a.dq = (float *)dq->data; a.dq_st = dq->stride_tok; a.dq_sh = dq->stride_head;
  a.dk = (float *)dk->data; a.dk_st = dk->stride_tok; a.dk_sh = dk->stride_head;
  a.dv = (float *)dv->data; a.dv_st = dv->stride_tok; a.dv_sh = dv->stride_head;
  a.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_diag_bwd", s, [&] { return launch_diag_bwd(a, s); }), "diagonal backward kernel");
}

attn_status attn_ulysses_reshard(int32_t uly, int32_t to_heads, const attn_tensor *src, const attn_tensor *dst,
                                 void *stream) {
  if (uly < 1 || uly > kMaxUly) return fail(ATTN_ERR_INVALID, "uly must be in [1, %d]", kMaxUly);
  if (!src || !dst) return fail(ATTN_ERR_NULL, "NULL descriptor array");
  for (int r = 0; r < uly; ++r) {
    TRY(check_tensor(&src[r], "src"));
    TRY(check_tensor(&dst[r], "dst"));
    if (src[r].dtype != src[0].dtype || dst[r].dtype != src[0].dtype) return fail(ATTN_ERR_DTYPE, "dtypes differ");
    if (src[r].n_tok != src[0].n_tok || src[r].n_head != src[0].n_head || src[r].head_dim != src[0].head_dim ||
        dst[r].n_tok != dst[0].n_tok || dst[r].n_head != dst[0].n_head || dst[r].head_dim != src[0].head_dim)
      return fail(ATTN_ERR_SHAPE, "every rank's shard must have the same shape");
  }
  const int64_t eb = src[0].dtype == ATTN_F32 ? 4 : 2;
  ReshardArgs a{};
  a.uly = uly; a.to_heads = to_heads ? 1 : 0;
  a.row_bytes = (int32_t)(src[0].head_dim * eb);
  if (to_heads) {  // src [S_l, H, D] -> dst [S, H / uly, D]
    if (src[0].n_head % uly) return fail(ATTN_ERR_SHAPE, "heads must divide by uly");
    if (dst[0].n_tok != src[0].n_tok * uly || dst[0].n_head != src[0].n_head / uly)
      return fail(ATTN_ERR_SHAPE, "head shard must be [S_l * uly, H / uly, D]");
    a.n_local = (int32_t)src[0].n_tok; a.h_local = (int32_t)dst[0].n_head;
  } else {         // src [S, H_l, D] -> dst [S / uly, H_l * uly, D]
    if (src[0].n_tok % uly) return fail(ATTN_ERR_SHAPE, "rows must divide by uly");
    if (dst[0].n_tok * uly != src[0].n_tok || dst[0].n_head != src[0].n_head * uly)
      return fail(ATTN_ERR_SHAPE, "sequence shard must be [S / uly, H_l * uly, D]");
    a.n_local = (int32_t)dst[0].n_tok; a.h_local = (int32_t)src[0].n_head;
  }
  if ((int64_t)a.n_local * uly >= ((int64_t)1 << 31)) return fail(ATTN_ERR_UNSUPPORTED, "2^31 rows or more");
  for (int r = 0; r < uly; ++r) {
    a.src[r] = (const char *)src[r].data; a.s_st[r] = src[r].stride_tok * eb; a.s_sh[r] = src[r].stride_head * eb;
    a.dst[r] = (char *)dst[r].data; a.d_st[r] = dst[r].stride_tok * eb; a.d_sh[r] = dst[r].stride_head * eb;
  }
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_reshard", s, [&] { return launch_reshard(a, s); }), "reshard kernel");
}

attn_status attn_ulysses_reshard_lse(int32_t uly, int32_t to_heads, const float *const *src, float *const *dst,
                                     int64_t n_local, int64_t n_head, void *stream) {
  if (uly < 1 || uly > kMaxUly) return fail(ATTN_ERR_INVALID, "uly must be in [1, %d]", kMaxUly);
  if (!src || !dst) return fail(ATTN_ERR_NULL, "NULL pointer array");
  if (n_local < 0 || n_head <= 0 || n_head % uly) return fail(ATTN_ERR_SHAPE, "heads must divide by uly");
  if (n_local * uly >= ((int64_t)1 << 31)) return fail(ATTN_ERR_UNSUPPORTED, "2^31 rows or more");
  LseReshardArgs a{};
  a.uly = uly; a.to_heads = to_heads ? 1 : 0; a.n_local = (int32_t)n_local; a.h_local = (int32_t)(n_head / uly);
  for (int r = 0; r < uly; ++r) {
    if (!src[r] || !dst[r]) return fail(ATTN_ERR_NULL, "NULL lse pointer");
    a.src[r] = src[r]; a.dst[r] = dst[r];
  }
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_reshard", s, [&] { return launch_lse_reshard(a, s); }), "lse reshard kernel");
}

attn_status attn_out_transpose(const attn_tensor *src, void *dst, void *stream) {
  TRY(check_tensor(src, "src"));
  if (!dst && src->n_tok > 0) return fail(ATTN_ERR_NULL, "dst is NULL");
  if (src->n_tok >= ((int64_t)1 << 31) || src->n_head * src->head_dim >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "sizes reach 2^31");
  TransposeArgs a;
  a.src = src->data; a.s_st = src->stride_tok; a.s_sh = src->stride_head; a.dst = dst;
  a.esize = src->dtype == ATTN_F32 ? 4 : 2;
  a.n = (int32_t)src->n_tok; a.h = (int32_t)src->n_head; a.d = (int32_t)src->head_dim;
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_transpose", s, [&] { return launch_out_transpose(a, s); }), "transpose kernel");
}

}  // extern "C"

namespace {

// delta, and with h16 (bf16 q and dout) the f16 copies of q and dout in the
// same pass over dout
attn_status bwd_delta_impl(const attn_tensor *dout, const attn_tensor *out, float *delta, const attn_tensor *q,
                           const HalfCopies *h16, void *stream) {
  TRY(check_tensor(dout, "dout"));
  TRY(check_tensor(out, "out"));
  TRY(check_hd(out->head_dim));
  if (dout->n_tok != out->n_tok || dout->n_head != out->n_head || dout->head_dim != out->head_dim)
    return fail(ATTN_ERR_SHAPE, "dout/out shapes differ");
  if (!delta && out->n_tok > 0) return fail(ATTN_ERR_NULL, "delta is NULL");
  DeltaArgs a;
  a.dout = dout->data; a.dtype_do = dout->dtype; a.do_st = dout->stride_tok; a.do_sh = dout->stride_head;
  a.out = out->data; a.dtype_o = out->dtype; a.o_st = out->stride_tok; a.o_sh = out->stride_head;
  a.delta = delta; a.n = out->n_tok; a.h = out->n_head; a.d = out->head_dim;
  if (h16 && h16->q16) {
    if (!q || q->dtype != ATTN_BF16 || dout->dtype != ATTN_BF16 || q->n_tok != out->n_tok || q->n_head != out->n_head)
      return fail(ATTN_ERR_INVALID, "internal: f16 copies need bf16 q and dout shaped like out");
    a.q = q->data; a.q_st = q->stride_tok; a.q_sh = q->stride_head;
    a.q16 = h16->q16; a.do16 = h16->do16; a.h16_flag = h16->flag;
  }
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_delta", s, [&] { return launch_delta(a, s); }), "delta kernel");
}

}  // namespace

extern "C" {

attn_status attn_bwd_delta(const attn_tensor *dout, const attn_tensor *out, float *delta, void *stream) {
  return bwd_delta_impl(dout, out, delta, nullptr, nullptr, stream);
}

}  // extern "C"

namespace {

// Schedules and lse2 computed once by a driver for several block backwards.
struct BwdPre {
  SchedBufs sq, sk;
  const float *lse2;
  HalfCopies h16;
};

attn_status block_bwd_impl(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                           const attn_tensor *out, const float *lse, const float *delta, const int32_t *cu_seqlens_q,
                           const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const attn_mask *mask, float scale, const attn_tensor *dq, const attn_tensor *dk,
                           const attn_tensor *dv, void *workspace, size_t workspace_bytes, void *stream,
                           const BwdPre *pre, bool set_q = false, bool set_kv = false, bool check_only = false) {
  TRY(check_qkv(q, k, v));
  TRY(check_mask(mask));
  if (mask && (mask->block_table || mask->seg_size > 0))
    return fail(ATTN_ERR_UNSUPPORTED, "paged keys and segments are forward-only");
  TRY(check_tensor(dout, "dout"));
  if (dout->dtype != q->dtype) return fail(ATTN_ERR_DTYPE, "dout dtype differs from q");
  if (dout->n_tok != q->n_tok || dout->n_head != q->n_head || dout->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "dout must be shaped like q");
  if (!delta) {
    TRY(check_tensor(out, "out"));
    if (out->n_tok != q->n_tok || out->n_head != q->n_head || out->head_dim != q->head_dim)
      return fail(ATTN_ERR_SHAPE, "out must be shaped like q");
  }
  if (!lse && q->n_tok > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  const attn_tensor *gr[3] = {dq, dk, dv};
  const char *gn[3] = {"dq", "dk", "dv"};
  for (int i = 0; i < 3; ++i) {
    TRY(check_tensor(gr[i], gn[i]));
    if (gr[i]->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "%s must be f32", gn[i]);
  }
  if (dq->n_tok != q->n_tok || dq->n_head != q->n_head || dq->head_dim != q->head_dim)
    return fail(ATTN_ERR_SHAPE, "dq must be shaped like q");
  for (int i = 1; i < 3; ++i)
    if (gr[i]->n_tok != k->n_tok || gr[i]->n_head != k->n_head || gr[i]->head_dim != k->head_dim)
      return fail(ATTN_ERR_SHAPE, "%s must be shaped like k", gn[i]);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative sizes");
  if (num_seqs > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(ATTN_ERR_INVALID, "scale must be positive and finite");
  TRY(check_ranges(q, k, v, mask, k->n_tok));
  if (dout->stride_tok >= (1 << 22)) return fail(ATTN_ERR_UNSUPPORTED, "a row stride of 2^22 elements or more");
  const int64_t capq = sched_capacity(q->n_tok, num_seqs, kBwdTile, 1);
  const int64_t capk = sched_capacity(k->n_tok, num_seqs, kBwdTile, 1);
  if (pre) {
    if (!delta) return fail(ATTN_ERR_INVALID, "internal: precomputed schedules need delta");
  } else {
    const size_t need = bwd_ws_bytes(q->n_tok, k->n_tok, q->n_head, q->head_dim, q->dtype, num_seqs, delta == nullptr);
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (((uintptr_t)workspace) % 256) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  hipStream_t s = (hipStream_t)stream;
  if (check_only || num_seqs == 0 || q->n_tok == 0 || k->n_tok == 0) return ok();

  MaskDev md = mask_dev(mask);
  SchedBufs sq, sk;
  const float *lse2;
  HalfCopies h16;
  if (pre) {
    if (pre->sq.capacity != capq || pre->sk.capacity != capk)
      return fail(ATTN_ERR_INVALID, "internal: schedule capacity differs");
    sq = pre->sq; sk = pre->sk; lse2 = pre->lse2; h16 = pre->h16;
  } else {
    char *w = (char *)workspace;
    sq = sched_carve(w, capq);
    w += align256(sched_bytes(capq));
    sk = sched_carve(w, capk);
    w += align256(sched_bytes(capk));
    float *l2 = (float *)w;
    w += align256((size_t)q->n_head * q->n_tok * 4);
    float *dl = nullptr;
    if (!delta) {
      dl = (float *)w;
      w += align256((size_t)q->n_head * q->n_tok * 4);
    }
    if (q->dtype == ATTN_BF16) h16 = half_carve(w, q->n_tok, q->n_head, q->head_dim);
    // lse2 first: it zeroes the f16 range flag the copies may set
    TRY(hip_check(timed("attn_lse2", s, [&] { return launch_lse2(lse, l2, q->n_head * q->n_tok, s, h16.flag); }),
                  "lse2"));
    lse2 = l2;
    if (dl) {
      TRY(bwd_delta_impl(dout, out, dl, q, &h16, stream));  // with the f16 copies in the same pass
      delta = dl;
    } else if (h16.q16) {
      TRY(hip_check(timed("attn_half_copy", s, [&] { return launch_half_copies(h16, q, dout, s); }), "f16 copies"));
    }
    const SchedJob jobs[2] = {
        {cu_seqlens_q, cu_seqlens_k, num_seqs, q->n_tok, k->n_tok, md, kBwdTile, kFwdBN, 0, 1, sq},
        {cu_seqlens_q, cu_seqlens_k, num_seqs, q->n_tok, k->n_tok, md, kBwdTile, kBwdBQ, 1, 1, sk}};
    TRY(hip_check(timed("attn_sched", s, [&] { return launch_schedules(jobs, 2, s); }), "scheduler"));
  }
  BwdArgs a;
  a.q = tdev(q); a.k = tdev(k); a.v = tdev(v); a.dout = tdev(dout);
  a.dtype = q->dtype; a.head_dim = (int32_t)q->head_dim; a.hq = (int32_t)q->n_head; a.hkv = (int32_t)k->n_head;
  a.scale = scale; a.mask = md; a.lse = lse; a.delta = delta; a.lse2 = lse2; a.n_q = q->n_tok; a.n_k = k->n_tok;
  a.dq = (float *)dq->data; a.dq_st = dq->stride_tok; a.dq_sh = dq->stride_head;
  a.dk = (float *)dk->data; a.dk_st = dk->stride_tok; a.dk_sh = dk->stride_head;
  a.dv = (float *)dv->data; a.dv_st = dv->stride_tok; a.dv_sh = dv->stride_head;
  a.qsched = sq; a.ksched = sk; a.q_items = capq; a.k_items = capk;
  a.set_q = set_q; a.set_kv = set_kv;
  a.q16 = h16.q16; a.do16 = h16.do16; a.h16_flag = h16.flag;
  TRY(hip_check(timed("attn_dkdv", s, [&] { return launch_bwd(a, 0, s); }), "dK/dV kernel"));
  return hip_check(timed("attn_dq", s, [&] { return launch_bwd(a, 1, s); }), "dQ kernel");
}

}  // namespace

extern "C" {

attn_status attn_block_bwd(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                           const attn_tensor *out, const float *lse, const float *delta, const int32_t *cu_seqlens_q,
                           const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const attn_mask *mask, float scale, const attn_tensor *dq, const attn_tensor *dk,
                           const attn_tensor *dv, void *workspace, size_t workspace_bytes, void *stream) {
  return block_bwd_impl(dout, q, k, v, out, lse, delta, cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q,
                        max_seqlen_k, mask, scale, dq, dk, dv, workspace, workspace_bytes, stream, nullptr);
}

attn_status attn_zigzag_shard(const attn_tensor *src, const int32_t *cu_seqlens_global, int32_t num_seqs,
                              int32_t max_seqlen, int32_t cp, int32_t rank, const attn_tensor *dst, void *stream) {
  TRY(check_tensor(src, "src"));
  TRY(check_tensor(dst, "dst"));
  if (cp < 1 || rank < 0 || rank >= cp) return fail(ATTN_ERR_INVALID, "need 0 <= rank < cp");
  if (src->dtype != dst->dtype || src->n_head != dst->n_head || src->head_dim != dst->head_dim)
    return fail(ATTN_ERR_SHAPE, "src/dst differ in dtype or head layout");
  if ((src->head_dim * esize(src->dtype)) % 16) return fail(ATTN_ERR_LAYOUT, "head rows must be 16-byte multiples");
  if (dst->n_tok * cp != src->n_tok) return fail(ATTN_ERR_SHAPE, "dst must hold n_src / cp rows");
  if (num_seqs < 0 || max_seqlen < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative sizes");
  if (num_seqs > 0 && !cu_seqlens_global) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  hipStream_t s = (hipStream_t)stream;
  return hip_check(timed("attn_zigzag_shard", s, [&] { return launch_zigzag_shard(src->data, src->stride_tok, src->stride_head, src->n_tok, dst->data,
                                       dst->stride_tok, dst->stride_head, dst->n_tok, esize(src->dtype),
                                       src->n_head, src->head_dim, cu_seqlens_global, num_seqs, max_seqlen, cp,
                                       rank, s); }),
                   "zigzag shard kernel");
}

// ---------------------------------------------------------------------------
// virtual-rank schedules
// ---------------------------------------------------------------------------
namespace {

attn_mask make_mask(uint32_t causal, uint32_t qv, uint32_t kv) {
  attn_mask m;
  memset(&m, 0, sizeof m);
  m.struct_size = sizeof(attn_mask);
  m.causal = causal;
  m.q_view = qv;
  m.k_view = kv;
  return m;
}

// Block kind of rank r at zig-zag step s (src = (r - s) mod cp):
// s == 0 causal over own rows; src < r: all q rows x src's front halves;
// src > r: q back halves x all of src's rows (both unmasked).
attn_mask zigzag_mask(int cp, int r, int s) {
  (void)cp;
  if (s == 0) return make_mask(1, ATTN_VIEW_ALL, ATTN_VIEW_ALL);
  if (s <= r) return make_mask(0, ATTN_VIEW_ALL, ATTN_VIEW_FRONT);
  return make_mask(0, ATTN_VIEW_BACK, ATTN_VIEW_ALL);
}

// The distinct block kinds (masks) of a ring schedule: at most three (the
// diagonal block, and one or two off-diagonal kinds), so the schedules of all
// steps are computed up front, in one launch.
constexpr int kRingKinds = 3;

struct RingLayout {
  size_t bout_off, blse_off, fwd_off, fsched_off, total;  // forward
  size_t delta_off, lse2_off, bsched_off, h16_off, btotal;  // backward
  int64_t fcap, qcap, kcap;
  size_t fsched_stride, bsched_stride;
};

RingLayout ring_layout(const attn_tensor *q, const attn_tensor *k, int32_t num_seqs) {
  Problem P;
  P.n_q = q->n_tok; P.hq = q->n_head; P.hkv = k->n_head; P.d = q->head_dim; P.nseg = 0; P.decode = false;
  P.paged = false; P.n_k_logical = k->n_tok;
  RingLayout L;
  L.bout_off = 0;
  L.blse_off = align256((size_t)q->n_tok * q->n_head * q->head_dim * esize(q->dtype));
  L.fwd_off = L.blse_off + align256((size_t)q->n_head * q->n_tok * 4);
  L.fsched_off = L.fwd_off + fwd_ws_bytes(P, num_seqs);
  L.fcap = sched_capacity(q->n_tok, num_seqs, kFwdBM, 0);
  L.fsched_stride = align256(sched_bytes(L.fcap));
  L.total = L.fsched_off + kRingKinds * L.fsched_stride;
  L.qcap = sched_capacity(q->n_tok, num_seqs, kBwdTile, 1);
  L.kcap = sched_capacity(k->n_tok, num_seqs, kBwdTile, 1);
  L.bsched_stride = align256(sched_bytes(L.qcap)) + align256(sched_bytes(L.kcap));
  L.delta_off = 0;
  L.lse2_off = align256((size_t)q->n_head * q->n_tok * 4);
  L.bsched_off = 2 * L.lse2_off;
  L.h16_off = L.bsched_off + kRingKinds * L.bsched_stride;
  L.btotal = L.h16_off + half_copy_bytes(q->n_tok, q->n_head, q->head_dim, q->dtype);
  return L;
}

// Masks of steps 0..n_steps-1 and the kind (index of the first equal mask) of each.
attn_status ring_kinds(int32_t cp, int32_t rank, int32_t n_steps, attn_mask (*mk)(int, int, int),
                       std::vector<attn_mask> &masks, std::vector<int> &kind_of, std::vector<attn_mask> &kinds) {
  masks.resize(n_steps);
  kind_of.resize(n_steps);
  kinds.clear();
  for (int s = 0; s < n_steps; ++s) {
    masks[s] = mk(cp, rank, s);
    int k = 0;
    while (k < (int)kinds.size() && memcmp(&kinds[k], &masks[s], sizeof(attn_mask))) ++k;
    if (k == (int)kinds.size()) {
      if (k == kRingKinds) return fail(ATTN_ERR_INVALID, "internal: more than %d block kinds", kRingKinds);
      kinds.push_back(masks[s]);
    }
    kind_of[s] = k;
  }
  return ok();
}

typedef attn_mask (*StepMask)(int cp, int r, int s);

attn_mask ring_mask(int cp, int r, int s) {
  (void)cp; (void)r;
  return make_mask(s == 0 ? 1 : 0, ATTN_VIEW_ALL, ATTN_VIEW_ALL);
}

attn_status check_ring_args(int32_t cp, int32_t rank, const attn_tensor *q, const attn_tensor *k_loc,
                            const attn_tensor *v_loc) {
  if (cp < 1 || rank < 0 || rank >= cp) return fail(ATTN_ERR_INVALID, "need 0 <= rank < cp");
  if (!k_loc || !v_loc) return fail(ATTN_ERR_NULL, "k_loc/v_loc is NULL");
  for (int i = 0; i < cp; ++i) {
    TRY(check_qkv(q, &k_loc[i], &v_loc[i]));
    if (k_loc[i].n_tok != q->n_tok) return fail(ATTN_ERR_SHAPE, "every rank's local K/V must have n_loc rows");
  }
  return ok();
}

attn_status run_ring_fwd(int32_t cp, int32_t rank, int32_t n_steps, StepMask mk, const attn_tensor *q,
                         const attn_tensor *k_loc, const attn_tensor *v_loc, const int32_t *cu, int32_t num_seqs,
                         int32_t max_local, float scale, const attn_tensor *out_acc, const attn_tensor *out,
                         float *lse, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_ring_args(cp, rank, q, k_loc, v_loc));
  TRY(check_tensor(out_acc, "out_acc"));
  if (out_acc->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "out_acc must be f32");
  TRY(check_tensor(out, "out"));
  if (num_seqs < 0 || max_local < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative num_seqs or max_seqlen");
  if (num_seqs > 0 && !cu) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  RingLayout L = ring_layout(q, &k_loc[0], num_seqs);
  if (!ws || ws_bytes < L.total) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed", L.total);
  if (((uintptr_t)ws) % 256) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  char *w = (char *)ws;
  attn_tensor bout = *q;
  bout.data = w + L.bout_off;
  bout.stride_head = q->head_dim;
  bout.stride_tok = q->n_head * q->head_dim;
  float *blse = (float *)(w + L.blse_off);
  void *fws = w + L.fwd_off;
  const size_t fws_bytes = L.fsched_off - L.fwd_off;
  Problem shp;
  shp.n_q = q->n_tok; shp.hq = q->n_head; shp.d = q->head_dim;
  TRY(check_out(out_acc, shp, "out_acc"));
  hipStream_t st = (hipStream_t)stream;
  // bf16: every block works on the running state in the forward's epilogue
  const bool fuse = can_fuse_merge(q, max_local, nullptr);
  // the tiled forward's schedules of every block kind, in one launch (the
  // one-query decode path needs none)
  std::vector<attn_mask> masks, kinds;
  std::vector<int> kind_of;
  TRY(ring_kinds(cp, rank, n_steps, mk, masks, kind_of, kinds));
  std::vector<SchedBufs> sch(kinds.size());
  const bool presched = max_local != 1 && num_seqs > 0 && q->n_tok > 0;
  if (presched) {
    SchedJob jobs[kRingKinds];
    for (size_t i = 0; i < kinds.size(); ++i) {
      TRY(check_mask(&kinds[i]));
      sch[i] = sched_carve(w + L.fsched_off + i * L.fsched_stride, L.fcap);
      jobs[i] = SchedJob{cu, cu, num_seqs, q->n_tok, k_loc[0].n_tok, mask_dev(&kinds[i]), kFwdBM, kFwdBN, 0, 1, sch[i]};
    }
    TRY(hip_check(timed("attn_sched", st, [&] { return launch_schedules(jobs, (int)kinds.size(), st); }),
                  "scheduler"));
  }
  // the last step that updates each half of the documents' rows: there the
  // fused epilogue writes the final output of that half
  int last_front = -1, last_back = -1;
  for (int s = 0; s < n_steps; ++s) {
    if (masks[s].q_view != ATTN_VIEW_BACK) last_front = s;
    if (masks[s].q_view != ATTN_VIEW_FRONT) last_back = s;
  }
  for (int s = 0; s < n_steps; ++s) {
    const int src = ((rank - s) % cp + cp) % cp;
    const attn_mask &m = masks[s];
    const SchedBufs *pre = presched ? &sch[kind_of[s]] : nullptr;
    const bool last = s == n_steps - 1;
    if (fuse) {
      const FusedMerge fm{out_acc, s > 0, (s == last_front ? 1 : 0) | (s == last_back ? 2 : 0)};
      TRY(block_fwd_impl(q, &k_loc[src], &v_loc[src], cu, cu, num_seqs, max_local, max_local, &m, scale, out, lse,
                         fws, fws_bytes, stream, &fm, pre, false));
      continue;
    }
    if (s == 0) {
      // the first block initialises the running state
      const attn_tensor *dst = (n_steps == 1) ? out : out_acc;
      TRY(block_fwd_impl(q, &k_loc[src], &v_loc[src], cu, cu, num_seqs, max_local, max_local, &m, scale, dst, lse,
                         fws, fws_bytes, stream, nullptr, pre, false));
      continue;
    }
    TRY(block_fwd_impl(q, &k_loc[src], &v_loc[src], cu, cu, num_seqs, max_local, max_local, &m, scale, &bout, blse,
                       fws, fws_bytes, stream, nullptr, pre, false));
    TRY(attn_merge_out_lse(out_acc, lse, &bout, blse, cu, num_seqs, m.q_view, nullptr, last ? out : nullptr, 0,
                           stream));
  }
  return ok();
}

attn_status run_ring_bwd(int32_t cp, int32_t rank, int32_t n_steps, StepMask mk, const attn_tensor *dout,
                         const attn_tensor *q, const attn_tensor *k_loc, const attn_tensor *v_loc,
                         const attn_tensor *out, const float *lse, const int32_t *cu, int32_t num_seqs,
                         int32_t max_local, float scale, const attn_tensor *dq, const attn_tensor *dk_loc,
                         const attn_tensor *dv_loc, void *ws, size_t ws_bytes, void *stream, uint32_t flags = 0) {
  TRY(check_ring_args(cp, rank, q, k_loc, v_loc));
  if (!dk_loc || !dv_loc) return fail(ATTN_ERR_NULL, "dk_loc/dv_loc is NULL");
  TRY(check_tensor(out, "out"));
  if (!lse && q->n_tok > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  if (num_seqs < 0 || max_local < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative num_seqs or max_seqlen");
  if (num_seqs > 0 && !cu) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  const RingLayout L = ring_layout(q, &k_loc[0], num_seqs);
  if (!ws || ws_bytes < L.btotal) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed", L.btotal);
  if (((uintptr_t)ws) % 256) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  char *w = (char *)ws;
  float *delta = (float *)(w + L.delta_off);
  float *lse2 = (float *)(w + L.lse2_off);
  hipStream_t st = (hipStream_t)stream;
  std::vector<attn_mask> masks, kinds;
  std::vector<int> kind_of;
  TRY(ring_kinds(cp, rank, n_steps, mk, masks, kind_of, kinds));
  for (size_t i = 0; i < kinds.size(); ++i) TRY(check_mask(&kinds[i]));
  const bool set = (flags & ATTN_BWD_SET) != 0;
  std::vector<ZeroRows> z;
  if (set) {
    // Every step's source is a different rank, so each block stores its dK / dV
    // into its owner's buffers, and step 0 (the diagonal block: every row of
    // every document) stores dq; what no block writes is zeroed before them.
    if (masks[0].q_view != ATTN_VIEW_ALL) return fail(ATTN_ERR_INVALID, "internal: step 0 must see every row");
    if (2 * cp + 1 > kMaxZeroRows) return fail(ATTN_ERR_UNSUPPORTED, "cp above %d with ATTN_BWD_SET", (kMaxZeroRows - 1) / 2);
    auto zr = [&](const attn_tensor *t, int32_t view) {
      z.push_back(ZeroRows{(float *)t->data, t->stride_tok, t->stride_head, t->n_tok, (int32_t)t->n_head,
                           (int32_t)t->head_dim, view});
    };
    // the zeroing writes f32 rows of every buffer, used by a block or not
    auto like = [&](const attn_tensor *t, const attn_tensor *ref, const char *name) -> attn_status {
      TRY(check_tensor(t, name));
      if (t->dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "%s must be f32", name);
      if (t->n_tok != ref->n_tok || t->n_head != ref->n_head || t->head_dim != ref->head_dim)
        return fail(ATTN_ERR_SHAPE, "%s must be shaped like its tensor", name);
      return ok();
    };
    TRY(like(dq, q, "dq"));
    zr(dq, 0);
    std::vector<int32_t> view_of(cp, 3);  // never a source: every row
    for (int s = 0; s < n_steps; ++s) view_of[((rank - s) % cp + cp) % cp] = (int32_t)masks[s].k_view;
    for (int c = 0; c < cp; ++c) {
      TRY(like(&dk_loc[c], &k_loc[c], "dk_loc"));
      TRY(like(&dv_loc[c], &v_loc[c], "dv_loc"));
      zr(&dk_loc[c], view_of[c]);
      zr(&dv_loc[c], view_of[c]);
    }
  }
  const BwdPre none{};
  for (int s = 0; s < n_steps; ++s) {  // every block's arguments, before anything is launched
    const int src = ((rank - s) % cp + cp) % cp;
    TRY(block_bwd_impl(dout, q, &k_loc[src], &v_loc[src], out, lse, delta, cu, cu, num_seqs, max_local, max_local,
                       &masks[s], scale, dq, &dk_loc[src], &dv_loc[src], nullptr, 0, stream, &none, false, false,
                       true));
  }
  std::vector<BwdPre> pre(kinds.size());
  HalfCopies h16;
  if (num_seqs > 0 && q->n_tok > 0 && q->dtype == ATTN_BF16) h16 = half_carve(w + L.h16_off, q->n_tok, q->n_head, q->head_dim);
  if (num_seqs > 0 && q->n_tok > 0)  // lse2 first: it zeroes the f16 range flag the delta pass may set
    TRY(hip_check(timed("attn_lse2", st, [&] { return launch_lse2(lse, lse2, q->n_head * q->n_tok, st, h16.flag); }),
                  "lse2"));
  TRY(bwd_delta_impl(dout, out, delta, q, &h16, stream));  // delta and the f16 copies in one pass
  if (num_seqs > 0 && q->n_tok > 0) {
    for (auto &pr : pre) pr.h16 = h16;
    SchedJob jobs[2 * kRingKinds];
    for (size_t i = 0; i < kinds.size(); ++i) {
      char *b = w + L.bsched_off + i * L.bsched_stride;
      pre[i].sq = sched_carve(b, L.qcap);
      pre[i].sk = sched_carve(b + align256(sched_bytes(L.qcap)), L.kcap);
      pre[i].lse2 = lse2;
      const MaskDev md = mask_dev(&kinds[i]);
      jobs[2 * i] = SchedJob{cu, cu, num_seqs, q->n_tok, k_loc[0].n_tok, md, kBwdTile, kFwdBN, 0, 1, pre[i].sq};
      jobs[2 * i + 1] = SchedJob{cu, cu, num_seqs, q->n_tok, k_loc[0].n_tok, md, kBwdTile, kBwdBQ, 1, 1, pre[i].sk};
    }
    TRY(hip_check(timed("attn_sched", st, [&] { return launch_schedules(jobs, 2 * (int)kinds.size(), st); }),
                  "scheduler"));
  }
  if (set) {
    TRY(hip_check(timed("attn_zero_rows", st, [&] { return launch_zero_rows(z.data(), (int)z.size(), cu, num_seqs, st); }),
                  "zero rows"));
  }
  for (int s = 0; s < n_steps; ++s) {
    const int src = ((rank - s) % cp + cp) % cp;
    TRY(block_bwd_impl(dout, q, &k_loc[src], &v_loc[src], out, lse, delta, cu, cu, num_seqs, max_local, max_local,
                       &masks[s], scale, dq, &dk_loc[src], &dv_loc[src], nullptr, 0, stream, &pre[kind_of[s]],
                       set && s == 0, set));
  }
  return ok();
}

}  // namespace

attn_status attn_zigzag_workspace_size(int32_t cp, const attn_tensor *q, const attn_tensor *k, int32_t num_seqs,
                                       int32_t max_seqlen_local, size_t *bytes) {
  if (!bytes) return fail(ATTN_ERR_NULL, "bytes is NULL");
  if (cp < 1) return fail(ATTN_ERR_INVALID, "cp must be >= 1");
  TRY(check_tensor(q, "q"));
  TRY(check_tensor(k, "k"));
  (void)max_seqlen_local;
  const RingLayout L = ring_layout(q, k, num_seqs);
  *bytes = L.total > L.btotal ? L.total : L.btotal;
  return ok();
}

attn_status attn_zigzag_fwd(int32_t cp, int32_t rank, const attn_tensor *q, const attn_tensor *k_loc,
                            const attn_tensor *v_loc, const int32_t *cu_local, int32_t num_seqs,
                            int32_t max_seqlen_local, float scale, const attn_tensor *out_acc, const attn_tensor *out,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  return run_ring_fwd(cp, rank, cp, zigzag_mask, q, k_loc, v_loc, cu_local, num_seqs, max_seqlen_local, scale, out_acc,
                      out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_zigzag_fwd_ranks(int32_t cp, int32_t n_ranks, const int32_t *ranks, const attn_tensor *q,
                                  const attn_tensor *k_loc, const attn_tensor *v_loc, const int32_t *cu_local,
                                  int32_t num_seqs, int32_t max_seqlen_local, float scale, const attn_tensor *out_acc,
                                  const attn_tensor *out, float *const *lse, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  if (n_ranks < 1 || n_ranks > cp) return fail(ATTN_ERR_INVALID, "need 1 <= n_ranks <= cp");
  if (!q || !out_acc || !out || !lse) return fail(ATTN_ERR_NULL, "NULL rank array");
  std::vector<int32_t> rk(n_ranks);
  for (int i = 0; i < n_ranks; ++i) {
    rk[i] = ranks ? ranks[i] : i;
    if (rk[i] < 0 || rk[i] >= cp) return fail(ATTN_ERR_INVALID, "ranks[%d] = %d outside [0, cp)", i, rk[i]);
    for (int j = 0; j < i; ++j)
      if (rk[j] == rk[i]) return fail(ATTN_ERR_INVALID, "rank %d listed twice", rk[i]);
    if (q[i].n_tok != q[0].n_tok || q[i].n_head != q[0].n_head || q[i].head_dim != q[0].head_dim ||
        q[i].dtype != q[0].dtype)
      return fail(ATTN_ERR_SHAPE, "every rank's q must be shaped like q[0]");
  }
  TRY(check_tensor(&q[0], "q"));
  TRY(check_ring_args(cp, rk[0], &q[0], k_loc, v_loc));
  const RingLayout L = ring_layout(&q[0], &k_loc[0], num_seqs);
  const size_t slice = align256(L.total > L.btotal ? L.total : L.btotal);
  if (!workspace || workspace_bytes < slice * n_ranks)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (n_ranks x attn_zigzag_workspace_size)",
                slice * n_ranks);
  if (((uintptr_t)workspace) % 256) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  char *w = (char *)workspace;
  const bool batch = can_fuse_merge(&q[0], max_seqlen_local, nullptr) && num_seqs > 0 && q[0].n_tok > 0;
  if (!batch) {  // f32 inputs, one query a document, or nothing to do: the ranks one after another
    for (int i = 0; i < n_ranks; ++i)
      TRY(run_ring_fwd(cp, rk[i], cp, zigzag_mask, &q[i], k_loc, v_loc, cu_local, num_seqs, max_seqlen_local, scale,
                       &out_acc[i], &out[i], lse[i], w + i * slice, slice, stream));
    return ok();
  }
  hipStream_t st = (hipStream_t)stream;
  // every rank's arguments checked, and its block kinds' schedules computed (all ranks' in few launches)
  std::vector<std::vector<attn_mask>> masks(n_ranks), kinds(n_ranks);
  std::vector<std::vector<int>> kind_of(n_ranks);
  std::vector<std::vector<SchedBufs>> sch(n_ranks);
  std::vector<SchedJob> jobs;
  std::vector<int> last_front(n_ranks, -1), last_back(n_ranks, -1);
  for (int i = 0; i < n_ranks; ++i) {
    TRY(check_ring_args(cp, rk[i], &q[i], k_loc, v_loc));
    TRY(check_tensor(&out_acc[i], "out_acc"));
    if (out_acc[i].dtype != ATTN_F32) return fail(ATTN_ERR_DTYPE, "out_acc must be f32");
    TRY(check_tensor(&out[i], "out"));
    if (!lse[i]) return fail(ATTN_ERR_NULL, "lse[%d] is NULL", i);
    if (!cu_local) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
    Problem shp;
    shp.n_q = q[i].n_tok; shp.hq = q[i].n_head; shp.d = q[i].head_dim;
    TRY(check_out(&out_acc[i], shp, "out_acc"));
    TRY(ring_kinds(cp, rk[i], cp, zigzag_mask, masks[i], kind_of[i], kinds[i]));
    sch[i].resize(kinds[i].size());
    for (size_t k = 0; k < kinds[i].size(); ++k) {
      TRY(check_mask(&kinds[i][k]));
      sch[i][k] = sched_carve(w + i * slice + L.fsched_off + k * L.fsched_stride, L.fcap);
      jobs.push_back(SchedJob{cu_local, cu_local, num_seqs, q[i].n_tok, k_loc[0].n_tok, mask_dev(&kinds[i][k]), kFwdBM,
                              kFwdBN, 0, 1, sch[i][k]});
    }
    for (int s = 0; s < cp; ++s) {
      if (masks[i][s].q_view != ATTN_VIEW_BACK) last_front[i] = s;
      if (masks[i][s].q_view != ATTN_VIEW_FRONT) last_back[i] = s;
    }
  }
  for (size_t j0 = 0; j0 < jobs.size(); j0 += kMaxSchedJobs) {
    const int nj = (int)(jobs.size() - j0 < (size_t)kMaxSchedJobs ? jobs.size() - j0 : kMaxSchedJobs);
    TRY(hip_check(timed("attn_sched", st, [&] { return launch_schedules(jobs.data() + j0, nj, st); }), "scheduler"));
  }
  // step by step: the ranks' blocks of one step in one launch (a step's
  // blocks are all causal (step 0) or all unmasked, of one shape)
  std::vector<FwdArgs> fa(n_ranks);
  for (int s = 0; s < cp; ++s) {
    for (int i = 0; i < n_ranks; ++i) {
      const int src = ((rk[i] - s) % cp + cp) % cp;
      const FusedMerge fm{&out_acc[i], s > 0, (s == last_front[i] ? 1 : 0) | (s == last_back[i] ? 2 : 0)};
      TRY(block_fwd_impl(&q[i], &k_loc[src], &v_loc[src], cu_local, cu_local, num_seqs, max_seqlen_local,
                         max_seqlen_local, &masks[i][s], scale, &out[i], lse[i], w + i * slice + L.fwd_off,
                         L.fsched_off - L.fwd_off, stream, &fm, &sch[i][kind_of[i][s]], false, nullptr, &fa[i]));
    }
    for (int i0 = 0; i0 < n_ranks; i0 += kMaxFwdBatch) {
      const int nb = n_ranks - i0 < kMaxFwdBatch ? n_ranks - i0 : kMaxFwdBatch;
      if (fwd_batchable(fa.data() + i0, nb)) {
        TRY(hip_check(timed("attn_fwd", st, [&] { return launch_fwd_batch(fa.data() + i0, nb, st); }),
                      "forward kernel"));
      } else {
        for (int i = i0; i < i0 + nb; ++i)
          TRY(hip_check(timed("attn_fwd", st, [&] { return launch_fwd(fa[i], st); }), "forward kernel"));
      }
    }
  }
  return ok();
}

attn_status attn_zigzag_bwd(int32_t cp, int32_t rank, const attn_tensor *dout, const attn_tensor *q,
                            const attn_tensor *k_loc, const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                            const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local, float scale,
                            const attn_tensor *dq, const attn_tensor *dk_loc, const attn_tensor *dv_loc,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return attn_zigzag_bwd_ex(cp, rank, dout, q, k_loc, v_loc, out, lse, cu_local, num_seqs, max_seqlen_local, scale, dq,
                            dk_loc, dv_loc, workspace, workspace_bytes, stream, 0);
}

attn_status attn_zigzag_bwd_ex(int32_t cp, int32_t rank, const attn_tensor *dout, const attn_tensor *q,
                               const attn_tensor *k_loc, const attn_tensor *v_loc, const attn_tensor *out,
                               const float *lse, const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                               float scale, const attn_tensor *dq, const attn_tensor *dk_loc, const attn_tensor *dv_loc,
                               void *workspace, size_t workspace_bytes, void *stream, uint32_t flags) {
  if (flags & ~(uint32_t)ATTN_BWD_SET) return fail(ATTN_ERR_INVALID, "unknown flags 0x%x", flags);
  return run_ring_bwd(cp, rank, cp, zigzag_mask, dout, q, k_loc, v_loc, out, lse, cu_local, num_seqs, max_seqlen_local,
                      scale, dq, dk_loc, dv_loc, workspace, workspace_bytes, stream, flags);
}

attn_status attn_ring_fwd(int32_t cp, int32_t rank, const attn_tensor *q, const attn_tensor *k_loc,
                          const attn_tensor *v_loc, const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                          float scale, const attn_tensor *out_acc, const attn_tensor *out, float *lse, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (cp < 1 || rank < 0 || rank >= cp) return fail(ATTN_ERR_INVALID, "need 0 <= rank < cp");
  return run_ring_fwd(cp, rank, rank + 1, ring_mask, q, k_loc, v_loc, cu_local, num_seqs, max_seqlen_local, scale,
                      out_acc, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_ring_bwd(int32_t cp, int32_t rank, const attn_tensor *dout, const attn_tensor *q,
                          const attn_tensor *k_loc, const attn_tensor *v_loc, const attn_tensor *out, const float *lse,
                          const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local, float scale,
                          const attn_tensor *dq, const attn_tensor *dk_loc, const attn_tensor *dv_loc, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return attn_ring_bwd_ex(cp, rank, dout, q, k_loc, v_loc, out, lse, cu_local, num_seqs, max_seqlen_local, scale, dq,
                          dk_loc, dv_loc, workspace, workspace_bytes, stream, 0);
}

attn_status attn_ring_bwd_ex(int32_t cp, int32_t rank, const attn_tensor *dout, const attn_tensor *q,
                             const attn_tensor *k_loc, const attn_tensor *v_loc, const attn_tensor *out,
                             const float *lse, const int32_t *cu_local, int32_t num_seqs, int32_t max_seqlen_local,
                             float scale, const attn_tensor *dq, const attn_tensor *dk_loc, const attn_tensor *dv_loc,
                             void *workspace, size_t workspace_bytes, void *stream, uint32_t flags) {
  if (cp < 1 || rank < 0 || rank >= cp) return fail(ATTN_ERR_INVALID, "need 0 <= rank < cp");
  if (flags & ~(uint32_t)ATTN_BWD_SET) return fail(ATTN_ERR_INVALID, "unknown flags 0x%x", flags);
  return run_ring_bwd(cp, rank, rank + 1, ring_mask, dout, q, k_loc, v_loc, out, lse, cu_local, num_seqs,
                      max_seqlen_local, scale, dq, dk_loc, dv_loc, workspace, workspace_bytes, stream, flags);
}

// KV-parallel: all R ranks' key parts in one buffer, merged by one pass (the
// same merge as parts then ranks, one launch instead of R + 1), when that
// buffer stays within 1 GiB; else each rank merges its parts and the ranks
// merge after.
static size_t kvp_parts_bytes(int32_t R, const Problem &P) {
  const int64_t n = (int64_t)R * (P.nseg > 0 ? P.nseg : 1);
  return align256((size_t)n * P.n_q * P.hq * P.d * 4) + align256((size_t)n * P.hq * P.n_q * 4);
}
static bool kvp_all_parts(int32_t R, const Problem &P) { return kvp_parts_bytes(R, P) <= ((size_t)1 << 30); }
// the R ranks' tile schedules (computed in one launch)
static size_t kvp_sched_bytes(int32_t R, const Problem &P, int32_t num_seqs) {
  return (size_t)R * align256(sched_bytes(sched_capacity(P.n_q, num_seqs, kFwdBM, P.nseg > 0 ? P.nseg : 1)));
}
// the R ranks' gathered K and V (contiguous logical rows; gathered in one launch)
static size_t kvp_gather_bytes(int32_t R, const Problem &P) {
  return (size_t)R * 2 * align256((size_t)P.n_k_logical * P.gather_row_bytes);
}

// The KV-parallel entries are always paged: the tables come in their own
// block_tables argument, so mask->block_table is ignored and the plan is made
// for paged keys (a host address stands in as the non-NULL table: plan_fwd
// only tests it, nothing dereferences it).
static const int32_t kKvpTableMarker[1] = {0};
static attn_mask kvp_paged_mask(const attn_mask *m) {
  attn_mask mk = *m;
  mk.block_table = kKvpTableMarker;
  return mk;
}

// The R ranks' forwards run as one batched launch, so a rank's keys need
// fewer parts than its own grid would ask for (the plan counts one rank's
// work items): at most the plan's count, and no more than keeps about
// kKvpItems work items over all R ranks. Every part a row sees is read by the
// one merge of the R ranks' parts, and each part costs its work item a
// prologue and an epilogue. (KV-parallel prefill of 2048 rows x 8 heads, R = 4: 16 parts a rank -> 3: W = 0 1.30 -> 1.08 ms,
// W = 4096 0.246 -> 0.170 ms; the merge 193 -> ~30 us.)
constexpr int64_t kKvpItems = 1536;
// A window bounds the keys one item's rows see on one rank: about window / R
// with round-robin keys, up to the window with contiguous ones. A part shorter
// than kKvpMinPartKeys only adds a prologue, an epilogue and merge reads
// (the prefill above with W = 4096, round-robin: 3 parts -> 1 part a rank,
// 0.173 -> 0.157 ms, the forward kernel unchanged and the merge 30 -> 16 us).
constexpr int64_t kKvpMinPartKeys = 1024;
// Returns the batched path's problem: kvp_all_parts(R, result) && result.gather
// selects it, else the ranks run one by one on the unadjusted plan.
Problem kvp_parts(int32_t R, Problem P, int32_t num_seqs, const attn_mask *m) {
  if (P.nseg <= 1) return P;
  const int64_t wgs = ((int64_t)P.n_q / kFwdBM + num_seqs) * P.hq * R;
  int64_t n = wgs > 0 ? (kKvpItems + wgs - 1) / wgs : 1;
  if (m->window > 0) {
    const int64_t span = (m->kv_interleave > 0 ? m->window / m->kv_interleave : m->window) + kFwdBM;
    const int64_t most = span / kKvpMinPartKeys;
    if (n > most) n = most;
  }
  if (n < 1) n = 1;
  if (n < P.nseg) {
    P.nseg = n;
    P.nsplit = n > 1 ? (int32_t)n : 0;
  }
  return P;
}

attn_status attn_kvp_workspace_size(int32_t R, const attn_tensor *q, const attn_tensor *k, int32_t num_seqs,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask_in,
                                    size_t *bytes) {
  if (!bytes) return fail(ATTN_ERR_NULL, "bytes is NULL");
  if (R < 1 || R > 16) return fail(ATTN_ERR_INVALID, "R must be in [1, 16]");
  if (!mask_in) return fail(ATTN_ERR_NULL, "mask is NULL");
  TRY(check_mask(mask_in));
  const attn_mask mk = kvp_paged_mask(mask_in);
  const attn_mask *mask = &mk;
  Problem P;
  TRY(plan_fwd(q, k, k, num_seqs, max_seqlen_q, max_seqlen_k, mask, P, true, false));
  P.decode = false;
  if (const Problem Pb = kvp_parts(R, P, num_seqs, mask); kvp_all_parts(R, Pb) && Pb.gather) {
    P = Pb;
    if (P.nseg == 0) P.nseg = 1;
    const size_t g = kvp_gather_bytes(R, P);
    P.gather = false;  // each rank's forward then runs on its gathered rows
    *bytes = kvp_parts_bytes(R, P) + kvp_sched_bytes(R, P, num_seqs) + g + fwd_ws_bytes(P, num_seqs, false);
  } else {
    const size_t part = align256((size_t)P.n_q * P.hq * P.d * 4) + align256((size_t)P.hq * P.n_q * 4);
    *bytes = (size_t)R * part + fwd_ws_bytes(P, num_seqs);
  }
  return ok();
}

attn_status attn_kvp_fwd(int32_t R, const attn_tensor *q, const attn_tensor *k_caches, const attn_tensor *v_caches,
                         const int32_t *const *block_tables, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                         int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k, const attn_mask *mask_in,
                         float scale, const attn_tensor *out, float *lse, void *workspace, size_t workspace_bytes,
                         void *stream) {
  if (R < 1 || R > 16) return fail(ATTN_ERR_INVALID, "R must be in [1, 16]");
  if (!k_caches || !v_caches || !block_tables || !mask_in) return fail(ATTN_ERR_NULL, "NULL argument");
  TRY(check_mask(mask_in));
  const attn_mask mk = kvp_paged_mask(mask_in);
  const attn_mask *mask = &mk;
  if (mask->kv_interleave != 0 && mask->kv_interleave != R)
    return fail(ATTN_ERR_INVALID, "kv_interleave must be 0 (contiguous) or R");
  size_t need = 0;
  TRY(attn_kvp_workspace_size(R, q, &k_caches[0], num_seqs, max_seqlen_q, max_seqlen_k, mask, &need));
  if (!workspace || workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  TRY(check_tensor(out, "out"));
  if (!lse && q->n_tok > 0) return fail(ATTN_ERR_NULL, "lse is NULL");
  char *w = (char *)workspace;
  Problem P;
  TRY(plan_fwd(q, &k_caches[0], &k_caches[0], num_seqs, max_seqlen_q, max_seqlen_k, mask, P, true, false));
  if (const Problem Pb = kvp_parts(R, P, num_seqs, mask); kvp_all_parts(R, Pb) && Pb.gather) {
    P = Pb;
    const int64_t n = P.nseg > 0 ? P.nseg : 1;
    const int64_t slice = P.n_q * P.hq * P.d, lslice = P.hq * P.n_q;
    float *pout = (float *)w;
    float *plse = (float *)(w + align256((size_t)R * n * slice * 4));
    if (P.nseg == 0) P.nseg = 1;
    const size_t pb = kvp_parts_bytes(R, P), sbb = kvp_sched_bytes(R, P, num_seqs), gbb = kvp_gather_bytes(R, P);
    const size_t gb = gbb / (2 * (size_t)R);
    const int64_t cap = sched_capacity(P.n_q, num_seqs, kFwdBM, n);
    char *gw = w + pb + sbb;
    std::vector<attn_mask> mr(R);
    std::vector<SchedBufs> sbr(R);
    std::vector<attn_tensor> kg(R), vg(R);
    std::vector<PageGatherArgs> ga(R);
    for (int r = 0; r < R; ++r) {
      const attn_tensor *kc = &k_caches[r], *vc = &v_caches[r];
      TRY(check_qkv(q, kc, vc));
      if (kc->n_head != k_caches[0].n_head || kc->dtype != k_caches[0].dtype)
        return fail(ATTN_ERR_SHAPE, "k_caches[%d] differs from k_caches[0]", r);
      if (vc->stride_tok != kc->stride_tok || vc->stride_head != kc->stride_head)
        return fail(ATTN_ERR_LAYOUT, "paged k and v caches must share their strides");
      mr[r] = *mask;
      if (!block_tables[r]) return fail(ATTN_ERR_NULL, "block_tables[%d] is NULL", r);
      if (mask->kv_interleave == R) mr[r].kv_rank = r;
      else mr[r].k_pos_offset = mask->k_pos_offset + (int64_t)r * max_seqlen_k;
      sbr[r] = sched_carve(w + pb + (size_t)r * (sbb / R), cap);
      // rank r's logical rows -> contiguous K, V
      PageGatherArgs &g = ga[r];
      g.src_k = kc->data; g.src_v = vc->data;
      g.page_stride = mask->page_stride; g.st = kc->stride_tok; g.sh = kc->stride_head;
      g.table = block_tables[r]; g.max_blocks = mask->max_blocks; g.n_pages = kc->n_tok / mask->block_size;
      g.shift = __builtin_ctz((unsigned)mask->block_size);
      g.dst_k = gw + (size_t)r * 2 * gb; g.dst_v = gw + ((size_t)r * 2 + 1) * gb;
      g.n_rows = P.n_k_logical; g.h = (int32_t)P.hkv; g.d = (int32_t)P.d; g.eb = esize(kc->dtype);
      g.cu = cu_seqlens_k; g.num_seqs = num_seqs;
      visible_key_rows(&mr[r], max_seqlen_q, max_seqlen_k, g.t_lo, g.t_hi);
      kg[r] = *kc;
      kg[r].data = g.dst_k; kg[r].n_tok = P.n_k_logical; kg[r].stride_head = P.d; kg[r].stride_tok = P.hkv * P.d;
      vg[r] = kg[r];
      vg[r].data = g.dst_v;
      mr[r].block_table = nullptr; mr[r].max_blocks = 0; mr[r].page_stride = 0;
    }
    hipStream_t s = (hipStream_t)stream;
    for (int r0 = 0; r0 < R; r0 += kMaxGatherBatch) {
      const int ng = R - r0 < kMaxGatherBatch ? R - r0 : kMaxGatherBatch;
      TRY(hip_check(timed("attn_gather", s, [&] { return launch_page_gathers(ga.data() + r0, ng, s); }),
                    "page gather"));
    }
    if (num_seqs > 0 && P.n_q > 0) {
      // the ranks' schedules (the same as each rank's forward would compute)
      SchedJob jobs[kMaxSchedJobs];
      for (int r0 = 0; r0 < R; r0 += kMaxSchedJobs) {
        const int nj = R - r0 < kMaxSchedJobs ? R - r0 : kMaxSchedJobs;
        for (int i = 0; i < nj; ++i) {
          MaskDev md = mask_dev(&mr[r0 + i]);
          md.seg_size = 0;
          jobs[i] = SchedJob{cu_seqlens_q, cu_seqlens_k, num_seqs, P.n_q, (int64_t)mask->max_blocks * mask->block_size,
                             md, kFwdBM, kFwdBN, 0, (int32_t)n, sbr[r0 + i]};
          jobs[i].nsplit = P.nsplit;
        }
        TRY(hip_check(timed("attn_sched", s, [&] { return launch_schedules(jobs, nj, s); }), "scheduler"));
      }
    }
    // the ranks' forwards: one launch when their shapes agree (each alone is
    // often too small to fill the chip), else one launch each
    std::vector<FwdArgs> fa(R);
    for (int r = 0; r < R; ++r) {
      const PartsOut po{pout + (int64_t)r * n * slice, plse + (int64_t)r * n * lslice, n};
      TRY(block_fwd_impl(q, &kg[r], &vg[r], cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, &mr[r],
                         scale, out, lse, gw + gbb, workspace_bytes - pb - sbb - gbb, stream, nullptr, &sbr[r], true,
                         &po, &fa[r]));
    }
    if (num_seqs > 0 && P.n_q > 0) {
      for (int r0 = 0; r0 < R; r0 += kMaxFwdBatch) {
        const int nb = R - r0 < kMaxFwdBatch ? R - r0 : kMaxFwdBatch;
        if (fwd_batchable(fa.data() + r0, nb)) {
          TRY(hip_check(timed("attn_fwd", s, [&] { return launch_fwd_batch(fa.data() + r0, nb, s); }),
                        "forward kernel"));
        } else {
          for (int r = r0; r < r0 + nb; ++r)
            TRY(hip_check(timed("attn_fwd", s, [&] { return launch_fwd(fa[r], s); }), "forward kernel"));
        }
      }
    }
    if (num_seqs == 0 || P.n_q == 0) return ok();
    MergeNArgs mn{};
    mn.n_parts = (int32_t)(R * n);
    mn.strided = 1;
    mn.out_stride = slice;
    mn.lse_stride = lslice;
    mn.pout[0] = pout; mn.pdtype[0] = ATTN_F32; mn.p_st[0] = P.hq * P.d; mn.p_sh[0] = P.d;
    mn.plse[0] = plse;
    mn.out = out->data; mn.out_dtype = out->dtype; mn.o_st = out->stride_tok; mn.o_sh = out->stride_head;
    mn.lse = lse; mn.n = P.n_q; mn.h = P.hq; mn.d = P.d;
    mn.cu = cu_seqlens_q; mn.num_seqs = num_seqs; mn.view = (int32_t)mask->q_view;
    return hip_check(timed("attn_merge_n", s, [&] { return launch_merge_n(mn, s); }), "rank merge");
  }
  const size_t obytes = align256((size_t)q->n_tok * q->n_head * q->head_dim * 4);
  const size_t lbytes = align256((size_t)q->n_head * q->n_tok * 4);
  std::vector<attn_tensor> parts(R);
  std::vector<const float *> plse(R);
  char *fws = w + (size_t)R * (obytes + lbytes);
  const size_t fws_bytes = workspace_bytes - (size_t)R * (obytes + lbytes);
  for (int r = 0; r < R; ++r) {
    attn_tensor &po = parts[r];
    po = *q;
    po.dtype = ATTN_F32;
    po.data = w + (size_t)r * (obytes + lbytes);
    po.stride_head = q->head_dim;
    po.stride_tok = q->n_head * q->head_dim;
    float *pl = (float *)(w + (size_t)r * (obytes + lbytes) + obytes);
    plse[r] = pl;
    attn_mask m = *mask;
    if (!block_tables[r]) return fail(ATTN_ERR_NULL, "block_tables[%d] is NULL", r);
    m.block_table = block_tables[r];
    if (mask->kv_interleave == R) m.kv_rank = r;
    else m.k_pos_offset = mask->k_pos_offset + (int64_t)r * max_seqlen_k;
    TRY(attn_block_fwd(q, &k_caches[r], &v_caches[r], cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k,
                       &m, scale, &po, pl, fws, fws_bytes, stream));
  }
  return attn_merge_n(R, parts.data(), plse.data(), out, lse, stream);
}

// ---------------------------------------------------------------------------
// device-content validation (synchronises)
// ---------------------------------------------------------------------------
attn_status attn_validate_inputs(const attn_tensor *q, const attn_tensor *k, const int32_t *cu_seqlens_q,
                                 const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, const attn_mask *mask, int32_t zigzag_cp, int32_t one_query,
                                 void *stream) {
  TRY(check_tensor(q, "q"));
  TRY(check_tensor(k, "k"));
  TRY(check_mask(mask));
  if (num_seqs < 0) return fail(ATTN_ERR_CU_SEQLENS, "negative num_seqs");
  if (num_seqs == 0) return ok();
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> cq(num_seqs + 1), ck(num_seqs + 1);
  TRY(hip_check(hipMemcpyAsync(cq.data(), cu_seqlens_q, cq.size() * 4, hipMemcpyDeviceToHost, s), "copy"));
  TRY(hip_check(hipMemcpyAsync(ck.data(), cu_seqlens_k, ck.size() * 4, hipMemcpyDeviceToHost, s), "copy"));
  std::vector<int32_t> bt;
  const bool paged = mask && mask->block_table;
  if (paged) {
    bt.resize(mask->max_blocks);
    TRY(hip_check(hipMemcpyAsync(bt.data(), mask->block_table, bt.size() * 4, hipMemcpyDeviceToHost, s), "copy"));
  }
  TRY(hip_check(hipStreamSynchronize(s), "sync"));
  const int64_t nk = paged ? (int64_t)mask->max_blocks * mask->block_size : k->n_tok;
  if (cq[0] != 0 || ck[0] != 0) return fail(ATTN_ERR_CONTENT, "cu_seqlens must start at 0");
  for (int d = 0; d < num_seqs; ++d) {
    const int64_t lq = (int64_t)cq[d + 1] - cq[d], lk = (int64_t)ck[d + 1] - ck[d];
    if (lq < 0 || lk < 0) return fail(ATTN_ERR_CONTENT, "cu_seqlens decreases at document %d", d);
    if (lq > max_seqlen_q || lk > max_seqlen_k)
      return fail(ATTN_ERR_CONTENT, "document %d longer than max_seqlen (%lld/%lld)", d, (long long)lq, (long long)lk);
    if (zigzag_cp > 0 && lq % (2 * zigzag_cp))
      return fail(ATTN_ERR_CONTENT, "document %d length %lld not a multiple of 2*cp", d, (long long)lq);
    if (one_query && lq != 1) return fail(ATTN_ERR_CONTENT, "document %d has %lld queries (decode needs 1)", d, (long long)lq);
  }
  if (cq[num_seqs] > q->n_tok || ck[num_seqs] > nk) return fail(ATTN_ERR_CONTENT, "cu_seqlens exceed the tensors");
  if (paged) {
    const int64_t pages = k->n_tok / mask->block_size;
    const int64_t used = (ck[num_seqs] + mask->block_size - 1) / mask->block_size;
    for (int64_t b = 0; b < used && b < (int64_t)bt.size(); ++b)
      if (bt[b] < 0 || bt[b] >= pages) return fail(ATTN_ERR_CONTENT, "block_table[%lld] = %d out of range", (long long)b, bt[b]);
  }
  return ok();
}

attn_status attn_timing_enable(int32_t on) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return ok();
}

attn_status attn_timing_report(char *buf, size_t len, size_t *written) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  auto &agg = t.agg;
  hipError_t err = hipSuccess;
  for (const Span &sp : t.spans) {
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventSynchronize(sp.b);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, sp.a, sp.b);
    auto &e = agg[sp.name];
    e.first += 1;
    e.second += ms;
    t.pool.push_back(sp.a);
    t.pool.push_back(sp.b);
  }
  t.spans.clear();
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "timing events: %s", hipGetErrorString(err));
  std::string out;
  char line[160];
  for (auto &kv : agg) {
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (written) *written = out.size();
  if (buf && len > 0) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
    if (out.size() >= len) return fail(ATTN_ERR_INVALID, "report needs %zu bytes", out.size() + 1);
    agg.clear();  // delivered
  }
  return ok();
}

}  // extern "C"
