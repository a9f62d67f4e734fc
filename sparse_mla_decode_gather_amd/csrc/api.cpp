// C-ABI of libsparsemla: argument validation, the split-K planner,
// workspace carving and kernel launches.  Host code only; everything here
// is shape arithmetic, so a call costs no device synchronisation and can be
// captured into a HIP graph.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.h"
#include "sparsemla.h"

namespace {

constexpr int kDefaultMaxSplits = 16;   // FlashInfer cake_* default max_splits
constexpr int kChunkCols = 64;          // split granularity in table columns

// Cost model, in units of half a gathered row of one workgroup's time (a
// row costs 2): a fixed cost per workgroup (Q load, compaction, epilogue),
// a split's partial write (kPartialPerHead per head), and the combine's
// reads of every partial row, spread over the CUs (kCombinePerRow per
// partial row).  The constants were fitted to forced-split timings over
// H = 64 / 128, BF16 and FP8 rows, K = 512 .. 2048 and T = 1 .. 192.
constexpr int64_t kWgOverheadRows = 96;
constexpr int64_t kPartialPerHead = 1;
constexpr int64_t kCombinePerRow = 4;
constexpr int64_t kHeadTileNum = 5, kHeadTileDen = 4;

// The model's cost of S = s splits for T tokens of H heads (one workgroup
// per CU): rounds of workgroups times a workgroup's fixed cost, its rows
// and its partial write, plus the combine's reads spread over the CUs.
int64_t split_cost(int64_t T, int H, int K, int num_chunks, int s, int64_t row_w,
                   int num_cus) {
  const int64_t cps = (num_chunks + s - 1) / s;
  const int64_t rows = std::min<int64_t>(cps * kChunkCols, K);
  const int64_t waves = (T * s + num_cus - 1) / num_cus;
  const int64_t per_wg = 2 * kWgOverheadRows + rows * row_w +
                         (s > 1 ? kPartialPerHead * (int64_t)H : 0);
  int64_t cost = waves * per_wg;
  if (s > 1) cost += (kCombinePerRow * T * H * s + num_cus - 1) / num_cus;
  return cost;
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

int query_cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SMLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (dev < 64 && g_cu_count[dev] > 0) {
    *out = g_cu_count[dev];
    return SMLA_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0)
    return SMLA_ERR_HIP;
  if (dev < 64) g_cu_count[dev] = n;
  *out = n;
  return SMLA_OK;
}

bool dtype_pair_ok(int q, int kv) {
  if (q == SMLA_DTYPE_BF16 && kv == SMLA_DTYPE_BF16) return true;
  if (q == SMLA_DTYPE_BF16 && kv == SMLA_DTYPE_PACKED_FP8_584) return true;
  if (q == SMLA_DTYPE_FP8_E4M3FN && kv == SMLA_DTYPE_FP8_E4M3FN) return true;
  if (q == SMLA_DTYPE_BF16 && kv == SMLA_DTYPE_FP8_E4M3FN) return true;
  return false;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
  size_t mid_lse, mid_out, total;
};

Layout layout_for(int S, int T, int H, int flags) {
  Layout L{0, 0, 0};
  if (S <= 1) {
    L.total = (flags & SMLA_FLAG_VALIDATE_INDICES) ? smla::kErrBlockBytes : 0;
    return L;
  }
  L.mid_lse = smla::kErrBlockBytes;
  const size_t lse_bytes = (size_t)T * H * S * sizeof(float);
  L.mid_out = round_up(L.mid_lse + lse_bytes, 256);
  L.total = L.mid_out + (size_t)T * H * S * smla::kHeadDim * 2;
  return L;
}

// Largest number of table columns a plan may span (num_splits x columns per
// split).  The kernels form column numbers s * split_cols + c in 32-bit
// ints, a table segment past the last one included, so the span stays far
// below INT_MAX.
constexpr int64_t kMaxPlanColumns = SMLA_MAX_PLAN_COLUMNS;

bool plan_ok(const smla_plan* p, int K) {
  if (p->num_splits < 1 || p->num_splits > SMLA_MAX_SPLITS) return false;
  if (p->head_tiles != 1 && p->head_tiles != 2) return false;
  if (p->chunk_cols < 1 || p->chunks_per_split < 1) return false;
  if (p->K != K) return false;
  const int64_t split_cols = (int64_t)p->chunks_per_split * p->chunk_cols;
  const int64_t cover = split_cols * p->num_splits;
  return cover >= K && cover <= kMaxPlanColumns;
}

// The QK scale must be a positive finite number (the kernels take the max of
// the raw logits and scale it afterwards, which needs a positive scale, and
// bmm1_scale * log2(e) must stay finite); the other scales must be finite.
bool scales_ok(float bmm1, float bmm2, float lse_scale) {
  const double s1 = (double)bmm1 * 1.4426950408889634;
  return std::isfinite(bmm1) && bmm1 > 0.f && s1 <= (double)FLT_MAX &&
         std::isfinite(bmm2) && std::isfinite(lse_scale);
}

}  // namespace

extern "C" {

int sparse_mla_plan_splits(int T, int H, int K, int q_dtype, int kv_dtype,
                           int max_splits, int num_splits_override,
                           int num_cus, smla_plan* out_plan) {
  if (!out_plan || T < 0 || K < 1 || K > kMaxPlanColumns) return SMLA_ERR_INVALID_ARG;
  if (H != 64 && H != 128) return SMLA_ERR_UNSUPPORTED_SHAPE;
  if (!dtype_pair_ok(q_dtype, kv_dtype)) return SMLA_ERR_UNSUPPORTED_DTYPE;
  if (num_cus <= 0) {
    const int st = query_cu_count(&num_cus);
    if (st != SMLA_OK) return st;
  }
  const int num_chunks = (K + kChunkCols - 1) / kChunkCols;
  int cap = max_splits > 0 ? max_splits : kDefaultMaxSplits;
  cap = std::min(std::min(cap, num_chunks), SMLA_MAX_SPLITS);

  int S = 1, head_tiles = 1;
  if (num_splits_override > 0) {
    S = std::min(std::max(num_splits_override, 1),
                 std::min(num_chunks, SMLA_MAX_SPLITS));
  } else if (T > 0) {
    // Per-row cost: the same for every row format at H=128.  Rows are
    // widened to BF16 and multiplied on the BF16 MFMA, whose work per row is
    // the same, so the row count and not its bytes sets a split's time
    // (weighting FP8 rows by their half-size bytes picked one split where
    // 4-8 ran up to 1.5x faster: H=128 FP8 rows, K=512, T=16-48).  At H=64
    // a BF16 row, gathered by LDS-DMA, costs half of one staged through
    // registers (FP8 and packed rows), which at H=128 the MFMA work hides
    // (fitted on sweeps of forced splits at H=64, BF16 and FP8 rows,
    // K = 512 .. 2048, T = 1 .. 512).
    const int64_t row_w64 = kv_dtype == SMLA_DTYPE_BF16 ? 1 : 2;
    const int64_t row_w = H == 64 ? row_w64 : 2;
    // An H=128 call may also run as head tiles: each token as two 64-head
    // halves on the H=64 kernel (2T virtual tokens, rows read twice, the
    // second time mostly from L2).  Their cost is the H=64 model's with a
    // row weight of 1 for every row format (against the H=128 kernel,
    // which stages FP8 and packed rows through registers too), and
    // one unit of it is worth kHeadTileNum / kHeadTileDen units of the
    // H=128 model (fitted on forced plans of both forms: BF16 rows,
    // K = 512 .. 2048, T = 1 .. 192, FP8 rows, K = 512 and 2048, T = 4 .. 128,
    // mean loss against the fastest 0.6%, worst 7.6%; packed rows, K = 512
    // and 2048, T = 1 .. 128: mean 1.5%, worst 10.6%).  Only while 2T
    // virtual tokens fit one round of CUs: beyond, the second row read and
    // the extra rounds lose (T=384, K=2048: BF16 rows 2% and FP8 rows 15%
    // slower than one workgroup per token, which the model misses).
    const bool try_head_tiles = H == 128 && 2 * (int64_t)T <= num_cus;
    const int64_t w_own = try_head_tiles ? kHeadTileDen : 1;
    int64_t best = INT64_MAX;
    for (int s = 1; s <= cap; ++s) {
      const int64_t cost =
          w_own * split_cost(T, H, K, num_chunks, s, row_w, num_cus);
      if (cost < best) {
        best = cost;
        S = s;
      }
    }
    if (try_head_tiles) {
      for (int s = 1; s <= cap; ++s) {
        const int64_t cost =
            kHeadTileNum * split_cost(2 * (int64_t)T, 64, K, num_chunks, s, 1, num_cus);
        if (cost < best) {
          best = cost;
          S = s;
          head_tiles = 2;
        }
      }
    }
  }
  const int cps = (num_chunks + S - 1) / S;
  out_plan->num_splits = S;
  out_plan->head_tiles = head_tiles;
  out_plan->chunk_cols = kChunkCols;
  out_plan->chunks_per_split = cps;
  out_plan->num_chunks = num_chunks;
  out_plan->K = K;
  out_plan->reserved[0] = out_plan->reserved[1] = 0;
  return SMLA_OK;
}

size_t sparse_mla_workspace_size(const smla_plan* plan, int T, int H,
                                 int flags) {
  if (!plan || T < 0 || (H != 64 && H != 128) || plan->num_splits < 1)
    return (size_t)-1;
  return layout_for(plan->num_splits, T, H, flags).total;
}

int sparse_mla_workspace_layout(const smla_plan* plan, int T, int H,
                                size_t* mid_lse_offset,
                                size_t* mid_out_offset) {
  if (!plan || T < 0 || (H != 64 && H != 128) || plan->num_splits < 1)
    return SMLA_ERR_INVALID_ARG;
  const Layout L = layout_for(plan->num_splits, T, H, 0);
  if (mid_lse_offset) *mid_lse_offset = L.mid_lse;
  if (mid_out_offset) *mid_out_offset = L.mid_out;
  return SMLA_OK;
}

}  // extern "C"

namespace {

// Argument checks shared by sparse_mla_decode and sparse_mla_gather_only,
// and the kernel parameters they resolve to.  *plan is replaced by
// *local when the caller passed none.  Returns SMLA_OK or a status.
// seg == pg == NULL: the combined table (args->indices, args->topk_lens);
// seg: the two-segment form; pg: the page-table form.  In both of the
// latter args->indices must be NULL; args->topk_lens must be NULL for seg
// and is the window + compressed slot count for pg.
int prepare_call(const smla_decode_args* a, const smla_segments* seg,
                 const smla_paged* pg, const smla_plan*& plan, smla_plan* local,
                 bool with_outputs, smla::DecodeParams* p, Layout* L) {
  if (!a) return SMLA_ERR_INVALID_ARG;
  if (a->T < 0 || a->K < 1) return SMLA_ERR_INVALID_ARG;
  if ((uint32_t)a->flags & ~(SMLA_FLAG_VALIDATE_INDICES | SMLA_FLAG_SERIAL_PIPELINE))
    return SMLA_ERR_INVALID_ARG;
  // the serialized pipeline is built for the combined table and the decode
  const bool serial = (a->flags & SMLA_FLAG_SERIAL_PIPELINE) != 0;
  if (serial && (seg || pg || !with_outputs)) return SMLA_ERR_INVALID_ARG;
  if (a->H != 64 && a->H != 128) return SMLA_ERR_UNSUPPORTED_SHAPE;
  if (!dtype_pair_ok(a->q_dtype, a->kv_dtype)) return SMLA_ERR_UNSUPPORTED_DTYPE;
  if (with_outputs && !scales_ok(a->bmm1_scale, a->bmm2_scale, a->lse_scale))
    return SMLA_ERR_INVALID_ARG;
  // the two tables: widths, rows, strides (in elements)
  int k1, k2;
  const int32_t *t1, *t2;
  int64_t s1, s2;
  int64_t t2_width;   // elements of a row of the second table that are read
  if (pg) {
    if (pg->swa_width < 0 || pg->max_pages < 0 || pg->page_size < 1)
      return SMLA_ERR_INVALID_ARG;
    const int64_t slots = (int64_t)pg->max_pages * pg->page_size;
    if (slots > INT_MAX / 2 || (int64_t)pg->swa_width + slots != a->K)
      return SMLA_ERR_INVALID_ARG;
    if (a->indices) return SMLA_ERR_INVALID_ARG;
    k1 = pg->swa_width;
    k2 = (int)slots;
    t1 = pg->swa_indices;
    t2 = pg->block_tables;
    s1 = pg->swa_row_stride == 0 ? k1 : pg->swa_row_stride;
    s2 = pg->block_table_stride == 0 ? pg->max_pages : pg->block_table_stride;
    t2_width = pg->max_pages;
  } else if (seg) {
    if (seg->swa_width < 0 || seg->extra_width < 0 ||
        (int64_t)seg->swa_width + seg->extra_width != a->K)
      return SMLA_ERR_INVALID_ARG;
    if (a->indices || a->topk_lens) return SMLA_ERR_INVALID_ARG;
    k1 = seg->swa_width;
    k2 = seg->extra_width;
    t1 = seg->swa_indices;
    t2 = seg->extra_indices;
    s1 = seg->swa_row_stride == 0 ? k1 : seg->swa_row_stride;
    s2 = seg->extra_row_stride == 0 ? k2 : seg->extra_row_stride;
    t2_width = k2;
  } else {
    k1 = std::min(a->K, smla::kSwaColumns);
    k2 = a->K - k1;
    t1 = a->indices;
    s1 = a->index_row_stride == 0 ? a->K : a->index_row_stride;
    if (s1 < a->K) return SMLA_ERR_INVALID_ARG;
    t2 = a->indices ? a->indices + k1 : nullptr;
    s2 = s1;
    t2_width = k2;
  }
  if (a->T == 0) return SMLA_OK;
  if (!a->q || (with_outputs && !a->out)) return SMLA_ERR_INVALID_ARG;
  if (k1 > 0 && (!t1 || !a->swa_pool || s1 < k1)) return SMLA_ERR_INVALID_ARG;
  if (k2 > 0 && (!t2 || !a->compressed_pool || s2 < t2_width)) return SMLA_ERR_INVALID_ARG;
  if (a->swa_rows < 0 || a->compressed_rows < 0) return SMLA_ERR_INVALID_ARG;
  if ((int64_t)a->T * a->H > INT_MAX / 2) return SMLA_ERR_INVALID_ARG;
  // A pool row is 512 elements, or 584 bytes for packed rows (its stride is
  // then counted in bytes).
  const bool packed = a->kv_dtype == SMLA_DTYPE_PACKED_FP8_584;
  const int64_t row_elems = packed ? SMLA_PACKED_ROW_BYTES : smla::kHeadDim;
  const int64_t row_stride = a->pool_row_stride == 0 ? row_elems : a->pool_row_stride;
  if (row_stride < row_elems) return SMLA_ERR_INVALID_ARG;
  if (a->cum_seq_lens_q && a->num_requests < 1) return SMLA_ERR_INVALID_ARG;
  const int kv_elem = a->kv_dtype == SMLA_DTYPE_BF16 ? 2 : 1;
  // rows start 16-B aligned (8-B for packed rows, whose loads are 8 and 16
  // bytes at 4-byte aligned offsets)
  const int64_t row_align = packed ? 8 : 16;
  if (!aligned(a->q, 16) || (with_outputs && !aligned(a->out, 16)) ||
      (a->swa_pool && !aligned(a->swa_pool, 16)) ||
      (a->compressed_pool && !aligned(a->compressed_pool, 16)) ||
      (row_stride * kv_elem) % row_align != 0 || (t1 && !aligned(t1, 4)) ||
      (t2 && !aligned(t2, 4)))
    return SMLA_ERR_MISALIGNED;

  if (!plan) {
    const int st = sparse_mla_plan_splits(a->T, a->H, a->K, a->q_dtype, a->kv_dtype,
                                          0, 0, 0, local);
    if (st != SMLA_OK) return st;
    plan = local;
  }
  if (!plan_ok(plan, a->K)) return SMLA_ERR_BAD_PLAN;
  const int S = plan->num_splits;
  if ((int64_t)a->T * S > INT_MAX / 2) return SMLA_ERR_INVALID_ARG;
  // head tiles: H=128 only; the gather alone has no heads and ignores them
  if (plan->head_tiles == 2 && a->H != 128) return SMLA_ERR_BAD_PLAN;
  const bool head_tiles = with_outputs && plan->head_tiles == 2;

  const bool validate = with_outputs && (a->flags & SMLA_FLAG_VALIDATE_INDICES) != 0;
  *L = layout_for(with_outputs ? S : 1, a->T, a->H, validate ? a->flags : 0);
  if (L->total > 0) {
    if (!a->workspace) return SMLA_ERR_WORKSPACE_TOO_SMALL;
    if (a->workspace_bytes < L->total) return SMLA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(a->workspace, 256)) return SMLA_ERR_MISALIGNED;
  }

  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  *p = smla::DecodeParams{};
  p->q = a->q;
  p->swa = static_cast<const uint8_t*>(a->swa_pool);
  p->comp = static_cast<const uint8_t*>(a->compressed_pool);
  p->swa_rows = a->swa_pool ? a->swa_rows : 0;
  p->comp_rows = a->compressed_pool ? a->compressed_rows : 0;
  p->row_stride_bytes = row_stride * kv_elem;
  // a table of width 0 is never read; point it at the other one so that
  // every pointer the kernel forms is a real address
  p->indices = k1 > 0 ? t1 : t2;
  p->index_row_stride = k1 > 0 ? s1 : s2;
  p->indices2 = k2 > 0 ? t2 : t1;
  p->index_row_stride2 = k2 > 0 ? s2 : s1;
  p->swa_cols = (seg || pg) ? k1 : smla::kSwaColumns;
  p->K2 = k2;
  p->segmented = pg ? 2 : seg ? 1 : 0;
  p->page_size = pg ? pg->page_size : 0;
  p->topk_lens = pg ? pg->swa_topk_lens : seg ? seg->swa_topk_lens : a->topk_lens;
  p->lens2 = pg ? a->topk_lens : seg ? seg->extra_topk_lens : nullptr;
  p->sinks = a->sinks;
  p->scale_log2 = (float)((double)a->bmm1_scale * 1.4426950408889634);
  p->bmm2 = a->bmm2_scale;
  p->lse_scale = a->lse_scale;
  p->out = a->out;
  p->out_lse = a->out_lse;
  p->err = validate ? reinterpret_cast<int32_t*>(ws) : nullptr;
  // head tiles: the H=64 kernel on 2T virtual tokens (same buffers)
  p->T = head_tiles ? 2 * a->T : a->T;
  p->H = head_tiles ? 64 : a->H;
  p->head_shift = head_tiles ? 1 : 0;
  p->K = a->K;
  p->S = S;
  p->split_cols = plan->chunks_per_split * plan->chunk_cols;
  p->validate = validate ? 1 : 0;
  // Longest-first starts only pay when some CU runs more than one item (one
  // H=128 workgroup fits a CU); without a device count, keep them.
  {
    int cus = 0;
    p->rank_items = (query_cu_count(&cus) != SMLA_OK || (int64_t)p->T * S > cus) ? 1 : 0;
  }
  p->serial = serial ? 1 : 0;
  if (with_outputs && S > 1) {
    p->mid_lse = reinterpret_cast<float*>(ws + L->mid_lse);
    p->mid_out = reinterpret_cast<uint16_t*>(ws + L->mid_out);
  }
  return SMLA_OK;
}

// The split kernel, then the combine when the plan splits.
int launch_all(const smla_decode_args* a, const smla_plan* plan,
               const smla::DecodeParams& p, hipStream_t stream) {
  const int S = plan->num_splits;
  if (p.validate && smla::launch_clear_error(p.err, stream) != hipSuccess)
    return SMLA_ERR_HIP;
  if (smla::launch_decode(p, a->q_dtype, a->kv_dtype, stream) != hipSuccess)
    return SMLA_ERR_HIP;
  if (S > 1) {
    smla::CombineParams c{};
    c.mid_out = p.mid_out;
    c.mid_lse = p.mid_lse;
    c.sinks = a->sinks;
    c.lse_scale = a->lse_scale;
    c.out = static_cast<uint16_t*>(a->out);
    c.out_lse = a->out_lse;
    c.T = a->T;
    c.H = a->H;
    c.S = S;
    c.stride = S;
    if (smla::launch_combine(c, stream) != hipSuccess) return SMLA_ERR_HIP;
  }
  return SMLA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_decode(const smla_decode_args* a, const smla_plan* plan,
                      smla_stream_t stream_handle) {
  smla_plan local;
  smla::DecodeParams p;
  Layout L;
  const int st = prepare_call(a, nullptr, nullptr, plan, &local, true, &p, &L);
  if (st != SMLA_OK || a->T == 0) return st;
  return launch_all(a, plan, p, reinterpret_cast<hipStream_t>(stream_handle));
}

int sparse_mla_decode_noalloc(const smla_decode_args* a, const smla_plan* plan,
                              smla_stream_t stream_handle) {
  if (!a) return SMLA_ERR_INVALID_ARG;
  // The caller brings no workspace; validation (whose error block the
  // caller would read back through a workspace pointer) is not offered.
  if (a->workspace != nullptr || a->workspace_bytes != 0 ||
      (a->flags & SMLA_FLAG_VALIDATE_INDICES) != 0)
    return SMLA_ERR_INVALID_ARG;
  smla_decode_args b = *a;
  smla_plan local;
  smla::DecodeParams p;
  Layout L;
  // First pass with no workspace: argument checks and the layout the call
  // needs (a call that needs none is complete right here).
  int st = prepare_call(&b, nullptr, nullptr, plan, &local, true, &p, &L);
  if (st == SMLA_OK) {
    if (a->T == 0) return SMLA_OK;
    return launch_all(&b, plan, p, reinterpret_cast<hipStream_t>(stream_handle));
  }
  if (st != SMLA_ERR_WORKSPACE_TOO_SMALL) return st;
  if (L.total > smla::kNoAllocScratchBytes) return SMLA_ERR_TOO_LARGE;
  void* scratch = nullptr;
  if (smla::noalloc_scratch(&scratch) != hipSuccess) return SMLA_ERR_HIP;
  b.workspace = scratch;
  b.workspace_bytes = smla::kNoAllocScratchBytes;
  st = prepare_call(&b, nullptr, nullptr, plan, &local, true, &p, &L);
  if (st != SMLA_OK) return st;
  return launch_all(&b, plan, p, reinterpret_cast<hipStream_t>(stream_handle));
}

int sparse_mla_decode_paged(const smla_decode_args* a, const smla_paged* pg,
                            const smla_plan* plan, smla_stream_t stream_handle) {
  if (!pg) return SMLA_ERR_INVALID_ARG;
  smla_plan local;
  smla::DecodeParams p;
  Layout L;
  const int st = prepare_call(a, nullptr, pg, plan, &local, true, &p, &L);
  if (st != SMLA_OK || a->T == 0) return st;
  return launch_all(a, plan, p, reinterpret_cast<hipStream_t>(stream_handle));
}

int sparse_mla_decode_segments(const smla_decode_args* a, const smla_segments* seg,
                               const smla_plan* plan, smla_stream_t stream_handle) {
  if (!seg) return SMLA_ERR_INVALID_ARG;
  smla_plan local;
  smla::DecodeParams p;
  Layout L;
  const int st = prepare_call(a, seg, nullptr, plan, &local, true, &p, &L);
  if (st != SMLA_OK || a->T == 0) return st;
  return launch_all(a, plan, p, reinterpret_cast<hipStream_t>(stream_handle));
}

int sparse_mla_gather_only(const smla_decode_args* a, const smla_plan* plan,
                           smla_stream_t stream_handle) {
  smla_plan local;
  smla::DecodeParams p;
  Layout L;
  const int st = prepare_call(a, nullptr, nullptr, plan, &local, false, &p, &L);
  if (st != SMLA_OK || a->T == 0) return st;
  if (a->H != 128) return SMLA_ERR_UNSUPPORTED_SHAPE;
  if (a->q_dtype != SMLA_DTYPE_BF16 || a->kv_dtype != SMLA_DTYPE_BF16)
    return SMLA_ERR_UNSUPPORTED_DTYPE;
  if (smla::launch_gather_only(p, reinterpret_cast<hipStream_t>(stream_handle)) !=
      hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_build_indices(const smla_build_args* a, smla_stream_t stream_handle) {
  if (!a) return SMLA_ERR_INVALID_ARG;
  if (a->T < 0 || a->swa_width < 0 || a->comp_width < 0) return SMLA_ERR_INVALID_ARG;
  const int64_t K = (int64_t)a->swa_width + a->comp_width;
  if (K < 1 || K > INT_MAX / 2) return SMLA_ERR_INVALID_ARG;
  if (a->T == 0) return SMLA_OK;
  const int64_t s1 = a->swa_row_stride == 0 ? a->swa_width : a->swa_row_stride;
  const int64_t s2 = a->comp_row_stride == 0 ? a->comp_width : a->comp_row_stride;
  const int64_t so = a->out_row_stride == 0 ? K : a->out_row_stride;
  if ((a->swa_width > 0 && (!a->swa_indices || s1 < a->swa_width)) ||
      (a->comp_width > 0 && (!a->comp_indices || s2 < a->comp_width)) ||
      !a->out_indices || !a->out_topk_lens || so < K)
    return SMLA_ERR_INVALID_ARG;
  const bool local = a->comp_local != 0;
  const int64_t sb = a->block_table_stride == 0 ? a->max_blocks : a->block_table_stride;
  if (local && a->comp_width > 0 &&
      (!a->block_tables || a->max_blocks < 1 || a->page_size < 1 ||
       a->num_requests < 1 || sb < a->max_blocks))
    return SMLA_ERR_INVALID_ARG;
  // one workgroup per 1024 columns of a token (the builder kernel's tile)
  if ((int64_t)a->T * ((K + 1023) / 1024) > INT_MAX) return SMLA_ERR_INVALID_ARG;
  const void* ptrs[] = {a->swa_indices, a->comp_indices, a->comp_topk_lens,
                        a->block_tables, a->token_to_req, a->valid_tokens,
                        a->out_indices, a->out_topk_lens, a->err};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return SMLA_ERR_MISALIGNED;
  smla::BuildParams p{};
  p.swa = a->swa_indices;
  p.swa_stride = s1;
  p.comp = a->comp_indices;
  p.comp_stride = s2;
  p.comp_lens = a->comp_topk_lens;
  p.block_tables = a->block_tables;
  p.bt_stride = sb;
  p.token_to_req = a->token_to_req;
  p.valid = a->valid_tokens;
  p.out = a->out_indices;
  p.out_stride = so;
  p.out_lens = a->out_topk_lens;
  p.err = a->err;
  p.T = a->T;
  p.W = a->swa_width;
  p.K2 = a->comp_width;
  p.local = (local && a->comp_width > 0) ? 1 : 0;
  p.max_blocks = a->max_blocks;
  p.page_size = a->page_size;
  p.num_requests = a->num_requests;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_handle);
  if (p.err && smla::launch_clear_error(p.err, stream) != hipSuccess) return SMLA_ERR_HIP;
  if (smla::launch_build_indices(p, stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_combine(const void* mid_out, const float* mid_lse, int T, int H,
                       int S, int split_stride, const float* sinks,
                       float lse_scale, void* out, float* out_lse,
                       smla_stream_t stream_handle) {
  if (T < 0 || S < 1 || S > SMLA_MAX_SPLITS || split_stride < S ||
      !std::isfinite(lse_scale))
    return SMLA_ERR_INVALID_ARG;
  if (H != 64 && H != 128) return SMLA_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return SMLA_OK;
  if (!mid_out || !mid_lse || !out) return SMLA_ERR_INVALID_ARG;
  if (!aligned(mid_out, 16) || !aligned(out, 16) || !aligned(mid_lse, 4))
    return SMLA_ERR_MISALIGNED;
  smla::CombineParams c{};
  c.mid_out = static_cast<const uint16_t*>(mid_out);
  c.mid_lse = mid_lse;
  c.sinks = sinks;
  c.lse_scale = lse_scale;
  c.out = static_cast<uint16_t*>(out);
  c.out_lse = out_lse;
  c.T = T;
  c.H = H;
  c.S = S;
  c.stride = split_stride;
  if (smla::launch_combine(c, reinterpret_cast<hipStream_t>(stream_handle)) !=
      hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_get_device_error(const void* workspace, smla_stream_t stream_handle,
                                int32_t* code, int32_t* token, int32_t* column) {
  if (!workspace) return SMLA_ERR_INVALID_ARG;
  int32_t host[4] = {0, -1, -1, 0};
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_handle);
  if (hipMemcpyAsync(host, workspace, sizeof(host), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SMLA_ERR_HIP;
  if (code) *code = host[0];
  if (token) *token = host[1];
  if (column) *column = host[2];
  return SMLA_OK;
}

const char* sparse_mla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_INVALID_ARG: return "invalid argument";
    case SMLA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype pair";
    case SMLA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (H must be 64 or 128)";
    case SMLA_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or too small";
    case SMLA_ERR_MISALIGNED: return "misaligned pointer or stride";
    case SMLA_ERR_BAD_PLAN: return "plan inconsistent with the call";
    case SMLA_ERR_HIP: return "HIP runtime error";
    case SMLA_ERR_TOO_LARGE:
      return "call needs more scratch than the allocation-free decode holds "
             "(SMLA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
