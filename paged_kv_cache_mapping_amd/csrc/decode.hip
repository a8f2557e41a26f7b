// Paged decode attention, host side: plans, argument checks, workspace
// layout and the C entry points (decode and chunked).  The kernels and their
// launch templates are in decode_kernels.h; decode_*.hip instantiate them.
#include <mutex>

#include "decode_kernels.h"
#include "prefill.h"

namespace pkv {

// --------------------------------------------------------------------------
// Host side.

static int log2_int(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Most visible blocks any row can have.  A window of W keys starting at the
// worst offset inside a block straddles ceil((W + bs - 1) / bs) blocks; a
// non-causal windowed row sees W + q_len - 1 keys.
static int max_visible_blocks(int max_seq_len, int bs, int window, int extra) {
  const int full = ceil_div(max_seq_len > 0 ? max_seq_len : 1, bs);
  if (window <= 0) return full;
  const long long win = ((long long)window + extra + bs - 1 + bs - 1) / bs;   // no int overflow
  return full < win ? full : (int)win;
}

// Query heads one vector-ALU work item handles.
static int heads_per_item_valu(int group) {
  if (group >= 8) return (group % 8 == 0) ? 8 : 0;
  return (group == 1 || group == 2 || group == 4) ? group : 0;
}

// MFMA rows one matrix-core work item may hold: 16 for bf16; 8 for fp8 and
// int4, whose lanes accumulate 16 elements per row (16 rows would need 256
// accumulator registers and spill).
static int max_item_rows(int kv_dtype) { return kv_dtype == PKV_BF16 ? 16 : 8; }

// Query heads one matrix-core work item handles (MFMA rows).
static int heads_per_item_mfma(int group, int kv_dtype) {
  const int cap = max_item_rows(kv_dtype);
  if (group >= cap) return (group % cap == 0) ? cap : 0;
  return (group == 1 || group == 2 || group == 4 || group == 8) ? group : 0;
}

// INT4 decode items may span two KV heads: head size 128, an even number of
// KV heads and at most 8 rows per pair.
static bool int4_pairs(int kv_dtype, int d, int hkv, int group) {
  return kv_dtype == PKV_INT4 && d == 128 && hkv % 2 == 0 && group >= 1 && 2 * group <= 8;
}

static bool mfma_eligible(int kv_dtype, int d, int bs) {
  if (bs % 16 != 0) return false;
  if (kv_dtype == PKV_INT4) return d == 128;   // the one INT4 head size built
  const int elt = dtype_size(kv_dtype);
  return (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3) && d % 32 == 0 && d * elt >= 64;
}

constexpr int kMaxStreamRows = 4096;   // prefix sums of the balanced scheme live in LDS
constexpr int kStreamMinUnits = 8;     // blocks per worker at least (bounds the pieces)
constexpr int kTrailPct = 90;            // second wave on a SIMD: share in percent
constexpr int kLdsPerCU = 160 * 1024;

// Resident waves per CU for the balanced kernels: two per SIMD while the
// registers allow it (two_waves: 4 rows per item; 8 with INT4, whose lanes
// keep 8 accumulators per row; 16 where P.V accumulates in the matrix
// cores), else one.  Multi-token plans count rows as heads (qt unknown
// here: any qt > 1 behaves alike).
static int stream_waves_per_cu(int heads_per_item, int kv_dtype, int d, bool multi) {
  return two_waves(d, kv_dtype, multi ? 1 : heads_per_item, multi ? heads_per_item : 1) ? 8 : 4;
}

static size_t partial_bytes(int rows, int hq, int splits, int d) {
  return (size_t)rows * hq * splits * ((size_t)d + 2) * sizeof(float);
}

static size_t plan_bytes(const pkv_decode_plan& p, int rows, int hq, int d) {
  // balanced: the partials, a piece count and output row per (row, head
  // group), and per row the decode step's own-token flag
  if (p.scheme == 1)
    return partial_bytes(rows, hq, p.max_splits, d) +
           (size_t)rows * (hq / p.heads_per_item) * 2 * sizeof(int32_t) + (size_t)rows * sizeof(int32_t);
  return p.max_splits > 1 ? partial_bytes(rows, hq, p.max_splits, d) : 0;
}

constexpr int kKnownPlanFlags = PKV_PLAN_BLOCKS_NOT_SHARED | PKV_PLAN_BLOCKS_SHARED;

// known bits only, and not both promises at once
static bool plan_flags_ok(int flags) {
  if (flags & ~kKnownPlanFlags) return false;
  return (flags & kKnownPlanFlags) != kKnownPlanFlags;
}

static int make_plan(int rows, int hq, int hkv, int d, int bs, int kv_dtype, int max_seq_len,
                     int window, int extra, bool allow_stream, pkv_decode_plan* plan, int force_hpi = 0,
                     int flags = 0) {
  if (!plan) return PKV_ERR_NULL;
  if (rows < 0 || hq <= 0 || hkv <= 0 || max_seq_len < 0 || window < 0) return PKV_ERR_SHAPE;
  if (!plan_flags_ok(flags)) return PKV_ERR_SHAPE;
  if (hq % hkv) return PKV_ERR_SHAPE;
  if (dtype_bits(kv_dtype) == 0) return PKV_ERR_DTYPE;
  if (!head_dim_supported(d) || !block_size_supported(bs)) return PKV_ERR_UNSUPPORTED;
  const int group = hq / hkv;
  const int nvis = max_visible_blocks(max_seq_len, bs, window, extra);
  const long long cus = device_cu_count();
  int gm = force_hpi > 0 ? force_hpi : heads_per_item_mfma(group, kv_dtype);
  // INT4 items over two adjacent KV heads (whole 128-byte lines) when the
  // pair's rows fit: heads_per_item = 2 * group marks them
  if (force_hpi == 0 && int4_pairs(kv_dtype, d, hkv, group)) gm = 2 * group;
  plan->flags = flags;
  if (allow_stream && mfma_eligible(kv_dtype, d, bs) && gm > 0 && rows <= kMaxStreamRows) {
    // balanced partition over resident wave slots
    const long long units = (long long)(rows > 0 ? rows : 1) * (hq / gm) * nvis;
    int per_cu = stream_waves_per_cu(gm, kv_dtype, d, force_hpi > 0);
    // Under PKV_PLAN_BLOCKS_SHARED every share is equal (the placement of
    // an eighth of the units per XCD needs equal shares), and bf16
    // single-query items of up to 4 rows run one wave per SIMD (shared-prefix
    // split 65.7 us against 68.0 with two waves and lead / trail shares).
    // PKV_PLAN_BLOCKS_NOT_SHARED leaves the shares alone, so that it changes
    // how blocks are loaded, not the bits.
    const bool shared = (flags & PKV_PLAN_BLOCKS_SHARED) != 0;
    if (shared && kv_dtype == PKV_BF16 && force_hpi == 0 && gm <= 4 && per_cu == 8) per_cu = 4;
    long long workers = cus * per_cu;
    const long long need = (units + kStreamMinUnits - 1) / kStreamMinUnits;
    plan->lead_workers = 0;
    plan->trail_share_pct = 100;
    if (workers > need) {
      workers = need;
    } else if (per_cu > 4 && !shared) {
      plan->lead_workers = (int32_t)(workers / 2);
      plan->trail_share_pct = kTrailPct;
    }
    if (workers < 1) workers = 1;
    plan->scheme = 1;
    plan->num_workers = (int32_t)workers;
    plan->split_blocks = kStreamMinUnits;
    plan->max_splits = ceil_div(nvis, kStreamMinUnits) + 1;
    plan->heads_per_item = gm;
  } else {
    const int gt = heads_per_item_valu(group);
    if (gt == 0) return PKV_ERR_UNSUPPORTED;
    if (kv_dtype == PKV_INT4) return PKV_ERR_UNSUPPORTED;   // matrix-core path only
    // fixed splits: about 16 single-wave work items per compute unit if
    // every row were as long as the longest; powers of two in [1, 64]
    const long long items1 = (long long)(rows > 0 ? rows : 1) * (hq / gt) * nvis;
    const long long target = cus * 16;
    int split = 1;
    while (split < 64 && items1 / split > target) split <<= 1;
    plan->scheme = 0;
    plan->num_workers = 0;
    plan->lead_workers = 0;
    plan->trail_share_pct = 100;
    plan->split_blocks = split;
    plan->max_splits = ceil_div(nvis, split);
    plan->heads_per_item = gt;
  }
  plan->workspace_bytes = plan_bytes(*plan, rows, hq, d);
  return PKV_OK;
}

static int check_plan(const pkv_decode_plan* plan, int rows, int hq, int hkv, int d, int bs,
                      int kv_dtype, int max_seq_len, int window, int extra) {
  if (!plan) return PKV_ERR_NULL;
  if (!plan_flags_ok(plan->flags)) return PKV_ERR_SHAPE;
  const int group = hq / hkv;
  const int nvis = max_visible_blocks(max_seq_len, bs, window, extra);
  if (plan->scheme == 1) {
    if (!mfma_eligible(kv_dtype, d, bs) || rows > kMaxStreamRows) return PKV_ERR_SHAPE;
    // any of 1, 2, 4, 8, 16 that divides the group (items of a KV head then
    // share its blocks); the planner picks the largest
    const int hpi = plan->heads_per_item;
    const bool pair = hpi == 2 * group && int4_pairs(kv_dtype, d, hkv, group);
    if (!pair && (hpi <= 0 || hpi > max_item_rows(kv_dtype) || (hpi & (hpi - 1)) || group % hpi))
      return PKV_ERR_SHAPE;
    if (plan->split_blocks < 1 || plan->num_workers < 1) return PKV_ERR_SHAPE;
    if (plan->lead_workers < 0 || plan->lead_workers > plan->num_workers) return PKV_ERR_SHAPE;
    if (plan->trail_share_pct < 1 || plan->trail_share_pct > 100) return PKV_ERR_SHAPE;
    if (plan->max_splits < ceil_div(nvis, plan->split_blocks) + 1) return PKV_ERR_SHAPE;
    return PKV_OK;
  }
  if (plan->scheme != 0) return PKV_ERR_SHAPE;
  if (kv_dtype == PKV_INT4) return PKV_ERR_UNSUPPORTED;
  if (plan->split_blocks < 1 || plan->split_blocks > 64) return PKV_ERR_SHAPE;
  const int gt = heads_per_item_valu(group);
  if (gt == 0) return PKV_ERR_UNSUPPORTED;
  if (plan->heads_per_item != gt) return PKV_ERR_SHAPE;
  if (plan->max_splits < ceil_div(nvis, plan->split_blocks)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// ---- dispatch to the per-(head_dim, KV dtype) instantiations
PKV_DECODE_ALL_D(extern, 8)
PKV_DECODE_ALL_D(extern, 16)
PKV_DECODE_ALL_D(extern, 32)
PKV_DECODE_ALL_D(extern, 64)
PKV_DECODE_ALL_D(extern, 128)
PKV_DECODE_ALL_D(extern, 256)
PKV_DECODE_STREAM_INST(extern, 128, PKV_INT4)
PKV_DECODE_PAIR_INST(extern, 128)
PKV_DECODE_MULTI_INST(extern, 128, PKV_BF16)
PKV_DECODE_MULTI_INST(extern, 128, PKV_FP8_E4M3)
PKV_DECODE_MULTI_INST(extern, 128, PKV_INT4)
PKV_DECODE_MERGE_MULTI_INST(extern, 128)

template <int D>
static int split_d(const DecodeArgs& a, int gt, int kv, hipStream_t s) {
  if (kv == PKV_F32) return run_split_dk<D, PKV_F32>(a, gt, s);
  if (kv == PKV_BF16) return run_split_dk<D, PKV_BF16>(a, gt, s);
  if (kv == PKV_FP8_E4M3) return run_split_dk<D, PKV_FP8_E4M3>(a, gt, s);
  return PKV_ERR_UNSUPPORTED;
}

static int dispatch_split(const DecodeArgs& a, int gt, int kv, hipStream_t s) {
  switch (a.head_dim) {
    case 8: return split_d<8>(a, gt, kv, s);
    case 16: return split_d<16>(a, gt, kv, s);
    case 32: return split_d<32>(a, gt, kv, s);
    case 64: return split_d<64>(a, gt, kv, s);
    case 128: return split_d<128>(a, gt, kv, s);
    case 256: return split_d<256>(a, gt, kv, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D>
static int stream_d(const DecodeArgs& a, int kv, int workers, hipStream_t s) {
  if (kv == PKV_BF16) return run_stream_dk<D, PKV_BF16>(a, workers, s);
  if (kv == PKV_FP8_E4M3) return run_stream_dk<D, PKV_FP8_E4M3>(a, workers, s);
  if constexpr (D == 128) {
    if (kv == PKV_INT4) return run_stream_dk<128, PKV_INT4>(a, workers, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

// Multi-token items (row mode 3), head size 128.
static int dispatch_multi(const DecodeArgs& a, int kv, int workers, hipStream_t s) {
  if (a.head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (kv == PKV_BF16) return run_multi_dk<128, PKV_BF16>(a, workers, s);
  if (kv == PKV_FP8_E4M3) return run_multi_dk<128, PKV_FP8_E4M3>(a, workers, s);
  if (kv == PKV_INT4) return run_multi_dk<128, PKV_INT4>(a, workers, s);
  return PKV_ERR_UNSUPPORTED;
}

static int dispatch_stream(const DecodeArgs& a, int kv, int workers, hipStream_t s) {
  if (a.pair) return a.head_dim == 128 ? run_stream_pair_d<128>(a, workers, s) : PKV_ERR_UNSUPPORTED;
  switch (a.head_dim) {
    case 32: return stream_d<32>(a, kv, workers, s);
    case 64: return stream_d<64>(a, kv, workers, s);
    case 128: return stream_d<128>(a, kv, workers, s);
    case 256: return stream_d<256>(a, kv, workers, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

static int dispatch_combine(const DecodeArgs& a, int ot, hipStream_t s) {
  if (a.qt > 1) return a.head_dim == 128 ? run_merge_multi_d<128>(a, ot, s) : PKV_ERR_UNSUPPORTED;
  switch (a.head_dim) {
    case 8: return run_combine_d<8>(a, ot, s);
    case 16: return run_combine_d<16>(a, ot, s);
    case 32: return run_combine_d<32>(a, ot, s);
    case 64: return run_combine_d<64>(a, ot, s);
    case 128: return run_combine_d<128>(a, ot, s);
    case 256: return run_combine_d<256>(a, ot, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

// Carve the partial arrays out of a workspace region.
static void bind_workspace(DecodeArgs& a, void* ws, int rows, int hq, int d, int splits, int gt) {
  float* wsf = reinterpret_cast<float*>(ws);
  const size_t nacc = (size_t)rows * hq * splits;
  a.ws_acc = wsf;
  a.ws_m = wsf ? wsf + nacc * d : nullptr;
  a.ws_l = wsf ? a.ws_m + nacc : nullptr;
  a.ws_np = wsf ? reinterpret_cast<int32_t*>(a.ws_l + nacc) : nullptr;
  a.ws_own = wsf && gt > 0 ? a.ws_np + (size_t)rows * (hq / gt) * 2 : nullptr;
}

// Validates everything host-visible and fills DecodeArgs (no launch).
// row_mode 0: decode rows; 1: chunked token rows; 2: chunked request rows.
static int prepare(DecodeArgs& a, void* out, const void* q, int q_dtype, int rows, int hq,
                   const pkv_cache* cache, const int32_t* bt, int bt_stride,
                   const int32_t* seq_lens, int max_seq_len, float scale, int window,
                   int row_mode, const int32_t* qsl, int num_reqs, int max_query_len, int causal,
                   const pkv_decode_plan* plan, void* ws, size_t ws_bytes) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (rows < 0 || hq <= 0 || bt_stride < 0 || max_seq_len < 0 || window < 0) return PKV_ERR_SHAPE;
  if (row_mode != 0 && (num_reqs < 0 || max_query_len < 0 || !qsl)) return PKV_ERR_SHAPE;
  if (hq % cache->num_kv_heads) return PKV_ERR_SHAPE;
  const int want_q = cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  if (q_dtype != want_q) return PKV_ERR_DTYPE;
  const int extra = ((row_mode == 1 && !causal) || row_mode == 3) && max_query_len > 0 ? max_query_len - 1 : 0;
  st = check_plan(plan, rows, hq, cache->num_kv_heads, cache->head_dim, cache->block_size,
                  cache->dtype, max_seq_len, window, extra);
  if (st != PKV_OK) return st;
  if (!(scale > 0.0f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  const int nrows_eff = (row_mode != 0 && num_reqs == 0) ? 0 : rows;
  if (nrows_eff > 0) {
    if (!out || !q || !bt || !seq_lens) return PKV_ERR_NULL;
    if (bt_stride == 0) return PKV_ERR_SHAPE;
  }
  const size_t need = plan_bytes(*plan, rows, hq, cache->head_dim);
  if (need > 0 && nrows_eff > 0 && (!ws || ws_bytes < need)) return PKV_ERR_WORKSPACE;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 15u)) return PKV_ERR_SHAPE;
  const long long items = plan->scheme == 1
      ? (long long)plan->num_workers
      : (long long)rows * hq / plan->heads_per_item * plan->max_splits;
  if (items > 0x7FFFFFFFLL) return PKV_ERR_SHAPE;

  const float log2e = 1.4426950408889634f;
  a = DecodeArgs{};
  a.out = out;
  a.q = q;
  a.row_mode = row_mode;
  a.causal = causal != 0;
  a.skip_single = 0;
  a.qsl = qsl;
  a.num_reqs = num_reqs;
  a.max_query_len = max_query_len;
  a.num_rows = nrows_eff;
  a.num_tokens = rows;
  a.num_q_heads = hq;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = hq / cache->num_kv_heads;
  a.pair = 0;
  if (plan->scheme == 1 && plan->heads_per_item == 2 * a.group && row_mode != 3) {
    // INT4 pair items (checked by check_plan): the kernels see Hkv / 2 heads
    // of two heads' rows each, every item holding both heads' query heads
    a.pair = 1;
    a.num_kv_heads /= 2;
    a.group *= 2;
  }
  a.sub_groups = a.group / plan->heads_per_item;
  a.head_dim = cache->head_dim;
  a.kbase = reinterpret_cast<const char*>(cache->k);
  a.vbase = reinterpret_cast<const char*>(cache->v);
  a.block_stride = cache->block_stride;
  a.num_blocks = cache->num_blocks;
  a.bs_log2 = log2_int(cache->block_size);
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.window = window;
  a.split_blocks = plan->split_blocks;
  a.max_splits = plan->max_splits;
  a.stream_loads = plan->scheme == 1 && (plan->flags & PKV_PLAN_BLOCKS_NOT_SHARED) != 0;
  a.xcd_local = plan->scheme == 1 && (plan->flags & PKV_PLAN_BLOCKS_SHARED) != 0;
  a.stream = plan->scheme == 1;
  a.heads_per_item = plan->heads_per_item;
  a.lead_workers = plan->lead_workers;
  a.trail_pct = plan->trail_share_pct;
  a.qt = 1;
  {
    // LDS one worker may take so that all workers stay resident
    const long long cus = device_cu_count();
    const long long per_cu = plan->num_workers > 0 ? (plan->num_workers + cus - 1) / cus : 1;
    long long budget = kLdsPerCU / (per_cu > 0 ? per_cu : 1);
    if (budget > 64 * 1024) budget = 64 * 1024;
    a.lds_budget = (int32_t)(budget & ~15LL);
  }
  const bool scaled = cache->dtype == PKV_FP8_E4M3 || cache->dtype == PKV_INT4;
  a.scale_log2 = scale * log2e * (scaled ? cache->k_scale : 1.0f);
  a.v_scale = scaled ? cache->v_scale : 1.0f;
  bind_workspace(a, ws, rows, hq, cache->head_dim, plan->max_splits, plan->heads_per_item);
  return PKV_OK;
}

static int run_split(const DecodeArgs& a, const pkv_decode_plan& plan, int kv_dtype, hipStream_t s) {
  if (a.num_rows == 0) return PKV_OK;
  int st;
  if (plan.scheme == 1 && a.qt > 1) st = dispatch_multi(a, kv_dtype, plan.num_workers, s);
  else if (plan.scheme == 1) st = dispatch_stream(a, kv_dtype, plan.num_workers, s);
  else st = dispatch_split(a, a.group / a.sub_groups, kv_dtype, s);
  if (st != PKV_OK) return st;
  return launch_status();
}

static int run_combine(const DecodeArgs& a, int out_dtype, hipStream_t s) {
  if (a.num_rows == 0 || a.max_splits <= 1) return PKV_OK;
  const int st = dispatch_combine(a, out_dtype, s);
  if (st != PKV_OK) return st;
  return launch_status();
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_decode_plan_make(int32_t num_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                                    int32_t max_seq_len, int32_t sliding_window, int32_t flags,
                                    pkv_decode_plan* plan) {
  return make_plan(num_rows, num_q_heads, num_kv_heads, head_dim, block_size, kv_dtype,
                   max_seq_len, sliding_window, 0, true, plan, 0, flags);
}

extern "C" int pkv_decode_plan_resize(int32_t num_rows, int32_t num_q_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_seq_len,
                                      int32_t sliding_window, pkv_decode_plan* plan) {
  if (!plan) return PKV_ERR_NULL;
  if (num_rows < 0 || num_q_heads <= 0 || max_seq_len < 0 || sliding_window < 0) return PKV_ERR_SHAPE;
  if (!head_dim_supported(head_dim) || !block_size_supported(block_size)) return PKV_ERR_UNSUPPORTED;
  if (!plan_flags_ok(plan->flags)) return PKV_ERR_SHAPE;
  if (plan->heads_per_item < 1 || num_q_heads % plan->heads_per_item) return PKV_ERR_SHAPE;
  const int nvis = max_visible_blocks(max_seq_len, block_size, sliding_window, 0);
  if (plan->scheme == 1) {
    if (plan->split_blocks < 1 || plan->num_workers < 1) return PKV_ERR_SHAPE;
    if (plan->lead_workers < 0 || plan->lead_workers > plan->num_workers) return PKV_ERR_SHAPE;
    if (plan->trail_share_pct < 1 || plan->trail_share_pct > 100) return PKV_ERR_SHAPE;
    plan->max_splits = ceil_div(nvis, plan->split_blocks) + 1;
  } else if (plan->scheme == 0) {
    if (plan->split_blocks < 1 || plan->split_blocks > 64) return PKV_ERR_SHAPE;
    plan->max_splits = ceil_div(nvis, plan->split_blocks);
  } else {
    return PKV_ERR_SHAPE;
  }
  plan->workspace_bytes = plan_bytes(*plan, num_rows, num_q_heads, head_dim);
  return PKV_OK;
}

extern "C" int pkv_paged_attention_decode_partials(
    void* out, const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
    const pkv_cache* cache, const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale, int32_t sliding_window,
    const pkv_decode_plan* plan, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeArgs a;
  int st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride,
                   seq_lens, max_seq_len, softmax_scale, sliding_window, 0, nullptr, 0, 0, 1, plan,
                   workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  return run_split(a, *plan, cache->dtype, stream);
}

extern "C" int pkv_paged_attention_decode_step(
    void* out, const void* q, int32_t q_dtype, const void* new_k, const void* new_v, int32_t num_seqs,
    int32_t num_q_heads, const pkv_cache* cache, const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale, int32_t sliding_window,
    const pkv_decode_plan* plan, void* workspace, size_t workspace_bytes, int64_t* slot_mapping,
    hipStream_t stream) {
  DecodeArgs a;
  int st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride,
                   seq_lens, max_seq_len, softmax_scale, sliding_window, 0, nullptr, 0, 0, 1, plan,
                   workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (plan->scheme != 1) return PKV_ERR_UNSUPPORTED;
  if (cache->dtype == PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs == 0) return PKV_OK;
  if (!new_k || !new_v) return PKV_ERR_NULL;
  if (!aligned16(new_k) || !aligned16(new_v)) return PKV_ERR_SHAPE;
  if (!workspace) return PKV_ERR_WORKSPACE;
  a.new_token = 1;
  a.new_k = new_k;
  a.new_v = new_v;
  a.slots_out = slot_mapping;
  a.kv_dtype = cache->dtype;
  a.kv_heads = cache->num_kv_heads;
  a.inv_k_scale = 1.0f / cache->k_scale;
  a.inv_v_scale = 1.0f / cache->v_scale;
  st = run_split(a, *plan, cache->dtype, stream);
  if (st != PKV_OK) return st;
  st = dispatch_combine(a, PKV_BF16, stream);
  if (st != PKV_OK) return st;
  return launch_status();
}

extern "C" int pkv_paged_attention_decode_combine(void* out, int32_t out_dtype, int32_t num_seqs,
                                                  int32_t num_q_heads, int32_t head_dim,
                                                  int32_t block_size, const int32_t* seq_lens,
                                                  int32_t sliding_window,
                                                  const pkv_decode_plan* plan,
                                                  const void* workspace, size_t workspace_bytes,
                                                  hipStream_t stream) {
  if (!plan) return PKV_ERR_NULL;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || sliding_window < 0) return PKV_ERR_SHAPE;
  if (!head_dim_supported(head_dim) || !block_size_supported(block_size)) return PKV_ERR_UNSUPPORTED;
  if (plan->split_blocks < 1 || plan->max_splits < 1 || plan->heads_per_item < 1 ||
      num_q_heads % plan->heads_per_item || (plan->scheme != 0 && plan->scheme != 1))
    return PKV_ERR_SHAPE;
  if (num_seqs == 0 || plan->max_splits == 1) return PKV_OK;
  if (!out || !seq_lens) return PKV_ERR_NULL;
  const size_t need = plan_bytes(*plan, num_seqs, num_q_heads, head_dim);
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  DecodeArgs a = {};
  a.out = out;
  a.num_rows = num_seqs;
  a.num_tokens = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.bs_log2 = log2_int(block_size);
  a.seq_lens = seq_lens;
  // Bounds are the split phase's business: rows it rejected carry NaN in
  // every split slot (fixed splits) or a piece count of 0 (balanced).
  a.max_seq_len = 0x7FFFFFFF;
  a.bt_stride = 0x7FFFFFFF;
  a.window = sliding_window;
  a.split_blocks = plan->split_blocks;
  a.max_splits = plan->max_splits;
  a.stream = plan->scheme == 1;
  a.heads_per_item = plan->heads_per_item;
  a.v_scale = 1.0f;
  bind_workspace(a, const_cast<void*>(workspace), num_seqs, num_q_heads, head_dim, plan->max_splits,
                 plan->heads_per_item);
  return run_combine(a, out_dtype, stream);
}

extern "C" int pkv_paged_attention_decode(void* out, const void* q, int32_t q_dtype,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          const pkv_cache* cache, const int32_t* block_table,
                                          int32_t bt_stride, const int32_t* seq_lens,
                                          int32_t max_seq_len, float softmax_scale,
                                          int32_t sliding_window, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (q_dtype != (cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16)) return PKV_ERR_DTYPE;
  pkv_decode_plan plan;
  st = make_plan(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim, cache->block_size,
                 cache->dtype, max_seq_len, sliding_window, 0, true, &plan);
  if (st != PKV_OK) return st;
  DecodeArgs a;
  st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride, seq_lens,
               max_seq_len, softmax_scale, sliding_window, 0, nullptr, 0, 0, 1, &plan, workspace,
               workspace_bytes);
  if (st != PKV_OK) return st;
  st = run_split(a, plan, cache->dtype, stream);
  if (st != PKV_OK) return st;
  return run_combine(a, q_dtype, stream);
}

// ---- decode with the library's own scratch (callers that cannot allocate)
//
// The decode's partials and piece counts live in this file-scope device
// array instead of a caller's workspace.  Every GPU the library runs on
// holds its own copy from module load until the process ends.  Host code
// never names the array directly (its host-side name is not a device
// address): the device address is looked up once per device, with that
// device current, and passed to the kernels like any workspace.
static __device__ __align__(256) char scratch[PKV_STATIC_SCRATCH_BYTES];

static int static_scratch(void** ptr) {
  static std::mutex mu;
  static void* dev_ptr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return PKV_OK;
}

extern "C" int pkv_paged_attention_decode_static(void* out, const void* q, int32_t q_dtype,
                                                 int32_t num_seqs, int32_t num_q_heads,
                                                 const pkv_cache* cache, const int32_t* block_table,
                                                 int32_t bt_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float softmax_scale,
                                                 int32_t sliding_window, hipStream_t stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (q_dtype != (cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16)) return PKV_ERR_DTYPE;
  pkv_decode_plan plan;
  st = make_plan(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim, cache->block_size,
                 cache->dtype, max_seq_len, sliding_window, 0, true, &plan);
  if (st != PKV_OK) return st;
  if (plan.workspace_bytes > PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (num_seqs > 0 && plan.workspace_bytes > 0) {
    st = static_scratch(&ws);
    if (st != PKV_OK) return st;
  }
  DecodeArgs a;
  st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride, seq_lens,
               max_seq_len, softmax_scale, sliding_window, 0, nullptr, 0, 0, 1, &plan, ws,
               plan.workspace_bytes);
  if (st != PKV_OK) return st;
  st = run_split(a, plan, cache->dtype, stream);
  if (st != PKV_OK) return st;
  return run_combine(a, q_dtype, stream);
}

// ---- a second stream per device, on which a chunked call runs its prefill
// part beside its decode part.  Events order the side stream after the
// caller's stream's earlier work and the caller's stream after the side
// stream's, so the call behaves as if it ran on the caller's stream alone.
// One mutex covers each fork / join sequence, so calls from several host
// threads never interleave their event records.  Default priority (the
// stream is created like any other).
struct SideStream {
  hipStream_t stream;
  hipEvent_t fork, join;
};
static std::mutex g_side_mu;

// Under g_side_mu.
static int side_stream(SideStream** out) {
  static SideStream side[64];
  static bool made[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_ERR_HIP;
  if (!made[dev]) {
    SideStream x;
    if (hipStreamCreateWithFlags(&x.stream, hipStreamNonBlocking) != hipSuccess) return PKV_ERR_HIP;
    if (hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) != hipSuccess) return PKV_ERR_HIP;
    if (hipEventCreateWithFlags(&x.join, hipEventDisableTiming) != hipSuccess) return PKV_ERR_HIP;
    side[dev] = x;
    made[dev] = true;
  }
  *out = &side[dev];
  return PKV_OK;
}

// The chunked form runs two passes over disjoint rows: requests with one
// query take the decode kernels (rows = requests), every other request's
// tokens take the per-token rows.  Each pass has its own workspace region.
struct ChunkPlans {
  pkv_decode_plan single, multi, spec;
  size_t single_bytes, multi_bytes;   // multi_bytes: the multi-query requests' region
  bool prefill;           // multi-query requests on the matrix-core prefill kernel
  int spec_qt;            // > 0: multi-query requests as multi-token decode items
  int spec_heads;         // query heads per multi-token item
};

// Query tokens per item when the step's multi-query requests are short
// enough to run as decode items (2 .. 8 tokens: a power of two at least
// max_query_len), else 0.  Items hold as many of the group's heads as fit
// in 16 MFMA rows.
static int multi_token_qt(const pkv_cache* c, int hq, int max_query_len, int num_reqs) {
  if (max_query_len < 2 || max_query_len > 8 || num_reqs > kMaxStreamRows) return 0;
  if (!mfma_eligible(c->dtype, c->head_dim, c->block_size)) return 0;
  if (c->head_dim != 128) return 0;
  const int g = hq / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return 0;
  int qt = 2;
  while (qt < max_query_len) qt <<= 1;
  return qt;
}

// flags: PKV_PLAN_* bits for the balanced plans (they change loads, not sizes)
static int chunk_plans(int num_tokens, int num_reqs, int hq, const pkv_cache* c, int max_query_len,
                       int max_seq_len, int window, ChunkPlans& p, int flags = 0) {
  int st = make_plan(num_reqs, hq, c->num_kv_heads, c->head_dim, c->block_size, c->dtype,
                     max_seq_len, window, 0, true, &p.single, 0, flags);
  if (st != PKV_OK) return st;
  // Non-causal windowed rows see up to W + q_len - 1 keys; size for that case.
  const int extra = max_query_len > 0 ? max_query_len - 1 : 0;
  st = make_plan(num_tokens, hq, c->num_kv_heads, c->head_dim, c->block_size, c->dtype,
                 max_seq_len, window, extra, false, &p.multi);
  // INT4 has no vector-ALU fallback: its multi-query requests need the
  // multi-token items (checked below)
  const bool multi_ok = st == PKV_OK;
  if (!multi_ok && !(st == PKV_ERR_UNSUPPORTED && c->dtype == PKV_INT4)) return st;
  p.single_bytes = (p.single.workspace_bytes + 255) & ~(size_t)255;
  p.spec_qt = multi_token_qt(c, hq, max_query_len, num_reqs);
  if (p.spec_qt > 0) {
    // one item per (request, head sub-group): its heads times the tokens
    const int g = hq / c->num_kv_heads;
    // the whole group where it fits in the item rows (bf16 measured fastest
    // with 16: items of 16 rows beat 8 and 4 on 64 x 4-token requests, 144
    // vs 149 vs 201 us)
    p.spec_heads = g;
    while (p.spec_heads > 1 && p.spec_heads * p.spec_qt > max_item_rows(c->dtype)) p.spec_heads >>= 1;
    st = make_plan(num_reqs, hq * p.spec_qt, c->num_kv_heads, c->head_dim, c->block_size, c->dtype,
                   max_seq_len, window, max_query_len - 1, true, &p.spec, p.spec_heads * p.spec_qt, flags);
    if (st != PKV_OK || p.spec.scheme != 1) p.spec_qt = 0;
  }
  p.prefill = p.spec_qt == 0 && prefill_supported(c->dtype, c->head_dim, hq / c->num_kv_heads,
                                                  max_seq_len, c->block_size, window, max_query_len);
  if (max_query_len > 1 && p.spec_qt == 0 && !p.prefill && !multi_ok) return PKV_ERR_UNSUPPORTED;
  p.multi_bytes = max_query_len <= 1 ? 0
                  : p.spec_qt > 0   ? p.spec.workspace_bytes
                  : p.prefill       ? prefill_workspace_bytes(c->head_dim)
                                    : p.multi.workspace_bytes;
  return PKV_OK;
}

extern "C" int pkv_chunked_workspace_size(int32_t num_tokens, int32_t num_reqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t kv_dtype, int32_t max_query_len,
                                          int32_t max_seq_len, int32_t sliding_window,
                                          size_t* bytes) {
  if (!bytes) return PKV_ERR_NULL;
  if (num_tokens < 0 || num_reqs < 0 || max_query_len < 0) return PKV_ERR_SHAPE;
  pkv_cache c = {};
  c.num_kv_heads = num_kv_heads;
  c.head_dim = head_dim;
  c.block_size = block_size;
  c.dtype = kv_dtype;
  ChunkPlans p;
  const int st = chunk_plans(num_tokens, num_reqs, num_q_heads, &c, max_query_len, max_seq_len,
                             sliding_window, p);
  if (st != PKV_OK) return st;
  *bytes = p.single_bytes + p.multi_bytes;
  return PKV_OK;
}

extern "C" int pkv_paged_attention_chunked(void* out, const void* q, int32_t q_dtype,
                                           int32_t num_tokens, int32_t num_q_heads,
                                           const int32_t* query_start_loc,
                                           const int32_t* seq_lens, int32_t num_reqs,
                                           int32_t max_query_len, const pkv_cache* cache,
                                           const int32_t* block_table, int32_t bt_stride,
                                           int32_t max_seq_len, float softmax_scale,
                                           int32_t causal, int32_t sliding_window, int32_t flags,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0 || num_reqs < 0 || max_query_len < 0) return PKV_ERR_SHAPE;
  if (q_dtype != (cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16)) return PKV_ERR_DTYPE;
  if (num_tokens == 0 || num_reqs == 0) return PKV_OK;
  if (!query_start_loc) return PKV_ERR_NULL;
  if (!plan_flags_ok(flags)) return PKV_ERR_SHAPE;
  ChunkPlans p;
  st = chunk_plans(num_tokens, num_reqs, num_q_heads, cache, max_query_len, max_seq_len,
                   sliding_window, p, flags);
  if (st != PKV_OK) return st;
  if (p.single_bytes + p.multi_bytes > 0 && (!workspace || workspace_bytes < p.single_bytes + p.multi_bytes))
    return PKV_ERR_WORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  // requests with a single query (causal or not, one query sees keys <= p)
  DecodeArgs a1;
  st = prepare(a1, out, q, q_dtype, num_reqs, num_q_heads, cache, block_table, bt_stride, seq_lens,
               max_seq_len, softmax_scale, sliding_window, 2, query_start_loc, num_reqs,
               max_query_len, 1, &p.single, ws, p.single_bytes);
  if (st != PKV_OK) return st;
  a1.num_tokens = num_tokens;
  if (max_query_len > 1 && p.spec_qt > 0) {
    // every request (1 .. 8 query tokens) as decode items of heads x query
    // tokens; the plan and workspace count one "head" per (token, head) pair
    if (!out || !q || !block_table || !seq_lens) return PKV_ERR_NULL;
    DecodeArgs a3;
    st = prepare(a3, out, q, q_dtype, num_reqs, num_q_heads * p.spec_qt, cache, block_table, bt_stride,
                 seq_lens, max_seq_len, softmax_scale, sliding_window, 3, query_start_loc, num_reqs,
                 max_query_len, causal, &p.spec, ws + p.single_bytes, p.multi_bytes);
    if (st != PKV_OK) return st;
    a3.num_q_heads = num_q_heads;
    a3.group = num_q_heads / cache->num_kv_heads;
    a3.sub_groups = a3.group / p.spec_heads;
    a3.heads_per_item = p.spec_heads;
    a3.qt = p.spec_qt;
    a3.num_tokens = num_tokens;
    st = run_split(a3, p.spec, cache->dtype, stream);
    if (st != PKV_OK) return st;
    // the items hold the single-query requests too: no separate pass
    return run_combine(a3, q_dtype, stream);
  } else if (max_query_len > 1 && p.prefill) {
    if (!out || !q || !block_table || !seq_lens) return PKV_ERR_NULL;
    if (bt_stride <= 0 || max_seq_len < 0 || sliding_window < 0) return PKV_ERR_SHAPE;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return PKV_ERR_SHAPE;
    if (num_q_heads % cache->num_kv_heads) return PKV_ERR_SHAPE;
    PrefillArgs pa = {};
    pa.out = out;
    pa.q = q;
    pa.qsl = query_start_loc;
    pa.seq_lens = seq_lens;
    pa.num_reqs = num_reqs;
    pa.num_tokens = num_tokens;
    pa.max_query_len = max_query_len;
    pa.max_seq_len = max_seq_len;
    pa.num_q_heads = num_q_heads;
    pa.num_kv_heads = cache->num_kv_heads;
    pa.kbase = reinterpret_cast<const char*>(cache->k);
    pa.vbase = reinterpret_cast<const char*>(cache->v);
    pa.block_stride = cache->block_stride;
    pa.num_blocks = cache->num_blocks;
    pa.bs_log2 = log2_int(cache->block_size);
    pa.bt = block_table;
    pa.bt_stride = bt_stride;
    pa.causal = causal != 0;
    pa.window = sliding_window;
    const float log2e = 1.4426950408889634f;
    const bool scaled = cache->dtype == PKV_FP8_E4M3 || cache->dtype == PKV_INT4;
    pa.scale_log2 = softmax_scale * log2e * (scaled ? cache->k_scale : 1.0f);
    pa.v_scale = scaled ? cache->v_scale : 1.0f;
    pa.part = reinterpret_cast<float*>(ws + p.single_bytes);
    // The prefill tile runs on the side stream, the single-query requests'
    // decode pass on the caller's stream: the two kernels are launched
    // together and the GPU runs whatever fits of the second beside the
    // first (their ramps and tails overlap; their full-occupancy bodies
    // cannot share a compute unit at these register counts).
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side = nullptr;
    st = side_stream(&side);
    if (st != PKV_OK) return st;
    if (hipEventRecord(side->fork, stream) != hipSuccess) return PKV_ERR_HIP;
    if (hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) return PKV_ERR_HIP;
    st = launch_prefill(pa, cache->dtype, cache->head_dim, side->stream);
    if (st == PKV_OK) st = launch_status();
    if (hipEventRecord(side->join, side->stream) != hipSuccess) return PKV_ERR_HIP;
    int st2 = run_split(a1, p.single, cache->dtype, stream);
    if (st2 == PKV_OK) st2 = run_combine(a1, q_dtype, stream);
    // the caller's stream waits for the prefill part whatever happened
    if (hipStreamWaitEvent(stream, side->join, 0) != hipSuccess) return PKV_ERR_HIP;
    return st != PKV_OK ? st : st2;
  } else if (max_query_len > 1) {
    DecodeArgs a2;
    st = prepare(a2, out, q, q_dtype, num_tokens, num_q_heads, cache, block_table, bt_stride,
                 seq_lens, max_seq_len, softmax_scale, sliding_window, 1, query_start_loc, num_reqs,
                 max_query_len, causal, &p.multi, ws ? ws + p.single_bytes : nullptr, p.multi_bytes);
    if (st != PKV_OK) return st;
    a2.skip_single = 1;
    st = run_split(a2, p.multi, cache->dtype, stream);
    if (st != PKV_OK) return st;
    st = run_combine(a2, q_dtype, stream);
    if (st != PKV_OK) return st;
  }
  st = run_split(a1, p.single, cache->dtype, stream);
  if (st != PKV_OK) return st;
  return run_combine(a1, q_dtype, stream);
}
