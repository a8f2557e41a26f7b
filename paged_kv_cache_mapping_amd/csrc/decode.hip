// Paged decode attention: split phase (per-split online softmax) and combine.
//
// Attention reads each sequence's past K/V by following its block table
// instead of assuming one contiguous tensor ("vLLM의 KV cache 연결 흐름",
// sections on slot mapping and on the metadata handed to the backend).  The
// softmax normaliser spans every block ("Understanding PageAttention Memory
// Optimization", section "Handling Softmax Across Blocks"); kernels tile the
// keys and keep a running (online) softmax (Chinese original of the
// worker-side page, section "Worker与ModelRunner的协作").  Grouped-query
// heads share a KV head and a sliding window limits keys to the most recent W
// positions ("Deep Dive into vLLM Worker-Side GPU KV Cache Initialization",
// section "Hybrid Attention Mechanisms").
//
// Work decomposition (MI355X): one wave per (row, KV head, group of query
// heads, split of consecutive visible blocks).  A wave reads a token row of
// one KV head with LPR lanes x 16 bytes (RPW = 64 / LPR rows per load), keeps
// one online-softmax state per lane for the rows it sees, and merges the
// lanes' states with cross-lane exchanges at the end.  Scores reduce over the
// LPR lanes of a row with DPP.  Sequences with more than one split leave base-2
// partial states (m, l, acc) in the workspace for the combine kernel.
#include <math.h>

#include "common.h"
#include "host_common.h"

namespace pkv {

constexpr float kLazyRescale = 8.0f;  // keep a stale max until a score beats it by 2^8

struct DecodeArgs {
  void* out;
  const void* q;
  // Row mode.  Decode: row b is sequence b, its query token is row b of q/out.
  // Chunked: row t is token t of the step; its request is found through
  // query_start_loc, its position is seq_len - q_len + (t - qsl[r]).
  int32_t chunked;
  int32_t causal;
  int32_t single_only;      // chunked: skip rows of requests with q_len != 1
  const int32_t* qsl;
  int32_t num_reqs;
  int32_t max_query_len;
  int32_t num_rows;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;            // query heads per KV head
  int32_t sub_groups;       // group / heads per work item
  int32_t head_dim;
  const char* kbase;
  const char* vbase;
  int64_t block_stride;     // elements
  int32_t num_blocks;
  int32_t bs_log2;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t window;
  int32_t split_blocks;
  int32_t max_splits;
  float scale_log2;         // softmax_scale * log2(e) (* k_scale for fp8)
  float v_scale;            // 1, or the fp8 V scale
  float* ws_acc;
  float* ws_m;
  float* ws_l;
};

// What one row attends to.
struct RowInfo {
  bool skip;      // not this kernel's row (padding, or handled elsewhere)
  bool valid;     // lengths and block-table row consistent
  int req;        // block-table row
  int lo, hi;     // inclusive visible key positions
  int first_blk;  // lo / block_size
  int nvis;       // visible logical blocks
};

__device__ __forceinline__ RowInfo row_info(const DecodeArgs& a, int row) {
  RowInfo r;
  r.skip = false;
  r.valid = false;
  r.req = row;
  int L, p;
  if (!a.chunked) {
    L = a.seq_lens[row];
    p = L - 1;
    if (L <= 0 || L > a.max_seq_len) return r;
  } else {
    const int end = a.qsl[a.num_reqs];
    if (row < a.qsl[0] || row >= end) { r.skip = true; return r; }
    int lo = 0, hi = a.num_reqs;  // largest q with qsl[q] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.qsl[mid] <= row) lo = mid; else hi = mid;
    }
    r.req = lo;
    const int ql = a.qsl[lo + 1] - a.qsl[lo];
    if (a.single_only && ql != 1) { r.skip = true; return r; }
    L = a.seq_lens[lo];
    if (L <= 0 || L > a.max_seq_len || ql > L || ql > a.max_query_len) return r;
    p = L - ql + (row - a.qsl[lo]);
  }
  r.hi = (a.chunked && !a.causal) ? L - 1 : p;
  r.lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  if (r.lo > r.hi) return r;
  r.first_blk = r.lo >> a.bs_log2;
  const int last = r.hi >> a.bs_log2;
  if (last >= a.bt_stride) return r;
  r.nvis = last - r.first_blk + 1;
  r.valid = true;
  return r;
}

template <typename T>
__device__ __forceinline__ T shfl_xor_t(T v, int m) { return __shfl_xor(v, m); }

// Store n consecutive floats of one output row as the output dtype.
template <int OT, int N>
__device__ __forceinline__ void store_out(void* base, int64_t elem, const float (&v)[N]) {
  if constexpr (OT == PKV_F32) {
    float* p = reinterpret_cast<float*>(base) + elem;
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = v[i];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base) + elem;
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        uint4 w;
        w.x = f32_to_bf16_rne(v[8 * i + 0]) | (f32_to_bf16_rne(v[8 * i + 1]) << 16);
        w.y = f32_to_bf16_rne(v[8 * i + 2]) | (f32_to_bf16_rne(v[8 * i + 3]) << 16);
        w.z = f32_to_bf16_rne(v[8 * i + 4]) | (f32_to_bf16_rne(v[8 * i + 5]) << 16);
        w.w = f32_to_bf16_rne(v[8 * i + 6]) | (f32_to_bf16_rne(v[8 * i + 7]) << 16);
        reinterpret_cast<uint4*>(p)[i] = w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i] = (uint16_t)f32_to_bf16_rne(v[i]);
    }
  }
}

// --------------------------------------------------------------------------
// Split phase.  D: head_dim; GT: query heads per work item; KV: cache dtype;
// QT: query/output dtype (F32 with an F32 cache, BF16 otherwise).
template <int D, int GT, int KV, int QT>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  constexpr int kElt = KV == PKV_F32 ? 4 : (KV == PKV_BF16 ? 2 : 1);
  constexpr int kRowBytes = D * kElt;
  constexpr int kVec = kRowBytes >= 16 ? 16 : kRowBytes;  // bytes per lane per row
  constexpr int LPR = kRowBytes / kVec;                    // lanes per row
  constexpr int EPL = kVec / kElt;                         // elements per lane
  constexpr int RPW = kWave / LPR;                         // rows per wave load
  constexpr int U = RPW >= 16 ? 1 : 16 / RPW;              // loads per step (>= 16 rows)
  constexpr bool kBf16Dot = (QT == PKV_BF16);              // q.k on packed bf16 pairs
  static_assert(EPL % 2 == 0 || !kBf16Dot, "bf16 dot needs pairs");
  constexpr int QW = kBf16Dot ? EPL / 2 : EPL;             // q registers per head

  const int lane = threadIdx.x;
  const int grp = lane / LPR;
  const int sub = lane % LPR;

  const int kvgroups = a.num_kv_heads * a.sub_groups;
  int w = blockIdx.x;
  const int s = w % a.max_splits;
  w /= a.max_splits;
  const int kvg = w % kvgroups;
  const int b = w / kvgroups;
  const int kvh = kvg / a.sub_groups;
  const int h0 = kvh * a.group + (kvg % a.sub_groups) * GT;

  const RowInfo span = row_info(a, b);
  if (span.skip) return;
  const int tok = b;
  const int64_t out_row = ((int64_t)tok * a.num_q_heads + h0) * D;
  if (!span.valid) {
    // Invalid row: NaN output (split 0) and NaN partials in every split slot,
    // so that a combine pass over this row can only produce NaN.
    if (grp == 0) {
      float nanv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) nanv[e] = __builtin_nanf("");
      for (int h = 0; h < GT; ++h) {
        if (s == 0) store_out<QT, EPL>(a.out, out_row + h * D + sub * EPL, nanv);
        if (a.max_splits > 1) {
          const int64_t pr = ((int64_t)b * a.num_q_heads + h0 + h) * a.max_splits + s;
          float* dst = a.ws_acc + pr * D + sub * EPL;
          for (int e = 0; e < EPL; ++e) dst[e] = nanv[e];
          if (sub == 0) {
            a.ws_m[pr] = 0.f;
            a.ws_l[pr] = nanv[0];
          }
        }
      }
    }
    return;
  }
  const int nsplit = ceil_div(span.nvis, a.split_blocks);
  if (s >= nsplit) return;

  const int blk_begin = span.first_blk + s * a.split_blocks;
  const int nb = min(a.split_blocks, span.first_blk + span.nvis - blk_begin);
  const int bs = 1 << a.bs_log2;

  // Stage this split's block ids in a register: lane i holds entry i.
  int tab = -1;
  if (lane < nb) tab = a.bt[(int64_t)span.req * a.bt_stride + blk_begin + lane];
  const bool bad = (lane < nb) && (tab < 0 || tab >= a.num_blocks);
  const bool any_bad = __ballot(bad) != 0;

  // Query slice of this lane: heads h0..h0+GT-1, elements sub*EPL .. +EPL.
  uint32_t qr[GT][QW];
  float qf[GT][kBf16Dot ? 1 : EPL];
  if constexpr (kBf16Dot) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)tok * a.num_q_heads + h0) * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int i = 0; i < QW; ++i)
        qr[h][i] = reinterpret_cast<const uint32_t*>(qp + h * D)[i];
    }
  } else {
    const float* qp = reinterpret_cast<const float*>(a.q) + ((int64_t)tok * a.num_q_heads + h0) * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] = qp[h * D + e];
  }
  (void)qr;
  (void)qf;

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  if (!any_bad) {
    const int pos0 = blk_begin << a.bs_log2;           // first position of the split
    const int pos_end = min((blk_begin + nb) << a.bs_log2, span.hi + 1);
    const int ntiles = ceil_div(pos_end - pos0, RPW);
    const int nsteps = ceil_div(ntiles, U);
    const int64_t head_off = (int64_t)kvh * D + sub * EPL;  // elements inside a token row
    const int64_t row_elems = (int64_t)a.num_kv_heads * D;

    uint4 ka[U], va[U], kb2[U], vb2[U];
    bool la[U], lb[U];

    auto issue = [&](int step, uint4 (&kd)[U], uint4 (&vd)[U], bool (&vl)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pos = pos0 + (step * U + u) * RPW + grp;
        const bool live = pos >= span.lo && pos < pos_end;
        const int local = (pos >> a.bs_log2) - blk_begin;
        const int phys = __shfl(tab, local < 0 ? 0 : (local > 63 ? 63 : local));
        vl[u] = live;
        kd[u] = make_uint4(0, 0, 0, 0);
        vd[u] = make_uint4(0, 0, 0, 0);
        if (live) {
          const int64_t e = (int64_t)phys * a.block_stride + (pos & (bs - 1)) * row_elems + head_off;
          if constexpr (kVec == 16) {
            kd[u] = *reinterpret_cast<const uint4*>(a.kbase + e * kElt);
            vd[u] = *reinterpret_cast<const uint4*>(a.vbase + e * kElt);
          } else if constexpr (kVec == 8) {
            uint2 k2 = *reinterpret_cast<const uint2*>(a.kbase + e * kElt);
            uint2 v2 = *reinterpret_cast<const uint2*>(a.vbase + e * kElt);
            kd[u] = make_uint4(k2.x, k2.y, 0, 0);
            vd[u] = make_uint4(v2.x, v2.y, 0, 0);
          }
        }
      }
    };

    // One step: U row loads of K and V per lane, folded into the state.
    auto compute = [&](const uint4 (&kd)[U], const uint4 (&vd)[U], const bool (&vl)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint4 kw = kd[u];
        const uint4 vw = vd[u];
        const bool live = vl[u];
        const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
        const uint32_t vwa[4] = {vw.x, vw.y, vw.z, vw.w};

        // K and V of this lane's row chunk in compute form.
        float vf[EPL];
        uint32_t kp[kBf16Dot ? EPL / 2 : 1];
        float kf[kBf16Dot ? 1 : EPL];
        (void)kp;
        (void)kf;
        if constexpr (KV == PKV_BF16) {
#pragma unroll
          for (int i = 0; i < EPL / 2; ++i) {
            vf[2 * i] = bf16_lo(vwa[i]);
            vf[2 * i + 1] = bf16_hi(vwa[i]);
            if constexpr (kBf16Dot) kp[i] = kwa[i];
            else { kf[2 * i] = bf16_lo(kwa[i]); kf[2 * i + 1] = bf16_hi(kwa[i]); }
          }
        } else if constexpr (KV == PKV_F32) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            vf[i] = as_float(vwa[i]);
            kf[i] = as_float(kwa[i]);
          }
        } else {  // fp8 codes, 4 per dword
#pragma unroll
          for (int i = 0; i < EPL / 4; ++i) {
            const f32x2 v01 = e4m3x2_to_f32<false>(vwa[i]);
            const f32x2 v23 = e4m3x2_to_f32<true>(vwa[i]);
            vf[4 * i] = v01.x; vf[4 * i + 1] = v01.y; vf[4 * i + 2] = v23.x; vf[4 * i + 3] = v23.y;
            if constexpr (kBf16Dot) {
              kp[2 * i] = e4m3x2_to_bf16x2<false>(kwa[i]);
              kp[2 * i + 1] = e4m3x2_to_bf16x2<true>(kwa[i]);
            } else {
              const f32x2 k01 = e4m3x2_to_f32<false>(kwa[i]);
              const f32x2 k23 = e4m3x2_to_f32<true>(kwa[i]);
              kf[4 * i] = k01.x; kf[4 * i + 1] = k01.y; kf[4 * i + 2] = k23.x; kf[4 * i + 3] = k23.y;
            }
          }
        }

#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float sc = 0.f;
          if constexpr (kBf16Dot) {
#pragma unroll
            for (int i = 0; i < EPL / 2; ++i) sc = dot2_bf16(qr[h][i], kp[i], sc);
          } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sc = fmaf(qf[h][e], kf[e], sc);
          }
          sc = group_sum<LPR>(sc);
          const float z = sc * a.scale_log2;
          if (live && z > m[h] + kLazyRescale) {
            const float alpha = __builtin_amdgcn_exp2f(m[h] - z);
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
            m[h] = z;
          }
          const float p = live ? __builtin_amdgcn_exp2f(z - m[h]) : 0.f;
          l[h] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    };

    // Two register sets: the next step's loads are in flight while the
    // current step is folded in.
    if (nsteps > 0) issue(0, ka, va, la);
    for (int st = 0; st < nsteps; st += 2) {
      if (st + 1 < nsteps) issue(st + 1, kb2, vb2, lb);
      compute(ka, va, la);
      if (st + 1 < nsteps) {
        if (st + 2 < nsteps) issue(st + 2, ka, va, la);
        compute(kb2, vb2, lb);
      }
    }

    // Merge the RPW row-lanes that share a column chunk (same `sub`).
#pragma unroll
    for (int step = LPR; step < kWave; step <<= 1) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float mo = shfl_xor_t(m[h], step);
        const float lo_ = shfl_xor_t(l[h], step);
        const float mn = fmaxf(m[h], mo);
        const float fa = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
        const float fb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l[h] = l[h] * fa + lo_ * fb;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float ao = shfl_xor_t(acc[h][e], step);
          acc[h][e] = acc[h][e] * fa + ao * fb;
        }
        m[h] = mn;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      m[h] = 0.f;
      l[h] = __builtin_nanf("");
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_nanf("");
    }
  }

  if (grp != 0) return;
  if (nsplit == 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float inv = a.v_scale / l[h];
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[h][e] * inv;
      store_out<QT, EPL>(a.out, out_row + h * D + sub * EPL, o);
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const int64_t pr = ((int64_t)b * a.num_q_heads + h0 + h) * a.max_splits + s;
    float* dst = a.ws_acc + pr * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = acc[h][e];
    if (sub == 0) {
      a.ws_m[pr] = m[h];
      a.ws_l[pr] = l[h];
    }
  }
}

// --------------------------------------------------------------------------
// Combine phase: one wave per (row, query head) with more than one split.
template <int D, int OT>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = D >= kWave ? D / kWave : 1;  // elements per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_q_heads;
  const int b = blockIdx.x / a.num_q_heads;
  // Rows the split phase rejected hold NaN in every split slot; the split
  // count is clamped to the slots that exist.
  const RowInfo span = row_info(a, b);
  if (span.skip || !span.valid) return;
  const int tok = b;
  const int nsplit = min(ceil_div(span.nvis, a.split_blocks), a.max_splits);
  if (nsplit <= 1) return;

  const int64_t pr0 = ((int64_t)b * a.num_q_heads + h) * a.max_splits;
  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, a.ws_m[pr0 + s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float den = 0.f;
  float num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  const bool active = D >= kWave || lane < D;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = a.ws_m[pr0 + s];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    den = fmaf(wgt, a.ws_l[pr0 + s], den);
    if (active) {
      const float* src = a.ws_acc + (pr0 + s) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) num[i] = fmaf(wgt, src[lane + i * kWave], num[i]);
    }
  }
  if (!active) return;
  const float inv = a.v_scale / den;
  const int64_t out_row = ((int64_t)tok * a.num_q_heads + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float v[1] = {num[i] * inv};
    store_out<OT, 1>(a.out, out_row + lane + i * kWave, v);
  }
}

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
  const int win = ceil_div(window + extra + bs - 1, bs);
  return full < win ? full : win;
}

static int heads_per_item(int group) {
  if (group >= 8) return (group % 8 == 0) ? 8 : 0;
  return (group == 1 || group == 2 || group == 4) ? group : 0;
}

static size_t partial_bytes(int rows, int hq, int splits, int d) {
  return (size_t)rows * hq * splits * ((size_t)d + 2) * sizeof(float);
}

static int make_plan(int rows, int hq, int hkv, int d, int bs, int max_seq_len, int window,
                     int extra, pkv_decode_plan* plan) {
  if (!plan) return PKV_ERR_NULL;
  if (rows < 0 || hq <= 0 || hkv <= 0 || max_seq_len < 0 || window < 0) return PKV_ERR_SHAPE;
  if (hq % hkv) return PKV_ERR_SHAPE;
  if (!head_dim_supported(d) || !block_size_supported(bs)) return PKV_ERR_UNSUPPORTED;
  const int gt = heads_per_item(hq / hkv);
  if (gt == 0) return PKV_ERR_UNSUPPORTED;
  const int nvis = max_visible_blocks(max_seq_len, bs, window, extra);
  const int kvgroups = hkv * (hq / hkv / gt);
  // Aim for about 16 single-wave work items per compute unit if every row
  // were as long as the longest; splits are powers of two in [1, 64] blocks.
  const long long cus = device_cu_count();
  const long long items1 = (long long)(rows > 0 ? rows : 1) * kvgroups * nvis;
  const long long target = cus * 16;
  int split = 1;
  while (split < 64 && items1 / split > target) split <<= 1;
  plan->split_blocks = split;
  plan->max_splits = ceil_div(nvis, split);
  plan->heads_per_item = gt;
  plan->reserved = 0;
  plan->workspace_bytes = plan->max_splits > 1 ? partial_bytes(rows, hq, plan->max_splits, d) : 0;
  return PKV_OK;
}

static int check_plan(const pkv_decode_plan* plan, int hq, int hkv, int bs, int max_seq_len,
                      int window, int extra) {
  if (!plan) return PKV_ERR_NULL;
  if (plan->split_blocks < 1 || plan->split_blocks > 64) return PKV_ERR_SHAPE;
  const int gt = heads_per_item(hq / hkv);
  if (gt == 0) return PKV_ERR_UNSUPPORTED;
  if (plan->heads_per_item != gt) return PKV_ERR_SHAPE;
  const int nvis = max_visible_blocks(max_seq_len, bs, window, extra);
  if (plan->max_splits < ceil_div(nvis, plan->split_blocks)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

template <int D, int GT, int KV, int QT>
static void launch_split(const DecodeArgs& a, hipStream_t s) {
  const long long kvgroups = (long long)a.num_kv_heads * a.sub_groups;
  const dim3 grid((unsigned)((long long)a.num_rows * kvgroups * a.max_splits));
  decode_split_kernel<D, GT, KV, QT><<<grid, 64, 0, s>>>(a);
}

template <int D, int KV, int QT>
static int dispatch_gt(const DecodeArgs& a, int gt, hipStream_t s) {
  switch (gt) {
    case 1: launch_split<D, 1, KV, QT>(a, s); return PKV_OK;
    case 2: launch_split<D, 2, KV, QT>(a, s); return PKV_OK;
    case 4: launch_split<D, 4, KV, QT>(a, s); return PKV_OK;
    case 8: launch_split<D, 8, KV, QT>(a, s); return PKV_OK;
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D>
static int dispatch_kv(const DecodeArgs& a, int gt, int kv, hipStream_t s) {
  if (kv == PKV_F32) return dispatch_gt<D, PKV_F32, PKV_F32>(a, gt, s);
  if (kv == PKV_BF16) return dispatch_gt<D, PKV_BF16, PKV_BF16>(a, gt, s);
  return dispatch_gt<D, PKV_FP8_E4M3, PKV_BF16>(a, gt, s);
}

static int dispatch_split(const DecodeArgs& a, int gt, int kv, hipStream_t s) {
  switch (a.head_dim) {
    case 8: return dispatch_kv<8>(a, gt, kv, s);
    case 16: return dispatch_kv<16>(a, gt, kv, s);
    case 32: return dispatch_kv<32>(a, gt, kv, s);
    case 64: return dispatch_kv<64>(a, gt, kv, s);
    case 128: return dispatch_kv<128>(a, gt, kv, s);
    case 256: return dispatch_kv<256>(a, gt, kv, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D>
static void launch_combine_d(const DecodeArgs& a, int ot, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.num_rows * a.num_q_heads));
  if (ot == PKV_F32) decode_combine_kernel<D, PKV_F32><<<grid, 64, 0, s>>>(a);
  else decode_combine_kernel<D, PKV_BF16><<<grid, 64, 0, s>>>(a);
}

static int dispatch_combine(const DecodeArgs& a, int ot, hipStream_t s) {
  switch (a.head_dim) {
    case 8: launch_combine_d<8>(a, ot, s); return PKV_OK;
    case 16: launch_combine_d<16>(a, ot, s); return PKV_OK;
    case 32: launch_combine_d<32>(a, ot, s); return PKV_OK;
    case 64: launch_combine_d<64>(a, ot, s); return PKV_OK;
    case 128: launch_combine_d<128>(a, ot, s); return PKV_OK;
    case 256: launch_combine_d<256>(a, ot, s); return PKV_OK;
  }
  return PKV_ERR_UNSUPPORTED;
}

// Validates everything host-visible and fills DecodeArgs (no launch).
// qsl == nullptr: decode rows; otherwise chunked rows (rows = tokens).
static int prepare(DecodeArgs& a, void* out, const void* q, int q_dtype, int rows, int hq,
                   const pkv_cache* cache, const int32_t* bt, int bt_stride,
                   const int32_t* seq_lens, int max_seq_len, float scale, int window,
                   const int32_t* qsl, int num_reqs, int max_query_len, int causal,
                   const pkv_decode_plan* plan, void* ws, size_t ws_bytes) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (rows < 0 || hq <= 0 || bt_stride < 0 || max_seq_len < 0 || window < 0) return PKV_ERR_SHAPE;
  if (qsl && (num_reqs < 0 || max_query_len < 0)) return PKV_ERR_SHAPE;
  if (hq % cache->num_kv_heads) return PKV_ERR_SHAPE;
  const int want_q = cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  if (q_dtype != want_q) return PKV_ERR_DTYPE;
  const int extra = (qsl && !causal && max_query_len > 0) ? max_query_len - 1 : 0;
  st = check_plan(plan, hq, cache->num_kv_heads, cache->block_size, max_seq_len, window, extra);
  if (st != PKV_OK) return st;
  if (!(scale > 0.0f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  const int nrows_eff = qsl ? (num_reqs > 0 ? rows : 0) : rows;
  if (nrows_eff > 0) {
    if (!out || !q || !bt || !seq_lens) return PKV_ERR_NULL;
    if (bt_stride == 0) return PKV_ERR_SHAPE;
  }
  const size_t need = plan->max_splits > 1 ? partial_bytes(rows, hq, plan->max_splits, cache->head_dim) : 0;
  if (need > 0 && nrows_eff > 0 && (!ws || ws_bytes < need)) return PKV_ERR_WORKSPACE;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 15u)) return PKV_ERR_SHAPE;
  const long long items = (long long)rows * hq / plan->heads_per_item * plan->max_splits;
  if (items > 0x7FFFFFFFLL) return PKV_ERR_SHAPE;

  const float log2e = 1.4426950408889634f;
  a.out = out;
  a.q = q;
  a.chunked = qsl != nullptr;
  a.causal = causal != 0;
  a.single_only = 0;
  a.qsl = qsl;
  a.num_reqs = num_reqs;
  a.max_query_len = max_query_len;
  a.num_rows = nrows_eff;
  a.num_q_heads = hq;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = hq / cache->num_kv_heads;
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
  a.scale_log2 = scale * log2e * (cache->dtype == PKV_FP8_E4M3 ? cache->k_scale : 1.0f);
  a.v_scale = cache->dtype == PKV_FP8_E4M3 ? cache->v_scale : 1.0f;
  float* wsf = reinterpret_cast<float*>(ws);
  const size_t nacc = (size_t)rows * hq * plan->max_splits;
  a.ws_acc = wsf;
  a.ws_m = wsf ? wsf + nacc * cache->head_dim : nullptr;
  a.ws_l = wsf ? a.ws_m + nacc : nullptr;
  return PKV_OK;
}

static int run_split(const DecodeArgs& a, int kv_dtype, hipStream_t s) {
  if (a.num_rows == 0) return PKV_OK;
  const int gt = a.group / a.sub_groups;
  const int st = dispatch_split(a, gt, kv_dtype, s);
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
                                    int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                    int32_t sliding_window, pkv_decode_plan* plan) {
  return make_plan(num_rows, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                   sliding_window, 0, plan);
}

extern "C" int pkv_paged_attention_decode_partials(
    void* out, const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
    const pkv_cache* cache, const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale, int32_t sliding_window,
    const pkv_decode_plan* plan, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeArgs a;
  int st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride,
                   seq_lens, max_seq_len, softmax_scale, sliding_window, nullptr, 0, 0, 1, plan,
                   workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  return run_split(a, cache->dtype, stream);
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
  if (plan->split_blocks < 1 || plan->split_blocks > 64 || plan->max_splits < 1) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || plan->max_splits == 1) return PKV_OK;
  if (!out || !seq_lens) return PKV_ERR_NULL;
  const size_t need = partial_bytes(num_seqs, num_q_heads, plan->max_splits, head_dim);
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  DecodeArgs a = {};
  a.out = out;
  a.num_rows = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.bs_log2 = log2_int(block_size);
  a.seq_lens = seq_lens;
  // Bounds are the split phase's business: rows it rejected carry NaN in
  // every split slot, so the merge reproduces NaN for them.
  a.max_seq_len = 0x7FFFFFFF;
  a.bt_stride = 0x7FFFFFFF;
  a.window = sliding_window;
  a.split_blocks = plan->split_blocks;
  a.max_splits = plan->max_splits;
  a.v_scale = 1.0f;
  float* wsf = reinterpret_cast<float*>(const_cast<void*>(workspace));
  const size_t nacc = (size_t)num_seqs * num_q_heads * plan->max_splits;
  a.ws_acc = wsf;
  a.ws_m = wsf + nacc * head_dim;
  a.ws_l = a.ws_m + nacc;
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
                 max_seq_len, sliding_window, 0, &plan);
  if (st != PKV_OK) return st;
  DecodeArgs a;
  st = prepare(a, out, q, q_dtype, num_seqs, num_q_heads, cache, block_table, bt_stride, seq_lens,
               max_seq_len, softmax_scale, sliding_window, nullptr, 0, 0, 1, &plan, workspace,
               workspace_bytes);
  if (st != PKV_OK) return st;
  st = run_split(a, cache->dtype, stream);
  if (st != PKV_OK) return st;
  return run_combine(a, q_dtype, stream);
}

extern "C" int pkv_chunked_workspace_size(int32_t num_tokens, int32_t num_reqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t max_query_len, int32_t max_seq_len,
                                          int32_t sliding_window, size_t* bytes) {
  if (!bytes) return PKV_ERR_NULL;
  if (num_tokens < 0 || num_reqs < 0 || max_query_len < 0) return PKV_ERR_SHAPE;
  pkv_decode_plan plan;
  // Non-causal windowed rows see up to W + q_len - 1 keys; size for that case.
  const int extra = max_query_len > 0 ? max_query_len - 1 : 0;
  int st = make_plan(num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                     sliding_window, extra, &plan);
  if (st != PKV_OK) return st;
  *bytes = plan.workspace_bytes;
  return PKV_OK;
}

extern "C" int pkv_paged_attention_chunked(void* out, const void* q, int32_t q_dtype,
                                           int32_t num_tokens, int32_t num_q_heads,
                                           const int32_t* query_start_loc,
                                           const int32_t* seq_lens, int32_t num_reqs,
                                           int32_t max_query_len, const pkv_cache* cache,
                                           const int32_t* block_table, int32_t bt_stride,
                                           int32_t max_seq_len, float softmax_scale,
                                           int32_t causal, int32_t sliding_window,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0 || num_reqs < 0) return PKV_ERR_SHAPE;
  if (q_dtype != (cache->dtype == PKV_F32 ? PKV_F32 : PKV_BF16)) return PKV_ERR_DTYPE;
  if (num_tokens == 0 || num_reqs == 0) return PKV_OK;
  if (!query_start_loc) return PKV_ERR_NULL;
  pkv_decode_plan plan;
  const int extra = max_query_len > 0 ? max_query_len - 1 : 0;
  st = make_plan(num_tokens, num_q_heads, cache->num_kv_heads, cache->head_dim,
                 cache->block_size, max_seq_len, sliding_window, extra, &plan);
  if (st != PKV_OK) return st;
  DecodeArgs a;
  st = prepare(a, out, q, q_dtype, num_tokens, num_q_heads, cache, block_table, bt_stride,
               seq_lens, max_seq_len, softmax_scale, sliding_window, query_start_loc, num_reqs,
               max_query_len, causal, &plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  st = run_split(a, cache->dtype, stream);
  if (st != PKV_OK) return st;
  return run_combine(a, q_dtype, stream);
}
