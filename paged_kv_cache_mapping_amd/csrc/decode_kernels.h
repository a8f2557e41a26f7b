// Paged decode attention kernels: split phase (per-split online softmax) and
// combine, with their launch templates.  Included by decode.hip (host side)
// and by the decode_*.hip files that instantiate the kernels per head size.
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
#pragma once

#include <math.h>

#include <type_traits>

#include "common.h"
#include "host_common.h"

namespace pkv {

constexpr float kLazyRescale = 8.0f;  // keep a stale max until a score beats it by 2^8

struct DecodeArgs {
  void* out;
  const void* q;
  // Row mode.  0 (decode): row b is sequence b, its query is row b of q/out.
  // 1 (chunked tokens): row t is token t of the step; its request is found
  //   through query_start_loc; position seq_len - q_len + (t - qsl[r]).
  //   Tokens of single-query requests are skipped when skip_single is set.
  // 2 (chunked requests): row r is request r; only requests with exactly one
  //   query are processed (their query token is qsl[r]).
  // 3 (chunked multi-token requests): row r is request r with 1 .. qt query
  //   tokens qsl[r] ..; one work item holds all of them for its heads.
  int32_t row_mode;
  int32_t causal;
  int32_t skip_single;
  const int32_t* qsl;
  int32_t num_reqs;
  int32_t max_query_len;
  int32_t num_tokens;       // rows of q / out
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
  int32_t stream_loads;     // balanced scheme, bf16: non-temporal K/V loads (no block read twice)
  int32_t xcd_local;        // balanced scheme: an eighth of the units per XCD (blocks shared by rows)
  int32_t stream;           // balanced partition (piece counts in ws_np)
  int32_t heads_per_item;
  int32_t* ws_np;           // balanced partition: pieces per (row, head group)
  int32_t* ws_own;          // decode step: per row, 1 when its own token has a slot
  int32_t lead_workers;     // balanced partition: workers with a full share (0: all)
  int32_t trail_pct;        // share of the other workers, percent of a full share
  int32_t lds_budget;       // bytes of LDS one worker may take
  int32_t qt;               // row mode 3: query tokens one item holds (else 1)
  int32_t pair;             // INT4: items span two adjacent KV heads (see kInt4Pair)
  // Decode step with its own token (pkv_paged_attention_decode_step, row
  // mode 0, balanced partition): the split leaves position seq_len - 1 out
  // and keeps every piece as a partial, and one worker per row writes that
  // token's key and value (new_k / new_v, [rows, Hkv, D] bf16, encoded as
  // the cache write does) to its slot, the slot to slots_out and whether it
  // had one to ws_own; the merge adds the token's term from new_k / new_v
  // rounded through the cache's format.
  int32_t new_token;
  const void* new_k;
  const void* new_v;
  int64_t* slots_out;
  int32_t kv_dtype;
  int32_t kv_heads;         // the cache's KV heads (pair items halve num_kv_heads)
  float inv_k_scale;
  float inv_v_scale;
};

// What one row attends to.
struct RowInfo {
  bool skip;      // not this kernel's row (padding, or handled elsewhere)
  bool valid;     // lengths and block-table row consistent
  int req;        // block-table row
  int tok;        // row of q / out
  int lo, hi;     // inclusive visible key positions
  int first_blk;  // lo / block_size
  int nvis;       // visible logical blocks
  int ntok;       // query tokens of the row (row mode 3; else 1)
};

__device__ __forceinline__ RowInfo row_info(const DecodeArgs& a, int row) {
  RowInfo r;
  r.skip = false;
  r.valid = false;
  r.req = row;
  r.tok = row;
  r.nvis = 0;
  r.ntok = 1;
  int L, p;
  if (a.row_mode == 3) {
    // keys of the request's query tokens together: from the first token's
    // window start to the last token (non-causal: to seq_len - 1, the same)
    const int t0 = a.qsl[row];
    const int ql = a.qsl[row + 1] - t0;
    if (ql < 1 || t0 < 0 || t0 + ql > a.num_tokens) { r.skip = true; return r; }
    r.tok = t0;
    r.ntok = ql;
    L = a.seq_lens[row];
    if (L <= 0 || L > a.max_seq_len || ql > L || ql > a.max_query_len || ql > a.qt) return r;
    r.hi = L - 1;
    r.lo = a.window > 0 ? max(0, L - ql - a.window + 1) : 0;
    r.first_blk = r.lo >> a.bs_log2;
    const int last3 = r.hi >> a.bs_log2;
    if (last3 >= a.bt_stride) return r;
    r.nvis = last3 - r.first_blk + 1;
    r.valid = true;
    return r;
  }
  if (a.row_mode == 0) {
    L = a.seq_lens[row];
    p = L - 1;
    if (L <= 0 || L > a.max_seq_len) return r;
    if (a.new_token) {
      // the cached keys end before the step's own token (the merge adds it);
      // a row with none of them is valid with no blocks
      r.hi = p - 1;
      r.lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
      r.valid = true;
      if (r.lo > r.hi) return r;
      r.first_blk = r.lo >> a.bs_log2;
      const int last0 = r.hi >> a.bs_log2;
      if (last0 >= a.bt_stride) { r.valid = false; return r; }
      r.nvis = last0 - r.first_blk + 1;
      return r;
    }
  } else if (a.row_mode == 2) {
    const int t0 = a.qsl[row];
    if (a.qsl[row + 1] - t0 != 1 || t0 < 0 || t0 >= a.num_tokens) { r.skip = true; return r; }
    r.tok = t0;
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
    if (a.skip_single && ql == 1) { r.skip = true; return r; }
    L = a.seq_lens[lo];
    if (L <= 0 || L > a.max_seq_len || ql > L || ql > a.max_query_len) return r;
    p = L - ql + (row - a.qsl[lo]);
  }
  r.hi = (a.row_mode != 0 && !a.causal) ? L - 1 : p;
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

// Lane H of each 16-lane row, handed to every lane of that row (DPP
// row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + H,
                                                               0xF, 0xF, false));
}

// f(std::integral_constant<int, I>{}) for I = B .. E - 1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Maximum over the four 16-lane rows (lanes l, l^16, l^32, l^48) on the
// lane-swap instructions: swapping a value with itself across the halves,
// then across odd and even rows, hands each lane its partners' copies.
__device__ __forceinline__ float rows4_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

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
  const int64_t out_row = ((int64_t)span.tok * a.num_q_heads + h0) * D;
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
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + out_row + sub * EPL;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int i = 0; i < QW; ++i)
        qr[h][i] = reinterpret_cast<const uint32_t*>(qp + h * D)[i];
    }
  } else {
    const float* qp = reinterpret_cast<const float*>(a.q) + out_row + sub * EPL;
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
    for (int e = 0; e < EPL; ++e) dst[e] = acc[h][e] * a.v_scale;   // partials hold dequantised V sums
    if (sub == 0) {
      a.ws_m[pr] = m[h];
      a.ws_l[pr] = l[h];
    }
  }
}

// --------------------------------------------------------------------------
// Split phase, uniform-block form: used when every wave load of RPW rows (and
// every step of 16 rows) lies inside one block, i.e. block_size >= 16 and a
// row takes >= 64 bytes.  The physical id of a step is wave-uniform, so it
// lives in a scalar register and every K/V load is one 16-byte vector load at
// a scalar base plus a per-lane constant offset.  Only a split's first and
// last steps can hold positions outside the visible range; they take a masked
// path.  The lazy-rescale test runs once per head per step on the lane's
// largest score of the step.
template <int D, int GT, int KV, int QT>
__global__ __launch_bounds__(64) void decode_split_uni_kernel(DecodeArgs a) {
  constexpr int kElt = KV == PKV_F32 ? 4 : (KV == PKV_BF16 ? 2 : 1);
  constexpr int kRowBytes = D * kElt;
  static_assert(kRowBytes >= 64, "uniform form needs rows of at least 64 bytes");
  constexpr int LPR = kRowBytes / 16;                      // lanes per row
  constexpr int EPL = 16 / kElt;                           // elements per lane
  constexpr int RPW = kWave / LPR;                         // rows per wave load
  constexpr int U = 16 / RPW;                              // loads per 16-row step
  constexpr int kStepRows = U * RPW;                       // == 16
  constexpr bool kBf16Dot = (QT == PKV_BF16);
  constexpr int QW = kBf16Dot ? EPL / 2 : EPL;

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
  const int64_t out_row = ((int64_t)span.tok * a.num_q_heads + h0) * D;
  if (!span.valid) {
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

  int tab = -1;
  if (lane < nb) tab = a.bt[(int64_t)span.req * a.bt_stride + blk_begin + lane];
  const bool bad = (lane < nb) && (tab < 0 || tab >= a.num_blocks);
  const bool any_bad = __ballot(bad) != 0;

  uint32_t qr[GT][QW];
  float qf[GT][kBf16Dot ? 1 : EPL];
  if constexpr (kBf16Dot) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(a.q) + out_row + sub * EPL);
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int i = 0; i < QW / 4; ++i) {
        const uint4 t = qp[h * (D * 2 / 16) + i];
        qr[h][4 * i] = t.x; qr[h][4 * i + 1] = t.y; qr[h][4 * i + 2] = t.z; qr[h][4 * i + 3] = t.w;
      }
    }
  } else {
    const float* qp = reinterpret_cast<const float*>(a.q) + out_row + sub * EPL;
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] = qp[h * D + e];
  }
  (void)qr;
  (void)qf;
  // The query and block-table loads must be complete before the pipelined
  // loop; otherwise the wait-count tracking cannot tell them apart from the
  // prefetched K/V loads and waits for everything at the top of each step.
  __builtin_amdgcn_s_waitcnt(0);

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  if (!any_bad) {
    const int steps_per_block = bs / kStepRows;
    const int nsteps = nb * steps_per_block;
    const int64_t blk_bytes = a.block_stride * kElt;
    const int row_bytes = a.num_kv_heads * kRowBytes;      // one token of all KV heads
    // per-lane byte offset inside a 16-row step (fits 32 bits: a block is
    // at most 32 rows x 64 heads x 512 bytes)
    const uint32_t lane_off = (uint32_t)((grp * a.num_kv_heads + kvh) * kRowBytes + sub * 16);
    const int pos_base = blk_begin << a.bs_log2;

    auto issue = [&](int st, uint4 (&kd)[U], uint4 (&vd)[U]) {
      const int blk = st / steps_per_block;
      const int r0 = (st - blk * steps_per_block) * kStepRows;
      const int phys = __builtin_amdgcn_readlane(tab, blk);
      const int64_t off = (int64_t)phys * blk_bytes + (int64_t)r0 * row_bytes;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // wave-uniform base (scalar registers) + 32-bit lane offset
        const char* kp = a.kbase + off + (int64_t)u * RPW * row_bytes;
        const char* vp = a.vbase + off + (int64_t)u * RPW * row_bytes;
        kd[u] = *reinterpret_cast<const uint4*>(kp + lane_off);
        vd[u] = *reinterpret_cast<const uint4*>(vp + lane_off);
      }
    };

    auto compute = [&](auto full_tag, int st, const uint4 (&kd)[U], const uint4 (&vd)[U]) {
      constexpr bool full = decltype(full_tag)::value;
      const int p0 = pos_base + st * kStepRows;                 // first row of the step
      float z[U][GT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t kwa[4] = {kd[u].x, kd[u].y, kd[u].z, kd[u].w};
        uint32_t kp[kBf16Dot ? EPL / 2 : 1];
        float kf[kBf16Dot ? 1 : EPL];
        (void)kp;
        (void)kf;
        if constexpr (KV == PKV_BF16) {
#pragma unroll
          for (int i = 0; i < EPL / 2; ++i) {
            if constexpr (kBf16Dot) kp[i] = kwa[i];
            else { kf[2 * i] = bf16_lo(kwa[i]); kf[2 * i + 1] = bf16_hi(kwa[i]); }
          }
        } else if constexpr (KV == PKV_F32) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) kf[i] = as_float(kwa[i]);
        } else {
#pragma unroll
          for (int i = 0; i < EPL / 4; ++i) {
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
          z[u][h] = sc;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < GT; ++h) z[u][h] = group_sum<LPR>(z[u][h]) * a.scale_log2;

      bool live[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pos = p0 + u * RPW + grp;
        live[u] = full || (pos >= span.lo && pos <= span.hi);
        if (!live[u]) {
#pragma unroll
          for (int h = 0; h < GT; ++h) z[u][h] = -INFINITY;
        }
      }

      // V rows in compute form; masked rows are zeroed so that stale or
      // poisoned bytes never reach the accumulators.
      float vf[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t vwa[4] = {vd[u].x, vd[u].y, vd[u].z, vd[u].w};
        if constexpr (KV == PKV_BF16) {
#pragma unroll
          for (int i = 0; i < EPL / 2; ++i) { vf[u][2 * i] = bf16_lo(vwa[i]); vf[u][2 * i + 1] = bf16_hi(vwa[i]); }
        } else if constexpr (KV == PKV_F32) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) vf[u][i] = as_float(vwa[i]);
        } else {
#pragma unroll
          for (int i = 0; i < EPL / 4; ++i) {
            const f32x2 v01 = e4m3x2_to_f32<false>(vwa[i]);
            const f32x2 v23 = e4m3x2_to_f32<true>(vwa[i]);
            vf[u][4 * i] = v01.x; vf[u][4 * i + 1] = v01.y; vf[u][4 * i + 2] = v23.x; vf[u][4 * i + 3] = v23.y;
          }
        }
        if (!full) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[u][e] = live[u] ? vf[u][e] : 0.f;
        }
      }

#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float zmax = z[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) zmax = fmaxf(zmax, z[u][h]);
        if (zmax > m[h] + kLazyRescale) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - zmax);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
          m[h] = zmax;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // a lane whose rows are all masked keeps m = -inf; its p must be 0
          const float p = (full || live[u]) ? __builtin_amdgcn_exp2f(z[u][h] - m[h]) : 0.f;
          l[h] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[u][e], acc[h][e]);
        }
      }
    };

    // Steps whose 16 rows are all visible skip every mask.
    auto step_is_full = [&](int st) {
      const int p0 = pos_base + st * kStepRows;
      return p0 >= span.lo && p0 + kStepRows - 1 <= span.hi;
    };
    auto run = [&](int st, const uint4 (&kd)[U], const uint4 (&vd)[U]) {
      if (step_is_full(st)) compute(std::true_type{}, st, kd, vd);
      else compute(std::false_type{}, st, kd, vd);
    };

    // Loads are issued unconditionally, one step ahead; past the end the last
    // step is fetched again (an L2 hit).  A branch around a prefetch would
    // make the wait-count tracking merge two paths and wait for everything.
    uint4 ka[U], va[U], kb2[U], vb2[U];
    const int last = nsteps - 1;
    issue(0, ka, va);
    for (int st = 0; st < nsteps; st += 2) {
      issue(min(st + 1, last), kb2, vb2);
      run(st, ka, va);
      issue(min(st + 2, last), ka, va);
      if (st + 1 < nsteps) run(st + 1, kb2, vb2);
    }

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
    for (int e = 0; e < EPL; ++e) dst[e] = acc[h][e] * a.v_scale;   // partials hold dequantised V sums
    if (sub == 0) {
      a.ws_m[pr] = m[h];
      a.ws_l[pr] = l[h];
    }
  }
}

// --------------------------------------------------------------------------
// Balanced split phase on the matrix cores, one load pipeline per worker.
//
// Work units are (KV-head group, row, visible block), ordered group-major:
// unit u is block u - g T - cum[r] of row r in group g, with T the visible
// blocks of all rows.  The grid is a fixed number of single-wave workers,
// one or two per SIMD; logical worker w takes a contiguous run of units,
// equal shares of P = max(ceil(U / workers), min_units) or, with two waves
// per SIMD, full shares for the first half of the workers and 90 % shares
// for the rest (a second wave on a SIMD loses instruction issue to the older
// one and lags it by a fifth); workgroup b is logical worker b,
// except under PKV_PLAN_BLOCKS_SHARED with equal shares and a worker count
// divisible by 8, where it is logical worker (b % 8) (W / 8) + b / 8:
// workgroups go to the eight XCDs round-robin, so each XCD then gets one
// contiguous eighth of the units, about one head group's, and blocks that
// several rows share (a common prompt) are reread from that XCD's L2 rather
// than from the memory-side cache (on unshared blocks that placement
// measured slower).  Each stretch
// of a worker's range that belongs to one (row, head group) is a "piece": it
// is folded with an online softmax and written either as the final output
// (when the piece covers the whole row) or as a partial (m, l, acc) in slot
// `piece` of that row, with the piece count stored for the combine kernel.
//
// A worker streams its range as one load pipeline that runs across piece
// boundaries.  Before any K/V load, lane i resolves unit wbase + i of a
// 64-unit window (its row through the prefix sums, the row's visible span,
// the block-table entry, the KV head) into registers, and the query rows of
// every piece that starts in the window are staged in LDS; the loop then
// reads the physical block of each step with one lane read, and crossing
// into the next piece costs an LDS read instead of a wait on memory.
//
// Scores of a 16-token step are one chain of 16x16x32 bf16 MFMAs, computed
// transposed (S^T = K Q^T, the same registers with the operands swapped):
// K rows load straight into one operand (lane l: token l % 16, 8 elements of
// a 32-element chunk) and the item's query rows, staged in LDS, are the other
// (unused rows zero).  Lane l then holds the scores of row l % 16 for tokens
// 4 (l / 16) .. + 3, so each row's running max and sum live in one lane.
// P.V runs on the matrix cores where mfma_pv says so (decode_flat_body
// describes the layout), else on the vector ALUs in fp32 with each weight
// arriving by a DPP row broadcast.  Requirements: bf16, fp8 or INT4 cache,
// bf16 query, head_dim % 32 == 0, row of at least 64 bytes, block size a
// multiple of 16, at most 16 MFMA rows per item.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));   // 4 bf16, 16x16x16 MFMA operand

// P.V on the matrix cores at head size 128: bf16, fp8 and INT4 caches (fp8
// and INT4 widened to bf16 in registers, exact), except bf16 / fp8
// single-query items of 8 rows (see decode_flat_body).
// K/V loads of the balanced kernel.  With NTL (bf16 caches whose blocks the
// caller declares unshared, PKV_PLAN_BLOCKS_NOT_SHARED) they carry a
// non-temporal hint: a stream read once then does not displace what is reused
// from the caches (table entries, staged queries, the partials the merge
// reads next); on the Llama-3-8B batch the split kernel went from 64.2 to
// 59.4 us.  Where blocks are shared by many rows (prefix sharing) the hint
// sends every row back to HBM (75 -> 146 us there), and 8-byte fp8 loads
// were slower with it too, so only the caller can ask for it.
template <typename T>
__device__ __forceinline__ T load_stream(const char* p) {
  if constexpr (sizeof(T) == 16) {
    typedef unsigned v4_t __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v4_t*>(p)));
  } else if constexpr (sizeof(T) == 8) {
    typedef unsigned v2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v2_t*>(p)));
  } else {
    static_assert(sizeof(T) == 4, "4, 8 or 16 bytes per lane");
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p)));
  }
}

template <typename T, bool NTL>
__device__ __forceinline__ T kv_load(const char* p) {
  if constexpr (NTL) return load_stream<T>(p);
  else return *reinterpret_cast<const T*>(p);
}

__host__ __device__ constexpr bool mfma_pv(int d, int kv, int gt, int qt) {
  return d == 128 && (kv_bits(kv) == 4 || ((kv == PKV_BF16 || kv == PKV_FP8_E4M3) && !(gt == 8 && qt == 1)));
}

// INT4 work items over two adjacent KV heads.  A 64-byte INT4 head row is
// half a 128-byte line, and the two halves belong to different items that
// different waves read at different times: the line was fetched twice (136.8
// MB per launch against 67.1 MB of K/V).  A pair item reads whole lines: its
// first GT / 2 rows are the query heads of the first KV head, the rest those
// of the second; the kernel sees the cache as Hkv / 2 heads of 128-byte rows.
constexpr int kInt4Pair = 0x100 | PKV_INT4;

template <int D, int GT, int KV>
struct MfmaShape {
  static constexpr bool kPair = KV == kInt4Pair;
  static constexpr int kBits = kv_bits(KV);          // 16 bf16, 8 fp8, 4 int4
  static constexpr int kHeadBytes = D * kBits / 8;   // one token of one KV head
  static constexpr int kRowBytes = kHeadBytes * (kPair ? 2 : 1);   // one token of an item
  static constexpr int NC = D / 32;                  // MFMA k-chunks
  // V: bytes per lane and load; INT4 takes 4 (8 elements, a 16-lane row per
  // token), so that a lane accumulates as many elements per row as with bf16
  // (fp8 at head size 128: 8, the bf16 lane layout for the matrix-core P.V)
  static constexpr int kVBytes = kBits == 4 ? 4 : (kBits == 8 && D == 128 ? 8 : 16);
  static constexpr int VLPR = kHeadBytes / kVBytes;  // V: lanes per row
  static constexpr int VRPW = kWave / VLPR;          // V: rows per load
  static constexpr int VU = 16 / VRPW;               // V: loads per 16-token step
  static constexpr int VEPL = kVBytes * 8 / kBits;   // V: elements per lane
  static constexpr int KB = kBits;                   // K: bytes per lane per chunk (8 elements)
  static constexpr int RG = (GT + 3) / 4;            // MFMA row groups in use
  static constexpr int QE = GT * D;                  // query elements of one piece
  static constexpr int QL = (QE + 8 * kWave - 1) / (8 * kWave);  // 16-byte loads per lane
  static_assert(VRPW <= 16 && VU * VRPW == 16, "V layout");
  static_assert(GT <= 16, "at most 16 query heads per item");
  static_assert(kBits != 4 || D % 128 == 0, "INT4 rows span whole 64-byte K loads");
  static_assert(!kPair || GT % 2 == 0, "pair items hold both heads' rows");
};

// INT4 K words for the matrix cores.  A word holds elements n = 0..7 of a
// lane's k-chunk as nibbles u (element n in bits 4n .. 4n + 3).  Each nibble
// becomes the bfloat16 value 128 + u (high byte 0x43, low byte u: exponent
// of 128, mantissa u, exact), so the products need a per-row correction of
// -136 * sum(q) to give (u - 8) . q.  The four dwords hold elements in the
// order 0, 2, 4, 6, 1, 3, 5, 7; the query operand is permuted to match
// (int4_q_perm).
// v_perm_b32 selects bytes of {S0 (high), S1 (low)}: selector 0..3 picks a
// byte of S1, 4..7 a byte of S0, 0x0C gives zero.
__device__ __forceinline__ uint4 int4_k_bf16(uint32_t w) {
  const uint32_t x = w & 0x0F0F0F0Fu;          // bytes u0, u2, u4, u6
  const uint32_t y = (w >> 4) & 0x0F0F0F0Fu;   // bytes u1, u3, u5, u7
  constexpr uint32_t kHi = 0x43434343u;                        // the high byte of each bf16
  return make_uint4(__builtin_amdgcn_perm(x, kHi, 0x00050004u), __builtin_amdgcn_perm(x, kHi, 0x00070006u),
                    __builtin_amdgcn_perm(y, kHi, 0x00050004u), __builtin_amdgcn_perm(y, kHi, 0x00070006u));
}

// Eight query elements (pairs q0q1, q2q3, q4q5, q6q7) into the order of
// int4_k_bf16: q0q2, q4q6, q1q3, q5q7.
__device__ __forceinline__ uint4 int4_q_perm(uint4 t) {
  return make_uint4((t.x & 0xFFFFu) | (t.y << 16), (t.z & 0xFFFFu) | (t.w << 16),
                    (t.x >> 16) | (t.y & 0xFFFF0000u), (t.z >> 16) | (t.w & 0xFFFF0000u));
}

// LDS layout of the balanced kernel (dynamic shared memory, 16-byte aligned
// sections) within a budget of bytes per worker: prefix sums cum[rows + 1];
// per-row records {req, tok, lo, hi} when rows <= kRowRecRows and they fit;
// query rows of as many pieces as the rest holds (2 to 64).
constexpr int kRowRecRows = 1024;

struct FlatLds {
  int cum_off, rec_off, q_off, qslots;
  bool recs;
  size_t bytes;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline FlatLds flat_lds_layout(int rows, int gt, int d, int budget) {
  FlatLds l;
  l.cum_off = 0;
  size_t off = align16(((size_t)rows + 1) * sizeof(int));
  const size_t per = (size_t)gt * d * 2;
  const size_t rec = align16((size_t)rows * 4 * sizeof(int));
  l.rec_off = (int)off;
  l.recs = rows <= kRowRecRows && off + rec + 2 * per <= (size_t)budget;
  if (l.recs) off += rec;
  l.q_off = (int)off;
  long long slots = off + 2 * per <= (size_t)budget ? (long long)(((size_t)budget - off) / per) : 2;
  if (slots > kWave) slots = kWave;
  if (slots < 2) slots = 2;
  l.qslots = (int)slots;
  l.bytes = off + (size_t)slots * per;
  return l;
}

// Contiguous shares of the unit range [0, U): workers w < lead take p_lead
// units each, the others p_trail (both at least min_units).  With lead equal
// to the worker count every share is equal.  range_of(u) numbers the shares;
// below 2^31 units (narrow) it divides in 32 bits, a few instructions
// instead of the long software sequence of a 64-bit division.
struct Shares {
  long long p_lead, p_trail, lead_end;
  int lead;
  bool narrow;
  __device__ __forceinline__ long long begin(long long w) const {
    return w <= lead ? w * p_lead : lead_end + (w - lead) * p_trail;
  }
  __device__ __forceinline__ long long range_of(long long u) const {
    if (narrow) {
      const uint32_t v = (uint32_t)u, le = (uint32_t)lead_end;
      return v < le ? v / (uint32_t)p_lead : lead + (v - le) / (uint32_t)p_trail;
    }
    return u < lead_end ? u / p_lead : lead + (u - lead_end) / p_trail;
  }
};

__device__ __forceinline__ Shares make_shares(long long U, int W, int lead, int pct, int min_units) {
  Shares s;
  if (lead <= 0 || lead >= W || pct >= 100 || pct <= 0) {
    s.lead = W;
    s.p_lead = (U + W - 1) / W;
  } else {
    s.lead = lead;
    const long long den = (long long)lead * 100 + (long long)(W - lead) * pct;
    s.p_lead = (U * 100 + den - 1) / den;
  }
  if (s.p_lead < min_units) s.p_lead = min_units;
  s.lead_end = (long long)s.lead * s.p_lead;
  const long long rest = U - s.lead_end;
  s.p_trail = (s.lead < W && rest > 0) ? (rest + (W - s.lead) - 1) / (W - s.lead) : 1;
  if (s.p_trail < min_units) s.p_trail = min_units;
  s.narrow = U < (1LL << 31);
  return s;
}

// The decode step's own token of row r (position seq_len - 1), written by
// one wave: its key and value rows from new_k / new_v, encoded exactly as
// the cache write does (bf16 as is; fp8 e4m3 and INT4 with the inverse
// scales), to the slot its block-table entry gives; the slot to slots_out
// (-1 for a block the table does not map, whose row the merge makes NaN)
// and the verdict to ws_own.  Rows whose lengths the split rejects are left
// to the rows-without-units pass.
template <int D>
__device__ __forceinline__ void write_own_token(const DecodeArgs& a, int r, int lane) {
  const int L = a.seq_lens[r];
  if (L <= 0 || L > a.max_seq_len) return;
  const int pos = L - 1;
  const int blk = pos >> a.bs_log2;
  const int phys = blk < a.bt_stride ? a.bt[(int64_t)r * a.bt_stride + blk] : -1;
  const bool ok = phys >= 0 && phys < a.num_blocks;
  const int in_blk = pos & ((1 << a.bs_log2) - 1);
  if (lane == 0) {
    a.ws_own[r] = ok ? 1 : 0;
    if (a.slots_out) a.slots_out[r] = ok ? ((int64_t)phys << a.bs_log2) + in_blk : -1;
  }
  if (!ok) return;
  const int bits = kv_bits(a.kv_dtype);
  const int n = a.kv_heads * D;                   // elements of one token row
  const int64_t row = (int64_t)phys * (a.block_stride * bits / 8) + (int64_t)in_blk * n * bits / 8;
  const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.new_k) + (int64_t)r * n;
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.new_v) + (int64_t)r * n;
  uint8_t* kd = reinterpret_cast<uint8_t*>(const_cast<char*>(a.kbase) + row);
  uint8_t* vd = reinterpret_cast<uint8_t*>(const_cast<char*>(a.vbase) + row);
  // eight elements per lane and pass (16 bytes of new_k / new_v)
  for (int e = lane * 8; e < n; e += kWave * 8) {
    const uint4 kw = *reinterpret_cast<const uint4*>(kn + e);
    const uint4 vw = *reinterpret_cast<const uint4*>(vn + e);
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vk[4] = {vw.x, vw.y, vw.z, vw.w};
    if (bits == 16) {
      *reinterpret_cast<uint4*>(kd + (int64_t)e * 2) = kw;
      *reinterpret_cast<uint4*>(vd + (int64_t)e * 2) = vw;
    } else if (bits == 8) {
      // the hardware conversion unless a NaN is among the eight (the
      // integer encoder keeps it), as the cache write does
      float kx[8], vx[8];
      bool nan = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kx[i] = as_float(((kk[i / 2] >> (16 * (i % 2))) & 0xFFFFu) << 16) * a.inv_k_scale;
        vx[i] = as_float(((vk[i / 2] >> (16 * (i % 2))) & 0xFFFFu) << 16) * a.inv_v_scale;
        nan |= kx[i] != kx[i] || vx[i] != vx[i];
      }
      uint32_t kc[2], vc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!nan) {
          kc[j] = e4m3x4_encode_no_nan(kx[4 * j], kx[4 * j + 1], kx[4 * j + 2], kx[4 * j + 3]);
          vc[j] = e4m3x4_encode_no_nan(vx[4 * j], vx[4 * j + 1], vx[4 * j + 2], vx[4 * j + 3]);
        } else {
          kc[j] = vc[j] = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kc[j] |= e4m3_encode(kx[4 * j + i]) << (8 * i);
            vc[j] |= e4m3_encode(vx[4 * j + i]) << (8 * i);
          }
        }
      }
      *reinterpret_cast<uint2*>(kd + e) = make_uint2(kc[0], kc[1]);
      *reinterpret_cast<uint2*>(vd + e) = make_uint2(vc[0], vc[1]);
    } else {   // two codes per byte, element 2j in the low nibble of byte j
      uint32_t kc = 0u, vc = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t kb = (kk[i / 2] >> (16 * (i % 2))) & 0xFFFFu, vb = (vk[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        kc |= int4_encode(as_float(kb << 16) * a.inv_k_scale) << (4 * i);
        vc |= int4_encode(as_float(vb << 16) * a.inv_v_scale) << (4 * i);
      }
      *reinterpret_cast<uint32_t*>(kd + e / 2) = kc;
      *reinterpret_cast<uint32_t*>(vd + e / 2) = vc;
    }
  }
}

template <int D, int GT, int KV, int DEPTH, int QT = 1, bool NTL = false>
__device__ __forceinline__ void decode_flat_body(const DecodeArgs& a) {
  using S = MfmaShape<D, GT, KV>;
  constexpr int NC = S::NC, VLPR = S::VLPR, VRPW = S::VRPW, VU = S::VU, VEPL = S::VEPL;
  constexpr int KB = S::KB, RG = S::RG;
  constexpr bool kI4 = S::kBits == 4;
  constexpr bool kPair = S::kPair;
  constexpr int NH = kPair ? 2 : 1;                  // KV heads of an item
  static_assert(!kPair || QT == 1, "pair items are single-query");
  // MFMA rows of an item: (query token t, head h) as row t * GT + h
  constexpr int RI = GT * QT;
  constexpr int QE = RI * D;                                   // query elements of one piece
  constexpr int QL = (QE + 8 * kWave - 1) / (8 * kWave);       // 16-byte loads per lane
  static_assert(RI <= 16, "at most 16 MFMA rows per item");
  static_assert(DEPTH >= 1 && DEPTH <= 4, "prefetch depth");
  // Row-broadcast scheme, when one V token row fits in a 16-lane row: the
  // scores come out transposed (S^T = K Q^T, same registers with the MFMA
  // operands swapped), so lane l holds tokens 4 (l / 16) .. + 3 of head
  // l % 16; V loads put tokens 4 R .. 4 R + 3 in row R; each probability a
  // lane needs then sits in its own row and arrives by DPP broadcast.
  // Otherwise (a token spans two rows) probabilities move by LDS permute.
  constexpr bool RB = VLPR <= 16;
  constexpr int TPRV = RB ? 16 / VLPR : 1;          // V tokens per 16-lane row and load
  static_assert(QT == 1 || RB, "multi-token items need the row-broadcast scheme");
  // P.V on the matrix cores (bf16, head size 128): the score MFMA leaves this
  // lane's weights where the A operand of v_mfma_f32_16x16x16_bf16 wants them
  // (row l % 16, tokens 4 (l / 16) + i), and with output column n of tile t
  // standing for dimension 8 n + t the lane's own V loads (tokens 4 R + u,
  // dimensions 8 (l % 16) .. + 7) are the B operand: no data moves.  The
  // lane then holds rows 4 R + i at dimensions 8 (l % 16) .. + 7.  P enters
  // as a bf16 high part plus a bf16 remainder.  bf16 and fp8 single-query
  // items of 8 rows keep the vector ALUs (measured faster there: 102-106
  // against 108-117 us on 32 x 4096 tokens with 64 query heads).
  constexpr bool kMPV = mfma_pv(D, KV, GT, QT) && RB && VLPR == 16 && VU == 4 && VEPL == 8;
  static_assert(!kI4 || kMPV, "INT4 runs on the matrix-core P.V");
  extern __shared__ __align__(16) char lds[];
  const FlatLds L = flat_lds_layout(a.num_rows, RI, D, a.lds_budget);
  int* cum = reinterpret_cast<int*>(lds + L.cum_off);     // cum[r]: visible blocks of rows < r
  int4* rrec = reinterpret_cast<int4*>(lds + L.rec_off);  // {req, tok, lo, hi}
  uint16_t* qst = reinterpret_cast<uint16_t*>(lds + L.q_off);
  const bool have_rec = L.recs;
  const int lane = threadIdx.x;
  const int kvgroups = a.num_kv_heads * a.sub_groups;

  // ---- visible blocks per row, prefix sums (and row records) in LDS
  int carry = 0;
  for (int r0 = 0; r0 < a.num_rows; r0 += kWave) {
    const int r = r0 + lane;
    int nv = 0;
    if (r < a.num_rows) {
      const RowInfo ri = row_info(a, r);
      nv = (!ri.skip && ri.valid) ? ri.nvis : 0;
      if (have_rec) rrec[r] = make_int4(ri.req, ri.tok, ri.lo, ri.hi);
    }
    int incl = nv;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (r < a.num_rows) cum[r] = carry + incl - nv;
    carry += __shfl(incl, kWave - 1);
  }
  if (lane == 0) cum[a.num_rows] = carry;
  __syncthreads();

  const long long U = (long long)carry * kvgroups;
  const int W = gridDim.x;
  const Shares sh = make_shares(U, W, a.lead_workers, a.trail_pct, a.split_blocks);
  // logical worker: an eighth of the units per XCD for shared blocks when
  // shares are equal (lead and trail shares keep the dispatch order they
  // are sized for)
  const int lw = (a.xcd_local && sh.lead >= W && W % 8 == 0)
                     ? (int)(blockIdx.x % 8) * (W / 8) + (int)(blockIdx.x / 8)
                     : (int)blockIdx.x;
  const long long u_lo = min(U, sh.begin(lw));
  const long long u_hi = min(U, sh.begin((long long)lw + 1));

  const int spb_log2 = a.bs_log2 - 4;                     // 16-token steps per block
  const int64_t blk_bytes = a.block_stride * S::kBits / 8;
  const int row_bytes = a.num_kv_heads * S::kRowBytes;      // one token, all KV heads
  const int vg = lane / VLPR, vsub = lane % VLPR;
  // K: lane l reads token l % 16; bf16 / fp8 take chunk c's elements
  // 32 c + 8 (l / 16) .. + 7, INT4 one 16-byte load of elements
  // 128 j + 32 (l / 16) .. + 31 per 64-byte half j (chunk 4 j + c' is the
  // load's word c')
  const uint32_t k_lane = (uint32_t)((lane % 16) * row_bytes + (lane / 16) * (kI4 ? 16 : KB));
  const uint32_t v_lane = RB ? (uint32_t)((4 * (lane / 16) + (lane % 16) / VLPR) * row_bytes + vsub * S::kVBytes)
                             : (uint32_t)(vg * row_bytes + vsub * S::kVBytes);

  // one lane's unit record
  int rec_phys = -1, rec_hoff = 0, rec_gid = -1, rec_pos0 = 0, rec_lo = 0, rec_hi = -1, rec_tok = 0;

  // running piece
  int cur = -1, s_lo = 0, s_hi = -1, s_tok = 0, s_ord = 0;
  int s_ql = 1, s_flo = 0, s_fhi = -1;   // query tokens; keys every row of the piece sees
  long long s_first = 0;
  bool s_bad = false;
  bf16x8_t qa[NC];
  float acc[kMPV ? 1 : RI][VEPL];     // vector-ALU P.V: row h, this lane's elements
  f32x4_t accm[kMPV ? VEPL : 1];      // matrix-core P.V: tile t, rows 4 R + i
  float m[GT];
  f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
  float m1 = -INFINITY, ls1 = 0.f;   // row-broadcast scheme: head lane % 16's max and sum
  float kqz = 0.f;                    // INT4: 136 * sum(q) of row lane % 16, times scale_log2

  // first query element of the piece (gid = row * kvgroups + head group)
  auto q_elem = [&](int gid, int tok) __attribute__((always_inline)) -> int64_t {
    const int kvg = gid % kvgroups;
    const int h0 = (kvg / a.sub_groups) * a.group + (kvg % a.sub_groups) * GT;
    return ((int64_t)tok * a.num_q_heads + h0) * D;
  };
  // query element offset of chunk c for this lane, matching the K layout
  auto q_chunk = [&](int c) __attribute__((always_inline)) -> int {
    return kI4 ? 128 * (c / 4) + 32 * (lane / 16) + 8 * (c % 4) : 32 * c + 8 * (lane / 16);
  };
  // INT4: reorder each chunk to the K operand's element order and form the
  // row's correction (the four lanes of a row hold a quarter of it each)
  auto q_int4 = [&]() __attribute__((always_inline)) {
    if constexpr (kI4) {
      float sq = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 t = __builtin_bit_cast(uint4, qa[c]);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) sq += bf16_lo(w[i]) + bf16_hi(w[i]);
        qa[c] = __builtin_bit_cast(bf16x8_t, int4_q_perm(t));
      }
      sq += shfl_xor_t(sq, 16);
      sq += shfl_xor_t(sq, 32);
      kqz = 136.0f * sq * a.scale_log2;
    }
  };
  // A operand of the piece's query rows: lane l takes row l % 16, elements
  // q_chunk(c) .. + 8 (rows past GT are zero)
  auto q_from_lds = [&](int slot) __attribute__((always_inline)) {
    const int row = lane % 16;
    const uint16_t* src = qst + (size_t)slot * QE + row * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (row < RI) t = *reinterpret_cast<const uint4*>(src + q_chunk(c));
      qa[c] = __builtin_bit_cast(bf16x8_t, t);
    }
    q_int4();
  };
  auto q_from_global = [&](int64_t qe) __attribute__((always_inline)) {
    const int row = lane % 16;
    const int64_t roff = (int64_t)(row / GT) * a.num_q_heads * D + (row % GT) * D;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.q) + qe + roff;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (row < RI && row / GT < s_ql) t = *reinterpret_cast<const uint4*>(src + q_chunk(c));
      qa[c] = __builtin_bit_cast(bf16x8_t, t);
    }
    // settle here, so that no wait for these loads lands inside the loop
    __builtin_amdgcn_s_waitcnt(0);
    q_int4();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 t = __builtin_bit_cast(uint4, qa[c]);
      asm volatile("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
      qa[c] = __builtin_bit_cast(bf16x8_t, t);
    }
  };
  auto start = [&](int unit, int gid) __attribute__((always_inline)) {
    cur = gid;
    s_lo = __builtin_amdgcn_readlane(rec_lo, unit);
    s_hi = __builtin_amdgcn_readlane(rec_hi, unit);
    s_tok = __builtin_amdgcn_readlane(rec_tok, unit);
    s_bad = false;
    s_flo = s_lo;
    s_fhi = s_hi;
    if constexpr (QT > 1) {
      // token t sits at s_hi - (ql - 1 - t); the first token sees the fewest
      // keys (causal), the last the latest window start
      const int b = gid / kvgroups;
      s_ql = a.qsl[b + 1] - a.qsl[b];
      if (a.causal) s_fhi = s_hi - (s_ql - 1);
      if (a.window > 0) s_flo = max(s_lo, s_hi - a.window + 1);
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) m[h] = -INFINITY;
    if constexpr (kMPV) {
#pragma unroll
      for (int t = 0; t < VEPL; ++t) accm[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int h = 0; h < RI; ++h)
#pragma unroll
        for (int e = 0; e < VEPL; ++e) acc[h][e] = 0.f;
    }
    lsum[0] = lsum[1] = lsum[2] = lsum[3] = 0.f;
    m1 = -INFINITY;
    ls1 = 0.f;
  };
  auto flush = [&]() __attribute__((always_inline)) {
    const int b = cur / kvgroups;
    const int kvg = cur % kvgroups;
    const int h0 = (kvg / a.sub_groups) * a.group + (kvg % a.sub_groups) * GT;
    const int nv = cum[b + 1] - cum[b];
    const long long seg_base = (long long)kvg * carry + cum[b];
    const long long r0 = sh.range_of(seg_base);
    const int piece = (int)(sh.range_of(s_first) - r0);
    const int npieces = (int)(sh.range_of(seg_base + nv - 1) - r0 + 1);
    // a piece that is its whole row writes the output, unless the merge still
    // adds the step's own token
    const bool whole = npieces == 1 && !a.new_token;
    if (s_bad) {
#pragma unroll
      for (int h = 0; h < GT; ++h) m[h] = 0.f;
      if constexpr (kMPV) {
        const float qn = __builtin_nanf("");
#pragma unroll
        for (int t = 0; t < VEPL; ++t) accm[t] = f32x4_t{qn, qn, qn, qn};
      } else {
#pragma unroll
        for (int h = 0; h < RI; ++h)
#pragma unroll
          for (int e = 0; e < VEPL; ++e) acc[h][e] = __builtin_nanf("");
      }
      lsum[0] = lsum[1] = lsum[2] = lsum[3] = __builtin_nanf("");
      m1 = 0.f;
      ls1 = __builtin_nanf("");
    }
    // the V layout's token groups hold partial sums under the same maxima
    // (the matrix-core form sums all tokens inside the products)
    if constexpr (!kMPV) {
#pragma unroll
      for (int step = VLPR; step < kWave; step <<= 1)
#pragma unroll
        for (int h = 0; h < RI; ++h)
#pragma unroll
          for (int e = 0; e < VEPL; ++e) acc[h][e] += shfl_xor_t(acc[h][e], step);
    }
    float lh[RI], mh[RI];   // each row's sum and max
    if constexpr (RB) {
      float lt = ls1;
      lt += shfl_xor_t(lt, 16);
      lt += shfl_xor_t(lt, 32);
#pragma unroll
      for (int h = 0; h < RI; ++h) {
        lh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lt), h));
        mh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m1), h));
      }
    } else {
      float lt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) lt[i] = group_sum<16>(lsum[i]);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        lh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lt[h % 4]), 16 * (h / 4)));
        mh[h] = m[h];
      }
    }
    if constexpr (kMPV) {
      // lane (R, c): rows 4 R + i, dimensions 8 c .. 8 c + 7
      const int R = lane / 16, c = lane % 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * R + i;
        if (r >= RI) continue;
        float lr = lh[i < RI ? i : 0];
#pragma unroll
        for (int rr = 1; rr < 4; ++rr)
          if (4 * rr + i < RI && R == rr) lr = lh[(4 * rr + i) % RI];
        // INT4 values entered as 128 + u: the row's values are u - 8
        const float off = kI4 ? -136.0f * lr : 0.0f;
        if (whole) {
          if (r / GT >= s_ql) continue;
          const int64_t out_row = ((int64_t)(s_tok + r / GT) * a.num_q_heads + h0 + r % GT) * D;
          const float inv = a.v_scale / lr;
          float o[VEPL];
#pragma unroll
          for (int t = 0; t < VEPL; ++t) o[t] = (accm[t][i] + off) * inv;
          store_out<PKV_BF16, VEPL>(a.out, out_row + c * VEPL, o);
        } else {
          const int64_t pr = (((int64_t)b * kvgroups + kvg) * RI + r) * a.max_splits + piece;
          float* dst = a.ws_acc + pr * D + c * VEPL;
#pragma unroll
          for (int t = 0; t < VEPL; t += 4) {
            const f32x4_t v4 = {(accm[t][i] + off) * a.v_scale, (accm[t + 1][i] + off) * a.v_scale,
                                (accm[t + 2][i] + off) * a.v_scale, (accm[t + 3][i] + off) * a.v_scale};
            *reinterpret_cast<f32x4_t*>(dst + t) = v4;
          }
        }
      }
    } else if (vg == 0) {
      if (whole) {
        // row r = t * GT + h: query token t of the piece, head h0 + h
#pragma unroll
        for (int h = 0; h < RI; ++h) {
          if (h / GT >= s_ql) continue;
          const int64_t out_row = ((int64_t)(s_tok + h / GT) * a.num_q_heads + h0 + h % GT) * D;
          const float inv = a.v_scale / lh[h];
          float o[VEPL];
#pragma unroll
          for (int e = 0; e < VEPL; ++e) o[e] = acc[h][e] * inv;
          store_out<PKV_BF16, VEPL>(a.out, out_row + vsub * VEPL, o);
        }
      } else {
        // acc rows: full 128-byte lines, written through the caches: the
        // merge reads them right after, mostly from L2 (streaming them past
        // the caches made the merge reread them from HBM)
#pragma unroll
        for (int h = 0; h < RI; ++h) {
          const int64_t pr = (((int64_t)b * kvgroups + kvg) * RI + h) * a.max_splits + piece;
          float* dst = a.ws_acc + pr * D + vsub * VEPL;
#pragma unroll
          for (int e = 0; e < VEPL; e += 4) {
            // partials hold dequantised V sums (the fp8 V scale applied)
            const f32x4_t v4 = {acc[h][e] * a.v_scale, acc[h][e + 1] * a.v_scale,
                                acc[h][e + 2] * a.v_scale, acc[h][e + 3] * a.v_scale};
            *reinterpret_cast<f32x4_t*>(dst + e) = v4;
          }
        }
      }
    }
    if (!whole) {
      // m and l of the piece's rows side by side: one record of 2 RI floats
      float* ml = a.ws_m + (((int64_t)b * kvgroups + kvg) * a.max_splits + piece) * (2 * RI);
      constexpr int NV = (2 * RI + 3) / 4;
      if (lane < NV) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 2 * RI; ++e)
          if (e / 4 == lane) v[e % 4] = e < RI ? mh[e] : lh[e - RI];
        if constexpr (2 * RI >= 4) {
          const f32x4_t v4 = {v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4_t*>(ml + 4 * lane) = v4;
        } else {
          ml[0] = v[0];
          ml[1] = v[1];
        }
      }
    }
    if (piece == 0 && lane == 0) {
      a.ws_np[2 * ((int64_t)b * kvgroups + kvg)] = npieces;
      a.ws_np[2 * ((int64_t)b * kvgroups + kvg) + 1] = s_tok;
    }
  };

  using VT = std::conditional_t<S::kVBytes == 16, uint4, std::conditional_t<S::kVBytes == 8, uint2, uint32_t>>;
  struct Buf {
    uint32_t k[NC * NH][KB / 4];   // chunks of the item's first KV head, then the second's
    VT v[VU][NH];
  };

  for (long long wbase = u_lo; wbase < u_hi; wbase += kWave) {
    const int nunits = (int)min((long long)kWave, u_hi - wbase);
    // ---- unit records of this window
    rec_phys = -1; rec_gid = -1;
    int bt_raw = -1;    // the unit's table entry, checked once the query loads are in flight too
    if (lane < nunits) {
      const long long u = wbase + lane;
      // head group, then the row: the largest b with cum[b] <= the unit's
      // block index within its group (carry > 0 whenever there are units)
      const int kvg = sh.narrow ? (int)((uint32_t)u / (uint32_t)carry) : (int)(u / carry);
      const int rel = (int)(u - (long long)kvg * carry);
      int lo = 0, hi = a.num_rows;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid] <= rel) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int j = rel - cum[b];
      int req, tok, klo, khi;
      if (have_rec) {
        const int4 rr = rrec[b];
        req = rr.x; tok = rr.y; klo = rr.z; khi = rr.w;
      } else {
        const RowInfo ri = row_info(a, b);
        req = ri.req; tok = ri.tok; klo = ri.lo; khi = ri.hi;
      }
      const int first_blk = klo >> a.bs_log2;
      bt_raw = a.bt[(int64_t)req * a.bt_stride + first_blk + j];
      rec_hoff = (kvg / a.sub_groups) * S::kRowBytes;
      rec_gid = b * kvgroups + kvg;
      rec_pos0 = (first_blk + j) << a.bs_log2;
      rec_lo = klo;
      rec_hi = khi;
      rec_tok = tok;
    }
    // ---- query rows of the pieces that start in this window (slot = order
    // of the piece in the window; the window's first unit always opens slot 0)
    const int gprev = __shfl_up(rec_gid, 1);
    unsigned long long starts = __ballot(lane < nunits && (lane == 0 || rec_gid != gprev));
    const int nstage = min(__popcll(starts), L.qslots);
    {
      uint4 qv[4][QL];
      unsigned long long sm = starts;
      for (int s0 = 0; s0 < nstage; s0 += 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (s0 + k < nstage) {
            const int ln = __builtin_ctzll(sm);
            sm &= sm - 1;
            const int gk = __builtin_amdgcn_readlane(rec_gid, ln);
            const int64_t qe = q_elem(gk, __builtin_amdgcn_readlane(rec_tok, ln));
            const uint16_t* src = reinterpret_cast<const uint16_t*>(a.q) + qe;
            int qlk = 1;                            // query tokens of the piece
            if constexpr (QT > 1) qlk = a.qsl[gk / kvgroups + 1] - a.qsl[gk / kvgroups];
#pragma unroll
            for (int i = 0; i < QL; ++i) {
              // element e: token e / (GT D) of the piece, then its GT heads
              const int e = (i * kWave + lane) * 8;
              const int t = e / (GT * D);
              const int64_t off = (int64_t)t * a.num_q_heads * D + (e - t * GT * D);
              qv[k][i] = (e < QE && t < qlk) ? *reinterpret_cast<const uint4*>(src + off)
                                              : make_uint4(0, 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (s0 + k < nstage) {
#pragma unroll
            for (int i = 0; i < QL; ++i) {
              const int e = (i * kWave + lane) * 8;
              if (e < QE) *reinterpret_cast<uint4*>(qst + (size_t)(s0 + k) * QE + e) = qv[k][i];
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    rec_phys = (lane < nunits && bt_raw >= 0 && bt_raw < a.num_blocks) ? bt_raw : -1;
    asm volatile("" : "+v"(rec_phys), "+v"(rec_gid), "+v"(rec_hoff), "+v"(rec_pos0),
                 "+v"(rec_lo), "+v"(rec_hi), "+v"(rec_tok));
    const int g0 = __builtin_amdgcn_readfirstlane(rec_gid);
    s_ord = 0;
    if (g0 != cur) {
      if (cur >= 0) flush();
      start(0, g0);
      s_first = wbase;
      q_from_lds(0);
    }

    const int nsteps = nunits << spb_log2;
    const int last = nsteps - 1;
    const int smask = (1 << spb_log2) - 1;

    // loads of step st; a step past the window's last one (issued only to
    // keep the pipeline's wait counts static, its data never used) reads
    // the first rows of block 0, which every such load shares, so it is
    // served by the caches instead of fetching the last step again
    auto issue = [&](int st, Buf& bf) __attribute__((always_inline)) {
      const bool past = st > last;
      const int unit = (past ? last : st) >> spb_log2;
      const int r0 = past ? 0 : (st & smask) * 16;
      int phys = __builtin_amdgcn_readlane(rec_phys, unit);
      const int hoff = past ? 0 : __builtin_amdgcn_readlane(rec_hoff, unit);
      phys = (phys < 0 || past) ? 0 : phys;   // bad ids are flagged at the fold; block 0 always exists
      const int64_t off = (int64_t)phys * blk_bytes + hoff + (int64_t)r0 * row_bytes;
      const char* kp = a.kbase + off;
      const char* vp = a.vbase + off;
      if constexpr (kI4) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int j = 0; j < NC / 4; ++j) {
            const uint4 t = kv_load<uint4, NTL>(kp + k_lane + hh * S::kHeadBytes + j * 64);
            const int c0 = hh * NC + 4 * j;
            bf.k[c0][0] = t.x; bf.k[c0 + 1][0] = t.y; bf.k[c0 + 2][0] = t.z; bf.k[c0 + 3][0] = t.w;
          }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if constexpr (KB == 16) {
            const uint4 t = kv_load<uint4, NTL>(kp + k_lane + c * 64);
            bf.k[c][0] = t.x; bf.k[c][1] = t.y; bf.k[c][2] = t.z; bf.k[c][3] = t.w;
          } else {
            const uint2 t = kv_load<uint2, NTL>(kp + k_lane + c * 32);
            bf.k[c][0] = t.x; bf.k[c][1] = t.y;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < VU; ++u)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          bf.v[u][hh] = kv_load<VT, NTL>(vp + v_lane + hh * S::kHeadBytes +
                                         (int64_t)u * (RB ? TPRV : VRPW) * row_bytes);
    };

    // V as floats, zero for keys outside the piece's span
    auto v_floats = [&](auto full_tag, int p0, int tok, const VT& raw, float (&vf)[VEPL])
        __attribute__((always_inline)) {
      constexpr bool full = decltype(full_tag)::value;
      uint32_t vwa[S::kVBytes / 4];
      __builtin_memcpy(vwa, &raw, sizeof(raw));
      if constexpr (KV == PKV_BF16) {
#pragma unroll
        for (int i = 0; i < VEPL / 2; ++i) { vf[2 * i] = bf16_lo(vwa[i]); vf[2 * i + 1] = bf16_hi(vwa[i]); }
      } else {
#pragma unroll
        for (int i = 0; i < VEPL / 4; ++i) {
          const f32x2 v01 = e4m3x2_to_f32<false>(vwa[i]);
          const f32x2 v23 = e4m3x2_to_f32<true>(vwa[i]);
          vf[4 * i] = v01.x; vf[4 * i + 1] = v01.y; vf[4 * i + 2] = v23.x; vf[4 * i + 3] = v23.y;
        }
      }
      if constexpr (!full) {
        const int pos = p0 + tok;
        const bool live = pos >= s_lo && pos <= s_hi;
#pragma unroll
        for (int e = 0; e < VEPL; ++e) vf[e] = live ? vf[e] : 0.f;
      }
    };

    // chunk c of the step's K rows as the MFMA operand (bf16 pairs)
    auto k_operand = [&](const Buf& bf, int c) __attribute__((always_inline)) -> uint4 {
      if constexpr (KV == PKV_BF16) {
        return make_uint4(bf.k[c][0], bf.k[c][1], bf.k[c][2], bf.k[c][3]);
      } else if constexpr (kI4) {
        return int4_k_bf16(bf.k[c][0]);
      } else {
        return make_uint4(e4m3x2_to_bf16x2<false>(bf.k[c][0]), e4m3x2_to_bf16x2<true>(bf.k[c][0]),
                          e4m3x2_to_bf16x2<false>(bf.k[c][1]), e4m3x2_to_bf16x2<true>(bf.k[c][1]));
      }
    };

    // row-broadcast fold of one 16-token step
    auto body_rb = [&](auto full_tag, int p0, const Buf& bf) __attribute__((always_inline)) {
      constexpr bool full = decltype(full_tag)::value;
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 kw = k_operand(bf, c);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), qa[c], sc, 0, 0, 0);
      }
      if constexpr (kPair) {
        // the second KV head's keys against the same query rows; its rows
        // are the upper half
        f32x4_t sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint4 kw = k_operand(bf, NC + c);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), qa[c], sb, 0, 0, 0);
        }
        const bool upper = (lane % 16) >= GT / 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = upper ? sb[i] : sc[i];
      }
      // lane l: tokens 4 (l / 16) + i of head l % 16
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = kI4 ? fmaf(sc[i], a.scale_log2, -kqz) : sc[i] * a.scale_log2;
      if constexpr (!full) {
        // this lane's row: token t of the piece (t >= ql: a padding row)
        int rlo = s_lo, rhi = s_hi;
        if constexpr (QT > 1) {
          const int t = (lane % 16) / GT;
          const int pt = s_hi - (s_ql - 1 - t);
          if (a.causal) rhi = pt;
          if (a.window > 0) rlo = max(s_lo, pt - a.window + 1);
          if (t >= s_ql) rhi = rlo - 1;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = p0 + 4 * (lane / 16) + i;
          if (pos < rlo || pos > rhi) z[i] = -INFINITY;
        }
      }
      const float mx = rows4_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      const bool grow = mx > m1 + kLazyRescale;
      if (__ballot(grow) != 0) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m1 - mx) : 1.0f;   // 0 when m = -inf
        if (grow) m1 = mx;
        ls1 *= alpha;
        if constexpr (kMPV) {
          // this lane's rows 4 R + i take the factors of lanes 4 R + i
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * (lane / 16) + i);
#pragma unroll
            for (int t = 0; t < VEPL; ++t) accm[t][i] *= ai;
          }
        } else {
          static_for<0, RI>([&](auto hc) __attribute__((always_inline)) {
            constexpr int h = decltype(hc)::value;
            const float ah = row_bcast<h>(alpha);
#pragma unroll
            for (int e = 0; e < VEPL; ++e) acc[h][e] *= ah;
          });
        }
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(z[i] - m1);
        if constexpr (!full) p = z[i] == -INFINITY ? 0.f : p;
        pv[i] = p;
      }
      // matrix-core P.V: each weight as a bf16 high part and the bf16
      // remainder, both rounded to nearest even by the hardware conversion
      // (pairs of weights per instruction, no branches)
      uint32_t phw[2], plw[2];
      if constexpr (kMPV) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x2_t h = {(__bf16)pv[2 * j], (__bf16)pv[2 * j + 1]};
          phw[j] = __builtin_bit_cast(uint32_t, h);
          const bf16x2_t l = {(__bf16)(pv[2 * j] - as_float(phw[j] << 16)),
                              (__bf16)(pv[2 * j + 1] - as_float(phw[j] & 0xFFFF0000u))};
          plw[j] = __builtin_bit_cast(uint32_t, l);
          // INT4 values enter with an offset that the flush takes off as a
          // multiple of the weight sum: the sum takes the weights the
          // products use
          if constexpr (kI4) {
            pv[2 * j] = as_float(phw[j] << 16) + as_float(plw[j] << 16);
            pv[2 * j + 1] = as_float(phw[j] & 0xFFFF0000u) + as_float(plw[j] & 0xFFFF0000u);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ls1 += pv[i];
      if constexpr (kMPV) {
        const s16x4_t pa_hi = __builtin_bit_cast(s16x4_t, make_uint2(phw[0], phw[1]));
        const s16x4_t pa_lo = __builtin_bit_cast(s16x4_t, make_uint2(plw[0], plw[1]));
        const s16x4_t zero4 = {0, 0, 0, 0};
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          // B operand of tile t: the bf16 values of dimension t of tokens
          // 4 R .. 4 R + 3, two to a dword (the first token in the low half)
          uint32_t bw[2][VEPL];
          if constexpr (kI4) {
            // nibble u as the bf16 value 128 + u (high byte 0x43, low byte u:
            // exponent of 128, mantissa u, exact); the flush takes 136 times
            // the weight sum off.  Every code is a finite value, so keys
            // outside the piece's span (weight 0) need no zeroing.  Bytes of
            // x: dimensions 0, 2, 4, 6; of y: 1, 3, 5, 7.  v_perm_b32 picks
            // bytes of {S0 (high), S1 (low)}: selector 0..3 a byte of S1,
            // 4..7 a byte of S0.
            constexpr uint32_t kHi = 0x43434343u;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const uint32_t r0 = bf.v[2 * pp][hh], r1 = bf.v[2 * pp + 1][hh];
              const uint32_t x0 = r0 & 0x0F0F0F0Fu, x1 = r1 & 0x0F0F0F0Fu;
              const uint32_t y0 = (r0 >> 4) & 0x0F0F0F0Fu, y1 = (r1 >> 4) & 0x0F0F0F0Fu;
              // bytes j, j + 1 of both tokens, interleaved (j = 0 and 2)
              const uint32_t nx[2] = {__builtin_amdgcn_perm(x1, x0, 0x05010400u),
                                      __builtin_amdgcn_perm(x1, x0, 0x07030602u)};
              const uint32_t ny[2] = {__builtin_amdgcn_perm(y1, y0, 0x05010400u),
                                      __builtin_amdgcn_perm(y1, y0, 0x07030602u)};
#pragma unroll
              for (int t = 0; t < VEPL; ++t) {
                const uint32_t n = (t & 1) ? ny[t / 4] : nx[t / 4];
                bw[pp][t] = __builtin_amdgcn_perm(kHi, n, ((t / 2) & 1) ? 0x04030402u : 0x04010400u);
              }
            }
          } else if constexpr (KV == PKV_FP8_E4M3) {
            // codes of two tokens interleaved byte by byte, so that each
            // hardware conversion of a code pair (exact; the V scale comes at
            // the flush) gives one dimension of both; keys outside the
            // piece's span are zeroed first (code 0 is +0)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              uint2 r0 = bf.v[2 * pp][hh], r1 = bf.v[2 * pp + 1][hh];
              if constexpr (!full) {
                const int pos = p0 + 4 * (lane / 16) + 2 * pp;
                const bool live0 = pos >= s_lo && pos <= s_hi, live1 = pos + 1 >= s_lo && pos + 1 <= s_hi;
                r0 = live0 ? r0 : make_uint2(0, 0);
                r1 = live1 ? r1 : make_uint2(0, 0);
              }
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const uint32_t c0 = w ? r0.y : r0.x, c1 = w ? r1.y : r1.x;   // dimensions 4 w .. 4 w + 3
                const uint32_t n01 = __builtin_amdgcn_perm(c1, c0, 0x05010400u);
                const uint32_t n23 = __builtin_amdgcn_perm(c1, c0, 0x07030602u);
                bw[pp][4 * w] = e4m3x2_to_bf16x2<false>(n01);
                bw[pp][4 * w + 1] = e4m3x2_to_bf16x2<true>(n01);
                bw[pp][4 * w + 2] = e4m3x2_to_bf16x2<false>(n23);
                bw[pp][4 * w + 3] = e4m3x2_to_bf16x2<true>(n23);
              }
            }
          } else {
          // V rows of tokens 4 R + u as bf16 pairs (elements 2k, 2k + 1 in
          // dword k); keys outside the piece's span are zeroed (their weights
          // are 0, but the slots may hold anything)
          uint32_t vw[4][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 raw = bf.v[u][hh];
            vw[u][0] = raw.x; vw[u][1] = raw.y; vw[u][2] = raw.z; vw[u][3] = raw.w;
            if constexpr (!full) {
              const int pos = p0 + 4 * (lane / 16) + u;
              const bool live = pos >= s_lo && pos <= s_hi;
#pragma unroll
              for (int k = 0; k < 4; ++k) vw[u][k] = live ? vw[u][k] : 0u;
            }
          }
#pragma unroll
          for (int t = 0; t < VEPL; ++t) {
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
            bw[0][t] = __builtin_amdgcn_perm(vw[1][t / 2], vw[0][t / 2], sel);
            bw[1][t] = __builtin_amdgcn_perm(vw[3][t / 2], vw[2][t / 2], sel);
          }
          }
          // pair items: each KV head's V meets only its own rows' weights
          s16x4_t ah = pa_hi, al = pa_lo;
          if constexpr (kPair) {
            const bool mine = ((lane % 16) >= GT / 2) == (hh == 1);
            ah = mine ? pa_hi : zero4;
            al = mine ? pa_lo : zero4;
          }
#pragma unroll
          for (int t = 0; t < VEPL; ++t) {
            const s16x4_t vb = __builtin_bit_cast(s16x4_t, make_uint2(bw[0][t], bw[1][t]));
            accm[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, vb, accm[t], 0, 0, 0);
            accm[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, vb, accm[t], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        // this lane's V token: 4 R + u TPRV + (l % 16) / VLPR, probability slot u TPRV + ...
        const int sub = (lane % 16) / VLPR;
        float vf[VEPL];
        v_floats(full_tag, p0, 4 * (lane / 16) + u * TPRV + sub, bf.v[u][0], vf);
        static_for<0, RI>([&](auto hc) __attribute__((always_inline)) {
          constexpr int h = decltype(hc)::value;
          float ph = row_bcast<h>(pv[u * TPRV]);
#pragma unroll
          for (int k = 1; k < TPRV; ++k) {
            const float t = row_bcast<h>(pv[u * TPRV + k]);
            ph = sub == k ? t : ph;
          }
#pragma unroll
          for (int e = 0; e < VEPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        });
      }
      }
    };

    auto body = [&](auto full_tag, int p0, const Buf& bf) __attribute__((always_inline)) {
      constexpr bool full = decltype(full_tag)::value;
      if constexpr (RB) {
        body_rb(full_tag, p0, bf);
      } else {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 kw = k_operand(bf, c);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], __builtin_bit_cast(bf16x8_t, kw), sc, 0, 0, 0);
      }
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = sc[i] * a.scale_log2;
      if constexpr (!full) {
        const int pos = p0 + (lane % 16);
        if (pos < s_lo || pos > s_hi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = -INFINITY;
        }
      }
      float mx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = z[i];
        v = fmaxf(v, dpp<kDppQuadXor1>(v));
        v = fmaxf(v, dpp<kDppQuadXor2>(v));
        v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
        v = fmaxf(v, dpp<kDppRowMirror>(v));
        mx[i] = v;
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float mb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, mx[h % 4]), 16 * (h / 4)));
        if (mb > m[h] + kLazyRescale) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - mb);   // 0 when m = -inf
#pragma unroll
          for (int e = 0; e < VEPL; ++e) acc[h][e] *= alpha;
          if (lane / 16 == h / 4) lsum[h % 4] *= alpha;
          m[h] = mb;
        }
      }
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mv = m[i < GT ? i : 0];
#pragma unroll
        for (int r = 1; r < RG; ++r)
          if (lane / 16 == r && 4 * r + i < GT) mv = m[4 * r + i];
        float pv = __builtin_amdgcn_exp2f(z[i] - mv);
        if constexpr (!full) pv = z[i] == -INFINITY ? 0.f : pv;
        pr[i] = pv;
        lsum[i] += pv;
      }
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int tok = u * VRPW + vg;                // token inside the step
        float vf[VEPL];
        v_floats(full_tag, p0, tok, bf.v[u][0], vf);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const int src = (tok + 16 * (h / 4)) * 4;
          const float ph = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
              src, __builtin_bit_cast(int, pr[h % 4])));
#pragma unroll
          for (int e = 0; e < VEPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        }
      }
      }
    };

    auto run = [&](int st, const Buf& bf) __attribute__((always_inline)) {
      const int unit = st >> spb_log2;
      const int gid = __builtin_amdgcn_readlane(rec_gid, unit);
      if (gid != cur) {                        // next piece of the window
        flush();
        start(unit, gid);
        s_first = wbase + unit;
        ++s_ord;
        if (s_ord < nstage) q_from_lds(s_ord);
        else q_from_global(q_elem(gid, s_tok));
      }
      s_bad |= __builtin_amdgcn_readlane(rec_phys, unit) < 0;
      const int p0 = __builtin_amdgcn_readlane(rec_pos0, unit) + (st & smask) * 16;
      if (p0 >= s_flo && p0 + 15 <= s_fhi) body(std::true_type{}, p0, bf);
      else body(std::false_type{}, p0, bf);
    };

    // loads run DEPTH steps ahead, unconditionally (past the end see issue),
    // so the wait counts stay static; the ring of DEPTH + 1 buffers is
    // unrolled so every index is a constant
    Buf ring[DEPTH + 1];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, ring[d]);
    for (int st = 0; st < nsteps; st += DEPTH + 1) {
#pragma unroll
      for (int k = 0; k <= DEPTH; ++k) {
        issue(st + k + DEPTH, ring[(k + DEPTH) % (DEPTH + 1)]);
        if (st + k < nsteps) run(st + k, ring[k]);
      }
    }
  }
  if (cur >= 0) flush();

  // ---- the decode step's own tokens: row r by worker W - 1 - r % W (the
  // last workers: when the plan has lead shares theirs are the smaller
  // ones), after its own units (no worker reads a slot being written: the
  // rows' visible keys end before their own token)
  if (a.new_token)
    for (int r = W - 1 - blockIdx.x; r < a.num_rows; r += W) write_own_token<D>(a, r, lane);

  // ---- rows without units, one worker each: rows this pass skips (another
  // pass owns them) get a piece count of 0 so that the merge phase leaves
  // them alone; rows that cannot be computed also get NaN output
  for (int r = blockIdx.x; r < a.num_rows; r += W) {
    if (cum[r + 1] != cum[r]) continue;       // a row with units: written by its pieces
    const RowInfo ri = row_info(a, r);
    if (a.new_token && ri.valid) {
      // no cached key: the merge makes the output from the step's own token
      for (int g = lane; g < kvgroups; g += kWave) {
        a.ws_np[2 * ((int64_t)r * kvgroups + g)] = 0;
        a.ws_np[2 * ((int64_t)r * kvgroups + g) + 1] = ri.tok;
      }
      continue;
    }
    if (ri.valid && !ri.skip) continue;
    if (!ri.skip) {
      const int64_t base = (int64_t)ri.tok * a.num_q_heads * D;
      for (int e = lane; e < ri.ntok * a.num_q_heads * D; e += kWave)
        reinterpret_cast<uint16_t*>(a.out)[base + e] = 0x7FC0;
    }
    for (int g = lane; g < kvgroups; g += kWave) {
      a.ws_np[2 * ((int64_t)r * kvgroups + g)] = 0;
      if (a.new_token) a.ws_np[2 * ((int64_t)r * kvgroups + g) + 1] = -1;   // the merge leaves it
    }
    if (a.new_token && a.slots_out && lane == 0) a.slots_out[r] = -1;    // nothing written
  }
}

// --------------------------------------------------------------------------
// The balanced kernel; decode_flat_kernel_2w asks the compiler to fit two
// waves per SIMD (used for eight query heads per item, where the default
// register allocation leaves room for only one).
template <int D, int GT, int KV, int DEPTH, int QT = 1, bool NTL = false>
__global__ __launch_bounds__(64) void decode_flat_kernel(DecodeArgs a) {
  decode_flat_body<D, GT, KV, DEPTH, QT, NTL>(a);
}

template <int D, int GT, int KV, int DEPTH, int QT = 1, bool NTL = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_flat_kernel_2w(
    DecodeArgs a) {
  decode_flat_body<D, GT, KV, DEPTH, QT, NTL>(a);
}

// Merge phase of the balanced scheme: one wave per (row, head group) with
// more than one piece.  The split phase leaves, per (row, group), the piece
// count and the output row, so the wave needs no row lookup.  The wave's
// four 16-lane parts take alternate pieces (part j pieces j, j + 4, ...);
// within a part, lane l takes DPL consecutive dims of the row, so it reads
// one (m, l) pair and one run of acc per piece and merges online, eight
// pieces' loads in flight per part (32 per wave, the first 32 issued with
// the piece count); the parts' states then combine across the wave, and for
// the decode step the first part adds the step's own token.
// Rows of an item one merge wave takes: one (an item of R rows is merged by
// R waves: more waves in flight, fewer loads per lane; measured faster than
// waves of 2 and 4 rows with halves or whole waves on every piece).
__host__ __device__ constexpr int merge_rows_per_wave(int rows) { return rows > 1 ? 1 : rows; }

// The step's own token (position seq_len - 1 of row b, pkv_paged_attention_
// decode_step) joining a merge wave's online softmax for its row h (query
// head `head`): its key and value are the row's new_k / new_v entries taken
// through the cache's format exactly as the split's write stores them (bf16
// as is; fp8 and INT4 encoded with the inverse scale, their code values then
// scaled as the cached keys' are).  The lane's query, key and value
// elements are loaded with the merge's first round of partials
// (OwnToken::load) and joined after the pieces (OwnToken::merge; every lane
// of the first part calls it: the dot product is reduced across a row's LPH
// lanes).
template <int D, int LPH, int DPL>
struct OwnToken {
  uint16_t qb[DPL], kb[DPL], vb[DPL];
  __device__ __forceinline__ void load(const DecodeArgs& a, int b, int head, int tok, int d0, bool active) {
    const int kvh = head / (a.num_q_heads / a.kv_heads);
    const int64_t src = ((int64_t)b * a.kv_heads + kvh) * D + (active ? d0 : 0);
    const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.new_k) + src;
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.new_v) + src;
    const uint16_t* qn = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)tok * a.num_q_heads + head) * D + (active ? d0 : 0);
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      qb[i] = active ? qn[i] : (uint16_t)0;
      kb[i] = active ? kn[i] : (uint16_t)0;
      vb[i] = active ? vn[i] : (uint16_t)0;
    }
  }
  __device__ __forceinline__ void merge(const DecodeArgs& a, float& M, float& den, float (&num)[DPL]) const {
    float dot = 0.f, vv[DPL];
    // fp8: the codes through the hardware conversion, four at a time, as
    // the write makes them (a group holding a NaN takes the integer encoder)
    float k8[DPL], v8[DPL];
    if (a.kv_dtype == PKV_FP8_E4M3) {
#pragma unroll
      for (int i0 = 0; i0 < DPL; i0 += 4) {
        constexpr int G4 = DPL < 4 ? DPL : 4;
        float kx[4], vx[4];
        bool nan = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kx[i] = i < G4 ? as_float((uint32_t)kb[i0 + i] << 16) * a.inv_k_scale : 0.f;
          vx[i] = i < G4 ? as_float((uint32_t)vb[i0 + i] << 16) * a.inv_v_scale : 0.f;
          nan |= kx[i] != kx[i] || vx[i] != vx[i];
        }
        uint32_t kc, vc;
        if (!nan) {
          kc = e4m3x4_encode_no_nan(kx[0], kx[1], kx[2], kx[3]);
          vc = e4m3x4_encode_no_nan(vx[0], vx[1], vx[2], vx[3]);
        } else {
          kc = vc = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kc |= e4m3_encode(kx[i]) << (8 * i);
            vc |= e4m3_encode(vx[i]) << (8 * i);
          }
        }
        const f32x2 ka = e4m3x2_to_f32<false>(kc), kh = e4m3x2_to_f32<true>(kc);
        const f32x2 va = e4m3x2_to_f32<false>(vc), vh = e4m3x2_to_f32<true>(vc);
        const float kd[4] = {ka.x, ka.y, kh.x, kh.y}, vd[4] = {va.x, va.y, vh.x, vh.y};
#pragma unroll
        for (int i = 0; i < G4; ++i) {
          k8[i0 + i] = kd[i];
          v8[i0 + i] = vd[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const float qx = as_float((uint32_t)qb[i] << 16);
      float kx = as_float((uint32_t)kb[i] << 16), vx = as_float((uint32_t)vb[i] << 16);
      if (a.kv_dtype == PKV_FP8_E4M3) {
        kx = k8[i];
        vx = v8[i];
      } else if (a.kv_dtype == PKV_INT4) {
        kx = (float)((int)int4_encode(kx * a.inv_k_scale) - 8);
        vx = (float)((int)int4_encode(vx * a.inv_v_scale) - 8);
      }
      dot = fmaf(qx, kx, dot);
      vv[i] = vx * a.v_scale;
    }
#pragma unroll
    for (int o = LPH / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
    const float s = dot * a.scale_log2;
    const float mn = fmaxf(M, s);
    const float c_old = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
    const float c_new = __builtin_amdgcn_exp2f(s - mn);
    den = den * c_old + c_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) num[i] = num[i] * c_old + vv[i] * c_new;
    M = mn;
  }
};

template <int D, int GT, int OT, int QT = 1, bool NT = false>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int RI = GT * QT;                       // rows of an item: (token, head)
  constexpr int RW = merge_rows_per_wave(RI);       // rows one wave merges
  constexpr int NH = 4;                             // wave parts taking alternate pieces
  constexpr int LPH = kWave / NH / RW;              // lanes per row within a part
  constexpr int DPL = D >= LPH ? D / LPH : 1;       // dims per lane
  constexpr int U = 8;                              // pieces per part and round of loads
  const int lane = threadIdx.x;
  const int half = lane / (kWave / NH);             // the wave part
  const int hl = lane % (kWave / NH);               // lane within its part
  const int groups = a.num_q_heads / GT;
  const int item = blockIdx.x / (RI / RW);
  const int b = item / groups;
  const int g = item % groups;
  const int64_t rg = (int64_t)b * groups + g;
  const int h = (blockIdx.x % (RI / RW)) * RW + hl / LPH;
  const int d0 = (hl % LPH) * DPL;
  const bool active = d0 < D;
  const float* ml = a.ws_m + rg * a.max_splits * (2 * RI);
  const float* accp = a.ws_acc + ((rg * RI + h) * a.max_splits) * D + (active ? d0 : 0);
  float mv[U], lv[U], av[U][DPL];
  // round r: this part's pieces r NH U + NH u + half; the first round is
  // read together with the piece count (the slots exist whatever the count;
  // words past it are ignored)
  auto load_round = [&](int s0, int np) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + NH * u + half, np - 1);   // past the end: repeat the last (skipped below)
      mv[u] = ml[s * (2 * RI) + h];
      lv[u] = ml[s * (2 * RI) + RI + h];
#pragma unroll
      for (int i = 0; i < DPL; ++i) av[u][i] = accp[(int64_t)s * D + i];
    }
  };
  const int np_word = a.ws_np[2 * rg];
  const int tok = a.ws_np[2 * rg + 1];
  // the step's own token: whether the split found it a slot, and this
  // lane's query, key and value elements, read with the first round
  int own_ok = 1;
  OwnToken<D, LPH, DPL> own;
  if constexpr (NT) {
    own_ok = a.ws_own[b];
    own.load(a, b, g * GT + h % GT, b, d0, active);   // decode rows: query row b
  }
  load_round(0, a.max_splits);
  const int np = min(np_word, a.max_splits);
  if (!NT && np <= 1) return;                       // written by the split phase (or rejected)
  if (tok < 0 || tok >= a.num_tokens) return;       // not a row this call wrote
  float M = -INFINITY, den = 0.f;
  float num[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) num[i] = 0.f;
  for (int s0 = 0; s0 < np; s0 += NH * U) {
    if (s0 > 0) load_round(s0, np);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + NH * u + half >= np) break;
      const float mn = fmaxf(M, mv[u]);
      const float c_old = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
      const float c_new = mv[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[u] - mn);
      den = den * c_old + lv[u] * c_new;
#pragma unroll
      for (int i = 0; i < DPL; ++i) num[i] = num[i] * c_old + av[u][i] * c_new;
      M = mn;
    }
  }
  if constexpr (NH > 1) {
    // the other parts' states for the same row and dims (lanes l ^ 16, l ^ 32)
#pragma unroll
    for (int o = kWave / NH; o < kWave; o <<= 1) {
      const float Mo = __shfl_xor(M, o);
      const float deno = __shfl_xor(den, o);
      const float mn = fmaxf(M, Mo);
      const float c_me = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
      const float c_ot = Mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mo - mn);
      den = den * c_me + deno * c_ot;
#pragma unroll
      for (int i = 0; i < DPL; ++i) num[i] = num[i] * c_me + __shfl_xor(num[i], o) * c_ot;
      M = mn;
    }
    if (half != 0) return;                           // one part writes
  }
  if constexpr (NT) {
    static_assert(QT == 1, "one query token per row");
    own.merge(a, M, den, num);
  }
  if (!active) return;
  // row h = t * GT + head: query token t of the row's request
  const int t = h / GT;
  if constexpr (QT > 1) {
    if (t >= a.qsl[b + 1] - a.qsl[b] || tok + t >= a.num_tokens) return;
  }
  const float inv = 1.0f / den;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = num[i] * inv;
  const int64_t out_elem = ((int64_t)(tok + t) * a.num_q_heads + g * GT + h % GT) * D + d0;
  store_out<OT, DPL>(a.out, out_elem, o);
  if constexpr (NT) {
    if (!own_ok) {   // the token has no slot: NaN row
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] = __builtin_nanf("");
      store_out<OT, DPL>(a.out, out_elem, o);
    }
  }
}

// Combine phase of the fixed splits: one wave per (row, query head) with
// more than one split.
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
  const int tok = span.tok;
  const int nsplit = min(ceil_div(span.nvis, a.split_blocks), a.max_splits);
  if (nsplit <= 1) return;

  const int64_t pr0 = ((int64_t)b * a.num_q_heads + h) * a.max_splits;
  const float* mp = a.ws_m + pr0;
  const float* lp = a.ws_l + pr0;
  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, mp[s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float den = 0.f;
  float num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  const bool active = D >= kWave || lane < D;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = mp[s];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    den = fmaf(wgt, lp[s], den);
    if (active) {
      const float* src = a.ws_acc + (pr0 + s) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) num[i] = fmaf(wgt, src[lane + i * kWave], num[i]);
    }
  }
  if (!active) return;
  const float inv = 1.0f / den;
  const int64_t out_row = ((int64_t)tok * a.num_q_heads + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float v[1] = {num[i] * inv};
    store_out<OT, 1>(a.out, out_row + lane + i * kWave, v);
  }
}

// ---- launch templates, one instantiation set per (head_dim, KV dtype)
template <int D, int GT, int KV, int QT>
void launch_split(const DecodeArgs& a, hipStream_t s) {
  const long long kvgroups = (long long)a.num_kv_heads * a.sub_groups;
  const dim3 grid((unsigned)((long long)a.num_rows * kvgroups * a.max_splits));
  constexpr int kRowBytes = D * (KV == PKV_F32 ? 4 : (KV == PKV_BF16 ? 2 : 1));
  if constexpr (kRowBytes >= 64) {
    if ((1 << a.bs_log2) >= 16) {
      decode_split_uni_kernel<D, GT, KV, QT><<<grid, 64, 0, s>>>(a);
      return;
    }
  }
  decode_split_kernel<D, GT, KV, QT><<<grid, 64, 0, s>>>(a);
}

// Fixed splits (vector ALUs), `gt` query heads per work item.
template <int D, int KV>
int run_split_dk(const DecodeArgs& a, int gt, hipStream_t s) {
  constexpr int QT = KV == PKV_F32 ? PKV_F32 : PKV_BF16;
  switch (gt) {
    case 1: launch_split<D, 1, KV, QT>(a, s); return PKV_OK;
    case 2: launch_split<D, 2, KV, QT>(a, s); return PKV_OK;
    case 4: launch_split<D, 4, KV, QT>(a, s); return PKV_OK;
    case 8: launch_split<D, 8, KV, QT>(a, s); return PKV_OK;
  }
  return PKV_ERR_UNSUPPORTED;
}

// Whether the balanced kernel fits two waves per SIMD (256 registers) for
// items of gt heads times qt query tokens.
__host__ __device__ constexpr bool two_waves(int d, int kv, int gt, int qt) {
  return mfma_pv(d, kv, gt, qt) ? gt * qt <= 16 : gt * qt <= (kv_bits(kv) == 4 ? 8 : 4);
}

template <int D, int GT, int KV, int QT = 1>
void launch_stream(const DecodeArgs& a, int workers, hipStream_t s) {
  const size_t lds = flat_lds_layout(a.num_rows, GT * QT, D, a.lds_budget).bytes;
  // loads one step ahead: deeper rings measured slower here (more requests in
  // flight raise the latency of all of them, and past 256 registers only one
  // wave fits on a SIMD)
  constexpr int kDepth = 1;
  if constexpr (KV == kInt4Pair) {   // one variant: items of 2 .. 8 rows, two waves per SIMD
    decode_flat_kernel_2w<D, GT, KV, kDepth, QT><<<workers, 64, lds, s>>>(a);
    return;
  }
  // non-temporal K/V loads when the caller promised that no block is read
  // by two rows (bf16 items; see kv_load)
  if constexpr (KV == PKV_BF16) {
    if (a.stream_loads) {
      if constexpr (two_waves(D, KV, GT, QT))
        decode_flat_kernel_2w<D, GT, KV, kDepth, QT, true><<<workers, 64, lds, s>>>(a);
      else decode_flat_kernel<D, GT, KV, kDepth, QT, true><<<workers, 64, lds, s>>>(a);
      return;
    }
  }
  // up to four rows per item the plan counts on two waves per SIMD, so the
  // kernel must fit in 256 registers (the fp8 build does not unless asked);
  // eight or more rows run one wave per SIMD (INT4 keeps 8 accumulators per
  // row and lane: two waves up to 8 rows; head size 128 accumulating in the
  // matrix cores: up to 16)
  if constexpr (two_waves(D, KV, GT, QT))
    decode_flat_kernel_2w<D, GT, KV, kDepth, QT><<<workers, 64, lds, s>>>(a);
  else decode_flat_kernel<D, GT, KV, kDepth, QT><<<workers, 64, lds, s>>>(a);
}

// Balanced partition (matrix cores), a.heads_per_item query heads per item.
template <int D, int KV>
int run_stream_dk(const DecodeArgs& a, int workers, hipStream_t s) {
  if constexpr (KV != PKV_F32 && D * kv_bits(KV) / 8 >= 64 && (KV != PKV_INT4 || D % 128 == 0)) {
    switch (a.heads_per_item) {
      case 1: launch_stream<D, 1, KV>(a, workers, s); return PKV_OK;
      case 2: launch_stream<D, 2, KV>(a, workers, s); return PKV_OK;
      case 4: launch_stream<D, 4, KV>(a, workers, s); return PKV_OK;
      case 8: launch_stream<D, 8, KV>(a, workers, s); return PKV_OK;
      case 16:
        // 16 rows of 16-element accumulators (fp8, int4) do not fit in the
        // registers; those caches take items of 8 rows
        if constexpr (MfmaShape<D, 16, KV>::VEPL <= 8) {
          launch_stream<D, 16, KV>(a, workers, s);
          return PKV_OK;
        }
        break;
    }
  }
  return PKV_ERR_UNSUPPORTED;
}

// INT4 pair items (a.pair): a.heads_per_item rows over two KV heads.
template <int D>
int run_stream_pair_d(const DecodeArgs& a, int workers, hipStream_t s) {
  switch (a.heads_per_item) {
    case 2: launch_stream<D, 2, kInt4Pair>(a, workers, s); return PKV_OK;
    case 4: launch_stream<D, 4, kInt4Pair>(a, workers, s); return PKV_OK;
    case 8: launch_stream<D, 8, kInt4Pair>(a, workers, s); return PKV_OK;
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D, int GT, int QT = 1>
void launch_merge(const DecodeArgs& a, int ot, hipStream_t s) {
  constexpr int kWaves = GT * QT / merge_rows_per_wave(GT * QT);   // waves per item
  const dim3 grid((unsigned)((long long)a.num_rows * (a.num_q_heads / GT) * kWaves));
  if constexpr (QT == 1) {
    if (a.new_token) {   // bf16 output (the step's queries are bf16)
      decode_merge_kernel<D, GT, PKV_BF16, 1, true><<<grid, 64, 0, s>>>(a);
      return;
    }
  }
  if (ot == PKV_F32) decode_merge_kernel<D, GT, PKV_F32, QT><<<grid, 64, 0, s>>>(a);
  else decode_merge_kernel<D, GT, PKV_BF16, QT><<<grid, 64, 0, s>>>(a);
}

// Multi-token items (row mode 3): a.heads_per_item query heads times a.qt
// query tokens as one item's MFMA rows.  Shapes where a V token row fits
// in 16 lanes (bf16 up to D 128, fp8 up to D 256, int4 D 128 and 256).
template <int D, int KV>
int run_multi_dk(const DecodeArgs& a, int workers, hipStream_t s) {
  if constexpr (KV != PKV_F32 && D * kv_bits(KV) / 8 >= 64 && D * kv_bits(KV) / 8 <= 256 &&
                (KV != PKV_INT4 || D % 128 == 0)) {
    switch (a.heads_per_item * 100 + a.qt) {
      case 102: launch_stream<D, 1, KV, 2>(a, workers, s); return PKV_OK;
      case 104: launch_stream<D, 1, KV, 4>(a, workers, s); return PKV_OK;
      case 108: launch_stream<D, 1, KV, 8>(a, workers, s); return PKV_OK;
      case 202: launch_stream<D, 2, KV, 2>(a, workers, s); return PKV_OK;
      case 204: launch_stream<D, 2, KV, 4>(a, workers, s); return PKV_OK;
      case 402: launch_stream<D, 4, KV, 2>(a, workers, s); return PKV_OK;
    }
    // items of 16 rows: bf16 only (see run_stream_dk)
    if constexpr (MfmaShape<D, 16, KV>::VEPL <= 8) {
      switch (a.heads_per_item * 100 + a.qt) {
        case 208: launch_stream<D, 2, KV, 8>(a, workers, s); return PKV_OK;
        case 404: launch_stream<D, 4, KV, 4>(a, workers, s); return PKV_OK;
        case 802: launch_stream<D, 8, KV, 2>(a, workers, s); return PKV_OK;
      }
    }
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D>
int run_merge_multi_d(const DecodeArgs& a, int ot, hipStream_t s) {
  switch (a.heads_per_item * 100 + a.qt) {
    case 102: launch_merge<D, 1, 2>(a, ot, s); return PKV_OK;
    case 104: launch_merge<D, 1, 4>(a, ot, s); return PKV_OK;
    case 108: launch_merge<D, 1, 8>(a, ot, s); return PKV_OK;
    case 202: launch_merge<D, 2, 2>(a, ot, s); return PKV_OK;
    case 204: launch_merge<D, 2, 4>(a, ot, s); return PKV_OK;
    case 208: launch_merge<D, 2, 8>(a, ot, s); return PKV_OK;
    case 402: launch_merge<D, 4, 2>(a, ot, s); return PKV_OK;
    case 404: launch_merge<D, 4, 4>(a, ot, s); return PKV_OK;
    case 802: launch_merge<D, 8, 2>(a, ot, s); return PKV_OK;
  }
  return PKV_ERR_UNSUPPORTED;
}

template <int D>
int run_combine_d(const DecodeArgs& a, int ot, hipStream_t s) {
  if (a.stream) {
    switch (a.heads_per_item) {
      case 1: launch_merge<D, 1>(a, ot, s); return PKV_OK;
      case 2: launch_merge<D, 2>(a, ot, s); return PKV_OK;
      case 4: launch_merge<D, 4>(a, ot, s); return PKV_OK;
      case 8: launch_merge<D, 8>(a, ot, s); return PKV_OK;
      case 16: launch_merge<D, 16>(a, ot, s); return PKV_OK;
    }
    return PKV_ERR_UNSUPPORTED;
  }
  const dim3 grid((unsigned)((long long)a.num_rows * a.num_q_heads));
  if (ot == PKV_F32) decode_combine_kernel<D, PKV_F32><<<grid, 64, 0, s>>>(a);
  else decode_combine_kernel<D, PKV_BF16><<<grid, 64, 0, s>>>(a);
  return PKV_OK;
}

// Every instantiation the host side calls; each source file decode_*.hip
// instantiates its share, the host side declares them extern.
#define PKV_DECODE_SPLIT_INST(EXT, D, KV) \
  EXT template int run_split_dk<D, KV>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_STREAM_INST(EXT, D, KV) \
  EXT template int run_stream_dk<D, KV>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_COMBINE_INST(EXT, D) \
  EXT template int run_combine_d<D>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_MULTI_INST(EXT, D, KV) \
  EXT template int run_multi_dk<D, KV>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_PAIR_INST(EXT, D) \
  EXT template int run_stream_pair_d<D>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_MERGE_MULTI_INST(EXT, D) \
  EXT template int run_merge_multi_d<D>(const DecodeArgs&, int, hipStream_t);
#define PKV_DECODE_ALL_D(EXT, D)                  \
  PKV_DECODE_SPLIT_INST(EXT, D, PKV_F32)          \
  PKV_DECODE_SPLIT_INST(EXT, D, PKV_BF16)         \
  PKV_DECODE_SPLIT_INST(EXT, D, PKV_FP8_E4M3)     \
  PKV_DECODE_STREAM_INST(EXT, D, PKV_BF16)        \
  PKV_DECODE_STREAM_INST(EXT, D, PKV_FP8_E4M3)    \
  PKV_DECODE_COMBINE_INST(EXT, D)

}  // namespace pkv
