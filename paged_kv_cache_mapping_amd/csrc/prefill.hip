// Chunked prefill attention on the matrix cores.
//
// A chunk of a prompt attends, causally (or not) and within an optional
// sliding window, to the request's cached keys, which it finds by walking the
// request's block table ("vLLM의 KV cache 연결 흐름", sections on slot mapping
// and on the metadata handed to the backend); the softmax spans every block
// and is kept online ("Understanding PageAttention Memory Optimization",
// "Handling Softmax Across Blocks"; Chinese worker-side page, section
// "Worker与ModelRunner的协作"); grouped-query heads share a KV head and a
// window keeps the most recent W positions ("Deep Dive into vLLM Worker-Side
// GPU KV Cache Initialization", "Hybrid Attention Mechanisms").
//
// Decomposition (MI355X): one persistent workgroup of eight waves per
// compute unit.  The work is cut into units of 32 keys of an item (request,
// KV head, tile of query tokens), and workgroup w takes a contiguous,
// balanced share of the units; a share that ends inside an item leaves its
// state in a slot for the merge kernel.  A wave owns NBW blocks of 16 rows;
// a row is one (query token, query head of the group).  Keys stream through
// LDS in tiles of 32 (K and V double-buffered, staged by the whole
// workgroup from the block table slice in LDS).  Per tile and 16-row block:
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q
//                 rows kept in registers): lane l holds keys 4(l/16)+i of
//                 row l%16, so each row's softmax state lives in one lane
//                 (replicated over the four lane groups);
//   O^T += V^T P^T on the same instruction: P^T needs no data movement -- its
//                 eight k slots per lane are the lane's own probabilities,
//                 which fixes the order of keys along k -- and V^T comes from
//                 the LDS tile through the gfx950 transpose read, which hands
//                 lane j of a 16-lane group element j of four consecutive
//                 key rows.
// The running max is lazy (rescale only when it grows by more than 2^8); P
// enters the product as a bf16 high part plus a bf16 remainder (about 16
// significant bits, so the result stays within the bf16 output's own
// rounding); everything else accumulates in fp32.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "host_common.h"
#include "prefill.h"

namespace pkv {

namespace {

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));
typedef short pf_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pf_i16x4 lds_i16x4;

// Waves per workgroup: two per SIMD, one computes while the other waits.  (A
// four-wave form, one per SIMD so that a decode wave fits beside it, folded
// at about 60 % of this one's rate and was slower overall.)  The merge kernel
// runs 512 threads.
constexpr int kPfWavesAlone = 8;
constexpr int kPfMergeThreads = 512;
constexpr int kPfKeys = 32;          // keys per tile
constexpr float kPfLazy = 8.0f;      // keep a stale max until a score beats it by 2^8

template <int D, int G, int NW>
struct PfShape {
  static constexpr int NT = NW * 64;             // threads per workgroup
  static constexpr int NBW = 2;                  // 16-row blocks per wave
  static constexpr int TPN = 16 / G;             // query tokens per row block
  static constexpr int TW = NBW * TPN;           // query tokens per wave
  static constexpr int TWG = NW * TW;            // query tokens per workgroup
  static constexpr int NC = D / 32;              // k-chunks of the score product
  static constexpr int MB = D / 16;              // 16-dim blocks of the output
  // LDS bytes per staged key row.  K rows are read 16 rows x 16 bytes per
  // pass (a 16-byte pad puts the rows on disjoint banks); V rows are read by
  // the transpose load, 8 rows x 32 bytes per pass (a 32-byte pad does).
  static constexpr int RSK = D * 2 + 16;
  static constexpr int RSV = D * 2 + 32;
  static constexpr int TILEK = kPfKeys * RSK;    // LDS bytes of one K tile
  static constexpr int TILEV = kPfKeys * RSV;    // LDS bytes of one V tile
  static constexpr int TILE = TILEK + TILEV;     // LDS bytes of one staged K + V tile
  static constexpr int CPR = D / 8;              // 16-byte bf16 chunks per key row
  static constexpr int CPT = kPfKeys * CPR;      // chunks per tile
  static constexpr int CPTH = (CPT + NT - 1) / NT;  // chunks per thread and plane
  static_assert(16 % G == 0, "group must divide 16");
};

inline size_t pf_align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Maximum over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), on the gfx950 lane-swap instructions instead of LDS permutes:
// swapping a value with itself across the two halves, then across odd and
// even rows, hands each lane its partner's copy.
__device__ __forceinline__ float pf_group4_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int G>
size_t pf_lds_bytes(int max_blocks) {
  return 2 * (size_t)PfShape<D, G, kPfWavesAlone>::TILE + pf_align16((size_t)max_blocks * sizeof(int));
}

// ---- the balanced partition
//
// Work units are key tiles of items; an item is (request, KV head, tile of
// query tokens), ordered request-major, then KV head, then query tile, so
// that neighbouring units read the same KV head's blocks.  Workgroup share
// w (of W) owns units [floor(U w / W), floor(U (w + 1) / W)).  A stretch of
// one item inside a share is a piece: a piece that is the whole item writes
// the output; a piece cut by a share boundary writes its unnormalised state
// into one of the share's two slots (2w: the piece that continues an item
// begun in an earlier share, 2w + 1: the piece whose item goes on into a
// later share) and the merge kernel combines the item's slots.

// One request as the partition sees it.
struct PfReq {
  int r;        // request index
  int q0, ql, L, p0;
  int ntq;      // query tiles with rows to write (0: not a multi-query request)
  bool valid;   // lengths agree with the arguments (otherwise its rows get NaN)
};

template <int TWG>
__device__ __forceinline__ PfReq pf_req(const PrefillArgs& a, int r) {
  PfReq q;
  q.r = r;
  q.q0 = a.qsl[r];
  const int end = a.qsl[r + 1];
  q.ql = end - q.q0;
  q.L = a.seq_lens[r];
  q.p0 = q.L - q.ql;
  const bool rows = q.ql > 1 && q.q0 >= 0 && end <= a.num_tokens;
  q.ntq = rows ? min((q.ql + TWG - 1) / TWG, a.tiles_per_req) : 0;
  q.valid = q.L > 0 && q.L <= a.max_seq_len && q.ql <= q.L && q.ql <= a.max_query_len;
  return q;
}

// Key tiles of query tile qt (one unit for an invalid request: its rows are
// written as NaN by whichever share owns that unit).
template <int TWG>
__device__ __forceinline__ int pf_item_units(const PrefillArgs& a, const PfReq& q, int qt) {
  if (!q.valid) return 1;
  const int tok_lo = qt * TWG, tok_hi = min(q.ql, tok_lo + TWG);
  const int khi = a.causal ? q.p0 + tok_hi - 1 : q.L - 1;
  const int klo = a.window > 0 ? max(0, q.p0 + tok_lo - a.window + 1) : 0;
  return khi / kPfKeys - klo / kPfKeys + 1;
}

// Units of one KV head's items of a request.
template <int TWG>
__device__ __forceinline__ long long pf_head_units(const PrefillArgs& a, const PfReq& q) {
  long long n = 0;
  for (int qt = 0; qt < q.ntq; ++qt) n += pf_item_units<TWG>(a, q, qt);
  return n;
}

// Whole workgroup: the total unit count; for target >= 0 also the request
// holding unit `target` and that request's first unit.
template <int TWG, int NW>
__device__ long long pf_scan(const PrefillArgs& a, long long target, int& req, long long& req_first) {
  constexpr int NT = NW * 64;
  __shared__ long long wsum[NW];
  __shared__ long long found[2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // an earlier call may still be reading `found`
  if (threadIdx.x == 0) {
    found[0] = -1;
    found[1] = 0;
  }
  __syncthreads();
  long long carry = 0;
  for (int base = 0; base < a.num_reqs; base += NT) {
    const int r = base + (int)threadIdx.x;
    long long u = 0;
    if (r < a.num_reqs) u = pf_head_units<TWG>(a, pf_req<TWG>(a, r)) * a.num_kv_heads;
    long long x = u;   // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    long long before = carry, chunk = 0;
    for (int i = 0; i < NW; ++i) {
      if (i < wave) before += wsum[i];
      chunk += wsum[i];
    }
    const long long first = before + x - u;
    if (target >= 0 && u > 0 && first <= target && target < first + u) {
      found[0] = r;
      found[1] = first;
    }
    carry += chunk;
    __syncthreads();
  }
  req = (int)found[0];
  req_first = found[1];
  return carry;
}

// The item holding unit u of request r (whose first unit is rfirst).
struct PfItem {
  int kvh, qt;
  long long first;   // the item's first unit
  int units;
};

template <int TWG>
__device__ __forceinline__ PfItem pf_item(const PrefillArgs& a, const PfReq& q, long long rfirst,
                                          long long u) {
  const long long per_head = pf_head_units<TWG>(a, q);
  PfItem it;
  const long long local = u - rfirst;
  it.kvh = (int)(local / per_head);
  long long rem = local - (long long)it.kvh * per_head;
  it.qt = 0;
  int n = pf_item_units<TWG>(a, q, 0);
  while (rem >= n) {
    rem -= n;
    ++it.qt;
    n = pf_item_units<TWG>(a, q, it.qt);
  }
  it.first = u - rem;
  it.units = n;
  return it;
}

// What share w tells the merge: the total unit count, and the item its first
// piece continues (head = 1) when that item began in an earlier share.
struct PfShareRec {
  long long units;   // U
  long long first;   // the item's first and one-past-last unit
  long long end;
  int q0, ql, kvh, qt;
  int head;
  int pad;
};
static_assert(sizeof(PfShareRec) == 48, "share record layout");

// Share boundaries and the XCD-aware order of shares: workgroups are dealt
// to the eight XCDs in turn, so share w goes to the workgroup that puts
// consecutive shares (which read the same KV head) on one XCD's L2.
__device__ __forceinline__ long long pf_bound(long long U, int w, int W) {
  return U * w / W;
}
// Floats of the slot region (accumulators, then (m, l) pairs); the share
// records follow it.
__host__ __device__ constexpr long long pf_slot_floats(int W, int D) {
  return (long long)2 * W * 256 * (D + 2);
}
__device__ __forceinline__ int pf_share_of_block(int b, int W) {
  return (W % 8 == 0) ? (b % 8) * (W / 8) + b / 8 : b;
}

// One piece: key tiles [ta, tb) of item (request q, KV head kvh, query tile
// qt), counted from the item's first key tile.  slot < 0: the piece is the
// whole item and writes the output; otherwise it writes its unnormalised
// state to that slot.
template <int D, int G, int KV, int NW>
__device__ __forceinline__ void pf_piece(const PrefillArgs& a, char* lds, const PfReq& rq, int kvh,
                                         int qt, int ta, int tb, int slot) {
  using S = PfShape<D, G, NW>;
  constexpr int kPfThreads = S::NT;
  constexpr int NBW = S::NBW, TPN = S::TPN, TW = S::TW, TWG = S::TWG;
  constexpr int NC = S::NC, MB = S::MB, RSK = S::RSK, RSV = S::RSV, TILE = S::TILE;
  constexpr int CPR = S::CPR, CPT = S::CPT, CPTH = S::CPTH;
  constexpr int kBits = kv_bits(KV);                    // 16 bf16, 8 fp8, 4 int4
  int* tab = reinterpret_cast<int*>(lds + 2 * TILE);   // phys block or -1, from block b0

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = lane >> 4;           // lane group of the MFMA layouts
  const int ln16 = lane & 15;
  const int q0 = rq.q0, ql = rq.ql, L = rq.L, p0 = rq.p0;   // p0: position of query 0
  const int tok_lo = qt * TWG;
  const int tok_hi = min(ql, tok_lo + TWG);
  const int hq = a.num_q_heads;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);

  if (!rq.valid) {
    // lengths inconsistent with the arguments: NaN rows, as the other paths
    // (such an item is one unit, so this piece is the whole item)
    const int n = (tok_hi - tok_lo) * G * D;
    for (int e = tid; e < n; e += kPfThreads) {
      const int t = e / (G * D);
      const int rem = e - t * G * D;
      out[((int64_t)(q0 + tok_lo + t) * hq + kvh * G) * D + rem] = 0x7FC0;
    }
    return;
  }

  // the item's keys, then this piece's share of them
  const int khi_item = a.causal ? p0 + tok_hi - 1 : L - 1;
  const int klo_item = a.window > 0 ? max(0, p0 + tok_lo - a.window + 1) : 0;
  const int kt0 = klo_item / kPfKeys + ta, kt1 = klo_item / kPfKeys + tb - 1;
  const int klo = max(klo_item, kt0 * kPfKeys);
  const int khi = min(khi_item, kt1 * kPfKeys + kPfKeys - 1);
  const int b0 = klo >> a.bs_log2;
  const int nblk = (khi >> a.bs_log2) - b0 + 1;
  // more table entries than the launch sized for: the rows are poisoned
  // instead of staging past the slice
  const bool poisoned = nblk > a.max_blocks;

  // ---- table slice of the blocks this piece can touch; whether any of
  // them is unmapped is decided once, for the whole workgroup
  int unmapped = 0;
  for (int i = tid; i < (poisoned ? 0 : nblk); i += kPfThreads) {
    const int j = b0 + i;
    int e = -1;
    if (j < a.bt_stride) e = a.bt[(int64_t)rq.r * a.bt_stride + j];
    const bool ok = e >= 0 && e < a.num_blocks;
    tab[i] = ok ? e : -1;
    unmapped |= ok ? 0 : 1;
  }
  const bool any_unmapped = __syncthreads_or(unmapped) != 0;

  // ---- this wave's rows
  const int tw0 = tok_lo + wave * TW;                 // first query token of the wave
  const bool wave_live = tw0 < tok_hi;
  const int tw_last = min(tw0 + TW, tok_hi) - 1;
  const int wqlo = p0 + tw0, wqhi = p0 + tw_last;     // positions of the wave's queries
  const int wkhi = a.causal ? wqhi : L - 1;
  const int wklo = a.window > 0 ? max(0, wqlo - a.window + 1) : 0;
  const bool wave_full_rows = tw0 + TW <= tok_hi;

  int row_t[NBW];        // query token (request-relative) of this lane's row per block
  int row_h[NBW];        // query head
  bool row_ok[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    row_t[nb] = tw0 + nb * TPN + ln16 / G;
    row_h[nb] = kvh * G + ln16 % G;
    row_ok[nb] = row_t[nb] < tok_hi;
  }

  // B operand of the score product: Q rows, lane l: row l % 16, dims 8 (l / 16) + 32 c
  pf_bf16x8 bq[NBW][NC];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(q0 + row_t[nb]) * hq + row_h[nb]) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (row_ok[nb]) t = *reinterpret_cast<const uint4*>(qp + 32 * c);
      bq[nb][c] = __builtin_bit_cast(pf_bf16x8, t);
    }
  }

  pf_f32x4 acc[NBW][MB];
  float m[NBW], lsum[NBW];
  bool bad[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    m[nb] = -INFINITY;
    lsum[nb] = 0.f;
    bad[nb] = false;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = pf_f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: chunk c = tid + 512 j of a tile is key c / CPR, 16 bytes
  // (8 bf16) at column chunk c % CPR; keys outside [klo, khi] or on an
  // unmapped block stage as zeros
  const int64_t blk_bytes = a.block_stride * kBits / 8;
  const int row_bytes = a.num_kv_heads * D * kBits / 8;
  const int bmask = (1 << a.bs_log2) - 1;
  // 8 elements of the cache: 16 bytes bf16, 8 fp8, 4 int4
  typedef typename std::conditional<kBits == 16, uint4,
                                    typename std::conditional<kBits == 8, uint2, uint32_t>::type>::type Raw;
  // Loads are issued unconditionally (keys outside [klo, khi] or on unmapped
  // blocks read block 0's first row, which always exists) and their data is
  // dropped afterwards: a load skipped under a branch would leave the wait
  // counters unknown at the store and make it wait for every load in flight.
  struct Stage {
    Raw k[CPTH], v[CPTH];
    bool ok[CPTH];
  };
  auto stage_load = [&](int kt, Stage& st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPTH; ++j) {
      const int c = (tid + kPfThreads * j) % CPT;     // threads past the tile repeat a chunk
      const int kp = kt * kPfKeys + c / CPR;
      const int cc = c % CPR;
      const bool in = kp >= klo && kp <= khi;
      const int phys = in ? tab[(kp >> a.bs_log2) - b0] : -1;
      const bool ok = phys >= 0;
      const int64_t off = ok ? (int64_t)phys * blk_bytes + (int64_t)(kp & bmask) * row_bytes +
                                   kvh * D * kBits / 8 + cc * kBits
                             : (int64_t)(cc * kBits);
      st.k[j] = *reinterpret_cast<const Raw*>(a.kbase + off);
      st.v[j] = *reinterpret_cast<const Raw*>(a.vbase + off);
      st.ok[j] = ok;
    }
  };
  auto widen = [&](const Raw& x) __attribute__((always_inline)) -> uint4 {
    if constexpr (KV == PKV_BF16) {
      return x;
    } else if constexpr (KV == PKV_INT4) {
      // nibble n (element n) holds u; the staged value is the integer u - 8,
      // exact in bf16 (the scales are applied to the scores and the output)
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = (float)((int)((x >> (8 * i)) & 0xFu) - 8);
        const float hi = (float)((int)((x >> (8 * i + 4)) & 0xFu) - 8);
        w[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
      }
      return make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      return make_uint4(e4m3x2_to_bf16x2<false>(x.x), e4m3x2_to_bf16x2<true>(x.x),
                        e4m3x2_to_bf16x2<false>(x.y), e4m3x2_to_bf16x2<true>(x.y));
    }
  };
  auto stage_store = [&](int buf, const Stage& st) __attribute__((always_inline)) {
    char* kt_l = lds + buf * TILE;
    char* vt_l = kt_l + S::TILEK;
#pragma unroll
    for (int j = 0; j < CPTH; ++j) {
      const int c = tid + kPfThreads * j;
      if (c < CPT) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(kt_l + (c / CPR) * RSK + (c % CPR) * 16) = st.ok[j] ? widen(st.k[j]) : z;
        *reinterpret_cast<uint4*>(vt_l + (c / CPR) * RSV + (c % CPR) * 16) = st.ok[j] ? widen(st.v[j]) : z;
      }
    }
  };

  auto compute = [&](int kt, int buf) __attribute__((always_inline)) {
    const int kbase = kt * kPfKeys;
    if (!wave_live || kbase > wkhi || kbase + kPfKeys - 1 < wklo) return;
    const char* kt_l = lds + buf * TILE;
    const char* vt_l = kt_l + S::TILEK;
    // an unmapped block among the tile's keys makes the rows that see it NaN
    bool tile_bad = false;
    if (any_unmapped) {
      const int lo = max(kbase, klo), hi = min(kbase + kPfKeys - 1, khi);
      for (int bi = (lo >> a.bs_log2) - b0; bi <= (hi >> a.bs_log2) - b0; ++bi)
        tile_bad |= tab[bi] < 0;
    }
    bool full = wave_full_rows && !tile_bad && kbase >= wklo && kbase + kPfKeys - 1 <= L - 1;
    if (a.causal) full = full && kbase + kPfKeys - 1 <= wqlo;
    if (a.window > 0) full = full && kbase >= wqhi - a.window + 1;

    // A operand of the score product: K rows 16 kh + l % 16, dims 8 (l / 16) + 32 c
    pf_bf16x8 ak[2][NC];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        ak[kh][c] = *reinterpret_cast<const pf_bf16x8*>(kt_l + (16 * kh + ln16) * RSK + (8 * grp + 32 * c) * 2);

    pf_bf16x8 pb[NBW], pl[NBW];   // P = bf16 high part + bf16 remainder
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      float z[2][4];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        pf_f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[kh][c], bq[nb][c], sc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[kh][i] = sc[i] * a.scale_log2;
      }
      if (!full) {
        const int qpos = p0 + row_t[nb];
        const int rhi = a.causal ? qpos : L - 1;
        const int rlo = a.window > 0 ? max(0, qpos - a.window + 1) : 0;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kp = kbase + 16 * kh + 4 * grp + i;
            const bool vis = row_ok[nb] && kp >= rlo && kp <= rhi;
            if (vis && tile_bad && tab[(kp >> a.bs_log2) - b0] < 0) bad[nb] = true;
            if (!vis) z[kh][i] = -INFINITY;
          }
      }
      float mt = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                       fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
      mt = pf_group4_max(mt);
      const bool grow = mt > m[nb] + kPfLazy;
      if (__ballot(grow) != 0) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[nb] - mt) : 1.0f;   // 0 when m = -inf
        if (grow) m[nb] = mt;
        lsum[nb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] *= alpha;
      }
      // a row with no visible key so far keeps m = -inf: subtract 0 instead,
      // so that masked scores (-inf) give exp2(-inf) = 0 without a select
      const float msub = m[nb] == -INFINITY ? 0.f : m[nb];
      float p[2][4];
      float ps = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kh][i] = __builtin_amdgcn_exp2f(z[kh][i] - msub);
          ps += p[kh][i];
        }
      lsum[nb] += ps;
      // k slots 8 (l / 16) + i: keys 4 (l / 16) + i, then 16 + 4 (l / 16) + i.
      // P goes in as two bf16 terms, so that the product keeps about 16 bits
      // of each probability: the high half of the binary32 bits (exact), and
      // the remainder x - high (exact in binary32) rounded to bf16.
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = p[(2 * k) / 4][(2 * k) % 4], x1 = p[(2 * k + 1) / 4][(2 * k + 1) % 4];
        const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
        hw[k] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // high halves of x0 (low), x1 (high)
        const float r0 = x0 - __uint_as_float(u0 & 0xFFFF0000u);
        const float r1 = x1 - __uint_as_float(u1 & 0xFFFF0000u);
        const pf_bf16x2 rb = {(__bf16)r0, (__bf16)r1};                 // nearest even
        lw[k] = __builtin_bit_cast(uint32_t, rb);
      }
      pb[nb] = __builtin_bit_cast(pf_bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      pl[nb] = __builtin_bit_cast(pf_bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }

    // O^T += V^T P^T: A = V^T from the tile by transpose reads.  Lane s of a
    // 16-lane group points at key k0 + s / 4, dims d0 + 4 (s % 4); lane j
    // then holds V[k0 + i][d0 + j], i = 0..3.
    const int vrow = 4 * grp + (ln16 >> 2);
    const int vcol = 4 * (ln16 & 3);
    // every V^T operand is read before the products, so the LDS latency is
    // paid once per tile rather than once per 16 dims
    pf_bf16x8 av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const char* v1 = vt_l + vrow * RSV + (16 * mb + vcol) * 2;
      const char* v2 = v1 + 16 * RSV;
      const pf_i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1));
      const pf_i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v2));
      av[mb] = __builtin_bit_cast(
          pf_bf16x8, (short __attribute__((ext_vector_type(8)))){lo4[0], lo4[1], lo4[2], lo4[3],
                                                                  hi4[0], hi4[1], hi4[2], hi4[3]});
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mb], pb[nb], acc[nb][mb], 0, 0, 0);
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mb], pl[nb], acc[nb][mb], 0, 0, 0);
      }
    }
  };

  // ---- key tiles: loads run three tiles ahead in a ring of register
  // stages, tiles are double-buffered in LDS, one barrier per tile.  Tile t
  // is loaded at step t - 3 into stage t % 3, stored to LDS buffer t % 2 at
  // step t - 1 and folded at step t.  The steps run in whole rounds of three
  // with no exit inside a round and every load and store unconditional
  // (past the last tile the last one is fetched and staged again and not
  // folded): a round with branches around the stages leads the compiler to
  // move stage registers around, and each such copy waits for the load in
  // flight.
  const int rounds = poisoned ? 0 : (kt1 - kt0 + 3) / 3;
  Stage s0, s1, s2;
  if (!poisoned) {
    stage_load(kt0, s0);
    stage_load(min(kt0 + 1, kt1), s1);
    stage_load(min(kt0 + 2, kt1), s2);
    stage_store(0, s0);
    __syncthreads();
  }
  auto step = [&](int rel, Stage& cur, const Stage& next) __attribute__((always_inline)) {
    stage_store((rel + 1) & 1, next);
    stage_load(min(kt0 + rel + 3, kt1), cur);
    if (kt0 + rel <= kt1) compute(kt0 + rel, rel & 1);
    __syncthreads();
  };
  for (int i = 0; i < rounds; ++i) {
    step(3 * i, s0, s1);
    step(3 * i + 1, s1, s2);
    step(3 * i + 2, s2, s0);
  }

  // ---- normalise and store (or hand the state to the merge):
  // lane l holds dims 16 mb + 4 (l / 16) + i of row l % 16
  if (!wave_live) return;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    float lt = lsum[nb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    // every lane takes part in both exchanges (no short-circuit: a lane that
    // skipped the exchange would not hand its flag to the others)
    int bi = (bad[nb] || poisoned) ? 1 : 0;
    bi |= __shfl_xor(bi, 16);
    bi |= __shfl_xor(bi, 32);
    const bool b = bi != 0;
    if (!row_ok[nb]) continue;
    if (slot >= 0) {
      // rows of a slot: wave, then row block, then row of the block
      const int rho = wave * (NBW * 16) + nb * 16 + ln16;
      float* pa = a.part + ((int64_t)slot * (TWG * G) + rho) * D + 4 * grp;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<pf_f32x4*>(pa + 16 * mb) = acc[nb][mb];
      if (grp == 0) {
        float* ml = a.part + (int64_t)2 * a.workers * (TWG * G) * D + ((int64_t)slot * (TWG * G) + rho) * 2;
        *reinterpret_cast<float2*>(ml) = make_float2(m[nb], b ? __builtin_nanf("") : lt);
      }
      continue;
    }
    const float inv = a.v_scale / lt;
    uint16_t* dst = out + ((int64_t)(q0 + row_t[nb]) * hq + row_h[nb]) * D + 4 * grp;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      uint2 w;
      if (b) {
        w = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
      } else {
        w.x = f32_to_bf16_rne(acc[nb][mb][0] * inv) | (f32_to_bf16_rne(acc[nb][mb][1] * inv) << 16);
        w.y = f32_to_bf16_rne(acc[nb][mb][2] * inv) | (f32_to_bf16_rne(acc[nb][mb][3] * inv) << 16);
      }
      *reinterpret_cast<uint2*>(dst + 16 * mb) = w;
    }
  }
}

template <int D, int G, int KV, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_tile_kernel(
    PrefillArgs a) {
  constexpr int TWG = PfShape<D, G, NW>::TWG;
  extern __shared__ __align__(16) char lds[];
  const int W = (int)gridDim.x;
  const int w = pf_share_of_block((int)blockIdx.x, W);
  int r;
  long long rfirst;
  const long long U = pf_scan<TWG, NW>(a, -1, r, rfirst);
  const long long b = pf_bound(U, w, W), e = pf_bound(U, w + 1, W);
  PfShareRec* rec = reinterpret_cast<PfShareRec*>(a.part + pf_slot_floats(W, D)) + w;
  if (b >= e) {
    if (threadIdx.x == 0) {
      PfShareRec x = {};
      x.units = U;
      *rec = x;
    }
    return;
  }
  pf_scan<TWG, NW>(a, b, r, rfirst);
  if (r < 0) return;   // (cannot happen: both scans count the same units)
  PfReq q = pf_req<TWG>(a, r);
  long long span = pf_head_units<TWG>(a, q) * a.num_kv_heads;
  for (long long u = b; u < e;) {
    while (u >= rfirst + span) {   // next request with units (single-query ones have none)
      if (r + 1 >= a.num_reqs) return;
      rfirst += span;
      ++r;
      q = pf_req<TWG>(a, r);
      span = pf_head_units<TWG>(a, q) * a.num_kv_heads;
    }
    const PfItem it = pf_item<TWG>(a, q, rfirst, u);
    const long long end = it.first + it.units;
    const long long pend = end < e ? end : e;
    const bool whole = u == it.first && end <= e;
    const int slot = whole ? -1 : (it.first < b ? 2 * w : 2 * w + 1);
    if (u == b && threadIdx.x == 0) {
      PfShareRec x = {};
      x.units = U;
      x.first = it.first;
      x.end = end;
      x.q0 = q.q0;
      x.ql = q.ql;
      x.kvh = it.kvh;
      x.qt = it.qt;
      x.head = it.first < b ? 1 : 0;
      *rec = x;
    }
    pf_piece<D, G, KV, NW>(a, lds, q, it.kvh, it.qt, (int)(u - it.first), (int)(pend - it.first), slot);
    u = pend;
  }
}

// Combines the slots of every item cut by share boundaries.  Workgroup j
// takes the item that share j's first piece continues when that item began
// in the closest earlier share j' holding units; its pieces are slot
// 2 j' + 1, then slot 2 w of every non-empty share w >= j that the item
// reaches.  Each thread merges one row's share of the dimensions.
template <int D, int G, int NW>
__global__ __launch_bounds__(kPfMergeThreads) void prefill_merge_kernel(PrefillArgs a) {
  using S = PfShape<D, G, NW>;
  constexpr int kPfThreads = kPfMergeThreads;
  constexpr int TWG = S::TWG, TW = S::TW, TPN = S::TPN, NBW = S::NBW;
  constexpr int ROWS = TWG * G;                 // rows of a slot (256)
  constexpr int TPR = kPfThreads / ROWS;        // threads per row
  constexpr int DPT = D / TPR;                  // dims per thread
  static_assert(kPfThreads % ROWS == 0 && D % (4 * TPR) == 0, "merge thread layout");
  const int W = a.workers;
  const int j = (int)blockIdx.x;
  if (j == 0 || j >= W) return;
  const PfShareRec it = reinterpret_cast<const PfShareRec*>(a.part + pf_slot_floats(W, D))[j];
  const long long U = it.units;
  if (!it.head || pf_bound(U, j, W) >= pf_bound(U, j + 1, W)) return;
  // the share before j that holds units (shares in between are empty); the
  // item must have begun there, or an earlier share merges it
  int jp = j - 1;
  while (jp >= 0 && pf_bound(U, jp, W) >= pf_bound(U, jp + 1, W)) --jp;
  if (jp < 0 || it.first < pf_bound(U, jp, W)) return;
  const long long end = it.end;

  const int rho = (int)threadIdx.x / TPR;
  const int d0 = ((int)threadIdx.x % TPR) * DPT;
  const int wv = rho / (NBW * 16), nb = (rho / 16) % NBW, l16 = rho % 16;
  const int tok = it.qt * TWG + wv * TW + nb * TPN + l16 / G;
  const int head = it.kvh * G + l16 % G;
  if (tok >= min(it.ql, it.qt * TWG + TWG)) return;
  const float* ml = a.part + (int64_t)2 * W * ROWS * D;
  auto for_slots = [&](auto&& f) __attribute__((always_inline)) {
    f(2 * jp + 1);
    for (int w = j; w < W; ++w) {
      const long long bw = pf_bound(U, w, W);
      if (bw >= end) break;
      if (bw < pf_bound(U, w + 1, W)) f(2 * w);
    }
  };
  float mx = -INFINITY;
  for_slots([&](int sl) { mx = fmaxf(mx, ml[((int64_t)sl * ROWS + rho) * 2]); });
  float den = 0.f;
  float num[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) num[i] = 0.f;
  for_slots([&](int sl) {
    const float2 rec = *reinterpret_cast<const float2*>(ml + ((int64_t)sl * ROWS + rho) * 2);
    const float wgt = rec.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rec.x - mx);
    den += wgt * rec.y;
    const float* src = a.part + ((int64_t)sl * ROWS + rho) * D + d0;
#pragma unroll
    for (int i = 0; i < DPT; i += 4) {
      const pf_f32x4 v = *reinterpret_cast<const pf_f32x4*>(src + i);
      num[i] += wgt * v[0];
      num[i + 1] += wgt * v[1];
      num[i + 2] += wgt * v[2];
      num[i + 3] += wgt * v[3];
    }
  });
  const float inv = a.v_scale / den;
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(it.q0 + tok) * a.num_q_heads + head) * D + d0;
#pragma unroll
  for (int i = 0; i < DPT; i += 4) {
    uint2 o;
    o.x = f32_to_bf16_rne(num[i] * inv) | (f32_to_bf16_rne(num[i + 1] * inv) << 16);
    o.y = f32_to_bf16_rne(num[i + 2] * inv) | (f32_to_bf16_rne(num[i + 3] * inv) << 16);
    *reinterpret_cast<uint2*>(dst + i) = o;
  }
}

template <int D, int G>
constexpr int pf_tokens_per_wg() { return PfShape<D, G, kPfWavesAlone>::TWG; }

int pf_tokens(int d, int g) {
  switch (d * 100 + g) {
    case 6401: return pf_tokens_per_wg<64, 1>();
    case 6402: return pf_tokens_per_wg<64, 2>();
    case 6404: return pf_tokens_per_wg<64, 4>();
    case 6408: return pf_tokens_per_wg<64, 8>();
    case 6416: return pf_tokens_per_wg<64, 16>();
    case 12801: return pf_tokens_per_wg<128, 1>();
    case 12802: return pf_tokens_per_wg<128, 2>();
    case 12804: return pf_tokens_per_wg<128, 4>();
    case 12808: return pf_tokens_per_wg<128, 8>();
    case 12816: return pf_tokens_per_wg<128, 16>();
    case 25601: return pf_tokens_per_wg<256, 1>();
    case 25602: return pf_tokens_per_wg<256, 2>();
    case 25604: return pf_tokens_per_wg<256, 4>();
    case 25608: return pf_tokens_per_wg<256, 8>();
    case 25616: return pf_tokens_per_wg<256, 16>();
  }
  return 0;
}

template <int D, int G, int KV>
int pf_launch(const PrefillArgs& a, hipStream_t s) {
  const size_t lds = pf_lds_bytes<D, G>(a.max_blocks);
  // past 64 KiB the kernel asks for the larger dynamic LDS explicitly
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_tile_kernel<D, G, KV, kPfWavesAlone>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return PKV_ERR_HIP;
  prefill_tile_kernel<D, G, KV, kPfWavesAlone><<<a.workers, kPfWavesAlone * 64, lds, s>>>(a);
  prefill_merge_kernel<D, G, kPfWavesAlone><<<a.workers, kPfMergeThreads, 0, s>>>(a);
  return PKV_OK;
}

template <int D, int KV>
int pf_launch_g(const PrefillArgs& a, int g, hipStream_t s) {
  switch (g) {
    case 1: return pf_launch<D, 1, KV>(a, s);
    case 2: return pf_launch<D, 2, KV>(a, s);
    case 4: return pf_launch<D, 4, KV>(a, s);
    case 8: return pf_launch<D, 8, KV>(a, s);
    case 16: return pf_launch<D, 16, KV>(a, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

// Table entries one workgroup may need: its keys span the longest context, or
// with a window the window plus the workgroup's own query tokens.
// (tokens: the query tokens one workgroup spans, or the longest query for
// rows that see up to the end of the context)
int pf_max_blocks(int max_seq_len, int bs, int window, int tokens) {
  const long long full = (max_seq_len + (long long)bs - 1) / bs + 1;
  if (window <= 0) return (int)full;
  const long long win = ((long long)window + tokens + 2 * bs - 2) / bs + 1;
  return (int)(full < win ? full : win);
}

}  // namespace

bool prefill_supported(int kv_dtype, int head_dim, int group, int max_seq_len, int block_size,
                       int window, int max_query_len) {
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3 && kv_dtype != PKV_INT4) return false;
  // 256: the accumulators and query rows of two row blocks alone would take
  // 192 of a wave's 256 registers
  if (head_dim != 64 && head_dim != 128) return false;
  if (kv_dtype == PKV_INT4 && head_dim != 128) return false;   // the INT4 head size built
  if (group < 1 || group > 16 || 16 % group) return false;
  if (max_query_len < 2) return false;
  const int tok = pf_tokens(head_dim, group);
  const int mb = pf_max_blocks(max_seq_len, block_size, window, tok > max_query_len ? tok : max_query_len);
  // the staged tiles plus the table slice within the LDS one workgroup may
  // take (one workgroup runs per CU: on gfx950 the CU's whole 160 KiB, which
  // holds the table slice of contexts up to about 500K tokens at head size
  // 128 and block size 16)
  const size_t bytes = 2 * (size_t)(32 * (head_dim * 4 + 48)) + pf_align16((size_t)mb * 4);
  return bytes <= (size_t)device_max_lds();
}

// One workgroup per compute unit (eight waves fill a CU at this kernel's
// register count); two slots of 256 rows x (D + 2) floats each, and one
// share record per workgroup.
static int pf_workers() {
  const int cus = device_cu_count();
  return cus > 0 ? cus : 1;
}

size_t prefill_workspace_bytes(int head_dim) {
  const int w = pf_workers();
  return (size_t)pf_slot_floats(w, head_dim) * sizeof(float) + (size_t)w * sizeof(PfShareRec);
}

int launch_prefill(const PrefillArgs& a0, int kv_dtype, int head_dim, hipStream_t s) {
  PrefillArgs a = a0;
  a.workers = pf_workers();
  if (!a.part) return PKV_ERR_WORKSPACE;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int tok = pf_tokens(head_dim, g);
  if (tok == 0) return PKV_ERR_UNSUPPORTED;
  a.tiles_per_req = (a.max_query_len + tok - 1) / tok;
  a.max_blocks = pf_max_blocks(a.max_seq_len, 1 << a.bs_log2, a.window,
                               tok > a.max_query_len ? tok : a.max_query_len);
  if (a.num_reqs == 0 || a.tiles_per_req == 0) return PKV_OK;
  const bool bf = kv_dtype == PKV_BF16;
  switch (head_dim) {
    case 64: return bf ? pf_launch_g<64, PKV_BF16>(a, g, s) : pf_launch_g<64, PKV_FP8_E4M3>(a, g, s);
    case 128:
      if (kv_dtype == PKV_INT4) return pf_launch_g<128, PKV_INT4>(a, g, s);
      return bf ? pf_launch_g<128, PKV_BF16>(a, g, s) : pf_launch_g<128, PKV_FP8_E4M3>(a, g, s);
  }
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
