// Slot mapping (step 1), KV cache write (step 2), block copies and the bulk FP8 and INT4 codecs.
//
// Slot mapping follows the page "Deep Dive into vLLM Worker-Side GPU KV Cache
// Initialization", section "Pinpointing the Token Slot": position p of a
// request lives in logical block p / block_size at offset p % block_size; with
// the block-table entry id for that logical block its slot is
// id * block_size + offset.  The tokens of one step start at the request's
// computed-token count ("vLLM의 KV cache 연결 흐름", section on EngineCore:
// new tokens = tokens with speculation - computed tokens).
//
// The cache write scatters each token's K/V rows to the slot's row of the
// paged planes ([num_blocks, block_size, kv_heads, head_dim], section
// "Summary" of the first page; layout from the Chinese original, section
// "Worker与ModelRunner的协作").
#include "common.h"
#include "host_common.h"

namespace pkv {

// ------------------------------------------------------------------ K1
// Slot of token t of the step, -1 for padding or a bad lookup; `owned` tells
// whether a request owns t.  q and ncs are query_start_loc and num_computed
// (in LDS or global memory).  Position p of request r lives in logical block
// p / block_size at offset p % block_size.
constexpr int kSlotStage = 1024;   // requests whose metadata a workgroup stages in LDS

__device__ __forceinline__ int64_t token_slot(int t, const int* q, const int* ncs,
                                              const int32_t* __restrict__ bt, int32_t bt_stride,
                                              int32_t num_reqs, int32_t bs_log2, int32_t num_blocks,
                                              bool& owned) {
  owned = t >= q[0] && t < q[num_reqs];
  if (!owned) return -1;
  int lo = 0, hi = num_reqs;  // largest r < num_reqs with qsl[r] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q[mid] <= t) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int64_t pos = (int64_t)ncs[r] + (t - q[r]);
  const int64_t logical = pos >> bs_log2;
  int64_t slot = -1;
  if (pos >= 0 && logical < bt_stride) {
    const int32_t id = bt[(int64_t)r * bt_stride + logical];
    if (id >= 0 && id < num_blocks)
      slot = ((int64_t)id << bs_log2) + (pos & ((1 << bs_log2) - 1));
  }
  return slot;
}

// One thread per token of the step.  The owning request is found by binary
// search over query_start_loc; all reads stay inside the arrays the caller
// described (block-table row index < bt_stride, request index < num_reqs).
// query_start_loc[0..R] and num_computed[0..R) into LDS by a workgroup of
// 256 threads, both loads of an entry issued before either store, so the
// staging costs one memory round trip (R <= kSlotStage).
__device__ __forceinline__ void stage_requests(const int32_t* qsl, const int32_t* nc, int num_reqs,
                                               int* sq, int* snc) {
  for (int i = threadIdx.x; i <= num_reqs; i += 256) {
    const int q = qsl[i];
    const int n = i < num_reqs ? nc[i] : 0;
    sq[i] = q;
    if (i < num_reqs) snc[i] = n;
  }
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ bt, int32_t bt_stride, int32_t num_reqs,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ nc,
    int32_t bs_log2, int32_t num_blocks, int32_t num_tokens,
    int64_t* __restrict__ out, int32_t* __restrict__ err) {
  // query_start_loc and num_computed go to LDS in one load round when they
  // fit, so a token's chain of dependent global loads is just the table entry
  __shared__ int sq[kSlotStage + 1];
  __shared__ int snc[kSlotStage];
  const bool staged = num_reqs <= kSlotStage;
  if (staged) {
    stage_requests(qsl, nc, num_reqs, sq, snc);
    __syncthreads();
  }
  const int* q = staged ? sq : qsl;
  const int* ncs = staged ? snc : nc;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= num_tokens) return;
  bool owned;
  const int64_t slot = token_slot(t, q, ncs, bt, bt_stride, num_reqs, bs_log2, num_blocks, owned);
  out[t] = slot;
  if (owned && slot < 0 && err) atomicAdd(err, 1);   // padding is not an error
}

// ------------------------------------------------------------------ K2
struct WriteArgs {
  const void* key;
  const void* value;
  int64_t tok_stride;   // source elements between tokens
  int64_t head_stride;  // source elements between heads
  const int64_t* slots;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t bs_log2;
  int64_t num_slots;    // num_blocks * block_size
  int64_t block_stride; // destination elements between blocks
  void* kdst;
  void* vdst;
  float inv_k_scale;
  float inv_v_scale;
  // fused slot mapping (cache_write_kernel<..., true>): the slots are
  // computed here and stored to slots_out
  const int32_t* bt;
  int32_t bt_stride;
  int32_t num_reqs;
  const int32_t* qsl;
  const int32_t* nc;
  int32_t num_blocks;
  int64_t* slots_out;
  int32_t* err;
};

template <int kBytes>
struct RawChunk;
template <> struct RawChunk<16> { using T = uint4; };
template <> struct RawChunk<8> { using T = uint2; };
template <> struct RawChunk<4> { using T = uint32_t; };

// Load `n` source elements starting at p as binary32 values.
template <int SRC, int N>
__device__ __forceinline__ void load_as_f32(const void* p, float (&x)[N]) {
  if constexpr (SRC == PKV_F32) {
    const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      uint4 w = v[i];
      x[4 * i + 0] = as_float(w.x); x[4 * i + 1] = as_float(w.y);
      x[4 * i + 2] = as_float(w.z); x[4 * i + 3] = as_float(w.w);
    }
  } else {  // bf16
    if constexpr (N >= 8) {
      const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        uint4 w = v[i];
        x[8 * i + 0] = bf16_lo(w.x); x[8 * i + 1] = bf16_hi(w.x);
        x[8 * i + 2] = bf16_lo(w.y); x[8 * i + 3] = bf16_hi(w.y);
        x[8 * i + 4] = bf16_lo(w.z); x[8 * i + 5] = bf16_hi(w.z);
        x[8 * i + 6] = bf16_lo(w.w); x[8 * i + 7] = bf16_hi(w.w);
      }
    }
  }
}

// SRC, DST: pkv_dtype; CE: destination elements per thread (16 bytes of
// destination, or the whole row when a row is shorter).
// FUSED: the token's slot is computed as in slot_mapping_kernel (and stored
// once per token) instead of read.
template <int SRC, int DST, int CE, bool FUSED = false>
__global__ __launch_bounds__(256) void cache_write_kernel(WriteArgs a) {
  constexpr int kDstBits = kv_bits(DST);
  constexpr int kSrcElt = SRC == PKV_F32 ? 4 : 2;
  constexpr int kSrcBytes = CE * kSrcElt;
  static_assert(kSrcBytes % 16 == 0, "source chunks are whole 16-byte vectors");
  const int chunks_per_head = a.head_dim / CE;
  const int chunks_per_plane = a.num_kv_heads * chunks_per_head;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.num_tokens * 2 * chunks_per_plane;
  const bool live = idx < total;
  const int t = live ? (int)(idx / (2 * chunks_per_plane)) : 0;
  const int rem = live ? (int)(idx - (int64_t)t * 2 * chunks_per_plane) : 0;
  const int kv = rem >= chunks_per_plane;
  const int j = rem - kv * chunks_per_plane;
  const int h = j / chunks_per_head;
  const int c = j - h * chunks_per_head;
  // The new row's bytes do not depend on its slot (padding tokens have rows
  // too): they are loaded first, so the load overlaps the slot lookup.
  uint4 raw[kSrcBytes / 16];
  if (live) {
    const uint4* s = reinterpret_cast<const uint4*>(
        reinterpret_cast<const char*>(kv ? a.value : a.key) +
        ((int64_t)t * a.tok_stride + (int64_t)h * a.head_stride + (int64_t)c * CE) * kSrcElt);
#pragma unroll
    for (int i = 0; i < kSrcBytes / 16; ++i) raw[i] = s[i];
  }
  int64_t slot;
  if constexpr (FUSED) {
    __shared__ int sq[kSlotStage + 1];
    __shared__ int snc[kSlotStage];
    const bool staged = a.num_reqs <= kSlotStage;   // uniform across the workgroup
    if (staged) {
      stage_requests(a.qsl, a.nc, a.num_reqs, sq, snc);
      __syncthreads();
    }
    if (!live) return;
    bool owned;
    slot = token_slot(t, staged ? sq : a.qsl, staged ? snc : a.nc, a.bt, a.bt_stride, a.num_reqs,
                      a.bs_log2, a.num_blocks, owned);
    if (rem == 0) {
      a.slots_out[t] = slot;
      if (owned && slot < 0 && a.err) atomicAdd(a.err, 1);
    }
  } else {
    if (!live) return;
    slot = a.slots[t];
  }
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);

  const char* src = reinterpret_cast<const char*>(raw);   // the row's bytes, in registers
  // element index times bits over 8 (INT4 chunks start at even elements)
  char* dst = reinterpret_cast<char*>(kv ? a.vdst : a.kdst) +
              (blk * a.block_stride + (off * a.num_kv_heads + h) * a.head_dim + (int64_t)c * CE) * kDstBits / 8;

  if constexpr (SRC == DST) {
    constexpr int kBytes = CE * kDstBits / 8;
    constexpr int kStep = kBytes >= 16 ? 16 : kBytes;
    using T = typename RawChunk<kStep>::T;
#pragma unroll
    for (int i = 0; i < kBytes / kStep; ++i)
      reinterpret_cast<T*>(dst)[i] = reinterpret_cast<const T*>(src)[i];
  } else if constexpr (DST == PKV_BF16) {  // f32 -> bf16, nearest even
    float x[CE];
    load_as_f32<SRC, CE>(src, x);
    uint32_t w[CE / 2];
#pragma unroll
    for (int i = 0; i < CE / 2; ++i)
      w[i] = f32_to_bf16_rne(x[2 * i]) | (f32_to_bf16_rne(x[2 * i + 1]) << 16);
    if constexpr (CE == 8) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int i = 0; i < CE / 8; ++i)
        reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    }
  } else if constexpr (DST == PKV_INT4) {  // 32 elements -> 16 bytes of nibbles
    static_assert(CE == 32, "INT4 chunks are 32 elements");
    const float inv = kv ? a.inv_v_scale : a.inv_k_scale;
    float x[CE];
    load_as_f32<SRC, CE>(src, x);
#pragma unroll
    for (int i = 0; i < CE; ++i) x[i] *= inv;
    *reinterpret_cast<uint4*>(dst) = make_uint4(int4_pack8(x), int4_pack8(x + 8), int4_pack8(x + 16),
                                                int4_pack8(x + 24));
  } else {  // -> fp8 e4m3 with the per-tensor inverse scale
    const float inv = kv ? a.inv_v_scale : a.inv_k_scale;
    float x[CE];
    load_as_f32<SRC, CE>(src, x);
    bool nan = false;
#pragma unroll
    for (int i = 0; i < CE; ++i) {
      x[i] *= inv;
      nan |= x[i] != x[i];
    }
    uint32_t w[CE / 4];
    if (!nan) {  // the hardware conversion (a few operations per element)
#pragma unroll
      for (int i = 0; i < CE / 4; ++i)
        w[i] = e4m3x4_encode_no_nan(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    } else {     // a NaN in the chunk: the integer encoder keeps it
#pragma unroll
      for (int i = 0; i < CE / 4; ++i)
        w[i] = e4m3_encode(x[4 * i]) | (e4m3_encode(x[4 * i + 1]) << 8) |
               (e4m3_encode(x[4 * i + 2]) << 16) | (e4m3_encode(x[4 * i + 3]) << 24);
    }
    if constexpr (CE == 16) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
  }
}

// ------------------------------------------------------------------ codec
template <int SRC>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void* __restrict__ x, int64_t n,
                                                           float inv, uint8_t* __restrict__ codes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v;
  if constexpr (SRC == PKV_F32) v = reinterpret_cast<const float*>(x)[i];
  else v = as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
  codes[i] = (uint8_t)e4m3_encode(v * inv);
}

__global__ __launch_bounds__(256) void fp8_dequantize_f32_kernel(const uint8_t* __restrict__ codes,
                                                                 int64_t n, float scale,
                                                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const f32x2 v = e4m3x2_to_f32<false>((uint32_t)codes[i]);
  out[i] = v.x * scale;
}

__global__ __launch_bounds__(256) void fp8_dequantize_bf16_kernel(const uint8_t* __restrict__ codes,
                                                                  int64_t n,
                                                                  uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint16_t)(e4m3x2_to_bf16x2<false>((uint32_t)codes[i]) & 0xFFFFu);
}

// INT4: one thread per output byte (two elements).
template <int SRC>
__global__ __launch_bounds__(256) void int4_quantize_kernel(const void* __restrict__ x, int64_t nbytes,
                                                            float inv, uint8_t* __restrict__ packed) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nbytes) return;
  float v0, v1;
  if constexpr (SRC == PKV_F32) {
    v0 = reinterpret_cast<const float*>(x)[2 * j];
    v1 = reinterpret_cast<const float*>(x)[2 * j + 1];
  } else {
    v0 = as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[2 * j] << 16);
    v1 = as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[2 * j + 1] << 16);
  }
  packed[j] = (uint8_t)(int4_encode(v0 * inv) | (int4_encode(v1 * inv) << 4));
}

__global__ __launch_bounds__(256) void int4_dequantize_kernel(const uint8_t* __restrict__ packed,
                                                              int64_t n, float scale,
                                                              float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = ((uint32_t)packed[i >> 1] >> (4 * (i & 1))) & 0xFu;
  out[i] = (float)((int)u - 8) * scale;
}

static int log2_int(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

template <int SRC, int DST, bool FUSED = false>
static void launch_write(const WriteArgs& a, int ce, hipStream_t s) {
  const int64_t threads = (int64_t)a.num_tokens * 2 * a.num_kv_heads * (a.head_dim / ce);
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (ce) {
    case 4: if constexpr (DST == PKV_F32) { cache_write_kernel<SRC, DST, 4, FUSED><<<grid, 256, 0, s>>>(a); } break;
    case 8: if constexpr (DST == PKV_BF16 || DST == PKV_FP8_E4M3) { cache_write_kernel<SRC, DST, 8, FUSED><<<grid, 256, 0, s>>>(a); } break;
    case 16: if constexpr (DST == PKV_FP8_E4M3) { cache_write_kernel<SRC, DST, 16, FUSED><<<grid, 256, 0, s>>>(a); } break;
    case 32: if constexpr (DST == PKV_INT4) { cache_write_kernel<SRC, DST, 32, FUSED><<<grid, 256, 0, s>>>(a); } break;
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_slot_mapping(const int32_t* block_table, int32_t bt_stride, int32_t num_reqs,
                                const int32_t* query_start_loc, const int32_t* num_computed,
                                int32_t block_size, int32_t num_blocks, int32_t num_tokens,
                                int64_t* slot_mapping, int32_t* err_count, hipStream_t stream) {
  if (num_tokens < 0 || num_reqs < 0 || bt_stride < 0 || num_blocks < 0) return PKV_ERR_SHAPE;
  if (!block_size_supported(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping || !query_start_loc) return PKV_ERR_NULL;
  if (num_reqs > 0 && (!block_table || !num_computed)) return PKV_ERR_NULL;
  if (num_reqs > 0 && bt_stride == 0) return PKV_ERR_SHAPE;
  const dim3 grid((unsigned)ceil_div(num_tokens, 256));
  slot_mapping_kernel<<<grid, 256, 0, stream>>>(block_table, bt_stride, num_reqs, query_start_loc,
                                                num_computed, log2_int(block_size), num_blocks,
                                                num_tokens, slot_mapping, err_count);
  return launch_status();
}

// Checks of a cache write and its arguments (no slots yet); fills `a` and
// the destination elements per thread.  PKV_OK with a.num_tokens == 0 means
// nothing to launch.
static int prepare_write(WriteArgs& a, int& ce, const void* key, const void* value, int32_t src_dtype,
                         int64_t src_token_stride, int64_t src_head_stride, int32_t num_tokens,
                         const pkv_cache* cache) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  const int dst = cache->dtype;
  if (dst == PKV_F32 && src_dtype != PKV_F32) return PKV_ERR_DTYPE;
  a = WriteArgs{};
  a.num_tokens = num_tokens;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value) return PKV_ERR_NULL;
  const int se = dtype_size(src_dtype);
  const int D = cache->head_dim;
  if (src_head_stride < D || src_token_stride < src_head_stride * (cache->num_kv_heads - 1) + D)
    return PKV_ERR_SHAPE;
  if (!aligned16(key) || !aligned16(value) || (src_token_stride * se) % 16 ||
      (src_head_stride * se) % 16)
    return PKV_ERR_SHAPE;
  // destination elements per thread: 16 bytes of destination, capped by the row
  ce = 128 / dtype_bits(dst);
  if (ce > D) ce = D;
  // sources narrower than 16 bytes per chunk are not vectorised: bf16 -> fp8
  // with D = 8 reads 16 bytes (fine); everything else keeps >= 16 source bytes.
  if (ce * se < 16) return PKV_ERR_UNSUPPORTED;

  a.key = key;
  a.value = value;
  a.tok_stride = src_token_stride;
  a.head_stride = src_head_stride;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = D;
  a.bs_log2 = log2_int(cache->block_size);
  a.num_slots = (int64_t)cache->num_blocks * cache->block_size;
  a.block_stride = cache->block_stride;
  a.kdst = cache->k;
  a.vdst = cache->v;
  a.inv_k_scale = 1.0f / cache->k_scale;
  a.inv_v_scale = 1.0f / cache->v_scale;
  return PKV_OK;
}

template <bool FUSED>
static int dispatch_write(const WriteArgs& a, int ce, int src_dtype, int dst, hipStream_t stream) {
  if (src_dtype == PKV_F32) {
    if (dst == PKV_F32) launch_write<PKV_F32, PKV_F32, FUSED>(a, ce, stream);
    else if (dst == PKV_BF16) launch_write<PKV_F32, PKV_BF16, FUSED>(a, ce, stream);
    else if (dst == PKV_FP8_E4M3) launch_write<PKV_F32, PKV_FP8_E4M3, FUSED>(a, ce, stream);
    else launch_write<PKV_F32, PKV_INT4, FUSED>(a, ce, stream);
  } else {
    if (dst == PKV_BF16) launch_write<PKV_BF16, PKV_BF16, FUSED>(a, ce, stream);
    else if (dst == PKV_FP8_E4M3) launch_write<PKV_BF16, PKV_FP8_E4M3, FUSED>(a, ce, stream);
    else launch_write<PKV_BF16, PKV_INT4, FUSED>(a, ce, stream);
  }
  return launch_status();
}

extern "C" int pkv_cache_write(const void* key, const void* value, int32_t src_dtype,
                               int64_t src_token_stride, int64_t src_head_stride,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               const pkv_cache* cache, hipStream_t stream) {
  WriteArgs a;
  int ce = 0;
  const int st = prepare_write(a, ce, key, value, src_dtype, src_token_stride, src_head_stride,
                               num_tokens, cache);
  if (st != PKV_OK || num_tokens == 0) return st;
  if (!slot_mapping) return PKV_ERR_NULL;
  a.slots = slot_mapping;
  return dispatch_write<false>(a, ce, src_dtype, cache->dtype, stream);
}

extern "C" int pkv_slot_mapping_cache_write(const int32_t* block_table, int32_t bt_stride,
                                            int32_t num_reqs, const int32_t* query_start_loc,
                                            const int32_t* num_computed, int32_t num_tokens,
                                            int64_t* slot_mapping, int32_t* err_count,
                                            const void* key, const void* value, int32_t src_dtype,
                                            int64_t src_token_stride, int64_t src_head_stride,
                                            const pkv_cache* cache, hipStream_t stream) {
  if (num_reqs < 0 || bt_stride < 0 || num_tokens < 0) return PKV_ERR_SHAPE;
  WriteArgs a;
  int ce = 0;
  const int st = prepare_write(a, ce, key, value, src_dtype, src_token_stride, src_head_stride,
                               num_tokens, cache);
  if (st != PKV_OK || num_tokens == 0) return st;
  if (!slot_mapping || !query_start_loc) return PKV_ERR_NULL;
  if (num_reqs > 0 && (!block_table || !num_computed)) return PKV_ERR_NULL;
  if (num_reqs > 0 && bt_stride == 0) return PKV_ERR_SHAPE;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.num_reqs = num_reqs;
  a.qsl = query_start_loc;
  a.nc = num_computed;
  a.num_blocks = cache->num_blocks;
  a.slots_out = slot_mapping;
  a.err = err_count;
  return dispatch_write<true>(a, ce, src_dtype, cache->dtype, stream);
}

extern "C" int pkv_fp8_e4m3_quantize(const void* x, int32_t src_dtype, int64_t n, float scale,
                                     uint8_t* codes, hipStream_t stream) {
  if (n < 0) return PKV_ERR_SHAPE;
  if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (!(scale > 0.0f && scale < 3.0e38f)) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!x || !codes) return PKV_ERR_NULL;
  const float inv = 1.0f / scale;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (src_dtype == PKV_F32) fp8_quantize_kernel<PKV_F32><<<grid, 256, 0, stream>>>(x, n, inv, codes);
  else fp8_quantize_kernel<PKV_BF16><<<grid, 256, 0, stream>>>(x, n, inv, codes);
  return launch_status();
}

extern "C" int pkv_fp8_e4m3_dequantize(const uint8_t* codes, int64_t n, float scale,
                                       int32_t out_dtype, void* out, hipStream_t stream) {
  if (n < 0) return PKV_ERR_SHAPE;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (out_dtype == PKV_BF16 && scale != 1.0f) return PKV_ERR_UNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (!codes || !out) return PKV_ERR_NULL;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (out_dtype == PKV_F32)
    fp8_dequantize_f32_kernel<<<grid, 256, 0, stream>>>(codes, n, scale, reinterpret_cast<float*>(out));
  else
    fp8_dequantize_bf16_kernel<<<grid, 256, 0, stream>>>(codes, n, reinterpret_cast<uint16_t*>(out));
  return launch_status();
}

extern "C" int pkv_int4_quantize(const void* x, int32_t src_dtype, int64_t n, float scale,
                                 uint8_t* packed, hipStream_t stream) {
  if (n < 0 || (n & 1)) return PKV_ERR_SHAPE;
  if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (!(scale > 0.0f && scale < 3.0e38f)) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!x || !packed) return PKV_ERR_NULL;
  const float inv = 1.0f / scale;
  const int64_t nb = n / 2;
  const dim3 grid((unsigned)((nb + 255) / 256));
  if (src_dtype == PKV_F32) int4_quantize_kernel<PKV_F32><<<grid, 256, 0, stream>>>(x, nb, inv, packed);
  else int4_quantize_kernel<PKV_BF16><<<grid, 256, 0, stream>>>(x, nb, inv, packed);
  return launch_status();
}

extern "C" int pkv_int4_dequantize(const uint8_t* packed, int64_t n, float scale, int32_t out_dtype,
                                   void* out, hipStream_t stream) {
  if (n < 0 || (n & 1)) return PKV_ERR_SHAPE;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (!(scale > 0.0f && scale < 3.0e38f)) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!packed || !out) return PKV_ERR_NULL;
  const dim3 grid((unsigned)((n + 255) / 256));
  int4_dequantize_kernel<<<grid, 256, 0, stream>>>(packed, n, scale, reinterpret_cast<float*>(out));
  return launch_status();
}

// ------------------------------------------------------------------ block copy
// Copy-on-write support for blocks shared between requests: every element of
// block src is copied to block dst in both planes.  One workgroup per (pair,
// plane), 16-byte moves (block bases and block data sizes are multiples of
// 16 bytes).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* k, char* v, int64_t stride_bytes,
                                                          int64_t data_bytes, const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int32_t num_blocks,
                                                          int32_t* err) {
  const int pair = blockIdx.x;
  const int s = src[pair];
  const int d = dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) {
    if (blockIdx.y == 0 && threadIdx.x == 0 && err) atomicAdd(err, 1);
    return;
  }
  char* base = blockIdx.y == 0 ? k : v;
  const uint4* from = reinterpret_cast<const uint4*>(base + (int64_t)s * stride_bytes);
  uint4* to = reinterpret_cast<uint4*>(base + (int64_t)d * stride_bytes);
  const int64_t n = data_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += 256) to[i] = from[i];
}

extern "C" int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src_ids, const int32_t* dst_ids,
                               int32_t num_pairs, int32_t* err_count, hipStream_t stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_ids || !dst_ids) return PKV_ERR_NULL;
  const int64_t data = elem_bytes((int64_t)cache->block_size * cache->num_kv_heads * cache->head_dim,
                                  cache->dtype);
  if (data % 16) return PKV_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)num_pairs, 2);
  copy_blocks_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<char*>(cache->k), reinterpret_cast<char*>(cache->v),
                                               elem_bytes(cache->block_stride, cache->dtype), data, src_ids, dst_ids,
                                               cache->num_blocks, err_count);
  return launch_status();
}
