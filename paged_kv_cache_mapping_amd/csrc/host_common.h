// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Compute units of the current device (cached per device id).
int device_cu_count();

// LDS bytes one workgroup may take on the current device (its attribute;
// 160 KiB, gfx950's per-CU LDS, when there is no device to ask).
int device_max_lds();

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes per element of a whole-byte type (0 for PKV_INT4 and unknown types).
inline int dtype_size(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

// Bits per element of a cache type (0: unknown).
inline int dtype_bits(int dt) { return dt == PKV_INT4 ? 4 : 8 * dtype_size(dt); }

// Bytes of n elements (n even for PKV_INT4).
inline int64_t elem_bytes(int64_t n, int dt) { return n * dtype_bits(dt) / 8; }

inline bool head_dim_supported(int d) {
  return d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
}

inline bool block_size_supported(int bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32; }

// Validate a cache descriptor (host data only).
inline int check_cache(const pkv_cache* c) {
  if (!c || !c->k || !c->v) return PKV_ERR_NULL;
  if (dtype_bits(c->dtype) == 0) return PKV_ERR_DTYPE;
  if (!block_size_supported(c->block_size) || !head_dim_supported(c->head_dim))
    return PKV_ERR_UNSUPPORTED;
  if (c->dtype == PKV_INT4 && c->head_dim < 32) return PKV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_SHAPE;
  const int64_t block_elems = (int64_t)c->block_size * c->num_kv_heads * c->head_dim;
  if (c->block_stride < block_elems) return PKV_ERR_SHAPE;
  if ((c->block_stride * dtype_bits(c->dtype)) % 128 != 0) return PKV_ERR_SHAPE;
  if (!aligned16(c->k) || !aligned16(c->v)) return PKV_ERR_SHAPE;
  if ((c->dtype == PKV_FP8_E4M3 || c->dtype == PKV_INT4) &&
      !(c->k_scale > 0.0f && c->v_scale > 0.0f && c->k_scale < 3.0e38f && c->v_scale < 3.0e38f))
    return PKV_ERR_SHAPE;
  return PKV_OK;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
