// Library-wide entry points: status strings, sizing closed form, device info.
#include <mutex>

#include "host_common.h"

namespace pkv {

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] > 0) return cached[dev];
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    cached[dev] = cus;
  }
  return cus;
}

int device_max_lds() {
  constexpr int kDefault = 160 * 1024;   // gfx950: a workgroup may take the whole CU's LDS
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kDefault;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] > 0) return cached[dev];
  }
  int bytes = 0;
  if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      bytes <= 0)
    bytes = kDefault;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    cached[dev] = bytes;
  }
  return bytes;
}

}  // namespace pkv

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_NULL: return "PKV_ERR_NULL: a required pointer is NULL";
    case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE: inconsistent sizes, strides or alignment";
    case PKV_ERR_DTYPE: return "PKV_ERR_DTYPE: unknown or unsupported dtype combination";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: head_dim, block_size or group size not built";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown pkv_status";
  }
}

// Per-token KV bytes over all layers: layers * kv_heads * head_dim * 2 * elt
// (elt half a byte for INT4).
extern "C" int64_t pkv_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t dtype) {
  const int bits = pkv::dtype_bits(dtype);
  if (bits == 0 || num_layers < 0 || num_kv_heads < 0 || head_dim < 0) return -1;
  int64_t bits_total;   // layers * heads * dim * 2 * bits, -1 past int64
  if (__builtin_mul_overflow((int64_t)num_layers * num_kv_heads, (int64_t)head_dim * 2 * bits, &bits_total))
    return -1;
  return bits_total / 8;
}

// Blocks a memory budget holds: floor(total * utilisation) - non-KV bytes,
// divided by one block's K+V bytes times the KV tensors sharing the pool.
extern "C" int64_t pkv_num_blocks_for_budget(int64_t total_bytes, double utilization,
                                             int64_t non_kv_bytes, int32_t num_tensors,
                                             int32_t block_size, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t dtype) {
  const int bits = pkv::dtype_bits(dtype);
  if (bits == 0) return PKV_ERR_DTYPE;
  if (total_bytes < 0 || non_kv_bytes < 0 || num_tensors <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || !(utilization > 0.0 && utilization <= 1.0))
    return PKV_ERR_SHAPE;
  // floor(total * utilization) <= total <= INT64_MAX, but the product is
  // rounded to a double first and 2^63 itself does not convert
  const double b = (double)total_bytes * utilization;
  const int64_t budget = b >= 0x1p63 ? INT64_MAX : (int64_t)b;
  const int64_t available = budget - non_kv_bytes;
  if (available <= 0) return 0;
  int64_t block_bits, per_block;
  if (__builtin_mul_overflow((int64_t)block_size * num_kv_heads, (int64_t)head_dim * 2 * bits, &block_bits) ||
      __builtin_mul_overflow(block_bits / 8, (int64_t)num_tensors, &per_block))
    return 0;   // one block is larger than any budget
  return available / per_block;
}
