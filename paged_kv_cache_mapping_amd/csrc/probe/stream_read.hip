// Streaming-read probe: how fast this GPU reads the bytes a paged decode
// step reads, in the same pieces, with nothing else to do.  It is the
// practical ceiling the decode's split kernel is measured against (the
// pages ask that block alignment "maximise bandwidth utilisation":
// "vLLM Worker侧GPU KV Cache初始化流程深度解析", section 第一步：物理分配).
//
// A unit is the K and the V rows of one KV head for `tokens` consecutive
// token slots of one block: `tokens` rows of `head_bytes`, `row_bytes` apart,
// starting `unit_off[u]` bytes into the K and the V plane.  Single-wave
// workers take equal contiguous shares of the units and stream them with
// 16-byte loads, DEPTH units ahead, folding every word into an XOR that is
// written once per worker (so the loads cannot be dropped).  Built as its
// own library (libpkvprobe.so); it is a measurement, not a step of the path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkvprobe.h"

namespace {

constexpr int kWave = 64;
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ __launch_bounds__(64) void stream_read_kernel(const char* kbase, const char* vbase,
                                                         const int64_t* unit_off, int num_units,
                                                         int row_bytes, int tokens, uint32_t* sink) {
  // per unit and plane: tokens x 256 bytes = 4 x 64 lanes x 16 bytes (the
  // host checks head_bytes == 256 and tokens == 16)
  const int lane = threadIdx.x;
  const int per = (num_units + gridDim.x - 1) / gridDim.x;
  const int u0 = min(num_units, (int)blockIdx.x * per);
  const int u1 = min(num_units, u0 + per);
  const int lane_off = (lane / 16) * row_bytes + (lane % 16) * 16;   // token lane/16 (+4 per load)
  v4u buf[DEPTH + 1][8];
  uint32_t acc = 0;
  const int64_t first_off = unit_off[0];       // past-the-end loads all read unit 0 (cached)
  for (int wbase = u0; wbase < u1; wbase += kWave) {
    // lane i holds the offset of unit wbase + i
    const int n = min(kWave, u1 - wbase);
    const int64_t my_off = lane < n ? unit_off[wbase + lane] : first_off;
    auto issue = [&](int k, v4u (&b)[8]) __attribute__((always_inline)) {
      const int kk = k < n ? k : 0;
      int64_t off = (int64_t)__builtin_amdgcn_readlane((int)(my_off & 0xFFFFFFFF), kk) |
                    ((int64_t)__builtin_amdgcn_readlane((int)(my_off >> 32), kk) << 32);
      off = (k < n ? off : first_off) + lane_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(kbase + off + (int64_t)i * 4 * row_bytes));
        b[4 + i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(vbase + off + (int64_t)i * 4 * row_bytes));
      }
    };
    auto fold = [&](const v4u (&b)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= b[i][0] ^ b[i][1] ^ b[i][2] ^ b[i][3];
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, buf[d]);
    for (int k0 = 0; k0 < n; k0 += DEPTH + 1) {
#pragma unroll
      for (int k = 0; k <= DEPTH; ++k) {
        issue(k0 + k + DEPTH, buf[(k + DEPTH) % (DEPTH + 1)]);
        if (k0 + k < n) fold(buf[k]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int pkvprobe_stream_read(const void* k_plane, const void* v_plane, const int64_t* unit_off,
                                    int32_t num_units, int32_t row_bytes, int32_t head_bytes,
                                    int32_t tokens, int32_t workers, int32_t depth, uint32_t* sink,
                                    hipStream_t stream) {
  if (!k_plane || !v_plane || !unit_off || !sink) return -1;
  if (num_units <= 0 || workers <= 0 || head_bytes != 256 || tokens != 16 || row_bytes < 256 ||
      row_bytes % 16)
    return -2;
  const char* k = reinterpret_cast<const char*>(k_plane);
  const char* v = reinterpret_cast<const char*>(v_plane);
  switch (depth) {
    case 1: stream_read_kernel<1><<<workers, kWave, 0, stream>>>(k, v, unit_off, num_units, row_bytes, tokens, sink); break;
    case 2: stream_read_kernel<2><<<workers, kWave, 0, stream>>>(k, v, unit_off, num_units, row_bytes, tokens, sink); break;
    case 3: stream_read_kernel<3><<<workers, kWave, 0, stream>>>(k, v, unit_off, num_units, row_bytes, tokens, sink); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
