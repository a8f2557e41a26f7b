// Chunked prefill attention on the matrix cores: the multi-query requests of
// a chunked step (the single-query ones take the decode kernels).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pkv {

struct PrefillArgs {
  void* out;                // [num_tokens, Hq, D] bf16
  const void* q;            // [num_tokens, Hq, D] bf16
  const int32_t* qsl;       // [num_reqs + 1]
  const int32_t* seq_lens;  // [num_reqs], including this step's tokens
  int32_t num_reqs;
  int32_t num_tokens;       // rows of q / out
  int32_t max_query_len;
  int32_t max_seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  const char* kbase;        // K plane (bytes)
  const char* vbase;        // V plane (bytes)
  int64_t block_stride;     // elements between physical blocks
  int32_t num_blocks;
  int32_t bs_log2;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t causal;
  int32_t window;           // 0: none
  int32_t tiles_per_req;    // query tiles per request (max_query_len over the tile height)
  int32_t max_blocks;       // table entries one piece may stage
  int32_t workers;          // workgroups of the balanced partition
  float* part;              // 2 * workers partial slots (prefill_workspace_bytes)
  float scale_log2;         // softmax_scale * log2(e) (* k_scale for fp8)
  float v_scale;            // 1, or the fp8 V scale
};

// True if the matrix-core prefill path takes this shape.
bool prefill_supported(int kv_dtype, int head_dim, int group, int max_seq_len, int block_size,
                       int window, int max_query_len);

// Workspace bytes of the partial slots (two per workgroup, one workgroup per
// compute unit of the current device).
size_t prefill_workspace_bytes(int head_dim);

// Launches the prefill kernel for every request with more than one query,
// then the merge of pieces cut by share boundaries; `part` must hold
// prefill_workspace_bytes(head_dim) bytes.
int launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, hipStream_t s);

}  // namespace pkv
