/*
 * pagedkv.h -- C ABI of libpagedkv.so: the paged KV-cache hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * Three steps, as the source pages describe them:
 *   1. turn each request's block table (logical block -> physical block id)
 *      into a per-token write slot: slot = physical_id * block_size +
 *      position % block_size;
 *   2. scatter this step's new K/V rows into the paged cache at those slots;
 *   3. attend over each request's cached K/V by walking its block table
 *      across non-contiguous physical blocks, with a softmax whose normaliser
 *      spans all blocks (computed online, split over long contexts and merged).
 *
 * Sources (web pages, cited by title and section):
 *   [W]  "Deep Dive into vLLM Worker-Side GPU KV Cache Initialization"
 *        (kongchang.com) and its Chinese original "vLLM Worker侧GPU KV
 *        Cache初始化流程深度解析" [W-zh].
 *   [E]  "vLLM의 KV cache 연결 흐름" (llm-engineer.pages.dev card
 *        vllm-kv-cache-engine-to-worker).
 *   [P]  "Understanding PageAttention Memory Optimization" (freaks.city).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers owned by the caller, except the
 *   pkv_cache descriptor and plan structs, which live in host memory and are
 *   read during the call only.  The library never allocates, frees or
 *   synchronises; each call enqueues its kernels on `stream` and returns.
 *   Inputs must stay alive until the stream has passed the call.
 * - Integer ids, lengths and offsets are int32 unless stated; slots are int64.
 * - Host-side argument checks run before anything is enqueued.  On failure a
 *   negative pkv_status is returned and nothing is launched.  A launch failure
 *   returns PKV_ERR_HIP.  Zero-sized work (no tokens, no sequences) returns
 *   PKV_OK and launches nothing.
 * - Data-dependent errors never fault: see each call.
 * - Library state: a per-device cache of the compute-unit count and, once a
 *   chunked call has run a prefill part on a device, one more stream and two
 *   events on that device (created on first use, default priority, kept
 *   until the process ends; see pkv_paged_attention_chunked).  Calls are
 *   reentrant.  Calls on one stream run in order; calls that share an output
 *   or workspace on different streams race.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from the shared library; nothing else is. */
#define PKV_API __attribute__((visibility("default")))

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL                     */
  PKV_ERR_SHAPE = -2,       /* sizes, strides or alignment inconsistent       */
  PKV_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
  PKV_ERR_UNSUPPORTED = -4, /* head_dim / block_size / group size not built   */
  PKV_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required        */
  PKV_ERR_HIP = -6          /* the HIP runtime reported an error              */
} pkv_status;

typedef enum {
  PKV_F32 = 0,       /* IEEE binary32                                        */
  PKV_BF16 = 1,      /* bfloat16                                             */
  PKV_FP8_E4M3 = 2,  /* OCP FP8 E4M3 ("FN"): bias 7, max 448, NaN = 0x7F/0xFF */
  PKV_INT4 = 3       /* 4-bit integer, zero point 8, two per byte (see pkv_cache) */
} pkv_dtype;

/*
 * One attention layer's view of a paged KV cache [W § Step 2: View
 * Transformation; W-zh § Worker与ModelRunner的协作: the
 * [num_blocks, block_size, num_heads, head_dim] layout].
 *
 * `k` and `v` each point at a plane of `num_blocks` physical blocks.  Block b
 * starts `b * block_stride` ELEMENTS after the plane base and holds
 * [block_size, num_kv_heads, head_dim] contiguous elements (token-major, then
 * head, then dim).  block_stride >= block_size * num_kv_heads * head_dim lets
 * K and V of one block interleave in one byte buffer.  Several layers may
 * share the same planes (layers of different groups in the same slot share a
 * tensor [W § Physical View: Two KVCacheTensors]); their block ids never
 * collide because the groups draw from one pool.
 *
 * Alignment: k, v and block_stride * element size must be multiples of 16 B
 * (256 B recommended [W-zh § 第一步：物理分配]).
 *
 * dtype PKV_FP8_E4M3: stored code c means value decode(c) * k_scale (or
 * v_scale); a write quantises x as encode(float(x) * (1.0f / scale)) with
 * round-to-nearest-even and saturation to +-448 [W-zh § KV Cache技术背景:
 * one byte per element halves the cache].
 *
 * dtype PKV_INT4 [W-zh § KV Cache技术背景: half a byte per element, scales
 * fixed offline from calibration data; § 第一步：物理分配: the byte buffer
 * is viewed per precision]: element 2j of a row is the low nibble of byte j,
 * element 2j + 1 the high nibble; nibble u means value (u - 8) * k_scale (or
 * v_scale).  A write stores u = clamp(rint(float(x) * (1.0f / scale)), -8, 7)
 * + 8, rint rounding half to even; NaN stores u = 8.  block_stride counts
 * elements (two per byte) and must be even; head_dim must be a multiple of
 * 32.  Scales are ignored for the other dtypes.
 */
typedef struct {
  void* k;
  void* v;
  int64_t block_stride;
  int32_t num_blocks;
  int32_t block_size;    /* 4, 8, 16 or 32 tokens [W § PagedAttention and Block Management] */
  int32_t num_kv_heads;
  int32_t head_dim;      /* 8, 16, 32, 64, 128 or 256 (PKV_INT4: 32 .. 256) */
  int32_t dtype;         /* pkv_dtype */
  float k_scale;
  float v_scale;
} pkv_cache;

/* Human-readable name of a pkv_status value (static storage). */
PKV_API const char* pkv_status_string(int status);

/*
 * KV bytes one token occupies across `num_layers` layers:
 * num_layers * num_kv_heads * head_dim * 2 (K and V) * element bytes
 * [W-zh § KV Cache技术背景, the 80-layer / 8-head / 128-dim example].
 * Host-only arithmetic.  Returns -1 for a bad dtype, negative sizes, or a
 * result past int64.
 */
PKV_API int64_t pkv_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype);

/*
 * Blocks a memory budget holds [P § Memory Pre-allocation Logic: the budget
 * is total GPU memory times the utilisation ratio; KV bytes are the budget
 * less the non-KV memory; the block count divides them by one block's size
 * and the number of layers].  With hybrid groups the layers that share one
 * block pool are the KV tensors (one per position within a group, W §
 * Hybrid Attention Mechanisms), so num_tensors takes their count.
 * One block = block_size * num_kv_heads * head_dim * 2 (K and V) * element
 * bytes.  budget = floor(total_bytes * utilization) (double arithmetic).
 * Host-only.  Returns the count (0 when the budget leaves no KV bytes, or
 * when one block's bytes are past int64), or
 * PKV_ERR_DTYPE / PKV_ERR_SHAPE (utilization outside (0, 1], sizes <= 0,
 * negative byte counts).
 */
PKV_API int64_t pkv_num_blocks_for_budget(int64_t total_bytes, double utilization,
                               int64_t non_kv_bytes, int32_t num_tensors,
                               int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype);

/*
 * Step 1 -- slot mapping [W § Pinpointing the Token Slot; E § Slot mapping은
 * 왜 필요한가; E § EngineCore가 하는 일 (num_new_tokens)].
 *
 * block_table      [num_reqs, bt_stride] int32; entry j of row r is the
 *                  physical id of request r's logical block j, -1 if none.
 * query_start_loc  [num_reqs + 1] int32, non-decreasing; request r owns the
 *                  step's tokens [query_start_loc[r], query_start_loc[r+1]).
 * num_computed     [num_reqs] int32: tokens of r already in the cache; token
 *                  t of r sits at position num_computed[r] + t - qsl[r].
 * slot_mapping     [num_tokens] int64 output; every element is written:
 *                  slot = id * block_size + position % block_size, or -1 for
 *                  padding tokens (t >= query_start_loc[num_reqs]) and for
 *                  tokens whose lookup is invalid (logical block >= bt_stride,
 *                  id < 0 or id >= num_blocks, negative position).
 * err_count        optional device int32; each invalid lookup adds 1 to it
 *                  (padding does not).  The caller zeroes it.
 */
PKV_API int pkv_slot_mapping(const int32_t* block_table, int32_t bt_stride,
                     int32_t num_reqs, const int32_t* query_start_loc,
                     const int32_t* num_computed, int32_t block_size,
                     int32_t num_blocks, int32_t num_tokens,
                     int64_t* slot_mapping, int32_t* err_count,
                     hipStream_t stream);

/*
 * Step 2 -- KV cache write ("reshape and cache") [W § Summary: the slot
 * decides where each new token is written; E § Slot mapping은 왜 필요한가].
 *
 * key, value       token t, head h, dim d at element
 *                  t * src_token_stride + h * src_head_stride + d, of dtype
 *                  src_dtype (PKV_F32 or PKV_BF16).  Strides in elements;
 *                  base pointers and strides 16-B aligned in bytes.
 * slot_mapping     [num_tokens] int64; slot s >= 0 writes row s % block_size of
 *                  block s / block_size; s < 0 is skipped; s >= num_blocks *
 *                  block_size is skipped too (never written out of range).
 * cache            destination planes.  Same dtype as the source: bit copy.
 *                  F32 -> BF16: round to nearest even.  -> FP8_E4M3 or INT4:
 *                  quantise with the cache's k_scale / v_scale.
 * Two tokens with one slot in a call race (the pages leave it undefined).
 */
PKV_API int pkv_cache_write(const void* key, const void* value, int32_t src_dtype,
                    int64_t src_token_stride, int64_t src_head_stride,
                    const int64_t* slot_mapping, int32_t num_tokens,
                    const pkv_cache* cache, hipStream_t stream);

/*
 * Steps 1 and 2 in one launch [W § Pinpointing the Token Slot and § Summary;
 * E § Slot mapping은 왜 필요한가]: exactly pkv_slot_mapping (block size and
 * pool size from `cache`) followed by pkv_cache_write with the slots it
 * produced.  Every argument means what it means in those two calls;
 * slot_mapping [num_tokens] is written (the caller may read it afterwards)
 * and err_count, when given, counts bad lookups as pkv_slot_mapping does.
 * Rows of key/value for padding tokens or bad lookups are not written.
 * Errors: those of either call, checked before anything is launched.
 */
PKV_API int pkv_slot_mapping_cache_write(const int32_t* block_table, int32_t bt_stride,
                                 int32_t num_reqs, const int32_t* query_start_loc,
                                 const int32_t* num_computed, int32_t num_tokens,
                                 int64_t* slot_mapping, int32_t* err_count,
                                 const void* key, const void* value, int32_t src_dtype,
                                 int64_t src_token_stride, int64_t src_head_stride,
                                 const pkv_cache* cache, hipStream_t stream);

/*
 * Block copy for prefix sharing [W-zh § PagedAttention与Block管理: requests
 * that share a prompt prefix point their tables' leading entries at the same
 * physical blocks, each block counting its references and returning to the
 * pool at zero].  A request about to write into a block it shares first
 * moves to a private copy (copy-on-write, this build's reading of the
 * sharing scheme); this call makes the copies.
 *
 * src_ids, dst_ids [num_pairs] device int32: block src_ids[i] is copied to
 *                  block dst_ids[i], every element of the K and the V plane
 *                  (block_size * num_kv_heads * head_dim elements each).
 * err_count        optional device int32; a pair with an id outside
 *                  [0, num_blocks) is skipped and adds 1.  The caller zeroes it.
 * A block that is a destination and also a source, or two pairs with one
 * destination, in one call: undefined (the copies race).
 */
PKV_API int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src_ids,
                    const int32_t* dst_ids, int32_t num_pairs,
                    int32_t* err_count, hipStream_t stream);

/*
 * Plan of the decode attention: how each row's visible blocks are cut into
 * pieces that are folded independently and merged afterwards, and the
 * workspace the partial results need [P § Handling Softmax Across Blocks:
 * one softmax normaliser spans every block of a row; W-zh §
 * Worker与ModelRunner的协作: kernels tile the keys with an online softmax].
 * Depends only on the arguments and on the current device's compute-unit
 * count.
 *
 * scheme 0 (fixed splits): row r's visible blocks are cut into splits of
 *   split_blocks blocks; one work item per (row, head group, split).
 * scheme 1 (balanced): num_workers workers each take a contiguous share (at
 *   least split_blocks blocks) of all (KV head group, row, block) units,
 *   ordered head group first; a row is cut wherever a share ends.  Used with block sizes that are
 *   multiples of 16 and bf16 / fp8 caches whose head_dim is a multiple of 32
 *   with rows of at least 64 bytes, or INT4 caches with head_dim 128, for at
 *   most 4096 rows (the rows' prefix sums are kept in LDS).  Other bf16 /
 *   fp8 / f32 shapes and more rows take scheme 0; INT4 has no scheme 0 and
 *   returns PKV_ERR_UNSUPPORTED there.
 *
 * The planner fills every field.  A caller may change split_blocks,
 * num_workers, lead_workers, trail_share_pct or heads_per_item (for tuning)
 * and must then call pkv_decode_plan_resize, which recomputes max_splits and
 * workspace_bytes from them.
 */

/* Flags of pkv_decode_plan_make. */
#define PKV_PLAN_BLOCKS_NOT_SHARED 1  /* the caller guarantees that no physical
                                         block is read by two rows of one call
                                         (no shared prefix blocks [W-zh §
                                         PagedAttention与Block管理]); bf16
                                         caches then read K/V with
                                         non-temporal loads, which stream past
                                         the caches.  Results are identical
                                         either way; a wrong promise costs
                                         time only (shared blocks are then
                                         re-read from HBM by every row).      */
#define PKV_PLAN_BLOCKS_SHARED 2      /* the caller says that many rows of one
                                         call read the same physical blocks (a
                                         common prompt [W-zh §
                                         PagedAttention与Block管理]).  The
                                         balanced scheme then runs each
                                         eighth of its units (about one KV
                                         head group's) on one XCD, so a block
                                         that several rows read is re-read
                                         from that XCD's L2 rather than from
                                         the memory-side cache.  Rows are cut
                                         at other places than without the
                                         flag, so results agree within the
                                         attention bounds, not bit for bit.
                                         Not together with
                                         PKV_PLAN_BLOCKS_NOT_SHARED
                                         (PKV_ERR_SHAPE).                     */

typedef struct {
  int32_t split_blocks;   /* scheme 0: blocks per split; 1: least blocks per worker */
  int32_t max_splits;     /* partial slots per (row, query head)                  */
  int32_t heads_per_item; /* query heads one work item processes (scheme 1: a
                             power of two dividing the group, up to 16 for
                             bf16 and 8 for fp8 / INT4; INT4 also takes
                             twice the group, up to 8, for items over two
                             adjacent KV heads, which read whole 128-byte
                             lines; the planner picks that when it can)      */
  int32_t flags;          /* PKV_PLAN_* bits given to pkv_decode_plan_make     */
  size_t workspace_bytes; /* partial (acc, m, l) storage (+ piece counts)         */
  int32_t scheme;         /* 0 or 1, see above                                    */
  int32_t num_workers;    /* scheme 1: workers launched                           */
  int32_t lead_workers;   /* scheme 1: the first lead_workers workers take a full
                             share each, the others trail_share_pct percent of
                             one (a second wave on a SIMD issues more slowly);
                             0 = all shares equal                             */
  int32_t trail_share_pct;/* scheme 1: 1..100, see lead_workers                   */
} pkv_decode_plan;

/*
 * Fill `plan` for a decode (one query token per row) over `num_rows` rows of
 * a cache of `kv_dtype`.  max_seq_len bounds every seq_lens entry;
 * sliding_window 0 = full attention; flags: PKV_PLAN_* bits (0 = none).
 * Returns PKV_ERR_SHAPE for unknown flags and for PKV_PLAN_BLOCKS_NOT_SHARED
 * together with PKV_PLAN_BLOCKS_SHARED.
 */
PKV_API int pkv_decode_plan_make(int32_t num_rows, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t kv_dtype,
                                 int32_t max_seq_len, int32_t sliding_window,
                                 int32_t flags, pkv_decode_plan* plan);

/*
 * After a caller changed a plan's tuning fields (split_blocks, num_workers,
 * lead_workers, trail_share_pct, heads_per_item), recompute max_splits and
 * workspace_bytes for the same num_rows, num_q_heads, head_dim, block_size,
 * max_seq_len and sliding_window that made it.  Host arithmetic only.
 * Returns PKV_ERR_SHAPE for fields no kernel takes (split_blocks outside
 * 1..64 for scheme 0 or below 1 for scheme 1, heads_per_item not dividing
 * num_q_heads, workers below 1, lead_workers outside 0..num_workers,
 * trail_share_pct outside 1..100); whether the heads_per_item suits the
 * cache is checked by the attention calls.
 */
PKV_API int pkv_decode_plan_resize(int32_t num_rows, int32_t num_q_heads,
                                   int32_t head_dim, int32_t block_size,
                                   int32_t max_seq_len, int32_t sliding_window,
                                   pkv_decode_plan* plan);

/*
 * Step 3 (decode form) -- paged attention, one query token per sequence
 * [E § Slot mapping은 왜 필요한가 (attention reads past K/V through the block
 * table) and § Forward 직전의 metadata; P § Handling Softmax Across Blocks;
 * W-zh § Worker与ModelRunner的协作 (tiling + online softmax); W § Hybrid
 * Attention Mechanisms (GQA, sliding window)].
 *
 * out, q           [num_seqs, num_q_heads, head_dim], dtype q_dtype.  q_dtype
 *                  is PKV_F32 for an F32 cache and PKV_BF16 for BF16 / FP8 /
 *                  INT4 caches; out has q's dtype.
 * INT4 caches take head_dim 128, block sizes 16 and 32, groups 1, 2, 4, 8
 * or multiples of 16, and at most 4096 rows; other shapes return
 * PKV_ERR_UNSUPPORTED.
 * block_table      [num_seqs, bt_stride] int32 physical ids.
 * seq_lens         [num_seqs] int32 in [1, max_seq_len]: tokens of the
 *                  sequence including this step's (already written) token.
 * softmax_scale    multiplies q.k before the softmax (usually 1/sqrt(D)).
 * sliding_window   0, or W > 0: a query at position p sees keys p-W+1 .. p.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * workspace        device scratch of at least plan.workspace_bytes
 *                  (pkv_decode_plan_make with the same arguments and
 *                  num_rows = num_seqs); need not be initialised.
 * A row whose seq_len is out of range, or that needs a block-table entry that
 * is past bt_stride, negative or >= num_blocks, gets NaN outputs; no memory
 * outside the cache planes is ever read for it.
 */
PKV_API int pkv_paged_attention_decode(void* out, const void* q, int32_t q_dtype,
                               int32_t num_seqs, int32_t num_q_heads,
                               const pkv_cache* cache,
                               const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, int32_t max_seq_len,
                               float softmax_scale, int32_t sliding_window,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under stream capture, serving loops
 * that must not call hipMalloc, harnesses that forbid allocation).  The
 * partial results go to a scratch array of PKV_STATIC_SCRATCH_BYTES that the
 * library holds in device memory (one per GPU, from the library's load until
 * the process ends); the call itself allocates nothing.  Every other
 * argument and the result are exactly those of pkv_paged_attention_decode
 * (same kernels, same plan).  Returns PKV_ERR_WORKSPACE when the plan for
 * these arguments needs more scratch than that (pkv_decode_plan_make with
 * the same arguments and flags 0 gives the size), PKV_ERR_HIP when the
 * scratch's address cannot be obtained.  The scratch needs no
 * initialisation and keeps the last call's partials; calls that overlap on
 * one GPU (different streams, or different host threads) share it and race.
 */
#define PKV_STATIC_SCRATCH_BYTES (64u << 20)

PKV_API int pkv_paged_attention_decode_static(void* out, const void* q, int32_t q_dtype,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      const pkv_cache* cache,
                                      const int32_t* block_table, int32_t bt_stride,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      float softmax_scale, int32_t sliding_window,
                                      hipStream_t stream);

/*
 * The two phases of pkv_paged_attention_decode as separate calls, for callers
 * that merge partial results themselves (for example across devices) or time
 * the phases.  Phase 1 writes, per (row, query head, split), the base-2
 * partial softmax state
 *     m,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
 *     s_j = softmax_scale * log2(e) * q.k_j,
 * into `workspace`; rows with a single split get their final output written
 * to `out` directly.  Phase 2 merges the splits of the remaining rows:
 *     out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
 * Both take the plan that pkv_decode_plan_make produced for these arguments.
 * Workspace layout (float32): acc [rows, Hq, max_splits, D], then for
 * scheme 0 m [rows, Hq, max_splits] and l [rows, Hq, max_splits]; for
 * scheme 1 (G = heads_per_item) records [rows, Hq / G, max_splits, 2, G]
 * holding the G heads' m then their l, followed by int32 pairs (piece
 * count, output row) [rows, Hq / G, 2] and an int32 per row (used by
 * pkv_paged_attention_decode_step: 1 when the row's new token has a slot).
 * acc holds dequantised V sums (for an
 * fp8 cache the V scale is already applied), so phase 2 needs no cache.
 */
PKV_API int pkv_paged_attention_decode_partials(void* out, const void* q,
                                        int32_t q_dtype, int32_t num_seqs,
                                        int32_t num_q_heads,
                                        const pkv_cache* cache,
                                        const int32_t* block_table,
                                        int32_t bt_stride,
                                        const int32_t* seq_lens,
                                        int32_t max_seq_len,
                                        float softmax_scale,
                                        int32_t sliding_window,
                                        const pkv_decode_plan* plan,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

PKV_API int pkv_paged_attention_decode_combine(void* out, int32_t out_dtype,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t head_dim, int32_t block_size,
                                       const int32_t* seq_lens,
                                       int32_t sliding_window,
                                       const pkv_decode_plan* plan,
                                       const void* workspace,
                                       size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * One decode step in two launches: the step's new K/V rows written to their
 * slots and every sequence's attention over its cache and that token
 * [W § Pinpointing the Token Slot and § Summary (write through the slot
 * mapping); P § Handling Softmax Across Blocks].  Sequence r's new token
 * sits at position seq_lens[r] - 1; its slot is
 * block_table[r][(seq_lens[r] - 1) / block_size] * block_size +
 * (seq_lens[r] - 1) % block_size.  The split pass attends to the cached
 * keys before that position and also writes each new token's K/V codes to
 * its slot and the slot to slot_mapping (one worker per sequence, after its
 * share of the attention; no sequence's visible keys include a slot being
 * written); the merge adds the new token's term (its key and value taken
 * through the cache's format as the write stores them: fp8 and INT4
 * encoded with the inverse scales).
 * Equivalent to pkv_slot_mapping_cache_write (query_start_loc 0..num_seqs,
 * num_computed = seq_lens - 1) followed by pkv_paged_attention_decode_partials
 * and _combine with the same plan: the same cache bytes and slots, and
 * outputs within the attention bounds of each other (the new token joins the
 * softmax in another order, so bits may differ).
 *   new_k, new_v  [num_seqs, Hkv, D] bf16, 16-byte aligned.
 *   slot_mapping  [num_seqs] int64 out, or NULL: -1 for a sequence whose new
 *                 token has no mapped block (its K/V are not written and its
 *                 output is NaN) or whose seq_len is out of range (NaN
 *                 output, nothing written).
 *   plan          a balanced plan (scheme 1) from pkv_decode_plan_make for
 *                 these sizes; others return PKV_ERR_UNSUPPORTED.
 * bf16, fp8 and INT4 caches (f32: PKV_ERR_DTYPE); q and out bf16.
 */
PKV_API int pkv_paged_attention_decode_step(void* out, const void* q, int32_t q_dtype,
                                    const void* new_k, const void* new_v,
                                    int32_t num_seqs, int32_t num_q_heads,
                                    const pkv_cache* cache,
                                    const int32_t* block_table, int32_t bt_stride,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    float softmax_scale, int32_t sliding_window,
                                    const pkv_decode_plan* plan,
                                    void* workspace, size_t workspace_bytes,
                                    int64_t* slot_mapping, hipStream_t stream);

/*
 * Workspace bytes pkv_paged_attention_chunked needs for these arguments.
 */
PKV_API int pkv_chunked_workspace_size(int32_t num_tokens, int32_t num_reqs,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t kv_dtype, int32_t max_query_len,
                               int32_t max_seq_len, int32_t sliding_window,
                               size_t* bytes);

/*
 * Step 3 (chunked form) -- paged attention for a mixed step: requests with
 * several query tokens (prefill chunks) and requests with one (decode)
 * [E § EngineCore가 하는 일 (num_new_tokens per request) and § Forward 직전의
 * metadata; W § Hybrid Attention Mechanisms; W-zh § 混合注意力机制].
 *
 * out, q           [num_tokens, num_q_heads, head_dim], dtype q_dtype (as in
 *                  the decode form).
 * query_start_loc  [num_reqs + 1] int32 as in pkv_slot_mapping; query_start_loc
 *                  [num_reqs] <= num_tokens; rows past it are left untouched.
 * seq_lens         [num_reqs] int32: tokens including this step's; query i of
 *                  request r sits at position seq_lens[r] - q_len_r + i.
 * max_query_len    bounds every q_len_r; max_seq_len bounds every seq_lens[r].
 * causal           1: query at p sees keys <= p.  0: all keys < seq_len.
 * sliding_window   0, or W: keys >= p - W + 1 only.
 * flags            0, PKV_PLAN_BLOCKS_NOT_SHARED or PKV_PLAN_BLOCKS_SHARED,
 *                  as for decode plans, for the decode-shaped parts (single
 *                  queries and multi-token items): no physical block read by
 *                  two requests of the call (their bf16 loads then bypass
 *                  the caches), or many requests reading the same blocks
 *                  (their units then run an eighth per XCD).  Other bits, or
 *                  both, return PKV_ERR_SHAPE.
 * workspace        at least pkv_chunked_workspace_size(...) bytes.
 * Invalid rows (q_len > seq_len, lengths out of range, missing blocks) get NaN.
 * INT4 caches: the decode form's shapes (head_dim 128, at most 4096
 * requests); others return PKV_ERR_UNSUPPORTED.
 * When max_query_len is above 8 (the matrix-core prefill path), the requests
 * with more than one query token run
 * on the library's second stream of the device, forked from `stream` by an
 * event and joined back into it by another, beside the single-query
 * requests' part on `stream`: later work on `stream` sees the whole result,
 * as if the call had run on `stream` alone (stream capture included).
 */
PKV_API int pkv_paged_attention_chunked(void* out, const void* q, int32_t q_dtype,
                                int32_t num_tokens, int32_t num_q_heads,
                                const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t num_reqs,
                                int32_t max_query_len, const pkv_cache* cache,
                                const int32_t* block_table, int32_t bt_stride,
                                int32_t max_seq_len, float softmax_scale,
                                int32_t causal, int32_t sliding_window,
                                int32_t flags, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 E4M3 bulk codec with the exact conversions the cache write and the
 * attention kernels use [W-zh § KV Cache技术背景].
 *   quantize:   codes[i] = encode(float(x[i]) * (1.0f / scale)), x of src_dtype
 *               (PKV_F32 or PKV_BF16); nearest-even, saturating to +-448,
 *               NaN kept.
 *   dequantize: out_dtype PKV_F32: out[i] = decode(codes[i]) * scale (the
 *               conversion the attention kernels apply to V);
 *               out_dtype PKV_BF16: out[i] = decode(codes[i]) as bfloat16,
 *               exact, scale must be 1.0f (the conversion applied to K before
 *               the bf16 dot products; the scale is applied to the score).
 */
PKV_API int pkv_fp8_e4m3_quantize(const void* x, int32_t src_dtype, int64_t n,
                          float scale, uint8_t* codes, hipStream_t stream);
PKV_API int pkv_fp8_e4m3_dequantize(const uint8_t* codes, int64_t n, float scale,
                            int32_t out_dtype, void* out, hipStream_t stream);

/*
 * INT4 bulk codec with the conversions the cache write uses [W-zh § KV
 * Cache技术背景, the INT4 format of pkv_cache].
 *   quantize:   packed[j] = u(2j) | u(2j + 1) << 4 with
 *               u(i) = clamp(rint(float(x[i]) * (1.0f / scale)), -8, 7) + 8,
 *               NaN -> 8; x of src_dtype (PKV_F32 or PKV_BF16); n elements,
 *               n even, packed holds n / 2 bytes.
 *   dequantize: out[i] = (u(i) - 8) * scale as float32 (out_dtype PKV_F32).
 * Returns PKV_ERR_SHAPE for odd n or a scale that is not positive and finite.
 */
PKV_API int pkv_int4_quantize(const void* x, int32_t src_dtype, int64_t n, float scale,
                      uint8_t* packed, hipStream_t stream);
PKV_API int pkv_int4_dequantize(const uint8_t* packed, int64_t n, float scale,
                        int32_t out_dtype, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
