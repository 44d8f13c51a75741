/*
 * mla_decode.h — C ABI of the MI355X (gfx950) paged-KV MLA decode library.
 *
 * The operation (page "深度剖析DeepSeek Infra开源全貌", jingzhunhuoke.net/55333.html,
 * section DAY1 FlashMLA):
 *   - MLA: all query heads of a request attend over ONE shared latent KV head
 *     (terminology paragraph on MLA).  A key row is 576 wide (512 latent + 64
 *     rope); the value row is the first 512 dims of the same cache row.
 *   - The KV cache is paged in blocks of 64 tokens (feature ②): token j of
 *     request b is row j % 64 of page block_table[b][j / 64].
 *   - The result is exact softmax attention computed tile by tile, as two
 *     products, scores then probabilities times values (FlashMLA terminology
 *     paragraph; feature ④).
 *   - Variable per-request lengths are balanced across compute units by
 *     splitting long requests' keys over several workers and merging the
 *     partial results (feature ⑤, dynamic load for variable-length input).
 *
 *   For query row r = t*h_q + h of request b (t < s_q, h < h_q):
 *     visible keys  J = { j < L_b - s_q + 1 + t }  if causal, else { j < L_b },
 *                   less the positions whose table slot holds no page (below)
 *     s_j  = scale * dot(q[b,t,h,0:576], K_b[j,0:576])
 *     LSE  = ln( sum_{j in J} exp(s_j) )                (natural log, fp32)
 *     O    = sum_{j in J} exp(s_j - LSE) * K_b[j,0:512]  (bf16, RNE)
 *   An empty J gives O = 0 and LSE = -inf.
 *
 * Conventions for every entry point:
 *   - All pointers named *_d are DEVICE pointers; the caller allocates and owns
 *     every buffer (inputs, outputs, metadata, workspace).  The library never
 *     allocates or frees and keeps no mutable global state, so calls on
 *     different streams may run concurrently (the one exception is
 *     mla_decode_fwd_noalloc and its static per-device array, below).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Enqueueing entry points are asynchronous: results are valid once the
 *     stream has been synchronised.  They never synchronise the host, except
 *     in the checked mode: with the environment variable MLA_DEBUG_SYNC set
 *     to anything but "" or "0" (read at every call), each launch is followed
 *     by a wait on its stream, so that a kernel fault is returned as
 *     MLA_ERR_HIP by the call that launched it, the launch named in
 *     mla_last_hip_error().  A stream under graph capture is not waited on.
 *   - All arguments are validated on the host BEFORE anything is enqueued; an
 *     invalid call returns a negative status and enqueues nothing.
 *   - Tensors are dense, row-major ("contiguous") with the stated shapes.
 *     q, kcache and out must be 16-byte aligned; int32 and fp32 buffers
 *     4-byte aligned; workspace 256-byte aligned.
 *   - Device data (seqlens, block_table) is not visible to host validation.
 *     A position whose table slot is at or beyond bt_stride, or whose slot
 *     holds a page id outside [0, num_blocks), holds no key: it is left out of
 *     the attention (nothing is read there), in the dense mode as in the
 *     sparse mode.  A row with no key left gets O = 0, LSE = -inf.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MLA_OK               0
#define MLA_ERR_INVALID_ARG (-1) /* null/misaligned pointer, bad size or enum */
#define MLA_ERR_UNSUPPORTED (-2) /* valid but not implemented shape (h_q) */
#define MLA_ERR_WORKSPACE   (-3) /* workspace smaller than mla_decode_workspace_bytes */
#define MLA_ERR_HIP         (-4) /* a HIP runtime call or launch failed */

/* Fixed shape constants. */
#define MLA_BLOCK_SIZE 64        /* tokens per KV page (feature ②) */
#define MLA_D_K 576              /* key width: 512 latent + 64 rope */
#define MLA_D_V 512              /* value width: first 512 dims of the key row */
#define MLA_TILE_META_INTS 8     /* int32 words per part in tile_meta */
#define MLA_MAX_S_Q 128          /* query tokens per request: 1 (decode), 2..8 (draft tokens), up to 128 (a prefill chunk) */

/*
 * mla_decode_num_parts — host only, no HIP call.
 * Recommended number of split-KV parts (workers) for a launch: one workgroup
 * per compute unit.  A workgroup carries one row tile of query rows: 128
 * rows when s_q*h_q is a multiple of 128 (s_q*h_q/128 tiles), else up to 64
 * (s_q*h_q <= 32 fits one tile, larger counts use ceil(s_q*h_q/64) tiles);
 * each part runs once per row tile, so parts = num_cus / row_tiles.
 *   h_q in {16,32,64,128}, 1 <= s_q <= MLA_MAX_S_Q, h_kv == 1, num_cus >= 1.
 * Returns MLA_OK and *num_parts_out >= 1, or an error status.
 */
int mla_decode_num_parts(int batch, int s_q, int h_q, int h_kv, int num_cus,
                         int* num_parts_out);

/*
 * mla_decode_workspace_bytes — host only, no HIP call.
 * Size of the split-partial workspace that mla_decode_fwd /
 * mla_decode_splitkv / mla_decode_combine need for `num_parts` parts:
 *   slots = 2*(num_parts-1) (an upper bound of the pieces of split requests),
 *   bytes = slots * s_q*h_q * (512*2 + 4), rounded up to 256.
 * May be 0 (num_parts == 1); then the workspace pointer may be NULL.
 * Layout (M = s_q*h_q, slots as above): bf16 partial outputs
 * O_part[slots][M][512], each normalised over its own keys and rounded to
 * bf16 as a whole request's output is (fp32 accumulation before; the merge
 * weights are at most 1 and sum to 1, so the rounding adds at most
 * 2^-8 * max|O_part| to a merged element), followed by fp32
 * LSE_part[slots][M] in BASE-2 (log2 of the sum of exp(scale*q.k)), -inf for a
 * piece with no visible key.  Request b's pieces occupy slots
 * [split_offsets[b], split_offsets[b+1]) in key order.
 */
int mla_decode_workspace_bytes(int batch, int s_q, int h_q, int num_parts,
                               size_t* bytes_out);

/*
 * mla_decode_metadata — enqueue the split-KV scheduler (one workgroup).
 * Passage: page "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA, feature ⑤
 * (dynamic load computation for variable-length input); the pages give no
 * rule, so the balancing rule below is this library's own.
 * Reads seqlens_d on the device (no host sync) and writes the partition of
 * all requests' pages over num_parts parts:
 *   tile_meta_d     int32 [num_parts][8] = {begin_req, begin_page, end_req,
 *                   end_page, first_split, 0, 0, 0}; part p covers the
 *                   (request, page) range [begin, end) in lexicographic order.
 *   split_offsets_d int32 [batch+1]: partial-slot prefix; request b owns slots
 *                   [split_offsets[b], split_offsets[b+1]) (empty when the
 *                   request is handled by one part and written directly).
 * Balancing rule (all integers): cost_b = ceil(L_b/64) + c for L_b > 0 and 0
 * otherwise, with the per-request overhead c = min(s_q*h_q, 128)/32 pages
 * (integer division: 0 for 16 rows); the total cost C is cut into num_parts
 * quotas of q = ceil(C/num_parts) units (a request's first c units are its
 * overhead, then one unit per page).
 * Deterministic.
 *   seqlens_d int32 [batch]; block_size must be 64; h_kv must be 1.
 */
int mla_decode_metadata(const int32_t* seqlens_d, int batch, int s_q, int h_q,
                        int h_kv, int block_size, int num_parts,
                        int32_t* tile_meta_d, int32_t* split_offsets_d,
                        void* stream);

/*
 * mla_decode_splitkv — enqueue the main decode kernel only.
 * Passage: page "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA: the MLA
 * terminology paragraph (one shared latent head), feature ② (64-token
 * pages), feature ④ (scores, then probabilities times values) and feature ⑤
 * (a long request's keys split over several workers).
 * For every part and row tile: gathers the part's pages through the block
 * table into LDS, computes scores (bf16 MFMA, fp32 accumulate), the online
 * softmax in fp32, and probabilities times values (bf16 MFMA).  A request
 * covered by one part is written to out_d / lse_d directly; pieces of split
 * requests are written as bf16 partials into the workspace, to be merged by
 * mla_decode_combine.
 *   q_d           bf16 [batch, s_q, h_q, 576]
 *   kcache_d      bf16 [num_blocks, 64, h_kv=1, 576]
 *   block_table_d int32 [batch, bt_stride]
 *   seqlens_d     int32 [batch]  (tokens in the cache, incl. the s_q new ones)
 *   scale         softmax scale multiplying q.k (finite)
 *   causal        0/1: with causal, query token t sees L - s_q + 1 + t keys
 *   tile_meta_d, split_offsets_d, num_parts: output of mla_decode_metadata
 *                 for the same seqlens/s_q/h_q/num_parts
 *   workspace_d   >= mla_decode_workspace_bytes(batch, s_q, h_q, num_parts)
 *   out_d         bf16 [batch, s_q, h_q, 512]
 *   lse_d         fp32 [batch, s_q, h_q]
 */
int mla_decode_splitkv(const void* q_d, const void* kcache_d, int64_t num_blocks,
                       const int32_t* block_table_d, int bt_stride,
                       const int32_t* seqlens_d, int batch, int s_q, int h_q,
                       int h_kv, float scale, int causal,
                       const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                       int num_parts, void* workspace_d, size_t workspace_bytes,
                       void* out_d, float* lse_d, void* stream);

/*
 * mla_decode_splitkv_timed — mla_decode_splitkv, and in addition the two
 * caller-created HIP events (hipEvent_t, timing enabled; either may be NULL)
 * are recorded at the decode kernel's own start and end (hipExtLaunchKernel),
 * so their elapsed time is the kernel's duration without the launch and
 * marker-packet overhead that separately recorded events include.  Same
 * arguments, validation and status codes as mla_decode_splitkv.
 */
int mla_decode_splitkv_timed(const void* q_d, const void* kcache_d, int64_t num_blocks,
                             const int32_t* block_table_d, int bt_stride,
                             const int32_t* seqlens_d, int batch, int s_q, int h_q,
                             int h_kv, float scale, int causal,
                             const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                             int num_parts, void* workspace_d, size_t workspace_bytes,
                             void* out_d, float* lse_d, void* start_event,
                             void* stop_event, void* stream);

/*
 * mla_decode_combine — enqueue the log-sum-exp merge of split partials.
 * Passage: page "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA, feature ⑤
 * (the pieces of a split request merged into one result).
 * For every request with split_offsets[b+1] > split_offsets[b]:
 *   LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) * O_i  (exact merge),
 * written to out_d (bf16) / lse_d.  Requests with seqlens[b] <= 0 get O = 0,
 * LSE = -inf.  Other rows are left untouched.  Arguments as in
 * mla_decode_splitkv.
 */
int mla_decode_combine(const int32_t* seqlens_d, int batch, int s_q, int h_q,
                       const int32_t* split_offsets_d, int num_parts,
                       const void* workspace_d, size_t workspace_bytes,
                       void* out_d, float* lse_d, void* stream);

/*
 * mla_decode_fwd — mla_decode_splitkv followed by mla_decode_combine on the
 * same stream: the whole decode attention for one batch (page
 * "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA: the operation defined at the
 * top of this file).
 */
int mla_decode_fwd(const void* q_d, const void* kcache_d, int64_t num_blocks,
                   const int32_t* block_table_d, int bt_stride,
                   const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                   float scale, int causal,
                   const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                   int num_parts, void* workspace_d, size_t workspace_bytes,
                   void* out_d, float* lse_d, void* stream);

/*
 * mla_kv_append — enqueue the write of the s_q new tokens' key rows into the
 * paged cache, the step that precedes decode.  Paging as for decode (page
 * "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA, feature ②: 64-token blocks):
 * token j of request b is row j % 64 of page block_table[b][j / 64].  The
 * lengths already count the new tokens, so new token t of request b is token
 * seqlens[b] - s_q + t; positions before 0, page slots at or beyond
 * bt_stride and page ids outside [0, num_blocks) are skipped (never written).
 *   new_kv_d      bf16 [batch, s_q, 576] (16-byte aligned), read only
 *   kcache_d      bf16 [num_blocks, 64, 1, 576] (16-byte aligned), written
 *   block_table_d int32 [batch, bt_stride]; seqlens_d int32 [batch]
 * 1 <= s_q <= MLA_MAX_S_Q.  Rows written by two requests (shared pages) get
 * one of the writes.  Returns MLA_OK or an error status; nothing is enqueued
 * on error.
 */
int mla_kv_append(const void* new_kv_d, void* kcache_d, int64_t num_blocks,
                  const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                  int batch, int s_q, void* stream);

/*
 * FP8 key cache.  Page "云上玩转DeepSeek系列之五：实测优化16%，体验FlashMLA加速
 * DeepSeek-V2-Lite推理" (ruibaoantu.com), section 四, item 2 (monitoring and
 * tuning), names FP8 precision as a further throughput step and gives no
 * format; this library's format keeps the attention defined above and stores
 * the 512 latent dims as OCP FP8 E4M3 codes with one fp32 scale per token,
 * the 64 rope dims in bf16.  One page of 64 tokens is MLA_FP8_PAGE_BYTES:
 *   [0, 32768)      codes uint8 [64][512]   E4M3 codes of latent dims 0..511
 *   [32768, 40960)  rope  bf16  [64][64]    dims 512..575
 *   [40960, 41216)  scale fp32  [64]        latent value = e4m3(code) * scale
 * E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0,
 * exponent 0 = subnormals m * 2^-9, S.1111.111 = NaN, no infinities, largest
 * finite 448.  The decode kernels accept any finite scale; mla_kv_append_fp8
 * writes power-of-two scales.
 */
#define MLA_FP8_PAGE_BYTES 41216
#define MLA_FP8_ROPE_OFFSET 32768
#define MLA_FP8_SCALE_OFFSET 40960

/*
 * mla_decode_splitkv_fp8 — mla_decode_splitkv over an FP8 cache:
 *   kcache_fp8_d  uint8 [num_blocks, MLA_FP8_PAGE_BYTES] (16-byte aligned)
 * The keys are K[j, 0:512] = e4m3(code) * scale, K[j, 512:576] = rope; the
 * products run on bf16 MFMA with fp32 accumulation (codes convert to bf16
 * exactly; the per-token scale multiplies the fp32 score sum and, for the
 * value product, the probability before its bf16 rounding).  start_event /
 * stop_event as in mla_decode_splitkv_timed (both may be NULL).  All other
 * arguments, validation and status codes as mla_decode_splitkv; the partials
 * go to the same workspace and are merged by mla_decode_combine.
 */
int mla_decode_splitkv_fp8(const void* q_d, const void* kcache_fp8_d, int64_t num_blocks,
                           const int32_t* block_table_d, int bt_stride,
                           const int32_t* seqlens_d, int batch, int s_q, int h_q,
                           int h_kv, float scale, int causal,
                           const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                           int num_parts, void* workspace_d, size_t workspace_bytes,
                           void* out_d, float* lse_d, void* start_event,
                           void* stop_event, void* stream);

/*
 * mla_decode_fwd_fp8 — mla_decode_splitkv_fp8 followed by mla_decode_combine
 * on the same stream.
 */
int mla_decode_fwd_fp8(const void* q_d, const void* kcache_fp8_d, int64_t num_blocks,
                       const int32_t* block_table_d, int bt_stride,
                       const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                       float scale, int causal,
                       const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                       int num_parts, void* workspace_d, size_t workspace_bytes,
                       void* out_d, float* lse_d, void* stream);

/*
 * mla_kv_append_fp8 — mla_kv_append into an FP8 cache.  Each new bf16 row x
 * (new_kv_d bf16 [batch, s_q, 576]) is quantised: amax = max |x[0:512]|, the
 * scale s is the smallest power of two with amax <= 448*s (1 if amax = 0),
 * code_d = E4M3 round-to-nearest-even of x_d / s (exact division, no
 * saturation needed); the rope dims are copied bit for bit and s is stored
 * as fp32.  Positions, skipping rules, arguments and status codes as
 * mla_kv_append; kcache_fp8_d uint8 [num_blocks, MLA_FP8_PAGE_BYTES].
 */
int mla_kv_append_fp8(const void* new_kv_d, void* kcache_fp8_d, int64_t num_blocks,
                      const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                      int batch, int s_q, void* stream);

/*
 * mla_decode_fwd_inline_plan — the whole decode in two launches instead of
 * three: the decode kernel derives its split plan itself (every workgroup
 * computes its part from seqlens with the rule of mla_decode_metadata; page
 * "深度剖析DeepSeek Infra开源全貌", DAY1 FlashMLA, feature ⑤: the dynamic load
 * split for variable lengths), then mla_decode_combine merges the pieces.
 * Arguments as mla_decode_fwd, except that tile_meta_d (int32 [num_parts, 8])
 * and split_offsets_d (int32 [batch + 1]) are OUTPUTS: the kernel writes the
 * same plan mla_decode_metadata would (the combine reads split_offsets_d
 * from it).  start_event / stop_event (may be NULL) as in
 * mla_decode_splitkv_timed.  num_parts from mla_decode_num_parts; batch at
 * most 1024 (MLA_ERR_UNSUPPORTED above: use the three-launch path); other
 * validation and status codes as mla_decode_fwd.
 */
int mla_decode_fwd_inline_plan(const void* q_d, const void* kcache_d, int64_t num_blocks,
                               const int32_t* block_table_d, int bt_stride,
                               const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                               float scale, int causal, int32_t* tile_meta_d,
                               int32_t* split_offsets_d, int num_parts, void* workspace_d,
                               size_t workspace_bytes, void* out_d, float* lse_d,
                               void* start_event, void* stop_event, void* stream);

/* mla_decode_fwd_inline_plan over an FP8 cache (the pages of mla_decode_splitkv_fp8). */
int mla_decode_fwd_inline_plan_fp8(const void* q_d, const void* kcache_fp8_d,
                                   int64_t num_blocks, const int32_t* block_table_d,
                                   int bt_stride, const int32_t* seqlens_d, int batch, int s_q,
                                   int h_q, int h_kv, float scale, int causal,
                                   int32_t* tile_meta_d, int32_t* split_offsets_d,
                                   int num_parts, void* workspace_d, size_t workspace_bytes,
                                   void* out_d, float* lse_d, void* start_event,
                                   void* stop_event, void* stream);

/*
 * Sparse (selected-keys) mode.  Page "云上玩转DeepSeek系列之五：实测
 * 优化16%，体验FlashMLA加速DeepSeek-V2-Lite推理" (ruibaoantu.com), section 四,
 * item 2, recommends FlashMLA's sparse attention mode beyond 8K tokens and
 * gives no algorithm; this library's reading: the caller selects, for every
 * query token, topk cache positions (any top-k selector; selection is not
 * part of the mode), and each head of that token attends exactly over them:
 *   indices_d int32 [batch, s_q, topk]: logical positions j in request b;
 *   an entry counts iff 0 <= j < vis(b, t) (the dense visible limit:
 *   L_b - s_q + 1 + t when causal, else L_b) and its page slot and page id
 *   are valid; counted entries form a multiset (a position listed twice
 *   counts twice); O and LSE as in the dense definition over the counted
 *   entries; none counted gives O = 0, LSE = -inf.
 * Work is split over (request, token) items of topk entries each:
 *   - parts: mla_decode_num_parts(batch * s_q, 1, h_q, 1, num_cus, ...)
 *   - workspace: mla_decode_sparse_workspace_bytes (partials as for
 *     mla_decode_workspace_bytes(batch*s_q, 1, h_q, num_parts), then the
 *     resolved row ids, validity bits and a zero row)
 *   - metadata: mla_decode_sparse_metadata (device, no host sync)
 * Constraints: topk a multiple of 32 in [32, 2^20]; batch*s_q*topk < 2^31;
 * num_blocks <= 2^25 (row ids are int32).
 */
int mla_decode_sparse_workspace_bytes(int batch, int s_q, int h_q, int topk, int num_parts,
                                      size_t* bytes_out);

int mla_decode_sparse_metadata(int batch, int s_q, int h_q, int topk, int num_parts,
                               int32_t* tile_meta_d, int32_t* split_offsets_d, void* stream);

/*
 * mla_decode_sparse_fwd — enqueue the sparse-mode decode: resolution of the
 * selected positions to cache rows, the split-KV kernel over the items
 * (rows gathered one by one into LDS, bf16 MFMA, fp32 online softmax) and the
 * combine.  Arguments as mla_decode_fwd plus indices_d / topk; tile_meta_d,
 * split_offsets_d and num_parts from mla_decode_sparse_metadata; workspace_d
 * 256-byte aligned, >= mla_decode_sparse_workspace_bytes.  start_event /
 * stop_event (hipEvent_t, may be NULL) are recorded at the decode kernel's
 * own start and end.
 */
int mla_decode_sparse_fwd(const void* q_d, const void* kcache_d, int64_t num_blocks,
                          const int32_t* block_table_d, int bt_stride,
                          const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                          float scale, int causal, const int32_t* indices_d, int topk,
                          const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                          int num_parts, void* workspace_d, size_t workspace_bytes,
                          void* out_d, float* lse_d, void* start_event, void* stop_event,
                          void* stream);

/*
 * mla_decode_sparse_fwd_fp8 — the sparse mode over an FP8 cache: kcache_d
 * an array of num_blocks FP8 pages (MLA_FP8_PAGE_BYTES each, the layout of
 * mla_decode_splitkv_fp8), every other argument, the workspace, metadata
 * and outputs as mla_decode_sparse_fwd.  A selected row is used exactly as
 * the dense FP8 path uses it (latent = e4m3(code) * scale, rope bf16);
 * its three fields are gathered row by row (codes, rope, scale).  Same
 * errors and constraints as mla_decode_sparse_fwd.
 */
int mla_decode_sparse_fwd_fp8(const void* q_d, const void* kcache_d, int64_t num_blocks,
                              const int32_t* block_table_d, int bt_stride,
                              const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                              float scale, int causal, const int32_t* indices_d, int topk,
                              const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                              int num_parts, void* workspace_d, size_t workspace_bytes,
                              void* out_d, float* lse_d, void* start_event, void* stop_event,
                              void* stream);

/*
 * mla_decode_fwd_noalloc — the whole decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It runs mla_decode_metadata, mla_decode_splitkv and
 * mla_decode_combine on `stream` with the plan (tile_meta, split_offsets) and
 * the split partials in one device array that the library holds for the life
 * of the process, MLA_NOALLOC_SCRATCH_BYTES per device, instead of caller
 * buffers; it allocates and frees nothing and calls no allocating routine.
 *   Arguments as mla_decode_fwd without tile_meta_d / split_offsets_d /
 *   num_parts / workspace_d / workspace_bytes; the caller still owns q, the
 *   cache, the table, the lengths and the outputs.  The stream must belong to
 *   the current device.
 *   Parts: mla_decode_num_parts for the current device, halved until the
 *   partials (mla_decode_workspace_bytes) fit in the array; results equal
 *   mla_decode_fwd's with that part count.
 *   batch above MLA_NOALLOC_MAX_BATCH returns MLA_ERR_INVALID_ARG; every other
 *   check and status code as mla_decode_fwd; nothing is enqueued on error.
 * All calls on one device share its array, which keeps the last call's
 * contents: two calls that overlap on one device (concurrent streams or host
 * threads) race and must be serialised by the caller.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
#define MLA_NOALLOC_MAX_BATCH 16384
int mla_decode_fwd_noalloc(const void* q_d, const void* kcache_d, int64_t num_blocks,
                           const int32_t* block_table_d, int bt_stride,
                           const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                           float scale, int causal, void* out_d, float* lse_d, void* stream);

/* Static text for a status code. */
const char* mla_status_string(int status);

/* Text of the last HIP error seen by this thread in the library ("" if none). */
const char* mla_last_hip_error(void);

/* Number of compute units of `device` (a HIP call). */
int mla_device_num_cus(int device, int* num_cus_out);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
