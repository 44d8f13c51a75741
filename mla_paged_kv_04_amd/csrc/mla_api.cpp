// Host side of the C ABI declared in include/mla_decode.h: argument
// validation, workspace sizing and kernel launches.  No allocation, no global
// mutable state except a thread-local error text, and no host synchronisation
// outside the checked mode (MLA_DEBUG_SYNC, below).
#include "../../include/mla_decode.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla_kernels.h"

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s", where, hipGetErrorString(e));
  return MLA_ERR_HIP;
}

// Checked mode: with MLA_DEBUG_SYNC set to anything but "" or "0" in the
// environment (read at every call), each launch is followed by a wait on its
// stream, so that a kernel fault is reported by the call that launched it, as
// MLA_ERR_HIP with that launch named in mla_last_hip_error().  A stream under
// graph capture is not waited on (the launch is only recorded there).
bool debug_sync() {
  const char* v = getenv("MLA_DEBUG_SYNC");
  return v != nullptr && v[0] != 0 && strcmp(v, "0") != 0;
}

// Status of a launch that returned `e` on `stream`.
int launched(hipError_t e, hipStream_t stream, const char* where) {
  if (e != hipSuccess) return hip_fail(e, where);
  if (!debug_sync()) return MLA_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, where);
  if (cs != hipStreamCaptureStatusNone) return MLA_OK;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, where);
  return MLA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_h_q(int h_q) { return h_q == 16 || h_q == 32 || h_q == 64 || h_q == 128; }

int check_shape(int batch, int s_q, int h_q, int h_kv) {
  if (batch < 1 || s_q < 1 || s_q > MLA_MAX_S_Q || h_kv != 1 || h_q < 1) return MLA_ERR_INVALID_ARG;
  if (!supported_h_q(h_q)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

constexpr int kMaxParts = 1 << 16;

int row_tiles(int s_q, int h_q) {
  const int M = s_q * h_q;
  const int t = mla::tile_rows_for(M);
  return (M + t - 1) / t;
}

size_t workspace_need(int s_q, int h_q, int num_parts) {
  const size_t slots = num_parts > 1 ? 2 * (size_t)(num_parts - 1) : 0;
  const size_t M = (size_t)s_q * h_q;
  size_t bytes = slots * M * (mla::kDV * sizeof(uint16_t) + sizeof(float));
  return (bytes + 255) / 256 * 256;
}

// Partial O (bf16) lives first, partial LSE (fp32) after it.
void split_workspace(void* ws, int s_q, int h_q, int num_parts, uint16_t** po, float** plse) {
  const size_t slots = num_parts > 1 ? 2 * (size_t)(num_parts - 1) : 0;
  const size_t M = (size_t)s_q * h_q;
  *po = static_cast<uint16_t*>(ws);
  *plse = ws ? reinterpret_cast<float*>(static_cast<uint16_t*>(ws) + slots * M * mla::kDV) : nullptr;
}

int check_common(const void* seqlens, const void* split_offsets, int batch, int s_q, int h_q,
                 int h_kv, int num_parts, const void* workspace, size_t workspace_bytes,
                 const void* out, const float* lse) {
  int st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_OK) return st;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  if (!seqlens || !split_offsets || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned(seqlens, 4) || !aligned(split_offsets, 4) || !aligned(lse, 4) ||
      !aligned(out, 16))
    return MLA_ERR_INVALID_ARG;
  const size_t need = workspace_need(s_q, h_q, num_parts);
  if (need > 0) {
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!workspace || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARG;
  }
  return MLA_OK;
}

// Validation and launch of the decode kernel for either cache format.
int splitkv_impl(const void* q_d, const void* kcache_d, int64_t num_blocks,
                 const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                 int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                 const int32_t* tile_meta_d, const int32_t* split_offsets_d, int num_parts,
                 void* workspace_d, size_t workspace_bytes, void* out_d, float* lse_d,
                 int kv_fp8, void* start_event, void* stop_event, void* stream,
                 int inplan = 0, int dry_run = 0) {
  int st = check_common(seqlens_d, split_offsets_d, batch, s_q, h_q, h_kv, num_parts,
                        workspace_d, workspace_bytes, out_d, lse_d);
  if (st != MLA_OK) return st;
  if (!q_d || !kcache_d || !block_table_d || !tile_meta_d) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_d, 16) || !aligned(kcache_d, 16) || !aligned(block_table_d, 4) ||
      !aligned(tile_meta_d, 4))
    return MLA_ERR_INVALID_ARG;
  if (num_blocks < 1 || bt_stride < 1 || !isfinite(scale) || (causal != 0 && causal != 1))
    return MLA_ERR_INVALID_ARG;
  if (dry_run) return MLA_OK;
  mla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q_d);
  a.kcache = kcache_d;
  a.num_blocks = num_blocks;
  a.block_table = block_table_d;
  a.seqlens = seqlens_d;
  a.tile_meta = tile_meta_d;
  a.split_offsets = split_offsets_d;
  split_workspace(workspace_d, s_q, h_q, num_parts, &a.part_o, &a.part_lse);
  a.out = static_cast<uint16_t*>(out_d);
  a.lse = lse_d;
  a.bt_stride = bt_stride;
  a.batch = batch;
  a.s_q = s_q;
  a.h_q = h_q;
  a.M = s_q * h_q;
  a.causal = causal;
  a.num_parts = num_parts;
  a.row_tiles = row_tiles(s_q, h_q);
  a.row_tile_rows = mla::tile_rows_for(s_q * h_q);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kv_fp8 = kv_fp8;
  a.sparse = 0;
  a.const_len = 0;
  a.rowids = nullptr;
  a.vmask = nullptr;
  a.zero_row = nullptr;
  a.inplan = inplan;
  a.c_fix = mla::fixed_cost_pages(mla::rows_per_tile(s_q, h_q));
  a.tile_meta_out = const_cast<int32_t*>(tile_meta_d);
  a.split_offsets_out = const_cast<int32_t*>(split_offsets_d);
  hipError_t e = mla::launch_splitkv(a, static_cast<hipStream_t>(stream),
                                     static_cast<hipEvent_t>(start_event),
                                     static_cast<hipEvent_t>(stop_event));
  return launched(e, static_cast<hipStream_t>(stream), "mla_decode_splitkv launch");
}

int check_append(const void* new_kv_d, void* kcache_d, int64_t num_blocks,
                 const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                 int batch, int s_q) {
  if (batch < 1 || s_q < 1 || s_q > MLA_MAX_S_Q || num_blocks < 1 || bt_stride < 1)
    return MLA_ERR_INVALID_ARG;
  if (!new_kv_d || !kcache_d || !block_table_d || !seqlens_d) return MLA_ERR_INVALID_ARG;
  if (!aligned(new_kv_d, 16) || !aligned(kcache_d, 16) || !aligned(block_table_d, 4) ||
      !aligned(seqlens_d, 4))
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// Sparse mode: items = batch * s_q (request, token) pairs of topk entries.
constexpr int kMaxTopk = 1 << 20;

int check_sparse_shape(int batch, int s_q, int h_q, int h_kv, int topk) {
  int st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_OK) return st;
  if (topk < 32 || topk > kMaxTopk || topk % 32 != 0) return MLA_ERR_INVALID_ARG;
  if ((long long)batch * s_q * (long long)topk > (1LL << 31) - 1) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct SparseWorkspace {
  size_t partial, rowids, vmask, zero_row, total;   // byte offsets and total size
};

SparseWorkspace sparse_workspace(int batch, int s_q, int h_q, int topk, int num_parts) {
  const size_t items = (size_t)batch * s_q;
  SparseWorkspace w;
  w.partial = 0;
  w.rowids = workspace_need(1, h_q, num_parts);
  w.vmask = w.rowids + round256(items * topk * 4);
  w.zero_row = w.vmask + round256(items * (topk / 32) * 4);
  w.total = w.zero_row + round256(mla::kRowBytes);
  return w;
}

}  // namespace

namespace mla {

int set_hip_error(hipError_t e, const char* where) { return hip_fail(e, where); }

int validate_decode(const void* q_d, const void* kcache_d, int64_t num_blocks,
                    const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                    int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                    const int32_t* tile_meta_d, const int32_t* split_offsets_d, int num_parts,
                    void* workspace_d, size_t workspace_bytes, void* out_d, float* lse_d) {
  return splitkv_impl(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                      s_q, h_q, h_kv, scale, causal, tile_meta_d, split_offsets_d, num_parts,
                      workspace_d, workspace_bytes, out_d, lse_d, 0, nullptr, nullptr, nullptr,
                      0, 1);
}

size_t decode_workspace_need(int s_q, int h_q, int num_parts) {
  return workspace_need(s_q, h_q, num_parts);
}

int decode_row_tiles(int s_q, int h_q) { return row_tiles(s_q, h_q); }

}  // namespace mla

extern "C" {

int mla_decode_num_parts(int batch, int s_q, int h_q, int h_kv, int num_cus,
                         int* num_parts_out) {
  if (!num_parts_out || num_cus < 1) return MLA_ERR_INVALID_ARG;
  int st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_OK) return st;
  int p = num_cus / row_tiles(s_q, h_q);
  if (p < 1) p = 1;
  if (p > kMaxParts) p = kMaxParts;
  *num_parts_out = p;
  return MLA_OK;
}

int mla_decode_workspace_bytes(int batch, int s_q, int h_q, int num_parts, size_t* bytes_out) {
  if (!bytes_out) return MLA_ERR_INVALID_ARG;
  int st = check_shape(batch, s_q, h_q, 1);
  if (st != MLA_OK) return st;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  *bytes_out = workspace_need(s_q, h_q, num_parts);
  return MLA_OK;
}

int mla_decode_metadata(const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                        int block_size, int num_parts, int32_t* tile_meta_d,
                        int32_t* split_offsets_d, void* stream) {
  int st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_OK) return st;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_INVALID_ARG;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  if (!seqlens_d || !tile_meta_d || !split_offsets_d) return MLA_ERR_INVALID_ARG;
  if (!aligned(seqlens_d, 4) || !aligned(tile_meta_d, 4) || !aligned(split_offsets_d, 4))
    return MLA_ERR_INVALID_ARG;
  const int c = mla::fixed_cost_pages(mla::rows_per_tile(s_q, h_q));
  hipError_t e = mla::launch_metadata(seqlens_d, batch, c, num_parts, tile_meta_d,
                                      split_offsets_d, static_cast<hipStream_t>(stream));
  return launched(e, static_cast<hipStream_t>(stream), "mla_decode_metadata launch");
}

int mla_decode_splitkv_timed(const void* q_d, const void* kcache_d, int64_t num_blocks,
                             const int32_t* block_table_d, int bt_stride,
                             const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                             float scale, int causal, const int32_t* tile_meta_d,
                             const int32_t* split_offsets_d, int num_parts, void* workspace_d,
                             size_t workspace_bytes, void* out_d, float* lse_d,
                             void* start_event, void* stop_event, void* stream) {
  return splitkv_impl(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                      s_q, h_q, h_kv, scale, causal, tile_meta_d, split_offsets_d, num_parts,
                      workspace_d, workspace_bytes, out_d, lse_d, 0, start_event, stop_event,
                      stream);
}

int mla_decode_splitkv_fp8(const void* q_d, const void* kcache_fp8_d, int64_t num_blocks,
                           const int32_t* block_table_d, int bt_stride,
                           const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                           float scale, int causal, const int32_t* tile_meta_d,
                           const int32_t* split_offsets_d, int num_parts, void* workspace_d,
                           size_t workspace_bytes, void* out_d, float* lse_d,
                           void* start_event, void* stop_event, void* stream) {
  return splitkv_impl(q_d, kcache_fp8_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                      s_q, h_q, h_kv, scale, causal, tile_meta_d, split_offsets_d, num_parts,
                      workspace_d, workspace_bytes, out_d, lse_d, 1, start_event, stop_event,
                      stream);
}

int mla_decode_splitkv(const void* q_d, const void* kcache_d, int64_t num_blocks,
                       const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                       int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                       const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                       int num_parts, void* workspace_d, size_t workspace_bytes, void* out_d,
                       float* lse_d, void* stream) {
  return mla_decode_splitkv_timed(q_d, kcache_d, num_blocks, block_table_d, bt_stride,
                                  seqlens_d, batch, s_q, h_q, h_kv, scale, causal, tile_meta_d,
                                  split_offsets_d, num_parts, workspace_d, workspace_bytes,
                                  out_d, lse_d, nullptr, nullptr, stream);
}

int mla_decode_combine(const int32_t* seqlens_d, int batch, int s_q, int h_q,
                       const int32_t* split_offsets_d, int num_parts, const void* workspace_d,
                       size_t workspace_bytes, void* out_d, float* lse_d, void* stream) {
  int st = check_common(seqlens_d, split_offsets_d, batch, s_q, h_q, 1, num_parts, workspace_d,
                        workspace_bytes, out_d, lse_d);
  if (st != MLA_OK) return st;
  mla::CombineArgs a;
  uint16_t* po;
  float* plse;
  split_workspace(const_cast<void*>(workspace_d), s_q, h_q, num_parts, &po, &plse);
  a.seqlens = seqlens_d;
  a.split_offsets = split_offsets_d;
  a.part_o = po;
  a.part_lse = plse;
  a.out = static_cast<uint16_t*>(out_d);
  a.lse = lse_d;
  a.batch = batch;
  a.M = s_q * h_q;
  a.const_len = 0;
  hipError_t e = mla::launch_combine(a, static_cast<hipStream_t>(stream));
  return launched(e, static_cast<hipStream_t>(stream), "mla_decode_combine launch");
}

int mla_decode_fwd(const void* q_d, const void* kcache_d, int64_t num_blocks,
                   const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                   int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                   const int32_t* tile_meta_d, const int32_t* split_offsets_d, int num_parts,
                   void* workspace_d, size_t workspace_bytes, void* out_d, float* lse_d,
                   void* stream) {
  int st = mla_decode_splitkv(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d,
                              batch, s_q, h_q, h_kv, scale, causal, tile_meta_d,
                              split_offsets_d, num_parts, workspace_d, workspace_bytes, out_d,
                              lse_d, stream);
  if (st != MLA_OK) return st;
  return mla_decode_combine(seqlens_d, batch, s_q, h_q, split_offsets_d, num_parts,
                            workspace_d, workspace_bytes, out_d, lse_d, stream);
}

int mla_decode_fwd_fp8(const void* q_d, const void* kcache_fp8_d, int64_t num_blocks,
                       const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                       int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                       const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                       int num_parts, void* workspace_d, size_t workspace_bytes, void* out_d,
                       float* lse_d, void* stream) {
  int st = mla_decode_splitkv_fp8(q_d, kcache_fp8_d, num_blocks, block_table_d, bt_stride,
                                  seqlens_d, batch, s_q, h_q, h_kv, scale, causal, tile_meta_d,
                                  split_offsets_d, num_parts, workspace_d, workspace_bytes,
                                  out_d, lse_d, nullptr, nullptr, stream);
  if (st != MLA_OK) return st;
  return mla_decode_combine(seqlens_d, batch, s_q, h_q, split_offsets_d, num_parts,
                            workspace_d, workspace_bytes, out_d, lse_d, stream);
}

int mla_decode_fwd_inline_plan(const void* q_d, const void* kcache_d, int64_t num_blocks,
                               const int32_t* block_table_d, int bt_stride,
                               const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                               float scale, int causal, int32_t* tile_meta_d,
                               int32_t* split_offsets_d, int num_parts, void* workspace_d,
                               size_t workspace_bytes, void* out_d, float* lse_d,
                               void* start_event, void* stop_event, void* stream) {
  if (batch > mla::kPlanMaxBatch) return MLA_ERR_UNSUPPORTED;
  int st = splitkv_impl(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                        s_q, h_q, h_kv, scale, causal, tile_meta_d, split_offsets_d, num_parts,
                        workspace_d, workspace_bytes, out_d, lse_d, 0, start_event, stop_event,
                        stream, 1);
  if (st != MLA_OK) return st;
  return mla_decode_combine(seqlens_d, batch, s_q, h_q, split_offsets_d, num_parts,
                            workspace_d, workspace_bytes, out_d, lse_d, stream);
}

int mla_decode_fwd_inline_plan_fp8(const void* q_d, const void* kcache_fp8_d,
                                   int64_t num_blocks, const int32_t* block_table_d,
                                   int bt_stride, const int32_t* seqlens_d, int batch, int s_q,
                                   int h_q, int h_kv, float scale, int causal,
                                   int32_t* tile_meta_d, int32_t* split_offsets_d,
                                   int num_parts, void* workspace_d, size_t workspace_bytes,
                                   void* out_d, float* lse_d, void* start_event,
                                   void* stop_event, void* stream) {
  if (batch > mla::kPlanMaxBatch) return MLA_ERR_UNSUPPORTED;
  int st = splitkv_impl(q_d, kcache_fp8_d, num_blocks, block_table_d, bt_stride, seqlens_d,
                        batch, s_q, h_q, h_kv, scale, causal, tile_meta_d, split_offsets_d,
                        num_parts, workspace_d, workspace_bytes, out_d, lse_d, 1, start_event,
                        stop_event, stream, 1);
  if (st != MLA_OK) return st;
  return mla_decode_combine(seqlens_d, batch, s_q, h_q, split_offsets_d, num_parts,
                            workspace_d, workspace_bytes, out_d, lse_d, stream);
}

int mla_kv_append(const void* new_kv_d, void* kcache_d, int64_t num_blocks,
                  const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                  int batch, int s_q, void* stream) {
  int st = check_append(new_kv_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d,
                        batch, s_q);
  if (st != MLA_OK) return st;
  hipError_t e = mla::launch_kv_append(static_cast<const uint16_t*>(new_kv_d),
                                       static_cast<uint16_t*>(kcache_d), num_blocks,
                                       block_table_d, bt_stride, seqlens_d, batch, s_q,
                                       static_cast<hipStream_t>(stream));
  return launched(e, static_cast<hipStream_t>(stream), "mla_kv_append launch");
}

int mla_kv_append_fp8(const void* new_kv_d, void* kcache_fp8_d, int64_t num_blocks,
                      const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                      int batch, int s_q, void* stream) {
  int st = check_append(new_kv_d, kcache_fp8_d, num_blocks, block_table_d, bt_stride, seqlens_d,
                        batch, s_q);
  if (st != MLA_OK) return st;
  hipError_t e = mla::launch_kv_append_fp8(static_cast<const uint16_t*>(new_kv_d),
                                           static_cast<uint8_t*>(kcache_fp8_d), num_blocks,
                                           block_table_d, bt_stride, seqlens_d, batch, s_q,
                                           static_cast<hipStream_t>(stream));
  return launched(e, static_cast<hipStream_t>(stream), "mla_kv_append_fp8 launch");
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported shape (h_q must be 16, 32, 64 or 128)";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* mla_last_hip_error(void) { return g_last_hip_error; }

int mla_device_num_cus(int device, int* num_cus_out) {
  if (!num_cus_out || device < 0) return MLA_ERR_INVALID_ARG;
  int v = 0;
  hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  *num_cus_out = v;
  return MLA_OK;
}

int mla_decode_sparse_workspace_bytes(int batch, int s_q, int h_q, int topk, int num_parts,
                                      size_t* bytes_out) {
  if (!bytes_out) return MLA_ERR_INVALID_ARG;
  int st = check_sparse_shape(batch, s_q, h_q, 1, topk);
  if (st != MLA_OK) return st;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  *bytes_out = sparse_workspace(batch, s_q, h_q, topk, num_parts).total;
  return MLA_OK;
}

int mla_decode_sparse_metadata(int batch, int s_q, int h_q, int topk, int num_parts,
                               int32_t* tile_meta_d, int32_t* split_offsets_d, void* stream) {
  int st = check_sparse_shape(batch, s_q, h_q, 1, topk);
  if (st != MLA_OK) return st;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  if (!tile_meta_d || !split_offsets_d || !aligned(tile_meta_d, 4) || !aligned(split_offsets_d, 4))
    return MLA_ERR_INVALID_ARG;
  const int c = mla::fixed_cost_pages(mla::rows_per_tile(1, h_q));
  hipError_t e = mla::launch_metadata(nullptr, batch * s_q, c, num_parts, tile_meta_d,
                                      split_offsets_d, static_cast<hipStream_t>(stream), topk);
  return launched(e, static_cast<hipStream_t>(stream), "mla_decode_sparse_metadata launch");
}

}  // extern "C"

namespace {

int sparse_fwd_impl(const void* q_d, const void* kcache_d, int64_t num_blocks,
                    const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                    int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                    const int32_t* indices_d, int topk, const int32_t* tile_meta_d,
                    const int32_t* split_offsets_d, int num_parts, void* workspace_d,
                    size_t workspace_bytes, void* out_d, float* lse_d, void* start_event,
                    void* stop_event, void* stream, int kv_fp8) {
  int st = check_sparse_shape(batch, s_q, h_q, h_kv, topk);
  if (st != MLA_OK) return st;
  if (num_parts < 1 || num_parts > kMaxParts) return MLA_ERR_INVALID_ARG;
  if (!q_d || !kcache_d || !block_table_d || !seqlens_d || !indices_d || !tile_meta_d ||
      !split_offsets_d || !out_d || !lse_d || !workspace_d)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_d, 16) || !aligned(kcache_d, 16) || !aligned(out_d, 16) ||
      !aligned(block_table_d, 4) || !aligned(seqlens_d, 4) || !aligned(indices_d, 4) ||
      !aligned(tile_meta_d, 4) || !aligned(split_offsets_d, 4) || !aligned(lse_d, 4) ||
      !aligned(workspace_d, 256))
    return MLA_ERR_INVALID_ARG;
  if (num_blocks < 1 || num_blocks > (1LL << 25) || bt_stride < 1 || !isfinite(scale) ||
      (causal != 0 && causal != 1))
    return MLA_ERR_INVALID_ARG;
  const SparseWorkspace w = sparse_workspace(batch, s_q, h_q, topk, num_parts);
  if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace_d);
  int32_t* rowids = reinterpret_cast<int32_t*>(ws + w.rowids);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(ws + w.vmask);
  void* zero_row = ws + w.zero_row;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_sparse_resolve(indices_d, block_table_d, bt_stride, seqlens_d,
                                            num_blocks, batch, s_q, topk, causal, rowids, vmask,
                                            zero_row, s);
  st = launched(e, s, "mla_decode_sparse_fwd resolve launch");
  if (st != MLA_OK) return st;
  const int items = batch * s_q;
  mla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q_d);
  a.kcache = kcache_d;
  a.num_blocks = num_blocks;
  a.block_table = block_table_d;
  a.seqlens = seqlens_d;
  a.tile_meta = tile_meta_d;
  a.split_offsets = split_offsets_d;
  split_workspace(workspace_d, 1, h_q, num_parts, &a.part_o, &a.part_lse);
  a.out = static_cast<uint16_t*>(out_d);
  a.lse = lse_d;
  a.bt_stride = bt_stride;
  a.batch = items;
  a.s_q = 1;
  a.h_q = h_q;
  a.M = h_q;
  a.causal = 0;
  a.num_parts = num_parts;
  a.row_tiles = row_tiles(1, h_q);
  a.row_tile_rows = mla::tile_rows_for(h_q);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kv_fp8 = kv_fp8;
  a.sparse = 1;
  a.const_len = topk;
  a.rowids = rowids;
  a.vmask = vmask;
  a.zero_row = zero_row;
  a.inplan = 0;
  a.c_fix = 0;
  a.tile_meta_out = nullptr;
  a.split_offsets_out = nullptr;
  e = mla::launch_splitkv(a, s, static_cast<hipEvent_t>(start_event),
                          static_cast<hipEvent_t>(stop_event));
  st = launched(e, s, "mla_decode_sparse_fwd decode launch");
  if (st != MLA_OK) return st;
  mla::CombineArgs c;
  c.seqlens = nullptr;
  c.split_offsets = split_offsets_d;
  c.part_o = a.part_o;
  c.part_lse = a.part_lse;
  c.out = a.out;
  c.lse = lse_d;
  c.batch = items;
  c.M = h_q;
  c.const_len = topk;
  e = mla::launch_combine(c, s);
  return launched(e, s, "mla_decode_sparse_fwd combine launch");
}

}  // namespace

extern "C" {

int mla_decode_sparse_fwd(const void* q_d, const void* kcache_d, int64_t num_blocks,
                          const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                          int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                          const int32_t* indices_d, int topk, const int32_t* tile_meta_d,
                          const int32_t* split_offsets_d, int num_parts, void* workspace_d,
                          size_t workspace_bytes, void* out_d, float* lse_d,
                          void* start_event, void* stop_event, void* stream) {
  return sparse_fwd_impl(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                         s_q, h_q, h_kv, scale, causal, indices_d, topk, tile_meta_d,
                         split_offsets_d, num_parts, workspace_d, workspace_bytes, out_d, lse_d,
                         start_event, stop_event, stream, 0);
}

int mla_decode_sparse_fwd_fp8(const void* q_d, const void* kcache_d, int64_t num_blocks,
                              const int32_t* block_table_d, int bt_stride,
                              const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                              float scale, int causal, const int32_t* indices_d, int topk,
                              const int32_t* tile_meta_d, const int32_t* split_offsets_d,
                              int num_parts, void* workspace_d, size_t workspace_bytes,
                              void* out_d, float* lse_d, void* start_event, void* stop_event,
                              void* stream) {
  return sparse_fwd_impl(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                         s_q, h_q, h_kv, scale, causal, indices_d, topk, tile_meta_d,
                         split_offsets_d, num_parts, workspace_d, workspace_bytes, out_d, lse_d,
                         start_event, stop_event, stream, 1);
}

}  // extern "C"
