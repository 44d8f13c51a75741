// Internal interface between the C-ABI host layer (mla_api.cpp) and the
// gfx950 kernels (mla_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kBlock = 64;                 // tokens per KV page
constexpr int kDK = 576;                   // key width (512 latent + 64 rope)
constexpr int kDV = 512;                   // value width (first 512 key dims)
constexpr int kRowBytes = kDK * 2;         // 1152 bytes per bf16 cache row
constexpr int kPageBytes = kBlock * kRowBytes;  // 73728 bytes per page
constexpr int kMaxRowsPerTile = 128;       // cap of the query rows charged in the split plan's per-request overhead
constexpr int kMetaInts = 8;

// Fixed per-request overhead of the balancing rule, in page units: one page
// per 32 query rows (none for 16-row tiles, whose start-up cost is below
// half a page; charging a whole page would unbalance equal requests).
inline int fixed_cost_pages(int rows_per_tile) { return rows_per_tile / 32; }

inline int rows_per_tile(int s_q, int h_q) {
  int m = s_q * h_q;
  return m < kMaxRowsPerTile ? m : kMaxRowsPerTile;
}

struct DecodeArgs {
  const uint16_t* q;          // bf16 [B, s_q, h_q, 576]
  const void* kcache;         // bf16 [num_blocks, 64, 1, 576], or FP8 pages [num_blocks, 41216 B]
  long long num_blocks;
  const int32_t* block_table; // [B, bt_stride]
  const int32_t* seqlens;     // [B]
  const int32_t* tile_meta;   // [P, 8]
  const int32_t* split_offsets;  // [B+1]
  uint16_t* part_o;           // bf16 [slots, M, 512]
  float* part_lse;            // [slots, M]   (log2 domain)
  uint16_t* out;              // bf16 [B, s_q, h_q, 512]
  float* lse;                 // [B, s_q, h_q] (natural log)
  int bt_stride;
  int batch;
  int s_q;
  int h_q;
  int M;                      // s_q * h_q
  int causal;
  int num_parts;
  int row_tiles;
  int row_tile_rows;          // query rows per workgroup tile (16, 32, 64, or 128 for the row-wave kernels)
  float scale_log2;           // scale * log2(e)
  int kv_fp8;                 // 1: kcache holds FP8 pages
  // Sparse mode (selected keys): requests are (request, token) items of
  // const_len entries each; entry e of item b is cache row rowids[b*const_len+e]
  // (page*64 + row, -1 = skipped), bit e%32 of vmask[(b*const_len+e)/32]
  // says whether it counts; skipped entries load zero_row (1152 zero bytes).
  int sparse;
  int const_len;              // > 0: every request has this many keys
  const int32_t* rowids;
  const uint32_t* vmask;
  const void* zero_row;
  // In-kernel plan: each workgroup derives its part of the split plan from
  // the lengths (the rule of mla_metadata_kernel, c_fix overhead pages per
  // request) instead of reading tile_meta / split_offsets; it writes its
  // part's tile_meta entry, and part 0 writes split_offsets for the combine.
  int inplan;
  int c_fix;
  int32_t* tile_meta_out;       // [P, 8]
  int32_t* split_offsets_out;   // [B+1]
};

// Largest batch whose plan a workgroup derives in-kernel (its lengths are
// held in registers, its split offsets in LDS).
constexpr int kPlanMaxBatch = 1024;

struct CombineArgs {
  const int32_t* seqlens;
  const int32_t* split_offsets;
  const uint16_t* part_o;     // bf16 [slots, M, 512]
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int batch;
  int M;
  int const_len;              // > 0: every request has this many keys (seqlens unused)
};

// Launchers (return hipGetLastError() of the launch).
// const_len > 0: every request has const_len keys and seqlens is not read.
hipError_t launch_metadata(const int32_t* seqlens, int batch, int c_fix, int num_parts,
                           int32_t* tile_meta, int32_t* split_offsets, hipStream_t stream,
                           int const_len = 0);

// Sparse mode: resolve selected positions to cache rows (rowids, vmask) and
// write the zero row.  items = batch * s_q; indices [items, topk].
hipError_t launch_sparse_resolve(const int32_t* indices, const int32_t* block_table,
                                 int bt_stride, const int32_t* seqlens, long long num_blocks,
                                 int batch, int s_q, int topk, int causal, int32_t* rowids,
                                 uint32_t* vmask, void* zero_row, hipStream_t stream);
// start/stop (may be null) are recorded at the kernel's own start and end.
hipError_t launch_splitkv(const DecodeArgs& a, hipStream_t stream, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

hipError_t launch_kv_append(const uint16_t* new_kv, uint16_t* kcache, long long num_blocks,
                            const int32_t* block_table, int bt_stride, const int32_t* seqlens,
                            int batch, int s_q, hipStream_t stream);

hipError_t launch_kv_append_fp8(const uint16_t* new_kv, uint8_t* kcache, long long num_blocks,
                                const int32_t* block_table, int bt_stride,
                                const int32_t* seqlens, int batch, int s_q, hipStream_t stream);

// Rows per workgroup tile for M query rows: 128 when M is a multiple of 128
// (the row-wave kernels: dense or sparse, either cache format), else 16, 32
// or 64 (mla_splitkv_ws_kernel).
int tile_rows_for(int M);

// Host layer helpers shared with the entry point that allocates nothing
// (mla_noalloc.hip); defined in mla_api.cpp.
// validate_decode: every check of mla_decode_splitkv, launching nothing.
int validate_decode(const void* q_d, const void* kcache_d, int64_t num_blocks,
                    const int32_t* block_table_d, int bt_stride, const int32_t* seqlens_d,
                    int batch, int s_q, int h_q, int h_kv, float scale, int causal,
                    const int32_t* tile_meta_d, const int32_t* split_offsets_d, int num_parts,
                    void* workspace_d, size_t workspace_bytes, void* out_d, float* lse_d);
// Records the HIP error text (mla_last_hip_error) and returns MLA_ERR_HIP.
int set_hip_error(hipError_t e, const char* where);
// Bytes of mla_decode_workspace_bytes, and the row tiles of a launch.
size_t decode_workspace_need(int s_q, int h_q, int num_parts);
int decode_row_tiles(int s_q, int h_q);

}  // namespace mla
