// The decode entry point that allocates nothing (mla_decode_fwd_noalloc):
// the scheduler's plan and the split partials live in one file-scope device
// array of fixed size instead of caller-provided buffers, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array's name is only a host-side stand-in: its device address is looked
// up once per device with hipGetSymbolAddress and every launch receives that
// address.  Every call on a GPU shares that GPU's array, so calls that
// overlap on one GPU (two streams, or two host threads) race on it.  Nothing
// in it needs clearing between calls: the scheduler writes every plan word it
// later reads and the decode kernel writes every partial that the combine
// reads.
#include "../../include/mla_decode.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_kernels.h"

namespace {

// Layout of the array: the plan (tile_meta for up to kNoAllocMaxParts parts,
// then split_offsets for up to MLA_NOALLOC_MAX_BATCH requests), then the
// partial workspace in the layout of mla_decode_workspace_bytes.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocMaxParts = 1024;
constexpr size_t kTileMetaOff = 0;
constexpr size_t kSplitOffsetsOff = (size_t)kNoAllocMaxParts * MLA_TILE_META_INTS * 4;
constexpr size_t kPartialsOff =
    kSplitOffsetsOff + ((size_t)(MLA_NOALLOC_MAX_BATCH + 1) * 4 + 255) / 256 * 256;
constexpr size_t kPartialsBytes = kScratchBytes - kPartialsOff;
static_assert(kPartialsOff % 256 == 0, "workspace must stay 256-byte aligned");

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of the array (looked up on the first
// call on each device, with that device current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mla::set_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return mla::set_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_fwd_noalloc(const void* q_d, const void* kcache_d, int64_t num_blocks,
                           const int32_t* block_table_d, int bt_stride,
                           const int32_t* seqlens_d, int batch, int s_q, int h_q, int h_kv,
                           float scale, int causal, void* out_d, float* lse_d, void* stream) {
  if (batch < 1 || batch > MLA_NOALLOC_MAX_BATCH) return MLA_ERR_INVALID_ARG;
  int num_cus = 0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mla::set_hip_error(e, "hipGetDevice");
  int st = mla_device_num_cus(dev, &num_cus);
  if (st != MLA_OK) return st;
  int parts = 0;
  st = mla_decode_num_parts(batch, s_q, h_q, h_kv, num_cus, &parts);
  if (st != MLA_OK) return st;
  if (parts > kNoAllocMaxParts) parts = kNoAllocMaxParts;
  // fewer parts when their partials would not fit in the array
  while (parts > 1 && mla::decode_workspace_need(s_q, h_q, parts) > kPartialsBytes) parts /= 2;

  void* base = nullptr;
  st = scratch_for_current_device(&base);
  if (st != MLA_OK) return st;
  char* sc = static_cast<char*>(base);
  int32_t* tile_meta = reinterpret_cast<int32_t*>(sc + kTileMetaOff);
  int32_t* split_offsets = reinterpret_cast<int32_t*>(sc + kSplitOffsetsOff);
  void* workspace = sc + kPartialsOff;
  const size_t ws_bytes = mla::decode_workspace_need(s_q, h_q, parts);

  // every check of the decode before anything is enqueued
  st = mla::validate_decode(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d,
                            batch, s_q, h_q, h_kv, scale, causal, tile_meta, split_offsets,
                            parts, workspace, ws_bytes, out_d, lse_d);
  if (st != MLA_OK) return st;
  st = mla_decode_metadata(seqlens_d, batch, s_q, h_q, h_kv, MLA_BLOCK_SIZE, parts, tile_meta,
                           split_offsets, stream);
  if (st != MLA_OK) return st;
  return mla_decode_fwd(q_d, kcache_d, num_blocks, block_table_d, bt_stride, seqlens_d, batch,
                        s_q, h_q, h_kv, scale, causal, tile_meta, split_offsets, parts,
                        workspace, ws_bytes, out_d, lse_d, stream);
}

}  // extern "C"
