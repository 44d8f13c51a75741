// gfx950 (MI355X) kernels of paged-KV MLA decode attention.
//
// Sources for what is computed: page "深度剖析DeepSeek Infra开源全貌"
// (jingzhunhuoke.net/55333.html), section DAY1 FlashMLA:
//   * MLA — every query head of a request attends over one shared latent KV
//     head (terminology paragraph on MLA);
//   * the KV cache is paged in 64-token blocks (feature ②);
//   * the kernel keeps a page on chip while it is used (feature ③, shared
//     memory; here LDS) and computes two products per page, scores and then
//     probabilities times values (feature ④, "Gemm1"/"Gemm2");
//   * variable lengths are balanced dynamically with double buffering
//     (feature ⑤) — here a split-KV partition plus a log-sum-exp merge.
//
// gfx950 design (not the page's Hopper design):
//   * one 512-thread workgroup (8 wave64, two per SIMD) per CU, in two roles:
//     four score waves (scores + softmax) and four value waves (values +
//     page loads), one half-page unit apart (see mla_splitkv_ws_kernel);
//   * half pages (32 x 576 bf16 = 36 KB) are streamed HBM -> LDS with 16-byte
//     direct-to-LDS buffer loads (no VGPR staging) into a ring of four unit
//     buffers (144 KB of the 160 KB LDS), two units in flight;
//   * scores are computed transposed, S^T = K . Q^T, on v_mfma_f32_16x16x32_bf16
//     with the page rows as the A operand (ds_read_b128) and Q held in VGPRs as
//     the B operand.  The MFMA output then holds, per lane, one query row and
//     four consecutive keys — so the online softmax needs only 2 cross-lane
//     steps per row, and the bf16 probabilities are already in the B-operand
//     layout of the second product;
//   * O^T += V^T . P^T on the same MFMA: V is the first 512 columns of the
//     same LDS page, read with ds_read_b64_tr_b16 (hardware 4x16 transpose),
//     so the key axis becomes the reduction axis without a second copy;
//   * LDS rows are XOR-swizzled in 16-byte units (see lds_swizzle) so the
//     row-wise A reads and the transposed V reads are bank-conflict free;
//   * the page's tail rows beyond the sequence length are zero-filled by the
//     buffer unit's range check (num_records), never read from memory.
#include "mla_kernels.h"

#include <hip/hip_ext.h>

#include <math.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kChunksPerRow = kRowBytes / 16;   // 72 16-byte units per row
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit format
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;           // lazy-rescale threshold (log2)

// 16-byte unit swizzle of LDS row r: unit c is stored at c ^ lds_swizzle(r).
// Chosen by measurement on gfx950 among XOR and rotation swizzles of the low
// three unit bits: with r & 7 both read patterns of the kernels run at the
// conflict-free rate — 16 consecutive rows at one unit (ds_read_b128, score
// operand: 4.9 clk per wave instruction per CU, against 8.1-8.6 for the other
// 8-row bijections tried and 16.1 unswizzled) and 4 rows x 32 bytes per
// 16-lane group (ds_read_b64_tr_b16, value operand: 3.3 clk, against 4.6-8.1).
// XOR stays inside an aligned group of 8 units; 72 units per row is a
// multiple of 8.
__device__ __forceinline__ int lds_swizzle(int r) { return r & 7; }

// Reductions over lanes {i, i^16, i^32, i^48}, the four lanes holding one
// query row, with the gfx950 row-swap permutes (VALU; a __shfl_xor would be a
// round trip through the LDS crossbar).  permlane16_swap(x, x) hands every
// lane x of lane i^16 in one of its two results and its own x in the other,
// permlane32_swap likewise for lane i^32, so combining the pair is the
// reduction step whichever way round the two come back.
__device__ __forceinline__ float wave_max_4lanes(float x) {
  const unsigned xi = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const unsigned yi = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

__device__ __forceinline__ float wave_sum_4lanes(float x) {
  const unsigned xi = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const unsigned yi = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// makes the compiler wait for ALL outstanding vector memory ops (vmcnt(0)),
// including the page prefetches that must stay in flight.  Callers wait
// explicitly for what the barrier publishes (vmcnt for direct-to-LDS page
// loads, lgkmcnt for ds_write); the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int n_pages(int L) {
  return L > 0 ? (L + kBlock - 1) / kBlock : 0;
}

// --------------------------------------------------------------------------
// Split-KV scheduler: one workgroup.  Implements the integer balancing rule
// documented with mla_decode_metadata (cost_b = pages + c, equal quotas).
// Every tile_meta word is written by exactly one thread.
// --------------------------------------------------------------------------
// One wave64: requests are taken 64 at a time; the cost scan inside a chunk
// fits 32 bits (a request has fewer than 2^25 pages), the running offsets are
// 64-bit.  No workgroup barriers.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// const_len > 0: every request has const_len keys (seqlens is not read).
__global__ __launch_bounds__(64) void mla_metadata_kernel(
    const int32_t* __restrict__ seqlens, int batch, int c_fix, int num_parts,
    int32_t* __restrict__ tile_meta, int32_t* __restrict__ split_offsets, int const_len) {
  const int lane = threadIdx.x;
  auto len = [&](int b) { return const_len > 0 ? const_len : seqlens[b]; };

  // total cost C
  long long local = 0;
  for (int b = lane; b < batch; b += 64) {
    const int n = n_pages(len(b));
    local += n > 0 ? (long long)(n + c_fix) : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
  const long long C = local;
  const long long P = num_parts;
  const long long q = C > 0 ? (C + P - 1) / P : 1;

  long long carry_cost = 0;
  int carry_slots = 0;
  for (int base = 0; base < batch; base += 64) {
    const int b = base + lane;
    const int n = b < batch ? n_pages(len(b)) : 0;
    const int cost = n > 0 ? n + c_fix : 0;
    const int incl = wave_incl_scan(cost);
    const long long start = carry_cost + (incl - cost);
    long long p0 = 0;   // first boundary index after the request's overhead units
    int nsplit = 1;
    if (n > 0) {
      const long long lo = start + c_fix;
      p0 = lo / q + 1;
      nsplit = 1 + (int)((lo + n - 1) / q - (p0 - 1));
    }
    const int slots = nsplit >= 2 ? nsplit : 0;
    const int slots_incl = wave_incl_scan(slots);
    if (b < batch) {
      split_offsets[b] = carry_slots + slots_incl - slots;
      if (cost > 0) {
        // boundaries p*q that fall inside [start, start + cost)
        const long long p_lo = (start + q - 1) / q;
        const long long p_hi = (start + cost + q - 1) / q;
        for (long long p = p_lo; p < p_hi && p < P; ++p) {
          long long k = p * q - start - c_fix;
          k = k < 0 ? 0 : (k > n ? n : k);
          const int first = (k > 0 && k < n) ? (int)(p - p0 + 1) : 0;
          int32_t* tm = tile_meta + p * kMetaInts;
          tm[0] = b;
          tm[1] = (int)k;
          tm[4] = first;
          if (p > 0) {
            tile_meta[(p - 1) * kMetaInts + 2] = b;
            tile_meta[(p - 1) * kMetaInts + 3] = (int)k;
          }
        }
      }
    }
    carry_cost += __shfl(incl, 63);
    carry_slots += __shfl(slots_incl, 63);
  }
  if (lane == 0) split_offsets[batch] = carry_slots;
  // parts whose boundary lies at or beyond C begin (and the last part ends) at (B, 0)
  const long long p_tail = (C + q - 1) / q;
  for (long long p = lane; p < P; p += 64) {
    int32_t* tm = tile_meta + p * kMetaInts;
    tm[5] = 0;
    tm[6] = 0;
    tm[7] = 0;
    if (p >= p_tail) {
      tm[0] = batch;
      tm[1] = 0;
      tm[4] = 0;
      if (p > 0) {
        tile_meta[(p - 1) * kMetaInts + 2] = batch;
        tile_meta[(p - 1) * kMetaInts + 3] = 0;
      }
    }
    if (p == P - 1) {
      tm[2] = batch;
      tm[3] = 0;
    }
  }
}

hipError_t launch_metadata(const int32_t* seqlens, int batch, int c_fix, int num_parts,
                           int32_t* tile_meta, int32_t* split_offsets, hipStream_t stream,
                           int const_len) {
  hipLaunchKernelGGL(mla_metadata_kernel, dim3(1), dim3(64), 0, stream, seqlens, batch, c_fix,
                     num_parts, tile_meta, split_offsets, const_len);
  return hipGetLastError();
}

// The split plan of part p, derived by one wave inside the decode kernel
// with the rule of mla_metadata_kernel (same scans, same boundary map, same
// split counts): plan[0..4] = b0, k0, b1, k1, first_split of the part, and
// so[b] = split_offsets[b] for every request b <= batch.  Requests are held
// kPlanMaxBatch / 64 per lane in registers, so the lengths are read once,
// all loads in flight together.
__device__ void plan_part_wave(const DecodeArgs& a, int p, int* plan, int* so) {
  constexpr int NC = kPlanMaxBatch / 64;
  const int lane = threadIdx.x & 63;
  const int B = a.batch, cf = a.c_fix;
  int n[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int b = 64 * c + lane;
    const int L = b < B ? (a.const_len > 0 ? a.const_len : a.seqlens[b]) : 0;
    n[c] = n_pages(L);
  }
  long long start[NC];
  long long carry = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (64 * c >= B) {
      start[c] = carry;
      continue;
    }
    const int cost = n[c] > 0 ? n[c] + cf : 0;
    const int incl = wave_incl_scan(cost);
    start[c] = carry + (incl - cost);
    carry += __shfl(incl, 63);
  }
  const long long C = carry;
  const long long P = a.num_parts;
  const long long q = C > 0 ? (C + P - 1) / P : 1;

  // Boundary x: (b, clamp(x - start_b - c, 0, n_b)) for the request whose
  // units contain x, (B, 0) for x >= C.
  auto boundary = [&](long long x, int& bb, int& kk, long long& st, int& nn) {
    bb = B;
    kk = 0;
    st = 0;
    nn = 0;
    if (x >= C) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (64 * c >= B) break;
      const int cost = n[c] > 0 ? n[c] + cf : 0;
      const bool hit = cost > 0 && start[c] <= x && x < start[c] + cost;
      const unsigned long long m = __ballot(hit);
      if (m) {
        const int l = __ffsll(static_cast<long long>(m)) - 1;
        bb = 64 * c + l;
        st = __shfl(start[c], l);
        nn = __shfl(n[c], l);
        long long k = x - st - cf;
        kk = static_cast<int>(k < 0 ? 0 : (k > nn ? nn : k));
        return;
      }
    }
  };
  int b0, k0, b1, k1, n0;
  long long st0, st1;
  int n1;
  boundary((long long)p * q, b0, k0, st0, n0);
  boundary((long long)(p + 1) * q, b1, k1, st1, n1);
  const int first = (b0 < B && k0 > 0 && k0 < n0) ? (int)(p - (st0 + cf) / q) : 0;
  if (lane == 0) {
    plan[0] = b0;
    plan[1] = k0;
    plan[2] = b1;
    plan[3] = k1;
    plan[4] = first;
  }
  // split offsets: prefix sums of the slot counts of split requests
  int carry_s = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (64 * c >= B) break;
    const int b = 64 * c + lane;
    int nsplit = 1;
    if (n[c] > 0) {
      const long long lo = start[c] + cf;
      nsplit = 1 + (int)((lo + n[c] - 1) / q - lo / q);
    }
    const int slots = nsplit >= 2 ? nsplit : 0;
    const int incl = wave_incl_scan(slots);
    if (b < B) so[b] = carry_s + incl - slots;
    carry_s += __shfl(incl, 63);
  }
  if (lane == 0) so[B] = carry_s;
}

// Values the hardware needs in SGPRs (buffer resources, M0) are read from
// global memory with vector loads (the kernel also stores, so loads are not
// provably invariant); readfirstlane tells the compiler they are wave-uniform
// so no waterfall loop is emitted.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Scalar (SMEM) load of read-only metadata: through the constant address
// space a wave-uniform address becomes s_load, tracked by lgkmcnt.  Vector
// loads would be tracked by vmcnt, which retires in issue order, so waiting
// for such a value would also wait for every page load issued before it.
// seqlens, block_table, tile_meta and split_offsets are never written while
// the kernel runs.
__device__ __forceinline__ int ldc(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

// Load 16 rows x 576 bf16 of Q (the B operand of the score product) for one
// lane: 18 x 16 bytes at a 64-byte stride.  Inline asm so the compiler does
// not place its own (in-order, hence pipeline-draining) vmcnt wait for it;
// the block waits for its own loads before it ends (its outputs are
// early-clobber so no load can overwrite the address of a later one).
__device__ __forceinline__ void load_q_rows(bf16x8 (&q)[18], const bf16x8* qp) {
  asm volatile(
      "global_load_dwordx4 %0, %18, off\n\t"
      "global_load_dwordx4 %1, %18, off offset:64\n\t"
      "global_load_dwordx4 %2, %18, off offset:128\n\t"
      "global_load_dwordx4 %3, %18, off offset:192\n\t"
      "global_load_dwordx4 %4, %18, off offset:256\n\t"
      "global_load_dwordx4 %5, %18, off offset:320\n\t"
      "global_load_dwordx4 %6, %18, off offset:384\n\t"
      "global_load_dwordx4 %7, %18, off offset:448\n\t"
      "global_load_dwordx4 %8, %18, off offset:512\n\t"
      "global_load_dwordx4 %9, %18, off offset:576\n\t"
      "global_load_dwordx4 %10, %18, off offset:640\n\t"
      "global_load_dwordx4 %11, %18, off offset:704\n\t"
      "global_load_dwordx4 %12, %18, off offset:768\n\t"
      "global_load_dwordx4 %13, %18, off offset:832\n\t"
      "global_load_dwordx4 %14, %18, off offset:896\n\t"
      "global_load_dwordx4 %15, %18, off offset:960\n\t"
      "global_load_dwordx4 %16, %18, off offset:1024\n\t"
      "global_load_dwordx4 %17, %18, off offset:1088\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]),
        "=&v"(q[6]), "=&v"(q[7]), "=&v"(q[8]), "=&v"(q[9]), "=&v"(q[10]), "=&v"(q[11]),
        "=&v"(q[12]), "=&v"(q[13]), "=&v"(q[14]), "=&v"(q[15]), "=&v"(q[16]), "=&v"(q[17])
      : "v"(qp)
      : "memory");
}

// A position in a part's page sequence is a (request b, page k) pair of
// wave-uniform ints; it is valid while (b, k) < (b1, k1) lexicographically.
__device__ __forceinline__ bool before_end(const DecodeArgs& a, int b, int k, int b1, int k1) {
  return b < a.batch && (b < b1 || (b == b1 && k < k1));
}

// Keys of request b: its length, or the fixed entry count of the sparse mode.
__device__ __forceinline__ int seqlen_of(const DecodeArgs& a, int b) {
  if (a.const_len > 0) return b < a.batch ? a.const_len : 0;
  return b < a.batch ? ldc(a.seqlens + b) : 0;
}

// Move (b, k) to the first page at or after it that belongs to the part.
__device__ __forceinline__ void seek(const DecodeArgs& a, int& b, int& k, int b1, int k1) {
  while (before_end(a, b, k, b1, k1)) {
    const int end = (b == b1) ? k1 : n_pages(seqlen_of(a, b));
    if (k < end) return;
    ++b;
    k = 0;
  }
}

// --------------------------------------------------------------------------
// Warp-specialised kernel for row tiles of 64 query rows (s_q*h_q >= 64).
// Eight waves, two per SIMD, in two roles that work one unit apart so that
// each SIMD always holds one wave of each and their matrix products, LDS
// reads and softmax interleave:
//   score waves 0..3:  rows 16q .. 16q+15 of the tile (q = w), all 32 keys
//                      of unit t: S^T = K . Q^T, online softmax (exact row
//                      max over the unit, lazy rescale), bf16 P to LDS;
//   value waves 4..7:  output dims 128j .. 128j+127 (j = w - 4) for all 64
//                      rows: O^T += V^T . P^T of unit t-1, and every direct
//                      page load, so no score wave ever waits on a load
//                      queue it did not fill.
// Work unit = half a page (32 keys, 36 KB) in a ring of four LDS buffers:
// while unit t is scored and unit t-1 multiplied, units t+1 and t+2 are in
// flight (each has two phases to land).  One workgroup barrier per unit.  Probabilities, rescale
// factors and final row sums are double-buffered by unit parity.
// --------------------------------------------------------------------------
constexpr int kHalfRows = 32;
constexpr int kHalfBytes = kHalfRows * kRowBytes;   // 36864
constexpr int kThreadsWS = 512;
constexpr int kWSBufs = 4;
constexpr int kHalfLoadsPerWave = 9;                // 36 1 KB slots over 4 value waves

// Issue the 9 direct-to-LDS loads of half `h` of page k of request b for
// value wave j: 1 KB slots j, j+4, ..., j+32 of the unit.  Rows at or beyond
// the sequence end are zero-filled by the buffer range check.
//
// Written as inline asm on purpose: the compiler then does not track these
// loads.  Tracked, every LDS read that it cannot prove disjoint from an
// in-flight direct load (the transposed V reads, for one) gets an
// "s_waitcnt vmcnt(0)", which would wait for the NEXT units' loads and
// serialise the pipeline.  All waits for these loads are therefore explicit
// (wait_unit in the kernel), and the asm clobbers "memory" so the compiler
// keeps LDS accesses on the right side of it.  M0 holds the LDS destination;
// nothing else in the kernels uses M0 (gfx9 LDS instructions do not), and one
// wait state separates each M0 write from the load that reads it.  The M0
// increments are SALU adds, which write SCC: SCC is declared clobbered.
// A unit's load set up for issue one slot at a time (half_load_slot): the
// buffer resource of the page half and the LDS address of this wave's first
// slot.  Spreading a unit's nine loads between the value product's MFMAs
// keeps the CU's load queue short, so that the issuing wave does not stall
// behind the loads of the other value waves.
struct HalfLoad {
  __amdgpu_buffer_rsrc_t r;
  uint32_t m0;
};

__device__ __forceinline__ HalfLoad half_load_setup(char* lds_buf, const DecodeArgs& a, int b,
                                                   int k, int h, int j) {
  const int L = ldc(a.seqlens + b);
  int rows = L - k * kBlock - h * kHalfRows;
  rows = rows > kHalfRows ? kHalfRows : rows;
  int page = -1;
  if (k < a.bt_stride) page = ldc(a.block_table + (long long)b * a.bt_stride + k);
  const bool ok = page >= 0 && (long long)page < a.num_blocks && rows > 0;
  const char* base = reinterpret_cast<const char*>(a.kcache) +
                     (ok ? (long long)page * kPageBytes + h * kHalfBytes : 0);
  const int nrec = uni(ok ? rows * kRowBytes : 0);
  HalfLoad d;
  d.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, nrec, kRsrcWord3);
  d.m0 = uni(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MLA_LDS char*)(lds_buf)) +
                                   j * 1024));
  return d;
}

// Slot m (0..8) of a unit set up by half_load_setup: 1 KB, 16 bytes per lane.
__device__ __forceinline__ void half_load_slot(const HalfLoad& d, int off, int m) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[o], %[r], 0 offen lds"
               :
               : [m] "s"(d.m0 + m * 0x1000), [r] "s"(d.r), [o] "v"(off)
               : "memory", "m0");
}

__device__ __forceinline__ void issue_half_load(char* lds_buf, const DecodeArgs& a, int b, int k,
                                                int h, const int (&off)[9], int j) {
  const int L = ldc(a.seqlens + b);
  int rows = L - k * kBlock - h * kHalfRows;
  rows = rows > kHalfRows ? kHalfRows : rows;
  int page = -1;
  if (k < a.bt_stride) page = ldc(a.block_table + (long long)b * a.bt_stride + k);
  const bool ok = page >= 0 && (long long)page < a.num_blocks && rows > 0;
  const char* base = reinterpret_cast<const char*>(a.kcache) +
                     (ok ? (long long)page * kPageBytes + h * kHalfBytes : 0);
  const int nrec = uni(ok ? rows * kRowBytes : 0);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, nrec, kRsrcWord3);
  const uint32_t m0 = uni(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((MLA_LDS char*)(lds_buf)) + j * 1024));
#define MLA_DMA(O) "s_nop 0\n\tbuffer_load_dwordx4 %[" #O "], %[r], 0 offen lds\n\t"
#define MLA_M0_NEXT "s_add_u32 m0, m0, 0x1000\n\t"
  asm volatile(
      "s_mov_b32 m0, %[m]\n\t"
      MLA_DMA(o0) MLA_M0_NEXT MLA_DMA(o1) MLA_M0_NEXT MLA_DMA(o2) MLA_M0_NEXT
      MLA_DMA(o3) MLA_M0_NEXT MLA_DMA(o4) MLA_M0_NEXT MLA_DMA(o5) MLA_M0_NEXT
      MLA_DMA(o6) MLA_M0_NEXT MLA_DMA(o7) MLA_M0_NEXT MLA_DMA(o8)
      :
      : [m] "s"(m0), [r] "s"(r), [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]),
        [o3] "v"(off[3]), [o4] "v"(off[4]), [o5] "v"(off[5]), [o6] "v"(off[6]),
        [o7] "v"(off[7]), [o8] "v"(off[8])
      : "memory", "m0", "scc");
#undef MLA_DMA
#undef MLA_M0_NEXT
}

// Unit positions: (request b, page k, half h); the second half of a page is a
// unit only if the page has keys in it.  The walk keeps the request length L
// cached and re-reads it only when the position moves to another request.
__device__ __forceinline__ void unit_next(const DecodeArgs& a, int& b, int& k, int& h, int& L,
                                          int b1, int k1) {
  if (h == 0 && L - k * kBlock > kHalfRows) {
    h = 1;
    return;
  }
  h = 0;
  ++k;
  while (before_end(a, b, k, b1, k1)) {
    const int end = (b == b1) ? k1 : n_pages(L);
    if (k < end) return;
    ++b;
    k = 0;
    L = seqlen_of(a, b);
  }
}

// Sparse mode: issue the loads of entries 64k + 32h .. +31 of item b for
// value wave j.  The unit has the dense layout in LDS (row r of the unit =
// entry r, units swizzled as lds_swizzle), but every row comes from its own
// cache row, so each lane carries a 64-bit address (global_load_lds_dwordx4:
// 16 bytes per lane to M0 + 16 * lane).  Slot j + 4m covers 64 consecutive
// 16-byte units of the unit buffer, i.e. rows r0 and r0 + 1 at most
// (72 units per row): their two row ids are wave-uniform scalar loads, and
// rsel[m] picks the lane's.  Skipped entries (row id -1) load the zero row,
// so every slot issues exactly one load and the vmcnt accounting of the
// dense path holds unchanged.  coff[m] is the lane's byte offset in its row;
// rlo / rhi are the row ids of rows r0(m), r0(m)+1 (load_sparse_rowids),
// loaded one unit ahead so that their latency is off the issue path.
__device__ __forceinline__ void load_sparse_rowids(const DecodeArgs& a, int b, int k, int h,
                                                   int j, int (&rlo)[9], int (&rhi)[9]) {
  const long long e0 = (long long)b * a.const_len + k * kBlock + h * kHalfRows;
#pragma unroll
  for (int m = 0; m < 9; ++m) {
    const int r0 = (256 * m + 64 * j) / kChunksPerRow;   // wave-uniform
    rlo[m] = ldc(a.rowids + e0 + r0);
    rhi[m] = r0 + 1 < kHalfRows ? ldc(a.rowids + e0 + r0 + 1) : -1;
  }
}

__device__ __forceinline__ void issue_half_load_sparse(char* lds_buf, const DecodeArgs& a,
                                                       const int (&rlo)[9], const int (&rhi)[9],
                                                       const int (&coff)[9],
                                                       const bool (&rsel)[9], int j) {
  const char* kc = reinterpret_cast<const char*>(a.kcache);
  const char* zr = reinterpret_cast<const char*>(a.zero_row);
  const char* src[9];
#pragma unroll
  for (int m = 0; m < 9; ++m) {
    const int rid = rsel[m] ? rhi[m] : rlo[m];
    src[m] = (rid >= 0 ? kc + (long long)rid * kRowBytes : zr) + coff[m];
  }
  const uint32_t m0 = uni(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((MLA_LDS char*)(lds_buf)) + j * 1024));
#define MLA_GDMA(O) "s_nop 0\n\tglobal_load_lds_dwordx4 %[" #O "], off\n\t"
#define MLA_M0_NEXT "s_add_u32 m0, m0, 0x1000\n\t"
  asm volatile(
      "s_mov_b32 m0, %[m]\n\t"
      MLA_GDMA(a0) MLA_M0_NEXT MLA_GDMA(a1) MLA_M0_NEXT MLA_GDMA(a2) MLA_M0_NEXT
      MLA_GDMA(a3) MLA_M0_NEXT MLA_GDMA(a4) MLA_M0_NEXT MLA_GDMA(a5) MLA_M0_NEXT
      MLA_GDMA(a6) MLA_M0_NEXT MLA_GDMA(a7) MLA_M0_NEXT MLA_GDMA(a8)
      :
      : [m] "s"(m0), [a0] "v"(src[0]), [a1] "v"(src[1]), [a2] "v"(src[2]), [a3] "v"(src[3]),
        [a4] "v"(src[4]), [a5] "v"(src[5]), [a6] "v"(src[6]), [a7] "v"(src[7]), [a8] "v"(src[8])
      : "memory", "m0", "scc");
#undef MLA_GDMA
#undef MLA_M0_NEXT
}

// --------------------------------------------------------------------------
// FP8 cache pages.  A page of 64 tokens is 41216 bytes:
//   [0, 32768)      E4M3 codes of latent dims 0..511, uint8 [64][512]
//   [32768, 40960)  rope dims 512..575 in bf16, [64][64]
//   [40960, 41216)  per-token fp32 scale, [64]; latent = e4m3(code) * scale
// A half-page unit in LDS holds its 32 rows of codes (16 KB), of rope (4 KB)
// and its 32 scales (a 256-byte slot): 20736 bytes.
// --------------------------------------------------------------------------
constexpr int kF8Latent = 512;
constexpr int kF8RopeOff = kBlock * kF8Latent;             // 32768
constexpr int kF8ScaleOff = kF8RopeOff + kBlock * 64 * 2;  // 40960
constexpr int kF8PageBytes = kF8ScaleOff + kBlock * 4;     // 41216
constexpr int kF8UnitCodes = 0;
constexpr int kF8UnitRope = kHalfRows * kF8Latent;         // 16384
constexpr int kF8UnitScale = kF8UnitRope + kHalfRows * 128;   // 20480
constexpr int kF8UnitBytes = kF8UnitScale + 256;           // 20736
// Sparse mode over FP8 pages: the scales of a unit's rows are gathered one
// row at a time, value wave j fetching rows 8j .. 8j+7 with one 64-lane dword
// load into its own 256-byte window (lanes 8..63 load zeros from the zero
// row), so a unit ends in four windows: scale of row r at window r / 8,
// byte 4 (r % 8).
constexpr int kF8SpUnitBytes = kF8UnitScale + 4 * 256;     // 21504
__device__ __forceinline__ int f8sp_scale_off(int r) { return (r >> 3) * 256 + (r & 7) * 4; }
// Ring depth for FP8 units.  The smaller units would leave room for six or
// seven buffers, but measured on gfx950 both are slower than four (membound
// 48.8 / 49.6 us against 46.7 us): with one 16-row tile the score wave's own
// chain, not the load latency, sets the phase.
constexpr int kWSBufsF8 = 4;

// Wait until at most `ahead` units of this wave's page loads (N loads each,
// issued after the unit waited for) are still outstanding; A is the largest
// number of units that can be ahead.
template <int K>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}
template <int N, int A>
__device__ __forceinline__ void wait_loads_behind(int ahead) {
  if constexpr (A <= 0) {
    vm_wait<0>();
  } else {
    if (ahead >= A)
      vm_wait<N * A>();
    else
      wait_loads_behind<N, A - 1>(ahead);
  }
}

// Swizzles of the FP8 unit, chosen by measurement on gfx950 (LDS throughput
// of the kernel's own read patterns under candidate XOR swizzles):
//  * code rows (512 B = 32 units): unit c of row r at c ^ f8_code_swizzle(r).
//    Both patterns run at the conflict-free rate — 16 rows at one unit
//    (ds_read_b128, score operand: 4.9 clk per wave instruction per CU) and
//    8 rows {4g..4g+3, 16+4g..16+4g+3} x 16 bytes per 16-lane group
//    (ds_read_b64_tr_b8, value operand: 2.9 clk, against 4.4 for r & 15);
//  * rope rows (128 B = 8 units): unit c of row r at c ^ ((r >> 1) & 7)
//    (4.8 clk, against 16.2 unswizzled).
__device__ __forceinline__ int f8_code_swizzle(int r) { return (r & 15) ^ (8 * ((r >> 4) & 1)); }
__device__ __forceinline__ int f8_rope_swizzle(int r) { return (r >> 1) & 7; }

// Issue the direct-to-LDS loads of half `h` of FP8 page k of request b for
// value wave j: code slots j, j+4, j+8, j+12 (1 KB each), rope slot j, and
// for wave 0 the unit's 32 scales (one dword per lane; lanes past the 32nd
// fall outside the range and write zeros).  Each of the three regions has
// its own buffer resource whose range ends at the sequence end, so rows
// past it are zero-filled: zero codes, rope and scale.  Same asm rationale
// as issue_half_load; M0 advances by 4 KB between all six loads.
__device__ __forceinline__ void issue_half_load_f8(char* lds_buf, const DecodeArgs& a, int b,
                                                   int k, int h, const int (&offc)[4], int offr,
                                                   int offs, int j) {
  const int L = ldc(a.seqlens + b);
  int rows = L - k * kBlock - h * kHalfRows;
  rows = rows > kHalfRows ? kHalfRows : rows;
  int page = -1;
  if (k < a.bt_stride) page = ldc(a.block_table + (long long)b * a.bt_stride + k);
  const bool ok = page >= 0 && (long long)page < a.num_blocks && rows > 0;
  const char* pg = reinterpret_cast<const char*>(a.kcache) + (ok ? (long long)page * kF8PageBytes : 0);
  const int nr = uni(ok ? rows : 0);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(pg + h * kHalfRows * kF8Latent), 0, nr * kF8Latent, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(pg + kF8RopeOff + h * kHalfRows * 128), 0, nr * 128, kRsrcWord3);
  const uint32_t m0 = uni(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((MLA_LDS char*)(lds_buf)) + j * 1024));
#define MLA_DMA(O, R) "s_nop 0\n\tbuffer_load_dwordx4 %[" #O "], %[" #R "], 0 offen lds\n\t"
#define MLA_M0_NEXT "s_add_u32 m0, m0, 0x1000\n\t"
  if (j == 0) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(pg + kF8ScaleOff + h * kHalfRows * 4), 0, nr * 4, kRsrcWord3);
    asm volatile(
        "s_mov_b32 m0, %[m]\n\t"
        MLA_DMA(o0, rc) MLA_M0_NEXT MLA_DMA(o1, rc) MLA_M0_NEXT MLA_DMA(o2, rc) MLA_M0_NEXT
        MLA_DMA(o3, rc) MLA_M0_NEXT MLA_DMA(o4, rr) MLA_M0_NEXT
        "s_nop 0\n\tbuffer_load_dword %[o5], %[rs], 0 offen lds\n\t"
        :
        : [m] "s"(m0), [rc] "s"(rc), [rr] "s"(rr), [rs] "s"(rs), [o0] "v"(offc[0]),
          [o1] "v"(offc[1]), [o2] "v"(offc[2]), [o3] "v"(offc[3]), [o4] "v"(offr), [o5] "v"(offs)
        : "memory", "m0", "scc");
  } else {
    asm volatile(
        "s_mov_b32 m0, %[m]\n\t"
        MLA_DMA(o0, rc) MLA_M0_NEXT MLA_DMA(o1, rc) MLA_M0_NEXT MLA_DMA(o2, rc) MLA_M0_NEXT
        MLA_DMA(o3, rc) MLA_M0_NEXT MLA_DMA(o4, rr)
        :
        : [m] "s"(m0), [rc] "s"(rc), [rr] "s"(rr), [o0] "v"(offc[0]), [o1] "v"(offc[1]),
          [o2] "v"(offc[2]), [o3] "v"(offc[3]), [o4] "v"(offr)
        : "memory", "m0", "scc");
  }
#undef MLA_DMA
#undef MLA_M0_NEXT
}

// Q rows for the FP8 score product.  A lane's 16-byte code read covers 16
// consecutive latent dims, 64p + 16g .. +16, which feed two MFMA steps; Q
// follows the same order: q[2p + e] = dims 64p + 16g + 8e .. +8 (p < 8), and
// q[16 + s] = rope dims 512 + 32s + 8g .. +8.  qlat points at dim 16g of the
// row, qrope at dim 512 + 8g.  Same asm rationale as load_q_rows.
__device__ __forceinline__ void load_q_rows_f8(bf16x8 (&q)[18], const bf16x8* qlat,
                                               const bf16x8* qrope) {
  asm volatile(
      "global_load_dwordx4 %0, %18, off\n\t"
      "global_load_dwordx4 %1, %18, off offset:16\n\t"
      "global_load_dwordx4 %2, %18, off offset:128\n\t"
      "global_load_dwordx4 %3, %18, off offset:144\n\t"
      "global_load_dwordx4 %4, %18, off offset:256\n\t"
      "global_load_dwordx4 %5, %18, off offset:272\n\t"
      "global_load_dwordx4 %6, %18, off offset:384\n\t"
      "global_load_dwordx4 %7, %18, off offset:400\n\t"
      "global_load_dwordx4 %8, %18, off offset:512\n\t"
      "global_load_dwordx4 %9, %18, off offset:528\n\t"
      "global_load_dwordx4 %10, %18, off offset:640\n\t"
      "global_load_dwordx4 %11, %18, off offset:656\n\t"
      "global_load_dwordx4 %12, %18, off offset:768\n\t"
      "global_load_dwordx4 %13, %18, off offset:784\n\t"
      "global_load_dwordx4 %14, %18, off offset:896\n\t"
      "global_load_dwordx4 %15, %18, off offset:912\n\t"
      "global_load_dwordx4 %16, %19, off\n\t"
      "global_load_dwordx4 %17, %19, off offset:64\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]),
        "=&v"(q[6]), "=&v"(q[7]), "=&v"(q[8]), "=&v"(q[9]), "=&v"(q[10]), "=&v"(q[11]),
        "=&v"(q[12]), "=&v"(q[13]), "=&v"(q[14]), "=&v"(q[15]), "=&v"(q[16]), "=&v"(q[17])
      : "v"(qlat), "v"(qrope)
      : "memory");
}

// Sparse mode over FP8 pages: row ids of the unit's rows that value wave j
// gathers (entries 64k + 32h .. +31 of item b): rc = rows 2(j + 4m) and
// 2(j + 4m) + 1 of code slot m, r8 = rows 8j .. 8j+7 (its rope slot and its
// scales).  Loaded one unit ahead, like load_sparse_rowids.
__device__ __forceinline__ void load_sparse_rowids_f8(const DecodeArgs& a, int b, int k, int h,
                                                      int j, int (&rc)[8], int (&r8)[8]) {
  const long long e0 = (long long)b * a.const_len + k * kBlock + h * kHalfRows;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    rc[2 * m] = ldc(a.rowids + e0 + 2 * (j + 4 * m));
    rc[2 * m + 1] = ldc(a.rowids + e0 + 2 * (j + 4 * m) + 1);
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) r8[x] = ldc(a.rowids + e0 + 8 * j + x);
}

// Select v[idx] from eight wave-uniform values with a per-lane idx (0..7).
__device__ __forceinline__ int select8(const int (&v)[8], int idx) {
  const int a0 = (idx & 1) ? v[1] : v[0], a1 = (idx & 1) ? v[3] : v[2];
  const int a2 = (idx & 1) ? v[5] : v[4], a3 = (idx & 1) ? v[7] : v[6];
  const int b0 = (idx & 2) ? a1 : a0, b1 = (idx & 2) ? a3 : a2;
  return (idx & 4) ? b1 : b0;
}

// Issue value wave j's six loads of a sparse FP8 unit: code slots j + 4m
// (rows 2s and 2s + 1, 512 bytes each, 32 lanes per row), rope slot j (rows
// 8j .. 8j+7, 128 bytes each, 8 lanes per row) and the scales of rows
// 8j .. 8j+7 (lanes 0..7).  Every row comes from its own cache row, so each
// lane carries a 64-bit address (global_load_lds); entries that do not
// count (row id -1) read the zero row, and every slot issues exactly one
// load, so a wave always has six loads per unit.  The LDS side keeps the
// dense FP8 unit layout and swizzles (code rows c ^ f8_code_swizzle(r), rope
// rows c ^ f8_rope_swizzle(r)); the scales go to f8sp_scale_off windows.
__device__ __forceinline__ void issue_half_load_f8_sparse(char* lds_buf, const DecodeArgs& a,
                                                          const int (&rc)[8], const int (&r8)[8],
                                                          int j) {
  const int lane = threadIdx.x & 63;
  const char* kc = reinterpret_cast<const char*>(a.kcache);
  const char* zr = reinterpret_cast<const char*>(a.zero_row);
  auto row_base = [&](int rid) {   // first byte of the row's page, and the row
    return kc + (long long)(rid >> 6) * kF8PageBytes;
  };
  const char* src[6];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = 2 * (j + 4 * m) + (lane >> 5);          // unit row of this lane
    const int rid = (lane >> 5) ? rc[2 * m + 1] : rc[2 * m];
    const int cb = ((lane & 31) ^ f8_code_swizzle(r)) << 4;
    src[m] = rid >= 0 ? row_base(rid) + (rid & 63) * kF8Latent + cb : zr + cb;
  }
  {
    const int r = 8 * j + (lane >> 3);
    const int rid = select8(r8, lane >> 3);
    const int cb = ((lane & 7) ^ f8_rope_swizzle(r)) << 4;
    src[4] = rid >= 0 ? row_base(rid) + kF8RopeOff + (rid & 63) * 128 + cb : zr + cb;
  }
  {
    const int rid = lane < 8 ? select8(r8, lane) : -1;
    src[5] = rid >= 0 ? row_base(rid) + kF8ScaleOff + (rid & 63) * 4 : zr;
  }
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MLA_LDS char*)(lds_buf)));
  const uint32_t m0c = uni(base + j * 1024);
  const uint32_t m0r = uni(base + kF8UnitRope + j * 1024);
  const uint32_t m0s = uni(base + kF8UnitScale + j * 256);
  asm volatile(
      "s_mov_b32 m0, %[c]\n\t"
      "s_nop 0\n\tglobal_load_lds_dwordx4 %[a0], off\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\tglobal_load_lds_dwordx4 %[a1], off\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\tglobal_load_lds_dwordx4 %[a2], off\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\tglobal_load_lds_dwordx4 %[a3], off\n\t"
      "s_mov_b32 m0, %[r]\n\t"
      "s_nop 0\n\tglobal_load_lds_dwordx4 %[a4], off\n\t"
      "s_mov_b32 m0, %[s]\n\t"
      "s_nop 0\n\tglobal_load_lds_dword %[a5], off\n\t"
      :
      : [c] "s"(m0c), [r] "s"(m0r), [s] "s"(m0s), [a0] "v"(src[0]), [a1] "v"(src[1]),
        [a2] "v"(src[2]), [a3] "v"(src[3]), [a4] "v"(src[4]), [a5] "v"(src[5])
      : "memory", "m0", "scc");
}

// Eight E4M3 codes (two dwords, code e in byte e) to bf16, exactly: every
// E4M3 value is a bf16 value.  Hardware conversion with a unit scale.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// RT: 16-row tiles in the workgroup tile (1, 2 or 4: 16, 32 or 64 query
// rows); score waves q >= RT have no rows and only keep step with the others.
// F8: the cache holds FP8 pages (layout above) instead of bf16 rows.
// SP: sparse mode: items of selected entries, rows gathered one by one
// (issue_half_load_sparse, or issue_half_load_f8_sparse over FP8 pages),
// entries that do not count masked.
template <int RT, bool F8, bool SP>
__global__ __launch_bounds__(kThreadsWS, 1) void mla_splitkv_ws_kernel(const DecodeArgs a) {
  constexpr int NBUF = F8 ? kWSBufsF8 : kWSBufs;          // ring of unit buffers
  constexpr int DL = 8;   // 16-dim output tiles per value wave (128 dims)
  constexpr int UB = F8 ? (SP ? kF8SpUnitBytes : kF8UnitBytes) : kHalfBytes;   // one unit buffer

  __shared__ __attribute__((aligned(1024))) char smem[NBUF * UB];
  __shared__ bf16x8 p_lds[2][RT][64];   // P^T operands: [unit parity][row tile][lane]
  __shared__ float alpha_lds[2][16 * RT];   // per-row rescale factor of the unit
  // per 16-row block q, byte q: any of its rows rescaled in the unit (one
  // dword, so the value waves test all blocks with one read; blocks without
  // rows keep the 0 written here)
  __shared__ uint32_t grow_lds[2];
  __shared__ float lfin_lds[2][16 * RT];    // per-row sum of a piece ending at the unit

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 2) grow_lds[tid] = 0u;   // ordered before every use by the first barrier
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int i = lane & 15;

  int part, rtile;
  const int x = blockIdx.x;
  const int R = a.row_tiles;
  if (R > 1 && (a.num_parts % 8) == 0) {
    part = (x / (8 * R)) * 8 + (x & 7);
    rtile = (x >> 3) % R;
  } else {
    part = x / R;
    rtile = x % R;
  }
  __shared__ int plan_lds[8];
  __shared__ int so_lds[kPlanMaxBatch + 1];   // split offsets (in-kernel plan)
  int b0, k0, b1, k1, first_split;
  const bool inplan = !SP && a.inplan;   // the sparse mode always reads its plan
  if (inplan) {
    if (w == 0) {
      plan_part_wave(a, part, plan_lds, so_lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (rtile == 0 && lane < kMetaInts)   // this part's entry, as the metadata kernel's
        a.tile_meta_out[part * kMetaInts + lane] = lane < 5 ? plan_lds[lane] : 0;
      if (part == 0 && rtile == 0)
        for (int b = lane; b <= a.batch; b += 64) a.split_offsets_out[b] = so_lds[b];
    }
    wg_barrier();   // the plan is in LDS for every wave
    b0 = uni(plan_lds[0]);
    k0 = uni(plan_lds[1]);
    b1 = uni(plan_lds[2]);
    k1 = uni(plan_lds[3]);
    first_split = uni(plan_lds[4]);
  } else {
    const int32_t* tm = a.tile_meta + part * kMetaInts;
    b0 = ldc(tm + 0);
    k0 = ldc(tm + 1);
    b1 = ldc(tm + 2);
    k1 = ldc(tm + 3);
    first_split = ldc(tm + 4);
  }

  int cb = b0, ck = k0, ch = 0;
  seek(a, cb, ck, b1, k1);
  if (!before_end(a, cb, ck, b1, k1)) return;  // uniform: empty part
  int cL = seqlen_of(a, cb);
  const int tile_row0 = rtile * 16 * RT;

  // Piece bookkeeping shared by both roles: a piece is the run of units of
  // one request inside the part.
  auto piece_slot = [&](int b, int pbeg, int pend, int n, bool& whole) {
    whole = pbeg == 0 && pend == n;
    const int sidx = (b == b0 && k0 > 0) ? first_split : 0;
    if (whole) return 0LL;
    return (long long)(inplan ? uni(so_lds[b]) : ldc(a.split_offsets + b)) + sidx;
  };

  if (w < 4) {
    // ======================= score waves =======================
    // The score waves carry the critical path of every phase (scores, then
    // the softmax chain); at a higher issue priority they take the SIMD first
    // and the value wave's products fill the gaps.
    __builtin_amdgcn_s_setprio(1);
    const int q = w;
    // uniform: this wave's 16-row block exists (s_q*h_q is a multiple of 16,
    // so a block is either all real rows or all beyond the last one)
    const bool active = q < RT && tile_row0 + 16 * q < a.M;
    const int row_own = tile_row0 + 16 * q + i;
    const int fi = lds_swizzle(i & 7);
    const int a_off0 = i * kRowBytes + (((0 + g) ^ fi) << 4);
    const int a_off1 = a_off0 ^ 64;   // unit 4+g instead of g (row bases are multiples of 128)
    // FP8 unit: code rows 16kt + i at unit (4p + g) ^ f8_code_swizzle(row),
    // i.e. address co[kt] ^ 64p; rope rows at unit (4s + g) ^ ((i >> 1) & 7),
    // i.e. (ro ^ 64s) + 2048kt
    int co[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      co[kt] = (16 * kt + i) * kF8Latent + ((g ^ f8_code_swizzle(16 * kt + i)) << 4);
    const int ro = kF8UnitRope + i * 128 + ((g ^ f8_rope_swizzle(i)) << 4);

    bf16x8 qreg[18];
    auto load_q = [&](int b) {
      const uint16_t* qrow = a.q + ((long long)b * a.M + row_own) * kDK;
      if constexpr (F8)
        load_q_rows_f8(qreg, reinterpret_cast<const bf16x8*>(qrow + 16 * g),
                       reinterpret_cast<const bf16x8*>(qrow + kF8Latent + 8 * g));
      else
        load_q_rows(qreg, reinterpret_cast<const bf16x8*>(qrow + 8 * g));
    };
    // Q of the first piece is loaded before the first barrier, so its latency
    // overlaps that of the first page loads instead of following them.
    if (active) load_q(cb);
    float m_run = -INFINITY, l_run = 0.f;
    int lim = 0, lim_min = 0, n = 0, pbeg = 0;
    bool new_piece = true;
    int t = 0;
    while (true) {
      wg_barrier();   // unit t landed; P of unit t-2 consumed
      const int b = cb, k = ck, h = ch;
      if (new_piece) {
        n = n_pages(cL);
        pbeg = k;
        lim_min = a.causal ? cL - a.s_q + 1 : cL;
        lim = a.causal ? cL - a.s_q + 1 + row_own / a.h_q : cL;
        m_run = -INFINITY;
        l_run = 0.f;
        if (active && t > 0) load_q(b);
      }
      const char* ubuf = smem + (t % NBUF) * UB;
      // sparse: which of the unit's 32 entries count (bit = key in the unit)
      const uint32_t vm = SP ? static_cast<uint32_t>(ldc(reinterpret_cast<const int32_t*>(a.vmask) +
                                                         (long long)b * (a.const_len / 32) + 2 * k + h))
                             : 0xffffffffu;
      if (active) {

      // ---- S^T[key][row] = K . Q^T: 32 keys x this wave's 16 rows ----
      f32x4 s[2];
      f32x4 sc[2];   // FP8: scales of the lane's keys 16kt + 4g + v
      if constexpr (!F8) {
        // Two accumulators per 16-key tile (even and odd 32-dim steps), so
        // four independent MFMA chains hide the accumulate latency.
        f32x4 sp[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 2; ++e) sp[kt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int D1 = 4;   // K steps read ahead of their products
        bf16x8 ka[D1 + 1][2];
#pragma unroll
        for (int ks = 0; ks < 18 + D1; ++ks) {
          if (ks < 18) {
            const char* ab = ubuf + ((ks & 1) ? a_off1 : a_off0) + 128 * (ks >> 1);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
              ka[ks % (D1 + 1)][kt] = *reinterpret_cast<const bf16x8*>(ab + kt * 16 * kRowBytes);
          }
          const int cs = ks - D1;
          if (cs >= 0) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
              sp[kt][cs & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  ka[cs % (D1 + 1)][kt], qreg[cs], sp[kt][cs & 1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[kt] = sp[kt][0] + sp[kt][1];
      } else {
        // Latent dims: raw E4M3 code products in two chains per key tile
        // (the scale is per key, so it multiplies the finished sum); rope
        // dims (bf16) in a third chain.
        f32x4 sp[2][2], sr[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          sp[kt][0] = sp[kt][1] = sr[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // Three-stage software pipeline over the 8 code reads (64 dims each):
        // read step ps, convert step ps-1, multiply step ps-2, so that the
        // conversions of one step overlap the products of the step before.
        u32x4 kc[2][2];
        bf16x8 kb[2][2][2];   // [step parity][kt][low / high 8 dims]
        bf16x8 ra[2][2];
#pragma unroll
        for (int ps = 0; ps < 8 + 2; ++ps) {
          if (ps < 8) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
              kc[ps & 1][kt] = *reinterpret_cast<const u32x4*>(ubuf + (co[kt] ^ (64 * ps)));
          }
          if (ps == 0) {
#pragma unroll
            for (int rs = 0; rs < 2; ++rs)
#pragma unroll
              for (int kt = 0; kt < 2; ++kt)
                ra[rs][kt] = *reinterpret_cast<const bf16x8*>(ubuf + (ro ^ (64 * rs)) + 2048 * kt);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
              sc[kt] = *reinterpret_cast<const f32x4*>(
                  ubuf + kF8UnitScale + (SP ? f8sp_scale_off(16 * kt + 4 * g) : 4 * (16 * kt + 4 * g)));
          }
          const int cv = ps - 1;   // step converted now
          if (cv >= 0 && cv < 8) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              const u32x4 w = kc[cv & 1][kt];
              kb[cv & 1][kt][0] = e4m3x8_to_bf16(w[0], w[1]);
              kb[cv & 1][kt][1] = e4m3x8_to_bf16(w[2], w[3]);
            }
          }
          const int cp = ps - 2;   // step multiplied now
          if (cp >= 0) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              sp[kt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[cp & 1][kt][0], qreg[2 * cp],
                                                                  sp[kt][0], 0, 0, 0);
              sp[kt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  kb[cp & 1][kt][1], qreg[2 * cp + 1], sp[kt][1], 0, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rs = 0; rs < 2; ++rs)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            sr[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[rs][kt], qreg[16 + rs], sr[kt],
                                                             0, 0, 0);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[kt] = sc[kt] * (sp[kt][0] + sp[kt][1]) + sr[kt];
      }

      // ---- online softmax of row_own (fp32, base 2, lazy rescale) ----
      {
        const int key0 = k * kBlock + h * kHalfRows + 4 * g;
        const bool need_mask = k * kBlock + (h + 1) * kHalfRows > lim_min;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float xv = s[kt][v] * a.scale_log2;
            if (need_mask && key0 + kt * 16 + v >= lim) xv = -INFINITY;
            if (SP && !((vm >> (kt * 16 + 4 * g + v)) & 1u)) xv = -INFINITY;
            s[kt][v] = xv;
            mx = fmaxf(mx, xv);
          }
        mx = wave_max_4lanes(mx);
        const float m_new = fmaxf(m_run, mx);
        // Keep the running max unless it grew by more than kRescaleSlack
        // (exact either way: numerator and denominator share it).
        const bool grow = m_new > m_run + kRescaleSlack;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        if (grow) m_run = m_new;
        l_run *= alpha;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float lsum = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = __builtin_amdgcn_exp2f(s[kt][v] - m_use);
            lsum += p;
            // FP8: the value operand holds raw codes, so P carries the key's scale
            pb[kt * 4 + v] = (__bf16)(F8 ? p * sc[kt][v] : p);
          }
        l_run += lsum;
        p_lds[t & 1][q][lane] = pb;
        if (g == 0) alpha_lds[t & 1][16 * q + i] = alpha;
        const int any = __any(grow) ? 1 : 0;
        if (lane == 0) reinterpret_cast<uint8_t*>(&grow_lds[t & 1])[q] = static_cast<uint8_t>(any);
      }
      }   // active

      // ---- next unit; at a piece end publish the row sum and write the LSE ----
      unit_next(a, cb, ck, ch, cL, b1, k1);
      const bool more = before_end(a, cb, ck, b1, k1);
      new_piece = !(more && cb == b);
      if (new_piece && active) {
        const float lt = wave_sum_4lanes(l_run);
        const float lse2 = lt > 0.f ? m_run + log2f(lt) : -INFINITY;
        bool whole;
        const long long slot = piece_slot(b, pbeg, (b == b1) ? k1 : n, n, whole);
        if (g == 0) {
          lfin_lds[t & 1][16 * q + i] = lt;
          if (whole)
            a.lse[(long long)b * a.M + row_own] = lse2 * kLn2;
          else
            a.part_lse[slot * a.M + row_own] = lse2;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // P, alpha, flags, sums written
      ++t;
      if (!more) break;
    }
    wg_barrier();   // the value waves' last product may start
  } else {
    // ======================= value waves =======================
    const int j = w - 4;
    const int tj = tid - 256;   // 0..255 within the value waves
    int off[9];
#pragma unroll
    for (int m = 0; m < 9; ++m) {
      const int p = 256 * m + tj;   // LDS 16-byte unit of the 36 KB unit buffer
      const int r = p / kChunksPerRow;
      const int pc = p - r * kChunksPerRow;
      off[m] = r * kRowBytes + ((pc ^ lds_swizzle(r)) << 4);
    }
    const int tr_row = 4 * g + (i >> 2);
    const int ft = lds_swizzle(tr_row & 7);
    const int hh = (i & 3) >> 1;
    int t_off[4];
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
      t_off[d4] = 256 * j + tr_row * kRowBytes + (((2 * d4 + hh) ^ ft) << 4) + ((i & 1) << 3);

    // FP8 unit: direct-load offsets (code slots j + 4m, rope slot j, scales)
    // and the transposed code read: lanes 2e, 2e+1 of a 16-lane group point
    // at the two 8-byte halves of key row kap(g, e) (the keys of P's element
    // e), dims 128j + 16dl .. +16, so lane i receives dim i of all 8 keys.
    // sparse: the lane's byte offset inside its row and whether its row is
    // the second one of the slot (see issue_half_load_sparse)
    int sp_coff[9];
    bool sp_rsel[9];
#pragma unroll
    for (int m = 0; m < 9; ++m) {
      const int p = 256 * m + tj;
      const int r = p / kChunksPerRow;
      sp_coff[m] = ((p - r * kChunksPerRow) ^ lds_swizzle(r)) << 4;
      sp_rsel[m] = r > (256 * m + 64 * j) / kChunksPerRow;
    }
    int offc[4], offr, offs, f8_t0;
    {
      const int lane = tid & 63;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int p = 64 * (j + 4 * m) + lane;   // 16-byte unit of the code region
        const int r = p >> 5;
        offc[m] = r * kF8Latent + (((p & 31) ^ f8_code_swizzle(r)) << 4);
      }
      const int pr = 64 * j + lane;               // 16-byte unit of the rope region
      const int rr = pr >> 3;
      offr = rr * 128 + (((pr & 7) ^ f8_rope_swizzle(rr)) << 4);
      offs = 4 * lane;
      const int e = i >> 1;
      const int kap = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
      f8_t0 = kap * kF8Latent + ((i & 1) << 3) + (((8 * j) ^ f8_code_swizzle(kap)) << 4);
    }

    f32x4 o[DL][RT];
#pragma unroll
    for (int dl = 0; dl < DL; ++dl)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) o[dl][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // issue cursor (ib, ik, ih); compute cursor (cb, ck, ch) is one unit behind
    // the score waves
    int ib = cb, ik = ck, ih = 0, iL = cL;
    int issued = 0;
    int sp_rlo[9], sp_rhi[9];   // sparse: row ids of the next unit to issue
    int f8_rc[8], f8_r8[8];     // sparse over FP8 pages: the same
    auto load_rowids = [&]() {
      if constexpr (SP && F8)
        load_sparse_rowids_f8(a, ib, ik, ih, j, f8_rc, f8_r8);
      else if constexpr (SP)
        load_sparse_rowids(a, ib, ik, ih, j, sp_rlo, sp_rhi);
    };
    if constexpr (SP) load_rowids();
    auto issue_next = [&]() {
      if (before_end(a, ib, ik, b1, k1)) {
        if constexpr (F8 && SP)
          issue_half_load_f8_sparse(smem + (issued % NBUF) * UB, a, f8_rc, f8_r8, j);
        else if constexpr (F8)
          issue_half_load_f8(smem + (issued % NBUF) * UB, a, ib, ik, ih, offc, offr, offs, j);
        else if constexpr (SP)
          issue_half_load_sparse(smem + (issued % NBUF) * UB, a, sp_rlo, sp_rhi, sp_coff,
                                 sp_rsel, j);
        else
          issue_half_load(smem + (issued % NBUF) * kHalfBytes, a, ib, ik, ih, off, j);
        ++issued;
        unit_next(a, ib, ik, ih, iL, b1, k1);
        if constexpr (SP)
          if (before_end(a, ib, ik, b1, k1)) load_rowids();
      }
    };
    // wait until unit u has landed (units issued after it stay in flight)
    // (loads per unit and wave: 9 for bf16; for FP8 6 on wave 0, 5 on the
    // others; 6 on every wave for sparse FP8)
    auto wait_unit = [&](int u) {
      const int ahead = issued - u - 1;
      if constexpr (!F8)
        wait_loads_behind<kHalfLoadsPerWave, NBUF - 2>(ahead);
      else if constexpr (SP)
        wait_loads_behind<6, NBUF - 2>(ahead);
      else if (j == 0)
        wait_loads_behind<6, NBUF - 2>(ahead);
      else
        wait_loads_behind<5, NBUF - 2>(ahead);
    };

    // Loads spread over the value product (bf16 dense cache, 32 or 64 rows):
    // slot 0 at the start of the phase, slot dl + 1 before the products of
    // output tile dl.
    constexpr bool kSpread = !F8 && !SP && RT >= 2;
    HalfLoad hl;
    bool hl_on = false;

    // V operands of the value product (bf16 cache), transposed reads
    bf16x8 va[DL];
    auto read_v = [&](const char* ub) {
#pragma unroll
      for (int dl = 0; dl < DL; ++dl) {
        const char* tb = ub + t_off[dl & 3] + 128 * (dl >> 2);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(tb));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(tb + 16 * kRowBytes));
        va[dl] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };

    for (int u = 0; u < NBUF - 1; ++u) issue_next();   // units 0 .. NBUF-2
    wait_unit(0);
    wg_barrier();   // b_0: unit 0 landed
    issue_next();   // unit NBUF-1 (its buffer is still unused)
    wait_unit(1);
    wg_barrier();   // b_1: unit 1 landed, P of unit 0 written

    int n = n_pages(cL), pbeg = ck;
    int t = 0;   // unit multiplied in this phase
    while (true) {
      // Unit t+NBUF-1 goes into the buffer of unit t-1, free since the last
      // barrier (its product ended in the previous phase); issued first so
      // that it has NBUF-2 phases to land.
      if (t >= 1) {
        if constexpr (kSpread) {
          hl_on = before_end(a, ib, ik, b1, k1);
          if (hl_on) {
            hl = half_load_setup(smem + (issued % NBUF) * kHalfBytes, a, ib, ik, ih, j);
            ++issued;
            unit_next(a, ib, ik, ih, iL, b1, k1);
            half_load_slot(hl, off[0], 0);
          }
        } else {
          issue_next();
        }
      }
      const int b = cb;
      const char* ubuf = smem + (t % NBUF) * UB;
      const int par = t & 1;

      // ---- O^T[dim][row] += V^T . P^T: this wave's 128 dims, all rows ----
      // With 32 or 64 rows every LDS operand of the unit is requested at once
      // (one round trip; the rescale factors read as volatile so that the
      // compiler does not sink them into the rescale branch, a second round
      // trip).  With 16 rows (memory-bound) V is read after the rescale, which
      // measured faster there.
      constexpr bool kEarlyV = RT >= 2;
      const bool grown = grow_lds[par] != 0u;
      float al[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        al[rt] = kEarlyV ? *(volatile MLA_LDS float*)(&alpha_lds[par][16 * rt + i])
                         : alpha_lds[par][16 * rt + i];
      bf16x8 pB[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) pB[rt] = p_lds[par][rt][lane];
      i32x2 vc[DL];   // FP8: transposed code reads
      auto read_vc = [&]() {
        if constexpr (F8) {
#pragma unroll
          for (int dl = 0; dl < DL; ++dl)
            vc[dl] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (MLA_LDS i32x2*)((MLA_LDS char*)(ubuf) + (f8_t0 ^ (dl << 4))));
        } else {
          read_v(ubuf);
        }
      };
      if constexpr (kEarlyV) read_vc();
      if (grown) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) o[dl][rt] *= al[rt];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!kEarlyV) read_vc();
      {
        if constexpr (F8) {
          // codes converted one 16-dim tile ahead of its products
          bf16x8 cur = e4m3x8_to_bf16(vc[0][0], vc[0][1]);
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) {
            bf16x8 nxt = cur;
            if (dl + 1 < DL) nxt = e4m3x8_to_bf16(vc[dl + 1][0], vc[dl + 1][1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              o[dl][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pB[rt], o[dl][rt], 0, 0, 0);
            cur = nxt;
          }
        } else {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) {
            if constexpr (kSpread) {
              if (hl_on) half_load_slot(hl, off[dl + 1], dl + 1);
              __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              o[dl][rt] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dl], pB[rt], o[dl][rt], 0, 0, 0);
          }
        }
      }

      // ---- next unit; at a piece end write O (by columns) and restart ----
      unit_next(a, cb, ck, ch, cL, b1, k1);
      const bool more = before_end(a, cb, ck, b1, k1);
      if (!(more && cb == b)) {
        bool whole;
        const long long slot = piece_slot(b, pbeg, (b == b1) ? k1 : n, n, whole);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float lt = lfin_lds[par][16 * rt + i];
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          const int row = tile_row0 + 16 * rt + i;
          if (tile_row0 + 16 * rt >= a.M) {   // rows past the last query row
          } else if (whole) {
            uint16_t* op = a.out + ((long long)b * a.M + row) * kDV + j * 128 + 4 * g;
#pragma unroll
            for (int dl = 0; dl < DL; ++dl) {
              const f32x4 v = o[dl][rt] * inv;
              const bf16x4 bv = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
              *reinterpret_cast<bf16x4*>(op + dl * 16) = bv;
            }
          } else {
            float* op = a.part_o + (slot * a.M + row) * kDV + j * 128 + 4 * g;
#pragma unroll
            for (int dl = 0; dl < DL; ++dl)
              *reinterpret_cast<f32x4*>(op + dl * 16) = o[dl][rt] * inv;
          }
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) o[dl][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          __builtin_amdgcn_sched_barrier(0);
        }
        if (more) {
          n = n_pages(cL);
          pbeg = ck;
        }
      }
      if (!more) break;
      wait_unit(t + 2);
      wg_barrier();   // b_{t+2}: unit t+2 landed, P of unit t+1 written
      ++t;
    }
  }
}

// Rows per workgroup tile.
int tile_rows_for(int M) {
  if (M <= 16) return 16;    // mla_splitkv_ws_kernel<1>
  if (M <= 32) return 32;    // mla_splitkv_ws_kernel<2>
  return 64;                 // mla_splitkv_ws_kernel<4> (M = 128, 256: 2 or 4 row tiles)
}

template <int RT, bool F8, bool SP = false>
hipError_t launch_ws(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 grid(a.num_parts * a.row_tiles);
  const dim3 block(kThreadsWS);
  if (start == nullptr && stop == nullptr) {
    // plain launch (also what a HIP graph capture records)
    hipLaunchKernelGGL((mla_splitkv_ws_kernel<RT, F8, SP>), grid, block, 0, stream, a);
  } else {
    // events recorded at the kernel's own start and end
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(&mla_splitkv_ws_kernel<RT, F8, SP>),
                                      grid, block, args, 0, stream, start, stop, 0);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_splitkv(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  if (a.sparse && a.kv_fp8) {
    if (a.row_tile_rows == 16) return launch_ws<1, true, true>(a, stream, start, stop);
    if (a.row_tile_rows == 32) return launch_ws<2, true, true>(a, stream, start, stop);
    return launch_ws<4, true, true>(a, stream, start, stop);
  }
  if (a.sparse) {
    if (a.row_tile_rows == 16) return launch_ws<1, false, true>(a, stream, start, stop);
    if (a.row_tile_rows == 32) return launch_ws<2, false, true>(a, stream, start, stop);
    return launch_ws<4, false, true>(a, stream, start, stop);
  }
  if (a.kv_fp8) {
    if (a.row_tile_rows == 16) return launch_ws<1, true>(a, stream, start, stop);
    if (a.row_tile_rows == 32) return launch_ws<2, true>(a, stream, start, stop);
    return launch_ws<4, true>(a, stream, start, stop);
  }
  if (a.row_tile_rows == 16) return launch_ws<1, false>(a, stream, start, stop);
  if (a.row_tile_rows == 32) return launch_ws<2, false>(a, stream, start, stop);
  return launch_ws<4, false>(a, stream, start, stop);
}

// --------------------------------------------------------------------------
// LSE combine: exact merge of the split partials of each split request.
// One workgroup per (request, 16 query rows, quarter of the 512 output dims):
// 16 threads per row, 8 dims each (2 x float4, interleaved so that a row's
// 16 threads read 256 contiguous bytes per step).  Splitting the dims keeps
// a few hundred workgroups in flight even for small batches.
// --------------------------------------------------------------------------
constexpr int kCombineQuarters = 4;

__global__ __launch_bounds__(kThreads) void mla_combine_kernel(const CombineArgs a) {
  const int b = blockIdx.x;
  const int r = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int dq = blockIdx.z * (kDV / kCombineQuarters);   // first dim of this quarter
  const int j = threadIdx.x & 15;
  if (r >= a.M) return;
  const int s0 = a.split_offsets[b];
  const int ns = a.split_offsets[b + 1] - s0;
  uint16_t* op = a.out + ((long long)b * a.M + r) * kDV + dq;
  if (ns == 0) {
    if ((a.const_len > 0 ? a.const_len : a.seqlens[b]) <= 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *reinterpret_cast<uint2*>(op + (j + 16 * c) * 4) = make_uint2(0u, 0u);
      if (j == 0 && blockIdx.z == 0) a.lse[(long long)b * a.M + r] = -INFINITY;
    }
    return;
  }
  // Merge in groups of four partials: each group's loads (LSEs and rows) go
  // out together, then fold into a running (max, weight sum, weighted row),
  // the same exact log-sum-exp merge in a streaming order.
  constexpr int G = 4;
  float mx = -INFINITY, tot = 0.f;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int s = 0; s < ns; s += G) {
    float ls[G];
    f32x4 po[G][2];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const bool ok = s + u < ns;
      const long long rowi = (long long)(s0 + (ok ? s + u : 0)) * a.M + r;
      ls[u] = ok ? a.part_lse[rowi] : -INFINITY;
      const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + rowi * kDV + dq);
#pragma unroll
      for (int c = 0; c < 2; ++c) po[u][c] = src[j + 16 * c];
    }
    float gm = mx;
#pragma unroll
    for (int u = 0; u < G; ++u) gm = fmaxf(gm, ls[u]);
    if (gm == -INFINITY) continue;   // every partial so far is empty
    const float al = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - gm);
    tot *= al;
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[c] *= al;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float wgt = ls[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[u] - gm);
      tot += wgt;
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[c] += wgt * po[u][c];
    }
    mx = gm;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const f32x4 v = acc[c] * inv;
    const bf16x4 bv = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4*>(op + (j + 16 * c) * 4) = bv;
  }
  if (j == 0 && blockIdx.z == 0)
    a.lse[(long long)b * a.M + r] = tot > 0.f ? (mx + log2f(tot)) * kLn2 : -INFINITY;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.batch, (a.M + 15) / 16, kCombineQuarters), block(kThreads);
  hipLaunchKernelGGL(mla_combine_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Paged-KV append: one workgroup per (request, new token); 72 lanes copy the
// 1152-byte row as 16-byte words.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(128) void mla_kv_append_kernel(
    const uint16_t* __restrict__ new_kv, uint16_t* __restrict__ kcache, long long num_blocks,
    const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ seqlens, int s_q) {
  const int b = blockIdx.x, t = blockIdx.y;
  const int c = threadIdx.x;
  if (c >= kChunksPerRow) return;
  const int pos = seqlens[b] - s_q + t;
  if (pos < 0 || pos / kBlock >= bt_stride) return;
  const int page = block_table[(long long)b * bt_stride + pos / kBlock];
  if (page < 0 || (long long)page >= num_blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(new_kv + ((long long)b * s_q + t) * kDK);
  uint4* dst = reinterpret_cast<uint4*>(kcache + ((long long)page * kBlock + pos % kBlock) * kDK);
  dst[c] = src[c];
}

hipError_t launch_kv_append(const uint16_t* new_kv, uint16_t* kcache, long long num_blocks,
                            const int32_t* block_table, int bt_stride, const int32_t* seqlens,
                            int batch, int s_q, hipStream_t stream) {
  hipLaunchKernelGGL(mla_kv_append_kernel, dim3(batch, s_q), dim3(128), 0, stream, new_kv,
                     kcache, num_blocks, block_table, bt_stride, seqlens, s_q);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Paged-KV append into FP8 pages: one wave per (request, new token).  Lane l
// quantises latent dims 8l .. 8l+7; the scale is the smallest power of two
// s with amax <= 448 s (1 for an all-zero latent), so x / s is exact and
// every code is the E4M3 round-to-nearest-even of an exact value.
// --------------------------------------------------------------------------
// E4M3 code of y (|y| <= 448), ties to even, from the format's fields: sign
// bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0
// holds the subnormals m * 2^-9.  The sign of -0 and of negative values that
// round to zero is kept.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) {                          // below 2^-6: grid of 2^-9
    return sign | static_cast<uint32_t>(rintf(a * 512.0f));   // 8 = smallest normal
  }
  int e;
  frexpf(a, &e);
  e -= 1;                                       // a in [2^e, 2^(e+1))
  uint32_t n = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));   // 8 .. 16
  if (n == 16) {
    n = 8;
    e += 1;
  }
  return sign | (static_cast<uint32_t>(e + 7) << 3) | (n - 8);
}

__global__ __launch_bounds__(64) void mla_kv_append_fp8_kernel(
    const uint16_t* __restrict__ new_kv, uint8_t* __restrict__ kcache, long long num_blocks,
    const int32_t* __restrict__ block_table, int bt_stride, const int32_t* __restrict__ seqlens,
    int s_q) {
  const int b = blockIdx.x, t = blockIdx.y;
  const int lane = threadIdx.x;
  const int pos = seqlens[b] - s_q + t;
  if (pos < 0 || pos / kBlock >= bt_stride) return;
  const int page = block_table[(long long)b * bt_stride + pos / kBlock];
  if (page < 0 || (long long)page >= num_blocks) return;
  const int r = pos % kBlock;
  const uint16_t* src = new_kv + ((long long)b * s_q + t) * kDK;
  uint8_t* pg = kcache + (long long)page * kF8PageBytes;

  const uint4 w = reinterpret_cast<const uint4*>(src)[lane];
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(wd[k] << 16);
    x[2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int ks = 0;   // s = 2^ks
  if (amax > 0.f) {
    int e;
    frexpf(amax, &e);   // amax = m 2^e, m in [0.5, 1); 448 = 0.875 * 2^9
    ks = (amax <= ldexpf(448.0f, e - 9)) ? e - 9 : e - 8;
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lo |= e4m3_rne(ldexpf(x[k], -ks)) << (8 * k);
    hi |= e4m3_rne(ldexpf(x[4 + k], -ks)) << (8 * k);
  }
  *reinterpret_cast<uint2*>(pg + r * kF8Latent + 8 * lane) = make_uint2(lo, hi);
  if (lane < 8)
    reinterpret_cast<uint4*>(pg + kF8RopeOff + r * 128)[lane] =
        reinterpret_cast<const uint4*>(src + kF8Latent)[lane];
  if (lane == 0) *reinterpret_cast<float*>(pg + kF8ScaleOff + 4 * r) = ldexpf(1.0f, ks);
}

hipError_t launch_kv_append_fp8(const uint16_t* new_kv, uint8_t* kcache, long long num_blocks,
                                const int32_t* block_table, int bt_stride,
                                const int32_t* seqlens, int batch, int s_q, hipStream_t stream) {
  hipLaunchKernelGGL(mla_kv_append_fp8_kernel, dim3(batch, s_q), dim3(64), 0, stream, new_kv,
                     kcache, num_blocks, block_table, bt_stride, seqlens, s_q);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Sparse mode, step 0: each selected position of item (request b, token t)
// becomes a cache row id (page * 64 + row) or -1 if the entry does not count
// (negative, at or beyond the token's visible limit, page slot outside the
// table or page id outside the pool), plus one validity bit per entry.
// One thread per entry; a wave covers 64 entries, i.e. two mask words.
// Block (0, 0) also writes the zero row that skipped entries are loaded from.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_sparse_resolve_kernel(
    const int32_t* __restrict__ indices, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ seqlens, long long num_blocks, int s_q, int topk, int causal,
    int32_t* __restrict__ rowids, uint32_t* __restrict__ vmask, uint4* __restrict__ zero_row) {
  const int item = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kChunksPerRow)
    zero_row[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  const int b = item / s_q, t = item - b * s_q;
  const int L = seqlens[b];
  int vis = causal ? L - s_q + 1 + t : L;
  vis = vis < 0 ? 0 : (vis > L ? L : vis);
  int rid = -1;
  if (e < topk) {
    const int pos = indices[(long long)item * topk + e];
    if (pos >= 0 && pos < vis && pos / kBlock < bt_stride) {
      const int page = block_table[(long long)b * bt_stride + pos / kBlock];
      if (page >= 0 && (long long)page < num_blocks) rid = page * kBlock + pos % kBlock;
    }
    rowids[(long long)item * topk + e] = rid;
  }
  const unsigned long long bal = __ballot(rid >= 0);
  const int lane = threadIdx.x & 63;
  if ((lane == 0 || lane == 32) && e < topk)
    vmask[((long long)item * topk + e) / 32] = static_cast<uint32_t>(lane == 0 ? bal : bal >> 32);
}

hipError_t launch_sparse_resolve(const int32_t* indices, const int32_t* block_table,
                                 int bt_stride, const int32_t* seqlens, long long num_blocks,
                                 int batch, int s_q, int topk, int causal, int32_t* rowids,
                                 uint32_t* vmask, void* zero_row, hipStream_t stream) {
  const dim3 grid(batch * s_q, (topk + 255) / 256);
  hipLaunchKernelGGL(mla_sparse_resolve_kernel, grid, dim3(256), 0, stream, indices, block_table,
                     bt_stride, seqlens, num_blocks, s_q, topk, causal, rowids, vmask,
                     static_cast<uint4*>(zero_row));
  return hipGetLastError();
}

}  // namespace mla
