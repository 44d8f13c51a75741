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

// Part and row tile of workgroup x (grid = num_parts x row tiles R).
// Workgroups are dealt to the eight XCDs in turn (x mod 8), each XCD with its
// own L2; with R > 1 the R row tiles of a part (which read the same pages)
// go to one XCD.  In the sparse mode (CONTIG; R = 1) every item is split into
// the same number of consecutive parts, which all read the item's Q, so each
// XCD takes a contiguous run of num_parts / 8 parts and reads an item's Q
// through one L2 (top-2048 sparse 2 % faster, both cache formats; the same
// map made the dense long-context workload 1.6 % slower, so dense parts keep
// x mod 8).
__device__ __forceinline__ void part_of_block(int x, int R, int P, bool contig, int& part,
                                              int& rtile) {
  if (P % 8 == 0 && R > 1) {
    part = (x / (8 * R)) * 8 + (x & 7);
    rtile = (x >> 3) % R;
  } else if (P % 8 == 0 && contig) {
    part = (x & 7) * (P / 8) + (x >> 3);
    rtile = 0;
  } else {
    part = x / R;
    rtile = x % R;
  }
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

// The page id in table slot k of request b; -1 for a slot at or beyond the
// table's column count.
__device__ __forceinline__ int unit_page(const DecodeArgs& a, int b, int k) {
  return k < a.bt_stride ? ldc(a.block_table + (long long)b * a.bt_stride + k) : -1;
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

// Advance (b, k) to the part's next page (L: the length of request b).
__device__ __forceinline__ void page_next(const DecodeArgs& a, int& b, int& k, int& L, int b1,
                                          int k1) {
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
// With one tile (dense mode) the unit's two 16-key tiles are split instead:
// score waves 0 and 1 both take the 16 rows, wave q the keys 16q .. 16q+15
// of every unit, each with its own online softmax over its key tile, and the
// value waves keep one accumulator per key tile; the two are merged exactly
// (the log-sum-exp merge of two key sets) when a piece ends.
// F8: the cache holds FP8 pages (layout above) instead of bf16 rows.
// SP: sparse mode: items of selected entries, rows gathered one by one
// (issue_half_load_sparse, or issue_half_load_f8_sparse over FP8 pages),
// entries that do not count masked.
template <int RT, bool F8, bool SP>
__global__ __launch_bounds__(kThreadsWS, 1) void mla_splitkv_ws_kernel(const DecodeArgs a) {
  constexpr int NBUF = F8 ? kWSBufsF8 : kWSBufs;          // ring of unit buffers
  constexpr int DL = 8;   // 16-dim output tiles per value wave (128 dims)
  constexpr int UB = F8 ? (SP ? kF8SpUnitBytes : kF8UnitBytes) : kHalfBytes;   // one unit buffer
  constexpr bool KS = RT == 1 && !SP;   // key tiles split over two score waves
  constexpr int NR = KS ? 2 : RT;       // softmax streams: row tiles, or key tiles

  __shared__ __attribute__((aligned(1024))) char smem[NBUF * UB];
  // P^T operands: [unit parity][row tile][lane]; with KS, score wave q fills
  // the 8-byte half q of every lane's operand (its key tile's elements)
  __shared__ bf16x8 p_lds[2][RT][64];
  __shared__ float alpha_lds[2][16 * NR];   // per-row rescale factor of the unit (per stream)
  // per 16-row block q, byte q: any of its rows rescaled in the unit (one
  // dword, so the value waves test all blocks with one read; blocks without
  // rows keep the 0 written here)
  __shared__ uint32_t grow_lds[2];
  __shared__ float lfin_lds[2][16 * NR];    // per-row sum of a piece ending at the unit
  __shared__ float mfin_lds[2][KS ? 32 : 1];  // KS: per-row reference of each key tile's sum

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 2) grow_lds[tid] = 0u;   // ordered before every use by the first barrier
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int i = lane & 15;

  int part, rtile;
  part_of_block(blockIdx.x, a.row_tiles, a.num_parts, SP, part, rtile);
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
    const bool active = KS ? (q < 2 && tile_row0 < a.M) : (q < RT && tile_row0 + 16 * q < a.M);
    const int row_own = tile_row0 + (KS ? 0 : 16 * q) + i;
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
    // dense mode: the page id of the unit (loaded before the barrier that
    // precedes the unit); a slot that names no page of the pool holds no keys
    int pg = SP ? 0 : unit_page(a, cb, ck);
    int t = 0;
    while (true) {
      wg_barrier();   // unit t landed; P of unit t-2 consumed
      const int b = cb, k = ck, h = ch;
      const bool pvalid = SP || (pg >= 0 && (long long)pg < a.num_blocks);
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
      if constexpr (KS) {
        if (active) {
          // ---- S^T[key][row] = K . Q^T: this wave's 16 keys x the 16 rows ----
          f32x4 s1;
          f32x4 sc1 = f32x4{1.f, 1.f, 1.f, 1.f};   // FP8: scales of the lane's keys 16q + 4g + v
          if constexpr (!F8) {
            f32x4 sp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            constexpr int D1 = 4;   // K steps read ahead of their products
            bf16x8 ka[D1 + 1];
            const char* kbase = ubuf + q * 16 * kRowBytes;
#pragma unroll
            for (int ks = 0; ks < 18 + D1; ++ks) {
              if (ks < 18)
                ka[ks % (D1 + 1)] = *reinterpret_cast<const bf16x8*>(
                    kbase + ((ks & 1) ? a_off1 : a_off0) + 128 * (ks >> 1));
              const int cs = ks - D1;
              if (cs >= 0)
                sp[cs & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[cs % (D1 + 1)], qreg[cs],
                                                                     sp[cs & 1], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
            s1 = sp[0] + sp[1];
          } else {
            // the same three-stage pipeline as below, over one key tile
            f32x4 sp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            f32x4 sr = f32x4{0.f, 0.f, 0.f, 0.f};
            const int cq = q ? co[1] : co[0];
            u32x4 kc[2];
            bf16x8 kb[2][2];
            bf16x8 ra[2];
#pragma unroll
            for (int ps = 0; ps < 8 + 2; ++ps) {
              if (ps < 8) kc[ps & 1] = *reinterpret_cast<const u32x4*>(ubuf + (cq ^ (64 * ps)));
              if (ps == 0) {
#pragma unroll
                for (int rs = 0; rs < 2; ++rs)
                  ra[rs] = *reinterpret_cast<const bf16x8*>(ubuf + (ro ^ (64 * rs)) + 2048 * q);
                sc1 = *reinterpret_cast<const f32x4*>(ubuf + kF8UnitScale + 4 * (16 * q + 4 * g));
              }
              const int cv = ps - 1;
              if (cv >= 0 && cv < 8) {
                const u32x4 wv = kc[cv & 1];
                kb[cv & 1][0] = e4m3x8_to_bf16(wv[0], wv[1]);
                kb[cv & 1][1] = e4m3x8_to_bf16(wv[2], wv[3]);
              }
              const int cp = ps - 2;
              if (cp >= 0) {
                sp[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[cp & 1][0], qreg[2 * cp], sp[0],
                                                                0, 0, 0);
                sp[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[cp & 1][1], qreg[2 * cp + 1],
                                                                sp[1], 0, 0, 0);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rs = 0; rs < 2; ++rs)
              sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[rs], qreg[16 + rs], sr, 0, 0, 0);
            s1 = sc1 * (sp[0] + sp[1]) + sr;
          }

          // ---- online softmax of row_own over this key tile ----
          const int key0 = k * kBlock + h * kHalfRows + 16 * q + 4 * g;
          const bool need_mask = !pvalid || k * kBlock + (h + 1) * kHalfRows > lim_min;
          const int lim_u = pvalid ? lim : -1;
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float xv = s1[v] * a.scale_log2;
            if (need_mask && key0 + v >= lim_u) xv = -INFINITY;
            s1[v] = xv;
            mx = fmaxf(mx, xv);
          }
          mx = wave_max_4lanes(mx);
          const float m_new = fmaxf(m_run, mx);
          const bool grow = m_new > m_run + kRescaleSlack;
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          if (grow) m_run = m_new;
          l_run *= alpha;
          const float m_use = m_run == -INFINITY ? 0.f : m_run;
          float lsum = 0.f;
          bf16x4 pb;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = __builtin_amdgcn_exp2f(s1[v] - m_use);
            lsum += p;
            pb[v] = (__bf16)(F8 ? p * sc1[v] : p);
          }
          l_run += lsum;
          reinterpret_cast<bf16x4*>(&p_lds[t & 1][0][lane])[q] = pb;
          if (g == 0) alpha_lds[t & 1][16 * q + i] = alpha;
          const int any = __any(grow) ? 1 : 0;
          if (lane == 0) reinterpret_cast<uint8_t*>(&grow_lds[t & 1])[q] = static_cast<uint8_t>(any);
        }
      } else {
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
        const bool need_mask = !pvalid || k * kBlock + (h + 1) * kHalfRows > lim_min;
        const int lim_u = pvalid ? lim : -1;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float xv = s[kt][v] * a.scale_log2;
            if (need_mask && key0 + kt * 16 + v >= lim_u) xv = -INFINITY;
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
      }   // !KS

      // ---- next unit; at a piece end publish the row sum and write the LSE ----
      unit_next(a, cb, ck, ch, cL, b1, k1);
      const bool more = before_end(a, cb, ck, b1, k1);
      new_piece = !(more && cb == b);
      if (new_piece && active) {
        const float lt = wave_sum_4lanes(l_run);
        if constexpr (KS) {
          // the value waves merge the two key tiles and write the LSE
          if (g == 0) {
            lfin_lds[t & 1][16 * q + i] = lt;
            mfin_lds[t & 1][16 * q + i] = m_run;
          }
        } else {
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
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // P, alpha, flags, sums written
      ++t;
      if (!more) break;
      if (!SP) pg = unit_page(a, cb, ck);
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
    f32x4 o2[KS ? DL : 1];   // KS: the accumulator of key tile 1 (o holds key tile 0)
#pragma unroll
    for (int dl = 0; dl < DL; ++dl) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) o[dl][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KS) o2[dl] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

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
      // KS: the two key tiles' operands, each with the other tile's keys zero
      float al2 = 1.f;
      bf16x8 pK0 = pB[0], pK1 = pB[0];
      if constexpr (KS) {
        al2 = alpha_lds[par][16 + i];
        const u32x4 pw = __builtin_bit_cast(u32x4, pB[0]);
        pK0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], 0u, 0u});
        pK1 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, pw[2], pw[3]});
      }
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
        if constexpr (KS) {
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) o2[dl] *= al2;
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
            if constexpr (KS) {
              o[dl][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pK0, o[dl][0], 0, 0, 0);
              o2[dl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pK1, o2[dl], 0, 0, 0);
            } else {
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                o[dl][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pB[rt], o[dl][rt], 0, 0, 0);
            }
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
            if constexpr (KS) {
              o[dl][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dl], pK0, o[dl][0], 0, 0, 0);
              o2[dl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dl], pK1, o2[dl], 0, 0, 0);
            } else {
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                o[dl][rt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dl], pB[rt], o[dl][rt], 0, 0, 0);
            }
          }
        }
      }

      // ---- next unit; at a piece end write O (by columns) and restart ----
      unit_next(a, cb, ck, ch, cL, b1, k1);
      const bool more = before_end(a, cb, ck, b1, k1);
      if (!(more && cb == b)) {
        bool whole;
        const long long slot = piece_slot(b, pbeg, (b == b1) ? k1 : n, n, whole);
        // KS: merge the key tiles' sums (each relative to its own reference)
        // into o[][0] and the row sum; value wave 0 writes the LSE
        float l_ks = 0.f;
        if constexpr (KS) {
          const float l0 = lfin_lds[par][i], l1 = lfin_lds[par][16 + i];
          const float m0 = mfin_lds[par][i], m1 = mfin_lds[par][16 + i];
          const float mm = fmaxf(m0, m1);
          const float e0 = l0 > 0.f ? __builtin_amdgcn_exp2f(m0 - mm) : 0.f;
          const float e1 = l1 > 0.f ? __builtin_amdgcn_exp2f(m1 - mm) : 0.f;
          l_ks = l0 * e0 + l1 * e1;
#pragma unroll
          for (int dl = 0; dl < DL; ++dl) {
            o[dl][0] = o[dl][0] * e0 + o2[dl] * e1;
            o2[dl] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if (j == 0 && g == 0 && tile_row0 < a.M) {
            const float lse2 = l_ks > 0.f ? mm + log2f(l_ks) : -INFINITY;
            const int row = tile_row0 + i;
            if (whole)
              a.lse[(long long)b * a.M + row] = lse2 * kLn2;
            else
              a.part_lse[slot * a.M + row] = lse2;
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float lt = KS ? l_ks : lfin_lds[par][16 * rt + i];
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
          } else {   // the same rounding to bf16 into the partial slot
            uint16_t* op = a.part_o + (slot * a.M + row) * kDV + j * 128 + 4 * g;
#pragma unroll
            for (int dl = 0; dl < DL; ++dl) {
              const f32x4 v = o[dl][rt] * inv;
              const bf16x4 bv = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
              *reinterpret_cast<bf16x4*>(op + dl * 16) = bv;
            }
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

// --------------------------------------------------------------------------
// Row-wave kernel for tiles of 128 query rows (s_q*h_q a multiple of 128,
// bf16 cache, dense mode).  Four waves, one per SIMD, each owning 32 query
// rows end to end, so nothing but the page ring is shared:
//   scores  S^T[key][row] = K . Q^T on v_mfma_f32_32x32x16_bf16: A = 32 keys x
//           16 dims of the LDS unit (ds_read_b128), B = Q^T held in VGPRs for
//           the piece (32 rows x 576 dims = 144 VGPRs);
//   softmax the C layout gives lane l row l % 32 and 16 of the unit's 32 keys
//           (the other 16 in lane l ^ 32): in-lane max, one permlane32 swap,
//           exp2; the running sum stays per lane until the piece ends;
//   values  O^T[dim][row] += V^T . P^T on the same MFMA: A = 32 dims x 16 keys
//           read with ds_read_b64_tr_b16 (two 4-key reads per operand), B = the
//           lane's own probabilities, in the key order the score C layout
//           already holds (key 8j + 4h + i of the unit is held by lane half h
//           as element 4j + i; step u of the value product takes j = 2u,
//           2u + 1), so P never leaves the registers; O^T (32 rows x 512 dims,
//           fp32) is 256 accumulator registers and every row's rescale and
//           normalisation are lane-local.
// The wave computes scores of unit t and values of unit t-1 in one phase,
// one workgroup barrier per unit, over the same four-buffer ring of 36 KB
// half-page units as the ws kernel (two units in flight; every wave issues
// 9 of a unit's 36 direct-to-LDS slots).  A 128-row tile puts each page into
// LDS once per part (the 64-row ws tiles load it twice, once per tile).
// --------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kRWThreads = 256;
constexpr int kRWRows = 128;

// 16-byte unit swizzle of row r in this kernel's unit buffers: unit c is
// stored at c ^ rw_swizzle(r), inside its aligned group of 8 (72 units per
// row).  A row is 1152 = 4.5 x 256 bytes, so even and odd rows start 128
// bytes apart in the 256 bytes the LDS serves at once.  Both read patterns
// of the kernel then hit every bank at most once per 256 bytes: the score
// operand (16 consecutive rows at one unit per 16 lanes: the XOR takes all
// eight values on the even and on the odd rows of any 16, bit 2 from row bit
// 1, bit 1 from row bit 2, bit 0 from row bit 3) and the transposed value
// operand (per 32 lanes 4 consecutive rows x 4 consecutive units of an
// aligned group of 4: rows r and r + 2 land in the two halves of the group
// of 8, and row bit 3 only permutes the units inside a group of 4).  With
// two bits (rows r and r + 8 alike) the score read measured a 2-way
// conflict: SQ_LDS_BANK_CONFLICT 1.05e7 cycles against 3.04e7 active on the
// 128-head ridge workload.
__device__ __forceinline__ int rw_swizzle(int r) {
  return ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
}

// Page validity of unit (b, k): its table slot exists and names a page of
// the pool.  Units of invalid pages are zero-filled by the loads and their
// keys do not count.
__device__ __forceinline__ bool page_ok(const DecodeArgs& a, int b, int k) {
  if (k >= a.bt_stride) return false;
  const int page = ldc(a.block_table + (long long)b * a.bt_stride + k);
  return page >= 0 && (long long)page < a.num_blocks;
}

// The score accumulator is kept in VGPRs (the softmax reads it with VALU
// instructions) while the 256 output accumulators take the AGPRs: the
// product is written as inline asm with a VGPR constraint on the
// accumulator (early-clobber where it is only written: a product's result
// must not share registers with its operands).  The compiler does not see
// these asm statements as matrix products, so the asm carries the hazard
// waits itself: two wait states before a product whose operand registers a
// VALU instruction may have written just before (MLA_MFMA below);
// consecutive products on the same accumulator of the same shape need none
// between them.  The last product of a chain, score_mfma_last, waits out
// the wait states before a VALU instruction may read its result (a 16-pass
// product: at most 19; 24 are inserted) inside its own asm block: the
// compiler may place a copy of the accumulator right after the statement
// that produced it, and that copy must already see the result.
// A product's asm statement, with (W) or without the two wait states that a
// VALU write of one of its operands needs when it is the instruction just
// before: kernels whose operands come straight from LDS or global loads
// (the bf16 cache) drop them, kernels that convert operands with VALU
// instructions (FP8 pages) keep them; the assembly lint checks every product
// of the built kernels for that hazard along every control-flow path.
#define MLA_MFMA(W, INSN, ...)                     \
  do {                                             \
    if constexpr (W)                               \
      asm volatile("s_nop 1\n\t" INSN __VA_ARGS__); \
    else                                           \
      asm volatile(INSN __VA_ARGS__);              \
  } while (0)
// Two fixed accumulator blocks (one per half of a page).
#define MLA_SACC0 "{v[236:251]}"
#define MLA_SACC1 "{v[220:235]}"
template <int BLK, bool W = true>
__device__ __forceinline__ void score_mfma_first(f32x16& s, const bf16x8& k, const bf16x8& q) {
  if constexpr (BLK == 0)
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0", : "=&" MLA_SACC0(s) : "v"(k), "v"(q));
  else
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0", : "=&" MLA_SACC1(s) : "v"(k), "v"(q));
}
template <int BLK, bool W = true>
__device__ __forceinline__ void score_mfma(f32x16& s, const bf16x8& k, const bf16x8& q) {
  if constexpr (BLK == 0)
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0", : "+" MLA_SACC0(s) : "v"(k), "v"(q));
  else
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0", : "+" MLA_SACC1(s) : "v"(k), "v"(q));
}
template <int BLK, bool W = true>
__device__ __forceinline__ void score_mfma_last(f32x16& s, const bf16x8& k, const bf16x8& q) {
  if constexpr (BLK == 0)
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7",
                 : "+" MLA_SACC0(s)
                 : "v"(k), "v"(q));
  else
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7",
                 : "+" MLA_SACC1(s)
                 : "v"(k), "v"(q));
}
// The 256 output accumulators of a wave (O^T for its 32 rows x 512 dims,
// fp32) live in fixed AGPRs, block db of 32 dims in a[16db .. 16db+15], and
// are touched only by the inline asm below, which names the registers it
// writes as clobbers.  The compiler therefore never holds them (it keeps Q,
// the scores and everything else in VGPRs, which fit) and never moves them
// through VGPRs.  A test checks the built code for AGPR writes outside these
// asm blocks.
// ---- output accumulators in fixed AGPRs (block db: a[16db .. 16db+15]) ----
#define MLA_AGPR_CLOBBERS_ALL \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", \
  "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", \
  "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", \
  "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", \
  "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", \
  "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", \
  "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", \
  "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", \
  "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", \
  "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", \
  "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", \
  "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191", \
  "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207", \
  "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223", \
  "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239", \
  "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255"

#define MLA_AGPR_CLOBBERS_B0 "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15"
#define MLA_AGPR_CLOBBERS_B1 "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31"
#define MLA_AGPR_CLOBBERS_B2 "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47"
#define MLA_AGPR_CLOBBERS_B3 "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63"
#define MLA_AGPR_CLOBBERS_B4 "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79"
#define MLA_AGPR_CLOBBERS_B5 "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95"
#define MLA_AGPR_CLOBBERS_B6 "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111"
#define MLA_AGPR_CLOBBERS_B7 "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127"
#define MLA_AGPR_CLOBBERS_B8 "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143"
#define MLA_AGPR_CLOBBERS_B9 "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159"
#define MLA_AGPR_CLOBBERS_B10 "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175"
#define MLA_AGPR_CLOBBERS_B11 "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191"
#define MLA_AGPR_CLOBBERS_B12 "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207"
#define MLA_AGPR_CLOBBERS_B13 "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223"
#define MLA_AGPR_CLOBBERS_B14 "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239"
#define MLA_AGPR_CLOBBERS_B15 "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255"

template <int DB, bool W = true>
__device__ __forceinline__ void acc_mfma(const bf16x8& v, const bf16x8& p) {
  if constexpr (DB == 0) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[0:15], %0, %1, a[0:15]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B0);
  } else if constexpr (DB == 1) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[16:31], %0, %1, a[16:31]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B1);
  } else if constexpr (DB == 2) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[32:47], %0, %1, a[32:47]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B2);
  } else if constexpr (DB == 3) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[48:63], %0, %1, a[48:63]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B3);
  } else if constexpr (DB == 4) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[64:79], %0, %1, a[64:79]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B4);
  } else if constexpr (DB == 5) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[80:95], %0, %1, a[80:95]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B5);
  } else if constexpr (DB == 6) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[96:111], %0, %1, a[96:111]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B6);
  } else if constexpr (DB == 7) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[112:127], %0, %1, a[112:127]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B7);
  } else if constexpr (DB == 8) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[128:143], %0, %1, a[128:143]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B8);
  } else if constexpr (DB == 9) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[144:159], %0, %1, a[144:159]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B9);
  } else if constexpr (DB == 10) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[160:175], %0, %1, a[160:175]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B10);
  } else if constexpr (DB == 11) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[176:191], %0, %1, a[176:191]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B11);
  } else if constexpr (DB == 12) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[192:207], %0, %1, a[192:207]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B12);
  } else if constexpr (DB == 13) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[208:223], %0, %1, a[208:223]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B13);
  } else if constexpr (DB == 14) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[224:239], %0, %1, a[224:239]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B14);
  } else if constexpr (DB == 15) {
    MLA_MFMA(W, "v_mfma_f32_32x32x16_bf16 a[240:255], %0, %1, a[240:255]", ::"v"(v), "v"(p)
                 : MLA_AGPR_CLOBBERS_B15);
  }
}

template <int DB>
__device__ __forceinline__ void acc_read(float (&e)[16]) {
  if constexpr (DB == 0) {
    asm volatile("v_accvgpr_read_b32 %0, a0\n\tv_accvgpr_read_b32 %1, a1\n\tv_accvgpr_read_b32 %2, a2\n\tv_accvgpr_read_b32 %3, a3\n\tv_accvgpr_read_b32 %4, a4\n\tv_accvgpr_read_b32 %5, a5\n\tv_accvgpr_read_b32 %6, a6\n\tv_accvgpr_read_b32 %7, a7\n\tv_accvgpr_read_b32 %8, a8\n\tv_accvgpr_read_b32 %9, a9\n\tv_accvgpr_read_b32 %10, a10\n\tv_accvgpr_read_b32 %11, a11\n\tv_accvgpr_read_b32 %12, a12\n\tv_accvgpr_read_b32 %13, a13\n\tv_accvgpr_read_b32 %14, a14\n\tv_accvgpr_read_b32 %15, a15"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 1) {
    asm volatile("v_accvgpr_read_b32 %0, a16\n\tv_accvgpr_read_b32 %1, a17\n\tv_accvgpr_read_b32 %2, a18\n\tv_accvgpr_read_b32 %3, a19\n\tv_accvgpr_read_b32 %4, a20\n\tv_accvgpr_read_b32 %5, a21\n\tv_accvgpr_read_b32 %6, a22\n\tv_accvgpr_read_b32 %7, a23\n\tv_accvgpr_read_b32 %8, a24\n\tv_accvgpr_read_b32 %9, a25\n\tv_accvgpr_read_b32 %10, a26\n\tv_accvgpr_read_b32 %11, a27\n\tv_accvgpr_read_b32 %12, a28\n\tv_accvgpr_read_b32 %13, a29\n\tv_accvgpr_read_b32 %14, a30\n\tv_accvgpr_read_b32 %15, a31"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 2) {
    asm volatile("v_accvgpr_read_b32 %0, a32\n\tv_accvgpr_read_b32 %1, a33\n\tv_accvgpr_read_b32 %2, a34\n\tv_accvgpr_read_b32 %3, a35\n\tv_accvgpr_read_b32 %4, a36\n\tv_accvgpr_read_b32 %5, a37\n\tv_accvgpr_read_b32 %6, a38\n\tv_accvgpr_read_b32 %7, a39\n\tv_accvgpr_read_b32 %8, a40\n\tv_accvgpr_read_b32 %9, a41\n\tv_accvgpr_read_b32 %10, a42\n\tv_accvgpr_read_b32 %11, a43\n\tv_accvgpr_read_b32 %12, a44\n\tv_accvgpr_read_b32 %13, a45\n\tv_accvgpr_read_b32 %14, a46\n\tv_accvgpr_read_b32 %15, a47"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 3) {
    asm volatile("v_accvgpr_read_b32 %0, a48\n\tv_accvgpr_read_b32 %1, a49\n\tv_accvgpr_read_b32 %2, a50\n\tv_accvgpr_read_b32 %3, a51\n\tv_accvgpr_read_b32 %4, a52\n\tv_accvgpr_read_b32 %5, a53\n\tv_accvgpr_read_b32 %6, a54\n\tv_accvgpr_read_b32 %7, a55\n\tv_accvgpr_read_b32 %8, a56\n\tv_accvgpr_read_b32 %9, a57\n\tv_accvgpr_read_b32 %10, a58\n\tv_accvgpr_read_b32 %11, a59\n\tv_accvgpr_read_b32 %12, a60\n\tv_accvgpr_read_b32 %13, a61\n\tv_accvgpr_read_b32 %14, a62\n\tv_accvgpr_read_b32 %15, a63"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 4) {
    asm volatile("v_accvgpr_read_b32 %0, a64\n\tv_accvgpr_read_b32 %1, a65\n\tv_accvgpr_read_b32 %2, a66\n\tv_accvgpr_read_b32 %3, a67\n\tv_accvgpr_read_b32 %4, a68\n\tv_accvgpr_read_b32 %5, a69\n\tv_accvgpr_read_b32 %6, a70\n\tv_accvgpr_read_b32 %7, a71\n\tv_accvgpr_read_b32 %8, a72\n\tv_accvgpr_read_b32 %9, a73\n\tv_accvgpr_read_b32 %10, a74\n\tv_accvgpr_read_b32 %11, a75\n\tv_accvgpr_read_b32 %12, a76\n\tv_accvgpr_read_b32 %13, a77\n\tv_accvgpr_read_b32 %14, a78\n\tv_accvgpr_read_b32 %15, a79"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 5) {
    asm volatile("v_accvgpr_read_b32 %0, a80\n\tv_accvgpr_read_b32 %1, a81\n\tv_accvgpr_read_b32 %2, a82\n\tv_accvgpr_read_b32 %3, a83\n\tv_accvgpr_read_b32 %4, a84\n\tv_accvgpr_read_b32 %5, a85\n\tv_accvgpr_read_b32 %6, a86\n\tv_accvgpr_read_b32 %7, a87\n\tv_accvgpr_read_b32 %8, a88\n\tv_accvgpr_read_b32 %9, a89\n\tv_accvgpr_read_b32 %10, a90\n\tv_accvgpr_read_b32 %11, a91\n\tv_accvgpr_read_b32 %12, a92\n\tv_accvgpr_read_b32 %13, a93\n\tv_accvgpr_read_b32 %14, a94\n\tv_accvgpr_read_b32 %15, a95"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 6) {
    asm volatile("v_accvgpr_read_b32 %0, a96\n\tv_accvgpr_read_b32 %1, a97\n\tv_accvgpr_read_b32 %2, a98\n\tv_accvgpr_read_b32 %3, a99\n\tv_accvgpr_read_b32 %4, a100\n\tv_accvgpr_read_b32 %5, a101\n\tv_accvgpr_read_b32 %6, a102\n\tv_accvgpr_read_b32 %7, a103\n\tv_accvgpr_read_b32 %8, a104\n\tv_accvgpr_read_b32 %9, a105\n\tv_accvgpr_read_b32 %10, a106\n\tv_accvgpr_read_b32 %11, a107\n\tv_accvgpr_read_b32 %12, a108\n\tv_accvgpr_read_b32 %13, a109\n\tv_accvgpr_read_b32 %14, a110\n\tv_accvgpr_read_b32 %15, a111"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 7) {
    asm volatile("v_accvgpr_read_b32 %0, a112\n\tv_accvgpr_read_b32 %1, a113\n\tv_accvgpr_read_b32 %2, a114\n\tv_accvgpr_read_b32 %3, a115\n\tv_accvgpr_read_b32 %4, a116\n\tv_accvgpr_read_b32 %5, a117\n\tv_accvgpr_read_b32 %6, a118\n\tv_accvgpr_read_b32 %7, a119\n\tv_accvgpr_read_b32 %8, a120\n\tv_accvgpr_read_b32 %9, a121\n\tv_accvgpr_read_b32 %10, a122\n\tv_accvgpr_read_b32 %11, a123\n\tv_accvgpr_read_b32 %12, a124\n\tv_accvgpr_read_b32 %13, a125\n\tv_accvgpr_read_b32 %14, a126\n\tv_accvgpr_read_b32 %15, a127"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 8) {
    asm volatile("v_accvgpr_read_b32 %0, a128\n\tv_accvgpr_read_b32 %1, a129\n\tv_accvgpr_read_b32 %2, a130\n\tv_accvgpr_read_b32 %3, a131\n\tv_accvgpr_read_b32 %4, a132\n\tv_accvgpr_read_b32 %5, a133\n\tv_accvgpr_read_b32 %6, a134\n\tv_accvgpr_read_b32 %7, a135\n\tv_accvgpr_read_b32 %8, a136\n\tv_accvgpr_read_b32 %9, a137\n\tv_accvgpr_read_b32 %10, a138\n\tv_accvgpr_read_b32 %11, a139\n\tv_accvgpr_read_b32 %12, a140\n\tv_accvgpr_read_b32 %13, a141\n\tv_accvgpr_read_b32 %14, a142\n\tv_accvgpr_read_b32 %15, a143"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 9) {
    asm volatile("v_accvgpr_read_b32 %0, a144\n\tv_accvgpr_read_b32 %1, a145\n\tv_accvgpr_read_b32 %2, a146\n\tv_accvgpr_read_b32 %3, a147\n\tv_accvgpr_read_b32 %4, a148\n\tv_accvgpr_read_b32 %5, a149\n\tv_accvgpr_read_b32 %6, a150\n\tv_accvgpr_read_b32 %7, a151\n\tv_accvgpr_read_b32 %8, a152\n\tv_accvgpr_read_b32 %9, a153\n\tv_accvgpr_read_b32 %10, a154\n\tv_accvgpr_read_b32 %11, a155\n\tv_accvgpr_read_b32 %12, a156\n\tv_accvgpr_read_b32 %13, a157\n\tv_accvgpr_read_b32 %14, a158\n\tv_accvgpr_read_b32 %15, a159"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 10) {
    asm volatile("v_accvgpr_read_b32 %0, a160\n\tv_accvgpr_read_b32 %1, a161\n\tv_accvgpr_read_b32 %2, a162\n\tv_accvgpr_read_b32 %3, a163\n\tv_accvgpr_read_b32 %4, a164\n\tv_accvgpr_read_b32 %5, a165\n\tv_accvgpr_read_b32 %6, a166\n\tv_accvgpr_read_b32 %7, a167\n\tv_accvgpr_read_b32 %8, a168\n\tv_accvgpr_read_b32 %9, a169\n\tv_accvgpr_read_b32 %10, a170\n\tv_accvgpr_read_b32 %11, a171\n\tv_accvgpr_read_b32 %12, a172\n\tv_accvgpr_read_b32 %13, a173\n\tv_accvgpr_read_b32 %14, a174\n\tv_accvgpr_read_b32 %15, a175"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 11) {
    asm volatile("v_accvgpr_read_b32 %0, a176\n\tv_accvgpr_read_b32 %1, a177\n\tv_accvgpr_read_b32 %2, a178\n\tv_accvgpr_read_b32 %3, a179\n\tv_accvgpr_read_b32 %4, a180\n\tv_accvgpr_read_b32 %5, a181\n\tv_accvgpr_read_b32 %6, a182\n\tv_accvgpr_read_b32 %7, a183\n\tv_accvgpr_read_b32 %8, a184\n\tv_accvgpr_read_b32 %9, a185\n\tv_accvgpr_read_b32 %10, a186\n\tv_accvgpr_read_b32 %11, a187\n\tv_accvgpr_read_b32 %12, a188\n\tv_accvgpr_read_b32 %13, a189\n\tv_accvgpr_read_b32 %14, a190\n\tv_accvgpr_read_b32 %15, a191"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 12) {
    asm volatile("v_accvgpr_read_b32 %0, a192\n\tv_accvgpr_read_b32 %1, a193\n\tv_accvgpr_read_b32 %2, a194\n\tv_accvgpr_read_b32 %3, a195\n\tv_accvgpr_read_b32 %4, a196\n\tv_accvgpr_read_b32 %5, a197\n\tv_accvgpr_read_b32 %6, a198\n\tv_accvgpr_read_b32 %7, a199\n\tv_accvgpr_read_b32 %8, a200\n\tv_accvgpr_read_b32 %9, a201\n\tv_accvgpr_read_b32 %10, a202\n\tv_accvgpr_read_b32 %11, a203\n\tv_accvgpr_read_b32 %12, a204\n\tv_accvgpr_read_b32 %13, a205\n\tv_accvgpr_read_b32 %14, a206\n\tv_accvgpr_read_b32 %15, a207"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 13) {
    asm volatile("v_accvgpr_read_b32 %0, a208\n\tv_accvgpr_read_b32 %1, a209\n\tv_accvgpr_read_b32 %2, a210\n\tv_accvgpr_read_b32 %3, a211\n\tv_accvgpr_read_b32 %4, a212\n\tv_accvgpr_read_b32 %5, a213\n\tv_accvgpr_read_b32 %6, a214\n\tv_accvgpr_read_b32 %7, a215\n\tv_accvgpr_read_b32 %8, a216\n\tv_accvgpr_read_b32 %9, a217\n\tv_accvgpr_read_b32 %10, a218\n\tv_accvgpr_read_b32 %11, a219\n\tv_accvgpr_read_b32 %12, a220\n\tv_accvgpr_read_b32 %13, a221\n\tv_accvgpr_read_b32 %14, a222\n\tv_accvgpr_read_b32 %15, a223"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 14) {
    asm volatile("v_accvgpr_read_b32 %0, a224\n\tv_accvgpr_read_b32 %1, a225\n\tv_accvgpr_read_b32 %2, a226\n\tv_accvgpr_read_b32 %3, a227\n\tv_accvgpr_read_b32 %4, a228\n\tv_accvgpr_read_b32 %5, a229\n\tv_accvgpr_read_b32 %6, a230\n\tv_accvgpr_read_b32 %7, a231\n\tv_accvgpr_read_b32 %8, a232\n\tv_accvgpr_read_b32 %9, a233\n\tv_accvgpr_read_b32 %10, a234\n\tv_accvgpr_read_b32 %11, a235\n\tv_accvgpr_read_b32 %12, a236\n\tv_accvgpr_read_b32 %13, a237\n\tv_accvgpr_read_b32 %14, a238\n\tv_accvgpr_read_b32 %15, a239"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  } else if constexpr (DB == 15) {
    asm volatile("v_accvgpr_read_b32 %0, a240\n\tv_accvgpr_read_b32 %1, a241\n\tv_accvgpr_read_b32 %2, a242\n\tv_accvgpr_read_b32 %3, a243\n\tv_accvgpr_read_b32 %4, a244\n\tv_accvgpr_read_b32 %5, a245\n\tv_accvgpr_read_b32 %6, a246\n\tv_accvgpr_read_b32 %7, a247\n\tv_accvgpr_read_b32 %8, a248\n\tv_accvgpr_read_b32 %9, a249\n\tv_accvgpr_read_b32 %10, a250\n\tv_accvgpr_read_b32 %11, a251\n\tv_accvgpr_read_b32 %12, a252\n\tv_accvgpr_read_b32 %13, a253\n\tv_accvgpr_read_b32 %14, a254\n\tv_accvgpr_read_b32 %15, a255"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15]));
  }
}
// all 256 accumulators to zero: 16 products of zero operands with no accumulation
// (the trailing wait states keep the operand register unwritten while the
// last products may still read it)
__device__ __forceinline__ void acc_zero_all(const bf16x8& z) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[0:15], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[16:31], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[32:47], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[48:63], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[64:79], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[80:95], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[96:111], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[112:127], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[128:143], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[144:159], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[160:175], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[176:191], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[192:207], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[208:223], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[224:239], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[240:255], %0, %0, 0\n\ts_nop 7\n\ts_nop 7" ::"v"(z) : MLA_AGPR_CLOBBERS_ALL);
}

// all 256 accumulators times the lane's x (the wait states of a 16-pass
// product before the first read, and of a VALU write before a product
// reads the register as its accumulator, are included)
__device__ __forceinline__ void acc_scale_all(float x) {
  float t0, t1, t2, t3;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read_b32 %0, a0\n\tv_accvgpr_read_b32 %1, a1\n\tv_accvgpr_read_b32 %2, a2\n\tv_accvgpr_read_b32 %3, a3\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a0, %0\n\tv_accvgpr_write_b32 a1, %1\n\tv_accvgpr_write_b32 a2, %2\n\tv_accvgpr_write_b32 a3, %3\n\tv_accvgpr_read_b32 %0, a4\n\tv_accvgpr_read_b32 %1, a5\n\tv_accvgpr_read_b32 %2, a6\n\tv_accvgpr_read_b32 %3, a7\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a4, %0\n\tv_accvgpr_write_b32 a5, %1\n\tv_accvgpr_write_b32 a6, %2\n\tv_accvgpr_write_b32 a7, %3\n\tv_accvgpr_read_b32 %0, a8\n\tv_accvgpr_read_b32 %1, a9\n\tv_accvgpr_read_b32 %2, a10\n\tv_accvgpr_read_b32 %3, a11\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a8, %0\n\tv_accvgpr_write_b32 a9, %1\n\tv_accvgpr_write_b32 a10, %2\n\tv_accvgpr_write_b32 a11, %3\n\tv_accvgpr_read_b32 %0, a12\n\tv_accvgpr_read_b32 %1, a13\n\tv_accvgpr_read_b32 %2, a14\n\tv_accvgpr_read_b32 %3, a15\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a12, %0\n\tv_accvgpr_write_b32 a13, %1\n\tv_accvgpr_write_b32 a14, %2\n\tv_accvgpr_write_b32 a15, %3\n\tv_accvgpr_read_b32 %0, a16\n\tv_accvgpr_read_b32 %1, a17\n\tv_accvgpr_read_b32 %2, a18\n\tv_accvgpr_read_b32 %3, a19\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a16, %0\n\tv_accvgpr_write_b32 a17, %1\n\tv_accvgpr_write_b32 a18, %2\n\tv_accvgpr_write_b32 a19, %3\n\tv_accvgpr_read_b32 %0, a20\n\tv_accvgpr_read_b32 %1, a21\n\tv_accvgpr_read_b32 %2, a22\n\tv_accvgpr_read_b32 %3, a23\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a20, %0\n\tv_accvgpr_write_b32 a21, %1\n\tv_accvgpr_write_b32 a22, %2\n\tv_accvgpr_write_b32 a23, %3\n\tv_accvgpr_read_b32 %0, a24\n\tv_accvgpr_read_b32 %1, a25\n\tv_accvgpr_read_b32 %2, a26\n\tv_accvgpr_read_b32 %3, a27\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a24, %0\n\tv_accvgpr_write_b32 a25, %1\n\tv_accvgpr_write_b32 a26, %2\n\tv_accvgpr_write_b32 a27, %3\n\tv_accvgpr_read_b32 %0, a28\n\tv_accvgpr_read_b32 %1, a29\n\tv_accvgpr_read_b32 %2, a30\n\tv_accvgpr_read_b32 %3, a31\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a28, %0\n\tv_accvgpr_write_b32 a29, %1\n\tv_accvgpr_write_b32 a30, %2\n\tv_accvgpr_write_b32 a31, %3\n\tv_accvgpr_read_b32 %0, a32\n\tv_accvgpr_read_b32 %1, a33\n\tv_accvgpr_read_b32 %2, a34\n\tv_accvgpr_read_b32 %3, a35\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a32, %0\n\tv_accvgpr_write_b32 a33, %1\n\tv_accvgpr_write_b32 a34, %2\n\tv_accvgpr_write_b32 a35, %3\n\tv_accvgpr_read_b32 %0, a36\n\tv_accvgpr_read_b32 %1, a37\n\tv_accvgpr_read_b32 %2, a38\n\tv_accvgpr_read_b32 %3, a39\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a36, %0\n\tv_accvgpr_write_b32 a37, %1\n\tv_accvgpr_write_b32 a38, %2\n\tv_accvgpr_write_b32 a39, %3\n\tv_accvgpr_read_b32 %0, a40\n\tv_accvgpr_read_b32 %1, a41\n\tv_accvgpr_read_b32 %2, a42\n\tv_accvgpr_read_b32 %3, a43\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a40, %0\n\tv_accvgpr_write_b32 a41, %1\n\tv_accvgpr_write_b32 a42, %2\n\tv_accvgpr_write_b32 a43, %3\n\tv_accvgpr_read_b32 %0, a44\n\tv_accvgpr_read_b32 %1, a45\n\tv_accvgpr_read_b32 %2, a46\n\tv_accvgpr_read_b32 %3, a47\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a44, %0\n\tv_accvgpr_write_b32 a45, %1\n\tv_accvgpr_write_b32 a46, %2\n\tv_accvgpr_write_b32 a47, %3\n\tv_accvgpr_read_b32 %0, a48\n\tv_accvgpr_read_b32 %1, a49\n\tv_accvgpr_read_b32 %2, a50\n\tv_accvgpr_read_b32 %3, a51\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a48, %0\n\tv_accvgpr_write_b32 a49, %1\n\tv_accvgpr_write_b32 a50, %2\n\tv_accvgpr_write_b32 a51, %3\n\tv_accvgpr_read_b32 %0, a52\n\tv_accvgpr_read_b32 %1, a53\n\tv_accvgpr_read_b32 %2, a54\n\tv_accvgpr_read_b32 %3, a55\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a52, %0\n\tv_accvgpr_write_b32 a53, %1\n\tv_accvgpr_write_b32 a54, %2\n\tv_accvgpr_write_b32 a55, %3\n\tv_accvgpr_read_b32 %0, a56\n\tv_accvgpr_read_b32 %1, a57\n\tv_accvgpr_read_b32 %2, a58\n\tv_accvgpr_read_b32 %3, a59\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a56, %0\n\tv_accvgpr_write_b32 a57, %1\n\tv_accvgpr_write_b32 a58, %2\n\tv_accvgpr_write_b32 a59, %3\n\tv_accvgpr_read_b32 %0, a60\n\tv_accvgpr_read_b32 %1, a61\n\tv_accvgpr_read_b32 %2, a62\n\tv_accvgpr_read_b32 %3, a63\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a60, %0\n\tv_accvgpr_write_b32 a61, %1\n\tv_accvgpr_write_b32 a62, %2\n\tv_accvgpr_write_b32 a63, %3\n\tv_accvgpr_read_b32 %0, a64\n\tv_accvgpr_read_b32 %1, a65\n\tv_accvgpr_read_b32 %2, a66\n\tv_accvgpr_read_b32 %3, a67\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a64, %0\n\tv_accvgpr_write_b32 a65, %1\n\tv_accvgpr_write_b32 a66, %2\n\tv_accvgpr_write_b32 a67, %3\n\tv_accvgpr_read_b32 %0, a68\n\tv_accvgpr_read_b32 %1, a69\n\tv_accvgpr_read_b32 %2, a70\n\tv_accvgpr_read_b32 %3, a71\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a68, %0\n\tv_accvgpr_write_b32 a69, %1\n\tv_accvgpr_write_b32 a70, %2\n\tv_accvgpr_write_b32 a71, %3\n\tv_accvgpr_read_b32 %0, a72\n\tv_accvgpr_read_b32 %1, a73\n\tv_accvgpr_read_b32 %2, a74\n\tv_accvgpr_read_b32 %3, a75\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a72, %0\n\tv_accvgpr_write_b32 a73, %1\n\tv_accvgpr_write_b32 a74, %2\n\tv_accvgpr_write_b32 a75, %3\n\tv_accvgpr_read_b32 %0, a76\n\tv_accvgpr_read_b32 %1, a77\n\tv_accvgpr_read_b32 %2, a78\n\tv_accvgpr_read_b32 %3, a79\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a76, %0\n\tv_accvgpr_write_b32 a77, %1\n\tv_accvgpr_write_b32 a78, %2\n\tv_accvgpr_write_b32 a79, %3\n\tv_accvgpr_read_b32 %0, a80\n\tv_accvgpr_read_b32 %1, a81\n\tv_accvgpr_read_b32 %2, a82\n\tv_accvgpr_read_b32 %3, a83\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a80, %0\n\tv_accvgpr_write_b32 a81, %1\n\tv_accvgpr_write_b32 a82, %2\n\tv_accvgpr_write_b32 a83, %3\n\tv_accvgpr_read_b32 %0, a84\n\tv_accvgpr_read_b32 %1, a85\n\tv_accvgpr_read_b32 %2, a86\n\tv_accvgpr_read_b32 %3, a87\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a84, %0\n\tv_accvgpr_write_b32 a85, %1\n\tv_accvgpr_write_b32 a86, %2\n\tv_accvgpr_write_b32 a87, %3\n\tv_accvgpr_read_b32 %0, a88\n\tv_accvgpr_read_b32 %1, a89\n\tv_accvgpr_read_b32 %2, a90\n\tv_accvgpr_read_b32 %3, a91\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a88, %0\n\tv_accvgpr_write_b32 a89, %1\n\tv_accvgpr_write_b32 a90, %2\n\tv_accvgpr_write_b32 a91, %3\n\tv_accvgpr_read_b32 %0, a92\n\tv_accvgpr_read_b32 %1, a93\n\tv_accvgpr_read_b32 %2, a94\n\tv_accvgpr_read_b32 %3, a95\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a92, %0\n\tv_accvgpr_write_b32 a93, %1\n\tv_accvgpr_write_b32 a94, %2\n\tv_accvgpr_write_b32 a95, %3\n\tv_accvgpr_read_b32 %0, a96\n\tv_accvgpr_read_b32 %1, a97\n\tv_accvgpr_read_b32 %2, a98\n\tv_accvgpr_read_b32 %3, a99\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a96, %0\n\tv_accvgpr_write_b32 a97, %1\n\tv_accvgpr_write_b32 a98, %2\n\tv_accvgpr_write_b32 a99, %3\n\tv_accvgpr_read_b32 %0, a100\n\tv_accvgpr_read_b32 %1, a101\n\tv_accvgpr_read_b32 %2, a102\n\tv_accvgpr_read_b32 %3, a103\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a100, %0\n\tv_accvgpr_write_b32 a101, %1\n\tv_accvgpr_write_b32 a102, %2\n\tv_accvgpr_write_b32 a103, %3\n\tv_accvgpr_read_b32 %0, a104\n\tv_accvgpr_read_b32 %1, a105\n\tv_accvgpr_read_b32 %2, a106\n\tv_accvgpr_read_b32 %3, a107\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a104, %0\n\tv_accvgpr_write_b32 a105, %1\n\tv_accvgpr_write_b32 a106, %2\n\tv_accvgpr_write_b32 a107, %3\n\tv_accvgpr_read_b32 %0, a108\n\tv_accvgpr_read_b32 %1, a109\n\tv_accvgpr_read_b32 %2, a110\n\tv_accvgpr_read_b32 %3, a111\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a108, %0\n\tv_accvgpr_write_b32 a109, %1\n\tv_accvgpr_write_b32 a110, %2\n\tv_accvgpr_write_b32 a111, %3\n\tv_accvgpr_read_b32 %0, a112\n\tv_accvgpr_read_b32 %1, a113\n\tv_accvgpr_read_b32 %2, a114\n\tv_accvgpr_read_b32 %3, a115\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a112, %0\n\tv_accvgpr_write_b32 a113, %1\n\tv_accvgpr_write_b32 a114, %2\n\tv_accvgpr_write_b32 a115, %3\n\tv_accvgpr_read_b32 %0, a116\n\tv_accvgpr_read_b32 %1, a117\n\tv_accvgpr_read_b32 %2, a118\n\tv_accvgpr_read_b32 %3, a119\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a116, %0\n\tv_accvgpr_write_b32 a117, %1\n\tv_accvgpr_write_b32 a118, %2\n\tv_accvgpr_write_b32 a119, %3\n\tv_accvgpr_read_b32 %0, a120\n\tv_accvgpr_read_b32 %1, a121\n\tv_accvgpr_read_b32 %2, a122\n\tv_accvgpr_read_b32 %3, a123\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a120, %0\n\tv_accvgpr_write_b32 a121, %1\n\tv_accvgpr_write_b32 a122, %2\n\tv_accvgpr_write_b32 a123, %3\n\tv_accvgpr_read_b32 %0, a124\n\tv_accvgpr_read_b32 %1, a125\n\tv_accvgpr_read_b32 %2, a126\n\tv_accvgpr_read_b32 %3, a127\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a124, %0\n\tv_accvgpr_write_b32 a125, %1\n\tv_accvgpr_write_b32 a126, %2\n\tv_accvgpr_write_b32 a127, %3\n\tv_accvgpr_read_b32 %0, a128\n\tv_accvgpr_read_b32 %1, a129\n\tv_accvgpr_read_b32 %2, a130\n\tv_accvgpr_read_b32 %3, a131\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a128, %0\n\tv_accvgpr_write_b32 a129, %1\n\tv_accvgpr_write_b32 a130, %2\n\tv_accvgpr_write_b32 a131, %3\n\tv_accvgpr_read_b32 %0, a132\n\tv_accvgpr_read_b32 %1, a133\n\tv_accvgpr_read_b32 %2, a134\n\tv_accvgpr_read_b32 %3, a135\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a132, %0\n\tv_accvgpr_write_b32 a133, %1\n\tv_accvgpr_write_b32 a134, %2\n\tv_accvgpr_write_b32 a135, %3\n\tv_accvgpr_read_b32 %0, a136\n\tv_accvgpr_read_b32 %1, a137\n\tv_accvgpr_read_b32 %2, a138\n\tv_accvgpr_read_b32 %3, a139\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a136, %0\n\tv_accvgpr_write_b32 a137, %1\n\tv_accvgpr_write_b32 a138, %2\n\tv_accvgpr_write_b32 a139, %3\n\tv_accvgpr_read_b32 %0, a140\n\tv_accvgpr_read_b32 %1, a141\n\tv_accvgpr_read_b32 %2, a142\n\tv_accvgpr_read_b32 %3, a143\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a140, %0\n\tv_accvgpr_write_b32 a141, %1\n\tv_accvgpr_write_b32 a142, %2\n\tv_accvgpr_write_b32 a143, %3\n\tv_accvgpr_read_b32 %0, a144\n\tv_accvgpr_read_b32 %1, a145\n\tv_accvgpr_read_b32 %2, a146\n\tv_accvgpr_read_b32 %3, a147\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a144, %0\n\tv_accvgpr_write_b32 a145, %1\n\tv_accvgpr_write_b32 a146, %2\n\tv_accvgpr_write_b32 a147, %3\n\tv_accvgpr_read_b32 %0, a148\n\tv_accvgpr_read_b32 %1, a149\n\tv_accvgpr_read_b32 %2, a150\n\tv_accvgpr_read_b32 %3, a151\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a148, %0\n\tv_accvgpr_write_b32 a149, %1\n\tv_accvgpr_write_b32 a150, %2\n\tv_accvgpr_write_b32 a151, %3\n\tv_accvgpr_read_b32 %0, a152\n\tv_accvgpr_read_b32 %1, a153\n\tv_accvgpr_read_b32 %2, a154\n\tv_accvgpr_read_b32 %3, a155\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a152, %0\n\tv_accvgpr_write_b32 a153, %1\n\tv_accvgpr_write_b32 a154, %2\n\tv_accvgpr_write_b32 a155, %3\n\tv_accvgpr_read_b32 %0, a156\n\tv_accvgpr_read_b32 %1, a157\n\tv_accvgpr_read_b32 %2, a158\n\tv_accvgpr_read_b32 %3, a159\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a156, %0\n\tv_accvgpr_write_b32 a157, %1\n\tv_accvgpr_write_b32 a158, %2\n\tv_accvgpr_write_b32 a159, %3\n\tv_accvgpr_read_b32 %0, a160\n\tv_accvgpr_read_b32 %1, a161\n\tv_accvgpr_read_b32 %2, a162\n\tv_accvgpr_read_b32 %3, a163\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a160, %0\n\tv_accvgpr_write_b32 a161, %1\n\tv_accvgpr_write_b32 a162, %2\n\tv_accvgpr_write_b32 a163, %3\n\tv_accvgpr_read_b32 %0, a164\n\tv_accvgpr_read_b32 %1, a165\n\tv_accvgpr_read_b32 %2, a166\n\tv_accvgpr_read_b32 %3, a167\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a164, %0\n\tv_accvgpr_write_b32 a165, %1\n\tv_accvgpr_write_b32 a166, %2\n\tv_accvgpr_write_b32 a167, %3\n\tv_accvgpr_read_b32 %0, a168\n\tv_accvgpr_read_b32 %1, a169\n\tv_accvgpr_read_b32 %2, a170\n\tv_accvgpr_read_b32 %3, a171\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a168, %0\n\tv_accvgpr_write_b32 a169, %1\n\tv_accvgpr_write_b32 a170, %2\n\tv_accvgpr_write_b32 a171, %3\n\tv_accvgpr_read_b32 %0, a172\n\tv_accvgpr_read_b32 %1, a173\n\tv_accvgpr_read_b32 %2, a174\n\tv_accvgpr_read_b32 %3, a175\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a172, %0\n\tv_accvgpr_write_b32 a173, %1\n\tv_accvgpr_write_b32 a174, %2\n\tv_accvgpr_write_b32 a175, %3\n\tv_accvgpr_read_b32 %0, a176\n\tv_accvgpr_read_b32 %1, a177\n\tv_accvgpr_read_b32 %2, a178\n\tv_accvgpr_read_b32 %3, a179\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a176, %0\n\tv_accvgpr_write_b32 a177, %1\n\tv_accvgpr_write_b32 a178, %2\n\tv_accvgpr_write_b32 a179, %3\n\tv_accvgpr_read_b32 %0, a180\n\tv_accvgpr_read_b32 %1, a181\n\tv_accvgpr_read_b32 %2, a182\n\tv_accvgpr_read_b32 %3, a183\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a180, %0\n\tv_accvgpr_write_b32 a181, %1\n\tv_accvgpr_write_b32 a182, %2\n\tv_accvgpr_write_b32 a183, %3\n\tv_accvgpr_read_b32 %0, a184\n\tv_accvgpr_read_b32 %1, a185\n\tv_accvgpr_read_b32 %2, a186\n\tv_accvgpr_read_b32 %3, a187\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a184, %0\n\tv_accvgpr_write_b32 a185, %1\n\tv_accvgpr_write_b32 a186, %2\n\tv_accvgpr_write_b32 a187, %3\n\tv_accvgpr_read_b32 %0, a188\n\tv_accvgpr_read_b32 %1, a189\n\tv_accvgpr_read_b32 %2, a190\n\tv_accvgpr_read_b32 %3, a191\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a188, %0\n\tv_accvgpr_write_b32 a189, %1\n\tv_accvgpr_write_b32 a190, %2\n\tv_accvgpr_write_b32 a191, %3\n\tv_accvgpr_read_b32 %0, a192\n\tv_accvgpr_read_b32 %1, a193\n\tv_accvgpr_read_b32 %2, a194\n\tv_accvgpr_read_b32 %3, a195\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a192, %0\n\tv_accvgpr_write_b32 a193, %1\n\tv_accvgpr_write_b32 a194, %2\n\tv_accvgpr_write_b32 a195, %3\n\tv_accvgpr_read_b32 %0, a196\n\tv_accvgpr_read_b32 %1, a197\n\tv_accvgpr_read_b32 %2, a198\n\tv_accvgpr_read_b32 %3, a199\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a196, %0\n\tv_accvgpr_write_b32 a197, %1\n\tv_accvgpr_write_b32 a198, %2\n\tv_accvgpr_write_b32 a199, %3\n\tv_accvgpr_read_b32 %0, a200\n\tv_accvgpr_read_b32 %1, a201\n\tv_accvgpr_read_b32 %2, a202\n\tv_accvgpr_read_b32 %3, a203\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a200, %0\n\tv_accvgpr_write_b32 a201, %1\n\tv_accvgpr_write_b32 a202, %2\n\tv_accvgpr_write_b32 a203, %3\n\tv_accvgpr_read_b32 %0, a204\n\tv_accvgpr_read_b32 %1, a205\n\tv_accvgpr_read_b32 %2, a206\n\tv_accvgpr_read_b32 %3, a207\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a204, %0\n\tv_accvgpr_write_b32 a205, %1\n\tv_accvgpr_write_b32 a206, %2\n\tv_accvgpr_write_b32 a207, %3\n\tv_accvgpr_read_b32 %0, a208\n\tv_accvgpr_read_b32 %1, a209\n\tv_accvgpr_read_b32 %2, a210\n\tv_accvgpr_read_b32 %3, a211\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a208, %0\n\tv_accvgpr_write_b32 a209, %1\n\tv_accvgpr_write_b32 a210, %2\n\tv_accvgpr_write_b32 a211, %3\n\tv_accvgpr_read_b32 %0, a212\n\tv_accvgpr_read_b32 %1, a213\n\tv_accvgpr_read_b32 %2, a214\n\tv_accvgpr_read_b32 %3, a215\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a212, %0\n\tv_accvgpr_write_b32 a213, %1\n\tv_accvgpr_write_b32 a214, %2\n\tv_accvgpr_write_b32 a215, %3\n\tv_accvgpr_read_b32 %0, a216\n\tv_accvgpr_read_b32 %1, a217\n\tv_accvgpr_read_b32 %2, a218\n\tv_accvgpr_read_b32 %3, a219\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a216, %0\n\tv_accvgpr_write_b32 a217, %1\n\tv_accvgpr_write_b32 a218, %2\n\tv_accvgpr_write_b32 a219, %3\n\tv_accvgpr_read_b32 %0, a220\n\tv_accvgpr_read_b32 %1, a221\n\tv_accvgpr_read_b32 %2, a222\n\tv_accvgpr_read_b32 %3, a223\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a220, %0\n\tv_accvgpr_write_b32 a221, %1\n\tv_accvgpr_write_b32 a222, %2\n\tv_accvgpr_write_b32 a223, %3\n\tv_accvgpr_read_b32 %0, a224\n\tv_accvgpr_read_b32 %1, a225\n\tv_accvgpr_read_b32 %2, a226\n\tv_accvgpr_read_b32 %3, a227\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a224, %0\n\tv_accvgpr_write_b32 a225, %1\n\tv_accvgpr_write_b32 a226, %2\n\tv_accvgpr_write_b32 a227, %3\n\tv_accvgpr_read_b32 %0, a228\n\tv_accvgpr_read_b32 %1, a229\n\tv_accvgpr_read_b32 %2, a230\n\tv_accvgpr_read_b32 %3, a231\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a228, %0\n\tv_accvgpr_write_b32 a229, %1\n\tv_accvgpr_write_b32 a230, %2\n\tv_accvgpr_write_b32 a231, %3\n\tv_accvgpr_read_b32 %0, a232\n\tv_accvgpr_read_b32 %1, a233\n\tv_accvgpr_read_b32 %2, a234\n\tv_accvgpr_read_b32 %3, a235\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a232, %0\n\tv_accvgpr_write_b32 a233, %1\n\tv_accvgpr_write_b32 a234, %2\n\tv_accvgpr_write_b32 a235, %3\n\tv_accvgpr_read_b32 %0, a236\n\tv_accvgpr_read_b32 %1, a237\n\tv_accvgpr_read_b32 %2, a238\n\tv_accvgpr_read_b32 %3, a239\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a236, %0\n\tv_accvgpr_write_b32 a237, %1\n\tv_accvgpr_write_b32 a238, %2\n\tv_accvgpr_write_b32 a239, %3\n\tv_accvgpr_read_b32 %0, a240\n\tv_accvgpr_read_b32 %1, a241\n\tv_accvgpr_read_b32 %2, a242\n\tv_accvgpr_read_b32 %3, a243\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a240, %0\n\tv_accvgpr_write_b32 a241, %1\n\tv_accvgpr_write_b32 a242, %2\n\tv_accvgpr_write_b32 a243, %3\n\tv_accvgpr_read_b32 %0, a244\n\tv_accvgpr_read_b32 %1, a245\n\tv_accvgpr_read_b32 %2, a246\n\tv_accvgpr_read_b32 %3, a247\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a244, %0\n\tv_accvgpr_write_b32 a245, %1\n\tv_accvgpr_write_b32 a246, %2\n\tv_accvgpr_write_b32 a247, %3\n\tv_accvgpr_read_b32 %0, a248\n\tv_accvgpr_read_b32 %1, a249\n\tv_accvgpr_read_b32 %2, a250\n\tv_accvgpr_read_b32 %3, a251\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a248, %0\n\tv_accvgpr_write_b32 a249, %1\n\tv_accvgpr_write_b32 a250, %2\n\tv_accvgpr_write_b32 a251, %3\n\tv_accvgpr_read_b32 %0, a252\n\tv_accvgpr_read_b32 %1, a253\n\tv_accvgpr_read_b32 %2, a254\n\tv_accvgpr_read_b32 %3, a255\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\tv_accvgpr_write_b32 a252, %0\n\tv_accvgpr_write_b32 a253, %1\n\tv_accvgpr_write_b32 a254, %2\n\tv_accvgpr_write_b32 a255, %3\n\ts_nop 7"
               : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
               : "v"(x)
               : MLA_AGPR_CLOBBERS_ALL);
}

// the wait states of a 16-pass product before its accumulators are read
__device__ __forceinline__ void acc_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

template <bool W = true>
__device__ __forceinline__ void acc_mfma_i(int db, const bf16x8& v, const bf16x8& p) {
  switch (db) {
    case 0: acc_mfma<0, W>(v, p); break;
    case 1: acc_mfma<1, W>(v, p); break;
    case 2: acc_mfma<2, W>(v, p); break;
    case 3: acc_mfma<3, W>(v, p); break;
    case 4: acc_mfma<4, W>(v, p); break;
    case 5: acc_mfma<5, W>(v, p); break;
    case 6: acc_mfma<6, W>(v, p); break;
    case 7: acc_mfma<7, W>(v, p); break;
    case 8: acc_mfma<8, W>(v, p); break;
    case 9: acc_mfma<9, W>(v, p); break;
    case 10: acc_mfma<10, W>(v, p); break;
    case 11: acc_mfma<11, W>(v, p); break;
    case 12: acc_mfma<12, W>(v, p); break;
    case 13: acc_mfma<13, W>(v, p); break;
    case 14: acc_mfma<14, W>(v, p); break;
    default: acc_mfma<15, W>(v, p); break;
  }
}

__device__ __forceinline__ void acc_read_i(int db, float (&e)[16]) {
  switch (db) {
    case 0: acc_read<0>(e); break;
    case 1: acc_read<1>(e); break;
    case 2: acc_read<2>(e); break;
    case 3: acc_read<3>(e); break;
    case 4: acc_read<4>(e); break;
    case 5: acc_read<5>(e); break;
    case 6: acc_read<6>(e); break;
    case 7: acc_read<7>(e); break;
    case 8: acc_read<8>(e); break;
    case 9: acc_read<9>(e); break;
    case 10: acc_read<10>(e); break;
    case 11: acc_read<11>(e); break;
    case 12: acc_read<12>(e); break;
    case 13: acc_read<13>(e); break;
    case 14: acc_read<14>(e); break;
    default: acc_read<15>(e); break;
  }
}

// Sparse mode of the row-wave kernel: one 1 KB slot of a half page, every
// lane's 16 bytes from its own address (global_load_lds_dwordx4: 64-bit
// address per lane, LDS destination M0 + 16 * lane), and the row ids of a
// page (global_load_lds_dword: 4 bytes per lane to M0 + 4 * lane).  Same asm
// rationale as half_load_slot: the compiler must not track these loads.
__device__ __forceinline__ void rowwave_sparse_slot(uint32_t m0, const char* src) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a], off"
               :
               : [m] "s"(m0), [a] "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void rowwave_sparse_dword(uint32_t m0, const char* src) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dword %[a], off"
               :
               : [m] "s"(m0), [a] "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void rowwave_rid_load(uint32_t m0, const int32_t* src) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dword %[a], off"
               :
               : [m] "s"(m0), [a] "v"(src)
               : "memory", "m0");
}

// The row-wave kernel's body.  SP: sparse mode (items of selected entries,
// every row gathered through its resolved row id; see rowwave_sparse_slot).
template <bool SP>
__device__ __forceinline__ void rowwave_body(const DecodeArgs& a) {
  constexpr int NBUF = kWSBufs;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kHalfBytes];
  __shared__ int plan_lds[8];
  __shared__ int so_lds[kPlanMaxBatch + 1];
  // sparse: each wave's copy of the row ids of the next two pages to issue
  // ([wave][page parity][entry]); a wave reads only what it loaded itself
  __shared__ int rid_lds[SP ? 4 : 1][2][kBlock];

  const int tid = threadIdx.x;
  const int w = uni(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;    // the lane's query row within the wave
  const int lh = lane >> 5;    // lane half: keys 4lh + 8j + i of a 32-key unit

  int part, rtile;
  part_of_block(blockIdx.x, a.row_tiles, a.num_parts, SP, part, rtile);
  int b0, k0, b1, k1, first_split;
  const bool inplan = !SP && a.inplan;   // the sparse mode always reads its plan
  if (inplan) {
    if (w == 0) {
      plan_part_wave(a, part, plan_lds, so_lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (rtile == 0 && lane < kMetaInts)
        a.tile_meta_out[part * kMetaInts + lane] = lane < 5 ? plan_lds[lane] : 0;
      if (part == 0 && rtile == 0)
        for (int b = lane; b <= a.batch; b += 64) a.split_offsets_out[b] = so_lds[b];
    }
    wg_barrier();
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
  if (!before_end(a, cb, ck, b1, k1)) return;   // uniform: empty part
  int cL = seqlen_of(a, cb);
  const int row = rtile * kRWRows + 32 * w + lr;   // < M (M is a multiple of 128)
  // Kernel arguments read again from the kernel argument segment where they
  // are used (through an opaque pointer; the argument block is the kernel's
  // only parameter), so that the compiler keeps neither them nor addresses
  // derived from them in registers across the page loop.  The sparse kernel
  // uses it for the arguments only it needs and for the outputs, which it
  // has no registers to spare for.
  auto args = [&]() {
    typedef const __attribute__((address_space(4))) DecodeArgs* KArgs;
    KArgs p = (KArgs)(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(p));
    return p;
  };
  const int tok = row / a.h_q;

  auto piece_slot = [&](int b, int pbeg, int pend, int n, bool& whole) {
    whole = pbeg == 0 && pend == n;
    const int sidx = (b == b0 && k0 > 0) ? first_split : 0;
    if (whole) return 0LL;
    return (long long)(inplan ? uni(so_lds[b]) : ldc(a.split_offsets + b)) + sidx;
  };

  // ---- LDS operand offsets (unit buffer relative; rows swizzled by rw_swizzle) ----
  // K (score A operand) of step s: row lr, 16-byte unit 2s + lh, i.e.
  // ko[s & 3] + 128 (s >> 2).
  int ko[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) ko[qd] = lr * kRowBytes + (((2 * qd + lh) ^ rw_swizzle(lr)) << 4);
  // V (value A operand) of dim block db, key step u, read jj: 16-lane group G
  // reads keys 16u + 8jj + 4(G >> 1) + (i >> 2), 8 bytes at dims
  // 32db + 16(G & 1) + 4(i & 3); the transpose hands lane i the four keys of
  // dim 32db + 16(G & 1) + i.  Offset: vo[db & 1] + (16u + 8jj) rows + 128 (db >> 1),
  // with vo[] ^ 16 for jj = 1: row bit 3 flips bit 0 of the swizzled unit,
  // i.e. bit 4 of the offset (rows are multiples of 128 bytes, the 8-byte
  // half sits below bit 4).
  int vo[2];
  {
    const int G = lane >> 4, i = lane & 15;
    const int vr = 4 * (G >> 1) + (i >> 2);
    const int c0 = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int d1 = 0; d1 < 2; ++d1)
      vo[d1] = vr * kRowBytes + (((4 * d1 + c0) ^ rw_swizzle(vr)) << 4) + ((i & 1) << 3);
  }

  // ---- Q of the first piece (B operand of the score product) ----
  bf16x8 qreg[36];
  auto load_q = [&](int b) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + ((long long)b * a.M + row) * kDK) + lh;
#pragma unroll
    for (int s = 0; s < 36; ++s) qreg[s] = qp[2 * s];
  };
  // The compiler's view of Q: every register has arrived (it then waits here,
  // once per piece, instead of before the score products of every phase,
  // where its count would also cover the page loads issued in between).
  auto q_ready = [&]() {
    asm volatile("" ::"v"(qreg[0]), "v"(qreg[1]), "v"(qreg[2]), "v"(qreg[3]), "v"(qreg[4]),
                 "v"(qreg[5]), "v"(qreg[6]), "v"(qreg[7]), "v"(qreg[8]), "v"(qreg[9]),
                 "v"(qreg[10]), "v"(qreg[11]), "v"(qreg[12]), "v"(qreg[13]), "v"(qreg[14]),
                 "v"(qreg[15]), "v"(qreg[16]), "v"(qreg[17]));
    asm volatile("" ::"v"(qreg[18]), "v"(qreg[19]), "v"(qreg[20]), "v"(qreg[21]), "v"(qreg[22]),
                 "v"(qreg[23]), "v"(qreg[24]), "v"(qreg[25]), "v"(qreg[26]), "v"(qreg[27]),
                 "v"(qreg[28]), "v"(qreg[29]), "v"(qreg[30]), "v"(qreg[31]), "v"(qreg[32]),
                 "v"(qreg[33]), "v"(qreg[34]), "v"(qreg[35]));
  };
  load_q(cb);

  // ---- page ring: two page slots of two 36 KB halves ----
  // Page p of the part lands in slot p & 1 (ring buffers 2(p & 1) and
  // 2(p & 1) + 1 hold its key rows 0-31 and 32-63).  Phase p computes page p
  // while page p + 1 streams into the other slot.  A page is issued in two
  // steps so that no scalar load waits on the issue path: prefetch_page()
  // (end of a phase, before its barrier) moves the issue cursor and loads the
  // page id; issue_page() (after the barrier) builds the two halves' buffer
  // resources, and this wave's 18 slots then go out one at a time between
  // the score products (issue_slot).
  int ib = cb, ik = ck, iL = cL;
  int issued = 0;           // pages issued
  int off[9];   // the global offsets of this wave's slots w, w + 4, ..., w + 32 of a half
#pragma unroll
  for (int m = 0; m < 9; ++m) {
    const int p = 256 * m + tid;
    const int r = p / kChunksPerRow;
    const int pc = p - r * kChunksPerRow;
    off[m] = r * kRowBytes + ((pc ^ rw_swizzle(r)) << 4);
  }
  bool pf_on = false;       // a page is at the issue cursor
  int pf_page = -1, pf_rows = 0;
  bool hl_on = false;       // the slots of an issued page are pending
  HalfLoad hla, hlb;
  uint32_t vring = 0;       // bit p & 1: page p's slot names a page of the pool
  auto prefetch_page = [&](bool advance) {
    if (advance) page_next(a, ib, ik, iL, b1, k1);
    pf_on = before_end(a, ib, ik, b1, k1);
    if (pf_on) {
      const int rows = iL - ik * kBlock;
      pf_rows = rows > kBlock ? kBlock : rows;

      if constexpr (!SP)
        pf_page = ik < a.bt_stride ? ldc(a.block_table + (long long)ib * a.bt_stride + ik) : -1;
    }
  };
  // sparse: the row ids of the page at the issue cursor are in rid_lds
  // (parity issued & 1); rid_pre holds the one this lane's next slot needs,
  // read a slot ahead so that the LDS latency stays off the issue path.
  // (Entries past the item's end hold entry 0's id: their rows load but
  // every key there is masked.)  The packed offsets pass through an empty
  // Slot m's chunk offset in its row (low half-word) and row of the half
  // (high half-word) are recomputed at each use from an opaque copy of tid,
  // so that the compiler keeps no per-slot values in registers across the
  // loop (the sparse kernel has no registers to spare for them).
  int rid_pre = -1;
  auto slot_word = [&](int m) {
    int t2 = tid;
    asm volatile("" : "+v"(t2));
    const int p = 256 * (m % 9) + t2;
    const int r = p / kChunksPerRow;
    return (((p - r * kChunksPerRow) ^ rw_swizzle(r)) << 4) | (r << 16);
  };
  auto read_rid = [&](int m) {
    const int e = (m / 9) * kHalfRows + (slot_word(m) >> 16);
    rid_pre = rid_lds[w][(issued - 1) & 1][e];
  };
  auto issue_page = [&]() {
    hl_on = pf_on;
    if constexpr (SP) {
      if (hl_on) {
        hla.m0 = uni(static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((MLA_LDS char*)(smem + 2 * (issued & 1) * kHalfBytes)) +
            w * 1024));
        hlb.m0 = hla.m0 + kHalfBytes;
        vring |= 1u << (issued & 1);
        ++issued;
        read_rid(0);
      }
    } else if (hl_on) {
      const bool in_pool = pf_page >= 0 && (long long)pf_page < a.num_blocks;
      const bool ok = in_pool && pf_rows > 0;
      const char* base = reinterpret_cast<const char*>(a.kcache) +
                         (ok ? (long long)pf_page * kPageBytes : 0);
      const int ra = ok ? (pf_rows > kHalfRows ? kHalfRows : pf_rows) : 0;
      const int rb = ok && pf_rows > kHalfRows ? pf_rows - kHalfRows : 0;
      hla.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, uni(ra * kRowBytes),
                                                kRsrcWord3);
      hlb.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + kHalfBytes), 0,
                                                uni(rb * kRowBytes), kRsrcWord3);
      hla.m0 = uni(static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((MLA_LDS char*)(smem + 2 * (issued & 1) * kHalfBytes)) +
          w * 1024));
      hlb.m0 = hla.m0 + kHalfBytes;
      const uint32_t bit = 1u << (issued & 1);
      vring = in_pool ? (vring | bit) : (vring & ~bit);
      ++issued;
    }
  };
  // slot m of the page: half m / 9, slot m % 9 of that half
  auto issue_slot = [&](int m) {
    if constexpr (SP) {
      if (hl_on) {
        const int rid = rid_pre;
        if (m + 1 < 18) read_rid(m + 1);
        // the lane's 16 bytes: its chunk of its row, read from the row's
        // cache row (the zero row for an entry that does not count)
        const int coff = slot_word(m) & 0xffff;
        const char* src = (rid >= 0 ? reinterpret_cast<const char*>(a.kcache) + (long long)rid * kRowBytes
                                    : reinterpret_cast<const char*>(a.zero_row)) + coff;
        rowwave_sparse_slot((m < 9 ? hla.m0 : hlb.m0) + (m % 9) * 0x1000, src);
      }
    } else {
      if (hl_on) half_load_slot(m < 9 ? hla : hlb, off[m % 9], m % 9);
    }
  };
  // sparse: the row ids of the page after the one at the issue cursor
  // (next = true) or of that page itself, into this wave's rid_lds copy of
  // parity par, one direct-to-LDS dword per lane; lanes past the item's end
  // reload entry 0.  An item has ceil(const_len / 64) pages.
  auto rid_load = [&](int par, bool next) {
    int rb = ib, rk = ik;
    if (next) {
      const int npi = (a.const_len + kBlock - 1) / kBlock;
      if (++rk == npi) {
        ++rb;
        rk = 0;
      }
    }
    if (before_end(a, rb, rk, b1, k1)) {
      const long long e0 = (long long)rb * a.const_len + rk * kBlock;
      const int rows = a.const_len - rk * kBlock;
      const int32_t* src = args()->rowids + e0 + (lane < rows ? lane : 0);
      const uint32_t m0 = uni(static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((MLA_LDS int*)(&rid_lds[w][par][0]))));
      rowwave_rid_load(m0, src);
    }
  };
  auto wait_page = [&](int p) {
    wait_loads_behind<2 * kHalfLoadsPerWave, 1>(issued - p - 1);
  };

  // page 0, all slots at once; page 1's id on its way
  prefetch_page(false);
  if constexpr (SP) {
    rid_load(0, false);   // pages 0 and 1
    rid_load(1, true);
    vm_wait<0>();
  }
  issue_page();
#pragma unroll
  for (int m = 0; m < 18; ++m) issue_slot(m);
  prefetch_page(true);
  wait_page(0);
  q_ready();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();

  const bf16x8 zero8 = bf16x8{};
  acc_zero_all(zero8);

  // ---- per piece (the run of the part's pages of one request) ----
  float m_run = -INFINITY, l_run = 0.f;   // running max (log2 units) and sum of the lane's row
  int pbeg = ck, npg = n_pages(cL);
  int lim = (!SP && a.causal) ? cL - a.s_q + 1 + tok : cL;   // (the sparse mode is never causal)
  int lim_min = (!SP && a.causal) ? cL - a.s_q + 1 : cL;
  bool first = true;        // the phase's page starts a piece

  // O / l of the finished piece: bf16 to out for a whole request, fp32
  // partial otherwise, with its LSE; then the accumulators restart
  auto piece_end = [&](int b) {
    float lt = l_run;
    {
      const unsigned li = __float_as_uint(lt);
      const auto p32 = __builtin_amdgcn_permlane32_swap(li, li, false, false);
      lt = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    }
    const float lse2 = lt > 0.f ? m_run + log2f(lt) : -INFINITY;
    bool whole;
    const long long slot = piece_slot(b, pbeg, (b == b1) ? k1 : npg, npg, whole);
    const float linv = lt > 0.f ? 1.f / lt : 0.f;
    float* const lse_p = SP ? args()->lse : a.lse;
    float* const plse_p = SP ? args()->part_lse : a.part_lse;
    uint16_t* const out_p = SP ? args()->out : a.out;
    uint16_t* const po_p = SP ? args()->part_o : a.part_o;
    if (lh == 0) {
      if (whole)
        lse_p[(long long)b * a.M + row] = lse2 * kLn2;
      else
        plse_p[slot * a.M + row] = lse2;
    }
    acc_drain();
    // O / l rounded to bf16: the output row of a whole request, else the
    // piece's partial row
    uint16_t* const op = whole ? out_p + ((long long)b * a.M + row) * kDV + 4 * lh
                               : po_p + (slot * a.M + row) * kDV + 4 * lh;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      float e[16];
      acc_read_i(db, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 bv = {(__bf16)(e[4 * j] * linv), (__bf16)(e[4 * j + 1] * linv),
                           (__bf16)(e[4 * j + 2] * linv), (__bf16)(e[4 * j + 3] * linv)};
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j) = bv;
      }
    }
    acc_zero_all(zero8);
  };

  // Softmax of one 32-key half, in steps placed between matrix products,
  // each small enough to issue within one product's execution: step 0 takes
  // the in-lane maximum (and masks, when the half holds keys past the
  // visible count or its page slot is invalid); step 1 the row maximum (one
  // permlane32 swap) and the lazy-rescale decision; steps 2-17 one
  // exponential each (the odd ones pack two probabilities into bf16);
  // step 18 the row-sum update.
  // Exponent: exp2(x * cx - m) as one fma.  An unmasked half keeps the raw
  // q.k sums (x = s, cx = scale * log2 e; for a scale >= 0 the scaled maximum
  // is the maximum of the raw sums times it); a masked half is rewritten in
  // place as scaled sums with -inf at the masked keys (cx = 1).
  constexpr int kSmxSteps = 19;
  const bool scale_neg = a.scale_log2 < 0.f;
  float mx = -INFINITY, neg_m = 0.f, cx = 1.f, alpha = 1.f, lsum = 0.f, p_even = 0.f;
  bool resc_any = false;
  // kbase: position of the half's first key; valid: its page is in the pool;
  // restart: the half starts a piece
  // vmh (sparse): bit e says whether entry kbase + e counts
  auto softmax_step = [&](int st, f32x16& sv, bf16x8 (&pv)[2], int kbase, bool valid,
                          bool restart, uint32_t vmh) {
    if (st == 0) {
      if (restart) {
        m_run = -INFINITY;
        l_run = 0.f;
      }
      const bool need_mask = scale_neg || !valid || kbase + kHalfRows > lim_min ||
                             (SP && vmh != ~0u);
      if (!need_mask) {
        float m0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
        float m1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
        float m2 = fmaxf(fmaxf(sv[6], sv[7]), sv[8]);
        float m3 = fmaxf(fmaxf(sv[9], sv[10]), sv[11]);
        float m4 = fmaxf(fmaxf(sv[12], sv[13]), sv[14]);
        m0 = fmaxf(fmaxf(m0, m1), m2);
        m3 = fmaxf(fmaxf(m3, m4), sv[15]);
        mx = fmaxf(m0, m3) * a.scale_log2;
        cx = a.scale_log2;
      } else {
        asm volatile("");   // a branch of its own: the unmasked path does none of this
        const int key0 = kbase + 4 * lh;   // element 4j + i: key key0 + 8j + i
        const int lim_u = valid ? lim : -1;
        mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float xv = sv[4 * j + i] * a.scale_log2;
            if (key0 + 8 * j + i >= lim_u) xv = -INFINITY;
            if (SP && !((vmh >> (8 * j + 4 * lh + i)) & 1u)) xv = -INFINITY;
            sv[4 * j + i] = xv;
            mx = fmaxf(mx, xv);
          }
        cx = 1.f;
      }
    } else if (st == 1) {
      const unsigned mi = __float_as_uint(mx);
      const auto p32 = __builtin_amdgcn_permlane32_swap(mi, mi, false, false);
      mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = m_new > m_run + kRescaleSlack;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      // O of a piece is still zero when its first maximum arrives
      resc_any = __any(grow && m_run != -INFINITY);
      if (grow) m_run = m_new;
      l_run *= alpha;
      neg_m = m_run == -INFINITY ? 0.f : -m_run;
      lsum = 0.f;
    } else if (st < 18) {
      const int e = st - 2;
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], cx, neg_m));
      lsum += p;
      if ((e & 1) == 0) {
        p_even = p;
      } else {
        pv[e >> 3][(e & 7) - 1] = (__bf16)p_even;
        pv[e >> 3][e & 7] = (__bf16)p;
      }
    } else {
      l_run += lsum;
    }
  };

  // The value product of one half: 16 dim blocks x 2 key steps, blocks
  // innermost, V read D2 products ahead; with SMX the softmax steps of
  // another half sit between its products.
  auto value_product = [&](const char* vbuf, bf16x8 (&pv)[2], bool smx, f32x16& s2,
                           bf16x8 (&p2)[2], int kb2, bool valid2, uint32_t vm2) {
    constexpr int D2 = 2;
    bf16x4 vlo[D2 + 1], vhi[D2 + 1];
    auto read_v = [&](int st) {
      const int u = st >> 4, db = st & 15;
      const char* vb = vbuf + vo[db & 1] + 128 * (db >> 1) + 16 * u * kRowBytes;
      const char* vb1 = vbuf + (vo[db & 1] ^ 16) + 128 * (db >> 1) + (16 * u + 8) * kRowBytes;
      vlo[st % (D2 + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(vb));
      vhi[st % (D2 + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(vb1));
    };
#pragma unroll
    for (int st = 0; st < D2; ++st) read_v(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + D2 < 32) read_v(i + D2);
      const bf16x4 lo = vlo[i % (D2 + 1)], hi = vhi[i % (D2 + 1)];
      const bf16x8 va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc_mfma_i<false>(i & 15, va, pv[i >> 4]);
      // the other half's exponentials come after the products that read
      // P[0], so that its P[0] can take those registers
      if (smx && i == 2) softmax_step(0, s2, p2, kb2, valid2, false, vm2);
      if (smx && i == 4) softmax_step(1, s2, p2, kb2, valid2, false, vm2);
      if (smx && i >= 16) softmax_step(i - 14, s2, p2, kb2, valid2, false, vm2);
      asm volatile("" ::"v"(va));   // operand registers held past the product's issue
      __builtin_amdgcn_sched_barrier(0);
    }
    if (smx) softmax_step(kSmxSteps - 1, s2, p2, kb2, valid2, false, vm2);
    // the last products may still read P: wait states before its registers
    // can be reused
    asm volatile("s_nop 7" ::"v"(pv[0]), "v"(pv[1]));
  };

  // The score product of one half (K read D1 products ahead), the page's
  // slots SLOT0 .. SLOT0 + 8 issued between its products; with SMX the
  // softmax steps of another half sit between them too.
  constexpr int D1 = 3;
  auto score_chain = [&](const char* kbuf, f32x16& sacc, int slot0, bool smx, f32x16& s2,
                         bf16x8 (&p2)[2], int kb2, bool valid2, bool restart2, uint32_t vm2) {
    constexpr int NK = D1 + 1;   // K operand ring: a slot is rewritten one step after its product
    bf16x8 ka[NK];
    auto read_k = [&](int ks) {
      ka[ks % NK] = *reinterpret_cast<const bf16x8*>(kbuf + ko[ks & 3] + 128 * (ks >> 2));
    };
#pragma unroll
    for (int ks = 0; ks < D1; ++ks) read_k(ks);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      if (i + D1 < 36) read_k(i + D1);
      if (slot0 == 0) {
        if (i == 0)
          score_mfma_first<0, false>(sacc, ka[0], qreg[0]);
        else if (i < 35)
          score_mfma<0, false>(sacc, ka[i % NK], qreg[i]);
        else
          score_mfma_last<0, false>(sacc, ka[i % NK], qreg[i]);
      } else {
        if (i == 0)
          score_mfma_first<1, false>(sacc, ka[0], qreg[0]);
        else if (i < 35)
          score_mfma<1, false>(sacc, ka[i % NK], qreg[i]);
        else
          score_mfma_last<1, false>(sacc, ka[i % NK], qreg[i]);
      }
      if ((i & 3) == 1) issue_slot(slot0 + (i >> 2));
      if (smx && i >= 2 && i - 2 < kSmxSteps)
        softmax_step(i - 2, s2, p2, kb2, valid2, restart2, vm2);
      // the product may still be reading its K operand: the register stays
      // allocated (no VALU result lands in it) until here.  (Only this step's
      // operand: naming the register of a read still in flight would make
      // the compiler wait for that read here.)
      asm volatile("" ::"v"(ka[i % NK]));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the pipeline: phase t computes page t (slot t & 1) ----
  //   scores of half A (page rows 0-31);
  //   scores of half B (rows 32-63) with A's softmax between the products;
  //   values of A with B's softmax between the products; values of B.
  // Page t + 1 is issued between the score products; a page with 32 rows or
  // fewer has no half B.
  int t = 0;
  while (true) {
    const bool valid = ((vring >> (t & 1)) & 1u) != 0;
    if (first && t > 0) {
      // Q of the new piece, before this phase's page loads (so that waiting
      // for it does not also wait for them: loads complete in order)
      load_q(cb);
      q_ready();
    }
    // sparse: validity words of page t's halves (bit e: entry e counts)
    uint32_t vm_a = ~0u, vm_b = ~0u;
    if constexpr (SP) {
      const uint32_t* vw = args()->vmask + (long long)cb * (a.const_len / 32) + 2 * ck;
      vm_a = static_cast<uint32_t>(ldc(reinterpret_cast<const int32_t*>(vw)));
      vm_b = (ck + 1) * kBlock > a.const_len ? 0u
                                              : static_cast<uint32_t>(ldc(reinterpret_cast<const int32_t*>(vw + 1)));
    }
    issue_page();   // page t + 1 into the other slot
    if constexpr (SP) rid_load(t & 1, true);   // page t + 2: lands by this phase's end
    const char* bufa = smem + 2 * (t & 1) * kHalfBytes;
    const char* bufb = bufa + kHalfBytes;
    const int kb = ck * kBlock;
    f32x16 sa, sb;
    bf16x8 pa[2], pb[2];
    // (a page of 32 rows or fewer runs half B too: its rows were loaded as
    // zeros and all of its keys are masked)
    score_chain(bufa, sa, 0, false, sa, pa, kb, valid, first, vm_a);
    score_chain(bufb, sb, 9, true, sa, pa, kb, valid, first, vm_a);
    if (resc_any) acc_scale_all(alpha);
    value_product(bufa, pa, true, sb, pb, kb + kHalfRows, valid, vm_b);
    if (resc_any) acc_scale_all(alpha);
    value_product(bufb, pb, false, sb, pb, kb + kHalfRows, valid, vm_b);

    // the compute cursor moves to the next page; a piece ends with its request
    const int pbi = cb;
    page_next(a, cb, ck, cL, b1, k1);
    const bool more = before_end(a, cb, ck, b1, k1);
    first = !(more && cb == pbi);
    if (first) piece_end(pbi);
    if (!more) break;
    if (first) {
      pbeg = ck;
      npg = n_pages(cL);
      lim = (!SP && a.causal) ? cL - a.s_q + 1 + tok : cL;
      lim_min = (!SP && a.causal) ? cL - a.s_q + 1 : cL;
    }
    prefetch_page(true);   // completes while this wave waits at the barrier
    wait_page(t + 1);
    wg_barrier();   // page t + 1 landed in every wave's slots; page t's slot is free
    ++t;
  }
}

__global__ __launch_bounds__(kRWThreads, 1) void mla_rowwave_kernel(const DecodeArgs a) {
  rowwave_body<false>(a);
}

// Sparse mode (bf16 cache): the item's selected entries in pages of 64, each
// row gathered from its resolved cache row (or the zero row), entries that do
// not count masked by their validity bits.
__global__ __launch_bounds__(kRWThreads, 1) void mla_rowwave_sparse_kernel(const DecodeArgs a) {
  rowwave_body<true>(a);
}

// FP8 unit of the row-wave kernel in LDS: code rows padded to 33 16-byte
// units (528 B) and rope rows to 9 (144 B), so that every operand read of the
// kernel is a per-lane base plus a constant and both read patterns hit
// distinct banks (16 consecutive rows at one unit land on (r + c) mod 16);
// the code region takes 17 one-kilobyte load slots, the rope region 5.
constexpr int kF8RwCodeRow = 33 * 16;                  // 528
constexpr int kF8RwRopeRow = 9 * 16;                   // 144
constexpr int kF8RwRope = 17 * 1024;                   // 17408: rope region
constexpr int kF8RwScale = kF8RwRope + 5 * 1024;       // 22528: 32 fp32 scales
constexpr int kF8RwUnit = kF8RwScale + 256;            // 22784

// One direct-to-LDS load of an FP8 unit region: 16 bytes per lane (a 1 KB
// slot), or 4 bytes per lane (the unit's scales).  Same asm rationale as
// half_load_slot.
__device__ __forceinline__ void f8_slot_x4(__amdgpu_buffer_rsrc_t r, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[o], %[r], 0 offen lds"
               :
               : [m] "s"(m0), [r] "s"(r), [o] "v"(voff)
               : "memory", "m0");
}
__device__ __forceinline__ void f8_slot_x1(__amdgpu_buffer_rsrc_t r, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tbuffer_load_dword %[o], %[r], 0 offen lds"
               :
               : [m] "s"(m0), [r] "s"(r), [o] "v"(voff)
               : "memory", "m0");
}

// mla_rowwave_kernel over an FP8 cache (pages of MLA_FP8_PAGE_BYTES: E4M3
// latent codes, bf16 rope, one fp32 scale per token).  Same rows per wave,
// phases and softmax as the bf16 kernel; what differs:
//  * a half page is an FP8 unit in LDS (kF8RwUnit: padded code and rope
//    rows and the 32 scales, 22,784 B), so the ring holds three pages: the
//    one computed and two in flight;
//  * scores: a 16-byte code read gives two 16-dim steps of K (codes
//    converted exactly to bf16); Q takes the same dim order (step 2p + e of
//    lane half h covers dims 32p + 16h + 8e .. +8).  The 32 latent products
//    give the raw code sum, which the key's scale multiplies before the four
//    rope products accumulate on top;
//  * values: the transposing 8-bit read hands a lane dim d of eight keys,
//    converted to bf16; P carries the key's scale (P' = bf16(p * scale)),
//    the row sum takes p itself.
template <bool SP>
__device__ __forceinline__ void rowwave_f8_body(const DecodeArgs& a) {
  constexpr int kSlots = 3;                      // page slots of the ring
  constexpr int kUnit = kF8RwUnit;               // one half page
  __shared__ __attribute__((aligned(1024))) char smem[kSlots * 2 * kUnit];
  __shared__ int plan_lds[8];
  __shared__ int so_lds[kPlanMaxBatch + 1];
  // sparse: each wave's copy of the row ids of two pages ([wave][page parity][entry])
  __shared__ int rid_lds[SP ? 4 : 1][2][kBlock];

  const int tid = threadIdx.x;
  const int w = uni(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;    // the lane's query row within the wave
  const int lh = lane >> 5;    // lane half: keys 4lh + 8j + i of a 32-key unit

  int part, rtile;
  part_of_block(blockIdx.x, a.row_tiles, a.num_parts, SP, part, rtile);
  int b0, k0, b1, k1, first_split;
  const bool inplan = !SP && a.inplan;   // the sparse mode always reads its plan
  if (inplan) {
    if (w == 0) {
      plan_part_wave(a, part, plan_lds, so_lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (rtile == 0 && lane < kMetaInts)
        a.tile_meta_out[part * kMetaInts + lane] = lane < 5 ? plan_lds[lane] : 0;
      if (part == 0 && rtile == 0)
        for (int b = lane; b <= a.batch; b += 64) a.split_offsets_out[b] = so_lds[b];
    }
    wg_barrier();
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
  if (!before_end(a, cb, ck, b1, k1)) return;   // uniform: empty part
  int cL = seqlen_of(a, cb);
  const int row = rtile * kRWRows + 32 * w + lr;   // < M (M is a multiple of 128)
  const int tok = row / a.h_q;
  // Kernel arguments read again from the kernel argument segment where they
  // are used (through an opaque pointer; the argument block is the kernel's
  // only parameter), so that the compiler keeps neither them nor addresses
  // derived from them in registers across the page loop (sparse mode).
  auto args = [&]() {
    typedef const __attribute__((address_space(4))) DecodeArgs* KArgs;
    KArgs p = (KArgs)(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(p));
    return p;
  };

  auto piece_slot = [&](int b, int pbeg, int pend, int n, bool& whole) {
    whole = pbeg == 0 && pend == n;
    const int sidx = (b == b0 && k0 > 0) ? first_split : 0;
    if (whole) return 0LL;
    return (long long)(inplan ? uni(so_lds[b]) : ldc(a.split_offsets + b)) + sidx;
  };

  // ---- LDS operand offsets (unit relative; padded rows, see kF8RwUnit) ----
  // Score, latent step pair p (steps 2p, 2p+1): code row lr, 16-byte unit
  // 2p + lh: kco + 32p.
  const int kco = lr * kF8RwCodeRow + 16 * lh;
  // Score, rope step s (dims 512 + 16s + 8lh): rope row lr, unit 2s + lh:
  // kro + 32s.
  const int kro = kF8RwRope + lr * kF8RwRopeRow + 16 * lh;
  // Value A operand of dim block db, key step u: 16-lane group G, lane i
  // reads 8 codes of key row 16u + 8(i >> 3) + 4(G >> 1) + ((i >> 1) & 3), its
  // half (i & 1) of code unit 2db + (G & 1); the 8-bit transpose hands lane i
  // dim 32db + 16(G & 1) + i of the group's eight keys, which are P's
  // elements 8(e >> 2) + 4(G >> 1) + (e & 3) of the step.  Offset:
  // vco + 16u rows + 32db.
  int vco;
  {
    const int G = lane >> 4, i = lane & 15;
    const int kr = 8 * (i >> 3) + 4 * (G >> 1) + ((i >> 1) & 3);   // key row in step 0
    vco = kr * kF8RwCodeRow + 16 * (G & 1) + 8 * (i & 1);
  }

  // ---- Q of the first piece (B operand of the score product) ----
  bf16x8 qreg[36];
  // qreg[2p + e] = dims 32p + 16lh + 8e .. +8 (latent), qreg[32 + s] = dims
  // 512 + 16s + 8lh .. +8 (rope)
  // Sparse: the lane id counted afresh where it is used (an asm the
  // compiler cannot merge with another), and the row rebuilt from it, so
  // that neither is kept, and spilled, across the page loop.
  auto lane_now = [&]() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto row_at = [&]() {
    if constexpr (SP)
      return uni(rtile * kRWRows + 32 * w) + (lane_now() & 31);
    else
      return row;
  };
  auto load_q = [&](int b) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + ((long long)b * a.M + row_at()) * kDK);
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) {
      qreg[2 * pp] = qp[4 * pp + 2 * lh];
      qreg[2 * pp + 1] = qp[4 * pp + 2 * lh + 1];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) qreg[32 + s] = qp[64 + 2 * s + lh];
  };
  // The compiler's view of Q: every register has arrived (it then waits here,
  // once per piece, instead of before the score products of every phase,
  // where its count would also cover the page loads issued in between).
  auto q_ready = [&]() {
    asm volatile("" ::"v"(qreg[0]), "v"(qreg[1]), "v"(qreg[2]), "v"(qreg[3]), "v"(qreg[4]),
                 "v"(qreg[5]), "v"(qreg[6]), "v"(qreg[7]), "v"(qreg[8]), "v"(qreg[9]),
                 "v"(qreg[10]), "v"(qreg[11]), "v"(qreg[12]), "v"(qreg[13]), "v"(qreg[14]),
                 "v"(qreg[15]), "v"(qreg[16]), "v"(qreg[17]));
    asm volatile("" ::"v"(qreg[18]), "v"(qreg[19]), "v"(qreg[20]), "v"(qreg[21]), "v"(qreg[22]),
                 "v"(qreg[23]), "v"(qreg[24]), "v"(qreg[25]), "v"(qreg[26]), "v"(qreg[27]),
                 "v"(qreg[28]), "v"(qreg[29]), "v"(qreg[30]), "v"(qreg[31]), "v"(qreg[32]),
                 "v"(qreg[33]), "v"(qreg[34]), "v"(qreg[35]));
  };
  load_q(cb);

  // ---- page ring: three page slots of two FP8 units ----
  // Page p lands in slot p % 3 (units 2(p % 3) and 2(p % 3) + 1: key rows
  // 0-31 and 32-63).  Phase p computes page p while pages p + 1 and p + 2
  // stream in.  Issue as in the bf16 kernel: prefetch_page() moves the issue
  // cursor and loads the page id before a barrier, issue_page() after it, and
  // the slots go out between the score products.  Per unit this wave loads
  // code slots w + 4k (k < 4, 1 KB each), rope slot w (1 KB) and, for wave
  // 0, the unit's 32 scales; each region of each unit has its own buffer
  // range, so rows past the request's length land as zeros.
  int ib = cb, ik = ck, iL = cL;
  int issued = 0;           // pages issued
  // A unit takes 23 loads of 64 lanes: code slots 0-16 and rope slots 0-4
  // (1 KB each, lane l of slot m carrying 16-byte unit 64m + l of the padded
  // region; pad units and units past the region read nothing and land as
  // zeros) and its 32 scales (4 bytes a lane).  Wave w issues code slots
  // 4k + w (k < 4) and rope slot w; the remaining three go to waves 0-2:
  // code slot 16, rope slot 4, the scales.  Per page: 12 loads per wave,
  // 10 for wave 3.
  constexpr int kNoLoad = 0x40000000;   // an offset past every buffer range
  auto code_off = [](int q) {           // 16-byte unit q of the padded code region
    const int r = q / 33, c = q - 33 * (q / 33);
    return (r < kHalfRows && c < 32) ? r * kF8Latent + 16 * c : kNoLoad;
  };
  auto rope_off = [](int q) {
    const int r = q / 9, c = q - 9 * (q / 9);
    return (r < kHalfRows && c < 8) ? r * 128 + 16 * c : kNoLoad;
  };
  int offc[4], offr, offx;
  // sparse: per slot m (0..5) a 16-bit word, two slots to a register
  // (spk[m >> 1], half m & 1): the row of the unit that the lane's bytes
  // belong to (bits 11-15), the region (bits 9-10: 0 codes, 1 rope, 2
  // scales, 3 nothing) and the 16-byte unit in the row (bits 0-8)
  int spk[3];
  if constexpr (SP) {
    auto word = [&](int m) {
      const bool code = m < 4 || (m == 5 && w == 0);
      const bool rope = m == 4 || (m == 5 && w == 1);
      int r = 0, kind = 3, c = 0;
      if (code) {
        const int q = 64 * (m < 4 ? 4 * m + w : 16) + lane;
        r = q / 33;
        c = q - 33 * r;
        kind = (r < kHalfRows && c < 32) ? 0 : 3;
      } else if (rope) {
        const int q = 64 * (m == 4 ? w : 4) + lane;
        r = q / 9;
        c = q - 9 * r;
        kind = (r < kHalfRows && c < 8) ? 1 : 3;
      } else if (w == 2) {
        r = lane;
        kind = lane < kHalfRows ? 2 : 3;
      }
      return ((r < kHalfRows ? r : 0) << 11) | (kind << 9) | c;
    };
#pragma unroll
    for (int k = 0; k < 3; ++k) spk[k] = word(2 * k) | (word(2 * k + 1) << 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) offc[k] = code_off(64 * (4 * k + w) + lane);
    offr = rope_off(64 * w + lane);
    offx = w == 0 ? code_off(64 * 16 + lane) : w == 1 ? rope_off(64 * 4 + lane)
                                               : (lane < kHalfRows ? 4 * lane : kNoLoad);
  }
  bool pf_on = false;       // a page is at the issue cursor
  int pf_page = -1, pf_rows = 0;
  bool hl_on = false;       // the slots of an issued page are pending
  const char* hl_pg = nullptr;   // the issued page (or the pool start when it reads nothing)
  int hl_rows = 0;          // its rows to load (0: none)
  uint32_t hl_m0 = 0;       // LDS address of its slot's unit 0
  uint32_t vring = 0;       // bit p % 3: page p's slot names a page of the pool
  auto prefetch_page = [&](bool advance) {
    if (advance) page_next(a, ib, ik, iL, b1, k1);
    pf_on = before_end(a, ib, ik, b1, k1);
    if (pf_on) {
      const int rows = iL - ik * kBlock;
      pf_rows = rows > kBlock ? kBlock : rows;
      if constexpr (!SP)
        pf_page = ik < a.bt_stride ? ldc(a.block_table + (long long)ib * a.bt_stride + ik) : -1;
    }
  };
  // Sparse: a lane's part of slot m (0..5) of unit u: the entry (row of the
  // page) it loads, and the byte offset in a cache page of its data relative
  // to that row's own (-1 for a lane that loads nothing), unpacked from the
  // slot's word through an empty asm so that the compiler keeps only the
  // packed words across the loop.
  // returns the byte offset of the lane's data in a cache page relative to
  // its row's own (-1: nothing to load); *e receives the entry; *stride the
  // region's row pitch
  auto sp_lane = [&](int u, int m, int* e, int* stride) {
    int pk = spk[m >> 1];
    asm volatile("" : "+v"(pk));
    // (unsigned: a row of 16 or more sets bit 31 of the upper word)
    const int wd = static_cast<int>((m & 1) ? (static_cast<uint32_t>(pk) >> 16)
                                            : (static_cast<uint32_t>(pk) & 0xffffu));
    *e = u * kHalfRows + (wd >> 11);
    const int kind = (wd >> 9) & 3, c = wd & 511;
    *stride = kind == 0 ? kF8Latent : kind == 1 ? 128 : 4;
    return kind == 3 ? -1 : kind == 0 ? 16 * c : kind == 1 ? kF8RopeOff + 16 * c : kF8ScaleOff;
  };
  // the row id of this lane's next slot, read from rid_lds a slot ahead
  int rid_pre = -1;
  auto read_rid = [&](int u, int m) {
    int e, st;
    (void)sp_lane(u, m, &e, &st);
    rid_pre = rid_lds[w][(issued - 1) & 1][e];
  };
  // the row ids of the page after the one at the issue cursor (next) or of
  // that page, into this wave's rid_lds copy of parity par, one
  // direct-to-LDS dword per lane; lanes past the item's end reload entry 0
  auto rid_load = [&](int par, bool next) {
    int rb = ib, rk = ik;
    if (next) {
      const int npi = (a.const_len + kBlock - 1) / kBlock;
      if (++rk == npi) {
        ++rb;
        rk = 0;
      }
    }
    if (before_end(a, rb, rk, b1, k1)) {
      const long long e0 = (long long)rb * a.const_len + rk * kBlock;
      const int rows = a.const_len - rk * kBlock;
      const int ln = lane_now();
      const int32_t* src = args()->rowids + e0 + (ln < rows ? ln : 0);
      const uint32_t m0 = uni(static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((MLA_LDS int*)(&rid_lds[w][par][0]))));
      rowwave_rid_load(m0, src);
    }
  };
  auto issue_page = [&]() {
    hl_on = pf_on;
    if constexpr (SP) {
      if (hl_on) {
        const int sl = issued % kSlots;
        hl_m0 = uni(static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((MLA_LDS char*)(smem + 2 * sl * kUnit))));
        vring |= 1u << sl;
        ++issued;
        read_rid(0, 0);
      }
    } else if (hl_on) {
      const bool in_pool = pf_page >= 0 && (long long)pf_page < a.num_blocks;
      const bool ok = in_pool && pf_rows > 0;
      hl_pg = reinterpret_cast<const char*>(a.kcache) + (ok ? (long long)pf_page * kF8PageBytes : 0);
      hl_rows = ok ? pf_rows : 0;
      const int sl = issued % kSlots;
      hl_m0 = uni(static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((MLA_LDS char*)(smem + 2 * sl * kUnit))));
      const uint32_t bit = 1u << sl;
      vring = in_pool ? (vring | bit) : (vring & ~bit);
      ++issued;
    }
  };
  // slot m (0..5) of unit u of the issued page for this wave: code slots
  // 4m + w (m < 4), rope slot w (m = 4), the extra one (m = 5)
  auto issue_slot = [&](int u, int m) {
    if (!hl_on || (m == 5 && w == 3)) return;
    if constexpr (SP) {
      const int rid = rid_pre;
      // the next slot's row id (unit 1 follows unit 0; wave 3 has no slot 5)
      const int last = w == 3 ? 4 : 5;
      if (m < last)
        read_rid(u, m + 1);
      else if (u == 0)
        read_rid(1, 0);
      int e, stride;
      const int off = sp_lane(u, m, &e, &stride);
      const char* src = (off >= 0 && rid >= 0)
                            ? reinterpret_cast<const char*>(a.kcache) +
                                  (long long)(rid >> 6) * kF8PageBytes + off + (rid & 63) * stride
                            : reinterpret_cast<const char*>(a.zero_row);
      const uint32_t ub = hl_m0 + u * kUnit;
      const bool code = m < 4 || (m == 5 && w == 0);
      const bool rope = m == 4 || (m == 5 && w == 1);
      if (code)
        rowwave_sparse_slot(ub + (m < 4 ? 4 * m + w : 16) * 1024, src);
      else if (rope)
        rowwave_sparse_slot(ub + kF8RwRope + (m == 4 ? w : 4) * 1024, src);
      else
        rowwave_sparse_dword(ub + kF8RwScale, src);
      return;
    }
    int ru = hl_rows - u * kHalfRows;
    ru = ru < 0 ? 0 : (ru > kHalfRows ? kHalfRows : ru);
    const uint32_t ub = hl_m0 + u * kUnit;
    const char* codes = hl_pg + u * kHalfRows * kF8Latent;
    const char* rope = hl_pg + kF8RopeOff + u * kHalfRows * 128;
    if (m < 4) {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(codes), 0,
                                                       uni(ru * kF8Latent), kRsrcWord3);
      f8_slot_x4(r, ub + (4 * m + w) * 1024, offc[m]);
    } else if (m == 4 || w == 1) {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rope), 0, uni(ru * 128),
                                                       kRsrcWord3);
      f8_slot_x4(r, ub + kF8RwRope + (m == 4 ? w : 4) * 1024, m == 4 ? offr : offx);
    } else if (w == 0) {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(codes), 0,
                                                       uni(ru * kF8Latent), kRsrcWord3);
      f8_slot_x4(r, ub + 16 * 1024, offx);
    } else {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(hl_pg + kF8ScaleOff + u * kHalfRows * 4), 0, uni(ru * 4), kRsrcWord3);
      f8_slot_x1(r, ub + kF8RwScale, offx);
    }
  };
  // this wave's loads of one page: 12, 10 for wave 3
  auto wait_page = [&](int p) {
    if (issued - p - 1 >= 1) {
      if (w == 3)
        vm_wait<10>();
      else
        vm_wait<12>();
    } else {
      vm_wait<0>();
    }
  };

  // pages 0 and 1, all slots at once; page 2's id on its way
  prefetch_page(false);
  if constexpr (SP) {
    rid_load(0, false);   // pages 0 and 1
    rid_load(1, true);
    vm_wait<0>();
  }
#pragma unroll
  for (int pg = 0; pg < 2; ++pg) {
    issue_page();
    if (SP && pg == 1) rid_load(0, true);   // page 2, ahead of page 1's slots
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int m = 0; m < 6; ++m) issue_slot(u, m);
    prefetch_page(true);
  }
  wait_page(0);
  q_ready();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();

  const bf16x8 zero8 = bf16x8{};
  acc_zero_all(zero8);

  // ---- per piece (the run of the part's pages of one request) ----
  float m_run = -INFINITY, l_run = 0.f;   // running max (log2 units) and sum of the lane's row
  int pbeg = ck, npg = n_pages(cL);
  int lim = (!SP && a.causal) ? cL - a.s_q + 1 + tok : cL;
  int lim_min = (!SP && a.causal) ? cL - a.s_q + 1 : cL;
  bool first = true;        // the phase's page starts a piece

  // O / l of the finished piece: bf16 to out for a whole request, fp32
  // partial otherwise, with its LSE; then the accumulators restart
  auto piece_end = [&](int b) {
    float lt = l_run;
    {
      const unsigned li = __float_as_uint(lt);
      const auto p32 = __builtin_amdgcn_permlane32_swap(li, li, false, false);
      lt = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    }
    const float lse2 = lt > 0.f ? m_run + log2f(lt) : -INFINITY;
    bool whole;
    const long long slot = piece_slot(b, pbeg, (b == b1) ? k1 : npg, npg, whole);
    const float linv = lt > 0.f ? 1.f / lt : 0.f;
    float* const lse_p = SP ? args()->lse : a.lse;
    float* const plse_p = SP ? args()->part_lse : a.part_lse;
    uint16_t* const out_p = SP ? args()->out : a.out;
    uint16_t* const po_p = SP ? args()->part_o : a.part_o;
    const int rr = row_at();
    if (lh == 0) {
      if (whole)
        lse_p[(long long)b * a.M + rr] = lse2 * kLn2;
      else
        plse_p[slot * a.M + rr] = lse2;
    }
    acc_drain();
    // O / l rounded to bf16: the output row of a whole request, else the
    // piece's partial row
    uint16_t* const op = whole ? out_p + ((long long)b * a.M + rr) * kDV + 4 * lh
                               : po_p + (slot * a.M + rr) * kDV + 4 * lh;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      float e[16];
      acc_read_i(db, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 bv = {(__bf16)(e[4 * j] * linv), (__bf16)(e[4 * j + 1] * linv),
                           (__bf16)(e[4 * j + 2] * linv), (__bf16)(e[4 * j + 3] * linv)};
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j) = bv;
      }
    }
    acc_zero_all(zero8);
  };

  // Softmax of one 32-key half, in steps placed between matrix products,
  // each small enough to issue within one product's execution: step 0 takes
  // the in-lane maximum (and masks, when the half holds keys past the
  // visible count or its page slot is invalid); step 1 the row maximum (one
  // permlane32 swap) and the lazy-rescale decision; steps 2-17 one
  // exponential each (the odd ones pack two probabilities into bf16);
  // step 18 the row-sum update.
  // Exponent: exp2(x * cx - m) as one fma.  An unmasked half keeps the raw
  // q.k sums (x = s, cx = scale * log2 e; for a scale >= 0 the scaled maximum
  // is the maximum of the raw sums times it); a masked half is rewritten in
  // place as scaled sums with -inf at the masked keys (cx = 1).
  constexpr int kSmxSteps = 19;
  const bool scale_neg = a.scale_log2 < 0.f;
  float mx = -INFINITY, neg_m = 0.f, cx = 1.f, alpha = 1.f, lsum = 0.f, p_even = 0.f;
  bool resc_any = false;
  // kbase: position of the half's first key; valid: its page is in the pool;
  // restart: the half starts a piece
  // ubuf: the half's unit (the key scales: element 4j + i is key 8j + 4lh + i)
  f32x4 ksc, ksc_n;   // scales of elements 4j .. 4j+3, and of the next group (read ahead)
  // vmh (sparse): bit e says whether entry kbase + e counts
  auto softmax_step = [&](int st, f32x16& sv, bf16x8 (&pv)[2], int kbase, bool valid,
                          bool restart, const char* ubuf, uint32_t vmh) {
    if (st == 0) {
      if (restart) {
        m_run = -INFINITY;
        l_run = 0.f;
      }
      const bool need_mask = scale_neg || !valid || kbase + kHalfRows > lim_min ||
                             (SP && vmh != ~0u);
      if (!need_mask) {
        float m0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
        float m1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
        float m2 = fmaxf(fmaxf(sv[6], sv[7]), sv[8]);
        float m3 = fmaxf(fmaxf(sv[9], sv[10]), sv[11]);
        float m4 = fmaxf(fmaxf(sv[12], sv[13]), sv[14]);
        m0 = fmaxf(fmaxf(m0, m1), m2);
        m3 = fmaxf(fmaxf(m3, m4), sv[15]);
        mx = fmaxf(m0, m3) * a.scale_log2;
        cx = a.scale_log2;
      } else {
        asm volatile("");   // a branch of its own: the unmasked path does none of this
        const int key0 = kbase + 4 * lh;   // element 4j + i: key key0 + 8j + i
        const int lim_u = valid ? lim : -1;
        mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float xv = sv[4 * j + i] * a.scale_log2;
            if (key0 + 8 * j + i >= lim_u) xv = -INFINITY;
            if (SP && !((vmh >> (8 * j + 4 * lh + i)) & 1u)) xv = -INFINITY;
            sv[4 * j + i] = xv;
            mx = fmaxf(mx, xv);
          }
        cx = 1.f;
      }
    } else if (st == 1) {
      const unsigned mi = __float_as_uint(mx);
      const auto p32 = __builtin_amdgcn_permlane32_swap(mi, mi, false, false);
      mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = m_new > m_run + kRescaleSlack;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      // O of a piece is still zero when its first maximum arrives
      resc_any = __any(grow && m_run != -INFINITY);
      if (grow) m_run = m_new;
      l_run *= alpha;
      neg_m = m_run == -INFINITY ? 0.f : -m_run;
      lsum = 0.f;
      if constexpr (SP)   // (sparse: no read-ahead, for the gather's registers)
        ksc = *reinterpret_cast<const f32x4*>(ubuf + kF8RwScale + 4 * (4 * lh));
      else
        ksc_n = *reinterpret_cast<const f32x4*>(ubuf + kF8RwScale + 4 * (4 * lh));
    } else if (st < 18) {
      const int e = st - 2;
      if constexpr (SP) {
        if ((e & 3) == 0 && e > 0)
          ksc = *reinterpret_cast<const f32x4*>(ubuf + kF8RwScale + 4 * (2 * e + 4 * lh));
      } else {
        if ((e & 3) == 0) ksc = ksc_n;
        if ((e & 3) == 1 && e < 12)   // the next group's scales, three steps ahead
          ksc_n = *reinterpret_cast<const f32x4*>(ubuf + kF8RwScale + 4 * (2 * (e + 3) + 4 * lh));
      }
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], cx, neg_m));
      lsum += p;
      // the value operand holds raw codes: P carries the key's scale
      const float ps = p * ksc[e & 3];
      if ((e & 1) == 0) {
        p_even = ps;
      } else {
        pv[e >> 3][(e & 7) - 1] = (__bf16)p_even;
        pv[e >> 3][e & 7] = (__bf16)ps;
      }
    } else {
      l_run += lsum;
    }
  };

  // The value product of one half: 16 dim blocks x 2 key steps, blocks
  // innermost; V^T is one 8-bit transposed read of codes per product (read
  // D2 products ahead), converted exactly to bf16.  With SMX the softmax
  // steps of another half sit between its products.
  auto value_product = [&](const char* vbuf, bf16x8 (&pv)[2], bool smx, f32x16& s2,
                           bf16x8 (&p2)[2], int kb2, bool valid2, const char* ubuf2,
                           uint32_t vm2) {
    constexpr int D2 = SP ? 1 : 2;   // (sparse: one read less in flight, for the gather's registers)
    i32x2 vc[D2 + 1];
    auto read_v = [&](int st) {
      const int u = st >> 4, db = st & 15;
      vc[st % (D2 + 1)] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (MLA_LDS i32x2*)((MLA_LDS char*)(vbuf) + vco + 16 * kF8RwCodeRow * u + 32 * db));
    };
#pragma unroll
    for (int st = 0; st < D2; ++st) read_v(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + D2 < 32) read_v(i + D2);
      const i32x2 c = vc[i % (D2 + 1)];
      const bf16x8 va = e4m3x8_to_bf16(static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1]));
      acc_mfma_i(i & 15, va, pv[i >> 4]);
      // the other half's exponentials come after the products that read
      // P[0], so that its P[0] can take those registers
      if (smx && i == 2) softmax_step(0, s2, p2, kb2, valid2, false, ubuf2, vm2);
      if (smx && i == 4) softmax_step(1, s2, p2, kb2, valid2, false, ubuf2, vm2);
      if (smx && i >= 16) softmax_step(i - 14, s2, p2, kb2, valid2, false, ubuf2, vm2);
      asm volatile("" ::"v"(va));   // operand registers held past the product's issue
      __builtin_amdgcn_sched_barrier(0);
    }
    if (smx) softmax_step(kSmxSteps - 1, s2, p2, kb2, valid2, false, ubuf2, vm2);
    // the last products may still read P: wait states before its registers
    // can be reused
    asm volatile("s_nop 7" ::"v"(pv[0]), "v"(pv[1]));
  };

  // The score product of one half: 32 latent steps (a 16-code read, two
  // reads ahead, gives two steps), the key scales applied to the code sum,
  // then the 4 rope steps.  This wave's slots of unit U of the issued page go
  // out between the latent products; with SMX the softmax steps of another
  // half sit between them too.  BLK: the half's pinned accumulator block.
  auto score_chain = [&](const char* kbuf, f32x16& sacc, int U, bool smx, f32x16& s2,
                         bf16x8 (&p2)[2], int kb2, bool valid2, bool restart2,
                         const char* ubuf2, uint32_t vm2) {
    u32x4 kc[2];
    auto read_c = [&](int pp) {
      kc[pp & 1] = *reinterpret_cast<const u32x4*>(kbuf + kco + 32 * pp);
    };
    auto mfma = [&](int i, const bf16x8& k, const bf16x8& q) {
      if (U == 0) {
        if (i == 0)
          score_mfma_first<0>(sacc, k, q);
        else if (i == 31 || i == 35)
          score_mfma_last<0>(sacc, k, q);
        else
          score_mfma<0>(sacc, k, q);
      } else {
        if (i == 0)
          score_mfma_first<1>(sacc, k, q);
        else if (i == 31 || i == 35)
          score_mfma_last<1>(sacc, k, q);
        else
          score_mfma<1>(sacc, k, q);
      }
    };
    read_c(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int pp = i >> 1;
      if ((i & 1) == 1 && pp + 1 < 16) read_c(pp + 1);   // the next pair, once this pair's
                                                         // first half is converted
      const u32x4 c = kc[pp & 1];
      const bf16x8 kv = (i & 1) ? e4m3x8_to_bf16(c[2], c[3]) : e4m3x8_to_bf16(c[0], c[1]);
      mfma(i, kv, qreg[i]);
      if (i % 6 == 1) issue_slot(U, i / 6);
      if (smx && i >= 2 && i - 2 < kSmxSteps)
        softmax_step(i - 2, s2, p2, kb2, valid2, restart2, ubuf2, vm2);
      asm volatile("" ::"v"(kv));   // the product's operand stays allocated until here
      __builtin_amdgcn_sched_barrier(0);
    }
    // the code sum times the key's scale (element 4j + i: key 8j + 4lh + i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(kbuf + kF8RwScale + 4 * (8 * j + 4 * lh));
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[4 * j + i] *= sc[i];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 kr = *reinterpret_cast<const bf16x8*>(kbuf + kro + 32 * st);
      mfma(32 + st, kr, qreg[32 + st]);
      asm volatile("" ::"v"(kr));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the pipeline: phase t computes page t (slot t % 3) ----
  //   scores of half A (page rows 0-31);
  //   scores of half B (rows 32-63) with A's softmax between the products;
  //   values of A with B's softmax between the products; values of B.
  // Page t + 2 is issued between the score products.
  int t = 0;
  while (true) {
    const int slot = t % kSlots;
    const bool valid = ((vring >> slot) & 1u) != 0;
    if (first && t > 0) {
      // Q of the new piece, before this phase's page loads (so that waiting
      // for it does not also wait for them: loads complete in order)
      load_q(cb);
      q_ready();
    }
    // sparse: validity words of page t's halves (bit e: entry e counts)
    uint32_t vm_a = ~0u, vm_b = ~0u;
    if constexpr (SP) {
      const uint32_t* vw = args()->vmask + (long long)cb * (a.const_len / 32) + 2 * ck;
      vm_a = static_cast<uint32_t>(ldc(reinterpret_cast<const int32_t*>(vw)));
      vm_b = (ck + 1) * kBlock > a.const_len ? 0u
                                              : static_cast<uint32_t>(ldc(reinterpret_cast<const int32_t*>(vw + 1)));
    }
    issue_page();   // page t + 2 into the slot of page t - 1
    if constexpr (SP) rid_load((t + 1) & 1, true);   // page t + 3, ahead of page t + 2's slots
    const char* bufa = smem + 2 * slot * kUnit;
    const char* bufb = bufa + kUnit;
    const int kb = ck * kBlock;
    f32x16 sa, sb;
    bf16x8 pa[2], pb[2];
    // (a page of 32 rows or fewer runs half B too: its rows were loaded as
    // zeros and all of its keys are masked)
    score_chain(bufa, sa, 0, false, sa, pa, kb, valid, first, bufa, vm_a);
    score_chain(bufb, sb, 1, true, sa, pa, kb, valid, first, bufa, vm_a);
    if (resc_any) acc_scale_all(alpha);
    value_product(bufa, pa, true, sb, pb, kb + kHalfRows, valid, bufb, vm_b);
    if (resc_any) acc_scale_all(alpha);
    value_product(bufb, pb, false, sb, pb, kb + kHalfRows, valid, bufb, vm_b);

    // the compute cursor moves to the next page; a piece ends with its request
    const int pbi = cb;
    page_next(a, cb, ck, cL, b1, k1);
    const bool more = before_end(a, cb, ck, b1, k1);
    first = !(more && cb == pbi);
    if (first) piece_end(pbi);
    if (!more) break;
    if (first) {
      pbeg = ck;
      npg = n_pages(cL);
      // (the sparse mode is never causal: its items carry their own limits)
      lim = (!SP && a.causal) ? cL - a.s_q + 1 + tok : cL;
      lim_min = (!SP && a.causal) ? cL - a.s_q + 1 : cL;
    }
    prefetch_page(true);   // completes while this wave waits at the barrier
    wait_page(t + 1);
    wg_barrier();   // page t + 1 landed in every wave's slots; page t's slot is free
    ++t;
  }
}

__global__ __launch_bounds__(kRWThreads, 1) void mla_rowwave_f8_kernel(const DecodeArgs a) {
  rowwave_f8_body<false>(a);
}

// Sparse mode over FP8 pages: each selected row's codes, rope and scale
// gathered from its own page through its resolved row id (the zero row for
// an entry that does not count), entries that do not count masked.
__global__ __launch_bounds__(kRWThreads, 1) void mla_rowwave_f8_sparse_kernel(const DecodeArgs a) {
  rowwave_f8_body<true>(a);
}

// Rows per workgroup tile of the split plan: 128 when s_q*h_q is a multiple
// of 128 (the row-wave kernels), else the ws kernel's 16, 32 or 64.
int tile_rows_for(int M) {
  if (M % kRWRows == 0) return kRWRows;
  if (M <= 16) return 16;    // mla_splitkv_ws_kernel<1>
  if (M <= 32) return 32;    // mla_splitkv_ws_kernel<2>
  return 64;                 // mla_splitkv_ws_kernel<4>
}

// Rows per tile of the ws kernel (16, 32 or 64).
static int ws_tile_rows(int M) { return M <= 16 ? 16 : M <= 32 ? 32 : 64; }

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

hipError_t launch_splitkv(const DecodeArgs& args, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  DecodeArgs a = args;
  // 128-row tiles: the row-wave kernels (dense or sparse, either cache format)
  if (a.M % kRWRows == 0) {
    a.row_tile_rows = kRWRows;
    a.row_tiles = a.M / kRWRows;
    const dim3 grid(a.num_parts * a.row_tiles);
    const dim3 block(kRWThreads);
    const void* kern =
        a.sparse ? (a.kv_fp8 ? reinterpret_cast<const void*>(&mla_rowwave_f8_sparse_kernel)
                             : reinterpret_cast<const void*>(&mla_rowwave_sparse_kernel))
        : a.kv_fp8 ? reinterpret_cast<const void*>(&mla_rowwave_f8_kernel)
                   : reinterpret_cast<const void*>(&mla_rowwave_kernel);
    void* kargs[] = {&a};
    if (start == nullptr && stop == nullptr) {
      if (a.sparse && a.kv_fp8)
        hipLaunchKernelGGL(mla_rowwave_f8_sparse_kernel, grid, block, 0, stream, a);
      else if (a.sparse)
        hipLaunchKernelGGL(mla_rowwave_sparse_kernel, grid, block, 0, stream, a);
      else if (a.kv_fp8)
        hipLaunchKernelGGL(mla_rowwave_f8_kernel, grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL(mla_rowwave_kernel, grid, block, 0, stream, a);
    } else {
      hipError_t e = hipExtLaunchKernel(kern, grid, block, kargs, 0, stream, start, stop, 0);
      if (e != hipSuccess) return e;
    }
    return hipGetLastError();
  }
  a.row_tile_rows = ws_tile_rows(a.M);
  a.row_tiles = (a.M + a.row_tile_rows - 1) / a.row_tile_rows;
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
// 16 threads per row, 8 contiguous dims each (one 16-byte bf16 load per
// partial, so a row's 16 threads read 256 contiguous bytes).  Splitting the dims keeps
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
      *reinterpret_cast<uint4*>(op + 8 * j) = make_uint4(0u, 0u, 0u, 0u);
      if (j == 0 && blockIdx.z == 0) a.lse[(long long)b * a.M + r] = -INFINITY;
    }
    return;
  }
  // Merge in groups of four partials: each group's loads (LSEs and bf16
  // rows) go out together, then fold into a running (max, weight sum,
  // weighted row), the same exact log-sum-exp merge in a streaming order.
  // Lane j holds dims dq + 8j .. dq + 8j + 7 of row r.
  constexpr int G = 4;
  float mx = -INFINITY, tot = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; s += G) {
    float ls[G];
    bf16x8 po[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const bool ok = s + u < ns;
      const long long rowi = (long long)(s0 + (ok ? s + u : 0)) * a.M + r;
      ls[u] = ok ? a.part_lse[rowi] : -INFINITY;
      po[u] = *reinterpret_cast<const bf16x8*>(a.part_o + rowi * kDV + dq + 8 * j);
    }
    float gm = mx;
#pragma unroll
    for (int u = 0; u < G; ++u) gm = fmaxf(gm, ls[u]);
    if (gm == -INFINITY) continue;   // every partial so far is empty
    const float al = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - gm);
    tot *= al;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= al;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float wgt = ls[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[u] - gm);
      tot += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)po[u][e];
    }
    mx = gm;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  bf16x8 ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(op + 8 * j) = ov;
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
