// Device-side helpers shared by the gfx950 kernels: vector types for the bf16 MFMA
// operands, the 32x32x16 MFMA, LDS/global tile movers and small math helpers.
//
// MFMA register layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//  * operand A (32 x 16): lane l holds row l % 32 and eight k-slots selected by l / 32;
//  * operand B (16 x 32): lane l holds column l % 32 and the same eight k-slots;
//  * result (32 x 32 fp32, 16 registers): lane l holds column l % 32; register r holds
//    row 8 * (r / 4) + 4 * (l / 32) + r % 4.
// Because A and B share the lane-half -> k-slot assignment, a contraction is correct for
// any consistent mapping of the contracted index onto (lane half, slot); the kernels
// choose that mapping to match the result layout of the previous MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fcp_types.h"

namespace fcp {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2_t __attribute__((__vector_size__(2 * sizeof(float))));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, z);
}

// Eight fp32 values -> eight bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8_t to_bf16x8(const float* x) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

__device__ __forceinline__ float bf16_to_f32(u16 x) {
  return __uint_as_float((uint32_t)x << 16);
}

__device__ __forceinline__ u16 f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(u16, b);
}

// Max / sum of x over lanes l % 32 and l % 32 + 32 (the two halves of a 32x32 MFMA result
// column), in every lane. v_permlane32_swap exchanges the upper half of one operand with
// the lower half of the other, so its two results hold x[l % 32] and x[l % 32 + 32];
// no LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16: within each group of 16 lanes, source lane i = 4a + b names 4
// consecutive 16-bit elements (row a, columns 4b..4b+3 of a 4 x 16 block); result lane j
// receives column j of that block, rows 0..3.
__device__ __forceinline__ u32x2_t lds_tr4(const u16* p) {
  const v4i16_t r =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
  return __builtin_bit_cast(u32x2_t, r);
}

// ---- LDS tiles ---------------------------------------------------------------------
//
// A tile is ROWS x D bf16 stored row-major without padding, each 16-byte chunk c of row
// r at chunk position c ^ swz<D>(r). gfx950 LDS has 64 four-byte banks and serves a
// 16-byte read for 16 lanes per cycle, an 8-byte read for 32. The swizzle makes both
// read patterns below conflict-free:
//  * 16-byte row reads of 16 consecutive rows at one chunk (D = 128: one row spans all
//    64 banks, so the 16 rows need 16 distinct chunk positions; D = 64: two rows share a
//    bank line, so the 8 rows of each parity need 8 distinct positions);
//  * transpose reads of 4 consecutive rows x 4 chunks (rows at distinct chunk quads).
// swz<D>(r) depends on r % 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Buffer resource over `num_bytes` bytes at `base` (raw, no stride): loads at offsets
// past num_bytes return zero.
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, num_bytes, 0x00020000u};
}

// LDS address (byte offset in the workgroup's LDS) of a __shared__ object.
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}

// Direct global -> LDS load: lane l's 16 bytes at rsrc + voff land at LDS lds + 16 l
// (buffer_load_dwordx4 ... lds; M0 holds the wave-uniform LDS address). Issued through
// inline assembly on purpose: the compiler then does not see an LDS write in flight and
// does not wait for it (vmcnt(0)) before every later LDS read -- which would serialise
// each prefetch with the compute it should overlap. The kernels order these copies
// themselves: s_waitcnt vmcnt (loads complete in issue order) + barrier before the data
// is read, and a barrier after the last read of a slot before it is refilled.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Asynchronous global -> LDS copies of ROWS-row tiles of bf16 tensors whose rows are
// `stride` elements apart (one head's D columns per row) into swizzled LDS tiles. The
// per-lane global offsets depend only on the lane and the stride, so they are computed
// once per kernel; a copy then costs the buffer descriptor (scalar) and its loads. Every
// wave of the NW-wave workgroup issues its share (INSTS loads per tile); the data may be
// read after this wave's s_waitcnt vmcnt and a barrier. Each wave instruction fills 1 KB
// of the tile and the lane picks the global chunk that belongs at its LDS position; rows
// at or past `valid` read as zero (buffer range check).
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;       // chunks per row
  static constexpr int RPI = 64 / CPR;    // rows per wave instruction
  static constexpr int NI = ROWS / RPI;   // instructions per tile
  static constexpr int INSTS = NI / NW;   // per wave
  static_assert(NI % NW == 0, "tile must split over the waves");
  uint32_t voff[INSTS];  // this lane's byte offset from the tile's first row
  uint32_t lds0;         // this wave's first 1 KB block, in bytes (wave-uniform)
  int64_t stride;
  __device__ TileCopy(int64_t stride_, int wave, int lane) : stride(stride_) {
    const int w = __builtin_amdgcn_readfirstlane(wave);
    lds0 = (uint32_t)(w * INSTS * 1024);
#pragma unroll
    for (int i = 0; i < INSTS; ++i) {
      const int r = (w * INSTS + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(r);
      voff[i] = (uint32_t)(((int64_t)r * stride + c * 8) * 2);
    }
  }
  // Rows [row0, row0 + ROWS) from column col0 of `src` into `tile`.
  __device__ __forceinline__ void operator()(const u16* src, int64_t row0, int valid,
                                             int64_t col0, u16* tile) const {
    const int vrows = valid < 0 ? 0 : (valid > ROWS ? ROWS : valid);
    const uint32_t nbytes =
        vrows > 0 ? (uint32_t)(((int64_t)(vrows - 1) * stride + D) * 2) : 0u;
    const u32x4_t rsrc = buffer_rsrc(src + row0 * stride + col0, nbytes);
    const uint32_t base = lds_addr(tile) + lds0;
#pragma unroll
    for (int i = 0; i < INSTS; ++i) dma16(rsrc, base + i * 1024, voff[i]);
  }
};

// Number of loads one wave issues for one TileCopy<D, ROWS, NW> copy.
template <int D, int ROWS, int NW>
constexpr int tile_copy_insts() {
  return TileCopy<D, ROWS, NW>::INSTS;
}

// MFMA operand reads from a swizzled tile, with the per-lane LDS element offsets shared
// by every tile a lane reads (D / 8 registers).
//  * rowop(tile, row0, kc): lane row/column l % 32 taken from tile row row0 + l % 32,
//    slots 16 kc + 8 (l / 32) + 0..7 along the row (row0 % 16 == 0): K for S^T = K Q^T,
//    Q or dO for S = Q K^T.
//  * trA(tile, k16, c32): the A operand (32 x 16) of a contraction over the tile's ROW
//    index: result rows are tile columns c32 .. c32 + 31, slot s of lane half h is tile
//    row k16 + 8 (s / 4) + 4 h + s % 4 -- the row order of a 32x32 MFMA result, so the
//    B operand can come straight from result registers. Two ds_read_b64_tr_b16 of 4 rows
//    each, rows k16 + 0..7 and k16 + 8..15 (k16 % 16 == 0, c32 % 32 == 0).
template <int D>
struct TileOffsets {
  static constexpr int NKC = D / 16, NCB = D / 32;
  int row[NKC];
  int tr[2][NCB];
  __device__ explicit TileOffsets(int lane) {
    const int r = lane & 31, s = swz<D>(r), h = lane >> 5;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) row[kc] = r * D + (((2 * kc + h) ^ s) << 3);
    const int j = lane & 15, grp = lane >> 4;
    const int x = 2 * (grp & 1) + ((j & 3) >> 1);  // chunk within a 32-column block
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tr_r = 8 * half + 4 * (grp >> 1) + (j >> 2);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        tr[half][cb] = tr_r * D + (((4 * cb + x) ^ swz<D>(tr_r)) << 3) + 4 * (j & 1);
    }
  }
  __device__ __forceinline__ bf16x8_t rowop(const u16* tile, int row0, int kc) const {
    return *reinterpret_cast<const bf16x8_t*>(tile + row0 * D + row[kc]);
  }
  __device__ __forceinline__ bf16x8_t trA(const u16* tile, int k16, int c32) const {
    const u16* p = tile + k16 * D;
    const u32x2_t lo = lds_tr4(p + tr[0][c32 >> 5]), hi = lds_tr4(p + tr[1][c32 >> 5]);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
  }
};

// Workgroup barrier for LDS tiles filled by dma16: waits for this wave's own LDS (and
// scalar) operations, then s_barrier. Unlike __syncthreads, whose release fence also
// waits for every outstanding global load (vmcnt(0)), it leaves prefetches in flight; the
// callers wait for the copies a tile needs (wait_vmem / wait_vmem_le) before it. The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Element i of a work-list table (read-only for the kernel's lifetime), for a wave-
// uniform i, through the scalar cache: a vector load would make the compiler wait for
// every outstanding tile copy before using the value.
template <class T>
__device__ __forceinline__ T load_uniform(const T* table, int i) {
  static_assert(sizeof(T) == sizeof(u32x4_t), "16-byte records");
  const __attribute__((address_space(4))) u32x4_t* t =
      (const __attribute__((address_space(4))) u32x4_t*)table;
  return __builtin_bit_cast(T, t[__builtin_amdgcn_readfirstlane(i)]);
}

// Entry i of a workgroup launch map, through the scalar cache.
__device__ __forceinline__ WgMap load_wg(const WgMap* map, int i) {
  const __attribute__((address_space(4))) u32x2_t* t =
      (const __attribute__((address_space(4))) u32x2_t*)map;
  return __builtin_bit_cast(WgMap, t[__builtin_amdgcn_readfirstlane(i)]);
}

// Entry i of an int32 table, read through the scalar cache (a wave-uniform value).
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* table, int i) {
  const __attribute__((address_space(4))) int32_t* t =
      (const __attribute__((address_space(4))) int32_t*)table;
  return t[__builtin_amdgcn_readfirstlane(i)];
}

// Waits for this wave's outstanding vector-memory operations (the async tile copies).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Waits until at most N of this wave's vector-memory loads are outstanding (loads
// complete in issue order), leaving the export and LDS/scalar counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Optional shader-clock sampling for measurement tools. With a non-null `clk`, thread 0
// of each workgroup reads the shader-clock counter (s_memtime) and the 100 MHz reference
// counter (s_memrealtime) when the workgroup starts and when it finishes, and adds the
// two differences to clk[0] and clk[1]: their ratio over a launch is the average shader
// clock in units of 100 MHz, weighted by workgroup lifetime. A null `clk` costs one
// scalar branch at each end.
struct ClockStamp {
  uint64_t c0 = 0, r0 = 0;
  __device__ explicit ClockStamp(unsigned long long* clk) {
    if (clk && threadIdx.x == 0) {
      c0 = __builtin_amdgcn_s_memtime();
      r0 = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ void done(unsigned long long* clk) const {
    if (clk && threadIdx.x == 0) {
      const uint64_t c1 = __builtin_amdgcn_s_memtime();
      const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(clk, (unsigned long long)(c1 - c0));
      atomicAdd(clk + 1, (unsigned long long)(r1 - r0));
    }
  }
};

}  // namespace fcp
