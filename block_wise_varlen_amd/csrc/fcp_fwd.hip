// Forward block attention on gfx950: bf16 MFMA for QK^T and PV, fp32 online softmax.
//
// Computes, for a tile of query rows of one Q range and a group of query heads sharing
// one KV head, softmax(Q K^T * scale, masked) V over the KV ranges of its pairs (FCP
// paper Sec. 2.2, attention over [H, L, D] with causal or non-causal masks; the formula
// is legible on the paper's review page, section "核心公式与建模"). With one KV range
// per item it writes that pair's normalised partial and its LSE (the per-slice result
// of Sec. 2.2); with all KV ranges of a Q range it writes the final output directly.
//
// Design (one workgroup = 256 query columns, 8 waves of one 32-column block each):
//  * The scores are computed transposed, S^T = K Q^T, so each lane owns one (token,
//    head) column: the row max / row sum of the online softmax are in-lane reductions
//    plus one exchange between lane l and l + 32.
//  * Q^T stays in registers for the whole item (B operand). A workgroup covers the
//    query heads of one KV head (grouped-query attention, Sec. 2.2 and Sec. 6.1), so each
//    K/V tile staged in LDS is reused by all of them.
//  * O^T = V^T P^T: P comes straight from the S^T registers as the B operand; the V^T
//    A operand is read from the row-major V tile with the LDS transpose read.
//  * K and V tiles move from HBM straight into (swizzled) LDS with buffer loads that
//    bypass registers.
//  * The running max is only raised (and the accumulator rescaled) when a new score
//    exceeds it by more than 2^8, so in steady state the accumulator is touched by MFMAs
//    only; P <= 2^8 meanwhile, which bf16 and fp32 hold exactly as well as P <= 1.
//  * K/V tiles of 64 keys go through a 3-deep LDS ring: the copy of tile n+2 is issued
//    before the MFMAs of tile n, and tile n+1 is waited for at the end of the iteration.
#include "fcp_common.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

// log2 headroom before the running max is raised.
constexpr float kRescaleSlack = 8.0f;

// Keys per K/V tile of the forward and depth of its LDS ring.
#ifndef FCP_FWD_KT
#define FCP_FWD_KT 128
#endif
constexpr int kFwdKt = FCP_FWD_KT;
constexpr int kFwdBuf = kFwdKt == 64 ? 3 : 2;

// Number of kFwdKt-key tiles of segment `s` visible to queries [q_off, q_off + rows).
__device__ __forceinline__ int seg_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / kFwdKt + 1;
}

// Position in the flattened (KV segment, 64-key tile) sequence of one work item, over
// the tiles visible to queries [q_off, q_off + rows).
struct TileCursor {
  KvSeg sg;
  int s, t, nt;
  bool valid;
  __device__ static TileCursor first(const KvSeg* segs, int s0, int s_end, int q_off,
                                     int rows) {
    TileCursor c{};
    c.valid = false;
    for (c.s = s0; c.s < s_end; ++c.s) {
      c.sg = segs[c.s];
      c.nt = seg_tiles(c.sg, q_off, rows);
      if (c.nt > 0) {
        c.valid = true;
        c.t = 0;
        break;
      }
    }
    return c;
  }
  __device__ TileCursor next(const KvSeg* segs, int s_end, int q_off, int rows) const {
    if (!valid) return *this;
    if (t + 1 < nt) {
      TileCursor c = *this;
      c.t = t + 1;
      return c;
    }
    return first(segs, s + 1, s_end, q_off, rows);
  }
};

template <int D, bool FINAL, int CB>
__global__ __launch_bounds__(64 * kColBlocksPerWG / CB)
__attribute__((amdgpu_waves_per_eu(CB == 1 ? 2 : 1, CB == 1 ? 2 : 1)))
void fwd_kernel(FwdArgs a) {
  constexpr int NW = kColBlocksPerWG / CB;  // waves per workgroup
  constexpr int NKC = D / 16;   // k-chunks of the QK^T contraction
  constexpr int NDB = D / 32;   // d-blocks of the output
  constexpr int NBUF = kFwdBuf;  // tile ring depth
  constexpr int COPY_INSTS = 2 * tile_copy_insts<D, kFwdKt, NW>();
  __shared__ __attribute__((aligned(16))) u16 sK[NBUF][kFwdKt * D];
  __shared__ __attribute__((aligned(16))) u16 sV[NBUF][kFwdKt * D];

  const int item_idx = blockIdx.x / a.n_hgroups;
  const int hg = blockIdx.x - item_idx * a.n_hgroups;
  const QItem it = a.items[item_idx];
  const int head_base = hg * a.hpw;
  const int kvh = head_base / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q_stride = (int64_t)a.hq * D;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const TileOffsets<D> to(lane);

  int tok[CB], head[CB];
  bool valid[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int cbg = wave * CB + cb;
    tok[cb] = (cbg / a.hpw) * kColBlock + l32;
    head[cb] = head_base + cbg % a.hpw;
    valid[cb] = tok[cb] < it.q_rows;
  }

  // Q^T as B operand: lane holds column (tok, head), k-slots d = 16*kc + 8*hi + 0..7.
  bf16x8_t qb[CB][NKC];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const u16* qrow = a.q + (int64_t)(it.q_row0 + tok[cb]) * q_stride + (int64_t)head[cb] * D;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      qb[cb][kc] = valid[cb] ? *reinterpret_cast<const bf16x8_t*>(qrow + 16 * kc + 8 * hi)
                             : zero_bf16x8();
  }

  f32x16_t acc[CB][NDB];
  float m[CB], l[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = -INFINITY;
    l[cb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[cb][db] = zero16();
  }

  const int seg_end = it.seg_begin + it.seg_count;
  const int64_t kv_col = (int64_t)kvh * D;
  // Cursors over the flattened (segment, tile) sequence: the tile being computed and the
  // two after it, whose copies are in flight.
  TileCursor cur = TileCursor::first(a.segs, it.seg_begin, seg_end, it.q_off, it.q_rows);
  TileCursor nx1 = cur.next(a.segs, seg_end, it.q_off, it.q_rows);
  TileCursor nx2 = nx1.next(a.segs, seg_end, it.q_off, it.q_rows);
  auto copy = [&](const TileCursor& tc, int b) {
    const int j0n = tc.t * kFwdKt;
    tile_copy_async<D, kFwdKt, NW>(a.k, (int64_t)tc.sg.kv_start + j0n, tc.sg.kv_len - j0n,
                                   kv_stride, kv_col, sK[b], wave, lane);
    tile_copy_async<D, kFwdKt, NW>(a.v, (int64_t)tc.sg.kv_start + j0n, tc.sg.kv_len - j0n,
                                   kv_stride, kv_col, sV[b], wave, lane);
  };
  if (cur.valid) copy(cur, 0);
  if (NBUF == 3 && nx1.valid) copy(nx1, 1);
  if (NBUF == 3 && nx1.valid)
    wait_vmem_le<COPY_INSTS>();
  else
    wait_vmem();
  __syncthreads();
  int buf = 0;
  const float c = a.scale_log2;

  while (cur.valid) {
    // The ring slot after the in-flight ones was last read in the previous iteration,
    // which every wave has left (barrier), so the next copy may overwrite it.
    if (NBUF == 3) {
      if (nx2.valid) copy(nx2, buf == 0 ? 2 : buf - 1);
    } else {
      if (nx1.valid) copy(nx1, buf ^ 1);
    }
    const KvSeg sg = cur.sg;
    const int t = cur.t;

    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    const int j0 = t * kFwdKt;
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kFwdKt > sg.kv_len) ||
                           (causal && j0 + kFwdKt - 1 - it.q_off > sg.mask_offset);
    // 32-key blocks, software-pipelined: the S^T = K Q^T MFMAs of block kb + 1 are issued
    // before the softmax of block kb, so the matrix pipe works while the VALU does.
    constexpr int NKB = kFwdKt / 32;
    f32x16_t Sn[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      Sn[cb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) Sn[cb] = mfma32(to.rowop(Kt, 0, kc), qb[cb][kc], Sn[cb]);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16_t S[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = Sn[cb];
      if (kb + 1 < NKB) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          Sn[cb] = zero16();
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc)
            Sn[cb] = mfma32(to.rowop(Kt, (kb + 1) * 32, kc), qb[cb][kc], Sn[cb]);
        }
      }
      // Mask: key j (within the KV range) visible to query i iff j < kv_len and, causal,
      // j - i <= mask_offset.
      if (need_mask) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int jb = j0 + kb * 32;
          const int lim_c = sg.mask_offset + it.q_off + tok[cb] - jb;
          const int lim = causal ? min(sg.kv_len - jb - 1, lim_c) : sg.kv_len - jb - 1;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + 4 * hi + (r & 3) > lim) S[cb][r] = -INFINITY;
        }
      }
      // Online softmax in base 2 with the scale folded into the exponent; the running
      // max m is raised only when the block's max exceeds it by more than kRescaleSlack.
      bool raise[CB];
      float m_new[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[cb][r]);
        mx = pair_max(mx) * c;
        if (m[cb] == -INFINITY) {
          m[cb] = mx;  // nothing accumulated yet: no rescale needed
          raise[cb] = false;
        } else {
          raise[cb] = mx > m[cb] + kRescaleSlack;
        }
        m_new[cb] = fmaxf(m[cb], mx);
      }
      bool any_raise = false;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) any_raise = any_raise || raise[cb];
      if (__any(any_raise)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const float alpha = raise[cb] ? __builtin_amdgcn_exp2f(m[cb] - m_new[cb]) : 1.f;
          m[cb] = raise[cb] ? m_new[cb] : m[cb];
          l[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][db][r] *= alpha;
        }
      }
      bf16x8_t pb[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float m_use = (m[cb] == -INFINITY) ? 0.f : m[cb];
        // The row sum uses the fp32 values (the LSE must not carry bf16 rounding).
        float p[16], rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(S[cb][r], c, -m_use));
          rs += p[r];
        }
        l[cb] += rs;
        pb[cb][0] = to_bf16x8(p);
        pb[cb][1] = to_bf16x8(p + 8);
      }
      // O^T += V^T P^T over the block's 32 keys.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8_t va = to.trA(Vt, kb * 32 + 16 * half, db * 32);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][db] = mfma32(va, pb[cb][half], acc[cb][db]);
        }
    }

    // The next tile must have landed (with three slots its copy is older than the one
    // just issued, which may stay in flight).
    if (NBUF == 3 && nx2.valid)
      wait_vmem_le<COPY_INSTS>();
    else
      wait_vmem();
    __syncthreads();
    buf = buf == NBUF - 1 ? 0 : buf + 1;
    cur = nx1;
    nx1 = nx2;
    nx2 = nx2.next(a.segs, seg_end, it.q_off, it.q_rows);
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) ln 2; no visible key -> O = 0, LSE = -inf.
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = pair_sum(l[cb]);
    if (!valid[cb]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m[cb] + __log2f(lt)) * kLn2 : -INFINITY;
    const int64_t row = it.out_row0 + tok[cb];
    const int64_t base = (row * a.hq + head[cb]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        const float o0 = acc[cb][db][4 * g4 + 0] * inv, o1 = acc[cb][db][4 * g4 + 1] * inv;
        const float o2 = acc[cb][db][4 * g4 + 2] * inv, o3 = acc[cb][db][4 * g4 + 3] * inv;
        if constexpr (FINAL) {
          const uint32_t w0 = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16(o2) | ((uint32_t)f32_to_bf16(o3) << 16);
          *reinterpret_cast<u32x2_t*>(a.o + base + d) = u32x2_t{w0, w1};
        } else {
          *reinterpret_cast<f32x4_t*>(a.o_part + base + d) = f32x4_t{o0, o1, o2, o3};
        }
      }
    if (hi == 0) {
      if constexpr (FINAL)
        a.lse[row * a.hq + head[cb]] = lse;
      else
        a.lse_part[row * a.hq + head[cb]] = lse;
    }
  }
}

}  // namespace

// Column blocks per wave of the launched forward: 1 (8 waves, two per SIMD, so one
// wave's softmax overlaps the other's MFMAs) or 2 (4 waves, one per SIMD).
constexpr int kFwdCB = 1;

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool final_out, hipStream_t stream) {
  if (a.n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_items * (unsigned)a.n_hgroups), block(64 * kColBlocksPerWG / kFwdCB);
  if (head_dim == 128) {
    if (final_out)
      hipLaunchKernelGGL((fwd_kernel<128, true, kFwdCB>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<128, false, kFwdCB>), grid, block, 0, stream, a);
  } else {
    if (final_out)
      hipLaunchKernelGGL((fwd_kernel<64, true, kFwdCB>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<64, false, kFwdCB>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fcp
