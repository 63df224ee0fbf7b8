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
//  * K/V tiles of 64 keys are double-buffered: the copy of tile n+1 is issued before
//    the MFMAs of tile n and waited for at the end of the iteration.
#include "fcp_common.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

// log2 headroom before the running max is raised.
constexpr float kRescaleSlack = 8.0f;

// Number of 64-key tiles of segment `s` visible to queries [q_off, q_off + rows).
__device__ __forceinline__ int seg_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / kKvTile + 1;
}

template <int D, bool FINAL, int CB>
__global__ __launch_bounds__(64 * kColBlocksPerWG / CB)
__attribute__((amdgpu_waves_per_eu(CB == 1 ? 2 : 1, CB == 1 ? 2 : 1)))
void fwd_kernel(FwdArgs a) {
  constexpr int NW = kColBlocksPerWG / CB;  // waves per workgroup
  constexpr int NKC = D / 16;   // k-chunks of the QK^T contraction
  constexpr int NDB = D / 32;   // d-blocks of the output
  __shared__ __attribute__((aligned(16))) u16 sK[2][kKvTile * D];
  __shared__ __attribute__((aligned(16))) u16 sV[2][kKvTile * D];

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
  int s = it.seg_begin, t = 0, nt = 0;
  KvSeg sg{};
  for (; s < seg_end; ++s) {
    sg = a.segs[s];
    nt = seg_tiles(sg, it.q_off, it.q_rows);
    if (nt > 0) break;
  }
  bool have = s < seg_end;
  const int64_t kv_col = (int64_t)kvh * D;
  if (have) {
    tile_copy_async<D, kKvTile, NW>(a.k, sg.kv_start, sg.kv_len, kv_stride, kv_col, sK[0], wave,
                                    lane);
    tile_copy_async<D, kKvTile, NW>(a.v, sg.kv_start, sg.kv_len, kv_stride, kv_col, sV[0], wave,
                                    lane);
    wait_vmem();
  }
  __syncthreads();
  int buf = 0;
  const float c = a.scale_log2;

  while (have) {
    int ns = s, ntile = t + 1, nnt = nt;
    KvSeg nsg = sg;
    if (ntile >= nnt) {
      ntile = 0;
      for (++ns; ns < seg_end; ++ns) {
        nsg = a.segs[ns];
        nnt = seg_tiles(nsg, it.q_off, it.q_rows);
        if (nnt > 0) break;
      }
    }
    const bool next = ns < seg_end;
    if (next) {
      const int j0n = ntile * kKvTile;
      tile_copy_async<D, kKvTile, NW>(a.k, (int64_t)nsg.kv_start + j0n, nsg.kv_len - j0n,
                                      kv_stride, kv_col, sK[buf ^ 1], wave, lane);
      tile_copy_async<D, kKvTile, NW>(a.v, (int64_t)nsg.kv_start + j0n, nsg.kv_len - j0n,
                                      kv_stride, kv_col, sV[buf ^ 1], wave, lane);
    }

    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    const int j0 = t * kKvTile;
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kKvTile > sg.kv_len) ||
                           (causal && j0 + kKvTile - 1 - it.q_off > sg.mask_offset);
    // One 32-key block at a time: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t S[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8_t ka = to.rowop(Kt, kb * 32, kc);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) S[cb] = mfma32(ka, qb[cb][kc], S[cb]);
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
        mx = fmaxf(mx, wave_xor32(mx)) * c;
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

    wait_vmem();
    __syncthreads();
    buf ^= 1;
    s = ns;
    t = ntile;
    nt = nnt;
    sg = nsg;
    have = next;
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) ln 2; no visible key -> O = 0, LSE = -inf.
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = l[cb] + wave_xor32(l[cb]);
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
