// Forward block attention on gfx950: bf16 MFMA for QK^T and PV, fp32 online softmax.
//
// Computes, for a tile of query rows of one Q range and a group of query heads sharing
// one KV head, softmax(Q K^T * scale, masked) V over the KV ranges of its pairs (FCP
// paper Sec. 2.2, attention over [H, L, D] with causal or non-causal masks; the formula
// is legible on the paper's review page, section "核心公式与建模"). With one KV range
// per item it writes that pair's normalised partial and its LSE (the per-slice result
// of Sec. 2.2); with all KV ranges of a Q range it writes the final output directly.
//
// Design (one workgroup = 4 waves = 256 query columns):
//  * The scores are computed transposed, S^T = K Q^T, so each lane owns one (token,
//    head) column: the row max / row sum of the online softmax are in-lane reductions
//    plus one exchange between lane l and l + 32, and rescaling the accumulator is a
//    per-lane multiply.
//  * Q^T stays in registers for the whole item (B operand). A workgroup covers the
//    query heads of one KV head (grouped-query attention, Sec. 2.2 and Sec. 6.1), so each
//    K/V tile staged in LDS is reused by all of them.
//  * O^T = V^T P^T: P comes straight from the S^T registers as the B operand; V is
//    written to LDS transposed, with keys ordered to match the S^T result layout.
//  * K/V tiles of 64 keys are double-buffered: global loads for tile n+1 are issued
//    before the MFMAs of tile n and written to the other LDS buffer afterwards.
#include "fcp_common.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

template <int D>
struct KvTileLoader {
  static constexpr int CPK = D / 8;                   // 16-byte chunks per key row
  static constexpr int KPT = kKvTile * CPK / 256;     // keys per thread (4 or 2)
  static constexpr int KLD = D + 8;                   // K tile row stride (elements)
  static constexpr int VLD = kKvTile + 8;             // V^T tile row stride (elements)
  u32x4_t rk[KPT], rv[KPT];
  int kg, dc;

  __device__ void init(int tid) {
    kg = tid / CPK;
    dc = tid % CPK;
  }

  __device__ void load(const u16* __restrict__ k, const u16* __restrict__ v, int64_t row_stride,
                       int kvh, const KvSeg& s, int t) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = t * kKvTile + kg * KPT + e;
      if (j < s.kv_len) {
        const int64_t off = (int64_t)(s.kv_start + j) * row_stride + (int64_t)kvh * D + dc * 8;
        rk[e] = *reinterpret_cast<const u32x4_t*>(k + off);
        rv[e] = *reinterpret_cast<const u32x4_t*>(v + off);
      } else {
        rk[e] = u32x4_t{0u, 0u, 0u, 0u};
        rv[e] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ void store(u16* sK, u16* sV) const {
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      *reinterpret_cast<u32x4_t*>(&sK[(kg * KPT + e) * KLD + dc * 8]) = rk[e];
    const int p = tpos(kg * KPT);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u16* lo = &sV[(dc * 8 + 2 * w) * VLD + p];
      u16* hi = &sV[(dc * 8 + 2 * w + 1) * VLD + p];
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2_t*>(lo) =
            u32x2_t{pack_lo(rv[0][w], rv[1][w]), pack_lo(rv[2][w], rv[3][w])};
        *reinterpret_cast<u32x2_t*>(hi) =
            u32x2_t{pack_hi(rv[0][w], rv[1][w]), pack_hi(rv[2][w], rv[3][w])};
      } else {
        *reinterpret_cast<uint32_t*>(lo) = pack_lo(rv[0][w], rv[1][w]);
        *reinterpret_cast<uint32_t*>(hi) = pack_hi(rv[0][w], rv[1][w]);
      }
    }
  }
};

// Number of 64-key tiles of segment `s` visible to queries [q_off, q_off + rows).
__device__ __forceinline__ int seg_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / kKvTile + 1;
}

template <int D, bool FINAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_kernel(FwdArgs a) {
  constexpr int CB = 2;         // column blocks per wave
  constexpr int NKC = D / 16;   // k-chunks of the QK^T contraction
  constexpr int NDB = D / 32;   // d-blocks of the output
  using Loader = KvTileLoader<D>;
  constexpr int KLD = Loader::KLD, VLD = Loader::VLD;
  __shared__ __attribute__((aligned(16))) u16 sK[2][kKvTile * KLD];
  __shared__ __attribute__((aligned(16))) u16 sV[2][D * VLD];

  const int item_idx = blockIdx.x / a.n_hgroups;
  const int hg = blockIdx.x - item_idx * a.n_hgroups;
  const QItem it = a.items[item_idx];
  const int head_base = hg * a.hpw;
  const int kvh = head_base / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q_stride = (int64_t)a.hq * D;
  const int64_t kv_stride = (int64_t)a.hkv * D;

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
  // First (segment, tile) with visible keys.
  for (; s < seg_end; ++s) {
    sg = a.segs[s];
    nt = seg_tiles(sg, it.q_off, it.q_rows);
    if (nt > 0) break;
  }
  bool have = s < seg_end;
  Loader ld;
  ld.init(tid);
  if (have) {
    ld.load(a.k, a.v, kv_stride, kvh, sg, 0);
    ld.store(sK[0], sV[0]);
  }
  __syncthreads();
  int buf = 0;
  const float c = a.scale_log2;

  while (have) {
    // Next tile position.
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
    if (next) ld.load(a.k, a.v, kv_stride, kvh, nsg, ntile);

    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    // S^T = K Q^T for two 32-key blocks.
    f32x16_t S[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) S[cb][0] = S[cb][1] = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8_t k0 =
          *reinterpret_cast<const bf16x8_t*>(&Kt[l32 * KLD + 16 * kc + 8 * hi]);
      const bf16x8_t k1 =
          *reinterpret_cast<const bf16x8_t*>(&Kt[(32 + l32) * KLD + 16 * kc + 8 * hi]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        S[cb][0] = mfma32(k0, qb[cb][kc], S[cb][0]);
        S[cb][1] = mfma32(k1, qb[cb][kc], S[cb][1]);
      }
    }

    // Mask: key j (within the KV range) visible to query i iff j < kv_len and, causal,
    // j - i <= mask_offset.
    const int j0 = t * kKvTile;
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kKvTile > sg.kv_len) ||
                           (causal && j0 + kKvTile - 1 - it.q_off > sg.mask_offset);
    if (need_mask) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int i = it.q_off + tok[cb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool vis = j < sg.kv_len && (!causal || j - i <= sg.mask_offset);
            if (!vis) S[cb][kb][r] = -INFINITY;
          }
      }
    }

    // Online softmax (base 2, scale folded into the exponent).
    bf16x8_t pb[CB][2][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[cb][kb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m[cb], mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[cb] - m_use);
      m[cb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(S[cb][kb][r], c, -m_use));
          rs += p[r];
        }
        pb[cb][kb][0] = to_bf16x8(p);
        pb[cb][kb][1] = to_bf16x8(p + 8);
      }
      l[cb] = l[cb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][db][r] *= alpha;
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(
              &Vt[(db * 32 + l32) * VLD + kb * 32 + 16 * half + 8 * hi]);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][db] = mfma32(va, pb[cb][kb][half], acc[cb][db]);
        }

    if (next) ld.store(sK[buf ^ 1], sV[buf ^ 1]);
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

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool final_out, hipStream_t stream) {
  if (a.n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_items * (unsigned)a.n_hgroups), block(256);
  if (head_dim == 128) {
    if (final_out)
      hipLaunchKernelGGL((fwd_kernel<128, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (final_out)
      hipLaunchKernelGGL((fwd_kernel<64, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fcp
