// Backward block attention on gfx950 (dQ; dK and dV), bf16 MFMA with fp32 accumulation.
//
// The FCP paper states that both passes are implemented but describes only the forward
// (Sec. 2.2); the gradient computed here is the exact one of the forward. With the
// merged LSE and Delta_i = sum_d dO_i O_i:
//   P_ij  = exp(S_ij * scale - LSE_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - Delta_i)
//   dQ_i += scale sum_j dS_ij k_j,  dK_j += scale sum_i dS_ij q_i,  dV_j += sum_i P_ij dO_i
// Every pair's contribution uses the final LSE, so contributions of different pairs add.
//
// Two kernels, so that each output has exactly one writer and no atomics are needed:
//  * dQ, Q-stationary: a work item is a tile of rows of one Q range (all pairs of that
//    range), like the fused forward. Scores are computed transposed (S^T = K Q^T,
//    dP^T = V dO^T) so each lane owns a (token, head) column; dQ^T = K^T dS^T takes dS^T
//    straight from registers and K^T from a transposed LDS copy.
//  * dK/dV, KV-stationary: a work item is up to 128 keys of one elementary KV interval
//    (keys covered by the same set of pairs) for one KV head; it streams every Q tile of
//    those pairs and every query head of the group. Scores are computed with keys as
//    columns (S = Q K^T, dP = dO V^T), so P and dS feed dV^T = dO^T P and
//    dK^T = Q^T dS from registers, with dO^T and Q^T read from transposed LDS copies.
// Recomputing S and dP in both kernels costs 4 of the 14 contractions per score; the
// counted work stays the 5 of the method.
#include "fcp_common.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

// ---------------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------------

template <int D>
struct DqTileLoader {
  static constexpr int CPK = D / 8;
  static constexpr int KPT = kKvTile * CPK / 256;  // keys per thread (4 or 2)
  static constexpr int RLD = D + 8;                // row-major tile stride
  static constexpr int TLD = kKvTile + 8;          // transposed tile stride
  u32x4_t rk[KPT], rv[KPT];
  int kg, dc;

  __device__ void init(int tid) {
    kg = tid / CPK;
    dc = tid % CPK;
  }
  __device__ void load(const u16* __restrict__ k, const u16* __restrict__ v, int64_t stride,
                       int kvh, const KvSeg& s, int t) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = t * kKvTile + kg * KPT + e;
      if (j < s.kv_len) {
        const int64_t off = (int64_t)(s.kv_start + j) * stride + (int64_t)kvh * D + dc * 8;
        rk[e] = *reinterpret_cast<const u32x4_t*>(k + off);
        rv[e] = *reinterpret_cast<const u32x4_t*>(v + off);
      } else {
        rk[e] = u32x4_t{0u, 0u, 0u, 0u};
        rv[e] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  // K row-major, K transposed (keys permuted), V row-major.
  __device__ void store(u16* sK, u16* sKt, u16* sV) const {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      *reinterpret_cast<u32x4_t*>(&sK[(kg * KPT + e) * RLD + dc * 8]) = rk[e];
      *reinterpret_cast<u32x4_t*>(&sV[(kg * KPT + e) * RLD + dc * 8]) = rv[e];
    }
    const int p = tpos(kg * KPT);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u16* lo = &sKt[(dc * 8 + 2 * w) * TLD + p];
      u16* hi = &sKt[(dc * 8 + 2 * w + 1) * TLD + p];
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2_t*>(lo) =
            u32x2_t{pack_lo(rk[0][w], rk[1][w]), pack_lo(rk[2][w], rk[3][w])};
        *reinterpret_cast<u32x2_t*>(hi) =
            u32x2_t{pack_hi(rk[0][w], rk[1][w]), pack_hi(rk[2][w], rk[3][w])};
      } else {
        *reinterpret_cast<uint32_t*>(lo) = pack_lo(rk[0][w], rk[1][w]);
        *reinterpret_cast<uint32_t*>(hi) = pack_hi(rk[0][w], rk[1][w]);
      }
    }
  }
};

__device__ __forceinline__ int seg_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / kKvTile + 1;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dq_kernel(BwdArgs a) {
  constexpr int CB = 2;
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  using Loader = DqTileLoader<D>;
  constexpr int RLD = Loader::RLD, TLD = Loader::TLD;
  __shared__ __attribute__((aligned(16))) u16 sK[2][kKvTile * RLD];
  __shared__ __attribute__((aligned(16))) u16 sV[2][kKvTile * RLD];
  __shared__ __attribute__((aligned(16))) u16 sKt[2][D * TLD];

  const int item_idx = blockIdx.x / a.n_hgroups;
  const int hg = blockIdx.x - item_idx * a.n_hgroups;
  const QItem it = a.qitems[item_idx];
  const int head_base = hg * a.hpw;
  const int kvh = head_base / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q_stride = (int64_t)a.hq * D;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const float c = a.scale_log2;

  int tok[CB], head[CB];
  bool valid[CB];
  float lse2[CB], dlt[CB];
  bf16x8_t qb[CB][NKC], gb[CB][NKC];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int cbg = wave * CB + cb;
    tok[cb] = (cbg / a.hpw) * kColBlock + l32;
    head[cb] = head_base + cbg % a.hpw;
    valid[cb] = tok[cb] < it.q_rows;
    const int64_t row = it.q_row0 + tok[cb];
    const u16* qrow = a.q + row * q_stride + (int64_t)head[cb] * D;
    const u16* grow = a.dout + row * q_stride + (int64_t)head[cb] * D;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      qb[cb][kc] = valid[cb] ? *reinterpret_cast<const bf16x8_t*>(qrow + 16 * kc + 8 * hi)
                             : zero_bf16x8();
      gb[cb][kc] = valid[cb] ? *reinterpret_cast<const bf16x8_t*>(grow + 16 * kc + 8 * hi)
                             : zero_bf16x8();
    }
    // Rows with LSE = -inf (or padding rows) get P = 0 through an infinite shift.
    const float L = valid[cb] ? a.lse[row * a.hq + head[cb]] : -INFINITY;
    lse2[cb] = L == -INFINITY ? INFINITY : L * kLog2e;
    dlt[cb] = valid[cb] ? a.delta[row * a.hq + head[cb]] : 0.f;
  }

  f32x16_t acc[CB][NDB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[cb][db] = zero16();

  const int seg_end = it.seg_begin + it.seg_count;
  int s = it.seg_begin, t = 0, nt = 0;
  KvSeg sg{};
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
    ld.store(sK[0], sKt[0], sV[0]);
  }
  __syncthreads();
  int buf = 0;

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
    if (next) ld.load(a.k, a.v, kv_stride, kvh, nsg, ntile);

    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    const u16* KTt = sKt[buf];
    const int j0 = t * kKvTile;
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kKvTile > sg.kv_len) ||
                           (causal && j0 + kKvTile - 1 - it.q_off > sg.mask_offset);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t S[CB], dP[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = dP[cb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t*>(&Kt[(kb * 32 + l32) * RLD + 16 * kc + 8 * hi]);
        const bf16x8_t va =
            *reinterpret_cast<const bf16x8_t*>(&Vt[(kb * 32 + l32) * RLD + 16 * kc + 8 * hi]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          S[cb] = mfma32(ka, qb[cb][kc], S[cb]);
          dP[cb] = mfma32(va, gb[cb][kc], dP[cb]);
        }
      }
      bf16x8_t dsb[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int i = it.q_off + tok[cb];
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(S[cb][r], c, -lse2[cb]));
          if (need_mask) {
            const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (!(j < sg.kv_len && (!causal || j - i <= sg.mask_offset))) p = 0.f;
          }
          ds[r] = p * (dP[cb][r] - dlt[cb]);
        }
        dsb[cb][0] = to_bf16x8(ds);
        dsb[cb][1] = to_bf16x8(ds + 8);
      }
      // dQ^T += K^T dS^T.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8_t kt = *reinterpret_cast<const bf16x8_t*>(
              &KTt[(db * 32 + l32) * TLD + kb * 32 + 16 * half + 8 * hi]);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][db] = mfma32(kt, dsb[cb][half], acc[cb][db]);
        }
    }

    if (next) ld.store(sK[buf ^ 1], sKt[buf ^ 1], sV[buf ^ 1]);
    __syncthreads();
    buf ^= 1;
    s = ns;
    t = ntile;
    nt = nnt;
    sg = nsg;
    have = next;
  }

#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (!valid[cb]) continue;
    const int64_t row = it.q_row0 + tok[cb];
    float* dst = a.dq + (row * a.hq + head[cb]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        f32x4_t cur = *reinterpret_cast<f32x4_t*>(dst + d);
        cur[0] += a.scale * acc[cb][db][4 * g4 + 0];
        cur[1] += a.scale * acc[cb][db][4 * g4 + 1];
        cur[2] += a.scale * acc[cb][db][4 * g4 + 2];
        cur[3] += a.scale * acc[cb][db][4 * g4 + 3];
        *reinterpret_cast<f32x4_t*>(dst + d) = cur;
      }
  }
}

// ---------------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------------

// Loads one Q tile (32 rows x D) and its dO tile for one query head, storing each both
// row-major and transposed (rows permuted), plus the tile's LSE (base 2) and Delta.
template <int D>
struct QTileLoader {
  static constexpr int CPK = D / 8;
  static constexpr int COMBOS = (kQTileBwd / 4) * CPK;  // (4-row group, d chunk) per tensor
  static constexpr int RLD = D + 8;
  static constexpr int TLD = kQTileBwd + 8;
  u32x4_t r[4];
  float lse2, dlt;
  int which;  // 0: q, 1: dout, -1: idle
  int rg, dc;

  __device__ void init(int tid) {
    which = tid < COMBOS ? 0 : (tid < 2 * COMBOS ? 1 : -1);
    const int c = which < 0 ? 0 : tid - which * COMBOS;
    rg = c / CPK;
    dc = c % CPK;
  }
  __device__ void load(const BwdArgs& a, const QSeg& s, int i0, int head, int tid) {
    if (which >= 0) {
      const u16* src = which == 0 ? a.q : a.dout;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + rg * 4 + e;
        if (i < s.q_len) {
          const int64_t off = ((int64_t)(s.q_start + i) * a.hq + head) * D + dc * 8;
          r[e] = *reinterpret_cast<const u32x4_t*>(src + off);
        } else {
          r[e] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    if (tid >= 256 - kQTileBwd) {
      const int i = i0 + tid - (256 - kQTileBwd);
      if (i < s.q_len) {
        const int64_t row = s.q_start + i;
        const float L = a.lse[row * a.hq + head];
        lse2 = L == -INFINITY ? INFINITY : L * kLog2e;
        dlt = a.delta[row * a.hq + head];
      } else {
        lse2 = INFINITY;
        dlt = 0.f;
      }
    }
  }
  __device__ void store(u16* sQ, u16* sG, u16* sQt, u16* sGt, float* sL, float* sD,
                        int tid) const {
    if (which >= 0) {
      u16* rowm = which == 0 ? sQ : sG;
      u16* tr = which == 0 ? sQt : sGt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x4_t*>(&rowm[(rg * 4 + e) * RLD + dc * 8]) = r[e];
      const int p = tpos(rg * 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<u32x2_t*>(&tr[(dc * 8 + 2 * w) * TLD + p]) =
            u32x2_t{pack_lo(r[0][w], r[1][w]), pack_lo(r[2][w], r[3][w])};
        *reinterpret_cast<u32x2_t*>(&tr[(dc * 8 + 2 * w + 1) * TLD + p]) =
            u32x2_t{pack_hi(r[0][w], r[1][w]), pack_hi(r[2][w], r[3][w])};
      }
    }
    if (tid >= 256 - kQTileBwd) {
      sL[tid - (256 - kQTileBwd)] = lse2;
      sD[tid - (256 - kQTileBwd)] = dlt;
    }
  }
};

// First query of segment `s` that sees any of keys [key_off, key_off + n).
__device__ __forceinline__ int first_query(const QSeg& s, int key_off) {
  return (s.flags & 1) ? max(0, key_off - s.mask_offset) : 0;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(BwdArgs a) {
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  using Loader = QTileLoader<D>;
  constexpr int RLD = Loader::RLD, TLD = Loader::TLD;
  __shared__ __attribute__((aligned(16))) u16 sQ[2][kQTileBwd * RLD];
  __shared__ __attribute__((aligned(16))) u16 sG[2][kQTileBwd * RLD];
  __shared__ __attribute__((aligned(16))) u16 sQt[2][D * TLD];
  __shared__ __attribute__((aligned(16))) u16 sGt[2][D * TLD];
  __shared__ float sL[2][kQTileBwd], sD[2][kQTileBwd];

  const int item_idx = blockIdx.x / a.hkv;
  const int kvh = blockIdx.x - item_idx * a.hkv;
  const KvItem it = a.kvitems[item_idx];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const float c = a.scale_log2;

  // This lane's key column; K^T and V^T as B operands (k-slots d = 16*kc + 8*hi + 0..7).
  const int key = wave * 32 + l32;  // within the item
  const bool kvalid = key < it.kv_rows;
  const int jkey = it.key_off + key;  // within the interval
  bf16x8_t kb[NKC], vb[NKC];
  {
    const int64_t off = (int64_t)(it.kv_row0 + key) * kv_stride + (int64_t)kvh * D;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      kb[kc] = kvalid ? *reinterpret_cast<const bf16x8_t*>(a.k + off + 16 * kc + 8 * hi)
                      : zero_bf16x8();
      vb[kc] = kvalid ? *reinterpret_cast<const bf16x8_t*>(a.v + off + 16 * kc + 8 * hi)
                      : zero_bf16x8();
    }
  }
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero16();

  // Iteration space: segments x Q tiles (from each segment's first visible query) x heads.
  const int seg_end = it.seg_begin + it.seg_count;
  const int G = a.group;
  auto first_tile = [&](int s0, int* s, int* i0, QSeg* sg) {
    for (*s = s0; *s < seg_end; ++*s) {
      *sg = a.qsegs[*s];
      *i0 = first_query(*sg, it.key_off);
      if (*i0 < sg->q_len) return true;
    }
    return false;
  };
  int s, i0, h = 0;
  QSeg sg;
  bool have = first_tile(it.seg_begin, &s, &i0, &sg);
  Loader ld;
  ld.init(tid);
  if (have) {
    ld.load(a, sg, i0, kvh * G, tid);
    ld.store(sQ[0], sG[0], sQt[0], sGt[0], sL[0], sD[0], tid);
  }
  __syncthreads();
  int buf = 0;

  while (have) {
    int ns = s, ni0 = i0, nh = h + 1;
    QSeg nsg = sg;
    bool next = true;
    if (nh == G) {
      nh = 0;
      ni0 = i0 + kQTileBwd;
      if (ni0 >= sg.q_len) next = first_tile(s + 1, &ns, &ni0, &nsg);
    }
    if (next) ld.load(a, nsg, ni0, kvh * G + nh, tid);

    const u16* Qt = sQ[buf];
    const u16* Gt = sG[buf];
    const u16* QTt = sQt[buf];
    const u16* GTt = sGt[buf];
    const float* L2 = sL[buf];
    const float* DL = sD[buf];

    // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
    f32x16_t S = zero16(), dP = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(&Qt[l32 * RLD + 16 * kc + 8 * hi]);
      const bf16x8_t ga = *reinterpret_cast<const bf16x8_t*>(&Gt[l32 * RLD + 16 * kc + 8 * hi]);
      S = mfma32(qa, kb[kc], S);
      dP = mfma32(ga, vb[kc], dP);
    }
    const bool causal = sg.flags & 1;
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 8 * (r >> 2) + 4 * hi + (r & 3);
      float pr = __builtin_amdgcn_exp2f(fmaf(S[r], c, -L2[qi]));
      if (causal && jkey - (i0 + qi) > sg.mask_offset) pr = 0.f;
      p[r] = pr;
      ds[r] = pr * (dP[r] - DL[qi]);
    }
    const bf16x8_t pb0 = to_bf16x8(p), pb1 = to_bf16x8(p + 8);
    const bf16x8_t sb0 = to_bf16x8(ds), sb1 = to_bf16x8(ds + 8);
    // dV^T += dO^T P, dK^T += Q^T dS (contracting over the 32 queries).
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u16* gt = &GTt[(db * 32 + l32) * TLD + 8 * hi];
      const u16* qt = &QTt[(db * 32 + l32) * TLD + 8 * hi];
      dv[db] = mfma32(*reinterpret_cast<const bf16x8_t*>(gt), pb0, dv[db]);
      dv[db] = mfma32(*reinterpret_cast<const bf16x8_t*>(gt + 16), pb1, dv[db]);
      dk[db] = mfma32(*reinterpret_cast<const bf16x8_t*>(qt), sb0, dk[db]);
      dk[db] = mfma32(*reinterpret_cast<const bf16x8_t*>(qt + 16), sb1, dk[db]);
    }

    if (next) ld.store(sQ[buf ^ 1], sG[buf ^ 1], sQt[buf ^ 1], sGt[buf ^ 1], sL[buf ^ 1],
                       sD[buf ^ 1], tid);
    __syncthreads();
    buf ^= 1;
    s = ns;
    i0 = ni0;
    h = nh;
    sg = nsg;
    have = next;
  }

  if (!kvalid) return;
  const int64_t base = ((int64_t)(it.kv_row0 + key) * a.hkv + kvh) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hi;
      f32x4_t ck = *reinterpret_cast<f32x4_t*>(a.dk + base + d);
      f32x4_t cv = *reinterpret_cast<f32x4_t*>(a.dv + base + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ck[e] += a.scale * dk[db][4 * g4 + e];
        cv[e] += dv[db][4 * g4 + e];
      }
      *reinterpret_cast<f32x4_t*>(a.dk + base + d) = ck;
      *reinterpret_cast<f32x4_t*>(a.dv + base + d) = cv;
    }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_qitems == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_qitems * (unsigned)a.n_hgroups), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL((dq_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dq_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_kvitems == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_kvitems * (unsigned)a.hkv), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL((dkdv_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dkdv_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace fcp
