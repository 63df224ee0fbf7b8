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
//    straight from registers and K^T through LDS transpose reads of the K tile.
//  * dK/dV, KV-stationary: a work item is up to 256 keys of one elementary KV interval
//    (keys covered by the same set of pairs) for one KV head; it streams every 64-row Q
//    tile of those pairs and every query head of the group. Scores are computed with
//    keys as columns (S = Q K^T, dP = dO V^T), so P and dS feed dV^T = dO^T P and
//    dK^T = Q^T dS from registers, with dO^T and Q^T read by LDS transpose reads of the
//    row-major Q and dO tiles. K^T is register-resident; the item's V block stays in LDS.
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

__device__ __forceinline__ int seg_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / kKvTile + 1;
}

template <int D, int CB>
__global__ __launch_bounds__(64 * kColBlocksPerWG / CB)
__attribute__((amdgpu_waves_per_eu(CB == 1 ? 2 : 1, CB == 1 ? 2 : 1)))
void dq_kernel(BwdArgs a) {
  constexpr int NW = kColBlocksPerWG / CB;  // waves per workgroup
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[2][kKvTile * D];
  __shared__ __attribute__((aligned(16))) u16 sV[2][kKvTile * D];

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
  const TileOffsets<D> to(lane);

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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t S[CB], dP[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = dP[cb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8_t ka = to.rowop(Kt, kb * 32, kc);
        const bf16x8_t va = to.rowop(Vt, kb * 32, kc);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          S[cb] = mfma32(ka, qb[cb][kc], S[cb]);
          dP[cb] = mfma32(va, gb[cb][kc], dP[cb]);
        }
      }
      bf16x8_t dsb[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int lim_c = sg.mask_offset + it.q_off + tok[cb] - j0 - kb * 32;
        const int lim_r = sg.kv_len - j0 - kb * 32 - 1;
        const int lim = causal ? min(lim_r, lim_c) : lim_r;
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(S[cb][r], c, -lse2[cb]));
          if (need_mask && 8 * (r >> 2) + 4 * hi + (r & 3) > lim) p = 0.f;
          ds[r] = p * (dP[cb][r] - dlt[cb]);
        }
        dsb[cb][0] = to_bf16x8(ds);
        dsb[cb][1] = to_bf16x8(ds + 8);
      }
      // dQ^T += K^T dS^T (contraction over the block's 32 keys).
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8_t kt = to.trA(Kt, kb * 32 + 16 * half, db * 32);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][db] = mfma32(kt, dsb[cb][half], acc[cb][db]);
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
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] += a.scale * acc[cb][db][4 * g4 + e];
        *reinterpret_cast<f32x4_t*>(dst + d) = cur;
      }
  }
}

// ---------------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------------

constexpr int kQRows = kQTileBwd;  // query rows per streamed tile (two 32-row blocks)
constexpr int kDkdvWaves = kKvTileBwd / 32;

// First query of segment `s` that sees any key of the item (causal), else 0.
__device__ __forceinline__ int first_query(const QSeg& s, int key_off) {
  return (s.flags & 1) ? max(0, key_off - s.mask_offset) : 0;
}

// 8 waves (two per SIMD), each owning 32 keys as MFMA columns. K^T stays in registers;
// the item's V block stays in LDS for the whole item and feeds dP = dO V^T.
template <int D>
__global__ __launch_bounds__(64 * kDkdvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_kernel(BwdArgs a) {
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NW = kDkdvWaves;
  __shared__ __attribute__((aligned(16))) u16 sV[kKvTileBwd * D];
  __shared__ __attribute__((aligned(16))) u16 sQ[2][kQRows * D];
  __shared__ __attribute__((aligned(16))) u16 sG[2][kQRows * D];
  __shared__ __attribute__((aligned(16))) float sL[2][kQRows];
  __shared__ __attribute__((aligned(16))) float sD[2][kQRows];

  const int item_idx = blockIdx.x / a.hkv;
  const int kvh = blockIdx.x - item_idx * a.hkv;
  const KvItem it = a.kvitems[item_idx];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const int64_t q_stride = (int64_t)a.hq * D;
  const float c = a.scale_log2;

  const TileOffsets<D> to(lane);
  // This lane's key column; K^T as B operand (k-slots d = 16*kc + 8*hi + 0..7).
  const int key = wave * 32 + l32;  // within the item
  const bool kvalid = key < it.kv_rows;
  const int jkey = it.key_off + key;  // within the interval
  bf16x8_t kb[NKC];
  {
    const int64_t off = (int64_t)(it.kv_row0 + key) * kv_stride + (int64_t)kvh * D;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      kb[kc] = kvalid ? *reinterpret_cast<const bf16x8_t*>(a.k + off + 16 * kc + 8 * hi)
                      : zero_bf16x8();
  }
  tile_copy_async<D, kKvTileBwd, NW>(a.v, it.kv_row0, it.kv_rows, kv_stride, (int64_t)kvh * D,
                                     sV, wave, lane);
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero16();

  // Iteration space: segments x 64-row Q tiles (from each segment's first visible
  // query) x query heads of the group.
  const int seg_end = it.seg_begin + it.seg_count;
  const int G = a.group;
  const int h_first = it.heads & 0xffff, h_end = h_first + (it.heads >> 16);
  int s = it.seg_begin, i0 = 0, h = h_first;
  QSeg sg{};
  for (; s < seg_end; ++s) {
    sg = a.qsegs[s];
    i0 = first_query(sg, it.key_off);
    if (i0 < sg.q_len) break;
  }
  bool have = s < seg_end;
  float stat = 0.f;  // tid < 64: LSE (base 2) of row tid; 64 <= tid < 128: Delta
  auto load_tile = [&](const QSeg& q, int r0, int head, int b) {
    const int64_t col = (int64_t)head * D;
    tile_copy_async<D, kQRows, NW>(a.q, (int64_t)q.q_start + r0, q.q_len - r0, q_stride, col,
                                   sQ[b], wave, lane);
    tile_copy_async<D, kQRows, NW>(a.dout, (int64_t)q.q_start + r0, q.q_len - r0, q_stride, col,
                                   sG[b], wave, lane);
    if (tid < 2 * kQRows) {
      const int r = tid & (kQRows - 1);
      const bool ok = r0 + r < q.q_len;
      const int64_t row = (int64_t)q.q_start + r0 + r;
      if (tid < kQRows) {
        const float L = ok ? a.lse[row * a.hq + head] : -INFINITY;
        stat = L == -INFINITY ? INFINITY : L * kLog2e;
      } else {
        stat = ok ? a.delta[row * a.hq + head] : 0.f;
      }
    }
  };
  auto store_stats = [&](int b) {
    if (tid < kQRows)
      sL[b][tid] = stat;
    else if (tid < 2 * kQRows)
      sD[b][tid - kQRows] = stat;
  };
  if (have) {
    load_tile(sg, i0, kvh * G + h_first, 0);
    store_stats(0);
  }
  wait_vmem();
  __syncthreads();
  int buf = 0;

  while (have) {
    int ns = s, ni0 = i0, nh = h + 1;
    QSeg nsg = sg;
    if (nh == h_end) {
      nh = h_first;
      ni0 = i0 + kQRows;
      if (ni0 >= sg.q_len) {
        for (++ns; ns < seg_end; ++ns) {
          nsg = a.qsegs[ns];
          ni0 = first_query(nsg, it.key_off);
          if (ni0 < nsg.q_len) break;
        }
      }
    }
    const bool next = ns < seg_end;
    if (next) load_tile(nsg, ni0, kvh * G + nh, buf ^ 1);

    const u16* Qt = sQ[buf];
    const u16* Gt = sG[buf];
    const bool causal = sg.flags & 1;
    // Causal: query i (within the segment) sees this lane's key iff i >= jkey - offset.
    const int thr = jkey - sg.mask_offset - i0;  // tile row index threshold
    const bool need_mask = causal && (it.key_off + kKvTileBwd - 1 - sg.mask_offset > i0);
#pragma unroll 1
    for (int rb = 0; rb < 2; ++rb) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      f32x16_t S = zero16(), dP = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        S = mfma32(to.rowop(Qt, rb * 32, kc), kb[kc], S);
        dP = mfma32(to.rowop(Gt, rb * 32, kc), to.rowop(sV, wave * 32, kc), dP);
      }
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = rb * 32 + 8 * g + 4 * hi;
        const f32x4_t L4 = *reinterpret_cast<const f32x4_t*>(&sL[buf][r0]);
        const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(&sD[buf][r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(S[r], c, -L4[e]));
          if (need_mask && r0 + e < thr) pr = 0.f;
          p[r] = pr;
          ds[r] = pr * (dP[r] - D4[e]);
        }
      }
      const bf16x8_t pb0 = to_bf16x8(p), pb1 = to_bf16x8(p + 8);
      const bf16x8_t sb0 = to_bf16x8(ds), sb1 = to_bf16x8(ds + 8);
      // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 queries.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = mfma32(to.trA(Gt, rb * 32, db * 32), pb0, dv[db]);
        dv[db] = mfma32(to.trA(Gt, rb * 32 + 16, db * 32), pb1, dv[db]);
        dk[db] = mfma32(to.trA(Qt, rb * 32, db * 32), sb0, dk[db]);
        dk[db] = mfma32(to.trA(Qt, rb * 32 + 16, db * 32), sb1, dk[db]);
      }
    }

    if (next) store_stats(buf ^ 1);
    wait_vmem();
    __syncthreads();
    buf ^= 1;
    s = ns;
    i0 = ni0;
    h = nh;
    sg = nsg;
    have = next;
  }

  if (!kvalid) return;
  if (it.slot < 0) {
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
  } else {
    // Part of a split item: write this part's (scaled) sums to its slot.
    const int64_t base = (((int64_t)it.slot * a.hkv + kvh) * kKvTileBwd + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        f32x4_t ck, cv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ck[e] = a.scale * dk[db][4 * g4 + e];
          cv[e] = dv[db][4 * g4 + e];
        }
        *reinterpret_cast<f32x4_t*>(a.part_dk + base + d) = ck;
        *reinterpret_cast<f32x4_t*>(a.part_dv + base + d) = cv;
      }
  }
}

// Adds the partial slots of each split dK/dV item into dk/dv, slots in increasing order
// (deterministic). One workgroup per (item, KV head); HBM-bound.
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(BwdArgs a) {
  const int ridx = blockIdx.x / a.hkv;
  const int kvh = blockIdx.x - ridx * a.hkv;
  const ReduceItem r = a.reduce[ridx];
  constexpr int V4 = D / 4;
  const int total = r.kv_rows * V4;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int key = e / V4, d4 = e - key * V4;
    f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < r.n_slots; ++p) {
      const int64_t src = (((int64_t)(r.slot_begin + p) * a.hkv + kvh) * kKvTileBwd + key) * V4 + d4;
      sk += reinterpret_cast<const f32x4_t*>(a.part_dk)[src];
      sv += reinterpret_cast<const f32x4_t*>(a.part_dv)[src];
    }
    const int64_t dst = ((int64_t)(r.kv_row0 + key) * a.hkv + kvh) * V4 + d4;
    reinterpret_cast<f32x4_t*>(a.dk)[dst] += sk;
    reinterpret_cast<f32x4_t*>(a.dv)[dst] += sv;
  }
}

}  // namespace

// Column blocks per wave of the launched dQ kernel (see the forward's kFwdCB).
constexpr int kDqCB = 1;

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_qitems == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_qitems * (unsigned)a.n_hgroups), block(64 * kColBlocksPerWG / kDqCB);
  if (head_dim == 128)
    hipLaunchKernelGGL((dq_kernel<128, kDqCB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dq_kernel<64, kDqCB>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_kvitems == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_kvitems * (unsigned)a.hkv), block(64 * kDkdvWaves);
  if (head_dim == 128)
    hipLaunchKernelGGL((dkdv_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dkdv_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_reduce == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_reduce * (unsigned)a.hkv), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL((dkdv_reduce_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dkdv_reduce_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace fcp
