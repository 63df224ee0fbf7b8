// Backward block attention on gfx950 (dQ; dK and dV), bf16 MFMA with fp32 accumulation.
//
// The FCP paper states that both passes are implemented but describes only the forward
// (Sec. 2.2); the gradient computed here is the exact one of the forward. With the
// merged LSE and Delta_i = sum_d dO_i O_i:
//   P_ij  = exp(S_ij * scale - LSE_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - Delta_i)
//   dQ_i += scale sum_j dS_ij k_j,  dK_j += scale sum_i dS_ij q_i,  dV_j += sum_i P_ij dO_i
// Every pair's contribution uses the final LSE, so contributions of different pairs add.
//
// Two kernels, so that each output has exactly one writer and no atomics are needed
// (the dQ kernel is in fcp_bwd_dq.hip, built with its own scheduling options):
//  * dQ, Q-stationary: a work item is a tile of rows of one Q range (all pairs of that
//    range), like the fused forward. Scores are computed transposed (S^T = K Q^T,
//    dP^T = V dO^T) so each lane owns a (token, head) column; dQ^T = K^T dS^T takes dS^T
//    straight from registers and K^T through LDS transpose reads of the K tile. Every
//    (row, head) belongs to exactly one dQ item, which also computes its Delta and stores
//    it with the LSE as the row statistics the dK/dV kernel reads.
//  * dK/dV, KV-stationary: a work item is up to 128 keys of one elementary KV interval
//    (keys covered by the same set of pairs) for one KV head, or a head subset of it; it
//    streams every 32-row Q tile of those pairs and every query head of the group.
//    Scores are computed with keys as columns (S = Q K^T, dP = dO V^T) by score waves
//    that keep K^T and V^T in registers; gradient waves on the same SIMDs take P and dS
//    through LDS and accumulate dV^T = dO^T P and dK^T = Q^T dS, reading dO^T and Q^T by
//    LDS transpose reads of the row-major Q and dO tiles.
// Recomputing S and dP in both kernels costs 4 of the 14 contractions per score; the
// counted work stays the 5 of the method.
#include "fcp_common.h"
#include "fcp_cursor.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {


// ---------------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------------

constexpr int kDkdvWaves = kKvTileBwd / 32;  // 4 SIMD pairs of waves, 32 keys each
static_assert(kQTileBwd == 32, "one 32-row MFMA block per streamed Q tile");

// First query of segment `s` that sees any key of the item (causal), else 0.
__device__ __forceinline__ int first_query(const QSeg& s, int key_off) {
  return (s.flags & 1) ? max(0, key_off - s.mask_offset) : 0;
}

// Position in the (Q segment, 32-row Q tile, query head) sequence of one dK/dV item,
// walked backwards over segments and tiles (heads innermost, ascending). Causally, every
// KV item of a sequence then starts on the same last Q tile and they stream in step, so
// concurrent workgroups share each Q / dO tile in L2; walking forwards, each would start
// at its own diagonal and re-read Q from HBM.
struct StepCursor {
  QSeg sg;
  int s, i0, lo, h;  // lo: first visible query of segment s
  bool valid;
  // Last tile of the last segment at or before `s_last` with a visible query.
  __device__ static StepCursor last(const QSeg* qsegs, int s_first, int s_last, int key_off,
                                    int h_first) {
    StepCursor c{};
    c.valid = false;
    c.h = h_first;
    for (c.s = s_last; c.s >= s_first; --c.s) {
      c.sg = load_uniform(qsegs, c.s);
      c.lo = first_query(c.sg, key_off);
      if (c.lo < c.sg.q_len) {
        c.i0 = c.lo + (c.sg.q_len - 1 - c.lo) / kQTileBwd * kQTileBwd;
        c.valid = true;
        break;
      }
    }
    return c;
  }
  __device__ StepCursor next(const QSeg* qsegs, int s_first, int key_off, int h_first,
                             int h_end) const {
    if (!valid) return *this;
    StepCursor c = *this;
    if (++c.h < h_end) return c;
    c.h = h_first;
    c.i0 -= kQTileBwd;
    if (c.i0 >= c.lo) return c;
    return last(qsegs, s_first, s - 1, key_off, h_first);
  }
};

// dK/dV with two waves per SIMD, each pair owning 32 keys as MFMA columns. Waves 0..3 (score waves) own the K^T / V^T
// registers of their 32 keys and, per tile, compute S and dP, then P and dS (the VALU
// side), handing P and dS in bf16 to waves 4..7 through LDS. Wave w + 4 runs on wave w's
// SIMD, owns the same 32 keys and accumulates dV^T += dO^T P and dK^T += Q^T dS for the
// tile the score wave finished one region earlier; it also issues the ring loads. The
// matrix pipe of each SIMD thus takes MFMAs from two instruction streams, and one wave's
// exp / convert / LDS waits no longer stall the other's MFMAs. Q / dO tiles and their
// (L2, Delta) rows stream through a ring of kDkdvSplitRing slots; all eight waves meet
// at one barrier per tile. In region t the score waves read tiles t and t + 1, the
// gradient waves tile t - 1, and tiles up to t + NB - 2 are in flight.
constexpr int kDkdvSplitWaves = 2 * kDkdvWaves;
constexpr int kDkdvSplitRing = 6;

template <int D>
__global__ __launch_bounds__(64 * kDkdvSplitWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_split_kernel(BwdArgs a) {
  const WgMap wm = load_wg(a.kvwg, blockIdx.x);
  if (wm.item < 0) return;  // placement padding
  // Thread 0 is a score wave's; it leaves after its last tile, when the gradient waves
  // have only their final accumulation and stores left.
  const ClockStamp clock(a.clk);
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NW = kDkdvWaves;
  constexpr int QR = kQTileBwd;
  constexpr int NB = kDkdvSplitRing;
  constexpr int LOADS = 2 * tile_copy_insts<D, QR, NW>() + 1;  // per tile, per loading wave
  __shared__ __attribute__((aligned(16))) u16 sQ[NB][QR * D];
  __shared__ __attribute__((aligned(16))) u16 sG[NB][QR * D];
  __shared__ __attribute__((aligned(16))) float sSt[NB][NW][256];
  // P (vectors 0, 1) and dS (2, 3) of one tile per SIMD pair, as the B operands of the
  // gradient MFMAs; two slots, written in region t and read in region t + 1.
  __shared__ __attribute__((aligned(16))) bf16x8_t sX[2][NW][4][64];

  const int kvh = wm.head;
  const KvItem it = a.kvitems[wm.item];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pw = wave & (NW - 1);  // SIMD pair: keys pw * 32 .. + 31
  const int l32 = lane & 31, hi = lane >> 5;
  const TileOffsets<D> to(lane);
  const int key = pw * 32 + l32;
  const bool kvalid = key < it.kv_rows;

  const int seg_end = it.seg_begin + it.seg_count;
  const int h_first = it.heads & 0xffff, h_end = h_first + (it.heads >> 16);
  auto advance = [&](const StepCursor& x) {
    return x.next(a.qsegs, it.seg_begin, it.key_off, h_first, h_end);
  };
  const StepCursor first =
      StepCursor::last(a.qsegs, it.seg_begin, seg_end - 1, it.key_off, h_first);
  auto next_slot = [](int b) { return b == NB - 1 ? 0 : b + 1; };

  if (wave < NW) {
    // ---- score waves
    const float c = a.scale_log2;
    const int jkey = it.key_off + key;
    bf16x8_t kb[NKC], vb[NKC];
    {
      const int64_t off =
          (int64_t)(it.kv_row0 + key) * ((int64_t)a.hkv * D) + (int64_t)kvh * D;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kb[kc] = kvalid ? *reinterpret_cast<const bf16x8_t*>(a.k + off + 16 * kc + 8 * hi)
                        : zero_bf16x8();
        vb[kc] = kvalid ? *reinterpret_cast<const bf16x8_t*>(a.v + off + 16 * kc + 8 * hi)
                        : zero_bf16x8();
      }
    }
    wait_vmem();
    __syncthreads();

    StepCursor cur = first;
    f32x16_t S = zero16(), dP = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      S = mfma32(to.rowop(sQ[0], 0, kc), kb[kc], S);
      dP = mfma32(to.rowop(sG[0], 0, kc), vb[kc], dP);
    }
    int buf = 0, x = 0;
    while (cur.valid) {
      const int nbuf = next_slot(buf);
      f32x4_t st[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* sp4 = &sSt[buf][pw][16 * g + 8 * hi];
        st[g][0] = *reinterpret_cast<const f32x4_t*>(sp4);
        st[g][1] = *reinterpret_cast<const f32x4_t*>(sp4 + 4);
      }
      // Causal: query i (within the segment) sees key jkey iff i >= jkey - mask_offset;
      // rows past the range see nothing. Only tiles on the diagonal or a ragged end mask.
      {
        const QSeg sg = cur.sg;
        const bool causal = sg.flags & 1;
        const int rows_left = sg.q_len - cur.i0;
        if ((causal && it.key_off + kKvTileBwd - 1 - sg.mask_offset > cur.i0) || rows_left < QR) {
          const int lo = causal ? jkey - sg.mask_offset - cur.i0 : -QR;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
            if (row < lo || row >= rows_left) S[r] = -INFINITY;
          }
        }
      }
      constexpr int NM = 2 * NKC;
      constexpr int PF = 2;
      const u16* Qn = sQ[nbuf];
      const u16* Gn = sG[nbuf];
      auto next_op = [&](int n) { return to.rowop((n & 1) ? Gn : Qn, 0, n >> 1); };
      // P and dS of tile t first, handed over before the S / dP MFMAs of tile t + 1 (row
      // reads PF MFMAs ahead), which then cover the exchange writes' latency.
      float p[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int g = i >> 2, e = i & 3;
        const float L2 = st[g][e >> 1][2 * (e & 1)];
        const float Dl = st[g][e >> 1][2 * (e & 1) + 1];
        p[i] = __builtin_amdgcn_exp2f(fmaf(S[i], c, -L2));
        ds[i] = p[i] * (dP[i] - Dl);
      }
      sX[x][pw][0][lane] = to_bf16x8(p);
      sX[x][pw][2][lane] = to_bf16x8(ds);
      sX[x][pw][1][lane] = to_bf16x8(p + 8);
      sX[x][pw][3][lane] = to_bf16x8(ds + 8);
      bf16x8_t an[NM];
#pragma unroll
      for (int i = 0; i < PF; ++i) an[i] = next_op(i);
      f32x16_t Sn = zero16(), dPn = zero16();
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i + PF < NM) an[i + PF] = next_op(i + PF);
        if (i & 1)
          dPn = mfma32(an[i], vb[i >> 1], dPn);
        else
          Sn = mfma32(an[i], kb[i >> 1], Sn);
      }
      S = Sn;
      dP = dPn;
      buf = nbuf;
      x ^= 1;
      lds_barrier();
      cur = advance(cur);
    }
    clock.done(a.clk);
    return;
  }

  // ---- gradient waves: ring loads, then dV / dK.
  const int G = a.group;
  const TileCopy<D, QR, NW> tcopy((int64_t)a.hq * D, pw, lane);
  const uint32_t st_off = lane < 16 ? lane * 16 : 0x7fffffffu;  // lanes past 15: no data
  auto load = [&](const StepCursor& y, int b) {
    const int head = kvh * G + y.h;
    const int64_t col = (int64_t)head * D;
    const int64_t r0 = (int64_t)y.sg.q_start + y.i0;
    tcopy(a.q, r0, y.sg.q_len - y.i0, col, sQ[b]);
    tcopy(a.dout, r0, y.sg.q_len - y.i0, col, sG[b]);
    // (L2, Delta) of the tile's 32 rows: 256 contiguous bytes, one 16-byte load per lane
    // for lanes 0..15; rows past the range and lanes past 15 read as zero.
    const uint32_t nbytes = (uint32_t)(min(y.sg.q_len - y.i0, QR) * 8);
    dma16(buffer_rsrc(a.stats + 2 * (head * a.q_rows + r0), nbytes),
          lds_addr(&sSt[b][pw][0]), st_off);
  };
  // Cursors of tiles t .. t + NB - 2 in region t.
  StepCursor cw[NB - 1];
  cw[0] = first;
#pragma unroll
  for (int k = 1; k < NB - 1; ++k) cw[k] = advance(cw[k - 1]);
#pragma unroll
  for (int k = 0; k < NB - 2; ++k)
    if (cw[k].valid) load(cw[k], k);
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero16();
  wait_vmem();
  __syncthreads();
  if (cw[NB - 2].valid) load(cw[NB - 2], NB - 2);

  // dV^T += dO^T P and dK^T += Q^T dS for the tile in ring slot b, with P / dS in
  // exchange slot xs.
  auto accumulate = [&](int b, int xs) {
    const bf16x8_t pp0 = sX[xs][pw][0][lane], pp1 = sX[xs][pw][1][lane];
    const bf16x8_t sp0 = sX[xs][pw][2][lane], sp1 = sX[xs][pw][3][lane];
    // Transpose operands PF MFMAs ahead, the order kept by scheduling barriers (the
    // compiler alone reads one operand ahead).
    constexpr int NM = 4 * NDB;
    constexpr int PF = 3;
    // Operand n: half n / (2 NDB), d block (n / 2) % NDB, dO^T (even) or Q^T (odd).
    auto op = [&](int n) {
      const int half = n / (2 * NDB), db = (n >> 1) % NDB;
      return to.trA((n & 1) ? sQ[b] : sG[b], 16 * half, db * 32);
    };
    bf16x8_t ap[NM];
#pragma unroll
    for (int i = 0; i < PF; ++i) ap[i] = op(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PF < NM) ap[i + PF] = op(i + PF);
      __builtin_amdgcn_sched_barrier(0);
      const int half = i / (2 * NDB), db = (i >> 1) % NDB;
      if (i & 1)
        dk[db] = mfma32(ap[i], half ? sp1 : sp0, dk[db]);
      else
        dv[db] = mfma32(ap[i], half ? pp1 : pp0, dv[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int buf = 0, pbuf = 0, x = 0;
  bool have_prev = false;
  while (cw[0].valid) {
    if (have_prev) accumulate(pbuf, x ^ 1);
    have_prev = true;
    pbuf = buf;
    buf = next_slot(buf);
    x ^= 1;
    // Tile t + 2 must have landed; tiles t + 3 .. t + NB - 2 may stay in flight.
    bool deep = false;
    if constexpr (NB == 6) deep = cw[4].valid;
    if (deep)
      wait_vmem_le<2 * LOADS>();
    else if (cw[3].valid)
      wait_vmem_le<LOADS>();
    else
      wait_vmem();
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NB - 2; ++k) cw[k] = cw[k + 1];
    cw[NB - 2] = advance(cw[NB - 3]);
    // The slot of tile t - 1 (read above) takes tile t + NB - 1.
    if (cw[NB - 2].valid) load(cw[NB - 2], (pbuf + NB - 1) % NB);
  }
  if (have_prev) accumulate(pbuf, x ^ 1);

  if (!kvalid) return;
  if (it.slot < 0 && a.accumulate) {
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
  } else if (it.slot < 0) {
    // Overwrite mode: the item is these rows' only writer.
    const int64_t base = ((int64_t)(it.kv_row0 + key) * a.hkv + kvh) * D;
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

// Adds the partial slots of each split dK/dV item into dk/dv (or, in overwrite mode,
// writes their sum), slots in increasing order (deterministic). One workgroup per
// (item, KV head); HBM-bound.
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
    if (a.accumulate) {
      reinterpret_cast<f32x4_t*>(a.dk)[dst] += sk;
      reinterpret_cast<f32x4_t*>(a.dv)[dst] += sv;
    } else {
      reinterpret_cast<f32x4_t*>(a.dk)[dst] = sk;
      reinterpret_cast<f32x4_t*>(a.dv)[dst] = sv;
    }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_kvwg == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_kvwg), block(64 * kDkdvSplitWaves);
  if (head_dim == 128)
    hipLaunchKernelGGL((dkdv_split_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dkdv_split_kernel<64>), grid, block, 0, stream, a);
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
