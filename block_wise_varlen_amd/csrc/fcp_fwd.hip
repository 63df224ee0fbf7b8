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
//  * K/V tiles of 128 keys go through a 2-slot LDS ring: the copy of tile n+1 is issued
//    once every wave has left tile n-1's slot, and is waited for before the last 32-key
//    block of tile n (whose QK^T reads tile n+1's first keys).
#include "fcp_common.h"
#include "fcp_cursor.h"
#include "fcp_kernels.h"
#include "fcp_types.h"


namespace fcp {
namespace {

// log2 headroom before the running max is raised.
constexpr float kRescaleSlack = 8.0f;

// Keys per K/V tile of the forward and depth of its LDS ring.
constexpr int kFwdKt = 128;

using TileCursor = KvTileCursor<kFwdKt>;

// Scheduling hints (LLVM AMDGPU sched_group_barrier masks).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

template <int D, bool FINAL, int CB>
__global__ __launch_bounds__(64 * kColBlocksPerWG / CB)
__attribute__((amdgpu_waves_per_eu(CB == 1 ? 2 : 1, CB == 1 ? 2 : 1)))
void fwd_kernel(FwdArgs a) {
  const WgMap wm = load_wg(a.wg, blockIdx.x);
  if (wm.item < 0) return;  // placement padding
  const ClockStamp clock(a.clk);
  constexpr int NW = kColBlocksPerWG / CB;  // waves per workgroup
  constexpr int NKC = D / 16;               // k-chunks of the QK^T contraction
  constexpr int NDB = D / 32;               // d-blocks of the output
  constexpr int NKB = kFwdKt / 32;          // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) u16 sK[2][kFwdKt * D];
  __shared__ __attribute__((aligned(16))) u16 sV[2][kFwdKt * D];

  const int hg = wm.head;
  const QItem it = a.items[wm.item];
  const int head_base = hg * a.hpw;
  const int kvh = head_base / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q_stride = (int64_t)a.hq * D;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const TileOffsets<D> to(lane);

  // Column block cbg = wave * CB + cb covers tokens (cbg / hpw) * 32 + 0..31 of head
  // head_base + cbg % hpw.
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
  const float c = a.scale_log2;
  // Cursors over the flattened (segment, tile) sequence: the tile being computed and the
  // one after it.
  TileCursor cur = TileCursor::first(a.segs, it.seg_begin, seg_end, it.q_off, it.q_rows);
  TileCursor nx = cur.next(a.segs, seg_end, it.q_off, it.q_rows);
  const TileCopy<D, kFwdKt, NW> tcopy(kv_stride, wave, lane);
  auto copy = [&](const TileCursor& tc, int b) {
    const int j0n = tc.t * kFwdKt;
    tcopy(a.k, (int64_t)tc.sg.kv_start + j0n, tc.sg.kv_len - j0n, kv_col, sK[b]);
    tcopy(a.v, (int64_t)tc.sg.kv_start + j0n, tc.sg.kv_len - j0n, kv_col, sV[b]);
  };

  // Software pipeline over 32-key blocks. Step kb runs two regions:
  //   A: the PV MFMAs of block kb - 1 | K operand reads for block kb + 1 | mask + row max
  //      of block kb;
  //   (rare branch: raise the running max, rescale the accumulator)
  //   B: the QK^T MFMAs of block kb + 1 | V^T operand reads for block kb | exp2, row sum
  //      and bf16 conversion of block kb.
  // Each region interleaves the wave's MFMAs with its own VALU work and with LDS reads
  // issued one region ahead of their use. The pipeline runs across tile boundaries; the
  // first pending PV multiplies zeros, the last QK^T (past the final tile) is discarded.
  f32x16_t S[CB];  // scores of the block whose softmax is next
  bf16x8_t pb[CB][2], va[2 * NDB], kop[NKC];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    S[cb] = zero16();
    pb[cb][0] = pb[cb][1] = zero_bf16x8();
  }
#pragma unroll
  for (int i = 0; i < 2 * NDB; ++i) va[i] = zero_bf16x8();

  if (cur.valid) copy(cur, 0);
  if (nx.valid) copy(nx, 1);
  // Everything issued so far (Q^T, both tiles) is complete after a full wait, which also
  // tells the compiler that no load of its own is still pending in the loop.
  wait_vmem();
  __syncthreads();
  if (cur.valid) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8_t kk = to.rowop(sK[0], 0, kc);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = mfma32(kk, qb[cb][kc], S[cb]);
    }
  }
  // Writes this item's rows of one output: O = acc / l, LSE = (m + log2 l) ln 2; no
  // visible key (or `empty`) -> O = 0, LSE = -inf. row0: output row of query tok 0.
  auto store = [&](int64_t row0, bool empty) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float lt = empty ? 0.f : pair_sum(l[cb]);
      if (!valid[cb]) continue;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (m[cb] + __log2f(lt)) * kLn2 : -INFINITY;
      const int64_t row = row0 + tok[cb];
      const int64_t base = (row * a.hq + head[cb]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          const float o0 = empty ? 0.f : acc[cb][db][4 * g4 + 0] * inv;
          const float o1 = empty ? 0.f : acc[cb][db][4 * g4 + 1] * inv;
          const float o2 = empty ? 0.f : acc[cb][db][4 * g4 + 2] * inv;
          const float o3 = empty ? 0.f : acc[cb][db][4 * g4 + 3] * inv;
          if (FINAL || a.o_part16) {
            // bf16 (RNE): the final output, or partials stored in bf16
            const uint32_t w0 = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16(o2) | ((uint32_t)f32_to_bf16(o3) << 16);
            *reinterpret_cast<u32x2_t*>((FINAL ? a.o : a.o_part16) + base + d) = u32x2_t{w0, w1};
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
  };
  // Per-pair partials: each KV segment is one pair with its own partial rows. seg_cur is
  // the segment being accumulated; segments without a visible tile get empty partials.
  auto part_row0 = [&](int sidx) { return (int64_t)load_uniform_i32(a.seg_out, sidx) + it.q_off; };
  int seg_cur = cur.valid ? cur.s : seg_end;
  if constexpr (!FINAL)
    for (int s2 = it.seg_begin; s2 < seg_cur; ++s2) store(part_row0(s2), true);

  int buf = 0;
  bool first_tile = true;
  // A store() issues 4 * NDB 16-byte (8-byte for bf16) stores per column block whose lane 0 holds a valid
  // row (the compiler skips the block only when no lane of the wave is valid), plus the
  // LSE store. kBurstStores counts the O stores of the wave's first column block: the
  // smallest number a store() of this wave issues, or 0 when it issues none.
  constexpr int kBurstStores = 4 * NDB;
  const bool wave_stores = (wave * CB / a.hpw) * kColBlock < it.q_rows;

  while (cur.valid) {
    // Tile n + 1 goes into the slot of tile n - 1, whose last reads (the V^T operands of
    // its final block) every wave has completed before this barrier.
    if (!first_tile && nx.valid) {
      lds_barrier();
      copy(nx, buf ^ 1);
    }
    const KvSeg sg = cur.sg;
    // Per-pair partials: this tile starts a new pair, whose predecessor is complete once
    // the first block's pending PV (the predecessor's last block) has been added.
    const bool boundary = !FINAL && cur.s != seg_cur;
    // The partial stores of a boundary come after this tile's copy of the next tile.
    const bool burst_after_copy = boundary && !first_tile && wave_stores;
    const int j0 = cur.t * kFwdKt;
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kFwdKt > sg.kv_len) ||
                           (causal && j0 + kFwdKt - 1 - it.q_off > sg.mask_offset);
    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    const u16* Kn = sK[buf ^ 1];

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb == NKB - 1 && nx.valid) {
        // The next tile's K is read from here on. Vector-memory operations retire in issue
        // order, so when this wave stored a finished partial after issuing that tile's
        // copy, waiting until only those stores are outstanding suffices: the partial
        // drains to memory while the next tile is computed.
        if (burst_after_copy)
          wait_vmem_le<kBurstStores>();
        else
          wait_vmem();
        lds_barrier();
      }
      if (need_mask) {
        // Key j (within the KV range) visible to query i iff j < kv_len and, causal,
        // j - i <= mask_offset. Only tiles on a diagonal or a ragged end take this branch.
        const int jb = j0 + kb * 32;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int lim_c = sg.mask_offset + it.q_off + tok[cb] - jb;
          const int lim = causal ? min(sg.kv_len - jb - 1, lim_c) : sg.kv_len - jb - 1;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + 4 * hi + (r & 3) > lim) S[cb][r] = -INFINITY;
        }
      }
      // ---- region A
      // Wave priority high in region A (MFMA-dense: PV, operand reads, row max) and low
      // in region B (QK^T beside the exp work): of the two waves on a SIMD, the one with
      // PV MFMAs ready issues first and the other's softmax VALU work fills in (-4 to -5%
      // forward time measured; the opposite assignment was no faster).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb][db] = mfma32(va[2 * db + half], pb[cb][half], acc[cb][db]);
      if constexpr (!FINAL) {
        if (kb == 0 && boundary) {
          store(part_row0(seg_cur), false);
          for (int s2 = seg_cur + 1; s2 < cur.s; ++s2) store(part_row0(s2), true);
          seg_cur = cur.s;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            m[cb] = -INFINITY;
            l[cb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[cb][db] = zero16();
          }
        }
      }
      {
        const u16* kt = kb + 1 < NKB ? Kt : Kn;
        const int kr = kb + 1 < NKB ? (kb + 1) * 32 : 0;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kop[kc] = to.rowop(kt, kr, kc);
      }
      bool raise[CB], any_raise = false;
      float mx[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        // Online softmax in base 2 with the scale folded into the exponent; the running
        // max is raised only when the block's max exceeds it by more than kRescaleSlack.
        float x = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, S[cb][r]);
        mx[cb] = pair_max(x) * c;
        raise[cb] = false;
        if (m[cb] == -INFINITY)
          m[cb] = mx[cb];  // nothing accumulated yet: no rescale needed
        else
          raise[cb] = mx[cb] > m[cb] + kRescaleSlack;
        any_raise = any_raise || raise[cb];
      }
#pragma unroll
      for (int i = 0; i < 2 * NDB * CB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (i < NKC) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 3, 0);
      }
      if (__any(any_raise)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const float alpha = raise[cb] ? __builtin_amdgcn_exp2f(m[cb] - mx[cb]) : 1.f;
          m[cb] = raise[cb] ? mx[cb] : m[cb];
          l[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][db][r] *= alpha;
        }
      }
      // ---- region B
      __builtin_amdgcn_s_setprio(0);
      f32x16_t Sn[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) Sn[cb] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) Sn[cb] = mfma32(kop[kc], qb[cb][kc], Sn[cb]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        va[2 * db] = to.trA(Vt, kb * 32, db * 32);
        va[2 * db + 1] = to.trA(Vt, kb * 32 + 16, db * 32);
      }
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
        S[cb] = Sn[cb];
      }
#pragma unroll
      for (int i = 0; i < NKC * CB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (i < 4 * NDB) __builtin_amdgcn_sched_group_barrier(kSgDsRead, (4 * NDB + NKC * CB - 1) / (NKC * CB), 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
      }
    }

    buf ^= 1;
    first_tile = false;
    cur = nx;
    nx = nx.next(a.segs, seg_end, it.q_off, it.q_rows);
  }
  // PV of the last block.
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[cb][db] = mfma32(va[2 * db + half], pb[cb][half], acc[cb][db]);

  if constexpr (FINAL) {
    store(it.out_row0, false);
  } else {
    if (seg_cur < seg_end) store(part_row0(seg_cur), false);
    for (int s2 = seg_cur + 1; s2 < seg_end; ++s2) store(part_row0(s2), true);
  }
  clock.done(a.clk);
}

}  // namespace

// Column blocks per wave of the launched forward: 2 (4 waves, one per SIMD, each K / V
// operand read from LDS feeds two MFMAs) or 1 (8 waves, two per SIMD).
#ifndef FCP_FWD_CB
#define FCP_FWD_CB 1
#endif
constexpr int kFwdCB = FCP_FWD_CB;

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool final_out, hipStream_t stream) {
  if (a.n_wg == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_wg), block(64 * kColBlocksPerWG / kFwdCB);
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
