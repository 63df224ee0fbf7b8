// Backward block attention on gfx950: the dQ kernel (Q-stationary), bf16 MFMA with fp32
// accumulation. The gradient and the two-kernel split (this kernel and the dK/dV kernel
// in fcp_bwd.hip) are described at the top of fcp_bwd.hip: with the merged LSE and
// Delta_i = sum_d dO_i O_i, P_ij = exp(S_ij * scale - LSE_i), dS_ij = P_ij (dP_ij -
// Delta_i) and dQ_i += scale sum_j dS_ij k_j (the exact gradient of the forward of the FCP
// paper, Sec. 2.2). This file is built with LLVM's max-ilp scheduling strategy, which
// measured 1.6% faster for this kernel (and no faster for the others).
#include "fcp_common.h"
#include "fcp_cursor.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

// ---------------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------------

// K/V tiles of the dQ kernel: 128 keys, two LDS slots. The copy of tile t + 2 goes into
// tile t's slot once every wave has left it (barrier at the end of tile t) and has the
// whole of tile t + 1's compute to land.
constexpr int kDqRing = 2;
constexpr int kDqKt = 128;

template <int D, int CB>
__global__ __launch_bounds__(64 * kColBlocksPerWG / CB)
__attribute__((amdgpu_waves_per_eu(CB == 1 ? 2 : 1, CB == 1 ? 2 : 1)))
void dq_kernel(BwdArgs a) {
  const WgMap wm = load_wg(a.qwg, blockIdx.x);
  if (wm.item < 0) return;  // placement padding
  const ClockStamp clock(a.clk);
  constexpr int NW = kColBlocksPerWG / CB;  // waves per workgroup
  constexpr int NKC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[kDqRing][kDqKt * D];
  __shared__ __attribute__((aligned(16))) u16 sV[kDqRing][kDqKt * D];

  const int hg = wm.head;
  const QItem it = a.qitems[wm.item];
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
    // Delta = dO . O over this lane's half of the head dimension (the same k-slots as its
    // dO^T registers), then over both halves; fp32 from the bf16 tensors.
    const u16* orow = a.o + row * q_stride + (int64_t)head[cb] * D;
    float dl = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8_t ob = valid[cb] ? *reinterpret_cast<const bf16x8_t*>(orow + 16 * kc + 8 * hi)
                                    : zero_bf16x8();
#pragma unroll
      for (int i = 0; i < 8; ++i) dl = fmaf((float)ob[i], (float)gb[cb][kc][i], dl);
    }
    dlt[cb] = pair_sum(dl);
    // LSE in base 2; rows with LSE = -inf (or padding rows) get P = 0 through an infinite
    // shift.
    const float L = valid[cb] ? a.lse[row * a.hq + head[cb]] : -INFINITY;
    lse2[cb] = L == -INFINITY ? INFINITY : L * kLog2e;
  }

  // Row statistics (LSE in base 2, Delta) for the dK/dV kernel, head-major.
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
    if (valid[cb] && hi == 0)
      *reinterpret_cast<f32x2_t*>(a.stats + 2 * (head[cb] * a.q_rows + it.q_row0 + tok[cb])) =
          f32x2_t{lse2[cb], dlt[cb]};

  f32x16_t acc[CB][NDB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[cb][db] = zero16();

  const int seg_end = it.seg_begin + it.seg_count;
  const int64_t kv_col = (int64_t)kvh * D;
  const TileCopy<D, kDqKt, NW> tcopy(kv_stride, wave, lane);
  static_assert(kDqRing == 2, "the loop alternates between two slots");
  using Cursor = KvTileCursor<kDqKt>;
  auto advance = [&](const Cursor& x) { return x.next(a.segs, seg_end, it.q_off, it.q_rows); };
  auto copy = [&](const Cursor& x, int b) {
    tcopy(a.k, (int64_t)x.sg.kv_start + x.j0(), x.sg.kv_len - x.j0(), kv_col, sK[b]);
    tcopy(a.v, (int64_t)x.sg.kv_start + x.j0(), x.sg.kv_len - x.j0(), kv_col, sV[b]);
  };
  // Cursors of the tile being computed and the one after it.
  Cursor cur = Cursor::first(a.segs, it.seg_begin, seg_end, it.q_off, it.q_rows);
  Cursor n1 = advance(cur);
  if (cur.valid) copy(cur, 0);
  if (n1.valid) copy(n1, 1);
  // Full wait: the first tiles and this lane's Q / dO / O registers; it also tells the
  // compiler that none of its own loads is pending in the loop.
  wait_vmem();
  __syncthreads();
  int buf = 0;

  while (cur.valid) {
    const KvSeg sg = cur.sg;
    const u16* Kt = sK[buf];
    const u16* Vt = sV[buf];
    const int j0 = cur.j0();
    const bool causal = sg.flags & 1;
    const bool need_mask = (j0 + kDqKt > sg.kv_len) ||
                           (causal && j0 + kDqKt - 1 - it.q_off > sg.mask_offset);
#pragma unroll
    for (int kb = 0; kb < kDqKt / 32; ++kb) {
      f32x16_t S[CB], dP[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) S[cb] = dP[cb] = zero16();
      // Wave priority: raised while this wave issues its MFMA runs, lowered for its
      // softmax VALU work, so that on a SIMD the wave with MFMAs ready issues them first
      // and the other wave's VALU work fills in beside them (dQ -4% measured).
      __builtin_amdgcn_s_setprio(1);
      // S^T and dP^T: operand rows are read PF MFMAs ahead; the scheduling barriers keep
      // that order (left alone, the compiler reads each operand one MFMA ahead and every
      // MFMA waits for LDS).
      {
        constexpr int NM = 2 * NKC, PF = 4;
        auto op = [&](int i) { return to.rowop((i & 1) ? Vt : Kt, kb * 32, i >> 1); };
        bf16x8_t ops[NM];
#pragma unroll
        for (int i = 0; i < PF; ++i) ops[i] = op(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i + PF < NM) ops[i + PF] = op(i + PF);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            if (i & 1)
              dP[cb] = mfma32(ops[i], gb[cb][i >> 1], dP[cb]);
            else
              S[cb] = mfma32(ops[i], qb[cb][i >> 1], S[cb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
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
      __builtin_amdgcn_s_setprio(1);
      // dQ^T += K^T dS^T (contraction over the block's 32 keys).
      {
        constexpr int NT = 2 * NDB, PT = 2;
        auto top = [&](int i) { return to.trA(Kt, kb * 32 + 16 * (i & 1), (i >> 1) * 32); };
        bf16x8_t kts[NT];
#pragma unroll
        for (int i = 0; i < PT; ++i) kts[i] = top(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i + PT < NT) kts[i + PT] = top(i + PT);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb][i >> 1] = mfma32(kts[i], dsb[cb][i & 1], acc[cb][i >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    // Tile t + 1 (the only copy in flight) must have landed, and every wave must be done
    // with tile t's slot, before tile t + 2 goes there.
    const Cursor n2 = advance(n1);
    if (n1.valid) wait_vmem();
    lds_barrier();
    if (n2.valid) copy(n2, buf);
    buf ^= 1;
    cur = n1;
    n1 = n2;
  }

#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (!valid[cb]) continue;
    const int64_t row = it.q_row0 + tok[cb];
    float* dst = a.dq + (row * a.hq + head[cb]) * D;
    if (a.accumulate) {
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
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          f32x4_t cur;
#pragma unroll
          for (int e = 0; e < 4; ++e) cur[e] = a.scale * acc[cb][db][4 * g4 + e];
          *reinterpret_cast<f32x4_t*>(dst + d) = cur;
        }
    }
  }
  clock.done(a.clk);
}

}  // namespace

// Column blocks per wave of the launched dQ kernel (see the forward's kFwdCB).
constexpr int kDqCB = 1;

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_qwg == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_qwg), block(64 * kColBlocksPerWG / kDqCB);
  if (head_dim == 128)
    hipLaunchKernelGGL((dq_kernel<128, kDqCB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((dq_kernel<64, kDqCB>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace fcp
