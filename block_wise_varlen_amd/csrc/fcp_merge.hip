// Streaming kernels: the LSE merge of per-pair partials and the backward's per-row
// Delta = sum_d dO * O. Both are bound by HBM bandwidth; one workgroup handles one query
// row across all heads so that every partial row is read as one contiguous run.
//
// Merge (FCP paper Sec. 2.2: per-slice results of a sequence reduce to the final output;
// the reduction is the log-sum-exp combine): for every head,
//   LSE = M + ln sum_p exp(LSE_p - M),  M = max_p LSE_p,
//   O   = sum_p exp(LSE_p - LSE) O_p,
// and a row whose partials are all empty (LSE_p = -inf) gets O = 0, LSE = -inf.
#include "fcp_common.h"
#include "fcp_kernels.h"
#include "fcp_types.h"

namespace fcp {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  extern __shared__ float s_lse[];
  const RowItem it = a.rows[blockIdx.x];
  const int hq = a.hq;
  const int32_t* parts = a.parts + it.part_begin;
  const int np = it.n_parts;

  for (int h = threadIdx.x; h < hq; h += 256) {
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p)
      mx = fmaxf(mx, a.lse_part[(int64_t)(parts[p] + it.row_in_group) * hq + h]);
    float out = -INFINITY;
    if (mx != -INFINITY) {
      float sum = 0.f;
      for (int p = 0; p < np; ++p)
        sum += __expf(a.lse_part[(int64_t)(parts[p] + it.row_in_group) * hq + h] - mx);
      out = mx + __logf(sum);
    }
    s_lse[h] = out;
    a.lse[(int64_t)it.q_row * hq + h] = out;
  }
  __syncthreads();

  constexpr int V4 = D / 4;
  const int total = hq * V4;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int h = e / V4;
    const float L = s_lse[h];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (L != -INFINITY) {
      int p = 0;
      for (; p + 4 <= np; p += 4) {
        f32x4_t x[4];
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t prow = parts[p + u] + it.row_in_group;
          w[u] = a.lse_part[prow * hq + h];
          x[u] = reinterpret_cast<const f32x4_t*>(a.o_part)[prow * total + e];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += __expf(w[u] - L) * x[u];
      }
      for (; p < np; ++p) {
        const int64_t prow = parts[p] + it.row_in_group;
        const float w = __expf(a.lse_part[prow * hq + h] - L);
        acc += w * reinterpret_cast<const f32x4_t*>(a.o_part)[prow * total + e];
      }
    }
    const uint32_t w0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    reinterpret_cast<u32x2_t*>(a.o)[(int64_t)it.q_row * total + e] = u32x2_t{w0, w1};
  }
}

// Delta_i = sum_d dO_i[d] * O_i[d] per (row, head), in fp32 from the bf16 tensors, stored
// beside the row's LSE in base 2 (+inf for a row that sees no key, so exp2(x - L2) = 0),
// head-major: the backward kernels read the pair with one 8-byte load per (row, head), and
// the stats of a run of rows of one head are contiguous.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int CPH = D / 8;  // 16-byte chunks per head
  const RowItem it = a.rows[blockIdx.x];
  const int total = a.hq * CPH;
  const int64_t base = (int64_t)it.q_row * a.hq * D;
  for (int e0 = 0; e0 < total; e0 += 256) {
    const int e = e0 + threadIdx.x;
    float s = 0.f;
    if (e < total) {
      const u32x4_t o = *reinterpret_cast<const u32x4_t*>(a.o + base + (int64_t)e * 8);
      const u32x4_t g = *reinterpret_cast<const u32x4_t*>(a.dout + base + (int64_t)e * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s += __uint_as_float(o[w] << 16) * __uint_as_float(g[w] << 16);
        s += __uint_as_float(o[w] & 0xffff0000u) * __uint_as_float(g[w] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int off = CPH / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (e < total && (e % CPH) == 0) {
      const int h = e / CPH;
      const float L = a.lse[(int64_t)it.q_row * a.hq + h];
      const float L2 = L == -INFINITY ? INFINITY : L * kLog2e;
      *reinterpret_cast<f32x2_t*>(a.stats + 2 * ((int64_t)h * a.q_rows + it.q_row)) =
          f32x2_t{L2, s};
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const size_t lds = (size_t)a.hq * sizeof(float);
  if (head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<128>), dim3(a.n_rows), dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((merge_kernel<64>), dim3(a.n_rows), dim3(256), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_delta(const DeltaArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL((delta_kernel<128>), dim3(a.n_rows), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((delta_kernel<64>), dim3(a.n_rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fcp
