// Streaming kernel: the LSE merge of per-pair partials, bound by HBM bandwidth; one
// workgroup handles one query row across all heads so that every partial row is read as
// one contiguous run.
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

// Four consecutive partial values (element e4 of 4-value groups), from fp32 or bf16
// partials.
template <bool PB>
__device__ __forceinline__ f32x4_t load4(const MergeArgs& a, int64_t e4) {
  if constexpr (PB) {
    const u32x2_t w = reinterpret_cast<const u32x2_t*>(a.o_part16)[e4];
    return f32x4_t{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                   __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
  } else {
    return reinterpret_cast<const f32x4_t*>(a.o_part)[e4];
  }
}

template <int D, bool PB>
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
          x[u] = load4<PB>(a, prow * total + e);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += __expf(w[u] - L) * x[u];
      }
      for (; p < np; ++p) {
        const int64_t prow = parts[p] + it.row_in_group;
        const float w = __expf(a.lse_part[prow * hq + h] - L);
        acc += w * load4<PB>(a, prow * total + e);
      }
    }
    const uint32_t w0 = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    reinterpret_cast<u32x2_t*>(a.o)[(int64_t)it.q_row * total + e] = u32x2_t{w0, w1};
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const size_t lds = (size_t)a.hq * sizeof(float);
  const bool pb = a.o_part16 != nullptr;
  if (head_dim == 128) {
    if (pb)
      hipLaunchKernelGGL((merge_kernel<128, true>), dim3(a.n_rows), dim3(256), lds, stream, a);
    else
      hipLaunchKernelGGL((merge_kernel<128, false>), dim3(a.n_rows), dim3(256), lds, stream, a);
  } else {
    if (pb)
      hipLaunchKernelGGL((merge_kernel<64, true>), dim3(a.n_rows), dim3(256), lds, stream, a);
    else
      hipLaunchKernelGGL((merge_kernel<64, false>), dim3(a.n_rows), dim3(256), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fcp
