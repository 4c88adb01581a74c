// Combine: gather-scale-accumulate of the expert rows back into token order.
//
//   y[t] = sum_j w[t,j] * (sum_c src[c][token_slot[t,j]])  (+ sum_c dense[c][t])
//
// src holds P partial blocks of the expert outputs (P = 1 for the GEMM path,
// one per 64-wide FFN slice for the decode path); dense is the residual MLP's
// output (Pd blocks) or null. Each output element is owned by one thread, sums
// run in a fixed order in fp32, and the result is rounded once to the I/O dtype.
#include "common.h"
#include "kernels.h"

namespace moe {

template <typename DT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ src, int P, long long prow,
                                                      const int* __restrict__ token_slot,
                                                      const float* __restrict__ w, int k,
                                                      const float* __restrict__ dense, int Pd,
                                                      typename DT::T* __restrict__ y, int T, int H) {
  using Tt = typename DT::T;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int s = token_slot[(long long)t * k + j];
    if (s < 0) continue;
    const float wt = w[(long long)t * k + j];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < P; ++c) {
      const float4 u = *reinterpret_cast<const float4*>(src + ((long long)c * prow + s) * H + h);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    acc.x = fmaf(wt, v.x, acc.x);
    acc.y = fmaf(wt, v.y, acc.y);
    acc.z = fmaf(wt, v.z, acc.z);
    acc.w = fmaf(wt, v.w, acc.w);
  }
  if (dense) {
    float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < Pd; ++c) {
      const float4 u = *reinterpret_cast<const float4*>(dense + ((long long)c * T + t) * H + h);
      d.x += u.x; d.y += u.y; d.z += u.z; d.w += u.w;
    }
    acc.x += d.x; acc.y += d.y; acc.z += d.z; acc.w += d.w;
  }
  Tt* dst = y + (long long)t * H + h;
  dst[0] = DT::from_f(pin_f32(acc.x));
  dst[1] = DT::from_f(pin_f32(acc.y));
  dst[2] = DT::from_f(pin_f32(acc.z));
  dst[3] = DT::from_f(pin_f32(acc.w));
  }
}

hipError_t launch_combine(int dtype, const float* ysrc, int P, long long prow, const int* token_slot,
                          const float* w, int k, const float* dense, int Pd, void* y, int T, int H,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / 4 + 255) / 256, T < 65535 ? T : 65535);
  switch (dtype) {
    case DT_F32:
      hipLaunchKernelGGL(combine_kernel<DtF32>, grid, dim3(256), 0, s, ysrc, P, prow, token_slot, w, k, dense,
                         Pd, (float*)y, T, H);
      break;
    case DT_F16:
      hipLaunchKernelGGL(combine_kernel<DtF16>, grid, dim3(256), 0, s, ysrc, P, prow, token_slot, w, k, dense,
                         Pd, (_Float16*)y, T, H);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<DtBF16>, grid, dim3(256), 0, s, ysrc, P, prow, token_slot, w, k, dense,
                         Pd, (__bf16*)y, T, H);
  }
  return hipGetLastError();
}

}  // namespace moe
