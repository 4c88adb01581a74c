// Combine: gather-scale-accumulate of the expert rows back into token order.
//
//   y[t] = sum_j w[t,j] * src[token_slot[t,j]]  (+ dense[t])
//
// src holds the expert outputs (fp32, one row per dispatched slot); dense is the
// residual MLP's output (fp32) or null. Each output element is owned by one
// thread, sums run in choice order in fp32, and the result is rounded once to
// the I/O dtype. Dropped and non-local assignments (slot -1) add nothing.
#include "common.h"
#include "kernels.h"

namespace moe {

// Each thread owns 8 consecutive columns of a token row (two 16-byte loads per
// source row, one 16-byte store for 16-bit outputs); H % 8 == 0.
#define COMB_V 8
template <typename DT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ src,
                                                      const int* __restrict__ token_slot,
                                                      const float* __restrict__ w, int k,
                                                      const float* __restrict__ dense,
                                                      typename DT::T* __restrict__ y, int T, int H) {
  using Tt = typename DT::T;
  const int h = (blockIdx.x * 256 + threadIdx.x) * COMB_V;
  if (h >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[COMB_V];
#pragma unroll
    for (int i = 0; i < COMB_V; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int s = token_slot[(long long)t * k + j];
      if (s < 0) continue;
      const float wt = w[(long long)t * k + j];
      const float* row = src + (long long)s * H + h;
      const float4 u0 = *reinterpret_cast<const float4*>(row);
      const float4 u1 = *reinterpret_cast<const float4*>(row + 4);
      const float v[COMB_V] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < COMB_V; ++i) acc[i] = fmaf(wt, v[i], acc[i]);
    }
    if (dense) {
      const float* row = dense + (long long)t * H + h;
      const float4 u0 = *reinterpret_cast<const float4*>(row);
      const float4 u1 = *reinterpret_cast<const float4*>(row + 4);
      const float d[COMB_V] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < COMB_V; ++i) acc[i] += d[i];
    }
    Tt o[COMB_V];
#pragma unroll
    for (int i = 0; i < COMB_V; ++i) o[i] = DT::from_f(pin_f32(acc[i]));
    Tt* dst = y + (long long)t * H + h;
    if constexpr (sizeof(Tt) == 2) {
      *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, o);
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

hipError_t launch_combine(int dtype, const float* ysrc, const int* token_slot, const float* w, int k,
                          const float* dense, void* y, int T, int H, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / COMB_V + 255) / 256, T < 65535 ? T : 65535);
  switch (dtype) {
    case DT_F32:
      hipLaunchKernelGGL(combine_kernel<DtF32>, grid, dim3(256), 0, s, ysrc, token_slot, w, k, dense, (float*)y, T, H);
      break;
    case DT_F16:
      hipLaunchKernelGGL(combine_kernel<DtF16>, grid, dim3(256), 0, s, ysrc, token_slot, w, k, dense, (_Float16*)y,
                         T, H);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<DtBF16>, grid, dim3(256), 0, s, ysrc, token_slot, w, k, dense, (__bf16*)y,
                         T, H);
  }
  return hipGetLastError();
}

}  // namespace moe
