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

// Each thread owns 8 consecutive columns of a token row (two 16-byte loads per
// source row, one 16-byte store for 16-bit outputs); H % 8 == 0.
#define COMB_V 8
template <typename DT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ src, int P, long long prow,
                                                      const int* __restrict__ token_slot,
                                                      const float* __restrict__ w, int k,
                                                      const float* __restrict__ dense, int Pd,
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
      float v[COMB_V];
#pragma unroll
      for (int i = 0; i < COMB_V; ++i) v[i] = 0.f;
      for (int c = 0; c < P; ++c) {
        const float* row = src + ((long long)c * prow + s) * H + h;
        const float4 u0 = *reinterpret_cast<const float4*>(row);
        const float4 u1 = *reinterpret_cast<const float4*>(row + 4);
        v[0] += u0.x; v[1] += u0.y; v[2] += u0.z; v[3] += u0.w;
        v[4] += u1.x; v[5] += u1.y; v[6] += u1.z; v[7] += u1.w;
      }
#pragma unroll
      for (int i = 0; i < COMB_V; ++i) acc[i] = fmaf(wt, v[i], acc[i]);
    }
    if (dense) {
      float d[COMB_V];
#pragma unroll
      for (int i = 0; i < COMB_V; ++i) d[i] = 0.f;
      for (int c = 0; c < Pd; ++c) {
        const float* row = dense + ((long long)c * T + t) * H + h;
        const float4 u0 = *reinterpret_cast<const float4*>(row);
        const float4 u1 = *reinterpret_cast<const float4*>(row + 4);
        d[0] += u0.x; d[1] += u0.y; d[2] += u0.z; d[3] += u0.w;
        d[4] += u1.x; d[5] += u1.y; d[6] += u1.z; d[7] += u1.w;
      }
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

hipError_t launch_combine(int dtype, const float* ysrc, int P, long long prow, const int* token_slot,
                          const float* w, int k, const float* dense, int Pd, void* y, int T, int H,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / COMB_V + 255) / 256, T < 65535 ? T : 65535);
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
