// Gate: fp32 logits z = x Wg^T (+ b) for small batches, and the wave-per-token
// softmax / top-k. (Large batches compute the logits with the MFMA grouped GEMM.)
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// One wave per expert, TB tokens per work-group row; every lane walks the
// hidden dimension in 16-byte vectors and the wave reduces at the end.
template <typename DT, int TB>
__global__ __launch_bounds__(256) void gate_logits_fma_kernel(
    const typename DT::T* __restrict__ x, const typename DT::T* __restrict__ wg,
    const float* __restrict__ bias, float* __restrict__ z, int T, int H, int E) {
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = lane_id();
  const int e = blockIdx.x * 4 + wave;
  const int t0 = blockIdx.y * TB;
  if (e >= E) return;
  const int nvec = H / DT::VEC;
  const uint4* wrow = reinterpret_cast<const uint4*>(wg + (long long)e * H);
  float acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.f;
  for (int c = lane; c < nvec; c += MOE_WAVE) {
    const uint4 wv = wrow[c];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      if (t0 + i < T) {
        const uint4 xv = reinterpret_cast<const uint4*>(x + (long long)(t0 + i) * H)[c];
        acc[i] = dot16<DT>(wv, xv, acc[i]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    float s = wave_sum(acc[i]);
    if (lane == 0 && t0 + i < T) z[(long long)(t0 + i) * E + e] = s + b;
  }
}

__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* z, int T, int E,
                                                           int k, int renorm, int* __restrict__ idx,
                                                           float* __restrict__ w,
                                                           float* probs) {
  const int t = blockIdx.x * 4 + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  int sel[2];
  wave_softmax_topk(z + (long long)t * E, E, k, renorm != 0, probs ? probs + (long long)t * E : nullptr,
                    idx + (long long)t * k, w + (long long)t * k, sel);
}

template <typename DT>
static hipError_t launch_gate_fma_t(const void* x, const void* wg, const float* bias, float* z, int T,
                                    int H, int E, hipStream_t s) {
  constexpr int TB = 8;
  dim3 grid((E + 3) / 4, (T + TB - 1) / TB);
  hipLaunchKernelGGL((gate_logits_fma_kernel<DT, TB>), grid, dim3(256), 0, s,
                     (const typename DT::T*)x, (const typename DT::T*)wg, bias, z, T, H, E);
  return hipGetLastError();
}

hipError_t launch_gate_logits_fma(int dtype, const void* x, const void* wg, const float* bias, float* z,
                                  int T, int H, int E, hipStream_t s) {
  switch (dtype) {
    case DT_F32: return launch_gate_fma_t<DtF32>(x, wg, bias, z, T, H, E, s);
    case DT_F16: return launch_gate_fma_t<DtF16>(x, wg, bias, z, T, H, E, s);
    default: return launch_gate_fma_t<DtBF16>(x, wg, bias, z, T, H, E, s);
  }
}

hipError_t launch_softmax_topk(const float* z, int T, int E, int k, int renorm, int* idx, float* w,
                               float* probs, hipStream_t s) {
  hipLaunchKernelGGL(softmax_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, T, E, k, renorm, idx,
                     w, probs);
  return hipGetLastError();
}

}  // namespace moe
