// Gate: fp32 logits z = x Wg^T (+ b) on the vector ALUs, and the wave-per-token
// softmax / top-k. (Large batches compute the logits with the MFMA grouped GEMM.)
#include "common.h"
#include "kernels.h"
#include "gate_dot.h"
#include "topk.h"

namespace moe {

// One 64-thread work-group (one wave) per block of 4 experts x 8 tokens, so the
// gate weights stream through many CUs at once. NQ in {1, 2} (H = 64 * NQ * VEC):
// every load of the block is issued before any arithmetic; NQ = 0: any H, with
// gate_block's loop. Both forms accumulate and reduce in the same order.
template <typename DT, int NQ>
__global__ __launch_bounds__(64) void gate_logits_fma_kernel(
    const typename DT::T* __restrict__ x, const typename DT::T* __restrict__ wg,
    const float* __restrict__ bias, float* __restrict__ z, int T, int H, int E) {
  const int lane = lane_id();
  const int t0 = blockIdx.x * GATE_TB;
  const int e0 = blockIdx.y * GATE_EB;
  float r;
  if constexpr (NQ == 0) {
    r = gate_block<DT>(wg, x, H, E, T, e0, t0);
  } else {
    uint4 wv[GATE_EB][NQ], xv[GATE_TB][NQ];
#pragma unroll
    for (int i = 0; i < GATE_EB; ++i)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        wv[i][q] = mask16(reinterpret_cast<const uint4*>(wg + (long long)min(e0 + i, E - 1) * H)[lane + 64 * q],
                          e0 + i < E);
#pragma unroll
    for (int t = 0; t < GATE_TB; ++t)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        xv[t][q] = mask16(reinterpret_cast<const uint4*>(x + (long long)min(t0 + t, T - 1) * H)[lane + 64 * q],
                          t0 + t < T);
    float acc[GATE_EB * GATE_TB];
#pragma unroll
    for (int i = 0; i < GATE_EB * GATE_TB; ++i) acc[i] = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < GATE_EB; ++i)
#pragma unroll
        for (int t = 0; t < GATE_TB; ++t) acc[i * GATE_TB + t] = dot16<DT>(wv[i][q], xv[t][q], acc[i * GATE_TB + t]);
    r = wave_reduce_multi<GATE_EB * GATE_TB>(acc);
  }
  const int e = e0 + gate_block_expert(lane);
  const int t = t0 + gate_block_token(lane);
  if ((lane & 1) == 0 && e < E && t < T) z[(long long)t * E + e] = r + (bias ? bias[e] : 0.f);
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
static hipError_t launch_gate_fma_t(const void* x, const void* wg, const float* bias, float* z, int T, int H, int E,
                                    hipStream_t s) {
  using T_ = typename DT::T;
  dim3 grid((T + GATE_TB - 1) / GATE_TB, (E + GATE_EB - 1) / GATE_EB);
  const int nq = (H % (64 * DT::VEC) == 0) ? H / (64 * DT::VEC) : 0;
  if (nq == 1)
    hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 1>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg, bias, z,
                       T, H, E);
  else if (nq == 2)
    hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 2>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg, bias, z,
                       T, H, E);
  else
    hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 0>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg, bias, z,
                       T, H, E);
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
