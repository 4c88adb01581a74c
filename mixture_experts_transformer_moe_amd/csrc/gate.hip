// Gate: fp32 logits z = x Wg^T (+ b) on the vector ALUs, and the wave-per-token
// softmax / top-k. (Large batches compute the logits with the MFMA grouped GEMM.)
#include "common.h"
#include "kernels.h"
#include "gate_dot.h"
#include "topk.h"

namespace moe {

// One 64-thread work-group (one wave) per block of EB experts x 8 tokens, so the
// gate weights stream through many CUs at once; small batches use EB = 1 or 2
// (more work-groups, fewer dot products per lane: the kernel is latency-bound).
// NQ in {1, 2} (H = 64 * NQ * VEC): every load of the block is issued before any
// arithmetic; NQ = 0 (EB = 4): any H, with gate_block's loop. For a given EB the
// accumulation and reduction order is fixed.
template <typename DT, int NQ, int EB>
__global__ __launch_bounds__(64) void gate_logits_fma_kernel(
    const typename DT::T* __restrict__ x, const typename DT::T* __restrict__ wg,
    const float* __restrict__ bias, float* __restrict__ z, int T, int H, int E, unsigned* __restrict__ fill,
    int nfill) {
  constexpr int NV = EB * GATE_TB;                 // logits per wave
  if (fill) {   // spread over the blocks
    const int b = blockIdx.y * gridDim.x + blockIdx.x, nb = gridDim.x * gridDim.y;
    for (int i = b * 64 + lane_id(); i < nfill; i += nb * 64) fill[i] = 0xFFFFFFFFu;
  }
  constexpr int SH = 6 - (NV == 8 ? 3 : NV == 16 ? 4 : 5);
  const int lane = lane_id();
  const int t0 = blockIdx.x * GATE_TB;
  const int e0 = blockIdx.y * EB;
  float r;
  if constexpr (NQ == 0) {
    static_assert(EB == GATE_EB, "the looped form reduces 4 x 8 blocks");
    r = gate_block<DT>(wg, x, H, E, T, e0, t0);
  } else {
    uint4 wv[EB][NQ], xv[GATE_TB][NQ];
#pragma unroll
    for (int i = 0; i < EB; ++i)
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
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < EB; ++i)
#pragma unroll
        for (int t = 0; t < GATE_TB; ++t) acc[i * GATE_TB + t] = dot16<DT>(wv[i][q], xv[t][q], acc[i * GATE_TB + t]);
    r = wave_reduce_multi<NV>(acc);
  }
  // after the reduction lane l holds logit number l >> SH: expert e0 + v / 8, token t0 + v % 8
  const int v = lane >> SH;
  const int e = e0 + v / GATE_TB;
  const int t = t0 + (v % GATE_TB);
  if ((lane & ((1 << SH) - 1)) == 0 && e < E && t < T) z[(long long)t * E + e] = r + (bias ? bias[e] : 0.f);
}

__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* z, int T, int E,
                                                           int k, int renorm, int* __restrict__ idx,
                                                           float* __restrict__ w,
                                                           float* probs, int zsplit) {
  const int t = blockIdx.x * 4 + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  int sel[2];
  wave_softmax_topk(z + (long long)t * E, E, k, renorm != 0, probs ? probs + (long long)t * E : nullptr,
                    idx + (long long)t * k, w + (long long)t * k, sel, zsplit, (long long)T * E);
}

template <typename DT, int EB>
static hipError_t launch_gate_fma_eb(const void* x, const void* wg, const float* bias, float* z, int T, int H, int E,
                                     int nq, hipStream_t s, unsigned* fill, int nfill) {
  using T_ = typename DT::T;
  dim3 grid((T + GATE_TB - 1) / GATE_TB, (E + EB - 1) / EB);
  if (nq == 1)
    hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 1, EB>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg, bias,
                       z, T, H, E, fill, nfill);
  else
    hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 2, EB>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg, bias,
                       z, T, H, E, fill, nfill);
  return hipGetLastError();
}

// experts per wave: 1 or 2 while that keeps the grid at <= 1024 / 2048 waves
static int gate_experts_per_wave(int T, int E, int H, int dtype) {
  const int vec = dtype == DT_F32 ? 4 : 8;
  if (H % (64 * vec) != 0 || H / (64 * vec) > 2) return GATE_EB;
  const long long tb = (T + GATE_TB - 1) / GATE_TB;
  if (tb * E <= 1024) return 1;
  if (tb * E <= 4096) return 2;
  return GATE_EB;
}

template <typename DT>
static hipError_t launch_gate_fma_t(const void* x, const void* wg, const float* bias, float* z, int T, int H, int E,
                                    hipStream_t s, unsigned* fill, int nfill) {
  using T_ = typename DT::T;
  const int nq = (H % (64 * DT::VEC) == 0) ? H / (64 * DT::VEC) : 0;
  const int eb = gate_experts_per_wave(T, E, H, sizeof(T_) == 4 ? DT_F32 : DT_F16);
  if (nq == 1 || nq == 2) {
    if (eb == 1) return launch_gate_fma_eb<DT, 1>(x, wg, bias, z, T, H, E, nq, s, fill, nfill);
    if (eb == 2) return launch_gate_fma_eb<DT, 2>(x, wg, bias, z, T, H, E, nq, s, fill, nfill);
    return launch_gate_fma_eb<DT, GATE_EB>(x, wg, bias, z, T, H, E, nq, s, fill, nfill);
  }
  dim3 grid((T + GATE_TB - 1) / GATE_TB, (E + GATE_EB - 1) / GATE_EB);
  hipLaunchKernelGGL((gate_logits_fma_kernel<DT, 0, GATE_EB>), grid, dim3(64), 0, s, (const T_*)x, (const T_*)wg,
                     bias, z, T, H, E, fill, nfill);
  return hipGetLastError();
}

hipError_t launch_gate_logits_fma(int dtype, const void* x, const void* wg, const float* bias, float* z,
                                  int T, int H, int E, hipStream_t s, unsigned* fill, int nfill) {
  switch (dtype) {
    case DT_F32: return launch_gate_fma_t<DtF32>(x, wg, bias, z, T, H, E, s, fill, nfill);
    case DT_F16: return launch_gate_fma_t<DtF16>(x, wg, bias, z, T, H, E, s, fill, nfill);
    default: return launch_gate_fma_t<DtBF16>(x, wg, bias, z, T, H, E, s, fill, nfill);
  }
}

hipError_t launch_softmax_topk(const float* z, int T, int E, int k, int renorm, int* idx, float* w,
                               float* probs, hipStream_t s, int zsplit) {
  hipLaunchKernelGGL(softmax_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, T, E, k, renorm, idx,
                     w, probs, zsplit < 1 ? 1 : zsplit);
  return hipGetLastError();
}

}  // namespace moe
