// Gate logits for a block of 4 experts x 8 tokens, computed by one wave.
//
// Every lane walks the hidden dimension in 16-byte vectors (vector c = lane,
// lane + 64, ...), accumulating 32 fp32 dot products in a fixed order; one
// multi-value wave reduction then leaves logit (e0 + (lane >> 4), t0 +
// ((lane >> 1) & 7)) in each lane. This is the looped form for hidden sizes that
// are not 64 * 8 or 128 * 8 elements.
#pragma once

#include "common.h"

namespace moe {

#define GATE_EB 4   // experts per wave block
#define GATE_TB 8   // tokens per wave block

template <typename DT>
__device__ inline float gate_block(const typename DT::T* __restrict__ wg, const typename DT::T* __restrict__ x,
                                   int H, int E, int T, int e0, int t0) {
  using T_ = typename DT::T;
  const int lane = threadIdx.x & 63;
  const int nvec = H / DT::VEC;
  float acc[GATE_EB * GATE_TB];
#pragma unroll
  for (int i = 0; i < GATE_EB * GATE_TB; ++i) acc[i] = 0.f;
  for (int c = lane; c < nvec; c += 64) {
    // rows past E or T are loaded from a valid row and masked to zero (no branches)
    uint4 wv[GATE_EB], xv[GATE_TB];
#pragma unroll
    for (int i = 0; i < GATE_EB; ++i)
      wv[i] = mask16(reinterpret_cast<const uint4*>(wg + (long long)min(e0 + i, E - 1) * H)[c], e0 + i < E);
#pragma unroll
    for (int t = 0; t < GATE_TB; ++t)
      xv[t] = mask16(reinterpret_cast<const uint4*>(x + (long long)min(t0 + t, T - 1) * H)[c], t0 + t < T);
#pragma unroll
    for (int i = 0; i < GATE_EB; ++i)
#pragma unroll
      for (int t = 0; t < GATE_TB; ++t) acc[i * GATE_TB + t] = dot16<DT>(wv[i], xv[t], acc[i * GATE_TB + t]);
  }
  (void)sizeof(T_);
  return wave_reduce_multi<GATE_EB * GATE_TB>(acc);
}

}  // namespace moe
