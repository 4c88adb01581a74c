// Wave-level softmax + top-k over one token's gate logits (one wave64 per token).
#pragma once

#include "common.h"

namespace moe {

#define MOE_MAX_EPL 8    // logits per lane: E <= 512

// Keep the better of two (value, index) pairs: larger value, ties to the lower index.
__device__ inline void better_of(float& v, int& idx, float ov, int oi) {
  if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
}
template <int CTRL>
__device__ inline void argmax_dpp_step(float& v, int& idx) {
  better_of(v, idx, dpp_mov<CTRL>(v), dpp_mov<CTRL>(idx));
}

// Reduce (value, index) pairs to the wave's best: larger value, ties to the
// lower index (the rule picks the same pair in any order). Rows by the DPP steps
// of wave_max, then the four row winners. Lanes holding no candidate pass
// idx = INT_MAX, v = -inf. Every lane returns the winner.
__device__ inline void wave_argmax(float& v, int& idx) {
  argmax_dpp_step<MOE_DPP_XOR1>(v, idx);
  argmax_dpp_step<MOE_DPP_XOR2>(v, idx);
  argmax_dpp_step<MOE_DPP_HMIRROR>(v, idx);
  argmax_dpp_step<MOE_DPP_MIRROR>(v, idx);
  float v0 = readlane_f(v, 0), v2 = readlane_f(v, 32);
  int i0 = __builtin_amdgcn_readlane(idx, 0), i2 = __builtin_amdgcn_readlane(idx, 32);
  better_of(v0, i0, readlane_f(v, 16), __builtin_amdgcn_readlane(idx, 16));
  better_of(v2, i2, readlane_f(v, 48), __builtin_amdgcn_readlane(idx, 48));
  better_of(v0, i0, v2, i2);
  v = v0;
  idx = i0;
}

// The k largest logits (ties to the lower index) of a token whose logits this lane
// holds in v[i] (expert lane + 64 i, i < epl). Every lane returns them in sel,
// and the winning logits in bvs.
__device__ inline void wave_select_topk(const float (&v)[MOE_MAX_EPL], int epl, int E, int k, int* sel, float* bvs) {
  const int lane = lane_id();
  sel[0] = sel[1] = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < MOE_MAX_EPL; ++i) {
      int e = lane + i * MOE_WAVE;
      bool ok = (i < epl) && (e < E) && (e != sel[0]);
      if (ok && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
    wave_argmax(bv, bi);
    if (bi >= E) bi = (j == 0 ? 0 : (sel[0] == 0 ? 1 : 0));  // only if every logit is NaN
    sel[j] = bi;
    bvs[j] = bv;
  }
}

// Only the top-k indices (no probabilities): the same choice as wave_softmax_topk.
__device__ inline void wave_topk_only(const float* z, int E, int k, int* idx_out) {
  const int lane = lane_id();
  float v[MOE_MAX_EPL];
  const int epl = (E + MOE_WAVE - 1) / MOE_WAVE;
#pragma unroll
  for (int i = 0; i < MOE_MAX_EPL; ++i) {
    int e = lane + i * MOE_WAVE;
    v[i] = (i < epl && e < E) ? z[e] : -INFINITY;
  }
  int sel[2];
  float bvs[2];
  wave_select_topk(v, epl, E, k, sel, bvs);
  if (lane == 0)
    for (int j = 0; j < k; ++j) idx_out[j] = sel[j];
}

// This lane's logits v[i] (expert lane + 64 i, i < epl; -inf past E), each the
// sum of NS partial sums nstride floats apart added in order 0, 1, ...: every
// load is issued before the first add.
template <int NS>
__device__ inline void load_logits(const float* z, int E, int epl, long long nstride, float (&v)[MOE_MAX_EPL]) {
  const int lane = lane_id();
  float part[NS][MOE_MAX_EPL];
#pragma unroll
  for (int i = 0; i < MOE_MAX_EPL; ++i) {
    const int e = lane + i * MOE_WAVE;
#pragma unroll
    for (int s = 0; s < NS; ++s) part[s][i] = (i < epl && e < E) ? z[s * nstride + e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < MOE_MAX_EPL; ++i) {
    const int e = lane + i * MOE_WAVE;
    float a = part[0][i];
#pragma unroll
    for (int s = 1; s < NS; ++s) a += part[s][i];
    v[i] = (i < epl && e < E) ? a : -INFINITY;
  }
}

// z: this token's E logits (fp32), or nsplit partial sums of them nstride floats
// apart, added in order 0, 1, ... . Writes idx_out[0..k), w_out[0..k) and, when
// probs != null, probs[0..E). Softmax is max-subtracted fp32; the choice is made
// on the logits (ties to the lower expert index), so exp rounding cannot tie.
// Every lane returns the chosen indices in sel[0..k).
__device__ inline void wave_softmax_topk(const float* z, int E, int k, bool renorm,
                                         float* probs, int* idx_out, float* w_out,
                                         int* sel, int nsplit = 1, long long nstride = 0) {
  const int lane = lane_id();
  float v[MOE_MAX_EPL];
  const int epl = (E + MOE_WAVE - 1) / MOE_WAVE;
  switch (nsplit) {
    case 2: load_logits<2>(z, E, epl, nstride, v); break;
    case 4: load_logits<4>(z, E, epl, nstride, v); break;
    case 8: load_logits<8>(z, E, epl, nstride, v); break;
    default:
      if (nsplit <= 1) {
        load_logits<1>(z, E, epl, nstride, v);
      } else {
#pragma unroll
        for (int i = 0; i < MOE_MAX_EPL; ++i) {
          const int e = lane + i * MOE_WAVE;
          float a = -INFINITY;
          if (i < epl && e < E) {
            a = z[e];
            for (int s = 1; s < nsplit; ++s) a += z[s * nstride + e];
          }
          v[i] = a;
        }
      }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < MOE_MAX_EPL; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MOE_MAX_EPL; ++i) {
    int e = lane + i * MOE_WAVE;
    if (i < epl && e < E) s += expf(v[i] - m);
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  if (probs) {
#pragma unroll
    for (int i = 0; i < MOE_MAX_EPL; ++i) {
      int e = lane + i * MOE_WAVE;
      if (i < epl && e < E) probs[e] = expf(v[i] - m) * inv;
    }
  }
  float wsel[2] = {0.f, 0.f};
  float bvs[2];
  wave_select_topk(v, epl, E, k, sel, bvs);
  for (int j = 0; j < k; ++j) wsel[j] = expf(bvs[j] - m) * inv;
  if (renorm) {
    float t = (k == 2) ? wsel[0] + wsel[1] : wsel[0];
    wsel[0] /= t;
    wsel[1] /= t;
  }
  if (lane == 0) {
    for (int j = 0; j < k; ++j) { idx_out[j] = sel[j]; w_out[j] = wsel[j]; }
  }
}

}  // namespace moe
