// Atomic-free building blocks of the dispatch (shared by the dispatch kernels
// and the decode expert kernel that routes its few tokens itself).
#pragma once

#include "common.h"

namespace moe {

#define DISP_BLOCK 1024

// Mask of the lanes whose key equals this lane's key (all 64 lanes active).
__device__ inline uint64_t match_lanes(int key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ inline int key_bits(int E) { return 32 - __clz(E); }   // keys 0..E fit

// Block-level stable ranking of NTH keys in [0, E] (E = "no expert").
// On return: wcnt[w * (E+1) + e] holds the number of keys e in waves < w of this
// block, *tot (per expert, E entries) the block's count, and the return value
// is the rank of this thread's key among equal keys of lower threads.
template <int NTH>
__device__ inline int block_rank(int key, int E, int* wcnt, int* tot) {
  constexpr int NW = NTH / MOE_WAVE;
  const int tid = threadIdx.x;
  const int w = tid / MOE_WAVE;
  const int lane = lane_id();
  const int stride = E + 1;
  for (int i = tid; i < NW * stride; i += NTH) wcnt[i] = 0;
  __syncthreads();
  const uint64_t m = match_lanes(key, key_bits(E));
  const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
  const int rank_w = __popcll(below);
  if (rank_w == 0) wcnt[w * stride + key] = __popcll(m);
  __syncthreads();
  for (int e = tid; e < E; e += NTH) {
    int c[NW];   // every wave's count read before the first write
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) c[ww] = wcnt[ww * stride + e];
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      wcnt[ww * stride + e] = run;
      run += c[ww];
    }
    tot[e] = run;
  }
  __syncthreads();
  return (key < E) ? wcnt[w * stride + key] + rank_w : -1;
}

// Exclusive scan of one int per thread over the whole block (NTH threads).
template <int NTH>
__device__ inline int block_excl_scan(int v, int* sh /* NTH / 64 + 1 ints */, int* total) {
  constexpr int NW = NTH / MOE_WAVE;
  const int lane = lane_id();
  const int w = threadIdx.x / MOE_WAVE;
  const int incl = wave_incl_scan(v);
  if (lane == MOE_WAVE - 1) sh[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int c[NW];   // every wave's total read before the first write
#pragma unroll
    for (int i = 0; i < NW; ++i) c[i] = sh[i];
    int run = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) { sh[i] = run; run += c[i]; }
    sh[NW] = run;
  }
  __syncthreads();
  const int r = sh[w] + incl - v;
  *total = sh[NW];
  __syncthreads();
  return r;
}

__device__ inline int load_key(const int* idx, int a, int T, int k, int E) {
  const int j = a / T;
  const int t = a - j * T;
  const int e = idx[(long long)t * k + j];
  return (e >= 0 && e < E) ? e : E;
}

// Zero the output rows of tokens with no kept local assignment (top-1 layers
// whose combine is folded into the expert kernel write every other row there).
template <int ESZ>
__device__ inline void zero_row(void* y, int t, int H) {
  uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(y) + (long long)t * H * ESZ);
  for (int c = 0; c < H * ESZ / 16; ++c) dst[c] = make_uint4(0, 0, 0, 0);
}

__device__ inline void zero_dropped(void* y_zero, int y_esz, int t, int H) {
  if (y_esz == 2) zero_row<2>(y_zero, t, H);
  else zero_row<4>(y_zero, t, H);
}

}  // namespace moe
