// Dispatch: capacity-limited, rank-major, atomic-free assignment of tokens to
// per-expert segments.
//
// Assignment a = j * T + t (choice j of token t) is ranked before every
// assignment with a larger a, so all first choices outrank all second choices
// and lower tokens outrank higher ones. pos(a) = number of earlier assignments
// to the same expert; the assignment keeps row offsets[e] + pos(a) of its local
// expert while pos(a) < C and is dropped otherwise.
//
// No atomics anywhere: inside a wave, lanes with the same expert find each other
// with one ballot per key bit; waves are combined by a per-expert scan in LDS;
// blocks by a per-expert scan over the blocks' histograms.
#include "common.h"
#include "kernels.h"
#include "dispatch_common.h"
#include "topk.h"
#include "tile_plan.h"

namespace moe {

#define DISP_WAVES (DISP_BLOCK / MOE_WAVE)

// -------------------------------------------------------------------- multi-block path
__global__ __launch_bounds__(DISP_BLOCK) void dispatch_count_kernel(const int* __restrict__ idx, int T,
                                                                    int k, int E, int* __restrict__ rank,
                                                                    int* __restrict__ blk_hist) {
  extern __shared__ int sh[];
  int* wcnt = sh;                                  // DISP_WAVES * (E + 1)
  int* tot = sh + DISP_WAVES * (E + 1);            // E
  const int kT = T * k;
  const int a = blockIdx.x * DISP_BLOCK + threadIdx.x;
  const int key = (a < kT) ? load_key(idx, a, T, k, E) : E;
  const int r = block_rank<DISP_BLOCK>(key, E, wcnt, tot);
  for (int e = threadIdx.x; e < E; e += DISP_BLOCK) blk_hist[(long long)blockIdx.x * E + e] = tot[e];
  if (a < kT) rank[a] = r;
}

// Column scan of the block histograms (becomes each block's per-expert base),
// demand, kept rows and the local segment offsets. One block. Each thread
// loads eight blocks' counts of its expert at a time before it scans them.
__global__ __launch_bounds__(DISP_BLOCK) void dispatch_scan_kernel(int* __restrict__ blk_hist, int nblk,
                                                                   int E, int e_lo, int E_loc, int C,
                                                                   int* __restrict__ demand,
                                                                   int* __restrict__ offsets) {
  __shared__ int sdem[1024];
  __shared__ int ssc[DISP_WAVES + 1];
  const int tid = threadIdx.x;
  if (tid < E) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = b0 + i < nblk ? blk_hist[(long long)(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b0 + i < nblk) blk_hist[(long long)(b0 + i) * E + tid] = run;
        run += c[i];
      }
    }
    demand[tid] = run;
    sdem[tid] = run;
  }
  __syncthreads();
  const int kept = (tid < E_loc) ? min(sdem[e_lo + tid], C) : 0;
  int total;
  const int off = block_excl_scan<DISP_BLOCK>(kept, ssc, &total);
  if (tid < E_loc) offsets[tid] = off;
  if (tid == 0) offsets[E_loc] = total;
}

// Slots of the assignments of block b < nblk; with tile lists to write, the
// blocks past every assignment (nplan of them) build the lists from the segment
// offsets while the others scatter.
__global__ __launch_bounds__(DISP_BLOCK) void dispatch_scatter_kernel(
    const int* __restrict__ idx, const int* __restrict__ rank, const int* __restrict__ base, int T, int k,
    int E, int e_lo, int E_loc, int C, const int* __restrict__ offsets, int R_max,
    int* __restrict__ slot_token, int* __restrict__ token_slot, void* y_zero, int y_esz, int H, int nblk,
    int nplan, TilePlanArgs plan) {
  if ((int)blockIdx.x >= nblk) {
    __shared__ int plds[tile_plan_lds_ints(DISP_BLOCK)];
    const int tid = threadIdx.x;
    const int rows = tid < E_loc ? offsets[tid + 1] - offsets[tid] : 0;
    tile_plan_body<DISP_BLOCK>(rows, E_loc, plan, plds, (int)blockIdx.x - nblk, nplan);
    return;
  }
  const int kT = T * k;
  const int a = blockIdx.x * DISP_BLOCK + threadIdx.x;
  if (a < kT) {
    const int j = a / T;
    const int t = a - j * T;
    const int e = load_key(idx, a, T, k, E);
    int slot = -1;
    if (e < E && e >= e_lo && e < e_lo + E_loc) {
      const int pos = base[(long long)blockIdx.x * E + e] + rank[a];
      if (pos < C) {
        slot = offsets[e - e_lo] + pos;
        slot_token[slot] = t;
      }
    }
    token_slot[(long long)t * k + j] = slot;
    if (y_zero && slot < 0) zero_dropped(y_zero, y_esz, t, H);
  }
  const int R = offsets[E_loc];
  for (int s = R + blockIdx.x * DISP_BLOCK + threadIdx.x; s < R_max; s += nblk * DISP_BLOCK)
    slot_token[s] = -1;
}

// -------------------------------------------------------------------- one-launch path
// Softmax / top-k, ranking, the scan over blocks, scatter and the tile lists of
// a batch of more than one block of assignments in one launch. Block roles, in
// the order the dispatcher starts them:
//   [0, nsoft)             one wave per token: softmax / top-k as
//                          softmax_topk_kernel; choice j of token t is then
//                          published as keys[j * T + t] = expert + 1;
//   [nsoft, nsoft + nblk)  ranker r: assignments r * DISP_BLOCK ... as the
//                          count kernel, publishes its per-expert counts + 1 as
//                          hist[r * E + e], adds up every ranker's counts (its
//                          base and the totals), then scatters as the scatter
//                          kernel;
//   the last nplan         the tile lists (and offsets) from the totals.
// A published word is written and read by agent-scope atomics (written through
// to memory, read past the XCD's L2); 0, left by the launch before, means not
// yet written. Softmax blocks wait for nothing and rankers publish before they
// wait, so once the rankers and list builders (at most ROUTE_MAX_BLOCKS + a
// few) are resident every wait ends. A wait that outlasts ROUTE_WAIT_TICKS gives
// up: a key counts as no expert (the ranker publishes what it used, so every
// block still sees the same counts), a count as 0. Blocks that gave up on a
// count may then disagree, but each writes only in-range values (its tokens,
// slots < R_max, offsets <= R_max) and leaves slot_token's tail of -1 to the
// others; every slot_token entry below the offsets' end holds a token (the
// launch before zeroed them), and the GEMMs skip any list entry that names no
// tile with rows under the offsets (tile_entry), so nothing downstream reads or
// writes out of bounds.
#define ROUTE_WAIT_TICKS 5000000ull   // 50 ms of the 100 MHz real-time counter
#define ROUTE_MAX_BLOCKS 64

__device__ inline int pub_load(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void pub_store(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// The published word at p, given its first read v; 0 if the wait gives up
// (ok then false; later waits of the thread give up at once).
__device__ inline int pub_wait(const int* p, int v, unsigned long long t0, bool& ok) {
  while (v == 0) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > ROUTE_WAIT_TICKS) {
      ok = false;
      return 0;
    }
    __builtin_amdgcn_s_sleep(1);
    v = pub_load(p);
  }
  return v;
}

// One lane polls the word at p (sleeping between reads) before the block reads
// all of its words: a hint, so that a block started early does not flood memory
// with reads; the per-word waits that follow decide.
__device__ inline void pub_hint(const int* p, unsigned long long t0) {
  if (threadIdx.x == 0) {
    while (pub_load(p) == 0 && __builtin_amdgcn_s_memrealtime() - t0 <= ROUTE_WAIT_TICKS)
      __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();
}

__global__ __launch_bounds__(DISP_BLOCK) void route_dispatch_kernel(RouteDispatchArgs a, int nsoft, int nblk,
                                                                    int nplan, TilePlanArgs plan) {
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (b < nsoft) {
    const int t = b * DISP_WAVES + tid / MOE_WAVE;
    if (t >= a.T) return;
    int sel[2];
    wave_softmax_topk(a.z + (long long)t * a.E, a.E, a.k, a.renorm != 0,
                      a.probs ? a.probs + (long long)t * a.E : nullptr, a.idx + (long long)t * a.k,
                      a.topk_w + (long long)t * a.k, sel, a.zsplit, (long long)a.T * a.E);
    if (lane_id() == 0)
      for (int j = 0; j < a.k; ++j) pub_store(a.keys + (long long)j * a.T + t, sel[j] + 1);
    return;
  }
  extern __shared__ int sh[];
  const int E = a.E;
  const bool ranker = b < nsoft + nblk;
  const int rb = ranker ? b - nsoft : nblk;   // list builders count every ranker as earlier
  int* wcnt = sh;                             // DISP_WAVES * (E + 1)
  int* tot = wcnt + DISP_WAVES * (E + 1);     // E
  int* sbase = tot + E;                       // E: counts of the earlier rankers
  int* stot = sbase + E;                      // E: every ranker's counts
  int* soff = stot + E;                       // E_loc + 1 (<= E + 1)
  int* ssc = soff + E + 1;                    // DISP_WAVES + 1
  int* plds = ssc + DISP_WAVES + 1;           // tile_plan_lds_ints(DISP_BLOCK)
  __shared__ int full;                        // every count this block waited for came
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  const int kT = a.T * a.k;
  const int as = rb * DISP_BLOCK + tid;
  int key = E, r = -1;
  if (ranker) {
    pub_hint(a.keys + min(rb * DISP_BLOCK + DISP_BLOCK, kT) - 1, t0);
    if (as < kT) {
      bool kok = true;
      const int* kp = a.keys + as;
      const int v = pub_wait(kp, pub_load(kp), t0, kok);
      key = (v >= 1 && v <= E) ? v - 1 : E;
    }
    r = block_rank<DISP_BLOCK>(key, E, wcnt, tot);
    for (int e = tid; e < E; e += DISP_BLOCK) pub_store(a.hist + (long long)rb * E + e, tot[e] + 1);
  } else {
    pub_hint(a.hist + (long long)nblk * E - 1, t0);
  }
  if (tid == 0) full = 1;
  __syncthreads();

  // every ranker's counts: thread (e, j) of the tpe threads of expert e (adjacent
  // lanes) adds rankers j, j + tpe, ..., four reads in flight at a time
  int tpe = 1;
  while (tpe < MOE_WAVE && E * tpe * 2 <= DISP_BLOCK) tpe *= 2;
  const int e = tid / tpe, jj = tid - (tid / tpe) * tpe;
  bool ok = true;
  int before = 0, total = 0;
  if (e < E) {
    for (int b0 = jj; b0 < nblk; b0 += 4 * tpe) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b2 = b0 + u * tpe;
        v[u] = b2 < nblk ? pub_load(a.hist + (long long)b2 * E + e) : 1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b2 = b0 + u * tpe;
        if (b2 < nblk) {
          const int c = pub_wait(a.hist + (long long)b2 * E + e, v[u], t0, ok);
          const int cnt = c > 0 ? c - 1 : 0;
          total += cnt;
          if (b2 < rb) before += cnt;
        }
      }
    }
  }
  for (int o = 1; o < tpe; o <<= 1) {
    before += __shfl_xor(before, o, MOE_WAVE);
    total += __shfl_xor(total, o, MOE_WAVE);
  }
  if (e < E && jj == 0) {
    sbase[e] = before;
    stot[e] = total;
  }
  if (!ok) full = 0;
  __syncthreads();

  const int kept = (tid < a.E_loc) ? min(stot[a.e_lo + tid], a.C) : 0;
  int R;
  const int off = block_excl_scan<DISP_BLOCK>(kept, ssc, &R);
  if (nplan > 0 ? b == nsoft + nblk : rb == 0) {
    for (int x = tid; x < E; x += DISP_BLOCK) a.demand[x] = stot[x];
    if (tid < a.E_loc) a.offsets[tid] = off;
    if (tid == 0) a.offsets[a.E_loc] = R;
  }
  if (!ranker) {
    tile_plan_body<DISP_BLOCK>(kept, a.E_loc, plan, plds, b - nsoft - nblk, nplan);
    return;
  }
  if (tid < a.E_loc) soff[tid] = off;
  __syncthreads();
  if (as < kT) {
    const int j = as / a.T;
    const int t = as - j * a.T;
    int slot = -1;
    if (key < E && key >= a.e_lo && key < a.e_lo + a.E_loc) {
      const int pos = sbase[key] + r;
      const int s2 = soff[key - a.e_lo] + pos;
      if (pos < a.C && s2 < a.R_max) {   // (s2 < R_max always holds once every count came)
        slot = s2;
        a.slot_token[slot] = t;
      }
    }
    a.token_slot[(long long)t * a.k + j] = slot;
    if (a.y_zero && slot < 0) zero_dropped(a.y_zero, a.y_esz, t, a.H);
  }
  if (full)
    for (int s = R + rb * DISP_BLOCK + tid; s < a.R_max; s += nblk * DISP_BLOCK) a.slot_token[s] = -1;
}

// -------------------------------------------------------------------- one-block path
// Whole dispatch for k*T <= NTH in one block of NTH threads. MODE 0: the routing
// comes from idx; MODE 1: softmax / top-k of every token first, from logits z
// (one wave per token). sh must hold small_lds_ints<NTH>(E) ints.
template <int MODE, int NTH>
__device__ inline void dispatch_small_body(int* sh, const float* z, int renorm, float* probs, float* topk_w, int* idx,
                                           int T, int k, int E, int e_lo, int E_loc, int C, int R_max,
                                           int* demand, int* offsets, int* slot_token, int* token_slot,
                                           void* y_zero, int y_esz, int H, const TilePlanArgs& plan, int zsplit) {
  constexpr int NW = NTH / MOE_WAVE;
  int* wcnt = sh;                                   // NW * (E + 1)
  int* tot = wcnt + NW * (E + 1);                   // E
  int* sidx = tot + E;                              // NTH
  int* ssc = sidx + NTH;                            // NW + 1
  int* plds = ssc + NW + 1;                         // tile_plan_lds_ints(NTH)
  const int tid = threadIdx.x;
  const int kT = T * k;
  if (MODE == 1) {
    const int w = tid / MOE_WAVE;
    for (int t = w; t < T; t += NW) {
      int sel[2];
      wave_softmax_topk(z + (long long)t * E, E, k, renorm != 0, probs ? probs + (long long)t * E : nullptr,
                        idx + (long long)t * k, topk_w + (long long)t * k, sel, zsplit, (long long)T * E);
      if (lane_id() == 0)
        for (int j = 0; j < k; ++j) sidx[j * T + t] = sel[j];
    }
    __syncthreads();
  }
  int key = E;
  if (tid < kT) {
    if (MODE == 1) {
      const int e = sidx[tid];
      key = (e >= 0 && e < E) ? e : E;
    } else {
      key = load_key(idx, tid, T, k, E);
    }
  }
  const int r = block_rank<NTH>(key, E, wcnt, tot);
  for (int e = tid; e < E; e += NTH) demand[e] = tot[e];
  const int kept = (tid < E_loc) ? min(tot[e_lo + tid], C) : 0;
  int total;
  const int off = block_excl_scan<NTH>(kept, ssc, &total);
  if (tid < E_loc) sidx[tid] = off;   // reuse: segment offsets (the keys are already in registers)
  if (tid < E_loc) offsets[tid] = off;
  if (tid == 0) offsets[E_loc] = total;
  __syncthreads();
  if (tid < kT) {
    const int j = tid / T;
    const int t = tid - j * T;
    int slot = -1;
    if (key < E && key >= e_lo && key < e_lo + E_loc && r < C) {
      slot = sidx[key - e_lo] + r;
      slot_token[slot] = t;
    }
    token_slot[(long long)t * k + j] = slot;
    if (y_zero && slot < 0) zero_dropped(y_zero, y_esz, t, H);
  }
  for (int s = total + tid; s < R_max; s += NTH) slot_token[s] = -1;
  if (plan.list1 || plan.list2) tile_plan_body<NTH>(kept, E_loc, plan, plds);
}

template <int MODE, int NTH>
__global__ __launch_bounds__(NTH) void dispatch_small_kernel(
    const float* z, int renorm, float* probs, float* __restrict__ topk_w, int* idx, int T, int k, int E,
    int e_lo, int E_loc, int C, int R_max, int* __restrict__ demand, int* __restrict__ offsets,
    int* __restrict__ slot_token, int* __restrict__ token_slot, void* y_zero, int y_esz, int H, TilePlanArgs plan,
    int zsplit) {
  extern __shared__ int sh[];
  dispatch_small_body<MODE, NTH>(sh, z, renorm, probs, topk_w, idx, T, k, E, e_lo, E_loc, C, R_max, demand, offsets,
                                 slot_token, token_slot, y_zero, y_esz, H, plan, zsplit);
}

// Gather x rows into the dispatched order (zero rows past the last one).
template <typename DT>
__global__ __launch_bounds__(256) void gather_rows_kernel(const typename DT::T* __restrict__ x,
                                                          const int* __restrict__ slot_token, int H,
                                                          typename DT::T* __restrict__ xd) {
  const int s = blockIdx.x;
  const int t = slot_token[s];
  const int nvec = H / DT::VEC;
  uint4* dst = reinterpret_cast<uint4*>(xd + (long long)s * H);
  if (t >= 0) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (long long)t * H);
    for (int c = threadIdx.x; c < nvec; c += 256) dst[c] = src[c];
  } else {
    for (int c = threadIdx.x; c < nvec; c += 256) dst[c] = make_uint4(0, 0, 0, 0);
  }
}

// -------------------------------------------------------------------- launchers
template <int NTH>
static size_t small_lds(int E) {
  return sizeof(int) * ((size_t)(NTH / MOE_WAVE) * (E + 1) + E + NTH + NTH / MOE_WAVE + 1 + tile_plan_lds_ints(NTH));
}
static TilePlanArgs plan_or_none(const TilePlanArgs* plan) {
  TilePlanArgs none{};
  return plan ? *plan : none;
}
size_t dispatch_small_lds(int E) { return small_lds<DISP_BLOCK>(E); }

template <int NTH>
static void launch_small_t(bool fuse_topk, const float* z, int renorm, float* probs, float* topk_w, int* idx, int T,
                           int k, int E, int e_lo, int E_loc, int C, int R_max, int* demand, int* offsets,
                           int* slot_token, int* token_slot, void* y_zero, int y_esz, int H,
                           const TilePlanArgs& plan, int zsplit, hipStream_t s) {
  const size_t lds = small_lds<NTH>(E);
  if (fuse_topk)
    hipLaunchKernelGGL((dispatch_small_kernel<1, NTH>), dim3(1), dim3(NTH), lds, s, z, renorm, probs, topk_w, idx, T,
                       k, E, e_lo, E_loc, C, R_max, demand, offsets, slot_token, token_slot, y_zero, y_esz, H, plan,
                       zsplit);
  else
    hipLaunchKernelGGL((dispatch_small_kernel<0, NTH>), dim3(1), dim3(NTH), lds, s, z, renorm, probs, topk_w, idx, T,
                       k, E, e_lo, E_loc, C, R_max, demand, offsets, slot_token, token_slot, y_zero, y_esz, H, plan,
                       zsplit);
}

// One block of 256 threads when the assignments and local experts fit, else 1024.
hipError_t launch_dispatch_small(bool fuse_topk, const float* z, int renorm, float* probs, float* topk_w,
                                 int* idx, int T, int k, int E, int e_lo, int E_loc, int C, int R_max,
                                 int* demand, int* offsets, int* slot_token, int* token_slot, void* y_zero,
                                 int y_esz, int H, const TilePlanArgs* plan, int zsplit, hipStream_t s) {
  if (T * k > DISP_BLOCK || E_loc > DISP_BLOCK) return hipErrorInvalidValue;
  const TilePlanArgs pl = plan_or_none(plan);
  if (zsplit < 1) zsplit = 1;
  if (T * k <= 256 && E_loc <= 256)
    launch_small_t<256>(fuse_topk, z, renorm, probs, topk_w, idx, T, k, E, e_lo, E_loc, C, R_max, demand, offsets,
                        slot_token, token_slot, y_zero, y_esz, H, pl, zsplit, s);
  else
    launch_small_t<DISP_BLOCK>(fuse_topk, z, renorm, probs, topk_w, idx, T, k, E, e_lo, E_loc, C, R_max, demand,
                               offsets, slot_token, token_slot, y_zero, y_esz, H, pl, zsplit, s);
  return hipGetLastError();
}

int dispatch_num_blocks(long long kT) { return (int)((kT + DISP_BLOCK - 1) / DISP_BLOCK); }
int dispatch_block_size() { return DISP_BLOCK; }

hipError_t launch_dispatch_multi(const int* idx, int T, int k, int E, int e_lo, int E_loc, int C, int R_max,
                                 int* rank, int* blk_hist, int* demand, int* offsets, int* slot_token,
                                 int* token_slot, void* y_zero, int y_esz, int H, const TilePlanArgs* plan,
                                 hipStream_t s) {
  const int nblk = dispatch_num_blocks((long long)T * k);
  const size_t lds = sizeof(int) * ((size_t)DISP_WAVES * (E + 1) + E);
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nblk), dim3(DISP_BLOCK), lds, s, idx, T, k, E, rank,
                     blk_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(DISP_BLOCK), 0, s, blk_hist, nblk, E, e_lo, E_loc,
                     C, demand, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const TilePlanArgs pl = plan_or_none(plan);
  const int nplan = (pl.list1 || pl.list2) ? std::max(1, pl.parts) : 0;   // blocks that write the tile lists
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nblk + nplan), dim3(DISP_BLOCK), 0, s, idx, rank, blk_hist, T,
                     k, E, e_lo, E_loc, C, offsets, R_max, slot_token, token_slot, y_zero, y_esz, H, nblk, nplan,
                     pl);
  return hipGetLastError();
}

bool route_dispatch_supported(long long kT) {
  return kT > DISP_BLOCK && kT <= (long long)ROUTE_MAX_BLOCKS * DISP_BLOCK;
}

size_t route_dispatch_lds(int E) {
  return sizeof(int) * ((size_t)DISP_WAVES * (E + 1) + 4 * (size_t)E + 1 + DISP_WAVES + 1 +
                        tile_plan_lds_ints(DISP_BLOCK));
}

hipError_t launch_route_dispatch(const RouteDispatchArgs& a, const TilePlanArgs* plan, hipStream_t s) {
  const long long kT = (long long)a.T * a.k;
  if (!route_dispatch_supported(kT) || a.E < 1 || a.E > DISP_BLOCK || a.E_loc > a.E || a.k < 1 || a.k > 2)
    return hipErrorInvalidValue;
  const int nsoft = (a.T + DISP_WAVES - 1) / DISP_WAVES;
  const int nblk = dispatch_num_blocks(kT);
  const TilePlanArgs pl = plan_or_none(plan);
  const int nplan = (pl.list1 || pl.list2) ? std::max(1, pl.parts) : 0;
  hipLaunchKernelGGL(route_dispatch_kernel, dim3(nsoft + nblk + nplan), dim3(DISP_BLOCK), route_dispatch_lds(a.E),
                     s, a, nsoft, nblk, nplan, pl);
  return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* x, const int* slot_token, int R_max, int H, void* xd,
                              hipStream_t s) {
  if (R_max <= 0) return hipSuccess;
  switch (dtype) {
    case DT_F32:
      hipLaunchKernelGGL(gather_rows_kernel<DtF32>, dim3(R_max), dim3(256), 0, s, (const float*)x, slot_token,
                         H, (float*)xd);
      break;
    case DT_F16:
      hipLaunchKernelGGL(gather_rows_kernel<DtF16>, dim3(R_max), dim3(256), 0, s, (const _Float16*)x,
                         slot_token, H, (_Float16*)xd);
      break;
    default:
      hipLaunchKernelGGL(gather_rows_kernel<DtBF16>, dim3(R_max), dim3(256), 0, s, (const __bf16*)x,
                         slot_token, H, (__bf16*)xd);
  }
  return hipGetLastError();
}

}  // namespace moe
