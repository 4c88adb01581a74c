// Expert FFN for segments of at most MAXM rows (decode-sized batches).
//
// With a handful of rows per expert the FFN is a stream over the active
// experts' weights: there is nothing for the matrix cores to reuse, so these
// kernels read each weight byte once with 16-byte non-temporal vector loads and
// do the arithmetic on the vector ALUs. Two launches, no barriers inside:
//
//   up    h[r, f] = GeLU(x_r . W1[f, :] + b1[f]), rounded to the I/O dtype
//   down  y[r, j] = h_r . W2[j, :] + b2[j]   (fp32), or, for a top-1 layer
//         without the dense MLP, the combine folded in: out[t, j] =
//         round(w_t * y[r, j]) with t the token of row r
//
// A wave owns RPW weight rows. Each lane loads its NQ 16-byte vectors of every
// row up front (all loads in flight at once), multiplies them with the
// segment's activation rows and a single multi-value wave reduction sums the
// RPW x MAXM dot products. Work-group g x c takes the g-th non-empty segment
// (found by each wave on its own from the offsets) and the c-th block of rows.
// Rows longer than 16 vectors per lane are split over 2 or 4 waves whose sums
// meet in LDS. A residual layer's dense MLP (all of the batch's rows) can ride
// in the same two launches as extra work-groups after the expert groups'.
#include <algorithm>

#include "common.h"
#include "dispatch_common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// The g-th non-empty segment of seg_off[0..nseg] (nseg <= 512), per wave. All
// offsets are loaded at once (clamped addresses, masked values, no branches).
__device__ inline bool find_active(const int* __restrict__ seg_off, int nseg, int g, int& seg, int& r0, int& r1) {
  const int lane = threadIdx.x & 63;
  int lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = min(i * 64 + lane, nseg - 1);
    lo[i] = seg_off[s];
    hi[i] = seg_off[s + 1];
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ne = (i * 64 + lane < nseg) && hi[i] > lo[i];
    const uint64_t bal = __ballot(ne);
    const int cnt = __popcll(bal);
    if (g < base + cnt) {
      const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
      const uint64_t pick = __ballot(ne && __popcll(below) == g - base);
      const int src = __ffsll((unsigned long long)pick) - 1;
      seg = i * 64 + src;
      r0 = __builtin_amdgcn_readlane(lo[i], src);   // (src is the same in every lane)
      r1 = __builtin_amdgcn_readlane(hi[i], src);
      return true;
    }
    base += cnt;
  }
  return false;
}

#ifndef DEC_WEIGHT_VECS
#define DEC_WEIGHT_VECS 16   // 16-byte weight vectors each lane holds in flight
#endif
template <int NQ, int MAXM>
struct DecRows {
  static constexpr int by_regs = (DEC_WEIGHT_VECS / NQ) > 0 ? DEC_WEIGHT_VECS / NQ : 1;
  static constexpr int by_red = 64 / MAXM;
  static constexpr int RPW = by_regs < by_red ? by_regs : by_red;    // weight rows per wave
};

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Issue every weight load of the wave: RPW rows of length K, NQ 16-byte vectors per lane.
template <typename DT, int NQ, int RPW>
__device__ inline void load_rows(uint4 (&wv)[RPW][NQ], const typename DT::T* __restrict__ wrow0, long long K) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      wv[i][q] = ld_nt16(wrow0 + (long long)i * K + (long long)(lane + 64 * q) * DT::VEC);
}

// Dot the wave's rows with MAXM activation rows and reduce: returns, in each
// lane, the sum for value v = lane >> (6 - log2(RPW * MAXM)) (row v / MAXM,
// activation v % MAXM).
template <typename DT, int MAXM, int NQ, int RPW>
__device__ inline float dot_rows(const uint4 (&wv)[RPW][NQ], const typename DT::T* const (&act)[MAXM]) {
  const int lane = threadIdx.x & 63;
  float acc[RPW * MAXM];
#pragma unroll
  for (int i = 0; i < RPW * MAXM; ++i) acc[i] = 0.f;
  if constexpr (MAXM * NQ <= 16) {
    // few activation vectors: load them all at once
    uint4 av[MAXM][NQ];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        av[m][q] = *reinterpret_cast<const uint4*>(act[m] + (long long)(lane + 64 * q) * DT::VEC);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float af[DT::VEC];
        unpack16<DT>(av[m][q], af);
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i * MAXM + m] = dot16f<DT>(wv[i][q], af, acc[i * MAXM + m]);
      }
    }
  } else {
    // many: one vector column q at a time
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      uint4 av[MAXM];
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        av[m] = *reinterpret_cast<const uint4*>(act[m] + (long long)(lane + 64 * q) * DT::VEC);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float af[DT::VEC];
        unpack16<DT>(av[m], af);
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i * MAXM + m] = dot16f<DT>(wv[i][q], af, acc[i * MAXM + m]);
      }
    }
  }
  return wave_reduce_multi<RPW * MAXM>(acc);
}

// Route a decode-sized batch (k*T <= 64) inside one work-group, entirely in LDS,
// in two phases so that the work-group's weight loads go out after the first:
//   phase 1: top-k of every token (one wave per token; work-group 0 also
//            computes the softmax weights); the expert of this work-group's
//            assignment a (rank-major a = j*T + t) is then known;
//   phase 2: with one thread per assignment b,
//            pos(b)  = earlier assignments to the same expert
//            kept(b) = local expert and pos(b) < C
//            slot(b) = kept assignments to lower local experts + pos(b)
//            which is the dispatch written out by direct counting (O(kT) per
//            thread, no scans). Assignment a leads its expert's segment when it
//            is kept with pos 0; the segment is rows [slot(a), slot(a) + kept
//            count of the expert). Work-group 0 also writes the routing out.
// Work-groups of assignments that do not lead a segment (duplicates of an
// expert, drops, non-local experts) end after phase 2; their weight loads, if
// any, read lines the leader reads too.
#ifndef UP_WAVES
#define UP_WAVES 8     // waves of a W1 work-group (W1 kernel 15.9 us against 17.1 with 4 and 16.6 with 16)
#endif
#ifndef DOWN_WAVES
#define DOWN_WAVES 8   // waves of a W2 work-group (W2 kernel 12.6 us against 12.8 with 4 and 12.7 with 2)
#endif
#define ROUTE_NTH (UP_WAVES * 64)
#define ROUTE_MAX_KT 64
__host__ __device__ inline size_t route_lds_ints(int T, int k, int R_max) {
  return 5 * (size_t)T * k + R_max + 4;
}

struct RouteLds {
  int* lidx;    // [T][k] chosen experts
  float* lw;    // [T][k] weights (work-group 0)
  int* lkey;    // [kT] rank-major keys (E = none)
  int* lpos;    // [kT] pos(b), or -1 when not kept
  int* lslot;   // [kT] slot(b) or -1
  int* lst;     // [R_max] slot -> token
  int* sinfo;   // seg, r0, r1, total
};

__device__ inline RouteLds route_lds(const RouteParams& rp, int* sh) {
  const int kT = rp.T * rp.k;
  RouteLds L;
  L.lidx = sh;
  L.lw = reinterpret_cast<float*>(L.lidx + kT);
  L.lkey = reinterpret_cast<int*>(L.lw + kT);
  L.lpos = L.lkey + kT;
  L.lslot = L.lpos + kT;
  L.lst = L.lslot + kT;
  L.sinfo = L.lst + rp.R_max;
  return L;
}

// Phase 1. Returns the local expert of assignment a, or -1 (a >= kT, non-local).
// all_weights: every work-group computes the softmax weights (in LDS), not only
// work-group 0.
__device__ inline int route_phase1(const RouteParams& rp, const RouteLds& L, int a, bool all_weights = false) {
  constexpr int NW = ROUTE_NTH / 64;
  const int E = rp.E, T = rp.T, k = rp.k;
  const int w = threadIdx.x >> 6;
  const bool writer = blockIdx.x == 0;
  for (int t = w; t < T; t += NW) {
    if (writer || all_weights) {
      int sel[2];
      wave_softmax_topk(rp.z + (long long)t * E, E, k, rp.renorm != 0, nullptr, L.lidx + t * k, L.lw + t * k, sel);
    } else {
      wave_topk_only(rp.z + (long long)t * E, E, k, L.lidx + t * k);
    }
  }
  __syncthreads();
  // retire every load of the top-k here (vmcnt 0): otherwise the paths with and
  // without weight loads merge with loads of unknown age in flight and phase 2
  // would wait for the weight loads too
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (a >= T * k) return -1;
  const int e = L.lidx[(a - (a / T) * T) * k + a / T];
  return (e >= rp.e_lo && e < rp.e_lo + rp.E_loc) ? e - rp.e_lo : -1;
}

// Phase 2. Returns false unless assignment a leads a segment; then seg, r0, r1
// and lst (slot -> token, in LDS).
__device__ inline bool route_phase2(const RouteParams& rp, const RouteLds& L, int H, int a, int& seg, int& r0,
                                    int& r1, const int*& lst_out) {
  const int E = rp.E, T = rp.T, k = rp.k, kT = T * k;
  const int tid = threadIdx.x;
  const bool writer = blockIdx.x == 0;
  if (tid == 0) L.sinfo[0] = -1;
  // keys in rank-major order
  int key = E;
  if (tid < kT) {
    const int j = tid / T, t = tid - (tid / T) * T;
    const int e = L.lidx[t * k + j];
    key = (e >= 0 && e < E) ? e : E;
    L.lkey[tid] = key;
  }
  __syncthreads();
  const bool local = key >= rp.e_lo && key < rp.e_lo + rp.E_loc;
  int pos = 0, cnt = 0;
  if (tid < kT) {
    for (int b = 0; b < kT; ++b) {
      const int kb = L.lkey[b];
      pos += (b < tid) & (kb == key);
      cnt += kb == key;
    }
    L.lpos[tid] = (local && pos < rp.C) ? pos : -1;
  }
  __syncthreads();
  if (tid < kT) {
    int slot = -1;
    if (L.lpos[tid] >= 0) {
      int below = 0;
      for (int b = 0; b < kT; ++b) below += (L.lpos[b] >= 0) & (L.lkey[b] < key);
      slot = below + pos;
      L.lst[slot] = tid - (tid / T) * T;
      if (tid == a && pos == 0) {               // this work-group's assignment leads its expert's segment
        L.sinfo[0] = key - rp.e_lo;
        L.sinfo[1] = below;
        L.sinfo[2] = below + min(cnt, rp.C);
      }
    }
    L.lslot[tid] = slot;
  }
  if (tid == 0) {
    int total = 0;
    for (int b = 0; b < kT; ++b) total += L.lpos[b] >= 0;
    L.sinfo[3] = total;
  }
  __syncthreads();
  if (writer) {
    const int total = L.sinfo[3];
    for (int b = tid; b < kT; b += ROUTE_NTH) {
      const int j = b / T, t = b - (b / T) * T;
      rp.idx[t * k + j] = L.lidx[t * k + j];
      rp.w[t * k + j] = L.lw[t * k + j];
      rp.token_slot[t * k + j] = L.lslot[b];
    }
    for (int e = tid; e < E; e += ROUTE_NTH) {
      int c = 0;
      for (int b = 0; b < kT; ++b) c += L.lkey[b] == e;
      rp.demand[e] = c;
    }
    for (int i = tid; i <= rp.E_loc; i += ROUTE_NTH) {
      int c = 0;
      for (int b = 0; b < kT; ++b) c += (L.lpos[b] >= 0) & (L.lkey[b] < rp.e_lo + i);
      rp.offsets[i] = c;
    }
    for (int s2 = tid; s2 < rp.R_max; s2 += ROUTE_NTH) rp.slot_token[s2] = s2 < total ? L.lst[s2] : -1;
    if (rp.y_zero) {
      for (int tt = tid; tt < T; tt += ROUTE_NTH) {
        bool any = false;
        for (int jj = 0; jj < k; ++jj) any |= L.lslot[jj * T + tt] >= 0;
        if (!any) zero_dropped(rp.y_zero, rp.y_esz, tt, H);
      }
    }
  }
  seg = L.sinfo[0];
  r0 = L.sinfo[1];
  r1 = L.sinfo[2];
  lst_out = L.lst;
  return seg >= 0;
}

// Loads whose address space the compiler cannot see through a pointer table or
// a pointer that may hold LDS are stated explicitly: a flat load also counts
// against lgkmcnt, and waiting for it would drain the weight loads in flight.
template <typename X>
__device__ inline X gload(const X* p) { return *(const __attribute__((address_space(1))) X*)p; }
__device__ inline int lds_load(const int* p) { return *(const __attribute__((address_space(3))) int*)p; }

// Every small load a work-group's epilogue needs (activation row indices, bias,
// the row's token and gate weight) is issued before or with the weight loads,
// so only the weight stream itself is left to wait for.
// KS waves share a block of weight rows, each taking 1 / KS of K (NQ vectors
// per lane per row), and add their sums through LDS in wave order: rows longer
// than 16 vectors per lane (K = 16384 or 32768 at 2-byte weights) keep the
// registers and loads in flight of one wave at K = 8192.
template <int KS, int NW>
__device__ inline float ksplit_sum(float s, int wave, int lane, bool& keep) {
  keep = true;
  if constexpr (KS > 1) {
    __shared__ float red[NW][64];
    red[wave][lane] = s;
    __syncthreads();
    keep = (wave % KS) == 0;
    float t = red[wave][lane];
#pragma unroll
    for (int i = 1; i < KS; ++i) t += red[wave + (keep ? i : 0)][lane];
    return t;
  }
  return s;
}

// The dense segment's work-groups (the residual MLP over the dM <= 8 rows of
// x, all of them at once: 8 activation rows per weight row, rows past dM
// repeat row 0 and are not stored). Chunk c covers the weight rows of one
// work-group, as for an expert segment.
#define DENSE_MAXM 8
template <typename DT, int NQ, int KS>
__device__ inline void dense_up_wg(const DecodeParams& p, int chunk) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, DENSE_MAXM>::RPW;
  constexpr int SH = 6 - ilog2(RPW * DENSE_MAXM);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long H = p.H, F = p.F;
  const int f0 = chunk * (UP_WAVES / KS) * RPW + (wave / KS) * RPW;
  const long long kofs = (long long)(wave % KS) * (H / KS);
  const int v = lane >> SH;
  const int oi = v / DENSE_MAXM, om = v - (v / DENSE_MAXM) * DENSE_MAXM;
  uint4 wv[RPW][NQ];
  load_rows<DT, NQ, RPW>(wv, reinterpret_cast<const T*>(p.dw1) + (long long)f0 * H + kofs, H);
  const T bias_raw = gload(reinterpret_cast<const T*>(p.db1) + f0 + oi);
  __builtin_amdgcn_sched_barrier(0);
  const int M = min(p.dM, DENSE_MAXM);
  const T* x = reinterpret_cast<const T*>(p.x);
  const T* act[DENSE_MAXM];
#pragma unroll
  for (int m = 0; m < DENSE_MAXM; ++m) act[m] = x + (long long)(m < M ? m : 0) * H + kofs;
  bool keep;
  const float s = ksplit_sum<KS, UP_WAVES>(dot_rows<DT, DENSE_MAXM, NQ, RPW>(wv, act), wave, lane, keep);
  if (keep && (lane & ((1 << SH) - 1)) == 0 && om < M)
    reinterpret_cast<T*>(p.dh)[(long long)om * F + f0 + oi] =
        DT::from_f(pin_f32(gelu_erf(s + DT::to_f(bias_raw))));
}

template <typename DT, int NQ, int KS>
__device__ inline void dense_down_wg(const DecodeParams& p, int chunk) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, DENSE_MAXM>::RPW;
  constexpr int SH = 6 - ilog2(RPW * DENSE_MAXM);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long H = p.H, F = p.F;
  const int j0 = chunk * (DOWN_WAVES / KS) * RPW + (wave / KS) * RPW;
  const long long kofs = (long long)(wave % KS) * (F / KS);
  const int v = lane >> SH;
  const int oi = v / DENSE_MAXM, om = v - (v / DENSE_MAXM) * DENSE_MAXM;
  uint4 wv[RPW][NQ];
  load_rows<DT, NQ, RPW>(wv, reinterpret_cast<const T*>(p.dw2) + (long long)j0 * F + kofs, F);
  const T bias_raw = gload(reinterpret_cast<const T*>(p.db2) + j0 + oi);
  __builtin_amdgcn_sched_barrier(0);
  const int M = min(p.dM, DENSE_MAXM);
  const T* h = reinterpret_cast<const T*>(p.dh);
  const T* act[DENSE_MAXM];
#pragma unroll
  for (int m = 0; m < DENSE_MAXM; ++m) act[m] = h + (long long)(m < M ? m : 0) * F + kofs;
  bool keep;
  const float s = ksplit_sum<KS, DOWN_WAVES>(dot_rows<DT, DENSE_MAXM, NQ, RPW>(wv, act), wave, lane, keep);
  if (keep && (lane & ((1 << SH) - 1)) == 0 && om < M)
    p.dout[(long long)om * H + j0 + oi] = s + DT::to_f(bias_raw);
}

template <typename DT, int MAXM, int NQ, int KS, bool DENSE>
__global__ __launch_bounds__(UP_WAVES * 64) void decode_up_kernel(RouteParams rp, DecodeParams p) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  constexpr int N = RPW * MAXM;
  constexpr int SH = 6 - ilog2(N);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = p.F / ((UP_WAVES / KS) * RPW);
  if constexpr (DENSE) {   // the dense segment's work-groups follow the expert groups'
    const int nexp = p.ngroups * nchunk;
    if ((int)blockIdx.x >= nexp) {
      dense_up_wg<DT, NQ, KS>(p, (int)blockIdx.x - nexp);
      return;
    }
  }
  const int g = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - g * nchunk;
  const long long H = p.H, F = p.F;
  const int f0 = chunk * (UP_WAVES / KS) * RPW + (wave / KS) * RPW;
  const long long kofs = (long long)(wave % KS) * (H / KS);   // this wave's share of K
  // after the reduction lane l holds value v = l >> SH: weight row f0 + oi, activation row om
  const int v = lane >> SH;
  const int oi = v / MAXM, om = v - (v / MAXM) * MAXM;
  uint4 wv[RPW][NQ];
  int rows[MAXM];
  T bias_raw = DT::from_f(0.f);
  int seg = 0, r0 = 0, r1 = p.M;
  if (rp.z) {
    // routed here: work-group g serves assignment g; its weight loads go out as
    // soon as the expert of g is known, the rest of the routing runs under them
    extern __shared__ int route_sh[];
    const RouteLds L = route_lds(rp, route_sh);
    const int e = route_phase1(rp, L, g);
    if (e >= 0) {
      const T* w1s = p.w1p ? reinterpret_cast<const T*>(p.w1p[e]) : reinterpret_cast<const T*>(p.w1) + (long long)e * F * H;
      const T* b1s = p.b1p ? reinterpret_cast<const T*>(p.b1p[e]) : reinterpret_cast<const T*>(p.b1) + (long long)e * F;
      load_rows<DT, NQ, RPW>(wv, w1s + (long long)f0 * H + kofs, H);
      bias_raw = gload(b1s + f0 + oi);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int* lst;
    if (!route_phase2(rp, L, p.H, g, seg, r0, r1, lst)) return;   // leads a segment: seg == e
    const int M = min(r1 - r0, MAXM);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) rows[m] = lds_load(lst + r0 + (m < M ? m : 0));
  } else {
    if (p.seg_off) {
      if (!find_active(p.seg_off, p.nseg, g, seg, r0, r1)) return;
    } else if (g > 0) {
      return;
    }
    const int M = min(r1 - r0, MAXM);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const int r = r0 + (m < M ? m : 0);
      rows[m] = p.a_rows ? gload(p.a_rows + r) : r;
    }
    const T* w1s = p.w1p ? reinterpret_cast<const T*>(p.w1p[seg]) : reinterpret_cast<const T*>(p.w1) + (long long)seg * F * H;
    const T* b1s = p.b1p ? reinterpret_cast<const T*>(p.b1p[seg]) : reinterpret_cast<const T*>(p.b1) + (long long)seg * F;
    bias_raw = gload(b1s + f0 + oi);
    load_rows<DT, NQ, RPW>(wv, w1s + (long long)f0 * H + kofs, H);
    __builtin_amdgcn_sched_barrier(0);   // every weight load is in flight before anything else
  }
  const int M = min(r1 - r0, MAXM);
  const T* x = reinterpret_cast<const T*>(p.x);
  const T* act[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) act[m] = x + (long long)rows[m] * H + kofs;
  bool keep;
  const float s = ksplit_sum<KS, UP_WAVES>(dot_rows<DT, MAXM, NQ, RPW>(wv, act), wave, lane, keep);
  if (keep && (lane & ((1 << SH) - 1)) == 0 && om < M) {
    const float u = s + DT::to_f(bias_raw);
    reinterpret_cast<T*>(p.h)[(long long)(r0 + om) * F + f0 + oi] = DT::from_f(pin_f32(gelu_erf(u)));
  }
}

template <typename DT, int MAXM, int NQ, bool FUSE, int KS, bool DENSE>
__global__ __launch_bounds__(DOWN_WAVES * 64) void decode_down_kernel(DecodeParams p) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  constexpr int N = RPW * MAXM;
  constexpr int SH = 6 - ilog2(N);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = p.H / ((DOWN_WAVES / KS) * RPW);
  if constexpr (DENSE) {   // the dense segment's work-groups follow the expert groups'
    const int nexp = p.ngroups * nchunk;
    if ((int)blockIdx.x >= nexp) {
      dense_down_wg<DT, NQ, KS>(p, (int)blockIdx.x - nexp);
      return;
    }
  }
  const int g = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - g * nchunk;
  int seg = 0, r0 = 0, r1 = p.M;
  if (p.seg_off) {
    if (!find_active(p.seg_off, p.nseg, g, seg, r0, r1)) return;
  } else if (g > 0) {
    return;
  }
  const long long H = p.H, F = p.F;
  const int j0 = chunk * (DOWN_WAVES / KS) * RPW + (wave / KS) * RPW;
  const long long kofs = (long long)(wave % KS) * (F / KS);   // this wave's share of K
  const int M = min(r1 - r0, MAXM);
  const int v = lane >> SH;
  const int oi = v / MAXM, om = v - (v / MAXM) * MAXM;
  const T* b2s = p.b2p ? reinterpret_cast<const T*>(p.b2p[seg]) : reinterpret_cast<const T*>(p.b2) + (long long)seg * H;
  const T bias_raw = gload(b2s + j0 + oi);
  int t_out = 0;
  if (FUSE) t_out = gload(p.slot_token + r0 + (om < M ? om : M - 1));   // a kept row: a token
  uint4 wv[RPW][NQ];
  const T* w2s = p.w2p ? reinterpret_cast<const T*>(p.w2p[seg]) : reinterpret_cast<const T*>(p.w2) + (long long)seg * H * F;
  load_rows<DT, NQ, RPW>(wv, w2s + (long long)j0 * F + kofs, F);
  __builtin_amdgcn_sched_barrier(0);
  float wt = 0.f;
  if (FUSE) {   // issued here, not after the dot: the token is back long before the weights
    wt = gload(p.topk_w + t_out);
    __builtin_amdgcn_sched_barrier(0);
  }
  const T* h = reinterpret_cast<const T*>(p.h);
  const T* act[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) act[m] = h + (long long)(r0 + (m < M ? m : 0)) * F + kofs;
  bool keep;
  const float s = ksplit_sum<KS, DOWN_WAVES>(dot_rows<DT, MAXM, NQ, RPW>(wv, act), wave, lane, keep);
  if (keep && (lane & ((1 << SH) - 1)) == 0 && om < M) {
    const float yv = s + DT::to_f(bias_raw);
    if (FUSE) {
      reinterpret_cast<T*>(p.out)[(long long)t_out * H + j0 + oi] = DT::from_f(pin_f32(fmaf(wt, yv, 0.f)));
    } else {
      reinterpret_cast<float*>(p.out)[(long long)(r0 + om) * H + j0 + oi] = yv;
    }
  }
}

// ---------------------------------------------------------------- one launch for both products
// Cache-policy bit of buffer loads and stores (gfx950): sc1 = agent scope. Such
// a store is written through the L2 of its XCD and such a load is served past
// it, so data handed from one work-group to another inside a launch never meets
// a stale line in another XCD's L2 (the same bit the compiler sets on relaxed
// agent-scope atomic loads and stores).
#define MOE_CPOL_AGENT 16
// Give-up time of the wait for another work-group's hidden rows: 50 ms of the
// 100 MHz real-time counter (a launch normally waits a few microseconds).
#define MOE_WAIT_TICKS 5000000ull

__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// Dot products of the wave's rows with MAXM activation rows held in LDS (row m
// at act + m * ld); same accumulation order as dot_rows.
template <typename DT, int MAXM, int NQ, int RPW>
__device__ inline float dot_rows_lds(const uint4 (&wv)[RPW][NQ],
                                     const __attribute__((address_space(3))) typename DT::T* act, int ld) {
  const int lane = threadIdx.x & 63;
  float acc[RPW * MAXM];
#pragma unroll
  for (int i = 0; i < RPW * MAXM; ++i) acc[i] = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const uint4 av = __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                                                     act + m * ld + (lane + 64 * q) * DT::VEC));
      float af[DT::VEC];
      unpack16<DT>(av, af);
#pragma unroll
      for (int i = 0; i < RPW; ++i) acc[i * MAXM + m] = dot16f<DT>(wv[i][q], af, acc[i * MAXM + m]);
    }
  }
  return wave_reduce_multi<RPW * MAXM>(acc);
}

// A 16-bit element still holding the fill pattern 0xFFFF (a NaN the layer never
// produces: NaN inputs are outside the layer's contract) has not been written.
__device__ inline bool has_unwritten(const uint4& v) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  bool u = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) u |= (w[i] & 0xFFFFu) == 0xFFFFu || (w[i] >> 16) == 0xFFFFu;
  return u;
}

// The expert FFN of a decode-sized batch in one launch. Work-group (g, c)
// routes the batch (as decode_up_kernel), streams chunk c of W1 of the expert
// whose segment assignment g leads and stores its part of h (agent-scope
// stores, written through to memory), then streams chunk c of W2 without
// waiting for anything. h starts out filled with 0xFFFF (the gate kernel of the
// same forward fills it), and every element is written once by one 2-byte
// store, so a 16-byte agent-scope load that finds no 0xFFFF element holds final
// values: each wave loads its share of the segment's h rows right behind its
// W2 loads, reloads any vector still unwritten, and the work-group assembles
// the rows in LDS for the second product. The W2 stream thus follows the W1
// stream inside one launch, and no work-group waits for a flag. Only groups
// that lead a segment read h, and every work-group writes its chunk before it
// reads, so the launch completes whatever the occupancy; a wait that outlasts
// MOE_WAIT_TICKS gives up and writes NaN, so no launch can hang.
// FUSE: top-1 combine folded in (writes y), else y_disp rows in fp32.
template <typename DT, int MAXM, int NQ1, int NQ2, bool FUSE>
__global__ __launch_bounds__(UP_WAVES * 64) void decode_fused_kernel(DecodeParams p, RouteParams rp, int nch,
                                                                     int h_lds_off) {
  using T = typename DT::T;
  constexpr int RPW1 = DecRows<NQ1, MAXM>::RPW;
  constexpr int RPW2 = DecRows<NQ2, MAXM>::RPW;
  constexpr int SH1 = 6 - ilog2(RPW1 * MAXM);
  constexpr int SH2 = 6 - ilog2(RPW2 * MAXM);
  constexpr int WVEC = NQ2 * 64 / UP_WAVES;   // 16-byte vectors of an h row each wave loads
  constexpr int HV = (WVEC + 63) / 64;        // ... per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = blockIdx.x / nch;
  const int c = blockIdx.x - g * nch;
  const long long H = p.H, F = p.F;
  const int nch1 = p.F / (UP_WAVES * RPW1);
  const int nch2 = p.H / (UP_WAVES * RPW2);
  const bool do1 = c < nch1, do2 = c < nch2;
  extern __shared__ int route_sh[];
  const RouteLds L = route_lds(rp, route_sh);
  __attribute__((address_space(3))) T* hs =
      reinterpret_cast<__attribute__((address_space(3))) T*>(
          reinterpret_cast<__attribute__((address_space(3))) char*>(
              (__attribute__((address_space(3))) int*)route_sh) + h_lds_off);
  __shared__ int wait_ok;

  // ---- routing; this group's W1 loads go out as soon as its expert is known
  const int f0 = c * UP_WAVES * RPW1 + wave * RPW1;
  const int v1 = lane >> SH1;
  const int oi1 = v1 / MAXM, om1 = v1 - (v1 / MAXM) * MAXM;
  uint4 wv1[RPW1][NQ1];
  T b1raw = DT::from_f(0.f);
  const int e = route_phase1(rp, L, g, FUSE);
  if (e >= 0 && do1) {
    const T* w1s = p.w1p ? reinterpret_cast<const T*>(p.w1p[e]) : reinterpret_cast<const T*>(p.w1) + (long long)e * F * H;
    const T* b1s = p.b1p ? reinterpret_cast<const T*>(p.b1p[e]) : reinterpret_cast<const T*>(p.b1) + (long long)e * F;
    load_rows<DT, NQ1, RPW1>(wv1, w1s + (long long)f0 * H, H);
    b1raw = gload(b1s + f0 + oi1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (threadIdx.x == 0) wait_ok = 1;   // (published by the barriers of route_phase2)
  int seg, r0, r1;
  const int* lst;
  if (!route_phase2(rp, L, p.H, g, seg, r0, r1, lst)) return;   // leads a segment: seg == e
  const int M = min(r1 - r0, MAXM);
  const __amdgpu_buffer_rsrc_t h_rsrc = raw_rsrc(p.h);

  // ---- first product: this chunk of h = GeLU(x W1^T + b1), stored past the L2s
  if (do1) {
    // activation rows of the segment: loads issued before the weights are waited for
    int rows[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) rows[m] = lds_load(lst + r0 + (m < M ? m : 0));
    const T* x = reinterpret_cast<const T*>(p.x);
    uint4 av[MAXM][NQ1];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
      for (int q = 0; q < NQ1; ++q)
        av[m][q] = __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4_t*)(
                                                 x + (long long)rows[m] * H + (long long)(lane + 64 * q) * DT::VEC));
    // the weights become opaque here: otherwise the compiler starts converting
    // them to fp32 right after their loads, which waits for them before the
    // routing above and holds twice the registers
#pragma unroll
    for (int i = 0; i < RPW1; ++i)
#pragma unroll
      for (int q = 0; q < NQ1; ++q) {
        u32x4_t t = __builtin_bit_cast(u32x4_t, wv1[i][q]);
        asm volatile("" : "+v"(t));
        wv1[i][q] = __builtin_bit_cast(uint4, t);
      }
    {
      unsigned short b = __builtin_bit_cast(unsigned short, b1raw);
      asm volatile("" : "+v"(b));
      b1raw = __builtin_bit_cast(T, b);
    }
    float acc[RPW1 * MAXM];
#pragma unroll
    for (int i = 0; i < RPW1 * MAXM; ++i) acc[i] = 0.f;
#pragma unroll
    for (int q = 0; q < NQ1; ++q)
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float af[DT::VEC];
        unpack16<DT>(av[m][q], af);
#pragma unroll
        for (int i = 0; i < RPW1; ++i) acc[i * MAXM + m] = dot16f<DT>(wv1[i][q], af, acc[i * MAXM + m]);
      }
    const float s1 = wave_reduce_multi<RPW1 * MAXM>(acc);
    if ((lane & ((1 << SH1) - 1)) == 0 && om1 < M) {
      const T hv = DT::from_f(pin_f32(gelu_erf(s1 + DT::to_f(b1raw))));
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hv), h_rsrc,
                                            (int)(((long long)(r0 + om1) * F + f0 + oi1) * 2), 0, MOE_CPOL_AGENT);
    }
  }

  // ---- second product: W2 loads first, then this wave's share of the h rows
  const int j0 = c * UP_WAVES * RPW2 + wave * RPW2;
  const int v2 = lane >> SH2;
  const int oi2 = v2 / MAXM, om2 = v2 - (v2 / MAXM) * MAXM;
  uint4 wv2[RPW2][NQ2];
  T b2raw = DT::from_f(0.f);
  if (do2) {
    const T* w2s = p.w2p ? reinterpret_cast<const T*>(p.w2p[seg]) : reinterpret_cast<const T*>(p.w2) + (long long)seg * H * F;
    const T* b2s = p.b2p ? reinterpret_cast<const T*>(p.b2p[seg]) : reinterpret_cast<const T*>(p.b2) + (long long)seg * H;
    load_rows<DT, NQ2, RPW2>(wv2, w2s + (long long)j0 * F, F);
    b2raw = gload(b2s + j0 + oi2);
    __builtin_amdgcn_sched_barrier(0);
  }
  // vector u of row m: elements (wave * WVEC + u * 64 + lane) * VEC .. + VEC - 1
  uint4 hv[MAXM][HV];
  auto h_off = [&](int m, int u) {
    return (int)(((long long)(r0 + m) * F + (long long)(wave * WVEC + u * 64 + lane) * DT::VEC) * 2);
  };
  auto h_mine = [&](int m, int u) { return m < M && u * 64 + lane < WVEC; };
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int u = 0; u < HV; ++u)
      if (h_mine(m, u))
        hv[m][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(h_rsrc, h_off(m, u), 0,
                                                                                   MOE_CPOL_AGENT));
  {
    // normally every element is written by now (its producer's W1 data came
    // in before this wave's W2 data); reload whatever is not
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      bool miss = false;
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int u = 0; u < HV; ++u) miss |= h_mine(m, u) && has_unwritten(hv[m][u]);
      if (__ballot(miss) == 0) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > MOE_WAIT_TICKS) {
        if (lane == 0) wait_ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int u = 0; u < HV; ++u)
          if (h_mine(m, u) && has_unwritten(hv[m][u]))
            hv[m][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(h_rsrc, h_off(m, u), 0,
                                                                                       MOE_CPOL_AGENT));
    }
  }
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int u = 0; u < HV; ++u)
      if (h_mine(m, u))
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(
            hs + (long long)m * F + (long long)(wave * WVEC + u * 64 + lane) * DT::VEC) =
            __builtin_bit_cast(u32x4_t, hv[m][u]);
  __syncthreads();
  if (!do2) return;
#pragma unroll
  for (int i = 0; i < RPW2; ++i)
#pragma unroll
    for (int q = 0; q < NQ2; ++q) {   // (as for W1: no conversion before the loads are needed)
      u32x4_t t = __builtin_bit_cast(u32x4_t, wv2[i][q]);
      asm volatile("" : "+v"(t));
      wv2[i][q] = __builtin_bit_cast(uint4, t);
    }
  {
    unsigned short b = __builtin_bit_cast(unsigned short, b2raw);
    asm volatile("" : "+v"(b));
    b2raw = __builtin_bit_cast(T, b);
  }
  const float s2 = dot_rows_lds<DT, MAXM, NQ2, RPW2>(wv2, hs, (int)F);
  if ((lane & ((1 << SH2) - 1)) == 0 && om2 < M) {
    const float yv = wait_ok ? s2 + DT::to_f(b2raw) : __builtin_nanf("");
    if constexpr (FUSE) {
      const int t_out = lds_load(lst + r0 + om2);
      const float wt = __builtin_bit_cast(float, lds_load(reinterpret_cast<const int*>(L.lw) + t_out));
      reinterpret_cast<T*>(p.out)[(long long)t_out * H + j0 + oi2] = DT::from_f(pin_f32(fmaf(wt, yv, 0.f)));
    } else {
      reinterpret_cast<float*>(p.out)[(long long)(r0 + om2) * H + j0 + oi2] = yv;
    }
  }
}

// ---------------------------------------------------------------- launchers
static int nq_of(int K, int vec) { return K / (64 * vec); }

struct LaunchEv {
  hipEvent_t start, stop;
};

// (p.dM > 0: the dense segment's work-groups are appended to the grid)
template <typename DT, int MAXM, int NQ, int KS>
static hipError_t launch_up_t(const DecodeParams& p, const RouteParams& rp, int grid_segs, hipStream_t s,
                              LaunchEv ev) {
  constexpr int RPW = DecRows<NQ, MAXM>::RPW, RPWD = DecRows<NQ, DENSE_MAXM>::RPW;
  const int grid = grid_segs * (p.F / ((UP_WAVES / KS) * RPW));
  const size_t lds = rp.z ? sizeof(int) * route_lds_ints(rp.T, rp.k, rp.R_max) : 0;
  if (p.dM > 0) {
    DecodeParams q = p;
    q.ngroups = grid_segs;
    const int gd = grid + p.F / ((UP_WAVES / KS) * RPWD);
    MOE_LAUNCH((decode_up_kernel<DT, MAXM, NQ, KS, true>), dim3(gd), dim3(UP_WAVES * 64), lds, s, ev.start, ev.stop,
               rp, q);
  } else {
    MOE_LAUNCH((decode_up_kernel<DT, MAXM, NQ, KS, false>), dim3(grid), dim3(UP_WAVES * 64), lds, s, ev.start,
               ev.stop, rp, p);
  }
  return hipGetLastError();
}

template <typename DT, int MAXM, int NQ, int KS>
static hipError_t launch_down_t(const DecodeParams& p, int grid_segs, bool fuse, hipStream_t s, LaunchEv ev) {
  constexpr int RPW = DecRows<NQ, MAXM>::RPW, RPWD = DecRows<NQ, DENSE_MAXM>::RPW;
  const int grid = grid_segs * (p.H / ((DOWN_WAVES / KS) * RPW));
  if (p.dM > 0) {   // (the dense output is added by the combine kernel: no folded combine here)
    if (fuse) return hipErrorInvalidValue;
    DecodeParams q = p;
    q.ngroups = grid_segs;
    const int gd = grid + p.H / ((DOWN_WAVES / KS) * RPWD);
    MOE_LAUNCH((decode_down_kernel<DT, MAXM, NQ, false, KS, true>), dim3(gd), dim3(DOWN_WAVES * 64), 0, s,
               ev.start, ev.stop, q);
  } else if (fuse) {
    MOE_LAUNCH((decode_down_kernel<DT, MAXM, NQ, true, KS, false>), dim3(grid), dim3(DOWN_WAVES * 64), 0, s,
               ev.start, ev.stop, p);
  } else {
    MOE_LAUNCH((decode_down_kernel<DT, MAXM, NQ, false, KS, false>), dim3(grid), dim3(DOWN_WAVES * 64), 0, s,
               ev.start, ev.stop, p);
  }
  return hipGetLastError();
}

// K = 512 q at 2-byte weights: q <= 16 vectors per lane per row in one wave;
// q = 32 / 64 split over 2 / 4 waves of 16 vectors each
template <typename DT, int MAXM>
static hipError_t launch_m(bool up, const DecodeParams& p, const RouteParams& rp, int grid_segs, bool fuse,
                           hipStream_t s, LaunchEv ev) {
  const int nq = up ? nq_of(p.H, DT::VEC) : nq_of(p.F, DT::VEC);
  switch (nq) {
#define CASE(Q, NQ, KS)                                                                              \
  case Q:                                                                                            \
    return up ? launch_up_t<DT, MAXM, NQ, KS>(p, rp, grid_segs, s, ev)                               \
              : launch_down_t<DT, MAXM, NQ, KS>(p, grid_segs, fuse, s, ev);
    CASE(1, 1, 1) CASE(2, 2, 1) CASE(4, 4, 1) CASE(8, 8, 1) CASE(16, 16, 1) CASE(32, 16, 2) CASE(64, 16, 4)
#undef CASE
  }
  return hipErrorInvalidValue;
}

template <typename DT>
static hipError_t launch_dt(bool up, int maxm, const DecodeParams& p, const RouteParams& rp, int grid_segs, bool fuse,
                            hipStream_t s, LaunchEv ev) {
  switch (maxm) {
    case 1: return launch_m<DT, 1>(up, p, rp, grid_segs, fuse, s, ev);
    case 2: return launch_m<DT, 2>(up, p, rp, grid_segs, fuse, s, ev);
    case 4: return launch_m<DT, 4>(up, p, rp, grid_segs, fuse, s, ev);
    case 8: return launch_m<DT, 8>(up, p, rp, grid_segs, fuse, s, ev);
  }
  return hipErrorInvalidValue;
}

template <typename DT, int MAXM, int NQ1, int NQ2>
static hipError_t launch_fused_t(const DecodeParams& p, const RouteParams& rp, int grid_segs, bool fuse,
                                 hipStream_t s, LaunchEv ev) {
  constexpr int RPW1 = DecRows<NQ1, MAXM>::RPW, RPW2 = DecRows<NQ2, MAXM>::RPW;
  const int nch = std::max(p.F / (UP_WAVES * RPW1), p.H / (UP_WAVES * RPW2));
  const int grid = grid_segs * nch;
  const int h_off = (int)((sizeof(int) * route_lds_ints(rp.T, rp.k, rp.R_max) + 15) / 16 * 16);
  const size_t lds = (size_t)h_off + (size_t)MAXM * p.F * sizeof(typename DT::T);
  if (fuse)
    MOE_LAUNCH((decode_fused_kernel<DT, MAXM, NQ1, NQ2, true>), dim3(grid), dim3(UP_WAVES * 64), lds, s, ev.start,
               ev.stop, p, rp, nch, h_off);
  else
    MOE_LAUNCH((decode_fused_kernel<DT, MAXM, NQ1, NQ2, false>), dim3(grid), dim3(UP_WAVES * 64), lds, s, ev.start,
               ev.stop, p, rp, nch, h_off);
  return hipGetLastError();
}

template <typename DT, int MAXM>
static hipError_t launch_fused_m(const DecodeParams& p, const RouteParams& rp, int grid_segs, bool fuse,
                                 hipStream_t s, LaunchEv ev) {
  const int nq1 = nq_of(p.H, DT::VEC), nq2 = nq_of(p.F, DT::VEC);
#define FCASE(Q1, Q2) \
  if (nq1 == Q1 && nq2 == Q2) return launch_fused_t<DT, MAXM, Q1, Q2>(p, rp, grid_segs, fuse, s, ev);
  FCASE(1, 4) FCASE(2, 8) FCASE(4, 16) FCASE(1, 2) FCASE(2, 4) FCASE(4, 8) FCASE(1, 1) FCASE(2, 2) FCASE(4, 4)
#undef FCASE
  return hipErrorInvalidValue;
}

// Shapes the one-launch decode kernel is built for: H and F from the streaming
// kernels' set with F / H in {1, 2, 4} (F = 4H is the pages' model shape), and
// the staged h rows (MAXM x F in the I/O dtype) within 32 KB of LDS.
bool decode_fused_supported(int dtype, int H, int F, int maxm) {
  if (dtype == DT_F32 || !decode_supported(dtype, H, F)) return false;
  if (!(F == H || F == 2 * H || F == 4 * H) || H > 2048) return false;
  if (maxm != 1 && maxm != 2 && maxm != 4 && maxm != 8) return false;
  return (long long)maxm * F * 2 <= 32768;
}

hipError_t launch_decode_fused(int dtype, int maxm, const DecodeParams& p, const RouteParams& rp, int grid_segs,
                               bool fuse_combine, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (grid_segs <= 0) return hipSuccess;
  if (!rp.z || (fuse_combine && !p.out)) return hipErrorInvalidValue;
  if (!decode_fused_supported(dtype, p.H, p.F, maxm)) return hipErrorInvalidValue;
  const LaunchEv ev{ev0, ev1};
#define FM(DT_)                                                                            \
  switch (maxm) {                                                                          \
    case 1: return launch_fused_m<DT_, 1>(p, rp, grid_segs, fuse_combine, s, ev);   \
    case 2: return launch_fused_m<DT_, 2>(p, rp, grid_segs, fuse_combine, s, ev);   \
    case 4: return launch_fused_m<DT_, 4>(p, rp, grid_segs, fuse_combine, s, ev);   \
    case 8: return launch_fused_m<DT_, 8>(p, rp, grid_segs, fuse_combine, s, ev);   \
  }
  if (dtype == DT_F16) {
    FM(DtF16)
  } else {
    FM(DtBF16)
  }
#undef FM
  return hipErrorInvalidValue;
}

bool decode_supported(int dtype, int H, int F) {
  if (dtype == DT_F32) return false;
  auto ok = [](int K) {
    if (K % 512) return false;
    const int q = K / 512;
    return q == 1 || q == 2 || q == 4 || q == 8 || q == 16 || q == 32 || q == 64;
  };
  return ok(H) && ok(F);
}

// Work-groups of the larger of the two decode expert launches (groups_up /
// groups_down segment groups): rows / (rows per work-group), with the K split
// the row length asks for.
long long decode_max_workgroups(int dtype, int H, int F, int maxm, long long groups_up, long long groups_down) {
  const int vec = dtype == DT_F32 ? 4 : 8;
  auto rows_per_wg = [&](int K, int waves) {
    int nq = K / (64 * vec), ks = 1;
    while (nq > 16) { nq /= 2; ks *= 2; }
    const int by_regs = std::max(DEC_WEIGHT_VECS / nq, 1), by_red = 64 / std::max(maxm, 1);
    return (long long)(waves / ks) * std::min(by_regs, by_red);
  };
  const long long up = groups_up * (F / rows_per_wg(H, UP_WAVES));
  const long long down = groups_down * (H / rows_per_wg(F, DOWN_WAVES));
  return std::max(up, down);
}

bool route_in_decode_supported(int T, int k, int E, int E_loc) {
  return T * k <= ROUTE_MAX_KT && E_loc <= ROUTE_NTH && E <= 512;
}

hipError_t launch_decode_up(int dtype, int maxm, const DecodeParams& p, int grid_segs, hipStream_t s,
                            hipEvent_t ev0, hipEvent_t ev1, const RouteParams* rp) {
  if (p.dM > DENSE_MAXM || p.dM < 0) return hipErrorInvalidValue;
  if (grid_segs <= 0 && p.dM == 0) return hipSuccess;
  if (grid_segs < 0) grid_segs = 0;
  const LaunchEv ev{ev0, ev1};
  const RouteParams none{};
  const RouteParams& r = rp ? *rp : none;
  return dtype == DT_F16 ? launch_dt<DtF16>(true, maxm, p, r, grid_segs, false, s, ev)
                         : launch_dt<DtBF16>(true, maxm, p, r, grid_segs, false, s, ev);
}

hipError_t launch_decode_down(int dtype, int maxm, const DecodeParams& p, int grid_segs, bool fuse_combine,
                              hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.dM > DENSE_MAXM || p.dM < 0) return hipErrorInvalidValue;
  if (grid_segs <= 0 && p.dM == 0) return hipSuccess;
  if (grid_segs < 0) grid_segs = 0;
  // the folded combine reads the row -> token map and the gate weights
  if (fuse_combine && (!p.slot_token || !p.topk_w || !p.out)) return hipErrorInvalidValue;
  const LaunchEv ev{ev0, ev1};
  const RouteParams none{};
  return dtype == DT_F16 ? launch_dt<DtF16>(false, maxm, p, none, grid_segs, fuse_combine, s, ev)
                         : launch_dt<DtBF16>(false, maxm, p, none, grid_segs, fuse_combine, s, ev);
}

}  // namespace moe
