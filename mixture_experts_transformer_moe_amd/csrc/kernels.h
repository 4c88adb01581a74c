// Host-side launchers of the HIP kernels (one definition per kernel file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "common.h"
#include "tile_plan.h"

namespace moe {

// gate.hip
// fill (nullable): nfill 32-bit words set to 0xFFFFFFFF by the launch (the
// one-launch decode kernel's hidden rows, marked unwritten in the launch before it)
hipError_t launch_gate_logits_fma(int dtype, const void* x, const void* wg, const float* bias, float* z,
                                  int T, int H, int E, hipStream_t s, unsigned* fill = nullptr, int nfill = 0);
// zsplit > 1: z holds that many partial logit sums, T * E floats apart (see GemmParams::ksplit)
hipError_t launch_softmax_topk(const float* z, int T, int E, int k, int renorm, int* idx, float* w,
                               float* probs, hipStream_t s, int zsplit = 1);

// dispatch.hip
size_t dispatch_small_lds(int E);
int dispatch_num_blocks(long long kT);
int dispatch_block_size();
// y_zero (nullable): output rows of tokens with no kept assignment are zeroed there.
// plan (nullable): the expert GEMMs' tile lists are built from the kept rows too.
hipError_t launch_dispatch_small(bool fuse_topk, const float* z, int renorm, float* probs, float* topk_w,
                                 int* idx, int T, int k, int E, int e_lo, int E_loc, int C, int R_max,
                                 int* demand, int* offsets, int* slot_token, int* token_slot, void* y_zero,
                                 int y_esz, int H, const TilePlanArgs* plan, int zsplit, hipStream_t s);
hipError_t launch_dispatch_multi(const int* idx, int T, int k, int E, int e_lo, int E_loc, int C, int R_max,
                                 int* rank, int* blk_hist, int* demand, int* offsets, int* slot_token,
                                 int* token_slot, void* y_zero, int y_esz, int H, const TilePlanArgs* plan,
                                 hipStream_t s);
hipError_t launch_gather_rows(int dtype, const void* x, const int* slot_token, int R_max, int H, void* xd,
                              hipStream_t s);
// Softmax / top-k of every token, the whole dispatch and the tile lists in one
// launch (more than one block of assignments). keys (k*T ints), hist (nblk*E
// ints) and slot_token (R_max ints) must hold 0 at launch (the gate launch
// before it zeroes them); z, zsplit and renorm as for launch_softmax_topk.
struct RouteDispatchArgs {
  const float* z;
  int zsplit, renorm;
  float* probs;   // nullable
  float* topk_w;
  int* idx;
  int T, k, E, e_lo, E_loc, C, R_max, H, y_esz;
  int* keys;
  int* hist;
  int* demand;
  int* offsets;
  int* slot_token;
  int* token_slot;
  void* y_zero;   // nullable, as for launch_dispatch_multi
};
bool route_dispatch_supported(long long kT);
size_t route_dispatch_lds(int E);
hipError_t launch_route_dispatch(const RouteDispatchArgs& a, const TilePlanArgs* plan, hipStream_t s);

// gemm.hip
enum { EPI_GELU = 0, EPI_F32 = 1 };
// Tile lists for segments [seg_off[s], seg_off[s+1]) (nseg <= 1024), see TilePlanArgs.
hipError_t launch_gemm_plan(const int* seg_off, int nseg, const TilePlanArgs& a, hipStream_t s);
// bias_f32 selects a float bias (gate) instead of a dtype bias.
// ev0 / ev1 (nullable): recorded by the kernel dispatch itself (start / end).
hipError_t launch_grouped_gemm(int dtype, int epi, bool bias_f32, int BM, int BN, const GemmParams& p,
                               int grid, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// decode_ffn.hip
bool decode_supported(int dtype, int H, int F);
// work-groups of the larger decode expert launch (segment groups of each)
long long decode_max_workgroups(int dtype, int H, int F, int maxm, long long groups_up, long long groups_down);
// rp (nullable): route the batch inside the kernel from the gate logits (see RouteParams).
bool route_in_decode_supported(int T, int k, int E, int E_loc);
hipError_t launch_decode_up(int dtype, int maxm, const DecodeParams& p, int grid_segs, hipStream_t s,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, const RouteParams* rp = nullptr);
hipError_t launch_decode_down(int dtype, int maxm, const DecodeParams& p, int grid_segs, bool fuse_combine,
                              hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Both expert products in one launch (routing inside, as launch_decode_up with rp);
// p.h must hold 0xFFFF in every 16-bit element at launch (the gate kernel fills it).
bool decode_fused_supported(int dtype, int H, int F, int maxm);
hipError_t launch_decode_fused(int dtype, int maxm, const DecodeParams& p, const RouteParams& rp, int grid_segs,
                               bool fuse_combine, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// combine.hip: y[t] = sum_j w[t,j] ysrc[token_slot[t,j]] (+ dense[t]); ysrc [*, H], dense [T, H] fp32
hipError_t launch_combine(int dtype, const float* ysrc, const int* token_slot, const float* w, int k,
                          const float* dense, void* y, int T, int H, hipStream_t s);

}  // namespace moe
