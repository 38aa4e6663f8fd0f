// Kernel launchers of the routed MoE layer.  Each launcher enqueues one
// kernel on `stream` and returns hipGetLastError(); callers have validated
// every size and pointer before.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

// Router: exact three-way bf16 split of the fp32 weight, the logits (or their
// per-chunk sums), then top-k and gates (optionally with the shared-expert
// gate).
// Permutation: one-workgroup counting sort when sort_small_fits, else the
// three passes hist / scan / scatter.
hipError_t launch_router_split(const float* wr, uint16_t* planes, int H, int E, hipStream_t stream);
// router_full(T): large batches take router_full (logits written directly),
// smaller ones router_part (per-chunk sums) with top-k forming the logits.
bool router_full(int64_t T);
hipError_t launch_router_part(const uint16_t* x, const uint16_t* planes, float* part, int64_t T,
                              int H, int E, hipStream_t stream);
hipError_t launch_router_full(const uint16_t* x, const uint16_t* planes, const float* bias,
                              float* logits, int64_t T, int H, int E, hipStream_t stream);
hipError_t launch_topk_gate(const float* src, int nchunk, const float* bias, float* logits_out,
                            int32_t* topk_idx, float* topk_gate, const uint16_t* x,
                            const uint16_t* w_sgate, float* sg, int64_t T, int H, int E, int K,
                            hipStream_t stream);
bool sort_small_fits(int64_t T, int E);
// Work lists: the permutation kernels (and launch_ffn_tiles) also write the
// up projection's list of up_rows-row tiles to tiles_up when it is not null
// (up_rows_per_tile(...) != kRowsPerTile); its count goes to meta[2].
hipError_t launch_route_sort_small(const int32_t* topk_idx, int32_t* offsets, int32_t* route_pos,
                                   int32_t* sorted_route, int32_t* tiles, int32_t* tiles_up,
                                   int up_rows, int32_t* meta, int* err_word, int64_t T, int E,
                                   int K, int has_shared, hipStream_t stream);
hipError_t launch_route_hist(const int32_t* topk_idx, int32_t* hist, int32_t* route_rank,
                             int64_t T, int E, int K, hipStream_t stream);
hipError_t launch_route_scan(const int32_t* hist, int32_t* block_base, int32_t* offsets,
                             int32_t* tiles, int32_t* tiles_up, int up_rows, int32_t* meta,
                             int nblocks, int E, int64_t T, int has_shared, int* err_word,
                             hipStream_t stream);
// Work list from caller-supplied offsets; offsets that are not a partition
// of [0, T*K) set *err_word and give an empty list.
// The shared expert's work list alone (rows-row tiles), length in *ntiles.
hipError_t launch_shared_tiles(int32_t* tiles, int32_t* ntiles, int64_t T, int E, int rows, hipStream_t stream);
// Offsets that are not a partition of [0, T*K) set *err_word = 1 and leave
// an empty list; with err_overwrite valid offsets clear it (0).
hipError_t launch_ffn_tiles(const int32_t* offsets, int32_t* tiles, int32_t* tiles_up, int up_rows,
                            int32_t* meta, int* err_word, int err_overwrite, int E, int64_t T, int K,
                            int has_shared, int rows_per_tile, hipStream_t stream);
hipError_t launch_route_scatter(const int32_t* topk_idx, const int32_t* block_base,
                                const int32_t* offsets, int32_t* route_pos, int32_t* sorted_route,
                                int64_t T, int E, int K, hipStream_t stream);
hipError_t launch_shared_gate(const uint16_t* x, const uint16_t* w_sgate, float* sg, int64_t T,
                              int H, hipStream_t stream);
// Rows per up-projection work item at this batch: kUpTallRows from
// kUpTallMin tokens at hidden size 2048, else kRowsPerTile.  Only the work
// split changes; every element's arithmetic is the same.
inline int up_rows_per_tile(int64_t T, int H) {
  return (T >= kUpTallMin && H == 2048) ? kUpTallRows : kRowsPerTile;
}
// tiles / ntiles: the up_rows-row work list and the int holding its length.
// mx: block-scaled FP8 expert weights (then w13 / ws13 resp. w2 / ws2 are
// not read), or null for bf16 weights.
hipError_t launch_ffn_up(const uint16_t* x, const uint16_t* w13, const uint16_t* ws13,
                         const MxWeights* mx, const LoraExpand* lora, const int32_t* offsets,
                         const int32_t* sorted_route, const int32_t* tiles, const int32_t* ntiles,
                         int up_rows, uint16_t* act_hi, uint16_t* act_lo, uint16_t* sact_hi,
                         uint16_t* sact_lo, float* gu, float* sgu, int64_t T, int H, int E, int K,
                         int I, int Is, int max_tiles, hipStream_t stream);
hipError_t launch_ffn_down(const uint16_t* act_hi, const uint16_t* act_lo,
                           const uint16_t* sact_hi, const uint16_t* sact_lo, const uint16_t* w2,
                           const uint16_t* ws2, const MxWeights* mx, const LoraExpand* lora,
                           const int32_t* offsets, const int32_t* sorted_route,
                           const int32_t* tiles, const int32_t* meta, float* y, float* sy,
                           int64_t T, int H, int E, int K, int I, int Is, int max_tiles,
                           hipStream_t stream);
// LoRA shrink of the routed experts' rows (lora_kernels.hip): z[p][j] =
// sum_k A_e[j][k] v_p[k] over the 64-row work list `tiles` (meta[0] items),
// stored as bf16 pairs zq[p][0 hi | 1 lo][16]; v_p = x[token of route
// sorted_route[p]] (v_lo null) or v_hi[p] + v_lo[p].
hipError_t launch_lora_shrink(const uint16_t* v_hi, const uint16_t* v_lo, const uint16_t* a,
                              const int32_t* offsets, const int32_t* sorted_route,
                              const int32_t* tiles, const int32_t* meta, uint16_t* z, int64_t T,
                              int Kd, int E, int K, int rank, int max_tiles, hipStream_t stream);
hipError_t launch_combine(const float* y, const float* gate, const float* sy, const float* sg,
                          float* out32, uint16_t* out16, int64_t T, int H, int K,
                          hipStream_t stream);

// Arguments of the backward's grouped GEMMs (see bwd_kernels.hip).
struct BwdLaunch {
  int64_t T;
  int H, E, K, I, Is;
  int max_tiles_bwd;
  const int32_t* offsets;
  const int32_t* sorted_route;
  const float* gate;
  const float* sg;
  const int32_t* tiles;  // kBwdRowsPerTile-row tiles
  const int32_t* meta;
  const uint16_t* x;
  const uint16_t* dout;
  const uint16_t* w13;
  const uint16_t* w2;
  const uint16_t* ws13;
  const uint16_t* ws2;
  const float* gu;
  const float* sgu;
  uint16_t* dgu[kGradPlanes];    // hi/lo planes
  uint16_t* sdgu[kGradPlanes];
  uint16_t* gact[kGradPlanes];
  uint16_t* sgact[kGradPlanes];
  double* dgp;  // [R][max(I, Is) / 128] partial route-weight gradients (kDact)
  double* dsp;  // [T][max(I, Is) / 128] partial shared-gate gradients (kDact)
  float *dx_route, *dx_shared;
  float *dw13, *dw2, *dws13, *dws2;
  // LoRA adapters of the routed experts (la13 = la2 = null: none): A13
  // [E][rank][H] and A2 [E][rank][I], and the shrink results (bf16 pairs
  // [R][hi, lo][kLoraMaxRank]) v2 = B2^T dOut, read by launch_bwd_dact, and
  // u13 = B13^T dGU, read by launch_bwd_gemms and launch_bwd_lora_grads
  const uint16_t* la13 = nullptr;
  const uint16_t* la2 = nullptr;
  const uint16_t* lv2 = nullptr;
  const uint16_t* lu13 = nullptr;
  float lscale = 0.f;
  int lrank = 0;
};

// Backward order: launch_bwd_dact (dGU and g*act planes, partial dot
// products), launch_bwd_gate (dl, dz from the partials), launch_bwd_gemms
// (dx, dW2, dW13), then the router, shared-gate and dX kernels.
hipError_t launch_bwd_dact(const BwdLaunch& L, hipStream_t stream);
hipError_t launch_bwd_gate(const double* dgp, const double* dsp, const float* gate, const float* sg,
                           float* dl, float* dz, int64_t T, int K, int I, int Is,
                           hipStream_t stream);
hipError_t launch_bwd_gemms(const BwdLaunch& L, hipStream_t stream);
// its three GEMMs one by one (independent of each other): dx, dW2, dW13
hipError_t launch_bwd_dx(const BwdLaunch& L, hipStream_t stream);
hipError_t launch_bwd_dw2(const BwdLaunch& L, hipStream_t stream);
hipError_t launch_bwd_dw13(const BwdLaunch& L, hipStream_t stream);
// With adapters: the shrinks of v2 (before launch_bwd_dact) and of u13, z13
// = A13 x and gz2 = A2 (g act) (after it) by launch_lora_shrink, then
// launch_bwd_lora_grads writes dA13 [E][rank][H], dB13 [E][2I][rank], dA2
// [E][rank][I] and dB2 [E][H][rank].
hipError_t launch_bwd_lora_grads(const BwdLaunch& L, const uint16_t* z13, const uint16_t* gz2, float* da13,
                                 float* db13, float* da2, float* db2, hipStream_t stream);
// dst[e][n][m] = src[e][m][n] for bf16 [E][M][N] matrices.
hipError_t launch_lora_transpose(const uint16_t* src, uint16_t* dst, int E, int M, int N, hipStream_t stream);
hipError_t launch_bwd_router(const uint16_t* x, const float* dl, const int32_t* offsets,
                             const int32_t* sorted_route, float* dwr, int64_t T, int H, int E,
                             int K, hipStream_t stream);
hipError_t launch_bwd_wsg(const uint16_t* x, const float* dz, double* partial, float* dwsg, int64_t T,
                          int H, hipStream_t stream);
hipError_t launch_bwd_dx_sum(const int32_t* topk_idx, const float* dl, const float* dx_route,
                             const float* dx_shared, const float* dz, const uint16_t* w_sgate,
                             const float* w_router, float* dx32, uint16_t* dx16, int64_t T, int H,
                             int E, int K, hipStream_t stream);

// Upper bound on grouped-GEMM row tiles for T tokens: every non-empty
// expert's last tile may be partial, plus the shared expert's tiles.
inline int64_t max_row_tiles(int64_t T, int K, int E, int has_shared, int rows = kRowsPerTile) {
  const int64_t R = T * K;
  return E + (R + rows - 1) / rows + (has_shared ? (T + rows - 1) / rows : 0);
}

}  // namespace moe
