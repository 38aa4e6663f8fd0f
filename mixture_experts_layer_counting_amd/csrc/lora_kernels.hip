// LoRA shrink of the routed experts (gfx950).
//
// ROLL pull request 502 page (Qwen3.8-Flash-Next adapter): the grouped
// expert adapters have rank r // top_k ("What this changes"), and the
// adapters' shrink, the A projection, runs with a single K partition, so no
// partial sums of a split contraction are ever combined by fp32 atomics
// (opening summary, numerical fixes).  Here a row's whole contraction
// belongs to one wave:
//
//   z[p][j] = sum_k A_e[j][k] v_p[k]   for j < rank, z[p][rank .. 16) = 0,
//
// for every routed row p (sorted position) of expert e.  v_p is the gathered
// token row x[t] (gate/up adapter, contraction H) or act_hi[p] + act_lo[p]
// (down adapter, contraction I; the sum of the bf16 pair is exact in fp32).
// Lane l of the row's wave takes the 8-element pieces l, l + 64, l + 128, ...
// of the contraction in ascending order, one fp32 fma chain from +0 per j;
// the 64 lane sums are then combined by a fixed xor butterfly (lane distance
// 32, 16, ..., 1), which leaves the same bits in every lane.  A row's result
// depends only on its own data, never on the batch or its position in it.
//
// The result leaves as a bf16 pair per element, hi = bf16(z), lo =
// bf16(z - hi) (z = hi + lo to about 2^-17 relative), which the grouped
// GEMMs' expand multiplies on the matrix cores: zq[p][0][j] = hi,
// zq[p][1][j] = lo, j < 16.
//
// A workgroup of eight waves takes one 64-row work item of an expert and
// stages all of A_e in LDS (rank * contraction <= kLoraShrinkLds elements,
// checked by the host); wave w computes rows w, w + 8, ....  Each wave
// issues its first row's loads before the staging barrier.
#include "moe_kernels.h"

namespace moe {

constexpr int kShrinkWaves = 8;

template <bool ACT>
__global__ __launch_bounds__(kShrinkWaves * 64) void lora_shrink_kernel(
    const uint16_t* __restrict__ v_hi, const uint16_t* __restrict__ v_lo,
    const uint16_t* __restrict__ a, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_route, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ meta, uint16_t* __restrict__ zq, int64_t T, int Kd, int E, int K,
    int rank) {
  const int item = xcd_item(blockIdx.x, meta[0]);
  if (item < 0) return;
  const GroupItem gi = group_item(item, 1, tiles, offsets, E, T, kRowsPerTile);
  if (gi.grp == E) return;  // the shared expert has no adapter
  const int rows = min(kRowsPerTile, gi.cnt - gi.row0);
  if (rows <= 0) return;
  extern __shared__ __attribute__((aligned(16))) uint16_t As[];  // A_e [rank][Kd]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t p0 = static_cast<int64_t>(gi.seg0) + gi.row0;
  const int npieces = Kd >> 3;  // 8-element pieces of a row; lane pieces q = lane + 64 c
  const int nc = (npieces + 63) >> 6;
  auto src_of = [&](int r) -> int64_t {
    if constexpr (ACT) {
      return (p0 + r) * Kd;
    } else {
      const int64_t rr = sorted_route[p0 + r];
      return ((rr >= 0 && rr < T * K) ? rr / K : 0) * Kd;
    }
  };
  u32x4_t vh[kLoraMaxPieces], vl[kLoraMaxPieces];
  auto load = [&](int r) {
    const int64_t src = src_of(r);
#pragma unroll
    for (int c = 0; c < kLoraMaxPieces; ++c) {
      const int q = lane + 64 * c;
      if (c < nc && q < npieces) {
        vh[c] = ld16(v_hi + src + 8 * q);
        if constexpr (ACT) vl[c] = ld16(v_lo + src + 8 * q);
      }
    }
  };
  if (wave < rows) load(wave);
  const uint16_t* ae = a + static_cast<int64_t>(gi.grp) * rank * Kd;
  for (int i = tid; i < rank * Kd / 8; i += kShrinkWaves * 64) st16(&As[8 * i], ld16(ae + 8 * i));
  __syncthreads();

  for (int r = wave; r < rows; r += kShrinkWaves) {
    if (r != wave) load(r);
    float s[kLoraMaxRank];
#pragma unroll
    for (int jj = 0; jj < kLoraMaxRank; ++jj) s[jj] = 0.f;
#pragma unroll
    for (int c = 0; c < kLoraMaxPieces; ++c) {
      const int q = lane + 64 * c;
      if (c < nc && q < npieces) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(vh[c][e] << 16);
          v[2 * e + 1] = __uint_as_float(vh[c][e] & 0xffff0000u);
          if constexpr (ACT) {
            v[2 * e] += __uint_as_float(vl[c][e] << 16);
            v[2 * e + 1] += __uint_as_float(vl[c][e] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int jj = 0; jj < kLoraMaxRank; ++jj) {
          if (jj < rank) {
            const u32x4_t a4 = ld16(&As[jj * Kd + 8 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s[jj] = fmaf(__uint_as_float(a4[e] << 16), v[2 * e], s[jj]);
              s[jj] = fmaf(__uint_as_float(a4[e] & 0xffff0000u), v[2 * e + 1], s[jj]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < kLoraMaxRank; ++jj) {
      if (jj < rank) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) s[jj] += __shfl_xor(s[jj], off, 64);
      }
    }
    // lanes 0..15 store hi of element j = lane, lanes 16..31 lo of j = lane - 16
    const int jj_out = lane & 15;
    float o = 0.f;
#pragma unroll
    for (int jj = 0; jj < kLoraMaxRank; ++jj)
      if (jj_out == jj) o = s[jj];
    uint16_t hi, lo;
    split_hi_lo(o, hi, lo);
    if (lane < 2 * kLoraMaxRank) zq[(p0 + r) * 2 * kLoraMaxRank + lane] = lane < kLoraMaxRank ? hi : lo;
  }
}

hipError_t launch_lora_shrink(const uint16_t* v_hi, const uint16_t* v_lo, const uint16_t* a,
                              const int32_t* offsets, const int32_t* sorted_route,
                              const int32_t* tiles, const int32_t* meta, uint16_t* z, int64_t T,
                              int Kd, int E, int K, int rank, int max_tiles, hipStream_t stream) {
  if (rank < 1 || rank > kLoraMaxRank || static_cast<int64_t>(rank) * Kd > kLoraShrinkLds ||
      Kd > 512 * kLoraMaxPieces || Kd % 8)
    return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(((static_cast<int64_t>(max_tiles) + 7) / 8) * 8);
  const size_t lds = static_cast<size_t>(rank) * Kd * 2;
  if (v_lo)
    lora_shrink_kernel<true><<<grid, kShrinkWaves * 64, lds, stream>>>(v_hi, v_lo, a, offsets, sorted_route, tiles,
                                                         meta, z, T, Kd, E, K, rank);
  else
    lora_shrink_kernel<false><<<grid, kShrinkWaves * 64, lds, stream>>>(v_hi, nullptr, a, offsets, sorted_route,
                                                          tiles, meta, z, T, Kd, E, K, rank);
  return hipGetLastError();
}

}  // namespace moe
