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
// A workgroup of 16 waves takes 16 rows of one 64-row work item (quarter q
// of the item: rows 16q .. 16q + 15) and stages A_e in LDS for them, 2048
// contraction elements at a time.
#include "moe_kernels.h"

namespace moe {

constexpr int kShrinkWaves = 16;
constexpr int kShrinkChunk = 2048;  // contraction elements of A_e staged at once

template <bool ACT>
__global__ __launch_bounds__(1024) void lora_shrink_kernel(
    const uint16_t* __restrict__ v_hi, const uint16_t* __restrict__ v_lo,
    const uint16_t* __restrict__ a, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_route, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ meta, float* __restrict__ z, int64_t T, int Kd, int E, int K,
    int rank) {
  constexpr int QPI = kRowsPerTile / kShrinkWaves;  // workgroups per 64-row item
  constexpr int CP = kShrinkChunk / 8;              // 8-element pieces per staged chunk
  const int item = xcd_item(blockIdx.x, meta[0] * QPI);
  if (item < 0) return;
  const GroupItem gi = group_item(item, QPI, tiles, offsets, E, T, kRowsPerTile);
  if (gi.grp == E) return;  // the shared expert has no adapter
  const int first = gi.row0 + kShrinkWaves * gi.nt;
  if (first >= gi.cnt) return;

  __shared__ __attribute__((aligned(16))) uint16_t As[kLoraMaxRank * kShrinkChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = first + wave;
  const bool valid = r < gi.cnt;  // waves past the segment compute a copy, store nothing
  const int64_t p = static_cast<int64_t>(gi.seg0) + (valid ? r : first);
  const uint16_t* vh;
  const uint16_t* vl = nullptr;
  if constexpr (ACT) {
    vh = v_hi + p * Kd;
    vl = v_lo + p * Kd;
  } else {
    const int64_t rr = sorted_route[p];
    const int64_t tok = (rr >= 0 && rr < T * K) ? rr / K : 0;
    vh = v_hi + tok * Kd;
  }
  const uint16_t* ae = a + static_cast<int64_t>(gi.grp) * rank * Kd;
  const int npieces = Kd >> 3;

  float s[kLoraMaxRank];
#pragma unroll
  for (int jj = 0; jj < kLoraMaxRank; ++jj) s[jj] = 0.f;

  for (int c0 = 0; c0 < Kd; c0 += kShrinkChunk) {
    const int q0 = c0 >> 3;
    // this lane's pieces of the chunk, loaded before the staging barrier
    u32x4_t vh4[CP / 64], vl4[CP / 64];
#pragma unroll
    for (int c = 0; c < CP / 64; ++c) {
      const int q = q0 + lane + 64 * c;
      if (q < npieces) {
        vh4[c] = ld16(vh + 8 * q);
        if constexpr (ACT) vl4[c] = ld16(vl + 8 * q);
      }
    }
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    for (int i = tid; i < rank * CP; i += 1024) {
      const int jj = i / CP, qq = i % CP;
      if (q0 + qq < npieces) st16(&As[jj * kShrinkChunk + 8 * qq], ld16(ae + static_cast<int64_t>(jj) * Kd + 8 * (q0 + qq)));
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CP / 64; ++c) {
      const int qq = lane + 64 * c;
      if (q0 + qq < npieces) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(vh4[c][e] << 16);
          v[2 * e + 1] = __uint_as_float(vh4[c][e] & 0xffff0000u);
          if constexpr (ACT) {
            v[2 * e] += __uint_as_float(vl4[c][e] << 16);
            v[2 * e + 1] += __uint_as_float(vl4[c][e] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int jj = 0; jj < kLoraMaxRank; ++jj) {
          if (jj < rank) {
            const u32x4_t a4 = ld16(&As[jj * kShrinkChunk + 8 * qq]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s[jj] = fmaf(__uint_as_float(a4[e] << 16), v[2 * e], s[jj]);
              s[jj] = fmaf(__uint_as_float(a4[e] & 0xffff0000u), v[2 * e + 1], s[jj]);
            }
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
  float o = 0.f;
#pragma unroll
  for (int jj = 0; jj < kLoraMaxRank; ++jj)
    if (lane == jj) o = s[jj];
  if (valid && lane < kLoraMaxRank) z[p * kLoraMaxRank + lane] = o;
}

hipError_t launch_lora_shrink(const uint16_t* v_hi, const uint16_t* v_lo, const uint16_t* a,
                              const int32_t* offsets, const int32_t* sorted_route,
                              const int32_t* tiles, const int32_t* meta, float* z, int64_t T,
                              int Kd, int E, int K, int rank, int max_tiles, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(max_tiles) * (kRowsPerTile / kShrinkWaves);
  const unsigned grid = static_cast<unsigned>(((items + 7) / 8) * 8);
  if (v_lo)
    lora_shrink_kernel<true><<<grid, 1024, 0, stream>>>(v_hi, v_lo, a, offsets, sorted_route, tiles,
                                                        meta, z, T, Kd, E, K, rank);
  else
    lora_shrink_kernel<false><<<grid, 1024, 0, stream>>>(v_hi, nullptr, a, offsets, sorted_route,
                                                         tiles, meta, z, T, Kd, E, K, rank);
  return hipGetLastError();
}

}  // namespace moe
