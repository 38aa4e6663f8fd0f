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
// token row x[t] (gate/up adapter, contraction H) or act_r as its bf16 pair
// act_hi + act_lo (down adapter, contraction I: two passes, hi first).
// The contraction runs on the matrix cores: wave w of a 64-row work item
// owns rows 32w .. 32w + 31 (two 16-row blocks sharing each A_e operand) and
// multiplies them by A_e^T (16 columns, zero past the rank) with 16x16x32
// bf16 MFMAs over K in ascending 32-wide steps, fp32 accumulation from zero.  A row's result depends only on its own data,
// never on the batch or its position in it.
//
// The result leaves as a bf16 pair per element, hi = bf16(z), lo =
// bf16(z - hi) (z = hi + lo to about 2^-17 relative), which the grouped
// GEMMs' expand multiplies on the matrix cores: zq[p][0][j] = hi,
// zq[p][1][j] = lo, j < 16.  Operands come straight from memory into
// registers (16 bytes per lane and step), four steps per batch with the
// next batch in flight.
#include "moe_kernels.h"

namespace moe {

constexpr int kShrinkSteps = 4;   // 32-wide K steps per batch of loads
constexpr int kShrinkBlocks = 2;  // 16-row blocks of a wave (sharing its A_e operands)

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4m_t;

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.  Lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]; it holds
// D[4*(l/16) + i][l%16] in element i.
__device__ __forceinline__ f32x4m_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4m_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <bool ACT>
__global__ __launch_bounds__(128) void lora_shrink_kernel(
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rb0 = kShrinkBlocks * wave;  // first 16-row block of this wave
  if (16 * rb0 >= rows) return;         // no barriers below: waves are independent
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t p0 = static_cast<int64_t>(gi.seg0) + gi.row0;
  // rows past the item's end repeat its last row (computed, not stored)
  const uint16_t* xh[kShrinkBlocks];
  const uint16_t* xl[kShrinkBlocks];
#pragma unroll
  for (int q = 0; q < kShrinkBlocks; ++q) {
    const int r = min(16 * (rb0 + q) + r16, rows - 1);
    int64_t src;
    if constexpr (ACT) {
      src = (p0 + r) * Kd;
    } else {
      const int64_t rr = sorted_route[p0 + r];
      src = ((rr >= 0 && rr < T * K) ? rr / K : 0) * Kd;
    }
    xh[q] = v_hi + src + 8 * kq;
    xl[q] = ACT ? v_lo + src + 8 * kq : nullptr;
  }
  const bool jv = r16 < rank;  // this lane's B column is a rank row of A_e
  const uint16_t* ar = a + (static_cast<int64_t>(gi.grp) * rank + (jv ? r16 : 0)) * Kd + 8 * kq;

  u32x4_t h0[kShrinkBlocks][kShrinkSteps], l0[kShrinkBlocks][kShrinkSteps], b0[kShrinkSteps];
  u32x4_t h1[kShrinkBlocks][kShrinkSteps], l1[kShrinkBlocks][kShrinkSteps], b1[kShrinkSteps];
  auto fetch = [&](u32x4_t (&h)[kShrinkBlocks][kShrinkSteps], u32x4_t (&l)[kShrinkBlocks][kShrinkSteps],
                   u32x4_t (&b)[kShrinkSteps], int k0) {
#pragma unroll
    for (int st = 0; st < kShrinkSteps; ++st) {
      const int k = k0 + 32 * st;
      b[st] = jv ? ld16(ar + k) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < kShrinkBlocks; ++q) {
        h[q][st] = ld16(xh[q] + k);
        if constexpr (ACT) l[q][st] = ld16(xl[q] + k);
      }
    }
  };
  f32x4m_t acc[kShrinkBlocks];
#pragma unroll
  for (int q = 0; q < kShrinkBlocks; ++q) acc[q] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4_t (&h)[kShrinkBlocks][kShrinkSteps],
                     const u32x4_t (&l)[kShrinkBlocks][kShrinkSteps], const u32x4_t (&b)[kShrinkSteps]) {
#pragma unroll
    for (int st = 0; st < kShrinkSteps; ++st) {
#pragma unroll
      for (int q = 0; q < kShrinkBlocks; ++q) {
        acc[q] = mfma16x16x32(h[q][st], b[st], acc[q]);
        if constexpr (ACT) acc[q] = mfma16x16x32(l[q][st], b[st], acc[q]);
      }
    }
  };
  constexpr int KB = 32 * kShrinkSteps;  // contraction elements per batch
  const int nb = Kd / KB;                // Kd % 128 == 0
  fetch(h0, l0, b0, 0);
  for (int bt = 0; bt < nb; bt += 2) {
    if (bt + 1 < nb) fetch(h1, l1, b1, (bt + 1) * KB);
    compute(h0, l0, b0);
    if (bt + 2 < nb) fetch(h0, l0, b0, (bt + 2) * KB);
    if (bt + 1 < nb) compute(h1, l1, b1);
  }

#pragma unroll
  for (int q = 0; q < kShrinkBlocks; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * (rb0 + q) + 4 * kq + i;
      if (row < rows) {
        uint16_t hi, lo;
        split_hi_lo(acc[q][i], hi, lo);
        uint16_t* o = zq + (p0 + row) * 2 * kLoraMaxRank;
        o[r16] = hi;
        o[kLoraMaxRank + r16] = lo;
      }
    }
  }
}

hipError_t launch_lora_shrink(const uint16_t* v_hi, const uint16_t* v_lo, const uint16_t* a,
                              const int32_t* offsets, const int32_t* sorted_route,
                              const int32_t* tiles, const int32_t* meta, uint16_t* z, int64_t T,
                              int Kd, int E, int K, int rank, int max_tiles, hipStream_t stream) {
  if (rank < 1 || rank > kLoraMaxRank || Kd % (32 * kShrinkSteps)) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(((static_cast<int64_t>(max_tiles) + 7) / 8) * 8);
  if (v_lo)
    lora_shrink_kernel<true><<<grid, 64 * kRowsPerTile / (16 * kShrinkBlocks), 0, stream>>>(v_hi, v_lo, a, offsets, sorted_route, tiles,
                                                       meta, z, T, Kd, E, K, rank);
  else
    lora_shrink_kernel<false><<<grid, 64 * kRowsPerTile / (16 * kShrinkBlocks), 0, stream>>>(v_hi, nullptr, a, offsets, sorted_route,
                                                        tiles, meta, z, T, Kd, E, K, rank);
  return hipGetLastError();
}

}  // namespace moe
