// Grouped expert FFN and combine kernels of the routed MoE layer (gfx950).
//
// Experts bullet of the "MoE route/combine contract" commit (RL-Kernel pull
// request 557 page): each route row gets its expert's gate_up and down
// projections with ONE fixed tile configuration, no gate multiply and no sum
// inside, exactly one writer per (token, route) row.  Here the fixed part is
// the per-element arithmetic: the 32x32x16 bf16 MFMA, the K order (64-wide
// blocks in ascending order, inside a block the lane-half/K-step order
// below) and fp32 accumulation from zero.  How rows are grouped into tiles
// (which depends on the batch) never changes a row's arithmetic, because an
// MFMA output row depends only on its own A row.
//
// Combine bullet: the route terms are summed in fp32 in route (slot) order
// with one bf16 cast at the end and no atomics.
#include "moe_kernels.h"

namespace moe {

// LDS row stride (bf16 elements) of a 64-wide K block: 64 + 8 of padding
// keeps the 16-byte MFMA operand reads of 16 consecutive rows on distinct
// banks.
constexpr int kLdsStride = 72;

// ---------------------------------------------------------------------------
// Up projection + SwiGLU.
// Work item = (row tile of one group, 128 activation columns).  Group g < E
// is routed expert g, its rows are the sorted positions offsets[g] + row0 ..;
// group E is the shared expert, rows are tokens row0 ...
// Wave w owns activation columns c = nt*128 + 32w .. +32 and computes both
// gate (W13 row c) and up (W13 row I + c) for every row of the tile, so the
// SwiGLU is elementwise on the two accumulators.  The weight rows stream from
// HBM straight into registers (each lane 64 contiguous bytes per block, the
// two lane halves one 128-byte line per row); the gathered activation rows
// are staged in LDS and shared by the four waves.
// Outputs: act as a bf16 hi/lo pair (row = sorted position, or token for the
// shared expert) and, if requested, the fp32 gate/up values.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void ffn_up_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const uint16_t* __restrict__ ws13, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_route, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ meta, uint16_t* __restrict__ act_hi,
    uint16_t* __restrict__ act_lo, uint16_t* __restrict__ sact_hi,
    uint16_t* __restrict__ sact_lo, float* __restrict__ gu, float* __restrict__ sgu, int64_t T,
    int H, int E, int K, int I, int Is, int ncol_tiles) {
  const int item = xcd_item(blockIdx.x, meta[0] * ncol_tiles);
  if (item < 0) return;
  const int tile = item / ncol_tiles, nt = item - tile * ncol_tiles;
  const int grp = tiles[2 * tile], row0 = tiles[2 * tile + 1];
  const bool shared = grp == E;
  const int Ie = shared ? Is : I;
  if (nt * kUpCols >= Ie) return;
  const int seg0 = shared ? 0 : offsets[grp];
  const int cnt = shared ? static_cast<int>(T) : offsets[grp + 1] - seg0;
  const int rows = min(kRowsPerTile, cnt - row0);
  if (rows <= 0) return;
  const int nmb = (rows + 31) >> 5;
  const uint16_t* W = shared ? ws13 : w13 + static_cast<int64_t>(grp) * 2 * I * H;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][kRowsPerTile][kLdsStride];
  __shared__ int s_tok[kRowsPerTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, half = lane >> 5;
  const int64_t R = T * K;

  if (tid < kRowsPerTile) {
    const int rr = min(tid, rows - 1);
    int64_t tok;
    if (shared) {
      tok = row0 + rr;
    } else {
      const int64_t r = sorted_route[seg0 + row0 + rr];
      tok = (r >= 0 && r < R) ? r / K : 0;
    }
    s_tok[tid] = static_cast<int>(tok);
  }
  __syncthreads();

  const int arow = tid >> 1, acol = (tid & 1) * 32;
  const bool aload = arow < nmb * 32;
  const uint16_t* xa = x + static_cast<int64_t>(s_tok[arow]) * H + acol;

  const int col = nt * kUpCols + wave * 32 + j;
  const uint16_t* wg = W + static_cast<int64_t>(col) * H + 32 * half;
  const uint16_t* wu = W + static_cast<int64_t>(Ie + col) * H + 32 * half;

  f32x16_t accg[4], accu[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    accg[mb] = zero16();
    accu[mb] = zero16();
  }
  u32x4_t ra[4], bg[4], bu[4], nbg[4], nbu[4];

  if (aload) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[q] = ld16(xa + 8 * q);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bg[s] = ld16(wg + 8 * s);
    bu[s] = ld16(wu + 8 * s);
  }
  if (aload) {
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(&As[0][arow][acol + 8 * q], ra[q]);
  }

  const int nkb = H >> 6;
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {
      const int k1 = (kb + 1) << 6;
      if (aload) {
#pragma unroll
        for (int q = 0; q < 4; ++q) ra[q] = ld16(xa + k1 + 8 * q);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        nbg[s] = ld16(wg + k1 + 8 * s);
        nbu[s] = ld16(wu + k1 + 8 * s);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          const u32x4_t a = ld16(&As[cur][mb * 32 + j][32 * half + 8 * s]);
          accg[mb] = mfma32x32x16(a, bg[s], accg[mb]);
          accu[mb] = mfma32x32x16(a, bu[s], accu[mb]);
        }
      }
    }
    if (more) {
      if (aload) {
#pragma unroll
        for (int q = 0; q < 4; ++q) st16(&As[cur ^ 1][arow][acol + 8 * q], ra[q]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bg[s] = nbg[s];
        bu[s] = nbu[s];
      }
    }
  }

  uint16_t* ohi = shared ? sact_hi : act_hi;
  uint16_t* olo = shared ? sact_lo : act_lo;
  float* ogu = shared ? sgu : gu;
  const int64_t p0 = shared ? row0 : static_cast<int64_t>(seg0) + row0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb < nmb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = mb * 32 + acc_row(v, half);
        if (row < rows) {
          const float g = accg[mb][v], u = accu[mb][v];
          const float a = silu_f32(g) * u;
          uint16_t hi, lo;
          split_hi_lo(a, hi, lo);
          const int64_t p = p0 + row;
          ohi[p * Ie + col] = hi;
          olo[p * Ie + col] = lo;
          if (ogu) {
            ogu[p * 2 * Ie + col] = g;
            ogu[p * 2 * Ie + Ie + col] = u;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection: y = act W2^T with act = hi + lo (two MFMA passes into the
// same fp32 accumulator, hi first), written to route row sorted_route[p] of y
// (or token row of shared_y).  Work item = (row tile, 256 hidden columns);
// wave w owns columns nt*256 + 64w .. +64 as two 32-column blocks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void ffn_down_kernel(
    const uint16_t* __restrict__ act_hi, const uint16_t* __restrict__ act_lo,
    const uint16_t* __restrict__ sact_hi, const uint16_t* __restrict__ sact_lo,
    const uint16_t* __restrict__ w2, const uint16_t* __restrict__ ws2,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_route,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta, float* __restrict__ y,
    float* __restrict__ sy, int64_t T, int H, int E, int K, int I, int Is) {
  const int ncol_tiles = H / kDownCols;
  const int item = xcd_item(blockIdx.x, meta[0] * ncol_tiles);
  if (item < 0) return;
  const int tile = item / ncol_tiles, nt = item - tile * ncol_tiles;
  const int grp = tiles[2 * tile], row0 = tiles[2 * tile + 1];
  const bool shared = grp == E;
  const int Ie = shared ? Is : I;
  const int seg0 = shared ? 0 : offsets[grp];
  const int cnt = shared ? static_cast<int>(T) : offsets[grp + 1] - seg0;
  const int rows = min(kRowsPerTile, cnt - row0);
  if (rows <= 0) return;
  const int nmb = (rows + 31) >> 5;
  const uint16_t* W = shared ? ws2 : w2 + static_cast<int64_t>(grp) * H * I;
  const int64_t p0 = shared ? row0 : static_cast<int64_t>(seg0) + row0;
  const uint16_t* Ahi = (shared ? sact_hi : act_hi) + p0 * Ie;
  const uint16_t* Alo = (shared ? sact_lo : act_lo) + p0 * Ie;
  float* out = shared ? sy : y;

  __shared__ __attribute__((aligned(16))) uint16_t Ah[2][kRowsPerTile][kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Al[2][kRowsPerTile][kLdsStride];
  __shared__ int s_dst[kRowsPerTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, half = lane >> 5;
  const int64_t R = T * K;

  if (tid < kRowsPerTile) {
    int dst = -1;
    if (tid < rows) {
      if (shared) {
        dst = row0 + tid;
      } else {
        const int64_t r = sorted_route[p0 + tid];
        dst = (r >= 0 && r < R) ? static_cast<int>(r) : -1;
      }
    }
    s_dst[tid] = dst;
  }

  const int arow = tid >> 1, acol = (tid & 1) * 32;
  const bool aload = arow < nmb * 32;
  const int64_t aoff = static_cast<int64_t>(min(arow, rows - 1)) * Ie + acol;

  const int n0 = nt * kDownCols + wave * 64;
  const uint16_t* wb0 = W + static_cast<int64_t>(n0 + j) * Ie + 32 * half;
  const uint16_t* wb1 = W + static_cast<int64_t>(n0 + 32 + j) * Ie + 32 * half;

  f32x16_t acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    acc[mb][0] = zero16();
    acc[mb][1] = zero16();
  }
  u32x4_t rh[4], rl[4], b0[4], b1[4], nb0[4], nb1[4];

  if (aload) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rh[q] = ld16(Ahi + aoff + 8 * q);
      rl[q] = ld16(Alo + aoff + 8 * q);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    b0[s] = ld16(wb0 + 8 * s);
    b1[s] = ld16(wb1 + 8 * s);
  }
  if (aload) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      st16(&Ah[0][arow][acol + 8 * q], rh[q]);
      st16(&Al[0][arow][acol + 8 * q], rl[q]);
    }
  }

  const int nkb = Ie >> 6;
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {
      const int k1 = (kb + 1) << 6;
      if (aload) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rh[q] = ld16(Ahi + aoff + k1 + 8 * q);
          rl[q] = ld16(Alo + aoff + k1 + 8 * q);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        nb0[s] = ld16(wb0 + k1 + 8 * s);
        nb1[s] = ld16(wb1 + k1 + 8 * s);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          const u32x4_t ah = ld16(&Ah[cur][mb * 32 + j][32 * half + 8 * s]);
          const u32x4_t al = ld16(&Al[cur][mb * 32 + j][32 * half + 8 * s]);
          acc[mb][0] = mfma32x32x16(ah, b0[s], acc[mb][0]);
          acc[mb][0] = mfma32x32x16(al, b0[s], acc[mb][0]);
          acc[mb][1] = mfma32x32x16(ah, b1[s], acc[mb][1]);
          acc[mb][1] = mfma32x32x16(al, b1[s], acc[mb][1]);
        }
      }
    }
    if (more) {
      if (aload) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          st16(&Ah[cur ^ 1][arow][acol + 8 * q], rh[q]);
          st16(&Al[cur ^ 1][arow][acol + 8 * q], rl[q]);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        b0[s] = nb0[s];
        b1[s] = nb1[s];
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb < nmb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = mb * 32 + acc_row(v, half);
        if (row < rows) {
          const int dst = s_dst[row];
          if (dst >= 0) {
            float* o = out + static_cast<int64_t>(dst) * H + n0 + j;
            o[0] = acc[mb][0][v];
            o[32] = acc[mb][1][v];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = fma chain over slots k = 0..K-1 of g[t][k] * y[t*K+k],
// from +0, then fma(sg[t], shared_y[t], .); fp32, one bf16 rounding.
// One workgroup per token; each thread owns 4 consecutive hidden columns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ sy,
                                                      const float* __restrict__ sg,
                                                      float* __restrict__ out32,
                                                      uint16_t* __restrict__ out16, int64_t T,
                                                      int H, int K) {
  const int64_t t = blockIdx.x;
  float g[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) g[k] = k < K ? gate[t * K + k] : 0.f;
  const float sgt = sy ? sg[t] : 0.f;
  const float* yt = y + t * K * H;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K) {
        const f32x4v_t v = *reinterpret_cast<const f32x4v_t*>(yt + static_cast<int64_t>(k) * H + c);
        a0 = fmaf(g[k], v[0], a0);
        a1 = fmaf(g[k], v[1], a1);
        a2 = fmaf(g[k], v[2], a2);
        a3 = fmaf(g[k], v[3], a3);
      }
    }
    if (sy) {
      const f32x4v_t v = *reinterpret_cast<const f32x4v_t*>(sy + t * H + c);
      a0 = fmaf(sgt, v[0], a0);
      a1 = fmaf(sgt, v[1], a1);
      a2 = fmaf(sgt, v[2], a2);
      a3 = fmaf(sgt, v[3], a3);
    }
    if (out32) {
      f32x4v_t o;
      o[0] = a0;
      o[1] = a1;
      o[2] = a2;
      o[3] = a3;
      *reinterpret_cast<f32x4v_t*>(out32 + t * H + c) = o;
    }
    if (out16) {
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(a0)) | (static_cast<uint32_t>(f32_to_bf16(a1)) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(a2)) | (static_cast<uint32_t>(f32_to_bf16(a3)) << 16);
      uint2 pk;
      pk.x = lo;
      pk.y = hi;
      *reinterpret_cast<uint2*>(out16 + t * H + c) = pk;
    }
  }
}

}  // namespace moe

// ---------------------------------------------------------------------------
// launchers: the grouped-GEMM grids cover the largest possible work list
// (rounded up to whole rounds of the 8 XCDs); workgroups past the actual
// list, which lives on the device, exit at once.
// ---------------------------------------------------------------------------
namespace moe {

hipError_t launch_ffn_up(const uint16_t* x, const uint16_t* w13, const uint16_t* ws13,
                         const int32_t* offsets, const int32_t* sorted_route, const int32_t* tiles,
                         const int32_t* meta, uint16_t* act_hi, uint16_t* act_lo,
                         uint16_t* sact_hi, uint16_t* sact_lo, float* gu, float* sgu, int64_t T,
                         int H, int E, int K, int I, int Is, int max_tiles, hipStream_t stream) {
  const int ncol = (I > Is ? I : Is) / kUpCols;
  const int64_t items = static_cast<int64_t>(max_tiles) * ncol;
  const unsigned grid = static_cast<unsigned>(((items + 7) / 8) * 8);
  ffn_up_kernel<<<grid, 256, 0, stream>>>(x, w13, ws13, offsets, sorted_route, tiles, meta, act_hi,
                                          act_lo, sact_hi, sact_lo, gu, sgu, T, H, E, K, I, Is,
                                          ncol);
  return hipGetLastError();
}

hipError_t launch_ffn_down(const uint16_t* act_hi, const uint16_t* act_lo,
                           const uint16_t* sact_hi, const uint16_t* sact_lo, const uint16_t* w2,
                           const uint16_t* ws2, const int32_t* offsets,
                           const int32_t* sorted_route, const int32_t* tiles,
                           const int32_t* meta, float* y, float* sy, int64_t T, int H, int E,
                           int K, int I, int Is, int max_tiles, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(max_tiles) * (H / kDownCols);
  const unsigned grid = static_cast<unsigned>(((items + 7) / 8) * 8);
  ffn_down_kernel<<<grid, 256, 0, stream>>>(act_hi, act_lo, sact_hi, sact_lo, w2, ws2, offsets,
                                            sorted_route, tiles, meta, y, sy, T, H, E, K, I, Is);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* gate, const float* sy, const float* sg,
                          float* out32, uint16_t* out16, int64_t T, int H, int K,
                          hipStream_t stream) {
  combine_kernel<<<static_cast<unsigned>(T), 256, 0, stream>>>(y, gate, sy, sg, out32, out16, T, H,
                                                              K);
  return hipGetLastError();
}

}  // namespace moe
