// Device helpers shared by the gfx950 kernels of the routed MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

namespace moe {

// Routed rows per grouped-GEMM work item (two 32-row MFMA blocks).
constexpr int kRowsPerTile = 64;
// Rows per up-projection work item from this many tokens on (hidden size
// 2048): three 32-row MFMA blocks, so an expert's ~160 routes at 8K tokens
// stream its gate/up weights twice instead of three times.  The down
// projection keeps kRowsPerTile.
constexpr int kUpTallRows = 96;
constexpr int64_t kUpTallMin = 4096;
// Activation columns per up-projection work item (four waves x 32).
constexpr int kUpCols = 128;
// Hidden columns per down-projection work item (four waves x 32).
constexpr int kDownCols = 128;
// Tokens per block of the permutation's counting sort.
constexpr int kSortBlock = 256;
// 32-bit token-mask words (experts x ceil(tokens / 32)) of the one-workgroup
// counting sort; larger batches take the three-kernel sort.
constexpr int kSortSmallWords = 16384;
// Rows per row tile of the backward's grouped GEMMs (and the edge of their
// 128x128 output tiles).
constexpr int kBwdRowsPerTile = 128;
// bf16 planes carrying each fp32 backward GEMM operand (dGU, g*act): the
// exact three-way split of split3 (hi, mid, lo; hi + mid + lo == v).  The
// weight gradients take all three planes; the input-gradient GEMM takes the
// first kDxPlanes (hi + mid = v to 16 significant bits).
constexpr int kGradPlanes = 3;
constexpr int kDxPlanes = 2;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Non-temporal 16-byte vector load and store, for data that is streamed
// (read or written once): it then does not push the operands that other
// work items re-read out of the caches.
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// D = A(32x16) * B(16x32) + C on the matrix cores, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; it holds
// D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v.
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator that element v of lane `half` (= lane/32) holds.
__device__ __forceinline__ int acc_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.f;
  return z;
}

// Split a float into the bf16 pair (hi, lo) with hi = bf16(a), lo = bf16(a - hi).
__device__ __forceinline__ void split_hi_lo(float a, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(a);
  lo = f32_to_bf16(a - bf16_to_f32(hi));
}

// Split a float exactly into three bf16 parts p[0] + p[1] + p[2] (hi, mid,
// lo): each step rounds the remainder to bf16, and an fp32 significand has
// 24 bits, so the third remainder fits in bf16 exactly.
__device__ __forceinline__ void split3(float a, uint16_t (&p)[3]) {
  p[0] = f32_to_bf16(a);
  const float r1 = a - bf16_to_f32(p[0]);
  p[1] = f32_to_bf16(r1);
  p[2] = f32_to_bf16(r1 - bf16_to_f32(p[1]));
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Block-scaled FP8 expert weights (OCP MX: E4M3 element codes, one E8M0 scale
// code per 32 consecutive elements along the contraction axis): routed
// experts' codes and scales, then the shared expert's.
struct MxWeights {
  const uint8_t* q;
  const uint8_t* s;
  const uint8_t* sq;
  const uint8_t* ss;
};

// LoRA adapters of the routed experts: largest rank, and the fp32 stride of
// a row of shrink results z (one 64-byte row per sorted route position).
constexpr int kLoraMaxRank = 16;
// The expand half of one projection's adapters as the grouped-GEMM
// epilogue applies it: B [E][out][rank] bf16, the rows' shrink results as
// bf16 pairs zq [sorted position][hi, lo][kLoraMaxRank], the update's scale
// and the rank.
struct LoraExpand {
  const uint16_t* b;
  const uint16_t* zq;
  float scale;
  int rank;
};

// Copy the expand rows b[0 .. n) (rank bf16 each, packed; n * rank a
// multiple of 8 and b 16-byte aligned) into LDS as they are, 16 bytes per
// thread and step.
__device__ __forceinline__ void lora_stage_b(uint16_t* lds, const uint16_t* b, int n, int rank, int tid) {
  for (int i = tid; i < n * rank / 8; i += 256) st16(lds + 8 * i, ld16(b + 8 * i));
}

// MFMA B operand of expand row `row` from the packed LDS copy: elements
// j = 8 * half .. 8 * half + 7 of the row, zero past the rank.
__device__ __forceinline__ u32x4_t lora_b_operand(const uint16_t* lds, int row, int half, int rank) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j0 = 8 * half + 2 * i;
    const uint32_t e0 = j0 < rank ? lds[row * rank + j0] : 0u;
    const uint32_t e1 = j0 + 1 < rank ? lds[row * rank + j0 + 1] : 0u;
    w[i] = e0 | (e1 << 16);
  }
  return u32x4_t{w[0], w[1], w[2], w[3]};
}

// E8M0 scale code -> 2^(code - 127) as a float (code 0 is the denormal 2^-127).
__device__ __forceinline__ float e8m0_scale(uint32_t code) {
  return __uint_as_float(code ? (code << 23) : 0x00400000u);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Sixteen E4M3 codes (one 16-byte load, element i in byte i) times `scale`
// -> sixteen bf16 (elements 0..7 in lo, 8..15 in hi), with the gfx950
// scaled conversion.  For a power-of-two scale the result is exact: an E4M3
// value has at most 4 significant bits.
__device__ __forceinline__ void mx_dequant16(u32x4_t codes, float scale, u32x4_t& lo, u32x4_t& hi) {
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[q], scale, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[q], scale, true);
    o[2 * q] = __builtin_bit_cast(uint32_t, a);
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, b);
  }
  lo = u32x4_t{o[0], o[1], o[2], o[3]};
  hi = u32x4_t{o[4], o[5], o[6], o[7]};
}

// XCD-aware mapping of a 1-D grid onto `items` work items.  The hardware
// deals workgroups round-robin over the 8 XCDs (workgroup g runs on XCD g%8);
// this gives each XCD one contiguous range of items, so items that share
// operands (the N-tiles of one row tile, the row tiles of one expert) meet in
// the same L2.  Returns -1 for workgroups with no item.
__device__ __forceinline__ int xcd_item(int g, int items) {
  const int per = (items + 7) >> 3;
  const int xcd = g & 7, slot = g >> 3;
  if (slot >= per) return -1;
  const int it = xcd * per + slot;
  return it < items ? it : -1;
}

// Work item -> (row tile, column tile) of a grouped GEMM whose work list
// `tiles` holds (group, first row) pairs, each group's row tiles contiguous
// and in row order.  Items [first*ncol, (first+nrt)*ncol) belong to the group
// whose row tiles are first .. first+nrt-1 (so a group's items stay one
// contiguous range: one XCD under xcd_item); inside that range the column
// tile is the slow index, so the row tiles that stream the same weight slice
// are dispatched next to each other and share its reads in L2.
struct GroupItem {
  int tile, nt, grp, row0, seg0, cnt;
};
__device__ __forceinline__ GroupItem group_item(int item, int ncol, const int32_t* tiles,
                                                const int32_t* offsets, int E, int64_t T,
                                                int rows_per_tile) {
  GroupItem g;
  const int tg = item / ncol;
  g.grp = tiles[2 * tg];
  const int first = tg - tiles[2 * tg + 1] / rows_per_tile;
  const bool shared = g.grp == E;
  g.seg0 = shared ? 0 : offsets[g.grp];
  g.cnt = shared ? static_cast<int>(T) : offsets[g.grp + 1] - g.seg0;
  const int nrt = max(1, (g.cnt + rows_per_tile - 1) / rows_per_tile);
  const int local = item - first * ncol;
  g.nt = local / nrt;
  const int rt = local - g.nt * nrt;
  g.tile = first + rt;
  g.row0 = rt * rows_per_tile;
  return g;
}

}  // namespace moe
