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

// ---------------------------------------------------------------------------
// Operand staging shared by both projections.
//
// Every operand row segment of one 64-wide K block is 128 contiguous bytes.
// Loads are issued so that each wave instruction reads 8 rows x 128 bytes
// (lane l: row l/8, 16-byte chunk l%8) -- whole cache lines of a few rows.
// Measured on MI355X, MFMA-fragment-shaped loads (32 rows x 32 bytes per
// instruction) stay at ~4.6 TB/s where this pattern streams ~5.1 TB/s.
// Every work item walks its K blocks in ascending order: a synthetic
// weight-only stream is faster when concurrent items start at different K
// offsets, but in these kernels starting together keeps the gathered
// activation blocks of concurrent items in L2, which measured faster.
//
// In LDS a row of a K block takes 64 bf16 (128 bytes); its 16-byte chunk c
// is stored at position c ^ ((row >> 1) & 7), which makes both the 8x128-byte
// stores and the 32-row fragment reads of ds_*_b128 conflict-free.
// Inside a K block, MFMA K step s and lane half h use chunk 4h + s, i.e.
// k = 32h + 8s .. +8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// ---------------------------------------------------------------------------
// Up projection + SwiGLU.
// Work item = (row tile of 32 * MBT rows of one group, 128 activation
// columns).  Group g < E is routed expert g, its rows are the sorted
// positions offsets[g] + row0 ..; group E is the shared expert, rows are
// tokens row0 ...  Wave w owns activation columns c = nt*128 + 32w .. +32
// and computes both gate (W13 row c) and up (W13 row I + c) for every row of
// the tile, so the SwiGLU is elementwise on the two accumulators.  Its 64
// weight rows go through a private LDS area; the gathered activation rows
// through a double-buffered area shared by the four waves.  64-row tiles
// (96 rows at large batches) keep registers and LDS small enough for two
// workgroups per CU, which with the loads of the next K blocks in flight
// keeps enough bytes moving.
// Outputs: act as a bf16 hi/lo pair (row = sorted position, or token for the
// shared expert) and, if requested, the fp32 gate/up values.
// NKB > 0 instantiates the K loop fully unrolled for H = 64 * NKB with a
// ring of NSET register sets of loads (blocks kb + 1 .. kb + NSET - 1 are in
// flight while kb is multiplied); NKB = 0 is the general loop with one block
// in flight (NSET = 1).  All run the same MFMA sequence on every element.
// LORA adds a routed expert's adapter update to gate and up before the
// SwiGLU: g = fma(scale, t, g) with t = sum_j z[p][j] B13[col][j] (u likewise
// with row I + col of B13), t taken on the matrix cores as z_hi B^T + z_lo
// B^T over 16 zero-padded rank columns (z: the rows' shrink results as bf16
// pairs).
// ---------------------------------------------------------------------------
template <int NKB, int NSET, int MBT, bool MX, bool LORA>
__global__ __launch_bounds__(256, 2) void ffn_up_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const uint16_t* __restrict__ ws13, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_route, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, uint16_t* __restrict__ act_hi,
    uint16_t* __restrict__ act_lo, uint16_t* __restrict__ sact_hi,
    uint16_t* __restrict__ sact_lo, float* __restrict__ gu, float* __restrict__ sgu, const MxWeights mx,
    const LoraExpand lx, int64_t T, int H, int E, int K, int I, int Is, int ncol_tiles) {
  constexpr int ROWS = 32 * MBT;  // rows of a work item
  const int item = xcd_item(blockIdx.x, ntiles[0] * ncol_tiles);
  if (item < 0) return;
  const GroupItem gi = group_item(item, ncol_tiles, tiles, offsets, E, T, ROWS);
  const int nt = gi.nt, grp = gi.grp;
  const bool shared = grp == E;
  const int Ie = shared ? Is : I;
  if (nt * kUpCols >= Ie) return;
  const int seg0 = gi.seg0;
  const int cnt = gi.cnt;
  // 96-row work lists: a group's routes are cut into its ceil(cnt / 96) row
  // tiles of (almost) equal length, so that the tiles that stream the same
  // weight slice do the same work per K block and stay close enough for the
  // later ones to find it in L2 (a row's arithmetic does not depend on its
  // tile)
  int row0 = gi.row0, span = ROWS;
  if constexpr (MBT == kUpTallRows / 32) {
    const int nrt = max(1, (cnt + ROWS - 1) / ROWS);
    span = (cnt + nrt - 1) / nrt;  // <= ROWS
    row0 = (gi.row0 / ROWS) * span;
  }
  const int rows = min(span, cnt - row0);
  // the group's only row tile reads each of its weights once: stream them
  const bool wstream = cnt <= ROWS;
  if (rows <= 0) return;
  const int nmb = (rows + 31) >> 5;
  const uint16_t* W = shared ? ws13 : w13 + static_cast<int64_t>(grp) * 2 * I * H;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[4][64 * 64];
  __shared__ int s_tok[ROWS];
  // the item's rows of shrink results (bf16 hi | lo) and its expand rows
  // (gate columns, then up columns; rank bf16 each, packed)
  __shared__ __attribute__((aligned(16))) uint16_t zs[LORA ? ROWS * 2 * kLoraMaxRank : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lbs[LORA ? 2 * kUpCols * kLoraMaxRank : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, half = lane >> 5;
  const int64_t R = T * K;
  const bool lora = LORA && !shared;  // the shared expert has no adapter
  if (lora) {
    // ordered before the epilogue by the K loop's barriers
    for (int i = tid; i < rows * 4; i += 256)
      st16(&zs[8 * i], ld16(lx.zq + (static_cast<int64_t>(seg0) + row0) * 2 * kLoraMaxRank + 8 * i));
    // gate rows nt*128 .. +128, then up rows I + nt*128 .. +128
    const uint16_t* b0 = lx.b + (static_cast<int64_t>(grp) * 2 * I + nt * kUpCols) * lx.rank;
    lora_stage_b(lbs, b0, kUpCols, lx.rank, tid);
    lora_stage_b(lbs + kUpCols * lx.rank, b0 + static_cast<int64_t>(I) * lx.rank, kUpCols, lx.rank, tid);
  }

  if (tid < ROWS) {
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

  const int nkb = NKB > 0 ? NKB : H >> 6;
  // A loader: rows ar0 + 32q, chunk ac
  const int ac = tid & 7, ar0 = tid >> 3;
  const uint16_t* xa[MBT];
#pragma unroll
  for (int q = 0; q < MBT; ++q) xa[q] = x + static_cast<int64_t>(s_tok[ar0 + 32 * q]) * H + ac * 8;
  // B loader: this wave's gate rows (Bs rows 0..31) and up rows (32..63),
  // eight rows x 128 bytes per instruction
  const int bc = lane & 7, br8 = lane >> 3;
  const int col = nt * kUpCols + wave * 32 + j;
  const uint16_t* wgp = W + static_cast<int64_t>(nt * kUpCols + wave * 32 + br8) * H + bc * 8;
  const uint16_t* wup = wgp + static_cast<int64_t>(Ie) * H;
  // MX B loader: the same 64 rows as 16 rows x 64 code bytes per
  // instruction (lane: row 16q + bq, 16-byte piece cq), with each row's
  // scale code for the piece's 32-element half.  The unrolled loop reads a
  // row's scale codes 16 at a time (8 K blocks) into a pair of register
  // groups; the general loop one byte per block.
  const int cq = lane & 3, bq = lane >> 2;
  const uint8_t* mq[4];
  const uint8_t* ms[4];
  const uint8_t* msr[4];
  if constexpr (MX) {
    const uint8_t* Wq = shared ? mx.sq : mx.q + static_cast<int64_t>(grp) * 2 * I * H;
    const uint8_t* Wsc = shared ? mx.ss : mx.s + static_cast<int64_t>(grp) * 2 * I * (H / 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = (q < 2 ? 0 : Ie) + nt * kUpCols + wave * 32 + 16 * (q & 1) + bq;
      mq[q] = Wq + r * H + cq * 16;
      ms[q] = Wsc + r * (H / 32) + (cq >> 1);
      msr[q] = Wsc + r * (H / 32);
    }
  }
  u32x4_t sg[2][4];
  // scale codes of K blocks 8g .. 8g + 7 of the wave's rows
  auto load_scales = [&](int g) {
#pragma unroll
    for (int q = 0; q < 4; ++q) sg[g & 1][q] = ld16(msr[q] + 16 * g);
  };
  // scale code of block kb for row group q (compile-time kb)
  auto group_scale = [&](int kb, int q) {
    const uint32_t w = sg[(kb >> 3) & 1][q][(kb & 7) >> 1];
    return (w >> (8 * (2 * (kb & 1) + (cq >> 1)))) & 0xffu;
  };

  f32x16_t accg[MBT], accu[MBT];
#pragma unroll
  for (int mb = 0; mb < MBT; ++mb) {
    accg[mb] = zero16();
    accu[mb] = zero16();
  }
  u32x4_t ra[NSET][MBT], rb[NSET][8];
  u32x4_t rq[NSET][4];
  uint32_t rs[NSET][4];

  auto issue = [&](int set, int kb) {
    const int kp = kb << 6;
    // row blocks past the item's last row are neither loaded nor multiplied
#pragma unroll
    for (int q = 0; q < MBT; ++q)
      if (q < nmb) ra[set][q] = ld16(xa[q] + kp);
    if constexpr (MX) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rq[set][q] = wstream ? ld16_nt(mq[q] + kp) : ld16(mq[q] + kp);
        if constexpr (NKB == 0) rs[set][q] = ms[q][2 * kb];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (wstream) {
          rb[set][q] = ld16_nt(wgp + static_cast<int64_t>(8 * q) * H + kp);
          rb[set][4 + q] = ld16_nt(wup + static_cast<int64_t>(8 * q) * H + kp);
        } else {
          rb[set][q] = ld16(wgp + static_cast<int64_t>(8 * q) * H + kp);
          rb[set][4 + q] = ld16(wup + static_cast<int64_t>(8 * q) * H + kp);
        }
      }
    }
  };
  // blk: the K block being staged (compile-time in the unrolled loop)
  auto stash = [&](int set, int buf, int blk) {
#pragma unroll
    for (int q = 0; q < MBT; ++q)
      if (q < nmb) st16(&As[buf][lds_off(ar0 + 32 * q, ac)], ra[set][q]);
    if constexpr (MX) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4_t lo, hi;
        const uint32_t sc = NKB > 0 ? group_scale(blk, q) : rs[set][q];
        mx_dequant16(rq[set][q], e8m0_scale(sc), lo, hi);
        st16(&Bs[wave][lds_off(16 * q + bq, 2 * cq)], lo);
        st16(&Bs[wave][lds_off(16 * q + bq, 2 * cq + 1)], hi);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) st16(&Bs[wave][lds_off(8 * q + br8, bc)], rb[set][q]);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 4 * half + s;
      const u32x4_t bg = ld16(&Bs[wave][lds_off(j, c)]);
      const u32x4_t bu = ld16(&Bs[wave][lds_off(32 + j, c)]);
#pragma unroll
      for (int mb = 0; mb < MBT; ++mb) {
        if (mb < nmb) {
          const u32x4_t a = ld16(&As[buf][lds_off(mb * 32 + j, c)]);
          accg[mb] = mfma32x32x16(a, bg, accg[mb]);
          accu[mb] = mfma32x32x16(a, bu, accu[mb]);
        }
      }
    }
  };

  // The B area is private to the wave: overwriting it after the reads of
  // the previous block is ordered by the wave's own LDS instruction order.
  if constexpr (NKB > 0) {
    static_assert(!MX || NKB % 8 == 0, "scale codes are read 8 K blocks at a time");
    if constexpr (MX) {
      load_scales(0);
      if (NKB > 8) load_scales(1);
    }
#pragma unroll
    for (int q = 0; q < NSET && q < NKB; ++q) issue(q, q);
    stash(0, 0, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      __syncthreads();
      if (kb + NSET < NKB) issue(kb % NSET, kb + NSET);
      // group g's registers are free once block 8g + 7 is staged
      if (MX && (kb & 7) == 7 && kb + 9 < NKB) load_scales((kb >> 3) + 2);
      compute(kb & 1);
      if (kb + 1 < NKB) stash((kb + 1) % NSET, (kb + 1) & 1, kb + 1);
    }
  } else {
    issue(0, 0);
    stash(0, 0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
      __syncthreads();
      const int cur = kb & 1;
      const bool more = kb + 1 < nkb;
      if (more) issue(0, kb + 1);
      compute(cur);
      if (more) stash(0, cur ^ 1, kb + 1);
    }
  }

  uint16_t* ohi = shared ? sact_hi : act_hi;
  uint16_t* olo = shared ? sact_lo : act_lo;
  float* ogu = shared ? sgu : gu;
  const int64_t p0 = shared ? row0 : static_cast<int64_t>(seg0) + row0;
#pragma unroll
  for (int mb = 0; mb < MBT; ++mb) {
    if (mb < nmb) {
      if constexpr (LORA) {
        if (lora) {
          // expand on the matrix cores: t = z_hi B^T + z_lo B^T over the 16
          // (zero-padded) rank columns, then acc += scale * t
          const u32x4_t zh = ld16(&zs[(mb * 32 + j) * 2 * kLoraMaxRank + 8 * half]);
          const u32x4_t zl = ld16(&zs[(mb * 32 + j) * 2 * kLoraMaxRank + kLoraMaxRank + 8 * half]);
          const u32x4_t bg = lora_b_operand(lbs, wave * 32 + j, half, lx.rank);
          const u32x4_t bu = lora_b_operand(lbs, kUpCols + wave * 32 + j, half, lx.rank);
          const f32x16_t tg = mfma32x32x16(zl, bg, mfma32x32x16(zh, bg, zero16()));
#pragma unroll
          for (int v = 0; v < 16; ++v) accg[mb][v] = fmaf(lx.scale, tg[v], accg[mb][v]);
          const f32x16_t tu = mfma32x32x16(zl, bu, mfma32x32x16(zh, bu, zero16()));
#pragma unroll
          for (int v = 0; v < 16; ++v) accu[mb][v] = fmaf(lx.scale, tu[v], accu[mb][v]);
        }
      }
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
// (or token row of shared_y).  Work item = (row tile, 128 * NBW hidden
// columns); wave w owns columns nt*128*NBW + 32*NBW*w .. + 32*NBW, as NBW
// MFMA column blocks.  Same staging as the up projection: the wave's W2 rows
// through a private LDS area, the act planes through a double-buffered
// shared one.  Wider items (NBW = 2) read each act block once per 256
// columns and keep twice the weight bytes in flight per workgroup.
// NKB > 0 instantiates the K loop fully unrolled for Ie = 64 * NKB with a
// ring of NSET register sets of loads (blocks kb + 1 .. kb + NSET - 1 in
// flight while kb is multiplied); NKB = 0 is the general loop with one block
// in flight (NSET = 1).  All run the same MFMA sequence on every element.
// LORA adds a routed expert's adapter update to every element before it is
// stored: y = fma(scale, t, y) with t = sum_j z[p][j] B2[col][j] taken on the
// matrix cores as z_hi B2^T + z_lo B2^T over 16 zero-padded rank columns (z:
// the rows' shrink results as bf16 pairs).
// ---------------------------------------------------------------------------
template <int NKB, int NSET, int NBW, bool MX, bool LORA>
__global__ __launch_bounds__(256, 2) void ffn_down_kernel(
    const uint16_t* __restrict__ act_hi, const uint16_t* __restrict__ act_lo,
    const uint16_t* __restrict__ sact_hi, const uint16_t* __restrict__ sact_lo,
    const uint16_t* __restrict__ w2, const uint16_t* __restrict__ ws2,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_route,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta, float* __restrict__ y,
    float* __restrict__ sy, const MxWeights mx, const LoraExpand lx, int64_t T, int H, int E, int K,
    int I, int Is) {
  constexpr int COLS = kDownCols * NBW;  // hidden columns of a work item
  constexpr int WROWS = 32 * NBW;        // W2 rows (hidden columns) of a wave
  const int ncol_tiles = H / COLS;
  const int item = xcd_item(blockIdx.x, meta[0] * ncol_tiles);
  if (item < 0) return;
  const GroupItem gi = group_item(item, ncol_tiles, tiles, offsets, E, T, kRowsPerTile);
  const int nt = gi.nt, grp = gi.grp, row0 = gi.row0;
  const bool shared = grp == E;
  const int Ie = shared ? Is : I;
  const int seg0 = gi.seg0;
  const int cnt = gi.cnt;
  const int rows = min(kRowsPerTile, cnt - row0);
  // the group's only row tile reads each of its weights once: stream them
  const bool wstream = cnt <= kRowsPerTile;
  if (rows <= 0) return;
  const int nmb = (rows + 31) >> 5;
  const uint16_t* W = shared ? ws2 : w2 + static_cast<int64_t>(grp) * H * I;
  const int64_t p0 = shared ? row0 : static_cast<int64_t>(seg0) + row0;
  float* out = shared ? sy : y;

  // LDS: act planes [buf][hi/lo][64 rows x 64 k], then the waves' W2 rows;
  // the epilogue stages the fp32 tile over both
  constexpr int kAsElems = 2 * 2 * kRowsPerTile * 64;
  constexpr int kBsElems = 4 * WROWS * 64;
  static_assert((kAsElems + kBsElems) * 2 >= kRowsPerTile * COLS * 4, "the epilogue tile fits");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kAsElems + kBsElems];
  __shared__ int s_dst[kRowsPerTile];
  // the item's rows of shrink results (bf16 hi | lo) and the expand rows of
  // its hidden columns (rank bf16 each, packed)
  __shared__ __attribute__((aligned(16))) uint16_t zs[LORA ? kRowsPerTile * 2 * kLoraMaxRank : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lbs[LORA ? COLS * kLoraMaxRank : 8];
  auto As = [&](int buf, int plane) { return smem + (buf * 2 + plane) * kRowsPerTile * 64; };
  uint16_t* const Bw = smem + kAsElems + (threadIdx.x >> 6) * WROWS * 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, half = lane >> 5;
  const int64_t R = T * K;
  const bool lora = LORA && !shared;  // the shared expert has no adapter
  if (lora) {
    // ordered before the epilogue by the K loop's barriers
    for (int i = tid; i < rows * 4; i += 256)
      st16(&zs[8 * i], ld16(lx.zq + p0 * 2 * kLoraMaxRank + 8 * i));
    lora_stage_b(lbs, lx.b + (static_cast<int64_t>(grp) * H + nt * COLS) * lx.rank, COLS, lx.rank, tid);
  }

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

  const int nkb = NKB > 0 ? NKB : Ie >> 6;
  const int ac = tid & 7, ar0 = tid >> 3;
  const uint16_t* ahi = (shared ? sact_hi : act_hi) + p0 * Ie + ac * 8;
  const uint16_t* alo = (shared ? sact_lo : act_lo) + p0 * Ie + ac * 8;
  int64_t aoff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) aoff[q] = static_cast<int64_t>(min(ar0 + 32 * q, rows - 1)) * Ie;
  const int bc = lane & 7, br8 = lane >> 3;
  const int n0 = nt * COLS + wave * WROWS;
  const uint16_t* wb = W + static_cast<int64_t>(n0 + br8) * Ie + bc * 8;
  // MX B loader: the wave's rows as 16 rows x 64 code bytes per instruction
  // (lane: row 16q + bq, 16-byte piece cq) with the piece's scale code.  The
  // unrolled loop (Ie = 512: 16 scale codes per row) reads all of a row's
  // scale codes once; the general loop one byte per block.
  constexpr int NQ = WROWS / 16;
  const int cq = lane & 3, bq = lane >> 2;
  const uint8_t* mq[NQ];
  const uint8_t* ms[NQ];
  u32x4_t sall[NQ];
  if constexpr (MX) {
    const uint8_t* Wq = shared ? mx.sq : mx.q + static_cast<int64_t>(grp) * H * I;
    const uint8_t* Wsc = shared ? mx.ss : mx.s + static_cast<int64_t>(grp) * H * (I / 32);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t r = n0 + 16 * q + bq;
      mq[q] = Wq + r * Ie + cq * 16;
      ms[q] = Wsc + r * (Ie / 32) + (cq >> 1);
      if constexpr (NKB > 0) {
        static_assert(NKB == 8, "a row's scale codes are one 16-byte load");
        sall[q] = ld16(Wsc + r * (Ie / 32));
      }
    }
  }
  auto row_scale = [&](int kb, int q) {
    return (sall[q][kb >> 1] >> (8 * (2 * (kb & 1) + (cq >> 1)))) & 0xffu;
  };

  f32x16_t acc[2][NBW];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = zero16();
  u32x4_t rh[NSET][2], rl[NSET][2], rb[NSET][4 * NBW];
  u32x4_t rq[NSET][NQ];
  uint32_t rs[NSET][NQ];

  // activation rows past the tile's end repeat its last row (unused)
  auto issue = [&](int set, int kb) {
    const int kp = kb << 6;
    // row blocks past the item's last row are neither loaded nor multiplied
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q < nmb) {
        rh[set][q] = ld16(ahi + aoff[q] + kp);
        rl[set][q] = ld16(alo + aoff[q] + kp);
      }
    }
    if constexpr (MX) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        rq[set][q] = wstream ? ld16_nt(mq[q] + kp) : ld16(mq[q] + kp);
        if constexpr (NKB == 0) rs[set][q] = ms[q][2 * kb];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4 * NBW; ++q)
        rb[set][q] = wstream ? ld16_nt(wb + static_cast<int64_t>(8 * q) * Ie + kp)
                             : ld16(wb + static_cast<int64_t>(8 * q) * Ie + kp);
    }
  };
  // blk: the K block being staged (compile-time in the unrolled loop)
  auto stash = [&](int set, int buf, int blk) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q < nmb) {
        st16(As(buf, 0) + lds_off(ar0 + 32 * q, ac), rh[set][q]);
        st16(As(buf, 1) + lds_off(ar0 + 32 * q, ac), rl[set][q]);
      }
    }
    if constexpr (MX) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        u32x4_t lo, hi;
        const uint32_t sc = NKB > 0 ? row_scale(blk, q) : rs[set][q];
        mx_dequant16(rq[set][q], e8m0_scale(sc), lo, hi);
        st16(Bw + lds_off(16 * q + bq, 2 * cq), lo);
        st16(Bw + lds_off(16 * q + bq, 2 * cq + 1), hi);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4 * NBW; ++q) st16(Bw + lds_off(8 * q + br8, bc), rb[set][q]);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 4 * half + s;
      u32x4_t b[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) b[nb] = ld16(Bw + lds_off(32 * nb + j, c));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (mb < nmb) {
          const u32x4_t ah = ld16(As(buf, 0) + lds_off(mb * 32 + j, c));
          const u32x4_t al = ld16(As(buf, 1) + lds_off(mb * 32 + j, c));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            acc[mb][nb] = mfma32x32x16(ah, b[nb], acc[mb][nb]);
            acc[mb][nb] = mfma32x32x16(al, b[nb], acc[mb][nb]);
          }
        }
      }
    }
  };

  // The B area is private to the wave: overwriting it after the reads of
  // the previous block is ordered by the wave's own LDS instruction order.
  if constexpr (NKB > 0) {
#pragma unroll
    for (int q = 0; q < NSET && q < NKB; ++q) issue(q, q);
    stash(0, 0, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      __syncthreads();
      if (kb + NSET < NKB) issue(kb % NSET, kb + NSET);
      compute(kb & 1);
      if (kb + 1 < NKB) stash((kb + 1) % NSET, (kb + 1) & 1, kb + 1);
    }
  } else {
    issue(0, 0);
    stash(0, 0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
      __syncthreads();
      const int cur = kb & 1;
      const bool more = kb + 1 < nkb;
      if (more) issue(0, kb + 1);
      compute(cur);
      if (more) stash(0, cur ^ 1, kb + 1);
    }
  }

  // Epilogue: the 64 x COLS fp32 tile is staged in LDS and each route row
  // goes out as 16-byte pieces, COLS * 4 contiguous bytes per row.
  if constexpr (LORA) {
    if (lora) {
      // expand on the matrix cores: t = z_hi B2^T + z_lo B2^T over the 16
      // (zero-padded) rank columns, then acc += scale * t
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (mb < nmb) {
          const u32x4_t zh = ld16(&zs[(mb * 32 + j) * 2 * kLoraMaxRank + 8 * half]);
          const u32x4_t zl = ld16(&zs[(mb * 32 + j) * 2 * kLoraMaxRank + kLoraMaxRank + 8 * half]);
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const u32x4_t b = lora_b_operand(lbs, wave * WROWS + 32 * nb + j, half, lx.rank);
            const f32x16_t t = mfma32x32x16(zl, b, mfma32x32x16(zh, b, zero16()));
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mb][nb][v] = fmaf(lx.scale, t[v], acc[mb][nb][v]);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the operand areas
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb < nmb) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          Cs[(mb * 32 + acc_row(v, half)) * COLS + wave * WROWS + nb * 32 + j] = acc[mb][nb][v];
    }
  }
  __syncthreads();
  constexpr int kPieces = COLS / 4;           // 16-byte pieces per row
  constexpr int kRowsPerPass = 256 / kPieces;  // rows stored per pass of the workgroup
  const int piece = tid % kPieces;
#pragma unroll
  for (int i = 0; i < kRowsPerTile / kRowsPerPass; ++i) {
    const int r = tid / kPieces + kRowsPerPass * i;
    if (r < rows) {
      const int dst = s_dst[r];
      if (dst >= 0) st16_nt(out + static_cast<int64_t>(dst) * H + nt * COLS + piece * 4, ld16(Cs + r * COLS + piece * 4));
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = fma chain over slots k = 0..K-1 of g[t][k] * y[t*K+k],
// from +0, then fma(sg[t], shared_y[t], .); fp32, one bf16 rounding.
// One workgroup per token; each thread owns 4 consecutive hidden columns of
// every 1024-column chunk.  The K route rows (KT >= K slots, surplus slots
// re-read the last row and are not used) and the shared row of NC chunks
// (NC = H / 1024 when instantiated, else one chunk at a time) are all loaded
// before the chains, so their latencies overlap.
// ---------------------------------------------------------------------------
template <int KT, int NC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ sy,
                                                      const float* __restrict__ sg,
                                                      float* __restrict__ out32,
                                                      uint16_t* __restrict__ out16, int64_t T,
                                                      int H, int K) {
  // NC > 0: H = 1024 * NC, every column chunk's route rows loaded in one
  // batch; NC = 0: general H, one chunk at a time
  constexpr int NB = NC > 0 ? NC : 1;
  const int64_t t = blockIdx.x;
  float g[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) g[k] = gate[t * K + min(k, K - 1)];
  const float sgt = sy ? sg[t] : 0.f;
  const float* yt = y + t * K * H;
  const float* st = sy ? sy + t * H : yt;  // read (unused) when there is no shared expert
  for (int c0 = threadIdx.x * 4; c0 < H; c0 += 1024 * NB) {
    f32x4v_t v[NB][KT], vs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = min(c0 + 1024 * b, H - 4);
#pragma unroll
      for (int k = 0; k < KT; ++k)
        v[b][k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(yt + static_cast<int64_t>(min(k, K - 1)) * H + c));
      vs[b] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(st + c));
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = c0 + 1024 * b;
      if (c >= H) break;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        if (k < K) {
          a0 = fmaf(g[k], v[b][k][0], a0);
          a1 = fmaf(g[k], v[b][k][1], a1);
          a2 = fmaf(g[k], v[b][k][2], a2);
          a3 = fmaf(g[k], v[b][k][3], a3);
        }
      }
      if (sy) {
        a0 = fmaf(sgt, vs[b][0], a0);
        a1 = fmaf(sgt, vs[b][1], a1);
        a2 = fmaf(sgt, vs[b][2], a2);
        a3 = fmaf(sgt, vs[b][3], a3);
      }
      if (out32) {
        f32x4v_t o;
        o[0] = a0;
        o[1] = a1;
        o[2] = a2;
        o[3] = a3;
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4v_t*>(out32 + t * H + c));
      }
      if (out16) {
        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(a0)) | (static_cast<uint32_t>(f32_to_bf16(a1)) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(a2)) | (static_cast<uint32_t>(f32_to_bf16(a3)) << 16);
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(out16 + t * H + c));
      }
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
                         const MxWeights* mx, const LoraExpand* lora, const int32_t* offsets,
                         const int32_t* sorted_route, const int32_t* tiles, const int32_t* ntiles,
                         int up_rows, uint16_t* act_hi, uint16_t* act_lo, uint16_t* sact_hi,
                         uint16_t* sact_lo, float* gu, float* sgu, int64_t T, int H, int E, int K,
                         int I, int Is, int max_tiles, hipStream_t stream) {
  const int ncol = (I > Is ? I : Is) / kUpCols;
  const int64_t items = static_cast<int64_t>(max_tiles) * ncol;
  const unsigned grid = static_cast<unsigned>(((items + 7) / 8) * 8);
  const MxWeights m = mx ? *mx : MxWeights{nullptr, nullptr, nullptr, nullptr};
  const LoraExpand lx = lora ? *lora : LoraExpand{nullptr, nullptr, 0.f, 0};
#define MOE_UP_ONE(NKB, NSET, MBT, MX, LORA)                                                          \
  ffn_up_kernel<NKB, NSET, MBT, MX, LORA><<<grid, 256, 0, stream>>>(                                 \
      x, w13, ws13, offsets, sorted_route, tiles, ntiles, act_hi, act_lo, sact_hi, sact_lo, gu, sgu, \
      m, lx, T, H, E, K, I, Is, ncol)
#define MOE_UP(NKB, NSET, MBT)                      \
  do {                                              \
    if (mx)                                         \
      MOE_UP_ONE(NKB, NSET, MBT, true, false);      \
    else if (lora)                                  \
      MOE_UP_ONE(NKB, NSET, MBT, false, true);      \
    else                                            \
      MOE_UP_ONE(NKB, NSET, MBT, false, false);     \
  } while (0)
  // the unrolled instantiations cover hidden size 2048 (64- and 96-row items)
  if (H == 2048 && up_rows == kUpTallRows)
    MOE_UP(32, 2, kUpTallRows / 32);
  else if (H == 2048)
    MOE_UP(32, 2, kRowsPerTile / 32);
  else
    MOE_UP(0, 1, kRowsPerTile / 32);
#undef MOE_UP
#undef MOE_UP_ONE
  return hipGetLastError();
}

hipError_t launch_ffn_down(const uint16_t* act_hi, const uint16_t* act_lo,
                           const uint16_t* sact_hi, const uint16_t* sact_lo, const uint16_t* w2,
                           const uint16_t* ws2, const MxWeights* mx, const LoraExpand* lora,
                           const int32_t* offsets, const int32_t* sorted_route,
                           const int32_t* tiles, const int32_t* meta, float* y, float* sy,
                           int64_t T, int H, int E, int K, int I, int Is, int max_tiles,
                           hipStream_t stream) {
  const MxWeights m = mx ? *mx : MxWeights{nullptr, nullptr, nullptr, nullptr};
  const LoraExpand lx = lora ? *lora : LoraExpand{nullptr, nullptr, 0.f, 0};
#define MOE_DOWN_ONE(NKB, NSET, NBW, MX, LORA)                                                       \
  ffn_down_kernel<NKB, NSET, NBW, MX, LORA><<<grid, 256, 0, stream>>>(                              \
      act_hi, act_lo, sact_hi, sact_lo, w2, ws2, offsets, sorted_route, tiles, meta, y, sy, m, lx, \
      T, H, E, K, I, Is)
#define MOE_DOWN(NKB, NSET, NBW, COLS)                                                  \
  do {                                                                                \
    const int64_t items = static_cast<int64_t>(max_tiles) * (H / (COLS));             \
    const unsigned grid = static_cast<unsigned>(((items + 7) / 8) * 8);               \
    if (mx)                                                                           \
      MOE_DOWN_ONE(NKB, NSET, NBW, true, false);                                      \
    else if (lora)                                                                    \
      MOE_DOWN_ONE(NKB, NSET, NBW, false, true);                                      \
    else                                                                              \
      MOE_DOWN_ONE(NKB, NSET, NBW, false, false);                                     \
  } while (0)
  // the unrolled instantiation covers expert and shared sizes of 512 (and
  // takes 256-column items when H allows); the general one 128 columns
  if (I == 512 && (Is == 0 || Is == 512) && H % (2 * kDownCols) == 0)
    MOE_DOWN(8, 2, 2, 2 * kDownCols);
  else
    MOE_DOWN(0, 1, 1, kDownCols);
#undef MOE_DOWN
#undef MOE_DOWN_ONE
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* gate, const float* sy, const float* sg,
                          float* out32, uint16_t* out16, int64_t T, int H, int K,
                          hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(T);
  if (K <= 10 && H == 2048)
    combine_kernel<10, 2><<<grid, 256, 0, stream>>>(y, gate, sy, sg, out32, out16, T, H, K);
  else if (K <= 10)
    combine_kernel<10, 0><<<grid, 256, 0, stream>>>(y, gate, sy, sg, out32, out16, T, H, K);
  else
    combine_kernel<16, 0><<<grid, 256, 0, stream>>>(y, gate, sy, sg, out32, out16, T, H, K);
  return hipGetLastError();
}

}  // namespace moe
