// Backward kernels of the routed MoE layer (gfx950).
//
// Backward bullet of the "MoE route/combine contract" commit (RL-Kernel pull
// request 557 page): weight gradients of every expert into one dense buffer,
// and each token's input gradient summed over its routes in ascending expert
// id.  The route-weight gradient is a per-token reduction with a fixed order
// (the page's H100 results note that a library sum over the hidden size was
// not batch invariant; here the order never depends on the batch).  There
// are no atomics: every output element has exactly one writer, and every sum
// runs in a fixed order.
//
// Precision: products of bf16 values are exact on the matrix cores; an fp32
// operand (activation gradients, gate-scaled activations) enters the weight
// gradients exactly, as three bf16 planes (hi + mid + lo == v), one MFMA per
// plane, and the input gradient as the first two (16 significant bits of v).
// The grouped GEMMs accumulate in fp32 on the matrix cores in a fixed K
// order; the small reductions (route weights, shared gate, router weights)
// accumulate in fp64.
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Route-weight and shared-gate gradients.
// dg[k] = <dOut[t], y[t*K+k]> and ds = <dOut[t], shared_y[t]>.  Since
// y = W2_e act, the same value is <W2_e^T dOut[t], act>, a sum over the
// intermediate dimension: the dact GEMM's epilogue forms it from its fp32
// product D = dOut W2_e and the fp32 activation recomputed from the saved
// gate/up values, as fp64 partial sums per 128-column tile (part[r][nt],
// nt < Ie / 128).  Here they are added in ascending tile order in fp64.
// dl[k] = g_k (dg_k - sum_j g_j dg_j) (softmax backward over the selected
// slots); dz = ds * sg * (1 - sg).
// One thread per route (a workgroup takes 256 / K whole tokens): it forms
// its dg[k] and leaves it and its gate in LDS; every thread of a token then
// forms sum_j g_j dg_j as an fma chain in ascending j (the same chain in
// every one of them) and its dl[k]; the token's first thread forms dz.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_gate_kernel(const double* __restrict__ dgp,
                                                       const double* __restrict__ dsp,
                                                       const float* __restrict__ gate,
                                                       const float* __restrict__ sg,
                                                       float* __restrict__ dl,
                                                       float* __restrict__ dz, int64_t T, int K,
                                                       int nt_route, int nt_shared, int nt_stride) {
  __shared__ double s_g[256], s_dg[256];
  const int per = 256 / K;  // tokens per workgroup
  const int lt = threadIdx.x / K, k = threadIdx.x - lt * K;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * per + lt;
  const bool live = lt < per && t < T;
  double dg = 0.0, g = 0.0;
  if (live) {
    const double* pr = dgp + (t * K + k) * nt_stride;
    for (int n = 0; n < nt_route; ++n) dg += pr[n];
    g = gate[t * K + k];
    s_g[threadIdx.x] = g;
    s_dg[threadIdx.x] = dg;
  }
  __syncthreads();
  if (!live) return;
  double mean = 0.0;
  for (int q = 0; q < K; ++q) mean = fma(s_g[lt * K + q], s_dg[lt * K + q], mean);
  dl[t * K + k] = static_cast<float>(g * (dg - mean));
  if (dsp && k == 0) {
    double ds = 0.0;
    for (int n = 0; n < nt_shared; ++n) ds += dsp[t * nt_stride + n];
    const double s = sg[t];
    dz[t] = static_cast<float>(ds * s * (1.0 - s));
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMMs of the expert backward: D[m][n] = sum_k A[m][k] B[k][n] over
// 32-wide K blocks, accumulated in fp32 on the matrix cores (MFMA 32x32x16).
// The input-gradient GEMMs (kDact, kDx: bwd_gemm_kernel) take 128x128
// output tiles, four waves in a 2x2 grid each owning a 64x64 block; the
// weight gradients (kDw2, kDw13: bwd_wgrad_kernel) take 256x128 / 128x256
// tiles, described with that kernel.
//
// bwd_gemm_kernel stages its operands in LDS, two stages: the next K block's
// global loads are issued before the current block's MFMAs and stored to the
// other stage after them, so one barrier per block separates the stages.
// Two LDS layouts:
//   * [row][k] (64-byte rows, XOR-swizzled 16-byte pieces: rk_off) for
//     sources stored k-contiguous (the routed or token rows of a dgrad);
//     fragments are 16-byte LDS loads;
//   * [k][col] (256-byte rows, XOR-swizzled 64-byte quarters: rc_off) for
//     sources whose rows are indexed by k (the expert weights read along
//     their output dimension, and both operands of a weight gradient, whose
//     contraction runs over the routes of an expert).  Rows are stored as
//     the 16-byte pieces they are loaded in and fragments are read with the
//     gfx950 LDS transpose read (ds_read_b64_tr_b16), two per fragment.
// An fp32 operand (dGU, g*act) is given as kGradPlanes bf16 planes, its
// exact split hi + mid + lo, and takes one MFMA per plane per K step in plane
// order: all three in the weight gradients, hi and mid in kDx.
//
// Modes (group g: routed expert g < E, shared expert g == E; p = row of the
// group's segment in sorted order, t(p) its token):
//   kDact: m = p (128-row tile), n = i < Ie, k = h < H.  A = dOut[t(p)][h]
//          ([row][k]); B = W2_g[h][i] ([k][col]).  Epilogue: dact = D * g_p,
//          SwiGLU backward with the saved gate/up pre-activations -> dGU
//          planes [p][2Ie] and g_p*act planes [p][Ie]; and the partial
//          route-weight gradient sum_i D[p][i] act[p][i] over the tile's
//          columns, fp64, in dgp[r][nt] (routed, r = sorted_route[p]) or
//          dsp[t][nt] (shared).
//   kDx:   m = p, n = h < H, k = j < 2Ie.  A = dGU planes ([row][k]);
//          B = W13_g[j][h] ([k][col]).  Epilogue: row of dx_route (route row
//          sorted_route[p]) or of dx_shared (token row).
//   kDw2:  m = h < H, n = i < Ie, k = p over the segment.  A = dOut[t(p)][h]
//          ([k][col], gathered rows); B = g*act planes [p][i] ([k][col]).
//          Epilogue: dW2_g[h][i].
//   kDw13: m = j < 2Ie, n = h < H, k = p.  A = dGU planes [p][j] ([k][col]);
//          B = x[t(p)][h] ([k][col], gathered rows).  Epilogue: dW13_g[j][h].
// The K order of every output element is fixed: K blocks in ascending order,
// in each block K step 0 then 1, and in each step the planes in order.  A
// dgrad row's result therefore depends only on its own row and its expert,
// never on the batch.
// ---------------------------------------------------------------------------
enum BwdMode { kDact = 0, kDx = 1, kDw2 = 2, kDw13 = 3 };

constexpr int kBT = kBwdRowsPerTile;  // edge of a dgrad tile and of the weight gradients' narrow side (128)
constexpr int kBwdTokLds = 256;       // weight-gradient segments up to this length keep their tokens in LDS
constexpr int kDactChunk = 16;        // K blocks per chunk of the general dact loop's two-level sum
constexpr int kBK = 32;
// [row][k] layout: 64-byte rows (32 k), 16-byte piece c of a row stored at
// c ^ ((row >> 2) & 3), which keeps both the loaders' stores (4 rows x 4
// pieces per 16 lanes) and the 32-row fragment reads free of bank conflicts.
__device__ __forceinline__ int rk_off(int row, int c) { return row * kBK + ((c ^ ((row >> 2) & 3)) << 3); }
// [k][col] layout: 128 columns per row; the 64-byte quarter of row `row`
// that holds column `col` is stored at quarter (col / 32) ^ (row % 4).  A
// transpose read's 32 lanes of a half-wave take 64 bytes of each of four
// consecutive rows (4-aligned), which the swizzle spreads over the four
// quarters, i.e. all 64 banks once; unswizzled 256-byte rows put them on
// the same 16 banks (measured with the LDS bank-conflict counter).  The
// loaders write whole 256-byte rows per 16 lanes, conflict-free either way.
constexpr int kRStride = 128;
__device__ __forceinline__ int rc_off(int row, int col) { return row * kRStride + (col ^ ((row & 3) << 5)); }
constexpr int kKPlane = kBT * kBK;
constexpr int kRPlane = kBK * kRStride;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// MFMA operand for lane `lane` from a [k][col] LDS plane: column
// col0 + lane%32, k = k0 + 8*(lane/32) .. +8.  Each transpose read gathers,
// in a group of 16 lanes, a 4x4 block of 16-bit elements (4 k rows x 4
// columns per lane address) and hands lane i the column i of it; the lane
// addresses below make the 16 columns of a group consecutive.
__device__ __forceinline__ u32x4_t frag_tr(const uint16_t* plane, int k0, int col0, int lane) {
  const int L = lane & 15;
  const int row = k0 + 8 * (lane >> 5) + (L >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
  // rows row and row + 4 share the swizzle
  const uint16_t* p = plane + rc_off(row, col);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p + 4 * kRStride));
  const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(u32x4_t, v);
}

struct BwdArgs {
  int64_t T;
  int H, E, K, I, Is;
  const int32_t* offsets;
  const int32_t* sorted_route;
  const float* gate;
  const float* sg;
  const int32_t* tiles;
  const int32_t* meta;
  const uint16_t* x;
  const uint16_t* dout;
  const uint16_t* w13;
  const uint16_t* w2;
  const uint16_t* ws13;
  const uint16_t* ws2;
  const float* gu;
  const float* sgu;
  uint16_t* dgu[kGradPlanes];    // planes of dGU [R][2I]
  uint16_t* sdgu[kGradPlanes];   // [T][2Is]
  uint16_t* gact[kGradPlanes];   // planes of g*act [R][I]
  uint16_t* sgact[kGradPlanes];  // [T][Is]
  double* dgp;                   // [R][nt_stride] partial <D, act> per column tile (routed)
  double* dsp;                   // [T][nt_stride] (shared)
  int nt_stride;
  float* dx_route;
  float* dx_shared;
  float* dw13;
  float* dw2;
  float* dws13;
  float* dws2;
  // LoRA term of the dgrad epilogues (LORA instantiations): the rows' shrink
  // results as bf16 pairs lzq [p][hi, lo][kLoraMaxRank] and the matrix
  // lbx [E][rank][out] they multiply (the adapter's A, row-major, out = the
  // GEMM's output columns)
  const uint16_t* lzq;
  const uint16_t* lbx;
  float lscale;
  int lrank;
};

// Work item of a grouped-GEMM launch.
struct BwdTile {
  int grp, m0, n0, nt;
  int rows;  // valid rows (dgrad) / contraction length (weight gradients)
  int seg0;  // first sorted position of the group (0 for the shared group)
  bool shared;
  bool wstream;  // dgrad: the group's only row tile, which reads each weight once
  int Ie;
};

template <int MODE>
__device__ __forceinline__ bool bwd_decode(const BwdArgs& a, int g, BwdTile& w) {
  static_assert(MODE == kDact || MODE == kDx, "dgrad modes");
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int ncol = MODE == kDact ? Imax / kBT : a.H / kBT;
  const int item = xcd_item(g, a.meta[0] * ncol);
  if (item < 0) return false;
  const int tile = item / ncol;
  w.nt = item - tile * ncol;
  w.grp = a.tiles[2 * tile];
  w.m0 = a.tiles[2 * tile + 1];
  w.n0 = w.nt * kBT;
  w.shared = w.grp == a.E;
  w.Ie = w.shared ? a.Is : a.I;
  if (MODE == kDact && w.n0 >= w.Ie) return false;
  w.seg0 = w.shared ? 0 : a.offsets[w.grp];
  const int cnt = w.shared ? static_cast<int>(a.T) : a.offsets[w.grp + 1] - w.seg0;
  w.rows = min(kBT, cnt - w.m0);
  w.wstream = cnt <= kBT;
  return w.rows > 0;
}

// token of sorted row p of a group (route ids outside [0, T*K) map to token 0)
__device__ __forceinline__ int64_t bwd_token(const BwdArgs& a, const BwdTile& w, int64_t p) {
  if (w.shared) return p;
  const int64_t r = a.sorted_route[p];
  return (r >= 0 && r < a.T * a.K) ? r / a.K : 0;
}

// LoRA term of a dgrad tile (routed groups; kDact: z = B2^T dOut with the
// adapter's A2, kDx: z = B13^T dGU with A13): the tile's rows' shrink
// results, bf16 hi | lo, into zs [128 rows][2][kLoraMaxRank] (zeros past
// the tile's rows), and the adapter matrix's rank rows for the tile's 128
// columns into lbs [rank][128].  nout: the adapter matrix's row length.
__device__ __forceinline__ void lora_stage_tile(const BwdArgs& a, const BwdTile& w, uint16_t* zs, uint16_t* lbs,
                                                int64_t nout, int tid) {
  const uint16_t* z0 = a.lzq + (static_cast<int64_t>(w.seg0) + w.m0) * 2 * kLoraMaxRank;
  for (int q = tid; q < kBT * 4; q += 256)
    st16(&zs[8 * q], q < w.rows * 4 ? ld16(z0 + 8 * q) : u32x4_t{0u, 0u, 0u, 0u});
  const uint16_t* b0 = a.lbx + static_cast<int64_t>(w.grp) * a.lrank * nout + w.n0;
  for (int q = tid; q < a.lrank * (kBT / 8); q += 256) {
    const int j = q / (kBT / 8), c = q - j * (kBT / 8);
    st16(&lbs[j * kBT + 8 * c], ld16(b0 + j * nout + 8 * c));
  }
}
// acc = fma(scale, z A, acc) on a wave's 64 x 64 block (2 x 2 MFMA blocks),
// the product as z_hi A then z_lo A over the 16 zero-padded rank columns.
__device__ __forceinline__ void lora_add_tile(const BwdArgs& a, const uint16_t* zs, const uint16_t* lbs,
                                              f32x16_t (&acc)[2][2], int wm, int wn, int lane) {
  const int i = lane & 31, half = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int zr = wm * 64 + mb * 32 + i;
    const u32x4_t zh = ld16(&zs[zr * 2 * kLoraMaxRank + 8 * half]);
    const u32x4_t zl = ld16(&zs[zr * 2 * kLoraMaxRank + kLoraMaxRank + 8 * half]);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // B[k][n] = A[k][n0 + col] for k < rank, else 0
      const int col = wn * 64 + nb * 32 + i;
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j0 = 8 * half + 2 * q;
        const uint32_t e0 = j0 < a.lrank ? lbs[j0 * kBT + col] : 0u;
        const uint32_t e1 = j0 + 1 < a.lrank ? lbs[(j0 + 1) * kBT + col] : 0u;
        bw[q] = e0 | (e1 << 16);
      }
      const u32x4_t b{bw[0], bw[1], bw[2], bw[3]};
      const f32x16_t t = mfma32x32x16(zl, b, mfma32x32x16(zh, b, zero16()));
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = fmaf(a.lscale, t[v], acc[mb][nb][v]);
    }
  }
}

// dact epilogue of one 64-row half (hh) of a tile and one 128-column group
// (columns n0 .. n0 + 127, column tile nt of the partial route-weight
// gradients), from the fp32 GEMM result staged at ep (row stride ES floats):
// each thread takes 8 consecutive columns of four rows for the SwiGLU
// backward, so the saved pre-activations are read and the gradient planes
// written 16 bytes at a time.
__device__ __forceinline__ void dact_epilogue(const BwdArgs& a, const BwdTile& w, const float* ep, int ES, int n0,
                                              int nt, int hh, int tid) {
  const int Ie = w.Ie;
  const int er = tid >> 4, ec = (tid & 15) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int lrow = hh * 64 + er + 16 * c;
    if (lrow >= w.rows) continue;
    float g;
    int64_t rowp;
    if (w.shared) {
      rowp = w.m0 + lrow;
      g = a.sg[rowp];
    } else {
      rowp = static_cast<int64_t>(w.seg0) + w.m0 + lrow;
      const int64_t r = a.sorted_route[rowp];
      g = (r >= 0 && r < a.T * a.K) ? a.gate[r] : 0.f;
    }
    const int col = n0 + ec;
    const float* gur = (w.shared ? a.sgu : a.gu) + rowp * 2 * Ie;
    const f32x4v_t* dsrc = reinterpret_cast<const f32x4v_t*>(ep + (er + 16 * c) * ES + ec);
    const f32x4v_t d0 = dsrc[0], d1 = dsrc[1];
    const f32x4v_t g0 = *reinterpret_cast<const f32x4v_t*>(gur + col);
    const f32x4v_t g1 = *reinterpret_cast<const f32x4v_t*>(gur + col + 4);
    const f32x4v_t u0 = *reinterpret_cast<const f32x4v_t*>(gur + Ie + col);
    const f32x4v_t u1 = *reinterpret_cast<const f32x4v_t*>(gur + Ie + col + 4);
    uint32_t pg[kGradPlanes][4], pu[kGradPlanes][4], pa[kGradPlanes][4];
    double dot = 0.0;  // this thread's 8 columns of <D, act>
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dv = e < 4 ? d0[e] : d1[e - 4];
      const float gv = e < 4 ? g0[e] : g1[e - 4];
      const float uv = e < 4 ? u0[e] : u1[e - 4];
      const float dact = dv * g;
      const float sgm = 1.0f / (1.0f + expf(-gv));
      const float dgate = dact * uv * sgm * (1.0f + gv * (1.0f - sgm));
      const float silu = silu_f32(gv);
      const float dup = dact * silu;
      const float act = silu * uv;
      const float gact = g * act;
      dot = fma(static_cast<double>(dv), static_cast<double>(act), dot);
      uint16_t sgp[3], sup[3], sap[3];
      split3(dgate, sgp);
      split3(dup, sup);
      split3(gact, sap);
      const int sh = 16 * (e & 1);
#pragma unroll
      for (int q = 0; q < kGradPlanes; ++q) {
        if ((e & 1) == 0) {
          pg[q][e >> 1] = sgp[q];
          pu[q][e >> 1] = sup[q];
          pa[q][e >> 1] = sap[q];
        } else {
          pg[q][e >> 1] |= static_cast<uint32_t>(sgp[q]) << sh;
          pu[q][e >> 1] |= static_cast<uint32_t>(sup[q]) << sh;
          pa[q][e >> 1] |= static_cast<uint32_t>(sap[q]) << sh;
        }
      }
    }
    // the 16 threads of this row (consecutive lanes) add their partial
    // sums in a fixed butterfly; the first writes the tile's sum
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 16);
    if ((tid & 15) == 0) {
      if (w.shared) {
        a.dsp[rowp * a.nt_stride + nt] = dot;
      } else {
        const int64_t r = a.sorted_route[rowp];
        if (r >= 0 && r < a.T * a.K) a.dgp[r * a.nt_stride + nt] = dot;
      }
    }
#pragma unroll
    for (int q = 0; q < kGradPlanes; ++q) {
      uint16_t* dq = (w.shared ? a.sdgu[q] : a.dgu[q]) + rowp * 2 * Ie;
      st16(dq + col, u32x4_t{pg[q][0], pg[q][1], pg[q][2], pg[q][3]});
      st16(dq + Ie + col, u32x4_t{pu[q][0], pu[q][1], pu[q][2], pu[q][3]});
      st16((w.shared ? a.sgact[q] : a.gact[q]) + rowp * Ie + col,
           u32x4_t{pa[q][0], pa[q][1], pa[q][2], pa[q][3]});
    }
  }
}

// The input-gradient GEMMs kDact and kDx for the shapes without a
// specialised kernel (bwd_dact_k64_kernel takes dact at hidden 2048,
// bwd_dx_wide_kernel dx at intermediate 512): a general K loop with the next
// block's loads in flight.  dact sums its long contraction in chunks of
// kDactChunk K blocks (below).
// LORA (routed groups): before the epilogue the routed rows'
// LoRA term is added on the matrix cores, acc = fma(scale, z A, acc) with z
// the rows' shrink results (bf16 hi + lo, two MFMAs) and A the adapter's
// rank x 128 slice of the tile's columns (zero past the rank).  kDact takes
// z = B2^T dOut and A2, so D + s A2^T B2^T dOut is the gradient of act and
// dact = g (D + s A2^T B2^T dOut) and the route-weight gradient
// <D + s A2^T B2^T dOut, act> include the adapter; kDx takes z = B13^T dGU
// and A13.
template <int MODE, bool LORA = false>
__global__ __launch_bounds__(256, 2) void bwd_gemm_kernel(const BwdArgs a) {
  static_assert(MODE == kDact || MODE == kDx, "dgrad modes");
  constexpr int NPA = MODE == kDx ? kDxPlanes : 1;
  constexpr int NPB = 1;
  constexpr int APLANE = kKPlane;
  constexpr int STAGE = NPA * APLANE + NPB * kRPlane;
  constexpr int NSTAGE = 2;
  // the epilogue stages a 64-row half of the fp32 tile (stride kBT + 4) in
  // the same area
  constexpr int EPI = 64 * (kBT + 4) * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI];
  // LoRA: the tile's rows' shrink results and its columns' expand rows
  __shared__ __attribute__((aligned(16))) uint16_t zs[LORA ? kBT * 2 * kLoraMaxRank : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lbs[LORA ? kLoraMaxRank * kBT : 8];

  BwdTile w;
  if (!bwd_decode<MODE>(a, blockIdx.x, w)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int Ie = w.Ie;
  const bool lora = LORA && !w.shared;  // the shared expert has no adapter
  // ordered before the epilogue by the K loop's barriers
  if (lora) lora_stage_tile(a, w, zs, lbs, MODE == kDact ? a.I : a.H, tid);

  const int kdim = MODE == kDact ? a.H : 2 * Ie;
  const int nkb = (kdim + kBK - 1) / kBK;

  // ---- load roles.  [row][k] operand (A): rows lr + 64c, 8 k at lc.
  // [k][col] operand (B): k rows kr + 16c, 8 columns at tc.
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const int kr = tid >> 4, tc = (tid & 15) * 8;

  // dgrad A: element offsets of this thread's two rows in the source
  int64_t a_off[2] = {0, 0};
  const uint16_t* a_base[NPA];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int rr = min(lr + 64 * c, w.rows - 1);
    if (MODE == kDact) {
      a_off[c] = bwd_token(a, w, static_cast<int64_t>(w.seg0) + w.m0 + rr) * a.H;
    } else {
      const int64_t rowp = w.shared ? (w.m0 + rr) : (static_cast<int64_t>(w.seg0) + w.m0 + rr);
      a_off[c] = rowp * 2 * Ie;
    }
  }
  if (MODE == kDact) {
    a_base[0] = a.dout;
  } else {
#pragma unroll
    for (int q = 0; q < NPA; ++q) a_base[q] = w.shared ? a.sdgu[q] : a.dgu[q];
  }
  // dgrad B: the expert's weight, rows indexed by k
  const uint16_t* wbase = nullptr;
  int wcols = 0;
  if (MODE == kDact) {
    wbase = w.shared ? a.ws2 : a.w2 + static_cast<int64_t>(w.grp) * a.H * a.I;
    wcols = Ie;
  }
  if (MODE == kDx) {
    wbase = w.shared ? a.ws13 : a.w13 + static_cast<int64_t>(w.grp) * 2 * a.I * a.H;
    wcols = a.H;
  }

  u32x4_t ra_set[1][NPA][2], rb_set[1][NPB][2];
  // dgrad operands of K block kb: A (routed or token rows) and B (weight)
  auto fetch_a = [&](int set, int kb) {
#pragma unroll
    for (int q = 0; q < NPA; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c) ra_set[set][q][c] = ld16(a_base[q] + a_off[c] + kb * kBK + lc);
  };
  auto fetch_b = [&](int set, int kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t* wp = wbase + static_cast<int64_t>(kb * kBK + kr + 16 * c) * wcols + w.n0 + tc;
      rb_set[set][0][c] = w.wstream ? ld16_nt(wp) : ld16(wp);
    }
  };
  auto fetch_set = [&](int set, int kb) {
    fetch_a(set, kb);
    fetch_b(set, kb);
  };
  auto stash_a = [&](int set, int stage) {
    uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < NPA; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c) st16(s + q * APLANE + rk_off(lr + 64 * c, lc >> 3), ra_set[set][q][c]);
  };
  auto stash_b = [&](int set, int stage) {
    uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < NPB; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c) st16(s + NPA * APLANE + q * kRPlane + rc_off(kr + 16 * c, tc), rb_set[set][q][c]);
  };
  auto stash_set = [&](int set, int stage) {
    stash_a(set, stage);
    stash_b(set, stage);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();

  auto compute = [&](int stage) {
    const uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4_t fa[2][NPA], fb[2][NPB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < NPA; ++q) fa[mb][q] = ld16(s + q * APLANE + rk_off(wm * 64 + mb * 32 + i, 2 * st + half));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < NPB; ++q) fb[nb][q] = frag_tr(s + NPA * APLANE + q * kRPlane, 16 * st, wn * 64 + nb * 32, lane);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int q = 0; q < NPA; ++q) acc[mb][nb] = mfma32x32x16(fa[mb][q], fb[nb][0], acc[mb][nb]);
        }
    }
  };

  if (nkb > 0) {
    fetch_set(0, 0);
    stash_set(0, 0);
  }
  // dact over a long hidden size: the matrix cores accumulate each chunk
  // of kDactChunk K blocks from zero and the chunk sums are added in
  // ascending order into a second fp32 sum, which keeps the rounding of
  // the long contraction near that of a kDactChunk * 32-term one
  constexpr bool CHUNKED = MODE == kDact;
  f32x16_t tot[2][2];
  if constexpr (CHUNKED) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) tot[mb][nb] = zero16();
  }
  for (int it = 0; it < nkb; ++it) {
    __syncthreads();
    const int cur = it & 1;
    const bool more = it + 1 < nkb;
    // the next block's loads are in flight during this block's MFMAs
    if (more) fetch_set(0, it + 1);
    compute(cur);
    if (CHUNKED && (it + 1) % kDactChunk == 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) tot[mb][nb][v] += acc[mb][nb][v];
          acc[mb][nb] = zero16();
        }
    }
    if (more) stash_set(0, cur ^ 1);
  }
  if constexpr (CHUNKED) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][nb][v] = tot[mb][nb][v] + acc[mb][nb][v];
  }

  if constexpr (LORA) {
    if (lora) lora_add_tile(a, zs, lbs, acc, wm, wn, lane);
  }

  if (MODE == kDact) {
    // D goes through LDS one 64-row half at a time (dact_epilogue)
    constexpr int ES = kBT + 4;  // fp32 row stride of a staged half
    static_assert(64 * ES * 2 <= EPI, "a staged half fits in the shared area");
    float* ep = reinterpret_cast<float*>(smem);
    for (int hh = 0; hh < 2; ++hh) {
      __syncthreads();
      if (wm == hh) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              ep[(mb * 32 + acc_row(v, half)) * ES + wn * 64 + nb * 32 + i] = acc[mb][nb][v];
      }
      __syncthreads();
      dact_epilogue(a, w, ep, ES, w.n0, w.nt, hh, tid);
    }
    return;
  }

  // ---- dx epilogue: the 128x128 fp32 tile goes through LDS one 64-row half at
  // a time (waves with wm == half write their accumulators), then each row
  // leaves as 16-byte pieces, 512 contiguous bytes per row per 32 lanes.
  constexpr int ES = kBT + 4;  // fp32 row stride of a staged half
  static_assert(64 * ES * 2 <= EPI, "a staged half fits in the shared area");
  float* ep = reinterpret_cast<float*>(smem);
  const int piece = tid & 31;
  for (int hh = 0; hh < 2; ++hh) {
    __syncthreads();
    if (wm == hh) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ep[(mb * 32 + acc_row(v, half)) * ES + wn * 64 + nb * 32 + i] = acc[mb][nb][v];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (tid >> 5) + 8 * j;
      const int lrow = hh * 64 + r;
      const u32x4_t val = ld16(ep + r * ES + piece * 4);
      const int col = w.n0 + piece * 4;
      if (lrow >= w.rows) continue;
      if (w.shared) {
        st16_nt(a.dx_shared + static_cast<int64_t>(w.m0 + lrow) * a.H + col, val);
      } else {
        const int64_t rt = a.sorted_route[static_cast<int64_t>(w.seg0) + w.m0 + lrow];
        if (rt >= 0 && rt < a.T * a.K) st16_nt(a.dx_route + rt * a.H + col, val);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dact at hidden 64 * NKB with 64-wide K blocks (half the K blocks, and so
// half the barriers and LDS round trips, of the 32-wide loop; each gathered
// dOut row contributes a whole 128-byte line per block).  Tiles, waves,
// epilogue and the MFMA sequence of every element (16-wide K steps in
// ascending order) are those of bwd_gemm_kernel<kDact>.  A (dOut rows) is
// staged [row][64 k] with 128-byte rows whose 16-byte pieces are swizzled
// by row (rk64_off; each wave instruction writes 8 whole rows, and the
// 32-row fragment reads are conflict-free), B (W2 rows h) [k][col] as in
// the other kernels.
// Register ring of three K blocks (two in flight while one is multiplied),
// two LDS stages.  LORA adds the routed rows' adapter term before the
// epilogue as bwd_gemm_kernel does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int rk64_off(int row, int c) { return row * 64 + ((c ^ ((row >> 1) & 7)) << 3); }

template <int NKB, bool LORA>
__global__ __launch_bounds__(256, 2) void bwd_dact_k64_kernel(const BwdArgs a) {
  constexpr int NS = 3;
  constexpr int APL = kBT * 64;  // A stage: 128 rows x 64 k
  constexpr int BPL = 64 * kRStride;  // B stage: 64 k rows x 128 columns
  constexpr int STAGE = APL + BPL;
  constexpr int ES = kBT + 4;  // fp32 row stride of a staged epilogue half
  constexpr int EPI = 64 * ES * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE > EPI ? 2 * STAGE : EPI];
  // LoRA: the tile's rows' shrink results and its columns' A2 rows
  __shared__ __attribute__((aligned(16))) uint16_t zs[LORA ? kBT * 2 * kLoraMaxRank : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lbs[LORA ? kLoraMaxRank * kBT : 8];

  BwdTile w;
  if (!bwd_decode<kDact>(a, blockIdx.x, w)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int Ie = w.Ie;
  const bool lora = LORA && !w.shared;  // the shared expert has no adapter
  // ordered before the epilogue by the K loop's barriers
  if (lora) lora_stage_tile(a, w, zs, lbs, a.I, tid);
  // A loader: rows wave * 32 + 8q + lane / 8, 16-byte piece ap = lane % 8,
  // so that each wave instruction writes 8 whole 128-byte rows; B loader: k
  // rows kr + 16c, 8 columns at tc
  const int ap = lane & 7;
  const int kr = tid >> 4, tc = (tid & 15) * 8;
  const uint16_t* arow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // rows past the tile repeat its last row, unused
    const int rr = min(wave * 32 + 8 * q + (lane >> 3), w.rows - 1);
    arow[q] = a.dout + bwd_token(a, w, static_cast<int64_t>(w.seg0) + w.m0 + rr) * a.H + ap * 8;
  }
  const uint16_t* wbase = (w.shared ? a.ws2 : a.w2 + static_cast<int64_t>(w.grp) * a.H * a.I) + w.n0 + tc;

  u32x4_t ra[NS][4], rb[NS][4];
  auto fetch = [&](int set, int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[set][q] = ld16(arow[q] + kb * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint16_t* wp = wbase + static_cast<int64_t>(kb * 64 + kr + 16 * c) * Ie;
      rb[set][c] = w.wstream ? ld16_nt(wp) : ld16(wp);
    }
  };
  auto stash = [&](int set, int stage) {
    uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(s + rk64_off(wave * 32 + 8 * q + (lane >> 3), ap), ra[set][q]);
#pragma unroll
    for (int c = 0; c < 4; ++c) st16(s + APL + rc_off(kr + 16 * c, tc), rb[set][c]);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();
  auto compute = [&](int stage) {
    const uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4_t fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = ld16(s + rk64_off(wm * 64 + mb * 32 + i, 2 * st + half));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = frag_tr(s + APL, 16 * st, wn * 64 + nb * 32, lane);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
    }
  };

#pragma unroll
  for (int q = 0; q < NS - 1 && q < NKB; ++q) fetch(q, q);
  stash(0, 0);
#pragma unroll
  for (int it = 0; it < NKB; ++it) {
    __syncthreads();
    if (it + NS - 1 < NKB) fetch((it + NS - 1) % NS, it + NS - 1);
    compute(it & 1);
    if (it + 1 < NKB) stash((it + 1) % NS, (it + 1) & 1);
  }
  if constexpr (LORA) {
    if (lora) lora_add_tile(a, zs, lbs, acc, wm, wn, lane);
  }

  // epilogue: D through LDS one 64-row half at a time, then dact_epilogue
  float* ep = reinterpret_cast<float*>(smem);
  for (int hh = 0; hh < 2; ++hh) {
    __syncthreads();
    if (wm == hh) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ep[(mb * 32 + acc_row(v, half)) * ES + wn * 64 + nb * 32 + i] = acc[mb][nb][v];
    }
    __syncthreads();
    dact_epilogue(a, w, ep, ES, w.n0, w.nt, hh, tid);
  }
}

// ---------------------------------------------------------------------------
// Input gradient per route (kDx) on 128 x 256 tiles, for a contraction of NKB
// 32-wide blocks (2Ie = 32 NKB for the routed and the shared expert alike).
// A = dGU planes hi, mid ([row][k] layout, 16 KB per block for 128 rows) is
// read once for 256 columns of dX; B = W13_g rows k, as two 128-column
// halves ([k][col] layout, 16 KB per block).  Waves 2 x 2, each owning
// 64 rows x 128 columns (eight 32x32 accumulators).  Register ring of two
// K blocks: blocks it + 1 and it + 2 are in flight while block it is
// multiplied, two LDS stages.  Every element's MFMA sequence is that of
// bwd_gemm_kernel<kDx>: K blocks ascending, K steps 0 then 1, planes hi, mid.
// LORA (routed groups): after the K loop the rows' shrink results z = B13^T
// dGU and the adapter's A13 rows for the tile's 256 columns are staged in
// the freed LDS, and acc = fma(scale, z A13, acc) with the product taken as
// z_hi A13 then z_lo A13 on the matrix cores, as in bwd_gemm_kernel.
// ---------------------------------------------------------------------------
template <int NKB, bool LORA>
__global__ __launch_bounds__(256, 2) void bwd_dx_wide_kernel(const BwdArgs a) {
  constexpr int NP = kDxPlanes;
  constexpr int TN = 2 * kBT;
  constexpr int STAGE = NP * kKPlane + 2 * kRPlane;
  constexpr int ES = TN + 4;  // fp32 row stride of a staged 64-row half
  constexpr int EPI = 64 * ES * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE > EPI ? 2 * STAGE : EPI];

  // ---- work item: (row tile of the work list, 256-column tile)
  const int ncol = a.H / TN;
  const int item = xcd_item(blockIdx.x, a.meta[0] * ncol);
  if (item < 0) return;
  const int tile = item / ncol;
  const int n0 = (item - tile * ncol) * TN;
  const int grp = a.tiles[2 * tile];
  const int m0 = a.tiles[2 * tile + 1];
  const bool shared = grp == a.E;
  const int Ie = shared ? a.Is : a.I;
  const int seg0 = shared ? 0 : a.offsets[grp];
  const int cnt = shared ? static_cast<int>(a.T) : a.offsets[grp + 1] - seg0;
  const int rows = min(kBT, cnt - m0);
  if (rows <= 0) return;
  const bool wstream = cnt <= kBT;  // the group's only row tile reads each weight once

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // load roles: A rows lr + 64c, 8 k at lc; B k rows kr + 16c, 8 columns at tc
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const int kr = tid >> 4, tc = (tid & 15) * 8;

  int64_t a_off[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int rr = min(lr + 64 * c, rows - 1);  // rows past the tile repeat its last row, unused
    const int64_t rowp = shared ? (m0 + rr) : (static_cast<int64_t>(seg0) + m0 + rr);
    a_off[c] = rowp * 2 * Ie;
  }
  const uint16_t* a_base[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) a_base[q] = shared ? a.sdgu[q] : a.dgu[q];
  const uint16_t* wbase = (shared ? a.ws13 : a.w13 + static_cast<int64_t>(grp) * 2 * a.I * a.H) + n0 + tc;

  u32x4_t ra[2][NP][2], rb[2][2][2];
  auto fetch = [&](int set, int kb) {
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c) ra[set][q][c] = ld16(a_base[q] + a_off[c] + kb * kBK + lc);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* wp = wbase + static_cast<int64_t>(kb * kBK + kr + 16 * c) * a.H + 128 * h;
        rb[set][h][c] = wstream ? ld16_nt(wp) : ld16(wp);
      }
  };
  auto stash = [&](int set, int stage) {
    uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int q = 0; q < NP; ++q) st16(s + q * kKPlane + rk_off(lr + 64 * c, lc >> 3), ra[set][q][c]);
#pragma unroll
      for (int h = 0; h < 2; ++h) st16(s + NP * kKPlane + h * kRPlane + rc_off(kr + 16 * c, tc), rb[set][h][c]);
    }
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = zero16();

  auto compute = [&](int stage) {
    const uint16_t* s = smem + stage * STAGE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4_t fa[2][NP];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < NP; ++q) fa[mb][q] = ld16(s + q * kKPlane + rk_off(wm * 64 + mb * 32 + i, 2 * st + half));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4_t fb = frag_tr(s + NP * kKPlane + wn * kRPlane, 16 * st, nb * 32, lane);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int q = 0; q < NP; ++q) acc[mb][nb] = mfma32x32x16(fa[mb][q], fb, acc[mb][nb]);
      }
    }
  };

  fetch(0, 0);
  if (NKB > 1) fetch(1, 1);
  stash(0, 0);
#pragma unroll
  for (int it = 0; it < NKB; ++it) {
    __syncthreads();
    if (it + 2 < NKB) fetch(it & 1, it + 2);
    compute(it & 1);
    if (it + 1 < NKB) stash((it + 1) & 1, (it + 1) & 1);
  }

  if constexpr (LORA) {
    if (!shared) {
      // zs [row][hi | lo][kLoraMaxRank] (rows past the tile: zeros), then
      // lbs [rank][256 columns]
      uint16_t* zs = smem;
      uint16_t* lbs = smem + kBT * 2 * kLoraMaxRank;
      __syncthreads();  // every wave is done with the K loop's stages
      const uint16_t* z0 = a.lzq + (static_cast<int64_t>(seg0) + m0) * 2 * kLoraMaxRank;
      for (int q = tid; q < kBT * 4; q += 256)
        st16(&zs[8 * q], q < rows * 4 ? ld16(z0 + 8 * q) : u32x4_t{0u, 0u, 0u, 0u});
      const uint16_t* b0 = a.lbx + static_cast<int64_t>(grp) * a.lrank * a.H + n0;
      for (int q = tid; q < a.lrank * (TN / 8); q += 256) {
        const int j = q / (TN / 8), c = q - j * (TN / 8);
        st16(&lbs[j * TN + 8 * c], ld16(b0 + static_cast<int64_t>(j) * a.H + 8 * c));
      }
      __syncthreads();
      u32x4_t zh[2], zl[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int zr = wm * 64 + mb * 32 + i;
        zh[mb] = ld16(&zs[zr * 2 * kLoraMaxRank + 8 * half]);
        zl[mb] = ld16(&zs[zr * 2 * kLoraMaxRank + kLoraMaxRank + 8 * half]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        // B[k][n] = A13[k][n0 + col] for k < rank, else 0
        const int col = wn * 128 + nb * 32 + i;
        uint32_t bw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j0 = 8 * half + 2 * q;
          const uint32_t e0 = j0 < a.lrank ? lbs[j0 * TN + col] : 0u;
          const uint32_t e1 = j0 + 1 < a.lrank ? lbs[(j0 + 1) * TN + col] : 0u;
          bw[q] = e0 | (e1 << 16);
        }
        const u32x4_t b{bw[0], bw[1], bw[2], bw[3]};
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const f32x16_t t = mfma32x32x16(zl[mb], b, mfma32x32x16(zh[mb], b, zero16()));
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mb][nb][v] = fmaf(a.lscale, t[v], acc[mb][nb][v]);
        }
      }
    }
  }

  // ---- epilogue: each 64-row half of the tile goes through LDS (the waves
  // with wm == hh stage theirs); each row leaves as 16-byte pieces, 1 KB
  // contiguous per row
  float* ep = reinterpret_cast<float*>(smem);
  const int piece = tid & 63;
  for (int hh = 0; hh < 2; ++hh) {
    __syncthreads();
    if (wm == hh) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ep[(mb * 32 + acc_row(v, half)) * ES + wn * 128 + nb * 32 + i] = acc[mb][nb][v];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = (tid >> 6) + 4 * j;
      const int lrow = hh * 64 + r;
      if (lrow >= rows) continue;
      const u32x4_t val = ld16(ep + r * ES + piece * 4);
      const int col = n0 + piece * 4;
      if (shared) {
        st16_nt(a.dx_shared + static_cast<int64_t>(m0 + lrow) * a.H + col, val);
      } else {
        const int64_t rt = a.sorted_route[static_cast<int64_t>(seg0) + m0 + lrow];
        if (rt >= 0 && rt < a.T * a.K) st16_nt(a.dx_route + rt * a.H + col, val);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Expert weight gradients on wide tiles.  One workgroup of four waves per
// output tile: kDw13 128 x 256 (gate/up rows j x hidden columns h), kDw2
// 256 x 128 (hidden rows h x intermediate columns i).  Of the two operands
// of each K block, the one stored in route order as kGradPlanes bf16 planes
// (dGU for kDw13, g*act for kDw2; 24 KB per block) spans 128 of the tile's
// edge and the gathered single-plane one (x rows for kDw13, dOut rows for
// kDw2; 16 KB) spans the 256-wide edge, so the three-plane operand is read
// once for twice the output of a 128 x 128 tile.  Waves: 2 x 2, each owning
// 64 x 128 (kDw13) or 128 x 64 (kDw2), i.e. eight 32x32 accumulators.  The
// next K block's loads are in flight in registers while a block is
// multiplied (one LDS stage, two workgroups per CU).  A work item is NT
// tiles of one group, computed one after the other.  The MFMA sequence of
// every output element is fixed: 32-route K blocks in ascending sorted
// position, K steps 0 then 1, planes hi, mid, lo; it does not depend on
// the tile shape or on which workgroup computes the tile.
// ---------------------------------------------------------------------------
template <int MODE, int NT>
__global__ __launch_bounds__(256, 2) void bwd_wgrad_kernel(const BwdArgs a) {
  static_assert(MODE == kDw2 || MODE == kDw13, "weight-gradient modes only");
  constexpr bool W13 = MODE == kDw13;
  constexpr int TM = W13 ? kBT : 2 * kBT;  // tile rows
  constexpr int TN = W13 ? 2 * kBT : kBT;  // tile columns
  constexpr int MB = W13 ? 2 : 4;          // 32-row blocks per wave
  constexpr int NB = W13 ? 4 : 2;          // 32-column blocks per wave
  // LDS: planes of the route-ordered operand, then the two 128-column halves
  // of the gathered one, each [32 k][128 columns] (rc_off layout)
  constexpr int PREG = kGradPlanes * kRPlane;
  constexpr int STAGE = PREG + 2 * kRPlane;
  // epilogue: one 64 x 256 (kDw13) or 128 x 128 (kDw2) fp32 half of the tile
  constexpr int ES = TN + 4;
  constexpr int EROWS = TM / 2;
  constexpr int EPI = EROWS * ES * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGE > EPI ? STAGE : EPI];
  __shared__ int s_tok[kBwdTokLds];

  // ---- work item (group, tile rows m0, tile columns n0).  The shared
  // expert's tiles contract over all T tokens, the routed ones over a few
  // blocks of routes: the shared tiles are dealt round-robin to the eight
  // XCDs and come first in each XCD's order (so they are not all left to the
  // end of one XCD's range), then each XCD takes a contiguous range of the
  // routed tiles (so an expert's tiles share its operands in one L2).
  if (a.meta[0] == 0) return;  // caller offsets failed the work-list check
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int mt = W13 ? 2 * Imax / TM : a.H / TM;
  const int ntl = W13 ? a.H / TN : Imax / TN;
  // A work item is NT consecutive tiles of one group (same rows m0 while
  // the group's column tiles last), run one after the other: the next
  // tile's first K block is loaded during the current tile's epilogue, and
  // the group's tokens are read once.
  const int per_grp = mt * ntl;
  const int ppg = (per_grp + NT - 1) / NT;  // items per group
  int grp, rem0;
  {
    const int nsh = a.Is > 0 ? ppg : 0;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int sx = (nsh - xcd + 7) >> 3;  // shared items xcd, xcd + 8, ... below nsh
    if (slot < sx) {
      grp = a.E;
      rem0 = xcd + 8 * slot;
    } else {
      const int nr = a.E * ppg;
      const int per = (nr + 7) >> 3;
      const int it = xcd * per + (slot - sx);
      if (slot - sx >= per || it >= nr) return;
      grp = it / ppg;
      rem0 = it - grp * ppg;
    }
  }
  const bool shared = grp == a.E;
  const int Ie = shared ? a.Is : a.I;
  // the item's tiles that exist for this group (a smaller shared expert has
  // fewer intermediate tiles)
  int tm0[NT] = {}, tn0[NT] = {};
  int ntiles = 0;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t = rem0 * NT + u;
    const int mm = (t / ntl) * TM, nn = (t % ntl) * TN;
    if (t < per_grp && (W13 ? mm < 2 * Ie : nn < Ie)) {
#pragma unroll
      for (int w = 0; w < NT; ++w)  // register arrays take constant indices only
        if (w == ntiles) {
          tm0[w] = mm;
          tn0[w] = nn;
        }
      ++ntiles;
    }
  }
  if (ntiles == 0) return;
  const int seg0 = shared ? 0 : a.offsets[grp];
  const int rows = shared ? static_cast<int>(a.T) : a.offsets[grp + 1] - seg0;
  const int nkb = (rows + kBK - 1) / kBK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;
  // loader role: k rows kr and kr + 16 of a block, 8 columns at tc
  const int kr = tid >> 4, tc = (tid & 15) * 8;

  // route-ordered operand: plane q, row p, columns pc0 + tc; gathered
  // operand: token row, columns g0 + 128 h + tc (pc0, g0: the tile being
  // fetched)
  const uint16_t* pbase[kGradPlanes];
#pragma unroll
  for (int q = 0; q < kGradPlanes; ++q)
    pbase[q] = W13 ? (shared ? a.sdgu[q] : a.dgu[q]) : (shared ? a.sgact[q] : a.gact[q]);
  const int64_t pstride = W13 ? 2 * Ie : Ie;
  const uint16_t* gsrc = W13 ? a.x : a.dout;
  int pc0 = 0, g0 = 0;
  auto aim = [&](int u) {
    pc0 = W13 ? tm0[u] : tn0[u];
    g0 = W13 ? tn0[u] : tm0[u];
  };
  aim(0);

  const bool tok_lds = rows <= kBwdTokLds;
  auto token_of = [&](int kk) -> int64_t {
    return tok_lds ? static_cast<int64_t>(s_tok[kk]) : bwd_token(a, BwdTile{grp, 0, 0, 0, rows, seg0, shared, false, Ie},
                                                              static_cast<int64_t>(seg0) + kk);
  };

  u32x4_t rp[kGradPlanes][2], rg[2][2];
  auto fetch_plain = [&](int kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int kk = kb * kBK + kr + 16 * c;
      const int64_t rowp = static_cast<int64_t>(seg0) + kk;
#pragma unroll
      for (int q = 0; q < kGradPlanes; ++q)
        rp[q][c] = kk < rows ? ld16(pbase[q] + rowp * pstride + pc0 + tc) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  int64_t tok[2] = {0, 0};
  auto fetch_gathered = [&](int kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool in = kb * kBK + kr + 16 * c < rows;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        rg[h][c] = in ? ld16(gsrc + tok[c] * a.H + g0 + 128 * h + tc) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto next_tokens = [&](int kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int kk = kb * kBK + kr + 16 * c;
      tok[c] = kk < rows ? token_of(kk) : 0;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int q = 0; q < kGradPlanes; ++q) st16(smem + q * kRPlane + rc_off(kr + 16 * c, tc), rp[q][c]);
#pragma unroll
      for (int h = 0; h < 2; ++h) st16(smem + PREG + h * kRPlane + rc_off(kr + 16 * c, tc), rg[h][c]);
    }
  };

  f32x16_t acc[MB][NB];

  auto compute = [&]() {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if constexpr (W13) {
        // A = dGU planes (rows m), B = x half wn (columns n)
        u32x4_t fa[MB][kGradPlanes];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int q = 0; q < kGradPlanes; ++q) fa[mb][q] = frag_tr(smem + q * kRPlane, 16 * st, wm * 64 + mb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4_t fb = frag_tr(smem + PREG + wn * kRPlane, 16 * st, nb * 32, lane);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < kGradPlanes; ++q) acc[mb][nb] = mfma32x32x16(fa[mb][q], fb, acc[mb][nb]);
        }
      } else {
        // A = dOut half wm (rows m), B = g*act planes (columns n)
        u32x4_t fb[NB][kGradPlanes];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < kGradPlanes; ++q) fb[nb][q] = frag_tr(smem + q * kRPlane, 16 * st, wn * 64 + nb * 32, lane);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4_t fa = frag_tr(smem + PREG + wm * kRPlane, 16 * st, mb * 32, lane);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < kGradPlanes; ++q) acc[mb][nb] = mfma32x32x16(fa, fb[nb][q], acc[mb][nb]);
        }
      }
    }
  };

  if (nkb > 0) {
    // the route-ordered operand of block 0 is in flight while the segment's
    // tokens are read
    fetch_plain(0);
    if (tok_lds) {
      if (tid < rows) s_tok[tid] = static_cast<int>(bwd_token(a, BwdTile{grp, 0, 0, 0, rows, seg0, shared, false, Ie},
                                                              static_cast<int64_t>(seg0) + tid));
      __syncthreads();
    }
    next_tokens(0);
    fetch_gathered(0);
    stash();
    if (nkb > 1) next_tokens(1);
  }

  float* ep = reinterpret_cast<float*>(smem);
  const int half = lane >> 5;
  float* out = W13 ? (shared ? a.dws13 : a.dw13 + static_cast<int64_t>(grp) * 2 * a.I * a.H)
                   : (shared ? a.dws2 : a.dw2 + static_cast<int64_t>(grp) * a.H * a.I);
  const int64_t ostride = W13 ? a.H : Ie;
  constexpr int PIECES = TN / 4;         // 16-byte pieces per tile row
  constexpr int RPP = 256 / PIECES;      // rows per pass of the workgroup
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    if (u >= ntiles) break;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = zero16();
    for (int it = 0; it < nkb; ++it) {
      __syncthreads();
      const bool more = it + 1 < nkb;
      if (more) {
        fetch_plain(it + 1);
        fetch_gathered(it + 1);
        if (it + 2 < nkb) next_tokens(it + 2);
      }
      compute();
      if (more) {
        __syncthreads();  // every wave is done reading the stage
        stash();
      }
    }
    // the next tile's first K block (the same routes) is in flight during
    // this tile's epilogue
    const bool next = u + 1 < ntiles && nkb > 0;
    if (next) {
      aim(u + 1);
      next_tokens(0);
      fetch_plain(0);
      fetch_gathered(0);
    }

    // ---- epilogue: the tile leaves through LDS one half at a time (the two
    // waves with wm == hh stage theirs), then each row as 16-byte pieces
    const int m0 = tm0[u], n0 = tn0[u];
    for (int hh = 0; hh < 2; ++hh) {
      __syncthreads();
      if (wm == hh) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              ep[(mb * 32 + acc_row(v, half)) * ES + wn * (NB * 32) + nb * 32 + i] = acc[mb][nb][v];
      }
      __syncthreads();
      const int piece = tid % PIECES;
#pragma unroll
      for (int j = 0; j < EROWS / RPP; ++j) {
        const int r = tid / PIECES + RPP * j;
        st16_nt(out + static_cast<int64_t>(m0 + hh * EROWS + r) * ostride + n0 + piece * 4,
                ld16(ep + r * ES + piece * 4));
      }
    }
    if (next) {
      __syncthreads();  // every wave is done reading the staged tile
      stash();
      if (nkb > 1) next_tokens(1);
    }
  }
}

// ---------------------------------------------------------------------------
// Router weight gradient: d_w_router[e][h] = sum over expert e's routes, in
// ascending route id, of dl[r] * x[t(r)][h] (fp64 accumulation).  One
// workgroup per (expert, 2048-column chunk); empty experts get zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_router_w_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ dl,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ sorted_route,
                                                           float* __restrict__ dwr, int64_t T,
                                                           int H, int K) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 2048 + threadIdx.x * 8;
  if (c >= H) return;
  const int64_t R = T * K;
  // segment bounds clamped to [0, R] (caller offsets are checked elsewhere;
  // this only keeps the reads in bounds)
  const int64_t p0 = min(max(static_cast<int64_t>(offsets[e]), int64_t{0}), R);
  const int64_t p1 = max(min(static_cast<int64_t>(offsets[e + 1]), R), p0);
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  // eight routes' loads are issued ahead of their additions, which keep the
  // ascending route order
  for (int64_t pb = p0; pb < p1; pb += 8) {
    int64_t rr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) rr[u] = sorted_route[min(pb + u, p1 - 1)];
    float sv[8];
    u32x4_t xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = rr[u] >= 0 && rr[u] < R;
      sv[u] = ok ? dl[rr[u]] : 0.f;
      xv[u] = ld16(x + (ok ? rr[u] / K : 0) * H + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (pb + u >= p1 || rr[u] < 0 || rr[u] >= R) continue;
      const double s = sv[u];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += s * bf16_to_f32(static_cast<uint16_t>(xv[u][q] & 0xffffu));
        acc[2 * q + 1] += s * bf16_to_f32(static_cast<uint16_t>(xv[u][q] >> 16));
      }
    }
  }
  float* o = dwr + static_cast<int64_t>(e) * H + c;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<float>(acc[j]);
}

// Shared-gate weight gradient, pass 1: partial[b][h] = sum over tokens
// 64b .. 64b+63 (ascending) of dz[t] * x[t][h], fp64.  A thread owns two
// columns; its tokens' loads are issued eight at a time, ahead of their
// additions, which keep the ascending token order.
__global__ __launch_bounds__(256) void bwd_wsg_partial_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ dz,
                                                              double* __restrict__ partial,
                                                              int64_t T, int H) {
  const int b = blockIdx.x;
  const int c = blockIdx.y * 512 + threadIdx.x * 2;
  if (c >= H) return;
  double a0 = 0.0, a1 = 0.0;
  const int64_t t0 = static_cast<int64_t>(b) * 64;
  const int64_t t1 = min(t0 + 64, T);
  for (int64_t tb = t0; tb < t1; tb += 8) {
    uint32_t xv[8];
    float sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t t = min(tb + u, t1 - 1);
      xv[u] = *reinterpret_cast<const uint32_t*>(x + t * H + c);
      sv[u] = dz[t];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (tb + u < t1) {
        const double sd = sv[u];
        a0 += sd * bf16_to_f32(static_cast<uint16_t>(xv[u] & 0xffffu));
        a1 += sd * bf16_to_f32(static_cast<uint16_t>(xv[u] >> 16));
      }
    }
  }
  double* o = partial + static_cast<int64_t>(b) * H + c;
  o[0] = a0;
  o[1] = a1;
}

// pass 2: d_w_sgate[h] = sum over blocks b (ascending) of partial[b][h];
// the partials are loaded sixteen at a time ahead of their additions.
__global__ __launch_bounds__(256) void bwd_wsg_final_kernel(const double* __restrict__ partial,
                                                            float* __restrict__ dwsg, int nb,
                                                            int H) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  double s = 0.0;
  for (int b0 = 0; b0 < nb; b0 += 16) {
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = partial[static_cast<int64_t>(min(b0 + u, nb - 1)) * H + h];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (b0 + u < nb) s += v[u];
  }
  dwsg[h] = static_cast<float>(s);
}

// ---------------------------------------------------------------------------
// Input gradient, one workgroup per token:
//   dX = ((sum of dx_route over the token's routes in ascending expert id)
//         + dx_shared) + dz * w_sgate + dx_router,
//   dx_router = sum over the same routes, same order, of dl * w_router[e]
// (fp32; the route order is fixed by sorting the token's expert ids).
// ---------------------------------------------------------------------------
template <int KT>
__global__ __launch_bounds__(256) void bwd_dx_sum_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
    const float* __restrict__ dx_route, const float* __restrict__ dx_shared,
    const float* __restrict__ dz, const uint16_t* __restrict__ w_sgate,
    const float* __restrict__ w_router, float* __restrict__ dx32, uint16_t* __restrict__ dx16,
    int H, int E, int K) {
  const int64_t t = blockIdx.x;
  // the token's valid slots in ascending expert id: rank[k] = number of
  // valid ids below slot k's (ids are distinct within a token, invalid ones
  // take no rank); slot_j / eid_j = the slot and id of rank j
  int e[KT], rank[KT];
  int n = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    e[k] = k < K ? topk_idx[t * K + k] : -1;
    if (e[k] >= E) e[k] = -1;
    n += e[k] >= 0 ? 1 : 0;
  }
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    int r = 0;
#pragma unroll
    for (int q = 0; q < KT; ++q) r += (e[q] >= 0 && e[q] < e[k]) ? 1 : 0;
    rank[k] = e[k] >= 0 ? r : -1;
  }
  const float* xrow[KT];
  const float* wrow[KT];
  float s[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    int slot = 0, id = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (rank[k] == j) {
        slot = k;
        id = e[k];
      }
    }
    // ranks past the valid count keep slot 0 / expert 0: loaded, unused
    xrow[j] = dx_route + (t * K + slot) * H;
    wrow[j] = w_router + static_cast<int64_t>(id) * H;
    s[j] = dl[t * K + slot];
  }
  const float dzt = dx_shared ? dz[t] : 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    f32x4v_t v[KT], wv[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      v[j] = *reinterpret_cast<const f32x4v_t*>(xrow[j] + c);
      wv[j] = *reinterpret_cast<const f32x4v_t*>(wrow[j] + c);
    }
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      if (j < n) {
        a0 += v[j][0];
        a1 += v[j][1];
        a2 += v[j][2];
        a3 += v[j][3];
        r0 = fmaf(s[j], wv[j][0], r0);
        r1 = fmaf(s[j], wv[j][1], r1);
        r2 = fmaf(s[j], wv[j][2], r2);
        r3 = fmaf(s[j], wv[j][3], r3);
      }
    }
    if (dx_shared) {
      const f32x4v_t v2 = *reinterpret_cast<const f32x4v_t*>(dx_shared + t * H + c);
      a0 += v2[0];
      a1 += v2[1];
      a2 += v2[2];
      a3 += v2[3];
      const uint2 w2v = *reinterpret_cast<const uint2*>(w_sgate + c);
      a0 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(w2v.x & 0xffffu)), a0);
      a1 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(w2v.x >> 16)), a1);
      a2 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(w2v.y & 0xffffu)), a2);
      a3 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(w2v.y >> 16)), a3);
    }
    a0 += r0;
    a1 += r1;
    a2 += r2;
    a3 += r3;
    f32x4v_t o;
    o[0] = a0;
    o[1] = a1;
    o[2] = a2;
    o[3] = a3;
    *reinterpret_cast<f32x4v_t*>(dx32 + t * H + c) = o;
    if (dx16) {
      uint2 pk;
      pk.x = static_cast<uint32_t>(f32_to_bf16(a0)) | (static_cast<uint32_t>(f32_to_bf16(a1)) << 16);
      pk.y = static_cast<uint32_t>(f32_to_bf16(a2)) | (static_cast<uint32_t>(f32_to_bf16(a3)) << 16);
      *reinterpret_cast<uint2*>(dx16 + t * H + c) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// LoRA adapter gradients of the routed experts.  Each is a sum over the
// expert's routes p of a rank vector r[p] (a shrink result, its bf16 hi +
// lo) times a feature row f[p], times the scale s:
//   kind 0  dA13[e][j][h] = s sum_p u13[p][j] x[t(p)][h]      u13 = B13^T dGU
//   kind 1  dB13[e][c][j] = s sum_p dGU[p][c] z13[p][j]        z13 = A13 x
//   kind 2  dA2[e][j][i]  = s sum_p v2[p][j] (g act)[p][i]     v2 = B2^T dOut
//   kind 3  dB2[e][h][j]  = s sum_p dOut[t(p)][h] gz2[p][j]    gz2 = A2 (g act)
// The gradient reaching the down adapter's output is g dOut, so kinds 2 and
// 3 carry the route's gate g in the feature (g act) or in the shrink (gz2 =
// g z2).  The fp32 features (dGU, g act) enter exactly: hi + mid + lo of
// their three bf16 planes is the fp32 value, and so is each partial sum.
//
// One launch covers the four kinds: blockIdx.y runs over each kind's
// feature tiles in turn.  Workgroup = (expert, 64 * FPT features): lane l of
// every wave owns
// features FPT l .. FPT l + FPT - 1 (one 16- or 8-byte load per plane and
// route), and wave w sums the w-th quarter of the expert's routes (in
// ascending sorted position, fp32 fma, rank vector from a wave-uniform
// load); the four partial sums are then added in wave order through LDS,
// ((q0 + q1) + q2) + q3.  RK = the rank rounded up to 4, 8 or 16 (the shrink
// results are zero past the rank).  No atomics; the result depends only on
// the expert's routes.
// ---------------------------------------------------------------------------
struct LoraGradOut {
  const uint16_t* rq[4];  // rank vectors of kinds 0..3 (u13, z13, v2, gz2)
  float* out[4];          // dA13, dB13, dA2, dB2
  int tiles[5];           // first feature tile of each kind; tiles[4] = total
};

template <int RK>
__global__ __launch_bounds__(256) void bwd_lora_grad_kernel(const BwdArgs a, const LoraGradOut o) {
  constexpr int FPT = RK == 16 ? 4 : 8;  // features per lane (registers)
  constexpr int NW = FPT / 2;            // 32-bit words per plane load
  // offsets that failed ffn_tiles_kernel's check left an empty work list
  if (a.meta[0] == 0) return;
  const int e = blockIdx.x;
  int kind = 0;
  while (kind < 3 && static_cast<int>(blockIdx.y) >= o.tiles[kind + 1]) ++kind;
  const int tile = blockIdx.y - o.tiles[kind];
  const uint16_t* __restrict__ rq = o.rq[kind];
  float* __restrict__ out = o.out[kind];
  const int nf = (kind == 0 || kind == 3) ? a.H : (kind == 1 ? 2 * a.I : a.I);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f = (tile * 64 + lane) * FPT;
  const bool live = f < nf;  // nf is a multiple of 128
  const int fo = live ? f : 0;
  const int64_t R = a.T * a.K;
  // segment bounds clamped to [0, R] (only keeps the reads in bounds)
  const int64_t p0 = min(max(static_cast<int64_t>(a.offsets[e]), int64_t{0}), R);
  const int64_t p1 = max(min(static_cast<int64_t>(a.offsets[e + 1]), R), p0);
  const int64_t per = (p1 - p0 + 3) >> 2;
  const int64_t q0 = min(p0 + wave * per, p1), q1 = min(q0 + per, p1);
  const bool gathered = kind == 0 || kind == 3;
  const uint16_t* src0 = gathered ? (kind == 0 ? a.x : a.dout) : (kind == 1 ? a.dgu[0] : a.gact[0]);
  const uint16_t* src1 = kind == 1 ? a.dgu[1] : a.gact[1];
  const uint16_t* src2 = kind == 1 ? a.dgu[2] : a.gact[2];

  float acc[FPT][RK];
#pragma unroll
  for (int c = 0; c < FPT; ++c)
#pragma unroll
    for (int j = 0; j < RK; ++j) acc[c][j] = 0.f;

  typedef uint32_t words_t __attribute__((ext_vector_type(NW)));
  auto ldw = [&](const uint16_t* p) { return *reinterpret_cast<const words_t*>(p); };
  // element offset of route p's feature row
  auto row_of = [&](int64_t p) -> int64_t {
    if (!gathered) return p * nf;
    const int64_t rt = a.sorted_route[p];
    return ((rt >= 0 && rt < R) ? rt / a.K : 0) * a.H;
  };
  auto feat = [&](int64_t o, float (&v)[FPT]) {
    const words_t w0 = ldw(src0 + o + fo);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w0[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w0[i] >> 16));
    }
    if (!gathered) {
      const words_t w1 = ldw(src1 + o + fo);
      const words_t w2 = ldw(src2 + o + fo);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        v[2 * i] = (v[2 * i] + bf16_to_f32(static_cast<uint16_t>(w1[i] & 0xffffu))) +
                   bf16_to_f32(static_cast<uint16_t>(w2[i] & 0xffffu));
        v[2 * i + 1] = (v[2 * i + 1] + bf16_to_f32(static_cast<uint16_t>(w1[i] >> 16))) +
                       bf16_to_f32(static_cast<uint16_t>(w2[i] >> 16));
      }
    }
  };
  auto accumulate = [&](int64_t p, const float (&v)[FPT]) {
    const uint16_t* z = rq + p * 2 * kLoraMaxRank;
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      const float r = bf16_to_f32(z[j]) + bf16_to_f32(z[kLoraMaxRank + j]);
#pragma unroll
      for (int c = 0; c < FPT; ++c) acc[c][j] = fmaf(r, v[c], acc[c][j]);
    }
  };
  constexpr int U = 4;  // routes per step: their feature loads in flight together
  int64_t p = q0;
  for (; p + U <= q1; p += U) {
    float v[U][FPT];
#pragma unroll
    for (int u = 0; u < U; ++u) feat(row_of(p + u), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) accumulate(p + u, v[u]);
  }
  for (; p < q1; ++p) {
    float v[FPT];
    feat(row_of(p), v);
    accumulate(p, v);
  }

  // the four waves' partial sums, added in wave order, one rank column at a
  // time
  __shared__ float part[4][64 * FPT];
  const float sc = a.lscale;
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    if (j < a.lrank) {  // uniform
      __syncthreads();
#pragma unroll
      for (int c = 0; c < FPT; ++c) part[wave][lane * FPT + c] = acc[c][j];
      __syncthreads();
      for (int t = threadIdx.x; t < 64 * FPT; t += 256) {
        const int ff = tile * 64 * FPT + t;
        if (ff < nf) {
          const float v = sc * (((part[0][t] + part[1][t]) + part[2][t]) + part[3][t]);
          if (kind == 0 || kind == 2) out[(static_cast<int64_t>(e) * a.lrank + j) * nf + ff] = v;
          else out[(static_cast<int64_t>(e) * nf + ff) * a.lrank + j] = v;
        }
      }
    }
  }
}

// dst[e][n][m] = src[e][m][n] (bf16), for the adapters' transposed copies.
__global__ __launch_bounds__(256) void lora_transpose_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int64_t total,
                                                             int M, int N) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q >= total) return;
  const int64_t mn = static_cast<int64_t>(M) * N;
  const int64_t e = q / mn, rem = q - e * mn;
  const int n = static_cast<int>(rem / M), m = static_cast<int>(rem - static_cast<int64_t>(n) * M);
  dst[q] = src[e * mn + static_cast<int64_t>(m) * N + n];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_bwd_gate(const double* dgp, const double* dsp, const float* gate, const float* sg,
                           float* dl, float* dz, int64_t T, int K, int I, int Is,
                           hipStream_t stream) {
  const int stride = (I > Is ? I : Is) / kBT;
  const int per = 256 / K;  // tokens per workgroup (K <= 16)
  bwd_gate_kernel<<<static_cast<unsigned>((T + per - 1) / per), 256, 0, stream>>>(
      dgp, dsp, gate, sg, dl, dz, T, K, I / kBT, Is / kBT, stride);
  return hipGetLastError();
}

namespace {
BwdArgs bwd_args(const BwdLaunch& L) {
  BwdArgs a;
  a.T = L.T;
  a.H = L.H;
  a.E = L.E;
  a.K = L.K;
  a.I = L.I;
  a.Is = L.Is;
  a.offsets = L.offsets;
  a.sorted_route = L.sorted_route;
  a.gate = L.gate;
  a.sg = L.sg;
  a.tiles = L.tiles;
  a.meta = L.meta;
  a.x = L.x;
  a.dout = L.dout;
  a.w13 = L.w13;
  a.w2 = L.w2;
  a.ws13 = L.ws13;
  a.ws2 = L.ws2;
  a.gu = L.gu;
  a.sgu = L.sgu;
  for (int q = 0; q < kGradPlanes; ++q) {
    a.dgu[q] = L.dgu[q];
    a.sdgu[q] = L.sdgu[q];
    a.gact[q] = L.gact[q];
    a.sgact[q] = L.sgact[q];
  }
  a.dgp = L.dgp;
  a.dsp = L.dsp;
  a.nt_stride = (L.I > L.Is ? L.I : L.Is) / kBT;
  a.dx_route = L.dx_route;
  a.dx_shared = L.dx_shared;
  a.dw13 = L.dw13;
  a.dw2 = L.dw2;
  a.dws13 = L.dws13;
  a.dws2 = L.dws2;
  a.lzq = nullptr;
  a.lbx = nullptr;
  a.lscale = L.lscale;
  a.lrank = L.lrank;
  return a;
}

unsigned rounds(int64_t items) { return static_cast<unsigned>(((items + 7) / 8) * 8); }

// tiles per weight-gradient work item: dW13 takes two (measured at 4096
// tokens: 1175 -> 1126 us), dW2 one (two measured 596 -> 722 us)
template <int MODE>
constexpr int wgrad_tiles() { return MODE == kDw13 ? 2 : 1; }

// weight-gradient grid: per XCD, its share of the shared expert's items plus
// its contiguous range of the routed items (per_grp tiles per group, nt tiles
// per item)
unsigned wgrad_grid(const BwdLaunch& L, int64_t per_grp, int nt) {
  const int64_t ppg = (per_grp + nt - 1) / nt;
  const int64_t nsh = L.Is > 0 ? ppg : 0;
  return static_cast<unsigned>(8 * ((nsh + 7) / 8 + (L.E * ppg + 7) / 8));
}
}  // namespace

hipError_t launch_bwd_dact(const BwdLaunch& L, hipStream_t stream) {
  BwdArgs a = bwd_args(L);
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const unsigned grid = rounds(static_cast<int64_t>(L.max_tiles_bwd) * (Imax / kBT));
  // the unrolled instantiations cover H = 2048
  if (L.la2) {
    a.lzq = L.lv2;
    a.lbx = L.la2;
    if (L.H == 2048) bwd_dact_k64_kernel<2048 / 64, true><<<grid, 256, 0, stream>>>(a);
    else bwd_gemm_kernel<kDact, true><<<grid, 256, 0, stream>>>(a);
  } else if (L.H == 2048) {
    bwd_dact_k64_kernel<2048 / 64, false><<<grid, 256, 0, stream>>>(a);
  } else {
    bwd_gemm_kernel<kDact><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdLaunch& L, hipStream_t stream) {
  BwdArgs a = bwd_args(L);
  const unsigned dx_grid = rounds(static_cast<int64_t>(L.max_tiles_bwd) * (L.H / kBT));
  // the unrolled dx instantiations cover expert and shared sizes of 512
  const bool unrolled = L.I == 512 && (L.Is == 0 || L.Is == 512);
  if (L.la13) {
    a.lzq = L.lu13;
    a.lbx = L.la13;
    if (unrolled) {
      const unsigned wide_grid = rounds(static_cast<int64_t>(L.max_tiles_bwd) * (L.H / (2 * kBT)));
      bwd_dx_wide_kernel<2 * 512 / kBK, true><<<wide_grid, 256, 0, stream>>>(a);
    } else {
      bwd_gemm_kernel<kDx, true><<<dx_grid, 256, 0, stream>>>(a);
    }
    a.lzq = nullptr;
    a.lbx = nullptr;
  } else if (unrolled) {
    const unsigned wide_grid = rounds(static_cast<int64_t>(L.max_tiles_bwd) * (L.H / (2 * kBT)));
    bwd_dx_wide_kernel<2 * 512 / kBK, false><<<wide_grid, 256, 0, stream>>>(a);
  } else {
    bwd_gemm_kernel<kDx><<<dx_grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dw2(const BwdLaunch& L, hipStream_t stream) {
  const BwdArgs a = bwd_args(L);
  const int Imax = L.I > L.Is ? L.I : L.Is;
  constexpr int nt = wgrad_tiles<kDw2>();
  bwd_wgrad_kernel<kDw2, nt><<<wgrad_grid(L, (L.H / (2 * kBT)) * (Imax / kBT), nt), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_dw13(const BwdLaunch& L, hipStream_t stream) {
  const BwdArgs a = bwd_args(L);
  const int Imax = L.I > L.Is ? L.I : L.Is;
  constexpr int nt = wgrad_tiles<kDw13>();
  bwd_wgrad_kernel<kDw13, nt><<<wgrad_grid(L, (2 * Imax / kBT) * (L.H / (2 * kBT)), nt), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_gemms(const BwdLaunch& L, hipStream_t stream) {
  if (launch_bwd_dx(L, stream) != hipSuccess) return hipErrorLaunchFailure;
  if (launch_bwd_dw2(L, stream) != hipSuccess) return hipErrorLaunchFailure;
  return launch_bwd_dw13(L, stream);
}

hipError_t launch_bwd_lora_grads(const BwdLaunch& L, const uint16_t* z13, const uint16_t* gz2, float* da13,
                                 float* db13, float* da2, float* db2, hipStream_t stream) {
  const BwdArgs a = bwd_args(L);
  LoraGradOut o{{L.lu13, z13, L.lv2, gz2}, {da13, db13, da2, db2}, {}};
  const int nf[4] = {L.H, 2 * L.I, L.I, L.H};
  // 64 lanes x 8 features per workgroup (x 4 at rank 16)
  const int per_wg = L.lrank <= 8 ? 512 : 256;
  o.tiles[0] = 0;
  for (int k = 0; k < 4; ++k) o.tiles[k + 1] = o.tiles[k] + (nf[k] + per_wg - 1) / per_wg;
  const dim3 grid(static_cast<unsigned>(L.E), static_cast<unsigned>(o.tiles[4]));
  if (L.lrank <= 4) bwd_lora_grad_kernel<4><<<grid, 256, 0, stream>>>(a, o);
  else if (L.lrank <= 8) bwd_lora_grad_kernel<8><<<grid, 256, 0, stream>>>(a, o);
  else bwd_lora_grad_kernel<16><<<grid, 256, 0, stream>>>(a, o);
  return hipGetLastError();
}

hipError_t launch_lora_transpose(const uint16_t* src, uint16_t* dst, int E, int M, int N, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(E) * M * N;
  if (total == 0) return hipSuccess;
  lora_transpose_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(src, dst, total, M, N);
  return hipGetLastError();
}

hipError_t launch_bwd_router(const uint16_t* x, const float* dl, const int32_t* offsets,
                             const int32_t* sorted_route, float* dwr, int64_t T, int H, int E,
                             int K, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(E), static_cast<unsigned>((H + 2047) / 2048));
  bwd_router_w_kernel<<<grid, 256, 0, stream>>>(x, dl, offsets, sorted_route, dwr, T, H, K);
  return hipGetLastError();
}

hipError_t launch_bwd_wsg(const uint16_t* x, const float* dz, double* partial, float* dwsg, int64_t T,
                          int H, hipStream_t stream) {
  const int nb = static_cast<int>((T + 63) / 64);
  dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>((H + 511) / 512));
  bwd_wsg_partial_kernel<<<grid, 256, 0, stream>>>(x, dz, partial, T, H);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_wsg_final_kernel<<<static_cast<unsigned>((H + 255) / 256), 256, 0, stream>>>(partial, dwsg, nb, H);
  return hipGetLastError();
}

hipError_t launch_bwd_dx_sum(const int32_t* topk_idx, const float* dl, const float* dx_route,
                             const float* dx_shared, const float* dz, const uint16_t* w_sgate,
                             const float* w_router, float* dx32, uint16_t* dx16, int64_t T, int H,
                             int E, int K, hipStream_t stream) {
  if (K <= 10)
    bwd_dx_sum_kernel<10><<<static_cast<unsigned>(T), 256, 0, stream>>>(
        topk_idx, dl, dx_route, dx_shared, dz, w_sgate, w_router, dx32, dx16, H, E, K);
  else
    bwd_dx_sum_kernel<16><<<static_cast<unsigned>(T), 256, 0, stream>>>(
        topk_idx, dl, dx_route, dx_shared, dz, w_sgate, w_router, dx32, dx16, H, E, K);
  return hipGetLastError();
}

}  // namespace moe
