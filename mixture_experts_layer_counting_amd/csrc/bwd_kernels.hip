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
// operand (activation gradients, gate-scaled activations) enters split
// exactly into three bf16 parts (hi + mid + lo), i.e. three MFMA passes.
// Each 32-wide K block is summed in fp32 on the matrix cores and the block
// sums are accumulated in fp64, so long contractions (weight gradients sum
// over every route of an expert, or every token for the shared expert) do
// not lose precision as the sum grows.
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Route-weight and shared-gate gradients, one workgroup per token.
// dg[k] = <dOut[t], y[t*K+k]>, ds = <dOut[t], shared_y[t]>, accumulated in
// fp64 (each thread over its columns in ascending order, then a fixed
// butterfly inside each wave, then the four waves in a fixed order).
// dl[k] = g_k (dg_k - sum_j g_j dg_j) (softmax backward over the selected
// slots); dz = ds * sg * (1 - sg).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_gate_kernel(const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ y,
                                                       const float* __restrict__ sy,
                                                       const float* __restrict__ gate,
                                                       const float* __restrict__ sg,
                                                       float* __restrict__ dl,
                                                       float* __restrict__ dz, int H, int K) {
  __shared__ double red[4][17];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* d = dout + t * H;
  const int nsum = K + (sy ? 1 : 0);
  double part[17];
#pragma unroll
  for (int k = 0; k < 17; ++k) part[k] = 0.0;
  for (int c = tid * 4; c < H; c += 1024) {
    const uint2 dv = *reinterpret_cast<const uint2*>(d + c);
    const double d0 = bf16_to_f32(static_cast<uint16_t>(dv.x & 0xffffu));
    const double d1 = bf16_to_f32(static_cast<uint16_t>(dv.x >> 16));
    const double d2 = bf16_to_f32(static_cast<uint16_t>(dv.y & 0xffffu));
    const double d3 = bf16_to_f32(static_cast<uint16_t>(dv.y >> 16));
#pragma unroll
    for (int k = 0; k < 17; ++k) {
      if (k < nsum) {
        const float* row = k < K ? y + (t * K + k) * H : sy + t * H;
        const f32x4v_t v = *reinterpret_cast<const f32x4v_t*>(row + c);
        part[k] += d0 * v[0];
        part[k] += d1 * v[1];
        part[k] += d2 * v[2];
        part[k] += d3 * v[3];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 17; ++k) {
    if (k < nsum) {
      double v = part[k];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) red[wave][k] = v;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double dg[17];
    for (int k = 0; k < nsum; ++k) dg[k] = (red[0][k] + red[1][k]) + (red[2][k] + red[3][k]);
    double mean = 0.0;
    for (int k = 0; k < K; ++k) mean += static_cast<double>(gate[t * K + k]) * dg[k];
    for (int k = 0; k < K; ++k) {
      const double g = gate[t * K + k];
      dl[t * K + k] = static_cast<float>(g * (dg[k] - mean));
    }
    if (sy) {
      const double s = sg[t];
      dz[t] = static_cast<float>(dg[K] * s * (1.0 - s));
    }
  }
}

// ---------------------------------------------------------------------------
// Generic grouped GEMM for the expert backward: D[m][n] = sum_k A[m][k] B[n][k]
// over 64x64 output tiles, 32-wide K blocks staged in LDS (one block of
// register prefetch), four waves each owning one 32x32 MFMA block.
//
// Operands are staged in LDS as [row][k] (row = m for A, n for B), loaded
// either from k-contiguous rows (one 16-byte store per thread) or from
// sources whose rows are indexed by k (transposed on the way into LDS).  An
// operand given as three bf16 planes (hi, mid, lo) takes three MFMA passes
// in that order.  Per K block the passes accumulate in fp32 from zero; the
// block sums are added in fp64 in ascending block order.
//
// Modes (group g: routed expert g < E, shared expert g == E; p = row of the
// group's segment, t(p) its token):
//   kDact: rows p, n = i < Ie, k = h < H.  A = dOut[t(p)][h]; B = W2_g[h][i]
//          (transposed).  Epilogue: dact = acc * g_p; SwiGLU backward with the
//          saved gate/up -> dGU planes [p][2Ie], and g_p*act planes [p][Ie].
//   kDx:   rows p, n = h < H, k = j < 2Ie.  A = dGU (3 planes); B = W13_g[j][h]
//          (transposed).  Epilogue: row p of dx_route (route-major, row
//          sorted_route[p]) or of dx_shared (token row).
//   kDw2:  m = h < H, n = i < Ie, k = p over the segment.  A = dOut[t(p)][h]
//          (transposed, gathered); B = g*act [p][i] (transposed, 3 planes).
//          Epilogue: dW2_g[h][i].
//   kDw13: m = j < 2Ie, n = h < H, k = p.  A = dGU[p][j] (transposed, 3 planes);
//          B = x[t(p)][h] (transposed, gathered).  Epilogue: dW13_g[j][h].
// The K order of every output element is fixed: ascending 32-wide blocks, in
// each block K-step 0 then 1, lane half 0 then 1 inside the MFMA.
// ---------------------------------------------------------------------------
enum BwdMode { kDact = 0, kDx = 1, kDw2 = 2, kDw13 = 3 };

constexpr int kBwdRows = 64;  // rows per dgrad row tile (and GEMM tile edge)
constexpr int kBK = 32;
constexpr int kBStride = 40;  // LDS row stride in bf16 (32 + 8 padding)

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
  uint16_t* dgu[3];    // planes of dGU [R][2I]
  uint16_t* sdgu[3];   // [T][2Is]
  uint16_t* gact[3];   // planes of g*act [R][I]
  uint16_t* sgact[3];  // [T][Is]
  float* dx_route;
  float* dx_shared;
  float* dw13;
  float* dw2;
  float* dws13;
  float* dws2;
};

// Work item of a grouped-GEMM launch.
struct BwdTile {
  int grp, m0, n0;
  int rows;     // valid rows (dgrad) / contraction length (wgrad)
  int seg0;     // first sorted position of the group (0 for the shared group)
  bool shared;
  int Ie;
};

template <int MODE>
__device__ __forceinline__ bool bwd_decode(const BwdArgs& a, int g, BwdTile& w) {
  const int Imax = a.I > a.Is ? a.I : a.Is;
  if (MODE == kDact || MODE == kDx) {
    const int ncol = MODE == kDact ? Imax / kBwdRows : a.H / kBwdRows;
    const int item = xcd_item(g, a.meta[0] * ncol);
    if (item < 0) return false;
    const int tile = item / ncol, nt = item - tile * ncol;
    w.grp = a.tiles[2 * tile];
    w.m0 = a.tiles[2 * tile + 1];
    w.n0 = nt * kBwdRows;
    w.shared = w.grp == a.E;
    w.Ie = w.shared ? a.Is : a.I;
    if (MODE == kDact && w.n0 >= w.Ie) return false;
    w.seg0 = w.shared ? 0 : a.offsets[w.grp];
    const int cnt = w.shared ? static_cast<int>(a.T) : a.offsets[w.grp + 1] - w.seg0;
    w.rows = min(kBwdRows, cnt - w.m0);
    return w.rows > 0;
  }
  const int groups = a.E + (a.Is > 0 ? 1 : 0);
  const int mt = MODE == kDw2 ? a.H / kBwdRows : 2 * Imax / kBwdRows;
  const int nt = MODE == kDw2 ? Imax / kBwdRows : a.H / kBwdRows;
  const int item = xcd_item(g, groups * mt * nt);
  if (item < 0) return false;
  w.grp = item / (mt * nt);
  const int rem = item - w.grp * (mt * nt);
  w.m0 = (rem / nt) * kBwdRows;
  w.n0 = (rem % nt) * kBwdRows;
  w.shared = w.grp == a.E;
  w.Ie = w.shared ? a.Is : a.I;
  if (MODE == kDw2 && w.n0 >= w.Ie) return false;
  if (MODE == kDw13 && w.m0 >= 2 * w.Ie) return false;
  w.seg0 = w.shared ? 0 : a.offsets[w.grp];
  w.rows = w.shared ? static_cast<int>(a.T) : a.offsets[w.grp + 1] - w.seg0;
  return true;
}

// token of sorted row p of a group (bounds-checked)
__device__ __forceinline__ int64_t bwd_token(const BwdArgs& a, const BwdTile& w, int64_t p) {
  if (w.shared) return p;
  const int64_t r = a.sorted_route[p];
  return (r >= 0 && r < a.T * a.K) ? r / a.K : 0;
}

template <int MODE>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(const BwdArgs a) {
  constexpr int NPA = (MODE == kDx || MODE == kDw13) ? 3 : 1;
  constexpr int NPB = MODE == kDw2 ? 3 : 1;
  constexpr bool A_TRANS = MODE == kDw2 || MODE == kDw13;
  constexpr bool B_TRANS = true;

  BwdTile w;
  if (!bwd_decode<MODE>(a, blockIdx.x, w)) return;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][NPA][kBwdRows][kBStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][NPB][kBwdRows][kBStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int Ie = w.Ie;

  // contraction length and number of K blocks
  int kdim;
  if (MODE == kDact) kdim = a.H;
  else if (MODE == kDx) kdim = 2 * Ie;
  else kdim = w.rows;
  const int nkb = (kdim + kBK - 1) / kBK;

  // ---- per-thread load roles
  // k-contiguous role: row lr = tid>>2 (0..63), k offset lc = (tid&3)*8
  // transposed role: k row kr = tid>>3 (0..31), m/n offset tc = (tid&7)*8
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const int kr = tid >> 3, tc = (tid & 7) * 8;

  // A source row pointers (k-contiguous modes)
  const uint16_t* a_row[NPA];
  if (!A_TRANS) {
    const int rr = min(lr, w.rows - 1);
    const int64_t p = static_cast<int64_t>(w.seg0) + w.m0 + rr;
    if (MODE == kDact) {
      a_row[0] = a.dout + bwd_token(a, w, p) * a.H;
    } else {  // kDx: dGU row p
      const int64_t rowp = w.shared ? (w.m0 + rr) : p;
#pragma unroll
      for (int q = 0; q < NPA; ++q) a_row[q] = (w.shared ? a.sdgu[q] : a.dgu[q]) + rowp * 2 * Ie;
    }
  }
  // B source base (all modes load B transposed: B[n][k] = src[k][n])
  const uint16_t* wbase = nullptr;
  if (MODE == kDact) wbase = w.shared ? a.ws2 : a.w2 + static_cast<int64_t>(w.grp) * a.H * a.I;
  if (MODE == kDx) wbase = w.shared ? a.ws13 : a.w13 + static_cast<int64_t>(w.grp) * 2 * a.I * a.H;

  auto fetch = [&](int kb, u32x4_t (&ra)[NPA], u32x4_t (&rb)[NPB]) {
    const int k0 = kb * kBK;
    // ---- A
    if (!A_TRANS) {
#pragma unroll
      for (int q = 0; q < NPA; ++q) ra[q] = ld16(a_row[q] + k0 + lc);
    } else {
      const int kk = k0 + kr;  // segment row
      if (kk < w.rows) {
        const int64_t p = static_cast<int64_t>(w.seg0) + kk;
        if (MODE == kDw2) {
          ra[0] = ld16(a.dout + bwd_token(a, w, p) * a.H + w.m0 + tc);
        } else {  // kDw13: dGU[p][m]
          const int64_t rowp = w.shared ? kk : p;
#pragma unroll
          for (int q = 0; q < NPA; ++q)
            ra[q] = ld16((w.shared ? a.sdgu[q] : a.dgu[q]) + rowp * 2 * Ie + w.m0 + tc);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NPA; ++q) ra[q] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    // ---- B (transposed)
    const int kk = k0 + kr;
    if (MODE == kDact || MODE == kDx) {
      const int ncols = MODE == kDact ? Ie : a.H;
      rb[0] = ld16(wbase + static_cast<int64_t>(kk) * ncols + w.n0 + tc);
    } else if (kk < w.rows) {
      const int64_t p = static_cast<int64_t>(w.seg0) + kk;
      if (MODE == kDw2) {
        const int64_t rowp = w.shared ? kk : p;
#pragma unroll
        for (int q = 0; q < NPB; ++q)
          rb[q] = ld16((w.shared ? a.sgact[q] : a.gact[q]) + rowp * Ie + w.n0 + tc);
      } else {  // kDw13: x[t(p)][n]
        rb[0] = ld16(a.x + bwd_token(a, w, p) * a.H + w.n0 + tc);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NPB; ++q) rb[q] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  auto stash = [&](int buf, const u32x4_t (&ra)[NPA], const u32x4_t (&rb)[NPB]) {
#pragma unroll
    for (int q = 0; q < NPA; ++q) {
      if (!A_TRANS) {
        st16(&As[buf][q][lr][lc], ra[q]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          As[buf][q][tc + e][kr] = static_cast<uint16_t>(ra[q][e >> 1] >> (16 * (e & 1)));
      }
    }
#pragma unroll
    for (int q = 0; q < NPB; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Bs[buf][q][tc + e][kr] = static_cast<uint16_t>(rb[q][e >> 1] >> (16 * (e & 1)));
    }
  };

  double acc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0;
  u32x4_t ra[NPA], rb[NPB];
  if (nkb > 0) {
    fetch(0, ra, rb);
    stash(0, ra, rb);
  }
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) fetch(kb + 1, ra, rb);
    f32x16_t part = zero16();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t fa[NPA], fb[NPB];
#pragma unroll
      for (int q = 0; q < NPA; ++q) fa[q] = ld16(&As[cur][q][wm * 32 + i][16 * s + 8 * half]);
#pragma unroll
      for (int q = 0; q < NPB; ++q) fb[q] = ld16(&Bs[cur][q][wn * 32 + i][16 * s + 8 * half]);
      // at most one operand has several planes
#pragma unroll
      for (int q = 0; q < NPA; ++q) part = mfma32x32x16(fa[q], fb[0], part);
#pragma unroll
      for (int q = 1; q < NPB; ++q) part = mfma32x32x16(fa[0], fb[q], part);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += static_cast<double>(part[v]);
    if (more) stash(cur ^ 1, ra, rb);
  }

  // ---- epilogue: lane holds D[m0 + wm*32 + acc_row(v)][n0 + wn*32 + i]
  const int col = w.n0 + wn * 32 + i;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int lrow = wm * 32 + acc_row(v, half);
    const float val = static_cast<float>(acc[v]);
    if (MODE == kDact) {
      if (lrow >= w.rows) continue;
      const int64_t p = static_cast<int64_t>(w.seg0) + w.m0 + lrow;  // sorted row / token
      float g;
      int64_t rowp;
      if (w.shared) {
        rowp = w.m0 + lrow;
        g = a.sg[rowp];
      } else {
        rowp = p;
        const int64_t r = a.sorted_route[p];
        g = (r >= 0 && r < a.T * a.K) ? a.gate[r] : 0.f;
      }
      const float* gur = (w.shared ? a.sgu : a.gu) + rowp * 2 * Ie;
      const float gv = gur[col], uv = gur[Ie + col];
      const float dact = val * g;
      const float sgm = 1.0f / (1.0f + expf(-gv));
      const float dgate = dact * uv * sgm * (1.0f + gv * (1.0f - sgm));
      const float silu = silu_f32(gv);
      const float dup = dact * silu;
      const float gact = g * (silu * uv);
      uint16_t pg[3], pu[3], pa[3];
      split3(dgate, pg);
      split3(dup, pu);
      split3(gact, pa);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        uint16_t* dq = (w.shared ? a.sdgu[q] : a.dgu[q]) + rowp * 2 * Ie;
        dq[col] = pg[q];
        dq[Ie + col] = pu[q];
        (w.shared ? a.sgact[q] : a.gact[q])[rowp * Ie + col] = pa[q];
      }
    } else if (MODE == kDx) {
      if (lrow >= w.rows) continue;
      if (w.shared) {
        a.dx_shared[static_cast<int64_t>(w.m0 + lrow) * a.H + col] = val;
      } else {
        const int64_t r = a.sorted_route[static_cast<int64_t>(w.seg0) + w.m0 + lrow];
        if (r >= 0 && r < a.T * a.K) a.dx_route[r * a.H + col] = val;
      }
    } else if (MODE == kDw2) {
      const int64_t hrow = w.m0 + lrow;
      float* o = w.shared ? a.dws2 : a.dw2 + static_cast<int64_t>(w.grp) * a.H * a.I;
      o[hrow * Ie + col] = val;
    } else {
      const int64_t jrow = w.m0 + lrow;
      float* o = w.shared ? a.dws13 : a.dw13 + static_cast<int64_t>(w.grp) * 2 * a.I * a.H;
      o[jrow * a.H + col] = val;
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
  const int p0 = offsets[e], p1 = offsets[e + 1];
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  const int64_t R = T * K;
  for (int p = p0; p < p1; ++p) {
    const int64_t r = sorted_route[p];
    if (r < 0 || r >= R) continue;
    const double s = dl[r];
    const u32x4_t xv = ld16(x + (r / K) * H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += s * bf16_to_f32(static_cast<uint16_t>(xv[q] & 0xffffu));
      acc[2 * q + 1] += s * bf16_to_f32(static_cast<uint16_t>(xv[q] >> 16));
    }
  }
  float* o = dwr + static_cast<int64_t>(e) * H + c;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<float>(acc[j]);
}

// Shared-gate weight gradient, pass 1: partial[b][h] = sum over tokens
// 64b .. 64b+63 (ascending) of dz[t] * x[t][h], fp64.
__global__ __launch_bounds__(256) void bwd_wsg_partial_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ dz,
                                                              double* __restrict__ partial,
                                                              int64_t T, int H) {
  const int b = blockIdx.x;
  const int c = blockIdx.y * 2048 + threadIdx.x * 8;
  if (c >= H) return;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  const int64_t t1 = min(static_cast<int64_t>(b + 1) * 64, T);
  for (int64_t t = static_cast<int64_t>(b) * 64; t < t1; ++t) {
    const double s = dz[t];
    const u32x4_t xv = ld16(x + t * H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += s * bf16_to_f32(static_cast<uint16_t>(xv[q] & 0xffffu));
      acc[2 * q + 1] += s * bf16_to_f32(static_cast<uint16_t>(xv[q] >> 16));
    }
  }
  double* o = partial + static_cast<int64_t>(b) * H + c;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = acc[j];
}

// pass 2: d_w_sgate[h] = sum over blocks b (ascending) of partial[b][h].
__global__ __launch_bounds__(256) void bwd_wsg_final_kernel(const double* __restrict__ partial,
                                                            float* __restrict__ dwsg, int nb,
                                                            int H) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  double s = 0.0;
  for (int b = 0; b < nb; ++b) s += partial[static_cast<int64_t>(b) * H + h];
  dwsg[h] = static_cast<float>(s);
}

// ---------------------------------------------------------------------------
// Input gradient, one workgroup per token:
//   dX = ((sum of dx_route over the token's routes in ascending expert id)
//         + dx_shared) + dz * w_sgate + dx_router,
//   dx_router = sum over the same routes, same order, of dl * w_router[e]
// (fp32; the route order is fixed by sorting the token's expert ids).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dx_sum_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
    const float* __restrict__ dx_route, const float* __restrict__ dx_shared,
    const float* __restrict__ dz, const uint16_t* __restrict__ w_sgate,
    const float* __restrict__ w_router, float* __restrict__ dx32, uint16_t* __restrict__ dx16,
    int H, int E, int K) {
  const int64_t t = blockIdx.x;
  // slots of this token in ascending expert id (insertion sort, K <= 16)
  int ord[16];
  int eid[16];
  int n = 0;
  for (int k = 0; k < K; ++k) {
    int e = topk_idx[t * K + k];
    if (e < 0 || e >= E) continue;
    int j = n++;
    while (j > 0 && eid[j - 1] > e) {
      eid[j] = eid[j - 1];
      ord[j] = ord[j - 1];
      --j;
    }
    eid[j] = e;
    ord[j] = k;
  }
  const float dzt = dx_shared ? dz[t] : 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    for (int j = 0; j < n; ++j) {
      const int k = ord[j];
      const f32x4v_t v = *reinterpret_cast<const f32x4v_t*>(dx_route + (t * K + k) * H + c);
      a0 += v[0];
      a1 += v[1];
      a2 += v[2];
      a3 += v[3];
      const float s = dl[t * K + k];
      const f32x4v_t wv = *reinterpret_cast<const f32x4v_t*>(w_router + static_cast<int64_t>(eid[j]) * H + c);
      r0 = fmaf(s, wv[0], r0);
      r1 = fmaf(s, wv[1], r1);
      r2 = fmaf(s, wv[2], r2);
      r3 = fmaf(s, wv[3], r3);
    }
    if (dx_shared) {
      const f32x4v_t v = *reinterpret_cast<const f32x4v_t*>(dx_shared + t * H + c);
      a0 += v[0];
      a1 += v[1];
      a2 += v[2];
      a3 += v[3];
      const uint2 wv = *reinterpret_cast<const uint2*>(w_sgate + c);
      a0 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(wv.x & 0xffffu)), a0);
      a1 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(wv.x >> 16)), a1);
      a2 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(wv.y & 0xffffu)), a2);
      a3 = fmaf(dzt, bf16_to_f32(static_cast<uint16_t>(wv.y >> 16)), a3);
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
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_bwd_gate(const uint16_t* dout, const float* y, const float* sy, const float* gate,
                           const float* sg, float* dl, float* dz, int64_t T, int H, int K,
                           hipStream_t stream) {
  bwd_gate_kernel<<<static_cast<unsigned>(T), 256, 0, stream>>>(dout, y, sy, gate, sg, dl, dz, H, K);
  return hipGetLastError();
}

hipError_t launch_bwd_gemms(const BwdLaunch& L, hipStream_t stream) {
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
  for (int q = 0; q < 3; ++q) {
    a.dgu[q] = L.dgu[q];
    a.sdgu[q] = L.sdgu[q];
    a.gact[q] = L.gact[q];
    a.sgact[q] = L.sgact[q];
  }
  a.dx_route = L.dx_route;
  a.dx_shared = L.dx_shared;
  a.dw13 = L.dw13;
  a.dw2 = L.dw2;
  a.dws13 = L.dws13;
  a.dws2 = L.dws2;
  const int Imax = L.I > L.Is ? L.I : L.Is;
  auto rounds = [](int64_t items) { return static_cast<unsigned>(((items + 7) / 8) * 8); };
  const int64_t dgrad_tiles = L.max_tiles64;
  bwd_gemm_kernel<kDact><<<rounds(dgrad_tiles * (Imax / kBwdRows)), 256, 0, stream>>>(a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_gemm_kernel<kDx><<<rounds(dgrad_tiles * (L.H / kBwdRows)), 256, 0, stream>>>(a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int64_t groups = L.E + (L.Is > 0 ? 1 : 0);
  bwd_gemm_kernel<kDw2><<<rounds(groups * (L.H / kBwdRows) * (Imax / kBwdRows)), 256, 0, stream>>>(a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_gemm_kernel<kDw13><<<rounds(groups * (2 * Imax / kBwdRows) * (L.H / kBwdRows)), 256, 0, stream>>>(a);
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
  dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>((H + 2047) / 2048));
  bwd_wsg_partial_kernel<<<grid, 256, 0, stream>>>(x, dz, partial, T, H);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_wsg_final_kernel<<<static_cast<unsigned>((H + 255) / 256), 256, 0, stream>>>(partial, dwsg, nb, H);
  return hipGetLastError();
}

hipError_t launch_bwd_dx_sum(const int32_t* topk_idx, const float* dl, const float* dx_route,
                             const float* dx_shared, const float* dz, const uint16_t* w_sgate,
                             const float* w_router, float* dx32, uint16_t* dx16, int64_t T, int H,
                             int E, int K, hipStream_t stream) {
  bwd_dx_sum_kernel<<<static_cast<unsigned>(T), 256, 0, stream>>>(topk_idx, dl, dx_route, dx_shared, dz,
                                                                 w_sgate, w_router, dx32, dx16, H, E, K);
  return hipGetLastError();
}

}  // namespace moe
