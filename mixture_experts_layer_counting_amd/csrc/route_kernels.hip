// Routing and permutation kernels of the routed MoE layer (gfx950).
//
// Routing follows the Routing bullet of the "MoE route/combine contract"
// commit on the RL-Kernel pull request 557 page: an FP32 router, softmax,
// stable descending selection with ties to the lower expert id, FP32
// renormalisation of the selected gates.  The permutation is the local
// selection of each expert's routes described in that page's "What" section,
// done as a stable counting sort so that an expert's rows keep ascending
// route id.
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router weight split: wr[e][h] (fp32) = hi + mid + lo exactly, each part a
// bf16, stored as three planes [3][E][H].  hi = bf16(w), mid = bf16(w - hi),
// lo = w - hi - mid (at most 8 significant bits, so exact in bf16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                           uint16_t* __restrict__ planes,
                                                           int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const f32x4v_t w0 = *reinterpret_cast<const f32x4v_t*>(wr + i);
  const f32x4v_t w1 = *reinterpret_cast<const f32x4v_t*>(wr + i + 4);
  u32x4_t ph, pm, pl;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t h2 = 0, m2 = 0, l2 = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 2 * q + u;
      const float w = r < 4 ? w0[r] : w1[r - 4];
      const uint16_t hi = f32_to_bf16(w);
      const float r1 = w - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
      h2 |= static_cast<uint32_t>(hi) << (16 * u);
      m2 |= static_cast<uint32_t>(mid) << (16 * u);
      l2 |= static_cast<uint32_t>(lo) << (16 * u);
    }
    ph[q] = h2;
    pm[q] = m2;
    pl[q] = l2;
  }
  st16(planes + i, ph);
  st16(planes + n + i, pm);
  st16(planes + 2 * n + i, pl);
}

// ---------------------------------------------------------------------------
// Router logits: l[t][e] = sum_h x[t][h] * wr[e][h] (+ bias[e]).
//
// With wr = hi + mid + lo (router_split_kernel) every product with the bf16
// activation is exact on the matrix cores.  K runs in 32-wide blocks staged through
// double-buffered LDS; inside a block, K step s and lane half h cover
// k = 16s + 8h .. +8, and each step adds hi, then mid, then lo.  K is cut
// into chunks of 256 (eight blocks): one workgroup computes one chunk's MFMA
// sum, from zero, in fp32, and writes it to part[t][c][e].  The top-k kernel
// then adds the chunk sums in ascending chunk order in fp64, adds the bias,
// and rounds once to fp32.  A logit's arithmetic depends only on its own
// token row and expert row, never on the batch or the tile it falls in.
//
// Workgroup tile: WM*64 tokens x 128 experts x one K chunk; four waves in a
// 2x2 grid, wave (wt, we) owning tokens wt*WM*32 .. +WM*32 and experts
// we*64 .. +64.
// ---------------------------------------------------------------------------
constexpr int kRtBK = 32;      // K block
constexpr int kRtChunk = 256;  // K chunk of one workgroup
constexpr int kRtStride = 40;  // LDS row stride (bf16): 32 + 8 padding, conflict-free fragment reads

template <int WM>
__global__ __launch_bounds__(256) void router_part_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          float* __restrict__ part, int64_t T,
                                                          int H, int E) {
  constexpr int BM = WM * 64;
  // work item (token tile, expert tile, chunk), chunk slowest: with the
  // XCD-aware mapping each XCD's L2 holds the weight planes of about one chunk
  const int ntt = static_cast<int>((T + BM - 1) / BM), net = (E + 127) / 128;
  const int item = xcd_item(blockIdx.x, ntt * net * (H / kRtChunk));
  if (item < 0) return;
  const int tt = item % ntt, et = (item / ntt) % net, chunk = item / (ntt * net);
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][BM][kRtStride];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][3][128][kRtStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wt = wave & 1, we = wave >> 1;
  const int64_t t0 = static_cast<int64_t>(tt) * BM;
  const int e0 = et * 128;
  const int kc = chunk * kRtChunk;
  const int ecount = min(128, E - e0);  // 64 or 128 (E is a multiple of 64)

  // loader roles: row r = tid >> 2 (0..63), 8 elements of K at lc
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const uint16_t* xsrc[WM];
#pragma unroll
  for (int q = 0; q < WM; ++q) {
    int64_t t = t0 + q * 64 + lr;
    if (t > T - 1) t = T - 1;
    xsrc[q] = x + t * H + kc + lc;
  }
  const int64_t n = static_cast<int64_t>(E) * H;
  const uint16_t* wsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = min(e0 + q * 64 + lr, E - 1);
    wsrc[q] = planes + static_cast<int64_t>(e) * H + kc + lc;
  }

  // two register sets: block kb + 2 is loaded while block kb is multiplied
  // and block kb + 1 waits in registers (the loop is fully unrolled, so the
  // set index is a constant)
  u32x4_t rx[2][WM], rw[2][3][2];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int q = 0; q < WM; ++q) rx[set][q] = ld16(xsrc[q] + k0);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
      for (int q = 0; q < 2; ++q) rw[set][pl][q] = ld16(wsrc[q] + pl * n + k0);
    }
  };
  auto stash = [&](int set, int buf) {
#pragma unroll
    for (int q = 0; q < WM; ++q) st16(&Xs[buf][q * 64 + lr][lc], rx[set][q]);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
      for (int q = 0; q < 2; ++q) st16(&Ws[buf][pl][q * 64 + lr][lc], rw[set][pl][q]);
    }
  };

  f32x16_t acc[WM][2];
#pragma unroll
  for (int mb = 0; mb < WM; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();

  constexpr int nkb = kRtChunk / kRtBK;
  fetch(0, 0);
  fetch(1, kRtBK);
  stash(0, 0);
#pragma unroll
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const int cur = kb & 1;
    if (kb + 2 < nkb) fetch(cur, (kb + 2) * kRtBK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t a[WM], b[2][3];
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
        a[mb] = ld16(&Xs[cur][wt * WM * 32 + mb * 32 + i][16 * s + 8 * half]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) b[nb][pl] = ld16(&Ws[cur][pl][we * 64 + nb * 32 + i][16 * s + 8 * half]);
      }
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int pl = 0; pl < 3; ++pl) acc[mb][nb] = mfma32x32x16(a[mb], b[nb][pl], acc[mb][nb]);
        }
      }
    }
    if (kb + 1 < nkb) stash(cur ^ 1, cur ^ 1);
  }

  if (we * 64 >= ecount) return;
  // part[t][chunk][e]: a token's chunk sums are contiguous for the top-k pass
  const int nchunk = H / kRtChunk;
  float* out = part + static_cast<int64_t>(chunk) * E;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int e = e0 + we * 64 + nb * 32 + i;
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + wt * WM * 32 + mb * 32 + acc_row(v, half);
        if (t < T) out[t * nchunk * E + e] = acc[mb][nb][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k selection and gates, one wave per token.
// Lane l first forms logits l, l+64, ... from the router's chunk sums (fp64,
// ascending chunk order, + bias, one rounding to fp32), writing them out if
// asked.  Each of the K rounds then takes the wave-wide maximum under the
// order (greater logit first, then lower expert id), so the result is the
// stable descending order with ties to the lower id.
// Gates: w_k = exp(l_k - l_0), summed in slot order, g_k = w_k / sum.
// ---------------------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ part, int nchunk,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_gate, int64_t T,
                                                        int E, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nq = E >> 6;  // logits per lane, <= NQ
  const int64_t cstride = E;
  // chunk sums in ascending chunk order; the loads of four chunks are issued
  // together, unconditionally (indices clamped into range, surplus values
  // unused), so that their latencies overlap
  double acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.0;
  const float* pp = part + t * nchunk * E + lane;
  for (int c0 = 0; c0 < nchunk; c0 += 4) {
    float pv[4][NQ];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        pv[c][q] = pp[min(c0 + c, nchunk - 1) * cstride + min(q, nq - 1) * 64];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c0 + c < nchunk) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] += static_cast<double>(pv[c][q]);
      }
    }
  }
  float v[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q < nq) {
      const int e = q * 64 + lane;
      v[q] = static_cast<float>(acc[q] + (bias ? static_cast<double>(bias[e]) : 0.0));
      if (logits) logits[t * E + e] = v[q];
    } else {
      v[q] = -INFINITY;
    }
  }
  uint32_t taken = 0;
  float my_val = 0.f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q < nq && !((taken >> q) & 1u)) {
        const int e = q * 64 + lane;
        if (v[q] > bv || (v[q] == bv && e < be)) {
          bv = v[q];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == k) {
      my_val = bv;
      my_id = be;
    }
  }
  const float top = __shfl(my_val, 0, 64);
  const float w = lane < K ? expf(my_val - top) : 0.f;
  float sum = 0.f;
  for (int k = 0; k < K; ++k) sum += __shfl(w, k, 64);
  if (lane < K) {
    topk_idx[t * K + lane] = my_id;
    topk_gate[t * K + lane] = w / sum;
  }
}

// ---------------------------------------------------------------------------
// Counting sort, pass 1: per block of 256 tokens, a 256-bit token mask per
// expert (LDS), giving each route its rank among the block's routes of the
// same expert (ranks follow token order, i.e. route id order since a token
// holds an expert at most once) and the block's count per expert.
// hist row layout: [E] counts, then one word of error bits
// (1: expert id out of range, 2: expert repeated within a token).
// route_rank receives the in-block rank (-1 for an invalid id).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ route_rank,
                                                         int64_t T, int E, int K) {
  __shared__ unsigned long long mask[1024 * 4];
  __shared__ int err;
  const int tid = threadIdx.x;
  for (int q = tid; q < E * 4; q += 256) mask[q] = 0ull;
  if (tid == 0) err = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kSortBlock + tid;
  const int word = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[t * K + k];
      if (e < 0 || e >= E) {
        atomicOr(&err, 1);
        continue;
      }
      const unsigned long long old = atomicOr(&mask[e * 4 + word], bit);
      if (old & bit) atomicOr(&err, 2);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[t * K + k];
      int rank = -1;
      if (e >= 0 && e < E) {
        rank = __popcll(mask[e * 4 + word] & (bit - 1ull));
        for (int w = 0; w < word; ++w) rank += __popcll(mask[e * 4 + w]);
      }
      route_rank[t * K + k] = rank;
    }
  }
  int32_t* hrow = hist + static_cast<int64_t>(blockIdx.x) * (E + 1);
  for (int e = tid; e < E; e += 256)
    hrow[e] = __popcll(mask[e * 4]) + __popcll(mask[e * 4 + 1]) + __popcll(mask[e * 4 + 2]) +
              __popcll(mask[e * 4 + 3]);
  if (tid == 0) hrow[E] = err;
}

// Inclusive scan of one int per thread over a 1024-thread block.
__device__ __forceinline__ int block_scan_incl(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

// Grouped-GEMM work list from per-group row counts (1024-thread block; thread
// e < E holds expert e's count).  Expert e's rows are split into row tiles of
// rows_per_tile, in expert order, followed by the shared expert's T rows as
// group E when has_shared.  tiles[2j] = group, tiles[2j+1] = first row;
// meta[0] = number of tiles.
__device__ void emit_tiles(int count, int E, int64_t T, int has_shared, int32_t* tiles,
                           int32_t* meta, int* buf, int rows_per_tile) {
  const int e = threadIdx.x;
  const int ntile = (count + rows_per_tile - 1) / rows_per_tile;
  const int tincl = block_scan_incl(ntile, buf);
  const int tfirst = tincl - ntile;
  for (int c = 0; c < ntile; ++c) {
    tiles[2 * (tfirst + c)] = e;
    tiles[2 * (tfirst + c) + 1] = c * rows_per_tile;
  }
  if (e == 1023) buf[0] = tincl;
  __syncthreads();
  const int routed_tiles = buf[0];
  __syncthreads();
  const int shared_tiles = has_shared ? static_cast<int>((T + rows_per_tile - 1) / rows_per_tile) : 0;
  for (int c = e; c < shared_tiles; c += 1024) {
    tiles[2 * (routed_tiles + c)] = E;
    tiles[2 * (routed_tiles + c) + 1] = c * rows_per_tile;
  }
  if (e == 0) meta[0] = routed_tiles + shared_tiles;
}

// ---------------------------------------------------------------------------
// Counting sort, pass 2 (one 1024-thread workgroup): per expert, the
// exclusive running count over blocks (block_base) and the expert segment
// offsets; the error bits of all blocks (meta[1] and the workspace error
// word, overwritten); and the grouped-GEMM work list (emit_tiles).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ block_base,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ meta, int nblocks,
                                                          int E, int64_t T, int has_shared,
                                                          int* __restrict__ err_word) {
  __shared__ int buf[1024];
  __shared__ int errs;
  const int e = threadIdx.x;
  if (e == 0) errs = 0;
  int run = 0;
  int errbits = 0;
  for (int b = e; b < nblocks; b += 1024) errbits |= hist[static_cast<int64_t>(b) * (E + 1) + E];
  if (e < E) {
    int b = 0;
    for (; b + 8 <= nblocks; b += 8) {
      int h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = hist[static_cast<int64_t>(b + q) * (E + 1) + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        block_base[static_cast<int64_t>(b + q) * E + e] = run;
        run += h[q];
      }
    }
    for (; b < nblocks; ++b) {
      const int h = hist[static_cast<int64_t>(b) * (E + 1) + e];
      block_base[static_cast<int64_t>(b) * E + e] = run;
      run += h;
    }
  }
  const int incl = block_scan_incl(run, buf);
  if (e < E) offsets[e] = incl - run;
  if (e == E - 1) offsets[E] = incl;
  if (errbits) atomicOr(&errs, errbits);
  emit_tiles(run, E, T, has_shared, tiles, meta, buf, kRowsPerTile);
  __syncthreads();
  if (e == 0) {
    meta[1] = errs;
    *err_word = errs ? 1 : 0;
  }
}

// Work list alone, from caller-supplied expert offsets (grouped FFN run on
// its own, or the backward's list).
__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ meta, int E,
                                                         int64_t T, int has_shared,
                                                         int rows_per_tile) {
  __shared__ int buf[1024];
  const int e = threadIdx.x;
  int count = 0;
  if (e < E) {
    count = offsets[e + 1] - offsets[e];
    if (count < 0) count = 0;
  }
  emit_tiles(count, E, T, has_shared, tiles, meta, buf, rows_per_tile);
}

// ---------------------------------------------------------------------------
// Counting sort, pass 3: scatter.  pos = offsets[e] + block_base[b][e] +
// in-block rank; sorted_route[pos] = r and route_pos[r] = pos.  route_pos
// holds the in-block rank on entry (written by pass 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                            const int32_t* __restrict__ block_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ route_pos,
                                                            int32_t* __restrict__ sorted_route,
                                                            int64_t T, int E, int K) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kSortBlock + threadIdx.x;
  if (t >= T) return;
  for (int k = 0; k < K; ++k) {
    const int64_t r = t * K + k;
    const int e = topk_idx[r];
    const int rank = route_pos[r];
    if (e < 0 || e >= E || rank < 0) {
      route_pos[r] = -1;
      continue;
    }
    const int pos = offsets[e] + block_base[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
    route_pos[r] = pos;
    sorted_route[pos] = static_cast<int32_t>(r);
  }
}

// ---------------------------------------------------------------------------
// Shared-expert gate sg[t] = sigmoid(sum_h w_sgate[h] x[t][h]), one wave per
// token: each lane sums its H/64 products in fp64 in ascending h, then a
// fixed butterfly adds the lanes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void shared_gate_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w_sgate,
                                                          float* __restrict__ sg, int64_t T,
                                                          int H) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xr = x + t * H;
  double acc = 0.0;
  for (int c = lane * 8; c < H; c += 512) {
    const u32x4_t xv = ld16(xr + c), wv = ld16(w_sgate + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(xv[q] & 0xffffu))) *
             static_cast<double>(bf16_to_f32(static_cast<uint16_t>(wv[q] & 0xffffu)));
      acc += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(xv[q] >> 16))) *
             static_cast<double>(bf16_to_f32(static_cast<uint16_t>(wv[q] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) sg[t] = static_cast<float>(1.0 / (1.0 + exp(-acc)));
}

}  // namespace moe

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace moe {

hipError_t launch_router_split(const float* wr, uint16_t* planes, int H, int E, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(E) * H;
  router_split_kernel<<<static_cast<unsigned>((n / 8 + 255) / 256), 256, 0, stream>>>(wr, planes, n);
  return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* planes, float* part, int64_t T,
                                int H, int E, hipStream_t stream) {
  const int64_t per_chunk = static_cast<int64_t>((E + 127) / 128) * (H / kRtChunk);
  auto grid = [&](int64_t bm) {
    const int64_t items = ((T + bm - 1) / bm) * per_chunk;
    return static_cast<unsigned>(((items + 7) / 8) * 8);
  };
  // the token tile only changes which tokens share a workgroup, never a
  // logit's arithmetic; small batches use the smaller tile to fill the GPU
  if (T >= 4096)
    router_part_kernel<2><<<grid(128), 256, 0, stream>>>(x, planes, part, T, H, E);
  else
    router_part_kernel<1><<<grid(64), 256, 0, stream>>>(x, planes, part, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk_gate(const float* part, const float* bias, float* logits, int32_t* topk_idx,
                            float* topk_gate, int64_t T, int H, int E, int K, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  const int nq = E / 64, nchunk = H / kRtChunk;
  if (nq <= 2)
    topk_gate_kernel<2><<<grid, 256, 0, stream>>>(part, nchunk, bias, logits, topk_idx, topk_gate, T, E, K);
  else if (nq <= 4)
    topk_gate_kernel<4><<<grid, 256, 0, stream>>>(part, nchunk, bias, logits, topk_idx, topk_gate, T, E, K);
  else if (nq <= 8)
    topk_gate_kernel<8><<<grid, 256, 0, stream>>>(part, nchunk, bias, logits, topk_idx, topk_gate, T, E, K);
  else
    topk_gate_kernel<16><<<grid, 256, 0, stream>>>(part, nchunk, bias, logits, topk_idx, topk_gate, T, E, K);
  return hipGetLastError();
}

hipError_t launch_route_hist(const int32_t* topk_idx, int32_t* hist, int32_t* route_rank,
                             int64_t T, int E, int K, hipStream_t stream) {
  const unsigned nb = static_cast<unsigned>((T + kSortBlock - 1) / kSortBlock);
  route_hist_kernel<<<nb, 256, 0, stream>>>(topk_idx, hist, route_rank, T, E, K);
  return hipGetLastError();
}

hipError_t launch_route_scan(const int32_t* hist, int32_t* block_base, int32_t* offsets,
                             int32_t* tiles, int32_t* meta, int nblocks, int E, int64_t T,
                             int has_shared, int* err_word, hipStream_t stream) {
  route_scan_kernel<<<1, 1024, 0, stream>>>(hist, block_base, offsets, tiles, meta, nblocks, E, T,
                                            has_shared, err_word);
  return hipGetLastError();
}

hipError_t launch_ffn_tiles(const int32_t* offsets, int32_t* tiles, int32_t* meta, int E, int64_t T,
                            int has_shared, int rows_per_tile, hipStream_t stream) {
  ffn_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, tiles, meta, E, T, has_shared, rows_per_tile);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t* topk_idx, const int32_t* block_base,
                                const int32_t* offsets, int32_t* route_pos, int32_t* sorted_route,
                                int64_t T, int E, int K, hipStream_t stream) {
  const unsigned nb = static_cast<unsigned>((T + kSortBlock - 1) / kSortBlock);
  route_scatter_kernel<<<nb, 256, 0, stream>>>(topk_idx, block_base, offsets, route_pos,
                                               sorted_route, T, E, K);
  return hipGetLastError();
}

hipError_t launch_shared_gate(const uint16_t* x, const uint16_t* w_sgate, float* sg, int64_t T,
                              int H, hipStream_t stream) {
  shared_gate_kernel<<<static_cast<unsigned>((T + 3) / 4), 256, 0, stream>>>(x, w_sgate, sg, T, H);
  return hipGetLastError();
}

}  // namespace moe
