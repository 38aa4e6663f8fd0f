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
// activation is exact on the matrix cores.  K is cut into chunks of 256.  A
// chunk is summed on the matrix cores in fp32 from zero: eight 32-wide K
// blocks, each two MFMA K steps (step s, lane half h: k = 16s + 8h .. +8),
// each step adding hi, then mid, then lo.  The chunk sums are added in fp64
// in ascending chunk order, the bias is added in fp64, and the result is
// rounded once to fp32.  A logit's arithmetic depends only on its own token
// row and expert row, never on the batch or the tile it falls in.
//
// Two kernels compute it, chosen by batch size only for speed (both give the
// same bits):
//   * router_part_kernel (small batches): one workgroup per (64 tokens,
//     128 experts, K chunk) writes the chunk's fp32 sums to part[t][c][e];
//     topk_gate_kernel then forms the logits from them;
//   * router_full_kernel (large batches): one workgroup per (128 tokens,
//     128 experts) runs all chunks, keeping the fp64 chain in registers, and
//     writes the logits.
// Operands are staged through double-buffered LDS (rt_off layout) with further K blocks' loads in flight in registers while a block is
// multiplied (three, from a ring of four register sets).
// ---------------------------------------------------------------------------
constexpr int kRtBK = 32;      // K block
constexpr int kRtChunk = 256;  // K chunk summed in fp32
constexpr int kRtFullMin = 4096;  // batches from this size take router_full_kernel

// LDS position (bf16 elements) of 16-byte piece c (k = 8c .. +8) of row `row`
// of a 32-wide K block: 64-byte rows, piece c stored at c ^ ((row >> 2) & 3).
// The loaders' stores (4 rows x 4 pieces per 16 lanes) and the fragment
// reads (16 rows, one piece) both touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int rt_off(int row, int c) { return row * 32 + ((c ^ ((row >> 2) & 3)) << 3); }

// Workgroup tile 64 tokens x 128 experts x one K chunk; four waves, wave w
// owning all 64 tokens and experts w*32 .. +32 (two 32-token MFMA blocks
// share each weight fragment read from LDS).
__global__ __launch_bounds__(256) void router_part_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          float* __restrict__ part, int64_t T,
                                                          int H, int E) {
  // work item (token tile, expert tile, chunk), chunk slowest: with the
  // XCD-aware mapping each XCD's L2 holds the weight planes of about one chunk
  const int ntt = static_cast<int>((T + 63) / 64), net = (E + 127) / 128;
  const int item = xcd_item(blockIdx.x, ntt * net * (H / kRtChunk));
  if (item < 0) return;
  const int tt = item % ntt, et = (item / ntt) % net, chunk = item / (ntt * net);
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][64 * kRtBK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][3][128 * kRtBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int we = wave;
  const int64_t t0 = static_cast<int64_t>(tt) * 64;
  const int e0 = et * 128;
  const int kc = chunk * kRtChunk;
  const int ecount = min(128, E - e0);  // 64 or 128 (E is a multiple of 64)

  // loader roles: row lr (0..63), 8 elements of K at lc
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const uint16_t* xsrc = x + min(t0 + lr, T - 1) * H + kc + lc;
  const int64_t n = static_cast<int64_t>(E) * H;
  const uint16_t* wsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = min(e0 + q * 64 + lr, E - 1);
    wsrc[q] = planes + static_cast<int64_t>(e) * H + kc + lc;
  }

  // four register sets: blocks kb + 1 .. kb + 3 are in flight while kb is
  // multiplied (the loop is fully unrolled, so set indices are constants)
  constexpr int kSets = 4;
  u32x4_t rx[kSets], rw[kSets][3][2];
  auto fetch = [&](int set, int k0) {
    rx[set] = ld16(xsrc + k0);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
      for (int q = 0; q < 2; ++q) rw[set][pl][q] = ld16(wsrc[q] + pl * n + k0);
    }
  };
  auto stash = [&](int set, int buf) {
    st16(&Xs[buf][rt_off(lr, lc >> 3)], rx[set]);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
      for (int q = 0; q < 2; ++q) st16(&Ws[buf][pl][rt_off(q * 64 + lr, lc >> 3)], rw[set][pl][q]);
    }
  };

  f32x16_t acc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) acc[mb] = zero16();

  constexpr int nkb = kRtChunk / kRtBK;
#pragma unroll
  for (int q = 0; q < kSets; ++q) fetch(q, q * kRtBK);
  stash(0, 0);
#pragma unroll
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const int cur = kb & 1;
    if (kb + kSets < nkb) fetch(kb % kSets, (kb + kSets) * kRtBK);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t a[2], b[3];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a[mb] = ld16(&Xs[cur][rt_off(mb * 32 + i, 2 * s + half)]);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) b[pl] = ld16(&Ws[cur][pl][rt_off(we * 32 + i, 2 * s + half)]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) acc[mb] = mfma32x32x16(a[mb], b[pl], acc[mb]);
      }
    }
    if (kb + 1 < nkb) stash((kb + 1) % kSets, cur ^ 1);
  }

  if (we * 32 >= ecount) return;
  // part[t][chunk][e]: a token's chunk sums are contiguous for the top-k pass
  const int nchunk = H / kRtChunk;
  float* out = part + static_cast<int64_t>(chunk) * E;
  const int e = e0 + we * 32 + i;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t t = t0 + mb * 32 + acc_row(v, half);
      if (t < T) out[t * nchunk * E + e] = acc[mb][v];
    }
  }
}

// Workgroup tile 128 tokens x 128 experts over all of K; eight waves, wave
// (wt, we) owning tokens wt*64 .. +64 (wt < 2) and experts we*32 .. +32
// (two 32-token MFMA blocks share each weight fragment read from LDS).
// Work items run expert tile slowest, so the XCD that owns a range of items
// keeps one expert tile's weight planes in its L2.
__global__ __launch_bounds__(512) void router_full_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int64_t T,
                                                          int H, int E) {
  const int ntt = static_cast<int>((T + 127) / 128), net = (E + 127) / 128;
  const int item = xcd_item(blockIdx.x, ntt * net);
  if (item < 0) return;
  const int tt = item % ntt, et = item / ntt;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][128 * kRtBK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][3][128 * kRtBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, half = lane >> 5;
  const int wt = wave & 1, we = wave >> 1;
  const int64_t t0 = static_cast<int64_t>(tt) * 128;
  const int e0 = et * 128;
  const int ecount = min(128, E - e0);  // 64 or 128

  // loader roles: row lr (0..127), 8 elements of K at lc
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const uint16_t* xsrc = x + min(t0 + lr, T - 1) * H + lc;
  const int64_t n = static_cast<int64_t>(E) * H;
  const uint16_t* wsrc = planes + static_cast<int64_t>(min(e0 + lr, E - 1)) * H + lc;

  // four register sets: blocks g + 1 .. g + 3 are in flight while g is
  // multiplied (block g uses set g & 3 and LDS buffer g & 1); blocks past the
  // end of K (the last prefetches) re-read the last one
  constexpr int kSets = 4;
  u32x4_t rx[kSets], rw[kSets][3];
  const int nkb = H / kRtBK;
  auto fetch = [&](int set, int g) {
    const int k0 = min(g, nkb - 1) * kRtBK;
    rx[set] = ld16(xsrc + k0);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) rw[set][pl] = ld16(wsrc + pl * n + k0);
  };
  auto stash = [&](int set, int buf) {
    st16(&Xs[buf][rt_off(lr, lc >> 3)], rx[set]);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) st16(&Ws[buf][pl][rt_off(lr, lc >> 3)], rw[set][pl]);
  };

  f32x16_t acc[2];
  double run[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    acc[mb] = zero16();
#pragma unroll
    for (int v = 0; v < 16; ++v) run[mb][v] = 0.0;
  }

  constexpr int kBlocks = kRtChunk / kRtBK;  // 8, a multiple of kSets
  const int nchunk = H / kRtChunk;
#pragma unroll
  for (int q = 0; q < kSets; ++q) fetch(q, q);
  stash(0, 0);
  for (int c = 0; c < nchunk; ++c) {
#pragma unroll
    for (int kb = 0; kb < kBlocks; ++kb) {
      __syncthreads();
      const int cur = kb & 1;
      fetch(kb % kSets, c * kBlocks + kb + kSets);
      // keep the next block's loads ahead of this block's LDS traffic
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4_t a[2], b[3];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) a[mb] = ld16(&Xs[cur][rt_off(wt * 64 + mb * 32 + i, 2 * s + half)]);
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) b[pl] = ld16(&Ws[cur][pl][rt_off(we * 32 + i, 2 * s + half)]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int pl = 0; pl < 3; ++pl) acc[mb] = mfma32x32x16(a[mb], b[pl], acc[mb]);
        }
      }
      stash((kb + 1) % kSets, cur ^ 1);
    }
    // this chunk's fp32 sums join the fp64 chains
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        run[mb][v] += static_cast<double>(acc[mb][v]);
        acc[mb][v] = 0.f;
      }
    }
  }

  if (we * 32 >= ecount) return;
  const int e = e0 + we * 32 + i;
  const double b = bias ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t t = t0 + wt * 64 + mb * 32 + acc_row(v, half);
      if (t < T) logits[t * E + e] = static_cast<float>(run[mb][v] + b);
    }
  }
}

// ---------------------------------------------------------------------------
// Shared-expert gate of one token, sg = sigmoid(sum_h w_sgate[h] x[h]), by
// one wave: lane l sums the products of h = 8l + 512j + (0..7), j ascending,
// in fp64, then a fixed butterfly adds the lanes.  Every lane returns sg.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shared_gate_of_row(const uint16_t* __restrict__ xr,
                                                    const uint16_t* __restrict__ w_sgate, int H,
                                                    int lane) {
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
  return static_cast<float>(1.0 / (1.0 + exp(-acc)));
}

// Wave-wide maximum / minimum of a 32-bit unsigned value, returned uniform:
// four DPP steps inside each row of 16 lanes (quad swaps, half-row and row
// mirrors), then the four row results.
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl_sel) {
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false); break;
  }
  return static_cast<uint32_t>(r);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) v = max(v, dpp_u32(v, q));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) v = min(v, dpp_u32(v, q));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// Order-preserving map of a finite float to an unsigned key (-0 and +0 share
// the key of +0, as they compare equal).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------------------
// Top-k selection and gates, one wave per token.
// Lane l first forms logits l, l+64, ...: from router_part_kernel's chunk
// sums (nchunk > 1: fp64 sum in ascending chunk order, + bias, one rounding
// to fp32, written to logits_out if given), or read as router_full_kernel
// wrote them (nchunk == 1, no bias).  Each of the K rounds then takes the
// largest untaken logit (a wave maximum of order-preserving keys), ties going
// to the lower expert id; that gives the stable descending order with ties
// to the lower id.  Gates: w_k = exp(l_k - l_0), summed in slot order from
// zero, g_k = w_k / sum.  With w_sgate given, waves 4..7 of the workgroup
// compute the shared-expert gates of its four tokens, beside the selection.
// ---------------------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(512) void topk_gate_kernel(const float* __restrict__ src, int nchunk,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_gate,
                                                        const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w_sgate,
                                                        float* __restrict__ sg, int64_t T, int H,
                                                        int E, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + ((threadIdx.x >> 6) & 3);
  if (t >= T) return;
  if (threadIdx.x >= 256) {  // a shared-gate wave (launched only with w_sgate)
    const float g = shared_gate_of_row(x + t * H, w_sgate, H, lane);
    if (lane == 0) sg[t] = g;
    return;
  }
  const int nq = E >> 6;  // logits per lane, <= NQ
  // loads are issued in batches, unconditionally (indices clamped into
  // range, surplus values unused), so that their latencies overlap
  float v[NQ];
  const float* pp = src + t * nchunk * E + lane;
  if (nchunk == 1 && !bias) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = pp[min(q, nq - 1) * 64];
  } else {
    double acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = 0.0;
    for (int c0 = 0; c0 < nchunk; c0 += 4) {
      float pv[4][NQ];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < NQ; ++q) pv[c][q] = pp[min(c0 + c, nchunk - 1) * E + min(q, nq - 1) * 64];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c0 + c < nchunk) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) acc[q] += static_cast<double>(pv[c][q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = min(q, nq - 1) * 64 + lane;
      v[q] = static_cast<float>(acc[q] + (bias ? static_cast<double>(bias[e]) : 0.0));
    }
  }
  if (logits_out) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (q < nq) logits_out[t * E + q * 64 + lane] = v[q];
  }
  uint32_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) key[q] = q < nq ? float_key(v[q]) : 0u;
  uint32_t taken = 0;
  float my_val = 0.f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    // this lane's best untaken logit (lowest q among equal keys)
    uint32_t bk = 0u;
    int bq = 0;
#pragma unroll
    for (int q = NQ - 1; q >= 0; --q) {
      if (q < nq && !((taken >> q) & 1u) && key[q] >= bk) {
        bk = key[q];
        bq = q;
      }
    }
    const uint32_t m = wave_max_u32(bk);
    const uint64_t cand = __ballot(bk == m);
    int win;
    if (__popcll(cand) == 1) {
      const int wl = __ffsll(static_cast<long long>(cand)) - 1;
      win = __builtin_amdgcn_readlane(bq * 64 + lane, wl);
    } else {
      win = static_cast<int>(wave_min_u32(bk == m ? static_cast<uint32_t>(bq * 64 + lane) : 0xffffffffu));
    }
    if ((win & 63) == lane) taken |= 1u << (win >> 6);
    if (lane == k) {
      my_val = key_float(m);
      my_id = win;
    }
  }
  const float top = __shfl(my_val, 0, 64);
  const float w = lane < K ? expf(my_val - top) : 0.f;
  float sum = 0.f;
  for (int k = 0; k < K; ++k) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
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

// Inclusive scan of one int per thread over a 1024-thread block: a scan
// inside each wave, then a scan of the 16 wave totals by the first wave.
// buf holds at least 16 ints; it is free again when this returns.
__device__ __forceinline__ int block_scan_incl(int v, int* buf) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? buf[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(w, off, 64);
      if (lane >= off) w += o;
    }
    if (lane < 16) buf[lane] = w;
  }
  __syncthreads();
  const int r = v + (wave > 0 ? buf[wave - 1] : 0);
  __syncthreads();
  return r;
}

// Grouped-GEMM work list from per-group row counts (1024-thread block; thread
// e < E holds expert e's count).  Expert e's rows are split into row tiles of
// rows_per_tile, in expert order, followed by the shared expert's T rows as
// group E when has_shared.  tiles[2j] = group, tiles[2j+1] = first row;
// *ntiles = number of tiles.
__device__ void emit_tiles(int count, int E, int64_t T, int has_shared, int32_t* tiles,
                           int32_t* ntiles, int* buf, int rows_per_tile) {
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
  if (e == 0) *ntiles = routed_tiles + shared_tiles;
}

// The forward's work lists: kRowsPerTile-row tiles (meta[0] of them) and,
// when tiles_up is given, the up projection's up_rows-row tiles (meta[2]).
__device__ void emit_work_lists(int count, int E, int64_t T, int has_shared, int32_t* tiles,
                                int32_t* tiles_up, int up_rows, int32_t* meta, int* buf) {
  emit_tiles(count, E, T, has_shared, tiles, &meta[0], buf, kRowsPerTile);
  if (tiles_up) emit_tiles(count, E, T, has_shared, tiles_up, &meta[2], buf, up_rows);
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
                                                          int32_t* __restrict__ tiles_up, int up_rows,
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
  emit_work_lists(run, E, T, has_shared, tiles, tiles_up, up_rows, meta, buf);
  __syncthreads();
  if (e == 0) {
    meta[1] = errs;
    *err_word = errs ? 1 : 0;
  }
}

// Work list alone, from caller-supplied expert offsets (grouped FFN run on
// its own, with the up projection's list when tiles_up is given, or the
// backward's list).  The offsets are checked first: offsets[0] == 0, never
// decreasing, offsets[E] == T*K.  Offsets that fail set the device-error
// word (it is never cleared here, so a permutation's error survives) and
// give an empty work list, so no kernel reads past the route arrays.
__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ tiles_up, int up_rows,
                                                         int32_t* __restrict__ meta, int* __restrict__ err_word,
                                                         int err_overwrite, int E, int64_t T, int K,
                                                         int has_shared, int rows_per_tile) {
  __shared__ int buf[1024];
  __shared__ int bad;
  const int e = threadIdx.x;
  if (e == 0) bad = 0;
  __syncthreads();
  int count = 0;
  if (e < E) {
    count = offsets[e + 1] - offsets[e];
    if (count < 0 || (e == 0 && offsets[0] != 0) || (e == E - 1 && offsets[E] != T * K)) bad = 1;
  }
  __syncthreads();
  if (bad) {
    if (e == 0) {
      meta[0] = 0;
      if (tiles_up) meta[2] = 0;
      *err_word = 1;
    }
    return;
  }
  if (err_overwrite && e == 0) *err_word = 0;
  emit_tiles(count, E, T, has_shared, tiles, &meta[0], buf, rows_per_tile);
  if (tiles_up) emit_tiles(count, E, T, has_shared, tiles_up, &meta[2], buf, up_rows);
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
// The whole counting sort in one 1024-thread workgroup, for batches whose
// per-expert token masks fit in LDS (E * ceil(T/32) <= kSortSmallWords):
// bit t%32 of mask word [t/32][e] marks that token t chose expert e.  The
// rank of route (t, k) among expert e's routes is the number of tokens below
// t in e's mask, i.e. routes keep ascending route id, the same order and the
// same outputs (expert_offsets, sorted_route, route_pos, work list, error
// bits) as the three-kernel sort.  A thread owns whole tokens (its K route
// ids loaded together); when every token fits one pass (T <= 1024) the ids
// stay in registers and sorted_route is assembled in LDS and written out in
// order instead of scattered.
// ---------------------------------------------------------------------------
template <int KT>
__global__ __launch_bounds__(1024) void route_sort_small_kernel(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ offsets,
    int32_t* __restrict__ route_pos, int32_t* __restrict__ sorted_route,
    int32_t* __restrict__ tiles, int32_t* __restrict__ tiles_up, int up_rows,
    int32_t* __restrict__ meta, int* __restrict__ err_word, int64_t T, int E, int K,
    int has_shared) {
  // mask[w * E + e]; the extra last word absorbs invalid routes' updates
  __shared__ uint32_t mask[kSortSmallWords + 1];
  __shared__ uint16_t below[kSortSmallWords];  // tokens of e in the words before w
  __shared__ int soff[1024];
  __shared__ int buf[1024];
  __shared__ int errs, total;
  const int tid = threadIdx.x;
  const int Ti = static_cast<int>(T);
  const int nw = (Ti + 31) >> 5;
  const bool one_pass = Ti <= 1024;
  for (int q = tid; q < E * nw; q += 1024) mask[q] = 0u;
  if (tid == 0) errs = 0;
  __syncthreads();

  int ev[KT];
  int my_err = 0;
  auto load_token = [&](int t) {
    const int tt = min(t, Ti - 1);
#pragma unroll
    for (int k = 0; k < KT; ++k) ev[k] = topk_idx[tt * K + min(k, K - 1)];
  };
  auto mark_token = [&](int t) {
    if (t >= Ti) return;
    const uint32_t bit = 1u << (t & 31);
    const int w0 = (t >> 5) * E;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (k < K) {
        const int e = ev[k];
        const bool valid = e >= 0 && e < E;
        if (!valid) my_err |= 1;
        const uint32_t b = valid ? bit : 0u;
        const uint32_t old = atomicOr(&mask[valid ? w0 + e : kSortSmallWords], b);
        if (old & b) my_err |= 2;
      }
    }
  };
  if (one_pass) {
    load_token(tid);
    mark_token(tid);
  } else {
    for (int t = tid; t < Ti; t += 1024) {
      load_token(t);
      mark_token(t);
    }
  }
  if (my_err) atomicOr(&errs, my_err);
  __syncthreads();

  int count = 0;
  if (tid < E) {
    for (int w = 0; w < nw; ++w) {
      below[w * E + tid] = static_cast<uint16_t>(count);
      count += __popc(mask[w * E + tid]);
    }
  }
  const int incl = block_scan_incl(count, buf);
  soff[tid] = incl - count;
  if (tid < E) offsets[tid] = incl - count;
  if (tid == E - 1) {
    offsets[E] = incl;
    total = incl;
  }
  emit_work_lists(count, E, T, has_shared, tiles, tiles_up, up_rows, meta, buf);
  __syncthreads();

  // positions of token t's routes (-1 for an invalid id)
  int pos[KT];
  auto place_token = [&](int t) {
    const uint32_t below_bits = (1u << (t & 31)) - 1u;
    const int w0 = (t >> 5) * E;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int e = ev[k];
      pos[k] = -1;
      if (k < K && e >= 0 && e < E)
        pos[k] = soff[e] + below[w0 + e] + __popc(mask[w0 + e] & below_bits);
    }
  };
  if (one_pass) {
    if (tid < Ti) {
      place_token(tid);
#pragma unroll
      for (int k = 0; k < KT; ++k)
        if (k < K) route_pos[tid * K + k] = pos[k];
    }
    __syncthreads();  // every mask read is done: the mask area becomes the staging area
    int* staged = reinterpret_cast<int*>(mask);
    if (tid < Ti) {
#pragma unroll
      for (int k = 0; k < KT; ++k)
        if (k < K && pos[k] >= 0) staged[pos[k]] = tid * K + k;
    }
    __syncthreads();
    for (int q = tid; q < total; q += 1024) sorted_route[q] = staged[q];
  } else {
    for (int t = tid; t < Ti; t += 1024) {
      load_token(t);
      place_token(t);
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        if (k < K) {
          route_pos[t * K + k] = pos[k];
          if (pos[k] >= 0) sorted_route[pos[k]] = t * K + k;
        }
      }
    }
  }
  if (tid == 0) {
    meta[1] = errs;
    *err_word = errs ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Shared-expert gate alone (grouped FFN stage run on its own), one wave per
// token, the same arithmetic as in topk_gate_kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void shared_gate_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w_sgate,
                                                          float* __restrict__ sg, int64_t T,
                                                          int H) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float g = shared_gate_of_row(x + t * H, w_sgate, H, lane);
  if (lane == 0) sg[t] = g;
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

bool router_full(int64_t T) { return T >= kRtFullMin; }

hipError_t launch_router_part(const uint16_t* x, const uint16_t* planes, float* part, int64_t T,
                              int H, int E, hipStream_t stream) {
  const int64_t items = ((T + 63) / 64) * ((E + 127) / 128) * (H / kRtChunk);
  router_part_kernel<<<static_cast<unsigned>(((items + 7) / 8) * 8), 256, 0, stream>>>(x, planes, part,
                                                                                       T, H, E);
  return hipGetLastError();
}

hipError_t launch_router_full(const uint16_t* x, const uint16_t* planes, const float* bias,
                              float* logits, int64_t T, int H, int E, hipStream_t stream) {
  const int64_t items = ((T + 127) / 128) * ((E + 127) / 128);
  router_full_kernel<<<static_cast<unsigned>(((items + 7) / 8) * 8), 512, 0, stream>>>(x, planes, bias,
                                                                                       logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk_gate(const float* src, int nchunk, const float* bias, float* logits_out,
                            int32_t* topk_idx, float* topk_gate, const uint16_t* x,
                            const uint16_t* w_sgate, float* sg, int64_t T, int H, int E, int K,
                            hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  const int nq = E / 64;
#define MOE_TOPK(NQ)                                                                           \
  topk_gate_kernel<NQ><<<grid, w_sgate ? 512 : 256, 0, stream>>>(src, nchunk, bias, logits_out, topk_idx, \
                                                                 topk_gate, x, w_sgate, sg, T, H, E, K)
  if (nq <= 2)
    MOE_TOPK(2);
  else if (nq <= 4)
    MOE_TOPK(4);
  else if (nq <= 8)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

bool sort_small_fits(int64_t T, int E) {
  return static_cast<int64_t>(E) * ((T + 31) / 32) <= kSortSmallWords;
}

hipError_t launch_route_sort_small(const int32_t* topk_idx, int32_t* offsets, int32_t* route_pos,
                                   int32_t* sorted_route, int32_t* tiles, int32_t* tiles_up,
                                   int up_rows, int32_t* meta, int* err_word, int64_t T, int E,
                                   int K, int has_shared, hipStream_t stream) {
  if (K <= 10)
    route_sort_small_kernel<10><<<1, 1024, 0, stream>>>(topk_idx, offsets, route_pos, sorted_route,
                                                        tiles, tiles_up, up_rows, meta, err_word, T,
                                                        E, K, has_shared);
  else
    route_sort_small_kernel<16><<<1, 1024, 0, stream>>>(topk_idx, offsets, route_pos, sorted_route,
                                                        tiles, tiles_up, up_rows, meta, err_word, T,
                                                        E, K, has_shared);
  return hipGetLastError();
}

hipError_t launch_route_hist(const int32_t* topk_idx, int32_t* hist, int32_t* route_rank,
                             int64_t T, int E, int K, hipStream_t stream) {
  const unsigned nb = static_cast<unsigned>((T + kSortBlock - 1) / kSortBlock);
  route_hist_kernel<<<nb, 256, 0, stream>>>(topk_idx, hist, route_rank, T, E, K);
  return hipGetLastError();
}

hipError_t launch_route_scan(const int32_t* hist, int32_t* block_base, int32_t* offsets,
                             int32_t* tiles, int32_t* tiles_up, int up_rows, int32_t* meta,
                             int nblocks, int E, int64_t T, int has_shared, int* err_word,
                             hipStream_t stream) {
  route_scan_kernel<<<1, 1024, 0, stream>>>(hist, block_base, offsets, tiles, tiles_up, up_rows, meta,
                                            nblocks, E, T, has_shared, err_word);
  return hipGetLastError();
}

// The shared expert's work list alone: tiles (E, c * rows) for c < ceil(T /
// rows), and its length in *ntiles.
__global__ __launch_bounds__(256) void shared_tiles_kernel(int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles, int64_t T, int E,
                                                           int rows) {
  const int64_t n = (T + rows - 1) / rows;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c < n) {
    tiles[2 * c] = E;
    tiles[2 * c + 1] = static_cast<int32_t>(c * rows);
  }
  if (c == 0) *ntiles = static_cast<int32_t>(n);
}

hipError_t launch_shared_tiles(int32_t* tiles, int32_t* ntiles, int64_t T, int E, int rows, hipStream_t stream) {
  const int64_t n = (T + rows - 1) / rows;
  shared_tiles_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(tiles, ntiles, T, E, rows);
  return hipGetLastError();
}

hipError_t launch_ffn_tiles(const int32_t* offsets, int32_t* tiles, int32_t* tiles_up, int up_rows,
                            int32_t* meta, int* err_word, int err_overwrite, int E, int64_t T, int K,
                            int has_shared, int rows_per_tile, hipStream_t stream) {
  ffn_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, tiles, tiles_up, up_rows, meta, err_word, err_overwrite,
                                           E, T, K, has_shared, rows_per_tile);
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
