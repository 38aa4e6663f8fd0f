// Host side of the C ABI declared in include/moe_mi355x.h: argument
// validation (everything is checked before anything is enqueued), workspace
// layout and the launch sequence of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe_mi355x.h"
#include "moe_kernels.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------------------
// workspace layout (byte offsets from the workspace base)
// ---------------------------------------------------------------------------
struct Layout {
  size_t err = 0;         // int error word (first 256 bytes)
  size_t rlogits = 0;     // router chunk sums [T][H/256][E] f32, or logits [T][E] f32 for large T
  size_t wsplit = 0;      // [3][E][H] bf16: exact hi/mid/lo split of the router weight
  size_t hist = 0;        // [NB][E+1] i32
  size_t block_base = 0;  // [NB][E] i32
  size_t tiles = 0;       // [2*max_tiles] i32
  size_t tiles_up = 0;    // [2*max_tiles_up] i32: the up projection's list when its rows differ
  size_t meta = 0;        // [64] i32
  // the shared expert's own work lists (moe_forward_side): 64-row tiles,
  // up_rows-row tiles when those differ, and their lengths (meta_sh[0], [2])
  size_t tiles_sh = 0, tiles_sh_up = 0, meta_sh = 0;
  size_t act_hi = 0, act_lo = 0;    // [R][I] bf16
  size_t sact_hi = 0, sact_lo = 0;  // [T][Is] bf16
  size_t fwd_end = 0;
  // LoRA shrink results (moe_forward_lora): [R][hi, lo][kLoraMaxRank] bf16 each
  size_t lora_z13 = 0, lora_z2 = 0;
  size_t lora_end = 0;
  // backward regions (after lora_end)
  size_t tiles_bwd = 0, meta_bwd = 0;  // work list of the backward's row tiles
  size_t dl = 0, dz = 0;             // [T][K], [T] f32
  size_t dgp = 0, dsp = 0;           // [R][NT], [T][NT] f64 partial dot products, NT = max(I, Is) / 128
  size_t dgu[moe::kGradPlanes] = {};    // [R][2I] bf16 planes (hi, mid, lo)
  size_t sdgu[moe::kGradPlanes] = {};   // [T][2Is]
  size_t gact[moe::kGradPlanes] = {};   // [R][I]
  size_t sgact[moe::kGradPlanes] = {};  // [T][Is]
  size_t dx_route = 0;               // [R][H] f32
  size_t dx_shared = 0;              // [T][H] f32
  size_t wsg_partial = 0;            // [ceil(T/64)][H] f64
  size_t bwd_end = 0;
  // LoRA backward (after bwd_end): shrink results v2 = B2^T dOut and u13 =
  // B13^T dGU ([R][hi, lo][kLoraMaxRank] bf16), and the transposed expand
  // matrices B2^T [E][rank][H] and B13^T [E][rank][2I] the shrinks read
  // (A13 x and A2 (g act) reuse lora_z13 and lora_z2, the 64-row work list
  // reuses tiles and meta)
  size_t lora_v2 = 0, lora_u13 = 0, lora_b2t = 0, lora_b13t = 0;
  size_t lora_bwd_end = 0;
  int nblocks = 0;
  int max_tiles = 0;
  int up_rows = 0;       // rows per up-projection item (moe::up_rows_per_tile)
  int max_tiles_up = 0;
  int max_tiles_bwd = 0;
};

Layout make_layout(const moe_dims& d) {
  Layout L;
  const int64_t T = d.tokens, R = T * d.top_k;
  const int E = d.experts, I = d.inter, Is = d.shared_inter;
  L.nblocks = static_cast<int>((T + moe::kSortBlock - 1) / moe::kSortBlock);
  L.max_tiles = static_cast<int>(moe::max_row_tiles(T, d.top_k, E, Is > 0));
  L.up_rows = moe::up_rows_per_tile(T, d.hidden);
  L.max_tiles_up = static_cast<int>(moe::max_row_tiles(T, d.top_k, E, Is > 0, L.up_rows));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.err = take(kAlign);
  L.rlogits = take(static_cast<size_t>(moe::router_full(T) ? 1 : d.hidden / 256) * T * E * 4);
  L.wsplit = take(static_cast<size_t>(3) * E * d.hidden * 2);
  L.hist = take(static_cast<size_t>(L.nblocks) * (E + 1) * 4);
  L.block_base = take(static_cast<size_t>(L.nblocks) * E * 4);
  L.tiles = take(static_cast<size_t>(L.max_tiles) * 2 * 4);
  L.tiles_up = take(L.up_rows != moe::kRowsPerTile ? static_cast<size_t>(L.max_tiles_up) * 2 * 4 : 0);
  L.meta = take(64 * 4);
  L.tiles_sh = take(static_cast<size_t>((T + moe::kRowsPerTile - 1) / moe::kRowsPerTile) * 2 * 4);
  L.tiles_sh_up = take(L.up_rows != moe::kRowsPerTile ? static_cast<size_t>((T + L.up_rows - 1) / L.up_rows) * 2 * 4 : 0);
  L.meta_sh = take(64 * 4);
  L.act_hi = take(static_cast<size_t>(R) * I * 2);
  L.act_lo = take(static_cast<size_t>(R) * I * 2);
  L.sact_hi = take(static_cast<size_t>(T) * Is * 2);
  L.sact_lo = take(static_cast<size_t>(T) * Is * 2);
  L.fwd_end = o;
  L.lora_z13 = take(static_cast<size_t>(R) * 2 * moe::kLoraMaxRank * 2);
  L.lora_z2 = take(static_cast<size_t>(R) * 2 * moe::kLoraMaxRank * 2);
  L.lora_end = o;
  const int64_t H = d.hidden;
  L.max_tiles_bwd = static_cast<int>(moe::max_row_tiles(T, d.top_k, E, Is > 0, moe::kBwdRowsPerTile));
  L.tiles_bwd = take(static_cast<size_t>(L.max_tiles_bwd) * 2 * 4);
  L.meta_bwd = take(64 * 4);
  L.dl = take(static_cast<size_t>(R) * 4);
  L.dz = take(static_cast<size_t>(T) * 4);
  const size_t nt = static_cast<size_t>(I > Is ? I : Is) / moe::kBwdRowsPerTile;
  L.dgp = take(static_cast<size_t>(R) * nt * 8);
  L.dsp = take(static_cast<size_t>(T) * nt * 8);
  for (int q = 0; q < moe::kGradPlanes; ++q) {
    L.dgu[q] = take(static_cast<size_t>(R) * 2 * I * 2);
    L.sdgu[q] = take(static_cast<size_t>(T) * 2 * Is * 2);
    L.gact[q] = take(static_cast<size_t>(R) * I * 2);
    L.sgact[q] = take(static_cast<size_t>(T) * Is * 2);
  }
  L.dx_route = take(static_cast<size_t>(R) * H * 4);
  L.dx_shared = take(static_cast<size_t>(T) * H * 4);
  L.wsg_partial = take(static_cast<size_t>((T + 63) / 64) * H * 8);
  L.bwd_end = o;
  L.lora_v2 = take(static_cast<size_t>(R) * 2 * moe::kLoraMaxRank * 2);
  L.lora_u13 = take(static_cast<size_t>(R) * 2 * moe::kLoraMaxRank * 2);
  L.lora_b2t = take(static_cast<size_t>(E) * moe::kLoraMaxRank * H * 2);
  L.lora_b13t = take(static_cast<size_t>(E) * moe::kLoraMaxRank * 2 * I * 2);
  L.lora_bwd_end = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
int check_dims(const moe_dims* d) {
  if (!d) return MOE_E_NULL;
  if (d->tokens < 0) return MOE_E_SHAPE;
  if (d->experts < 64 || d->experts > 1024 || d->experts % 64) return MOE_E_SHAPE;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->experts) return MOE_E_SHAPE;
  if (d->hidden < 256 || d->hidden > 16384 || d->hidden % 256) return MOE_E_SHAPE;
  if (d->inter < 128 || d->inter > 4096 || d->inter % 128) return MOE_E_SHAPE;
  if (d->shared_inter != 0 &&
      (d->shared_inter < 128 || d->shared_inter > 4096 || d->shared_inter % 128))
    return MOE_E_SHAPE;
  if (d->tokens * static_cast<int64_t>(d->top_k) >= (int64_t{1} << 31)) return MOE_E_SHAPE;
  return MOE_OK;
}

struct Buf {
  const void* p;
  size_t bytes;
  bool out;
};

// Collects the buffers of one call, then checks presence, alignment and
// overlap (an output may overlap nothing else).
class Args {
 public:
  void in(const void* p, size_t bytes, bool required = true) { add(p, bytes, false, required); }
  void out(const void* p, size_t bytes, bool required = true) { add(p, bytes, true, required); }
  int status() const {
    if (null_) return MOE_E_NULL;
    if (misaligned_) return MOE_E_ALIGN;
    for (size_t a = 0; a < bufs_.size(); ++a) {
      for (size_t b = a + 1; b < bufs_.size(); ++b) {
        if (!bufs_[a].out && !bufs_[b].out) continue;
        const auto pa = reinterpret_cast<uintptr_t>(bufs_[a].p);
        const auto pb = reinterpret_cast<uintptr_t>(bufs_[b].p);
        if (pa < pb + bufs_[b].bytes && pb < pa + bufs_[a].bytes) return MOE_E_ALIAS;
      }
    }
    return MOE_OK;
  }

 private:
  void add(const void* p, size_t bytes, bool out, bool required) {
    if (!p) {
      if (required && bytes) null_ = true;
      return;
    }
    if (reinterpret_cast<uintptr_t>(p) % 16) misaligned_ = true;
    if (bytes) bufs_.push_back({p, bytes, out});
  }
  std::vector<Buf> bufs_;
  bool null_ = false;
  bool misaligned_ = false;
};

int check_ws(const moe_dims& d, const void* ws, size_t ws_bytes, int op) {
  if (!ws) return MOE_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_E_ALIGN;
  if (ws_bytes < moe_workspace_bytes(&d, op)) return MOE_E_WORKSPACE;
  return MOE_OK;
}

// gfx950 check of the current device, cached per device id.
int check_device() {
  static std::mutex mu;
  static std::vector<int> arch_ok;  // 0 unknown, 1 ok, 2 bad
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MOE_E_DEVICE;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= arch_ok.size()) arch_ok.resize(dev + 1, 0);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_E_DEVICE;
    }
    arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return arch_ok[dev] == 1 ? MOE_OK : MOE_E_DEVICE;
}

#define MOE_TRY(expr)                       \
  do {                                      \
    const int _st = (expr);                 \
    if (_st != MOE_OK) return _st;          \
  } while (0)

// Optional per-kernel events of moe_forward_profiled: when set, event i is
// recorded before launch i (NULL entries are skipped).
struct Marks {
  hipEvent_t* ev = nullptr;
  int n = 0;
  int next = 0;
  hipStream_t s = nullptr;
  hipError_t mark() {
    if (!ev || next >= n) return hipSuccess;
    hipEvent_t e = ev[next++];
    return e ? hipEventRecord(e, s) : hipSuccess;
  }
};
thread_local Marks* g_marks = nullptr;

#define MOE_LAUNCH(expr)                                                  \
  do {                                                                    \
    if (g_marks && g_marks->mark() != hipSuccess) return MOE_E_LAUNCH;    \
    if ((expr) != hipSuccess) return MOE_E_LAUNCH;                        \
  } while (0)

size_t bytes_x(const moe_dims& d) { return static_cast<size_t>(d.tokens) * d.hidden * 2; }

void add_weights(Args& a, const moe_dims& d, const moe_weights* w, bool router, bool experts) {
  const size_t E = d.experts, H = d.hidden, I = d.inter, Is = d.shared_inter;
  if (router) {
    a.in(w->w_router, E * H * 4);
    a.in(w->router_bias, E * 4, false);
    a.in(w->w_router_planes, 3 * E * H * 2, false);
  }
  if (experts) {
    a.in(w->w13, E * 2 * I * H * 2);
    a.in(w->w2, E * H * I * 2);
    if (Is) {
      a.in(w->ws13, 2 * Is * H * 2);
      a.in(w->ws2, H * Is * 2);
      a.in(w->w_sgate, H * 2);
    }
  }
}

// ---------------------------------------------------------------------------
// launch sequences (arguments already validated)
// ---------------------------------------------------------------------------
// sg: when non-null, the top-k kernel also writes the shared-expert gate.
int run_route(const moe_dims& d, const uint16_t* x, const moe_weights* w, moe_routes* r, void* ws,
              const Layout& L, float* sg, hipStream_t s) {
  const uint16_t* planes = w->w_router_planes;
  float* rbuf = at<float>(ws, L.rlogits);
  const uint16_t* xs = sg ? x : nullptr;
  const uint16_t* wsg = sg ? w->w_sgate : nullptr;
  if (planes) {
    MOE_LAUNCH(hipSuccess);  // the caller's split: the profiling marker only
  } else {
    uint16_t* own = at<uint16_t>(ws, L.wsplit);
    MOE_LAUNCH(moe::launch_router_split(w->w_router, own, d.hidden, d.experts, s));
    planes = own;
  }
  if (moe::router_full(d.tokens)) {
    float* logits = r->logits ? r->logits : rbuf;
    MOE_LAUNCH(moe::launch_router_full(x, planes, w->router_bias, logits, d.tokens, d.hidden,
                                       d.experts, s));
    MOE_LAUNCH(moe::launch_topk_gate(logits, 1, nullptr, nullptr, r->topk_idx, r->topk_gate, xs,
                                     wsg, sg, d.tokens, d.hidden, d.experts, d.top_k, s));
  } else {
    MOE_LAUNCH(moe::launch_router_part(x, planes, rbuf, d.tokens, d.hidden, d.experts, s));
    MOE_LAUNCH(moe::launch_topk_gate(rbuf, d.hidden / 256, w->router_bias, r->logits,
                                     r->topk_idx, r->topk_gate, xs, wsg, sg, d.tokens, d.hidden,
                                     d.experts, d.top_k, s));
  }
  return MOE_OK;
}

// The up projection's own work list (null when it uses the common one).
int32_t* tiles_up_of(void* ws, const Layout& L) {
  return L.up_rows != moe::kRowsPerTile ? at<int32_t>(ws, L.tiles_up) : nullptr;
}

// with_shared: the work lists also take the shared expert's tiles (false
// when it runs on a side stream with lists of its own)
int run_permute(const moe_dims& d, moe_routes* r, void* ws, const Layout& L, hipStream_t s,
                bool with_shared = true) {
  const int has_shared = with_shared && d.shared_inter > 0;
  if (moe::sort_small_fits(d.tokens, d.experts)) {
    MOE_LAUNCH(moe::launch_route_sort_small(r->topk_idx, r->expert_offsets, r->route_pos,
                                            r->sorted_route, at<int32_t>(ws, L.tiles),
                                            tiles_up_of(ws, L), L.up_rows, at<int32_t>(ws, L.meta),
                                            at<int>(ws, L.err), d.tokens, d.experts, d.top_k,
                                            has_shared, s));
    return MOE_OK;
  }
  MOE_LAUNCH(moe::launch_route_hist(r->topk_idx, at<int32_t>(ws, L.hist), r->route_pos, d.tokens,
                                    d.experts, d.top_k, s));
  MOE_LAUNCH(moe::launch_route_scan(at<int32_t>(ws, L.hist), at<int32_t>(ws, L.block_base),
                                    r->expert_offsets, at<int32_t>(ws, L.tiles), tiles_up_of(ws, L),
                                    L.up_rows, at<int32_t>(ws, L.meta), L.nblocks, d.experts,
                                    d.tokens, has_shared, at<int>(ws, L.err), s));
  MOE_LAUNCH(moe::launch_route_scatter(r->topk_idx, at<int32_t>(ws, L.block_base),
                                       r->expert_offsets, r->route_pos, r->sorted_route, d.tokens,
                                       d.experts, d.top_k, s));
  return MOE_OK;
}

// whole_forward: the work list in the workspace was built by run_permute and
// the shared-expert gate by run_route.
// mx13 / mx2: block-scaled FP8 expert weights of the two projections (then
// w's expert matrices are not read), or null.
// lora: the routed experts' adapters (shrink kernels before each grouped
// GEMM, expand in its epilogue), or null.
int run_ffn(const moe_dims& d, const uint16_t* x, const moe_weights* w, const moe_routes* r,
            moe_saved* sv, void* ws, const Layout& L, bool whole_forward, hipStream_t s,
            const moe::MxWeights* mx13 = nullptr, const moe::MxWeights* mx2 = nullptr,
            const moe_lora* lora = nullptr) {
  const int has_shared = d.shared_inter > 0;
  if (!whole_forward)
    MOE_LAUNCH(moe::launch_ffn_tiles(r->expert_offsets, at<int32_t>(ws, L.tiles), tiles_up_of(ws, L),
                                     L.up_rows, at<int32_t>(ws, L.meta), at<int>(ws, L.err), 0,
                                     d.experts, d.tokens, d.top_k, has_shared, moe::kRowsPerTile, s));
  if (has_shared && !whole_forward)
    MOE_LAUNCH(moe::launch_shared_gate(x, w->w_sgate, sv->shared_gate, d.tokens, d.hidden, s));
  const bool own_up = tiles_up_of(ws, L) != nullptr;
  moe::LoraExpand e13{}, e2{};
  if (lora) {
    e13 = {lora->b13, at<uint16_t>(ws, L.lora_z13), lora->scale, lora->rank};
    e2 = {lora->b2, at<uint16_t>(ws, L.lora_z2), lora->scale, lora->rank};
    MOE_LAUNCH(moe::launch_lora_shrink(x, nullptr, lora->a13, r->expert_offsets, r->sorted_route,
                                       at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.meta),
                                       at<uint16_t>(ws, L.lora_z13), d.tokens, d.hidden, d.experts,
                                       d.top_k, lora->rank, L.max_tiles, s));
  }
  MOE_LAUNCH(moe::launch_ffn_up(x, w->w13, w->ws13, mx13, lora ? &e13 : nullptr,
                                r->expert_offsets, r->sorted_route,
                                own_up ? tiles_up_of(ws, L) : at<int32_t>(ws, L.tiles),
                                at<int32_t>(ws, L.meta) + (own_up ? 2 : 0), L.up_rows,
                                at<uint16_t>(ws, L.act_hi), at<uint16_t>(ws, L.act_lo),
                                at<uint16_t>(ws, L.sact_hi), at<uint16_t>(ws, L.sact_lo), sv->gu,
                                has_shared ? sv->shared_gu : nullptr, d.tokens, d.hidden,
                                d.experts, d.top_k, d.inter, d.shared_inter,
                                own_up ? L.max_tiles_up : L.max_tiles, s));
  if (lora)
    MOE_LAUNCH(moe::launch_lora_shrink(at<uint16_t>(ws, L.act_hi), at<uint16_t>(ws, L.act_lo),
                                       lora->a2, r->expert_offsets, r->sorted_route,
                                       at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.meta),
                                       at<uint16_t>(ws, L.lora_z2), d.tokens, d.inter, d.experts,
                                       d.top_k, lora->rank, L.max_tiles, s));
  MOE_LAUNCH(moe::launch_ffn_down(at<uint16_t>(ws, L.act_hi), at<uint16_t>(ws, L.act_lo),
                                  at<uint16_t>(ws, L.sact_hi), at<uint16_t>(ws, L.sact_lo), w->w2,
                                  w->ws2, mx2, lora ? &e2 : nullptr, r->expert_offsets,
                                  r->sorted_route,
                                  at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.meta), sv->y,
                                  has_shared ? sv->shared_y : nullptr, d.tokens, d.hidden,
                                  d.experts, d.top_k, d.inter, d.shared_inter, L.max_tiles, s));
  return MOE_OK;
}

// The shared expert's two GEMMs alone, on their own work lists (it does not
// depend on the routing): the side-stream half of moe_forward_side.
int run_shared_ffn(const moe_dims& d, const uint16_t* x, const moe_weights* w, const moe_routes* r,
                   moe_saved* sv, void* ws, const Layout& L, hipStream_t s) {
  const bool own_up = L.up_rows != moe::kRowsPerTile;
  int32_t* meta = at<int32_t>(ws, L.meta_sh);
  const int n64 = static_cast<int>((d.tokens + moe::kRowsPerTile - 1) / moe::kRowsPerTile);
  const int nup = static_cast<int>((d.tokens + L.up_rows - 1) / L.up_rows);
  MOE_LAUNCH(moe::launch_shared_tiles(at<int32_t>(ws, L.tiles_sh), meta, d.tokens, d.experts,
                                      moe::kRowsPerTile, s));
  if (own_up)
    MOE_LAUNCH(moe::launch_shared_tiles(at<int32_t>(ws, L.tiles_sh_up), meta + 2, d.tokens, d.experts,
                                        L.up_rows, s));
  MOE_LAUNCH(moe::launch_ffn_up(x, w->w13, w->ws13, nullptr, nullptr, r->expert_offsets, r->sorted_route,
                                at<int32_t>(ws, own_up ? L.tiles_sh_up : L.tiles_sh), meta + (own_up ? 2 : 0),
                                L.up_rows, at<uint16_t>(ws, L.act_hi), at<uint16_t>(ws, L.act_lo),
                                at<uint16_t>(ws, L.sact_hi), at<uint16_t>(ws, L.sact_lo), sv->gu,
                                sv->shared_gu, d.tokens, d.hidden, d.experts, d.top_k, d.inter,
                                d.shared_inter, own_up ? nup : n64, s));
  MOE_LAUNCH(moe::launch_ffn_down(at<uint16_t>(ws, L.act_hi), at<uint16_t>(ws, L.act_lo),
                                  at<uint16_t>(ws, L.sact_hi), at<uint16_t>(ws, L.sact_lo), w->w2, w->ws2,
                                  nullptr, nullptr, r->expert_offsets, r->sorted_route,
                                  at<int32_t>(ws, L.tiles_sh), meta, sv->y, sv->shared_y, d.tokens, d.hidden,
                                  d.experts, d.top_k, d.inter, d.shared_inter, n64, s));
  return MOE_OK;
}

int run_combine(const moe_dims& d, const moe_routes* r, const moe_saved* sv, float* o32,
                uint16_t* o16, hipStream_t s) {
  const bool sh = d.shared_inter > 0;
  MOE_LAUNCH(moe::launch_combine(sv->y, r->topk_gate, sh ? sv->shared_y : nullptr,
                                 sh ? sv->shared_gate : nullptr, o32, o16, d.tokens, d.hidden,
                                 d.top_k, s));
  return MOE_OK;
}

// buffer registration per stage
void add_routes_out(Args& a, const moe_dims& d, const moe_routes* r) {
  const size_t T = d.tokens, K = d.top_k, E = d.experts;
  a.out(r->topk_idx, T * K * 4);
  a.out(r->topk_gate, T * K * 4);
  a.out(r->logits, T * E * 4, false);
}

void add_perm_out(Args& a, const moe_dims& d, const moe_routes* r) {
  const size_t T = d.tokens, K = d.top_k, E = d.experts;
  a.out(r->expert_offsets, (E + 1) * 4);
  a.out(r->sorted_route, T * K * 4);
  a.out(r->route_pos, T * K * 4);
}

void add_saved(Args& a, const moe_dims& d, const moe_saved* sv, bool out) {
  const size_t T = d.tokens, K = d.top_k, H = d.hidden, I = d.inter, Is = d.shared_inter;
  auto add = [&](const void* p, size_t b, bool req) { out ? a.out(p, b, req) : a.in(p, b, req); };
  add(sv->y, T * K * H * 4, true);
  add(sv->gu, T * K * 2 * I * 4, false);
  if (Is) {
    add(sv->shared_y, T * H * 4, true);
    add(sv->shared_gate, T * 4, true);
    add(sv->shared_gu, T * 2 * Is * 4, false);
  }
}

// side streams and events: all present, all distinct, none the call's stream
int check_side(const moe_side_streams* side, hipStream_t stream) {
  if (!side || !side->side[0] || !side->side[1] || !side->fork || !side->join[0] || !side->join[1])
    return MOE_E_NULL;
  if (side->side[0] == side->side[1] || side->side[0] == stream || side->side[1] == stream)
    return MOE_E_ALIAS;
  if (side->fork == side->join[0] || side->fork == side->join[1] || side->join[0] == side->join[1])
    return MOE_E_ALIAS;
  return MOE_OK;
}

// moe_backward (lora null), moe_backward_lora (rank already checked) and
// moe_backward_side (ss: the caller's side streams and events; null: one
// stream).
int run_backward(const moe_dims* dims, const moe_weights* w, const moe_lora* lora, const uint16_t* x,
                 const moe_routes* routes, const moe_saved* saved, const uint16_t* d_out,
                 float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads, moe_lora_grads* lg, void* ws,
                 size_t ws_bytes, hipStream_t stream, const moe_side_streams* ss = nullptr) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved || !grads) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, K = d.top_k, E = d.experts, H = d.hidden, I = d.inter,
               Is = d.shared_inter;
  Args a;
  a.in(x, bytes_x(d));
  a.in(d_out, bytes_x(d));
  add_weights(a, d, w, true, true);
  a.in(routes->topk_idx, T * K * 4);
  a.in(routes->topk_gate, T * K * 4);
  a.in(routes->expert_offsets, (E + 1) * 4);
  a.in(routes->sorted_route, T * K * 4);
  a.in(saved->y, T * K * H * 4, false);  // not read: dg is formed from D and act
  a.in(saved->gu, T * K * 2 * I * 4);
  if (Is) {
    a.in(saved->shared_y, T * H * 4, false);  // not read: ds is formed from D and act
    a.in(saved->shared_gate, T * 4);
    a.in(saved->shared_gu, T * 2 * Is * 4);
  }
  a.out(d_x_f32, T * H * 4);
  a.out(d_x_bf16, T * H * 2, false);
  a.out(grads->d_w_router, E * H * 4);
  a.out(grads->d_w13, E * 2 * I * H * 4);
  a.out(grads->d_w2, E * H * I * 4);
  if (Is) {
    a.out(grads->d_ws13, 2 * Is * H * 4);
    a.out(grads->d_ws2, H * Is * 4);
    a.out(grads->d_w_sgate, H * 4);
  }
  const size_t rk = lora ? lora->rank : 0;
  if (lora) {
    a.in(lora->a13, E * rk * H * 2);
    a.in(lora->b13, E * 2 * I * rk * 2);
    a.in(lora->a2, E * rk * I * 2);
    a.in(lora->b2, E * H * rk * 2);
    a.out(lg->d_a13, E * rk * H * 4);
    a.out(lg->d_b13, E * 2 * I * rk * 4);
    a.out(lg->d_a2, E * rk * I * 4);
    a.out(lg->d_b2, E * H * rk * 4);
  }
  const int op = lora ? MOE_OP_BACKWARD_LORA : MOE_OP_BACKWARD;
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, op)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, op));
  MOE_TRY(check_device());
  const Layout L = make_layout(d);
  const bool sh = Is > 0;
  hipStream_t s = stream;
  // the backward's first kernel also overwrites the workspace's error word
  MOE_LAUNCH(moe::launch_ffn_tiles(routes->expert_offsets, at<int32_t>(ws, L.tiles_bwd), nullptr, 0,
                                   at<int32_t>(ws, L.meta_bwd), at<int>(ws, L.err), 1, d.experts, d.tokens,
                                   d.top_k, sh, moe::kBwdRowsPerTile, s));
  moe::BwdLaunch b;
  b.T = d.tokens;
  b.H = d.hidden;
  b.E = d.experts;
  b.K = d.top_k;
  b.I = d.inter;
  b.Is = d.shared_inter;
  b.max_tiles_bwd = L.max_tiles_bwd;
  b.offsets = routes->expert_offsets;
  b.sorted_route = routes->sorted_route;
  b.gate = routes->topk_gate;
  b.sg = sh ? saved->shared_gate : nullptr;
  b.tiles = at<int32_t>(ws, L.tiles_bwd);
  b.meta = at<int32_t>(ws, L.meta_bwd);
  b.x = x;
  b.dout = d_out;
  b.w13 = w->w13;
  b.w2 = w->w2;
  b.ws13 = sh ? w->ws13 : nullptr;
  b.ws2 = sh ? w->ws2 : nullptr;
  b.gu = saved->gu;
  b.sgu = sh ? saved->shared_gu : nullptr;
  for (int q = 0; q < moe::kGradPlanes; ++q) {
    b.dgu[q] = at<uint16_t>(ws, L.dgu[q]);
    b.sdgu[q] = at<uint16_t>(ws, L.sdgu[q]);
    b.gact[q] = at<uint16_t>(ws, L.gact[q]);
    b.sgact[q] = at<uint16_t>(ws, L.sgact[q]);
  }
  b.dgp = at<double>(ws, L.dgp);
  b.dsp = sh ? at<double>(ws, L.dsp) : nullptr;
  b.dx_route = at<float>(ws, L.dx_route);
  b.dx_shared = sh ? at<float>(ws, L.dx_shared) : nullptr;
  b.dw13 = grads->d_w13;
  b.dw2 = grads->d_w2;
  b.dws13 = sh ? grads->d_ws13 : nullptr;
  b.dws2 = sh ? grads->d_ws2 : nullptr;
  // the adapters' shrinks run over the 64-row work list of the forward
  auto shrink = [&](const uint16_t* vh, const uint16_t* vl, const uint16_t* am, size_t z, int kd) {
    return moe::launch_lora_shrink(vh, vl, am, routes->expert_offsets, routes->sorted_route,
                                   at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.meta), at<uint16_t>(ws, z),
                                   d.tokens, kd, d.experts, d.top_k, lora->rank, L.max_tiles, s);
  };
  if (lora) {
    b.la13 = lora->a13;
    b.la2 = lora->a2;
    b.lv2 = at<uint16_t>(ws, L.lora_v2);
    b.lu13 = at<uint16_t>(ws, L.lora_u13);
    b.lscale = lora->scale;
    b.lrank = lora->rank;
    MOE_LAUNCH(moe::launch_ffn_tiles(routes->expert_offsets, at<int32_t>(ws, L.tiles), nullptr, 0,
                                     at<int32_t>(ws, L.meta), at<int>(ws, L.err), 0, d.experts, d.tokens,
                                     d.top_k, sh, moe::kRowsPerTile, s));
    MOE_LAUNCH(moe::launch_lora_transpose(lora->b2, at<uint16_t>(ws, L.lora_b2t), d.experts, d.hidden,
                                          lora->rank, s));
    MOE_LAUNCH(moe::launch_lora_transpose(lora->b13, at<uint16_t>(ws, L.lora_b13t), d.experts,
                                          2 * d.inter, lora->rank, s));
    MOE_LAUNCH(shrink(d_out, nullptr, at<uint16_t>(ws, L.lora_b2t), L.lora_v2, d.hidden));
  }
  MOE_LAUNCH(moe::launch_bwd_dact(b, s));
  MOE_LAUNCH(moe::launch_bwd_gate(b.dgp, b.dsp, routes->topk_gate, sh ? saved->shared_gate : nullptr,
                                  at<float>(ws, L.dl), at<float>(ws, L.dz), d.tokens, d.top_k, d.inter,
                                  d.shared_inter, s));
  if (lora) {
    MOE_LAUNCH(shrink(b.dgu[0], b.dgu[1], at<uint16_t>(ws, L.lora_b13t), L.lora_u13, 2 * d.inter));
    MOE_LAUNCH(shrink(x, nullptr, lora->a13, L.lora_z13, d.hidden));
    MOE_LAUNCH(shrink(b.gact[0], b.gact[1], lora->a2, L.lora_z2, d.inter));
  }
  if (ss) {
    // the weight gradients on the side streams, from the point where dGU and
    // g*act exist; dx and everything after it stay on `stream`
    if (hipEventRecord(ss->fork, s) != hipSuccess) return MOE_E_LAUNCH;
    for (int i = 0; i < 2; ++i)
      if (hipStreamWaitEvent(ss->side[i], ss->fork, 0) != hipSuccess) return MOE_E_LAUNCH;
    MOE_LAUNCH(moe::launch_bwd_dw13(b, ss->side[0]));
    MOE_LAUNCH(moe::launch_bwd_dw2(b, ss->side[1]));
    for (int i = 0; i < 2; ++i)
      if (hipEventRecord(ss->join[i], ss->side[i]) != hipSuccess) return MOE_E_LAUNCH;
    MOE_LAUNCH(moe::launch_bwd_dx(b, s));
  } else {
    MOE_LAUNCH(moe::launch_bwd_gemms(b, s));
  }
  if (lora)
    MOE_LAUNCH(moe::launch_bwd_lora_grads(b, at<uint16_t>(ws, L.lora_z13), at<uint16_t>(ws, L.lora_z2),
                                          lg->d_a13, lg->d_b13, lg->d_a2, lg->d_b2, s));
  MOE_LAUNCH(moe::launch_bwd_router(x, at<float>(ws, L.dl), routes->expert_offsets,
                                    routes->sorted_route, grads->d_w_router, d.tokens, d.hidden,
                                    d.experts, d.top_k, s));
  if (sh)
    MOE_LAUNCH(moe::launch_bwd_wsg(x, at<float>(ws, L.dz), at<double>(ws, L.wsg_partial),
                                   grads->d_w_sgate, d.tokens, d.hidden, s));
  MOE_LAUNCH(moe::launch_bwd_dx_sum(routes->topk_idx, at<float>(ws, L.dl), at<float>(ws, L.dx_route),
                                    sh ? at<float>(ws, L.dx_shared) : nullptr, at<float>(ws, L.dz),
                                    sh ? w->w_sgate : nullptr, w->w_router, d_x_f32, d_x_bf16,
                                    d.tokens, d.hidden, d.experts, d.top_k, s));
  if (ss)
    for (int i = 0; i < 2; ++i)
      if (hipStreamWaitEvent(s, ss->join[i], 0) != hipSuccess) return MOE_E_LAUNCH;
  return MOE_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "required pointer is NULL";
    case MOE_E_SHAPE: return "dimension out of the supported range";
    case MOE_E_UNSUPPORTED: return "unsupported combination";
    case MOE_E_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_DEVICE: return "device is not gfx950, or device data error";
    case MOE_E_LAUNCH: return "kernel launch failed";
    case MOE_E_ALIAS: return "an output overlaps another buffer";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_dims* dims, int op) {
  if (check_dims(dims) != MOE_OK) return 0;
  const Layout L = make_layout(*dims);
  switch (op) {
    case MOE_OP_ROUTE:
    case MOE_OP_PERMUTE:
    case MOE_OP_FFN:
    case MOE_OP_FORWARD: return L.fwd_end;
    case MOE_OP_FORWARD_LORA: return L.lora_end;
    case MOE_OP_BACKWARD_LORA: return L.lora_bwd_end;
    case MOE_OP_BACKWARD: return L.bwd_end;
    default: return 0;
  }
}

int moe_route(const moe_dims* dims, const uint16_t* x, const moe_weights* w, moe_routes* routes,
              void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes) return MOE_E_NULL;
  const moe_dims& d = *dims;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, true, false);
  add_routes_out(a, d, routes);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_ROUTE)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_ROUTE));
  MOE_TRY(check_device());
  return run_route(d, x, w, routes, ws, make_layout(d), nullptr, stream);
}

int moe_permute(const moe_dims* dims, moe_routes* routes, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!routes) return MOE_E_NULL;
  const moe_dims& d = *dims;
  Args a;
  a.in(routes->topk_idx, static_cast<size_t>(d.tokens) * d.top_k * 4);
  add_perm_out(a, d, routes);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_PERMUTE)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_PERMUTE));
  MOE_TRY(check_device());
  return run_permute(d, routes, ws, make_layout(d), stream);
}

int moe_grouped_ffn(const moe_dims* dims, const uint16_t* x, const moe_weights* w,
                    const moe_routes* routes, moe_saved* saved, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, K = d.top_k, E = d.experts;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, false, true);
  a.in(routes->expert_offsets, (E + 1) * 4);
  a.in(routes->sorted_route, T * K * 4);
  add_saved(a, d, saved, true);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FFN)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FFN));
  MOE_TRY(check_device());
  return run_ffn(d, x, w, routes, saved, ws, make_layout(d), false, stream);
}

int moe_grouped_ffn_lora(const moe_dims* dims, const uint16_t* x, const moe_weights* w,
                         const moe_lora* lora, const moe_routes* routes, moe_saved* saved, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (!lora) return MOE_E_NULL;
  if (lora->rank < 1 || lora->rank > moe::kLoraMaxRank) return MOE_E_SHAPE;
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, K = d.top_k, E = d.experts, H = d.hidden, I = d.inter, rk = lora->rank;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, false, true);
  a.in(lora->a13, E * rk * H * 2);
  a.in(lora->b13, E * 2 * I * rk * 2);
  a.in(lora->a2, E * rk * I * 2);
  a.in(lora->b2, E * H * rk * 2);
  a.in(routes->expert_offsets, (E + 1) * 4);
  a.in(routes->sorted_route, T * K * 4);
  add_saved(a, d, saved, true);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FORWARD_LORA)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FORWARD_LORA));
  MOE_TRY(check_device());
  return run_ffn(d, x, w, routes, saved, ws, make_layout(d), false, stream, nullptr, nullptr, lora);
}

int moe_combine(const moe_dims* dims, const moe_routes* routes, const moe_saved* saved,
                float* out_f32, uint16_t* out_bf16, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!routes || !saved) return MOE_E_NULL;
  if (!out_f32 && !out_bf16) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, K = d.top_k, H = d.hidden;
  Args a;
  a.in(routes->topk_gate, T * K * 4);
  a.in(saved->y, T * K * H * 4);
  if (d.shared_inter) {
    a.in(saved->shared_y, T * H * 4);
    a.in(saved->shared_gate, T * 4);
  }
  a.out(out_f32, T * H * 4, false);
  a.out(out_bf16, T * H * 2, false);
  MOE_TRY(a.status());
  MOE_TRY(check_device());
  return run_combine(d, routes, saved, out_f32, out_bf16, stream);
}

int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, moe_routes* routes,
                moe_saved* saved, float* out_f32, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  if (!out_f32 && !out_bf16) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, H = d.hidden;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, true, true);
  add_routes_out(a, d, routes);
  add_perm_out(a, d, routes);
  add_saved(a, d, saved, true);
  a.out(out_f32, T * H * 4, false);
  a.out(out_bf16, T * H * 2, false);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FORWARD)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FORWARD));
  MOE_TRY(check_device());
  const Layout L = make_layout(d);
  MOE_TRY(run_route(d, x, w, routes, ws, L, d.shared_inter > 0 ? saved->shared_gate : nullptr,
                    stream));
  MOE_TRY(run_permute(d, routes, ws, L, stream));
  MOE_TRY(run_ffn(d, x, w, routes, saved, ws, L, true, stream));
  return run_combine(d, routes, saved, out_f32, out_bf16, stream);
}

int moe_forward_side(const moe_dims* dims, const moe_weights* w, const uint16_t* x, moe_routes* routes,
                     moe_saved* saved, float* out_f32, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                     hipStream_t stream, const moe_side_streams* side) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  if (!out_f32 && !out_bf16) return MOE_E_NULL;
  MOE_TRY(check_side(side, stream));
  const moe_dims& d = *dims;
  const size_t T = d.tokens, H = d.hidden;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, true, true);
  add_routes_out(a, d, routes);
  add_perm_out(a, d, routes);
  add_saved(a, d, saved, true);
  a.out(out_f32, T * H * 4, false);
  a.out(out_bf16, T * H * 2, false);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FORWARD)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FORWARD));
  MOE_TRY(check_device());
  const Layout L = make_layout(d);
  const bool sh = d.shared_inter > 0;
  if (sh) {
    // the shared expert on side[0], from this point of the call's stream
    if (hipEventRecord(side->fork, stream) != hipSuccess) return MOE_E_LAUNCH;
    if (hipStreamWaitEvent(side->side[0], side->fork, 0) != hipSuccess) return MOE_E_LAUNCH;
    MOE_TRY(run_shared_ffn(d, x, w, routes, saved, ws, L, side->side[0]));
    if (hipEventRecord(side->join[0], side->side[0]) != hipSuccess) return MOE_E_LAUNCH;
  }
  MOE_TRY(run_route(d, x, w, routes, ws, L, sh ? saved->shared_gate : nullptr, stream));
  MOE_TRY(run_permute(d, routes, ws, L, stream, false));
  MOE_TRY(run_ffn(d, x, w, routes, saved, ws, L, true, stream));
  if (sh && hipStreamWaitEvent(stream, side->join[0], 0) != hipSuccess) return MOE_E_LAUNCH;
  return run_combine(d, routes, saved, out_f32, out_bf16, stream);
}

int moe_forward_lora(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                     const uint16_t* x, moe_routes* routes, moe_saved* saved, float* out_f32,
                     uint16_t* out_bf16, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (!lora) return MOE_E_NULL;
  if (lora->rank < 1 || lora->rank > moe::kLoraMaxRank) return MOE_E_SHAPE;
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  if (!out_f32 && !out_bf16) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, H = d.hidden, E = d.experts, I = d.inter, rk = lora->rank;
  Args a;
  a.in(x, bytes_x(d));
  add_weights(a, d, w, true, true);
  a.in(lora->a13, E * rk * H * 2);
  a.in(lora->b13, E * 2 * I * rk * 2);
  a.in(lora->a2, E * rk * I * 2);
  a.in(lora->b2, E * H * rk * 2);
  add_routes_out(a, d, routes);
  add_perm_out(a, d, routes);
  add_saved(a, d, saved, true);
  a.out(out_f32, T * H * 4, false);
  a.out(out_bf16, T * H * 2, false);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FORWARD_LORA)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FORWARD_LORA));
  MOE_TRY(check_device());
  const Layout L = make_layout(d);
  MOE_TRY(run_route(d, x, w, routes, ws, L, d.shared_inter > 0 ? saved->shared_gate : nullptr,
                    stream));
  MOE_TRY(run_permute(d, routes, ws, L, stream));
  MOE_TRY(run_ffn(d, x, w, routes, saved, ws, L, true, stream, nullptr, nullptr, lora));
  return run_combine(d, routes, saved, out_f32, out_bf16, stream);
}

int moe_forward_mx(const moe_dims* dims, const moe_weights_mx* w, const uint16_t* x,
                   moe_routes* routes, moe_saved* saved, float* out_f32, uint16_t* out_bf16,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!w || !routes || !saved) return MOE_E_NULL;
  if (!out_f32 && !out_bf16) return MOE_E_NULL;
  const moe_dims& d = *dims;
  const size_t T = d.tokens, H = d.hidden, E = d.experts, I = d.inter, Is = d.shared_inter;
  Args a;
  a.in(x, bytes_x(d));
  a.in(w->w_router, E * H * 4);
  a.in(w->router_bias, E * 4, false);
  a.in(w->w_router_planes, 3 * E * H * 2, false);
  a.in(w->w13_q, E * 2 * I * H);
  a.in(w->w13_s, E * 2 * I * (H / 32));
  a.in(w->w2_q, E * H * I);
  a.in(w->w2_s, E * H * (I / 32));
  if (Is) {
    a.in(w->ws13_q, 2 * Is * H);
    a.in(w->ws13_s, 2 * Is * (H / 32));
    a.in(w->ws2_q, H * Is);
    a.in(w->ws2_s, H * (Is / 32));
    a.in(w->w_sgate, H * 2);
  }
  add_routes_out(a, d, routes);
  add_perm_out(a, d, routes);
  add_saved(a, d, saved, true);
  a.out(out_f32, T * H * 4, false);
  a.out(out_bf16, T * H * 2, false);
  a.in(ws, std::min(ws_bytes, moe_workspace_bytes(dims, MOE_OP_FORWARD)), false);
  MOE_TRY(a.status());
  MOE_TRY(check_ws(d, ws, ws_bytes, MOE_OP_FORWARD));
  MOE_TRY(check_device());
  moe_weights wr = {};
  wr.w_router = w->w_router;
  wr.router_bias = w->router_bias;
  wr.w_sgate = w->w_sgate;
  wr.w_router_planes = w->w_router_planes;
  const moe::MxWeights mx13{w->w13_q, w->w13_s, w->ws13_q, w->ws13_s};
  const moe::MxWeights mx2{w->w2_q, w->w2_s, w->ws2_q, w->ws2_s};
  const Layout L = make_layout(d);
  MOE_TRY(run_route(d, x, &wr, routes, ws, L, d.shared_inter > 0 ? saved->shared_gate : nullptr,
                    stream));
  MOE_TRY(run_permute(d, routes, ws, L, stream));
  MOE_TRY(run_ffn(d, x, &wr, routes, saved, ws, L, true, stream, &mx13, &mx2));
  return run_combine(d, routes, saved, out_f32, out_bf16, stream);
}

namespace {
const char* const kFwdSmall[] = {"router_split", "router_logits", "topk_gate", "route_sort",
                                 "ffn_up", "ffn_down", "combine"};
const char* const kFwdLarge[] = {"router_split", "router_logits", "topk_gate", "route_hist",
                                 "route_scan", "route_scatter", "ffn_up", "ffn_down", "combine"};
}  // namespace

int moe_forward_kernel_count(const moe_dims* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return moe::sort_small_fits(dims->tokens, dims->experts) ? 7 : 9;
}

const char* moe_forward_kernel_name(const moe_dims* dims, int i) {
  const int n = moe_forward_kernel_count(dims);
  if (i < 0 || i >= n) return nullptr;
  return n == 7 ? kFwdSmall[i] : kFwdLarge[i];
}

int moe_forward_profiled(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                         moe_routes* routes, moe_saved* saved, float* out_f32,
                         uint16_t* out_bf16, void* ws, size_t ws_bytes, hipEvent_t* events,
                         int n_events, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (!events) return MOE_E_NULL;
  if (n_events < moe_forward_kernel_count(dims) + 1) return MOE_E_SHAPE;
  Marks marks;
  marks.ev = events;
  marks.n = n_events;
  marks.s = stream;
  g_marks = &marks;
  const int st = moe_forward(dims, w, x, routes, saved, out_f32, out_bf16, ws, ws_bytes, stream);
  g_marks = nullptr;
  if (st != MOE_OK) return st;
  if (dims->tokens > 0 && marks.mark() != hipSuccess) return MOE_E_LAUNCH;
  return MOE_OK;
}

int moe_backward(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                 const moe_routes* routes, const moe_saved* saved, const uint16_t* d_out,
                 float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  return run_backward(dims, w, nullptr, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, nullptr, ws,
                      ws_bytes, stream);
}

int moe_backward_side(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                      const moe_routes* routes, const moe_saved* saved, const uint16_t* d_out,
                      float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads, void* ws, size_t ws_bytes,
                      hipStream_t stream, const moe_side_streams* side) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  MOE_TRY(check_side(side, stream));
  return run_backward(dims, w, nullptr, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, nullptr, ws,
                      ws_bytes, stream, side);
}

int moe_backward_lora_side(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                           const uint16_t* x, const moe_routes* routes, const moe_saved* saved,
                           const uint16_t* d_out, float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads,
                           moe_lora_grads* lora_grads, void* ws, size_t ws_bytes, hipStream_t stream,
                           const moe_side_streams* side) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!lora || !lora_grads) return MOE_E_NULL;
  if (lora->rank < 1 || lora->rank > moe::kLoraMaxRank) return MOE_E_SHAPE;
  MOE_TRY(check_side(side, stream));
  return run_backward(dims, w, lora, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, lora_grads, ws,
                      ws_bytes, stream, side);
}

int moe_backward_lora(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                      const uint16_t* x, const moe_routes* routes, const moe_saved* saved,
                      const uint16_t* d_out, float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads,
                      moe_lora_grads* lora_grads, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  if (dims->tokens == 0) return MOE_OK;
  if (!lora || !lora_grads) return MOE_E_NULL;
  if (lora->rank < 1 || lora->rank > moe::kLoraMaxRank) return MOE_E_SHAPE;
  return run_backward(dims, w, lora, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, lora_grads, ws,
                      ws_bytes, stream);
}

int moe_split_router(const moe_dims* dims, const float* w_router, uint16_t* planes,
                     hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const size_t E = dims->experts, H = dims->hidden;
  Args a;
  a.in(w_router, E * H * 4);
  a.out(planes, 3 * E * H * 2);
  MOE_TRY(a.status());
  MOE_TRY(check_device());
  MOE_LAUNCH(moe::launch_router_split(w_router, planes, dims->hidden, dims->experts, stream));
  return MOE_OK;
}

int moe_last_device_error(void* ws, hipStream_t stream) {
  if (!ws) return MOE_E_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_E_LAUNCH;
  int v = 0;
  if (hipMemcpy(&v, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_E_LAUNCH;
  return v ? MOE_E_DEVICE : MOE_OK;
}

}  // extern "C"
