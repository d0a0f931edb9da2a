// C ABI of the MoE layer: validation, workspace layout and launch sequences.
// Every entry point validates its arguments completely before it enqueues
// anything, so a rejected call leaves the stream and all outputs untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOE_HIP(call, where)                          \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

constexpr size_t kAlign = 256;
size_t al(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Validated shape and the sizes derived from it.
struct Shape {
  int T, d, E, k, dff, nsh, dffs;
  int gate_all, bf16, elt;
  long long C;          // capacity, -1 when it cannot bind
  int R;                // T*k routed rows (buffer size)
  int rows_total;       // R + n_shared*T
  int act_stride;
  int BM, max_tiles;
  bool n256;            // d % 256 == 0 and d_ff, d_ff_shared % 128 == 0 (large tiles)
  int nb_sel, nb_idx, nkeys;
  int ep;               // simulated expert-parallel ranks (1: off)
  int G;                // row groups: E, or ep*E in the expert-parallel layout
};

moe_status validate(const moe_config* c, Shape* s) {
  if (c == nullptr) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->reserved2 != 0.0f) return fail(MOE_ERR_INVALID_ARG, "reserved fields must be 0");
  if (c->ep_ranks < 0) return fail(MOE_ERR_INVALID_ARG, "ep_ranks=%d < 0", c->ep_ranks);
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", c->T);
  if (c->E < 1 || c->E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d not in [1, 1024]", c->E);
  if (c->k < 1 || c->k > c->E || c->k > 16)
    return fail(MOE_ERR_INVALID_ARG, "k=%d not in [1, min(E, 16)]", c->k);
  if (c->d < 1 || c->d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "d=%d, d_ff=%d must be > 0", c->d, c->d_ff);
  if (c->n_shared != 0 && c->n_shared != 1)
    return fail(MOE_ERR_INVALID_ARG, "n_shared=%d must be 0 or 1", c->n_shared);
  if (c->n_shared == 1 && c->d_ff_shared < 1)
    return fail(MOE_ERR_INVALID_ARG, "d_ff_shared=%d must be > 0", c->d_ff_shared);
  if (c->gate_mode != MOE_GATE_SOFTMAX_SELECTED && c->gate_mode != MOE_GATE_SOFTMAX_ALL)
    return fail(MOE_ERR_INVALID_ARG, "gate_mode=%d unknown", c->gate_mode);
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype=%d unknown", c->dtype);
  if (std::isnan(c->capacity_factor) || std::isinf(c->capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if (!std::isfinite(c->aux_alpha)) return fail(MOE_ERR_INVALID_ARG, "aux_alpha must be finite");
  const int dffs = c->n_shared ? c->d_ff_shared : 0;
  if (c->d % 64 || c->d_ff % 64 || dffs % 64)
    return fail(MOE_ERR_UNSUPPORTED, "d=%d, d_ff=%d, d_ff_shared=%d must be multiples of 64",
                c->d, c->d_ff, dffs);
  const long long R = static_cast<long long>(c->T) * c->k;
  const long long rows = R + static_cast<long long>(c->n_shared) * c->T;
  if (rows > (1LL << 30)) return fail(MOE_ERR_INVALID_ARG, "T*k + n_shared*T = %lld too large", rows);

  s->T = c->T; s->d = c->d; s->E = c->E; s->k = c->k; s->dff = c->d_ff;
  s->nsh = c->n_shared; s->dffs = dffs;
  s->gate_all = c->gate_mode == MOE_GATE_SOFTMAX_ALL;
  s->bf16 = c->dtype == MOE_BF16;
  s->elt = s->bf16 ? 2 : 4;
  s->R = static_cast<int>(R);
  s->rows_total = static_cast<int>(rows);
  s->act_stride = c->d_ff > dffs ? c->d_ff : dffs;
  // C = ceil(k*T/E * cf) in double; it cannot bind when C >= T (a token picks an
  // expert at most once), so that case runs the capacity-free path.
  s->C = -1;
  if (c->capacity_factor > 0) {
    const double cd = std::ceil(static_cast<double>(R) / c->E * c->capacity_factor);
    if (cd < static_cast<double>(c->T)) s->C = static_cast<long long>(cd);
  }
  s->ep = c->ep_ranks > 1 ? c->ep_ranks : 1;
  s->G = s->E;
  if (s->ep > 1) {
    if (s->E % s->ep || s->T % s->ep)
      return fail(MOE_ERR_INVALID_ARG, "ep_ranks=%d must divide E=%d and T=%d", s->ep, s->E, s->T);
    if (c->capacity_factor > 0)
      return fail(MOE_ERR_UNSUPPORTED, "capacity with ep_ranks > 1 is not supported");
    if (static_cast<long long>(s->ep) * s->E > 1024)
      return fail(MOE_ERR_UNSUPPORTED, "ep_ranks*E=%lld > 1024 row groups",
                  static_cast<long long>(s->ep) * s->E);
    s->G = s->ep * s->E;
  }
  s->nkeys = moe::index_keys(s->G, s->k, s->C >= 0);
  if (s->nkeys > moe::kIndexMaxKeys)
    return fail(MOE_ERR_UNSUPPORTED, "capacity with E*k=%d > %d is not supported", s->nkeys,
                moe::kIndexMaxKeys);
  s->n256 = (s->d % 256 == 0) && (s->dff % 128 == 0) && (s->dffs % 128 == 0);
  s->BM = moe::gemm_tile_rows(s->bf16, s->R, s->G, s->n256);
  s->max_tiles = moe::gemm_max_tiles(s->BM, s->R, s->G);
  s->nb_sel = moe::router_select_blocks(s->T);
  s->nb_idx = moe::index_blocks(s->T);
  return MOE_OK;
}

// workspace sizes per stage
size_t zpart_bytes(const Shape& s) {
  return al(moe::router_scores_part_floats(s.bf16, s.T, s.d, s.E) * 4);
}
size_t route_bytes(const Shape& s) {
  return al(static_cast<size_t>(s.T) * s.E * 4) + 2 * al(static_cast<size_t>(s.nb_sel) * s.E * 4) +
         al(static_cast<size_t>(s.E) * 4) +
         al(static_cast<size_t>(s.nb_sel) * moe::kScaleStats * 4) + zpart_bytes(s);
}
size_t permute_bytes(const Shape& s) {
  return al(static_cast<size_t>(s.nb_idx + 1) * s.nkeys * 4) + 2 * al(static_cast<size_t>(s.k) * s.G * 4) +
         (s.ep > 1 ? al(static_cast<size_t>(s.R) * 4) : 0);
}
size_t tiles_bytes(const Shape& s) { return al(static_cast<size_t>(s.max_tiles) * 16); }
// stream-K partial tiles of the down product (256-row tiles only)
size_t sk_bytes(const Shape& s) { return s.bf16 && s.BM == 256 ? moe::kStreamKPartBytes : 0; }
size_t act_bytes(const Shape& s) {
  return al(static_cast<size_t>(s.rows_total) * s.act_stride * s.elt);
}
size_t yperm_bytes(const Shape& s) { return al(static_cast<size_t>(s.rows_total) * s.d * 4); }
size_t forward_fixed_bytes(const Shape& s) {
  const size_t R4 = al(static_cast<size_t>(s.R) * 4);
  return 4 * R4 + al(static_cast<size_t>(s.G + 1) * 4) + yperm_bytes(s) + act_bytes(s);
}

struct Carver {
  char* p;
  template <typename T>
  T* take(size_t bytes) {
    T* r = reinterpret_cast<T*>(p);
    p += al(bytes);
    return r;
  }
};

// Workspace of moe_backward: every buffer of the recomputed forward and of the
// backward, carved in this order (a null base only measures the size).
struct BwdBufs {
  float *z, *zpart, *gates, *h1, *h3, *row_gate, *dg_row, *dz, *u, *dxp, *dxp2, *wpart, *rpart;
  int32_t *idx, *dest, *src, *offsets, *counts, *kept, *ndrop, *soff, *tiles, *tiles256;
  int32_t *blk, *slot_base, *slot_keep, *chunk_off;
  uint16_t *act, *dyb, *dyp, *dH, *xp, *dzs;
  int max_tiles256;
  int rchunks;      // > 0: the router's gradients as MFMA products over this many token chunks
  bool split_dx;    // routed dX_perm in two halves (W1 part, W3 part), summed by unpermute_dx
};

// The activation products (u = dy W2, dX = dH [W1; W3]) read the experts' weights
// K-major (gemm_kmajor_w4_kernel, through the LDS transpose read). Measured
// against transposing the weights in memory once per call (on a side stream,
// beside the recomputed gate/up product) and running the forward's K-contiguous
// kernel: Mixtral layer at 4096 tokens 10.45 -> 9.21 ms with 2.9 GB less
// workspace; the shared expert of the DeepSeek layer u 140 + dX 321 us
// transposed (plus three transposes of 0.2 ms each) against 186 + 231 us.

// The routed dX_perm product (N = d) has few output tiles per CU when the groups
// are long: at the Mixtral shape (4096 tokens) 35 x 16 tiles, 2.2 per CU, so its
// last round of workgroups ran a fifth full. Below four tiles per CU the grid
// runs twice, each copy over half of K (W1, then W3), into two buffers that
// unpermute_dx adds.
constexpr int kSplitDxTilesPerCU = 4;

size_t backward_layout(const Shape& s, char* base, BwdBufs* b) {
  Carver cv{base};
  const size_t T = s.T, E = s.E, k = s.k, R = s.R, d = s.d, As = s.act_stride;
  const size_t rows = s.rows_total;
  b->max_tiles256 = moe::gemm_max_tiles(256, s.R, s.E);
  const long long dx_tiles =
      static_cast<long long>(s.BM == 256 ? s.max_tiles : b->max_tiles256) * (s.d / 256);
  b->split_dx = dx_tiles < static_cast<long long>(kSplitDxTilesPerCU) * 256;
  b->z = cv.take<float>(T * E * 4);
  b->zpart = cv.take<float>(zpart_bytes(s));
  b->idx = cv.take<int32_t>(T * k * 4);
  b->gates = cv.take<float>(T * k * 4);
  b->dest = cv.take<int32_t>(T * k * 4);
  b->src = cv.take<int32_t>(R * 4);
  b->offsets = cv.take<int32_t>((E + 1) * 4);
  b->counts = cv.take<int32_t>(E * 4);
  b->kept = cv.take<int32_t>(E * 4);
  b->ndrop = cv.take<int32_t>(4);
  b->soff = cv.take<int32_t>(2 * 4);
  b->tiles = cv.take<int32_t>(static_cast<size_t>(s.max_tiles) * 16);
  b->tiles256 = cv.take<int32_t>(static_cast<size_t>(b->max_tiles256) * 16);
  b->blk = cv.take<int32_t>(static_cast<size_t>(s.nb_idx + 1) * s.nkeys * 4);
  b->slot_base = cv.take<int32_t>(k * E * 4);
  b->slot_keep = cv.take<int32_t>(k * E * 4);
  b->h1 = cv.take<float>(rows * As * 4);
  b->h3 = cv.take<float>(rows * As * 4);
  b->act = cv.take<uint16_t>(rows * As * 2);
  b->dyb = cv.take<uint16_t>(T * d * 2);
  b->dyp = cv.take<uint16_t>(R * d * 2);
  b->xp = cv.take<uint16_t>(R * d * 2);
  b->row_gate = cv.take<float>(R * 4);
  b->dg_row = cv.take<float>(R * 4);
  b->dz = cv.take<float>(T * E * 4);
  b->u = cv.take<float>(rows * As * 4);
  b->dH = cv.take<uint16_t>(rows * 2 * As * 2);
  b->dxp = cv.take<float>(rows * d * 4);
  b->dxp2 = cv.take<float>(b->split_dx ? R * d * 4 : 0);
  // wide routers: dz W_r and dz^T x on the MFMA kernels, the token chunks of dW_r
  // sized so the grouped-K product has about one tile per CU
  b->rchunks = 0;
  if (moe::router_grad_mfma(s.E)) {
    const int per_chunk = (2 * s.E / 256) * (s.d / 256);
    const int want = per_chunk < 256 ? 256 / per_chunk : 1;
    const int most = (s.T + 255) / 256;
    b->rchunks = want < most ? want : most;
  }
  b->dzs = cv.take<uint16_t>(b->rchunks ? T * 2 * E * 2 : 0);
  b->chunk_off = cv.take<int32_t>(b->rchunks ? (static_cast<size_t>(b->rchunks) + 1) * 4 : 0);
  b->rpart = cv.take<float>(static_cast<size_t>(b->rchunks) * 2 * E * d * 4);
  b->wpart = cv.take<float>(b->rchunks ? 0 :
                            static_cast<size_t>(moe::router_wgrad_plan(s.T, s.E, s.d).chunks) *
                            E * d * 4);
  return static_cast<size_t>(cv.p - base);
}

size_t stage_bytes(const Shape& s, moe_stage st) {
  size_t b = 0;
  switch (st) {
    case MOE_STAGE_ROUTE: b = route_bytes(s); break;
    case MOE_STAGE_PERMUTE: b = permute_bytes(s); break;
    case MOE_STAGE_EXPERT_GATEUP: b = tiles_bytes(s); break;
    case MOE_STAGE_EXPERT_DOWN: b = tiles_bytes(s) + sk_bytes(s); break;
    case MOE_STAGE_EXPERT_FFN: b = act_bytes(s) + tiles_bytes(s) + sk_bytes(s); break;
    case MOE_STAGE_COMBINE: b = 0; break;
    case MOE_STAGE_FORWARD: {
      size_t scratch = route_bytes(s);
      // the index writes the tile table at the start of the scratch while its own
      // buffers (after the table) are still in use
      if (tiles_bytes(s) + permute_bytes(s) > scratch) scratch = tiles_bytes(s) + permute_bytes(s);
      if (tiles_bytes(s) + sk_bytes(s) > scratch) scratch = tiles_bytes(s) + sk_bytes(s);
      b = forward_fixed_bytes(s) + scratch;
      break;
    }
    case MOE_STAGE_BACKWARD: {
      BwdBufs bb;
      b = backward_layout(s, nullptr, &bb);
      break;
    }
  }
  return b < kAlign ? kAlign : b;
}



moe_status check_ws(const Shape& s, moe_stage st, const void* ws, size_t ws_bytes) {
  if (st == MOE_STAGE_COMBINE) return MOE_OK;   // uses no scratch: ws may be NULL
  const size_t need = stage_bytes(s, st);
  if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

#define REQUIRE(ptr)                                                            \
  do {                                                                          \
    if ((ptr) == nullptr) return fail(MOE_ERR_INVALID_ARG, #ptr " is NULL");    \
    if (!aligned16(ptr)) return fail(MOE_ERR_INVALID_ARG, #ptr " not 16-byte aligned"); \
  } while (0)

bool want_route_stats(const moe_stats* st) {
  return st != nullptr && (st->f != nullptr || st->P != nullptr || st->aux != nullptr ||
                           st->z_loss != nullptr || st->entropy != nullptr ||
                           st->max_prob != nullptr || st->top_gap != nullptr ||
                           st->margin != nullptr);
}

// ---- stage bodies (arguments already validated)

moe_status do_route(const Shape& s, float alpha, const void* x, const void* wr, const float* bias,
                    int32_t* idx, float* gates, const moe_stats* st, void* ws, hipStream_t stream) {
  Carver cv{static_cast<char*>(ws)};
  float* z = cv.take<float>(static_cast<size_t>(s.T) * s.E * 4);
  float* p_part = cv.take<float>(static_cast<size_t>(s.nb_sel) * s.E * 4);
  int32_t* c_part = cv.take<int32_t>(static_cast<size_t>(s.nb_sel) * s.E * 4);
  float* fp = cv.take<float>(static_cast<size_t>(s.E) * 4);
  float* q_part = cv.take<float>(static_cast<size_t>(s.nb_sel) * moe::kScaleStats * 4);
  float* zpart = cv.take<float>(zpart_bytes(s));
  const bool stats = want_route_stats(st);
  const bool scale = stats && (st->z_loss || st->entropy || st->max_prob || st->top_gap);
  MOE_HIP(moe::launch_router_scores(s.bf16, x, wr, s.T, s.d, s.E, z, zpart, stream),
          "router_scores");
  MOE_HIP(moe::launch_router_select(z, bias, s.T, s.E, s.k, s.gate_all, idx, gates,
                                    stats ? p_part : nullptr, stats ? c_part : nullptr,
                                    scale ? q_part : nullptr, stats ? st->margin : nullptr,
                                    stream),
          "router_select");
  if (stats)
    MOE_HIP(moe::launch_router_stats(p_part, c_part, scale ? q_part : nullptr, s.nb_sel, s.T, s.E,
                                     alpha, st->f, st->P, st->aux, fp, st->z_loss, st->entropy,
                                     st->max_prob, st->top_gap, stream),
            "router_stats");
  return MOE_OK;
}

// the load statistics of `st` (nullable) that the index kernels write
moe::LoadOut load_out(const moe_stats* st) {
  moe::LoadOut o;
  if (st != nullptr) {
    o.counts = st->counts;
    o.kept = st->kept;
    o.n_dropped = st->n_dropped;
    o.touched = st->touched;
    o.max_over_mean = st->max_over_mean;
  }
  return o;
}

// tiles (nullable): also build the grouped GEMM tile table there; it may alias
// the workspace (written after the index kernels are done with it)
moe_status do_permute(const Shape& s, const int32_t* idx, const void* x, int32_t* offsets,
                      int32_t* dest, int32_t* src, void* x_perm, const moe_stats* st, void* ws,
                      int32_t* tiles, hipStream_t stream) {
  Carver cv{static_cast<char*>(ws)};
  int32_t* blk = cv.take<int32_t>(static_cast<size_t>(s.nb_idx + 1) * s.nkeys * 4);
  int32_t* slot_base = cv.take<int32_t>(static_cast<size_t>(s.k) * s.G * 4);
  int32_t* slot_keep = cv.take<int32_t>(static_cast<size_t>(s.k) * s.G * 4);
  const int32_t* keys = idx;
  if (s.ep > 1) {
    // expert-parallel layout: group (destination rank, source rank, local expert)
    int32_t* gid = cv.take<int32_t>(static_cast<size_t>(s.R) * 4);
    MOE_HIP(moe::launch_ep_group_ids(idx, s.T, s.k, s.E, s.ep, gid, stream), "ep_group_ids");
    keys = gid;
  }
  MOE_HIP(moe::launch_index(keys, s.T, s.k, s.G, s.C, blk, slot_base, slot_keep, offsets, dest,
                            src, load_out(st), s.BM, s.max_tiles, s.ep, tiles, stream),
          "index");
  if (x_perm != nullptr)
    MOE_HIP(moe::launch_gather_rows(s.elt, x, src, offsets, s.G, s.R, s.d, x_perm, stream),
            "gather_rows");
  return MOE_OK;
}

struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;   // held by a call from its fork to its join
constexpr int kMaxDevices = 64;

// The device's side stream, or nullptr if it cannot be created (the caller then
// keeps that work on its own stream). Call with g_side_mu held.
SideStream* side_stream() {
  static SideStream side[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = side[dev];
  if (ss.s == nullptr) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f != nullptr) (void)hipEventDestroy(f);
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    ss.s = st;
    ss.fork = f;
    ss.join = j;
  }
  return &ss;
}

// rows per non-empty group on average (at most R groups hold rows)
int avg_group_rows(const Shape& s) {
  const int g = s.G < s.R ? s.G : s.R;
  return g > 0 ? s.R / g : 0;
}

// Decode-sized layers with a shared expert: where both products take the 16-row
// streaming tiles, the shared expert's items join the routed launch (DeepSeek
// shape, one token: 0.179 -> 0.165 ms). Otherwise, over more than 16 tokens, the
// shared expert's product (one dense group, too few tiles to fill the device
// alone) runs on the side stream beside the routed one: both only stream weights
// from HBM, and side by side each fills the other's idle CUs, ramp and tail
// (DeepSeek shape at 64 tokens: 3.34 -> 3.27 ms before the joint launch took its
// gate/up product; at one token the side stream only added the fork). It is forked
// from the caller's stream before either launch and joined back after both, so
// the call's work stays ordered on the caller's stream; it uses no scratch
// (no stream-K) and writes rows of its own (the shared block).
struct SharedOnSide {
  std::unique_lock<std::mutex> lock{g_side_mu, std::defer_lock};
  SideStream* side = nullptr;

  moe_status fork(const Shape& s, int shared_bm, hipStream_t stream) {
    if (!(s.nsh && s.bf16 && s.BM == 16 && s.T > 16 && shared_bm != 256)) return MOE_OK;
    return fork_now(stream);
  }
  // fork whatever the shape (side stays nullptr if there is no side stream)
  moe_status fork_now(hipStream_t stream) {
    lock.lock();
    side = side_stream();
    if (side == nullptr) { lock.unlock(); return MOE_OK; }
    MOE_HIP(hipEventRecord(side->fork, stream), "fork");
    MOE_HIP(hipStreamWaitEvent(side->s, side->fork, 0), "fork");
    return MOE_OK;
  }
  hipStream_t stream_for_shared(hipStream_t stream) const { return side ? side->s : stream; }
  moe_status join(hipStream_t stream) {
    if (side == nullptr) return MOE_OK;
    MOE_HIP(hipEventRecord(side->join, side->s), "join");
    MOE_HIP(hipStreamWaitEvent(stream, side->join, 0), "join");
    side = nullptr;
    lock.unlock();
    return MOE_OK;
  }
};

// Tile rows of the shared expert's gate/up product (one group of T rows): the
// 16-row streaming kernel up to 128 rows, where it beats the 32-row tiles at
// every measured size (DeepSeek shape, 64 rows: 96 -> 43 us); else as routed.
int shared_gateup_rows(const Shape& s) {
  const int bm = moe::gemm_tile_rows(s.bf16, s.T, 1, s.n256);
  return s.bf16 && s.T <= 128 ? 16 : bm;
}

// shared_done: the shared expert's rows of act are already being written (the
// fused forward's decode steps start that product on the side stream first)
moe_status do_gateup(const Shape& s, const void* x, const int32_t* src, const int32_t* tiles,
                     const void* w1, const void* w3, const void* ws1, const void* ws3, void* act,
                     hipStream_t stream, bool shared_done = false) {
  moe::GemmTileMap map{tiles, s.max_tiles, 0, moe::gemm_n_fast(s.BM, s.R, s.E), avg_group_rows(s)};
  moe::GateUpArgs a{x, src, w1, w3, static_cast<long long>(s.dff) * s.d, act, s.act_stride, 0,
                    s.d, s.dff};
  if (shared_done) {
    MOE_HIP(moe::launch_gemm_gateup_bf16(map, a, s.BM, stream), "gemm_gateup");
    return MOE_OK;
  }
  const int bm_sh = shared_gateup_rows(s);
  if (s.nsh && s.bf16 && s.BM == 16 && bm_sh == 16) {
    // both stream weights in 16-row tiles: one launch for the two
    moe::GateUpArgs b{x, nullptr, ws1, ws3, 0, act, s.act_stride, s.R, s.d, s.dffs};
    MOE_HIP(moe::launch_gemm_gateup_bf16_with_shared(map, a, b, s.T, stream), "gemm_gateup");
    return MOE_OK;
  }
  SharedOnSide sh;
  moe_status st = sh.fork(s, bm_sh, stream);
  if (st != MOE_OK) return st;
  if (s.nsh) {
    const hipStream_t ss = sh.stream_for_shared(stream);
    moe::GemmTileMap m1{nullptr, 0, s.T};
    moe::GateUpArgs b{x, nullptr, ws1, ws3, 0, act, s.act_stride, s.R, s.d, s.dffs};
    if (s.bf16) MOE_HIP(moe::launch_gemm_gateup_bf16(m1, b, bm_sh, ss), "gemm_gateup_shared");
    else MOE_HIP(moe::launch_gemm_gateup_f32(m1, b, ss), "gemm_gateup_shared");
  }
  if (s.bf16) MOE_HIP(moe::launch_gemm_gateup_bf16(map, a, s.BM, stream), "gemm_gateup");
  else MOE_HIP(moe::launch_gemm_gateup_f32(map, a, stream), "gemm_gateup");
  return sh.join(stream);
}

moe_status do_down(const Shape& s, const void* act, const int32_t* tiles, const void* w2,
                   const void* ws2, float* y_perm, float* sk_part, hipStream_t stream) {
  moe::GemmTileMap map{tiles, s.max_tiles, 0, moe::gemm_n_fast(s.BM, s.R, s.E), avg_group_rows(s)};
  moe::DownArgs a{act, s.act_stride, 0, w2, static_cast<long long>(s.d) * s.dff, y_perm, 0, s.dff, s.d};
  a.sk_part = sk_part;
  a.act_f16 = true;   // the gate/up products wrote the activation as IEEE half
  const int bm_sh = moe::gemm_tile_rows(1, s.T, 1, s.n256);
  if (s.nsh && s.bf16 && s.BM == 16 && bm_sh == 16) {
    moe::DownArgs b{act, s.act_stride, s.R, ws2, 0, y_perm, s.R, s.dffs, s.d};
    b.act_f16 = true;
    MOE_HIP(moe::launch_gemm_down_bf16_with_shared(map, a, b, s.T, stream), "gemm_down");
    return MOE_OK;
  }
  SharedOnSide sh;
  moe_status st = sh.fork(s, bm_sh, stream);
  if (st != MOE_OK) return st;
  if (s.nsh) {
    const hipStream_t ss = sh.stream_for_shared(stream);
    moe::GemmTileMap m1{nullptr, 0, s.T};
    moe::DownArgs b{act, s.act_stride, s.R, ws2, 0, y_perm, s.R, s.dffs, s.d};
    b.act_f16 = true;
    // the stream-K partials are shared scratch: only on the caller's stream
    b.sk_part = sh.side ? nullptr : sk_part;
    if (s.bf16) MOE_HIP(moe::launch_gemm_down_bf16(m1, b, bm_sh, ss), "gemm_down_shared");
    else MOE_HIP(moe::launch_gemm_down_f32(m1, b, ss), "gemm_down_shared");
  }
  if (s.bf16) MOE_HIP(moe::launch_gemm_down_bf16(map, a, s.BM, stream), "gemm_down");
  else MOE_HIP(moe::launch_gemm_down_f32(map, a, stream), "gemm_down");
  st = sh.join(stream);
  if (st != MOE_OK) return st;
  return MOE_OK;
}

}  // namespace

namespace moe {

moe_status report_error(moe_status s, const char* msg) { return fail(s, "%s", msg); }

hipError_t allow_large_lds(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::set<std::tuple<const void*, int, size_t>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kernel, dev, bytes);
  if (done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(bytes));
  if (e == hipSuccess) done.insert(key);
  return e;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_workspace_size(const moe_config* cfg, moe_stage stage, size_t* bytes) {
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (stage < MOE_STAGE_ROUTE || stage > MOE_STAGE_BACKWARD)
    return fail(MOE_ERR_INVALID_ARG, "unknown stage %d", static_cast<int>(stage));
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  *bytes = stage_bytes(s, stage);
  return MOE_OK;
}

int32_t moe_act_stride(const moe_config* cfg) {
  Shape s;
  if (validate(cfg, &s) != MOE_OK) return -1;
  return s.act_stride;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* sel_bias, int32_t* idx, float* gates, const moe_stats* stats,
                     void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(x); REQUIRE(w_router); REQUIRE(idx); REQUIRE(gates);
  st = check_ws(s, MOE_STAGE_ROUTE, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  return do_route(s, cfg->aux_alpha, x, w_router, sel_bias, idx, gates, stats, ws,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_config* cfg, const int32_t* idx, const void* x, int32_t* offsets,
                       int32_t* dest, int32_t* src, void* x_perm, const moe_stats* stats, void* ws,
                       size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(idx); REQUIRE(offsets); REQUIRE(dest); REQUIRE(src);
  if (x_perm != nullptr) { REQUIRE(x); REQUIRE(x_perm); }
  st = check_ws(s, MOE_STAGE_PERMUTE, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  return do_permute(s, idx, x, offsets, dest, src, x_perm, stats, ws, nullptr,
                    static_cast<hipStream_t>(stream));
}

moe_status moe_expert_gateup(const moe_config* cfg, const void* x, const int32_t* src,
                             const int32_t* offsets, const void* w1, const void* w3,
                             const void* ws1, const void* ws3, void* act, void* ws,
                             size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(x); REQUIRE(offsets); REQUIRE(w1); REQUIRE(w3); REQUIRE(act);
  if (s.nsh) {
    REQUIRE(ws1); REQUIRE(ws3);
    if (src == nullptr) return fail(MOE_ERR_INVALID_ARG, "a shared expert needs src (x unpermuted)");
  }
  st = check_ws(s, MOE_STAGE_EXPERT_GATEUP, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  int32_t* tiles = static_cast<int32_t*>(ws);
  MOE_HIP(moe::launch_tile_map(offsets, s.G, s.BM, s.max_tiles, s.ep, tiles, strm), "tile_map");
  return do_gateup(s, x, src, tiles, w1, w3, ws1, ws3, act, strm);
}

moe_status moe_expert_down(const moe_config* cfg, const void* act, const int32_t* offsets,
                           const void* w2, const void* ws2, float* y_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(act); REQUIRE(offsets); REQUIRE(w2); REQUIRE(y_perm);
  if (s.nsh) REQUIRE(ws2);
  st = check_ws(s, MOE_STAGE_EXPERT_DOWN, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  int32_t* tiles = static_cast<int32_t*>(ws);
  float* sk = sk_bytes(s) ? reinterpret_cast<float*>(static_cast<char*>(ws) + tiles_bytes(s)) : nullptr;
  MOE_HIP(moe::launch_tile_map(offsets, s.G, s.BM, s.max_tiles, s.ep, tiles, strm), "tile_map");
  return do_down(s, act, tiles, w2, ws2, y_perm, sk, strm);
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* src,
                          const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                          const void* ws1, const void* ws3, const void* ws2, float* y_perm,
                          void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(x); REQUIRE(offsets); REQUIRE(w1); REQUIRE(w3); REQUIRE(w2); REQUIRE(y_perm);
  if (s.nsh) {
    REQUIRE(ws1); REQUIRE(ws3); REQUIRE(ws2);
    if (src == nullptr) return fail(MOE_ERR_INVALID_ARG, "a shared expert needs src (x unpermuted)");
  }
  st = check_ws(s, MOE_STAGE_EXPERT_FFN, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  Carver cv{static_cast<char*>(ws)};
  void* act = cv.take<char>(static_cast<size_t>(s.rows_total) * s.act_stride * s.elt);
  int32_t* tiles = cv.take<int32_t>(static_cast<size_t>(s.max_tiles) * 16);
  float* sk = sk_bytes(s) ? cv.take<float>(sk_bytes(s)) : nullptr;
  MOE_HIP(moe::launch_tile_map(offsets, s.G, s.BM, s.max_tiles, s.ep, tiles, strm), "tile_map");
  st = do_gateup(s, x, src, tiles, w1, w3, ws1, ws3, act, strm);
  if (st != MOE_OK) return st;
  return do_down(s, act, tiles, w2, ws2, y_perm, sk, strm);
}

moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* dest,
                       const float* gates, float* y, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(y_perm); REQUIRE(dest); REQUIRE(gates); REQUIRE(y);
  st = check_ws(s, MOE_STAGE_COMBINE, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  MOE_HIP(moe::launch_combine(y_perm, dest, gates, s.T, s.k, s.d, s.nsh ? s.R : -1, y,
                              static_cast<hipStream_t>(stream)),
          "combine");
  return MOE_OK;
}

moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const float* sel_bias, const void* w1, const void* w3, const void* w2,
                        const void* ws1, const void* ws3, const void* ws2, const float* dy,
                        float* dx, float* dw_router, float* dw1, float* dw3, float* dw2,
                        float* dws1, float* dws3, float* dws2, void* ws, size_t ws_bytes,
                        void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (!s.bf16) return fail(MOE_ERR_UNSUPPORTED, "the backward runs on bf16 inputs");
  if (s.ep > 1) return fail(MOE_ERR_UNSUPPORTED, "the backward does not take ep_ranks > 1");
  if (s.d % 256 || s.dff % 256 || s.dffs % 256)
    return fail(MOE_ERR_UNSUPPORTED, "the backward needs d, d_ff, d_ff_shared multiples of 256");
  REQUIRE(x); REQUIRE(w_router); REQUIRE(w1); REQUIRE(w3); REQUIRE(w2); REQUIRE(dy);
  REQUIRE(dx); REQUIRE(dw_router); REQUIRE(dw1); REQUIRE(dw3); REQUIRE(dw2);
  if (s.nsh) { REQUIRE(ws1); REQUIRE(ws3); REQUIRE(ws2); REQUIRE(dws1); REQUIRE(dws3); REQUIRE(dws2); }
  if (sel_bias != nullptr && (reinterpret_cast<uintptr_t>(sel_bias) & 3))
    return fail(MOE_ERR_INVALID_ARG, "sel_bias not 4-byte aligned");
  st = check_ws(s, MOE_STAGE_BACKWARD, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  BwdBufs b;
  backward_layout(s, static_cast<char*>(ws), &b);
  const int T = s.T, E = s.E, k = s.k, R = s.R, d = s.d, dff = s.dff, dffs = s.dffs;
  const int As = s.act_stride;
  const int sh_row0 = s.nsh ? R : -1;
  auto u16 = [](const void* p) { return static_cast<const uint16_t*>(p); };

  // ---- forward, recomputed: routing, index, pre-activations, activation
  MOE_HIP(moe::launch_router_scores(1, x, w_router, T, d, E, b.z, b.zpart, strm), "router_scores");
  MOE_HIP(moe::launch_router_select(b.z, sel_bias, T, E, k, s.gate_all, b.idx, b.gates, nullptr,
                                    nullptr, nullptr, nullptr, strm),
          "router_select");
  moe::LoadOut load;
  load.counts = b.counts;
  load.kept = b.kept;
  load.n_dropped = b.ndrop;
  MOE_HIP(moe::launch_index(b.idx, T, k, E, s.C, b.blk, b.slot_base, b.slot_keep, b.offsets, b.dest,
                            b.src, load, s.BM, s.max_tiles, 1, b.tiles, strm),
          "index");
  const moe::GemmTileMap map{b.tiles, s.max_tiles, 0, moe::gemm_n_fast(s.BM, s.R, E),
                            avg_group_rows(s)};
  const moe::GemmTileMap map1{nullptr, 0, T};
  const int bm1 = moe::gemm_tile_rows(1, T, 1, s.n256);
  // the K-major products run 256-row tiles
  moe::GemmTileMap map256 = map;
  if (s.BM != 256) {
    MOE_HIP(moe::launch_tile_map(b.offsets, E, 256, b.max_tiles256, 1, b.tiles256, strm),
            "tile_map 256");
    map256 = moe::GemmTileMap{b.tiles256, b.max_tiles256, 0};
  }
  // h1 = X W1^T, h3 = X W3^T (fp32) and act on the gathered token rows: with 256-row
  // tiles the forward's gate/up kernel stores all three; else two plain products
  // and the activation pass
  auto preact = [&](const moe::GemmTileMap& m, int bm, const void* wa, const void* wb,
                    long long wst, const int32_t* rows, int row0, int nrows, int n) -> moe_status {
    if (bm == 256) {
      moe::GateUpArgs g{x, rows, wa, wb, wst, b.act, As, row0, d, n};
      g.h1 = b.h1;
      g.h3 = b.h3;
      MOE_HIP(moe::launch_gemm_gateup_bf16(m, g, bm, strm), "h1/h3/act");
      return MOE_OK;
    }
    moe::DownArgs a{x, d, 0, wa, wst, b.h1, row0, d, n, rows, As};
    MOE_HIP(moe::launch_gemm_down_bf16(m, a, bm, strm), "h1");
    a.w2 = wb;
    a.y = b.h3;
    MOE_HIP(moe::launch_gemm_down_bf16(m, a, bm, strm), "h3");
    MOE_HIP(moe::launch_swiglu_fwd(b.h1, b.h3, As, row0, nrows, n, b.act, strm), "swiglu_fwd");
    return MOE_OK;
  };
  st = preact(map, s.BM, w1, w3, static_cast<long long>(dff) * d, b.src, 0, R, dff);
  if (st != MOE_OK) return st;
  if (s.nsh) {
    st = preact(map1, bm1, ws1, ws3, 0, nullptr, R, T, dffs);
    if (st != MOE_OK) return st;
  }

  // ---- down: u = dy W2 per row (W2 read K-major), then the SwiGLU backward with
  // the row's gate, which also yields the gates' gradient <dy_t, y_perm[r]> =
  // <act_r, u_r>; then the logits' gradient.
  MOE_HIP(moe::launch_dy_rows(dy, b.dest, b.gates, T, k, d, b.dyb, b.dyp, b.row_gate, strm),
          "dy_rows");
  {
    moe::KmDataArgs a{b.dyb, d, b.src, 0, u16(w2), nullptr, d, dff,
                      static_cast<long long>(d) * dff, b.u, As, 0, d, dff};
    MOE_HIP(moe::launch_gemm_kmajor_data(map256, a, strm), "u");
  }
  MOE_HIP(moe::launch_swiglu_bwd(b.u, b.h1, b.h3, b.act, b.row_gate, As, 0, R, dff, b.dH,
                                 b.dg_row, strm),
          "swiglu_bwd");
  if (s.nsh) {
    {
      moe::KmDataArgs a{b.dyb, d, nullptr, 0, u16(ws2), nullptr, d, dffs, 0, b.u, As, R, d, dffs};
      MOE_HIP(moe::launch_gemm_kmajor_data(map1, a, strm), "u shared");
    }
    MOE_HIP(moe::launch_swiglu_bwd(b.u, b.h1, b.h3, b.act, nullptr, As, R, T, dffs, b.dH, nullptr,
                                   strm),
            "swiglu_bwd shared");
  }
  MOE_HIP(moe::launch_gate_bwd(b.z, b.idx, b.gates, b.dest, b.dg_row, b.counts, T, E, k,
                               s.gate_all, cfg->aux_alpha, b.dz, strm),
          "gate_bwd");
  if (b.rchunks > 0)
    MOE_HIP(moe::launch_dz_split(b.dz, T, E, b.rchunks, b.dzs, b.chunk_off, strm), "dz_split");

  // ---- gate/up: dX_perm = [dh1 dh3] [W1; W3], K = 2 d_ff over W1 then W3 (K-major)
  {
    moe::KmDataArgs a{b.dH, 2 * As, nullptr, 0, u16(w1), u16(w3), dff, d,
                      static_cast<long long>(dff) * d, b.dxp, d, 0, 2 * dff, d};
    if (b.split_dx) a.y2 = b.dxp2;
    MOE_HIP(moe::launch_gemm_kmajor_data(map256, a, strm), "dx_perm");
  }
  if (s.nsh) {
    moe::KmDataArgs a{b.dH, 2 * As, nullptr, R, u16(ws1), u16(ws3), dffs, d, 0, b.dxp, d, R,
                      2 * dffs, d};
    MOE_HIP(moe::launch_gemm_kmajor_data(map1, a, strm), "dx_perm shared");
  }
  // dx = the rows' dX_perm in slot order (+ shared) + dz W_r; a wide router's
  // dz W_r = [hi | lo] [W_r; W_r] is written into dx first and read back there
  if (b.rchunks > 0) {
    moe::KmDataArgs a{b.dzs, 2 * E, nullptr, 0, u16(w_router), u16(w_router), E, d, 0, dx, d, 0,
                      2 * E, d};
    MOE_HIP(moe::launch_gemm_kmajor_data(map1, a, strm), "dz W_r");
  }
  MOE_HIP(moe::launch_unpermute_dx(1, b.dxp, b.split_dx ? b.dxp2 : nullptr, b.dest, b.dz,
                                   b.rchunks > 0 ? nullptr : w_router, T, k, E, d, sh_row0, dx,
                                   strm),
          "unpermute_dx");
  if (b.rchunks > 0) {
    MOE_HIP(moe::launch_gemm_kmajor_groupk(b.chunk_off, b.rchunks, b.dzs, 2 * E, 2 * E, u16(x), d,
                                           d, b.rpart, false, strm),
            "dz^T x");
    MOE_HIP(moe::launch_router_wgrad_pairs(b.rpart, b.rchunks, E, d, dw_router, strm), "dW_r");
  } else {
    MOE_HIP(moe::launch_router_wgrad(1, b.dz, x, T, E, d, b.wpart, dw_router, strm),
            "router_wgrad");
  }

  // ---- weight gradients over each expert's rows: dW2 = dY_perm^T act,
  // dW1 = dH1^T X_perm, dW3 = dH3^T X_perm (both operands K-major)
  MOE_HIP(moe::launch_gather_rows(2, x, b.src, b.offsets, E, R, d, b.xp, strm), "x_perm");
  const bool gk_stream = moe::gemm_n_fast(256, s.R, E);
  MOE_HIP(moe::launch_gemm_kmajor_groupk(b.offsets, E, b.dyp, d, d, b.act, As, dff, dw2, gk_stream,
                                         strm),
          "dW2");
  MOE_HIP(moe::launch_gemm_kmajor_groupk(b.offsets, E, b.dH, 2 * As, dff, b.xp, d, d, dw1, gk_stream,
                                         strm),
          "dW1");
  MOE_HIP(moe::launch_gemm_kmajor_groupk(b.offsets, E, b.dH + dff, 2 * As, dff, b.xp, d, d, dw3,
                                         gk_stream, strm),
          "dW3");
  if (s.nsh) {
    const size_t r0 = static_cast<size_t>(R);
    MOE_HIP(moe::launch_single_group_offsets(T, b.soff, strm), "shared offsets");
    MOE_HIP(moe::launch_gemm_kmajor_groupk(b.soff, 1, b.dyb, d, d, b.act + r0 * As, As, dffs, dws2,
                                           false, strm),
            "dWs2");
    MOE_HIP(moe::launch_gemm_kmajor_groupk(b.soff, 1, b.dH + r0 * 2 * As, 2 * As, dffs, u16(x), d,
                                           d, dws1, false, strm),
            "dWs1");
    MOE_HIP(moe::launch_gemm_kmajor_groupk(b.soff, 1, b.dH + r0 * 2 * As + dffs, 2 * As, dffs,
                                           u16(x), d, d, dws3, false, strm),
            "dWs3");
  }
  return MOE_OK;
}

moe_status moe_ep_traffic(const moe_config* cfg, const int32_t* offsets, int32_t* rows,
                          void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (s.ep <= 1) return fail(MOE_ERR_INVALID_ARG, "ep_ranks must be > 1");
  REQUIRE(offsets); REQUIRE(rows);
  if (s.T == 0) return MOE_OK;   // nothing routed: outputs untouched, as everywhere
  MOE_HIP(moe::launch_ep_traffic(offsets, s.ep, s.E, rows, static_cast<hipStream_t>(stream)),
          "ep_traffic");
  return MOE_OK;
}

moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma, float* bias,
                           void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(counts); REQUIRE(bias);
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite");
  if (s.T == 0) return MOE_OK;   // no load to balance
  MOE_HIP(moe::launch_bias_update(counts, s.T, s.k, s.E, s.ep, gamma, bias,
                                  static_cast<hipStream_t>(stream)),
          "bias_update");
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* sel_bias, const void* w1, const void* w3, const void* w2,
                       const void* ws1, const void* ws3, const void* ws2, float* y,
                       int32_t* idx_out, float* gates_out, const moe_stats* stats, void* ws,
                       size_t ws_bytes, void* stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  REQUIRE(x); REQUIRE(w_router); REQUIRE(w1); REQUIRE(w3); REQUIRE(w2); REQUIRE(y);
  if (s.nsh) { REQUIRE(ws1); REQUIRE(ws3); REQUIRE(ws2); }
  if (idx_out != nullptr) REQUIRE(idx_out);
  if (gates_out != nullptr) REQUIRE(gates_out);
  st = check_ws(s, MOE_STAGE_FORWARD, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  Carver cv{static_cast<char*>(ws)};
  const size_t R4 = static_cast<size_t>(s.R) * 4;
  int32_t* idx = cv.take<int32_t>(R4);
  float* gates = cv.take<float>(R4);
  int32_t* dest = cv.take<int32_t>(R4);
  int32_t* src = cv.take<int32_t>(R4);
  int32_t* offsets = cv.take<int32_t>(static_cast<size_t>(s.G + 1) * 4);
  float* y_perm = cv.take<float>(static_cast<size_t>(s.rows_total) * s.d * 4);
  void* act = cv.take<char>(static_cast<size_t>(s.rows_total) * s.act_stride * s.elt);
  void* scratch = cv.p;   // shared by the stages in turn (stream order)
  if (idx_out) idx = idx_out;
  if (gates_out) gates = gates_out;

  int32_t* tiles = static_cast<int32_t*>(scratch);
  // Decode steps of more than 16 tokens with a shared expert: its gate/up product
  // does not depend on the routing, so it starts on the side stream before the
  // router and runs beside the scores, the selection and the index, and the routed
  // gate/up launch holds the routed items only. Joined before the down launch, which
  // reads both; it writes only the shared rows of act, with the K split of the joint
  // launch (bit for bit the staged result). DeepSeek shape at 64 tokens: 3.29 ->
  // 3.20 ms; at one token the router phase is too short to hide it (+2 %), so up to
  // 16 tokens the shared items stay in the routed launch.
  SharedOnSide early;
  bool shared_done = false;
  if (s.nsh && s.bf16 && s.BM == 16 && s.T > 16 && shared_gateup_rows(s) == 16) {
    st = early.fork_now(strm);
    if (st != MOE_OK) return st;
    if (early.side != nullptr) {
      moe::GemmTileMap m1{nullptr, 0, s.T};
      moe::GateUpArgs b{x, nullptr, ws1, ws3, 0, act, s.act_stride, s.R, s.d, s.dffs};
      // the K split of the joint launch the staged entry point runs (same bits)
      b.stream_ks = moe::stream_gateup_split(s.max_tiles, avg_group_rows(s), s.dff, s.T, s.dffs);
      MOE_HIP(moe::launch_gemm_gateup_bf16(m1, b, 16, early.side->s), "gemm_gateup_shared");
      shared_done = true;
    } else {
      st = early.join(strm);   // no side stream: the joint launch below
      if (st != MOE_OK) return st;
    }
  }
  if (s.ep == 1 && !want_route_stats(stats) && moe::route_index_single_ok(s.T, s.E, s.k, s.C >= 0)) {
    // small batch, no routing statistics: selection and index in one launch after
    // the scores. The tile table is written over the logits at the start of the
    // scratch, after the kernel's barrier, when every logit has been read.
    Carver rc{static_cast<char*>(scratch)};
    float* z = rc.take<float>(static_cast<size_t>(s.T) * s.E * 4);
    rc.take<float>(static_cast<size_t>(s.nb_sel) * s.E * 4);              // p_part
    rc.take<int32_t>(static_cast<size_t>(s.nb_sel) * s.E * 4);            // c_part
    rc.take<float>(static_cast<size_t>(s.E) * 4);                         // fp
    rc.take<float>(static_cast<size_t>(s.nb_sel) * moe::kScaleStats * 4); // q_part
    float* zpart = rc.take<float>(zpart_bytes(s));
    // a small router's scores in the same launch (Mixtral shape, one token)
    const bool scores_here = moe::route_scores_in_index_ok(s.bf16, s.T, s.d, s.E);
    if (!scores_here)
      MOE_HIP(moe::launch_router_scores(s.bf16, x, w_router, s.T, s.d, s.E, z, zpart, strm),
              "router_scores");
    MOE_HIP(moe::launch_route_index_single(
                z, sel_bias, s.T, s.k, s.E, s.gate_all, idx, gates, s.C, offsets, dest, src,
                load_out(stats), s.BM, s.max_tiles, tiles, strm, scores_here ? x : nullptr,
                scores_here ? w_router : nullptr, s.d),
            "route_index");
  } else {
    st = do_route(s, cfg->aux_alpha, x, w_router, sel_bias, idx, gates, stats, scratch, strm);
    if (st != MOE_OK) return st;
    st = do_permute(s, idx, x, offsets, dest, src, nullptr, stats,
                    static_cast<char*>(scratch) + tiles_bytes(s), tiles, strm);
    if (st != MOE_OK) return st;
  }
  st = do_gateup(s, x, src, tiles, w1, w3, ws1, ws3, act, strm, shared_done);
  if (st != MOE_OK) return st;
  if (shared_done) {
    st = early.join(strm);
    if (st != MOE_OK) return st;
  }
  if (!s.nsh && s.bf16 && s.BM == 16 && s.ep == 1) {
    // one or two tokens of a layer with few experts per token: the down product
    // and the combine in one launch (the same y bit for bit, no y_perm round trip)
    moe::GemmTileMap map{tiles, s.max_tiles, 0, false, avg_group_rows(s)};
    moe::DownArgs a{act, s.act_stride, 0, w2, static_cast<long long>(s.d) * s.dff, y_perm, 0,
                    s.dff, s.d};
    a.act_f16 = true;
    const hipError_t e = moe::launch_gemm_down_combine_bf16(map, a, dest, gates, s.T, s.k, y, strm);
    if (e == hipSuccess) return MOE_OK;
    if (e != hipErrorNotSupported) return hip_fail(e, "gemm_down_combine");
  }
  float* sk = sk_bytes(s) ? reinterpret_cast<float*>(static_cast<char*>(scratch) + tiles_bytes(s))
                         : nullptr;
  st = do_down(s, act, tiles, w2, ws2, y_perm, sk, strm);
  if (st != MOE_OK) return st;
  MOE_HIP(moe::launch_combine(y_perm, dest, gates, s.T, s.k, s.d, s.nsh ? s.R : -1, y, strm),
          "combine");
  return MOE_OK;
}

}  // extern "C"
