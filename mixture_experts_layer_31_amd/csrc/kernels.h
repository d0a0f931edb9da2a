// Internal launchers of the MoE kernels. Every launcher enqueues on `s` and
// returns hipGetLastError() of its launch(es); shapes are validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Raise a kernel's dynamic-LDS limit above 64 KiB, once per (kernel, device):
// setting the attribute before every launch measurably slows the launches.
hipError_t allow_large_lds(const void* kernel, size_t bytes);

// ---- backward (backward.hip)
hipError_t launch_single_group_offsets(int rows, int32_t* off, hipStream_t s);
// Router gradients as MFMA products (E a multiple of 128): dz split into bf16
// halves dzs [T][2E] (hi | lo) and the C + 1 token-chunk offsets c T / C; then,
// after the grouped-K product part [C][2E][d] = per chunk [hi | lo]^T x, dW_r as
// the chunk-ordered sum of its hi and lo rows.
constexpr int kRouterMfmaExperts = 128;
inline bool router_grad_mfma(int E) { return E >= kRouterMfmaExperts && E % kRouterMfmaExperts == 0; }
hipError_t launch_dz_split(const float* dz, int T, int E, int C, uint16_t* dzs, int32_t* chunk_off,
                           hipStream_t s);
hipError_t launch_router_wgrad_pairs(const float* part, int C, int E, int d, float* dwr,
                                     hipStream_t s);
hipError_t launch_swiglu_fwd(const float* h1, const float* h3, int stride, int row0, int rows,
                             int n, uint16_t* act, hipStream_t s);
hipError_t launch_swiglu_bwd(const float* u, const float* h1, const float* h3,
                             const uint16_t* act, const float* row_gate, int stride, int row0,
                             int rows, int n, uint16_t* dH, float* dg_row, hipStream_t s);
hipError_t launch_dy_rows(const float* dy, const int32_t* dest, const float* gates, int T, int k,
                          int d, uint16_t* dyb, uint16_t* dyp, float* row_gate, hipStream_t s);
hipError_t launch_gate_bwd(const float* z, const int32_t* idx, const float* gates,
                           const int32_t* dest, const float* dg_row, const int32_t* counts, int T,
                           int E, int k, int gate_all, float alpha, float* dz, hipStream_t s);
hipError_t launch_unpermute_dx(int dtype_bf16, const float* dxp, const float* dxp2,
                               const int32_t* dest, const float* dz, const void* wr, int T, int k,
                               int E, int d, int shared_row0, float* dx, hipStream_t s);
// dW_r = dz^T x in token chunks (part: chunks * E * d floats of scratch), then the
// chunks summed in order.
struct RouterWgradPlan {
  int eb = 8, tc = 16, chunks = 0;
};
RouterWgradPlan router_wgrad_plan(int T, int E, int d);
hipError_t launch_router_wgrad(int dtype_bf16, const float* dz, const void* x, int T, int E, int d,
                               float* part, float* dwr, hipStream_t s);

// ---- router (router.hip)
constexpr int kSelectMaxBlocks = 1024;
int router_select_tokens(int T);   // tokens per router_select workgroup
int router_select_blocks(int T);
// bf16 scores: the vector-unit kernel for a few tokens (gemv), the one-block
// MFMA kernel for up to 16 experts (narrow), else the tiled MFMA kernel's tile
// shape (32 wt tokens x 32 we experts), expert tiles and K-splits; groups =
// workgroups launched
struct RouterScorePlan {
  bool gemv = false, narrow = false;
  int wt = 2, we = 2, n_et = 0, S = 1;
  long long groups = 0;
};
RouterScorePlan router_score_plan(int T, int d, int E);
// floats of scratch the scores need for split-K partial sums (0: none)
size_t router_scores_part_floats(int dtype_bf16, int T, int d, int E);
// part: router_scores_part_floats(...) floats (may be null when that is 0)
hipError_t launch_router_scores(int dtype_bf16, const void* x, const void* w, int T, int d, int E,
                                float* z, float* part, hipStream_t s);
// q_part (nullable): per-block sums of the four scale statistics (z-loss,
// entropy, top probability, top-2 gap), [blocks][kScaleStats]; margin
// (nullable): s_(k) - s_(k+1) per token, [T]
constexpr int kScaleStats = 4;
hipError_t launch_router_select(const float* z, const float* bias, int T, int E, int k,
                                int gate_all, int32_t* idx, float* gates, float* p_part,
                                int32_t* c_part, float* q_part, float* margin, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, int T, int k, int E, int ep, float gamma,
                              float* bias, hipStream_t s);
hipError_t launch_router_stats(const float* p_part, const int32_t* c_part, const float* q_part,
                               int nblocks, int T, int E, float alpha, float* f, float* P,
                               float* aux, float* fp, float* z_loss, float* entropy,
                               float* max_prob, float* top_gap, hipStream_t s);

// ---- index: histogram, scan, rank (index.hip)
constexpr int kIndexTokensPerBlock = 256;
int index_blocks(int T);
// number of histogram keys: E without capacity, k*E with capacity
inline int index_keys(int E, int k, bool cap) { return cap ? E * k : E; }
constexpr int kIndexMaxKeys = 4096;   // LDS bitmaps: 32 bytes per key
// Single-workgroup index (one launch) when T <= 256 and the keys fit in LDS.
constexpr int kIndexSingleMaxKeys = 1024;
bool index_single_ok(int T, int E, int k, bool cap);
// With `tiles` set, also writes the grouped GEMM tile table for BM-row tiles
// (as launch_tile_map does), in the same launch on the single-workgroup path.
// Selection and index of a small batch in one single-workgroup launch (the
// fused forward's decode steps; no routing statistics, no expert-parallel
// layout): idx and gates as launch_router_select writes them, then what
// launch_index writes, with the tile table.
constexpr int kRouteIndexMaxTokens = 64;
bool route_index_single_ok(int T, int E, int k, bool cap);
// Load statistics the index writes where a pointer is set (each nullable):
// per key the assignments before drops (counts) and after capacity (kept), the
// dropped total, the number of experts that keep at least one assignment
// (touched) and the largest expert load over the mean T*k/E (max_over_mean).
struct LoadOut {
  int32_t* counts = nullptr;
  int32_t* kept = nullptr;
  int32_t* n_dropped = nullptr;
  int32_t* touched = nullptr;
  float* max_over_mean = nullptr;
};
// With x set (bf16 [T][d], and w_router [E][d]) the logits are computed in the
// same launch, bit for bit as launch_router_scores computes them, where
// route_scores_in_index_ok holds (a small router: T * E <= kRouteScoresMaxPairs,
// the scores' single-token vector plan); z is then unused.
constexpr int kRouteScoresMaxPairs = 8;
bool route_scores_in_index_ok(int dtype_bf16, int T, int d, int E);
hipError_t launch_route_index_single(const float* z, const float* bias, int T, int k, int E,
                                     int gate_all, int32_t* idx, float* gates,
                                     long long capacity, int32_t* offsets, int32_t* dest,
                                     int32_t* src, const LoadOut& load, int BM, int max_tiles,
                                     int32_t* tiles, hipStream_t s, const void* x = nullptr,
                                     const void* w_router = nullptr, int d = 0);
hipError_t launch_index(const int32_t* idx, int T, int k, int E, long long capacity,
                        int32_t* blk, int32_t* slot_base, int32_t* slot_keep, int32_t* offsets,
                        int32_t* dest, int32_t* src, const LoadOut& load, int BM, int max_tiles,
                        int ep, int32_t* tiles, hipStream_t s);
// Simulated expert parallelism (ep > 1 ranks): row-group ids and send-row matrix.
hipError_t launch_ep_group_ids(const int32_t* idx, int T, int k, int E, int n, int32_t* gid,
                               hipStream_t s);
hipError_t launch_ep_traffic(const int32_t* offsets, int n, int E, int32_t* rows, hipStream_t s);
// Tile table entries are int4 (weights group, first row, rows, order block). The
// fourth field packs the tile's block of the blocked launch order (first tile of
// the block << 8 | tiles in it): a group of nt tiles forms ceil(nt / 8) blocks of
// ceil(nt / blocks) consecutive tiles (the last one shorter), so a group of up to
// eight tiles is one block and is walked as a whole.
constexpr int kTileOrderBlock = 8;
__host__ __device__ inline int tile_block_word(int start, int nt, int i) {
  const int nb = (nt + kTileOrderBlock - 1) / kTileOrderBlock;
  const int c = (nt + nb - 1) / nb;
  const int lo = (i / c) * c;
  return ((start + lo) << 8) | (nt - lo < c ? nt - lo : c);
}

// Weights index of row group g of G groups: g itself, or with ep > 1 ranks the
// expert of group (r*ep + s)*El + l, namely r*El + l with El = G / ep^2.
__host__ __device__ inline int tile_group_weights(int g, int G, int ep) {
  if (ep <= 1) return g;
  const int El = G / (ep * ep);
  return (g / (ep * El)) * El + g % El;
}

// ---- row movement (rows.hip)
hipError_t launch_gather_rows(int elt_bytes, const void* x, const int32_t* src,
                              const int32_t* offsets, int E, int R_max, int d, void* x_perm,
                              hipStream_t s);
hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* gates, int T,
                          int k, int d, int shared_row0 /* -1: none */, float* y,
                          hipStream_t s);

// ---- grouped GEMMs (gemm_bf16.hip, gemm_f32.hip)
//
// Tile table entry: {group, first row, rows, 0}. An entry with rows == 0 ends
// the work of its workgroup.
struct GemmTileMap {
  const int32_t* tiles;   // [max_tiles][4], or nullptr for one group of n_single rows
  int max_tiles;
  int n_single;
  bool n_fast = false;    // 256-row tiles: run the n tiles of each m tile together
  int avg_rows = 0;       // rows per non-empty group on average (decode kernels; 0: unknown)
};

// Tile order of the 256-row kernels for R_max rows over `experts` weight
// matrices: n tiles fastest (gemm_bf16.hip, xcd_tile_nfast) when there are many
// experts of at most one tile each on average, which makes those products
// weight-streaming. It counts experts, not row groups: groups that share an
// expert's weights (the expert-parallel layout) want the m-fastest order, which
// runs them side by side on one weight panel.
bool gemm_n_fast(int BM, long long R_max, int experts);

// BM of the grouped GEMMs for R_max rows in `groups` groups; n256_ok: d is a
// multiple of 256 and d_ff (and d_ff_shared) of 128, as the large tiles need
int gemm_tile_rows(int dtype_bf16, int R_max, int groups, bool n256_ok);
int gemm_max_tiles(int BM, int R_max, int E);
hipError_t launch_tile_map(const int32_t* offsets, int E, int BM, int max_tiles, int ep,
                           int32_t* tiles, hipStream_t s);

struct GateUpArgs {
  const void* x;          // activation rows source
  const int32_t* src;     // row -> x row (nullable: identity)
  const void* w1;         // [G][N][K]
  const void* w3;
  long long w_stride;     // elements between groups' weight matrices
  void* act;              // [rows][act_stride]: IEEE half, or bf16 when h1 is set
  int act_stride;
  int out_row0;           // output row = out_row0 + grouped row
  int K, N;               // K = d, N = d_ff
  float* h1 = nullptr;    // optional fp32 pre-activations X W1^T, X W3^T at the
  float* h3 = nullptr;    // activation's rows and stride (256-row tiles only)
  int stream_ks = 0;      // 16-row streaming tiles: the K split to use (0: the
                          // launch's own rule; stream_gateup_split() gives another's)
};
// The K split that a 16-row streaming launch of a tile table (max_tiles tiles,
// avg_rows rows per group, N columns) plus a dense segment of seg_rows rows and
// seg_N columns chooses: a product run on its own gets this value in
// GateUpArgs::stream_ks to compute bit for bit as it would in that joint launch.
int stream_gateup_split(int max_tiles, int avg_rows, int N, int seg_rows, int seg_N);
struct DownArgs {
  const void* act;        // [rows][act_stride]
  int act_stride;
  int in_row0;            // input row = in_row0 + grouped row (after src, if set)
  const void* w2;         // [G][N][K]
  long long w_stride;
  float* y;               // [rows][N]
  int out_row0;
  int K, N;               // K = d_ff, N = d
  const int32_t* src = nullptr;   // grouped row -> input row (nullable: identity)
  int out_stride = 0;             // y row stride in floats (0: N)
  float* sk_part = nullptr;       // stream-K partial tiles (streamk_part_bytes), nullable
  bool act_f16 = false;           // act rows are IEEE half (the forward's SwiGLU
                                  // activation): the bf16 weights are widened to half
                                  // and the product runs on half MFMAs
};
// Workgroups of a persistent launch: one per CU (a multiple of 8), at most cap; 0 if
// the CU count is unavailable.
int persistent_workgroups(int cap);
// Stream-K down products: at most this many workgroups, each with one partial
// 256 x 256 fp32 tile of scratch.
constexpr int kStreamKMaxWorkgroups = 256;
constexpr size_t kStreamKPartBytes = static_cast<size_t>(kStreamKMaxWorkgroups) * 256 * 256 * 4;
// K-major grouped GEMMs (gemm_kmajor.hip), 256 x 256 tiles.
// Data mode: y[y_row0 + row][n] = sum_k x[x_row0 + row(r)][k] * W_g[k][n] for the
// rows of a 256-row tile table (row(r) = src[r] when src is set), with
// W_g[k] = wa + g w_stride + k ldw for k < ksplit, wb + g w_stride + (k - ksplit) ldw
// after; K and ksplit multiples of 32, N of 256. With y2 set (0 < ksplit < K)
// the sum is split at ksplit: y gets the k < ksplit part, y2 (same stride and
// rows) the rest, each from its own half of a doubled grid.
struct KmDataArgs {
  const uint16_t* x;
  int lda;
  const int32_t* src;   // nullable
  int x_row0;
  const uint16_t* wa;
  const uint16_t* wb;   // used for k >= ksplit
  int ksplit, ldw;
  long long w_stride;
  float* y;
  int y_stride, y_row0;
  int K, N;
  float* y2 = nullptr;
};
hipError_t launch_gemm_kmajor_data(const GemmTileMap& map, const KmDataArgs& a, hipStream_t s);
// Grouped K: out[g][m][n] = sum over rows r in [offsets[g], offsets[g+1]) of
// A[r][m] * B[r][n] (fp32 out, [G][N1][N2]); A [rows][lda], B [rows][ldb] bf16,
// N1 and N2 multiples of 256.
// rows_stream: the groups are short (gemm_n_fast), so the products are bound by
// writing the fp32 output: tiles go out n-fastest with plain stores.
hipError_t launch_gemm_kmajor_groupk(const int32_t* offsets, int G, const uint16_t* A, int lda,
                                     int N1, const uint16_t* B, int ldb, int N2, float* out,
                                     bool rows_stream, hipStream_t s);
hipError_t launch_gemm_gateup_bf16(const GemmTileMap& map, const GateUpArgs& a, int BM,
                                   hipStream_t s);
hipError_t launch_gemm_down_bf16(const GemmTileMap& map, const DownArgs& a, int BM,
                                 hipStream_t s);
// Decode-sized steps: the grouped rows (16-row tiles, streaming kernel) and one
// dense group of sh_rows rows with its own weights (sh: the shared expert; no
// src, same activation / output buffers and strides) in one launch.
hipError_t launch_gemm_gateup_bf16_with_shared(const GemmTileMap& map, const GateUpArgs& a,
                                               const GateUpArgs& sh, int sh_rows, hipStream_t s);
hipError_t launch_gemm_down_bf16_with_shared(const GemmTileMap& map, const DownArgs& a,
                                             const DownArgs& sh, int sh_rows, hipStream_t s);
// Decode steps of at most 16 tokens whose tile bound times the streaming K split
// fits one workgroup: the down product and the gate-weighted combine in one launch,
// y written directly (bit for bit the streaming down product then combine); y_perm
// is not written. hipErrorNotSupported (nothing launched) where it does not apply.
hipError_t launch_gemm_down_combine_bf16(const GemmTileMap& map, const DownArgs& a,
                                         const int32_t* dest, const float* gates, int T, int k,
                                         float* y, hipStream_t s);
hipError_t launch_gemm_gateup_f32(const GemmTileMap& map, const GateUpArgs& a, hipStream_t s);
hipError_t launch_gemm_down_f32(const GemmTileMap& map, const DownArgs& a, hipStream_t s);

}  // namespace moe
