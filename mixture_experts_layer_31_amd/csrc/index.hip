// Per-expert histogram, capacity and the token permutation.
//
// The CMU 15-779 Lecture 21 notes, §3.3: the destination row of every
// (token, expert) assignment is the prefix sum of the transposed 0/1 selection
// mask taken expert-major, so rows are grouped by expert, tokens in order inside
// a group, and the group boundaries (CSR indptr) come out of the same scan.
// §3.5: with a capacity C an expert keeps at most C assignments, every first
// choice before any second choice, tokens in order; the rest are dropped.
//
// GPU formulation. Tokens are cut into blocks of 256. Each block builds, in LDS,
// one 256-bit token bitmap per key (key = expert, or (slot, expert) with
// capacity) with LDS atomics; counts are popcounts. A single-workgroup scan
// turns the per-block counts into per-block bases (exclusive prefix over
// blocks, in block order) and the expert offsets. The rank of a token among the
// earlier tokens of its key is then base + popcount of the bitmap bits below it.
// Atomics only ever set bits, so every output is deterministic and equal to the
// sequential definition.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {

constexpr int kTB = kIndexTokensPerBlock;   // tokens per block = threads per block
constexpr int kWords = kTB / 32;            // 32-bit bitmap words per key

int index_blocks(int T) { return (T + kTB - 1) / kTB; }

__device__ __forceinline__ void build_bitmaps(uint32_t* bm, const int32_t* idx, int T, int k,
                                              int E, int nkeys, bool cap) {
  for (int i = threadIdx.x; i < nkeys * kWords; i += kTB) bm[i] = 0u;
  __syncthreads();
  const int t = blockIdx.x * kTB + threadIdx.x;
  if (t < T) {
    const uint32_t bit = 1u << (threadIdx.x & 31);
    const int w = threadIdx.x >> 5;
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) continue;  // not an expert
      const int key = cap ? j * E + e : e;
      atomicOr(&bm[key * kWords + w], bit);
    }
  }
  __syncthreads();
}

// number of set bits of key's bitmap strictly below local token position p
__device__ __forceinline__ int bits_below(const uint32_t* bm, int key, int p, int stride = kWords) {
  const uint32_t* b = bm + key * stride;
  int r = 0;
  const int w = p >> 5;
  for (int i = 0; i < w; ++i) r += __popc(b[i]);
  return r + __popc(b[w] & ((1u << (p & 31)) - 1u));
}

// Expert load summary, called by every thread of a 1024-thread workgroup once the
// per-key totals are final. With ep == 1 thread e holds expert e's assignments
// before drops (cnt) and after capacity (keep). With ep = n > 1 the G keys are
// the groups of the expert-parallel layout, with no capacity (kept = counts),
// and expert e of the E = G / n sums its n groups (r*n + s)*(E/n) + l, r = e div
// (E/n), l = e mod (E/n), over the source ranks s, read from tot. touched counts
// the experts with a kept assignment; max_over_mean is max_e load_e * E / (T*k),
// the quotient taken in double and rounded once to float.
__device__ __forceinline__ void load_summary(int cnt, int keep, const int32_t* tot, int G, int ep,
                                             int T, int k, const LoadOut& o, int* part) {
  if (o.touched == nullptr && o.max_over_mean == nullptr) return;   // uniform
  const int e = threadIdx.x;
  const int E = G / ep;
  int load = 0, used = 0;
  if (ep > 1) {
    if (e < E) {
      const int per = E / ep, r = e / per, l = e - r * per;
      for (int src_rank = 0; src_rank < ep; ++src_rank) load += tot[(r * ep + src_rank) * per + l];
      used = load > 0;
    }
  } else if (e < G) {
    load = cnt;
    used = keep > 0;
  }
  int n_used = 0;
  block_scan_1024(used, part, &n_used);
  const int mx = block_max_1024(load, part);
  if (threadIdx.x == 0) {
    if (o.touched) o.touched[0] = n_used;
    if (o.max_over_mean)
      o.max_over_mean[0] = static_cast<float>(static_cast<double>(mx) * E /
                                              (static_cast<double>(T) * k));
  }
}

__global__ __launch_bounds__(kTB) void index_count_kernel(const int32_t* __restrict__ idx, int T,
                                                          int k, int E, int cap,
                                                          int32_t* __restrict__ blk) {
  extern __shared__ uint32_t bm[];
  const int nkeys = cap ? E * k : E;
  build_bitmaps(bm, idx, T, k, E, nkeys, cap);
  for (int key = threadIdx.x; key < nkeys; key += kTB) {
    int c = 0;
    for (int w = 0; w < kWords; ++w) c += __popc(bm[key * kWords + w]);
    blk[static_cast<size_t>(blockIdx.x) * nkeys + key] = c;
  }
}

// One workgroup. blk[b][key] (counts) becomes the exclusive prefix over blocks.
// With a tile table (tiles != nullptr) it also writes the GEMM tiles of BM rows
// from the kept counts, as tile_map_kernel does from the offsets (one launch less).
__global__ __launch_bounds__(1024) void index_scan_kernel(
    int32_t* __restrict__ blk, int nb, int T, int k, int E, long long C,
    int32_t* __restrict__ slot_base, int32_t* __restrict__ slot_keep,
    int32_t* __restrict__ offsets, LoadOut o, int ep, int BM, int max_tiles,
    int4* __restrict__ tiles) {
  __shared__ int32_t part[16];
  const int cap = C >= 0;
  const int nkeys = cap ? E * k : E;
  int32_t* tot = blk + static_cast<size_t>(nb) * nkeys;   // row nb holds the key totals
  // per key, the blocks in chunks of 16: the chunk's loads go out together, then
  // the running sum (one load latency per chunk, not per block: 64 blocks took
  // 12 us one by one)
  constexpr int kChunk = 16;
  for (int key = threadIdx.x; key < nkeys; key += blockDim.x) {
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += kChunk) {
      int c[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        c[i] = b0 + i < nb ? blk[static_cast<size_t>(b0 + i) * nkeys + key] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (b0 + i < nb) blk[static_cast<size_t>(b0 + i) * nkeys + key] = run;
        run += c[i];
      }
    }
    tot[key] = run;
  }
  __threadfence_block();
  __syncthreads();
  // per expert: count before drops and kept after capacity
  const int e = threadIdx.x;
  int keep_e = 0, cnt = 0;
  if (e < E) {
    if (cap) {
      // all j-th choices are served before any (j+1)-th choice
      for (int j = 0; j < k; ++j) {
        const int tj = tot[j * E + e];
        long long room = C - cnt;
        room = room < 0 ? 0 : room;
        const int keep_j = static_cast<int>(room < tj ? room : tj);
        slot_base[j * E + e] = cnt;
        slot_keep[j * E + e] = keep_j;
        keep_e += keep_j;
        cnt += tj;
      }
    } else {
      cnt = tot[e];
      keep_e = cnt;
    }
    if (o.counts) o.counts[e] = cnt;
    if (o.kept) o.kept[e] = keep_e;
  }
  // scan of kept over experts (E <= 1024 = blockDim.x)
  int kept_total = 0;
  const int incl = block_scan_1024((e < E) ? keep_e : 0, part, &kept_total);
  if (e < E) offsets[e + 1] = incl;
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    if (o.n_dropped) o.n_dropped[0] = T * k - kept_total;
  }
  if (tiles != nullptr) {
    const int nt = (e < E) ? (keep_e + BM - 1) / BM : 0;
    int tiles_total = 0;
    const int start = block_scan_1024(nt, part, &tiles_total) - nt;
    const int lo = incl - keep_e;
    const int w = tile_group_weights(e, E, ep);
    for (int i = 0; i < nt && start + i < max_tiles; ++i)
      tiles[start + i] =
          make_int4(w, lo + i * BM, min(BM, keep_e - i * BM), tile_block_word(start, nt, i));
    for (int i = tiles_total + threadIdx.x; i < max_tiles; i += 1024) tiles[i] = make_int4(0, 0, 0, 0);
  }
  load_summary(cnt, keep_e, tot, E, ep, T, k, o, part);
}

__global__ __launch_bounds__(kTB) void index_rank_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, long long C,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ slot_base,
    const int32_t* __restrict__ slot_keep, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  extern __shared__ uint32_t bm[];
  const int cap = C >= 0;
  const int nkeys = cap ? E * k : E;
  build_bitmaps(bm, idx, T, k, E, nkeys, cap);
  const int t = blockIdx.x * kTB + threadIdx.x;
  if (t >= T) return;
  const int p = threadIdx.x;
  const int32_t* base = blk + static_cast<size_t>(blockIdx.x) * nkeys;
  for (int j = 0; j < k; ++j) {
    const int e = idx[static_cast<size_t>(t) * k + j];
    int row;
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {
      row = -1;   // an out-of-range index is never given a row
    } else if (!cap) {
      row = offsets[e] + base[e] + bits_below(bm, e, p);
    } else {
      const int key = j * E + e;
      const int rank_j = base[key] + bits_below(bm, key, p);
      if (static_cast<long long>(slot_base[key]) + rank_j >= C) {
        row = -1;
      } else {
        // kept rows of e held by earlier tokens: in each slot j', the kept ones
        // are the first slot_keep[j'][e] tokens of that slot (token order)
        int before = 0;
        for (int j2 = 0; j2 < k; ++j2) {
          const int key2 = j2 * E + e;
          const int r2 = base[key2] + bits_below(bm, key2, p);
          const int kk = slot_keep[key2];
          before += r2 < kk ? r2 : kk;
        }
        row = offsets[e] + before;
      }
    }
    dest[static_cast<size_t>(t) * k + j] = row;
    if (row >= 0) src[row] = t;
  }
}

// ---------------------------------------------------------------- expert parallelism
//
// Simulated expert parallelism over n ranks (CMU 15-779 notes §5.1): rank r
// holds experts [r*E/n, (r+1)*E/n) and tokens [r*T/n, (r+1)*T/n). Assignment
// (t, e) goes from source rank s = t / (T/n) to destination rank
// r = e / (E/n); its row group is (r*n + s)*(E/n) + e % (E/n), so the index
// over these n*E groups lays each rank's send and receive rows out
// contiguously. An out-of-range expert id stays out of range.
__global__ __launch_bounds__(256) void ep_group_ids_kernel(const int32_t* __restrict__ idx,
                                                           int T, int k, int E, int n,
                                                           int32_t* __restrict__ gid) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(T) * k) return;
  const int e = idx[i];
  const int t = static_cast<int>(i / k);
  const int El = E / n, Tl = T / n;
  gid[i] = static_cast<unsigned>(e) < static_cast<unsigned>(E)
               ? ((e / El) * n + t / Tl) * El + e % El
               : -1;
}

hipError_t launch_ep_group_ids(const int32_t* idx, int T, int k, int E, int n, int32_t* gid,
                               hipStream_t s) {
  const long long R = static_cast<long long>(T) * k;
  if (R == 0) return hipSuccess;
  ep_group_ids_kernel<<<dim3((R + 255) / 256), dim3(256), 0, s>>>(idx, T, k, E, n, gid);
  return hipGetLastError();
}

// rows[s*n + r] = rows of the groups (r, s, *): offsets over n*E groups
__global__ __launch_bounds__(256) void ep_traffic_kernel(const int32_t* __restrict__ offsets,
                                                         int n, int El,
                                                         int32_t* __restrict__ rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n * n) return;
  const int src = i / n, dst = i % n;
  const int g0 = (dst * n + src) * El;
  rows[i] = offsets[g0 + El] - offsets[g0];
}

hipError_t launch_ep_traffic(const int32_t* offsets, int n, int E, int32_t* rows, hipStream_t s) {
  ep_traffic_kernel<<<dim3((n * n + 255) / 256), dim3(256), 0, s>>>(offsets, n, E / n, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------- one workgroup
//
// T <= 256 tokens and at most kIndexSingleMaxKeys keys (decode and small
// batches): the three steps above in one 1024-thread workgroup with every
// intermediate in LDS, so a decode step pays one launch instead of three. The
// arithmetic and its order are those of the three kernels with one token block
// (every per-block base is 0). When `tiles` is set it also writes the grouped
// GEMM tile table of BM-row tiles (group, first row, rows) from the offsets, as
// tile_map_kernel does, and zero entries up to max_tiles.
// The workgroup's body; idx may point to global memory or to LDS.
__device__ __forceinline__ void index_single_body(
    const int32_t* __restrict__ idx, int T, int k, int E, long long C,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src,
    const LoadOut& o, int BM, int max_tiles, int ep, int4* __restrict__ tiles, uint32_t* smem) {
  const int cap = C >= 0;
  const int nkeys = cap ? E * k : E;
  const int nw = (T + 31) >> 5;                                     // bitmap words per key
  uint32_t* bm = smem;                                              // [nkeys][nw]
  int32_t* tot = reinterpret_cast<int32_t*>(bm + nkeys * kWords);   // [nkeys]
  int32_t* sbase = tot + nkeys;                                     // [nkeys]
  int32_t* skeep = sbase + nkeys;                                   // [nkeys]
  int32_t* off = skeep + nkeys;                                     // [E + 1]
  int32_t* part = off + (E + 1);                                    // [16]
  const int tid = threadIdx.x;

  for (int i = tid; i < nkeys * nw; i += 1024) bm[i] = 0u;
  __syncthreads();
  if (tid < T) {
    const uint32_t bit = 1u << (tid & 31);
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(tid) * k + j];
      if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) continue;
      atomicOr(&bm[(cap ? j * E + e : e) * nw + (tid >> 5)], bit);
    }
  }
  __syncthreads();
  for (int key = tid; key < nkeys; key += 1024) {
    int c = 0;
    for (int w = 0; w < nw; ++w) c += __popc(bm[key * nw + w]);
    tot[key] = c;
  }
  __syncthreads();
  const int e = tid;
  int keep_e = 0, cnt = 0;
  if (e < E) {
    if (cap) {
      for (int j = 0; j < k; ++j) {
        const int tj = tot[j * E + e];
        long long room = C - cnt;
        room = room < 0 ? 0 : room;
        const int keep_j = static_cast<int>(room < tj ? room : tj);
        sbase[j * E + e] = cnt;
        skeep[j * E + e] = keep_j;
        keep_e += keep_j;
        cnt += tj;
      }
    } else {
      cnt = tot[e];
      keep_e = cnt;
    }
    if (o.counts) o.counts[e] = cnt;
    if (o.kept) o.kept[e] = keep_e;
  }
  // offsets: inclusive scan of the kept counts; tile table: exclusive scan of
  // ceil(kept / BM). Both in one scan of (kept | tiles << 16) while every partial
  // sum fits in 15 bits (tiles <= kept <= T k), else in two.
  const int keep_v = (e < E) ? keep_e : 0;
  const int nt = (tiles != nullptr && e < E) ? (keep_e + BM - 1) / BM : 0;
  int kept_total = 0, incl, tiles_total = 0, tiles_incl = 0;
  if (T * k < 32768) {
    int tot2 = 0;
    const int v2 = block_scan_1024(keep_v | (nt << 16), part, &tot2);
    incl = v2 & 0xFFFF;
    kept_total = tot2 & 0xFFFF;
    tiles_incl = v2 >> 16;
    tiles_total = tot2 >> 16;
  } else {
    incl = block_scan_1024(keep_v, part, &kept_total);
    if (tiles != nullptr) tiles_incl = block_scan_1024(nt, part, &tiles_total);
  }
  if (e < E) { off[e + 1] = incl; offsets[e + 1] = incl; }
  if (tid == 0) {
    off[0] = 0;
    offsets[0] = 0;
    if (o.n_dropped) o.n_dropped[0] = T * k - kept_total;
  }
  if (tiles != nullptr) {
    const int start = tiles_incl - nt, lo = incl - keep_v;
    const int w = tile_group_weights(e, E, ep);
    for (int i = 0; i < nt && start + i < max_tiles; ++i)
      tiles[start + i] =
          make_int4(w, lo + i * BM, min(BM, keep_v - i * BM), tile_block_word(start, nt, i));
    for (int i = tiles_total + tid; i < max_tiles; i += 1024) tiles[i] = make_int4(0, 0, 0, 0);
  }
  load_summary(cnt, keep_e, tot, E, ep, T, k, o, part);
  __syncthreads();

  // one thread per (token, slot): every slot's row depends only on the bitmaps,
  // the offsets and (with capacity) the slot bases
  for (int p = tid; p < T * k; p += 1024) {
    const int t = p / k, j = p - t * k;
    const int ej = idx[p];
    int row;
    if (static_cast<unsigned>(ej) >= static_cast<unsigned>(E)) {
      row = -1;
    } else if (!cap) {
      row = off[ej] + bits_below(bm, ej, t, nw);
    } else {
      const int key = j * E + ej;
      const int rank_j = bits_below(bm, key, t, nw);
      if (static_cast<long long>(sbase[key]) + rank_j >= C) {
        row = -1;
      } else {
        int before = 0;
        for (int j2 = 0; j2 < k; ++j2) {
          const int key2 = j2 * E + ej;
          const int r2 = bits_below(bm, key2, t, nw);
          const int kk = skeep[key2];
          before += r2 < kk ? r2 : kk;
        }
        row = off[ej] + before;
      }
    }
    dest[p] = row;
    if (row >= 0) src[row] = t;
  }

}

// LDS words of index_single_body
__host__ __device__ constexpr size_t index_single_words(int E, int nkeys) {
  return static_cast<size_t>(nkeys) * (kWords + 3) + (E + 1) + 16;
}

__global__ __launch_bounds__(1024) void index_single_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, long long C,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src,
    LoadOut o, int BM, int max_tiles, int ep, int4* __restrict__ tiles) {
  extern __shared__ uint32_t smem[];
  index_single_body(idx, T, k, E, C, offsets, dest, src, o, BM, max_tiles, ep, tiles, smem);
}

// Small batches in one launch: selection (as router_select_kernel, without the
// statistics) and then the single-workgroup index. Wave w selects the tokens
// w, w + 16, ...; their choices go to idx and gates and to LDS, from where the
// index body reads them after a barrier. One launch instead of two for the
// decode-sized steps of the fused forward. The caller may place the tile table
// over the logits (z and tiles may alias, hence no __restrict__ on either): every
// logit is read before the barrier that precedes the first tile store.
// J > 0 (a small bf16 router, T * E <= kRouteScoresMaxPairs): the logits are
// computed here first, into LDS, each by four waves exactly as
// router_scores_gemv_kernel<1, J> does (256 threads, chunk c on thread c % 256,
// J chunks each in order, a wave butterfly, the four wave sums in order), so z is
// the same bit for bit and the scores' launch is saved.
template <int NE, int J>
__global__ __launch_bounds__(1024) void route_index_single_kernel(
    const float* z, const uint16_t* __restrict__ xr, const uint16_t* __restrict__ wr, int d,
    const float* __restrict__ bias, int T, int k, int E,
    int gate_all, int32_t* __restrict__ idx, float* __restrict__ gates, long long C,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src,
    LoadOut o, int BM, int max_tiles, int4* tiles) {
  extern __shared__ uint32_t smem[];
  const int nkeys = C >= 0 ? E * k : E;   // as index_keys()
  int32_t* sidx = reinterpret_cast<int32_t*>(smem + index_single_words(E, nkeys));   // [T][k]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if constexpr (J > 0) {
    static_assert(kRouteScoresMaxPairs <= 8, "two rounds of four pairs");
    float* zl = reinterpret_cast<float*>(sidx + T * k);   // [T][E]
    float* red = zl + T * E;                                // [2][16] wave sums
    const int g = wv >> 2, wg = wv & 3, vt = threadIdx.x & 255;
    const int npairs = T * E, nchunk = d >> 3;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 wc[2][J], xc[2][J];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int p = 4 * r + g;
      const int t = p < npairs ? p / E : 0, e = p < npairs ? p % E : 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = vt + 256 * j;
        const bool in = p < npairs && c < nchunk;
        wc[r][j] = in ? *reinterpret_cast<const u32x4*>(wr + static_cast<size_t>(e) * d + c * 8)
                      : zero4;
        xc[r][j] = in ? *reinterpret_cast<const u32x4*>(xr + static_cast<size_t>(t) * d + c * 8)
                      : zero4;
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float w0 = __uint_as_float(wc[r][j][q] << 16);
          const float w1 = __uint_as_float(wc[r][j][q] & 0xFFFF0000u);
          acc = fmaf(__uint_as_float(xc[r][j][q] << 16), w0, acc);
          acc = fmaf(__uint_as_float(xc[r][j][q] & 0xFFFF0000u), w1, acc);
        }
      acc = wave_allsum(acc);
      if (lane == 0) red[16 * r + 4 * g + wg] = acc;
    }
    __syncthreads();
    if (vt == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int p = 4 * r + g;
        const float* rr = red + 16 * r + 4 * g;
        if (p < npairs) zl[p] = ((rr[0] + rr[1]) + rr[2]) + rr[3];
      }
    }
    __syncthreads();
    z = zl;
  }
  float b[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    b[i] = (bias != nullptr && e < E) ? bias[e] : 0.f;
  }
  for (int t = wv; t < T; t += 16) {
    TokenSelect<NE> ts;
    select_token<NE>(z + static_cast<size_t>(t) * E, b, E, k, gate_all, lane, ts);
    if (lane < k) {
      idx[static_cast<size_t>(t) * k + lane] = ts.e;
      gates[static_cast<size_t>(t) * k + lane] = ts.g;
      sidx[t * k + lane] = ts.e;
    }
  }
  __syncthreads();
  index_single_body(sidx, T, k, E, C, offsets, dest, src, o, BM, max_tiles, 1, tiles, smem);
}

bool route_scores_in_index_ok(int dtype_bf16, int T, int d, int E) {
  return dtype_bf16 && T * E <= kRouteScoresMaxPairs && d % 8 == 0 && d / 8 <= 512 &&
         router_score_plan(T, d, E).gemv;
}

static size_t index_single_lds(int E, int nkeys) {
  return index_single_words(E, nkeys) * sizeof(uint32_t);
}

bool index_single_ok(int T, int E, int k, bool cap) {
  return T <= kTB && E <= 1024 && index_keys(E, k, cap) <= kIndexSingleMaxKeys;
}

bool route_index_single_ok(int T, int E, int k, bool cap) {
  return T <= kRouteIndexMaxTokens && index_single_ok(T, E, k, cap);
}

hipError_t launch_route_index_single(const float* z, const float* bias, int T, int k, int E,
                                     int gate_all, int32_t* idx, float* gates,
                                     long long capacity, int32_t* offsets, int32_t* dest,
                                     int32_t* src, const LoadOut& load, int BM, int max_tiles,
                                     int32_t* tiles, hipStream_t s, const void* x,
                                     const void* w_router, int d) {
  const bool cap = capacity >= 0;
  if (!route_index_single_ok(T, E, k, cap)) return hipErrorInvalidValue;
  const bool scores = x != nullptr;
  if (scores && !route_scores_in_index_ok(1, T, d, E)) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const size_t lds = index_single_lds(E, index_keys(E, k, cap)) +
                     static_cast<size_t>(T) * k * sizeof(int32_t) +
                     (scores ? (static_cast<size_t>(T) * E + 32) * sizeof(float) : 0);
  const int ne = (E + 63) / 64;
  const auto* xr = static_cast<const uint16_t*>(x);
  const auto* wr = static_cast<const uint16_t*>(w_router);
#define MOE_RIS(NE_, J_)                                                                     \
  do {                                                                                       \
    auto kern = route_index_single_kernel<NE_, J_>;                                          \
    if (lds > 65536) {                                                                       \
      const hipError_t e1 = allow_large_lds(reinterpret_cast<const void*>(kern), lds);       \
      if (e1 != hipSuccess) return e1;                                                       \
    }                                                                                        \
    kern<<<dim3(1), dim3(1024), lds, s>>>(z, xr, wr, d, bias, T, k, E, gate_all, idx, gates, \
                                          cap ? capacity : -1, offsets, dest, src, load, BM, \
                                          max_tiles, reinterpret_cast<int4*>(tiles));        \
  } while (0)
  if (scores) {   // E <= kRouteScoresMaxPairs: one selection chunk per lane
    if (d / 8 <= 256) MOE_RIS(1, 1);
    else MOE_RIS(1, 2);
  } else if (ne <= 1) {
    MOE_RIS(1, 0);
  } else if (ne <= 2) {
    MOE_RIS(2, 0);
  } else if (ne <= 4) {
    MOE_RIS(4, 0);
  } else {
    MOE_RIS(16, 0);
  }
#undef MOE_RIS
  return hipGetLastError();
}

hipError_t launch_index(const int32_t* idx, int T, int k, int E, long long capacity,
                        int32_t* blk, int32_t* slot_base, int32_t* slot_keep, int32_t* offsets,
                        int32_t* dest, int32_t* src, const LoadOut& load, int BM, int max_tiles,
                        int ep, int32_t* tiles, hipStream_t s) {
  const bool cap = capacity >= 0;
  if (index_single_ok(T, E, k, cap)) {
    const size_t lds = index_single_lds(E, index_keys(E, k, cap));
    if (lds > 65536) {
      hipError_t e1 = allow_large_lds(reinterpret_cast<const void*>(index_single_kernel), lds);
      if (e1 != hipSuccess) return e1;
    }
    index_single_kernel<<<dim3(1), dim3(1024), lds, s>>>(
        idx, T, k, E, cap ? capacity : -1, offsets, dest, src, load, BM, max_tiles, ep,
        reinterpret_cast<int4*>(tiles));
    return hipGetLastError();
  }
  const int nb = index_blocks(T);
  const int nkeys = index_keys(E, k, cap);
  const size_t lds = static_cast<size_t>(nkeys) * kWords * sizeof(uint32_t);
  if (lds > 65536) {
    hipError_t e1 = allow_large_lds(reinterpret_cast<const void*>(index_count_kernel), lds);
    if (e1 != hipSuccess) return e1;
    hipError_t e2 = allow_large_lds(reinterpret_cast<const void*>(index_rank_kernel), lds);
    if (e2 != hipSuccess) return e2;
  }
  index_count_kernel<<<dim3(nb), dim3(kTB), lds, s>>>(idx, T, k, E, cap ? 1 : 0, blk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  index_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(blk, nb, T, k, E, cap ? capacity : -1,
                                                   slot_base, slot_keep, offsets, load, ep, BM,
                                                   max_tiles, reinterpret_cast<int4*>(tiles));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  index_rank_kernel<<<dim3(nb), dim3(kTB), lds, s>>>(idx, T, k, E, cap ? capacity : -1, blk,
                                                     slot_base, slot_keep, offsets, dest, src);
  return hipGetLastError();
}

}  // namespace moe
