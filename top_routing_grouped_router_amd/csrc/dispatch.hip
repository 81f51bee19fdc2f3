// Token counts per expert, expert offsets, the stable permutation of the token copies and
// the per-expert M-tile list of the grouped GEMMs.
//
// "Как устроен Olmo-core 3: обучение больших MoE-моделей":
//   * section "Балансировка нагрузки и вспомогательные штрафы": the selected indices are
//     histogrammed over all tokens into one count per expert;
//   * section "Пересылка токенов между экспертами": the expert indices are sorted, which
//     orders the tokens by expert, and the bins are the cumulative sum of the counts;
//   * section "Вычисления экспертов и точность": offsets are int32 cumulative sums.
// The sort is stable over the flat assignment index a = t*k + j, so the permutation is
// unique and identical on every run.
//
// Design (no sort, no order-dependent atomics):
//   rank_kernel     256 tokens per block, one wavefront per 64 tokens. Each wavefront ORs
//                   a bit per (expert, lane) into a 64-bit LDS mask (OR commutes, so the
//                   masks are exact); a copy's rank inside the block is the popcount of the
//                   lower lanes' bits plus the earlier wavefronts' counts. Block counts go
//                   to an (E, nblocks) table.
//   scan_cols       one block per expert: exclusive scan of its row of block counts ->
//                   per-block bases; total -> counts[e].
//   offsets_tiles   one block: exclusive scan of counts -> offsets; M-tiles per expert
//                   (TilePlan: whole tiles, the remainder on one more tile or on the
//                   remainder list, a thin last round moved there) -> the two tile lists,
//                   one thread per tile entry. Experts with no tokens get no tile, so their
//                   weights are never read.
//   permute         one thread per copy: position = offset + block base + rank.
//   dispatch_small  all of the above in one workgroup for batches of at most 1024 tokens,
//                   where four launches would cost more than the work.
// Entries that the routing never produces are handled alike by both paths: an index out of
// [0, E), or one that repeats an earlier index of its token, is not counted and gets no
// position (inverse -1). A repeat is seen in the mask ORs: the thread that owns the token ORs
// its bit once per entry, in entry order, so a repeated expert finds its bit already set.
// Everything here moves O(T*k) int32 words: a few MB at the largest shapes.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kRankTokens = 256;  // tokens per rank block (4 wavefronts)

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ idx, int64_t T, int k,
                                                   int E, int nblk, int32_t* __restrict__ rank,
                                                   int32_t* __restrict__ blk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* bits = reinterpret_cast<uint64_t*>(smem);            // [4][E]
  int32_t* pre = reinterpret_cast<int32_t*>(bits + 4 * E);       // [4][E]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += kWave) bits[wave * E + e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(b) * kRankTokens + wave * kWave + lane;
  uint32_t rep = 0;  // bit j: entry j repeats an earlier expert of the token (k <= 16)
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) {
        const unsigned long long old = atomicOr(reinterpret_cast<unsigned long long*>(&bits[wave * E + e]),
                                                1ull << lane);
        if (old & (1ull << lane)) rep |= 1u << j;
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pre[w * E + e] = run;
      run += __popcll(bits[w * E + e]);
    }
    blk[static_cast<int64_t>(e) * nblk + b] = run;
  }
  __syncthreads();
  if (t < T) {
    const uint64_t below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E)
        rank[t * k + j] = ((rep >> j) & 1u) ? -1 : pre[wave * E + e] + __popcll(bits[wave * E + e] & below);
    }
  }
}

// Inclusive scan across a 256- or 1024-thread block; `sh` holds one int per wavefront.
__device__ int block_inclusive_scan(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int x = lane < nw ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(x, o, kWave);
      if (lane >= o) x += u;
    }
    if (lane < nw) sh[lane] = x;  // inclusive wave totals
  }
  __syncthreads();
  const int add = wave > 0 ? sh[wave - 1] : 0;
  const int total = sh[nw - 1];
  __syncthreads();
  sh[16] = total;  // published for the caller after the next barrier
  return v + add;
}

__global__ __launch_bounds__(256) void scan_cols_kernel(int32_t* __restrict__ blk, int nblk,
                                                        int32_t* __restrict__ counts) {
  __shared__ int sh[17];
  const int e = blockIdx.x;
  int32_t* row = blk + static_cast<int64_t>(e) * nblk;
  int carry = 0;
  for (int base = 0; base < nblk; base += 256) {
    const int i = base + threadIdx.x;
    const int v = i < nblk ? row[i] : 0;
    const int incl = block_inclusive_scan(v, sh);
    if (i < nblk) row[i] = carry + incl - v;
    __syncthreads();
    carry += sh[16];
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Tiles of one expert with c rows under a plan: nb in the main list, ns in the remainder list.
__device__ __forceinline__ void expert_tile_counts(int c, const TilePlan& p, int& nb, int& ns) {
  const int full = c / p.bm, r = c - full * p.bm;
  if (r == 0 || r > p.small_max) {
    nb = full + (r > 0 ? 1 : 0);
    ns = 0;
  } else {
    nb = full;
    ns = (r + p.bs - 1) / p.bs;
  }
}

// Writes expert e's tiles (rows [excl, excl + c) of the sorted order) at list positions tb / ts.
__device__ __forceinline__ void write_expert_tiles(int e, int excl, int c, const TilePlan& p, int nb, int ns,
                                                   int tb, int ts, const TileList& big, const TileList& small) {
  for (int i = 0; i < nb; ++i) {
    const int ti = tb + i;
    if (ti >= big.cap) break;
    big.expert[ti] = e;
    big.row0[ti] = excl + i * p.bm;
    big.rows[ti] = min(p.bm, c - i * p.bm);
  }
  const int r0 = nb * p.bm;
  for (int i = 0; i < ns; ++i) {
    const int ti = ts + i;
    if (ti >= small.cap) break;
    small.expert[ti] = e;
    small.row0[ti] = excl + r0 + i * p.bs;
    small.rows[ti] = min(p.bs, c - r0 - i * p.bs);
  }
}

// counts -> offsets (or offsets given) -> M-tile lists. One block of 1024 threads, E <= 1024.
// With a capacity (> 0) the offsets are those of the kept counts min(count, capacity), and
// drop_off (E + 1) receives the exclusive scan of the dropped counts. With perm, the positions
// past the kept and dropped assignments (those of entries that get no position) are set to -1
// before permute_kernel writes the others.
__global__ __launch_bounds__(1024) void offsets_tiles_kernel(const int32_t* __restrict__ counts_in,
                                                             const int32_t* __restrict__ offsets_in,
                                                             int32_t* __restrict__ offsets_out,
                                                             int E, TilePlan plan, TileList tiles,
                                                             TileList small_tiles, int capacity,
                                                             int32_t* __restrict__ drop_off,
                                                             int32_t* __restrict__ perm, int64_t A) {
  __shared__ int sh[17];
  const int e = threadIdx.x;
  int c = 0, excl = 0;
  if (offsets_in) {
    if (e < E) {
      excl = offsets_in[e];
      c = offsets_in[e + 1] - excl;
    }
  } else {
    const int n = e < E ? counts_in[e] : 0;
    c = capacity > 0 ? min(n, capacity) : n;
    excl = block_inclusive_scan(c, sh) - c;
    if (e < E) offsets_out[e] = excl;
    if (e == E - 1) offsets_out[E] = excl + c;
    __syncthreads();
    int64_t placed = sh[16];  // kept assignments
    __syncthreads();
    if (capacity > 0) {
      const int dc = n - c;
      const int dexcl = block_inclusive_scan(dc, sh) - dc;
      if (e < E) drop_off[e] = dexcl;
      if (e == E - 1) drop_off[E] = dexcl + dc;
      __syncthreads();
      placed += sh[16];      // + dropped assignments
      __syncthreads();
    }
    if (perm)
      for (int64_t p = placed + threadIdx.x; p < A; p += blockDim.x) perm[p] = -1;
  }
  if (tiles.cap <= 0) return;
  c = c < 0 ? 0 : c;
  int nb = 0, ns = 0;
  if (e < E) expert_tile_counts(c, plan, nb, ns);
  // Thin last round of the main list (TilePlan): move m whole M-tiles of one expert to the
  // remainder list. The rule reads only the block-wide total, so every thread agrees on m.
  block_inclusive_scan(nb, sh);
  __syncthreads();
  const int total0 = sh[16];
  __syncthreads();
  const int R = plan.tail_round, ntn = plan.tail_ntn;
  int m = 0;
  if (small_tiles.cap > 0 && plan.small_max > 0 && R > 0 && R <= kTailRoundMax && ntn > 0) {
    const int64_t work = static_cast<int64_t>(total0) * ntn;
    const int tail = static_cast<int>(work % R);
    if (work > R && tail > 0 && 8 * tail <= R) m = (tail + ntn - 1) / ntn;
  }
  if (m > 0) {
    __shared__ int s_pick;
    if (threadIdx.x == 0) s_pick = 0x7fffffff;
    __syncthreads();
    // experts that already have remainder tiles first, then by index
    if (e < E && nb >= m) atomicMin(&s_pick, (ns > 0 ? 0 : E) + e);
    __syncthreads();
    const int pick = s_pick;
    if (pick != 0x7fffffff && e == pick % E) {
      nb -= m;
      ns = (c - nb * plan.bm + plan.bs - 1) / plan.bs;
    }
  }
  const int tb = block_inclusive_scan(nb, sh) - nb;
  __syncthreads();
  const int total = sh[16];
  __syncthreads();
  const int ts = block_inclusive_scan(ns, sh) - ns;
  __syncthreads();
  const int total_s = sh[16];
  __syncthreads();
  block_inclusive_scan(nb >= kSpreadMinMTiles ? nb : 0, sh);  // M-tiles of large experts
  __syncthreads();
  const int in_large = sh[16];
  // Tile entries, one thread per tile: tile t of a list belongs to the last expert whose first
  // tile is at or before t (experts without tiles share their start with the next expert).
  __shared__ int s_tb[MOE_MAX_EXPERTS], s_ts[MOE_MAX_EXPERTS], s_row[MOE_MAX_EXPERTS], s_cnt[MOE_MAX_EXPERTS],
      s_srow[MOE_MAX_EXPERTS];
  if (e < E) {
    s_tb[e] = tb;
    s_ts[e] = ts;
    s_row[e] = excl;
    s_cnt[e] = c;
    s_srow[e] = nb * plan.bm;  // first row (inside the expert) of its remainder tiles
  }
  __syncthreads();
  auto owner = [&](const int* start, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  const int nbig = min(total, tiles.cap);
  for (int t = threadIdx.x; t < nbig; t += blockDim.x) {
    const int x = owner(s_tb, t), i = t - s_tb[x];
    tiles.expert[t] = x;
    tiles.row0[t] = s_row[x] + i * plan.bm;
    tiles.rows[t] = min(plan.bm, s_cnt[x] - i * plan.bm);
  }
  const int nsmall = min(total_s, small_tiles.cap);
  for (int t = threadIdx.x; t < nsmall; t += blockDim.x) {
    const int x = owner(s_ts, t), r = s_srow[x] + (t - s_ts[x]) * plan.bs;
    small_tiles.expert[t] = x;
    small_tiles.row0[t] = s_row[x] + r;
    small_tiles.rows[t] = min(plan.bs, s_cnt[x] - r);
  }
  if (threadIdx.x == 0) {
    tiles.count[0] = nbig;
    tiles.count[1] = total > 0 && 2 * in_large >= total ? 1 : 0;
    if (small_tiles.cap > 0) {
      small_tiles.count[0] = nsmall;
      small_tiles.count[1] = 0;
    }
  }
}

// Position of an assignment whose rank inside its expert's stable order is r: the kept rows
// (r < capacity, or no capacity) follow the expert offsets; the dropped ones come after all
// kept rows, grouped by expert in the same order.
__device__ __forceinline__ int64_t sorted_position(int64_t r, int e, int E, const int32_t* off,
                                                   const int32_t* drop_off, int capacity) {
  if (capacity <= 0 || r < capacity) return static_cast<int64_t>(off[e]) + r;
  return static_cast<int64_t>(off[E]) + drop_off[e] + (r - capacity);
}

__global__ __launch_bounds__(256) void permute_kernel(const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ blk, int nblk,
                                                      const int32_t* __restrict__ offsets, int64_t A,
                                                      int k, int E, int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inv, int capacity,
                                                      const int32_t* __restrict__ drop_off) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= A) return;
  const int e = idx[a];
  if (e < 0 || e >= E || rank[a] < 0) {  // out of range, or a repeat within the token
    inv[a] = -1;
    return;
  }
  const int64_t t = a / k;
  const int64_t b = t / kRankTokens;
  const int64_t r = static_cast<int64_t>(blk[static_cast<int64_t>(e) * nblk + b]) + rank[a];
  const int64_t pos = sorted_position(r, e, E, offsets, drop_off, capacity);
  if (pos >= 0 && pos < A) perm[pos] = static_cast<int32_t>(a);
  inv[a] = static_cast<int32_t>(pos);
}

// Rows of the expert output (assignment order) of dropped assignments are zero: sorted
// positions p in [offsets[E], A) hold them, row perm[p] of y (row_bytes each, a multiple of 16).
__global__ __launch_bounds__(256) void zero_dropped_kernel(const int32_t* __restrict__ offsets, int E,
                                                           const int32_t* __restrict__ perm, int64_t A,
                                                           unsigned char* __restrict__ y, int64_t row_bytes) {
  const int64_t p0 = min(max(static_cast<int64_t>(offsets[E]), int64_t(0)), A);
  const int64_t cpr = row_bytes / 16;
  const int64_t n = (A - p0) * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t a = perm[p0 + i / cpr];
    if (a >= 0 && a < A) *reinterpret_cast<uint4*>(y + a * row_bytes + (i % cpr) * 16) = make_uint4(0, 0, 0, 0);
  }
}

int num_rank_blocks(int64_t T) { return static_cast<int>((T + kRankTokens - 1) / kRankTokens); }

// Exclusive scan over the E <= 1024 entries v[0..E) of an LDS array by one 256-thread block
// (four consecutive entries per thread); writes the scan to out[0..E] (out[E] = total).
__device__ void block_exclusive_scan_e(const int32_t* v, int E, int32_t* out, int* sh) {
  const int e0 = threadIdx.x * 4;
  int loc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    loc[q] = e0 + q < E ? v[e0 + q] : 0;
    sum += loc[q];
  }
  int run = block_inclusive_scan(sum, sh) - sum;
  __syncthreads();
  const int total = sh[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e0 + q < E) out[e0 + q] = run;
    run += loc[q];
  }
  if (threadIdx.x == 0) out[E] = total;
}

// The whole dispatch of a small batch (T <= kSmallTokens) in one 256-thread workgroup:
// histogram, offsets, M-tile list and stable permutation, with no intermediate global
// buffers. Pass 1 counts with LDS atomics (exact); pass 2 walks the tokens in chunks of 256
// in order and ranks each copy like rank_kernel (64-bit per-wavefront masks), on top of the
// running count of its expert from the earlier chunks. The first 256 tokens' entries are read
// from memory once for both passes, and each pair of per-expert counts is scanned as one packed
// value.
constexpr int kSmallTokens = 1024;
constexpr int kMaxTopK = MOE_MAX_TOP_K;  // entries per token (top_k is validated against it)

__global__ __launch_bounds__(256) void dispatch_small_kernel(const int32_t* __restrict__ idx, int64_t T, int k,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv, TileList tiles,
                                                             TileList small_tiles, TilePlan plan, int capacity) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* bits = reinterpret_cast<uint64_t*>(smem);  // [4][E]
  int32_t* pre = reinterpret_cast<int32_t*>(bits + 4 * E);  // [4][E]
  int32_t* run = pre + 4 * E;                           // [E] counts, then running rank base
  int32_t* off = run + E;                               // [E + 1] offsets (of the kept counts)
  int32_t* doff = off + E + 1;                          // [E + 1] offsets of the dropped counts
  int32_t* kc = pre;                                    // [E] kept counts (pass 1 only)
  int32_t* dc = pre + E;                                // [E] dropped counts (pass 1 only)
  int32_t* mt = pre + 2 * E;                            // [E] main-list tiles per expert (pass 1 only)
  int32_t* ms = pre + 3 * E;                            // [E] remainder-list tiles per expert (pass 1)
  int32_t* tb = pre;                                    // [E + 1] first main-list tile (pass 1)
  int32_t* ts = reinterpret_cast<int32_t*>(bits);       // [E + 1] first remainder tile (pass 1; bits is free)
  __shared__ int sh[17];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t A = T * k;
  // Two counts packed in one scan (16 bits each): A <= kSmallTokens * kMaxTopK assignments.
  static_assert(kSmallTokens * kMaxTopK < 65536, "packed scans");

  // Each token's k entries are read as independent loads; those of the first 256 tokens (all of
  // a decode-sized batch) stay in registers for the second pass. The zeroing below overlaps the
  // first chunk's loads.
  int ek0[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) ek0[j] = (tid < T && j < k) ? idx[static_cast<int64_t>(tid) * k + j] : -1;
  for (int e = tid; e < E; e += 256) run[e] = 0;
  __syncthreads();
  // An entry repeating an earlier expert of its token is not counted.
  for (int64_t t = tid; t < T; t += 256) {
    int ek[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) ek[j] = t < 256 ? ek0[j] : (j < k ? idx[t * k + j] : -1);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ek[j];
      if (e < 0 || e >= E) continue;
      bool repeat = false;
#pragma unroll
      for (int q = 0; q < j; ++q) repeat |= ek[q] == e;
      if (!repeat) atomicAdd(&run[e], 1);
    }
  }
  __syncthreads();
  // kept | dropped << 16, scanned once
  for (int e = tid; e < E; e += 256) {
    const int kept = capacity > 0 ? min(run[e], capacity) : run[e];
    kc[e] = kept | ((run[e] - kept) << 16);
  }
  __syncthreads();
  block_exclusive_scan_e(kc, E, off, sh);
  __syncthreads();
  for (int e = tid; e <= E; e += 256) {
    const int v = off[e];
    off[e] = v & 0xFFFF;
    doff[e] = v >> 16;
  }
  __syncthreads();
  // positions past the kept and dropped assignments belong to no entry
  for (int64_t p = static_cast<int64_t>(off[E]) + doff[E] + tid; p < A; p += 256) perm[p] = -1;
  for (int e = tid; e < E; e += 256) {
    counts[e] = run[e];
    offsets[e] = off[e];
    int nb, ns;
    expert_tile_counts(off[e + 1] - off[e], plan, nb, ns);
    mt[e] = nb;
    ms[e] = ns;
    dc[e] = nb | (ns << 16);
  }
  if (tid == 0) offsets[E] = off[E];
  __syncthreads();
  if (tiles.cap > 0) {
    // first tile of each list, scanned once (packed as above); tb[E] overwrites dc[0] only
    // after every thread has read its entries of dc
    block_exclusive_scan_e(dc, E, tb, sh);
    __syncthreads();
    if (tid == 0) sh[16] = 0;
    for (int e = tid; e <= E; e += 256) {
      const int v = tb[e];
      tb[e] = v & 0xFFFF;
      ts[e] = v >> 16;
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      write_expert_tiles(e, off[e], off[e + 1] - off[e], plan, mt[e], ms[e], tb[e], ts[e], tiles, small_tiles);
      if (mt[e] >= kSpreadMinMTiles) atomicAdd(&sh[16], mt[e]);  // M-tiles of large experts
    }
    __syncthreads();
    if (tid == 0) {
      tiles.count[0] = min(tb[E], tiles.cap);
      tiles.count[1] = tb[E] > 0 && 2 * sh[16] >= tb[E] ? 1 : 0;
      if (small_tiles.cap > 0) {
        small_tiles.count[0] = min(ts[E], small_tiles.cap);
        small_tiles.count[1] = 0;
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += 256) run[e] = 0;
  __syncthreads();

  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    // only the wavefronts holding tokens of this chunk keep masks
    const int nwa = static_cast<int>(min(static_cast<int64_t>(4), (T - t0 + 63) / 64));
    for (int i = tid; i < nwa * E; i += 256) bits[i] = 0;
    __syncthreads();
    const int64_t t = t0 + tid;
    uint32_t rep = 0;  // bit j: entry j repeats an earlier expert of the token
    int ek[kMaxTopK];  // the token's entries
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) ek[j] = t0 == 0 ? ek0[j] : ((t < T && j < k) ? idx[t * k + j] : -1);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ek[j];
      if (e >= 0 && e < E) {
        const unsigned long long old =
            atomicOr(reinterpret_cast<unsigned long long*>(&bits[wave * E + e]), 1ull << lane);
        if (old & (1ull << lane)) rep |= 1u << j;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      int r = run[e];
      for (int w = 0; w < nwa; ++w) {
        pre[w * E + e] = r;
        r += __popcll(bits[w * E + e]);
      }
      run[e] = r;
    }
    __syncthreads();
    if (t < T) {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k) break;
        const int64_t a = t * k + j;
        const int e = ek[j];
        if (e < 0 || e >= E || ((rep >> j) & 1u)) {
          inv[a] = -1;
          continue;
        }
        const int64_t r = static_cast<int64_t>(pre[wave * E + e]) + __popcll(bits[wave * E + e] & below);
        const int64_t pos = sorted_position(r, e, E, off, doff, capacity);
        if (pos >= 0 && pos < A) perm[pos] = static_cast<int32_t>(a);
        inv[a] = static_cast<int32_t>(pos);
      }
    }
    __syncthreads();
  }
}

}  // namespace

size_t dispatch_scratch_bytes(const Layer& ly) {
  const size_t A = static_cast<size_t>(ly.T) * ly.k;
  const size_t nblk = static_cast<size_t>(num_rank_blocks(ly.T));
  // rank (A), block counts (E, nblk), dropped-count offsets (E + 1)
  return (A + static_cast<size_t>(ly.E) * nblk + static_cast<size_t>(ly.E) + 1) * sizeof(int32_t) + 256;
}

namespace {
// The plan with its thin-last-round fields (TilePlan) for the bf16 large tiles of this device.
// (The one-workgroup dispatch of small batches builds its lists without the move.)
TilePlan with_tail(const Layer& ly, const TilePlan& plan) {
  TilePlan p = plan;
  if (ly.bf16 && !ly.mx && p.small_max > 0) {
    p.tail_round = gemm_bf16_round_tiles();
    const int64_t cols = gemm_bf16_swiglu_tile_cols();
    p.tail_ntn = static_cast<int>((ly.h + cols - 1) / cols);
  }
  return p;
}
}  // namespace

hipError_t launch_dispatch(const Layer& ly, const int32_t* idx, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* inv, void* scratch, const TileList& tiles,
                           const TileList& small_tiles, const TilePlan& plan, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  const int cap = static_cast<int>(ly.capacity);  // <= T rounded up to 8, below 2^31
  if (ly.T <= kSmallTokens) {
    // bits [4][E] u64, pre [4][E], run [E], off [E + 1], doff [E + 1]: 60 E + 8 bytes
    // (61 KiB at E = 1024)
    const size_t lds = static_cast<size_t>(ly.E) * 4 * (sizeof(uint64_t) + sizeof(int32_t)) +
                       static_cast<size_t>(3 * ly.E + 2) * sizeof(int32_t);
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(256), lds, s, idx, ly.T, ly.k, ly.E, counts, offsets,
                       perm, inv, tiles, small_tiles, plan, cap);
    return hipGetLastError();
  }
  const int nblk = num_rank_blocks(ly.T);
  const int64_t A = ly.T * ly.k;
  int32_t* rank = static_cast<int32_t*>(scratch);
  int32_t* blk = rank + A;
  int32_t* drop_off = blk + static_cast<int64_t>(ly.E) * nblk;
  const size_t lds = static_cast<size_t>(ly.E) * 4 * (sizeof(uint64_t) + sizeof(int32_t));
  hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(256), lds, s, idx, ly.T, ly.k, ly.E, nblk, rank,
                     blk);
  hipLaunchKernelGGL(scan_cols_kernel, dim3(ly.E), dim3(256), 0, s, blk, nblk, counts);
  hipLaunchKernelGGL(offsets_tiles_kernel, dim3(1), dim3(1024), 0, s, counts, nullptr, offsets, ly.E,
                     with_tail(ly, plan), tiles, small_tiles, cap, drop_off, perm, A);
  hipLaunchKernelGGL(permute_kernel, dim3(static_cast<unsigned>((A + 255) / 256)), dim3(256), 0, s,
                     idx, rank, blk, nblk, offsets, A, ly.k, ly.E, perm, inv, cap, drop_off);
  return hipGetLastError();
}

hipError_t launch_zero_dropped(const Layer& ly, const int32_t* offsets, const int32_t* perm, void* y,
                               hipStream_t s) {
  const int64_t A = ly.T * ly.k;
  if (ly.capacity <= 0 || A <= 0) return hipSuccess;
  const int64_t row_bytes = ly.K * (ly.bf16 ? 2 : 4);
  const int64_t chunks = A * (row_bytes / 16);
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((chunks + 255) / 256, 2048));
  hipLaunchKernelGGL(zero_dropped_kernel, dim3(grid), dim3(256), 0, s, offsets, ly.E, perm, A,
                     static_cast<unsigned char*>(y), row_bytes);
  return hipGetLastError();
}

namespace {
// counts (E) and offsets (E + 1) of an empty batch, zeroed by a kernel rather than memset nodes so
// that a caller may capture the call in a graph.
__global__ __launch_bounds__(256) void zero_counts_offsets_kernel(int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets, int E) {
  for (int e = blockIdx.x * 256 + threadIdx.x; e <= E; e += gridDim.x * 256) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}
}  // namespace

hipError_t launch_zero_counts_offsets(int32_t* counts, int32_t* offsets, int E, hipStream_t s) {
  hipLaunchKernelGGL(zero_counts_offsets_kernel, dim3(static_cast<unsigned>((E + 256) / 256)), dim3(256), 0, s,
                     counts, offsets, E);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const Layer& ly, const int32_t* offsets, const TileList& tiles,
                              const TileList& small_tiles, const TilePlan& plan, hipStream_t s) {
  hipLaunchKernelGGL(offsets_tiles_kernel, dim3(1), dim3(1024), 0, s, nullptr, offsets, nullptr,
                     ly.E, with_tail(ly, plan), tiles, small_tiles, 0, nullptr, nullptr, int64_t(0));
  return hipGetLastError();
}

}  // namespace moe
