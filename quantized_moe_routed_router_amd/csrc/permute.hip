// Token-by-expert permutation: stable counting sort of the T*k (token, slot)
// pairs by expert, so each expert's weights are read once per batch and its
// rows form one contiguous group for the grouped GEMM.  (Every picked expert
// is computed: forum repost, paragraph "Where it stands".)
//
// Three passes, no host round trip (one launch up to PSB_MAX_N entries):
//   1. per 1024-entry chunk, a histogram over experts (LDS atomics);
//   2. per expert, the exclusive prefix of its chunk counts (chunk order), and
//      the exclusive prefix over experts -> offsets, counts, tile prefix and
//      one record per row tile (with a second list, experts below split_rows
//      rows are tiled by BM2 rows there instead, the others by BM rows);
//   3. per chunk, one wave walks its entries 64 at a time in order; equal-
//      expert lanes are found with ballots over the id bits, so ranks inside a
//      step and across steps keep the original order (stable).
// Ids outside [0, E) are sorted into a trailing bin after expert E-1.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int PCH = 1024;   // entries per chunk

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ ids, int N,
                                                         int E, int32_t* __restrict__ chunk_counts) {
  extern __shared__ int hist[];                        // [E+1]
  for (int e = threadIdx.x; e <= E; e += 256) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * PCH;
  for (int i = threadIdx.x; i < PCH; i += 256) {
    const int g = base + i;
    if (g < N) {
      int e = ids[g];
      if ((unsigned)e >= (unsigned)E) e = E;
      atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += 256) chunk_counts[(size_t)blockIdx.x * (E + 1) + e] = hist[e];
}

// One wave per bin: lane l owns a contiguous run of chunks; per-lane sums,
// an exclusive scan of them across the wave, then each lane writes the
// running prefix over its chunks (chunk order, so the sort stays stable).
__global__ __launch_bounds__(256) void perm_chunk_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                              int nchunks, int E,
                                                              int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e > E) return;                                    // wave-uniform; no block barrier below
  const int per = (nchunks + 63) / 64;
  const int c0 = min(lane * per, nchunks), c1 = min(c0 + per, nchunks);
  int mine = 0;
#pragma unroll 8
  for (int c = c0; c < c1; ++c) mine += chunk_counts[(size_t)c * (E + 1) + e];
  int incl = mine;                                      // inclusive scan over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - mine;
#pragma unroll 8
  for (int c = c0; c < c1; ++c) {
    const size_t o = (size_t)c * (E + 1) + e;
    const int v = chunk_counts[o];
    chunk_base[o] = run;
    run += v;
  }
  if (lane == 63) totals[e] = incl;
}

// An expert's row-tile counts: BM-row tiles, or with a second list (sp.tile_map
// set) BM-row tiles from sp.split_rows rows up and sp.BM-row tiles below.
__device__ __forceinline__ void tile_counts(int rows, bool expert, int BM, const TileSplit& sp, int& n1, int& n2) {
  n1 = n2 = 0;
  if (!expert) return;
  if (sp.tile_map && rows < sp.split_rows) n2 = (rows + sp.BM - 1) / sp.BM;
  else if (BM > 0) n1 = (rows + BM - 1) / BM;
}

// Expert e's prefix entry and tile records {e, first row of the tile, end of
// the expert's rows} from the inclusive tile-count scan incl (of 1056 slots).
__device__ __forceinline__ void write_tiles(int e, int E, int first_row, int end_row, const int* incl, int BM,
                                            int32_t* tile_prefix, int32_t* tile_map) {
  const int t0 = e ? incl[e - 1] : 0;
  if (tile_prefix) tile_prefix[e] = t0;
  if (tile_map && e < E) {
    const int nt = incl[e] - t0;
    for (int i = 0; i < nt; ++i)
      *reinterpret_cast<int4*>(tile_map + (size_t)(t0 + i) * 4) = int4{e, first_row + i * BM, end_row, 0};
  }
}

// Single block: exclusive scan over bins (E+1 <= 1025 values).
__global__ __launch_bounds__(1024) void perm_offsets_kernel(const int32_t* __restrict__ totals, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ bin_start,
                                                            int32_t* __restrict__ tile_prefix,
                                                            int32_t* __restrict__ tile_map, int BM,
                                                            const TileSplit sp) {
  __shared__ int sc[2][1056];
  __shared__ int st[2][1056];
  __shared__ int st2[2][1056];
  const int tid = threadIdx.x;
  for (int e = tid; e < 1056; e += 1024) { sc[0][e] = 0; st[0][e] = 0; st2[0][e] = 0; }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) {
    const int v = totals[e];
    sc[0][e] = v;
    tile_counts(v, e < E, BM, sp, st[0][e], st2[0][e]);
  }
  __syncthreads();
  // Hillis-Steele inclusive scan over 1056 slots, ping-pong buffers
  int cur = 0;
  for (int off = 1; off < 1056; off <<= 1) {
    for (int e = tid; e < 1056; e += 1024) {
      sc[cur ^ 1][e] = sc[cur][e] + (e >= off ? sc[cur][e - off] : 0);
      st[cur ^ 1][e] = st[cur][e] + (e >= off ? st[cur][e - off] : 0);
      st2[cur ^ 1][e] = st2[cur][e] + (e >= off ? st2[cur][e - off] : 0);
    }
    __syncthreads();
    cur ^= 1;
  }
  for (int e = tid; e <= E; e += 1024) {
    const int excl = e ? sc[cur][e - 1] : 0;
    bin_start[e] = excl;
    if (e < E) counts[e] = totals[e];
    offsets[e] = excl;                               // offsets[E] = entries with valid ids
    write_tiles(e, E, excl, sc[cur][e], st[cur], BM, tile_prefix, tile_map);
    if (sp.tile_map) write_tiles(e, E, excl, sc[cur][e], st2[cur], sp.BM, sp.tile_prefix, sp.tile_map);
  }
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ bin_start,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  extern __shared__ int run[];                          // [E+1]
  const int lane = threadIdx.x;
  for (int e = lane; e <= E; e += 64) run[e] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) <= E) ++nbits;                   // bins 0..E need nbits bits
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int base = blockIdx.x * PCH;
  for (int s = 0; s < PCH; s += 64) {
    const int g = base + s + lane;
    const bool valid = g < N;
    int e = valid ? ids[g] : 0;
    if ((unsigned)e >= (unsigned)E) e = E;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      mask &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(mask & below);
      const int pos = bin_start[e] + chunk_base[(size_t)blockIdx.x * (E + 1) + e] + run[e] + rank;
      perm[pos] = g;
      inv[g] = pos;
      const bool last = (mask >> lane) == 1ull;        // highest lane of its group
      if (last) run[e] += __popcll(mask);
    }
    __syncthreads();
  }
}

// Small batches (N <= PSB_MAX_N) in one launch: one block of 16 waves, wave
// w owns the w-th contiguous sixteenth of the entries.  Per-wave histograms
// in LDS, their exclusive prefix per bin in wave order, the scan over bins
// (counts, offsets, tile prefix and records as above), then each wave places
// its entries 64 at a time with the same ballot ranks.  Entry order inside
// a wave, then wave order, is the original order, so the sort stays stable.
// Every wave runs the same number of steps, so the per-step barrier is
// uniform.
constexpr int PSB_WAVES = 16, PSB_MAX_N = 16384;

__global__ __launch_bounds__(64 * PSB_WAVES) void perm_small_kernel(const int32_t* __restrict__ ids, int N,
                                                                     int E, int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv,
                                                                     int32_t* __restrict__ tile_prefix,
                                                                     int32_t* __restrict__ tile_map, int BM,
                                                                     const TileSplit sp) {
  __shared__ int hist[PSB_WAVES][1025];                // per wave and bin: count, then running position
  __shared__ int sc[2][1056];
  __shared__ int st[2][1056];
  __shared__ int st2[2][1056];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < PSB_WAVES * 1025; i += 64 * PSB_WAVES) (&hist[0][0])[i] = 0;
  for (int e = tid; e < 1056; e += 64 * PSB_WAVES) { sc[0][e] = 0; st[0][e] = 0; st2[0][e] = 0; }
  __syncthreads();
  const int per = (N + PSB_WAVES - 1) / PSB_WAVES;
  const int c0 = min(wv * per, N), c1 = min(c0 + per, N);
  for (int g = c0 + lane; g < c1; g += 64) {
    int e = ids[g];
    if ((unsigned)e >= (unsigned)E) e = E;
    atomicAdd(&hist[wv][e], 1);
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 64 * PSB_WAVES) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < PSB_WAVES; ++w) {
      const int v = hist[w][e];
      hist[w][e] = run;
      run += v;
    }
    sc[0][e] = run;
    tile_counts(run, e < E, BM, sp, st[0][e], st2[0][e]);
  }
  __syncthreads();
  int cur = 0;                                          // Hillis-Steele inclusive scan
  for (int off = 1; off < 1056; off <<= 1) {
    for (int e = tid; e < 1056; e += 64 * PSB_WAVES) {
      sc[cur ^ 1][e] = sc[cur][e] + (e >= off ? sc[cur][e - off] : 0);
      st[cur ^ 1][e] = st[cur][e] + (e >= off ? st[cur][e - off] : 0);
      st2[cur ^ 1][e] = st2[cur][e] + (e >= off ? st2[cur][e - off] : 0);
    }
    __syncthreads();
    cur ^= 1;
  }
  for (int e = tid; e <= E; e += 64 * PSB_WAVES) {
    const int excl = e ? sc[cur][e - 1] : 0;
    if (e < E) counts[e] = sc[cur][e] - excl;
    offsets[e] = excl;
    write_tiles(e, E, excl, sc[cur][e], st[cur], BM, tile_prefix, tile_map);
    if (sp.tile_map) write_tiles(e, E, excl, sc[cur][e], st2[cur], sp.BM, sp.tile_prefix, sp.tile_map);
  }
  int nbits = 0;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = 0; s < per; s += 64) {
    const int g = c0 + s + lane;
    const bool valid = g < c1;
    int e = valid ? ids[g] : 0;
    if ((unsigned)e >= (unsigned)E) e = E;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      mask &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(mask & below);
      const int pos = (e ? sc[cur][e - 1] : 0) + hist[wv][e] + rank;
      perm[pos] = g;
      inv[g] = pos;
      const bool last = (mask >> lane) == 1ull;         // highest lane of its group
      if (last) hist[wv][e] += __popcll(mask);
    }
    __syncthreads();
  }
}

size_t permute_workspace_bytes(int T, int k, int E) {
  const size_t N = (size_t)T * k;
  const size_t nch = (N + PCH - 1) / PCH;
  return (2 * nch * (E + 1) + 2 * (size_t)(E + 1)) * sizeof(int32_t) + 256;
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                          int32_t* tile_prefix, int32_t* tile_map, int BM, hipStream_t s,
                          const TileSplit& split) {
  const int N = T * k;
  if (N <= PSB_MAX_N) {
    perm_small_kernel<<<1, 64 * PSB_WAVES, 0, s>>>(ids, N, E, counts, offsets, perm, inv, tile_prefix, tile_map, BM,
                                                   split);
    return hipGetLastError();
  }
  const int nch = (N + PCH - 1) / PCH;
  int32_t* cc = reinterpret_cast<int32_t*>(ws);
  int32_t* cb = cc + (size_t)nch * (E + 1);
  int32_t* totals = cb + (size_t)nch * (E + 1);
  int32_t* bin_start = totals + (E + 1);
  if (nch > 0) {
    perm_count_kernel<<<nch, 256, (E + 1) * sizeof(int), s>>>(ids, N, E, cc);
    perm_chunk_scan_kernel<<<(E + 1 + 3) / 4, 256, 0, s>>>(cc, nch, E, cb, totals);
  } else {
    perm_chunk_scan_kernel<<<(E + 1 + 3) / 4, 256, 0, s>>>(cc, 0, E, cb, totals);
  }
  perm_offsets_kernel<<<1, 1024, 0, s>>>(totals, E, counts, offsets, bin_start, tile_prefix, tile_map, BM, split);
  if (nch > 0)
    perm_scatter_kernel<<<nch, 64, (E + 1) * sizeof(int), s>>>(ids, N, E, cb, bin_start, perm, inv);
  return hipGetLastError();
}

}  // namespace moe
