// permute.hip — stable counting sort of the S = M*k (token, slot) pairs by
// expert id, over as many workgroups as the pairs need.
//
// Pass 1 (k_perm_count): workgroup g counts its segment of kPermSeg pairs
// per expert into ghist[g][e].  Pass 2 (k_perm_scatter): every workgroup
// reads all of ghist, so it knows each expert's start (an exclusive scan of
// the totals over experts) and its own base inside each expert's run (the
// counts of the segments before it).  Inside the workgroup, wavefront w owns
// a contiguous sub-segment: a per-wavefront LDS histogram gives its base, and
// equal ids inside each group of 64 pairs are ranked with ballots over the id
// bits.  The output is grouped by expert and ascending in pair index inside
// each expert — bit-identical on every run, whatever the number of
// workgroups.
#include "launch.hpp"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermSub = kPermSeg / kPermWaves;  // pairs per wavefront

__global__ __launch_bounds__(kPermThreads) void k_perm_count(const int32_t* __restrict__ ids, int S, int E,
                                                             int32_t* __restrict__ ghist, int32_t* __restrict__ err) {
  __shared__ int hist[kMaxExperts];
  __shared__ int bad;
  const int tid = threadIdx.x, g = blockIdx.x;
  for (int e = tid; e < E; e += kPermThreads) hist[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int lo = g * kPermSeg, hi = min(S, lo + kPermSeg);
  for (int p = lo + tid; p < hi; p += kPermThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    else atomicAdd(&bad, 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) ghist[(size_t)g * E + e] = hist[e];
  if (tid == 0 && bad) atomicOr(err, 1);
}

// Exclusive scan over v[0..n) in LDS (n <= kPermThreads), whole workgroup;
// v[n] receives the total.  Wavefront prefix sums with shuffles, then a scan
// of the wavefront totals.
__device__ void block_exclusive_scan(int* v, int n, int* wsum) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int x = tid < n ? v[tid] : 0;
  int inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < kPermWaves ? wsum[lane] : 0;
    int ti = t;
#pragma unroll
    for (int off = 1; off < kPermWaves; off <<= 1) {
      const int y = __shfl_up(ti, off, kWave);
      if (lane >= off) ti += y;
    }
    if (lane < kPermWaves) wsum[lane] = ti - t;  // exclusive over wavefronts
    if (lane == kPermWaves - 1) wsum[kPermWaves] = ti;
  }
  __syncthreads();
  if (tid < n) v[tid] = wsum[wave] + inc - x;
  if (tid == 0) v[n] = wsum[kPermWaves];
  __syncthreads();
}

struct PermOut {
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* perm;     // [S] pair at each sorted position (-1 past the valid pairs)
  int32_t* inv;      // [S] sorted position of each pair (-1 for invalid ids), or null
  int32_t* tile_e;   // [items] work items of kItemRows rows, or null
  int32_t* tile_j;
  int32_t* ntile;
};

__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(const int32_t* __restrict__ ids, int S, int E,
                                                               const int32_t* __restrict__ ghist, PermOut o) {
  __shared__ int whist[kPermWaves][kMaxExperts];
  __shared__ int start[kMaxExperts + 1];  // exclusive scan of the totals
  __shared__ int mine[kMaxExperts + 1];   // this workgroup's base inside each expert's run
  __shared__ int wsum[kPermWaves + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = blockIdx.x, G = gridDim.x;
  for (int e = tid; e < E; e += kPermThreads) {
    int tot = 0, before = 0;
    for (int gg = 0; gg < G; ++gg) {
      const int v = ghist[(size_t)gg * E + e];
      before += gg < g ? v : 0;
      tot += v;
    }
    start[e] = tot;
    mine[e] = before;
  }
  for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermThreads) (&whist[0][0])[i] = 0;
  __syncthreads();
  block_exclusive_scan(start, E, wsum);
  const int lo = g * kPermSeg + wave * kPermSub;
  const int hi = min(S, lo + kPermSub);
  for (int p = lo + lane; p < hi; p += kWave) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&whist[wave][e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    int run = start[e] + mine[e];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = whist[w][e];
      whist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = lo; b0 < hi; b0 += kWave) {
    const int p = b0 + lane;
    const int e = p < hi ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool b = valid && ((e >> bit) & 1);
      const uint64_t bal = __ballot(b);
      m &= b ? bal : ~bal;
    }
    const int rank = __popcll(m & lt);
    // every lane reads the cursor of its id before the group's leader (rank 0)
    // advances it: one wavefront's LDS instructions execute in program order
    const int cur = valid ? whist[wave][e] : 0;
    if (valid) o.perm[cur + rank] = p;
    if (o.inv && p < hi) o.inv[p] = valid ? cur + rank : -1;
    if (valid && rank == 0) whist[wave][e] = cur + __popcll(m);
  }
  if (g != 0) return;
  for (int e = tid; e < E; e += kPermThreads) {
    o.counts[e] = start[e + 1] - start[e];
    o.offsets[e] = start[e];
  }
  if (tid == 0) o.offsets[E] = start[E];
  for (int p = start[E] + tid; p < S; p += kPermThreads) o.perm[p] = -1;
  if (o.tile_e == nullptr) return;
  // work items: expert e owns ceil(count_e / kItemRows) consecutive items
  __syncthreads();
  if (tid < E) mine[tid] = (start[tid + 1] - start[tid] + kItemRows - 1) / kItemRows;  // reused: items of e
  __syncthreads();
  block_exclusive_scan(mine, E, wsum);  // first item of each expert; mine[E] = total
  if (tid == 0) *o.ntile = mine[E];
  for (int e = tid; e < E; e += kPermThreads) {
    const int n = (start[e + 1] - start[e] + kItemRows - 1) / kItemRows;
    for (int j = 0; j < n; ++j) {
      o.tile_e[mine[e] + j] = e;
      o.tile_j[mine[e] + j] = j;
    }
  }
}

static hipError_t permute_impl(const Shape& s, const int32_t* ids, int M, int32_t* ghist, int32_t* err,
                               const PermOut& o, hipStream_t st) {
  const int S = M * s.k;
  const int G = perm_groups(S);
  if (G < 1) return hipSuccess;
  hipLaunchKernelGGL(k_perm_count, dim3(G), dim3(kPermThreads), 0, st, ids, S, s.E, ghist, err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_perm_scatter, dim3(G), dim3(kPermThreads), 0, st, ids, S, s.E, ghist, o);
  return hipGetLastError();
}

hipError_t launch_permute(const Shape& s, const int32_t* ids, int M, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* ghist, int32_t* err, hipStream_t st) {
  PermOut o{counts, offsets, perm, nullptr, nullptr, nullptr, nullptr};
  return permute_impl(s, ids, M, ghist, err, o, st);
}

hipError_t launch_permute_items(const Shape& s, const int32_t* ids, int M, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* tile_e, int32_t* tile_j, int32_t* ntile,
                                int32_t* ghist, int32_t* err, hipStream_t st) {
  PermOut o{counts, offsets, perm, inv, tile_e, tile_j, ntile};
  return permute_impl(s, ids, M, ghist, err, o, st);
}

}  // namespace moe
