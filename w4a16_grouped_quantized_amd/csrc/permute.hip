// permute.hip — stable counting sort of the M*k (token, slot) pairs by
// expert id, in one workgroup of 16 wavefronts.
//
// Wavefront w owns a contiguous segment of pairs.  Pass 1 counts its
// segment per expert (LDS histogram [16][E]); a scan turns the histogram into
// per-(expert, wavefront) write bases; pass 2 walks each segment again in
// order, 64 pairs at a time, and ranks equal ids inside the 64 with ballots
// over the id bits, so the output is grouped by expert and ascending in pair
// index inside each expert — bit-identical on every run.
#include "launch.hpp"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ ids, int S, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ err) {
  __shared__ int hist[kPermWaves][kMaxExperts];
  __shared__ int scan[kMaxExperts + 1];
  __shared__ int bad;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermThreads) (&hist[0][0])[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int seg = (S + kPermWaves - 1) / kPermWaves;
  const int lo = wave * seg, hi = min(S, lo + seg);
  for (int p = lo + lane; p < hi; p += kWave) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[wave][e], 1);
    else atomicAdd(&bad, 1);
  }
  __syncthreads();
  // per-expert totals and per-(wave, expert) exclusive bases
  for (int e = tid; e < E; e += kPermThreads) {
    int c = 0;
    for (int w = 0; w < kPermWaves; ++w) c += hist[w][e];
    scan[e] = c;
  }
  __syncthreads();
  if (tid == 0) {  // E <= 512: a serial scan is a few hundred cycles
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = scan[e];
      scan[e] = run;
      run += c;
    }
    scan[E] = run;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    int run = scan[e];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = lo; base < hi; base += kWave) {
    const int p = base + lane;
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
    const int cur = valid ? hist[wave][e] : 0;
    if (valid) perm[cur + rank] = p;
    if (valid && rank == 0) hist[wave][e] = cur + __popcll(m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    counts[e] = scan[e + 1] - scan[e];
    offsets[e] = scan[e];
  }
  if (tid == 0) {
    offsets[E] = scan[E];
    if (bad) atomicOr(err, 1);
  }
  for (int p = scan[E] + tid; p < S; p += kPermThreads) perm[p] = -1;
}

hipError_t launch_permute(const Shape& s, const int32_t* ids, int M, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, st, ids, M * s.k, s.E, counts, offsets, perm, err);
  return hipGetLastError();
}

}  // namespace moe
