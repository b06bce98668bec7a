// Token -> expert permutation: a stable counting sort of the (token, slot)
// pairs by expert id, so that every expert's tokens are contiguous and each
// expert's weights are streamed once per layer (per-expert dispatch: page 3
// "The 'Doorbell' Mechanism").
//
// Stability (pairs of one expert in increasing pair index) comes from ranking
// each pair among the lanes of its wave with the same expert (ballots over the
// id bits) and walking a chunk of pairs in order with one wave.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kChunk = 1024;          // pairs per chunk in the multi-block path
constexpr int kSmallMaxPairs = 4096;  // single-wave path up to this many pairs

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Mask of the valid lanes of this wave holding the same id as this lane.
__device__ __forceinline__ uint64_t match_same(int e, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(valid && bit);
    same &= bit ? bal : ~bal;
  }
  return same;
}

__device__ __forceinline__ int id_bits(int E) {
  int nb = 0;
  while ((1 << nb) < E) ++nb;
  return nb;
}

// One wave scatters pairs [p0, p1) in order; running[e] holds the next free
// sorted position of expert e (LDS, owned by this wave).  The ids of 16
// rounds of 64 pairs are requested together, before the first round.  The
// caller is a one-wave block: the wave's LDS accesses complete in order, so a
// round's reads of running[] come before its update without a barrier (a block
// barrier would also wait for the round's global stores).
__device__ void scatter_chunk(const PermuteArgs& a, int* running, int p0, int p1, int lane, int nbits) {
  constexpr int kRounds = 16;
  for (int b0 = p0; b0 < p1; b0 += 64 * kRounds) {
    int ev[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int p = b0 + 64 * i + lane;
      ev[i] = p < p1 ? a.ids[p] : 0;
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int base = b0 + 64 * i;
      if (base >= p1) break;  // uniform
      const int p = base + lane;
      const bool valid = p < p1;
      const int e = ev[i];
      const uint64_t same = match_same(e, valid, nbits);
      const int rank = __popcll(same & lanemask_lt(lane));
      const int cnt = __popcll(same);
      int pos = 0;
      if (valid) pos = running[e] + rank;
      if (valid) {
        a.sorted_pairs[pos] = p;
        a.pair_pos[p] = pos;
        if (rank == 0) running[e] = pos + cnt;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Exclusive scan of v over one wave; returns the prefix, total in *tot.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* tot) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  *tot = __shfl(incl, 63, 64);
  return incl - v;
}

// Small path: one wave does histogram, scan and scatter.
__global__ __launch_bounds__(64) void k_perm_small(PermuteArgs a) {
  extern __shared__ int lds[];
  int* cnt = lds;  // [E]: counts, then running positions
  const int lane = threadIdx.x;
  const int n = a.T * a.K, E = a.E;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  // the ids of 16 rounds are requested together before their counts are
  // added (a load per round, waiting for each, costs a memory latency each)
  constexpr int kRounds = 16;
  for (int p0 = 0; p0 < n; p0 += 64 * kRounds) {
    int ev[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int p = p0 + 64 * i + lane;
      ev[i] = p < n ? a.ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
      if (ev[i] >= 0) atomicAdd(&cnt[ev[i]], 1);
  }
  __syncthreads();
  // lane owns experts [lane*per, (lane+1)*per)
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) sum += cnt[e];
  }
  int tot;
  int off = wave_excl_scan(sum, lane, &tot);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt[e];
      a.offsets[e] = off;
      cnt[e] = off;
      off += c;
    }
  }
  if (lane == 0) a.offsets[E] = tot;
  __syncthreads();
  scatter_chunk(a, cnt, 0, n, lane, id_bits(E));
}

// Up to kSmallMaxPairs pairs and E <= kBlockMaxE experts: one block of
// kBlockWaves waves, wave w taking the contiguous chunk [w cs, (w+1) cs) of
// the pairs (cs a multiple of 64).  Phase 1: each wave counts its chunk's ids
// into its own LDS row; phase 2: thread e turns expert e's counts into
// running sums over the waves in wave order, a block scan of the totals
// gives the expert offsets, and row w of expert e becomes the first sorted
// position of chunk w's pairs of e; phase 3: each wave scatters its chunk in
// order from its own row (scatter_chunk: a one-wave owner of its LDS row).
// Chunks in wave order and pairs in order within a chunk keep the sort stable.
constexpr int kBlockWaves = 16, kBlockMaxE = 512;

__global__ __launch_bounds__(64 * kBlockWaves) void k_perm_block(PermuteArgs a) {
  extern __shared__ int rows[];  // [kBlockWaves][E]
  __shared__ int wsum[kBlockWaves];
  const int E = a.E, n = a.T * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cs = (n + 64 * kBlockWaves - 1) / (64 * kBlockWaves) * 64;
  const int p0 = min(wave * cs, n), p1 = min(p0 + cs, n);
  for (int i = tid; i < kBlockWaves * E; i += 64 * kBlockWaves) rows[i] = 0;
  __syncthreads();
  int* row = rows + wave * E;
  // the chunk's ids (at most kSmallMaxPairs / kBlockWaves of them) requested
  // together before their counts are added
  constexpr int kRounds = kSmallMaxPairs / kBlockWaves / 64;
  int ev[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int p = p0 + 64 * i + lane;
    ev[i] = p < p1 ? a.ids[p] : -1;
  }
#pragma unroll
  for (int i = 0; i < kRounds; ++i)
    if (ev[i] >= 0) atomicAdd(&row[ev[i]], 1);
  __syncthreads();
  int total = 0;
  if (tid < E) {
    for (int w = 0; w < kBlockWaves; ++w) {
      const int c = rows[w * E + tid];
      rows[w * E + tid] = total;
      total += c;
    }
  }
  int wtot;
  const int pre = wave_excl_scan(total, lane, &wtot);
  if (lane == 0) wsum[wave] = wtot;
  __syncthreads();
  int off = pre;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  if (tid < E) {
    a.offsets[tid] = off;
    for (int w = 0; w < kBlockWaves; ++w) rows[w * E + tid] += off;
  }
  if (tid == 0) a.offsets[E] = n;
  __syncthreads();
  scatter_chunk(a, row, p0, p1, lane, id_bits(E));
}

// Multi-block path, phase 1: per-chunk histograms -> chunk_base[c][e].
__global__ __launch_bounds__(256) void k_perm_hist(PermuteArgs a) {
  extern __shared__ int hist[];
  const int E = a.E, n = a.T * a.K, c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int p0 = c * kChunk, p1 = min(n, p0 + kChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += 256) atomicAdd(&hist[a.ids[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) a.chunk_base[(size_t)c * E + e] = hist[e];
}

// Phase 2 (one block): per expert, the exclusive prefix over chunks; expert
// offsets from a block scan of the totals; finally
// chunk_base[c][e] <- first sorted position of chunk c's pairs of expert e.
__global__ __launch_bounds__(1024) void k_perm_scan(PermuteArgs a, int n_chunks) {
  __shared__ int part[1024];
  const int E = a.E, tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  // the chunk counts go through in batches of kBatch, all loaded before any is
  // stored, so that the loads of a batch are in flight together
  constexpr int kBatch = 32;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    int run = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < n_chunks ? a.chunk_base[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (c0 + j < n_chunks) {
          a.chunk_base[(size_t)(c0 + j) * E + e] = run;
          run += v[j];
        }
    }
    a.offsets[e] = run;  // count for now, rewritten below by this same thread
    sum += run;
  }
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int off = part[tid] - sum;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int cnt = a.offsets[e];
    a.offsets[e] = off;
    for (int c0 = 0; c0 < n_chunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < n_chunks ? a.chunk_base[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (c0 + j < n_chunks) a.chunk_base[(size_t)(c0 + j) * E + e] = v[j] + off;
    }
    off += cnt;
  }
  if (tid == 1023) a.offsets[E] = part[1023];
}

__global__ __launch_bounds__(64) void k_perm_scatter(PermuteArgs a) {
  extern __shared__ int running[];
  const int E = a.E, n = a.T * a.K, c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) running[e] = a.chunk_base[(size_t)c * E + e];
  __syncthreads();
  const int p0 = c * kChunk, p1 = min(n, p0 + kChunk);
  scatter_chunk(a, running, p0, p1, lane, id_bits(E));
}

size_t permute_scratch_ints(int T, int K, int E) {
  const size_t n = (size_t)T * K;
  if (n <= (size_t)kSmallMaxPairs) return 0;
  const size_t chunks = (n + kChunk - 1) / kChunk;
  return chunks * (size_t)E;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int n = a.T * a.K;
  if (n <= kSmallMaxPairs) {
    // a block of 16 waves from 4 rounds of pairs on; one wave below that, or
    // for more experts than the block's LDS rows hold
    if (n > 256 && a.E <= kBlockMaxE) k_perm_block<<<1, 64 * kBlockWaves, (size_t)kBlockWaves * a.E * 4, s>>>(a);
    else k_perm_small<<<1, 64, (size_t)a.E * 4, s>>>(a);
    return hipGetLastError();
  }
  const int chunks = (n + kChunk - 1) / kChunk;
  k_perm_hist<<<chunks, 256, (size_t)a.E * 4, s>>>(a);
  k_perm_scan<<<1, 1024, 0, s>>>(a, chunks);
  k_perm_scatter<<<chunks, 64, (size_t)a.E * 4, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
