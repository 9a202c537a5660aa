// Expert bucketing of (token, slot) pairs: the sparse active sets K_t of the
// router (papernotes.org notes, Method, key design 1) turned into one
// contiguous row list per expert, so that the projection can run as a grouped
// GEMM over active pairs only.
//
// Two launches, all integer work and all deterministic:
//   count - per block of pairs, a histogram over E experts plus one extra
//           bucket for out-of-range indices (LDS integer atomics: the counts
//           do not depend on their order). The decode path gets these from
//           the router instead.
//   place - per block: bucket starts and earlier blocks' counts from the
//           histograms, then the stable rank of every pair among the block's
//           pairs of the same expert (wave ballots, then wave order), so
//           every expert's list is sorted by pair id m*k + j. Block 0 also
//           writes the GEMM's tile schedule. A pair whose expert index is out
//           of range gets zero outputs here.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

int bucket_blocks(int pairs) { return (pairs + kBucketPairs - 1) / kBucketPairs; }

__device__ __forceinline__ int bucket_of(int e, int E) { return (e >= 0 && e < E) ? e : E; }

__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t* __restrict__ idx,
                                                           int pairs, int E,
                                                           int32_t* __restrict__ counts) {
  extern __shared__ int hist[];  // [E + 1]
  for (int e = threadIdx.x; e <= E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kBucketPairs;
  for (int i = threadIdx.x; i < kBucketPairs; i += blockDim.x) {
    const int p = p0 + i;
    if (p < pairs) atomicAdd(&hist[bucket_of(idx[p], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x)
    counts[(size_t)blockIdx.x * (E + 1) + e] = hist[e];
}

// Merged scan + scatter. Every workgroup owns one block of `bp` pairs; it
// derives, from the per-block histograms, the start of every bucket (bucket E
// = out-of-range indices) and the number of pairs of each bucket in the
// blocks before its own, then places its pairs in stable order (pair id).
// Workgroup 0 also writes the bucket offsets and the GEMM tile schedule:
//   offsets[0..E+1]: start of each bucket and the end;
//   tile_info[t] = {expert, first sorted row, rows} for the row tiles of bm
//   pairs of every real expert in order, {-1, 0, 0} up to ntiles_max, and
//   tile_info[ntiles_max] = {number of real tiles, 0, 0, 0}.
// Next to each sorted pair id goes its top-k weight (sorted_w), so the GEMM
// reads a tile's rows with one round trip.
template <typename T>
__global__ __launch_bounds__(256) void bucket_place_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w, int pairs, int E, int bp,
    int nblk, const int32_t* __restrict__ counts, int bm, int ntiles_max,
    int32_t* __restrict__ offsets, int4v* __restrict__ tile_info, int32_t* __restrict__ sorted,
    float* __restrict__ sorted_w, T* __restrict__ X_hat, int HP, T* __restrict__ B_hat, int GN,
    float* __restrict__ c_part) {
  extern __shared__ int sh[];
  const int EP = E + 1;
  int* before = sh;            // [EP] pairs of each bucket in earlier blocks (then: running base)
  int* total = sh + EP;        // [EP]
  int* wcnt = sh + 2 * EP;     // [4][EP] per-wave counts of the current round
  int* scan = sh + 6 * EP;     // [256] scan scratch
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int blk = blockIdx.x;

  // ---- per-bucket sums over blocks, split over threads
  const int nparts = EP <= 256 ? 256 / EP : 1;
  for (int e = threadIdx.x; e < EP; e += blockDim.x) { before[e] = 0; total[e] = 0; }
  for (int e = threadIdx.x; e < 4 * EP; e += blockDim.x) wcnt[e] = 0;
  __syncthreads();
  // bucket e's counts of blocks b0, b0 + step, ...: loads issued kColumnLoads
  // at a time (a thread walks nblk / nparts blocks, more as E grows; one load
  // in flight at a time made this loop's latency grow with E)
  constexpr int kColumnLoads = 16;
  auto column = [&](int e, int b0, int step, int& sb, int& st) {
    for (int b = b0; b < nblk; b += kColumnLoads * step) {
      int v[kColumnLoads];
#pragma unroll
      for (int q = 0; q < kColumnLoads; ++q) {
        const int bq = b + q * step;
        v[q] = bq < nblk ? counts[(size_t)bq * EP + e] : 0;
      }
#pragma unroll
      for (int q = 0; q < kColumnLoads; ++q) {
        st += v[q];
        sb += b + q * step < blk ? v[q] : 0;
      }
    }
  };
  {
    const int part = threadIdx.x / EP, e = threadIdx.x % EP;
    if (part < nparts) {
      int sb = 0, st = 0;
      column(e, part, nparts, sb, st);
      atomicAdd(&before[e], sb);
      atomicAdd(&total[e], st);
    }
    if (EP > 256) {  // one thread per bucket when buckets outnumber threads
      for (int e2 = threadIdx.x; e2 < EP; e2 += blockDim.x) {
        if (e2 < 256) continue;
        int sb = 0, st = 0;
        column(e2, 0, 1, sb, st);
        before[e2] = sb;
        total[e2] = st;
      }
    }
  }
  __syncthreads();
  // ---- exclusive scan of the totals (one bucket per thread, EP <= 257)
  int tv = threadIdx.x < EP ? total[threadIdx.x] : 0;
  scan[threadIdx.x] = tv;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  const int excl = scan[threadIdx.x] - tv;
  const int last_total = EP > 256 ? total[256] : 0;  // E = 256: bucket 256 is the invalid one
  if (blk == 0) {
    if (threadIdx.x < EP) offsets[threadIdx.x] = excl;
    if (threadIdx.x == 0) {
      if (EP > 256) offsets[256] = scan[255];
      offsets[EP] = scan[255] + last_total;
    }
  }
  __syncthreads();
  if (threadIdx.x < EP) before[threadIdx.x] += excl;  // becomes the running base of this block
  if (EP > 256 && threadIdx.x == 0) before[256] += scan[255];
  __syncthreads();
  if (blk == 0) {
    // tile prefix over experts (scan scratch is free again), then each
    // expert's tiles written by its own thread
    __shared__ int tprefix[257];
    if (threadIdx.x == 0) {
      int tiles = 0;
      for (int e = 0; e < E; ++e) {
        tprefix[e] = tiles;
        tiles += (total[e] + bm - 1) / bm;
      }
      tprefix[E] = tiles;
    }
    __syncthreads();
    if (threadIdx.x < E) {  // E <= 256: thread e holds bucket e's start in excl
      const int e = threadIdx.x;
      const int nt = (total[e] + bm - 1) / bm;
      for (int j = 0; j < nt; ++j)
        tile_info[tprefix[e] + j] = int4v{e, excl + j * bm, min(bm, total[e] - j * bm), 0};
    }
    for (int t = tprefix[E] + threadIdx.x; t < ntiles_max; t += blockDim.x)
      tile_info[t] = int4v{-1, 0, 0, 0};
    if (threadIdx.x == 0) tile_info[ntiles_max] = int4v{tprefix[E], 0, 0, 0};
  }

  // ---- stable placement of this block's pairs
  const int p0 = blk * bp;
  for (int r0 = 0; r0 < bp; r0 += 256) {
    const int p = p0 + r0 + threadIdx.x;
    const bool ok = r0 + threadIdx.x < bp && p < pairs;
    const int bkt = ok ? bucket_of(idx[p], E) : -1;
    int rank = 0;
    uint64_t todo = __ballot(ok);
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int lb = __shfl(bkt, leader);
      const uint64_t same = __ballot(ok && bkt == lb);
      if (ok && bkt == lb) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        rank = __popcll(same & below);
      }
      if (lane == leader) wcnt[wave * EP + lb] = __popcll(same);
      todo &= ~same;
    }
    __syncthreads();
    if (ok) {
      int pos = before[bkt] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w * EP + bkt];
      sorted[pos] = p;
      sorted_w[pos] = topk_w[p];
      if (bkt == E) {
        // An out-of-range expert index: this slot contributes nothing.
        for (int i = 0; i < HP; ++i) X_hat[(size_t)p * HP + i] = from_f32<T>(0.f);
        for (int i = 0; i < GN; ++i) {
          B_hat[(size_t)p * GN + i] = from_f32<T>(0.f);
          c_part[(size_t)p * GN + i] = 0.f;
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < EP; e += blockDim.x) {
      before[e] += wcnt[e] + wcnt[EP + e] + wcnt[2 * EP + e] + wcnt[3 * EP + e];
      wcnt[e] = wcnt[EP + e] = wcnt[2 * EP + e] = wcnt[3 * EP + e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_bucket(bool is_bf16, const int32_t* idx, const float* topk_w, int pairs, int E,
                         int bm, int ntiles_max, int32_t* counts, int32_t* offsets,
                         int32_t* tile_info_i, int32_t* sorted, float* sorted_w, void* X_hat,
                         int HP, void* B_hat, int GN, float* c_part, hipStream_t s,
                         int block_pairs, bool counted) {
  int4v* tile_info = reinterpret_cast<int4v*>(tile_info_i);
  const int bp = block_pairs > 0 ? block_pairs : kBucketPairs;
  const int nblk = (pairs + bp - 1) / bp;
  const size_t hl = (size_t)(E + 1) * sizeof(int);
  if (nblk > 0 && !counted) {
    prof_begin("bucket_count", s);
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nblk), dim3(256), hl, s, idx, pairs, E, counts);
    prof_end(s);
  }
  const size_t pl = (size_t)(6 * (E + 1) + 256) * sizeof(int);
  prof_begin("bucket_place", s);
  const dim3 grid(nblk > 0 ? nblk : 1);
  if (is_bf16)
    hipLaunchKernelGGL(bucket_place_kernel<f16>, grid, dim3(256), pl, s, idx, topk_w, pairs, E, bp,
                       nblk, counts, bm, ntiles_max, offsets, tile_info, sorted, sorted_w,
                       (f16*)X_hat, HP, (f16*)B_hat, GN, c_part);
  else
    hipLaunchKernelGGL(bucket_place_kernel<float>, grid, dim3(256), pl, s, idx, topk_w, pairs, E,
                       bp, nblk, counts, bm, ntiles_max, offsets, tile_info, sorted, sorted_w,
                       (float*)X_hat, HP, (float*)B_hat, GN, c_part);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
