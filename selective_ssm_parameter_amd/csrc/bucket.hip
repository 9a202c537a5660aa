// Expert bucketing of (token, slot) pairs: the sparse active sets K_t of the
// router (papernotes.org notes, Method, key design 1) turned into one
// contiguous row list per expert, so that the projection can run as a grouped
// GEMM over active pairs only.
//
// Three launches, all integer work and all deterministic:
//   count   - per block of 1024 pairs, a histogram over E experts plus one
//             extra bucket for out-of-range indices (LDS integer atomics:
//             the counts do not depend on their order);
//   scan    - one workgroup: expert offsets, per-block bases, and the number
//             of BM-row tiles per expert with their prefix (the GEMM's tile
//             schedule);
//   scatter - per block, the stable rank of every pair among the block's
//             pairs of the same expert (wave ballots, then wave order), so
//             every expert's list is sorted by pair id m*k + j. A pair whose
//             expert index is out of range gets zero outputs here.
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

// offsets[0..E+1]: start of each bucket (bucket E = invalid pairs) and the end.
// tile_offsets[0..E]: prefix of ceil(count_e / bm) over real experts.
__global__ __launch_bounds__(256) void bucket_scan_kernel(const int32_t* __restrict__ counts,
                                                          int nblk, int E, int bm,
                                                          int32_t* __restrict__ bases,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_offsets) {
  extern __shared__ int tot[];  // [E + 1]
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int s = 0;
    for (int b = 0; b < nblk; ++b) s += counts[(size_t)b * (E + 1) + e];
    tot[e] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0, tiles = 0;
    for (int e = 0; e <= E; ++e) {
      offsets[e] = run;
      if (e < E) {
        tile_offsets[e] = tiles;
        tiles += (tot[e] + bm - 1) / bm;
      }
      run += tot[e];
    }
    offsets[E + 1] = run;
    tile_offsets[E] = tiles;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int run = offsets[e];
    for (int b = 0; b < nblk; ++b) {
      bases[(size_t)b * (E + 1) + e] = run;
      run += counts[(size_t)b * (E + 1) + e];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ idx,
                                                             int pairs, int E,
                                                             const int32_t* __restrict__ bases,
                                                             int32_t* __restrict__ sorted,
                                                             T* __restrict__ X_hat, int HP,
                                                             T* __restrict__ B_hat, int GN,
                                                             float* __restrict__ c_part) {
  extern __shared__ int sh[];
  int* run = sh;                // [E + 1] running count of this block per bucket
  int* wcnt = sh + (E + 1);     // [4][E + 1] per-wave counts of the current round
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) run[e] = 0;
  for (int e = threadIdx.x; e < 4 * (E + 1); e += blockDim.x) wcnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kBucketPairs;
  for (int r0 = 0; r0 < kBucketPairs; r0 += 256) {
    const int p = p0 + r0 + threadIdx.x;
    const bool ok = p < pairs;
    const int b = ok ? bucket_of(idx[p], E) : -1;
    // Rank among earlier lanes of this wave with the same bucket.
    int rank = 0;
    uint64_t todo = __ballot(ok);
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int lb = __shfl(b, leader);
      const uint64_t same = __ballot(ok && b == lb);
      if (ok && b == lb) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        rank = __popcll(same & below);
      }
      if (lane == leader) wcnt[wave * (E + 1) + lb] = __popcll(same);
      todo &= ~same;
    }
    __syncthreads();
    if (ok) {
      int pos = bases[(size_t)blockIdx.x * (E + 1) + b] + run[b] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w * (E + 1) + b];
      sorted[pos] = p;
      if (b == E) {
        // An out-of-range expert index: this slot contributes nothing.
        for (int i = 0; i < HP; ++i) X_hat[(size_t)p * HP + i] = from_f32<T>(0.f);
        for (int i = 0; i < GN; ++i) {
          B_hat[(size_t)p * GN + i] = from_f32<T>(0.f);
          c_part[(size_t)p * GN + i] = 0.f;
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      run[e] += wcnt[e] + wcnt[(E + 1) + e] + wcnt[2 * (E + 1) + e] + wcnt[3 * (E + 1) + e];
      wcnt[e] = wcnt[(E + 1) + e] = wcnt[2 * (E + 1) + e] = wcnt[3 * (E + 1) + e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_bucket(bool is_bf16, const int32_t* idx, int pairs, int E, int bm,
                         int32_t* counts, int32_t* bases, int32_t* offsets, int32_t* tile_offsets,
                         int32_t* sorted, void* X_hat, int HP, void* B_hat, int GN,
                         float* c_part, hipStream_t s) {
  const int nblk = bucket_blocks(pairs);
  const size_t hl = (size_t)(E + 1) * sizeof(int);
  if (nblk > 0) {
    prof_begin("bucket_count", s);
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nblk), dim3(256), hl, s, idx, pairs, E, counts);
    prof_end(s);
  }
  prof_begin("bucket_scan", s);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(256), hl, s, counts, nblk, E, bm, bases,
                     offsets, tile_offsets);
  prof_end(s);
  if (nblk > 0) {
    prof_begin("bucket_scatter", s);
    if (is_bf16)
      hipLaunchKernelGGL(bucket_scatter_kernel<f16>, dim3(nblk), dim3(256), 5 * hl, s, idx,
                         pairs, E, bases, sorted, (f16*)X_hat, HP, (f16*)B_hat, GN, c_part);
    else
      hipLaunchKernelGGL(bucket_scatter_kernel<float>, dim3(nblk), dim3(256), 5 * hl, s, idx,
                         pairs, E, bases, sorted, (float*)X_hat, HP, (float*)B_hat, GN, c_part);
    prof_end(s);
  }
  return hipGetLastError();
}

}  // namespace swimba
