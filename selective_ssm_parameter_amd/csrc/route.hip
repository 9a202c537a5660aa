// Router and top-k active set (papernotes.org notes on "Swimba: Switch Mamba
// Model Scales State Space Models", Method, key design 1: pi_t = softmax(g_t)
// with a top-k sparse active set; gist.science English summary, Technical
// Summary section 2, Expert Routing).
//
// One workgroup routes 64 tokens (16 when there are few tokens, as in
// decode, so that more workgroups share the work). Wave w computes the logits
// of tokens [16w, 16w + 16) against every expert with 16x16 matrix-core tiles
// (a workgroup with fewer tokens splits d_model over its waves instead): the A
// operand is the token rows of u, the B operand the router rows (both are
// contiguous along d_model, so every lane loads 16 bytes). Products of bf16
// values are exact in fp32 and accumulate in fp32, so the logits are never
// rounded to bf16. The logits go through LDS; a group of lanes per token then
// picks the top-k (strictly greater wins, so equal logits keep the lower
// index) and evaluates the softmax over all E experts in fp32.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

__device__ void route_tokens(const float* lg, int ldl, int tok0, int tpw, int M, int E, int k,
                             int32_t* __restrict__ idx, float* __restrict__ wout,
                             float* __restrict__ logits, int* hcnt);

// GT: expert tiles per pass (1, 2 or 4; tiles past E read zeros). The K loop
// issues the loads of RB steps together (A rows and every tile's router rows)
// before their matrix-core ops, so a wave waits for memory once per batch
// rather than once per load (8 steps of 2-byte data, 4 of fp32).

template <typename T, int GT, int NW>
__global__ __launch_bounds__(64 * NW) void route_kernel(const T* __restrict__ u,
                                                    const T* __restrict__ wr, int M, int D,
                                                    int E, int k, int32_t* __restrict__ idx,
                                                    float* __restrict__ wout,
                                                    float* __restrict__ logits,
                                                    int32_t* __restrict__ hist, int tpw,
                                                    int ksplit) {
  extern __shared__ float lg[];  // [ksplit][tpw][E + 1] partial logits
  typedef typename Vec<T>::x8 F;
  constexpr int RB = sizeof(T) == 2 ? 8 : 4;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tok0 = blockIdx.x * tpw;
  const int ET = (E + 15) / 16;
  const int ldl = E + 1;
  // Waves over (token tile, K slice): with few tokens per workgroup d_model
  // is split over the waves that would otherwise be idle (ksplit * ntt <=
  // the workgroup's waves).
  const int ntt = tpw / 16;
  const int tt = wave % ntt, ks = wave / ntt;
  const int nsteps = D / 32;
  const int s0 = ks * nsteps / ksplit, s1 = (ks + 1) * nsteps / ksplit;

  const int row = tok0 + tt * 16 + c;
  constexpr uint32_t ES = sizeof(T);
  // Out-of-range rows (tokens beyond M, experts beyond E, d past the slice)
  // read zeros.
  const BufRes ru = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rw = make_rsrc(wr, (uint64_t)E * D * ES);
  const uint32_t uoff = row < M ? ((uint32_t)row * D + 8 * g) * ES : kOOB;
  float* mylg = lg + (size_t)ks * tpw * ldl;

  if (ks < ksplit && tt < ntt) {
    for (int et0 = 0; et0 < ET; et0 += GT) {
      floatx4 acc[GT];
#pragma unroll
      for (int i = 0; i < GT; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      uint32_t woff[GT];
#pragma unroll
      for (int i = 0; i < GT; ++i) {
        const int e = (et0 + i) * 16 + c;
        woff[i] = e < E ? ((uint32_t)e * D + 8 * g) * ES : kOOB;
      }
      for (int st0 = s0; st0 < s1; st0 += RB) {
        F a[RB], b[RB][GT];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          const bool ok = st0 + q < s1;
          const uint32_t k0 = 32u * (st0 + q) * ES;
          a[q] = load8_buf<T>(ru, (ok && uoff != kOOB) ? uoff + k0 : kOOB);
#pragma unroll
          for (int i = 0; i < GT; ++i)
            b[q][i] = load8_buf<T>(rw, (ok && woff[i] != kOOB) ? woff[i] + k0 : kOOB);
        }
        __builtin_amdgcn_sched_barrier(0);  // all of the batch's loads before its first use
#pragma unroll
        for (int q = 0; q < RB; ++q)
#pragma unroll
          for (int i = 0; i < GT; ++i) acc[i] = mma16(a[q], b[q][i], acc[i]);
      }
      // acc[i][q] = partial logit of token (16 tt + 4g + q) for expert (16 (et0+i) + c)
#pragma unroll
      for (int i = 0; i < GT; ++i) {
        const int e = (et0 + i) * 16 + c;
        if (e < E) {
#pragma unroll
          for (int q = 0; q < 4; ++q) mylg[(tt * 16 + 4 * g + q) * ldl + e] = acc[i][q];
        }
      }
    }
  }
  __syncthreads();
  // sum the K slices in slice order (deterministic)
  if (ksplit > 1) {
    for (int q = threadIdx.x; q < ntt * 16 * ldl; q += blockDim.x) {
      float sacc = lg[q];
      for (int j = 1; j < ksplit; ++j) sacc += lg[(size_t)j * tpw * ldl + q];
      lg[q] = sacc;
    }
    __syncthreads();
  }

  int* hcnt = reinterpret_cast<int*>(lg + (size_t)ksplit * tpw * ldl);  // [E + 1]
  if (hist) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) hcnt[e] = 0;
    __syncthreads();
  }
  route_tokens(lg, ldl, tok0, tpw, M, E, k, idx, wout, logits, hist ? hcnt : nullptr);
  if (hist) {
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) hist[(size_t)blockIdx.x * (E + 1) + e] = hcnt[e];
  }
}

// Prefill-sized batches: a workgroup routes 64 tokens with 4 waves that split
// d_model four ways, every wave computing all 64 tokens (four token tiles)
// against GT expert tiles for its quarter of d_model, so each router-row
// fragment serves four token tiles (with 16 tokens per wave over all of
// d_model, every wave read all of W_r: at E = 64 and d_model 2048, four times
// the bytes of u). The partial logits are summed in LDS in slice order. The
// loads of RB K steps are issued together before their matrix-core ops.
template <typename T, int GT, int RB>
__global__ __launch_bounds__(256) void route_big_kernel(const T* __restrict__ u,
                                                        const T* __restrict__ wr, int M, int D,
                                                        int E, int k, int32_t* __restrict__ idx,
                                                        float* __restrict__ wout,
                                                        float* __restrict__ logits) {
  constexpr int TPW = 64, TM = 4, KS = 4;
  extern __shared__ float lg[];  // [KS][TPW][E + 1] partial logits
  typedef typename Vec<T>::x8 F;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tok0 = blockIdx.x * TPW;
  const int ET = (E + 15) / 16;
  const int ldl = E + 1;
  const int nsteps = D / 32;
  const int s0 = wave * nsteps / KS, s1 = (wave + 1) * nsteps / KS;
  constexpr uint32_t ES = sizeof(T);
  const BufRes ru = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rw = make_rsrc(wr, (uint64_t)E * D * ES);
  float* mylg = lg + (size_t)wave * TPW * ldl;
  uint32_t uoff[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = tok0 + i * 16 + c;
    uoff[i] = row < M ? ((uint32_t)row * D + 8 * g) * ES : kOOB;
  }
  for (int et0 = 0; et0 < ET; et0 += GT) {
    floatx4 acc[TM][GT];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < GT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint32_t woff[GT];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      const int e = (et0 + j) * 16 + c;
      woff[j] = e < E ? ((uint32_t)e * D + 8 * g) * ES : kOOB;
    }
    for (int st0 = s0; st0 < s1; st0 += RB) {
      F a[RB][TM], b[RB][GT];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const bool ok = st0 + q < s1;
        const uint32_t k0 = 32u * (st0 + q) * ES;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          a[q][i] = load8_buf<T>(ru, (ok && uoff[i] != kOOB) ? uoff[i] + k0 : kOOB);
#pragma unroll
        for (int j = 0; j < GT; ++j)
          b[q][j] = load8_buf<T>(rw, (ok && woff[j] != kOOB) ? woff[j] + k0 : kOOB);
      }
      __builtin_amdgcn_sched_barrier(0);  // all of the batch's loads before its first use
#pragma unroll
      for (int q = 0; q < RB; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < GT; ++j) acc[i][j] = mma16(a[q][i], b[q][j], acc[i][j]);
    }
    // acc[i][j][q] = partial logit of token 16 i + 4g + q for expert 16 (et0 + j) + c
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < GT; ++j) {
        const int e = (et0 + j) * 16 + c;
        if (e < E) {
#pragma unroll
          for (int q = 0; q < 4; ++q) mylg[(i * 16 + 4 * g + q) * ldl + e] = acc[i][j][q];
        }
      }
  }
  __syncthreads();
  // the slices' partial logits summed in slice order (deterministic)
  for (int q = threadIdx.x; q < TPW * ldl; q += blockDim.x) {
    float sacc = lg[q];
#pragma unroll
    for (int j = 1; j < KS; ++j) sacc += lg[(size_t)j * TPW * ldl + q];
    lg[q] = sacc;
  }
  __syncthreads();
  route_tokens(lg, ldl, tok0, TPW, M, E, k, idx, wout, logits, nullptr);
}

// Top-k and softmax of the workgroup's tokens from their logits in LDS. A
// group of sg lanes (a power of two with E <= 4 sg) shares a token: lane sl
// holds experts sl, sl + sg, sl + 2 sg, sl + 3 sg. Each of the k rounds takes
// the group's maximum over the experts not yet chosen (equal logits: the lower
// expert index wins), so the choice is exactly that of a sequential scan; the
// softmax denominator is summed over the group in a fixed butterfly order.
__device__ void route_tokens(const float* lg, int ldl, int tok0, int tpw, int M, int E, int k,
                             int32_t* __restrict__ idx, float* __restrict__ wout,
                             float* __restrict__ logits, int* hcnt) {
  constexpr int kNone = 0x7fffffff;
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int sg = 1;
  while (4 * sg < E) sg *= 2;
  const int per_wave = 64 / sg;
  const int sub = lane / sg, sl = lane % sg;
  for (int t0 = wave * per_wave; t0 < tpw; t0 += nw * per_wave) {
    const int t = t0 + sub;
    const int m = tok0 + t;
    const bool valid = t < tpw && m < M;
    const float* l = lg + (valid ? t : 0) * ldl;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = sl + sg * j;
      v[j] = (valid && e < E) ? l[e] : -INFINITY;
      if (logits && valid && e < E) logits[(size_t)m * E + e] = v[j];
    }
    int taken = 0;
    // the group's best expert not yet taken: (value, index), ties to the lower index
    auto best = [&](float& bv, int& be) {
      bv = -INFINITY;
      be = kNone;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = sl + sg * j;
        if (!((taken >> j) & 1) && e < E && (be == kNone || v[j] > bv)) {
          bv = v[j];
          be = e;
        }
      }
      for (int off = sg >> 1; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, sg);
        const int oe = __shfl_xor(be, off, sg);
        if (oe != kNone && (be == kNone || ov > bv || (ov == bv && oe < be))) {
          bv = ov;
          be = oe;
        }
      }
      if (be != kNone && be % sg == sl) taken |= 1 << (be / sg);
    };
    float bv;
    int be;
    best(bv, be);
    const float mx = bv;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sl + sg * j < E) sum += expf(v[j] - mx);
    for (int off = sg >> 1; off > 0; off >>= 1) sum += __shfl_xor(sum, off, sg);
    const float inv = 1.f / sum;
    for (int j = 0; j < k; ++j) {
      if (j > 0) best(bv, be);
      if (valid && sl == 0) {
        idx[(size_t)m * k + j] = be;
        wout[(size_t)m * k + j] = expf(bv - mx) * inv;
        if (hcnt) atomicAdd(&hcnt[be], 1);
      }
    }
  }
}

hipError_t launch_route(bool is_bf16, const void* u, const void* w_router, int M, int D, int E, int k,
                        int32_t* idx, float* w, float* logits, hipStream_t s, int32_t* hist) {
  if (M == 0) return hipSuccess;
  if (!hist && M > 1024 && E <= 64) {
    // prefill: 64 tokens per workgroup, d_model split over the 4 waves
    const size_t lds = (size_t)4 * 64 * (E + 1) * sizeof(float);
    const dim3 grid((M + 63) / 64);
    const int ET = (E + 15) / 16;
    const void* fn;
    if (is_bf16)
      fn = ET > 2 ? (const void*)route_big_kernel<bf16, 4, 2>
                  : (ET > 1 ? (const void*)route_big_kernel<bf16, 2, 2>
                            : (const void*)route_big_kernel<bf16, 1, 2>);
    else
      fn = ET > 2 ? (const void*)route_big_kernel<float, 4, 1>
                  : (ET > 1 ? (const void*)route_big_kernel<float, 2, 1>
                            : (const void*)route_big_kernel<float, 1, 1>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    prof_begin("route_topk", s);
#define SWIMBA_ROUTE_BIG(TT, G, RBQ)                                                           \
  hipLaunchKernelGGL((route_big_kernel<TT, G, RBQ>), grid, dim3(256), lds, s, (const TT*)u,   \
                     (const TT*)w_router, M, D, E, k, idx, w, logits)
    if (is_bf16) {
      if (ET > 2) SWIMBA_ROUTE_BIG(bf16, 4, 2);
      else if (ET > 1) SWIMBA_ROUTE_BIG(bf16, 2, 2);
      else SWIMBA_ROUTE_BIG(bf16, 1, 2);
    } else {
      if (ET > 2) SWIMBA_ROUTE_BIG(float, 4, 1);
      else if (ET > 1) SWIMBA_ROUTE_BIG(float, 2, 1);
      else SWIMBA_ROUTE_BIG(float, 1, 1);
    }
#undef SWIMBA_ROUTE_BIG
    prof_end(s);
    return hipGetLastError();
  }
  const int tpw = route_tokens_per_wg(M);
  const int ET = (E + 15) / 16;
  const int GT = ET >= 4 ? 4 : (ET >= 2 ? 2 : 1);
  // Decode-sized batches (16 tokens per workgroup, up to 32 experts): 16
  // waves, d_model split 16 ways, so each wave's slice of the K loop is one
  // batch of reads; otherwise 4 waves. The split shrinks while the partial
  // logits would not fit 64 KiB of LDS.
  const bool wide = tpw == 16 && GT <= 2;
  const int nwaves = wide ? 16 : 4;
  dim3 grid((M + tpw - 1) / tpw), block(64 * nwaves);
  int ksplit = nwaves / (tpw / 16);
  while (ksplit > 1 && (size_t)ksplit * tpw * (E + 1) * sizeof(float) > 65536) ksplit /= 2;
  size_t lds = (size_t)ksplit * tpw * (E + 1) * sizeof(float) + (size_t)(E + 1) * sizeof(int);
  const void* fn;
#define SWIMBA_ROUTE_FN(TT)                                                                     \
  (wide ? (GT == 2 ? (const void*)route_kernel<TT, 2, 16> : (const void*)route_kernel<TT, 1, 16>) \
        : (GT == 4 ? (const void*)route_kernel<TT, 4, 4>                                         \
                   : (GT == 2 ? (const void*)route_kernel<TT, 2, 4> : (const void*)route_kernel<TT, 1, 4>)))
  if (is_bf16) fn = SWIMBA_ROUTE_FN(bf16);
  else fn = SWIMBA_ROUTE_FN(float);
#undef SWIMBA_ROUTE_FN
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  prof_begin("route_topk", s);
#define SWIMBA_ROUTE(TT, G, W)                                                                  \
  hipLaunchKernelGGL((route_kernel<TT, G, W>), grid, block, lds, s, (const TT*)u,              \
                     (const TT*)w_router, M, D, E, k, idx, w, logits, hist, tpw, ksplit)
#define SWIMBA_ROUTE_T(TT)                       \
  if (wide) {                                    \
    if (GT == 2) SWIMBA_ROUTE(TT, 2, 16);        \
    else SWIMBA_ROUTE(TT, 1, 16);                \
  } else if (GT == 4) SWIMBA_ROUTE(TT, 4, 4);    \
  else if (GT == 2) SWIMBA_ROUTE(TT, 2, 4);      \
  else SWIMBA_ROUTE(TT, 1, 4);
  if (is_bf16) {
    SWIMBA_ROUTE_T(bf16)
  } else {
    SWIMBA_ROUTE_T(float)
  }
#undef SWIMBA_ROUTE_T
#undef SWIMBA_ROUTE
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
