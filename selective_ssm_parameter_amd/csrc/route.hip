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
// rounded to bf16. The logits go through LDS; one thread per token then picks
// the top-k (strictly greater wins, so equal logits keep the lower index) and
// evaluates the softmax over all E experts in fp32.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

__device__ void route_token(const float* l, int m, int E, int k, int32_t* __restrict__ idx,
                            float* __restrict__ wout, float* __restrict__ logits, int* hcnt);

template <typename T>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ u,
                                                    const T* __restrict__ wr, int M, int D,
                                                    int E, int k, int32_t* __restrict__ idx,
                                                    float* __restrict__ wout,
                                                    float* __restrict__ logits,
                                                    int32_t* __restrict__ hist, int tpw,
                                                    int ksplit) {
  extern __shared__ float lg[];  // [ksplit][tpw][E + 1] partial logits
  typedef typename Vec<T>::x8 F;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tok0 = blockIdx.x * tpw;
  const int ET = (E + 15) / 16;
  const int ldl = E + 1;
  // Waves over (token tile, K slice): with few tokens per workgroup d_model
  // is split over the waves that would otherwise be idle (ksplit * ntt <= 4).
  const int ntt = tpw / 16;
  const int tt = wave % ntt, ks = wave / ntt;
  const int nsteps = D / 32;
  const int s0 = ks * nsteps / ksplit, s1 = (ks + 1) * nsteps / ksplit;

  const int row = tok0 + tt * 16 + c;
  constexpr uint32_t ES = sizeof(T);
  // Out-of-range rows (tokens beyond M, experts beyond E) read zeros.
  const BufRes ru = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rw = make_rsrc(wr, (uint64_t)E * D * ES);
  const uint32_t uoff = row < M ? ((uint32_t)row * D + 8 * g) * ES : kOOB;
  float* mylg = lg + (size_t)ks * tpw * ldl;

  // Expert tiles are processed 4 at a time (16 accumulators per lane); the K
  // loop is unrolled so several steps' loads are in flight together.
  if (ks < ksplit && tt < ntt) {
    for (int et0 = 0; et0 < ET; et0 += 4) {
      floatx4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      uint32_t woff[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (et0 + i) * 16 + c;
        woff[i] = (et0 + i < ET && e < E) ? ((uint32_t)e * D + 8 * g) * ES : kOOB;
      }
#pragma unroll 4
      for (int st = s0; st < s1; ++st) {
        const int k0 = 32 * st;
        const F a = load8_buf<T>(ru, uoff == kOOB ? kOOB : uoff + k0 * ES);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (et0 + i < ET) {
            const F b = load8_buf<T>(rw, woff[i] == kOOB ? kOOB : woff[i] + k0 * ES);
            acc[i] = mma16(a, b, acc[i]);
          }
        }
      }
      // acc[i][q] = partial logit of token (16 tt + 4g + q) for expert (16 (et0+i) + c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (et0 + i) * 16 + c;
        if (et0 + i < ET && e < E) {
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
  const int t = threadIdx.x;
  if (t < tpw && tok0 + t < M) route_token(lg + t * ldl, tok0 + t, E, k, idx, wout, logits,
                                                 hist ? hcnt : nullptr);
  if (hist) {
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) hist[(size_t)blockIdx.x * (E + 1) + e] = hcnt[e];
  }
}

// Top-k and softmax of one token from its logits in LDS.
__device__ void route_token(const float* l, int m, int E, int k, int32_t* __restrict__ idx,
                            float* __restrict__ wout, float* __restrict__ logits, int* hcnt) {
  if (logits) {
    for (int e = 0; e < E; ++e) logits[(size_t)m * E + e] = l[e];
  }
  int chosen[8];
  for (int j = 0; j < k; ++j) {
    int bi = -1;
    float best = 0.f;
    for (int e = 0; e < E; ++e) {
      bool taken = false;
      for (int q = 0; q < j; ++q) taken |= (chosen[q] == e);
      if (taken) continue;
      if (bi < 0 || l[e] > best) {
        bi = e;
        best = l[e];
      }
    }
    chosen[j] = bi;
  }
  const float mx = l[chosen[0]];
  float sum = 0.f;
  for (int e = 0; e < E; ++e) sum += expf(l[e] - mx);
  const float inv = 1.f / sum;
  for (int j = 0; j < k; ++j) {
    idx[(size_t)m * k + j] = chosen[j];
    wout[(size_t)m * k + j] = expf(l[chosen[j]] - mx) * inv;
    if (hcnt) atomicAdd(&hcnt[chosen[j]], 1);
  }
}

hipError_t launch_route(bool is_bf16, const void* u, const void* w_router, int M, int D, int E, int k,
                        int32_t* idx, float* w, float* logits, hipStream_t s, int32_t* hist) {
  if (M == 0) return hipSuccess;
  const int tpw = route_tokens_per_wg(M);
  dim3 grid((M + tpw - 1) / tpw), block(256);
  // 16 (32) tokens per workgroup: d_model split 4 (2) ways over the waves, as
  // long as the partial logits fit 64 KiB of LDS
  int ksplit = 64 / tpw;
  while (ksplit > 1 && (size_t)ksplit * tpw * (E + 1) * sizeof(float) > 65536) ksplit /= 2;
  size_t lds = (size_t)ksplit * tpw * (E + 1) * sizeof(float) + (size_t)(E + 1) * sizeof(int);
  hipError_t err = hipFuncSetAttribute(
      is_bf16 ? (const void*)route_kernel<bf16> : (const void*)route_kernel<float>,
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  prof_begin("route_topk", s);
  if (is_bf16)
    hipLaunchKernelGGL(route_kernel<bf16>, grid, block, lds, s, (const bf16*)u,
                       (const bf16*)w_router, M, D, E, k, idx, w, logits, hist, tpw, ksplit);
  else
    hipLaunchKernelGGL(route_kernel<float>, grid, block, lds, s, (const float*)u,
                       (const float*)w_router, M, D, E, k, idx, w, logits, hist, tpw, ksplit);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
