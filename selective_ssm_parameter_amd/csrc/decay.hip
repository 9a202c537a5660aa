// Expert-mixed decay (papernotes.org notes on "Swimba: Switch Mamba Model
// Scales State Space Models", Limitations and outlook: the parameter-space mix
// extended to the diagonal of the transition, under the stability condition).
//
// For token t of sequence b and head h the decay is the convex mix over the
// token's selected experts, weights renormalised over the k slots (summed in
// slot order, fp32):
//     a_{t,h} = sum_j w_{t,j} a^(idx_{t,j})_h / sum_j w_{t,j}
// and the kernel writes what the chunked scan consumes: the inclusive running
// sum of log2 a within t's chunk of L tokens,
//     ld[b, h, t] = sum_{u = c0}^{t} max(log2 a_{u,h}, -126)
// (a zero decay is taken as 2^-126, which the scan's products carry as zero).
// An expert index outside [0, E) contributes decay 0 with its weight.
// One wave per (sequence, chunk, head): lane l owns PT = ceil(L / 64)
// consecutive tokens, sums them in order, and a wave-wide inclusive scan of
// the lane totals (fixed order, deterministic) supplies each lane's offset.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

template <int PT>
__global__ __launch_bounds__(256) void mix_decay_kernel(const int32_t* __restrict__ idx,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ a_experts,
                                                        float* __restrict__ ld, int T, int H,
                                                        int E, int k, int L) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  const int b = blockIdx.z;
  if (h >= H) return;
  const int c0 = blockIdx.x * L;
  const int Lc = min(L, T - c0);
  float v[PT];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int tl = lane * PT + i;
    float lv = 0.f;
    if (tl < Lc) {
      const size_t m = (size_t)b * T + c0 + tl;
      float num = 0.f, den = 0.f;
      for (int j = 0; j < k; ++j) {
        const float wj = w[m * k + j];
        const int e = idx[m * k + j];
        num += (e >= 0 && e < E) ? wj * a_experts[(size_t)e * H + h] : 0.f;
        den += wj;
      }
      lv = fmaxf(log2f(num / den), -126.f);
    }
    run += lv;
    v[i] = run;
  }
  float tot = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(tot, off);
    if (lane >= off) tot += o;
  }
  const float before = tot - run;  // sum over the lanes below this one
  float* out = ld + ((size_t)b * H + h) * T + c0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int tl = lane * PT + i;
    if (tl < Lc) out[tl] = v[i] + before;
  }
}

hipError_t launch_mix_decay(const int32_t* idx, const float* w, const float* a_experts,
                            float* ld, int Bt, int T, int H, int E, int k, int L,
                            hipStream_t s) {
  if (Bt == 0 || T == 0) return hipSuccess;
  if (L < 1 || L > 256) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + L - 1) / L), (unsigned)((H + 3) / 4), (unsigned)Bt);
  prof_begin("mix_decay", s);
  if (L <= 64)
    hipLaunchKernelGGL(mix_decay_kernel<1>, grid, dim3(256), 0, s, idx, w, a_experts, ld, T, H,
                       E, k, L);
  else if (L <= 128)
    hipLaunchKernelGGL(mix_decay_kernel<2>, grid, dim3(256), 0, s, idx, w, a_experts, ld, T, H,
                       E, k, L);
  else
    hipLaunchKernelGGL(mix_decay_kernel<4>, grid, dim3(256), 0, s, idx, w, a_experts, ld, T, H,
                       E, k, L);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
