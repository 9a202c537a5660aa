// Recurrent decode: in-place state update and readout for one token per
// sequence (papernotes.org notes on "Swimba: Switch Mamba Model Scales State
// Space Models", Method, key design 1, h_t = A h_{t-1} + U~_t, Y_t = C~_t^T h_t;
// key findings: token-by-token decoding).
//
// One workgroup per (sequence, head) streams that head's fp32 N x P state from
// HBM once and writes it back once (C~ is summed here from the projection's
// per-slot fp32 parts, in slot order):
//     h[n, p] <- a_h h[n, p] + sum_j B_hat[j, n] X[j, p]      (fp32)
//     y[p]     = sum_n C~[n] h[n, p]
// Thread t handles columns p = 4(t % 16) .. +3 and rows n = t/16 + 16 i, so
// each wave moves 4 full rows (1 KiB contiguous) per load. The k injections
// and C~ are staged in LDS as fp32; the readout sums over n in a fixed order
// (per thread, then over the 16 row groups), so results are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

constexpr int kDecMaxK = 8;
constexpr int kDecMaxN = 128;

template <typename S, typename TY>
__global__ __launch_bounds__(256) void decode_state_kernel(
    const S* __restrict__ B_hat, const S* __restrict__ X_hat, const float* __restrict__ c_part,
    const float* __restrict__ a, float* __restrict__ hstate, TY* __restrict__ y, int H, int G,
    int N, int k) {
  constexpr int P = 64;
  __shared__ float sB[kDecMaxK][kDecMaxN];
  __shared__ float sX[kDecMaxK][P];
  __shared__ float sC[kDecMaxN];
  __shared__ floatx4 red[16][16];

  const int h = blockIdx.x, b = blockIdx.y;
  const int grp = h / (H / G);
  const int GN = G * N;
  const int p4 = 4 * (threadIdx.x & 15);
  const int n0 = threadIdx.x >> 4;
  float* hs = hstate + ((size_t)b * H + h) * (size_t)N * P;
  // this thread's state rows, all in flight together with the staging loads
  constexpr int NR = kDecMaxN / 16;
  floatx4 hv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    if (n0 + 16 * i < N) hv[i] = *reinterpret_cast<const floatx4*>(hs + (size_t)(n0 + 16 * i) * P + p4);
  for (int q = threadIdx.x; q < k * N; q += 256) {
    const int j = q / N, n = q % N;
    sB[j][n] = to_f32(B_hat[((size_t)b * k + j) * GN + grp * N + n]);
  }
  for (int q = threadIdx.x; q < k * P; q += 256) {
    const int j = q / P, p = q % P;
    sX[j][p] = to_f32(X_hat[((size_t)b * k + j) * H * P + (size_t)h * P + p]);
  }
  // C~ = sum_j c_part[b, j] in slot order (fp32), rounded to the stream type
  for (int n = threadIdx.x; n < N; n += 256) {
    float cs = 0.f;
    for (int j = 0; j < k; ++j) cs += c_part[((size_t)b * k + j) * GN + grp * N + n];
    sC[n] = to_f32(from_f32<S>(cs));
  }
  __syncthreads();

  const float ah = a[h];
  floatx4 xj[kDecMaxK];
  for (int j = 0; j < k; ++j) xj[j] = floatx4{sX[j][p4], sX[j][p4 + 1], sX[j][p4 + 2], sX[j][p4 + 3]};
  floatx4 yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int n = n0 + 16 * i;
    if (n < N) {
      floatx4 v = hv[i] * ah;
      for (int j = 0; j < k; ++j) v += sB[j][n] * xj[j];
      *reinterpret_cast<floatx4*>(hs + (size_t)n * P + p4) = v;
      yacc += sC[n] * v;
    }
  }
  red[n0][threadIdx.x & 15] = yacc;
  __syncthreads();
  if (threadIdx.x < 16) {
    floatx4 s = red[0][threadIdx.x];
    for (int r = 1; r < 16; ++r) s += red[r][threadIdx.x];
    TY* yo = y + ((size_t)b * H + h) * P + 4 * threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) yo[i] = from_f32<TY>(s[i]);
  }
}

hipError_t launch_decode_state(bool is_bf16, int Bt, int H, int G, int N, int P, int k,
                               const void* B_hat, const void* X_hat, const float* c_part,
                               const float* a, float* h, void* y, hipStream_t s) {
  (void)P;
  if (Bt == 0) return hipSuccess;
  prof_begin("decode_state", s);
  if (is_bf16)
    hipLaunchKernelGGL((decode_state_kernel<f16, bf16>), dim3(H, Bt), dim3(256), 0, s,
                       (const f16*)B_hat, (const f16*)X_hat, c_part, a, h, (bf16*)y,
                       H, G, N, k);
  else
    hipLaunchKernelGGL((decode_state_kernel<float, float>), dim3(H, Bt), dim3(256), 0, s,
                       (const float*)B_hat, (const float*)X_hat, c_part, a, h,
                       (float*)y, H, G, N, k);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
