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

// N (state size) and KM (a bound on k; k itself is a run-time argument) are
// compile-time so every load is issued up front and the row loop unrolls.
// With a_experts non-null the decay is the expert-mixed one (papernotes.org
// notes, Limitations and outlook): a = sum_j w_j a_experts[idx_j, h] / sum_j w_j
// over the sequence's k slots, in slot order (an index outside [0, E) adds
// decay 0 with its weight).
template <typename S, typename TY, int N, int KM>
__global__ __launch_bounds__(256, 4) void decode_state_kernel(
    const S* __restrict__ B_hat, const S* __restrict__ X_hat, const float* __restrict__ c_part,
    const float* __restrict__ a, float* __restrict__ hstate, TY* __restrict__ y, int H, int G,
    int k, const int32_t* __restrict__ idx, const float* __restrict__ tw,
    const float* __restrict__ a_experts, int E) {
  constexpr int P = 64;
  constexpr int NR = N / 16;                  // state rows per thread
  constexpr int QN = (KM * N + 255) / 256;    // B_hat / c_part staging loads per thread
  constexpr int QP = (KM * P + 255) / 256;    // X_hat staging loads per thread
  __shared__ float sB[KM][N];
  __shared__ float sCp[KM][N];
  __shared__ float sX[KM][P];
  __shared__ float sC[N];
  __shared__ floatx4 red[16][16];

  const int t = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int grp = h / (H / G);
  const int GN = G * N;
  const int p4 = 4 * (t & 15);
  const int n0 = t >> 4;
  float* hs = hstate + ((size_t)b * H + h) * (size_t)N * P;

  // every HBM read of this workgroup is in flight before the first wait. The
  // state is read non-temporally: it is used once per step, and keeping it out
  // of the caches leaves them to the data that other kernels reuse (measured:
  // the step is 3-4% faster whether or not other traffic runs between steps;
  // non-temporal stores as well help only when steps run back to back and hurt
  // when other writes come between them, so the write-back stays ordinary)
  floatx4 hv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    hv[i] = __builtin_nontemporal_load(
        reinterpret_cast<const floatx4*>(hs + (size_t)(n0 + 16 * i) * P + p4));
  // staging loads are unconditional (clamped index) so none waits behind a branch
  float bq[QN], cq[QN], xq[QP];
#pragma unroll
  for (int r = 0; r < QN; ++r) {
    const int q = min(t + 256 * r, k * N - 1);
    const size_t row = ((size_t)b * k + q / N) * GN + grp * N + q % N;
    bq[r] = to_f32(B_hat[row]);
    cq[r] = c_part[row];
  }
#pragma unroll
  for (int r = 0; r < QP; ++r) {
    const int q = min(t + 256 * r, k * P - 1);
    xq[r] = to_f32(X_hat[((size_t)b * k + q / P) * H * P + (size_t)h * P + q % P]);
  }
#pragma unroll
  for (int r = 0; r < QN; ++r) {
    const int q = t + 256 * r;
    if (q < k * N) {
      sB[q / N][q % N] = bq[r];
      sCp[q / N][q % N] = cq[r];
    }
  }
#pragma unroll
  for (int r = 0; r < QP; ++r) {
    const int q = t + 256 * r;
    if (q < k * P) sX[q / P][q % P] = xq[r];
  }
  __syncthreads();
  // C~ = sum_j c_part[b, j] in slot order (fp32), rounded to the stream type
  if (t < N) {
    float cs = 0.f;
    for (int j = 0; j < k; ++j) cs += sCp[j][t];
    sC[t] = to_f32(from_f32<S>(cs));
  }
  __syncthreads();

  float ah;
  if (a_experts) {
    float num = 0.f, den = 0.f;
    for (int j = 0; j < k; ++j) {
      const float wj = tw[(size_t)b * k + j];
      const int e = idx[(size_t)b * k + j];
      num += (e >= 0 && e < E) ? wj * a_experts[(size_t)e * H + h] : 0.f;
      den += wj;
    }
    ah = num / den;
  } else {
    ah = a[h];
  }
  floatx4 xj[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    xj[j] = j < k ? floatx4{sX[j][p4], sX[j][p4 + 1], sX[j][p4 + 2], sX[j][p4 + 3]}
                  : floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int n = n0 + 16 * i;
    floatx4 v = hv[i] * ah;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) v += sB[j][n] * xj[j];
    *reinterpret_cast<floatx4*>(hs + (size_t)n * P + p4) = v;
    yacc += sC[n] * v;
  }
  red[n0][t & 15] = yacc;
  __syncthreads();
  if (t < 16) {
    floatx4 s = red[0][t];
    for (int r = 1; r < 16; ++r) s += red[r][t];
    TY* yo = y + ((size_t)b * H + h) * P + 4 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) yo[i] = from_f32<TY>(s[i]);
  }
}

struct DecayMix {
  const int32_t* idx;
  const float* w;
  const float* a_experts;
  int E;
};

template <int N, int KM>
static void launch_decode_state_t(bool is_bf16, dim3 grid, const void* B_hat, const void* X_hat,
                                  const float* c_part, const float* a, float* h, void* y, int H,
                                  int G, int k, hipStream_t s, DecayMix m) {
  if (is_bf16)
    hipLaunchKernelGGL((decode_state_kernel<f16, bf16, N, KM>), grid, dim3(256), 0, s,
                       (const f16*)B_hat, (const f16*)X_hat, c_part, a, h, (bf16*)y, H, G, k,
                       m.idx, m.w, m.a_experts, m.E);
  else
    hipLaunchKernelGGL((decode_state_kernel<float, float, N, KM>), grid, dim3(256), 0, s,
                       (const float*)B_hat, (const float*)X_hat, c_part, a, h, (float*)y, H, G,
                       k, m.idx, m.w, m.a_experts, m.E);
}

template <int N>
static void launch_decode_state_n(bool is_bf16, dim3 grid, const void* B_hat, const void* X_hat,
                                  const float* c_part, const float* a, float* h, void* y, int H,
                                  int G, int k, hipStream_t s, DecayMix m) {
  if (k <= 1)
    launch_decode_state_t<N, 1>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m);
  else if (k <= 2)
    launch_decode_state_t<N, 2>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m);
  else if (k <= 4)
    launch_decode_state_t<N, 4>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m);
  else
    launch_decode_state_t<N, 8>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m);
}

hipError_t launch_decode_state(bool is_bf16, int Bt, int H, int G, int N, int P, int k,
                               const void* B_hat, const void* X_hat, const float* c_part,
                               const float* a, float* h, void* y, hipStream_t s,
                               const int32_t* idx, const float* w, const float* a_experts,
                               int E) {
  const DecayMix m{idx, w, a_experts, E};
  if (Bt == 0) return hipSuccess;
  if (P != 64 || k < 1 || k > 8 || (N != 16 && N != 32 && N != 64 && N != 128))
    return hipErrorInvalidValue;
  prof_begin("decode_state", s);
  const dim3 grid(H, Bt);
  switch (N) {
    case 16: launch_decode_state_n<16>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m); break;
    case 32: launch_decode_state_n<32>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m); break;
    case 64: launch_decode_state_n<64>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m); break;
    default: launch_decode_state_n<128>(is_bf16, grid, B_hat, X_hat, c_part, a, h, y, H, G, k, s, m); break;
  }
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
