// MoE over separated SSMs, the comparison design of the pages (papernotes.org
// notes on "Swimba: Switch Mamba Model Scales State Space Models", research
// background and motivation: one state trajectory per expert, every expert's
// recursion advanced at every step; Method, key design 2, Theorem 3.4: the
// output is the routing-weighted sum of the experts' readouts of their own
// states).
//
// Per expert e and head h:  h^(e)_t = a_h h^(e)_{t-1} + [e in K_t] B^(e)_t X^(e)_t^T,
//                           y_t = sum_{e in K_t} pi_{t,e} C^(e)_t^T h^(e)_t.
// It reuses the Swimba kernels: the router, the grouped projection of the
// selected (token, slot) pairs (with B left unweighted), then these two
// kernels around the chunked scan run over Bt * E sequences with k = 1:
//   scatter: the per-expert streams of sequence (b, e) at row (b E + e) T + t:
//            the selected pair's X, B and pi * C, zeros when e is not in K_t;
//   sum:     y[b, t] = sum_e y^(e)[b, t] over the experts in order (fp32).
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

// One thread moves 8 elements of one output row. Row layout: X (HP) | B (GN)
// | C (GN) chunks of 8.
template <typename S>
__global__ __launch_bounds__(256) void sep_scatter_kernel(
    const int32_t* __restrict__ idx, const S* __restrict__ X_hat, const S* __restrict__ B_hat,
    const float* __restrict__ c_part, int Bt, int T, int E, int k, int HP, int GN,
    S* __restrict__ Xs, S* __restrict__ Bs, S* __restrict__ Cs) {
  typedef typename Vec<S>::x8 V;
  const int CX = HP / 8, CB = GN / 8, CR = CX + 2 * CB;
  const size_t rows = (size_t)Bt * E * T;
  const size_t n = rows * CR;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t o = i / CR;
    const int ch = (int)(i - o * CR);
    const int t = (int)(o % T);
    const size_t be = o / T;
    const int e = (int)(be % E);
    const size_t b = be / E;
    const size_t m = b * T + t;
    int j = -1;
    for (int q = 0; q < k; ++q)
      if (idx[m * k + q] == e) j = q;
    const size_t pr = m * k + (j < 0 ? 0 : j);
    if (ch < CX) {
      store8<S>(Xs + o * HP + 8 * ch, j < 0 ? zero8<S>() : load8<S>(X_hat + pr * HP + 8 * ch));
    } else if (ch < CX + CB) {
      const int c = ch - CX;
      store8<S>(Bs + o * GN + 8 * c, j < 0 ? zero8<S>() : load8<S>(B_hat + pr * GN + 8 * c));
    } else {
      const int c = ch - CX - CB;
      V v = zero8<S>();
      if (j >= 0) v = convert8<S, float>(load8<float>(c_part + pr * GN + 8 * c));
      store8<S>(Cs + o * GN + 8 * c, v);
    }
  }
}

// y[m, :] = sum_{e = 0..E-1} yp[(b E + e) T + t, :] in fp32, in expert order.
template <typename TY>
__global__ __launch_bounds__(256) void sep_sum_kernel(const float* __restrict__ yp, int Bt, int T,
                                                      int E, int HP, TY* __restrict__ y) {
  const size_t n4 = (size_t)Bt * T * HP / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t m = (i * 4) / HP, c = (i * 4) % HP;
    const size_t b = m / T, t = m % T;
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < E; ++e)
      s += *reinterpret_cast<const floatx4*>(yp + ((b * E + e) * T + t) * HP + c);
    typename Vec<TY>::x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = from_f32<TY>(s[q]);
    *reinterpret_cast<typename Vec<TY>::x4*>(y + m * HP + c) = o;
  }
}

static unsigned grid_for(size_t n) {
  const size_t g = (n + 255) / 256;
  return (unsigned)(g < 16384 ? (g > 0 ? g : 1) : 16384);
}

hipError_t launch_sep_scatter(bool is_bf16, const int32_t* idx, const void* X_hat,
                              const void* B_hat, const float* c_part, int Bt, int T, int E, int k,
                              int HP, int GN, void* Xs, void* Bs, void* Cs, hipStream_t s) {
  const size_t n = (size_t)Bt * E * T * (HP / 8 + 2 * (GN / 8));
  if (n == 0) return hipSuccess;
  prof_begin("sep_scatter", s);
  if (is_bf16)
    hipLaunchKernelGGL(sep_scatter_kernel<f16>, dim3(grid_for(n)), dim3(256), 0, s, idx,
                       (const f16*)X_hat, (const f16*)B_hat, c_part, Bt, T, E, k, HP, GN, (f16*)Xs,
                       (f16*)Bs, (f16*)Cs);
  else
    hipLaunchKernelGGL(sep_scatter_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, idx,
                       (const float*)X_hat, (const float*)B_hat, c_part, Bt, T, E, k, HP, GN,
                       (float*)Xs, (float*)Bs, (float*)Cs);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_sep_sum(bool is_bf16, const float* yp, int Bt, int T, int E, int HP, void* y,
                          hipStream_t s) {
  const size_t n4 = (size_t)Bt * T * HP / 4;
  if (n4 == 0) return hipSuccess;
  prof_begin("sep_sum", s);
  if (is_bf16)
    hipLaunchKernelGGL(sep_sum_kernel<bf16>, dim3(grid_for(n4)), dim3(256), 0, s, yp, Bt, T, E, HP,
                       (bf16*)y);
  else
    hipLaunchKernelGGL(sep_sum_kernel<float>, dim3(grid_for(n4)), dim3(256), 0, s, yp, Bt, T, E,
                       HP, (float*)y);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace swimba
