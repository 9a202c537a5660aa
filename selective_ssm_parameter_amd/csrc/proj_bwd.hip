// Backward of the expert projections, the parameter-space mix and the router
// (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
// Models", Method, key design 1: z_j = W^(e_j) u with rows X | B | C,
// B_hat_j = w_j B_j, C~ = sum_j w_j C_j, w_j = softmax(W_r u)[e_j];
// Experiments: the converted model is fine-tuned, which needs these
// gradients). Given dB_hat, dX_hat and dC~ (from the scan's backward):
//   dz_j  = [dX_hat_j | w_j dB_hat_j | w_j dC~]          (per (token, slot))
//   dw_j  = <B_j, dB_hat_j> + <C_j, dC~>                   (B_j, C_j unweighted)
//   dg    = pi o (dpi - <pi, dpi>),  dpi = dw at the selected experts
//   du    = sum_j W^(e_j)^T dz_j + W_r^T dg
//   dW^(e) = sum over the pairs of expert e of dz_j u^T,   dW_r = dg^T u
// The top-k set is piecewise constant in the logits and has no gradient.
// The forward routing and projection are recomputed (same kernels, so the
// same bits); the pairs come sorted by expert from the bucketing, and
// dz is materialised in that order so both grouped GEMMs read contiguous
// rows. GEMM operands bf16 (fp32 for fp32 problems), fp32 accumulation, fp32
// outputs; every sum over slots, tokens or splits runs in a fixed order.
#include "common.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace swimba {


// ---------------------------------------------------------------- dz and dw

// One wave per sorted pair: dz in sorted order, and the pair's share of the
// router gradient s_j = w_j dw_j = <w B_j, dB_hat_j> + <w C_j, dC~> (the
// weighted streams are what the forward keeps, so no division by w).
template <typename T, typename S>
__global__ __launch_bounds__(256) void pbwd_dz_kernel(ProjBwdArgs A) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int pairs = A.M * A.k;
  if (i >= pairs) return;
  const int p = A.sorted[i], m = p / A.k;
  const float wj = A.sorted_w[i];
  T* row = static_cast<T*>(A.dz) + (size_t)i * A.W;
  for (int c = lane; c < A.W; c += 64) {
    float v;
    if (c < A.HP) v = A.dX[(size_t)p * A.HP + c];
    else if (c < A.HP + A.GN) v = wj * A.dB[(size_t)p * A.GN + (c - A.HP)];
    else v = wj * A.dC[(size_t)m * A.GN + (c - A.HP - A.GN)];
    row[c] = from_f32<T>(v);
  }
  float sum = 0.f;
  const S* bh = static_cast<const S*>(A.B_hat) + (size_t)p * A.GN;
  for (int n = lane; n < A.GN; n += 64)
    sum += to_f32(bh[n]) * A.dB[(size_t)p * A.GN + n] +
           A.c_part[(size_t)p * A.GN + n] * A.dC[(size_t)m * A.GN + n];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) A.sw[p] = sum;
}

// ---------------------------------------------------------------- router

// One wave per token. With pi = softmax(logits) and q_e = pi_e dpi_e (the sum
// of s_j over the slots routed to e), dg_e = q_e - pi_e sum_f q_f. Then du is
// initialised with W_r^T dg, lanes over d.
template <typename T>
__global__ __launch_bounds__(256) void pbwd_router_kernel(ProjBwdArgs A) {
  __shared__ float sdg[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + wave;
  const int E = A.E;
  if (m < A.M) {
    float pi[4], q[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;
      pi[r] = e < E ? A.logits[(size_t)m * E + e] : -INFINITY;
      mx = fmaxf(mx, pi[r]);
      q[r] = 0.f;
      if (e < E)
        for (int j = 0; j < A.k; ++j)
          if (A.idx[(size_t)m * A.k + j] == e) q[r] += A.sw[(size_t)m * A.k + j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float se = 0.f, sq = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pi[r] = lane + 64 * r < E ? expf(pi[r] - mx) : 0.f;
      se += pi[r];
      sq += q[r];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      se += __shfl_xor(se, off);
      sq += __shfl_xor(sq, off);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;
      if (e < E) {
        const float g = q[r] - (pi[r] / se) * sq;
        sdg[wave][e] = g;
        A.dg[(size_t)m * E + e] = g;
      }
    }
  }
  __syncthreads();
  if (m >= A.M) return;
  const T* wr = static_cast<const T*>(A.w_router);
  for (int d = lane; d < A.D; d += 64) {
    float acc = 0.f;
    for (int e = 0; e < E; ++e) acc += sdg[wave][e] * to_f32(wr[(size_t)e * A.D + d]);
    A.du[(size_t)m * A.D + d] = acc;
  }
}

// ---------------------------------------------------------------- grouped GEMMs

// 128 x 128 output tiles, K steps of 32, four waves of 64 x 64 each. Tiles
// are staged through LDS as 16-byte chunks (one stage, registers in between).
//   MODE 0 (du): rows = one expert's sorted pairs, columns = d, K = w:
//     A(i, w) = dz[i][w] (rows of dz, k contiguous), B(w, d) = W^(e)[w][d].
//   MODE 1 (dW): rows = w, columns = d, K = the expert's sorted pairs:
//     A(w, i) = dz[i][w] (K-major), B(i, d) = u[token of pair i][d].
// K-major tiles ([k][row]) are read back with load_kmajor (the transposing LDS
// read for 2-byte types) and stored with its swizzle; the k-contiguous A tile
// of MODE 0 with the row swizzle.
constexpr int kGB = 128, kGK = 32;

template <typename T, int MODE>
__global__ __launch_bounds__(256) void pbwd_gemm_kernel(ProjBwdArgs A) {
  typedef typename Vec<T>::x8 F;
  constexpr int ES = sizeof(T), EPC = 16 / ES;  // bytes, elements per 16-byte chunk
  constexpr int ACPR = MODE == 0 ? kGK / EPC : kGB / EPC;  // chunks per LDS row
  constexpr int BCPR = kGB / EPC;
  constexpr int NCH = kGB * kGK / EPC;  // chunks per tile
  __shared__ __align__(16) unsigned char As[kGB * kGK * ES];
  __shared__ __align__(16) unsigned char Bs[kGB * kGK * ES];

  const int E = A.E, D = A.D, W = A.W;
  const int ncol = (D + kGB - 1) / kGB;
  int e = -1, r0 = 0, nrows = 0, c0 = 0;  // expert, first row, rows, first column
  int kbeg = 0, klen = 0;                  // MODE 1: the expert's sorted pair range
  if constexpr (MODE == 0) {
    int t = blockIdx.x / ncol;
    c0 = (blockIdx.x % ncol) * kGB;
    for (int q = 0; q < E; ++q) {
      const int cnt = A.offsets[q + 1] - A.offsets[q];
      const int nt = (cnt + kGB - 1) / kGB;
      if (t < nt) {
        e = q;
        r0 = A.offsets[q] + t * kGB;
        nrows = min(kGB, cnt - t * kGB);
        break;
      }
      t -= nt;
    }
    if (e < 0) return;
    klen = W;
  } else {
    const int nwt = (W + kGB - 1) / kGB;
    e = blockIdx.x / (nwt * ncol);
    const int rem = blockIdx.x % (nwt * ncol);
    r0 = (rem / ncol) * kGB;
    c0 = (rem % ncol) * kGB;
    if (e >= E) return;
    nrows = min(kGB, W - r0);
    kbeg = A.offsets[e];
    klen = A.offsets[e + 1] - kbeg;
  }
  const T* dz = static_cast<const T*>(A.dz);
  const T* we = static_cast<const T*>(A.w_experts) + (size_t)e * W * D;
  const T* u = static_cast<const T*>(A.u);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, cl = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int k0 = 0; k0 < klen; k0 += kGK) {
    int4v va[NCH / 256], vb[NCH / 256];
#pragma unroll
    for (int it = 0; it < NCH / 256; ++it) {
      const int q = threadIdx.x + 256 * it;
      va[it] = int4v{0, 0, 0, 0};
      vb[it] = int4v{0, 0, 0, 0};
      if constexpr (MODE == 0) {
        const int r = q / ACPR, kk = k0 + (q % ACPR) * EPC;
        if (r < nrows && kk < klen)
          va[it] = *reinterpret_cast<const int4v*>(dz + (size_t)(r0 + r) * W + kk);
      } else {
        const int r = q / ACPR, kk = k0 + r, w = r0 + (q % ACPR) * EPC;
        if (kk < klen && w < W)
          va[it] = *reinterpret_cast<const int4v*>(dz + (size_t)(kbeg + kk) * W + w);
      }
      const int r = q / BCPR, kk = k0 + r, d = c0 + (q % BCPR) * EPC;
      if (kk < klen && d < D) {
        if constexpr (MODE == 0) {
          vb[it] = *reinterpret_cast<const int4v*>(we + (size_t)kk * D + d);
        } else {
          const int tok = A.sorted[kbeg + kk] / A.k;
          vb[it] = *reinterpret_cast<const int4v*>(u + (size_t)tok * D + d);
        }
      }
    }
    __syncthreads();  // the previous step's fragments are read
#pragma unroll
    for (int it = 0; it < NCH / 256; ++it) {
      const int q = threadIdx.x + 256 * it;
      {
        const int r = q / ACPR, ch = q % ACPR;
        const int sw = MODE == 0 ? swz_row<T, ACPR>(r) : swz_tr<T, ACPR>(r);
        *reinterpret_cast<int4v*>(As + (r * ACPR + (ch ^ sw)) * 16) = va[it];
      }
      {
        const int r = q / BCPR, ch = q % BCPR;
        *reinterpret_cast<int4v*>(Bs + (r * BCPR + (ch ^ swz_tr<T, BCPR>(r))) * 16) = vb[it];
      }
    }
    __syncthreads();
    F bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = load_kmajor<T, BCPR>(Bs, 0, wn * 64 + 16 * j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      F af;
      const int row = wm * 64 + 16 * i;
      if constexpr (MODE == 0) {
        // lane (g, c): k = 8g .. 8g + 7 of row row + c
        const int r = row + cl;
        if constexpr (ES == 2)
          af = load8<T>(reinterpret_cast<const T*>(As + (r * ACPR + (g ^ swz_row<T, ACPR>(r))) * 16));
        else
          af = load8<T>(reinterpret_cast<const T*>(As + r * ACPR * 16 + 32 * g));
      } else {
        af = load_kmajor<T, ACPR>(As, 0, row, lane);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mma16(af, bf[j], acc[i][j]);
    }
  }

  // lane (g, c) of tile (i, j) holds rows 16 i + 4 g + q, column 16 j + c
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = c0 + wn * 64 + 16 * j + cl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * 64 + 16 * i + 4 * g + q;
        if (d < D && r < nrows) {
          if constexpr (MODE == 0) A.du_part[(size_t)A.sorted[r0 + r] * D + d] = acc[i][j][q];
          else A.dW[((size_t)e * W + r0 + r) * D + d] = acc[i][j][q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- sums

// du[m] += sum_j du_part[m, j] in slot order (pairs of out-of-range experts
// contribute nothing).
__global__ void pbwd_du_sum_kernel(ProjBwdArgs A) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (q >= (size_t)A.M * A.D) return;
  const size_t m = q / A.D, d = q % A.D;
  float s = A.du[q];
  for (int j = 0; j < A.k; ++j) {
    const int e = A.idx[m * A.k + j];
    if (e >= 0 && e < A.E) s += A.du_part[(m * A.k + j) * A.D + d];
  }
  A.du[q] = s;
}

// dW_r partials: split sp of the tokens, thread d, experts in groups of 16.
template <typename T>
__global__ __launch_bounds__(256) void pbwd_dwr_kernel(ProjBwdArgs A, int per) {
  const int d = blockIdx.x * 256 + threadIdx.x, sp = blockIdx.y;
  if (d >= A.D) return;
  const int m0 = sp * per, m1 = min(A.M, m0 + per);
  const T* u = static_cast<const T*>(A.u);
  for (int e0 = 0; e0 < A.E; e0 += 16) {
    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    for (int m = m0; m < m1; ++m) {
      const float uv = to_f32(u[(size_t)m * A.D + d]);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (e0 + q < A.E) acc[q] += A.dg[(size_t)m * A.E + e0 + q] * uv;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (e0 + q < A.E) A.dwr_part[((size_t)sp * A.E + e0 + q) * A.D + d] = acc[q];
  }
}

__global__ void pbwd_dwr_sum_kernel(ProjBwdArgs A) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (q >= (size_t)A.E * A.D) return;
  float s = 0.f;
  for (int sp = 0; sp < A.nsplit; ++sp) s += A.dwr_part[(size_t)sp * A.E * A.D + q];
  A.dWr[q] = s;
}

__global__ void fill_zero_kernel(float* dst, size_t n) {
  for (size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    dst[q] = 0.f;
}

hipError_t launch_fill_zero(float* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launch

constexpr int kDwrTokens = 512;  // tokens per dW_r split

int proj_bwd_splits(int M) { return (M + kDwrTokens - 1) / kDwrTokens; }

template <typename T, typename S>
static hipError_t launch_pbwd_t(const ProjBwdArgs& A, hipStream_t s) {
  const int pairs = A.M * A.k;
  prof_begin("proj_bwd_dz", s);
  hipLaunchKernelGGL((pbwd_dz_kernel<T, S>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("proj_bwd_router", s);
  hipLaunchKernelGGL(pbwd_router_kernel<T>, dim3((unsigned)((A.M + 3) / 4)), dim3(256), 0, s, A);
  prof_end(s);
  const int ncol = (A.D + kGB - 1) / kGB;
  // row tiles over all experts: sum_e ceil(n_e / 128) <= pairs / 128 + E
  const int ntr = pairs / kGB + A.E;
  prof_begin("proj_bwd_du", s);
  hipLaunchKernelGGL((pbwd_gemm_kernel<T, 0>), dim3((unsigned)(ntr * ncol)), dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("proj_bwd_du_sum", s);
  hipLaunchKernelGGL(pbwd_du_sum_kernel, dim3((unsigned)(((size_t)A.M * A.D + 255) / 256)),
                     dim3(256), 0, s, A);
  prof_end(s);
  const int nwt = (A.W + kGB - 1) / kGB;
  prof_begin("proj_bwd_dw", s);
  hipLaunchKernelGGL((pbwd_gemm_kernel<T, 1>), dim3((unsigned)(A.E * nwt * ncol)), dim3(256), 0,
                     s, A);
  prof_end(s);
  prof_begin("proj_bwd_dwr", s);
  hipLaunchKernelGGL(pbwd_dwr_kernel<T>, dim3((unsigned)((A.D + 255) / 256), (unsigned)A.nsplit),
                     dim3(256), 0, s, A, kDwrTokens);
  hipLaunchKernelGGL(pbwd_dwr_sum_kernel, dim3((unsigned)(((size_t)A.E * A.D + 255) / 256)),
                     dim3(256), 0, s, A);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_project_backward(bool is_bf16, ProjBwdArgs A, hipStream_t s) {
  A.nsplit = proj_bwd_splits(A.M);
  if (is_bf16) return launch_pbwd_t<bf16, f16>(A, s);
  return launch_pbwd_t<float, float>(A, s);
}

}  // namespace swimba
