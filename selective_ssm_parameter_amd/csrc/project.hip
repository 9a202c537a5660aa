// Expert projections with the parameter-space mix fused into the epilogue
// (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
// Models", Method, key design 1: every selected expert maps the token to its
// own B, C, X streams, mixed as U~ = sum pi B X^T and C~ = sum pi C; the
// notes' outlook asks for exactly this: a fused MoE operator for the SSM input
// projection that avoids extra HBM round trips of router and slicing).
//
// Grouped GEMM over active pairs only. The bucketing kernels give every expert
// a contiguous list of (token, slot) pairs; each workgroup owns BM pairs of one
// expert and BN = 128 of the W = H*P + 2*G*N output columns:
//     Z[r, c] = sum_d u[token(r), d] * W_e[c, d]
// Both operands are contiguous along d, so global loads are 16 bytes per lane
// and the tiles sit in LDS in [row][d] order, which is exactly the fragment
// order of the matrix cores (8 consecutive d per lane). Accumulation is fp32.
// The K loop double-buffers LDS and keeps the next K tile's global loads in
// flight (in registers) while the current tile is multiplied, so there is one
// barrier per K tile and memory latency overlaps the matrix-core work.
// Epilogue, by column region (S = stream type: fp16 for bf16 inputs, else fp32):
//     c <  H*P          -> X_hat[token, slot, c]            (S)
//     c <  H*P + G*N    -> B_hat[token, slot, .] = w * Z     (S, w folded)
//     otherwise         -> c_part[token, slot, .] = w * Z    (fp32)
// and a last small kernel sums c_part over the slots in slot order
// (0..k-1, fp32) into C_mix, so C~ never depends on which workgroup ran first.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

constexpr int kBN = 128;

int proj_bm(int pairs, int E) { return (pairs / (E > 0 ? E : 1)) >= 96 ? 128 : 64; }

int proj_row_tiles_max(int pairs, int E, int bm) { return (pairs + bm - 1) / bm + E; }

// K-tile depth: 64 for 2-byte inputs, 32 for fp32 (same bytes per row).
template <typename T> struct ProjK { static constexpr int BK = sizeof(T) == 2 ? 64 : 32; };

template <typename T, int BM>
struct ProjLds {
  static constexpr int BK = ProjK<T>::BK;
  static constexpr int LDK = BK + 8;  // LDS row stride in elements
  static constexpr size_t bytes = (size_t)2 * (BM + kBN) * LDK * sizeof(T);
};

template <typename T, int BM>
__global__ __launch_bounds__(256) void proj_kernel(
    const T* __restrict__ u, const T* __restrict__ wexp, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_offsets,
    const float* __restrict__ topk_w, int M, int D, int W, int HP, int GN, int E, int k,
    typename StreamOf<T>::type* __restrict__ X_hat, typename StreamOf<T>::type* __restrict__ B_hat,
    float* __restrict__ c_part) {
  typedef typename StreamOf<T>::type S;
  constexpr int BK = ProjK<T>::BK, LDK = ProjLds<T, BM>::LDK;
  constexpr int CH = BK / 8;                 // 8-element chunks per row and K tile
  constexpr int WAVES_M = BM / 64;           // 2 (BM=128) or 1 (BM=64)
  constexpr int WAVES_N = 4 / WAVES_M;       // 2 or 4
  constexpr int WN = kBN / WAVES_N;          // 64 or 32
  constexpr int TM = 4, TN = WN / 16;        // 16x16 tiles per wave
  constexpr int AU = BM * CH / 256;          // A chunks per thread per K tile
  constexpr int BU = kBN * CH / 256;         // B chunks per thread per K tile
  typedef typename Vec<T>::x8 F;

  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* As = reinterpret_cast<T*>(lds_raw);              // [2][BM][LDK]
  T* Bs = As + 2 * BM * LDK;                          // [2][kBN][LDK]
  __shared__ int rtok[BM];
  __shared__ int rslot[BM];
  __shared__ float rw[BM];
  __shared__ int sh_e, sh_row0, sh_nrows;

  const int tile = blockIdx.x;
  if (threadIdx.x == 0) {
    int e = -1;
    if (tile < tile_offsets[E]) {
      int lo = 0, hi = E - 1;  // last e with tile_offsets[e] <= tile
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (tile_offsets[mid] <= tile) lo = mid; else hi = mid - 1;
      }
      e = lo;
      const int row0 = offsets[e] + (tile - tile_offsets[e]) * BM;
      sh_row0 = row0;
      sh_nrows = min(BM, offsets[e + 1] - row0);
    }
    sh_e = e;
  }
  __syncthreads();
  const int e = sh_e;
  if (e < 0) return;
  const int row0 = sh_row0, nrows = sh_nrows;
  for (int r = threadIdx.x; r < BM; r += 256) {
    if (r < nrows) {
      const int p = sorted[row0 + r];
      rtok[r] = p / k;
      rslot[r] = p - (p / k) * k;
      rw[r] = topk_w[p];
    } else {
      rtok[r] = -1;
      rslot[r] = 0;
      rw[r] = 0.f;
    }
  }
  __syncthreads();

  const int col0 = blockIdx.y * kBN;
  const T* We = wexp + (size_t)e * W * D;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Per-thread byte offsets of the A (gathered tokens) and B (weight) chunks;
  // out-of-range chunks read zeros through the buffer resources.
  constexpr uint32_t ES = sizeof(T);
  const BufRes rA = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rW = make_rsrc(We, (uint64_t)W * D * ES);
  uint32_t aoff[AU], boff[BU];
  int ach[AU], bch[BU];
#pragma unroll
  for (int i = 0; i < AU; ++i) {
    const int q = threadIdx.x + 256 * i, r = q / CH;
    ach[i] = q % CH;
    const int tok = rtok[r];
    aoff[i] = tok >= 0 ? ((uint32_t)tok * D + 8 * ach[i]) * ES : kOOB;
  }
#pragma unroll
  for (int i = 0; i < BU; ++i) {
    const int q = threadIdx.x + 256 * i, r = q / CH;
    bch[i] = q % CH;
    const int col = col0 + r;
    boff[i] = col < W ? ((uint32_t)col * D + 8 * bch[i]) * ES : kOOB;
  }
  F areg[AU], breg[BU];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AU; ++i)
      areg[i] = load8_buf<T>(rA, (aoff[i] != kOOB && k0 + 8 * ach[i] < D) ? aoff[i] + k0 * ES : kOOB);
#pragma unroll
    for (int i = 0; i < BU; ++i)
      breg[i] = load8_buf<T>(rW, (boff[i] != kOOB && k0 + 8 * bch[i] < D) ? boff[i] + k0 * ES : kOOB);
  };
  auto store_tile = [&](int buf) {
    T* a = As + buf * BM * LDK;
    T* bb = Bs + buf * kBN * LDK;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int q = threadIdx.x + 256 * i, r = q / CH, ch = q % CH;
      store8<T>(&a[r * LDK + 8 * ch], areg[i]);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
      const int q = threadIdx.x + 256 * i, r = q / CH, ch = q % CH;
      store8<T>(&bb[r * LDK + 8 * ch], breg[i]);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (D + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tile((kt + 1) * BK);  // next tile in flight during compute
    __syncthreads();  // tile kt is in LDS; everyone is done with tile kt - 1
    const T* a = As + (kt & 1) * BM * LDK;
    const T* bb = Bs + (kt & 1) * kBN * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      F af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = load8<T>(&a[(wm * 64 + i * 16 + c) * LDK + 32 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = load8<T>(&bb[(wn * WN + j * 16 + c) * LDK + 32 * ks + 8 * g]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_tile((kt + 1) & 1);
  }

  // Epilogue: lane holds Z[4g + q][c] of every 16x16 tile.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wm * 64 + i * 16 + 4 * g + q;
      const int tok = rtok[r];
      if (tok < 0) continue;
      const size_t pair = (size_t)tok * k + rslot[r];
      const float w = rw[r];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = col0 + wn * WN + j * 16 + c;
        const float z = acc[i][j][q];
        if (col < HP) {
          X_hat[pair * HP + col] = from_f32<S>(z);
        } else if (col < HP + GN) {
          B_hat[pair * GN + (col - HP)] = from_f32<S>(w * z);
        } else if (col < W) {
          c_part[pair * GN + (col - HP - GN)] = w * z;
        }
      }
    }
  }
}

// C_mix[m, :] = sum_{j = 0..k-1} c_part[m, j, :], in slot order, fp32.
template <typename T>
__global__ __launch_bounds__(256) void mix_c_kernel(const float* __restrict__ c_part, int M,
                                                    int k, int GN, T* __restrict__ C_mix) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // one group of 4 values
  const size_t n4 = (size_t)M * GN / 4;
  if (i >= n4) return;
  const size_t m = (i * 4) / GN, n = (i * 4) % GN;
  floatx4 s = *reinterpret_cast<const floatx4*>(c_part + (m * k) * GN + n);
  for (int j = 1; j < k; ++j) {
    floatx4 v = *reinterpret_cast<const floatx4*>(c_part + (m * k + j) * GN + n);
    s += v;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) C_mix[m * GN + n + q] = from_f32<T>(s[q]);
}

template <typename T>
static hipError_t launch_project_t(const ProjGeom& g, const T* u, const T* wexp,
                                   const int32_t* sorted, const int32_t* offsets,
                                   const int32_t* tile_offsets, const float* w, int bm,
                                   typename StreamOf<T>::type* B_hat,
                                   typename StreamOf<T>::type* X_hat, float* c_part,
                                   typename StreamOf<T>::type* C_mix, hipStream_t s) {
  typedef typename StreamOf<T>::type S;
  const int pairs = g.M * g.k;
  const dim3 grid(proj_row_tiles_max(pairs, g.E, bm), (g.W + kBN - 1) / kBN);
  const size_t lds = bm == 128 ? ProjLds<T, 128>::bytes : ProjLds<T, 64>::bytes;
  const void* kfn = bm == 128 ? (const void*)proj_kernel<T, 128> : (const void*)proj_kernel<T, 64>;
  hipError_t err = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  prof_begin("expert_project", s);
  if (bm == 128)
    hipLaunchKernelGGL((proj_kernel<T, 128>), grid, dim3(256), lds, s, u, wexp, sorted, offsets,
                       tile_offsets, w, g.M, g.D, g.W, g.HP(), g.GN(), g.E, g.k, X_hat, B_hat, c_part);
  else
    hipLaunchKernelGGL((proj_kernel<T, 64>), grid, dim3(256), lds, s, u, wexp, sorted, offsets,
                       tile_offsets, w, g.M, g.D, g.W, g.HP(), g.GN(), g.E, g.k, X_hat, B_hat, c_part);
  prof_end(s);
  if (!C_mix) return hipGetLastError();
  const size_t n4 = (size_t)g.M * g.GN() / 4;
  prof_begin("mix_c", s);
  hipLaunchKernelGGL(mix_c_kernel<S>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, c_part,
                     g.M, g.k, g.GN(), C_mix);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_project(bool is_bf16, const ProjGeom& g, const void* u, const void* w_experts,
                          const int32_t* sorted, const int32_t* offsets,
                          const int32_t* tile_offsets, const int32_t* /*idx*/, const float* w,
                          int bm, void* B_hat, void* X_hat, float* c_part, void* C_mix,
                          hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  if (is_bf16)
    return launch_project_t<bf16>(g, (const bf16*)u, (const bf16*)w_experts, sorted, offsets,
                                  tile_offsets, w, bm, (f16*)B_hat, (f16*)X_hat, c_part,
                                  (f16*)C_mix, s);
  return launch_project_t<float>(g, (const float*)u, (const float*)w_experts, sorted, offsets,
                                 tile_offsets, w, bm, (float*)B_hat, (float*)X_hat, c_part,
                                 (float*)C_mix, s);
}

}  // namespace swimba
