// Expert projections with the parameter-space mix fused into the epilogue
// (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
// Models", Method, key design 1: every selected expert maps the token to its
// own B, C, X streams, mixed as U~ = sum pi B X^T and C~ = sum pi C; the
// notes' outlook asks for exactly this: a fused MoE operator for the SSM input
// projection that avoids extra HBM round trips of router and slicing).
//
// Grouped GEMM over active pairs only. The bucketing kernels give every expert
// a contiguous list of (token, slot) pairs; each workgroup owns BM pairs of one
// expert and BN of the W = H*P + 2*G*N output columns (256 x 256 with 8 waves
// for large groups, smaller tiles when an expert has few rows):
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
// written as whole row segments after staging each wave's results in LDS; a
// last small kernel sums c_part over the slots in slot order (0..k-1, fp32)
// into C_mix, so C~ never depends on which workgroup ran first.
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

// Tile configurations: BM pairs x BN columns per workgroup, WM x WN waves, each
// wave computing (BM/WM) x (BN/WN) with 16x16x32 matrix-core tiles.
template <int BM_, int BN_, int WM_, int WN_>
struct ProjCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NTH = 64 * NW;
  static constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
};
typedef ProjCfg<256, 256, 2, 4> ProjBig;    // large expert groups (prefill), 8 waves
typedef ProjCfg<128, 128, 2, 2> ProjMid;
typedef ProjCfg<64, 128, 1, 4> ProjSmall;  // few rows per expert (decode)

int proj_bm(int pairs, int E) {
  const int per = pairs / (E > 0 ? E : 1);
  return per >= 192 ? 256 : (per >= 96 ? 128 : 64);
}

int proj_row_tiles_max(int pairs, int E, int bm) { return (pairs + bm - 1) / bm + E; }

// K-tile depth: 64 for 2-byte inputs, 32 for fp32 (same bytes per row).
template <typename T> struct ProjK { static constexpr int BK = sizeof(T) == 2 ? 64 : 32; };

template <typename T, class C>
struct ProjLds {
  static constexpr int BK = ProjK<T>::BK;
  static constexpr int LDK = BK + 8;          // LDS row stride of the K tiles (elements)
  static constexpr int RR = C::TM >= 4 ? 4 : C::TM;  // epilogue row tiles per round
  static constexpr int EPS = C::TN * 16 + 4;  // epilogue row stride (floats)
  static constexpr size_t main_bytes = (size_t)2 * (C::BM + C::BN) * LDK * sizeof(T);
  static constexpr size_t epi_bytes = (size_t)C::NW * RR * 16 * EPS * sizeof(float);
  static constexpr size_t bytes = main_bytes > epi_bytes ? main_bytes : epi_bytes;
};

template <typename T, class C>
__global__ __launch_bounds__(C::NTH) void proj_kernel(
    const T* __restrict__ u, const T* __restrict__ wexp, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_offsets,
    const float* __restrict__ topk_w, int M, int D, int W, int HP, int GN, int E, int k,
    int ntiles, typename StreamOf<T>::type* __restrict__ X_hat,
    typename StreamOf<T>::type* __restrict__ B_hat, float* __restrict__ c_part) {
  typedef typename StreamOf<T>::type S;
  typedef ProjLds<T, C> Lay;
  constexpr int BM = C::BM, BN = C::BN, NTH = C::NTH, TM = C::TM, TN = C::TN;
  constexpr int BK = Lay::BK, LDK = Lay::LDK;
  constexpr int CH = BK / 8;                 // 8-element chunks per row and K tile
  constexpr int AU = BM * CH / NTH;          // A chunks per thread per K tile
  constexpr int BU = BN * CH / NTH;          // B chunks per thread per K tile
  typedef typename Vec<T>::x8 F;

  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* As = reinterpret_cast<T*>(lds_raw);              // [2][BM][LDK]
  T* Bs = As + 2 * BM * LDK;                          // [2][BN][LDK]
  __shared__ int rtok[BM];
  __shared__ int rslot[BM];
  __shared__ float rw[BM];
  __shared__ int sh_e, sh_row0, sh_nrows;

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so give
  // XCD x the contiguous logical range [x * per, (x + 1) * per): its tiles
  // share an expert's weights and, column tile fastest, a row tile of tokens.
  const int CT = (W + BN - 1) / BN;
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (logical >= ntiles) return;
  const int tile = logical / CT, ctile = logical % CT;
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
  for (int r = threadIdx.x; r < BM; r += NTH) {
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

  const int col0 = ctile * BN;
  const T* We = wexp + (size_t)e * W * D;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // Per-thread byte offsets of the A (gathered tokens) and B (weight) chunks;
  // out-of-range chunks read zeros through the buffer resources.
  constexpr uint32_t ES = sizeof(T);
  const BufRes rA = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rW = make_rsrc(We, (uint64_t)W * D * ES);
  uint32_t aoff[AU], boff[BU];
  int ach[AU], bch[BU];
#pragma unroll
  for (int i = 0; i < AU; ++i) {
    const int q = threadIdx.x + NTH * i, r = q / CH;
    ach[i] = q % CH;
    const int tok = rtok[r];
    aoff[i] = tok >= 0 ? ((uint32_t)tok * D + 8 * ach[i]) * ES : kOOB;
  }
#pragma unroll
  for (int i = 0; i < BU; ++i) {
    const int q = threadIdx.x + NTH * i, r = q / CH;
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
    T* bb = Bs + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int q = threadIdx.x + NTH * i, r = q / CH, ch = q % CH;
      store8<T>(&a[r * LDK + 8 * ch], areg[i]);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
      const int q = threadIdx.x + NTH * i, r = q / CH, ch = q % CH;
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
    const T* a = As + (kt & 1) * BM * LDK + (wm * TM * 16 + c) * LDK + 8 * g;
    const T* bb = Bs + (kt & 1) * BN * LDK + (wn * TN * 16 + c) * LDK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      F bfr[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = load8<T>(bb + j * 16 * LDK + 32 * ks);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const F af = load8<T>(a + i * 16 * LDK + 32 * ks);
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma16(af, bfr[j], acc[i][j]);
      }
    }
    if (kt + 1 < nk) store_tile((kt + 1) & 1);
  }

  // ---- epilogue through LDS: each wave stages RR row tiles x TN column tiles
  // of fp32 results, then writes whole row segments (4 columns per lane).
  constexpr int RR = Lay::RR, EPS = Lay::EPS;
  float* ep = reinterpret_cast<float*>(lds_raw) + (size_t)wave * RR * 16 * EPS;
  __syncthreads();  // the K tiles are no longer read
#pragma unroll
  for (int round = 0; round < TM / RR; ++round) {
#pragma unroll
    for (int i = 0; i < RR; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) ep[(16 * i + 4 * g + q) * EPS + 16 * j + c] = acc[round * RR + i][j][q];
    __syncthreads();
    constexpr int CPR = TN * 4;  // 4-column chunks per staged row
    for (int it = lane; it < RR * 16 * CPR; it += 64) {
      const int rl = it / CPR, ch = it % CPR;
      const int r = wm * TM * 16 + round * RR * 16 + rl;
      const int col = col0 + wn * TN * 16 + 4 * ch;
      const int tok = rtok[r];
      if (tok < 0 || col >= W) continue;
      const size_t pair = (size_t)tok * k + rslot[r];
      const floatx4 v = *reinterpret_cast<const floatx4*>(&ep[rl * EPS + 4 * ch]);
      typedef typename Vec<S>::x4 S4;
      if (col < HP) {
        S4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = from_f32<S>(v[q]);
        *reinterpret_cast<S4*>(&X_hat[pair * HP + col]) = o;
      } else if (col < HP + GN) {
        const float w = rw[r];
        S4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = from_f32<S>(w * v[q]);
        *reinterpret_cast<S4*>(&B_hat[pair * GN + (col - HP)]) = o;
      } else {
        *reinterpret_cast<floatx4*>(&c_part[pair * GN + (col - HP - GN)]) = v * rw[r];
      }
    }
    __syncthreads();
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

template <typename T, class C>
static hipError_t launch_proj_cfg(const ProjGeom& g, const T* u, const T* wexp,
                                  const int32_t* sorted, const int32_t* offsets,
                                  const int32_t* tile_offsets, const float* w,
                                  typename StreamOf<T>::type* B_hat,
                                  typename StreamOf<T>::type* X_hat, float* c_part,
                                  hipStream_t s) {
  const int pairs = g.M * g.k;
  const int ntiles = proj_row_tiles_max(pairs, g.E, C::BM) * ((g.W + C::BN - 1) / C::BN);
  const dim3 grid((unsigned)((ntiles + 7) / 8 * 8));  // a multiple of the 8 XCDs
  const size_t lds = ProjLds<T, C>::bytes;
  hipError_t err = hipFuncSetAttribute((const void*)proj_kernel<T, C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  prof_begin("expert_project", s);
  hipLaunchKernelGGL((proj_kernel<T, C>), grid, dim3(C::NTH), lds, s, u, wexp, sorted, offsets,
                     tile_offsets, w, g.M, g.D, g.W, g.HP(), g.GN(), g.E, g.k, ntiles, X_hat,
                     B_hat, c_part);
  prof_end(s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_project_t(const ProjGeom& g, const T* u, const T* wexp,
                                   const int32_t* sorted, const int32_t* offsets,
                                   const int32_t* tile_offsets, const float* w, int bm,
                                   typename StreamOf<T>::type* B_hat,
                                   typename StreamOf<T>::type* X_hat, float* c_part,
                                   typename StreamOf<T>::type* C_mix, hipStream_t s) {
  typedef typename StreamOf<T>::type S;
  hipError_t err;
  if constexpr (sizeof(T) == 2) {
    // the 256 x 256 tile needs 2-byte K tiles to fit LDS
    if (bm == 256)
      err = launch_proj_cfg<T, ProjBig>(g, u, wexp, sorted, offsets, tile_offsets, w, B_hat, X_hat, c_part, s);
    else if (bm == 128)
      err = launch_proj_cfg<T, ProjMid>(g, u, wexp, sorted, offsets, tile_offsets, w, B_hat, X_hat, c_part, s);
    else
      err = launch_proj_cfg<T, ProjSmall>(g, u, wexp, sorted, offsets, tile_offsets, w, B_hat, X_hat, c_part, s);
  } else {
    if (bm >= 128)
      err = launch_proj_cfg<T, ProjMid>(g, u, wexp, sorted, offsets, tile_offsets, w, B_hat, X_hat, c_part, s);
    else
      err = launch_proj_cfg<T, ProjSmall>(g, u, wexp, sorted, offsets, tile_offsets, w, B_hat, X_hat, c_part, s);
  }
  if (err != hipSuccess) return err;
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
