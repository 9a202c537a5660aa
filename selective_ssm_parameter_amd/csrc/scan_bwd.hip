// Backward of the single-trajectory scan (the reverse-time chunked solve).
// (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
// Models", Method, key design 1: h_t = a h_{t-1} + sum_j B_hat_j X_j^T,
// y_t = C~_t^T h_t; Experiments: the converted model is fine-tuned, which
// needs these gradients.)
//
// With g_t = dl/dh_t (gradient of the loss through every later readout):
//   g_t = C~_t dy_t^T + a g_{t+1} (+ dh_T at t = T-1)
//   dX_j = g_t^T B_hat_j,  dB_hat_j = sum_{heads of the group} g_t X_j,
//   dC~_t = sum_{heads} h_t dy_t,  da = sum_t <g_t, h_{t-1}>,  dh_init = a g_0.
// Chunks of BL tokens (a fixed internal length: the result does not depend
// on it). For chunk c = [c0, c1), entering state H_c = h_{c0-1} and F_c =
// a g_{c1} (dh_T for the last chunk: the gradient entering from the right),
// with local times:
//   g_t = sum_{s >= t} a^{s-t} C~_s dy_s^T + a^{c1-1-t} F_c
//   h_t = sum_{s <= t} a^{t-s} U_s      + a^{t-c0+1} H_c
// so, with Gm[s, r] = C~_s . B_hat_r and D[s, r] = dy_s . X_r over the chunk's
// (token, slot) pairs r of token t(r), masked to t(r) <= s:
//   dX_r^T   = sum_s dy_s^T a^{s-t} Gm[s, r]     + a^{c1-1-t} F_c^T B_hat_r
//   dB_hat_r = sum_s C~_s   a^{s-t} D[s, r]      + a^{c1-1-t} F_c X_r
//   dC~_s    = sum_r B_hat_r a^{s-t} D[s, r]     + a^{s-c0+1} H_c dy_s
//   da       = sum_{t(r) < s} (s-t) a^{s-t-1} Gm[s, r] D[s, r]
//            + sum_r (c1-1-t) a^{c1-2-t} B_hat_r . (F_c X_r)
//            + sum_s (s-c0+1) a^{s-c0} C~_s . (H_c dy_s) + Lc a^{Lc-1} <F_c, H_c>.
// Kernels: local chunk states S_c = sum_r a^{c1-1-t} B_hat_r X_r^T and
// R_c = sum_s a^{s-c0} C~_s dy_s^T (matrix cores); a sequential sweep per
// state element turning S into H_c (forwards: H_{c+1} = a^{Lc} H_c + S_c) and
// R into F_c (backwards: F_{c-1} = a R_c + a^{Lc} F_c, ending at F_{-1} =
// dh_init); per (sequence, chunk, group, slice of the group's heads)
// the gradients above on matrix cores, the slice's heads visited in order so
// dB_hat and dC~ are summed over them in registers, then (with several
// slices) a fixed-order sum of the slices' parts; a fixed-order sum of da.
// Everything is deterministic.
//
// LDS tiles are row-major with 16-byte chunks XOR-swizzled per row (the
// swizzle of the transposing read): a contraction along a tile row is one
// 16-byte read per fragment, one down a tile column is the transposing read.
// Tiles come in with 16-byte global reads, all of a thread's reads issued
// before the first is used; powers of the decay come from a per-head table.
// Matrix-core operands are fp16 (fp32 for fp32 problems) with fp32
// accumulation and fp32 outputs: the streams are fp16 already, and dy and the
// states are scaled per (chunk, head) by a power of two that brings their
// largest magnitude into [1/2, 1) (exact, and undone in fp32 on the results),
// so the gradients keep fp16's precision whatever their range.
#include "common.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace swimba {

constexpr int kBP = 64;        // head dim
constexpr int kGradWaves = 8;  // waves of the gradient kernel

// The local chunk states S_c and R_c go to HBM in the operand type (fp16 for
// bf16 problems), each (chunk, head) tile scaled by the power of two that
// brings its largest magnitude into [1/2, 1); the sweep restores them and
// sums in fp32, and writes H_c and F_c in the same type: for bf16 problems
// fp16 rows of P elements, each row with its own power-of-two factor (the
// gradient kernel rounds them to fp16 tiles under a power-of-two scale
// anyway); fp32 for fp32 problems.

struct BwdArgs {
  const void* B_hat;    // [M, k, G, N] stream type
  const void* X_hat;    // [M, k, H, P] stream type
  const void* C_mix;    // [M, G, N] stream type
  const void* dy;       // [M, H, P] dtype
  const float* a;       // [H]
  const float* h_init;  // [Bt, H, N, P] or null
  const float* dh_final;
  float* dB;            // [M, k, G, N]
  float* dX;            // [M, k, H, P]
  float* dC;            // [M, G, N]
  float* da;            // [H]
  float* dh_init;       // [Bt, H, N, P] or null
  void* Sl;             // [Bt, nb, H, N, P] local type: S_c (scaled by 1 / S_u)
  void* Rl;             // [Bt, nb, H, N, P] local type: R_c (scaled by 1 / R_u)
  float* Su;            // [Bt, nb, H]: the factor that restores S_c
  float* Ru;            // [Bt, nb, H]: the factor that restores R_c
  void* S;              // [Bt, nb, H, N, P] local type: H_c (entering state of chunk c)
  void* R;              // [Bt, nb, H, N, P] local type: F_c (gradient entering chunk c
                        // from the right); fp16 rows are scaled by 1 / Hu, 1 / Fu
  float* Hu;            // [Bt, nb, H, N]: the factor that restores row n of H_c (fp16 only)
  float* Fu;            // [Bt, nb, H, N]: the factor that restores row n of F_c (fp16 only)
  float* da_part;       // [Bt, nb, H]
  float* dBp;           // [hs, M, k, G, N] slice parts (hs > 1)
  float* dCp;           // [hs, M, G, N]
  int T, H, G, N, k, nb, hs;
};

// ---------------------------------------------------------------- LDS tiles

template <typename T, int CPR>
__device__ __forceinline__ int chunk_off(int r, int j) {
  return (r * CPR + (j ^ swz_tr<T, CPR>(r))) * 16;
}
template <typename T, int CPR>
__device__ __forceinline__ int elem_off(int r, int col) {
  constexpr int EPC = 16 / (int)sizeof(T);
  return chunk_off<T, CPR>(r, col / EPC) + (col % EPC) * (int)sizeof(T);
}
// Elements col .. col + 3 of row r (col a multiple of 4: one 8-byte piece of a
// 16-byte chunk for 2-byte types, a whole chunk for fp32), as fp32.
template <typename T, int CPR>
__device__ __forceinline__ floatx4 lds_get4(const unsigned char* t, int r, int col) {
  floatx4 v;
  if constexpr (sizeof(T) == 2) {
    typedef T T4 __attribute__((ext_vector_type(4)));
    const T4 x = *reinterpret_cast<const T4*>(t + elem_off<T, CPR>(r, col));
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = to_f32(x[q]);
  } else {
    v = *reinterpret_cast<const floatx4*>(t + elem_off<T, CPR>(r, col));
  }
  return v;
}
// Elements col .. col + 3 of row r (col a multiple of 4) from fp32 values:
// one 8-byte write for 2-byte types, one 16-byte write for fp32.
template <typename T, int CPR>
__device__ __forceinline__ void lds_put4(unsigned char* t, int r, int col, floatx4 v) {
  if constexpr (sizeof(T) == 2) {
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 x;
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = from_f32<T>(v[q]);
    *reinterpret_cast<T4*>(t + elem_off<T, CPR>(r, col)) = x;
  } else {
    *reinterpret_cast<floatx4*>(t + elem_off<T, CPR>(r, col)) = v;
  }
}

// Fragment along tile rows: lane (g, c) gets row r0 + c, elements
// k0 + 8g .. k0 + 8g + 7 (k0 a multiple of 32).
template <typename T, int CPR>
__device__ __forceinline__ typename Vec<T>::x8 frag_row(const unsigned char* t, int r0, int k0,
                                                        int lane) {
  const int g = lane >> 4, c = lane & 15;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename Vec<T>::x8*>(
        t + chunk_off<T, CPR>(r0 + c, (k0 >> 3) + g));
  } else {
    const int j = (k0 + 8 * g) >> 2;
    const floatx4 lo = *reinterpret_cast<const floatx4*>(t + chunk_off<T, CPR>(r0 + c, j));
    const floatx4 hi = *reinterpret_cast<const floatx4*>(t + chunk_off<T, CPR>(r0 + c, j + 1));
    return floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// One 16 x 16 tile: acc + sum over k < K (a multiple of 32) of A(m0 + i, k)
// B(k, n0 + j). AROW: A(m, k) = At[m][k], else At[k][m]; BROW: B(k, n) =
// Bt[n][k], else Bt[k][n]. Lane (g, c) gets D[m0 + 4g + i][n0 + c].
template <typename T, bool AROW, int ACPR, bool BROW, int BCPR>
__device__ __forceinline__ floatx4 tmm(const unsigned char* At, const unsigned char* Bt, int m0,
                                       int n0, int K, int lane) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 32) {
    typename Vec<T>::x8 fa, fb;
    if constexpr (AROW) fa = frag_row<T, ACPR>(At, m0, k0, lane);
    else fa = load_kmajor<T, ACPR>(At, k0, m0, lane);
    if constexpr (BROW) fb = frag_row<T, BCPR>(Bt, n0, k0, lane);
    else fb = load_kmajor<T, BCPR>(Bt, k0, n0, lane);
    acc = mma16(fa, fb, acc);
  }
  return acc;
}

// The NK = K / 32 fragments of one operand of a tile column (or row) block:
// ROW: along tile rows (frag_row at row c0), else down tile columns
// (load_kmajor at column c0).
template <typename T, bool ROW, int CPR, int NK>
__device__ __forceinline__ void load_frags(const unsigned char* t, int c0,
                                           typename Vec<T>::x8* f, int lane) {
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if constexpr (ROW) f[s] = frag_row<T, CPR>(t, c0, 32 * s, lane);
    else f[s] = load_kmajor<T, CPR>(t, 32 * s, c0, lane);
  }
}

// One 16 x 16 tile with the B operand's fragments given (loaded once for all
// the tiles of a wave that share them); A as in tmm.
template <typename T, bool AROW, int ACPR, int NK>
__device__ __forceinline__ floatx4 tmm_b(const unsigned char* At, int m0,
                                         const typename Vec<T>::x8* bf, int lane) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    typename Vec<T>::x8 fa;
    if constexpr (AROW) fa = frag_row<T, ACPR>(At, m0, 32 * s, lane);
    else fa = load_kmajor<T, ACPR>(At, 32 * s, m0, lane);
    acc = mma16(fa, bf[s], acc);
  }
  return acc;
}

template <typename SRC> struct Raw16;
template <> struct Raw16<f16> { typedef f16x8 type; };
template <> struct Raw16<bf16> { typedef bf16x8 type; };
template <> struct Raw16<float> { typedef floatx4 type; };

// Global -> LDS tile of ROWS x COLS elements of T from src (row stride
// gstride elements), each scaled by f(row) * sc; rows >= valid and columns
// >= cvalid (a multiple of 8) are zeros. 16-byte reads, all issued first.
template <typename T, int ROWS, int COLS, int NT, typename SRC>
struct TileLoad {
  static constexpr int V = 16 / (int)sizeof(SRC);  // elements per read
  static constexpr int RPR = COLS / V;             // reads per row
  static constexpr int NV = ROWS * RPR;
  static constexpr int IT = (NV + NT - 1) / NT;
  static constexpr int CPR = COLS * (int)sizeof(T) / 16;
  typedef typename Raw16<SRC>::type RV;
  RV raw[IT];

  __device__ __forceinline__ void fetch(const SRC* src, size_t gstride, int valid, int cvalid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int q = threadIdx.x + NT * i;
      const int r = q / RPR, c = (q % RPR) * V;
      raw[i] = RV{};
      if ((NV % NT == 0 || q < NV) && r < valid && c < cvalid)
        raw[i] = *reinterpret_cast<const RV*>(src + (size_t)r * gstride + c);
    }
  }
  // absmax and store take the factor of read i of this thread, row r, as
  // f(i, r); absmax and store take it per row.
  template <class F>
  __device__ __forceinline__ float absmax_ir(F f) const {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int q = threadIdx.x + NT * i;
      if (NV % NT != 0 && q >= NV) continue;
      const float s = f(i, q / RPR);
#pragma unroll
      for (int j = 0; j < V; ++j) mx = fmaxf(mx, fabsf(to_f32(raw[i][j]) * s));
    }
    return mx;
  }
  template <class F>
  __device__ __forceinline__ float absmax(F f) const {
    return absmax_ir([&](int, int r) { return f(r); });
  }
  template <class F>
  __device__ __forceinline__ void store(unsigned char* tile, F f, float sc) const {
    store_ir(tile, [&](int, int r) { return f(r); }, sc);
  }
  template <class F>
  __device__ __forceinline__ void store_ir(unsigned char* tile, F f, float sc) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int q = threadIdx.x + NT * i;
      if (NV % NT != 0 && q >= NV) continue;
      const int r = q / RPR, c = (q % RPR) * V;
      const float s = f(i, r) * sc;
      if constexpr (sizeof(T) == 2 && V == 8) {
        typename Vec<T>::x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = from_f32<T>(to_f32(raw[i][j]) * s);
        *reinterpret_cast<typename Vec<T>::x8*>(tile + chunk_off<T, CPR>(r, c / 8)) = o;
      } else if constexpr (sizeof(T) == 2) {  // fp32 source: half a chunk
        typename Vec<T>::x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = from_f32<T>(raw[i][j] * s);
        *reinterpret_cast<typename Vec<T>::x4*>(tile + elem_off<T, CPR>(r, c)) = o;
      } else {  // fp32 tile
        floatx4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = to_f32(raw[i][j]) * s;
        *reinterpret_cast<floatx4*>(tile + chunk_off<T, CPR>(r, c / 4)) = o;
      }
    }
  }
};

template <typename T, int ROWS, int COLS, int NT, typename SRC, class F>
__device__ __forceinline__ void tile_load(unsigned char* tile, const SRC* src, size_t gstride,
                                          int valid, int cvalid, F f) {
  TileLoad<T, ROWS, COLS, NT, SRC> L;
  L.fetch(src, gstride, valid, cvalid);
  L.store(tile, f, 1.f);
}

// tile_load with the tile scaled by the power of two that brings its largest
// magnitude into [1/2, 1) (1 for an all-zero tile; the exponent is capped so
// a subnormal maximum still gives a finite scale). Returns the scale. Every
// thread of the workgroup calls it (two barriers; red: NT / 64 floats).
template <typename T, int ROWS, int COLS, int NT, typename SRC, class F>
__device__ __forceinline__ float tile_load_scaled(unsigned char* tile, const SRC* src,
                                                  size_t gstride, int valid, int cvalid, F f,
                                                  float* red) {
  TileLoad<T, ROWS, COLS, NT, SRC> L;
  L.fetch(src, gstride, valid, cvalid);
  float mx = L.absmax(f);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  const float sc = mx > 0.f ? ldexpf(1.f, min(-(ilogbf(mx) + 1), 126)) : 1.f;
  L.store(tile, f, sc);
  return sc;
}

__device__ __forceinline__ float powi(float a, int d) {
  float r = 1.f, b = a;
  for (int e = d; e > 0; e >>= 1) {
    if (e & 1) r *= b;
    b *= b;
  }
  return r;
}

// ---------------------------------------------------------------- local states

template <typename T, typename S, typename TY, int NP, int KS, int BL>
__global__ __launch_bounds__(256) void bwd_local_kernel(BwdArgs A) {
  constexpr int R = KS * BL, ES = sizeof(T);
  constexpr int CB = NP * ES / 16, CX = kBP * ES / 16;
  __shared__ __align__(16) unsigned char Bs[R * NP * ES];
  __shared__ __align__(16) unsigned char Xd[R * kBP * ES];
  __shared__ __align__(16) unsigned char Cs[BL * NP * ES];
  __shared__ __align__(16) unsigned char Dyd[BL * kBP * ES];
  __shared__ float pw[BL + 1];
  __shared__ float red[4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = A.H, G = A.G, N = A.N, Tl = A.T;
  const int grp = h / (H / G);
  const int c0 = c * BL, Lc = min(BL, Tl - c0);
  const float a = A.a[h];
  const size_t m0 = (size_t)b * Tl + c0;  // first token row of the chunk
  for (int d = threadIdx.x; d <= BL; d += 256) pw[d] = powi(a, d);
  __syncthreads();
  const auto one = [](int) { return 1.f; };
  const auto xdec = [&](int r) { return r < Lc * KS ? pw[Lc - 1 - r / KS] : 0.f; };
  const auto ydec = [&](int s) { return s < Lc ? pw[s] : 0.f; };
  // every tile's reads in flight at once, then dy's scale, then the stores
  TileLoad<T, R, NP, 256, S> LB;
  TileLoad<T, R, kBP, 256, S> LX;
  TileLoad<T, BL, NP, 256, S> LC;
  TileLoad<T, BL, kBP, 256, TY> LY;
  LB.fetch(static_cast<const S*>(A.B_hat) + (m0 * KS) * G * N + grp * N, (size_t)G * N, Lc * KS,
           N);
  LX.fetch(static_cast<const S*>(A.X_hat) + (m0 * KS) * H * kBP + h * kBP, (size_t)H * kBP,
           Lc * KS, kBP);
  LC.fetch(static_cast<const S*>(A.C_mix) + m0 * G * N + grp * N, (size_t)G * N, Lc, N);
  LY.fetch(static_cast<const TY*>(A.dy) + m0 * H * kBP + h * kBP, (size_t)H * kBP, Lc, kBP);
  float my = LY.absmax(ydec);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) my = fmaxf(my, __shfl_xor(my, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = my;
  __syncthreads();
  my = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // 2^-e brings dy's largest decayed magnitude into [1/2, 1); capped for subnormals
  const float sdy = my > 0.f ? ldexpf(1.f, min(-(ilogbf(my) + 1), 126)) : 1.f;
  LB.store(Bs, one, 1.f);
  LX.store(Xd, xdec, 1.f);
  LC.store(Cs, one, 1.f);
  LY.store(Dyd, ydec, sdy);
  __syncthreads();
  const float udy = 1.f / sdy;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, cl = lane & 15;
  const size_t sbase = (((size_t)b * A.nb + c) * H + h) * (size_t)N * kBP;
  constexpr int TILES = (NP / 16) * (kBP / 16), TI = TILES / 4;
  // S[n][p] = sum_r B_hat[r][n] xd[r][p];  R[n][p] = sum_s C~[s][n] dyd[s][p]
  // (wave w owns column block p0 = 16 w of every tile it computes, so the
  // xd and dyd fragments are read once)
  typedef typename Vec<T>::x8 F;
  F fx[R / 32], fy[BL / 32];
  load_frags<T, false, CX, R / 32>(Xd, 16 * wave, fx, lane);
  load_frags<T, false, CX, BL / 32>(Dyd, 16 * wave, fy, lane);
  floatx4 s4[TI], r4[TI];
  float ms = 0.f, mr = 0.f;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int t = wave + 4 * i;
    const int n0 = 16 * (t / (kBP / 16));
    s4[i] = r4[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (n0 < N) {
      s4[i] = tmm_b<T, false, CB, R / 32>(Bs, n0, fx, lane);
      r4[i] = tmm_b<T, false, CB, BL / 32>(Cs, n0, fy, lane) * udy;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ms = fmaxf(ms, fabsf(s4[i][q]));
      mr = fmaxf(mr, fabsf(r4[i][q]));
    }
  }
  float ss = 1.f, sr = 1.f;  // storage scales (1 for fp32 tiles)
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      ms = fmaxf(ms, __shfl_xor(ms, off));
      mr = fmaxf(mr, __shfl_xor(mr, off));
    }
    __syncthreads();  // red is free again
    if (lane == 0) {
      red[wave] = ms;
      pw[wave] = mr;  // the decay table is no longer read
    }
    __syncthreads();
    ms = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    mr = fmaxf(fmaxf(pw[0], pw[1]), fmaxf(pw[2], pw[3]));
    ss = ms > 0.f ? ldexpf(1.f, min(-(ilogbf(ms) + 1), 126)) : 1.f;
    sr = mr > 0.f ? ldexpf(1.f, min(-(ilogbf(mr) + 1), 126)) : 1.f;
  }
  if (threadIdx.x == 0) {
    A.Su[((size_t)b * A.nb + c) * H + h] = 1.f / ss;
    A.Ru[((size_t)b * A.nb + c) * H + h] = 1.f / sr;
  }
  T* Sl = static_cast<T*>(A.Sl) + sbase;
  T* Rl = static_cast<T*>(A.Rl) + sbase;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int t = wave + 4 * i;
    const int n0 = 16 * (t / (kBP / 16)), p0 = 16 * (t % (kBP / 16));
    if (n0 >= N) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 4 * g + q;
      Sl[(size_t)n * kBP + p0 + cl] = from_f32<T>(s4[i][q] * ss);
      Rl[(size_t)n * kBP + p0 + cl] = from_f32<T>(r4[i][q] * sr);
    }
  }
}

// ---------------------------------------------------------------- state sweep

// DPP move of x from the lane that control word CTRL names (all rows and banks).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Largest x over each aligned group of G lanes (G a power of two up to 64),
// every lane of the group receiving it. Within 16 lanes the steps are DPP
// moves (quad permutations [1,0,3,2] and [2,3,0,1], then the half-row and row
// mirrors, each pairing a block of lanes whose maximum is already known with
// its neighbour); only the steps between 16-lane rows go through the
// cross-lane permute.
template <int G>
__device__ __forceinline__ float group_max(float m) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "power-of-two group up to 64 lanes");
  if constexpr (G >= 2) m = fmaxf(m, dpp_f<0xB1>(m));
  if constexpr (G >= 4) m = fmaxf(m, dpp_f<0x4E>(m));
  if constexpr (G >= 8) m = fmaxf(m, dpp_f<0x141>(m));
  if constexpr (G >= 16) m = fmaxf(m, dpp_f<0x140>(m));
  if constexpr (G >= 32) m = fmaxf(m, __shfl_xor(m, 16));
  if constexpr (G >= 64) m = fmaxf(m, __shfl_xor(m, 32));
  return m;
}

// Per state element: the states entering each chunk, H_c going forwards
// (H_{c+1} = a^{Lc} H_c + S_c from h_init) and F_c going backwards (F_{c-1} =
// a R_c + a^{Lc} F_c from dh_final, ending at F_{-1} = a g_0 = dh_init). Each
// thread owns V elements of a (sequence, head) state (16 bytes of the local
// states, or fewer when there are few states, so that enough threads share
// the walk) and reads those of SU chunks before it uses any (the walk over
// chunks is serial, so the reads of several chunks are kept in flight); sums
// in fp32. H_c and F_c are written in the local states' type, fp16 rows of
// kBP elements each with its own power-of-two factor: the gradient kernel
// rounds them to fp16 tiles for the matrix cores in any case.
template <typename LT, int BL, int V>
__global__ __launch_bounds__(256) void bwd_sweep_kernel(BwdArgs A) {
  constexpr int SU = V >= 4 ? 8 : 16;  // chunks whose reads are in flight together
  typedef LT RV __attribute__((ext_vector_type(V)));
  const int h = blockIdx.y, b = blockIdx.z;
  const int NPsz = A.N * kBP;
  const int e0 = (blockIdx.x * 256 + threadIdx.x) * V;
  if (e0 >= NPsz) return;
  const float a = A.a[h];
  const float aL = powi(a, BL);
  const int Tl = A.T, nb = A.nb, H = A.H;
  const float aLast = powi(a, Tl - (nb - 1) * BL);
  const size_t hb = ((size_t)b * H + h) * NPsz + e0;
  const size_t cstride = (size_t)H * NPsz;
  const size_t base = (size_t)b * nb * cstride + (size_t)h * NPsz + e0;
  const float* Su = A.Su + (size_t)b * nb * H + h;
  const float* Ru = A.Ru + (size_t)b * nb * H + h;
  float st[V], gr[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    st[j] = A.h_init ? A.h_init[hb + j] : 0.f;
    gr[j] = A.dh_final ? A.dh_final[hb + j] : 0.f;
  }
  const LT* Sl = static_cast<const LT*>(A.Sl) + base;
  const LT* Rl = static_cast<const LT*>(A.Rl) + base;
  LT* Hp = static_cast<LT*>(A.S) + base;
  LT* Fp = static_cast<LT*>(A.R) + base;
  // row n of the state: factors at ((b nb + c) H + h) N + n
  const size_t ubase = ((size_t)b * nb * H + h) * A.N + e0 / kBP;
  const size_t ustride = (size_t)H * A.N;
  auto put = [&](LT* dst, float* uf, const float* v) {
    if constexpr (sizeof(LT) == 4) {
      if constexpr (V % 4 == 0) {
#pragma unroll
        for (int j = 0; j < V; j += 4)
          *reinterpret_cast<floatx4*>(dst + j) = floatx4{v[j], v[j + 1], v[j + 2], v[j + 3]};
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) dst[j] = v[j];
      }
    } else {
      // fp16: the row (the kBP / V lanes holding it, all in one wave) is
      // scaled by the power of two that brings its largest magnitude into
      // [1/2, 1); the factor that restores it goes beside the state
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < V; ++j) m = fmaxf(m, fabsf(v[j]));
      m = group_max<kBP / V>(m);
      const float sc = m > 0.f ? ldexpf(1.f, min(-(ilogbf(m) + 1), 126)) : 1.f;
      RV o;
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = from_f32<LT>(v[j] * sc);
      *reinterpret_cast<RV*>(dst) = o;
      if (e0 % kBP == 0) *uf = 1.f / sc;
    }
  };
  for (int c0 = 0; c0 < nb; c0 += SU) {
    RV v[SU];
    float us[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      if (c0 + u < nb) {
        v[u] = *reinterpret_cast<const RV*>(Sl + (size_t)(c0 + u) * cstride);
        us[u] = Su[(size_t)(c0 + u) * H];
      }
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int c = c0 + u;
      if (c >= nb) break;
      put(Hp + (size_t)c * cstride, A.Hu + ubase + (size_t)c * ustride, st);
      const float ac = c == nb - 1 ? aLast : aL;
#pragma unroll
      for (int j = 0; j < V; ++j) st[j] = st[j] * ac + to_f32(v[u][j]) * us[u];
    }
  }
  for (int c1 = nb - 1; c1 >= 0; c1 -= SU) {
    RV v[SU];
    float us[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      if (c1 - u >= 0) {
        v[u] = *reinterpret_cast<const RV*>(Rl + (size_t)(c1 - u) * cstride);
        us[u] = Ru[(size_t)(c1 - u) * H] * a;
      }
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int c = c1 - u;
      if (c < 0) break;
      put(Fp + (size_t)c * cstride, A.Fu + ubase + (size_t)c * ustride, gr);
      const float ac = c == nb - 1 ? aLast : aL;
#pragma unroll
      for (int j = 0; j < V; ++j) gr[j] = gr[j] * ac + to_f32(v[u][j]) * us[u];
    }
  }
  if (A.dh_init) {
#pragma unroll
    for (int j = 0; j < V; ++j) A.dh_init[hb + j] = gr[j];
  }
}

// ---------------------------------------------------------------- chunk gradients

template <typename T, typename S, typename TY, int NP, int KS, int BL>
__global__ __launch_bounds__(64 * kGradWaves) void bwd_grad_kernel(BwdArgs A) {
  constexpr int NW = kGradWaves, NT = 64 * NW;
  constexpr int R = KS * BL, ES = sizeof(T);
  constexpr int CB = NP * ES / 16, CX = kBP * ES / 16, CG = R * ES / 16, CD = BL * ES / 16;
  constexpr int NGT = (BL / 16) * (R / 16);   // Gm and D tiles
  constexpr int NXT = (kBP / 16) * (R / 16);  // dX tiles
  constexpr int NBT = (NP / 16) * (R / 16);   // dB_hat tiles
  constexpr int NCT = (NP / 16) * (BL / 16);  // dC~ tiles
  constexpr int GI = (NGT + NW - 1) / NW, BI = (NBT + NW - 1) / NW, CI = (NCT + NW - 1) / NW;
  __shared__ __align__(16) unsigned char Bs[R * NP * ES];    // B_hat [r][n]
  __shared__ __align__(16) unsigned char Cs[BL * NP * ES];   // C~ [s][n]
  __shared__ __align__(16) unsigned char Xs[R * kBP * ES];   // X_r of the head [r][p]
  __shared__ __align__(16) unsigned char Dys[BL * kBP * ES]; // dy_s of the head [s][p]
  __shared__ __align__(16) unsigned char Dm[R * BL * ES];    // masked, decayed D [r][s]
  __shared__ __align__(16) unsigned char GmM[R * BL * ES];   // masked, decayed Gm [r][s]
  __shared__ __align__(16) unsigned char Ss[NP * kBP * ES];  // F_c [n][p]
  __shared__ __align__(16) unsigned char Hs[NP * kBP * ES];  // H_c [n][p]
  __shared__ float pw[BL + 2];                               // a^d of the head
  __shared__ float red[NW];
  __shared__ float redm[3][NW];

  const int c = blockIdx.x, y = blockIdx.y, b = blockIdx.z;
  const int H = A.H, G = A.G, N = A.N, Tl = A.T, HG = H / G, HS = A.hs, HPS = HG / HS;
  const int grp = y / HS, slice = y % HS;
  const int c0 = c * BL, Lc = min(BL, Tl - c0);
  const size_t m0 = (size_t)b * Tl + c0;
  const int lane0 = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const auto one = [](int) { return 1.f; };

  tile_load<T, R, NP, NT>(Bs, static_cast<const S*>(A.B_hat) + (m0 * KS) * G * N + grp * N,
                          (size_t)G * N, Lc * KS, N, one);
  tile_load<T, BL, NP, NT>(Cs, static_cast<const S*>(A.C_mix) + m0 * G * N + grp * N,
                           (size_t)G * N, Lc, N, one);
  __syncthreads();
  // Gm[s][r] = C~_s . B_hat_r: this wave's tiles, kept in registers for every head
  floatx4 gm[GI];
#pragma unroll
  for (int i = 0; i < GI; ++i) {
    const int t = wave + NW * i;
    gm[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (t < NGT)
      gm[i] = tmm<T, true, CB, true, CB>(Cs, Bs, 16 * (t / (R / 16)), 16 * (t % (R / 16)), NP,
                                         lane0);
  }

  floatx4 dBa[BI], dCa[CI];
#pragma unroll
  for (int i = 0; i < BI; ++i) dBa[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CI; ++i) dCa[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int hi = 0; hi < HPS; ++hi) {
    const int h = grp * HG + slice * HPS + hi;
    const float a = A.a[h];
    // lane made opaque per head: the tiles' address arithmetic is then redone
    // for each head instead of being held in registers across the loop
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int g = lane >> 4, cl = lane & 15;
    const size_t sbase = (((size_t)b * A.nb + c) * H + h) * (size_t)N * kBP;
    __syncthreads();  // the previous head is done with Xs, Dys, Dm, GmM, Ss, Hs, pw
    for (int d = threadIdx.x; d < BL + 2; d += NT) pw[d] = powi(a, d);
    // the head's tiles, every read in flight at once; dy, F_c and H_c are
    // scaled by powers of two, and <F_c, H_c> is taken in fp32 on the way
    TileLoad<T, R, kBP, NT, S> LX;
    TileLoad<T, BL, kBP, NT, TY> LD;
    TileLoad<T, NP, kBP, NT, T> LF, LH;
    LX.fetch(static_cast<const S*>(A.X_hat) + (m0 * KS) * H * kBP + h * kBP, (size_t)H * kBP,
             Lc * KS, kBP);
    LD.fetch(static_cast<const TY*>(A.dy) + m0 * H * kBP + h * kBP, (size_t)H * kBP, Lc, kBP);
    LF.fetch(static_cast<const T*>(A.R) + sbase, (size_t)kBP, N, kBP);
    LH.fetch(static_cast<const T*>(A.S) + sbase, (size_t)kBP, N, kBP);
    // fp16 states: the factor of each read's row (1 for fp32 states)
    float fu[LF.IT], hu[LF.IT];
#pragma unroll
    for (int i = 0; i < LF.IT; ++i) {
      fu[i] = hu[i] = 1.f;
      if constexpr (sizeof(T) == 2) {
        const int r = (threadIdx.x + NT * i) / LF.RPR;
        if (r < N) {
          const size_t ui = sbase / kBP + r;  // ((b nb + c) H + h) N + r
          fu[i] = A.Fu[ui];
          hu[i] = A.Hu[ui];
        }
      }
    }
    auto fsc = [&](int i, int) { return fu[i]; };
    auto hsc = [&](int i, int) { return hu[i]; };
    float eh = 0.f;
#pragma unroll
    for (int i = 0; i < LF.IT; ++i) {
      float e = 0.f;
#pragma unroll
      for (int j = 0; j < LF.V; ++j) e += to_f32(LF.raw[i][j]) * to_f32(LH.raw[i][j]);
      eh += e * (fu[i] * hu[i]);
    }
    float mx[3] = {LD.absmax(one), LF.absmax_ir(fsc), LH.absmax_ir(hsc)};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], off));
      if (lane == 0) redm[j][wave] = mx[j];
    }
    __syncthreads();
    float scl[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      float m = redm[j][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = fmaxf(m, redm[j][w]);
      // 2^-e brings the largest magnitude into [1/2, 1); capped for subnormals
      scl[j] = m > 0.f ? ldexpf(1.f, min(-(ilogbf(m) + 1), 126)) : 1.f;
    }
    LX.store(Xs, one, 1.f);
    LD.store(Dys, one, scl[0]);
    LF.store_ir(Ss, fsc, scl[1]);
    LH.store_ir(Hs, hsc, scl[2]);
    const float udy = 1.f / scl[0], uF = 1.f / scl[1], uHdy = 1.f / (scl[2] * scl[0]);
    __syncthreads();
    float dap = eh * (float)Lc * pw[Lc - 1];  // this lane's part of da for the head
    // Every phase's tiles t = wave + NW i of a wave share one column block
    // (NW is a multiple of the column blocks), so that operand's fragments
    // are loaded once per phase.
    static_assert(NW % (R / 16) == 0 && NW % (BL / 16) == 0, "fixed column block per wave");
    typedef typename Vec<T>::x8 F;
    // D[s][r] = dy_s . X_r; the masked, decayed D and Gm; the Gm D term of da
    F fx[kBP / 32];
    load_frags<T, true, CX, kBP / 32>(Xs, 16 * (wave % (R / 16)), fx, lane);
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      const int t = wave + NW * i;
      if (t >= NGT) continue;
      const int s0 = 16 * (t / (R / 16)), r0 = 16 * (t % (R / 16));
      const floatx4 v = tmm_b<T, true, CX, kBP / 32>(Dys, s0, fx, lane);
      const int r = r0 + cl, tr = r / KS;
      floatx4 dv, dg;  // this lane's 4 consecutive s of row r, stored [r][s]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = s0 + 4 * g + q;
        const bool in = tr <= s && s < Lc;
        const float dec = in ? pw[s - tr] : 0.f;
        if (in && tr < s) dap += (float)(s - tr) * pw[s - tr - 1] * gm[i][q] * v[q] * udy;
        dv[q] = dec * v[q];
        dg[q] = dec * gm[i][q];
      }
      lds_put4<T, CD>(Dm, r, s0 + 4 * g, dv);
      lds_put4<T, CD>(GmM, r, s0 + 4 * g, dg);
    }
    __syncthreads();
    // dX_r^T[p] = sum_s dy_s[p] GmM(s, r) + a^{Lc-1-t} (F_c^T B_hat_r)[p]
    {
      F fg[BL / 32], fb[NP / 32];
      load_frags<T, true, CD, BL / 32>(GmM, 16 * (wave % (R / 16)), fg, lane);
      load_frags<T, true, CB, NP / 32>(Bs, 16 * (wave % (R / 16)), fb, lane);
    for (int t = wave; t < NXT; t += NW) {
      const int p0 = 16 * (t / (R / 16)), r0 = 16 * (t % (R / 16));
      floatx4 v = tmm_b<T, false, CX, BL / 32>(Dys, p0, fg, lane);
      const floatx4 w = tmm_b<T, false, CX, NP / 32>(Ss, p0, fb, lane);
      const int r = r0 + cl, tr = r / KS;
      if (tr < Lc) {
        v = v * udy + w * (pw[Lc - 1 - tr] * uF);
        const size_t row = (m0 * KS + r) * H + h;  // pair row of X_hat
        *reinterpret_cast<floatx4*>(A.dX + row * kBP + p0 + 4 * g) = v;
      }
    }
    }
    // dB_hat_r[n] += sum_s C~_s[n] Dm(s, r) + a^{Lc-1-t} (F_c X_r)[n]
    F fd[BL / 32];
    load_frags<T, true, CD, BL / 32>(Dm, 16 * (wave % (R / 16)), fd, lane);
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int t = wave + NW * i;
      const int n0 = 16 * (t / (R / 16)), r0 = 16 * (t % (R / 16));
      if (t >= NBT || n0 >= N) continue;
      const floatx4 v = tmm_b<T, false, CB, BL / 32>(Cs, n0, fd, lane);
      const floatx4 w = tmm_b<T, true, CX, kBP / 32>(Ss, n0, fx, lane);
      const int r = r0 + cl, tr = r / KS;
      const float sc = tr < Lc ? pw[Lc - 1 - tr] : 0.f;
      const float wt = tr + 1 < Lc ? (float)(Lc - 1 - tr) * pw[Lc - 2 - tr] : 0.f;
      const floatx4 bq = lds_get4<T, CB>(Bs, r, n0 + 4 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) dap += wt * uF * w[q] * bq[q];
      dBa[i] = dBa[i] + v * udy + w * (sc * uF);
      __builtin_amdgcn_sched_barrier(0);  // keep the tiles' reads from piling up in registers
    }
    // dC~_s[n] += sum_r B_hat_r[n] Dm(s, r) + a^{s+1} (H_c dy_s)[n]
    F fm[R / 32], fy[kBP / 32];
    load_frags<T, false, CD, R / 32>(Dm, 16 * (wave % (BL / 16)), fm, lane);
    load_frags<T, true, CX, kBP / 32>(Dys, 16 * (wave % (BL / 16)), fy, lane);
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      const int t = wave + NW * i;
      const int n0 = 16 * (t / (BL / 16)), s0 = 16 * (t % (BL / 16));
      if (t >= NCT || n0 >= N) continue;
      const floatx4 v = tmm_b<T, false, CB, R / 32>(Bs, n0, fm, lane);
      const floatx4 w = tmm_b<T, true, CX, kBP / 32>(Hs, n0, fy, lane);
      const int s = s0 + cl;
      const float sc = s < Lc ? pw[s + 1] : 0.f;
      const float wt = s < Lc ? (float)(s + 1) * pw[s] : 0.f;
      const floatx4 cq = lds_get4<T, CB>(Cs, s, n0 + 4 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) dap += wt * uHdy * w[q] * cq[q];
      dCa[i] = dCa[i] + v * udy + w * (sc * uHdy);
      __builtin_amdgcn_sched_barrier(0);
    }
    // da of this (sequence, chunk, head): wave sums, then the waves in order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dap += __shfl_xor(dap, off);
    if (lane == 0) red[wave] = dap;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = red[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w];
      A.da_part[((size_t)b * A.nb + c) * H + h] = s;
    }
  }

  // dB_hat and dC~ of the chunk, summed over the slice's heads
  const int g = lane0 >> 4, cl = lane0 & 15;
  float* dB = HS > 1 ? A.dBp + (size_t)slice * ((size_t)Tl * gridDim.z * KS * G * N) : A.dB;
  float* dC = HS > 1 ? A.dCp + (size_t)slice * ((size_t)Tl * gridDim.z * G * N) : A.dC;
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int t = wave + NW * i;
    const int n0 = 16 * (t / (R / 16)), r0 = 16 * (t % (R / 16));
    const int r = r0 + cl;
    if (t >= NBT || n0 >= N || r / KS >= Lc) continue;
    *reinterpret_cast<floatx4*>(dB + ((m0 * KS + r) * G + grp) * N + n0 + 4 * g) = dBa[i];
  }
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int t = wave + NW * i;
    const int n0 = 16 * (t / (BL / 16)), s0 = 16 * (t % (BL / 16));
    const int s = s0 + cl;
    if (t >= NCT || n0 >= N || s >= Lc) continue;
    *reinterpret_cast<floatx4*>(dC + ((m0 + s) * G + grp) * N + n0 + 4 * g) = dCa[i];
  }
}

// dB_hat and dC~ from the head slices' parts, slices in order (float4 units;
// the first nb4 units are dB_hat's, the rest dC~'s).
__global__ void bwd_slice_sum_kernel(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                     float* __restrict__ dB, float* __restrict__ dC, size_t nb4,
                                     size_t nc4, int hs) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (q >= nb4 + nc4) return;
  const bool isb = q < nb4;
  const size_t i = isb ? q : q - nb4, n4 = isb ? nb4 : nc4;
  const floatx4* src = reinterpret_cast<const floatx4*>(isb ? dBp : dCp);
  floatx4 s = src[i];
  for (int k = 1; k < hs; ++k) s = s + src[(size_t)k * n4 + i];
  reinterpret_cast<floatx4*>(isb ? dB : dC)[i] = s;
}

// da[h] = sum over sequences and chunks: one wave per head, lane j summing
// the parts j, j + 64, ... in order, then a fixed butterfly over the lanes.
__global__ void bwd_da_kernel(const float* __restrict__ part, float* __restrict__ da, int Bt,
                              int nb, int H) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const int n = Bt * nb;
  float s = 0.f;
  for (int i = lane; i < n; i += 64) s += part[(size_t)i * H + h];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) da[h] = s;
}

// ---------------------------------------------------------------- launch

int scan_bwd_block(bool is_bf16) { return is_bf16 ? 64 : 32; }

// Slices of each group's heads: the fewest (a divisor of the group's heads)
// that give the gradient kernel at least 1024 workgroups.
int scan_bwd_slices(bool is_bf16, int Bt, int T, int H, int G) {
  const int BL = scan_bwd_block(is_bf16);
  const long base = (long)((T + BL - 1) / BL) * G * Bt;
  const int HG = H / G;
  for (int d = 1; d <= HG; ++d)
    if (HG % d == 0 && base * d >= 1024) return d;
  return HG;
}

// Workspace: H_c and F_c in the local-state type (fp16 rows for bf16 problems)
// with one fp32 factor per row of P elements (Hu, Fu), the local states S_c
// and R_c (same type) with their per-(chunk, head) factors, da's parts, and
// the head slices' dB_hat / dC~ parts.
struct BwdWs {
  size_t H, F, Hu, Fu, Sl, Rl, Su, Ru, dap, parts, total;
};

static BwdWs bwd_ws(bool is_bf16, int Bt, int T, int H, int G, int N, int k) {
  const int BL = scan_bwd_block(is_bf16);
  const size_t nb = (size_t)((T + BL - 1) / BL);
  const size_t al = 255;
  auto up = [&](size_t x) { return (x + al) & ~al; };
  const size_t elems = (size_t)Bt * nb * H * N * kBP;
  const size_t les = is_bf16 ? 2 : 4;  // local-state element bytes
  const int hs = scan_bwd_slices(is_bf16, Bt, T, H, G);
  const size_t M = (size_t)Bt * T;
  BwdWs w{};
  size_t off = 0;
  w.H = off; off += up(elems * les);
  w.F = off; off += up(elems * les);
  w.Hu = off; off += up((size_t)Bt * nb * H * N * 4);
  w.Fu = off; off += up((size_t)Bt * nb * H * N * 4);
  w.Sl = off; off += up(elems * les);
  w.Rl = off; off += up(elems * les);
  w.Su = off; off += up((size_t)Bt * nb * H * 4);
  w.Ru = off; off += up((size_t)Bt * nb * H * 4);
  w.dap = off; off += up((size_t)Bt * nb * H * 4);
  w.parts = off;
  off += up(hs > 1 ? (size_t)hs * (M * k * G * N + M * G * N) * sizeof(float) : 0);
  w.total = off;
  return w;
}

size_t scan_bwd_ws_bytes(bool is_bf16, int Bt, int T, int H, int G, int N, int k) {
  return bwd_ws(is_bf16, Bt, T, H, G, N, k).total;
}

template <typename T, typename S, typename TY, int NP, int KS, int BL>
static hipError_t launch_bwd_t(const BwdArgs& A, int Bt, hipStream_t s) {
  const dim3 g1((unsigned)A.nb, (unsigned)A.H, (unsigned)Bt);
  prof_begin("scan_bwd_local", s);
  hipLaunchKernelGGL((bwd_local_kernel<T, S, TY, NP, KS, BL>), g1, dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("scan_bwd_sweep", s);
  {
    // 16 bytes of local state per thread, or 4 elements when that leaves
    // fewer than 128K threads for the walk
    constexpr int V16 = 16 / (int)sizeof(T);
    const bool narrow = (size_t)Bt * A.H * A.N * kBP / V16 < (size_t)131072;
    const int V = narrow ? 4 : V16;
    const dim3 gs((unsigned)((A.N * kBP / V + 255) / 256), A.H, Bt);
    if (narrow) hipLaunchKernelGGL((bwd_sweep_kernel<T, BL, 4>), gs, dim3(256), 0, s, A);
    else hipLaunchKernelGGL((bwd_sweep_kernel<T, BL, V16>), gs, dim3(256), 0, s, A);
  }
  prof_end(s);
  prof_begin("scan_bwd_grad", s);
  hipLaunchKernelGGL((bwd_grad_kernel<T, S, TY, NP, KS, BL>),
                     dim3((unsigned)A.nb, (unsigned)(A.G * A.hs), (unsigned)Bt),
                     dim3(64 * kGradWaves), 0, s, A);
  prof_end(s);
  if (A.hs > 1) {
    const size_t M = (size_t)Bt * A.T;
    const size_t nb4 = M * A.k * A.G * A.N / 4, nc4 = M * A.G * A.N / 4;
    prof_begin("scan_bwd_slice_sum", s);
    hipLaunchKernelGGL(bwd_slice_sum_kernel, dim3((unsigned)((nb4 + nc4 + 255) / 256)),
                       dim3(256), 0, s, A.dBp, A.dCp, A.dB, A.dC, nb4, nc4, A.hs);
    prof_end(s);
  }
  prof_begin("scan_bwd_da", s);
  hipLaunchKernelGGL(bwd_da_kernel, dim3((unsigned)A.H), dim3(64), 0, s, A.da_part, A.da, Bt,
                     A.nb, A.H);
  prof_end(s);
  return hipGetLastError();
}

template <typename T, typename S, typename TY, int NP>
static hipError_t launch_bwd_np(const BwdArgs& A, int Bt, hipStream_t s) {
  constexpr int BL = sizeof(T) == 2 ? 64 : 32;
  if (A.k == 1) return launch_bwd_t<T, S, TY, NP, 1, BL>(A, Bt, s);
  return launch_bwd_t<T, S, TY, NP, 2, BL>(A, Bt, s);
}

template <typename T, typename S, typename TY>
static hipError_t launch_bwd_ty(const BwdArgs& A, int Bt, hipStream_t s) {
  if (A.N <= 32) return launch_bwd_np<T, S, TY, 32>(A, Bt, s);
  if (A.N <= 64) return launch_bwd_np<T, S, TY, 64>(A, Bt, s);
  return launch_bwd_np<T, S, TY, 128>(A, Bt, s);
}

__global__ void bwd_empty_kernel(const float* __restrict__ dh_final, float* __restrict__ dh_init,
                                 float* __restrict__ da, size_t n, int H) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (dh_init && i < n) dh_init[i] = dh_final ? dh_final[i] : 0.f;
  if (i < (size_t)H) da[i] = 0.f;
}

hipError_t launch_scan_backward(bool is_bf16, int Bt, int T, int H, int G, int N, int k,
                                const void* B_hat, const void* X_hat, const void* C_mix,
                                const void* dy, const float* a, const float* h_init,
                                const float* dh_final, float* dB, float* dX, float* dC, float* da,
                                float* dh_init, void* ws, hipStream_t s) {
  if (Bt == 0) {
    if (H > 0)
      hipLaunchKernelGGL(bwd_empty_kernel, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, s,
                         nullptr, nullptr, da, (size_t)0, H);
    return hipGetLastError();
  }
  if (T == 0) {
    const size_t n = (size_t)Bt * H * N * kBP;
    const size_t m = n > (size_t)H ? n : (size_t)H;
    hipLaunchKernelGGL(bwd_empty_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s,
                       dh_final, dh_init, da, n, H);
    return hipGetLastError();
  }
  const int BL = scan_bwd_block(is_bf16);
  const int nb = (T + BL - 1) / BL;
  const int hs = scan_bwd_slices(is_bf16, Bt, T, H, G);
  const BwdWs w = bwd_ws(is_bf16, Bt, T, H, G, N, k);
  const size_t M = (size_t)Bt * T;
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  float* dBp = reinterpret_cast<float*>(w8 + w.parts);
  float* dCp = dBp + (size_t)hs * M * k * G * N;
  BwdArgs A{B_hat, X_hat, C_mix, dy, a, h_init, dh_final, dB, dX, dC, da, dh_init,
            w8 + w.Sl, w8 + w.Rl, reinterpret_cast<float*>(w8 + w.Su),
            reinterpret_cast<float*>(w8 + w.Ru), w8 + w.H, w8 + w.F,
            reinterpret_cast<float*>(w8 + w.Hu), reinterpret_cast<float*>(w8 + w.Fu),
            reinterpret_cast<float*>(w8 + w.dap), dBp, dCp,
            T, H, G, N, k, nb, hs};
  if (is_bf16) return launch_bwd_ty<f16, f16, bf16>(A, Bt, s);
  return launch_bwd_ty<float, float, float>(A, Bt, s);
}

}  // namespace swimba
