// Single-trajectory scan of the Swimba mixer, solved chunk by chunk (SSD).
// (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
// Models", Method, key design 1: h_t = A h_{t-1} + U~_t, Y_t = C~_t^T h_t, one
// state trajectory solved with the chunked SSD algorithm; key design 2: A is
// shared by every expert and every step, here a scalar a_h per head.)
//
// For head h (group g), a chunk of Lc tokens starting at c0 with entering
// state H (N x P, fp32), and (token, slot) pairs r = (s, j) of the chunk:
//   y_t   = a^{t-c0+1} C~_t^T H
//         + sum_{r : s <= t} a^{t-s} (C~_t . B_hat_r) X_r          (intra)
//   H'    = a^{Lc} H + sum_r a^{c0+Lc-1-s} B_hat_r X_r^T          (carry)
// U~_t = sum_j B_hat_{t,j} X_{t,j}^T is never formed: the contraction runs over
// the k-concatenated pair axis (k*BT rows per block of BT tokens).
//
// Work split (MI355X-first rather than the three separate SSD passes of the
// prior art): a workgroup owns (sequence, segment of chunks, head). It walks
// its chunks in order with the state in fp32 registers, so per-chunk states
// never go to HBM. Segments of one sequence run in parallel; their boundary
// states come from two small passes:
//   pass 1: every segment but the last computes its end state from zero
//           (the carry recurrence only) into the workspace;
//   pass 2: per (sequence, head, element), a sequential, coalesced sweep over
//           segments: Hin_0 = h_init, Hin_{s+1} = a^{len_s} Hin_s + S_s;
//   pass 3: every segment recomputes its chunks from Hin_s and writes y; the
//           last segment also writes h_final.
//
// Wave w of the 4 owns output columns p in [16w, 16w+16): its slice of H and of
// the carry lives in matrix-core accumulator layout (rows n, column p), which
// is also the A-operand layout of the readout C~ H once the contraction order
// over n is permuted to {4g..4g+3, 16+4g..16+4g+3} per 32-step (the C~ operand
// is read in the same permuted order). Per block pair (tau, sigma):
//   Gram^T[r, t] = B_hat_r . C~_t          (matrix cores, K = N)
//   Gm[t, r]     = Gram^T[r, t] a^{t-s}, zero above the diagonal (LDS table)
//   y^T         += X^T Gm^T                 (K = pairs)
//   carry       += B_hat^T (decay * X)      (K = pairs, diagonal block only)
#include "common.hpp"
#include "launch.hpp"

namespace swimba {

constexpr int kP = 64;  // head dim served by these kernels

struct ScanArgs {
  const void* B_hat;
  const void* X_hat;
  const void* C_mix;
  const float* a;
  const float* h_init;
  void* y;
  float* h_final;
  float* ws;  // [Bt, segs, H, N, P] fp32 segment states
  int T, H, G, N, k, L, segs, seg_chunks;
};

template <typename T, int NP, int KS, int BT, bool WITH_Y>
struct ScanLds {
  static constexpr int R = KS * BT;      // pair rows per block
  static constexpr int LDN = NP + 8;     // row stride of [.][n] buffers
  static constexpr int LDR = R + 8;      // row stride of [.][r] buffers
  static constexpr int CS = WITH_Y ? BT * LDN : 0;
  static constexpr int BS = WITH_Y ? R * LDN : 0;
  static constexpr int BST = NP * LDR;
  static constexpr int XST = kP * LDR;
  static constexpr int GM = WITH_Y ? BT * LDR : 0;
  static constexpr int ELEMS = CS + BS + BST + XST + GM;
  static size_t bytes(int L) { return (size_t)ELEMS * sizeof(T) + (size_t)(L + 1) * sizeof(float); }
};

template <typename T, typename TY, int NP, int KS, int BT, bool WITH_Y>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs A, int pass) {
  typedef ScanLds<T, NP, KS, BT, WITH_Y> Lay;
  constexpr int R = Lay::R, LDN = Lay::LDN, LDR = Lay::LDR;
  constexpr int NT = NP / 16;  // 16-row tiles of the state
  typedef typename Vec<T>::x8 F;
  typedef typename Vec<T>::x4 F4;

  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* Cs = reinterpret_cast<T*>(lds_raw);
  T* Bs = Cs + Lay::CS;
  T* BsT = Bs + Lay::BS;
  T* XsT = BsT + Lay::BST;
  T* Gm = XsT + Lay::XST;
  float* pw = reinterpret_cast<float*>(Gm + Lay::GM);

  const int h = blockIdx.x, seg = blockIdx.y, b = blockIdx.z;
  const int H = A.H, G = A.G, N = A.N, L = A.L, Tlen = A.T;
  const int grp = h / (H / G);
  const int GN = G * N;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, c = lane & 15;
  const int pcol = 16 * wave + c;  // this lane's state column

  const T* Bh = reinterpret_cast<const T*>(A.B_hat);
  const T* Xh = reinterpret_cast<const T*>(A.X_hat);
  const T* Cm = reinterpret_cast<const T*>(A.C_mix);
  const size_t tok_base = (size_t)b * Tlen;
  const size_t NPsz = (size_t)N * kP;

  const float ah = A.a[h];
  for (int j = threadIdx.x; j <= L; j += 256) pw[j] = pow_int(ah, j);

  // Entering state of this segment.
  floatx4 Hr[NT], Sn[NT];
  {
    const float* src = nullptr;
    if (!WITH_Y) {
      src = nullptr;  // pass 1 starts from zero
    } else if (A.segs == 1) {
      src = A.h_init;
      if (src) src += ((size_t)b * H + h) * NPsz;
    } else {
      src = A.ws + (((size_t)b * A.segs + seg) * H + h) * NPsz;
    }
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * ni + 4 * g4 + i;
        Hr[ni][i] = (src && n < N) ? src[(size_t)n * kP + pcol] : 0.f;
      }
      Sn[ni] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int nc = (Tlen + L - 1) / L;
  const int ch0 = seg * A.seg_chunks;
  const int ch1 = min(nc, ch0 + A.seg_chunks);

  for (int ch = ch0; ch < ch1; ++ch) {
    const int c0 = ch * L;
    const int Lc = min(L, Tlen - c0);
    const int nb = (Lc + BT - 1) / BT;

    // The entering state as a matrix-core operand. In fp16 it is first scaled
    // by 2^-e (per wave, e >= 0 chosen from the wave's max |H|) so that it stays
    // below 2^14; the readout is multiplied back by 2^e in fp32.
    F hfrag[NT / 2];
    float hscale = 1.f;
    if (WITH_Y) {
      float hin = 1.f;
      if (sizeof(T) == 2) {
        float m = 0.f;
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Hr[ni][i]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        int e = 0;
        if (m > 16384.f) e = (int)ceilf(log2f(m * (1.f / 16384.f)));
        hin = ldexpf(1.f, -e);
        hscale = ldexpf(1.f, e);
      }
#pragma unroll
      for (int q = 0; q < NT / 2; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hfrag[q][i] = from_f32<T>(Hr[2 * q][i] * hin);
          hfrag[q][4 + i] = from_f32<T>(Hr[2 * q + 1][i] * hin);
        }
      }
    }

    for (int tau = WITH_Y ? 0 : nb - 1; tau < nb; ++tau) {
      floatx4 accY[BT / 16];
      const int sig0 = WITH_Y ? 0 : 0;
      const int sig1 = WITH_Y ? tau : nb - 1;
      for (int sig = sig0; sig <= sig1; ++sig) {
        const bool diag = WITH_Y ? (sig == tau) : true;
        __syncthreads();  // previous users of the LDS buffers are done
        // ---- stage C~ of block tau (first sigma only)
        if (WITH_Y && sig == 0) {
          for (int q = threadIdx.x; q < BT * (NP / 8); q += 256) {
            const int t = q / (NP / 8), n0 = 8 * (q % (NP / 8));
            const int tl = tau * BT + t;
            F v = zero8<T>();
            if (tl < Lc && n0 < N) v = load8<T>(Cm + (tok_base + c0 + tl) * GN + grp * N + n0);
            store8<T>(&Cs[t * LDN + n0], v);
          }
        }
        // ---- stage B_hat (rows and/or transposed) and X^T of block sigma
        for (int q = threadIdx.x; q < (R / 4) * (NP / 8); q += 256) {
          const int r0 = 4 * (q / (NP / 8)), n0 = 8 * (q % (NP / 8));
          F v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = r0 + i, s = r / KS, j = r - s * KS;
            const int sl = sig * BT + s;
            v[i] = zero8<T>();
            if (sl < Lc && n0 < N)
              v[i] = load8<T>(Bh + ((tok_base + c0 + sl) * KS + j) * GN + grp * N + n0);
          }
          if (WITH_Y) {
#pragma unroll
            for (int i = 0; i < 4; ++i) store8<T>(&Bs[(r0 + i) * LDN + n0], v[i]);
          }
          if (diag) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              F4 col = {v[0][e], v[1][e], v[2][e], v[3][e]};
              *reinterpret_cast<F4*>(&BsT[(n0 + e) * LDR + r0]) = col;
            }
          }
        }
        for (int q = threadIdx.x; q < (R / 4) * (kP / 8); q += 256) {
          const int r0 = 4 * (q / (kP / 8)), p0 = 8 * (q % (kP / 8));
          F v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = r0 + i, s = r / KS, j = r - s * KS;
            const int sl = sig * BT + s;
            v[i] = zero8<T>();
            if (sl < Lc) v[i] = load8<T>(Xh + ((tok_base + c0 + sl) * KS + j) * (size_t)H * kP +
                                         (size_t)h * kP + p0);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            F4 col = {v[0][e], v[1][e], v[2][e], v[3][e]};
            *reinterpret_cast<F4*>(&XsT[(p0 + e) * LDR + r0]) = col;
          }
        }
        __syncthreads();

        if (WITH_Y) {
          // ---- readout of the entering state, once per tau
          if (sig == 0) {
#pragma unroll
            for (int tt = 0; tt < BT / 16; ++tt) {
              floatx4 acc = {0.f, 0.f, 0.f, 0.f};
              const T* crow = &Cs[(16 * tt + c) * LDN];
#pragma unroll
              for (int q = 0; q < NT / 2; ++q) {
                F bf = load4x2<T>(crow + 32 * q + 4 * g4, crow + 32 * q + 16 + 4 * g4);
                acc = mma16(hfrag[q], bf, acc);
              }
              const float alpha = pw[min(tau * BT + 16 * tt + c + 1, L)] * hscale;
              accY[tt] = acc * alpha;
            }
          }
          // ---- masked Gram^T tiles -> Gm[t][r]
          constexpr int RT = R / 16, TT = BT / 16;
          for (int tix = wave; tix < RT * TT; tix += 4) {
            const int rt = tix / TT, tt = tix % TT;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NP / 32; ++q) {
              F af = load8<T>(&Bs[(16 * rt + c) * LDN + 32 * q + 8 * g4]);
              F bf = load8<T>(&Cs[(16 * tt + c) * LDN + 32 * q + 8 * g4]);
              acc = mma16(af, bf, acc);
            }
            const int t = 16 * tt + c;
            const int tpos = tau * BT + t;
            F4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rt + 4 * g4 + i;
              const int spos = sig * BT + r / KS;
              const int d = tpos - spos;
              out[i] = from_f32<T>(d >= 0 ? acc[i] * pw[d] : 0.f);
            }
            *reinterpret_cast<F4*>(&Gm[t * LDR + 16 * rt + 4 * g4]) = out;
          }
          __syncthreads();
          // ---- y^T[p, t] += X^T[p, r] Gm[t, r]
#pragma unroll
          for (int tt = 0; tt < BT / 16; ++tt) {
#pragma unroll
            for (int q = 0; q < R / 32; ++q) {
              F af = load8<T>(&XsT[pcol * LDR + 32 * q + 8 * g4]);
              F bf = load8<T>(&Gm[(16 * tt + c) * LDR + 32 * q + 8 * g4]);
              accY[tt] = mma16(af, bf, accY[tt]);
            }
          }
        }
        // ---- carry: Sn[n, p] += sum_r B_hat[r, n] a^{Lc-1-s} X[r, p]
        if (diag) {
#pragma unroll
          for (int q = 0; q < R / 32; ++q) {
            F xf = load8<T>(&XsT[pcol * LDR + 32 * q + 8 * g4]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 32 * q + 8 * g4 + e;
              const int d = Lc - 1 - (sig * BT + r / KS);
              xf[e] = from_f32<T>(d >= 0 ? to_f32(xf[e]) * pw[d] : 0.f);
            }
#pragma unroll
            for (int ni = 0; ni < NT; ++ni) {
              F af = load8<T>(&BsT[(16 * ni + c) * LDR + 32 * q + 8 * g4]);
              Sn[ni] = mma16(af, xf, Sn[ni]);
            }
          }
        }
      }
      if (WITH_Y) {
        // ---- store y for block tau: lane holds y[t = 16tt + c][p = 16w + 4g + i]
        typedef typename Vec<TY>::x4 Y4;
        TY* y = reinterpret_cast<TY*>(A.y);
#pragma unroll
        for (int tt = 0; tt < BT / 16; ++tt) {
          const int tl = tau * BT + 16 * tt + c;
          if (tl < Lc) {
            Y4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = from_f32<TY>(accY[tt][i]);
            *reinterpret_cast<Y4*>(y + (tok_base + c0 + tl) * (size_t)H * kP + (size_t)h * kP +
                                   16 * wave + 4 * g4) = o;
          }
        }
      }
    }
    // ---- chunk end: H <- a^{Lc} H + carry
    const float aL = pw[Lc];
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      Hr[ni] = Hr[ni] * aL + Sn[ni];
      Sn[ni] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // ---- write the end state
  float* dst = nullptr;
  if (!WITH_Y) {
    dst = A.ws + (((size_t)b * A.segs + seg + 1) * H + h) * NPsz;  // slot s+1 holds S_s
  } else if (seg == A.segs - 1 && A.h_final) {
    dst = A.h_final + ((size_t)b * H + h) * NPsz;
  }
  if (dst) {
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * ni + 4 * g4 + i;
        if (n < N) dst[(size_t)n * kP + pcol] = Hr[ni][i];
      }
  }
  (void)pass;
}

// Pass 2: Hin_0 = h_init (or 0), Hin_{s+1} = a^{len_s} Hin_s + S_s, for every
// (sequence, head, element), walking the segments in order. Slot s of the
// workspace holds S_{s-1} on entry (s >= 1) and Hin_s on exit.
__global__ __launch_bounds__(256) void scan_combine_kernel(const float* __restrict__ a,
                                                           const float* __restrict__ h_init,
                                                           float* __restrict__ ws, int H,
                                                           int NPsz, int T, int L, int segs,
                                                           int seg_chunks) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int e4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e4 >= NPsz) return;
  const float ah = a[h];
  floatx4 Hc = {0.f, 0.f, 0.f, 0.f};
  if (h_init) Hc = *reinterpret_cast<const floatx4*>(h_init + ((size_t)b * H + h) * NPsz + e4);
  float* base = ws + (size_t)b * segs * H * NPsz + (size_t)h * NPsz + e4;
  const size_t sstride = (size_t)H * NPsz;
  *reinterpret_cast<floatx4*>(base) = Hc;
  for (int s = 0; s + 1 < segs; ++s) {
    const int t0 = s * seg_chunks * L;
    const int len = min(T, t0 + seg_chunks * L) - t0;
    floatx4* slot = reinterpret_cast<floatx4*>(base + (size_t)(s + 1) * sstride);
    Hc = Hc * pow_int(ah, len) + *slot;
    *slot = Hc;
  }
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                  size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_copy(const float* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0 || src == dst) return hipSuccess;
  prof_begin("state_copy", s);
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src,
                     dst, n);
  prof_end(s);
  return hipGetLastError();
}

ScanGeom scan_geom(int Bt, int T, int H, int G, int N, int P, int k, int L) {
  ScanGeom g{Bt, T, H, G, N, P, k, L, 1, 1};
  const int nc = (T + L - 1) / L;
  if (nc <= 0) return g;
  const int units = Bt * H;
  int want = (1024 + units - 1) / units;
  if (want > nc) want = nc;
  if (want < 1) want = 1;
  g.seg_chunks = (nc + want - 1) / want;
  g.segs = (nc + g.seg_chunks - 1) / g.seg_chunks;
  return g;
}

size_t scan_ws_bytes(const ScanGeom& g) {
  if (g.segs <= 1) return 0;
  return (size_t)g.Bt * g.segs * g.H * g.N * g.P * sizeof(float);
}

template <typename T, typename TY, int NP, int KS, int BT>
static hipError_t launch_scan_t(const ScanGeom& g, const ScanArgs& args, hipStream_t s) {
  auto k3 = scan_kernel<T, TY, NP, KS, BT, true>;
  auto k1 = scan_kernel<T, TY, NP, KS, BT, false>;
  const size_t l3 = ScanLds<T, NP, KS, BT, true>::bytes(g.L);
  const size_t l1 = ScanLds<T, NP, KS, BT, false>::bytes(g.L);
  hipError_t err = hipFuncSetAttribute((const void*)k3, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)l3);
  if (err != hipSuccess) return err;
  err = hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)l1);
  if (err != hipSuccess) return err;
  if (g.segs > 1) {
    prof_begin("scan_segment_state", s);
    hipLaunchKernelGGL(k1, dim3(g.H, g.segs - 1, g.Bt), dim3(256), l1, s, args, 1);
    prof_end(s);
    const int NPsz = g.N * g.P;
    prof_begin("scan_state_pass", s);
    hipLaunchKernelGGL(scan_combine_kernel, dim3((NPsz / 4 + 255) / 256, g.H, g.Bt), dim3(256), 0,
                       s, args.a, args.h_init, args.ws, g.H, NPsz, g.T, g.L, g.segs, g.seg_chunks);
    prof_end(s);
  }
  prof_begin("scan_chunk_output", s);
  hipLaunchKernelGGL(k3, dim3(g.H, g.segs, g.Bt), dim3(256), l3, s, args, 3);
  prof_end(s);
  return hipGetLastError();
}

template <typename T, typename TY, int NP>
static hipError_t dispatch_ks(const ScanGeom& g, const ScanArgs& a, hipStream_t s, bool bt32) {
  if (g.k == 1)
    return bt32 ? launch_scan_t<T, TY, NP, 1, 32>(g, a, s) : launch_scan_t<T, TY, NP, 1, 64>(g, a, s);
  return bt32 ? launch_scan_t<T, TY, NP, 2, 32>(g, a, s) : launch_scan_t<T, TY, NP, 2, 64>(g, a, s);
}

template <typename T, typename TY>
static hipError_t dispatch_np(const ScanGeom& g, const ScanArgs& a, hipStream_t s, bool bt32) {
  const int np = g.N <= 32 ? 32 : (g.N <= 64 ? 64 : 128);
  if (np == 32) return dispatch_ks<T, TY, 32>(g, a, s, bt32);
  if (np == 64) return dispatch_ks<T, TY, 64>(g, a, s, bt32);
  return dispatch_ks<T, TY, 128>(g, a, s, bt32);
}

hipError_t launch_scan(bool is_bf16, const ScanGeom& g, const void* B_hat, const void* X_hat,
                       const void* C_mix, const float* a, const float* h_init, void* y,
                       float* h_final, float* ws, hipStream_t s) {
  if (g.Bt == 0) return hipSuccess;
  if (g.T == 0) {
    if (h_final) return launch_state_copy(h_init, h_final, (size_t)g.Bt * g.H * g.N * g.P, s);
    return hipSuccess;
  }
  ScanArgs args{B_hat, X_hat, C_mix, a, h_init, y, h_final, ws,
                g.T, g.H, g.G, g.N, g.k, g.L, g.segs, g.seg_chunks};
  // bf16 inputs (fp16 streams) use 64-token blocks (32 when the chunk is 32);
  // fp32 always 32, to fit LDS.
  const bool bt32 = !is_bf16 || g.L == 32;
  if (is_bf16) return dispatch_np<f16, bf16>(g, args, s, bt32);
  return dispatch_np<float, float>(g, args, s, bt32);
}

}  // namespace swimba
