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
// same bits); the pairs come sorted by expert from the bucketing, and dz and
// the pairs' token rows of u are materialised in that order so both grouped
// GEMMs read contiguous rows. GEMM operands bf16 (fp32 for fp32 problems),
// fp32 accumulation, fp32 outputs; every sum over slots, tokens or splits
// runs in a fixed order.
#include "common.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace swimba {

// ---------------------------------------------------------------- dz and dw

// One wave per sorted pair: dz and the pair's token row of u in sorted order,
// and the pair's share of the router gradient s_j = w_j dw_j = <w B_j,
// dB_hat_j> + <w C_j, dC~> (the weighted streams are what the forward keeps,
// so no division by w).
template <typename T, typename S>
__global__ __launch_bounds__(256) void pbwd_dz_kernel(ProjBwdArgs A) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int pairs = A.M * A.k;
  if (i >= pairs) return;
  const int p = A.sorted[i], m = p / A.k;
  const float wj = A.sorted_w[i];
  T* row = static_cast<T*>(A.dz) + (size_t)i * A.W;
  // four columns per lane (H*P and G*N are multiples of 4, so a group of
  // four never straddles the X | B | C boundaries)
  for (int c = 4 * lane; c < A.W; c += 256) {
    floatx4 v;
    if (c < A.HP) {
      v = *reinterpret_cast<const floatx4*>(A.dX + (size_t)p * A.HP + c);
    } else if (c < A.HP + A.GN) {
      v = *reinterpret_cast<const floatx4*>(A.dB + (size_t)p * A.GN + (c - A.HP)) * wj;
    } else {
      v = *reinterpret_cast<const floatx4*>(A.dC + (size_t)m * A.GN + (c - A.HP - A.GN)) * wj;
    }
    typename Vec<T>::x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = from_f32<T>(v[j]);
    *reinterpret_cast<typename Vec<T>::x4*>(row + c) = o;
  }
  // the pair's token row of u, in sorted order (the dW GEMM's B operand)
  {
    const int4v* src = reinterpret_cast<const int4v*>(static_cast<const T*>(A.u) + (size_t)m * A.D);
    int4v* dst = reinterpret_cast<int4v*>(static_cast<T*>(A.us) + (size_t)i * A.D);
    for (int q = lane; q < A.D * (int)sizeof(T) / 16; q += 64) dst[q] = src[q];
  }
  float sum = 0.f;
  const S* bh = static_cast<const S*>(A.B_hat) + (size_t)p * A.GN;
  for (int n = 4 * lane; n < A.GN; n += 256) {
    const floatx4 db = *reinterpret_cast<const floatx4*>(A.dB + (size_t)p * A.GN + n);
    const floatx4 cp = *reinterpret_cast<const floatx4*>(A.c_part + (size_t)p * A.GN + n);
    const floatx4 dc = *reinterpret_cast<const floatx4*>(A.dC + (size_t)m * A.GN + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) sum += to_f32(bh[n + j]) * db[j] + cp[j] * dc[j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) A.sw[p] = sum;
}

// ---------------------------------------------------------------- router

// Router gradient, 32 tokens per workgroup. Phase 1, a group of sg lanes
// per token (sg a power of two with E <= 4 sg; lane l of a group holds
// experts l, l + sg, l + 2 sg, l + 3 sg), so a wave covers 64 / sg tokens per
// pass: pi = softmax(logits), q_e = pi_e dpi_e (the sum of s_j over the slots
// routed to e), dg_e = q_e - pi_e sum_f q_f, into LDS and dg; the group's sums
// run in a fixed butterfly order. Phase 2, threads over d: du[t, d] =
// sum_e dg[t, e] W_r[e, d] for the 32 tokens, each router element read once
// per workgroup (du is initialised here).
constexpr int kRouterTok = 32;

template <typename T>
__global__ __launch_bounds__(256) void pbwd_router_kernel(ProjBwdArgs A) {
  __shared__ float sdg[kRouterTok][257];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouterTok;
  const int E = A.E;
  int sg = 1;
  while (4 * sg < E) sg *= 2;
  const int tpp = 64 / sg, sl = lane % sg;
  for (int tl = wave * tpp + lane / sg; tl < kRouterTok; tl += 4 * tpp) {
    const int m = t0 + tl;
    const bool ok = m < A.M;
    float pi[4], q[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = sl + sg * r;
      pi[r] = (ok && e < E) ? A.logits[(size_t)m * E + e] : -INFINITY;
      mx = fmaxf(mx, pi[r]);
      q[r] = 0.f;
      if (ok && e < E)
        for (int j = 0; j < A.k; ++j)
          if (A.idx[(size_t)m * A.k + j] == e) q[r] += A.sw[(size_t)m * A.k + j];
    }
    for (int off = sg >> 1; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, sg));
    float se = 0.f, sq = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pi[r] = (ok && sl + sg * r < E) ? expf(pi[r] - mx) : 0.f;
      se += pi[r];
      sq += q[r];
    }
    for (int off = sg >> 1; off > 0; off >>= 1) {
      se += __shfl_xor(se, off, sg);
      sq += __shfl_xor(sq, off, sg);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = sl + sg * r;
      if (e < E) {
        const float g = ok ? q[r] - (pi[r] / se) * sq : 0.f;
        sdg[tl][e] = g;
        if (ok) A.dg[(size_t)m * E + e] = g;
      }
    }
  }
  __syncthreads();
  const T* wr = static_cast<const T*>(A.w_router);
  const int nt = min(kRouterTok, A.M - t0);
  for (int d = threadIdx.x; d < A.D; d += 256) {
    float acc[kRouterTok];
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) acc[t] = 0.f;
    for (int e = 0; e < E; ++e) {
      const float w = to_f32(wr[(size_t)e * A.D + d]);
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t) acc[t] += sdg[t][e] * w;
    }
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t)
      if (t < nt) A.du[(size_t)(t0 + t) * A.D + d] = acc[t];
  }
}

// ---------------------------------------------------------------- grouped GEMMs

// 128 x 128 output tiles, four waves of 64 x 64 each. Tiles go from HBM to
// LDS by buffer-to-LDS copies into a ring of stages, issued ahead of the
// products that read them; each lane's part of a
// copy's offset is planned once and the K step enters as the copy's scalar
// offset (every operand is a strided run of rows).
//   MODE 0 (du): rows = one expert's sorted pairs, columns = d, K = w:
//     A(i, w) = dz[i][w] (tile [row][k], read along rows),
//     B(w, d) = W^(e)[w][d] (tile [k][col], read with the transposing read).
//   MODE 1 (dW): rows = w, columns = d, K = the expert's sorted pairs:
//     A(w, i) = dz[i][w], B(i, d) = us[i][d] (both tiles [k][row]).
// The buffer of a MODE 1 operand ends at the expert's last pair, so the rows
// of a partial last K step read zeros; the K steps past the end of a turn of
// the ring read zeros or are not multiplied.
constexpr int kGB = 128;

// MODE 0 takes K steps of 64 (its dz rows then arrive as 128-byte segments)
// in a ring of two stages; MODE 1 K steps of 32 in a ring of four.
template <typename T, int MODE>
struct GemmTiles {
  static constexpr int BK = MODE == 0 ? 64 : 32, NS = MODE == 0 ? 2 : 4;
  static constexpr int ES = sizeof(T), EPC = 16 / ES;  // bytes, elements per 16-byte chunk
  static constexpr int ACPR = MODE == 0 ? BK / EPC : kGB / EPC;  // chunks per LDS row
  static constexpr int AROWS = MODE == 0 ? kGB : BK;
  static constexpr int BCPR = kGB / EPC, BROWS = BK;
  static constexpr int AB = AROWS * ACPR * 16, BB = BROWS * BCPR * 16, STAGE = AB + BB;
  static constexpr int MA = AROWS * ACPR / 256, MB = BROWS * BCPR / 256;  // copies per wave
  static constexpr int CPW = MA + MB;
};

template <typename T, int MODE>
__global__ __launch_bounds__(256) void pbwd_gemm_kernel(ProjBwdArgs A) {
  typedef typename Vec<T>::x8 F;
  typedef GemmTiles<T, MODE> G;
  constexpr int ACPR = G::ACPR, BCPR = G::BCPR;
  constexpr uint32_t ES = G::ES;
  // stage arrays (NS of them are used): copies into one are known not to
  // touch the others
  __shared__ __align__(16) unsigned char stg0[G::STAGE];
  __shared__ __align__(16) unsigned char stg1[G::STAGE];
  __shared__ __align__(16) unsigned char stg2[G::NS == 4 ? G::STAGE : 16];
  __shared__ __align__(16) unsigned char stg3[G::NS == 4 ? G::STAGE : 16];

  const int E = A.E, D = A.D, W = A.W;
  const int ncol = (D + kGB - 1) / kGB;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so XCD x
  // takes the contiguous logical range [x per, (x + 1) per) of the units,
  // which run row tile by row tile (all column tiles of one row tile
  // together): an XCD's workgroups share dz rows and one expert's weights
  // (du), or one expert's dz and token rows (dW), in its L2.
  int units;
  if constexpr (MODE == 0) {
    int nt = 0;
    for (int q = 0; q < E; ++q) nt += (A.offsets[q + 1] - A.offsets[q] + kGB - 1) / kGB;
    units = nt * ncol;
  } else {
    units = E * ((W + kGB - 1) / kGB) * ncol;
  }
  const int per = (units + 7) / 8, slot = blockIdx.x / 8;
  const int logical = (blockIdx.x % 8) * per + slot;
  if (slot >= per || logical >= units) return;
  int e = -1, r0 = 0, nrows = 0, c0 = 0;  // expert, first row, rows, first column
  int kbeg = 0, klen = 0;                  // MODE 1: the expert's sorted pair range
  if constexpr (MODE == 0) {
    int t = logical / ncol;
    c0 = (logical % ncol) * kGB;
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
    e = logical / (nwt * ncol);
    const int rem = logical % (nwt * ncol);
    r0 = (rem / ncol) * kGB;
    c0 = (rem % ncol) * kGB;
    nrows = min(kGB, W - r0);
    kbeg = A.offsets[e];
    klen = A.offsets[e + 1] - kbeg;
  }
  const T* dz = static_cast<const T*>(A.dz);
  const int pairs = A.M * A.k;
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- operands: buffers, planned lane offsets, and the bytes one K step moves
  BufRes rA, rB;
  uint32_t aoff[G::MA], boff[G::MB];
  uint32_t astep, bstep;
  if constexpr (MODE == 0) {
    const T* we = static_cast<const T*>(A.w_experts) + (size_t)e * W * D;
    rA = make_rsrc(dz + (size_t)r0 * W, (uint64_t)(pairs - r0) * W * ES);
    rB = make_rsrc(we + c0, (uint64_t)((size_t)W * D - c0) * ES);
    dma_plan<G::AROWS, ACPR>((uint32_t)W * ES, wave, lane,
                             [](int r) { return swz_row<T, ACPR>(r); }, aoff);
    astep = G::BK * ES;
    bstep = G::BK * (uint32_t)D * ES;
  } else {
    const T* us = static_cast<const T*>(A.us);
    // (an expert without pairs gets empty buffers: every read is zero)
    const size_t na = (size_t)klen * W, nb = (size_t)klen * D;
    rA = make_rsrc(dz + (size_t)kbeg * W + r0, (uint64_t)(na > (size_t)r0 ? na - r0 : 0) * ES);
    rB = make_rsrc(us + (size_t)kbeg * D + c0, (uint64_t)(nb > (size_t)c0 ? nb - c0 : 0) * ES);
    dma_plan<G::AROWS, ACPR>((uint32_t)W * ES, wave, lane,
                             [](int r) { return swz_tr<T, ACPR>(r); }, aoff);
    astep = G::BK * (uint32_t)W * ES;
    bstep = G::BK * (uint32_t)D * ES;
  }
  dma_plan<G::BROWS, BCPR>((uint32_t)D * ES, wave, lane,
                           [](int r) { return swz_tr<T, BCPR>(r); }, boff);
  auto fetch = [&](unsigned char* st, int kt) {
    dma_tile_full<G::AROWS, ACPR>(rA, (uint32_t)kt * astep, aoff, st, wave);
    dma_tile_full<G::BROWS, BCPR>(rB, (uint32_t)kt * bstep, boff, st + G::AB, wave);
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](const unsigned char* st) {
    const unsigned char* As = st;
    const unsigned char* Bs = st + G::AB;
#pragma unroll
    for (int ks = 0; ks < G::BK; ks += 32) {
      F bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = load_kmajor<T, BCPR>(Bs, ks, wn * 64 + 16 * j, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        F af;
        const int row = wm * 64 + 16 * i;
        if constexpr (MODE == 0) {
          // lane (g, c): k = ks + 8g .. ks + 8g + 7 of row row + c
          const int r = row + cl;
          if constexpr (ES == 2)
            af = load8<T>(reinterpret_cast<const T*>(
                As + (r * ACPR + (((ks >> 3) + g) ^ swz_row<T, ACPR>(r))) * 16));
          else
            af = load8<T>(reinterpret_cast<const T*>(As + r * ACPR * 16 + (ks + 8 * g) * 4));
        } else {
          af = load_kmajor<T, ACPR>(As, ks, row, lane);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma16(af, bf[j], acc[i][j]);
      }
    }
  };

  const int nk = (klen + G::BK - 1) / G::BK;
  if constexpr (G::NS == 4) {
    // whole turns of the four stages, every copy unconditional (steps past
    // the end read zeros or are not multiplied)
    const int nk4 = (nk + 3) / 4 * 4;
    fetch(stg0, 0);
    fetch(stg1, 1);
    fetch(stg2, 2);
    auto iter = [&](int kt, const unsigned char* cur, unsigned char* far) {
      wait_vm<2 * G::CPW>();  // step kt landed (steps kt + 1, kt + 2 may be in flight)
      stage_barrier();        // step kt visible to all waves; step kt - 1 no longer read
      fetch(far, kt + 3);
      if (kt < nk) compute(cur);
    };
    for (int kt = 0; kt < nk4; kt += 4) {
      iter(kt, stg0, stg3);
      iter(kt + 1, stg1, stg0);
      iter(kt + 2, stg2, stg1);
      iter(kt + 3, stg3, stg2);
    }
  } else {
    // two stages: the copies of step kt + 1 run during the products of step kt
    const int nk2 = (nk + 1) / 2 * 2;
    fetch(stg0, 0);
    auto iter = [&](int kt, const unsigned char* cur, unsigned char* far) {
      wait_vm<0>();     // step kt landed
      stage_barrier();  // step kt visible to all waves; step kt - 1 no longer read
      fetch(far, kt + 1);
      if (kt < nk) compute(cur);
    };
    for (int kt = 0; kt < nk2; kt += 2) {
      iter(kt, stg0, stg1);
      iter(kt + 1, stg1, stg0);
    }
  }
  wait_vm<0>();  // the copies past the end land before the workgroup's LDS is released

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

// du[m] += sum_j du_part[m, j] in slot order, four columns per thread.
__global__ void pbwd_du_sum_kernel(ProjBwdArgs A) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t D4 = A.D / 4;
  if (q >= (size_t)A.M * D4) return;
  const size_t m = q / D4, d = (q % D4) * 4;
  floatx4 s = *reinterpret_cast<const floatx4*>(A.du + m * A.D + d);
  for (int j = 0; j < A.k; ++j)
    s = s + *reinterpret_cast<const floatx4*>(A.du_part + (m * A.k + j) * A.D + d);
  *reinterpret_cast<floatx4*>(A.du + m * A.D + d) = s;
}

// dW_r partials over splits of kDwrTokens tokens: block (column tile of 64,
// split). The split's u columns (all their 16-byte reads in flight at once)
// and, 16 experts at a time, its router gradients are staged in LDS; thread
// (sub, c) takes column c and every fourth token of the split starting at
// sub; the four subs are added in order.
constexpr int kDwrTokens = 256;

template <typename T>
__global__ __launch_bounds__(256) void pbwd_dwr_kernel(ProjBwdArgs A) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CPT = 64 / EPC;              // chunks per token row of the tile
  constexpr int IT = kDwrTokens * CPT / 256; // chunks per thread
  __shared__ float part[4][16][64];
  __shared__ __align__(16) float sdg[kDwrTokens][16];
  __shared__ __align__(16) T su[kDwrTokens][64];
  const int c = threadIdx.x & 63, sub = threadIdx.x >> 6;
  const int d0 = blockIdx.x * 64, d = d0 + c, sp = blockIdx.y;
  const int m0 = sp * kDwrTokens, m1 = min(A.M, m0 + kDwrTokens);
  const T* u = static_cast<const T*>(A.u);
  {
    int4v v[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int q = threadIdx.x + 256 * i;
      const int t = q / CPT, cc = (q % CPT) * EPC;
      v[i] = int4v{0, 0, 0, 0};
      if (m0 + t < m1 && d0 + cc < A.D)
        v[i] = *reinterpret_cast<const int4v*>(u + (size_t)(m0 + t) * A.D + d0 + cc);
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int q = threadIdx.x + 256 * i;
      *reinterpret_cast<int4v*>(&su[q / CPT][(q % CPT) * EPC]) = v[i];
    }
  }
  for (int e0 = 0; e0 < A.E; e0 += 16) {
    __syncthreads();  // su is written; the previous group's sdg and part are read
    for (int q = threadIdx.x; q < kDwrTokens * 16; q += 256) {
      const int t = q / 16, e = e0 + q % 16;
      sdg[t][q % 16] = (m0 + t < m1 && e < A.E) ? A.dg[(size_t)(m0 + t) * A.E + e] : 0.f;
    }
    __syncthreads();
    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll 4
    for (int t = sub; t < m1 - m0; t += 4) {
      const float uv = to_f32(su[t][c]);
      const floatx4* g4 = reinterpret_cast<const floatx4*>(sdg[t]);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const floatx4 gv = g4[q4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * q4 + j] += gv[j] * uv;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) part[sub][q][c] = acc[q];
    __syncthreads();
    for (int q = sub; q < 16; q += 4) {
      if (e0 + q < A.E && d < A.D)
        A.dwr_part[((size_t)sp * A.E + e0 + q) * A.D + d] =
            ((part[0][q][c] + part[1][q][c]) + part[2][q][c]) + part[3][q][c];
    }
  }
}

// dW_r = the splits' partials added in split order; the reads of 16 splits
// are issued together (64-thread workgroups, so that many CUs share the sum).
__global__ __launch_bounds__(64) void pbwd_dwr_sum_kernel(ProjBwdArgs A) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t ED = (size_t)A.E * A.D;
  if (q >= ED) return;
  float s = 0.f;
  int sp = 0;
  for (; sp + 16 <= A.nsplit; sp += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = A.dwr_part[(size_t)(sp + j) * ED + q];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  for (; sp < A.nsplit; ++sp) s += A.dwr_part[(size_t)sp * ED + q];
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

int proj_bwd_splits(int M) { return (M + kDwrTokens - 1) / kDwrTokens; }

template <typename T, typename S>
static hipError_t launch_pbwd_t(const ProjBwdArgs& A, hipStream_t s) {
  const int pairs = A.M * A.k;
  prof_begin("proj_bwd_dz", s);
  hipLaunchKernelGGL((pbwd_dz_kernel<T, S>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("proj_bwd_router", s);
  hipLaunchKernelGGL(pbwd_router_kernel<T>, dim3((unsigned)((A.M + kRouterTok - 1) / kRouterTok)),
                     dim3(256), 0, s, A);
  prof_end(s);
  const int ncol = (A.D + kGB - 1) / kGB;
  // row tiles over all experts: sum_e ceil(n_e / 128) <= pairs / 128 + E
  const int ntr = pairs / kGB + A.E;
  prof_begin("proj_bwd_du", s);
  hipLaunchKernelGGL((pbwd_gemm_kernel<T, 0>), dim3((unsigned)((ntr * ncol + 7) / 8 * 8)),
                     dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("proj_bwd_du_sum", s);
  hipLaunchKernelGGL(pbwd_du_sum_kernel, dim3((unsigned)(((size_t)A.M * A.D / 4 + 255) / 256)),
                     dim3(256), 0, s, A);
  prof_end(s);
  const int nwt = (A.W + kGB - 1) / kGB;
  prof_begin("proj_bwd_dw", s);
  hipLaunchKernelGGL((pbwd_gemm_kernel<T, 1>), dim3((unsigned)((A.E * nwt * ncol + 7) / 8 * 8)),
                     dim3(256), 0, s, A);
  prof_end(s);
  prof_begin("proj_bwd_dwr", s);
  hipLaunchKernelGGL(pbwd_dwr_kernel<T>, dim3((unsigned)((A.D + 63) / 64), (unsigned)A.nsplit),
                     dim3(256), 0, s, A);
  hipLaunchKernelGGL(pbwd_dwr_sum_kernel, dim3((unsigned)(((size_t)A.E * A.D + 63) / 64)),
                     dim3(64), 0, s, A);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_project_backward(bool is_bf16, ProjBwdArgs A, hipStream_t s) {
  A.nsplit = proj_bwd_splits(A.M);
  if (is_bf16) return launch_pbwd_t<bf16, f16>(A, s);
  return launch_pbwd_t<float, float>(A, s);
}

}  // namespace swimba
