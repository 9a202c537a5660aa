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
// the k-concatenated pair axis (k*BT rows per block of BT = 32 tokens).
//
// Kernels (MI355X-first rather than the three separate SSD passes of the prior
// art):
//   scan_gram:   G[t, r] = C~_t . B_hat_r for the block pairs the output walk
//                reads, once per group: it does not depend on the head, so the
//                heads of a group share it instead of recomputing it.
//   pass 1:      (several segments per sequence only) every segment but the
//                last computes its end state from zero, carry recurrence only;
//   pass 2:      per (sequence, head, element), a sequential, coalesced sweep
//                over segments: Hin_0 = h_init, Hin_{s+1} = a^{len_s} Hin_s + S_s;
//   pass 3:      every segment walks its chunks from Hin_s and writes y; the
//                last segment also writes h_final.
// Passes 1 and 3 have two forms. For 2-byte streams, k <= 2 and the shared
// decay (the prefill hot path), two heads of a group share a workgroup of 8
// waves and walk one 32-token block per step (scan_carry_kernel,
// scan_block_kernel, described at their definitions). Otherwise (fp32
// streams, k = 3 or 4, the expert-mixed decay, an odd number of heads per
// group) scan_kernel below walks one head per workgroup:
// a workgroup of passes 1 and 3 is 4 waves and owns (sequence, segment, head);
// wave w owns the head columns p in [16w, 16w + 16). Its slice of the state
// lives in fp32 matrix-core accumulators (rows n, column p) for the whole
// segment, so per-chunk states never go to HBM or LDS: the readout C~ H takes
// its A operand straight from those registers, with the contraction over n
// visited in the order {4g..4g+3, 16+4g..16+4g+3} per 32-step (and the C~
// operand read in the same order). Per block pair (tau, sigma) of a chunk:
//   y^T[p, t]  = a^{t+1} H^T C~^T                  (sigma = 0: readout)
//   y^T[p, t] += X^T (G o decay)^T                 (intra, K = pairs)
//   H[n, p]   += (a^{Lc-1-s} B_hat)^T X            (carry, last block row)
// The carry of every block of a chunk is applied in the chunk's last block
// row, after all readouts of the chunk have used the entering state.
#include <cstdlib>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace swimba {

constexpr int kP = 64;             // head dim served by these kernels
constexpr int kScanThreads = 256;  // 4 waves

struct ScanArgs {
  const void* B_hat;
  const void* X_hat;
  const void* C_mix;
  const float* a;
  const float* h_init;
  void* y;
  float* h_final;
  float* ws;          // [Bt, segs, H, N, P] fp32 segment states
  const void* gram;   // [Bt, nc, G, npairs, BT, k*BT] Gram tiles (stream type)
  const float* ld;    // expert-mixed decay: [Bt, H, T] running log2 decay within each
                      // chunk (inclusive); nullptr for the shared decay a
  int T, H, G, N, k, L, segs, seg_chunks, nc, npairs, Bt;
  int sub;  // pass 1 splits each segment into `sub` pieces of seg_chunks / sub chunks
};

// LDS of the walk: two stages, each holding one step's row-major tiles as they
// arrive from HBM (copied by the buffer-to-LDS path, no registers involved):
//   X   [R][64]   pair rows of this head's X_hat      (every step)
//   B   [R][NP]   pair rows of B_hat                   (last block row: carry)
//   C   [BT][NP]  token rows of C~                     (sigma = 0: readout)
//   G   [BT][R]   the Gram tile of the block pair      (every step)
//   Lam [L]       the chunk's running log2 decay        (every step; expert-mixed decay)
// Rows are sequences of 16-byte chunks; chunk c of row r sits at c ^ swz(r).
template <typename T, int NP, int KS, int BT, bool WITH_Y, bool TV = false>
struct ScanLds {
  static constexpr int R = KS * BT;
  static constexpr int XROW = kP * (int)sizeof(T), BROW = NP * (int)sizeof(T);
  static constexpr int GROW = R * (int)sizeof(T);
  static constexpr int XB = R * XROW, BB = R * BROW;
  static constexpr int CB = WITH_Y ? BT * BROW : 0, GB = WITH_Y ? BT * GROW : 0;
  static constexpr int LB = TV ? 256 * 4 : 0;  // the chunk's running log2 decay (TV)
  static constexpr int XO = 0, BO = XB, CO = XB + BB, GO = XB + BB + CB, LO = GO + GB;
  static constexpr int STAGE = XB + BB + CB + GB + LB;
  static constexpr size_t bytes = 2 * (size_t)STAGE;
};

// a^d for integer d >= 0 from la = log2(a) (la = -1e30 encodes a = 0).
__device__ __forceinline__ float apow(float la, int d) {
  return d == 0 ? 1.f : exp2f((float)d * la);
}
// The same with the bare hardware exp2 (no denormal range reduction: results
// below 2^-126 may come out as zero), for the per-step factors of the walk.
__device__ __forceinline__ float apow_step(float la, int d) {
  return d == 0 ? 1.f : __builtin_amdgcn_exp2f((float)d * la);
}

// Fragments (t-tile tt, pair k-step q) of a diagonal block pair: a fragment is
// zero when every (t, r) in it has s > t; the others get a per-lane mask.
template <int KS, int BT>
struct DiagFrags {
  static constexpr int TT = BT / 16, RQ = KS * BT / 32;  // k-steps of 32 pairs per block
  static constexpr bool zero(int tt, int q) { return 16 * tt + 15 - (32 * q) / KS < 0; }
  static constexpr int index(int tt, int q) {
    int n = 0;
    for (int a = 0; a < TT; ++a)
      for (int b = 0; b < RQ; ++b) {
        if (a == tt && b == q) return zero(a, b) ? -1 : n;
        if (!zero(a, b)) ++n;
      }
    return -1;
  }
  static constexpr int count() {
    int n = 0;
    for (int a = 0; a < TT; ++a)
      for (int b = 0; b < RQ; ++b) n += zero(a, b) ? 0 : 1;
    return n;
  }
};

// One step of the walk over a segment: chunk ch, output block tau, source
// block sig (sig <= tau). Pass 1 visits (ch, sig) with tau = the last block.
struct ScanStep {
  int ch, tau, sig;
};

// Gram tiles G[t, r] = C~[c0 + tau*BT + t] . B_hat[(c0 + sig*BT)*k + r] (fp32
// accumulation, stored in the stream type) for one (block pair, chunk, batch).
template <typename T, int NP, int KS, int BT>
__global__ __launch_bounds__(256) void scan_gram_kernel(const T* __restrict__ B_hat,
                                                        const T* __restrict__ C_mix,
                                                        T* __restrict__ gram, int Tlen, int G,
                                                        int N, int L, int nc, int npairs, int Bt,
                                                        int diag) {
  constexpr int R = KS * BT, TT = BT / 16, RT = R / 16;
  constexpr uint32_t ES = sizeof(T);
  typedef typename Vec<T>::x8 F;
  typedef typename Vec<T>::x4 F4;
  // 1-D grid, dealt XCD-contiguously with (group, block pair) fastest: the
  // tiles of one chunk are computed on one XCD and read its B_hat and C~ rows
  // from that XCD's L2 once.
  // diag: only the diagonal pairs (tau, tau), for the walk one block per step
  const int npw = diag ? L / BT : npairs;  // pairs computed per chunk
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (logical >= G * npw * nc * Bt) return;
  const int grp = logical % G, ip = (logical / G) % npw;
  const int ch = (logical / (G * npw)) % nc, b = logical / (G * npw * nc);
  int tau = 0, sig = 0, pidx = 0;
  if (diag) {
    tau = sig = ip;
    pidx = ip * (ip + 1) / 2 + ip;
  } else {
    pidx = ip;
    while ((tau + 1) * (tau + 2) / 2 <= pidx) ++tau;
    sig = pidx - tau * (tau + 1) / 2;
  }
  const int c0 = ch * L, Lc = min(L, Tlen - c0);
  if (tau * BT >= Lc) return;  // block beyond the (last, partial) chunk
  const int GN = G * N;
  const BufRes rB = make_rsrc(B_hat + (size_t)b * Tlen * KS * GN, (uint64_t)Tlen * KS * GN * ES);
  const BufRes rC = make_rsrc(C_mix + (size_t)b * Tlen * GN, (uint64_t)Tlen * GN * ES);
  const int wave = threadIdx.x >> 6, lane = lane_id(), g4 = lane >> 4, c = lane & 15;
  T* out = gram + ((((size_t)b * nc + ch) * G + grp) * npairs + pidx) * (size_t)(BT * R);
  for (int tix = wave; tix < RT * TT; tix += 4) {
    const int rt = tix / TT, tt = tix % TT;
    const int rl = sig * BT * KS + 16 * rt + c;  // pair row within the chunk
    const int tl = tau * BT + 16 * tt + c;       // token within the chunk
    const uint32_t rrow = (uint32_t)(c0 * KS + rl), trow = (uint32_t)(c0 + tl);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NP / 32; ++q) {
      const int n0 = 32 * q + 8 * g4;
      const F af = load8_buf<T>(rB, (rl < Lc * KS && n0 < N) ? (rrow * GN + grp * N + n0) * ES : kOOB);
      const F bf = load8_buf<T>(rC, (tl < Lc && n0 < N) ? (trow * GN + grp * N + n0) * ES : kOOB);
      acc = mma16(af, bf, acc);
    }
    // lane holds G[t = 16tt + c][r = 16rt + 4g + i]
    F4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[i]);
    *reinterpret_cast<F4*>(&out[(16 * tt + c) * R + 16 * rt + 4 * g4]) = o;
  }
}

// TV: the expert-mixed decay. Every decay factor of a step is 2 to a
// difference of the chunk's running log2 decay Lam (inclusive sums from the
// chunk's first token), split as in the shared-decay walk into a row factor,
// a block scalar and a column factor so that each stays <= 1:
//   token t of block tau, pair row s of block sig < tau:
//     prod_{u=s+1}^{t} a_u = 2^{Lam_t - Lam_send} * 2^{Lam_send - Lam_s}
//   (send = last token of block sig), readout 2^{Lam_t}, carry to the chunk
//   end 2^{Lam_end - Lam_send} * 2^{Lam_send - Lam_s}, H <- 2^{Lam_end} H.
template <typename T, typename TY, int NP, int KS, int BT, bool WITH_Y, bool TV = false>
// Two workgroups per CU where their LDS fits (2-byte streams, k <= 2).
__global__ __launch_bounds__(kScanThreads, sizeof(T) == 2 && KS <= 2 ? 2 : 1) void scan_kernel(ScanArgs A) {
  typedef ScanLds<T, NP, KS, BT, WITH_Y, TV> Lay;
  constexpr int R = Lay::R;
  constexpr int TT = BT / 16, RQ = R / 32, NT = NP / 16, NQ = NP / 32;
  constexpr int XC = Lay::XROW / 16, BC = Lay::BROW / 16, GC = Lay::GROW / 16;  // chunks per row
  typedef DiagFrags<KS, BT> DF;
  constexpr int NDF = DF::count() > 0 ? DF::count() : 1;
  constexpr uint32_t ES = sizeof(T);
  typedef typename Vec<T>::x8 F;

  // two stages, separate arrays: the copies into one are known not to touch the
  // tiles being read from the other
  __shared__ __align__(16) unsigned char stage0[Lay::STAGE];
  __shared__ __align__(16) unsigned char stage1[Lay::STAGE];

  const int H = A.H, G = A.G, N = A.N, L = A.L, Tlen = A.T;
  // 1-D grid over (head, segment, sequence), head fastest, dealt so that XCD x
  // owns the contiguous range [x * per, (x + 1) * per): the heads of one
  // (sequence, segment) share an XCD and walk its chunks together, so the
  // B_hat, C~ and Gram tiles they all read come from that XCD's L2.
  // pass 1 walks the pieces of every segment but the last (sub per segment),
  // pass 3 the segments; the workspace holds one state slot per piece
  // boundary (slot 0: h_init), segment s entering at slot s * sub
  const int nseg = WITH_Y ? A.segs : (A.segs - 1) * A.sub;
  const int nslot = (A.segs - 1) * A.sub + 1;
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (logical >= H * nseg * A.Bt) return;
  const int h = logical % H, seg = (logical / H) % nseg, b = logical / (H * nseg);
  const int grp = h / (H / G);
  const int GN = G * N;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, c = lane & 15;
  const size_t NPsz = (size_t)N * kP;
  const size_t HPsz = (size_t)H * kP;
  const int prow_x = 16 * w + c;  // this lane's head column p

  const float ah = TV ? 1.f : A.a[h];  // TV: the decay comes per token from A.ld
  const float la = ah > 0.f ? log2f(ah) : -1e30f;

  const BufRes rB = make_rsrc(reinterpret_cast<const T*>(A.B_hat) + (size_t)b * Tlen * KS * GN,
                              (uint64_t)Tlen * KS * GN * ES);
  const BufRes rX = make_rsrc(reinterpret_cast<const T*>(A.X_hat) + (size_t)b * Tlen * KS * HPsz,
                              (uint64_t)Tlen * KS * HPsz * ES);
  const BufRes rC = make_rsrc(reinterpret_cast<const T*>(A.C_mix) + (size_t)b * Tlen * GN,
                              (uint64_t)Tlen * GN * ES);
  const BufRes rL = make_rsrc(TV ? A.ld + ((size_t)b * H + h) * Tlen : A.a,
                              TV ? (uint64_t)Tlen * 4 : 0);
  const size_t gtile = (size_t)BT * R;
  const BufRes rG = make_rsrc(
      reinterpret_cast<const T*>(A.gram) + (size_t)b * A.nc * G * A.npairs * gtile,
      WITH_Y ? (uint64_t)A.nc * G * A.npairs * gtile * ES : 0);

  // ---- per-lane decay tables (constant over the segment)
  // er[q][j] = a^{BT-1-s} for the pair row r = 32q + 8g + j of a block (s = r / k):
  // the carry weight of that row relative to the block end, and the row factor
  // of the off-diagonal intra term a^{dblk + t - s} = a^{dblk-(BT-1)} a^t a^{BT-1-s}.
  F er[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) er[q][j] = from_f32<T>(apow(la, BT - 1 - (32 * q + 8 * g4 + j) / KS));
  float at[WITH_Y ? TT : 1];   // a^t of the lane's output token t = 16tt + c
  F dm[WITH_Y ? NDF : 1];      // diagonal block: a^{t-s} for s <= t, else 0
  if (WITH_Y) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) at[tt] = apow(la, 16 * tt + c);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        const int ix = DF::index(tt, q);
        if (ix >= 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int d = 16 * tt + c - (32 * q + 8 * g4 + j) / KS;
            dm[ix][j] = from_f32<T>(d >= 0 ? apow(la, d) : 0.f);
          }
        }
      }
  }

  // ---- entering state of this segment (this wave's columns, accumulator layout)
  floatx4 Hr[NT];
  {
    const float* src = nullptr;
    if (WITH_Y) {
      if (A.segs == 1) {
        src = A.h_init;
        if (src) src += ((size_t)b * H + h) * NPsz;
      } else {
        src = A.ws + (((size_t)b * nslot + seg * A.sub) * H + h) * NPsz;
      }
    }
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * a + 4 * g4 + i;
        Hr[a][i] = (src && n < N) ? src[(size_t)n * kP + prow_x] : 0.f;
      }
  }

  const int nc = A.nc;
  const int span = WITH_Y ? A.seg_chunks : A.seg_chunks / A.sub;  // chunks walked
  const int ch0 = seg * span;
  const int ch1 = min(nc, ch0 + span);
  if (ch0 >= ch1) return;
  auto nblocks = [&](int ch) { return (min(L, Tlen - ch * L) + BT - 1) / BT; };
  auto advance = [&](ScanStep s) {
    if (WITH_Y) {
      if (++s.sig > s.tau) {
        s.sig = 0;
        if (++s.tau == nblocks(s.ch)) { s.tau = 0; ++s.ch; }
      }
    } else {
      if (++s.sig == nblocks(s.ch)) { s.sig = 0; ++s.ch; }
      s.tau = s.ch < ch1 ? nblocks(s.ch) - 1 : 0;
    }
    return s;
  };

  // ---- HBM -> LDS stage for one step (the tiles this step reads). Whole
  // tiles (every row and chunk valid: all but a sequence's last partial chunk,
  // and N = NP) are copied from per-lane offsets planned once, with the tile
  // position as the scalar offset; the others go through the checked copy.
  constexpr int NXI = (R * XC / 64 + 3) / 4, NBI = (R * BC / 64 + 3) / 4;
  constexpr int NCI = (BT * BC / 64 + 3) / 4, NGI = (BT * GC / 64 + 3) / 4;
  uint32_t xoff[NXI], boff[NBI], coff[WITH_Y ? NCI : 1], goff[WITH_Y ? NGI : 1];
  dma_plan<R, XC>((uint32_t)HPsz * ES, w, lane, [](int r) { return swz_tr<T, XC>(r); }, xoff);
  dma_plan<R, BC>((uint32_t)GN * ES, w, lane, [](int r) { return swz_tr<T, BC>(r); }, boff);
  if (WITH_Y) {
    dma_plan<BT, BC>((uint32_t)GN * ES, w, lane, [](int r) { return swz_row<T, BC>(r); }, coff);
    dma_plan<BT, GC>((uint32_t)R * ES, w, lane, [](int r) { return swz_row<T, GC>(r); }, goff);
  }
  const bool nfull = N == NP;
  auto fetch = [&](unsigned char* st, ScanStep s) {
    const int c0 = s.ch * L;
    const int Lc = min(L, Tlen - c0);
    const bool last = s.tau == (Lc + BT - 1) / BT - 1;
    const uint32_t prow = (uint32_t)(c0 + s.sig * BT) * KS;  // first pair row of block sig
    const int rlim = (Lc - s.sig * BT) * KS;                  // valid pair rows in the block
    const bool rows_full = rlim >= R;
    const uint32_t xb = (prow * (uint32_t)HPsz + h * kP) * ES;
    if (rows_full)
      dma_tile_full<R, XC>(rX, xb, xoff, st + Lay::XO, w);
    else
      dma_tile<R, XC>(rX, xb, (uint32_t)HPsz * ES, st + Lay::XO, rlim, XC, w, lane,
                      [](int r) { return swz_tr<T, XC>(r); });
    if (last) {
      const uint32_t bb = (prow * GN + grp * N) * ES;
      if (rows_full && nfull)
        dma_tile_full<R, BC>(rB, bb, boff, st + Lay::BO, w);
      else
        dma_tile<R, BC>(rB, bb, GN * ES, st + Lay::BO, rlim, (int)(N * ES / 16), w, lane,
                        [](int r) { return swz_tr<T, BC>(r); });
    }
    if (WITH_Y) {
      if (s.sig == 0) {
        const uint32_t cb = ((uint32_t)(c0 + s.tau * BT) * GN + grp * N) * ES;
        if (Lc - s.tau * BT >= BT && nfull)
          dma_tile_full<BT, BC>(rC, cb, coff, st + Lay::CO, w);
        else
          dma_tile<BT, BC>(rC, cb, GN * ES, st + Lay::CO, Lc - s.tau * BT, (int)(N * ES / 16), w,
                           lane, [](int r) { return swz_row<T, BC>(r); });
      }
      const int pidx = s.tau * (s.tau + 1) / 2 + s.sig;
      const uint32_t gbase = (uint32_t)((((size_t)s.ch * G + grp) * A.npairs + pidx) * gtile);
      dma_tile_full<BT, GC>(rG, gbase * ES, goff, st + Lay::GO, w);
    }
    if constexpr (TV) {
      // every slot of the chunk's Lam is written (zeros past its last token),
      // so no value of another chunk is left in the stage
      if (64 * w < L) {
        const int tl = 64 * w + lane;
        const uint32_t off = tl < Lc ? (uint32_t)(c0 + tl) * 4u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rL, (__attribute__((address_space(3))) void*)(st + Lay::LO + 256 * w), 4, off, 0, 0,
            0);
      }
    }
  };

  float hin = 1.f, hscale = 1.f;
  floatx4 accY[WITH_Y ? TT : 1];
  bool ypend = false;
  size_t yrow0 = 0;
  int ylim = 0;

  // ---- compute one step from the stage at LDS byte offset st
  auto compute = [&](const unsigned char* st, const ScanStep cur) {
    const unsigned char* Xs = st + Lay::XO;
    const unsigned char* Bs = st + Lay::BO;
    const unsigned char* Cs = st + Lay::CO;
    const unsigned char* Gs = st + Lay::GO;
    const int c0 = cur.ch * L;
    const int Lc = min(L, Tlen - c0);
    const int nb = (Lc + BT - 1) / BT;
    const bool last = cur.tau == nb - 1;
    const bool dg = cur.sig == cur.tau;

    if (WITH_Y && cur.tau == 0 && cur.sig == 0) {
      hin = 1.f;
      hscale = 1.f;
      if (sizeof(T) == 2) {
        // The entering state as an fp16 operand, scaled by 2^-e (e >= 0 from
        // this wave's max |H|) so it stays below 2^14; the readout is
        // multiplied back by 2^e in fp32.
        float mx = 0.f;
#pragma unroll
        for (int a = 0; a < NT; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(Hr[a][i]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (mx > 16384.f) {
          const int e = (int)ceilf(log2f(mx * (1.f / 16384.f)));
          hin = ldexpf(1.f, -e);
          hscale = ldexpf(1.f, e);
        }
      }
    }

    F xq[RQ];  // X^T fragment of this wave's columns: rows r = 32q + 8g + j
#pragma unroll
    for (int q = 0; q < RQ; ++q) xq[q] = load_kmajor<T, XC>(Xs, 32 * q, 16 * w, lane);

    // TV: the step's decay factors from the chunk's running log2 decay (zero
    // past the chunk's last token). ev[q] = 2^{Lam_send - Lam_s} for the pair
    // rows of block sig; lt[tt] = Lam at the lane's output tokens of block tau.
    F ev[TV ? RQ : 1];
    float lt[TV ? TT : 1], l_send = 0.f, l_end = 0.f;
    if constexpr (TV) {
      const float* Ls = reinterpret_cast<const float*>(st + Lay::LO);
      const int sig0 = cur.sig * BT, tau0 = cur.tau * BT;
      l_send = Ls[min(sig0 + BT, Lc) - 1];
      l_end = Ls[Lc - 1];
#pragma unroll
      for (int q = 0; q < RQ; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          ev[q][j] = from_f32<T>(__builtin_amdgcn_exp2f(l_send - Ls[sig0 + (32 * q + 8 * g4 + j) / KS]));
      if (WITH_Y) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) lt[tt] = Ls[tau0 + 16 * tt + c];
      }
    }

    if (WITH_Y) {
      if (cur.sig == 0) {
        // ---- readout of the entering state: y^T[p, t] = H^T[p, n] C~^T[n, t]
        const float ablk =
            TV ? hscale : (cur.tau == 0 ? 1.f : apow_step(la, cur.tau * BT)) * hscale * ah;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) accY[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
        const bool scaled = hin != 1.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          F hf;
          if (scaled) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hf[i] = from_f32<T>(Hr[2 * q][i] * hin);
              hf[4 + i] = from_f32<T>(Hr[2 * q + 1][i] * hin);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hf[i] = from_f32<T>(Hr[2 * q][i]);
              hf[4 + i] = from_f32<T>(Hr[2 * q + 1][i]);
            }
          }
          // the C~ fragments of every token tile first, then the matrix-core ops
          F cf[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            // C~ operand in the same n order: {32q + 4g .. +3, 32q + 16 + 4g .. +3}
            const int t = 16 * tt + c;
            const int n0 = 32 * q + 4 * g4;
            const int e0 = n0 * (int)ES, e1 = (n0 + 16) * (int)ES;
            const int sw = swz_row<T, BC>(t);
            const T* p0 = reinterpret_cast<const T*>(Cs + (t * BC + ((e0 >> 4) ^ sw)) * 16 + (e0 & 15));
            const T* p1 = reinterpret_cast<const T*>(Cs + (t * BC + ((e1 >> 4) ^ sw)) * 16 + (e1 & 15));
            cf[tt] = load4x2<T>(p0, p1);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) accY[tt] = mma16(hf, cf[tt], accY[tt]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          accY[tt] = accY[tt] * ((TV ? __builtin_amdgcn_exp2f(lt[tt]) : at[tt]) * ablk);
      }
      // ---- intra-chunk: y^T[p, t] += X^T[p, r] (G o decay)[t, r]
      auto gfrag = [&](int tt, int q) {
        const int t = 16 * tt + c;
        const int e0 = (32 * q + 8 * g4) * (int)ES;
        const unsigned char* p = Gs + (t * GC + ((e0 >> 4) ^ swz_row<T, GC>(t))) * 16 + (e0 & 15);
        return load8<T>(reinterpret_cast<const T*>(p));
      };
      // Gram fragments: all of a q-step's token tiles read before their
      // matrix-core ops
      if (dg) {
        if constexpr (TV) {
          // a^{t-s} for s <= t as 2^{Lam_t - Lam_s} (zero above the diagonal
          // and for tokens past the chunk)
          const float* Ls = reinterpret_cast<const float*>(st + Lay::LO);
          const int tau0 = cur.tau * BT;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int q = 0; q < RQ; ++q) {
              const int ix = DF::index(tt, q);
              if (ix >= 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                  const int t = 16 * tt + c, sj = (32 * q + 8 * g4 + j) / KS;
                  dm[ix][j] = from_f32<T>((sj <= t && tau0 + t < Lc)
                                              ? __builtin_amdgcn_exp2f(lt[tt] - Ls[tau0 + sj])
                                              : 0.f);
                }
              }
            }
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          F gf[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            if (DF::index(tt, q) >= 0) gf[tt] = gfrag(tt, q);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int ix = DF::index(tt, q);
            if (ix >= 0) accY[tt] = mma16(xq[q], gf[tt] * dm[ix], accY[tt]);
          }
        }
      } else {
        floatx4 tmp[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) tmp[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          F gf[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) gf[tt] = gfrag(tt, q);
          __builtin_amdgcn_sched_barrier(0);
          const F xs = xq[q] * (TV ? ev[q] : er[q]);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) tmp[tt] = mma16(xs, gf[tt], tmp[tt]);
        }
        const float u = TV ? 0.f : apow_step(la, (cur.tau - cur.sig) * BT - (BT - 1));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          accY[tt] = accY[tt] + tmp[tt] * (TV ? __builtin_amdgcn_exp2f(lt[tt] - l_send) : u * at[tt]);
      }
    }
    if (last) {
      // The carry accumulates straight into the state: H <- a^{Lc} H first
      // (after the readouts of this chunk, which all use the entering state).
      if (cur.sig == 0) {
        const float aL = TV ? __builtin_amdgcn_exp2f(l_end) : apow_step(la, Lc);
#pragma unroll
        for (int a = 0; a < NT; ++a) Hr[a] = Hr[a] * aL;
      }
      // ---- carry: H[n, p] += sum_r B_hat[r, n] (a^{Lc-1-s} X[r, p])
      const bool full = TV || Lc == L;  // TV: ev is already relative to the valid rows
      const float blk = TV ? __builtin_amdgcn_exp2f(l_end - l_send) : apow_step(la, (nb - 1 - cur.sig) * BT);
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        F xd;
        if (full) {
          xd = xq[q] * ((TV ? ev[q] : er[q]) * from_f32<T>(blk));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int d = Lc - 1 - (cur.sig * BT + (32 * q + 8 * g4 + j) / KS);
            xd[j] = from_f32<T>(to_f32(xq[q][j]) * (d >= 0 ? apow_step(la, d) : 0.f));
          }
        }
        // B_hat fragments four at a time: their LDS reads are all in flight
        // before the first matrix-core op needs one
        constexpr int CG = NT < 4 ? NT : 4;
#pragma unroll
        for (int a0 = 0; a0 < NT; a0 += CG) {
          F bf[CG];
#pragma unroll
          for (int i = 0; i < CG; ++i) bf[i] = load_kmajor<T, BC>(Bs, 32 * q, 16 * (a0 + i), lane);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < CG; ++i) Hr[a0 + i] = mma16(bf[i], xd, Hr[a0 + i]);
        }
      }
    }
    if (WITH_Y && dg) {
      // y of block tau is complete; it is stored at the start of the next step
      ypend = true;
      yrow0 = (size_t)b * Tlen + c0 + cur.tau * BT;
      ylim = Lc - cur.tau * BT;
    }
  };
  // ---- store the pending y block: lane holds y[t = 16tt + c][p = 16w + 4g + i]
  auto store_y = [&]() {
    if (!WITH_Y || !ypend) return;
    typedef typename Vec<TY>::x4 Y4;
    TY* yb = reinterpret_cast<TY*>(A.y) + yrow0 * HPsz + (size_t)h * kP + 16 * w + 4 * g4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tl = 16 * tt + c;
      if (tl < ylim) {
        Y4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = from_f32<TY>(accY[tt][i]);
        *reinterpret_cast<Y4*>(yb + (size_t)tl * HPsz) = o;
      }
    }
    ypend = false;
  };

  // ---- the walk: the copy of the next step's tiles into the other stage runs
  // while this step computes; one barrier per step. Unrolled by two so that
  // every access names its stage array.
  ScanStep s0{ch0, WITH_Y ? 0 : nblocks(ch0) - 1, 0};
  ScanStep s1 = advance(s0);
  fetch(stage0, s0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](const unsigned char* cur_st, unsigned char* next_st) {
    store_y();
    if (s1.ch < ch1) fetch(next_st, s1);
    compute(cur_st, s0);
    __builtin_amdgcn_s_waitcnt(0);  // the next stage has landed
    __syncthreads();
    s0 = s1;
    if (s1.ch < ch1) s1 = advance(s1);
    return s0.ch < ch1;
  };
  while (step(stage0, stage1) && step(stage1, stage0)) {
  }
  store_y();

  // ---- write the end state
  float* dst = nullptr;
  if (!WITH_Y) {
    dst = A.ws + (((size_t)b * nslot + seg + 1) * H + h) * NPsz;  // slot j+1 holds S_j
  } else if (seg == A.segs - 1 && A.h_final) {
    dst = A.h_final + ((size_t)b * H + h) * NPsz;
  }
  if (dst) {
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * a + 4 * g4 + i;
        if (n < N) dst[(size_t)n * kP + prow_x] = Hr[a][i];
      }
  }
}

// N copies that read nothing (an offset past the buffer) and write 4-byte
// zeros into `sink` (kSinkBytes of LDS): they keep a wave's count of copies in
// flight fixed when a step needs fewer tiles, so that a fixed vmcnt wait still
// covers the previous step's copies. Each goes to its own 256 bytes of the
// sink: identical calls were merged into one by the compiler, which left the
// wait short by N - 1 and let a walk's last two steps read tiles still in
// flight.
constexpr int kSinkBytes = 2048;
template <int N>
__device__ __forceinline__ void dma_dummies(BufRes rs, unsigned char* sink) {
  static_assert(N * 256 <= kSinkBytes, "one 256-byte sink slot per dummy copy");
#pragma unroll
  for (int m = 0; m < N; ++m) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(sink + 256 * m), 4, kOOB, 0, 0, 0);
  }
}

constexpr int kBlockThreads = 512;
// K-major fragments of 2-byte tiles with planned lane offsets: lane (g, c)
// gets rows k0 + 8g .. k0 + 8g + 7 of column col0 + c through two transposing
// reads (as load_kmajor). kmajor_off is the byte offset within the tile of
// the lane's half hh at k0 = 0; the swizzle depends on the row's low four bits
// only, so the read at k0 (a multiple of 32) lies k0 * CPR * 16 bytes further
// on.
template <typename T, int CPR>
__device__ __forceinline__ int kmajor_off(int col0, int hh, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const int r = 8 * g + 4 * hh + (c >> 2);
  const int col = col0 + 4 * (c & 3);
  const int ch = col >> 3, half = (col >> 2) & 1;
  return (r * CPR + (ch ^ swz_tr<T, CPR>(r))) * 16 + 8 * half;
}
// The fragment at lane offsets off[0], off[1] plus kb bytes (a constant). The
// offsets are made opaque to the optimiser once, where they are planned, so
// that each read's LDS address is one step from its stage array: the LDS
// lowering gives an access its alias scope only within a few address steps of
// the variable, and a transposing read without one is taken to alias every
// buffer-to-LDS copy in flight (the compiler then waits for all of them first).
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 load_kmajor_at(const unsigned char* stage,
                                                              const int (&off)[2], int kb) {
  typedef typename Vec<T>::x8 F;
  typedef short s4 __attribute__((__vector_size__(8)));
  F v;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const typename Vec<T>::x4 w4 = __builtin_bit_cast(
        typename Vec<T>::x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                 (__attribute__((address_space(3))) s4*)(stage + off[hh] + kb)));
#pragma unroll
    for (int m = 0; m < 4; ++m) v[4 * hh + m] = w4[m];
  }
  return v;
}

// The output walk one 32-token block per step, two heads per workgroup (8
// waves; the heads share one copy of the group's B_hat, C~ and Gram tiles).
// Every block is its own sub-chunk: the SSD split is exact for any chunk
// length, so block sig's tokens take the cross-block part of y from the state
// after the carry of block sig - 1, and only the diagonal Gram tiles are
// needed. Step s copies block s's X_hat rows (both heads), B_hat rows, C~ rows
// and its diagonal Gram tile, and computes
//   y^T[p, t]  = a^{t+1} H^T C~^T + X^T (G o decay)^T     (readout + intra)
//   H         <- a^{Ls} H + B_hat^T (a^{Ls-1-s} X)         (carry)
// with the readout's fp16 operand converted from the state registers at the
// step's start. Against walking 64-token sub-chunks: no fp16 copy of the
// state in LDS (its writes and reads), no cross-block intra term, half the
// Gram tiles, and the LDS left free holds a third stage, so the copies of
// step s + 2 are in flight while step s computes.
template <typename T, int NP, int KS, int BT>
struct BlockLds {
  static constexpr int R = KS * BT;
  static constexpr int XROW = kP * (int)sizeof(T), BROW = NP * (int)sizeof(T);
  static constexpr int GROW = R * (int)sizeof(T);
  static constexpr int XB = R * XROW, BB = R * BROW, CB = BT * BROW, GB = BT * GROW;
  static constexpr int XO = 0, BO = 2 * XB, CO = BO + BB, GO = CO + CB;
  static constexpr int STAGE = GO + GB;
};

template <typename T, typename TY, int NP, int KS, int BT>
__global__ __launch_bounds__(kBlockThreads, 1) void scan_block_kernel(ScanArgs A) {
  typedef BlockLds<T, NP, KS, BT> Lay;
  constexpr int R = Lay::R;
  constexpr int TT = BT / 16, RQ = R / 32, NT = NP / 16, NQ = NP / 32;
  constexpr int XC = Lay::XROW / 16, BC = Lay::BROW / 16, GC = Lay::GROW / 16;
  typedef DiagFrags<KS, BT> DF;
  constexpr int NDF = DF::count() > 0 ? DF::count() : 1;
  constexpr uint32_t ES = sizeof(T);
  typedef typename Vec<T>::x8 F;
  constexpr int CX = dma_count<2 * R, XC, 8>(), CBn = dma_count<R, BC, 8>();
  constexpr int CCn = dma_count<BT, BC, 8>(), CG = dma_count<BT, GC, 8>();
  constexpr int NCOPY = CX + CBn + CCn + CG;

  __shared__ __align__(16) unsigned char stage0[Lay::STAGE];
  __shared__ __align__(16) unsigned char stage1[Lay::STAGE];
  __shared__ __align__(16) unsigned char stage2[Lay::STAGE];
  __shared__ __align__(16) unsigned char sink[kSinkBytes];

  const int H = A.H, G = A.G, N = A.N, L = A.L, Tlen = A.T;
  const int HU = H / 2;
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (logical >= HU * A.segs * A.Bt) return;
  const int hp = logical % HU, seg = (logical / HU) % A.segs, b = logical / (HU * A.segs);
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w >> 2, wc = w & 3;  // head of the pair, column block of the head
  const int h = 2 * hp + hw;
  const int grp = h / (H / G);
  const int GN = G * N;
  const int g4 = lane >> 4, c = lane & 15;
  const size_t NPsz = (size_t)N * kP;
  const size_t HPsz = (size_t)H * kP;
  const int prow_x = 16 * wc + c;
  // lane offsets of the transposing reads within a stage: this wave's X
  // columns of its head, and the B_hat columns of each 16-wide n tile
  int xo[2], bo[NT][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    xo[hh] = Lay::XO + hw * Lay::XB + kmajor_off<T, XC>(16 * wc, hh, lane);
    asm("" : "+v"(xo[hh]));
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      bo[a][hh] = Lay::BO + kmajor_off<T, BC>(16 * a, hh, lane);
      asm("" : "+v"(bo[a][hh]));
    }
  }
  // lane offsets of the readout's C~ reads within a stage: token t = 16 tt + c,
  // n0 = 32 q + 4 g4 and n0 + 16, four elements each (one opaque offset per
  // read, so that the two tiles' reads are not merged into one whose halves
  // then have to be moved into place)
  int co[TT][NQ][2];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int t = 16 * tt + c;
        const int e0 = (32 * q + 16 * m + 4 * g4) * (int)ES;
        co[tt][q][m] = Lay::CO + (t * BC + ((e0 >> 4) ^ swz_row<T, BC>(t))) * 16 + (e0 & 15);
        asm("" : "+v"(co[tt][q][m]));
      }

  const float ah = A.a[h];
  const float la = ah > 0.f ? log2f(ah) : -1e30f;

  const BufRes rB = make_rsrc(reinterpret_cast<const T*>(A.B_hat) + (size_t)b * Tlen * KS * GN,
                              (uint64_t)Tlen * KS * GN * ES);
  const BufRes rX = make_rsrc(reinterpret_cast<const T*>(A.X_hat) + (size_t)b * Tlen * KS * HPsz,
                              (uint64_t)Tlen * KS * HPsz * ES);
  const BufRes rC = make_rsrc(reinterpret_cast<const T*>(A.C_mix) + (size_t)b * Tlen * GN,
                              (uint64_t)Tlen * GN * ES);
  const size_t gtile = (size_t)BT * R;
  const BufRes rG = make_rsrc(
      reinterpret_cast<const T*>(A.gram) + (size_t)b * A.nc * G * A.npairs * gtile,
      (uint64_t)A.nc * G * A.npairs * gtile * ES);

  // ---- per-lane decay tables: carry a^{BT-1-s} of pair row r = 32q + 8 g4 + j
  // (s = r / k), readout a^t of token t = 16 tt + c, diagonal block a^{t-s}
  F er[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) er[q][j] = from_f32<T>(apow(la, BT - 1 - (32 * q + 8 * g4 + j) / KS));
  float at[TT];
  F dm[NDF];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) at[tt] = apow(la, 16 * tt + c) * ah;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int ix = DF::index(tt, q);
      if (ix >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = 16 * tt + c - (32 * q + 8 * g4 + j) / KS;
          dm[ix][j] = from_f32<T>(d >= 0 ? apow(la, d) : 0.f);
        }
      }
    }
  const float aBT = apow(la, BT);

  // ---- entering state of this segment (this wave's columns)
  floatx4 Hr[NT];
  {
    const float* src = nullptr;
    if (A.segs == 1) {
      src = A.h_init;
      if (src) src += ((size_t)b * H + h) * NPsz;
    } else {
      src = A.ws + (((size_t)b * ((A.segs - 1) * A.sub + 1) + seg * A.sub) * H + h) * NPsz;
    }
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * a + 4 * g4 + i;
        Hr[a][i] = (src && n < N) ? src[(size_t)n * kP + prow_x] : 0.f;
      }
  }

  // the walk goes over the segment's 32-token blocks by their index in the
  // sequence: chunk lengths are multiples of BT, so block j starts at token
  // j * BT, belongs to chunk j / LB and is block j % LB of it
  const int LB = L / BT;  // 1, 2, 4 or 8
  const int lbs = __builtin_ctz((unsigned)LB);
  const int j0 = seg * A.seg_chunks * LB;
  const int j1 = min((Tlen + BT - 1) / BT, (seg + 1) * A.seg_chunks * LB);
  if (j0 >= j1) return;

  // ---- copies of one step into a stage (every wave takes its share of each
  // tile; X of both heads as one tile of 2R rows)
  uint32_t xoff[CX], boff[CBn], coff[CCn], goff[CG];
  int xrow[CX];
#pragma unroll
  for (int m = 0; m < CX; ++m) {
    const int slot = 64 * dma_group<2 * R, XC, 8>(m, w) + lane;
    const int r = slot / XC, pc = slot % XC, rr = r % R;
    xrow[m] = rr;
    xoff[m] = rr * (uint32_t)HPsz * ES + (r / R) * kP * ES + 16 * (pc ^ swz_tr<T, XC>(rr));
  }
  dma_plan_n<R, BC, 8>((uint32_t)GN * ES, w, lane, [](int r) { return swz_tr<T, BC>(r); }, boff);
  dma_plan_n<BT, BC, 8>((uint32_t)GN * ES, w, lane, [](int r) { return swz_row<T, BC>(r); }, coff);
  dma_plan_n<BT, GC, 8>((uint32_t)R * ES, w, lane, [](int r) { return swz_row<T, GC>(r); }, goff);
  const bool nfull = N == NP;

  const uint32_t gpair = (uint32_t)(gtile * ES);                     // one Gram tile
  const uint32_t gbase = (uint32_t)grp * (uint32_t)A.npairs * gpair;  // this group's
  const uint32_t gchunk = (uint32_t)G * (uint32_t)A.npairs * gpair;   // one chunk's
  auto fetch = [&](unsigned char* st, int jb) {
    const int c0 = jb * BT;  // the block's first token
    const int ch = jb >> lbs, sig = jb & (LB - 1);
    const uint32_t prow = (uint32_t)c0 * KS;
    const uint32_t xb = (prow * (uint32_t)HPsz + 2 * hp * kP) * ES;
    const uint32_t bb = (prow * GN + grp * N) * ES;
    const uint32_t cb = ((uint32_t)c0 * GN + grp * N) * ES;
    if (c0 + BT <= Tlen && nfull) {  // a whole block: every row and chunk valid
      int wx = 1024 * dma_group<2 * R, XC, 8>(0, w), wb = 1024 * dma_group<R, BC, 8>(0, w);
      int wcc = 1024 * dma_group<BT, BC, 8>(0, w);
      asm volatile("" : "+s"(wx), "+s"(wb), "+s"(wcc));
      dma_tile_full_w<2 * R, XC, 8>(rX, xb, xoff, st + Lay::XO, wx);
      dma_tile_full_w<R, BC, 8>(rB, bb, boff, st + Lay::BO, wb);
      dma_tile_full_w<BT, BC, 8>(rC, cb, coff, st + Lay::CO, wcc);
    } else {
      const int Ls = min(BT, Tlen - c0);
      const int rlim = Ls * KS;
      if (rlim >= R)
        dma_tile_full_n<2 * R, XC, 8>(rX, xb, xoff, st + Lay::XO, w);
      else
        dma_rows_n<2 * R, XC, 8>(rX, xb, xoff, xrow, rlim, st + Lay::XO, w);
      dma_tile_n<R, BC, 8>(rB, bb, GN * ES, st + Lay::BO, rlim, (int)(N * ES / 16), w, lane,
                           [](int r) { return swz_tr<T, BC>(r); });
      dma_tile_n<BT, BC, 8>(rC, cb, GN * ES, st + Lay::CO, Ls, (int)(N * ES / 16), w, lane,
                            [](int r) { return swz_row<T, BC>(r); });
    }
    // the diagonal Gram tile (sig, sig) of chunk ch: pair index sig (sig + 3) / 2
    // (32-bit offsets: the Gram buffer of a sequence is below 4 GiB)
    const uint32_t pidx = ((uint32_t)sig * (uint32_t)(sig + 3)) >> 1;
    const uint32_t gb = (uint32_t)ch * gchunk + gbase + pidx * gpair;
    int wg = 1024 * dma_group<BT, GC, 8>(0, w);
    asm volatile("" : "+s"(wg));
    dma_tile_full_w<BT, GC, 8>(rG, gb, goff, st + Lay::GO, wg);
  };

  floatx4 accY[TT];
  bool ypend = false;  // y of the previous step waiting to be stored
  size_t yrow0 = 0;
  int ylim = 0;
  auto store_y = [&]() {
    if (!ypend) return;
    typedef typename Vec<TY>::x4 Y4;
    TY* yb = reinterpret_cast<TY*>(A.y) + yrow0 * HPsz + (size_t)h * kP + 16 * wc + 4 * g4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tl = 16 * tt + c;
      if (tl < ylim) {
        Y4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = from_f32<TY>(accY[tt][i]);
        *reinterpret_cast<Y4*>(yb + (size_t)tl * HPsz) = o;
      }
    }
    ypend = false;
  };

  auto gfrag = [&](const unsigned char* Gt, int tt, int q) {
    const int t = 16 * tt + c;
    const int e0 = (32 * q + 8 * g4) * (int)ES;
    return load8<T>(reinterpret_cast<const T*>(
        Gt + (t * GC + ((e0 >> 4) ^ swz_row<T, GC>(t))) * 16 + (e0 & 15)));
  };

  auto compute = [&](const unsigned char* st, int jb) {
    const unsigned char* Gd = st + Lay::GO;
    const int c0 = jb * BT;
    const int Ls = min(BT, Tlen - c0);

    // ---- the block's entering state as fp16 operands; past 2^14 (found from
    // this wave's max |H| with one ballot) they are scaled by 2^-e, e >= 0, and
    // the readout by 2^e
    bool scaled = false;
    float hin = 1.f, hscale = 1.f;
    if (sizeof(T) == 2) {
      float mx = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(Hr[a][i]));
      }
      if (__ballot(mx > 16384.f)) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const int e = (int)ceilf(log2f(mx * (1.f / 16384.f)));
        hin = ldexpf(1.f, -e);
        hscale = ldexpf(1.f, e);
        scaled = true;
      }
    }

    F xq[RQ];  // X^T fragments of this wave's columns
#pragma unroll
    for (int q = 0; q < RQ; ++q) xq[q] = load_kmajor_at<T>(st, xo, 32 * q * XC * 16);

    // ---- readout: y^T[p, t] = H^T[p, n] C~^T[n, t], n visited in the order
    // {4 g4 .. 4 g4 + 3, 16 + 4 g4 .. 16 + 4 g4 + 3} per 32 (the accumulator's)
    auto readout = [&](auto scale_tag) {
      constexpr bool SC = decltype(scale_tag)::value;
      floatx4 ro[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) ro[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        F cf[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          cf[tt] = load4x2<T>(reinterpret_cast<const T*>(st + co[tt][q][0]),
                              reinterpret_cast<const T*>(st + co[tt][q][1]));
        F hq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hq[i] = from_f32<T>(SC ? Hr[2 * q][i] * hin : Hr[2 * q][i]);
          hq[4 + i] = from_f32<T>(SC ? Hr[2 * q + 1][i] * hin : Hr[2 * q + 1][i]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) ro[tt] = mma16(hq, cf[tt], ro[tt]);
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) accY[tt] = ro[tt] * (SC ? at[tt] * hscale : at[tt]);
    };
    if (scaled)
      readout(std::true_type{});
    else
      readout(std::false_type{});
    // ---- intra term of the block
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      F gf[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (DF::index(tt, q) >= 0) gf[tt] = gfrag(Gd, tt, q);
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int ix = DF::index(tt, q);
        if (ix >= 0) accY[tt] = mma16(xq[q], gf[tt] * dm[ix], accY[tt]);
      }
    }

    // ---- carry: H <- a^{Ls} H + sum_r B_hat[r, n] (a^{Ls-1-s} X[r, p])
    const bool full = Ls == BT;
    const float aL = full ? aBT : apow_step(la, Ls);
#pragma unroll
    for (int a = 0; a < NT; ++a) Hr[a] = Hr[a] * aL;
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      F xd;
      if (full) {
        xd = xq[q] * er[q];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = Ls - 1 - (32 * q + 8 * g4 + j) / KS;
          xd[j] = from_f32<T>(to_f32(xq[q][j]) * (d >= 0 ? apow_step(la, d) : 0.f));
        }
      }
      // the K step's B_hat fragments read together, left to the compiler's
      // schedule (in groups of four with a scheduling fence between: 1-2 %
      // slower)
      F bf[NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) bf[a] = load_kmajor_at<T>(st, bo[a], 32 * q * BC * 16);
#pragma unroll
      for (int a = 0; a < NT; ++a) Hr[a] = mma16(bf[a], xd, Hr[a]);
    }
    ypend = true;
    yrow0 = (size_t)b * Tlen + c0;
    ylim = Ls;
  };

  // ---- the walk: step s computes from stage s % 3 while the copies of step
  // s + 2 go into stage (s + 2) % 3; one barrier per step
  int jc = j0;
  fetch(stage0, jc);
  if (jc + 1 < j1)
    fetch(stage1, jc + 1);
  else
    dma_dummies<NCOPY>(rX, sink);
  wait_vm<0>();
  stage_barrier();
  auto step = [&](const unsigned char* cur_st, unsigned char* far_st) {
    store_y();  // the previous block's y, before this step's copies
    if (jc + 2 < j1)
      fetch(far_st, jc + 2);
    else
      dma_dummies<NCOPY>(rX, sink);
    compute(cur_st, jc);
    wait_vm<NCOPY>();  // the next step's copies have landed
    stage_barrier();
    return ++jc < j1;
  };
  while (step(stage0, stage2) && step(stage1, stage0) && step(stage2, stage1)) {
  }
  store_y();
  wait_vm<0>();  // the copies past the end land before the workgroup's LDS is released

  if (seg == A.segs - 1 && A.h_final) {
    float* dst = A.h_final + ((size_t)b * H + h) * NPsz;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * a + 4 * g4 + i;
        if (n < N) dst[(size_t)n * kP + prow_x] = Hr[a][i];
      }
  }
}

// Pass 1 with two heads per workgroup (8 waves; the heads share one copy of
// the group's B_hat rows): the carry-only walk over the chunks of one piece of
// a segment, one step per 32-token block (its X_hat rows for both heads and
// its B_hat rows), H <- a^{Lc} H at a chunk's first block and
// H += B_hat^T (a^{Lc-1-s} X_hat) for every block, from a zero state; the
// piece's end state goes to its workspace slot. Three LDS stages with a fixed
// number of copies per step, so the copies of step s + 2 are in flight while
// step s computes and a stage is waited for with one count.
constexpr int kCarryThreads = 512;
template <typename T, int NP, int KS, int BT>
struct CarryLds {
  static constexpr int R = KS * BT;
  static constexpr int XROW = kP * (int)sizeof(T), BROW = NP * (int)sizeof(T);
  static constexpr int XB = R * XROW, BB = R * BROW;
  static constexpr int XO = 0, BO = 2 * XB;
  static constexpr int STAGE = BO + BB;
};

template <typename T, int NP, int KS, int BT>
__global__ __launch_bounds__(kCarryThreads, 1) void scan_carry_kernel(ScanArgs A) {
  typedef CarryLds<T, NP, KS, BT> Lay;
  constexpr int R = Lay::R, RQ = R / 32, NT = NP / 16;
  constexpr int XC = Lay::XROW / 16, BC = Lay::BROW / 16;
  constexpr uint32_t ES = sizeof(T);
  typedef typename Vec<T>::x8 F;
  constexpr int CX = dma_count<2 * R, XC, 8>(), CBn = dma_count<R, BC, 8>();
  constexpr int NCOPY = CX + CBn;

  __shared__ __align__(16) unsigned char stage0[Lay::STAGE];
  __shared__ __align__(16) unsigned char stage1[Lay::STAGE];
  __shared__ __align__(16) unsigned char stage2[Lay::STAGE];
  __shared__ __align__(16) unsigned char sink[kSinkBytes];

  const int H = A.H, G = A.G, N = A.N, L = A.L, Tlen = A.T;
  const int HU = H / 2;
  const int nseg = (A.segs - 1) * A.sub;  // pieces
  const int nslot = nseg + 1;
  const int per = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (logical >= HU * nseg * A.Bt) return;
  const int hp = logical % HU, seg = (logical / HU) % nseg, b = logical / (HU * nseg);
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w >> 2, wc = w & 3;
  const int h = 2 * hp + hw;
  const int grp = h / (H / G);
  const int GN = G * N;
  const int g4 = lane >> 4, c = lane & 15;
  const size_t NPsz = (size_t)N * kP;
  const size_t HPsz = (size_t)H * kP;
  const int prow_x = 16 * wc + c;
  const float la = A.a[h] > 0.f ? log2f(A.a[h]) : -1e30f;
  // lane offsets of the transposing reads within a stage (planned once, as in
  // the output walk)
  int xo[2], bo[NT][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    xo[hh] = Lay::XO + hw * Lay::XB + kmajor_off<T, XC>(16 * wc, hh, lane);
    asm("" : "+v"(xo[hh]));
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      bo[a][hh] = Lay::BO + kmajor_off<T, BC>(16 * a, hh, lane);
      asm("" : "+v"(bo[a][hh]));
    }
  }

  const BufRes rB = make_rsrc(reinterpret_cast<const T*>(A.B_hat) + (size_t)b * Tlen * KS * GN,
                              (uint64_t)Tlen * KS * GN * ES);
  const BufRes rX = make_rsrc(reinterpret_cast<const T*>(A.X_hat) + (size_t)b * Tlen * KS * HPsz,
                              (uint64_t)Tlen * KS * HPsz * ES);

  F er[RQ];  // a^{BT-1-s} of the pair row r = 32q + 8g + j of a block (s = r / k)
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) er[q][j] = from_f32<T>(apow(la, BT - 1 - (32 * q + 8 * g4 + j) / KS));

  floatx4 Hr[NT];
#pragma unroll
  for (int a = 0; a < NT; ++a) Hr[a] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int span = A.seg_chunks / A.sub;
  const int ch0 = seg * span;
  const int ch1 = min(A.nc, ch0 + span);
  if (ch0 >= ch1) return;
  auto nblocks = [&](int ch) { return (min(L, Tlen - ch * L) + BT - 1) / BT; };
  struct Blk {
    int ch, sig;
  };
  auto advance = [&](Blk s) {
    if (++s.sig == nblocks(s.ch)) {
      s.sig = 0;
      ++s.ch;
    }
    return s;
  };

  uint32_t xoff[CX], boff[CBn];
  int xrow[CX];
#pragma unroll
  for (int m = 0; m < CX; ++m) {
    const int slot = 64 * dma_group<2 * R, XC, 8>(m, w) + lane;
    const int r = slot / XC, pc = slot % XC, rr = r % R;
    xrow[m] = rr;
    xoff[m] = rr * (uint32_t)HPsz * ES + (r / R) * kP * ES + 16 * (pc ^ swz_tr<T, XC>(rr));
  }
  dma_plan_n<R, BC, 8>((uint32_t)GN * ES, w, lane, [](int r) { return swz_tr<T, BC>(r); }, boff);
  const bool nfull = N == NP;
  auto fetch = [&](unsigned char* st, Blk s) {
    const int c0 = s.ch * L;
    const int Lc = min(L, Tlen - c0);
    const uint32_t prow = (uint32_t)(c0 + s.sig * BT) * KS;
    const int rlim = (Lc - s.sig * BT) * KS;
    const bool rows_full = rlim >= R;
    const uint32_t xb = (prow * (uint32_t)HPsz + 2 * hp * kP) * ES;
    if (rows_full)
      dma_tile_full_n<2 * R, XC, 8>(rX, xb, xoff, st + Lay::XO, w);
    else
      dma_rows_n<2 * R, XC, 8>(rX, xb, xoff, xrow, rlim, st + Lay::XO, w);
    const uint32_t bb = (prow * GN + grp * N) * ES;
    if (rows_full && nfull)
      dma_tile_full_n<R, BC, 8>(rB, bb, boff, st + Lay::BO, w);
    else
      dma_tile_n<R, BC, 8>(rB, bb, GN * ES, st + Lay::BO, rlim, (int)(N * ES / 16), w, lane,
                           [](int r) { return swz_tr<T, BC>(r); });
  };
  auto compute = [&](const unsigned char* st, Blk cur) {
    const int Lc = min(L, Tlen - cur.ch * L);
    const int nb = (Lc + BT - 1) / BT;
    if (cur.sig == 0) {
      const float aL = apow_step(la, Lc);
#pragma unroll
      for (int a = 0; a < NT; ++a) Hr[a] = Hr[a] * aL;
    }
    const bool full = Lc == nb * BT;
    const float blk = apow_step(la, (nb - 1 - cur.sig) * BT);
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const F xq = load_kmajor_at<T>(st, xo, 32 * q * XC * 16);
      F xd;
      if (full) {
        xd = xq * (er[q] * from_f32<T>(blk));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = Lc - 1 - (cur.sig * BT + (32 * q + 8 * g4 + j) / KS);
          xd[j] = from_f32<T>(to_f32(xq[j]) * (d >= 0 ? apow_step(la, d) : 0.f));
        }
      }
      constexpr int CGR = NT < 4 ? NT : 4;
#pragma unroll
      for (int a0 = 0; a0 < NT; a0 += CGR) {
        F bf[CGR];
#pragma unroll
        for (int i = 0; i < CGR; ++i) bf[i] = load_kmajor_at<T>(st, bo[a0 + i], 32 * q * BC * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CGR; ++i) Hr[a0 + i] = mma16(bf[i], xd, Hr[a0 + i]);
      }
    }
  };

  // ---- the walk: step s computes from stage s % 3 while the copies of step
  // s + 2 go into stage (s + 2) % 3; one barrier per step
  Blk s0{ch0, 0};
  Blk s1 = advance(s0);
  Blk s2 = s1.ch < ch1 ? advance(s1) : s1;
  fetch(stage0, s0);
  if (s1.ch < ch1)
    fetch(stage1, s1);
  else
    dma_dummies<NCOPY>(rX, sink);
  wait_vm<0>();
  stage_barrier();
  auto step = [&](const unsigned char* cur_st, unsigned char* far_st) {
    if (s2.ch < ch1)
      fetch(far_st, s2);
    else
      dma_dummies<NCOPY>(rX, sink);
    compute(cur_st, s0);
    wait_vm<NCOPY>();  // the next step's copies have landed
    stage_barrier();
    s0 = s1;
    s1 = s2;
    if (s2.ch < ch1) s2 = advance(s2);
    return s0.ch < ch1;
  };
  while (step(stage0, stage2) && step(stage1, stage0) && step(stage2, stage1)) {
  }
  wait_vm<0>();  // the copies past the end land before the workgroup's LDS is released

  float* dst = A.ws + (((size_t)b * nslot + seg + 1) * H + h) * NPsz;  // slot j+1 holds S_j
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 16 * a + 4 * g4 + i;
      if (n < N) dst[(size_t)n * kP + prow_x] = Hr[a][i];
    }
}

// Pass 2: Hin_0 = h_init (or 0), Hin_{s+1} = a^{len_s} Hin_s + S_s, for every
// (sequence, head, element), walking the pieces of pass 1 in order (`segs`
// slots here, pieces of `seg_chunks` chunks). Slot s of the workspace holds
// S_{s-1} on entry (s >= 1) and Hin_s on exit.
// With the expert-mixed decay (ld non-null) a segment's decay is the product
// over its chunks of 2^{Lam at the chunk's last token}, the exponents summed in
// chunk order.
__global__ __launch_bounds__(256) void scan_combine_kernel(const float* __restrict__ a,
                                                           const float* __restrict__ h_init,
                                                           float* __restrict__ ws, int H,
                                                           int NPsz, int T, int L, int segs,
                                                           int seg_chunks,
                                                           const float* __restrict__ ld) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int e4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e4 >= NPsz) return;
  const float ah = ld ? 1.f : a[h];
  const float* lrow = ld ? ld + ((size_t)b * H + h) * T : nullptr;
  floatx4 Hc = {0.f, 0.f, 0.f, 0.f};
  if (h_init) Hc = *reinterpret_cast<const floatx4*>(h_init + ((size_t)b * H + h) * NPsz + e4);
  float* base = ws + (size_t)b * segs * H * NPsz + (size_t)h * NPsz + e4;
  const size_t sstride = (size_t)H * NPsz;
  *reinterpret_cast<floatx4*>(base) = Hc;
  for (int s = 0; s + 1 < segs; ++s) {
    const int t0 = s * seg_chunks * L;
    const int len = min(T, t0 + seg_chunks * L) - t0;
    floatx4* slot = reinterpret_cast<floatx4*>(base + (size_t)(s + 1) * sstride);
    float dec;
    if (lrow) {
      float e = 0.f;
      for (int c0 = t0; c0 < t0 + len; c0 += L) e += lrow[min(T, c0 + L) - 1];
      dec = exp2f(e);
    } else {
      dec = pow_int(ah, len);
    }
    Hc = Hc * dec + *slot;
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

// Tuning knob (environment, read once): SWIMBA_SCAN_WGS = the most workgroups
// the output pass may have; the segment count per sequence is the largest that
// keeps (sequences x heads x segments) within it. The default, 512, is what the
// MI355X holds at once (two workgroups per CU): more segments than one round
// of workgroups measured slower (a second, partial round), fewer leave CUs idle.
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}
// Workgroups the prefill walk aims at (segments per sequence follow from it).
// Measured on MI355X: chunks of 64 tokens (3 block pairs each) run fastest
// with about 1024 (8 x 2048 tokens, 24 heads: 5 segments of 7 chunks, chunk
// output 94 -> 80 us), longer chunks with 512 (4 x 8192 tokens with L = 128
// and 65536 tokens with L = 256 both lose 2-10 % at 384, 768 or 1024).
static int scan_target_wgs(int L) {
  static const int w = env_int("SWIMBA_SCAN_WGS", 0);
  if (w > 0) return w;
  return L <= 64 ? 1024 : 512;
}

static int scan_npairs(int L, int bt) {
  const int nb = (L + bt - 1) / bt;
  return nb * (nb + 1) / 2;
}

// Tokens per block. 64-token blocks (one step per 64-token chunk, two stages
// of 80 KiB) measured slower than 32-token blocks with two workgroups per CU,
// so the walk uses 32; the kernels stay templated on the block size.
static int scan_block(int N, int k, int L, int es) {
  (void)N, (void)k, (void)L, (void)es;
  return 32;
}

// The walk one block per step (scan_block_kernel, two heads per workgroup)
// serves 2-byte streams with k <= 2 and the shared decay when the heads of a
// group pair up (H / G even). Measured on MI355X against the walks it
// replaced: 4 x 8192 tokens, 64 heads, L = 128: chunk output 323 -> 300 us
// (a walk of 64-token sub-chunks by source block, whose fp16 copy of the
// entering state lived in LDS); 65536 tokens, 32 heads, L = 256: 319 -> 296
// us; 8 x 2048 tokens, 24 heads, L = 64: 81 -> 78 us (one head per
// workgroup). SWIMBA_SCAN_WALK = 0 forces one head per workgroup.
static int scan_walk(int H, int G, int k, int es, bool tv) {
  static const int forced = env_int("SWIMBA_SCAN_WALK", -1);
  const bool two = es == 2 && k <= 2 && !tv && (H / G) % 2 == 0;
  if (forced == 0) return 0;
  return two ? 1 : 0;
}
static int walk_target_wgs(int L) {
  static const int w = env_int("SWIMBA_SCAN_WGS", 0);
  if (w > 0) return w;
  (void)L;
  return 256;
}

// Pass 1 (the carry-only walk to each segment's end state) runs one head per
// workgroup; with few segments it leaves CUs idle (4 x 8192 tokens, 64 heads,
// two segments: 256 workgroups). It splits every segment into equal pieces
// (a divisor of its chunk count), as many as bring it closest to 512
// workgroups, and the combine then sweeps the pieces. Measured on MI355X:
// 4 x 8192 tokens, 64 heads: 2 pieces took pass 1 + combine from 128 to 95 us
// (4 pieces: 123 us); 65536 tokens, 32 heads (480 workgroups already): 2
// pieces were slower (168 -> 202 us).
static int scan_pieces(int units1, int seg_chunks) {
  static const int forced = env_int("SWIMBA_SCAN_SUB", 0);
  if (units1 <= 0) return 1;
  int best = 1;
  for (int m = 1; m <= seg_chunks; ++m) {
    if (seg_chunks % m) continue;
    if (forced > 0) {
      if (m >= forced) return m;
      continue;
    }
    if (std::abs(units1 * m - 512) < std::abs(units1 * best - 512)) best = m;
  }
  return forced > 0 ? seg_chunks : best;
}

// Pass 1 with two heads per workgroup (scan_carry_kernel) goes with the
// two-head output walk (2-byte streams, k <= 2, the shared decay, heads of a
// group in pairs). Measured on MI355X: 4 x 8192 tokens, 64 heads: 84 -> 75
// us; 65536 tokens, 32 heads: 156 -> 136 us; 8 x 2048 tokens, 24 heads, L =
// 64: 29 -> 25 us. SWIMBA_SCAN_CARRY = 0 keeps one head per workgroup.
static bool carry_two(const ScanGeom& g) {
  static const int on = env_int("SWIMBA_SCAN_CARRY", 1);
  return on > 0 && g.walk == 1;
}

ScanGeom scan_geom(int Bt, int T, int H, int G, int N, int P, int k, int L, int es, bool tv) {
  ScanGeom g{Bt, T, H, G, N, P, k, L, es, scan_block(N, k, L, es), 1, 1, 0, 1};
  const int nc = (T + L - 1) / L;
  if (nc <= 0) return g;
  g.walk = scan_walk(H, G, k, es, tv);
  const int units = g.walk ? Bt * (H / 2) : Bt * H;
  int want = (g.walk ? walk_target_wgs(L) : scan_target_wgs(L)) / units;
  if (want > nc) want = nc;
  if (want < 1) want = 1;
  g.seg_chunks = (nc + want - 1) / want;
  g.segs = (nc + g.seg_chunks - 1) / g.seg_chunks;
  g.sub = scan_pieces(Bt * H * (g.segs - 1), g.seg_chunks);
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t scan_state_bytes(const ScanGeom& g) {
  if (g.segs <= 1) return 0;
  const size_t nslot = (size_t)(g.segs - 1) * g.sub + 1;
  return align256((size_t)g.Bt * nslot * g.H * g.N * g.P * sizeof(float));
}

static size_t scan_gram_bytes(const ScanGeom& g) {
  const size_t nc = (size_t)((g.T + g.L - 1) / g.L);
  return align256((size_t)g.Bt * nc * g.G * scan_npairs(g.L, g.bt) * g.bt * (g.k * g.bt) * g.es);
}

size_t scan_ws_bytes(const ScanGeom& g) {
  if (g.Bt == 0 || g.T == 0) return 0;
  return scan_state_bytes(g) + scan_gram_bytes(g);
}

template <typename T, typename TY, int NP, int KS, int BT, bool TV>
static hipError_t launch_scan_t(const ScanGeom& g, ScanArgs args, hipStream_t s) {
  auto k3 = scan_kernel<T, TY, NP, KS, BT, true, TV>;
  auto k1 = scan_kernel<T, TY, NP, KS, BT, false, TV>;
  const size_t l3 = 0, l1 = 0;  // static LDS (two stage arrays)
  prof_begin("scan_gram", s);
  const int diag = (sizeof(T) == 2 && KS <= 2 && !TV && g.walk == 1) ? 1 : 0;
  const int ng = (diag ? g.L / BT : args.npairs) * g.G * args.nc * g.Bt;
  hipLaunchKernelGGL((scan_gram_kernel<T, NP, KS, BT>), dim3((unsigned)((ng + 7) / 8 * 8)),
                     dim3(256), 0, s, static_cast<const T*>(args.B_hat),
                     static_cast<const T*>(args.C_mix), static_cast<T*>(const_cast<void*>(args.gram)),
                     g.T, g.G, g.N, g.L, args.nc, args.npairs, g.Bt,
                     diag);
  prof_end(s);
  if (g.segs > 1) {
    prof_begin("scan_segment_state", s);
    bool done = false;
    if constexpr (sizeof(T) == 2 && KS <= 2 && !TV) {
      if (carry_two(g)) {
        const int n1 = (g.H / 2) * (g.segs - 1) * g.sub * g.Bt;
        hipLaunchKernelGGL((scan_carry_kernel<T, NP, KS, BT>), dim3((unsigned)((n1 + 7) / 8 * 8)),
                           dim3(kCarryThreads), 0, s, args);
        done = true;
      }
    }
    if (!done) {
      const int n1 = g.H * (g.segs - 1) * g.sub * g.Bt;
      hipLaunchKernelGGL(k1, dim3((unsigned)((n1 + 7) / 8 * 8)), dim3(kScanThreads), l1, s, args);
    }
    prof_end(s);
    const int NPsz = g.N * g.P;
    prof_begin("scan_state_pass", s);
    hipLaunchKernelGGL(scan_combine_kernel, dim3((NPsz / 4 + 255) / 256, g.H, g.Bt), dim3(256), 0,
                       s, args.a, args.h_init, args.ws, g.H, NPsz, g.T, g.L,
                       (g.segs - 1) * g.sub + 1, g.seg_chunks / g.sub, args.ld);
    prof_end(s);
  }
  hipEvent_t e0, e1;
  prof_kernel("scan_chunk_output", &e0, &e1);
  if constexpr (sizeof(T) == 2 && KS <= 2 && !TV) {
    if (g.walk == 1) {
      const int n3 = (g.H / 2) * g.segs * g.Bt;
      hipExtLaunchKernelGGL((scan_block_kernel<T, TY, NP, KS, BT>),
                            dim3((unsigned)((n3 + 7) / 8 * 8)), dim3(kBlockThreads), 0, s, e0, e1,
                            0, args);
      return hipGetLastError();
    }
  }
  const int n3 = g.H * g.segs * g.Bt;
  hipExtLaunchKernelGGL(k3, dim3((unsigned)((n3 + 7) / 8 * 8)), dim3(kScanThreads), l3, s, e0, e1,
                        0, args);
  return hipGetLastError();
}

template <typename T, typename TY, int NP, int KS>
static hipError_t dispatch_bt(const ScanGeom& g, const ScanArgs& a, hipStream_t s) {
  if (a.ld) return launch_scan_t<T, TY, NP, KS, 32, true>(g, a, s);
  return launch_scan_t<T, TY, NP, KS, 32, false>(g, a, s);
}

template <typename T, typename TY, int NP>
static hipError_t dispatch_ks(const ScanGeom& g, const ScanArgs& a, hipStream_t s) {
  if (g.k == 1) return dispatch_bt<T, TY, NP, 1>(g, a, s);
  if constexpr (sizeof(T) == 2) {
    // 2-byte streams: k = 3 and 4 fit two stages in LDS (fp32 ones do not)
    if (g.k == 3) return dispatch_bt<T, TY, NP, 3>(g, a, s);
    if (g.k == 4) return dispatch_bt<T, TY, NP, 4>(g, a, s);
  }
  return dispatch_bt<T, TY, NP, 2>(g, a, s);
}

template <typename T, typename TY>
static hipError_t dispatch_np(const ScanGeom& g, const ScanArgs& a, hipStream_t s) {
  const int np = g.N <= 32 ? 32 : (g.N <= 64 ? 64 : 128);
  if (np == 32) return dispatch_ks<T, TY, 32>(g, a, s);
  if (np == 64) return dispatch_ks<T, TY, 64>(g, a, s);
  return dispatch_ks<T, TY, 128>(g, a, s);
}

hipError_t launch_scan(bool is_bf16, const ScanGeom& g, const void* B_hat, const void* X_hat,
                       const void* C_mix, const float* a, const float* h_init, void* y,
                       float* h_final, float* ws, hipStream_t s, const float* ld, bool y_f32) {
  if (g.Bt == 0) return hipSuccess;
  if (g.T == 0) {
    if (h_final) return launch_state_copy(h_init, h_final, (size_t)g.Bt * g.H * g.N * g.P, s);
    return hipSuccess;
  }
  const int nc = (g.T + g.L - 1) / g.L;
  unsigned char* gram = reinterpret_cast<unsigned char*>(ws) + scan_state_bytes(g);
  ScanArgs args{B_hat, X_hat, C_mix, a, h_init, y, h_final, ws, gram, ld,
                g.T, g.H, g.G, g.N, g.k, g.L, g.segs, g.seg_chunks, nc, scan_npairs(g.L, g.bt),
                g.Bt, g.sub};
  if (is_bf16 && y_f32) {
    // fp16 streams with an fp32 y (the separated-SSM trajectories, summed
    // over experts afterwards): shared decay, one slot per token
    if (g.k != 1 || ld) return hipErrorInvalidValue;
    const int np = g.N <= 32 ? 32 : (g.N <= 64 ? 64 : 128);
    if (np == 32) return launch_scan_t<f16, float, 32, 1, 32, false>(g, args, s);
    if (np == 64) return launch_scan_t<f16, float, 64, 1, 32, false>(g, args, s);
    return launch_scan_t<f16, float, 128, 1, 32, false>(g, args, s);
  }
  if (is_bf16) return dispatch_np<f16, bf16>(g, args, s);
  return dispatch_np<float, float>(g, args, s);
}

}  // namespace swimba
