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
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

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

// Staged K loop: per stage, BK = 32 elements of d for the BM gathered token rows
// (A) and the BN weight rows (B), row-major, 16-byte chunk c of row r at
// c ^ swz_row(r). Four stages: the copies of a K tile are issued three tiles
// ahead of its multiply.
constexpr int kProjStages = 4;
template <typename T, class C>
struct ProjLay {
  static constexpr int BK = 32;
  static constexpr int ROWB = BK * (int)sizeof(T);  // bytes per tile row
  static constexpr int CPR = ROWB / 16;             // chunks per row
  static constexpr int AB = C::BM * ROWB, BB = C::BN * ROWB;
  static constexpr int STAGE = AB + BB;
  static constexpr int NIA = AB / 1024, NIB = BB / 1024;  // copy instructions per stage
  static constexpr int MA = NIA / C::NW, MB = NIB / C::NW;  // ... per wave
  static constexpr int CPW = MA + MB;
  static_assert(NIA % C::NW == 0 && NIB % C::NW == 0, "copies split evenly over the waves");
};

// XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so XCD x
// gets the contiguous logical range [x * per, (x + 1) * per) of the real
// (row tile, column tile) units. Units are ordered in groups of GR row tiles,
// column tile by column tile within a group, so the workgroups one XCD runs at
// a time share a few row tiles of tokens and a few column tiles of weights
// (both stay in its L2 while they move along d together; GR = 1 when every
// weight tile is read once anyway). The grid is
// sized for the most row tiles there can be; the number that exist (written
// by the bucketing kernel after the tile table) spreads them over all XCDs, so
// no XCD is left with only empty slots. Returns false for a workgroup without
// a unit.
// GR (environment SWIMBA_PROJ_GR, read once; default 4) matters little on
// MI355X: 4 x 8192 tokens, E = 16: GR 1, 2, 4, 8, 16 took 1158, 1134, 1129,
// 1140, 1149 us; 65536 tokens, E = 8: GR 4 636 us, GR 8 613 us.
constexpr int kProjGroupRows = 4;
static int proj_group_rows() {
  static const int g = [] {
    const char* v = getenv("SWIMBA_PROJ_GR");
    const int x = v ? atoi(v) : 0;
    return x > 0 ? x : kProjGroupRows;
  }();
  return g;
}
__device__ __forceinline__ bool xcd_unit(int GR, int nt, int CT, int& tile, int& ctile) {
  const int units = nt * CT;
  const int per = (units + 7) / 8;
  const int slot = blockIdx.x / 8;
  if (slot >= per) return false;
  const int logical = (blockIdx.x % 8) * per + slot;
  if (logical >= units) return false;
  const int group = logical / (GR * CT);
  const int rem = logical - group * (GR * CT);
  const int gm = min(GR, nt - group * GR);  // row tiles in this group
  ctile = rem / gm;
  tile = group * GR + (rem - ctile * gm);
  return true;
}
__device__ __forceinline__ bool xcd_tile(int GR, const int4v* __restrict__ tile_info,
                                         int nrow_tiles, int CT, int& tile, int& ctile) {
  return xcd_unit(GR, tile_info[nrow_tiles][0], CT, tile, ctile);
}

// PLAIN: the same kernel as a plain GEMM out[M, W] = u[M, D] wexp[W, D]^T (the
// output projection): rows are u's own rows in order (nrow_tiles row tiles),
// one weight matrix, and the epilogue writes out in TO.
// KFULL: d is a multiple of kProjStages K tiles, so no copy ever needs a K
// bound: the per-lane part of every copy offset is fixed for the workgroup and
// the K tile enters as the copy's scalar offset (no vector arithmetic per copy).
template <typename T, class C, bool PLAIN = false, typename TO = float, bool KFULL = false>
__global__ __launch_bounds__(C::NTH) void proj_kernel(
    const T* __restrict__ u, const T* __restrict__ wexp, const int32_t* __restrict__ sorted,
    const float* __restrict__ sorted_w, const int4v* __restrict__ tile_info, int M, int D, int W,
    int HP, int GN, int k, int nrow_tiles, typename StreamOf<T>::type* __restrict__ X_hat,
    typename StreamOf<T>::type* __restrict__ B_hat, float* __restrict__ c_part,
    TO* __restrict__ out, int bw_one, int gr) {
  typedef typename StreamOf<T>::type S;
  typedef ProjLay<T, C> Lay;
  constexpr int BM = C::BM, BN = C::BN, NTH = C::NTH, NW = C::NW, TM = C::TM, TN = C::TN;
  constexpr int BK = Lay::BK, CPR = Lay::CPR, ROWB = Lay::ROWB, MA = Lay::MA, MB = Lay::MB;
  constexpr uint32_t ES = sizeof(T);
  typedef typename Vec<T>::x8 F;

  // four stage arrays: copies into one are known not to touch the others
  __shared__ __align__(16) unsigned char stg0[Lay::STAGE];
  __shared__ __align__(16) unsigned char stg1[Lay::STAGE];
  __shared__ __align__(16) unsigned char stg2[Lay::STAGE];
  __shared__ __align__(16) unsigned char stg3[Lay::STAGE];
  __shared__ int rtok[BM];
  __shared__ int rslot[BM];
  __shared__ float rw[BM];

  const int CT = (W + BN - 1) / BN;
  int tile, ctile, e, row0, nrows;
  if constexpr (PLAIN) {
    if (!xcd_unit(gr, nrow_tiles, CT, tile, ctile)) return;
    e = 0;
    row0 = tile * BM;
    nrows = min(BM, M - row0);
  } else {
    if (!xcd_tile(gr, tile_info, nrow_tiles, CT, tile, ctile)) return;
    const int4v ti = tile_info[tile];  // {expert, first sorted row, rows}
    e = ti[0];
    if (e < 0) return;
    row0 = ti[1];
    nrows = ti[2];
  }
  for (int r = threadIdx.x; r < BM; r += NTH) {
    if (r < nrows) {
      const int p = PLAIN ? row0 + r : sorted[row0 + r];
      rtok[r] = p / k;
      rslot[r] = p - (p / k) * k;
      rw[r] = PLAIN ? 1.f : sorted_w[row0 + r];
    } else {
      rtok[r] = -1;
      rslot[r] = 0;
      rw[r] = 0.f;
    }
  }
  __syncthreads();

  const int col0 = ctile * BN;
  const T* We = wexp + (size_t)e * W * D;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // ---- copy plan (independent of the K tile): instruction m of this wave
  // fills LDS chunk slots 64 (wave + NW m) + lane of a tile.
  const BufRes rA = make_rsrc(u, (uint64_t)M * D * ES);
  const BufRes rW = make_rsrc(We, (uint64_t)W * D * ES);
  uint32_t abase[MA], bbase[MB];
  int alc[MA], blc[MB];
#pragma unroll
  for (int m = 0; m < MA; ++m) {
    const int slot = 64 * (wave + NW * m) + lane;
    const int r = slot / CPR;
    alc[m] = (slot % CPR) ^ swz_row<T, CPR>(r);
    const int tok = rtok[r];
    abase[m] = tok >= 0 ? (uint32_t)tok * D * ES : kOOB;
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int slot = 64 * (wave + NW * m) + lane;
    const int r = slot / CPR;
    blc[m] = (slot % CPR) ^ swz_row<T, CPR>(r);
    const int col = col0 + r;
    bbase[m] = col < W ? (uint32_t)col * D * ES : kOOB;
  }
  // KFULL: lane offsets with the row and chunk folded in (rows past the group
  // or columns past W keep an offset beyond the buffer whatever the K tile)
  uint32_t aoff[MA], boff[MB];
#pragma unroll
  for (int m = 0; m < MA; ++m) aoff[m] = abase[m] != kOOB ? abase[m] + 16u * alc[m] : kOOB;
#pragma unroll
  for (int m = 0; m < MB; ++m) boff[m] = bbase[m] != kOOB ? bbase[m] + 16u * blc[m] : kOOB;
  // MAV: the A copies of the tile's rows (MA, or MA / 2 for a half tile: the
  // copies m < MA / 2 cover rows 0 .. BM / 2 - 1)
  auto fetch = [&](unsigned char* st, int k0, auto mav_tag) {
    constexpr int MAV = decltype(mav_tag)::value;
    if constexpr (KFULL) {
      // the look-ahead of the last turn re-reads the last K tile (never used)
      const int ks = __builtin_amdgcn_readfirstlane(min(k0, D - BK) * (int)ES);
#pragma unroll
      for (int m = 0; m < MAV; ++m) {
        const uint32_t off = aoff[m];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(st + 1024 * (wave + NW * m)), 16, off,
            ks, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint32_t off = boff[m];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rW, (__attribute__((address_space(3))) void*)(st + Lay::AB + 1024 * (wave + NW * m)),
            16, off, ks, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < MAV; ++m) {
        const int kk = k0 + alc[m] * (16 / (int)ES);
        const uint32_t off = (abase[m] != kOOB && kk < D) ? abase[m] + kk * ES : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(st + 1024 * (wave + NW * m)), 16, off, 0,
            0, 0);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int kk = k0 + blc[m] * (16 / (int)ES);
        const uint32_t off = (bbase[m] != kOOB && kk < D) ? bbase[m] + kk * ES : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rW, (__attribute__((address_space(3))) void*)(st + Lay::AB + 1024 * (wave + NW * m)),
            16, off, 0, 0, 0);
      }
    }
  };

  // ---- fragments: lane (g, c) reads row c of a 16-row tile, elements 8g .. 8g+7
  auto frag = [&](const unsigned char* tilebase, int r) {
    if constexpr (sizeof(T) == 2) {
      return load8<T>(reinterpret_cast<const T*>(tilebase + r * ROWB + 16 * (g ^ swz_row<T, CPR>(r))));
    } else {
      return load8<T>(reinterpret_cast<const T*>(tilebase + r * ROWB + 32 * g));
    }
  };

  // The K loop and epilogue for TMV fragment rows per wave: TM, or TM / 2 or
  // TM / 4 for a half or quarter tile (an expert's last row tile with at most
  // BM / 2 or BM / 4 rows: the waves' rows are 16 TMV apart and only the A
  // copies of the first BM / 2 rows are issued, rows past the tile's reading
  // zeros), so that a short tail costs about half or a quarter of a tile.
  auto run = [&](auto tmv_tag) {
    constexpr int TMV = decltype(tmv_tag)::value;
    constexpr int MAV = MA * TMV / TM > 0 ? MA * TMV / TM : 1;
    static_assert(MAV * (BM / MA) >= C::WM * TMV * 16, "the A copies cover the rows computed");
    const std::integral_constant<int, MAV> mav{};
    // acc[i][j] holds, in lane (g, c), out[pair row 16i + c][columns 16j + 4g .. +3]
    // of this wave's block: the weight fragment is the matrix-core A operand.
    floatx4 acc[TMV][TN];
#pragma unroll
    for (int i = 0; i < TMV; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Column tiles are used in pairs (2jj, 2jj + 1) covering 32 columns: row m of
    // the pair's first matrix-core tile is column 8 (m / 4) + m % 4 and of the
    // second 8 (m / 4) + 4 + m % 4, so lane group g ends up with the 8
    // consecutive columns 8g .. 8g + 7 of the pair (one 16-byte store).
    auto bcol = [&](int j) {
      return wn * TN * 16 + 32 * (j >> 1) + 8 * (c >> 2) + 4 * (j & 1) + (c & 3);
    };
    // The matrix-core ops of the last DEF fragment rows of K tile kt are issued
    // after the reads of tile kt + 1 (past its barrier), so that they cover the
    // wait for those reads: 1-2 % at c3 and c4 (4 x 8192 and 65536 tokens),
    // bit-identical results.
    constexpr int DEF = TMV > 1 ? 1 : 0;
    F bfr[TN], afr[TMV];
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = zero8<T>();
#pragma unroll
    for (int i = 0; i < TMV; ++i) afr[i] = zero8<T>();
    auto mma_tail = [&]() {
#pragma unroll
      for (int i = TMV - DEF; i < TMV; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma16(bfr[j], afr[i], acc[i][j]);
    };
    auto compute = [&](const unsigned char* st) {
      F nb[TN], na[TMV];
#pragma unroll
      for (int j = 0; j < TN; ++j) nb[j] = frag(st + Lay::AB, bcol(j));
#pragma unroll
      for (int i = 0; i < TMV; ++i) na[i] = frag(st, wm * TMV * 16 + 16 * i + c);
      __builtin_amdgcn_sched_barrier(0);
      mma_tail();
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = nb[j];
#pragma unroll
      for (int i = 0; i < TMV; ++i) afr[i] = na[i];
#pragma unroll
      for (int i = 0; i < TMV - DEF; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma16(bfr[j], afr[i], acc[i][j]);
    };

    // The K loop runs in whole turns of the four stages and issues every copy
    // unconditionally (tiles past d read zeros, and multiply to nothing): with
    // no branches in the loop the compiler's own wait counts see which stage a
    // copy fills, and never drain all copies before reading a stage.
    const int nk = (D + BK - 1) / BK;
    const int nk4 = (nk + kProjStages - 1) / kProjStages * kProjStages;  // == nk when KFULL
    fetch(stg0, 0, mav);
    fetch(stg1, BK, mav);
    fetch(stg2, 2 * BK, mav);
    auto iter = [&](int kt, const unsigned char* cur, unsigned char* far) {
      wait_vm<2 * (MAV + MB)>();  // tile kt landed (tiles kt + 1, kt + 2 may be in flight)
      stage_barrier();          // tile kt visible to all waves; tile kt - 1 no longer read
      fetch(far, (kt + 3) * BK, mav);
      compute(cur);
    };
    for (int kt = 0; kt < nk4; kt += kProjStages) {
      iter(kt, stg0, stg3);
      iter(kt + 1, stg1, stg0);
      iter(kt + 2, stg2, stg1);
      iter(kt + 3, stg3, stg2);
    }
    mma_tail();
    wait_vm<0>();  // the copies past the end land before the workgroup's LDS is released

    // ---- epilogue: each lane stores 8 consecutive columns of one pair row per
    // column-tile pair (H*P and G*N are multiples of 16, so 8 columns never
    // straddle two regions).
    static_assert(TN % 2 == 0, "column tiles are used in pairs");
    typedef typename Vec<S>::x8 S8;
#pragma unroll
    for (int i = 0; i < TMV; ++i) {
      const int r = wm * TMV * 16 + 16 * i + c;
      const int tok = rtok[r];
      const size_t pair = (size_t)(tok < 0 ? 0 : tok) * k + rslot[r];
      const float wv = rw[r];
#pragma unroll
      for (int jj = 0; jj < TN / 2; ++jj) {
        const int cbase = __builtin_amdgcn_readfirstlane(col0 + wn * TN * 16 + 32 * jj);
        if (cbase >= W) continue;
        const int col = cbase + 8 * g;
        if (col >= W) continue;
        floatx8 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc[i][2 * jj][q];
          v[4 + q] = acc[i][2 * jj + 1][q];
        }
        if (tok < 0) continue;
        if constexpr (PLAIN) {
          typename Vec<TO>::x8 o;
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = from_f32<TO>(v[q]);
          store8<TO>(&out[pair * W + col], o);
        } else if (col < HP) {
          S8 o;
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = from_f32<S>(v[q]);
          store8<S>(&X_hat[pair * HP + col], o);
        } else if (col < HP + GN) {
          S8 o;
          const float wb = bw_one ? 1.f : wv;
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = from_f32<S>(wb * v[q]);
          store8<S>(&B_hat[pair * GN + (col - HP)], o);
        } else {
          floatx8 o = v * wv;
          store8<float>(&c_part[pair * GN + (col - HP - GN)], o);
        }
      }
    }
  };
  if constexpr (!PLAIN && TM % 4 == 0 && MA % 2 == 0) {
    if (nrows <= BM / 4)
      run(std::integral_constant<int, TM / 4>{});
    else if (nrows <= BM / 2)
      run(std::integral_constant<int, TM / 2>{});
    else
      run(std::integral_constant<int, TM>{});
  } else if constexpr (!PLAIN && TM % 2 == 0 && MA % 2 == 0) {
    if (nrows <= BM / 2)
      run(std::integral_constant<int, TM / 2>{});
    else
      run(std::integral_constant<int, TM>{});
  } else {
    run(std::integral_constant<int, TM>{});
  }
}

// Skinny variant for expert groups of at most 64 rows (decode batches, where
// every expert has a few dozen (token, slot) pairs and the step is bound by
// streaming all experts' weights from HBM once). The weights go from HBM
// straight into registers in bursts: every kSkGroup K steps a wave issues the
// next group's kSkGroup loads back to back, a whole group ahead of their use,
// so each of its 16 columns is requested as one contiguous 512-byte run. The
// gathered token rows (read again by every column tile, so mostly L2 hits)
// are staged in LDS in chunks of kSkKC elements of d, double buffered,
// written from registers one chunk ahead. Workgroup = one row tile x kSkBN
// columns; wave w owns columns 16w .. 16w + 15 of the tile and all four
// 16-row fragments. The epilogue is the one of proj_kernel with four
// consecutive columns per lane.
constexpr int kSkBN = 64;
constexpr int kSkKC = 128;
constexpr int kSkSteps = kSkKC / 32;   // K steps per token-row chunk
constexpr int kSkGroup = 2 * kSkSteps;  // K steps per weight burst (two chunks)
constexpr int kSkRowB = kSkKC * 2;      // LDS bytes per token row of a chunk

// DIRECT (decode batches of at most kSkDirectPairs pairs): no bucketing
// launch. A workgroup owns one expert and kSkBN columns; it finds its
// expert's pairs itself by reading the router's idx (all of it, a few KiB
// from L2), in pair order (wave ballots, then wave order), and walks them in
// row tiles of 64. Otherwise a workgroup owns one row tile of the bucketing
// kernel's schedule.
constexpr int kSkDirectPairs = 4096;
int proj_direct_max_pairs() { return kSkDirectPairs; }

template <bool DIRECT>
__global__ __launch_bounds__(256, 3) void proj_skinny_kernel(
    const bf16* __restrict__ u, const bf16* __restrict__ wexp, const int32_t* __restrict__ sorted,
    const float* __restrict__ sorted_w, const int4v* __restrict__ tile_info, int M, int D, int W,
    int HP, int GN, int k, int nrow_tiles, f16* __restrict__ X_hat, f16* __restrict__ B_hat,
    float* __restrict__ c_part, int bw_one, const int32_t* __restrict__ idx,
    const float* __restrict__ topk_w, int E) {
  typedef bf16x8 F;
  // chunk rows: 16-byte piece ch of row r at piece ch ^ (r % 16)
  __shared__ __align__(16) unsigned char abuf0[64 * kSkRowB];
  __shared__ __align__(16) unsigned char abuf1[64 * kSkRowB];
  __shared__ int rtok[64];
  __shared__ int rslot[64];
  __shared__ float rw[64];
  constexpr int NPL = DIRECT ? kSkDirectPairs : 1;
  __shared__ int plist[NPL];  // DIRECT: the expert's pair ids, ascending
  __shared__ int wcnt[16];

  const int CT = (W + kSkBN - 1) / kSkBN;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int ctile, e, nrt, total = 0;
  int4v ti = int4v{0, 0, 0, 0};
  if constexpr (DIRECT) {
    if (!xcd_unit(1, E, CT, e, ctile)) return;
    // rounds of 1024 pairs: p = r0 + 256 i + threadIdx.x, the round's four
    // loads issued before their first use
    const int pairs = M * k;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int run = 0;
    for (int r0 = 0; r0 < pairs; r0 += 1024) {
      int hit[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = r0 + 256 * i + threadIdx.x;
        hit[i] = p < pairs ? idx[p] : -1;
      }
      uint64_t bal[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bal[i] = __ballot(hit[i] == e);
        if (lane == 0) wcnt[4 * i + wave] = __popcll(bal[i]);
      }
      __syncthreads();
      // rank = hits of earlier rounds and quarters, earlier waves of this
      // quarter, earlier lanes of this wave
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int before = run;
        for (int w2 = 0; w2 < wave; ++w2) before += wcnt[4 * i + w2];
        if (hit[i] == e) plist[before + __popcll(bal[i] & below)] = r0 + 256 * i + threadIdx.x;
        run += wcnt[4 * i] + wcnt[4 * i + 1] + wcnt[4 * i + 2] + wcnt[4 * i + 3];
      }
      __syncthreads();  // wcnt is rewritten by the next round
    }
    total = run;
    nrt = (total + 63) / 64;
  } else {
    int tile;
    if (!xcd_tile(1, tile_info, nrow_tiles, CT, tile, ctile)) return;
    ti = tile_info[tile];  // {expert, first sorted row, rows}
    e = ti[0];
    if (e < 0) return;
    nrt = 1;
  }

  const int g = lane >> 4, c = lane & 15;
  const int col0 = ctile * kSkBN + 16 * wave;  // W is a multiple of 16: whole waves drop out
  const bool active = col0 < W;
  const int nsteps = D / 32;
  const int ngroups = (nsteps + kSkGroup - 1) / kSkGroup;
  const BufRes rA = make_rsrc(u, (uint64_t)M * D * 2);
  const BufRes rW = make_rsrc(wexp + (size_t)e * W * D, (uint64_t)W * D * 2);
  // weights: lane (g, c) reads column col0 + c, elements 32 s + 8 g .. + 7 of
  // K step s; steps past d read zeros
  const uint32_t wbase = active ? ((uint32_t)(col0 + c) * D + 8 * g) * 2 : kOOB;

  F wq[2 * kSkGroup];  // two bursts: the group in use and the next one
  auto burst = [&](auto par, int grp) {
    constexpr int PAR = decltype(par)::value;
#pragma unroll
    for (int j = 0; j < kSkGroup; ++j) {
      const int s = kSkGroup * grp + j;
      wq[kSkGroup * PAR + j] =
          load8_buf<bf16>(rW, (wbase == kOOB || s >= nsteps) ? kOOB : wbase + 64u * s);
    }
  };

  for (int rt = 0; rt < nrt; ++rt) {
  // the row tile's first weight burst does not depend on its rows: it is in
  // flight while the row table is filled
  burst(std::integral_constant<int, 0>(), 0);
  int nrows;
  if constexpr (DIRECT) {
    nrows = min(64, total - 64 * rt);
    if (threadIdx.x < 64) {
      const int r = threadIdx.x;
      if (r < nrows) {
        const int p = plist[64 * rt + r];
        rtok[r] = p / k;
        rslot[r] = p - (p / k) * k;
        rw[r] = topk_w[p];
      } else {
        rtok[r] = -1;
        rslot[r] = 0;
        rw[r] = 0.f;
      }
    }
  } else {
    const int row0 = ti[1];
    nrows = ti[2];
    if (threadIdx.x < 64) {
      const int r = threadIdx.x;
      if (r < nrows) {
        const int p = sorted[row0 + r];
        rtok[r] = p / k;
        rslot[r] = p - (p / k) * k;
        rw[r] = sorted_w[row0 + r];
      } else {
        rtok[r] = -1;
        rslot[r] = 0;
        rw[r] = 0.f;
      }
    }
  }
  __syncthreads();

  // token rows: thread t copies pieces q = t + 256 m of a chunk's 64 x 16 pieces
  uint32_t abase[4];
  int apiece[4], alds[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int q = threadIdx.x + 256 * m;
    const int r = q >> 4, ch = q & 15;
    apiece[m] = 8 * ch;
    abase[m] = r < nrows ? ((uint32_t)rtok[r] * D + 8 * ch) * 2 : kOOB;
    alds[m] = r * kSkRowB + 16 * (ch ^ (r & 15));
  }
  F ar[4];
  auto aload = [&](int chunk) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bool ok = abase[m] != kOOB && chunk * kSkKC + apiece[m] < D;
      ar[m] = load8_buf<bf16>(rA, ok ? abase[m] + chunk * kSkRowB : kOOB);
    }
  };
  auto awrite = [&](unsigned char* buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m) *reinterpret_cast<F*>(buf + alds[m]) = ar[m];
  };

  floatx4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the K steps of one chunk: weights from slots first .. first + 3
  auto steps = [&](auto first, const unsigned char* buf) {
    constexpr int S0 = decltype(first)::value;
#pragma unroll
    for (int j = 0; j < kSkSteps; ++j) {
      F a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const F*>(buf + (16 * i + c) * kSkRowB + 16 * ((4 * j + g) ^ c));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = mma16(wq[S0 + j], a[i], acc[i]);
    }
  };
  // One group (two chunks) with its weights in slot half PAR. Token rows of
  // the second chunk are requested before the next burst, so writing them to
  // LDS waits for them alone; the next group's burst is waited for only at
  // the end of this group.
  auto group = [&](auto par, int grp) {
    constexpr int PAR = decltype(par)::value;
    aload(2 * grp + 1);
    burst(std::integral_constant<int, 1 - PAR>(), grp + 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the burst's loads together
    steps(std::integral_constant<int, kSkGroup * PAR>(), abuf0);
    awrite(abuf1);
    __syncthreads();  // chunk 2 grp + 1 visible; abuf0 no longer read
    aload(2 * grp + 2);
    steps(std::integral_constant<int, kSkGroup * PAR + kSkSteps>(), abuf1);
    awrite(abuf0);
    __syncthreads();  // chunk 2 grp + 2 visible; abuf1 no longer read
  };
  aload(0);
  awrite(abuf0);
  __syncthreads();
  for (int grp = 0; grp < ngroups; grp += 2) {
    group(std::integral_constant<int, 0>(), grp);
    if (grp + 1 >= ngroups) break;
    group(std::integral_constant<int, 1>(), grp + 1);
  }

  // ---- epilogue: acc[i] holds, in lane (g, c), columns col0 + 4g .. + 3 of
  // pair row 16 i + c (H*P and G*N are multiples of 16: no region straddles)
  if (active) {
    const int col = col0 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + c;
      if (r >= nrows) continue;
      const size_t pair = (size_t)rtok[r] * k + rslot[r];
      const float wv = rw[r];
      const floatx4 v = acc[i];
      if (col < HP) {
        f16x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = from_f32<f16>(v[q]);
        *reinterpret_cast<f16x4*>(&X_hat[pair * HP + col]) = o;
      } else if (col < HP + GN) {
        f16x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = from_f32<f16>((bw_one ? 1.f : wv) * v[q]);
        *reinterpret_cast<f16x4*>(&B_hat[pair * GN + (col - HP)]) = o;
      } else {
        *reinterpret_cast<floatx4*>(&c_part[pair * GN + (col - HP - GN)]) = v * wv;
      }
    }
  }
  __syncthreads();  // the next row tile rewrites the row table and both chunk buffers
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
                                  const int32_t* sorted, const float* sorted_w,
                                  const int4v* tile_info, typename StreamOf<T>::type* B_hat,
                                  typename StreamOf<T>::type* X_hat, float* c_part,
                                  hipStream_t s) {
  const int pairs = g.M * g.k;
  const int nrow = proj_row_tiles_max(pairs, g.E, C::BM);
  const int ntiles = nrow * ((g.W + C::BN - 1) / C::BN);
  const dim3 grid((unsigned)((ntiles + 7) / 8 * 8));  // a multiple of the 8 XCDs
  hipEvent_t e0, e1;
  prof_kernel("expert_project", &e0, &e1);
  if (g.D % (kProjStages * ProjLay<T, C>::BK) == 0)
    hipExtLaunchKernelGGL((proj_kernel<T, C, false, float, true>), grid, dim3(C::NTH), 0, s, e0, e1,
                          0, u, wexp, sorted, sorted_w, tile_info, g.M, g.D, g.W, g.HP(), g.GN(),
                          g.k, nrow, X_hat, B_hat, c_part, (float*)nullptr, g.bw_one,
                          proj_group_rows());
  else
    hipExtLaunchKernelGGL((proj_kernel<T, C>), grid, dim3(C::NTH), 0, s, e0, e1, 0, u, wexp, sorted,
                          sorted_w, tile_info, g.M, g.D, g.W, g.HP(), g.GN(), g.k, nrow, X_hat,
                          B_hat, c_part, (float*)nullptr, g.bw_one, proj_group_rows());
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_project_t(const ProjGeom& g, const T* u, const T* wexp,
                                   const int32_t* sorted, const float* sorted_w,
                                   const int4v* ti, int bm, typename StreamOf<T>::type* B_hat,
                                   typename StreamOf<T>::type* X_hat, float* c_part,
                                   typename StreamOf<T>::type* C_mix, hipStream_t s) {
  typedef typename StreamOf<T>::type S;
  hipError_t err;
  if constexpr (sizeof(T) == 2) {
    // the 256 x 256 tile needs 2-byte K tiles to fit LDS
    if (bm == 64) {
      const int nrow = proj_row_tiles_max(g.M * g.k, g.E, 64);
      const int ntiles = nrow * ((g.W + kSkBN - 1) / kSkBN);
      hipEvent_t e0, e1;
      prof_kernel("expert_project", &e0, &e1);
      hipExtLaunchKernelGGL(proj_skinny_kernel<false>, dim3((unsigned)((ntiles + 7) / 8 * 8)),
                            dim3(256), 0, s, e0, e1, 0, u, wexp, sorted, sorted_w, ti, g.M, g.D,
                            g.W, g.HP(), g.GN(), g.k, nrow, X_hat, B_hat, c_part, g.bw_one,
                            (const int32_t*)nullptr, (const float*)nullptr, g.E);
      err = hipGetLastError();
    } else if (bm == 256)
      err = launch_proj_cfg<T, ProjBig>(g, u, wexp, sorted, sorted_w, ti, B_hat, X_hat, c_part, s);
    else if (bm == 128)
      err = launch_proj_cfg<T, ProjMid>(g, u, wexp, sorted, sorted_w, ti, B_hat, X_hat, c_part, s);
    else
      err = launch_proj_cfg<T, ProjSmall>(g, u, wexp, sorted, sorted_w, ti, B_hat, X_hat, c_part, s);
  } else {
    if (bm >= 128)
      err = launch_proj_cfg<T, ProjMid>(g, u, wexp, sorted, sorted_w, ti, B_hat, X_hat, c_part, s);
    else
      err = launch_proj_cfg<T, ProjSmall>(g, u, wexp, sorted, sorted_w, ti, B_hat, X_hat, c_part, s);
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

// Output projection out[M, N] = y[M, K] w_out[N, K]^T (fp32 accumulation, out in
// the input type): the expert projection's GEMM with rows in order.
template <typename T, class C>
static hipError_t launch_outproj_cfg(int M, int K, int N, const T* y, const T* w, T* out,
                                     hipStream_t s) {
  const int nrow = (M + C::BM - 1) / C::BM;
  const int units = nrow * ((N + C::BN - 1) / C::BN);
  prof_begin("output_project", s);
  const dim3 grid((unsigned)((units + 7) / 8 * 8));
  typedef typename StreamOf<T>::type S;
  if (K % (kProjStages * ProjLay<T, C>::BK) == 0)
    hipLaunchKernelGGL((proj_kernel<T, C, true, T, true>), grid, dim3(C::NTH), 0, s, y, w,
                       (const int32_t*)nullptr, (const float*)nullptr, (const int4v*)nullptr, M, K,
                       N, 0, 0, 1, nrow, (S*)nullptr, (S*)nullptr, (float*)nullptr, out, 0,
                       proj_group_rows());
  else
    hipLaunchKernelGGL((proj_kernel<T, C, true, T>), grid, dim3(C::NTH), 0, s, y, w,
                       (const int32_t*)nullptr, (const float*)nullptr, (const int4v*)nullptr, M, K,
                       N, 0, 0, 1, nrow, (S*)nullptr, (S*)nullptr, (float*)nullptr, out, 0,
                       proj_group_rows());
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_output_project(bool is_bf16, int M, int K, int N, const void* y,
                                 const void* w_out, void* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (is_bf16) {
    const bf16* yb = static_cast<const bf16*>(y);
    const bf16* wb = static_cast<const bf16*>(w_out);
    bf16* ob = static_cast<bf16*>(out);
    if (M >= 4096) return launch_outproj_cfg<bf16, ProjBig>(M, K, N, yb, wb, ob, s);
    if (M >= 512) return launch_outproj_cfg<bf16, ProjMid>(M, K, N, yb, wb, ob, s);
    return launch_outproj_cfg<bf16, ProjSmall>(M, K, N, yb, wb, ob, s);
  }
  const float* yf = static_cast<const float*>(y);
  const float* wf = static_cast<const float*>(w_out);
  float* of = static_cast<float*>(out);
  if (M >= 512) return launch_outproj_cfg<float, ProjMid>(M, K, N, yf, wf, of, s);
  return launch_outproj_cfg<float, ProjSmall>(M, K, N, yf, wf, of, s);
}

hipError_t launch_project_direct(const ProjGeom& g, const void* u, const void* w_experts,
                                 const int32_t* idx, const float* topk_w, void* B_hat,
                                 void* X_hat, float* c_part, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  const int units = g.E * ((g.W + kSkBN - 1) / kSkBN);
  hipEvent_t e0, e1;
  prof_kernel("expert_project", &e0, &e1);
  hipExtLaunchKernelGGL(proj_skinny_kernel<true>, dim3((unsigned)((units + 7) / 8 * 8)), dim3(256),
                        0, s, e0, e1, 0, (const bf16*)u, (const bf16*)w_experts,
                        (const int32_t*)nullptr, (const float*)nullptr, (const int4v*)nullptr, g.M,
                        g.D, g.W, g.HP(), g.GN(), g.k, 0, (f16*)X_hat, (f16*)B_hat, c_part,
                        g.bw_one, idx, topk_w, g.E);
  return hipGetLastError();
}

hipError_t launch_project(bool is_bf16, const ProjGeom& g, const void* u, const void* w_experts,
                          const int32_t* sorted, const float* sorted_w, const int32_t* tile_info,
                          int bm, void* B_hat, void* X_hat, float* c_part, void* C_mix,
                          hipStream_t s) {
  const int4v* ti = reinterpret_cast<const int4v*>(tile_info);
  if (is_bf16)
    return launch_project_t<bf16>(g, (const bf16*)u, (const bf16*)w_experts, sorted, sorted_w, ti,
                                  bm, (f16*)B_hat, (f16*)X_hat, c_part, (f16*)C_mix, s);
  return launch_project_t<float>(g, (const float*)u, (const float*)w_experts, sorted, sorted_w, ti,
                                 bm, (float*)B_hat, (float*)X_hat, c_part, (float*)C_mix, s);
}

}  // namespace swimba
