// Host-side launchers of the Swimba kernels. Each returns the hipError_t of
// its launch(es); arguments are validated by the API layer before any call.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swimba {

// Optional per-kernel timing (see swimba_profile_enable in the public header).
void prof_begin(const char* name, hipStream_t s);  // no-op unless profiling is on
void prof_end(hipStream_t s);
// One kernel timed under `name`: when profiling selects it, *start and *stop
// are events for the kernel's launch (hipExtLaunchKernelGGL), which takes the
// kernel's own start and end times, so no event packet goes between kernels
// (each such packet held the stream for several microseconds); otherwise both
// are null, and the launch behaves as a plain one.
void prof_kernel(const char* name, hipEvent_t* start, hipEvent_t* stop);

struct ProjGeom {
  int M, D, H, P, G, N, E, k, W;
  int bw_one = 0;  // B_hat without the routing weight (the separated-SSM layout)
  int HP() const { return H * P; }
  int GN() const { return G * N; }
};

// Router: logits (fp32), softmax, top-k. With `hist` non-null it also writes
// the expert histogram of each workgroup's route_tokens_per_wg(M) tokens
// ([nblk][E+1]).
constexpr int kRouteTok = 64;
// tokens per router workgroup: 16 for up to 1024 tokens (decode batches),
// so at least a few dozen workgroups share the router weights' reads
inline int route_tokens_per_wg(int64_t M) { return M <= 1024 ? 16 : kRouteTok; }
hipError_t launch_route(bool is_bf16, const void* u, const void* w_router, int M, int D, int E, int k,
                        int32_t* idx, float* w, float* logits, hipStream_t s,
                        int32_t* hist = nullptr);

// Bucketing of (token, slot) pairs by expert.
constexpr int kBucketPairs = 256;  // pairs per bucketing block
int bucket_blocks(int pairs);
// block_pairs: pairs per bucketing block (0 = kBucketPairs); counted: the
// histograms [nblk][E+1] are already in `counts` (written by the router).
// tile_info: 4 ints per GEMM row tile {expert (-1: none), first sorted row, rows, 0},
// ntiles_max + 1 entries (the last holds the number of real tiles).
hipError_t launch_bucket(bool is_bf16, const int32_t* idx, const float* topk_w, int pairs, int E,
                         int bm, int ntiles_max, int32_t* counts, int32_t* offsets,
                         int32_t* tile_info, int32_t* sorted, float* sorted_w, void* X_hat, int HP,
                         void* B_hat, int GN, float* c_part, hipStream_t s, int block_pairs = 0,
                         bool counted = false);

// Grouped expert projection with the mix epilogue, then the slot-ordered C sum.
int proj_row_tiles_max(int pairs, int E, int bm);
int proj_bm(int pairs, int E);
// C_mix == nullptr skips the slot sum (the caller consumes c_part itself).
// Decode batches (bf16, at most proj_direct_max_pairs() pairs): the skinny
// projection with every workgroup finding its expert's pairs in idx itself,
// with no bucketing launch before it.
int proj_direct_max_pairs();
hipError_t launch_project_direct(const ProjGeom& g, const void* u, const void* w_experts,
                                 const int32_t* idx, const float* topk_w, void* B_hat,
                                 void* X_hat, float* c_part, hipStream_t s);
hipError_t launch_project(bool is_bf16, const ProjGeom& g, const void* u, const void* w_experts,
                          const int32_t* sorted, const float* sorted_w, const int32_t* tile_info,
                          int bm, void* B_hat, void* X_hat, float* c_part, void* C_mix,
                          hipStream_t s);

// Chunked scan.
struct ScanGeom {
  int Bt, T, H, G, N, P, k, L;
  int es;            // bytes per stream element (2: fp16, 4: fp32)
  int bt;            // tokens per block of the scan (32 or 64)
  int segs;          // segments per sequence
  int seg_chunks;    // chunks per segment
  int walk;          // output walk: 0 one head per workgroup, 1 two heads, one block per step
  int sub;           // pass 1 walks each segment in `sub` pieces
};
// tv: the expert-mixed decay (its output pass walks one head per workgroup).
ScanGeom scan_geom(int Bt, int T, int H, int G, int N, int P, int k, int L, int es,
                   bool tv = false);
size_t scan_ws_bytes(const ScanGeom& g);
// ld: the expert-mixed decay's running log2 decay [Bt, H, T] (then a is not
// read), or nullptr for the shared decay a [H].
// y_f32: fp32 y for bf16 problems (k = 1 and the shared decay only).
hipError_t launch_scan(bool is_bf16, const ScanGeom& g, const void* B_hat, const void* X_hat,
                       const void* C_mix, const float* a, const float* h_init, void* y,
                       float* h_final, float* ws, hipStream_t s, const float* ld = nullptr,
                       bool y_f32 = false);

// Separated-SSM MoE (one trajectory per expert): per-expert dense streams of
// the Bt * E sequences (row (b E + e) T + t) from the selected pairs' X_hat,
// unweighted B_hat and weighted C parts, zeros where the expert is not
// selected; and y = the sum over experts of the trajectories' fp32 outputs.
hipError_t launch_sep_scatter(bool is_bf16, const int32_t* idx, const void* X_hat,
                              const void* B_hat, const float* c_part, int Bt, int T, int E, int k,
                              int HP, int GN, void* Xs, void* Bs, void* Cs, hipStream_t s);
hipError_t launch_sep_sum(bool is_bf16, const float* yp, int Bt, int T, int E, int HP, void* y,
                          hipStream_t s);

// Expert-mixed decay: running log2 of the per-token decay within each chunk
// of L tokens, ld [Bt, H, T], from the routing (idx, w [Bt*T, k]) and the
// per-expert decays a_experts [E, H].
hipError_t launch_mix_decay(const int32_t* idx, const float* w, const float* a_experts,
                            float* ld, int Bt, int T, int H, int E, int k, int L,
                            hipStream_t s);
hipError_t launch_state_copy(const float* src, float* dst, size_t n, hipStream_t s);
// dst[0 .. n) = 0 with a fill kernel (safe under stream capture).
hipError_t launch_fill_zero(float* dst, size_t n, hipStream_t s);

// Output projection out[M, N] = y[M, K] w_out[N, K]^T (out in the input type).
hipError_t launch_output_project(bool is_bf16, int M, int K, int N, const void* y,
                                 const void* w_out, void* out, hipStream_t s);

// Backward of the chunked scan (see swimba_ssd_chunk_scan_backward).
size_t scan_bwd_ws_bytes(bool is_bf16, int Bt, int T, int H, int G, int N, int k);
hipError_t launch_scan_backward(bool is_bf16, int Bt, int T, int H, int G, int N, int k,
                                const void* B_hat, const void* X_hat, const void* C_mix,
                                const void* dy, const float* a, const float* h_init,
                                const float* dh_final, float* dB, float* dX, float* dC, float* da,
                                float* dh_init, void* ws, hipStream_t s);

// Backward of the expert projections, the mix and the router (see
// swimba_expert_project_mix_backward). The forward's routing (idx, topk_w,
// logits), bucketing (sorted, sorted_w, offsets) and weighted streams (B_hat,
// c_part) are recomputed by the caller; dz, us, sw, dg, du_part and dwr_part
// are scratch (dwr_part of proj_bwd_splits(M) dW_r splits).
struct ProjBwdArgs {
  const void* u;          // [M, D] input type
  const void* w_router;   // [E, D]
  const void* w_experts;  // [E, W, D]
  const int32_t* idx;     // [M, k]
  const float* topk_w;    // [M, k]
  const float* dB;        // [M, k, G*N] gradient of B_hat
  const float* dX;        // [M, k, H*P] gradient of X_hat
  const float* dC;        // [M, G*N] gradient of C~
  float* du;              // [M, D]
  float* dWr;             // [E, D]
  float* dW;              // [E, W, D]
  const float* logits;    // [M, E]
  const void* B_hat;      // [M, k, G*N] stream type
  const float* c_part;    // [M, k, G*N]
  const int32_t* sorted;  // [M*k] pair ids grouped by expert
  const float* sorted_w;  // [M*k]
  const int32_t* offsets; // [E + 2]
  void* dz;               // [M*k, W] input type, sorted order
  void* us;               // [M*k, D] input type: the pairs' token rows of u, sorted order
  float* sw;              // [M*k] w_j dw_j by pair id
  float* dg;              // [M, E]
  float* du_part;         // [M*k, D] by pair id
  float* dwr_part;        // [nsplit, E, D]
  int M, D, E, k, W, HP, GN, nsplit;
};
int proj_bwd_splits(int M);
hipError_t launch_project_backward(bool is_bf16, ProjBwdArgs a, hipStream_t s);

// Decode: in-place state update and readout for one token per sequence.
// C~ is summed here from the per-slot fp32 parts c_part [Bt, k, G*N], in slot order.
// a_experts non-null: the expert-mixed decay, a_t = sum_j w_j a_experts[idx_j]
// / sum_j w_j from the routing (idx, w [Bt, k]); a is then not read.
hipError_t launch_decode_state(bool is_bf16, int Bt, int H, int G, int N, int P, int k,
                               const void* B_hat, const void* X_hat, const float* c_part,
                               const float* a, float* h, void* y, hipStream_t s,
                               const int32_t* idx = nullptr, const float* w = nullptr,
                               const float* a_experts = nullptr, int E = 0);

}  // namespace swimba
