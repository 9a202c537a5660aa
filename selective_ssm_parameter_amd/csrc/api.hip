// C ABI of the Swimba mixer: argument validation, workspace carving, dispatch.
// Every check runs before the first launch; no HIP call is made on an invalid
// argument, so outputs stay untouched and the call is safe without a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "swimba.h"

using namespace swimba;

// Scratch of swimba_decode_step_noalloc (see scratch_ptr below).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

swimba_status fail(swimba_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

swimba_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SWIMBA_OK;
  return fail(SWIMBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- dims

struct Dims {
  int64_t Bt, T, D, H, P, N, G, E, k, L, M, W, HP, GN;
  bool bf16;
  size_t esize;
};

swimba_status read_dims(const swimba_dims* d, Dims& o) {
  if (!d) return fail(SWIMBA_ERR_NULL, "dims is NULL");
  if (d->reserved != 0) return fail(SWIMBA_ERR_DIMS, "dims.reserved must be 0");
  if (d->dtype != SWIMBA_F32 && d->dtype != SWIMBA_BF16)
    return fail(SWIMBA_ERR_DIMS, "dims.dtype %d is not a swimba_dtype", d->dtype);
  if (d->batch < 0 || d->seqlen < 0) return fail(SWIMBA_ERR_DIMS, "batch and seqlen must be >= 0");
  if (d->d_model < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1 ||
      d->n_experts < 1 || d->chunk < 1)
    return fail(SWIMBA_ERR_DIMS, "d_model, nheads, headdim, dstate, ngroups, n_experts and chunk must be >= 1");
  if (d->nheads % d->ngroups != 0) return fail(SWIMBA_ERR_DIMS, "ngroups must divide nheads");
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(SWIMBA_ERR_DIMS, "top_k must lie in [1, n_experts]");
  o.Bt = d->batch; o.T = d->seqlen; o.D = d->d_model; o.H = d->nheads; o.P = d->headdim;
  o.N = d->dstate; o.G = d->ngroups; o.E = d->n_experts; o.k = d->top_k; o.L = d->chunk;
  o.M = o.Bt * o.T;
  o.HP = o.H * o.P;
  o.GN = o.G * o.N;
  o.W = o.HP + 2 * o.GN;
  o.bf16 = d->dtype == SWIMBA_BF16;
  o.esize = o.bf16 ? 2 : 4;  // stream element: fp16 for bf16 inputs, else fp32
  if (o.M * o.k >= (int64_t(1) << 30) || o.W * o.D >= (int64_t(1) << 31) ||
      o.HP > (1 << 20))
    return fail(SWIMBA_ERR_DIMS, "problem too large for 32-bit pair indexing");
  return SWIMBA_OK;
}

swimba_status check_kernel_shape(const Dims& d) {
  if (d.P != 64) return fail(SWIMBA_ERR_UNSUPPORTED, "headdim %lld: only 64 has a kernel", (long long)d.P);
  if (d.N != 16 && d.N != 32 && d.N != 64 && d.N != 128)
    return fail(SWIMBA_ERR_UNSUPPORTED, "dstate %lld: supported 16, 32, 64, 128", (long long)d.N);
  if (d.D % 32 != 0) return fail(SWIMBA_ERR_UNSUPPORTED, "d_model must be a multiple of 32");
  if (d.E > 256) return fail(SWIMBA_ERR_UNSUPPORTED, "n_experts must be <= 256");
  if (d.k > 8) return fail(SWIMBA_ERR_UNSUPPORTED, "top_k must be <= 8");
  return SWIMBA_OK;
}

// The kernels address HBM through buffer resources with 32-bit byte offsets:
// the token rows of u, the router and each expert's weight matrix as a whole,
// and the scan's streams of one sequence. Rows, columns and K steps a load must
// not read take the offset 2^31 (kOOB), which returns zeros only while it lies
// past the record, so records stay below 2^31 bytes (0x7FFFFFF0, "2 GiB"
// below). Larger tensors are rejected here instead of being read wrongly.
constexpr int64_t kMaxRecord = 0x7FFFFFF0ll;

swimba_status check_records(const Dims& d, bool router, bool experts) {
  const int64_t ein = d.bf16 ? 2 : 4;  // u and weight elements
  if (d.M * d.D * ein > kMaxRecord)
    return fail(SWIMBA_ERR_DIMS, "u is %lld bytes; the kernels address at most 2 GiB of it",
                (long long)(d.M * d.D * ein));
  if (router && d.E * d.D * ein > kMaxRecord)
    return fail(SWIMBA_ERR_DIMS, "w_router is larger than 2 GiB");
  if (experts && d.W * d.D * ein > kMaxRecord)
    return fail(SWIMBA_ERR_DIMS, "one expert's weights (%lld bytes) exceed 2 GiB",
                (long long)(d.W * d.D * ein));
  return SWIMBA_OK;
}

// Per sequence, the scan addresses B_hat, X_hat, C_mix and its Gram tiles
// with 32-bit byte offsets.
swimba_status check_scan_records(const Dims& d) {
  const int64_t es = (int64_t)d.esize;
  const int64_t nc = (d.T + d.L - 1) / d.L;
  const int64_t nb = (d.L + 31) / 32;
  const int64_t gram = nc * d.G * (nb * (nb + 1) / 2) * 32 * (32 * d.k) * es;
  if (d.T * d.k * d.HP * es > kMaxRecord || d.T * d.k * d.GN * es > kMaxRecord || gram > kMaxRecord)
    return fail(SWIMBA_ERR_DIMS,
                "one sequence's X_hat (%lld bytes) or Gram tiles (%lld bytes) exceed 2 GiB; "
                "split the sequence and pass the state on (h_final -> h_init)",
                (long long)(d.T * d.k * d.HP * es), (long long)gram);
  return SWIMBA_OK;
}

// kmax: the scans take top_k <= 4, the scan backward top_k <= 2.
swimba_status check_scan_shape(const Dims& d, int kmax = 4) {
  if (!d.bf16 && kmax > 2) kmax = 2;  // fp32 streams: two LDS stages fit for k <= 2 only
  if (d.k > kmax)
    return fail(SWIMBA_ERR_UNSUPPORTED, "this scan supports top_k <= %d for this dtype", kmax);
  if (d.L != 32 && d.L != 64 && d.L != 128 && d.L != 256)
    return fail(SWIMBA_ERR_UNSUPPORTED, "chunk must be 32, 64, 128 or 256");
  return SWIMBA_OK;
}

// ---------------------------------------------------------------- workspace

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ProjWs {
  size_t counts, offsets, tiles, sorted, sortw, cpart, total;
};

ProjWs proj_ws(const Dims& d) {
  const int64_t pairs = d.M * d.k;
  // histograms: blocks of kBucketPairs pairs, or of the router's workgroup
  // tokens when the router wrote them (decode)
  const int64_t tpw = route_tokens_per_wg(d.M);
  const int64_t nblk = std::max<int64_t>(bucket_blocks((int)pairs), (d.M + tpw - 1) / tpw);
  ProjWs w{};
  size_t off = 0;
  w.counts = off; off += align256(sizeof(int32_t) * nblk * (d.E + 1));
  w.offsets = off; off += align256(sizeof(int32_t) * (d.E + 2));
  // tile table: 4 ints per row tile, for the smallest row tile (most tiles)
  w.tiles = off; off += align256(sizeof(int32_t) * 4 * ((size_t)proj_row_tiles_max((int)pairs, (int)d.E, 64) + 1));
  w.sorted = off; off += align256(sizeof(int32_t) * pairs);
  w.sortw = off; off += align256(sizeof(float) * pairs);
  w.cpart = off; off += align256(sizeof(float) * pairs * d.GN);
  w.total = off;
  return w;
}

struct DecWs {
  size_t idx, w, bhat, xhat, proj, total;
};

DecWs dec_ws(const Dims& d) {
  DecWs w{};
  size_t off = 0;
  const int64_t pairs = d.Bt * d.k;
  w.idx = off; off += align256(sizeof(int32_t) * pairs);
  w.w = off; off += align256(sizeof(float) * pairs);
  w.bhat = off; off += align256(d.esize * pairs * d.GN);
  w.xhat = off; off += align256(d.esize * pairs * d.HP);
  w.proj = off;
  Dims one = d;
  one.T = 1;
  one.M = d.Bt;
  off += proj_ws(one).total;
  w.total = off;
  return w;
}

// Backward of projection, mix and router: the recomputed forward (routing,
// bucketing, weighted streams) and the backward's scratch.
struct PbwdWs {
  size_t idx, w, logits, proj, bhat, xhat, dz, us, sw, dg, dupart, dwrpart, total;
};

// saved: the forward's routing, B_hat and projection workspace are passed in
// (swimba_expert_project_mix_backward_saved), so none of them is recomputed.
PbwdWs pbwd_ws(const Dims& d, bool saved = false) {
  PbwdWs w{};
  size_t off = 0;
  const int64_t pairs = d.M * d.k;
  if (!saved) {
    w.idx = off; off += align256(sizeof(int32_t) * pairs);
    w.w = off; off += align256(sizeof(float) * pairs);
    w.logits = off; off += align256(sizeof(float) * d.M * d.E);
    w.proj = off; off += proj_ws(d).total;
    w.bhat = off; off += align256(d.esize * pairs * d.GN);
    w.xhat = off; off += align256(d.esize * pairs * d.HP);
  }
  w.dz = off; off += align256(d.esize * pairs * d.W);
  w.us = off; off += align256(d.esize * pairs * d.D);
  w.sw = off; off += align256(sizeof(float) * pairs);
  w.dg = off; off += align256(sizeof(float) * d.M * d.E);
  w.dupart = off; off += align256(sizeof(float) * pairs * d.D);
  w.dwrpart = off; off += align256(sizeof(float) * proj_bwd_splits((int)d.M) * d.E * d.D);
  w.total = off;
  return w;
}

// Separated-SSM MoE: the routing, the projection of the selected pairs, the
// per-expert dense streams of the Bt * E trajectories, their fp32 outputs and
// the scan's own workspace for them.
Dims sep_dims(const Dims& d) {
  Dims s = d;
  s.Bt = d.Bt * d.E;
  s.k = 1;
  s.M = s.Bt * d.T;
  return s;
}

size_t scan_bytes(const Dims& d);

struct SepWs {
  size_t idx, w, proj, xhat, bhat, xs, bs, cs, yp, scan, total;
};

SepWs sep_ws(const Dims& d) {
  SepWs w{};
  size_t off = 0;
  const int64_t pairs = d.M * d.k, rows = d.Bt * d.E * d.T;
  w.idx = off; off += align256(sizeof(int32_t) * pairs);
  w.w = off; off += align256(sizeof(float) * pairs);
  w.proj = off; off += proj_ws(d).total;
  w.xhat = off; off += align256(d.esize * pairs * d.HP);
  w.bhat = off; off += align256(d.esize * pairs * d.GN);
  w.xs = off; off += align256(d.esize * rows * d.HP);
  w.bs = off; off += align256(d.esize * rows * d.GN);
  w.cs = off; off += align256(d.esize * rows * d.GN);
  w.yp = off; off += align256(sizeof(float) * rows * d.HP);
  w.scan = off; off += scan_bytes(sep_dims(d));
  w.total = off;
  return w;
}

// The shared-decay and the expert-mixed scans may walk different segment
// counts; one workspace query (SWIMBA_CALL_SCAN) serves both.
size_t scan_bytes(const Dims& d) {
  return std::max(scan_ws_bytes(scan_geom((int)d.Bt, (int)d.T, (int)d.H, (int)d.G, (int)d.N,
                                          (int)d.P, (int)d.k, (int)d.L, (int)d.esize, false)),
                  scan_ws_bytes(scan_geom((int)d.Bt, (int)d.T, (int)d.H, (int)d.G, (int)d.N,
                                          (int)d.P, (int)d.k, (int)d.L, (int)d.esize, true)));
}

swimba_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SWIMBA_OK;
  if (!ws) return fail(SWIMBA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (have < need) return fail(SWIMBA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, have);
  if (!aligned16(ws)) return fail(SWIMBA_ERR_ALIGN, "workspace is not 16-byte aligned");
  return SWIMBA_OK;
}

#define REQUIRE_PTR(p)                                                  \
  do {                                                                  \
    if (!(p)) return fail(SWIMBA_ERR_NULL, "%s is NULL", #p);           \
    if (!aligned16(p)) return fail(SWIMBA_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)
#define OPTIONAL_PTR(p)                                                 \
  do {                                                                  \
    if ((p) && !aligned16(p)) return fail(SWIMBA_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

ProjGeom proj_geom(const Dims& d, int64_t M, bool bw_one = false) {
  ProjGeom g;
  g.bw_one = bw_one ? 1 : 0;
  g.M = (int)M; g.D = (int)d.D; g.H = (int)d.H; g.P = (int)d.P; g.G = (int)d.G; g.N = (int)d.N;
  g.E = (int)d.E; g.k = (int)d.k; g.W = (int)d.W;
  return g;
}

// Runs bucketing, the grouped projection and (with C_mix non-null) the
// slot-ordered C sum for M tokens. routed: the router already wrote the
// expert histograms of its workgroups' tokens into the workspace.
hipError_t run_project(const Dims& d, int64_t M, const void* u, const void* w_experts,
                       const int32_t* idx, const float* w, void* B_hat, void* X_hat, void* C_mix,
                       unsigned char* ws, hipStream_t s, bool routed = false, bool bw_one = false) {
  Dims dm = d;
  dm.M = M;
  const ProjWs lay = proj_ws(dm);
  const int pairs = (int)(M * d.k);
  int bm = proj_bm(pairs, (int)d.E);
  if (!d.bf16 && bm > 128) bm = 128;  // fp32 tiles of 256 x 256 do not fit LDS
  int32_t* counts = reinterpret_cast<int32_t*>(ws + lay.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + lay.offsets);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + lay.tiles);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + lay.sorted);
  float* sortw = reinterpret_cast<float*>(ws + lay.sortw);
  float* cpart = reinterpret_cast<float*>(ws + lay.cpart);
  const int ntiles_max = proj_row_tiles_max(pairs, (int)d.E, bm);
  hipError_t e = launch_bucket(d.bf16, idx, w, pairs, (int)d.E, bm, ntiles_max, counts, offsets,
                               tiles, sorted, sortw, X_hat, (int)d.HP, B_hat, (int)d.GN, cpart, s,
                               routed ? (int)(route_tokens_per_wg(M) * d.k) : 0, routed);
  if (e != hipSuccess) return e;
  return launch_project(d.bf16, proj_geom(d, M, bw_one), u, w_experts, sorted, sortw, tiles, bm,
                        B_hat, X_hat, cpart, C_mix, s);
}

// ---------------------------------------------------------------- profiling

struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<std::string> g_prof_only;  // record only these kernel names (empty: all)
thread_local const char* g_prof_prefix = "";  // "decode_" inside swimba_decode_step
bool g_prof_open = false;                      // a begin without its end yet
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t ev = g_prof_pool.back();
    g_prof_pool.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

}  // namespace

namespace swimba {

void prof_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  std::string full = std::string(g_prof_prefix) + name;
  if (!g_prof_only.empty() &&
      std::find(g_prof_only.begin(), g_prof_only.end(), full) == g_prof_only.end())
    return;
  ProfRec r{full, prof_event(), prof_event()};
  if (!r.start || !r.stop) return;
  g_prof_open = true;
  hipEventRecord(r.start, s);
  g_prof_recs.push_back(r);
}

void prof_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || !g_prof_open || g_prof_recs.empty()) return;
  g_prof_open = false;
  hipEventRecord(g_prof_recs.back().stop, s);
}

void prof_kernel(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  std::string full = std::string(g_prof_prefix) + name;
  if (!g_prof_only.empty() &&
      std::find(g_prof_only.begin(), g_prof_only.end(), full) == g_prof_only.end())
    return;
  ProfRec r{full, prof_event(), prof_event()};
  if (!r.start || !r.stop) return;
  g_prof_recs.push_back(r);
  *start = r.start;
  *stop = r.stop;
}

}  // namespace swimba

// ---------------------------------------------------------------- C ABI

extern "C" {

int32_t swimba_abi_version(void) { return SWIMBA_ABI_VERSION; }

const char* swimba_last_error(void) { return g_err.c_str(); }

size_t swimba_workspace_size(const swimba_dims* dims, int32_t call) {
  Dims d;
  std::string saved = g_err;
  const swimba_status st = read_dims(dims, d);
  g_err = saved;
  if (st != SWIMBA_OK) return 0;
  switch (call) {
    case SWIMBA_CALL_ROUTE: return 0;
    case SWIMBA_CALL_PROJECT: return d.M == 0 ? 0 : proj_ws(d).total;
    case SWIMBA_CALL_SCAN: return scan_bytes(d);
    case SWIMBA_CALL_DECODE: return d.Bt == 0 ? 0 : dec_ws(d).total;
    case SWIMBA_CALL_SCAN_BACKWARD:
      return d.M == 0 ? 0 : scan_bwd_ws_bytes(d.bf16, (int)d.Bt, (int)d.T, (int)d.H, (int)d.G, (int)d.N, (int)d.k);
    case SWIMBA_CALL_PROJECT_BACKWARD: return d.M == 0 ? 0 : pbwd_ws(d).total;
    case SWIMBA_CALL_PROJECT_BACKWARD_SAVED: return d.M == 0 ? 0 : pbwd_ws(d, true).total;
    case SWIMBA_CALL_SEPARATED: return d.M == 0 ? 0 : sep_ws(d).total;
    default: return 0;
  }
}

swimba_status swimba_route_topk(const swimba_dims* dims, const void* u, const void* w_router,
                                int32_t* topk_idx, float* topk_w, float* logits,
                                hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_records(d, true, false)) != SWIMBA_OK) return st;
  if (d.M == 0) return SWIMBA_OK;
  REQUIRE_PTR(u);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  OPTIONAL_PTR(logits);
  return hip_status(launch_route(d.bf16, u, w_router, (int)d.M, (int)d.D, (int)d.E, (int)d.k,
                                 topk_idx, topk_w, logits, stream),
                    "route_topk launch");
}

swimba_status swimba_expert_project_mix(const swimba_dims* dims, const void* u,
                                        const void* w_experts, const int32_t* topk_idx,
                                        const float* topk_w, void* B_hat, void* X_hat,
                                        void* C_mix, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_records(d, false, true)) != SWIMBA_OK) return st;
  if (d.M == 0) return SWIMBA_OK;
  REQUIRE_PTR(u);
  REQUIRE_PTR(w_experts);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(B_hat);
  REQUIRE_PTR(X_hat);
  REQUIRE_PTR(C_mix);
  if ((st = check_ws(ws, ws_bytes, proj_ws(d).total)) != SWIMBA_OK) return st;
  return hip_status(run_project(d, d.M, u, w_experts, topk_idx, topk_w, B_hat, X_hat, C_mix,
                                static_cast<unsigned char*>(ws), stream),
                    "expert_project_mix launch");
}

}  // extern "C"

namespace {

// The backward of router, projections and mix. saved == false: the forward's
// routing and projection are recomputed into the workspace; saved == true:
// they come from the caller (the router's outputs, the forward's B_hat and
// the workspace of the swimba_expert_project_mix call that produced it).
swimba_status pbwd_impl(bool saved, const swimba_dims* dims, const void* u, const void* w_router,
                        const void* w_experts, const int32_t* topk_idx, const float* topk_w,
                        const float* logits, const void* B_hat, const void* fwd_ws,
                        size_t fwd_ws_bytes, const float* dB_hat, const float* dX_hat,
                        const float* dC_mix, float* du, float* dW_router, float* dW_experts,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_records(d, true, true)) != SWIMBA_OK) return st;
  // the backward GEMMs address an expert's pair rows with 32-bit byte offsets
  if (d.M * d.k * d.D * (int64_t)d.esize >= (int64_t(1) << 31) ||
      d.M * d.k * d.W * (int64_t)d.esize >= (int64_t(1) << 31))
    return fail(SWIMBA_ERR_DIMS, "problem too large for 31-bit pair-row offsets");
  REQUIRE_PTR(dW_router);
  REQUIRE_PTR(dW_experts);
  if (d.M == 0) {
    // no tokens: the weight gradients are zero
    hipError_t e = launch_fill_zero(dW_router, (size_t)(d.E * d.D), stream);
    if (e == hipSuccess) e = launch_fill_zero(dW_experts, (size_t)(d.E * d.W * d.D), stream);
    return hip_status(e, "expert_project_mix_backward launch");
  }
  REQUIRE_PTR(u);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(w_experts);
  REQUIRE_PTR(dB_hat);
  REQUIRE_PTR(dX_hat);
  REQUIRE_PTR(dC_mix);
  REQUIRE_PTR(du);
  const ProjWs play = proj_ws(d);
  if (saved) {
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(logits);
    REQUIRE_PTR(B_hat);
    if ((st = check_ws(const_cast<void*>(fwd_ws), fwd_ws_bytes, play.total)) != SWIMBA_OK) {
      g_err = "forward " + g_err;
      return st;
    }
  }
  const PbwdWs lay = pbwd_ws(d, saved);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != SWIMBA_OK) return st;
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  const int32_t* idx = topk_idx;
  const float* tw = topk_w;
  const float* lg = logits;
  const void* bhat = B_hat;
  const unsigned char* pws = static_cast<const unsigned char*>(fwd_ws);
  if (!saved) {
    // the forward's routing and weighted streams, recomputed with its own kernels
    int32_t* ridx = reinterpret_cast<int32_t*>(w8 + lay.idx);
    float* rw = reinterpret_cast<float*>(w8 + lay.w);
    float* rlg = reinterpret_cast<float*>(w8 + lay.logits);
    hipError_t e = launch_route(d.bf16, u, w_router, (int)d.M, (int)d.D, (int)d.E, (int)d.k,
                                ridx, rw, rlg, stream);
    if (e != hipSuccess) return hip_status(e, "expert_project_mix_backward route launch");
    e = run_project(d, d.M, u, w_experts, ridx, rw, w8 + lay.bhat, w8 + lay.xhat, nullptr,
                    w8 + lay.proj, stream);
    if (e != hipSuccess) return hip_status(e, "expert_project_mix_backward projection launch");
    idx = ridx;
    tw = rw;
    lg = rlg;
    bhat = w8 + lay.bhat;
    pws = w8 + lay.proj;
  }
  ProjBwdArgs a{};
  a.u = u; a.w_router = w_router; a.w_experts = w_experts;
  a.idx = idx; a.topk_w = tw; a.dB = dB_hat; a.dX = dX_hat; a.dC = dC_mix;
  a.du = du; a.dWr = dW_router; a.dW = dW_experts; a.logits = lg;
  a.B_hat = bhat;
  a.c_part = reinterpret_cast<const float*>(pws + play.cpart);
  a.sorted = reinterpret_cast<const int32_t*>(pws + play.sorted);
  a.sorted_w = reinterpret_cast<const float*>(pws + play.sortw);
  a.offsets = reinterpret_cast<const int32_t*>(pws + play.offsets);
  a.dz = w8 + lay.dz;
  a.us = w8 + lay.us;
  a.sw = reinterpret_cast<float*>(w8 + lay.sw);
  a.dg = reinterpret_cast<float*>(w8 + lay.dg);
  a.du_part = reinterpret_cast<float*>(w8 + lay.dupart);
  a.dwr_part = reinterpret_cast<float*>(w8 + lay.dwrpart);
  a.M = (int)d.M; a.D = (int)d.D; a.E = (int)d.E; a.k = (int)d.k; a.W = (int)d.W;
  a.HP = (int)d.HP; a.GN = (int)d.GN;
  return hip_status(launch_project_backward(d.bf16, a, stream),
                    "expert_project_mix_backward launch");
}

}  // namespace

extern "C" {

swimba_status swimba_expert_project_mix_backward(
    const swimba_dims* dims, const void* u, const void* w_router, const void* w_experts,
    const float* dB_hat, const float* dX_hat, const float* dC_mix, float* du, float* dW_router,
    float* dW_experts, void* ws, size_t ws_bytes, hipStream_t stream) {
  return pbwd_impl(false, dims, u, w_router, w_experts, nullptr, nullptr, nullptr, nullptr,
                   nullptr, 0, dB_hat, dX_hat, dC_mix, du, dW_router, dW_experts, ws, ws_bytes,
                   stream);
}

swimba_status swimba_expert_project_mix_backward_saved(
    const swimba_dims* dims, const void* u, const void* w_router, const void* w_experts,
    const int32_t* topk_idx, const float* topk_w, const float* logits, const void* B_hat,
    const void* fwd_ws, size_t fwd_ws_bytes, const float* dB_hat, const float* dX_hat,
    const float* dC_mix, float* du, float* dW_router, float* dW_experts, void* ws,
    size_t ws_bytes, hipStream_t stream) {
  return pbwd_impl(true, dims, u, w_router, w_experts, topk_idx, topk_w, logits, B_hat, fwd_ws,
                   fwd_ws_bytes, dB_hat, dX_hat, dC_mix, du, dW_router, dW_experts, ws,
                   ws_bytes, stream);
}

}  // extern "C"

namespace {

// The chunked scan with the shared decay a [H] (mixed false) or the
// expert-mixed decay given as running log2 sums log_decay [Bt, H, T] (a unused).
swimba_status scan_impl(bool mixed, const swimba_dims* dims, const void* B_hat,
                        const void* X_hat, const void* C_mix, const float* a, const float* log_decay,
                        const float* h_init, void* y, float* h_final, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_scan_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_scan_records(d)) != SWIMBA_OK) return st;
  if (d.Bt == 0) return SWIMBA_OK;
  if (mixed) {
    if (d.T > 0) REQUIRE_PTR(log_decay);
  } else {
    REQUIRE_PTR(a);
  }
  OPTIONAL_PTR(h_init);
  OPTIONAL_PTR(h_final);
  if (d.M > 0) {
    REQUIRE_PTR(B_hat);
    REQUIRE_PTR(X_hat);
    REQUIRE_PTR(C_mix);
    REQUIRE_PTR(y);
  }
  if ((st = check_ws(ws, ws_bytes, scan_bytes(d))) != SWIMBA_OK) return st;
  const ScanGeom g = scan_geom((int)d.Bt, (int)d.T, (int)d.H, (int)d.G, (int)d.N, (int)d.P,
                               (int)d.k, (int)d.L, (int)d.esize, mixed);
  return hip_status(launch_scan(d.bf16, g, B_hat, X_hat, C_mix, a, h_init, y, h_final,
                                static_cast<float*>(ws), stream, log_decay),
                    "ssd_chunk_scan launch");
}

}  // namespace

extern "C" {

swimba_status swimba_ssd_chunk_scan(const swimba_dims* dims, const void* B_hat,
                                    const void* X_hat, const void* C_mix, const float* a,
                                    const float* h_init, void* y, float* h_final, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  return scan_impl(false, dims, B_hat, X_hat, C_mix, a, nullptr, h_init, y, h_final, ws,
                   ws_bytes, stream);
}

swimba_status swimba_ssd_chunk_scan_mixed(const swimba_dims* dims, const void* B_hat,
                                          const void* X_hat, const void* C_mix,
                                          const float* log_decay, const float* h_init, void* y,
                                          float* h_final, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  // with no tokens the scan only copies the state and never reads the decay;
  // the launcher takes a non-null decay as the mixed mode
  alignas(16) static const float kNoTokens[4] = {0.f, 0.f, 0.f, 0.f};
  const float* ld = log_decay;
  if (!ld && dims && dims->seqlen == 0) ld = kNoTokens;
  return scan_impl(true, dims, B_hat, X_hat, C_mix, nullptr, ld, h_init, y, h_final, ws,
                   ws_bytes, stream);
}

swimba_status swimba_ssd_chunk_scan_backward(const swimba_dims* dims, const void* B_hat,
                                             const void* X_hat, const void* C_mix,
                                             const float* a, const float* h_init, const void* dy,
                                             const float* dh_final, float* dB_hat, float* dX_hat,
                                             float* dC_mix, float* da, float* dh_init, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_scan_shape(d, 2)) != SWIMBA_OK) return st;
  if (d.M * d.HP * 4 >= (int64_t(1) << 40)) return fail(SWIMBA_ERR_DIMS, "problem too large");
  REQUIRE_PTR(da);
  REQUIRE_PTR(a);
  OPTIONAL_PTR(h_init);
  OPTIONAL_PTR(dh_final);
  OPTIONAL_PTR(dh_init);
  if (d.M > 0) {
    REQUIRE_PTR(B_hat);
    REQUIRE_PTR(X_hat);
    REQUIRE_PTR(C_mix);
    REQUIRE_PTR(dy);
    REQUIRE_PTR(dB_hat);
    REQUIRE_PTR(dX_hat);
    REQUIRE_PTR(dC_mix);
  }
  const size_t need =
      d.M == 0 ? 0 : scan_bwd_ws_bytes(d.bf16, (int)d.Bt, (int)d.T, (int)d.H, (int)d.G, (int)d.N, (int)d.k);
  if ((st = check_ws(ws, ws_bytes, need)) != SWIMBA_OK) return st;
  return hip_status(launch_scan_backward(d.bf16, (int)d.Bt, (int)d.T, (int)d.H, (int)d.G,
                                         (int)d.N, (int)d.k, B_hat, X_hat, C_mix, dy, a, h_init,
                                         dh_final, dB_hat, dX_hat, dC_mix, da, dh_init, ws,
                                         stream),
                    "ssd_chunk_scan_backward launch");
}

swimba_status swimba_mix_decay(const swimba_dims* dims, const int32_t* topk_idx,
                               const float* topk_w, const float* a_experts, float* log_decay,
                               hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if (d.L != 32 && d.L != 64 && d.L != 128 && d.L != 256)
    return fail(SWIMBA_ERR_UNSUPPORTED, "chunk must be 32, 64, 128 or 256");
  if (d.M * d.H >= (int64_t(1) << 31)) return fail(SWIMBA_ERR_DIMS, "batch * seqlen * nheads too large");
  if (d.M == 0) return SWIMBA_OK;
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(a_experts);
  REQUIRE_PTR(log_decay);
  return hip_status(launch_mix_decay(topk_idx, topk_w, a_experts, log_decay, (int)d.Bt,
                                     (int)d.T, (int)d.H, (int)d.E, (int)d.k, (int)d.L, stream),
                    "mix_decay launch");
}

}  // extern "C"

namespace {

// Scratch of swimba_decode_step_noalloc: the decode workspace (routing,
// streams, bucketing, per-slot C parts) of one call, in a file-scope device
// array instead of caller memory. Each device holds its own copy for the life
// of the process; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in). Nothing in it needs to start at zero: every byte a
// decode step reads was written earlier in the same step.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
swimba_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SWIMBA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SWIMBA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SWIMBA_OK;
}

// noalloc: the workspace is the device's static scratch (ws is ignored).
swimba_status decode_impl(bool mixed, const swimba_dims* dims, const void* u,
                          const void* w_router, const void* w_experts, const float* a,
                          const float* a_experts, float* h, void* y, int32_t* topk_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream, bool noalloc = false) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if (d.T != 1) return fail(SWIMBA_ERR_DIMS, "decode_step needs seqlen == 1");
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_records(d, true, true)) != SWIMBA_OK) return st;
  if (d.Bt == 0) return SWIMBA_OK;
  REQUIRE_PTR(u);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(w_experts);
  if (mixed) {
    REQUIRE_PTR(a_experts);
  } else {
    REQUIRE_PTR(a);
  }
  REQUIRE_PTR(h);
  REQUIRE_PTR(y);
  OPTIONAL_PTR(topk_idx);
  const DecWs lay = dec_ws(d);
  if (noalloc) {
    if (lay.total > kScratchBytes)
      return fail(SWIMBA_ERR_WORKSPACE,
                  "decode_step_noalloc: these dims need %zu bytes of scratch; the static "
                  "scratch holds %zu (use swimba_decode_step with a workspace)",
                  lay.total, kScratchBytes);
    if ((st = scratch_ptr(&ws)) != SWIMBA_OK) return st;
    ws_bytes = kScratchBytes;
  } else if ((st = check_ws(ws, ws_bytes, lay.total)) != SWIMBA_OK) {
    return st;
  }
  struct PrefixGuard {
    PrefixGuard() { g_prof_prefix = "decode_"; }
    ~PrefixGuard() { g_prof_prefix = ""; }
  } prefix_guard;
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w8 + lay.idx);
  float* tw = reinterpret_cast<float*>(w8 + lay.w);
  void* bhat = w8 + lay.bhat;
  void* xhat = w8 + lay.xhat;
  Dims d1 = d;
  d1.M = d.Bt;
  const ProjWs play = proj_ws(d1);
  unsigned char* pws = w8 + lay.proj;
  // bf16 batches whose experts get a few dozen pairs each: the skinny
  // projection finds every expert's pairs in idx itself (no bucketing launch)
  const int pairs = (int)(d.Bt * d.k);
  const bool direct = d.bf16 && proj_bm(pairs, (int)d.E) == 64 && pairs <= proj_direct_max_pairs();
  hipError_t e = launch_route(d.bf16, u, w_router, (int)d.Bt, (int)d.D, (int)d.E, (int)d.k, idx,
                              tw, nullptr, stream,
                              direct ? nullptr : reinterpret_cast<int32_t*>(pws + play.counts));
  if (e != hipSuccess) return hip_status(e, "decode_step route launch");
  if (direct)
    e = launch_project_direct(proj_geom(d, d.Bt), u, w_experts, idx, tw, bhat, xhat,
                              reinterpret_cast<float*>(pws + play.cpart), stream);
  else
    e = run_project(d, d.Bt, u, w_experts, idx, tw, bhat, xhat, nullptr, pws, stream, true);
  if (e != hipSuccess) return hip_status(e, "decode_step projection launch");
  e = launch_decode_state(d.bf16, (int)d.Bt, (int)d.H, (int)d.G, (int)d.N, (int)d.P, (int)d.k,
                          bhat, xhat, reinterpret_cast<const float*>(pws + play.cpart), a, h, y,
                          stream, idx, tw, a_experts, (int)d.E);
  return hip_status(e, "decode_step state launch");
}

}  // namespace

extern "C" {

swimba_status swimba_decode_step(const swimba_dims* dims, const void* u, const void* w_router,
                                 const void* w_experts, const float* a, float* h, void* y,
                                 int32_t* topk_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  return decode_impl(false, dims, u, w_router, w_experts, a, nullptr, h, y, topk_idx, ws,
                     ws_bytes, stream);
}

swimba_status swimba_decode_step_noalloc(const swimba_dims* dims, const void* u,
                                         const void* w_router, const void* w_experts,
                                         const float* a, float* h, void* y, int32_t* topk_idx,
                                         hipStream_t stream) {
  return decode_impl(false, dims, u, w_router, w_experts, a, nullptr, h, y, topk_idx, nullptr, 0,
                     stream, true);
}

swimba_status swimba_decode_step_mixed(const swimba_dims* dims, const void* u,
                                       const void* w_router, const void* w_experts,
                                       const float* a_experts, float* h, void* y,
                                       int32_t* topk_idx, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  return decode_impl(true, dims, u, w_router, w_experts, nullptr, a_experts, h, y, topk_idx, ws,
                     ws_bytes, stream);
}

swimba_status swimba_separated_forward(const swimba_dims* dims, const void* u,
                                       const void* w_router, const void* w_experts,
                                       const float* a, const float* h_init, void* y,
                                       float* h_final, int32_t* topk_idx, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if ((st = check_kernel_shape(d)) != SWIMBA_OK) return st;
  if ((st = check_records(d, true, true)) != SWIMBA_OK) return st;
  const Dims ds = sep_dims(d);
  if (ds.Bt > INT32_MAX || ds.M * d.HP >= (int64_t(1) << 40))
    return fail(SWIMBA_ERR_DIMS, "batch * n_experts trajectories too large");
  if ((st = check_scan_shape(ds)) != SWIMBA_OK) return st;
  if ((st = check_scan_records(ds)) != SWIMBA_OK) return st;
  if (d.Bt == 0) return SWIMBA_OK;
  REQUIRE_PTR(a);
  OPTIONAL_PTR(h_init);
  OPTIONAL_PTR(h_final);
  const ScanGeom g = scan_geom((int)ds.Bt, (int)ds.T, (int)ds.H, (int)ds.G, (int)ds.N, (int)ds.P,
                               1, (int)ds.L, (int)ds.esize);
  if (d.M == 0)  // no tokens: the states pass through unchanged
    return hip_status(launch_scan(d.bf16, g, nullptr, nullptr, nullptr, a, h_init, nullptr,
                                  h_final, nullptr, stream),
                      "separated_forward launch");
  REQUIRE_PTR(u);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(w_experts);
  REQUIRE_PTR(y);
  OPTIONAL_PTR(topk_idx);
  const SepWs lay = sep_ws(d);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != SWIMBA_OK) return st;
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w8 + lay.idx);
  float* tw = reinterpret_cast<float*>(w8 + lay.w);
  hipError_t e = launch_route(d.bf16, u, w_router, (int)d.M, (int)d.D, (int)d.E, (int)d.k, idx,
                              tw, nullptr, stream);
  if (e != hipSuccess) return hip_status(e, "separated_forward route launch");
  // the selected pairs' X, B (unweighted) and pi * C parts
  e = run_project(d, d.M, u, w_experts, idx, tw, w8 + lay.bhat, w8 + lay.xhat, nullptr,
                  w8 + lay.proj, stream, false, true);
  if (e != hipSuccess) return hip_status(e, "separated_forward projection launch");
  const ProjWs play = proj_ws(d);
  e = launch_sep_scatter(d.bf16, idx, w8 + lay.xhat, w8 + lay.bhat,
                         reinterpret_cast<const float*>(w8 + lay.proj + play.cpart), (int)d.Bt,
                         (int)d.T, (int)d.E, (int)d.k, (int)d.HP, (int)d.GN, w8 + lay.xs,
                         w8 + lay.bs, w8 + lay.cs, stream);
  if (e != hipSuccess) return hip_status(e, "separated_forward scatter launch");
  float* yp = reinterpret_cast<float*>(w8 + lay.yp);
  e = launch_scan(d.bf16, g, w8 + lay.bs, w8 + lay.xs, w8 + lay.cs, a, h_init, yp, h_final,
                  reinterpret_cast<float*>(w8 + lay.scan), stream, nullptr, true);
  if (e != hipSuccess) return hip_status(e, "separated_forward scan launch");
  return hip_status(launch_sep_sum(d.bf16, yp, (int)d.Bt, (int)d.T, (int)d.E, (int)d.HP, y, stream),
                    "separated_forward sum launch");
}

swimba_status swimba_output_project(const swimba_dims* dims, const void* y, const void* w_out,
                                    void* out, hipStream_t stream) {
  Dims d;
  swimba_status st = read_dims(dims, d);
  if (st != SWIMBA_OK) return st;
  if (d.D % 32 != 0) return fail(SWIMBA_ERR_UNSUPPORTED, "d_model must be a multiple of 32");
  if (d.HP % 8 != 0) return fail(SWIMBA_ERR_UNSUPPORTED, "nheads * headdim must be a multiple of 8");
  const int64_t in_bytes = d.bf16 ? 2 : 4;  // y, w_out and out elements
  if (d.M * d.HP * in_bytes >= (int64_t(1) << 31) || d.D * d.HP * in_bytes >= (int64_t(1) << 31) ||
      d.M * d.D >= (int64_t(1) << 31))
    return fail(SWIMBA_ERR_DIMS, "problem too large for 31-bit byte offsets");
  if (d.M == 0) return SWIMBA_OK;
  REQUIRE_PTR(y);
  REQUIRE_PTR(w_out);
  REQUIRE_PTR(out);
  return hip_status(launch_output_project(d.bf16, (int)d.M, (int)d.HP, (int)d.D, y, w_out, out,
                                          stream),
                    "output_project launch");
}

swimba_status swimba_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return SWIMBA_OK;
}

swimba_status swimba_profile_select(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only.clear();
  const std::string list = kernel ? kernel : "";
  size_t pos = 0;
  while (pos < list.size()) {
    size_t end = list.find(',', pos);
    if (end == std::string::npos) end = list.size();
    if (end > pos) g_prof_only.emplace_back(list.substr(pos, end - pos));
    pos = end + 1;
  }
  return SWIMBA_OK;
}

int32_t swimba_profile_report(char* buf, size_t cap) {
  if (!buf || cap == 0) return fail(SWIMBA_ERR_NULL, "report buffer is NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<std::string> names;
  std::vector<double> ms;
  std::vector<int> cnt;
  for (const ProfRec& r : g_prof_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      t = -1.f;
    size_t i = 0;
    while (i < names.size() && names[i] != r.name) ++i;
    if (i == names.size()) {
      names.emplace_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  std::string out = "{";
  for (size_t i = 0; i < names.size(); ++i) {
    char item[256];
    snprintf(item, sizeof(item), "%s\"%s\": {\"launches\": %d, \"ms\": %.6f}", i ? ", " : "",
             names[i].c_str(), cnt[i], ms[i]);
    out += item;
  }
  out += "}";
  if (out.size() + 1 > cap) return fail(SWIMBA_ERR_DIMS, "report buffer too small");
  snprintf(buf, cap, "%s", out.c_str());
  return (int32_t)out.size();
}

}  // extern "C"
