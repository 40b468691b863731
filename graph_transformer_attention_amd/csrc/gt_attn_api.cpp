// C ABI of libgt_attn.so: argument validation, workspace sizing, kernel dispatch and
// per-thread error messages. Validation runs on the host before anything is
// enqueued, so every argument error is reported without touching the GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/gt_attn.h"
#include "gt_internal.h"

namespace gt {
std::string spd_validate(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C);
void spd_fill(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C, uint8_t* spd,
              int nthreads);
std::vector<int64_t> components(const int64_t* indptr, const int32_t* indices, int64_t N);
}  // namespace gt

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by all device entry points; returns GT_OK or an error.
int check_shape(int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  if (N < 1 || N > 0x7FFFFFFFll) return fail(GT_EINVAL, "N=%lld must lie in [1, 2^31-1]", (long long)N);
  if (H < 1) return fail(GT_EINVAL, "H=%d must be >= 1", H);
  if (D < 1) return fail(GT_EINVAL, "D=%d must be >= 1", D);
  if (NB < 2 || NB > 255) return fail(GT_EINVAL, "NB=%d must lie in [2, 255]", NB);
  if (dtype != GT_F32 && dtype != GT_BF16) return fail(GT_EINVAL, "dtype=%d is not GT_F32 or GT_BF16", dtype);
  if (D != 8 && D != 16 && D != 32 && D != 64)
    return fail(GT_EUNSUPPORTED, "D=%d: supported head dimensions are 8, 16, 32, 64", D);
  if (H > 64 || H * D > 512) return fail(GT_EUNSUPPORTED, "H=%d, D=%d: needs H <= 64 and H*D <= 512", H, D);
  if (NB > 64 || H * NB > 4096)
    return fail(GT_EUNSUPPORTED, "NB=%d, H=%d: needs NB <= 64 and H*NB <= 4096", NB, H);
  return GT_OK;
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(GT_EINVAL, "%s is null", name);
  if (!aligned16(p)) return fail(GT_EINVAL, "%s is not 16-byte aligned", name);
  return GT_OK;
}

#define GT_CHECK(expr)          \
  do {                          \
    const int rc_ = (expr);     \
    if (rc_ != GT_OK) return rc_; \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GT_OK;
  return fail(GT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Kernel timing records of the calling thread (gt_trace_enable / gt_trace_collect).
struct TraceRec {
  int id;
  hipEvent_t begin, end;
};
thread_local bool g_trace_on = false;
thread_local bool g_trace_failed = false;
thread_local std::vector<hipEvent_t> g_trace_pool;
thread_local std::vector<TraceRec> g_trace_recs;
thread_local hipEvent_t g_trace_open = nullptr;

hipEvent_t trace_event() {
  if (!g_trace_pool.empty()) {
    hipEvent_t e = g_trace_pool.back();
    g_trace_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    g_trace_failed = true;
    return nullptr;
  }
  return e;
}

const char* const kKernelNames[GT_KERNEL_COUNT] = {"fwd",        "bwd_delta",  "bwd_kv",     "bwd_q",
                                                   "bwd_dtable", "qkv_fwd",    "qkv_bwd_dx", "qkv_bwd_dw",
                                                   "store",      "merge",      "fwd_merge",  "bwd_finish",
                                                   "spd_device", "layer_fwd",  "layer_bwd",  "layer_wgrad",
                                                   "bwd_fused"};

int check_dtype(int32_t dtype) {
  if (dtype != GT_F32 && dtype != GT_BF16) return fail(GT_EINVAL, "dtype=%d is not GT_F32 or GT_BF16", dtype);
  return GT_OK;
}

int check_proj(int64_t N, int32_t hid, int32_t dtype) {
  if (N < 1 || N > 0x7FFFFFFFll) return fail(GT_EINVAL, "N=%lld must lie in [1, 2^31-1]", (long long)N);
  if (hid < 8 || hid > 512 || hid % 8 != 0) return fail(GT_EINVAL, "hid=%d must be a multiple of 8 in [8, 512]", hid);
  return check_dtype(dtype);
}

int check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return GT_OK;  // a call that needs no workspace accepts a null one
  if (ws == nullptr) return fail(GT_EINVAL, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(GT_EINVAL, "workspace is not 256-byte aligned");
  if (have < need) return fail(GT_EINVAL, "workspace_bytes=%zu < %zu required", have, need);
  return GT_OK;
}

size_t up256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Shapes of a block step: Nq queries against Nk keys.
int check_block(int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  if (Nq < 1 || Nq > 0x7FFFFFFFll) return fail(GT_EINVAL, "Nq=%lld must lie in [1, 2^31-1]", (long long)Nq);
  if (Nk < 1 || Nk > 0x7FFFFFFFll) return fail(GT_EINVAL, "Nk=%lld must lie in [1, 2^31-1]", (long long)Nk);
  return check_shape(Nq, H, D, NB, dtype);
}

int check_ld(int64_t ld, int64_t n, const char* name, const char* nname) {
  if (ld < n) return fail(GT_EINVAL, "%s=%lld must be >= %s=%lld", name, (long long)ld, nname, (long long)n);
  return GT_OK;
}

// Workspace of gt_stack_fwd_bwd: per layer the saved activations (Q, K, V and the
// next layer's input in storage type, out and lse in float32), then the backward's
// scratch shared by all layers.
struct StackLayout {
  size_t q, k, v, out, lse, xn, layer;    // offsets within one layer's block, block size
  size_t g, dob, dq, dk, dv, attn, proj, fwd;  // offsets of the shared scratch
  size_t bytes;
  gt::BwdWorkspace attn_ws;
};

StackLayout stack_layout(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  StackLayout s{};
  const size_t hid = static_cast<size_t>(H) * D, n = static_cast<size_t>(N);
  const size_t st = dtype == GT_BF16 ? 2 : 4;
  size_t o = 0;
  s.q = o;
  o += up256(n * hid * st);
  s.k = o;
  o += up256(n * hid * st);
  s.v = o;
  o += up256(n * hid * st);
  s.out = o;
  o += up256(n * hid * 4);
  s.lse = o;
  o += up256(n * H * 4);
  s.xn = o;
  o += up256(n * hid * st);
  s.layer = o;
  o = s.layer * static_cast<size_t>(L);
  s.g = o;
  o += up256(n * hid * 4);
  s.dob = o;
  o += up256(n * hid * st);
  s.dq = o;
  o += up256(n * hid * 4);
  s.dk = o;
  o += up256(n * hid * 4);
  s.dv = o;
  o += up256(n * hid * 4);
  s.attn_ws = gt::bwd_workspace(N, N, H, D, NB, dtype);
  s.attn = o;
  o += up256(s.attn_ws.bytes);
  s.proj = o;
  o += up256(gt::qkv_bwd_workspace(N, static_cast<int>(hid)));
  s.fwd = o;
  o += up256(gt::fwd_workspace_bytes(N, N, H, D, dtype, false));
  s.bytes = o;
  return s;
}

// Workspace of gt_model_fwd_bwd: per layer the saved values of the forward (LN
// statistics, Q, K, V in storage type, attention out and lse, X1, Hd and the layer's
// output), then the backward's scratch shared by all layers.
struct ModelLayout {
  size_t st1, q, k, v, o, lse, x1, st2, hd, xout, layer;  // offsets within one layer's block
  size_t dxa, dxb, dx1, dob, dq, dk, dv, fac, attn, fwd, part, bytes;
  gt::BwdWorkspace attn_ws;
};

ModelLayout model_layout(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  ModelLayout m{};
  const size_t n = static_cast<size_t>(N), hid = static_cast<size_t>(H) * D;
  const size_t st = dtype == GT_BF16 ? 2 : 4, row = n * hid * 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  m.st1 = take(n * 8);
  m.q = take(n * hid * st);
  m.k = take(n * hid * st);
  m.v = take(n * hid * st);
  m.o = take(row);
  m.lse = take(n * H * 4);
  m.x1 = take(row);
  m.st2 = take(n * 8);
  m.hd = take(row);
  m.xout = take(row);
  m.layer = o;
  o = m.layer * static_cast<size_t>(L);
  m.dxa = take(row);
  m.dxb = take(row);
  m.dx1 = take(row);
  m.dob = take(n * hid * st);
  m.dq = take(row);
  m.dk = take(row);
  m.dv = take(row);
  m.fac = take(8 * row);  // g, b, dh, bhat, db, a, ahat, da
  m.attn_ws = gt::bwd_workspace(N, N, H, D, NB, dtype);
  m.attn = take(m.attn_ws.bytes);
  m.fwd = take(gt::fwd_workspace_bytes(N, N, H, D, dtype, false));
  m.part = take(static_cast<size_t>(gt::model_wgrad_chunks(N)) * gt::model_params(static_cast<int>(hid),
                                                                                    static_cast<int>(hid)) * 4);
  m.bytes = o;
  return m;
}

int check_model(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  GT_CHECK(check_shape(N, H, D, NB, dtype));
  if (L < 1 || L > 1024) return fail(GT_EINVAL, "L=%d must lie in [1, 1024]", L);
  if (gt::model_params(H * D, H * D) == 0)
    return fail(GT_EUNSUPPORTED, "H*D=%d: the full layer is built for hidden = feed-forward = 64", H * D);
  return GT_OK;
}

hipError_t attn_fwd(const gt::FwdArgs& a, hipStream_t s) {
  if (!gt::mfma_supported(a.H, a.D, a.dtype)) return gt::launch_fwd_valu(a, s);
  return a.D == 32 ? gt::launch_fwd_mfma_d32(a, s) : gt::launch_fwd_mfma(a, s);
}

hipError_t attn_bwd(const gt::BwdArgs& a, const gt::BwdWorkspace& w, hipStream_t s) {
  if (!gt::mfma_supported(a.H, a.D, a.dtype)) return gt::launch_bwd_valu(a, w, s);
  return a.D == 32 ? gt::launch_bwd_mfma_d32(a, w, s) : gt::launch_bwd_mfma(a, w, s);
}

}  // namespace

namespace gt {

void trace_begin(int kernel_id, hipStream_t s) {
  (void)kernel_id;
  if (!g_trace_on) return;
  g_trace_open = trace_event();
  if (g_trace_open != nullptr && hipEventRecord(g_trace_open, s) != hipSuccess) g_trace_failed = true;
}

void trace_end(int kernel_id, hipStream_t s) {
  if (!g_trace_on || g_trace_open == nullptr) return;
  hipEvent_t e = trace_event();
  if (e == nullptr) return;
  if (hipEventRecord(e, s) != hipSuccess) g_trace_failed = true;
  g_trace_recs.push_back({kernel_id, g_trace_open, e});
  g_trace_open = nullptr;
}

// A matrix-core launch may be split along its inner loop into S grid rows (each keeping at
// least 256 inner nodes). S minimises a time model of the launch in units of one 32-node
// tile: ceil(W*S / R) rounds of workgroups, each costing a fixed overhead plus its
// inner tiles, with W workgroups per row (128 outer nodes x one head pair) and R
// workgroups resident at once (the kernel's occupancy). The one-pass D = 8 backward's
// workgroups are 8 waves of one or two 32-key sets (256 or 512 keys, fused_sets), one
// per CU: W counts those, each costing 2 or 4 of the others' workgroups (fixed part and
// tiles alike). Measured per-workgroup costs
// are a fixed ~10-20 us plus ~1.7-1.8 us per tile, so the fixed part is about 12 tiles.
// This both fills the GPU when the outer dimension is short and evens out the last
// round when W is not a multiple of R.
// The forward's CUs do not finish a round together: launched as exactly one round at
// 32768 nodes, it kept 11 of 16 waves resident on average, the rest idle at the tail;
// smaller workgroups in more rounds let the faster CUs take more of them (4 key splits:
// 1.72 -> 1.59 ms). The model charges the forward's last round a tail of 2/10 of a
// workgroup's tiles (the backward kernels kept 7.4 of 8 waves resident: no tail term).
constexpr int64_t kSplitMinInner = 256;
constexpr int64_t kSplitFixedTiles = 12;
constexpr int64_t kFwdTailTenths = 2;

// 4-wave workgroups resident per CU, from each kernel's VGPR use (512 per SIMD lane):
// D = 8: forward 128 -> 4, key-outer 192-212 -> 2, query-outer 142 -> 3; D = 32: forward 156
// -> 3, key-outer 238-243 and query-outer 226 -> 2.
int64_t resident_wgs(int kind, int D) {
  if (kind == kSplitFused) return 256;
  const int per_cu = D == 32 ? (kind == kSplitFwd ? 3 : 2) : (kind == kSplitFwd ? 4 : kind == kSplitKv ? 2 : 3);
  return 256 * per_cu;
}

Split inner_split(int64_t outer, int64_t inner, int H, int D, int dtype, int kind) {
  Split sp{1, inner};
  if (!mfma_supported(H, D, dtype)) return sp;
  const int64_t R = resident_wgs(kind, D);
  const int64_t sets = kind == kSplitFused ? fused_sets(outer) : 0;
  const int64_t wg_nodes = sets ? 256 * sets : 128, cost = sets ? 2 * sets : 1;
  const int64_t W = (outer + wg_nodes - 1) / wg_nodes * (H / 2);
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(64, inner / kSplitMinInner));
  int64_t best_t = -1;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t chunk = S == 1 ? inner : ((inner + S - 1) / S + 31) / 32 * 32;
    const int64_t parts = (inner + chunk - 1) / chunk;
    const int64_t rounds = (W * parts + R - 1) / R;
    const int64_t tiles = (chunk + 31) / 32;
    const int64_t t = 10 * rounds * cost * (kSplitFixedTiles + tiles) + (kind == kSplitFwd ? kFwdTailTenths * tiles : 0);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      sp.S = static_cast<int>(parts);
      sp.chunk = chunk;
    }
  }
  return sp;
}

size_t fwd_workspace_bytes(int64_t N, int64_t Nk, int H, int D, int dtype, bool block) {
  const Split sp = inner_split(N, Nk, H, D, dtype, kSplitFwd);
  if (sp.S == 1 && !block) return 0;
  const size_t rows = static_cast<size_t>(N) * H;
  return up256(static_cast<size_t>(sp.S) * rows * D * sizeof(float)) + up256(static_cast<size_t>(sp.S) * rows * sizeof(float));
}

BwdWorkspace bwd_workspace(int64_t N, int64_t Nk, int H, int D, int NB, int dtype, bool fused_ok) {
  BwdWorkspace w{};
  const bool mfma = mfma_supported(H, D, dtype);
  w.fused = fused_ok && mfma && D == 8;
  const int64_t kb = valu_kv_block(H);
  w.n_kv_blocks = mfma ? (D == 32 ? mfma_d32_kv_blocks(Nk) : mfma_kv_blocks(Nk)) : (Nk + kb - 1) / kb;
  w.kv = inner_split(Nk, N, H, D, dtype, w.fused ? kSplitFused : kSplitKv);
  w.q = inner_split(N, Nk, H, D, dtype, kSplitQ);
  const size_t f = sizeof(float);
  w.delta_off = 0;
  w.ops_off = up256(static_cast<size_t>(N) * H * f);
  w.partial_off = w.ops_off + (mfma ? up256(D == 32 ? mfma_d32_ops_bytes(N, Nk) : mfma_ops_bytes(N, Nk)) : 0);
  w.dkv_off = w.partial_off + up256(static_cast<size_t>(w.kv.S) * w.n_kv_blocks * H * NB * f);
  const size_t dkv = w.kv.S > 1 ? up256(2 * static_cast<size_t>(w.kv.S) * Nk * H * D * f) : 0;
  w.dq_off = w.dkv_off + dkv;
  const size_t dq = w.q.S > 1 ? up256(static_cast<size_t>(w.q.S) * N * H * D * f) : 0;
  w.dqf_off = w.dq_off + dq;
  // the one-pass backward's dQ partials: one [N][H][D] array per workgroup (256 or 512 keys)
  const size_t dqf = w.fused ? up256(static_cast<size_t>(mfma_fused_dq_parts(Nk)) * N * H * D * f) : 0;
  w.flag_off = w.dqf_off + dqf;  // one device word the kernels of a call share (code-range flag)
  w.bytes = w.flag_off + 256;
  return w;
}

}  // namespace gt

namespace gt {
void set_last_error(const char* msg) { g_error = msg; }
}  // namespace gt

extern "C" {

const char* gt_last_error(void) { return g_error.c_str(); }

const char* gt_version(void) { return "gt_attn 0.1 (gfx950)"; }

int gt_trace_enable(int32_t on) {
  g_trace_on = on != 0;
  return GT_OK;
}

int gt_trace_collect(int32_t* counts, double* total_ms, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    if (counts) counts[i] = 0;
    if (total_ms) total_ms[i] = 0.0;
  }
  int rc = GT_OK;
  for (const TraceRec& r : g_trace_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess)
      rc = fail(GT_EHIP, "gt_trace_collect: could not read a kernel timing event");
    if (r.id >= 0 && r.id < n) {
      if (counts) counts[r.id] += 1;
      if (total_ms) total_ms[r.id] += ms;
    }
    g_trace_pool.push_back(r.begin);
    g_trace_pool.push_back(r.end);
  }
  g_trace_recs.clear();
  if (g_trace_failed) {
    g_trace_failed = false;
    rc = fail(GT_EHIP, "gt_trace: an event could not be created or recorded");
  }
  return rc;
}

int gt_probe_peak(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (kind < 0 || kind > 4) return fail(GT_EINVAL, "probe kind=%d must lie in [0, 4]", kind);
  if (blocks < 1 || blocks > (1 << 20)) return fail(GT_EINVAL, "probe blocks=%d out of range", blocks);
  if (iters < 1) return fail(GT_EINVAL, "probe iters=%d must be >= 1", iters);
  if (sink == nullptr) return fail(GT_EINVAL, "probe sink is null");
  return hip_status(gt::launch_probe(kind, blocks, iters, sink, static_cast<hipStream_t>(stream)),
                    "gt_probe_peak launch");
}

const char* gt_kernel_name(int32_t id) {
  return (id >= 0 && id < GT_KERNEL_COUNT) ? kKernelNames[id] : "";
}

size_t gt_attn_fwd_workspace_bytes(int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_shape(N, H, D, NB, dtype);
  g_error = saved;
  return rc != GT_OK ? 0 : gt::fwd_workspace_bytes(N, N, H, D, dtype, false);
}

int gt_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* spd, const float* table,
                float* out, float* lse, int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype,
                void* stream) {
  GT_CHECK(check_shape(N, H, D, NB, dtype));
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  GT_CHECK(check_ptr(spd, "spd"));
  GT_CHECK(check_ptr(table, "table"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  gt::FwdArgs a{q, k, v, spd, table, out, lse, N, H, D, NB, dtype, N, N, nullptr, 0};
  return hip_status(attn_fwd(a, static_cast<hipStream_t>(stream)), "gt_attn_fwd launch");
}

int gt_attn_fwd_ws(const void* q, const void* k, const void* v, const uint8_t* spd, const float* table,
                   float* out, float* lse, void* workspace, size_t workspace_bytes, int64_t N, int32_t H,
                   int32_t D, int32_t NB, int32_t dtype, void* stream) {
  GT_CHECK(check_shape(N, H, D, NB, dtype));
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  GT_CHECK(check_ptr(spd, "spd"));
  GT_CHECK(check_ptr(table, "table"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  const size_t need = gt::fwd_workspace_bytes(N, N, H, D, dtype, false);
  GT_CHECK(check_workspace(workspace, workspace_bytes, need));
  gt::FwdArgs a{q, k, v, spd, table, out, lse, N, H, D, NB, dtype, N, N, need > 0 ? workspace : nullptr, 0};
  return hip_status(attn_fwd(a, static_cast<hipStream_t>(stream)), "gt_attn_fwd_ws launch");
}

size_t gt_attn_bwd_workspace_bytes(int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_shape(N, H, D, NB, dtype);
  g_error = saved;
  if (rc != GT_OK) return 0;
  return gt::bwd_workspace(N, N, H, D, NB, dtype).bytes;
}

int gt_attn_bwd(const void* q, const void* k, const void* v, const uint8_t* spd, const uint8_t* spd_t,
                const float* table,
                const float* out, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                float* dtable, void* workspace, size_t workspace_bytes, int64_t N, int32_t H,
                int32_t D, int32_t NB, int32_t dtype, void* stream) {
  return gt::bwd_call(q, k, v, spd, spd_t, table, out, lse, dout, dq, dk, dv, dtable, workspace, workspace_bytes, N, H,
                      D, NB, dtype, stream, true);
}

}  // extern "C"

int gt::bwd_call(const void* q, const void* k, const void* v, const uint8_t* spd, const uint8_t* spd_t,
                 const float* table, const float* out, const float* lse, const void* dout, float* dq, float* dk,
                 float* dv, float* dtable, void* workspace, size_t workspace_bytes, int64_t N, int32_t H, int32_t D,
                 int32_t NB, int32_t dtype, void* stream, bool fused_ok) {
  GT_CHECK(check_shape(N, H, D, NB, dtype));
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  GT_CHECK(check_ptr(spd, "spd"));
  GT_CHECK(check_ptr(spd_t, "spd_t"));
  GT_CHECK(check_ptr(table, "table"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  GT_CHECK(check_ptr(dout, "dout"));
  GT_CHECK(check_ptr(dq, "dq"));
  GT_CHECK(check_ptr(dk, "dk"));
  GT_CHECK(check_ptr(dv, "dv"));
  GT_CHECK(check_ptr(dtable, "dtable"));
  const gt::BwdWorkspace w = gt::bwd_workspace(N, N, H, D, NB, dtype, fused_ok);
  GT_CHECK(check_workspace(workspace, workspace_bytes, w.bytes));
  gt::BwdArgs a{q, k, v, spd, spd_t, table, out, lse, dout, dq, dk, dv, dtable, workspace, N, H, D, NB, dtype,
                N, N, N, 0};
  return hip_status(attn_bwd(a, w, static_cast<hipStream_t>(stream)), "gt_attn_bwd launch");
}

extern "C" {

size_t gt_attn_fwd_block_workspace_bytes(int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_block(Nq, Nk, H, D, NB, dtype);
  g_error = saved;
  return rc != GT_OK ? 0 : gt::fwd_workspace_bytes(Nq, Nk, H, D, dtype, true);
}

int gt_attn_fwd_block(const void* q, const void* k, const void* v, const uint8_t* spd, int64_t ld,
                      const float* table, float* out, float* lse, void* workspace, size_t workspace_bytes,
                      int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB, int32_t dtype, int32_t accumulate,
                      void* stream) {
  GT_CHECK(check_block(Nq, Nk, H, D, NB, dtype));
  GT_CHECK(check_ld(ld, Nk, "ld", "Nk"));
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  if (spd == nullptr) return fail(GT_EINVAL, "spd is null");
  GT_CHECK(check_ptr(table, "table"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  if (accumulate != 0 && accumulate != 1) return fail(GT_EINVAL, "accumulate=%d must be 0 or 1", accumulate);
  GT_CHECK(check_workspace(workspace, workspace_bytes, gt::fwd_workspace_bytes(Nq, Nk, H, D, dtype, true)));
  gt::FwdArgs a{q, k, v, spd, table, out, lse, Nq, H, D, NB, dtype, Nk, ld, workspace, accumulate};
  return hip_status(attn_fwd(a, static_cast<hipStream_t>(stream)), "gt_attn_fwd_block launch");
}

int gt_attn_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b, float* out,
                  float* lse, int64_t Nq, int32_t H, int32_t D, void* stream) {
  if (Nq < 1 || Nq > 0x7FFFFFFFll) return fail(GT_EINVAL, "Nq=%lld must lie in [1, 2^31-1]", (long long)Nq);
  if (H < 1 || H > 64) return fail(GT_EINVAL, "H=%d must lie in [1, 64]", H);
  if (D != 8 && D != 16 && D != 32 && D != 64)
    return fail(GT_EUNSUPPORTED, "D=%d: supported head dimensions are 8, 16, 32, 64", D);
  GT_CHECK(check_ptr(out_a, "out_a"));
  GT_CHECK(check_ptr(lse_a, "lse_a"));
  GT_CHECK(check_ptr(out_b, "out_b"));
  GT_CHECK(check_ptr(lse_b, "lse_b"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  return hip_status(gt::launch_merge(out_a, lse_a, out_b, lse_b, out, lse, Nq * H, D, static_cast<hipStream_t>(stream)),
                    "gt_attn_merge launch");
}

size_t gt_attn_bwd_block_workspace_bytes(int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_block(Nq, Nk, H, D, NB, dtype);
  g_error = saved;
  if (rc != GT_OK) return 0;
  return gt::bwd_workspace(Nq, Nk, H, D, NB, dtype).bytes;
}

int gt_attn_bwd_block(const void* q, const void* k, const void* v, const uint8_t* spd, int64_t ld,
                      const uint8_t* spd_t, int64_t ld_t, const float* table, const float* out, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, float* dtable, void* workspace,
                      size_t workspace_bytes, int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB,
                      int32_t dtype, int32_t accumulate, void* stream) {
  GT_CHECK(check_block(Nq, Nk, H, D, NB, dtype));
  GT_CHECK(check_ld(ld, Nk, "ld", "Nk"));
  GT_CHECK(check_ld(ld_t, Nq, "ld_t", "Nq"));
  if (accumulate < 0 || accumulate > GT_ACC_ALL)
    return fail(GT_EINVAL, "accumulate=%d must be a combination of the GT_ACC_* bits", accumulate);
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  if (spd == nullptr) return fail(GT_EINVAL, "spd is null");
  if (spd_t == nullptr) return fail(GT_EINVAL, "spd_t is null");
  GT_CHECK(check_ptr(table, "table"));
  GT_CHECK(check_ptr(out, "out"));
  GT_CHECK(check_ptr(lse, "lse"));
  GT_CHECK(check_ptr(dout, "dout"));
  GT_CHECK(check_ptr(dq, "dq"));
  GT_CHECK(check_ptr(dk, "dk"));
  GT_CHECK(check_ptr(dv, "dv"));
  GT_CHECK(check_ptr(dtable, "dtable"));
  const gt::BwdWorkspace w = gt::bwd_workspace(Nq, Nk, H, D, NB, dtype);
  GT_CHECK(check_workspace(workspace, workspace_bytes, w.bytes));
  gt::BwdArgs a{q, k, v, spd, spd_t, table, out, lse, dout, dq, dk, dv, dtable, workspace, Nq, H, D, NB, dtype,
                Nk, ld, ld_t, accumulate};
  return hip_status(attn_bwd(a, w, static_cast<hipStream_t>(stream)), "gt_attn_bwd_block launch");
}

int gt_spd_build(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C, uint8_t* spd,
                 int32_t nthreads) {
  if (indptr == nullptr) return fail(GT_EINVAL, "indptr is null");
  if (spd == nullptr) return fail(GT_EINVAL, "spd is null");
  const std::string why = gt::spd_validate(indptr, indices, N, C);
  if (!why.empty()) return fail(GT_EINVAL, "gt_spd_build: %s", why.c_str());
  gt::spd_fill(indptr, indices, N, C, spd, nthreads);
  return GT_OK;
}

size_t gt_spd_build_device_workspace_bytes(int64_t N, int64_t nnz, int32_t C) {
  if (N < 1 || N > 0x7FFFFFFFll || nnz < 0 || C < 1 || C > 254) return 0;
  return gt::spd_device_layout(N, nnz).bytes;
}

int gt_spd_build_device(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C, uint8_t* spd,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (indptr == nullptr) return fail(GT_EINVAL, "indptr is null");
  if (spd == nullptr) return fail(GT_EINVAL, "spd is null");
  if (N < 1 || N > 0x7FFFFFFFll) return fail(GT_EINVAL, "N=%lld must lie in [1, 2^31-1]", (long long)N);
  const std::string why = gt::spd_validate(indptr, indices, N, C);
  if (!why.empty()) return fail(GT_EINVAL, "gt_spd_build_device: %s", why.c_str());
  const int64_t nnz = indptr[N];
  const gt::SpdDeviceLayout lay = gt::spd_device_layout(N, nnz);
  GT_CHECK(check_workspace(workspace, workspace_bytes, lay.bytes));
  const std::vector<int64_t> comp64 = gt::components(indptr, indices, N);
  const std::vector<int32_t> comp(comp64.begin(), comp64.end());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  // the graph goes to the workspace first; the host arrays (and the labels above) are
  // no longer needed once the copies are complete
  GT_CHECK(hip_status(hipMemcpyAsync(base + lay.indptr_off, indptr, static_cast<size_t>(N + 1) * 8,
                                     hipMemcpyHostToDevice, s), "gt_spd_build_device copy"));
  if (nnz > 0)
    GT_CHECK(hip_status(hipMemcpyAsync(base + lay.indices_off, indices, static_cast<size_t>(nnz) * 4,
                                       hipMemcpyHostToDevice, s), "gt_spd_build_device copy"));
  GT_CHECK(hip_status(hipMemcpyAsync(base + lay.comp_off, comp.data(), static_cast<size_t>(N) * 4,
                                     hipMemcpyHostToDevice, s), "gt_spd_build_device copy"));
  GT_CHECK(hip_status(hipStreamSynchronize(s), "gt_spd_build_device copy"));
  return hip_status(gt::launch_spd_device(workspace, lay, N, C, spd, s), "gt_spd_build_device launch");
}

int gt_qkv_fwd(const void* x, const void* w, void* q, void* k, void* v, int64_t N, int32_t hid, int32_t dtype,
               void* stream) {
  GT_CHECK(check_proj(N, hid, dtype));
  GT_CHECK(check_ptr(x, "x"));
  GT_CHECK(check_ptr(w, "w"));
  GT_CHECK(check_ptr(q, "q"));
  GT_CHECK(check_ptr(k, "k"));
  GT_CHECK(check_ptr(v, "v"));
  return hip_status(gt::launch_qkv_fwd(x, w, q, k, v, N, hid, dtype, static_cast<hipStream_t>(stream)),
                    "gt_qkv_fwd launch");
}

size_t gt_qkv_bwd_workspace_bytes(int64_t N, int32_t hid) {
  const std::string saved = g_error;
  const int rc = check_proj(N, hid, GT_F32);
  g_error = saved;
  return rc != GT_OK ? 0 : up256(gt::qkv_bwd_workspace(N, hid));
}

int gt_qkv_bwd(const void* x, const void* w, const float* dq, const float* dk, const float* dv, float* dx, float* dw,
               void* workspace, size_t workspace_bytes, int64_t N, int32_t hid, int32_t dtype, void* stream) {
  GT_CHECK(check_proj(N, hid, dtype));
  GT_CHECK(check_ptr(x, "x"));
  GT_CHECK(check_ptr(w, "w"));
  GT_CHECK(check_ptr(dq, "dq"));
  GT_CHECK(check_ptr(dk, "dk"));
  GT_CHECK(check_ptr(dv, "dv"));
  GT_CHECK(check_ptr(dx, "dx"));
  GT_CHECK(check_ptr(dw, "dw"));
  GT_CHECK(check_workspace(workspace, workspace_bytes, gt::qkv_bwd_workspace(N, hid)));
  return hip_status(
      gt::launch_qkv_bwd(x, w, dq, dk, dv, dx, dw, workspace, N, hid, dtype, static_cast<hipStream_t>(stream)),
      "gt_qkv_bwd launch");
}

int gt_store(const float* src, void* dst, int64_t n, int32_t dtype, void* stream) {
  GT_CHECK(check_dtype(dtype));
  if (n < 0) return fail(GT_EINVAL, "n=%lld must be >= 0", (long long)n);
  if (n == 0) return GT_OK;
  GT_CHECK(check_ptr(src, "src"));
  GT_CHECK(check_ptr(dst, "dst"));
  return hip_status(gt::launch_store(src, dst, n, dtype, static_cast<hipStream_t>(stream)), "gt_store launch");
}

int32_t gt_model_param_count(int32_t hid, int32_t ffn) { return gt::model_params(hid, ffn); }

size_t gt_model_workspace_bytes(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_model(N, L, H, D, NB, dtype);
  g_error = saved;
  return rc != GT_OK ? 0 : model_layout(N, L, H, D, NB, dtype).bytes;
}

int gt_model_fwd_bwd(const float* x0, const float* params, const float* tables, const uint8_t* spd,
                     const uint8_t* spd_t, const float* dout, float* x_last, float* dx0, float* dparams,
                     float* dtables, void* workspace, size_t workspace_bytes, int64_t N, int32_t L, int32_t H,
                     int32_t D, int32_t NB, int32_t dtype, void* stream) {
  GT_CHECK(check_model(N, L, H, D, NB, dtype));
  GT_CHECK(check_ptr(x0, "x0"));
  GT_CHECK(check_ptr(params, "params"));
  GT_CHECK(check_ptr(tables, "tables"));
  GT_CHECK(check_ptr(spd, "spd"));
  GT_CHECK(check_ptr(spd_t, "spd_t"));
  GT_CHECK(check_ptr(dout, "dout"));
  GT_CHECK(check_ptr(x_last, "x_last"));
  GT_CHECK(check_ptr(dx0, "dx0"));
  GT_CHECK(check_ptr(dparams, "dparams"));
  GT_CHECK(check_ptr(dtables, "dtables"));
  const ModelLayout m = model_layout(N, L, H, D, NB, dtype);
  GT_CHECK(check_workspace(workspace, workspace_bytes, m.bytes));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int P = gt::model_params(H * D, H * D);
  char* base = static_cast<char*>(workspace);
  auto at = [&](int l, size_t off) { return base + static_cast<size_t>(l) * m.layer + off; };
  auto f32 = [](char* p) { return reinterpret_cast<float*>(p); };
  const size_t row = static_cast<size_t>(N) * H * D;
  // forward: X_{l+1} = layer_l(X_l); the last layer writes x_last
  const float* X = x0;
  for (int l = 0; l < L; ++l) {
    const float* p = params + static_cast<size_t>(l) * P;
    float* Xn = l == L - 1 ? x_last : f32(at(l, m.xout));
    GT_CHECK(hip_status(gt::launch_layer_pre_fwd(X, p, at(l, m.q), at(l, m.k), at(l, m.v), f32(at(l, m.st1)), N,
                                                 dtype, s),
                        "gt_model_fwd_bwd layer forward"));
    const gt::FwdArgs fa{at(l, m.q), at(l, m.k), at(l, m.v), spd, tables + static_cast<size_t>(l) * H * NB,
                         f32(at(l, m.o)), f32(at(l, m.lse)), N, H, D, NB, dtype, N, N, base + m.fwd, 0};
    GT_CHECK(hip_status(attn_fwd(fa, s), "gt_model_fwd_bwd attention forward"));
    GT_CHECK(hip_status(gt::launch_layer_post_fwd(X, f32(at(l, m.o)), p, f32(at(l, m.x1)), f32(at(l, m.st2)),
                                                  f32(at(l, m.hd)), Xn, N, s),
                        "gt_model_fwd_bwd layer forward"));
    X = Xn;
  }
  // backward of sum(dout * X_L)
  float* fac = f32(base + m.fac);
  float* const post_bufs[5] = {fac, fac + row, fac + 2 * row, fac + 3 * row, fac + 4 * row};  // g, b, dh, bhat, db
  float* const pre_bufs[3] = {fac + 5 * row, fac + 6 * row, fac + 7 * row};                   // a, ahat, da
  float* dxbuf[2] = {f32(base + m.dxa), f32(base + m.dxb)};
  float* dx1 = f32(base + m.dx1);
  float *dq = f32(base + m.dq), *dk = f32(base + m.dk), *dv = f32(base + m.dv);
  const float* G = dout;
  for (int l = L - 1; l >= 0; --l) {
    const float* p = params + static_cast<size_t>(l) * P;
    const float* Xl = l == 0 ? x0 : f32(at(l - 1, m.xout));
    float* dXl = l == 0 ? dx0 : dxbuf[l & 1];
    GT_CHECK(hip_status(gt::launch_layer_post_bwd(G, f32(at(l, m.x1)), f32(at(l, m.st2)), f32(at(l, m.hd)), p, dx1,
                                                  base + m.dob, post_bufs, N, dtype, s),
                        "gt_model_fwd_bwd layer backward"));
    const gt::BwdArgs ba{at(l, m.q), at(l, m.k), at(l, m.v), spd, spd_t, tables + static_cast<size_t>(l) * H * NB,
                         f32(at(l, m.o)), f32(at(l, m.lse)), base + m.dob, dq, dk, dv,
                         dtables + static_cast<size_t>(l) * H * NB, base + m.attn, N, H, D, NB, dtype, N, N, N, 0};
    GT_CHECK(hip_status(attn_bwd(ba, m.attn_ws, s), "gt_model_fwd_bwd attention backward"));
    GT_CHECK(hip_status(gt::launch_layer_pre_bwd(dq, dk, dv, Xl, f32(at(l, m.st1)), p, dx1, dXl, pre_bufs, N, s),
                        "gt_model_fwd_bwd layer backward"));
    const gt::LayerGradFactors fg{pre_bufs[1], pre_bufs[2], pre_bufs[0], dq, dk, dv, f32(at(l, m.o)), dx1,
                                  post_bufs[3], post_bufs[4], post_bufs[1], post_bufs[2], post_bufs[0], G};
    GT_CHECK(hip_status(gt::launch_layer_wgrad(fg, f32(base + m.part), dparams + static_cast<size_t>(l) * P, N, s),
                        "gt_model_fwd_bwd weight gradients"));
    G = dXl;
  }
  return GT_OK;
}

size_t gt_stack_workspace_bytes(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype) {
  const std::string saved = g_error;
  const int rc = check_shape(N, H, D, NB, dtype);
  g_error = saved;
  if (rc != GT_OK || L < 1 || L > 1024) return 0;
  return stack_layout(N, L, H, D, NB, dtype).bytes;
}

int gt_stack_fwd_bwd(const void* x0, const void* w, const float* tables, const uint8_t* spd, const uint8_t* spd_t,
                     const void* dout, void* x_last, float* dx0, float* dw, float* dtable, void* workspace,
                     size_t workspace_bytes, int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype,
                     void* stream) {
  GT_CHECK(check_shape(N, H, D, NB, dtype));
  if (L < 1 || L > 1024) return fail(GT_EINVAL, "L=%d must lie in [1, 1024]", L);
  GT_CHECK(check_ptr(x0, "x0"));
  GT_CHECK(check_ptr(w, "w"));
  GT_CHECK(check_ptr(tables, "tables"));
  GT_CHECK(check_ptr(spd, "spd"));
  GT_CHECK(check_ptr(spd_t, "spd_t"));
  GT_CHECK(check_ptr(dout, "dout"));
  GT_CHECK(check_ptr(x_last, "x_last"));
  GT_CHECK(check_ptr(dx0, "dx0"));
  GT_CHECK(check_ptr(dw, "dw"));
  GT_CHECK(check_ptr(dtable, "dtable"));
  const StackLayout lay = stack_layout(N, L, H, D, NB, dtype);
  GT_CHECK(check_workspace(workspace, workspace_bytes, lay.bytes));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int hid = H * D;
  const size_t st = dtype == GT_BF16 ? 2 : 4;
  const size_t wsz = static_cast<size_t>(3) * hid * hid;
  char* base = static_cast<char*>(workspace);
  auto layer = [&](int l, size_t off) { return base + static_cast<size_t>(l) * lay.layer + off; };
  float* G = reinterpret_cast<float*>(base + lay.g);
  void* dO = base + lay.dob;
  float* dq = reinterpret_cast<float*>(base + lay.dq);
  float* dk = reinterpret_cast<float*>(base + lay.dk);
  float* dv = reinterpret_cast<float*>(base + lay.dv);
  const int64_t nel = N * hid;
  // forward: X_{l+1} = store(attention_l(X_l W_l)); the last layer writes x_last
  const void* X = x0;
  for (int l = 0; l < L; ++l) {
    const void* wl = static_cast<const char*>(w) + l * wsz * st;
    void *q = layer(l, lay.q), *k = layer(l, lay.k), *v = layer(l, lay.v);
    float* out = reinterpret_cast<float*>(layer(l, lay.out));
    float* lse = reinterpret_cast<float*>(layer(l, lay.lse));
    void* xn = l == L - 1 ? x_last : layer(l, lay.xn);
    GT_CHECK(hip_status(gt::launch_qkv_fwd(X, wl, q, k, v, N, hid, dtype, s), "gt_stack_fwd_bwd qkv"));
    const gt::FwdArgs fa{q, k, v, spd, tables + static_cast<size_t>(l) * H * NB, out, lse, N, H, D, NB, dtype, N, N,
                         base + lay.fwd, 0};
    GT_CHECK(hip_status(attn_fwd(fa, s), "gt_stack_fwd_bwd attention forward"));
    GT_CHECK(hip_status(gt::launch_store(out, xn, nel, dtype, s), "gt_stack_fwd_bwd store"));
    X = xn;
  }
  // backward of sum(dout * X_L): layer l gets store(dX_{l+1}) as its attention dout
  for (int l = L - 1; l >= 0; --l) {
    const void* wl = static_cast<const char*>(w) + l * wsz * st;
    const void* dol = dout;
    if (l < L - 1) {
      GT_CHECK(hip_status(gt::launch_store(G, dO, nel, dtype, s), "gt_stack_fwd_bwd store"));
      dol = dO;
    }
    const gt::BwdArgs ba{layer(l, lay.q), layer(l, lay.k), layer(l, lay.v), spd, spd_t,
                         tables + static_cast<size_t>(l) * H * NB, reinterpret_cast<float*>(layer(l, lay.out)),
                         reinterpret_cast<float*>(layer(l, lay.lse)), dol, dq, dk, dv,
                         dtable + static_cast<size_t>(l) * H * NB, base + lay.attn, N, H, D, NB, dtype,
                         N, N, N, 0};
    GT_CHECK(hip_status(attn_bwd(ba, lay.attn_ws, s), "gt_stack_fwd_bwd attention backward"));
    const void* Xl = l == 0 ? x0 : layer(l - 1, lay.xn);
    float* dxl = l == 0 ? dx0 : G;
    GT_CHECK(hip_status(gt::launch_qkv_bwd(Xl, wl, dq, dk, dv, dxl, dw + static_cast<size_t>(l) * wsz,
                                           base + lay.proj, N, hid, dtype, s),
                        "gt_stack_fwd_bwd qkv backward"));
  }
  return GT_OK;
}

}  // extern "C"
