// Internal interface between the C-ABI layer (gt_attn_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gt {

// N is the number of query nodes, Nk the number of key nodes (N for a whole graph,
// a key block's size for one GA-CP block step); spd[i * ld + j] is the code of query
// i and key j (ld >= Nk), spd_t[j * ld_t + i] the same code (ld_t >= N).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* spd;
  const float* table;
  float* out;
  float* lse;
  int64_t N;
  int H, D, NB, dtype;
  int64_t Nk, ld;
  void* workspace;  // fwd_workspace_bytes(N, Nk, ...) bytes, or null: then the launch is never split
  int acc;          // nonzero: merge the result into out/lse (a running result over other keys)
};

// Split of a kernel's inner loop (keys of the forward and query-outer pass, queries of
// the key-outer pass) over S workgroup rows of `chunk` nodes (a multiple of 32) each,
// used when the outer dimension alone gives too few workgroups to fill the GPU. The
// partial results go to the workspace and a reduction kernel combines them.
struct Split {
  int S;
  int64_t chunk;
};
// kind: which matrix-core kernel (its occupancy sets how many workgroups fit at once).
enum SplitKind { kSplitFwd = 0, kSplitKv = 1, kSplitQ = 2, kSplitFused = 3 };
Split inner_split(int64_t outer, int64_t inner, int H, int D, int dtype, int kind);
// block: room for at least one partial result (a block step may merge into out/lse)
size_t fwd_workspace_bytes(int64_t N, int64_t Nk, int H, int D, int dtype, bool block);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* spd;
  const uint8_t* spd_t;
  const float* table;
  const float* out;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* dtable;
  void* workspace;
  int64_t N;
  int H, D, NB, dtype;
  int64_t Nk, ld, ld_t;
  int acc;  // bits kAcc*: add into dq / dk and dv / dtable instead of overwriting
};

// Accumulate bits of BwdArgs::acc (the header's GT_ACC_* values).
enum { kAccDq = 1, kAccDkv = 2, kAccDtable = 4 };

// Workspace layout of the backward (each region 256-byte aligned): delta [N*H] float
// (vector-ALU kernels), operand copies of the MFMA kernels (mfma_ops_bytes), per-key-
// block bucket partial sums [kv.S * n_kv_blocks * H * NB] float, then when split the
// key-outer pass's dK, dV partials [kv.S][2][Nk*H*D] and the query-outer pass's dQ
// partials [q.S][N*H*D] float.
struct BwdWorkspace {
  size_t delta_off, ops_off, partial_off, dkv_off, dq_off, dqf_off, flag_off, bytes;
  int64_t n_kv_blocks;  // partial rows of one split
  Split kv, q;
  bool fused;  // head dimension 8 on the matrix cores: the one-pass backward's dQ partials at dqf_off
};

// Kernel timing ids (gt_trace_enable); the first five are the header's GT_KERNEL_* ids.
enum {
  kTraceFwd = 0,
  kTraceBwdDelta = 1,
  kTraceBwdKv = 2,
  kTraceBwdQ = 3,
  kTraceBwdDtable = 4,
  kTraceQkvFwd = 5,
  kTraceQkvDx = 6,
  kTraceQkvDw = 7,
  kTraceStore = 8,
  kTraceMerge = 9,
  kTraceFwdSplits = 10,
  kTraceBwdSplits = 11,
  kTraceSpd = 12,
  kTraceLayerFwd = 13,
  kTraceLayerBwd = 14,
  kTraceLayerWgrad = 15,
  kTraceBwdFused = 16,
};

// Kernel timing hook (gt_trace_enable): bracket one launch with events on its stream.
void trace_begin(int kernel_id, hipStream_t s);
void trace_end(int kernel_id, hipStream_t s);

// fused_ok = false: the three-pass layout only (no room for the one-pass backward's dQ
// partials, which take N*H*D floats per 128-key block)
BwdWorkspace bwd_workspace(int64_t N, int64_t Nk, int H, int D, int NB, int dtype, bool fused_ok = true);

// Whether every code row base p + i * ld is 16-byte aligned (whole-row vector loads).
inline bool codes_aligned(const uint8_t* p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ld % 16 == 0;
}

hipError_t launch_fwd_valu(const FwdArgs& a, hipStream_t s);
// matrix-core kernels exist for bf16, H = 8, D in {8, 32}
bool mfma_supported(int H, int D, int dtype);
int64_t mfma_npad(int64_t N);
int64_t mfma_kv_blocks(int64_t Nk);
int64_t mfma_fused_dq_parts(int64_t Nk);
int fused_sets(int64_t Nk);  // 32-key sets per wave of the one-pass D = 8 backward (1 or 2)
size_t mfma_ops_bytes(int64_t N, int64_t Nk);
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_mfma(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s);
// head dimension 32 (attn_mfma_d32.hip)
size_t mfma_d32_ops_bytes(int64_t N, int64_t Nk);
int64_t mfma_d32_kv_blocks(int64_t Nk);
hipError_t launch_fwd_mfma_d32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_mfma_d32(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_dtable_reduce(const float* partial, float* dtable, int64_t nblocks, int HNB, int acc,
                                hipStream_t s);
// out, lse from S partial results over disjoint key ranges: opart [S][rows*D], lpart [S][rows];
// with acc, out/lse on entry are one more partial result
hipError_t launch_merge_splits(const float* opart, const float* lpart, int S, float* out, float* lse, int64_t rows,
                               int D, int acc, hipStream_t s);
// dst[x] = sum_s part[s*n + x] (+ dst[x] when acc), n a multiple of 4
struct SumSplits {
  const float* part;
  float* dst;
  int64_t n;
  int S, acc;
};
// The backward's last step after a split launch: up to three partial sums (S = 0 marks
// an unused one) and the dtable reduction over `nblocks` partial rows, in one launch.
// gate: when given, the launch does nothing unless *gate is nonzero (the rerun of a pass
// that met codes beyond its private bins)
hipError_t launch_bwd_finish(const SumSplits& a, const SumSplits& b, const SumSplits& c, const float* partial,
                             float* dtable, int64_t nblocks, int HNB, int dacc, hipStream_t s,
                             const uint32_t* gate = nullptr);
// out = merge of two partial attention results over disjoint key sets by their lse
hipError_t launch_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b, float* out,
                        float* lse, int64_t rows, int D, hipStream_t s);
hipError_t launch_bwd_valu(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s);
int64_t valu_kv_block(int H);
hipError_t launch_probe(int kind, int blocks, int iters, float* sink, hipStream_t s);

// GPU builder of the distance codes (spd_device.hip). Workspace regions (256-byte
// aligned): the CSR graph and component labels copied from the host, per-level flags,
// then three [N][G] masks (visited, frontier, fresh) for groups of G 64-source batches.
constexpr size_t kSpdMaskBudget = size_t(1) << 30;  // bytes of masks per group
struct SpdDeviceLayout {
  size_t indptr_off, indices_off, comp_off, flags_off, masks_off, bytes;
  int G;
};
SpdDeviceLayout spd_device_layout(int64_t N, int64_t nnz);
hipError_t launch_spd_device(void* workspace, const SpdDeviceLayout& l, int64_t N, int32_t C, uint8_t* spd,
                             hipStream_t s);

// Q/K/V projections and storage rounding (proj.hip). dtype 1 = bfloat16 storage.
size_t qkv_bwd_workspace(int64_t N, int hid);
hipError_t launch_qkv_fwd(const void* x, const void* w, void* q, void* k, void* v, int64_t N, int hid, int dtype,
                          hipStream_t s);
hipError_t launch_qkv_bwd(const void* x, const void* w, const float* dq, const float* dk, const float* dv, float* dx,
                          float* dw, void* workspace, int64_t N, int hid, int dtype, hipStream_t s);
hipError_t launch_store(const float* src, void* dst, int64_t n, int dtype, hipStream_t s);

// Dense parts of the full Graph-Transformer layer (gt_layer.hip); hidden = feed-forward
// = 64. model_params: floats per layer's parameter vector (0 for other sizes).
int model_params(int hid, int ffn);
int64_t model_wgrad_chunks(int64_t N);
struct WgradJob {
  const float* a;  // [N][64] input factor
  const float* d;  // [N][64] gradient factor
  int diag;        // 0: 64 x 64 outer-product sum, 1: 64 column-wise products
  int w_off;       // offset of the result in the layer's parameter gradient
  int c_off;       // offset of the column sums of d, or -1
};
struct WgradJobs {
  WgradJob j[8];
  int n;       // jobs used
  int stride;  // floats per partial row (the parameter count)
};
hipError_t launch_layer_pre_fwd(const float* x, const float* p, void* q, void* k, void* v, float* stats, int64_t N,
                                int dtype, hipStream_t s);
hipError_t launch_layer_post_fwd(const float* x, const float* o, const float* p, float* x1, float* stats, float* hd,
                                 float* x2, int64_t N, hipStream_t s);
hipError_t launch_layer_post_bwd(const float* dx2, const float* x1, const float* stats, const float* hd,
                                 const float* p, float* dx1, void* dout_attn, float* const bufs[5], int64_t N,
                                 int dtype, hipStream_t s);
hipError_t launch_layer_pre_bwd(const float* dq, const float* dk, const float* dv, const float* x, const float* stats,
                                const float* p, const float* dx1, float* dx, float* const bufs[3], int64_t N,
                                hipStream_t s);
hipError_t launch_wgrad_jobs(const WgradJobs& jobs, float* partial, float* grad, int64_t N, hipStream_t s);
// The factors of one layer's parameter gradients, each [N][64] float32: LN1 (ahat, da),
// the Q/K/V projections (a with dq, dk, dv), Wo (o, dx1), LN2 (bhat, db), W1 and c1
// (b, dh), W2 and c2 (g, dx2). grad: the layer's parameter gradient (overwritten);
// partial: model_wgrad_chunks(N) x model_params floats of scratch.
struct LayerGradFactors {
  const float *ahat, *da, *a, *dq, *dk, *dv, *o, *dx1, *bhat, *db, *b, *dh, *g, *dx2;
};
hipError_t launch_layer_wgrad(const LayerGradFactors& f, float* partial, float* grad, int64_t N, hipStream_t s);

// Message for gt_last_error() on the calling thread (entry points outside gt_attn_api.cpp).
void set_last_error(const char* msg);
// gt_attn_bwd with a choice of workspace layout: fused_ok = false takes the three-pass
// backward, whose workspace (bwd_workspace(..., false)) has no room for the one-pass
// backward's dQ partials.
int bwd_call(const void* q, const void* k, const void* v, const uint8_t* spd, const uint8_t* spd_t,
             const float* table, const float* out, const float* lse, const void* dout, float* dq, float* dk, float* dv,
             float* dtable, void* workspace, size_t workspace_bytes, int64_t N, int32_t H, int32_t D, int32_t NB,
             int32_t dtype, void* stream, bool fused_ok);

}  // namespace gt
