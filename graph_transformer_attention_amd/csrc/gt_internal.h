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
};

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
// (vector-ALU kernels), operand copies of the MFMA kernels (mfma_ops_bytes), then
// per-key-block bucket partial sums [n_kv_blocks * H * NB] float.
struct BwdWorkspace {
  size_t delta_off, ops_off, partial_off, bytes;
  int64_t n_kv_blocks;
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
};

// Kernel timing hook (gt_trace_enable): bracket one launch with events on its stream.
void trace_begin(int kernel_id, hipStream_t s);
void trace_end(int kernel_id, hipStream_t s);

BwdWorkspace bwd_workspace(int64_t N, int64_t Nk, int H, int D, int NB, int dtype);

// Whether every code row base p + i * ld is 16-byte aligned (whole-row vector loads).
inline bool codes_aligned(const uint8_t* p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ld % 16 == 0;
}

hipError_t launch_fwd_valu(const FwdArgs& a, hipStream_t s);
// matrix-core kernels exist for bf16, H = 8, D in {8, 32}
bool mfma_supported(int H, int D, int dtype);
int64_t mfma_npad(int64_t N);
int64_t mfma_kv_blocks(int64_t Nk);
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
// out = merge of two partial attention results over disjoint key sets by their lse
hipError_t launch_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b, float* out,
                        float* lse, int64_t rows, int D, hipStream_t s);
hipError_t launch_bwd_valu(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s);
int64_t valu_kv_block(int H);
hipError_t launch_probe(int kind, int blocks, int iters, float* sink, hipStream_t s);

// Q/K/V projections and storage rounding (proj.hip). dtype 1 = bfloat16 storage.
size_t qkv_bwd_workspace(int64_t N, int hid);
hipError_t launch_qkv_fwd(const void* x, const void* w, void* q, void* k, void* v, int64_t N, int hid, int dtype,
                          hipStream_t s);
hipError_t launch_qkv_bwd(const void* x, const void* w, const float* dq, const float* dk, const float* dv, float* dx,
                          float* dw, void* workspace, int64_t N, int hid, int dtype, hipStream_t s);
hipError_t launch_store(const float* src, void* dst, int64_t n, int dtype, hipStream_t s);

}  // namespace gt
