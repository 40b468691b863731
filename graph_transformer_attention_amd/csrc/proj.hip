// Q/K/V projections of a stacked Graph Transformer (MegaGraph pages, Fig. 8 caption:
// 16 layers, 8 heads, hidden size 64) and the float32 -> storage-type rounding used
// at the stack's storage points.
//
//   forward     T = store(X W_t)            t in {q, k, v}; X [N, hid], W_t [hid, hid]
//   backward    dX = sum_t dT W_t^T         dW_t = X^T dT   (float32)
//
// At hidden 64 a projection is 2*N*hid*3*hid flops against H*N^2 attention entries
// per layer (under 1% of the layer at N = 6800), so these are plain LDS-tiled GEMMs
// on the vector ALU: 256 threads compute a 64 x 64 output tile, 4 x 4 per thread,
// over 16-deep slices of the contraction staged in LDS as float32.
#include "gt_internal.h"

namespace gt {
namespace {

constexpr int kTile = 64;
constexpr int kSlice = 16;
constexpr int kChunk = 256;  // nodes per dW partial sum

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ void put(float* p, float x) { *p = x; }
__device__ __forceinline__ void put(uint16_t* p, float x) { *p = bf16_rne(x); }

// acc[i][j] += sum_kk A[kk][4ty+i] * B[kk][4tx+j] over one staged slice.
__device__ __forceinline__ void slice_fma(float (&acc)[4][4], const float (*A)[kTile + 1], const float (*B)[kTile],
                                          int tx, int ty) {
#pragma unroll
  for (int kk = 0; kk < kSlice; ++kk) {
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = A[kk][4 * ty + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = B[kk][4 * tx + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
  }
}

// T_t[n, c] = sum_k X[n, k] W_t[k, c]; grid (row tiles, column tiles, 3).
template <typename T>
__global__ __launch_bounds__(256) void qkv_fwd_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                      T* __restrict__ q, T* __restrict__ k, T* __restrict__ v,
                                                      int64_t N, int hid) {
  __shared__ float As[kSlice][kTile + 1];  // [k][row]
  __shared__ float Bs[kSlice][kTile];      // [k][column]
  const int t = blockIdx.z;
  const T* W = w + static_cast<int64_t>(t) * hid * hid;
  T* out = t == 0 ? q : (t == 1 ? k : v);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < hid; k0 += kSlice) {
    for (int e = tid; e < kTile * kSlice; e += 256) {
      const int r = e >> 4, kk = e & 15;
      const int64_t n = r0 + r;
      As[kk][r] = (n < N && k0 + kk < hid) ? to_f(x[n * hid + k0 + kk]) : 0.f;
      const int kb = e >> 6, c = e & 63;
      Bs[kb][c] = (k0 + kb < hid && c0 + c < hid) ? to_f(W[static_cast<int64_t>(k0 + kb) * hid + c0 + c]) : 0.f;
    }
    __syncthreads();
    slice_fma(acc, As, Bs, tx, ty);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = r0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + 4 * tx + j;
      if (n < N && c < hid) put(out + n * hid + c, acc[i][j]);
    }
  }
}

// dX[n, c] = sum_t sum_j dT_t[n, j] W_t[c, j]; grid (row tiles, column tiles).
template <typename T>
__global__ __launch_bounds__(256) void qkv_dx_kernel(const T* __restrict__ w, const float* __restrict__ dq,
                                                     const float* __restrict__ dk, const float* __restrict__ dv,
                                                     float* __restrict__ dx, int64_t N, int hid) {
  __shared__ float As[kSlice][kTile + 1];
  __shared__ float Bs[kSlice][kTile];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int c0 = blockIdx.y * kTile;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int t = 0; t < 3; ++t) {
    const float* G = t == 0 ? dq : (t == 1 ? dk : dv);
    const T* W = w + static_cast<int64_t>(t) * hid * hid;
    for (int k0 = 0; k0 < hid; k0 += kSlice) {
      for (int e = tid; e < kTile * kSlice; e += 256) {
        const int r = e >> 4, kk = e & 15;
        const int64_t n = r0 + r;
        As[kk][r] = (n < N && k0 + kk < hid) ? G[n * hid + k0 + kk] : 0.f;
        const int c = e >> 4, kb = e & 15;  // W_t[c, j]: consecutive threads walk j
        Bs[kb][c] = (k0 + kb < hid && c0 + c < hid) ? to_f(W[static_cast<int64_t>(c0 + c) * hid + k0 + kb]) : 0.f;
      }
      __syncthreads();
      slice_fma(acc, As, Bs, tx, ty);
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = r0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + 4 * tx + j;
      if (n < N && c < hid) dx[n * hid + c] = acc[i][j];
    }
  }
}

// Partial dW_t[a, b] = sum over nodes n of chunk blockIdx.x of X[n, a] dT_t[n, b];
// grid (node chunks, a tiles * b tiles, 3). Written to part[chunk][t][a][b].
template <typename T>
__global__ __launch_bounds__(256) void qkv_dw_partial_kernel(const T* __restrict__ x, const float* __restrict__ dq,
                                                             const float* __restrict__ dk,
                                                             const float* __restrict__ dv, float* __restrict__ part,
                                                             int64_t N, int hid) {
  __shared__ float As[kSlice][kTile + 1];  // [node][a]
  __shared__ float Bs[kSlice][kTile];      // [node][b]
  const int t = blockIdx.z;
  const float* G = t == 0 ? dq : (t == 1 ? dk : dv);
  const int tiles = (hid + kTile - 1) / kTile;
  const int a0 = (blockIdx.y / tiles) * kTile, b0 = (blockIdx.y % tiles) * kTile;
  const int64_t n_begin = static_cast<int64_t>(blockIdx.x) * kChunk;
  const int64_t n_end = n_begin + kChunk < N ? n_begin + kChunk : N;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int64_t n0 = n_begin; n0 < n_end; n0 += kSlice) {
    for (int e = tid; e < kTile * kSlice; e += 256) {
      const int kk = e >> 6, c = e & 63;
      const int64_t n = n0 + kk;
      const bool in = n < n_end;
      As[kk][c] = (in && a0 + c < hid) ? to_f(x[n * hid + a0 + c]) : 0.f;
      Bs[kk][c] = (in && b0 + c < hid) ? G[n * hid + b0 + c] : 0.f;
    }
    __syncthreads();
    slice_fma(acc, As, Bs, tx, ty);
    __syncthreads();
  }
  float* P = part + (static_cast<int64_t>(blockIdx.x) * 3 + t) * hid * hid;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = a0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = b0 + 4 * tx + j;
      if (a < hid && b < hid) P[a * hid + b] = acc[i][j];
    }
  }
}

// dW[e] = sum over chunks c, in order, of part[c][e]; e < 3*hid*hid.
__global__ __launch_bounds__(256) void qkv_dw_reduce_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                            int64_t nchunks, int64_t per_chunk) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= per_chunk) return;
  float s = 0.f;
  for (int64_t c = 0; c < nchunks; ++c) s += part[c * per_chunk + e];
  dw[e] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void store_kernel(const float* __restrict__ src, T* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) put(dst + i, src[i]);
}

int64_t n_chunks(int64_t N) { return (N + kChunk - 1) / kChunk; }

}  // namespace

size_t qkv_bwd_workspace(int64_t N, int hid) {
  return static_cast<size_t>(n_chunks(N)) * 3 * hid * hid * sizeof(float);
}

hipError_t launch_qkv_fwd(const void* x, const void* w, void* q, void* k, void* v, int64_t N, int hid, int dtype,
                          hipStream_t s) {
  const int tiles = (hid + kTile - 1) / kTile;
  const dim3 grid(static_cast<unsigned>((N + kTile - 1) / kTile), tiles, 3);
  trace_begin(kTraceQkvFwd, s);
  if (dtype == 1)
    hipLaunchKernelGGL(qkv_fwd_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w), static_cast<uint16_t*>(q), static_cast<uint16_t*>(k),
                       static_cast<uint16_t*>(v), N, hid);
  else
    hipLaunchKernelGGL(qkv_fwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(w), static_cast<float*>(q), static_cast<float*>(k),
                       static_cast<float*>(v), N, hid);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceQkvFwd, s);
  return e;
}

hipError_t launch_qkv_bwd(const void* x, const void* w, const float* dq, const float* dk, const float* dv, float* dx,
                          float* dw, void* workspace, int64_t N, int hid, int dtype, hipStream_t s) {
  const int tiles = (hid + kTile - 1) / kTile;
  const dim3 grid_dx(static_cast<unsigned>((N + kTile - 1) / kTile), tiles);
  trace_begin(kTraceQkvDx, s);
  if (dtype == 1)
    hipLaunchKernelGGL(qkv_dx_kernel<uint16_t>, grid_dx, dim3(256), 0, s, static_cast<const uint16_t*>(w), dq, dk,
                       dv, dx, N, hid);
  else
    hipLaunchKernelGGL(qkv_dx_kernel<float>, grid_dx, dim3(256), 0, s, static_cast<const float*>(w), dq, dk, dv,
                       dx, N, hid);
  hipError_t e = hipGetLastError();
  trace_end(kTraceQkvDx, s);
  if (e != hipSuccess) return e;
  float* part = static_cast<float*>(workspace);
  const int64_t nch = n_chunks(N);
  const dim3 grid_dw(static_cast<unsigned>(nch), tiles * tiles, 3);
  trace_begin(kTraceQkvDw, s);
  if (dtype == 1)
    hipLaunchKernelGGL(qkv_dw_partial_kernel<uint16_t>, grid_dw, dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       dq, dk, dv, part, N, hid);
  else
    hipLaunchKernelGGL(qkv_dw_partial_kernel<float>, grid_dw, dim3(256), 0, s, static_cast<const float*>(x), dq, dk,
                       dv, part, N, hid);
  e = hipGetLastError();
  if (e == hipSuccess) {
    const int64_t per = 3ll * hid * hid;
    hipLaunchKernelGGL(qkv_dw_reduce_kernel, dim3(static_cast<unsigned>((per + 255) / 256)), dim3(256), 0, s, part,
                       dw, nch, per);
    e = hipGetLastError();
  }
  trace_end(kTraceQkvDw, s);
  return e;
}

hipError_t launch_store(const float* src, void* dst, int64_t n, int dtype, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  trace_begin(kTraceStore, s);
  if (dtype == 1)
    hipLaunchKernelGGL(store_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                       static_cast<uint16_t*>(dst), n);
  else
    hipLaunchKernelGGL(store_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                       static_cast<float*>(dst), n);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceStore, s);
  return e;
}

}  // namespace gt
