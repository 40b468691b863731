// The dense parts of a full Graph-Transformer layer around the biased attention
// (MegaGraph pages, Fig. 8 caption: 16 layers, 8 heads, hidden and feed-forward
// dimension 64), read as the pre-norm Transformer layer:
//
//   A  = LN(X; g1, b1)                   Q, K, V = store(A Wq), store(A Wk), store(A Wv)
//   O  = attention(Q, K, V)              (the attention kernels)
//   X1 = X + O Wo                        B = LN(X1; g2, b2)
//   X2 = X1 + gelu(B W1 + c1) W2 + c2
//
// LN normalises over the hidden dimension with a biased variance and eps = 1e-5;
// gelu(x) = x Phi(x). Hidden and feed-forward sizes are both 64, so every dense step
// is a product of a node's 64-vector with a 64 x 64 matrix: a few percent of a
// layer's work next to the H*N^2 attention entries. These kernels therefore fuse all
// per-node steps of one side of the attention into one launch, with the weights in
// LDS: a workgroup of 128 threads holds 16 nodes, 8 threads per node, each thread 8
// of the node's 64 columns. A product reads the node's input vector from an LDS row
// buffer (one broadcast per node) and the weight columns of its thread's 8 outputs
// (consecutive threads read consecutive 32-byte runs); transposed products use a
// transposed copy staged in LDS. Row reductions (mean, variance) use shuffles across
// a node's 8 lanes.
//
// Weight gradients are sums over nodes of outer products; wgrad_partial_kernel forms
// them per 256-node chunk for up to 8 (input, gradient) pairs in one launch and
// wgrad_reduce_kernel adds the chunks in order, so they are reproducible.
//
// Parameter vector of one layer (floats): g1[64], b1[64], Wq, Wk, Wv, Wo [64][64],
// g2[64], b2[64], W1 [64][64], c1[64], W2 [64][64], c2[64]; W[a][b] multiplies input
// column a into output column b.
#include "gt_internal.h"

#include <algorithm>

namespace gt {
namespace {

constexpr int kHid = 64;
constexpr int kRows = 16;            // nodes per workgroup
constexpr int kLThreads = 8 * kRows; // 8 threads per node
constexpr int kRb = kHid + 4;        // LDS row stride (floats) of row buffers and staged matrices
constexpr int kMat = kHid * kHid;    // floats of a matrix in global memory
constexpr int kMatL = kHid * kRb;    // floats of a staged matrix in LDS
constexpr float kLnEps = 1e-5f;

// offsets of the parameter vector
constexpr int kG1 = 0, kB1 = 64, kWq = 128, kWk = kWq + kMat, kWv = kWk + kMat, kWo = kWv + kMat;
constexpr int kG2 = kWo + kMat, kB2 = kG2 + 64, kW1 = kB2 + 64, kC1 = kW1 + kMat, kW2 = kC1 + 64;
constexpr int kC2 = kW2 + kMat, kParams = kC2 + 64;
static_assert(kParams == 24960, "parameter layout");

__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ uint16_t f_to_bf16(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

struct V8 {
  float v[8];
};

__device__ __forceinline__ V8 load8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return V8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ void store8(float* p, const V8& x) {
  *reinterpret_cast<float4*>(p) = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x.v[4], x.v[5], x.v[6], x.v[7]);
}
// eight values in the attention's storage type (dtype 1: bfloat16, rounded)
__device__ __forceinline__ void store8_t(void* base, int64_t off, const V8& x, int dtype) {
  if (dtype == 1) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f_to_bf16(x.v[2 * i])) | (static_cast<uint32_t>(f_to_bf16(x.v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    store8(static_cast<float*>(base) + off, x);
  }
}

// Sum over the 8 lanes of one node (consecutive lanes).
__device__ __forceinline__ float node_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// out[j] = sum_k row[k] M[k][c0 + j], j < 8; row and M in LDS (M row stride kRb).
__device__ __forceinline__ V8 matvec(const float* row, const float* M, int c0) {
  V8 o{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
  for (int k = 0; k < kHid; k += 4) {
    const float4 x = *reinterpret_cast<const float4*>(row + k);
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const V8 w = load8(M + (k + u) * kRb + c0);
#pragma unroll
      for (int j = 0; j < 8; ++j) o.v[j] = fmaf(xs[u], w.v[j], o.v[j]);
    }
  }
  return o;
}

// Stage a 64 x 64 matrix into LDS (row stride kRb) as is or transposed, four floats per
// load; the padded stride spreads a transposed write's lanes over the banks.
__device__ __forceinline__ void stage_mat(float* dst, const float* src, bool transpose, int tid) {
  for (int e = 4 * tid; e < kMat; e += 4 * kLThreads) {
    const int a = e >> 6, b = e & 63;
    const float4 x = *reinterpret_cast<const float4*>(src + e);
    if (transpose) {
      dst[b * kRb + a] = x.x;
      dst[(b + 1) * kRb + a] = x.y;
      dst[(b + 2) * kRb + a] = x.z;
      dst[(b + 3) * kRb + a] = x.w;
    } else {
      *reinterpret_cast<float4*>(dst + a * kRb + b) = x;
    }
  }
}

struct RowCtx {
  int64_t n;   // node
  int rl, c0;  // node within the workgroup, first column of this thread
  bool valid;
};
__device__ __forceinline__ RowCtx row_ctx(int64_t N) {
  RowCtx c;
  c.rl = threadIdx.x >> 3;
  c.c0 = 8 * (threadIdx.x & 7);
  c.n = static_cast<int64_t>(blockIdx.x) * kRows + c.rl;
  c.valid = c.n < N;
  return c;
}

// Normalise one node's row: returns xhat (8 columns of this thread) and mean, rstd.
__device__ __forceinline__ V8 normalise(const V8& x, float& mean, float& rstd) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x.v[j];
  mean = node_sum(s) * (1.f / kHid);
  float ss = 0.f;
  V8 d;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    d.v[j] = x.v[j] - mean;
    ss = fmaf(d.v[j], d.v[j], ss);
  }
  rstd = 1.f / sqrtf(node_sum(ss) * (1.f / kHid) + kLnEps);
#pragma unroll
  for (int j = 0; j < 8; ++j) d.v[j] *= rstd;
  return d;
}

// LN backward for one node: dx = rstd * (dxh - mean(dxh) - xhat * mean(dxh * xhat)),
// dxh = dy * g.
__device__ __forceinline__ V8 ln_backward(const V8& dy, const V8& xhat, const float* g, int c0, float rstd) {
  V8 dxh;
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dxh.v[j] = dy.v[j] * g[c0 + j];
    s1 += dxh.v[j];
    s2 = fmaf(dxh.v[j], xhat.v[j], s2);
  }
  const float m1 = node_sum(s1) * (1.f / kHid), m2 = node_sum(s2) * (1.f / kHid);
  V8 dx;
#pragma unroll
  for (int j = 0; j < 8; ++j) dx.v[j] = rstd * (dxh.v[j] - m1 - xhat.v[j] * m2);
  return dx;
}

__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad(float x) {
  return 0.5f * (1.f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * expf(-0.5f * x * x);
}

// Pre-attention side, forward: A = LN(X; g1, b1) and Q, K, V = store(A W_t); saves the
// node's mean and 1/std.
__global__ __launch_bounds__(kLThreads) void pre_fwd_kernel(const float* __restrict__ x, const float* __restrict__ p,
                                                            void* q, void* k, void* v, float* __restrict__ stats,
                                                            int64_t N, int dtype) {
  __shared__ __align__(16) float W[3][kMatL];
  __shared__ __align__(16) float rb[kRows][kRb];
  const int tid = threadIdx.x;
  for (int t = 0; t < 3; ++t) stage_mat(W[t], p + kWq + t * kMat, false, tid);
  const RowCtx c = row_ctx(N);
  const V8 xv = c.valid ? load8(x + c.n * kHid + c.c0) : V8{};
  float mean, rstd;
  V8 a = normalise(xv, mean, rstd);
#pragma unroll
  for (int j = 0; j < 8; ++j) a.v[j] = fmaf(a.v[j], p[kG1 + c.c0 + j], p[kB1 + c.c0 + j]);
  store8(&rb[c.rl][c.c0], a);
  if (c.valid && (tid & 7) == 0) {
    stats[2 * c.n] = mean;
    stats[2 * c.n + 1] = rstd;
  }
  __syncthreads();
  void* outs[3] = {q, k, v};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const V8 o = matvec(rb[c.rl], W[t], c.c0);
    if (c.valid) store8_t(outs[t], c.n * kHid + c.c0, o, dtype);
  }
}

// Post-attention side, forward: X1 = X + O Wo, B = LN(X1; g2, b2), Hd = B W1 + c1,
// X2 = X1 + gelu(Hd) W2 + c2. Saves X1, the node's LN statistics and Hd.
__global__ __launch_bounds__(kLThreads) void post_fwd_kernel(const float* __restrict__ x, const float* __restrict__ o,
                                                             const float* __restrict__ p, float* __restrict__ x1,
                                                             float* __restrict__ stats, float* __restrict__ hd,
                                                             float* __restrict__ x2, int64_t N) {
  __shared__ __align__(16) float W[3][kMatL];  // Wo, W1, W2
  __shared__ __align__(16) float rb[kRows][kRb];
  const int tid = threadIdx.x;
  stage_mat(W[0], p + kWo, false, tid);
  stage_mat(W[1], p + kW1, false, tid);
  stage_mat(W[2], p + kW2, false, tid);
  const RowCtx c = row_ctx(N);
  const int64_t off = c.n * kHid + c.c0;
  store8(&rb[c.rl][c.c0], c.valid ? load8(o + off) : V8{});
  __syncthreads();
  const V8 y = matvec(rb[c.rl], W[0], c.c0);
  const V8 xv = c.valid ? load8(x + off) : V8{};
  V8 r1;
#pragma unroll
  for (int j = 0; j < 8; ++j) r1.v[j] = xv.v[j] + y.v[j];
  if (c.valid) store8(x1 + off, r1);
  float mean, rstd;
  V8 b = normalise(r1, mean, rstd);
#pragma unroll
  for (int j = 0; j < 8; ++j) b.v[j] = fmaf(b.v[j], p[kG2 + c.c0 + j], p[kB2 + c.c0 + j]);
  if (c.valid && (tid & 7) == 0) {
    stats[2 * c.n] = mean;
    stats[2 * c.n + 1] = rstd;
  }
  __syncthreads();  // every node's O row has been read
  store8(&rb[c.rl][c.c0], b);
  __syncthreads();
  V8 h = matvec(rb[c.rl], W[1], c.c0);
#pragma unroll
  for (int j = 0; j < 8; ++j) h.v[j] += p[kC1 + c.c0 + j];
  if (c.valid) store8(hd + off, h);
  V8 g;
#pragma unroll
  for (int j = 0; j < 8; ++j) g.v[j] = gelu(h.v[j]);
  __syncthreads();
  store8(&rb[c.rl][c.c0], g);
  __syncthreads();
  const V8 f = matvec(rb[c.rl], W[2], c.c0);
  V8 out;
#pragma unroll
  for (int j = 0; j < 8; ++j) out.v[j] = r1.v[j] + f.v[j] + p[kC2 + c.c0 + j];
  if (c.valid) store8(x2 + off, out);
}

// Post-attention side, backward, for the output gradient dX2: writes dX1, the
// attention's output gradient dO = store(dX1 Wo^T), and per node the factors of the
// weight gradients: G = gelu(Hd), B, dHd, Bhat, dB.
__global__ __launch_bounds__(kLThreads) void post_bwd_kernel(const float* __restrict__ dx2,
                                                             const float* __restrict__ x1,
                                                             const float* __restrict__ stats,
                                                             const float* __restrict__ hd, const float* __restrict__ p,
                                                             float* __restrict__ dx1, void* dout_attn,
                                                             float* __restrict__ gbuf, float* __restrict__ bbuf,
                                                             float* __restrict__ dhbuf, float* __restrict__ bhbuf,
                                                             float* __restrict__ dbbuf, int64_t N, int dtype) {
  __shared__ __align__(16) float W[3][kMatL];  // W2^T, W1^T, Wo^T
  __shared__ __align__(16) float rb[kRows][kRb];
  const int tid = threadIdx.x;
  stage_mat(W[0], p + kW2, true, tid);
  stage_mat(W[1], p + kW1, true, tid);
  stage_mat(W[2], p + kWo, true, tid);
  const RowCtx c = row_ctx(N);
  const int64_t off = c.n * kHid + c.c0;
  const float mean = c.valid ? stats[2 * c.n] : 0.f, rstd = c.valid ? stats[2 * c.n + 1] : 1.f;
  const V8 r1 = c.valid ? load8(x1 + off) : V8{};
  V8 bh, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bh.v[j] = (r1.v[j] - mean) * rstd;
    b.v[j] = fmaf(bh.v[j], p[kG2 + c.c0 + j], p[kB2 + c.c0 + j]);
  }
  const V8 h = c.valid ? load8(hd + off) : V8{};
  V8 g;
#pragma unroll
  for (int j = 0; j < 8; ++j) g.v[j] = gelu(h.v[j]);
  const V8 d2 = c.valid ? load8(dx2 + off) : V8{};
  if (c.valid) {
    store8(bhbuf + off, bh);
    store8(bbuf + off, b);
    store8(gbuf + off, g);
  }
  store8(&rb[c.rl][c.c0], d2);
  __syncthreads();
  V8 dh = matvec(rb[c.rl], W[0], c.c0);  // dG = dX2 W2^T
#pragma unroll
  for (int j = 0; j < 8; ++j) dh.v[j] *= gelu_grad(h.v[j]);
  if (c.valid) store8(dhbuf + off, dh);
  __syncthreads();
  store8(&rb[c.rl][c.c0], dh);
  __syncthreads();
  const V8 db = matvec(rb[c.rl], W[1], c.c0);  // dB = dHd W1^T
  if (c.valid) store8(dbbuf + off, db);
  const V8 dln = ln_backward(db, bh, p + kG2, c.c0, rstd);
  V8 d1;
#pragma unroll
  for (int j = 0; j < 8; ++j) d1.v[j] = d2.v[j] + dln.v[j];
  if (c.valid) store8(dx1 + off, d1);
  __syncthreads();
  store8(&rb[c.rl][c.c0], d1);
  __syncthreads();
  const V8 dO = matvec(rb[c.rl], W[2], c.c0);  // dO = dX1 Wo^T
  if (c.valid) store8_t(dout_attn, off, dO, dtype);
}

// Pre-attention side, backward: dA = dQ Wq^T + dK Wk^T + dV Wv^T, then
// dX = dX1 + LN1 backward(dA). Writes the factors A, Ahat and dA of the weight
// gradients.
__global__ __launch_bounds__(kLThreads) void pre_bwd_kernel(const float* __restrict__ dq, const float* __restrict__ dk,
                                                            const float* __restrict__ dv, const float* __restrict__ x,
                                                            const float* __restrict__ stats,
                                                            const float* __restrict__ p, const float* __restrict__ dx1,
                                                            float* __restrict__ dx, float* __restrict__ abuf,
                                                            float* __restrict__ ahbuf, float* __restrict__ dabuf,
                                                            int64_t N) {
  __shared__ __align__(16) float W[3][kMatL];  // Wq^T, Wk^T, Wv^T
  __shared__ __align__(16) float rb[kRows][kRb];
  const int tid = threadIdx.x;
  for (int t = 0; t < 3; ++t) stage_mat(W[t], p + kWq + t * kMat, true, tid);
  const RowCtx c = row_ctx(N);
  const int64_t off = c.n * kHid + c.c0;
  const float* grads[3] = {dq, dk, dv};
  V8 da{};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (t > 0) __syncthreads();
    store8(&rb[c.rl][c.c0], c.valid ? load8(grads[t] + off) : V8{});
    __syncthreads();
    const V8 part = matvec(rb[c.rl], W[t], c.c0);
#pragma unroll
    for (int j = 0; j < 8; ++j) da.v[j] += part.v[j];
  }
  const float mean = c.valid ? stats[2 * c.n] : 0.f, rstd = c.valid ? stats[2 * c.n + 1] : 1.f;
  const V8 xv = c.valid ? load8(x + off) : V8{};
  V8 ah, a;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ah.v[j] = (xv.v[j] - mean) * rstd;
    a.v[j] = fmaf(ah.v[j], p[kG1 + c.c0 + j], p[kB1 + c.c0 + j]);
  }
  const V8 dln = ln_backward(da, ah, p + kG1, c.c0, rstd);
  if (c.valid) {
    const V8 d1 = load8(dx1 + off);
    V8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o.v[j] = d1.v[j] + dln.v[j];
    store8(dx + off, o);
    store8(abuf + off, a);
    store8(ahbuf + off, ah);
    store8(dabuf + off, da);
  }
}

// Weight gradients, per chunk of kChunkRows nodes: for each job, either
//   outer: out[a][b] = sum_n A[n][a] D[n][b]   (64 x 64 at w_off) and, if c_off >= 0,
//          colsum[b] = sum_n D[n][b]           (64 at c_off)
//   diag:  out[b] = sum_n A[n][b] D[n][b]      (64 at w_off), colsum at c_off
// written to partial[chunk][...]; grid (chunks, jobs).
constexpr int kChunkRows = 256;
constexpr int kSub = 64;        // nodes staged in LDS at a time
constexpr int kWThreads = 256;  // thread t owns the 4 x 4 outer-product block at [4*(t/16)][4*(t%16)]

__global__ __launch_bounds__(kWThreads) void wgrad_partial_kernel(WgradJobs jobs, float* __restrict__ partial,
                                                                  int64_t N) {
  __shared__ __align__(16) float As[kSub][kHid];
  __shared__ __align__(16) float Ds[kSub][kHid];
  WgradJob job = jobs.j[0];  // jobs.j[blockIdx.y], selected with static indices (no private copy)
#pragma unroll
  for (int i = 1; i < 8; ++i)
    if (i == static_cast<int>(blockIdx.y)) job = jobs.j[i];
  const float* A = job.a;
  const float* Dm = job.d;
  const int diag = job.diag;
  const int tid = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kChunkRows;
  const int a0 = 4 * (tid >> 4), b0 = 4 * (tid & 15);  // outer: entries [a0 .. a0+3][b0 .. b0+3]
  float acc[4][4] = {};
  float cs = 0.f, dg = 0.f;
  for (int s = 0; s < kChunkRows; s += kSub) {
    for (int e = tid; e < kSub * kHid / 4; e += kWThreads) {
      const int r = e >> 4, c4 = 4 * (e & 15);
      const int64_t n = n0 + s + r;
      float4 av = make_float4(0.f, 0.f, 0.f, 0.f), dv = av;
      if (n < N) {
        av = *reinterpret_cast<const float4*>(A + n * kHid + c4);
        dv = *reinterpret_cast<const float4*>(Dm + n * kHid + c4);
      }
      *reinterpret_cast<float4*>(&As[r][c4]) = av;
      *reinterpret_cast<float4*>(&Ds[r][c4]) = dv;
    }
    __syncthreads();
    if (!diag) {
#pragma unroll 4
      for (int r = 0; r < kSub; ++r) {
        const float4 av = *reinterpret_cast<const float4*>(&As[r][a0]);
        const float4 dv = *reinterpret_cast<const float4*>(&Ds[r][b0]);
        const float ar[4] = {av.x, av.y, av.z, av.w}, dr[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], dr[j], acc[i][j]);
      }
    }
    if (tid < kHid) {
      for (int r = 0; r < kSub; ++r) {
        cs += Ds[r][tid];
        dg = fmaf(As[r][tid], Ds[r][tid], dg);
      }
    }
    __syncthreads();
  }
  float* out = partial + static_cast<int64_t>(blockIdx.x) * jobs.stride;
  if (!diag) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(out + job.w_off + (a0 + i) * kHid + b0) =
          make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  } else if (tid < kHid) {
    out[job.w_off + tid] = dg;
  }
  if (job.c_off >= 0 && tid < kHid) out[job.c_off + tid] = cs;
}

// grad[x] = sum over chunks of partial[chunk][x], in chunk order.
__global__ __launch_bounds__(kWThreads) void wgrad_reduce_kernel(const float* __restrict__ partial, int64_t chunks,
                                                                 int stride, float* __restrict__ grad) {
  const int x = blockIdx.x * kWThreads + threadIdx.x;
  if (x >= stride) return;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += partial[c * stride + x];
  grad[x] = s;
}

}  // namespace

int model_params(int hid, int ffn) { return hid == kHid && ffn == kHid ? kParams : 0; }
int64_t model_wgrad_chunks(int64_t N) { return (N + kChunkRows - 1) / kChunkRows; }

hipError_t launch_layer_pre_fwd(const float* x, const float* p, void* q, void* k, void* v, float* stats, int64_t N,
                                int dtype, hipStream_t s) {
  trace_begin(kTraceLayerFwd, s);
  hipLaunchKernelGGL(pre_fwd_kernel, dim3(static_cast<unsigned>((N + kRows - 1) / kRows)), dim3(kLThreads), 0, s, x,
                     p, q, k, v, stats, N, dtype);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceLayerFwd, s);
  return e;
}

hipError_t launch_layer_post_fwd(const float* x, const float* o, const float* p, float* x1, float* stats, float* hd,
                                 float* x2, int64_t N, hipStream_t s) {
  trace_begin(kTraceLayerFwd, s);
  hipLaunchKernelGGL(post_fwd_kernel, dim3(static_cast<unsigned>((N + kRows - 1) / kRows)), dim3(kLThreads), 0, s,
                     x, o, p, x1, stats, hd, x2, N);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceLayerFwd, s);
  return e;
}

hipError_t launch_layer_post_bwd(const float* dx2, const float* x1, const float* stats, const float* hd,
                                 const float* p, float* dx1, void* dout_attn, float* const bufs[5], int64_t N,
                                 int dtype, hipStream_t s) {
  trace_begin(kTraceLayerBwd, s);
  hipLaunchKernelGGL(post_bwd_kernel, dim3(static_cast<unsigned>((N + kRows - 1) / kRows)), dim3(kLThreads), 0, s,
                     dx2, x1, stats, hd, p, dx1, dout_attn, bufs[0], bufs[1], bufs[2], bufs[3], bufs[4], N, dtype);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceLayerBwd, s);
  return e;
}

hipError_t launch_layer_pre_bwd(const float* dq, const float* dk, const float* dv, const float* x, const float* stats,
                                const float* p, const float* dx1, float* dx, float* const bufs[3], int64_t N,
                                hipStream_t s) {
  trace_begin(kTraceLayerBwd, s);
  hipLaunchKernelGGL(pre_bwd_kernel, dim3(static_cast<unsigned>((N + kRows - 1) / kRows)), dim3(kLThreads), 0, s,
                     dq, dk, dv, x, stats, p, dx1, dx, bufs[0], bufs[1], bufs[2], N);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceLayerBwd, s);
  return e;
}

hipError_t launch_layer_wgrad(const LayerGradFactors& f, float* partial, float* grad, int64_t N, hipStream_t s) {
  WgradJobs jobs{};
  jobs.stride = kParams;
  const WgradJob list[8] = {{f.ahat, f.da, 1, kG1, kB1},  {f.a, f.dq, 0, kWq, -1},  {f.a, f.dk, 0, kWk, -1},
                            {f.a, f.dv, 0, kWv, -1},      {f.o, f.dx1, 0, kWo, -1}, {f.bhat, f.db, 1, kG2, kB2},
                            {f.b, f.dh, 0, kW1, kC1},     {f.g, f.dx2, 0, kW2, kC2}};
  for (int i = 0; i < 8; ++i) jobs.j[i] = list[i];
  jobs.n = 8;
  return launch_wgrad_jobs(jobs, partial, grad, N, s);
}

hipError_t launch_wgrad_jobs(const WgradJobs& jobs, float* partial, float* grad, int64_t N, hipStream_t s) {
  const int64_t chunks = model_wgrad_chunks(N);
  trace_begin(kTraceLayerWgrad, s);
  hipLaunchKernelGGL(wgrad_partial_kernel, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(jobs.n)),
                     dim3(kWThreads), 0, s, jobs, partial, N);
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(static_cast<unsigned>((jobs.stride + kWThreads - 1) / kWThreads)),
                     dim3(kWThreads), 0, s, partial, chunks, jobs.stride, grad);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceLayerWgrad, s);
  return e;
}

}  // namespace gt
