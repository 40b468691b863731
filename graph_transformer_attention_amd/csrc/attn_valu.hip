// General biased-attention kernels on the vector ALU (any supported H and D, float32
// or bfloat16 storage). One thread owns one (node, head) pair; tiles of the other
// operand and of the uint8 code matrix are staged in LDS, and the bias table
// (premultiplied by log2 e) sits in LDS for the whole kernel.
//
// MegaGraph pages, Fig. 4 caption: attention is computed block by block over the
// keys with the bias columns sliced to each block — here each key tile of the
// forward pulls exactly the matching code columns and merges its softmax
// statistics into a running (max, sum) pair.
#include "gt_internal.h"

#include <algorithm>

namespace gt {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr size_t kLdsDefault = 65536;

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------
// Forward: thread (r, h) owns query row i = blockIdx.x*R + r and head h.
// LDS: table*log2e [H*NB] | K tile [BN][H][D] | V tile | codes [R][BN].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint8_t* __restrict__ spd, const float* __restrict__ table, float* __restrict__ out,
    float* __restrict__ lse, int64_t N, int64_t Nk, int64_t ldc, int H, int NB, int BN, float qscale) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int HD = H * D;
  const int R = kThreads / H;
  float* tb = reinterpret_cast<float*>(smem);
  float* Ks = tb + ((H * NB + 3) & ~3);
  float* Vs = Ks + BN * HD;
  uint8_t* cs = reinterpret_cast<uint8_t*>(Vs + BN * HD);

  const int t = threadIdx.x;
  const int r = t / H, h = t - r * H;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
  const int64_t i = row0 + r;
  const bool valid = (r < R) && (i < N);

  for (int x = t; x < H * NB; x += kThreads) tb[x] = table[x] * kLog2e;

  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = valid ? ld(q, (i * H + h) * D + d) * qscale : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* tbh = tb + h * NB;

  for (int64_t j0 = 0; j0 < Nk; j0 += BN) {
    const int nk = static_cast<int>(std::min<int64_t>(BN, Nk - j0));
    __syncthreads();
    for (int x = t; x < BN * HD; x += kThreads) {
      const int jj = x / HD;
      float kx = 0.f, vx = 0.f;
      if (jj < nk) {
        const int64_t g = (j0 + jj) * HD + (x - jj * HD);
        kx = ld(k, g);
        vx = ld(v, g);
      }
      Ks[x] = kx;
      Vs[x] = vx;
    }
    for (int x = t; x < R * BN; x += kThreads) {
      const int rr = x / BN, jj = x - rr * BN;
      const int64_t ii = row0 + rr;
      cs[x] = (ii < N && jj < nk) ? spd[ii * ldc + j0 + jj] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    const uint8_t* crow = cs + r * BN;
    for (int jc = 0; jc < nk; jc += 8) {
      float s[8];
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = jc + u;
        float sv = -INFINITY;
        if (j < nk) {
          const float* kp = Ks + (j * H + h) * D;
          float dot = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) dot = fmaf(qr[d], kp[d], dot);
          const int code = min(static_cast<int>(crow[j]), NB - 1);
          sv = dot + tbh[code];
        }
        s[u] = sv;
        cmax = fmaxf(cmax, sv);
      }
      const float mn = fmaxf(m, cmax);
      const float alpha = exp2_hw(m - mn);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = jc + u;
        if (j < nk) {
          const float p = exp2_hw(s[u] - mn);
          l += p;
          const float* vp = Vs + (j * H + h) * D;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vp[d], acc[d]);
        }
      }
      m = mn;
    }
  }
  if (valid) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) out[(i * H + h) * D + d] = acc[d] * inv;
    lse[i * H + h] = (m + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------
// Backward, step 1: delta[i,h] = sum_d dout[i,h,d] * out[i,h,d].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const float* __restrict__ out,
                                                             const T* __restrict__ dout,
                                                             float* __restrict__ delta,
                                                             int64_t NH) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (x >= NH) return;
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) s = fmaf(ld(dout, x * D + d), out[x * D + d], s);
  delta[x] = s;
}

// Backward, step 2 (key-outer): thread (c, h) owns key j = blockIdx.x*CK + c and head h,
// loops over all query rows and accumulates dK, dV and per-thread bucket sums of dS.
// LDS: table*log2e | bins [NB][256] | Q tile [BM][H][D] | dO tile | lse*log2e [BM][H]
//      | delta [BM][H] | codes [BM][CK].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_kv_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint8_t* __restrict__ spd, const float* __restrict__ table,
    const float* __restrict__ lse, const float* __restrict__ delta, const T* __restrict__ dout,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ partial, int64_t N,
    int64_t Nk, int64_t ldc, int H, int NB, int BM, float qscale, float scale, int acc) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int HD = H * D;
  const int CK = kThreads / H;
  float* tb = reinterpret_cast<float*>(smem);
  float* bins = tb + ((H * NB + 3) & ~3);
  float* Qs = bins + NB * kThreads;
  float* Os = Qs + BM * HD;
  float* Ls = Os + BM * HD;
  float* Ds = Ls + BM * H;
  uint8_t* cs = reinterpret_cast<uint8_t*>(Ds + BM * H);

  const int t = threadIdx.x;
  const int c = t / H, h = t - c * H;
  const int64_t col0 = static_cast<int64_t>(blockIdx.x) * CK;
  const int64_t j = col0 + c;
  const bool valid = (c < CK) && (j < Nk);

  for (int x = t; x < H * NB; x += kThreads) tb[x] = table[x] * kLog2e;
  for (int b = 0; b < NB; ++b) bins[b * kThreads + t] = 0.f;

  float kr[D], vr[D], dka[D], dva[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = valid ? ld(k, (j * H + h) * D + d) : 0.f;
    vr[d] = valid ? ld(v, (j * H + h) * D + d) : 0.f;
    dka[d] = 0.f;
    dva[d] = 0.f;
  }
  const float* tbh = tb + h * NB;

  for (int64_t i0 = 0; i0 < N; i0 += BM) {
    const int nq = static_cast<int>(std::min<int64_t>(BM, N - i0));
    __syncthreads();
    for (int x = t; x < BM * HD; x += kThreads) {
      const int ii = x / HD;
      float qx = 0.f, ox = 0.f;
      if (ii < nq) {
        const int64_t g = (i0 + ii) * HD + (x - ii * HD);
        qx = ld(q, g);
        ox = ld(dout, g);
      }
      Qs[x] = qx;
      Os[x] = ox;
    }
    for (int x = t; x < BM * H; x += kThreads) {
      const int ii = x / H;
      const bool ok = ii < nq;
      Ls[x] = ok ? lse[i0 * H + x] * kLog2e : 0.f;
      Ds[x] = ok ? delta[i0 * H + x] : 0.f;
    }
    for (int x = t; x < BM * CK; x += kThreads) {
      const int ii = x / CK, cc = x - ii * CK;
      cs[x] = (ii < nq && col0 + cc < Nk) ? spd[(i0 + ii) * ldc + col0 + cc] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    for (int ii = 0; ii < nq; ++ii) {
      const float* qp = Qs + (ii * H + h) * D;
      const float* op = Os + (ii * H + h) * D;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dot = fmaf(qp[d], kr[d], dot);
        dp = fmaf(op[d], vr[d], dp);
      }
      const int code = min(static_cast<int>(cs[ii * CK + c]), NB - 1);
      const float p = exp2_hw(fmaf(dot, qscale, tbh[code]) - Ls[ii * H + h]);
      const float ds = p * (dp - Ds[ii * H + h]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dva[d] = fmaf(p, op[d], dva[d]);
        dka[d] = fmaf(ds, qp[d], dka[d]);
      }
      bins[code * kThreads + t] += ds;
    }
  }
  if (valid) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t o = (j * H + h) * D + d;
      dk[o] = acc ? dk[o] + dka[d] * scale : dka[d] * scale;
      dv[o] = acc ? dv[o] + dva[d] : dva[d];
    }
  }
  __syncthreads();
  for (int x = t; x < H * NB; x += kThreads) {
    const int hh = x / NB, b = x - hh * NB;
    float s = 0.f;
    for (int cc = 0; cc < CK; ++cc) s += bins[b * kThreads + cc * H + hh];
    partial[static_cast<int64_t>(blockIdx.x) * H * NB + x] = s;
  }
}

// Backward, step 3 (query-outer): thread (r, h) owns query row i and head h and
// accumulates dQ over all keys. LDS: table*log2e | K tile | V tile | codes [R][BN].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_q_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint8_t* __restrict__ spd, const float* __restrict__ table,
    const float* __restrict__ lse, const float* __restrict__ delta, const T* __restrict__ dout,
    float* __restrict__ dq, int64_t N, int64_t Nk, int64_t ldc, int H, int NB, int BN, float qscale, float scale,
    int acc) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int HD = H * D;
  const int R = kThreads / H;
  float* tb = reinterpret_cast<float*>(smem);
  float* Ks = tb + ((H * NB + 3) & ~3);
  float* Vs = Ks + BN * HD;
  uint8_t* cs = reinterpret_cast<uint8_t*>(Vs + BN * HD);

  const int t = threadIdx.x;
  const int r = t / H, h = t - r * H;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
  const int64_t i = row0 + r;
  const bool valid = (r < R) && (i < N);

  for (int x = t; x < H * NB; x += kThreads) tb[x] = table[x] * kLog2e;
  float qr[D], orr[D], dqa[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = valid ? ld(q, (i * H + h) * D + d) : 0.f;
    orr[d] = valid ? ld(dout, (i * H + h) * D + d) : 0.f;
    dqa[d] = 0.f;
  }
  const float l2 = valid ? lse[i * H + h] * kLog2e : 0.f;
  const float dl = valid ? delta[i * H + h] : 0.f;
  const float* tbh = tb + h * NB;

  for (int64_t j0 = 0; j0 < Nk; j0 += BN) {
    const int nk = static_cast<int>(std::min<int64_t>(BN, Nk - j0));
    __syncthreads();
    for (int x = t; x < BN * HD; x += kThreads) {
      const int jj = x / HD;
      float kx = 0.f, vx = 0.f;
      if (jj < nk) {
        const int64_t g = (j0 + jj) * HD + (x - jj * HD);
        kx = ld(k, g);
        vx = ld(v, g);
      }
      Ks[x] = kx;
      Vs[x] = vx;
    }
    for (int x = t; x < R * BN; x += kThreads) {
      const int rr = x / BN, jj = x - rr * BN;
      const int64_t ii = row0 + rr;
      cs[x] = (ii < N && jj < nk) ? spd[ii * ldc + j0 + jj] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    const uint8_t* crow = cs + r * BN;
    for (int jj = 0; jj < nk; ++jj) {
      const float* kp = Ks + (jj * H + h) * D;
      const float* vp = Vs + (jj * H + h) * D;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dot = fmaf(qr[d], kp[d], dot);
        dp = fmaf(orr[d], vp[d], dp);
      }
      const int code = min(static_cast<int>(crow[jj]), NB - 1);
      const float p = exp2_hw(fmaf(dot, qscale, tbh[code]) - l2);
      const float ds = p * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) dqa[d] = fmaf(ds, kp[d], dqa[d]);
    }
  }
  if (valid) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t o = (i * H + h) * D + d;
      dq[o] = acc ? dq[o] + dqa[d] * scale : dqa[d] * scale;
    }
  }
}

// Backward, step 4: dtable[x] = sum over key blocks of partial[block][x], in block
// order within each thread and a fixed tree across the workgroup (deterministic).
__global__ __launch_bounds__(kThreads) void dtable_reduce_kernel(const float* __restrict__ partial,
                                                                 float* __restrict__ dtable,
                                                                 int64_t nblocks, int HNB, int acc) {
  __shared__ float red[kThreads];
  const int x = blockIdx.x;
  float s = 0.f;
  for (int64_t b = threadIdx.x; b < nblocks; b += kThreads) s += partial[b * HNB + x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dtable[x] = acc ? dtable[x] + red[0] : red[0];
}

// out = (exp(lse_a - lse) out_a + exp(lse_b - lse) out_b), lse = log(exp(lse_a) + exp(lse_b)),
// one thread per (node, head) row of D values; out and lse may alias either input.
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* out_a, const float* lse_a,
                                                         const float* out_b, const float* lse_b, float* out,
                                                         float* lse, int64_t rows, int D) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (r >= rows) return;
  const float la = lse_a[r], lb = lse_b[r];
  const float m = fmaxf(la, lb);
  // a side with lse = -inf (no keys) gets weight 0; both -inf cannot be normalised
  const float wa = la == -INFINITY ? 0.f : expf(la - m);
  const float wb = lb == -INFINITY ? 0.f : expf(lb - m);
  const float sum = wa + wb;
  const float fa = wa / sum, fb = wb / sum;
  for (int d = 0; d < D; d += 4) {
    const float4 a = *reinterpret_cast<const float4*>(out_a + r * D + d);
    const float4 b = *reinterpret_cast<const float4*>(out_b + r * D + d);
    *reinterpret_cast<float4*>(out + r * D + d) =
        make_float4(fa * a.x + fb * b.x, fa * a.y + fb * b.y, fa * a.z + fb * b.z, fa * a.w + fb * b.w);
  }
  lse[r] = m + logf(sum);
}

// out, lse from S partial results over disjoint key ranges (one thread per (node, head)
// row): lse = log sum_s exp(lse_s), out = sum_s exp(lse_s - lse) out_s.
// With acc, out/lse on entry are one more partial result (a running merge); a partial
// with lse = -inf has weight 0.
__global__ __launch_bounds__(kThreads) void merge_splits_kernel(const float* __restrict__ opart,
                                                                const float* __restrict__ lpart, int S,
                                                                float* __restrict__ out, float* __restrict__ lse,
                                                                int64_t rows, int D, int acc) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (r >= rows) return;
  const float l_old = acc ? lse[r] : -INFINITY;
  float m = l_old;
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, lpart[sp * rows + r]);
  float sum = l_old == -INFINITY ? 0.f : expf(l_old - m);
  for (int sp = 0; sp < S; ++sp) sum += expf(lpart[sp * rows + r] - m);
  const float inv = 1.f / sum;
  const float w_old = l_old == -INFINITY ? 0.f : expf(l_old - m) * inv;
  for (int d = 0; d < D; d += 4) {
    float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (w_old != 0.f) {
      const float4 o = *reinterpret_cast<const float4*>(out + r * D + d);
      o4 = make_float4(w_old * o.x, w_old * o.y, w_old * o.z, w_old * o.w);
    }
    for (int sp = 0; sp < S; ++sp) {
      const float wgt = expf(lpart[sp * rows + r] - m) * inv;
      const float4 o = *reinterpret_cast<const float4*>(opart + (sp * rows + r) * D + d);
      o4.x = fmaf(wgt, o.x, o4.x);
      o4.y = fmaf(wgt, o.y, o4.y);
      o4.z = fmaf(wgt, o.z, o4.z);
      o4.w = fmaf(wgt, o.w, o4.w);
    }
    *reinterpret_cast<float4*>(out + r * D + d) = o4;
  }
  lse[r] = m + logf(sum);
}

// The backward's finishing launch after split kernels. Workgroups [0, e0) sum the
// partials of a, [e0, e1) those of b, [e1, e2) those of c (dst = sum over S partial
// arrays of n floats, + dst when acc, four floats per thread, partials in order);
// workgroup e2 + x reduces dtable entry x over the partial rows (as dtable_reduce_kernel).
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(SumSplits a, SumSplits b, SumSplits c, int64_t e0,
                                                              int64_t e1, int64_t e2, const float* __restrict__ partial,
                                                              float* __restrict__ dtable, int64_t nblocks, int HNB,
                                                              int dacc, const uint32_t* __restrict__ gate) {
  if (gate != nullptr && *gate == 0u) return;
  const int64_t bid = blockIdx.x;
  if (bid < e2) {
    // select the descriptor by value (workgroup-uniform)
    const bool in_a = bid < e0, in_b = !in_a && bid < e1;
    const float* part = in_a ? a.part : (in_b ? b.part : c.part);
    float* dst = in_a ? a.dst : (in_b ? b.dst : c.dst);
    const int64_t n = in_a ? a.n : (in_b ? b.n : c.n);
    const int S = in_a ? a.S : (in_b ? b.S : c.S);
    const int acc = in_a ? a.acc : (in_b ? b.acc : c.acc);
    const int64_t b0 = in_a ? 0 : (in_b ? e0 : e1);
    const int64_t x = ((bid - b0) * kThreads + threadIdx.x) * 4;
    if (x >= n) return;
    float4 s = acc ? *reinterpret_cast<const float4*>(dst + x) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < S; ++sp) {
      const float4 p = *reinterpret_cast<const float4*>(part + sp * n + x);
      s.x += p.x;
      s.y += p.y;
      s.z += p.z;
      s.w += p.w;
    }
    *reinterpret_cast<float4*>(dst + x) = s;
    return;
  }
  __shared__ float red[kThreads];
  const int x = static_cast<int>(bid - e2);
  float s = 0.f;
  for (int64_t r = threadIdx.x; r < nblocks; r += kThreads) s += partial[r * HNB + x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dtable[x] = dacc ? dtable[x] + red[0] : red[0];
}

int fwd_tile_keys(int H, int D, int NB) {
  const int HD = H * D;
  int bn = std::max(8, std::min(64, 4096 / HD));
  bn &= ~7;
  const size_t fixed = 4 * ((H * NB + 3) & ~3);
  while (bn > 8 && fixed + 8ull * bn * HD + static_cast<size_t>(kThreads / H) * bn > kLdsDefault)
    bn -= 8;
  return bn;
}

size_t fwd_lds(int H, int D, int NB, int BN) {
  return 4 * ((H * NB + 3) & ~3) + 8ull * BN * H * D + static_cast<size_t>(kThreads / H) * BN;
}

size_t kv_lds(int H, int D, int NB, int BM) {
  const int CK = kThreads / H;
  return 4 * ((H * NB + 3) & ~3) + 4ull * NB * kThreads + 8ull * BM * H * D + 8ull * BM * H +
         static_cast<size_t>(BM) * CK;
}

int kv_tile_rows(int H, int D, int NB) {
  int bm = 32;
  while (bm > 1 && kv_lds(H, D, NB, bm) > kLdsDefault) bm >>= 1;
  return bm;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= kLdsDefault) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

template <typename T, int D>
hipError_t fwd_typed(const FwdArgs& a, hipStream_t s) {
  const int BN = fwd_tile_keys(a.H, D, a.NB);
  const size_t lds = fwd_lds(a.H, D, a.NB, BN);
  const int R = kThreads / a.H;
  const unsigned grid = static_cast<unsigned>((a.N + R - 1) / R);
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
  trace_begin(0, s);
  hipLaunchKernelGGL((fwd_valu_kernel<T, D>), dim3(grid), dim3(kThreads), lds, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.spd, a.table, a.out, a.lse,
                     a.N, a.Nk, a.ld, a.H, a.NB, BN, qscale);
  const hipError_t e = hipGetLastError();
  trace_end(0, s);
  return e;
}

template <typename T, int D>
hipError_t bwd_typed(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  float* delta = reinterpret_cast<float*>(ws + w.delta_off);
  float* partial = reinterpret_cast<float*>(ws + w.partial_off);
  const int64_t NH = a.N * a.H;
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* dout = static_cast<const T*>(a.dout);

  trace_begin(1, s);
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(static_cast<unsigned>((NH + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, a.out, dout, delta, NH);
  hipError_t e = hipGetLastError();
  trace_end(1, s);
  if (e != hipSuccess) return e;

  const int BM = kv_tile_rows(a.H, D, a.NB);
  const size_t lds_kv = kv_lds(a.H, D, a.NB, BM);
  e = allow_lds(bwd_kv_valu_kernel<T, D>, lds_kv);
  if (e != hipSuccess) return e;
  trace_begin(2, s);
  hipLaunchKernelGGL((bwd_kv_valu_kernel<T, D>), dim3(static_cast<unsigned>(w.n_kv_blocks)),
                     dim3(kThreads), lds_kv, s, q, k, v, a.spd, a.table, a.lse, delta, dout, a.dk,
                     a.dv, partial, a.N, a.Nk, a.ld, a.H, a.NB, BM, qscale, scale, a.acc & kAccDkv);
  e = hipGetLastError();
  trace_end(2, s);
  if (e != hipSuccess) return e;

  const int BN = fwd_tile_keys(a.H, D, a.NB);
  const size_t lds_q = fwd_lds(a.H, D, a.NB, BN);
  const int R = kThreads / a.H;
  trace_begin(3, s);
  hipLaunchKernelGGL((bwd_q_valu_kernel<T, D>), dim3(static_cast<unsigned>((a.N + R - 1) / R)),
                     dim3(kThreads), lds_q, s, q, k, v, a.spd, a.table, a.lse, delta, dout, a.dq,
                     a.N, a.Nk, a.ld, a.H, a.NB, BN, qscale, scale, a.acc & kAccDq);
  e = hipGetLastError();
  trace_end(3, s);
  if (e != hipSuccess) return e;

  return launch_dtable_reduce(partial, a.dtable, w.n_kv_blocks, a.H * a.NB, a.acc & kAccDtable, s);
}

template <typename T>
hipError_t fwd_by_d(const FwdArgs& a, hipStream_t s) {
  switch (a.D) {
    case 8: return fwd_typed<T, 8>(a, s);
    case 16: return fwd_typed<T, 16>(a, s);
    case 32: return fwd_typed<T, 32>(a, s);
    default: return fwd_typed<T, 64>(a, s);
  }
}

template <typename T>
hipError_t bwd_by_d(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
  switch (a.D) {
    case 8: return bwd_typed<T, 8>(a, w, s);
    case 16: return bwd_typed<T, 16>(a, w, s);
    case 32: return bwd_typed<T, 32>(a, w, s);
    default: return bwd_typed<T, 64>(a, w, s);
  }
}

}  // namespace

int64_t valu_kv_block(int H) { return kThreads / H; }

hipError_t launch_dtable_reduce(const float* partial, float* dtable, int64_t nblocks, int HNB, int acc,
                                hipStream_t s) {
  trace_begin(kTraceBwdDtable, s);
  hipLaunchKernelGGL(dtable_reduce_kernel, dim3(static_cast<unsigned>(HNB)), dim3(kThreads), 0, s, partial,
                     dtable, nblocks, HNB, acc);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceBwdDtable, s);
  return e;
}

hipError_t launch_merge_splits(const float* opart, const float* lpart, int S, float* out, float* lse, int64_t rows,
                               int D, int acc, hipStream_t s) {
  trace_begin(kTraceFwdSplits, s);
  hipLaunchKernelGGL(merge_splits_kernel, dim3(static_cast<unsigned>((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, opart, lpart, S, out, lse, rows, D, acc);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceFwdSplits, s);
  return e;
}

hipError_t launch_bwd_finish(const SumSplits& a, const SumSplits& b, const SumSplits& c, const float* partial,
                             float* dtable, int64_t nblocks, int HNB, int dacc, hipStream_t s, const uint32_t* gate) {
  auto blocks = [](const SumSplits& g) { return g.S > 0 ? (g.n / 4 + kThreads - 1) / kThreads : 0; };
  const int64_t e0 = blocks(a), e1 = e0 + blocks(b), e2 = e1 + blocks(c);
  trace_begin(kTraceBwdSplits, s);
  hipLaunchKernelGGL(bwd_finish_kernel, dim3(static_cast<unsigned>(e2 + HNB)), dim3(kThreads), 0, s, a, b, c, e0, e1,
                     e2, partial, dtable, nblocks, HNB, dacc, gate);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceBwdSplits, s);
  return e;
}

hipError_t launch_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b, float* out,
                        float* lse, int64_t rows, int D, hipStream_t s) {
  trace_begin(kTraceMerge, s);
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>((rows + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, out_a, lse_a, out_b, lse_b, out, lse, rows, D);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceMerge, s);
  return e;
}

hipError_t launch_fwd_valu(const FwdArgs& a0, hipStream_t s) {
  FwdArgs a = a0;
  if (a0.acc) {  // partial result into the workspace, then merged into out/lse
    a.out = static_cast<float*>(a0.workspace);
    a.lse = a.out + a0.N * a0.H * a0.D;
  }
  const hipError_t e = a.dtype == 0 ? fwd_by_d<float>(a, s) : fwd_by_d<uint16_t>(a, s);
  if (e != hipSuccess || !a0.acc) return e;
  return launch_merge_splits(a.out, a.lse, 1, a0.out, a0.lse, a0.N * a0.H, a0.D, 1, s);
}

hipError_t launch_bwd_valu(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
  return a.dtype == 0 ? bwd_by_d<float>(a, w, s) : bwd_by_d<uint16_t>(a, w, s);
}

}  // namespace gt
