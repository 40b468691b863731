// Biased attention on the bf16 matrix cores (gfx950 MFMA): head dimension 8, bf16
// inputs, float32 accumulation and outputs.
//
// MegaGraph pages, abstract: the score matrix and the topology-aware bias matrix are
// what make full-graph attention expensive; Fig. 4 caption: work proceeds over key
// blocks with the bias columns sliced to each block. Neither matrix exists here
// outside registers: each 32x32 score tile of a head is one MFMA whose accumulator
// starts from the tile's bias, table[h, code] read from LDS by the uint8 code, so
// adding the bias costs no vector instruction.
//
// Work split: one 64-lane wave per workgroup owns 32 nodes of the outer loop and two
// heads (blockIdx.y selects the head pair). Lane l holds column c = l % 32 of every
// 32x32 tile and one half hp = l / 32 of its rows.
//
// Row order inside a 32-row tile: MFMA row r stands for node offset
//     a(r) = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3),
// so the 16 accumulator entries of lane half hp are exactly offsets 16*hp + 0..15.
// The lane's codes are then one contiguous 16-byte load, and each 8-entry half of
// its accumulator is directly a bf16 operand of the 32x32x16 MFMA that contracts
// over those nodes, whose other operand is read as 8 consecutive nodes of a
// transposed [d][node] tile in LDS.
//
// Table in LDS: for each of the wave's two heads, 256 floats: entry b holds
// table[h, min(b, NB-1)] * sqrt(D), so every byte value indexes it without a clamp.
#include "gt_internal.h"

#include <algorithm>

namespace gt {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kD = 8;
constexpr int kH = 8;
constexpr int kHD = kH * kD;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int node_of_row(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// 16 consecutive codes of one row starting at column col; zero past column `limit`.
template <bool kAligned>
__device__ __forceinline__ u32x4 load_codes16(const uint8_t* row, int64_t col, int64_t limit) {
  if (kAligned && col + 16 <= limit) return *reinterpret_cast<const u32x4*>(row + col);
  u32x4 r = {0u, 0u, 0u, 0u};
  for (int b = 0; b < 16; ++b) {
    const uint32_t x = (col + b < limit) ? row[col + b] : 0u;
    r[b >> 2] |= x << (8 * (b & 3));
  }
  return r;
}

__device__ __forceinline__ uint32_t code_byte(const u32x4& cw, int v) { return (cw[v >> 2] >> (8 * (v & 3))) & 0xffu; }

// Four bf16 of one (node, head) row at d = 4*hp .. 4*hp+3, or zeros past N.
__device__ __forceinline__ s16x4 load_op4(const uint16_t* base, int64_t node, int64_t N, int h, int hp) {
  if (node < N) return *reinterpret_cast<const s16x4*>(base + node * kHD + h * kD + 4 * hp);
  return s16x4{0, 0, 0, 0};
}

__device__ __forceinline__ s16x8 pack_bf16x8(const f32x16& a, int first) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(a[first + e]);
  return __builtin_bit_cast(s16x8, r);
}

__device__ __forceinline__ f32x16 mfma_x8(s16x4 a, s16x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_x16(s16x8 a, s16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
}

// Stage the transposed tile T[hl][d][0..31] (bf16) of nodes n0..n0+31 for the wave's
// heads h0, h0+1 from a node-major [N][H][D] bf16 tensor: lane (hl, group g of 4 nodes,
// d-pair dp) loads 4 dwords and packs them into two 8-byte rows of the tile.
__device__ __forceinline__ void stage_transposed(uint16_t* tile, const uint16_t* src, int64_t n0,
                                                 int64_t N, int h0, int lane) {
  const int hl = lane >> 5, g = (lane >> 2) & 7, dp = lane & 3;
  uint32_t w[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t n = n0 + 4 * g + r;
    w[r] = n < N ? *reinterpret_cast<const uint32_t*>(src + n * kHD + (h0 + hl) * kD + 2 * dp) : 0u;
  }
  // low halves are d = 2dp, high halves d = 2dp+1
  const u32x2 lo = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u)};
  const u32x2 hi = {__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
  *reinterpret_cast<u32x2*>(tile + (hl * kD + 2 * dp) * 32 + 4 * g) = lo;
  *reinterpret_cast<u32x2*>(tile + (hl * kD + 2 * dp + 1) * 32 + 4 * g) = hi;
}

// A operand of the contraction over 8 nodes: rows m < 8 are T[hl][m][first..first+7];
// row 8 is all ones when `ones_row` (it yields the row sums); other rows are zero.
__device__ __forceinline__ s16x8 read_operand_t(const uint16_t* tile, int hl, int m, int first, bool ones_row) {
  if (m < kD) return *reinterpret_cast<const s16x8*>(tile + (hl * kD + m) * 32 + first);
  const short one = ones_row && m == kD ? static_cast<short>(0x3F80) : static_cast<short>(0);
  return s16x8{one, one, one, one, one, one, one, one};
}

// ---------------------------------------------------------------------------------
// Forward. S^T = K Q^T per 32-key tile (rows = keys in the order above, columns =
// queries); running max and sum per query column; O^T += V^T P^T with a ones row in
// V^T so the MFMA also accumulates the row sum l.
template <bool kAligned>
__global__ __launch_bounds__(64) void fwd_mfma_d8_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint8_t* __restrict__ spd,
                                                         const float* __restrict__ table,
                                                         float* __restrict__ out, float* __restrict__ lse,
                                                         int64_t N, int NB) {
  __shared__ float tb[2 * 256];
  __shared__ __align__(16) uint16_t vt[2 * kD * 32];
  const int lane = threadIdx.x;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * blockIdx.y;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int64_t i = i0 + c;
  const bool qvalid = i < N;
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int x = lane; x < 512; x += 64) {
    const int hl = x >> 8, b = x & 255;
    tb[x] = table[(h0 + hl) * NB + min(b, NB - 1)] * sqd;
  }
  const s16x4 qop0 = load_op4(q, qvalid ? i : N, N, h0, hp);
  const s16x4 qop1 = load_op4(q, qvalid ? i : N, N, h0 + 1, hp);
  const uint8_t* srow = spd + (qvalid ? i : 0) * N;

  f32x16 o0 = {}, o1 = {};
  float m0 = -INFINITY, m1 = -INFINITY;
  const int kr = node_of_row(c);  // the key this lane feeds as A-operand row c

  for (int64_t j0 = 0; j0 < N; j0 += 32) {
    const bool tail = j0 + 32 > N;
    const u32x4 cw = qvalid ? load_codes16<kAligned>(srow, j0 + 16 * hp, N) : u32x4{0u, 0u, 0u, 0u};
    const s16x4 kop0 = load_op4(k, j0 + kr, N, h0, hp);
    const s16x4 kop1 = load_op4(k, j0 + kr, N, h0 + 1, hp);
    __syncthreads();
    stage_transposed(vt, v, j0, N, h0, lane);
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t cb = code_byte(cw, e);
      s0[e] = tb[cb];
      s1[e] = tb[256 + cb];
    }
    s0 = mfma_x8(kop0, qop0, s0);
    s1 = mfma_x8(kop1, qop1, s1);
    if (tail) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (j0 + 16 * hp + e >= N) {
          s0[e] = -INFINITY;
          s1[e] = -INFINITY;
        }
      }
    }
    float x0 = s0[0], x1 = s1[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      x0 = fmaxf(x0, s0[e]);
      x1 = fmaxf(x1, s1[e]);
    }
    x0 = fmaxf(x0, __shfl_xor(x0, 32));
    x1 = fmaxf(x1, __shfl_xor(x1, 32));
    const float n0 = fmaxf(m0, x0), n1 = fmaxf(m1, x1);
    if (n0 > m0) {
      const float a0 = __builtin_amdgcn_exp2f((m0 - n0) * sc2);
#pragma unroll
      for (int e = 0; e < 5; ++e) o0[e] *= a0;
      m0 = n0;
    }
    if (n1 > m1) {
      const float a1 = __builtin_amdgcn_exp2f((m1 - n1) * sc2);
#pragma unroll
      for (int e = 0; e < 5; ++e) o1[e] *= a1;
      m1 = n1;
    }
    const float b0 = -m0 * sc2, b1 = -m1 * sc2;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, b0));
      s1[e] = __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, b1));
    }
    __syncthreads();
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1) {
      const s16x8 va = read_operand_t(vt, 0, c, 16 * hp + 8 * k1, true);
      const s16x8 vb = read_operand_t(vt, 1, c, 16 * hp + 8 * k1, true);
      o0 = mfma_x16(va, pack_bf16x8(s0, 8 * k1), o0);
      o1 = mfma_x16(vb, pack_bf16x8(s1, 8 * k1), o1);
    }
  }
  // O^T rows: d = 4hp + e in entries e = 0..3; row 8 (lane half 0, entry 4) is l.
  const float l0 = __shfl(o0[4], c), l1 = __shfl(o1[4], c);
  if (qvalid) {
    float* op = out + i * kHD + h0 * kD + 4 * hp;
    const float r0 = 1.f / l0, r1 = 1.f / l1;
    *reinterpret_cast<float4*>(op) = make_float4(o0[0] * r0, o0[1] * r0, o0[2] * r0, o0[3] * r0);
    *reinterpret_cast<float4*>(op + kD) = make_float4(o1[0] * r1, o1[1] * r1, o1[2] * r1, o1[3] * r1);
    if (hp == 0) {
      lse[i * kH + h0] = (m0 * sc2 + log2f(l0)) * kLn2;
      lse[i * kH + h0 + 1] = (m1 * sc2 + log2f(l1)) * kLn2;
    }
  }
}

}  // namespace

bool mfma_supported(int H, int D, int dtype) { return H == kH && D == kD && dtype == 1; }

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.N + 31) / 32), kH / 2);
  trace_begin(0, s);
  if (a.N % 16 == 0)
    hipLaunchKernelGGL(fwd_mfma_d8_kernel<true>, grid, dim3(64), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table,
                       a.out, a.lse, a.N, a.NB);
  else
    hipLaunchKernelGGL(fwd_mfma_d8_kernel<false>, grid, dim3(64), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table,
                       a.out, a.lse, a.N, a.NB);
  const hipError_t e = hipGetLastError();
  trace_end(0, s);
  return e;
}

}  // namespace gt
