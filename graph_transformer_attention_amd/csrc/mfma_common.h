// Helpers shared by the matrix-core (MFMA) attention kernels for gfx950: operand
// types, the row order of a 32x32 MFMA tile, code loads, half-precision packing,
// the MFMA wrappers and the XCD-aware workgroup order.
#pragma once

#include "gt_internal.h"

namespace gt {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Running-max slack of the forward's lazy rescale, in log2 units.
constexpr float kLazy = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Row order inside a 32-row MFMA tile: row r stands for node offset
//     a(r) = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3),
// so the 16 accumulator entries of lane half hp = l / 32 are exactly the node offsets
// 16*hp + 0..15. A lane's codes for those nodes are then one contiguous 16-byte load,
// and each 8-entry half of its accumulator is directly an operand of the 32x32x16
// MFMA that contracts over those nodes.
__device__ __forceinline__ int node_of_row(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

__host__ __device__ constexpr int slot_of_node(int n) {  // inverse of node_of_row
  return (((n >> 2) & 3) << 3) | (((n >> 4) & 1) << 2) | (n & 3);
}
// Position (halves) of 16-byte chunk `chunk` of 64-byte row `row` in an LDS tile whose
// chunks are XOR-swizzled so that 8 lanes reading rows 0..7 at one chunk index hit 8
// distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 32 + 8 * (chunk ^ ((row >> 1) & 3)); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). Issued once before a
// software-pipelined loop: with a load of the first tile still pending at loop entry,
// the compiler's wait analysis would otherwise merge that state into the loop header
// and wait for every outstanding load (the next tile's prefetch included) at the top
// of each iteration.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// 16 codes of one row from column col (col is a multiple of 16); kGuard zero-fills past N.
template <bool kGuard, bool kAligned>
__device__ __forceinline__ u32x4 codes_at(const uint8_t* row, int64_t col, int64_t N) {
  if (kGuard || !kAligned) return load_codes16<false>(row, col, N);
  return *reinterpret_cast<const u32x4*>(row + col);
}

__device__ __forceinline__ s16x8 pack_f16x8(const f32x16& a, int first) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<_Float16>(a[first + e]);
  return __builtin_bit_cast(s16x8, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two bf16 in one dword -> two halves in one dword (same element order).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r = {static_cast<_Float16>(bf16_lo(w)), static_cast<_Float16>(bf16_hi(w))};
  return __builtin_bit_cast(uint32_t, r);
}

// Half precision for the backward's operand copies, with overflow turned into NaN: a
// value at or beyond half's range (|x| >= 65520 rounds to infinity) would otherwise
// become an infinity that can vanish from a product (exp2(-inf) = 0 makes a whole row's
// probabilities 0) and leave finite, wrong gradients. NaN reaches every output it
// touches instead.
__device__ __forceinline__ _Float16 to_half_or_nan(float x) {
  return fabsf(x) < 65520.0f ? static_cast<_Float16>(x) : static_cast<_Float16>(__builtin_nanf(""));
}
__device__ __forceinline__ uint16_t half_bits_or_nan(float x) { return __builtin_bit_cast(uint16_t, to_half_or_nan(x)); }
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_or_nan(uint32_t w) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r = {to_half_or_nan(bf16_lo(w)), to_half_or_nan(bf16_hi(w))};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma_h16(s16x8 a, s16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_b16(s16x8 a, s16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ s16x8 load_h8(const uint16_t* p) { return *reinterpret_cast<const s16x8*>(p); }

// Epilogue store of four float results: overwrite, or add into what is there (acc).
__device__ __forceinline__ void store4(float* p, float4 x, int acc) {
  if (acc) {
    const float4 o = *reinterpret_cast<const float4*>(p);
    x = make_float4(o.x + x.x, o.y + x.y, o.z + x.z, o.w + x.w);
  }
  *reinterpret_cast<float4*>(p) = x;
}

// Workgroup -> (node block, head pair) mapping. Workgroups are dispatched round-robin
// over the 8 XCDs (each with its own L2). The 4 head pairs of one node block read
// the same code rows, so they are placed on one XCD, in consecutive dispatch slots.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_map(int wg, int nblocks, int& blk, int& hpair) {
  const int xcd = wg % kXcds, slot = wg / kXcds;
  hpair = slot & 3;
  blk = (slot >> 2) * kXcds + xcd;
  if (blk >= nblocks) blk = -1;  // padding workgroup (grid rounded up to whole groups)
}
__host__ __device__ constexpr int xcd_grid(int nblocks) {
  return ((nblocks + kXcds - 1) / kXcds) * kXcds * 4;
}

template <typename K>
hipError_t allow_lds_mfma(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

}  // namespace
}  // namespace gt
