// Biased attention on the gfx950 matrix cores (MFMA) for head dimension 32, 8 heads,
// bfloat16 inputs, float32 accumulation and outputs.
//
// MegaGraph pages, abstract: the score matrix and the topology-aware bias matrix make
// full-graph attention expensive; Fig. 4 caption: work proceeds over key blocks with
// the bias columns sliced to each block. As at D = 8, neither matrix is stored: each
// 32x32 score tile of a head starts its MFMA accumulator from table[h, code] read from
// LDS, and the contractions over D (QK^T, dO V^T) and over nodes (PV, P^T dO, dS^T Q,
// dS K) run on 32x32x16 MFMAs, all 32 accumulator rows carrying head dimensions.
//
// Precision as at D = 8: QK^T multiplies the bf16 inputs exactly (bf16 MFMA in the
// forward, inputs converted exactly to half in the backward), P and dS enter the
// contractions over nodes as IEEE half, lse*sqrt(D) and delta enter the backward's
// score MFMAs split into two halves (an extra 16-deep contraction chunk).
//
// Work split: 4-wave workgroups over 128 nodes of one head pair (xcd_map); lane l
// holds column l % 32 of every tile and half l / 32 of its rows in the order of
// node_of_row.
#include "mfma_common.h"

#include <algorithm>
#include <type_traits>

namespace gt {
namespace {

constexpr int kD = 32;
constexpr int kH = 8;
constexpr int kHD = kH * kD;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------------
// Staged tiles: one 32-node tile of a head pair, 16-byte chunks (the forward stages
// k as a row tile, the backward its operand copies):
//   row tile      [slot][head][32] half, slot s holding node a(s): 32 rows of 128 bytes,
//                 chunk k of row s stored at chunk position k ^ rswz(s)
// The swizzle gives the 8 (or 16) lanes of one LDS cycle distinct bank groups when they
// read consecutive rows at one chunk index: t = (s >> 1) & 7, with bit 2 flipped when
// bit 0 is set (a permutation of 0..7). The backward also reads row tiles transposed
// (ds_read_b64_tr_b16), 4 consecutive slots s0..s0+3 (s0 a multiple of 4) at a time; the
// flip moves slots s0+2 and s0+3 to the other head's half of the row, so those reads
// cover all 64 banks once.
constexpr int kRowTile = 32 * 2 * kD;  // halves

__device__ __forceinline__ int rswz(int s) {
  const int t = (s >> 1) & 7;
  return t ^ ((t & 1) << 2);
}
__device__ __forceinline__ int row_pos(int slot, int chunk) { return slot * 64 + 8 * (chunk ^ rswz(slot)); }

// global chunk x of a row tile: node = x >> 3, chunk = x & 7 (head = chunk >> 2, 8 halves of d)
__device__ __forceinline__ const uint16_t* row_src(const uint16_t* base, int64_t n0, int h0, int x) {
  return base + ((n0 + (x >> 3)) * kH + h0) * kD + 8 * (x & 7);
}
// Row tile operand of MFMA row c (node a(c)): head hl, d chunk ci (16 wide), half hp.
__device__ __forceinline__ s16x8 row_op(const uint16_t* tile, int c, int hl, int ci, int hp) {
  return load_h8(tile + row_pos(c, 4 * hl + 2 * ci + hp));
}

// ---------------------------------------------------------------------------------
// Forward: per 32-key tile, S^T = K Q^T (two bf16 MFMAs over D), online softmax per
// query column, O^T += V^T P^T (two half MFMAs over the tile's keys). The row sum l
// is accumulated on the vector ALU (all 32 rows of V^T are head dimensions). The 4 waves
// of a workgroup share each key tile: its k rows are staged in LDS as a row tile (one
// 16-byte chunk per thread, read back as the MFMA operands of every wave), and V^T as
// half, rows of 40 halves (80 bytes) so that the 16 lanes of an LDS cycle reading rows
// d..d+15 hit distinct banks.
constexpr int kVtRow = 40;
constexpr int kVtHead = kD * kVtRow;  // halves per head in one buffer

struct FwdTileD32 {
  u32x4 cw;           // 16 codes: query row, keys 16*hp .. 16*hp+15 of the tile
  s16x8 ks;           // staging: chunk tid of the tile's k row tile
  u32x2 va, vb;       // staging: 4 d values of keys 2kp and 2kp+1 (bf16)
};

template <bool kGuard, bool kAligned>
__device__ __forceinline__ void fwd_load_d32(FwdTileD32& t, const uint8_t* srow, const uint16_t* k,
                                             const uint16_t* v, int64_t j0, int64_t N, int h0, int hp, int tid,
                                             int shl, int sdq, int skp) {
  t.cw = codes_at<kGuard, kAligned>(srow, j0 + 16 * hp, N);
  t.ks = (!kGuard || j0 + (tid >> 3) < N) ? load_h8(row_src(k, j0, h0, tid)) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t v0 = j0 + 2 * skp, v1 = v0 + 1;
  const uint16_t* vp = v + (h0 + shl) * kD + 4 * sdq;
  t.va = (!kGuard || v0 < N) ? *reinterpret_cast<const u32x2*>(vp + v0 * kHD) : u32x2{0u, 0u};
  t.vb = (!kGuard || v1 < N) ? *reinterpret_cast<const u32x2*>(vp + v1 * kHD) : u32x2{0u, 0u};
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void fwd_mfma_d32_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                const uint8_t* __restrict__ spd,
                                                                const float* __restrict__ table,
                                                                float* __restrict__ out, float* __restrict__ lse,
                                                                int64_t N, int64_t Nk, int64_t ldc, int NB,
                                                                int64_t kchunk, int64_t ostride, int64_t lstride) {
  __shared__ float2 tb[256];  // both heads' bias for each byte value (forward: * sqrt(D), query-outer: * log2e)
  __shared__ __align__(16) uint16_t vt[2][2 * kVtHead];  // [buffer][head][d][key], rows of kVtRow
  __shared__ __align__(16) uint16_t kt[2][kRowTile];     // [buffer] k row tile
  // workgroup row y of a split launch: keys [y*kchunk, min(Nk, (y+1)*kchunk)), partial
  // results at out + y*ostride, lse + y*lstride
  {
    const int64_t jb = static_cast<int64_t>(blockIdx.y) * kchunk;
    k += jb * kHD;
    v += jb * kHD;
    spd += jb;
    Nk = Nk - jb < kchunk ? Nk - jb : kchunk;
    out += blockIdx.y * ostride;
    lse += blockIdx.y * lstride;
  }
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int c = lane & 31, hp = lane >> 5;
  const int nqb = static_cast<int>((N + 32 * kWaves - 1) / (32 * kWaves));
  int qb, hpair;
  xcd_map(blockIdx.x, nqb, qb, hpair);
  if (qb < 0) return;
  const int h0 = 2 * hpair;
  const int64_t i = static_cast<int64_t>(qb) * (32 * kWaves) + 32 * w + c;
  const bool qvalid = i < N;
  const int64_t irow = qvalid ? i : N - 1;
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < 256; b += kThreads) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * sqd, table[(h0 + 1) * NB + c] * sqd);
  }
  s16x8 qop[2][2];
#pragma unroll
  for (int hl = 0; hl < 2; ++hl)
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
      qop[hl][ci] = qvalid ? load_h8(q + i * kHD + (h0 + hl) * kD + 16 * ci + 8 * hp)
                           : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* srow = spd + irow * ldc;
  // staging role: head shl, d quad sdq (d = 4*sdq .. +3), key pair skp (keys 2*skp, 2*skp+1)
  const int shl = tid >> 7, sdq = (tid >> 4) & 7, skp = tid & 15;
  auto stage = [&](int buf, const u32x2& va, const u32x2& vb) {
    // halves of (key 2skp, key 2skp+1) for each of the four d values
    const uint32_t a0 = bf16x2_to_f16x2(va[0]), a1 = bf16x2_to_f16x2(va[1]);
    const uint32_t b0 = bf16x2_to_f16x2(vb[0]), b1 = bf16x2_to_f16x2(vb[1]);
    uint32_t* base = reinterpret_cast<uint32_t*>(&vt[buf][shl * kVtHead + (4 * sdq) * kVtRow + 2 * skp]);
    constexpr int kRowWords = kVtRow / 2;
    base[0 * kRowWords] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
    base[1 * kRowWords] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
    base[2 * kRowWords] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
    base[3 * kRowWords] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
  };
  // k row tile: thread tid moves chunk tid (node tid >> 3, chunk tid & 7) to its row slot
  const int kpos = row_pos(slot_of_node(tid >> 3), tid & 7);
  auto stage_k = [&](int buf, const s16x8& ks) { *reinterpret_cast<s16x8*>(&kt[buf][kpos]) = ks; };

  const int ntiles = static_cast<int>((Nk + 31) / 32), nfull = static_cast<int>(Nk / 32);  // scalar loop tests
  FwdTileD32 cur, nxt;
  if (nfull > 0)
    fwd_load_d32<false, kAligned>(cur, srow, k, v, 0, Nk, h0, hp, tid, shl, sdq, skp);
  else
    fwd_load_d32<true, kAligned>(cur, srow, k, v, 0, Nk, h0, hp, tid, shl, sdq, skp);
  stage(0, cur.va, cur.vb);
  stage_k(0, cur.ks);
  wait_vm0();
  __syncthreads();

  f32x16 o0 = {}, o1 = {};
  // nb0, nb1: the softmax shift of both heads as the exp2 argument's addend,
  // -m * log2(e)/sqrt(D) for the running max m of the raw scores (set by the first tile);
  // l0, l1: this lane half's share of the row sums, in float32 from the unrounded P (a sum
  // of the half-precision P would carry their rounding into lse).
  float nb0 = 0.f, nb1 = 0.f, l0 = 0.f, l1 = 0.f;
  auto tile = [&](int t, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    const int64_t j0 = static_cast<int64_t>(t) * 32;
    const int buf = t & 1;
    if (t + 1 < nfull)
      fwd_load_d32<false, kAligned>(nxt, srow, k, v, j0 + 32, Nk, h0, hp, tid, shl, sdq, skp);
    else if (t + 1 < ntiles)
      fwd_load_d32<true, kAligned>(nxt, srow, k, v, j0 + 32, Nk, h0, hp, tid, shl, sdq, skp);
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float2 t = tb[code_byte(cur.cw, e)];
      s0[e] = t.x;
      s1[e] = t.y;
    }
    s0 = mfma_b16(row_op(kt[buf], c, 0, 0, hp), qop[0][0], s0);
    s1 = mfma_b16(row_op(kt[buf], c, 1, 0, hp), qop[1][0], s1);
    s0 = mfma_b16(row_op(kt[buf], c, 0, 1, hp), qop[0][1], s0);
    s1 = mfma_b16(row_op(kt[buf], c, 1, 1, hp), qop[1][1], s1);
    if (t >= nfull) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (j0 + 16 * hp + e >= Nk) {
          s0[e] = -INFINITY;
          s1[e] = -INFINITY;
        }
      }
    }
    if constexpr (kFirst) {  // the shift starts at the query column's largest score of this tile
      float x0 = s0[0], x1 = s1[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) {
        x0 = fmaxf(x0, s0[e]);
        x1 = fmaxf(x1, s1[e]);
      }
      nb0 = -fmaxf(x0, __shfl_xor(x0, 32)) * sc2;
      nb1 = -fmaxf(x1, __shfl_xor(x1, 32)) * sc2;
    }
    // exp2 arguments against the current shift
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = fmaf(s0[e], sc2, nb0);
      s1[e] = fmaf(s1[e], sc2, nb1);
    }
    if constexpr (!kFirst) {
      // The lazy running max, tested on the arguments: one above kLazy is a score that far
      // above the shift. Each lane tests its own 16 keys; the two lane halves of a query
      // column are combined only on the rare rescale path.
      float x0 = s0[0], x1 = s1[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) {
        x0 = fmaxf(x0, s0[e]);
        x1 = fmaxf(x1, s1[e]);
      }
      if (__builtin_expect(__any(x0 > kLazy || x1 > kLazy), 0)) {  // rare: keep it a branch
        // the shift rises by d to the column's largest score (whose argument becomes 0)
        const float d0 = fmaxf(fmaxf(x0, __shfl_xor(x0, 32)), 0.f);
        const float d1 = fmaxf(fmaxf(x1, __shfl_xor(x1, 32)), 0.f);
        const float a0 = __builtin_amdgcn_exp2f(-d0), a1 = __builtin_amdgcn_exp2f(-d1);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          o0[e] *= a0;
          o1[e] *= a1;
          s0[e] -= d0;
          s1[e] -= d1;
        }
        l0 *= a0;
        l1 *= a1;
        nb0 -= d0;
        nb1 -= d1;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = __builtin_amdgcn_exp2f(s0[e]);
      s1[e] = __builtin_amdgcn_exp2f(s1[e]);
      l0 += s0[e];
      l1 += s1[e];
    }
    const uint16_t* vb0 = &vt[buf][c * kVtRow + 16 * hp];
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1) {
      o0 = mfma_h16(load_h8(vb0 + 8 * k1), pack_f16x8(s0, 8 * k1), o0);
      o1 = mfma_h16(load_h8(vb0 + kVtHead + 8 * k1), pack_f16x8(s1, 8 * k1), o1);
    }
    if (t + 1 < ntiles) {
      stage(buf ^ 1, nxt.va, nxt.vb);
      stage_k(buf ^ 1, nxt.ks);
      cur = nxt;
    }
    __syncthreads();
  };
  tile(0, std::true_type{});
  for (int t = 1; t < ntiles; ++t) tile(t, std::false_type{});
  // each lane half summed its 16 keys of every tile
  l0 += __shfl_xor(l0, 32);
  l1 += __shfl_xor(l1, 32);
  if (qvalid) {
    // O^T rows held by this lane: d = 8*j + 4*hp + (0..3), entries 4*j .. 4*j+3
    const float r0 = 1.f / l0, r1 = 1.f / l1;
    float* op0 = out + i * kHD + h0 * kD + 4 * hp;
    float* op1 = op0 + kD;
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      *reinterpret_cast<float4*>(op0 + 8 * jq) =
          make_float4(o0[4 * jq] * r0, o0[4 * jq + 1] * r0, o0[4 * jq + 2] * r0, o0[4 * jq + 3] * r0);
      *reinterpret_cast<float4*>(op1 + 8 * jq) =
          make_float4(o1[4 * jq] * r1, o1[4 * jq + 1] * r1, o1[4 * jq + 2] * r1, o1[4 * jq + 3] * r1);
    }
    if (hp == 0) {
      lse[i * kH + h0] = (log2f(l0) - nb0) * kLn2;
      lse[i * kH + h0 + 1] = (log2f(l1) - nb1) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------------
// Backward operand copies, written once per call: query-side arrays (q, dout, lse,
// delta) for the N queries rounded up to 32 (npq), key-side arrays (k, v) for the Nk
// keys rounded up to 32 (npk); padded rows are zero:
//   qd, kd, vd, od   [node][head][32] half      q, k, v, dout (the contractions over
//                                               nodes read them transposed from their
//                                               staged row tiles)
//   lq, dl           [head][node] two halves    (-L_hi, -L_lo), L = lse*sqrt(D), and
//                                               (-delta_hi, -delta_lo), delta = <dout, out>
// The score MFMAs contract over 48: the 32 head dimensions, then a chunk holding
// [-L_hi, -L_lo, 1, 0...] on the query side against [1, 1, pen, 0...] on the key
// side (pen = -inf for padded keys), so S comes out as q.k - lse*sqrt(D); likewise
// [-delta_hi, -delta_lo, 0...] against [1, 1, 0...] gives dout.v - delta. Padded
// queries get -L_hi = -inf.
struct OpsD32 {
  uint16_t *qd, *kd, *vd, *od;
  uint32_t *lq, *dl;
  int64_t npq, npk;
};

// half bits of a constant (exact: 1, -inf); data go through half_bits_or_nan
__device__ __forceinline__ uint16_t hbits(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

__global__ __launch_bounds__(256) void bwd_prep_mfma_d32_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                const float* __restrict__ out,
                                                                const uint16_t* __restrict__ dout,
                                                                const float* __restrict__ lse, OpsD32 ops,
                                                                int64_t N, int64_t Nk, uint32_t* __restrict__ flag) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x == 0) *flag = 0u;  // the key-outer pass's code-range flag starts clear
  const int64_t nmax = ops.npq > ops.npk ? ops.npq : ops.npk;
  if (x >= nmax * kH) return;
  const int h = static_cast<int>(x / nmax);
  const int64_t n = x - h * nmax;
  const int64_t row = (n * kH + h) * kD;
  const uint16_t ninf = hbits(-INFINITY);
  // One node's row of 32 bf16 values -> half row; with o given, also returns <row, o's row>.
  auto copy = [&](const uint16_t* src, uint16_t* dst, const float* o) {
    float dot = 0.f;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const u32x4 wv = *reinterpret_cast<const u32x4*>(src + row + 8 * part);
      u32x4 hv;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) hv[wi] = bf16x2_to_f16x2_or_nan(wv[wi]);
      *reinterpret_cast<u32x4*>(dst + row + 8 * part) = hv;
      if (o != nullptr) {
        const float4 oa = *reinterpret_cast<const float4*>(o + row + 8 * part);
        const float4 ob = *reinterpret_cast<const float4*>(o + row + 8 * part + 4);
        dot = fmaf(bf16_lo(wv[0]), oa.x, dot);
        dot = fmaf(bf16_hi(wv[0]), oa.y, dot);
        dot = fmaf(bf16_lo(wv[1]), oa.z, dot);
        dot = fmaf(bf16_hi(wv[1]), oa.w, dot);
        dot = fmaf(bf16_lo(wv[2]), ob.x, dot);
        dot = fmaf(bf16_hi(wv[2]), ob.y, dot);
        dot = fmaf(bf16_lo(wv[3]), ob.z, dot);
        dot = fmaf(bf16_hi(wv[3]), ob.w, dot);
      }
    }
    return dot;
  };
  auto zero = [&](uint16_t* dst) {
#pragma unroll
    for (int part = 0; part < 4; ++part) *reinterpret_cast<u32x4*>(dst + row + 8 * part) = u32x4{0u, 0u, 0u, 0u};
  };
  if (n < ops.npq) {
    const int64_t lrow = static_cast<int64_t>(h) * ops.npq + n;
    if (n < N) {
      copy(q, ops.qd, nullptr);
      const float delta = copy(dout, ops.od, out);
      const float L = lse[n * kH + h] * sqrtf(static_cast<float>(kD));
      const _Float16 lh = to_half_or_nan(L);
      ops.lq[lrow] = pack2(hbits(-static_cast<float>(lh)), half_bits_or_nan(-(L - static_cast<float>(lh))));
      const _Float16 dh = to_half_or_nan(delta);
      ops.dl[lrow] = pack2(hbits(-static_cast<float>(dh)), half_bits_or_nan(-(delta - static_cast<float>(dh))));
    } else {
      zero(ops.qd);
      zero(ops.od);
      ops.lq[lrow] = pack2(ninf, 0);
      ops.dl[lrow] = 0u;
    }
  }
  if (n < ops.npk) {
    if (n < Nk) {
      copy(k, ops.kd, nullptr);
      copy(v, ops.vd, nullptr);
    } else {
      zero(ops.kd);
      zero(ops.vd);
    }
  }
}

// A tile set: kRows row tiles of 256 chunks each, so thread tid (of kThreads = 256)
// moves chunk tid of every tile.
template <int kRows>
struct StageSetD32 {
  static constexpr int kPer = kRows;
  static constexpr int kHalves = kRows * kRowTile;
  const uint16_t* rows[kRows];
  int h0;

  __device__ __forceinline__ void load(s16x8 (&r)[kPer], int64_t n0, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) r[u] = load_h8(row_src(rows[u], n0, h0, tid));  // chunk tid of tile u
  }
  __device__ __forceinline__ void store(uint16_t* buf, const s16x8 (&r)[kPer], int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      *reinterpret_cast<s16x8*>(buf + u * kRowTile + row_pos(slot_of_node(tid >> 3), tid & 7)) = r[u];
  }
};

// The third 16-deep contraction chunk of a lane: lanes of half 0 carry
// [a, b, c, 0, 0, 0, 0, 0] (halves), lanes of half 1 carry zeros.
__device__ __forceinline__ s16x8 aug_chunk(uint32_t ab, uint16_t cc, int hp) {
  if (hp != 0) return s16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const u32x4 w = {ab, static_cast<uint32_t>(cc), 0u, 0u};
  return __builtin_bit_cast(s16x8, w);
}

// ---------------------------------------------------------------------------------
// Backward, key-outer: a wave owns 32 keys (lane c keeps key c) and a head pair; the
// 4 waves share each staged query tile (q and dout rows, 8 KB), staged once per tile in
// LDS. S and dP - delta come from 3 MFMAs each (rows = queries, columns = keys),
// P = exp2(S log2e / sqrt(D)), dS = P (dP - delta); dV^T += dO^T P and dK^T += Q^T dS
// contract over the tile's queries, their dO^T and Q^T operands read from the same row
// tiles with ds_read_b64_tr_b16 (below), so no transposed copy is staged. Bucket sums of
// dS go to LDS bins in one of two layouts:
//  * kPrivate: [bucket][64 lanes][2 heads], one bin row per lane, so every lane updates
//    its own bins in the same instruction. Only buckets below kPrivBins fit in LDS at this
//    occupancy; a lane that meets a larger code raises *flag, and the launch is then
//    redone by the shared layout, which overwrites every output of this one.
//  * shared: [bucket][32 keys][2 heads], the two lane halves of a wave (which hold the
//    same 32 keys) updating it one half after the other, so no two lanes touch a bin at
//    once. Any NB. As the rerun of a private launch (flag given) it returns at once unless
//    *flag was raised.
constexpr int kKvTbD32 = 64;  // key-outer table entries (float2: both heads), codes clamped to NB-1 <= 63
constexpr int kPrivBins = 16;  // buckets of the private layout

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

// Transposed operand from a row tile: 4 consecutive nodes of one d for each lane. In a
// 16-lane group, ds_read_b64_tr_b16 gives lane j element j % 4 of the 8-byte pieces that
// lanes 4e + j / 4 address (e = 0..3): when lane 4e + r of group G addresses node n0 + e,
// head hl, d = 16 (G % 2) + 4r .. +3, lane j receives nodes n0 .. n0+3 at d = 16 (G % 2) + j,
// i.e. at its own column c. tr_lane_base gives that address (halves) for the 4-node group
// n0 = 16 (G / 2) + 8 k1 + 4 half without its slot term 512 (2 k1 + half): the row
// swizzle makes the rest depend on (hl, half) only through hl ^ half (x below).
__device__ __forceinline__ int tr_lane_base(int lane, int x) {
  const int G = lane >> 4, e4 = (lane >> 2) & 3, r4 = lane & 3;
  const int pos = ((r4 >> 1) ^ (e4 >> 1)) | (((G & 1) ^ (G >> 1)) << 1) | (((e4 >> 1) ^ x) << 2);
  return 64 * (4 * (G >> 1) + e4) + 8 * pos + 4 * (r4 & 1);
}
// 8 consecutive nodes 16 hp + 8 k1 .. +7 of head hl at the lane's d, as an MFMA operand
__device__ __forceinline__ s16x8 tr_row_op(const uint16_t* tile, int tb0, int tb1, int hl, int k1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(tile + 512 * (2 * k1) + (hl ? tb1 : tb0)));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(tile + 512 * (2 * k1 + 1) + (hl ? tb0 : tb1)));
  return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool kAligned, bool kPrivate>
__global__ __launch_bounds__(kThreads) void bwd_kv_mfma_d32_kernel(const uint8_t* __restrict__ spd_t,
                                                                   const float* __restrict__ table, OpsD32 ops,
                                                                   float* __restrict__ dk, float* __restrict__ dv,
                                                                   float* __restrict__ partial, int64_t N, int64_t Nk,
                                                                   int64_t ldt, int NB, int acc, int64_t qchunk,
                                                                   int64_t gstride, int64_t pstride,
                                                                   uint32_t* __restrict__ flag) {
  constexpr int kBinLanes = kPrivate ? 64 : 32;                          // bin rows per bucket
  // Three separate LDS arrays (bins sized for the layout's largest bucket count, NB <= 64):
  // as distinct objects the compiler knows the bin updates never touch the table or the
  // staged tile, so it may issue the stage reads of the dK/dV operands among them.
  __shared__ __align__(16) float bins_all[kWaves * 2 * (kPrivate ? kPrivBins : kKvTbD32) * kBinLanes];
  __shared__ __align__(16) float2 tb[kKvTbD32];  // both heads' bias * log2e: the exp2 arguments' addends
  __shared__ __align__(16) uint16_t stage[StageSetD32<2>::kHalves];
  if (!kPrivate && flag != nullptr && *flag == 0u) return;  // the private launch was exact
  // workgroup row y of a split launch: queries [y*qchunk, min(N, (y+1)*qchunk)), partial
  // dK, dV at + y*gstride and bucket partials at + y*pstride
  const int64_t ib = static_cast<int64_t>(blockIdx.y) * qchunk;
  N = N - ib < qchunk ? N - ib : qchunk;
  ops.qd += ib * kH * kD;
  ops.od += ib * kH * kD;
  ops.lq += ib;
  ops.dl += ib;
  dk += blockIdx.y * gstride;
  dv += blockIdx.y * gstride;
  partial += blockIdx.y * pstride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nbins = kPrivate ? kPrivBins : NB;
  float* bins = bins_all + w * (2 * nbins * kBinLanes);  // [nbins][rows][2 heads] per wave

  const int npad32 = static_cast<int>(ops.npk / 32);
  const int nkb = (npad32 + kWaves - 1) / kWaves;
  int kb, hpair;
  xcd_map(blockIdx.x, nkb, kb, hpair);
  if (kb < 0) return;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * hpair;
  const int64_t jw = static_cast<int64_t>(kb) * (32 * kWaves) + 32 * w;
  const int64_t j = jw + c;
  const bool wave_live = jw < ops.npk;
  const int64_t jj = wave_live ? j : 0;
  const int64_t npad = ops.npq;  // staged tiles (and lse, delta) are over queries
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < kKvTbD32; b += kThreads) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * kLog2e, table[(h0 + 1) * NB + c] * kLog2e);
  }
  for (int x = lane; x < 2 * nbins * kBinLanes; x += 64) bins[x] = 0.f;
  s16x8 kop[2][2], vop[2][2];
#pragma unroll
  for (int hl = 0; hl < 2; ++hl)
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      kop[hl][ci] = load_h8(ops.kd + (jj * kH + h0 + hl) * kD + 16 * ci + 8 * hp);
      vop[hl][ci] = load_h8(ops.vd + (jj * kH + h0 + hl) * kD + 16 * ci + 8 * hp);
    }
  const uint16_t one = 0x3C00u, ninf = 0xFC00u;
  const s16x8 kaug = aug_chunk(pack2(one, one), j < Nk ? 0 : ninf, hp);
  const s16x8 vaug = aug_chunk(pack2(one, one), 0, hp);
  f32x16 dv0 = {}, dv1 = {}, dk0 = {}, dk1 = {};
  const uint32_t nbm1 = static_cast<uint32_t>(NB - 1);
  float2* mybins = reinterpret_cast<float2*>(bins) + (kPrivate ? lane : c);
  // private layout: bytes >= kPrivBins seen by this lane (a clamped code >= kPrivBins needs
  // a raw byte >= kPrivBins; with NB <= kPrivBins every clamped code fits)
  const bool check_range = kPrivate && NB > kPrivBins;
  uint32_t over = 0u;
  const uint8_t* crow = spd_t + (j < Nk ? j : Nk - 1) * ldt + ib;
  const int64_t cc = 16 * hp;
  const int qr = node_of_row(c);

  StageSetD32<2> set;
  set.rows[0] = ops.qd;
  set.rows[1] = ops.od;
  set.h0 = h0;
  const int tb0 = tr_lane_base(lane, 0), tb1 = tr_lane_base(lane, 1);
  const int ntiles = static_cast<int>((N + 31) / 32), nfull = static_cast<int>(N / 32);  // scalar loop tests
  s16x8 sr[StageSetD32<2>::kPer];
  set.load(sr, 0, tid);
  u32x4 cw = nfull > 0 ? codes_at<false, kAligned>(crow, cc, N) : codes_at<true, kAligned>(crow, cc, N);
  uint32_t lw0 = ops.lq[static_cast<int64_t>(h0) * npad + qr], lw1 = ops.lq[static_cast<int64_t>(h0 + 1) * npad + qr];
  uint32_t dw0 = ops.dl[static_cast<int64_t>(h0) * npad + qr], dw1 = ops.dl[static_cast<int64_t>(h0 + 1) * npad + qr];
  wait_vm0();

  for (int t = 0; t < ntiles; ++t) {
    const int64_t i0 = static_cast<int64_t>(t) * 32;
    set.store(stage, sr, tid);
    __syncthreads();
    u32x4 cwn = cw;
    uint32_t lwn0 = lw0, lwn1 = lw1, dwn0 = dw0, dwn1 = dw1;
    if (t + 1 < ntiles) {
      set.load(sr, i0 + 32, tid);
      cwn = (t + 1 < nfull) ? codes_at<false, kAligned>(crow, i0 + 32 + cc, N)
                            : codes_at<true, kAligned>(crow, i0 + 32 + cc, N);
      const int64_t qn = i0 + 32 + qr;
      lwn0 = ops.lq[static_cast<int64_t>(h0) * npad + qn];
      lwn1 = ops.lq[static_cast<int64_t>(h0 + 1) * npad + qn];
      dwn0 = ops.dl[static_cast<int64_t>(h0) * npad + qn];
      dwn1 = ops.dl[static_cast<int64_t>(h0 + 1) * npad + qn];
    }
    if (wave_live) {
      const uint16_t* q_t = stage;
      const uint16_t* o_t = stage + kRowTile;
      uint32_t code[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) code[e] = min(code_byte(cw, e), nbm1);
      f32x16 s0 = {}, s1 = {};
      if (check_range) over |= (cw[0] | cw[1] | cw[2] | cw[3]) & 0xF0F0F0F0u;
      f32x16 p0 = {}, p1 = {};
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) {
        s0 = mfma_h16(row_op(q_t, c, 0, ci, hp), kop[0][ci], s0);
        s1 = mfma_h16(row_op(q_t, c, 1, ci, hp), kop[1][ci], s1);
        p0 = mfma_h16(row_op(o_t, c, 0, ci, hp), vop[0][ci], p0);
        p1 = mfma_h16(row_op(o_t, c, 1, ci, hp), vop[1][ci], p1);
      }
      s0 = mfma_h16(aug_chunk(lw0, one, hp), kaug, s0);
      s1 = mfma_h16(aug_chunk(lw1, one, hp), kaug, s1);
      p0 = mfma_h16(aug_chunk(dw0, 0, hp), vaug, p0);
      p1 = mfma_h16(aug_chunk(dw1, 0, hp), vaug, p1);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float2 tv = tb[code[e]];  // read straight into the FMAs' addends: no moves
        const float pa = __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, tv.x));
        const float pb = __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, tv.y));
        s0[e] = pa;
        s1[e] = pb;
        p0[e] *= pa;
        p1[e] *= pb;
      }
      if constexpr (kPrivate) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t b = min(code[e], static_cast<uint32_t>(kPrivBins - 1));  // in range even when flagged
          float2 bin = mybins[b * 64];
          bin.x += p0[e];
          bin.y += p1[e];
          mybins[b * 64] = bin;
        }
      } else {
        // lane half 0 first, then half 1: the two halves hold the same 32 keys
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          if (hp == half) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float2 bin = mybins[code[e] * 32];
              bin.x += p0[e];
              bin.y += p1[e];
              mybins[code[e] * 32] = bin;
            }
          }
        }
      }
#pragma unroll
      for (int k1 = 0; k1 < 2; ++k1) {
        dv0 = mfma_h16(tr_row_op(o_t, tb0, tb1, 0, k1), pack_f16x8(s0, 8 * k1), dv0);
        dv1 = mfma_h16(tr_row_op(o_t, tb0, tb1, 1, k1), pack_f16x8(s1, 8 * k1), dv1);
        dk0 = mfma_h16(tr_row_op(q_t, tb0, tb1, 0, k1), pack_f16x8(p0, 8 * k1), dk0);
        dk1 = mfma_h16(tr_row_op(q_t, tb0, tb1, 1, k1), pack_f16x8(p1, 8 * k1), dk1);
      }
    }
    cw = cwn;
    lw0 = lwn0;
    lw1 = lwn1;
    dw0 = dwn0;
    dw1 = dwn1;
    __syncthreads();
  }
  if (wave_live && j < Nk) {
    const float rs = 1.f / sqd;
    float* kp0 = dk + j * kHD + h0 * kD + 4 * hp;
    float* vp0 = dv + j * kHD + h0 * kD + 4 * hp;
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      store4(kp0 + 8 * jq, make_float4(dk0[4 * jq] * rs, dk0[4 * jq + 1] * rs, dk0[4 * jq + 2] * rs, dk0[4 * jq + 3] * rs),
             acc);
      store4(kp0 + kD + 8 * jq,
             make_float4(dk1[4 * jq] * rs, dk1[4 * jq + 1] * rs, dk1[4 * jq + 2] * rs, dk1[4 * jq + 3] * rs), acc);
      store4(vp0 + 8 * jq, make_float4(dv0[4 * jq], dv0[4 * jq + 1], dv0[4 * jq + 2], dv0[4 * jq + 3]), acc);
      store4(vp0 + kD + 8 * jq, make_float4(dv1[4 * jq], dv1[4 * jq + 1], dv1[4 * jq + 2], dv1[4 * jq + 3]), acc);
    }
  }
  if (kPrivate && over != 0u) *flag = 1u;  // every writer stores the same value
  // per-wave bins -> one partial row per 32-key block and head (a wave past the last key
  // block writes its zero bins too, so every partial row is defined); buckets past the
  // private layout's bins had no entries unless the flag was raised
  for (int x = lane; x < 2 * NB; x += 64) {
    const int hl = x / NB, b = x - hl * NB;
    float sum = 0.f;
    if (b < nbins) {
      const float* srcb = bins + b * (2 * kBinLanes) + hl;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains, fixed order
#pragma unroll
      for (int l = 0; l < kBinLanes; l += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s4[u] += srcb[2 * (l + u)];
      }
      sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    partial[((jw / 32) * kH + h0 + hl) * NB + b] = sum;
  }
}

// ---------------------------------------------------------------------------------
// Backward, query-outer: a wave owns 32 queries (lane c keeps query c) and a head
// pair; the 4 waves share each staged key tile (k and v rows), double-buffered.
// S^T and dP^T - delta come from 3 MFMAs each (rows = keys, columns = queries);
// dQ^T += K^T dS^T per key tile, K^T read from the k row tile with ds_read_b64_tr_b16
// as in the key-outer pass.
template <bool kAligned>
__global__ __launch_bounds__(kThreads) void bwd_q_mfma_d32_kernel(const uint8_t* __restrict__ spd,
                                                                  const float* __restrict__ table, OpsD32 ops,
                                                                  float* __restrict__ dq, int64_t N, int64_t Nk,
                                                                  int64_t ldc, int NB, int acc, int64_t kchunk,
                                                                  int64_t gstride) {
  using Set = StageSetD32<2>;
  __shared__ float2 tb[256];  // both heads' bias for each byte value (forward: * sqrt(D), query-outer: * log2e)
  __shared__ __align__(16) uint16_t stage[2 * Set::kHalves];
  // workgroup row y of a split launch: keys [y*kchunk, min(Nk, (y+1)*kchunk)), partial dQ
  // at dq + y*gstride
  const int64_t jb = static_cast<int64_t>(blockIdx.y) * kchunk;
  Nk = Nk - jb < kchunk ? Nk - jb : kchunk;
  ops.kd += jb * kH * kD;
  ops.vd += jb * kH * kD;
  spd += jb;
  dq += blockIdx.y * gstride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int npad32 = static_cast<int>(ops.npq / 32);
  const int nqb = (npad32 + kWaves - 1) / kWaves;
  int qb, hpair;
  xcd_map(blockIdx.x, nqb, qb, hpair);
  if (qb < 0) return;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * hpair;
  const int64_t iw = static_cast<int64_t>(qb) * (32 * kWaves) + 32 * w;
  const int64_t i = iw + c;
  const bool wave_live = iw < ops.npq;
  const int64_t ii = wave_live ? i : 0;
  const bool qvalid = i < N;
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < 256; b += kThreads) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * kLog2e, table[(h0 + 1) * NB + c] * kLog2e);
  }
  s16x8 qop[2][2], oop[2][2], qaug[2], oaug[2];
  const uint16_t one = 0x3C00u, ninf = 0xFC00u;
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      qop[hl][ci] = load_h8(ops.qd + (ii * kH + h0 + hl) * kD + 16 * ci + 8 * hp);
      oop[hl][ci] = load_h8(ops.od + (ii * kH + h0 + hl) * kD + 16 * ci + 8 * hp);
    }
    qaug[hl] = aug_chunk(ops.lq[static_cast<int64_t>(h0 + hl) * ops.npq + ii], one, hp);
    oaug[hl] = aug_chunk(ops.dl[static_cast<int64_t>(h0 + hl) * ops.npq + ii], 0, hp);
  }
  const s16x8 vaug = aug_chunk(pack2(one, one), 0, hp);
  f32x16 dq0 = {}, dq1 = {};
  const uint8_t* srow = spd + (qvalid ? i : N - 1) * ldc;
  const int64_t cc = 16 * hp;
  const int kr = node_of_row(c);

  Set set;
  set.rows[0] = ops.kd;
  set.rows[1] = ops.vd;
  set.h0 = h0;
  const int tb0 = tr_lane_base(lane, 0), tb1 = tr_lane_base(lane, 1);
  const int ntiles = static_cast<int>((Nk + 31) / 32), nfull = static_cast<int>(Nk / 32);  // scalar loop tests
  s16x8 sr[Set::kPer];
  set.load(sr, 0, tid);
  set.store(stage, sr, tid);
  u32x4 cw = nfull > 0 ? codes_at<false, kAligned>(srow, cc, Nk) : codes_at<true, kAligned>(srow, cc, Nk);
  wait_vm0();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int64_t j0 = static_cast<int64_t>(t) * 32;
    const uint16_t* cur = stage + (t & 1) * Set::kHalves;
    u32x4 cwn = cw;
    if (t + 1 < ntiles) {
      set.load(sr, j0 + 32, tid);
      cwn = (t + 1 < nfull) ? codes_at<false, kAligned>(srow, j0 + 32 + cc, Nk)
                            : codes_at<true, kAligned>(srow, j0 + 32 + cc, Nk);
    }
    if (wave_live) {
      const uint16_t* k_t = cur;
      const uint16_t* v_t = cur + kRowTile;
      f32x16 s0 = {}, s1 = {};
      f32x16 p0 = {}, p1 = {};
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) {
        s0 = mfma_h16(row_op(k_t, c, 0, ci, hp), qop[0][ci], s0);
        s1 = mfma_h16(row_op(k_t, c, 1, ci, hp), qop[1][ci], s1);
        p0 = mfma_h16(row_op(v_t, c, 0, ci, hp), oop[0][ci], p0);
        p1 = mfma_h16(row_op(v_t, c, 1, ci, hp), oop[1][ci], p1);
      }
      const s16x8 kaug = aug_chunk(pack2(one, one), j0 + kr < Nk ? 0 : ninf, hp);
      s0 = mfma_h16(kaug, qaug[0], s0);
      s1 = mfma_h16(kaug, qaug[1], s1);
      p0 = mfma_h16(vaug, oaug[0], p0);
      p1 = mfma_h16(vaug, oaug[1], p1);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float2 t = tb[code_byte(cw, e)];  // both heads' log2e-scaled bias: the FMA addends
        p0[e] *= __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, t.x));
        p1[e] *= __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, t.y));
      }
#pragma unroll
      for (int k1 = 0; k1 < 2; ++k1) {
        dq0 = mfma_h16(tr_row_op(k_t, tb0, tb1, 0, k1), pack_f16x8(p0, 8 * k1), dq0);
        dq1 = mfma_h16(tr_row_op(k_t, tb0, tb1, 1, k1), pack_f16x8(p1, 8 * k1), dq1);
      }
    }
    if (t + 1 < ntiles) set.store(stage + ((t + 1) & 1) * Set::kHalves, sr, tid);
    cw = cwn;
    __syncthreads();
  }
  if (wave_live && qvalid) {
    const float rs = 1.f / sqd;
    float* qp0 = dq + i * kHD + h0 * kD + 4 * hp;
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      store4(qp0 + 8 * jq, make_float4(dq0[4 * jq] * rs, dq0[4 * jq + 1] * rs, dq0[4 * jq + 2] * rs, dq0[4 * jq + 3] * rs),
             acc);
      store4(qp0 + kD + 8 * jq,
             make_float4(dq1[4 * jq] * rs, dq1[4 * jq + 1] * rs, dq1[4 * jq + 2] * rs, dq1[4 * jq + 3] * rs), acc);
    }
  }
}

OpsD32 carve_ops_d32(void* base, int64_t N, int64_t Nk) {
  OpsD32 o{};
  o.npq = (N + 31) / 32 * 32;
  o.npk = (Nk + 31) / 32 * 32;
  const size_t nq = static_cast<size_t>(o.npq) * kH * kD;  // halves per query-side array
  const size_t nk = static_cast<size_t>(o.npk) * kH * kD;  // halves per key-side array
  uint16_t* p = static_cast<uint16_t*>(base);
  o.qd = p;
  o.od = o.qd + nq;
  o.kd = o.od + nq;
  o.vd = o.kd + nk;
  o.lq = reinterpret_cast<uint32_t*>(o.vd + nk);
  o.dl = o.lq + static_cast<size_t>(o.npq) * kH;
  return o;
}

}  // namespace

size_t mfma_d32_ops_bytes(int64_t N, int64_t Nk) {
  const size_t npq = static_cast<size_t>((N + 31) / 32 * 32), npk = static_cast<size_t>((Nk + 31) / 32 * 32);
  return (2 * npq + 2 * npk) * kH * kD * 2 + npq * kH * 4 * 2;
}

int64_t mfma_d32_kv_blocks(int64_t Nk) {
  const int64_t nblk = ((Nk + 31) / 32 + kWaves - 1) / kWaves;
  return nblk * kWaves;
}

hipError_t launch_fwd_mfma_d32(const FwdArgs& a, hipStream_t s) {
  // no workspace (gt_attn_fwd): never split
  const Split sp = a.workspace != nullptr ? inner_split(a.N, a.Nk, kH, kD, a.dtype, kSplitFwd) : Split{1, a.Nk};
  const int64_t rows = a.N * kH;
  float* out = a.out;
  float* lse = a.lse;
  const bool part = sp.S > 1 || a.acc;
  if (part) {  // partial results per key range, merged (into out/lse when acc) below
    out = static_cast<float*>(a.workspace);
    lse = out + static_cast<size_t>(sp.S) * rows * kD;
  }
  const dim3 grid(static_cast<unsigned>(xcd_grid(static_cast<int>((a.N + 32 * kWaves - 1) / (32 * kWaves)))),
                  static_cast<unsigned>(sp.S));
  trace_begin(kTraceFwd, s);
  if (codes_aligned(a.spd, a.ld))
    hipLaunchKernelGGL(fwd_mfma_d32_kernel<true>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table, out, lse,
                       a.N, a.Nk, a.ld, a.NB, sp.chunk, rows * kD, rows);
  else
    hipLaunchKernelGGL(fwd_mfma_d32_kernel<false>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table, out, lse,
                       a.N, a.Nk, a.ld, a.NB, sp.chunk, rows * kD, rows);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceFwd, s);
  if (e != hipSuccess || !part) return e;
  return launch_merge_splits(out, lse, sp.S, a.out, a.lse, rows, kD, a.acc, s);
}

hipError_t launch_bwd_mfma_d32(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
  char* base = static_cast<char*>(a.workspace);
  const OpsD32 ops = carve_ops_d32(base + w.ops_off, a.N, a.Nk);
  float* partial = reinterpret_cast<float*>(base + w.partial_off);
  uint32_t* flag = reinterpret_cast<uint32_t*>(base + w.flag_off);
  const int64_t prep_threads = std::max(ops.npq, ops.npk) * kH;
  trace_begin(kTraceBwdDelta, s);
  hipLaunchKernelGGL(bwd_prep_mfma_d32_kernel, dim3(static_cast<unsigned>((prep_threads + 255) / 256)), dim3(256), 0,
                     s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.out, static_cast<const uint16_t*>(a.dout), a.lse, ops, a.N,
                     a.Nk, flag);
  hipError_t e = hipGetLastError();
  trace_end(kTraceBwdDelta, s);
  if (e != hipSuccess) return e;

  // key-outer: split over query ranges writes partial dK, dV ([2][S][Nk*H*D] in the
  // workspace) that are summed afterwards; unsplit it writes (or adds) directly
  const int64_t nk_el = a.Nk * kHD, nq_el = a.N * kHD;
  const bool kv_split = w.kv.S > 1;
  float* dkp = kv_split ? reinterpret_cast<float*>(base + w.dkv_off) : a.dk;
  float* dvp = kv_split ? dkp + static_cast<size_t>(w.kv.S) * nk_el : a.dv;
  const int kv_acc = kv_split ? 0 : (a.acc & kAccDkv);
  const int64_t pstride = w.n_kv_blocks * kH * a.NB;
  const int nkb = static_cast<int>((ops.npk / 32 + kWaves - 1) / kWaves);
  const dim3 kgrid(static_cast<unsigned>(xcd_grid(nkb)), static_cast<unsigned>(w.kv.S));
  // Private bins first when its outputs may be overwritten by a rerun (no accumulation
  // into dK, dV); the shared-bin launch after it runs only if a code fell outside the
  // private bins (never when NB <= kPrivBins, so it is then not launched).
  const bool priv = kv_acc == 0;
  const bool aligned = codes_aligned(a.spd_t, a.ld_t);
  auto kv_launch = [&](auto private_tag, uint32_t* f) {
    constexpr bool kP = decltype(private_tag)::value;
    if (aligned)
      hipLaunchKernelGGL((bwd_kv_mfma_d32_kernel<true, kP>), kgrid, dim3(kThreads), 0, s, a.spd_t, a.table, ops,
                         dkp, dvp, partial, a.N, a.Nk, a.ld_t, a.NB, kv_acc, w.kv.chunk, nk_el, pstride, f);
    else
      hipLaunchKernelGGL((bwd_kv_mfma_d32_kernel<false, kP>), kgrid, dim3(kThreads), 0, s, a.spd_t, a.table, ops,
                         dkp, dvp, partial, a.N, a.Nk, a.ld_t, a.NB, kv_acc, w.kv.chunk, nk_el, pstride, f);
  };
  trace_begin(kTraceBwdKv, s);
  if (priv) {
    kv_launch(std::true_type{}, flag);
    e = hipGetLastError();
    if (e == hipSuccess && a.NB > kPrivBins) {
      kv_launch(std::false_type{}, flag);
      e = hipGetLastError();
    }
  } else {
    kv_launch(std::false_type{}, nullptr);
    e = hipGetLastError();
  }
  trace_end(kTraceBwdKv, s);
  if (e != hipSuccess) return e;

  const bool q_split = w.q.S > 1;
  float* dqp = q_split ? reinterpret_cast<float*>(base + w.dq_off) : a.dq;
  const int q_acc = q_split ? 0 : (a.acc & kAccDq);
  const int nqb = static_cast<int>((ops.npq / 32 + kWaves - 1) / kWaves);
  const dim3 qgrid(static_cast<unsigned>(xcd_grid(nqb)), static_cast<unsigned>(w.q.S));
  trace_begin(kTraceBwdQ, s);
  if (codes_aligned(a.spd, a.ld))
    hipLaunchKernelGGL(bwd_q_mfma_d32_kernel<true>, qgrid, dim3(kThreads), 0, s, a.spd, a.table, ops, dqp, a.N, a.Nk,
                       a.ld, a.NB, q_acc, w.q.chunk, nq_el);
  else
    hipLaunchKernelGGL(bwd_q_mfma_d32_kernel<false>, qgrid, dim3(kThreads), 0, s, a.spd, a.table, ops, dqp, a.N,
                       a.Nk, a.ld, a.NB, q_acc, w.q.chunk, nq_el);
  e = hipGetLastError();
  trace_end(kTraceBwdQ, s);
  if (e != hipSuccess) return e;
  if (!kv_split && !q_split)
    return launch_dtable_reduce(partial, a.dtable, w.n_kv_blocks, kH * a.NB, a.acc & kAccDtable, s);
  const SumSplits none{nullptr, nullptr, 0, 0, 0};
  const int dkv = a.acc & kAccDkv;
  const SumSplits sk = kv_split ? SumSplits{dkp, a.dk, nk_el, w.kv.S, dkv} : none;
  const SumSplits sv = kv_split ? SumSplits{dvp, a.dv, nk_el, w.kv.S, dkv} : none;
  const SumSplits sq = q_split ? SumSplits{dqp, a.dq, nq_el, w.q.S, a.acc & kAccDq} : none;
  return launch_bwd_finish(sk, sv, sq, partial, a.dtable, w.kv.S * w.n_kv_blocks, kH * a.NB, a.acc & kAccDtable, s);
}

}  // namespace gt
