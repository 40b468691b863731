// Biased attention on the gfx950 matrix cores (MFMA): head dimension 8, 8 heads,
// bfloat16 inputs, float32 accumulation and outputs.
//
// Precision: the scores QK^T and dO V^T multiply the bf16 inputs exactly. Softmax
// probabilities P and score gradients dS enter the contractions over nodes (P.V,
// P^T dO, dS^T Q, dS K) as IEEE half precision (11-bit significand; bf16's 8 bits
// leave a max error near 4-7% of the gradients' RMS on heavy-tailed rows), and the
// bf16 inputs they meet are converted to half exactly (inputs must lie within
// half's range, |x| < 65504).
//
// MegaGraph pages, abstract: the score matrix and the topology-aware bias matrix are
// what make full-graph attention expensive; Fig. 4 caption: work proceeds over key
// blocks with the bias columns sliced to each block. Neither matrix exists here
// outside registers: each score MFMA's accumulator starts from the tile's bias,
// table[h, code] read from LDS by the uint8 code, so adding the bias costs no vector
// instruction.
//
// Work split: workgroups of 4 waves (8 in the one-pass backward); each wave owns 32
// nodes of its outer loop and two heads (the head pair follows from the workgroup
// order, xcd_map). Lane l holds
// column c = l % 32 of every 32x32 tile and one half hp = l / 32 of its rows. In the
// backward, rows follow node_of_row (mfma_common.h): the lane's 16 accumulator entries
// are 16 consecutive nodes, so its codes are one 16-byte load and each 8-entry half of
// its accumulator is directly an operand of the 32x32x16 MFMA that contracts over those
// nodes, whose other operand is read as 8 consecutive nodes of a transposed [d][node]
// tile in LDS. The forward interleaves the two heads in its score tiles (below).
//
// Table in LDS: for each byte value b, both heads' table[h, min(b, NB-1)] * sqrt(D) as one
// float2 (one 8-byte read per entry), so every byte value indexes it without a clamp.
#include "mfma_common.h"

#include <algorithm>
#include <type_traits>

namespace gt {
namespace {

constexpr int kD = 8;
constexpr int kH = 8;
constexpr int kHD = kH * kD;

// ---------------------------------------------------------------------------------
// Forward. Per 32-key tile, S^T = K Q^T for both heads as two MFMAs over 16 keys each
// (rows = key and head pairs, columns = queries; see kop below); running max per query
// column and head; O^T += V^T P^T with a ones row in V^T so the MFMA also accumulates
// the row sum l.
//
// A workgroup is 4 waves = 128 queries x 2 heads (ordered as in xcd_map); the waves
// share each key tile's K rows and transposed half-precision V in LDS (double-buffered,
// one barrier per key tile; every thread stages one dword of each, V converted to half),
// and each wave prefetches the next tile's codes and its staging share into registers
// while it computes the current one. Only the last key tile can be partial, so only it
// takes the guarded loads and the -inf mask.
//
// The running max is updated lazily: the first tile sets it, and a wave rescales its
// accumulators only when some lane's score exceeds it by more than kLazy (in log2 units),
// so the probabilities fed to the MFMA stay below 2^kLazy and rescales are rare. The test
// reads the exp2 arguments, which carry the shift already: no per-tile threshold.
constexpr int kFwdWaves = 4;

struct FwdTile {
  u32x4 cw;       // 16 codes: query row, keys 16*hp .. 16*hp+15 of the tile
  uint32_t kw;    // one dword of K (two d values of one key and head) to stage
  uint32_t vw;    // the same dword of V
};

// Staged K tile of a head pair: [key][8 dwords], 32 bytes per key: head h's 8 d values
// (16 bytes) at half h ^ ((key >> 4) & 1), so the 16 lanes of one score MFMA that read
// 16-byte halves of keys {8g..8g+7} and {16+8g..16+8g+7} cover all banks once.
__device__ __forceinline__ int kt_pos(int key, int head) { return key * 8 + 4 * (head ^ ((key >> 4) & 1)); }

// 8 of 16 accumulator entries (first, first+2, ..., first+14) as an f16 MFMA operand
__device__ __forceinline__ s16x8 pack_f16x8_odd_even(const f32x16& a, int first) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<_Float16>(a[first + 2 * e]);
  return __builtin_bit_cast(s16x8, r);
}

template <bool kGuard, bool kAligned>
__device__ __forceinline__ void fwd_load(FwdTile& t, const uint8_t* srow, const uint16_t* k,
                                         const uint16_t* v, int64_t j0, int64_t N, int h0, int hp,
                                         int sk, int shl, int sdp) {
  if (kGuard || !kAligned) {
    t.cw = load_codes16<false>(srow, j0 + 16 * hp, N);
  } else {
    t.cw = *reinterpret_cast<const u32x4*>(srow + j0 + 16 * hp);
  }
  const int64_t vn = j0 + sk;
  const int64_t off = vn * kHD + (h0 + shl) * kD + 2 * sdp;
  t.kw = (!kGuard || vn < N) ? *reinterpret_cast<const uint32_t*>(k + off) : 0u;
  t.vw = (!kGuard || vn < N) ? *reinterpret_cast<const uint32_t*>(v + off) : 0u;
}

template <bool kAligned>
__global__ __launch_bounds__(64 * kFwdWaves, 4) void fwd_mfma_d8_kernel(const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ k,
                                                                    const uint16_t* __restrict__ v,
                                                                    const uint8_t* __restrict__ spd,
                                                                    const float* __restrict__ table,
                                                                    float* __restrict__ out,
                                                                    float* __restrict__ lse, int64_t N, int64_t Nk,
                                                                    int64_t ldc, int NB, int64_t kchunk,
                                                                    int64_t ostride, int64_t lstride) {
  __shared__ float2 tb[256];  // both heads' bias for each byte value
  __shared__ __align__(16) uint16_t vt[2][2][kD + 1][32];  // [buffer][head][d or ones][key]
  __shared__ __align__(16) uint32_t kt[2][32 * 8];         // [buffer] staged K tile (kt_pos)
  __shared__ __align__(16) uint32_t kzero[4];              // the zero half of a score operand
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
  const int nqb = static_cast<int>((N + 32 * kFwdWaves - 1) / (32 * kFwdWaves));
  int qb, hpair;
  xcd_map(blockIdx.x, nqb, qb, hpair);
  if (qb < 0) return;
  const int h0 = 2 * hpair;
  const int64_t i = static_cast<int64_t>(qb) * (32 * kFwdWaves) + 32 * w + c;
  const bool qvalid = i < N;
  const int64_t irow = qvalid ? i : N - 1;
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < 256; b += 64 * kFwdWaves) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * sqd, table[(h0 + 1) * NB + c] * sqd);
  }
  for (int x = tid; x < 2 * 2 * 32; x += 64 * kFwdWaves) vt[x >> 6][(x >> 5) & 1][kD][x & 31] = 0x3C00;  // 1.0
  if (tid < 4) kzero[tid] = 0u;
  // query operand of the score MFMAs: the 8 d values of head h0 + hp (k-group hp)
  const s16x8 qop = qvalid ? load_h8(q + i * kHD + (h0 + hp) * kD) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* srow = spd + irow * ldc;
  // staging role: key sk of the tile, head shl, d pair sdp (one dword per thread)
  const int sk = 8 * w + (lane >> 3), shl = (lane >> 2) & 1, sdp = lane & 3;
  const int kdw = kt_pos(sk, shl) + sdp;  // this thread's K dword
  auto stage = [&](int buf, uint32_t kw, uint32_t vw) {
    kt[buf][kdw] = kw;
    const uint32_t hh = bf16x2_to_f16x2(vw);
    vt[buf][shl][2 * sdp][sk] = static_cast<uint16_t>(hh & 0xffffu);
    vt[buf][shl][2 * sdp + 1][sk] = static_cast<uint16_t>(hh >> 16);
  };
  // Score MFMA g (g = 0, 1) of a tile covers 16 keys of both heads: accumulator row r
  // stands for key 16*((r >> 2) & 1) + 8g + 2*(r >> 3) + ((r & 3) >> 1) and head r & 1, so a
  // lane's entries 2m and 2m+1 are key 16*hp + 8g + m of heads 0 and 1: one 8-byte table
  // read fills both. The contraction runs over the 16 d values of both heads (k-group =
  // head): row c's operand is its key's k for its head, zero for the other head.
  const bool kown = (c & 1) == hp;
  const int krow0 = 16 * ((c >> 2) & 1) + 2 * (c >> 3) + ((c & 3) >> 1);  // key of row c at g = 0
  auto kop = [&](int buf, int g) {
    const uint32_t* p = kown ? &kt[buf][kt_pos(krow0 + 8 * g, hp)] : kzero;
    return *reinterpret_cast<const s16x8*>(p);
  };

  const int ntiles = static_cast<int>((Nk + 31) / 32), nfull = static_cast<int>(Nk / 32);
  FwdTile cur, nxt;
  if (nfull > 0)
    fwd_load<false, kAligned>(cur, srow, k, v, 0, Nk, h0, hp, sk, shl, sdp);
  else
    fwd_load<true, kAligned>(cur, srow, k, v, 0, Nk, h0, hp, sk, shl, sdp);
  stage(0, cur.kw, cur.vw);
  wait_vm0();
  __syncthreads();

  f32x16 o0 = {}, o1 = {};
  // The softmax shift of both heads, kept as the exp2 argument's addend: -m * log2(e)/sqrt(D)
  // for the running max m of the raw scores (set by the first tile).
  float nb0 = 0.f, nb1 = 0.f;
  // One key tile; kMask (the partial last tile only) sets the scores of keys past Nk to
  // -inf. The full tiles run without that code: kept in the loop, the compiler turns the
  // tile-uniform test into per-entry selects executed on every tile. kFirst: the first
  // tile, which sets the shift from its largest score.
  auto tile = [&](int t, auto mask_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
    const int64_t j0 = static_cast<int64_t>(t) * 32;
    const int buf = t & 1;
    if (t + 1 < nfull)
      fwd_load<false, kAligned>(nxt, srow, k, v, j0 + 32, Nk, h0, hp, sk, shl, sdp);
    else if (t + 1 < ntiles)
      fwd_load<true, kAligned>(nxt, srow, k, v, j0 + 32, Nk, h0, hp, sk, shl, sdp);
    // sg[g]: entries 2m, 2m+1 = key 16*hp + 8g + m, heads 0 and 1
    f32x16 sg[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float2 tv = tb[code_byte(cur.cw, 8 * g + m)];
        sg[g][2 * m] = tv.x;
        sg[g][2 * m + 1] = tv.y;
      }
      sg[g] = mfma_b16(kop(buf, g), qop, sg[g]);
    }
    if constexpr (kMask) {
      const int64_t lim = Nk - (j0 + 16 * hp);  // lane keys 8g + m >= lim are past the last key
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (8 * g + (e >> 1) >= lim) sg[g][e] = -INFINITY;
    }
    if constexpr (kFirst) {  // the shift starts at the query column's largest score of this tile
      float x0 = sg[0][0], x1 = sg[0][1];
#pragma unroll
      for (int j = 1; j < 16; ++j) {
        x0 = fmaxf(x0, sg[j >> 3][2 * (j & 7)]);
        x1 = fmaxf(x1, sg[j >> 3][2 * (j & 7) + 1]);
      }
      nb0 = -fmaxf(x0, __shfl_xor(x0, 32)) * sc2;
      nb1 = -fmaxf(x1, __shfl_xor(x1, 32)) * sc2;
    }
    // exp2 arguments against the current shift
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        sg[g][e] = fmaf(sg[g][e], sc2, nb0);
        sg[g][e + 1] = fmaf(sg[g][e + 1], sc2, nb1);
      }
    if constexpr (!kFirst) {
      // The running max is tested on the arguments: an argument above kLazy means a score
      // that far above the shift. Each lane tests its own 16 keys; the two lane halves of
      // a query column are combined only on the rare rescale path.
      float x0 = sg[0][0], x1 = sg[0][1];
#pragma unroll
      for (int j = 1; j < 16; ++j) {
        x0 = fmaxf(x0, sg[j >> 3][2 * (j & 7)]);
        x1 = fmaxf(x1, sg[j >> 3][2 * (j & 7) + 1]);
      }
      if (__builtin_expect(__any(x0 > kLazy || x1 > kLazy), 0)) {  // rare: keep it a branch
        // the shift rises by d to the column's largest score (whose argument becomes 0)
        const float d0 = fmaxf(fmaxf(x0, __shfl_xor(x0, 32)), 0.f);
        const float d1 = fmaxf(fmaxf(x1, __shfl_xor(x1, 32)), 0.f);
        const float a0 = __builtin_amdgcn_exp2f(-d0), a1 = __builtin_amdgcn_exp2f(-d1);
#pragma unroll
        for (int e = 0; e < 5; ++e) {
          o0[e] *= a0;
          o1[e] *= a1;
        }
        nb0 -= d0;
        nb1 -= d1;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            sg[g][e] -= d0;
            sg[g][e + 1] -= d1;
          }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) sg[g][e] = __builtin_amdgcn_exp2f(sg[g][e]);
    // rows >= 9 of the V^T operand only feed output rows that are never read; PV MFMA g
    // contracts over keys 16*hp + 8g .. +7 (k-group hp), the lane's keys of score MFMA g
    const int vr = min(c, kD);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const s16x8 va = *reinterpret_cast<const s16x8*>(&vt[buf][0][vr][16 * hp + 8 * g]);
      const s16x8 vb = *reinterpret_cast<const s16x8*>(&vt[buf][1][vr][16 * hp + 8 * g]);
      o0 = mfma_h16(va, pack_f16x8_odd_even(sg[g], 0), o0);
      o1 = mfma_h16(vb, pack_f16x8_odd_even(sg[g], 1), o1);
    }
    if (t + 1 < ntiles) {
      stage(buf ^ 1, nxt.kw, nxt.vw);
      cur = nxt;
    }
    __syncthreads();
  };
  if (nfull > 0) tile(0, std::false_type{}, std::true_type{});
  for (int t = 1; t < nfull; ++t) tile(t, std::false_type{}, std::false_type{});
  if (nfull < ntiles) {
    if (nfull == 0)
      tile(nfull, std::true_type{}, std::true_type{});
    else
      tile(nfull, std::true_type{}, std::false_type{});
  }
  // O^T rows: d = 4hp + e in entries e = 0..3; row 8 (lane half 0, entry 4) is l.
  const float l0 = __shfl(o0[4], c), l1 = __shfl(o1[4], c);
  if (qvalid) {
    float* op = out + i * kHD + h0 * kD + 4 * hp;
    const float r0 = 1.f / l0, r1 = 1.f / l1;
    *reinterpret_cast<float4*>(op) = make_float4(o0[0] * r0, o0[1] * r0, o0[2] * r0, o0[3] * r0);
    *reinterpret_cast<float4*>(op + kD) = make_float4(o1[0] * r1, o1[1] * r1, o1[2] * r1, o1[3] * r1);
    if (hp == 0) {
      lse[i * kH + h0] = (log2f(l0) - nb0) * kLn2;
      lse[i * kH + h0 + 1] = (log2f(l1) - nb1) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------------
// Backward operand copies, written once per call into the workspace: query-side rows
// for the N queries rounded up to 32 (npq), key-side rows for the Nk keys rounded up
// to 32 (npk); padded rows let the main loops run without bounds checks. Augmented half-precision rows [node][head][16] fold the per-query terms of
// the backward into the score MFMAs (contraction index 8.. holds the extra columns):
//   qa  = [q(8), -L_hi, -L_lo, 1, 0..]    L = lse * sqrt(D), split into two halves
//   ka  = [k(8),  1,     1,  pen, 0..]    pen = 0, or -inf for padded keys
//   doa = [do(8), -dl_hi, -dl_lo, 0..]    dl = delta = <dout, out>
//   va  = [v(8),  1,     1,   0, 0..]
// so that qa.ka = q.k - lse*sqrt(D) (+ -inf past Nk) and doa.va = dout.v - delta. The bf16
// inputs are exact in half precision, so the score products carry no rounding; the scale
// log2(e)/sqrt(D) is applied in float32 before the exp2 (folding it into q would round
// q to half precision and cost about 1e-3 of P). Padded
// queries get -L_hi = -inf. The contractions over queries read Q^T and dO^T from the
// staged qa and doa row tiles transposed (ds_read_b64_tr_b16); a transposed half copy
// kt [head][d][node] of k (over npk nodes) serves the contraction over keys.
struct BwdOps {
  uint16_t *qa, *ka, *doa, *va, *kt;
  int64_t npq, npk;
};

__global__ __launch_bounds__(256) void bwd_prep_mfma_d8_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const float* __restrict__ out,
                                                               const uint16_t* __restrict__ dout,
                                                               const float* __restrict__ lse, BwdOps ops,
                                                               int64_t N, int64_t Nk, uint32_t* __restrict__ flag) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x == 0) *flag = 0u;  // the fused pass's code-range flag starts clear
  const int64_t nmax = ops.npq > ops.npk ? ops.npq : ops.npk;
  if (x >= nmax * kH) return;
  const int h = static_cast<int>(x / nmax);
  const int64_t n = x - h * nmax;
  // Rows are assembled as raw half bit patterns (uint16) and stored as two dwordx4;
  // values beyond half's range become NaN (half_bits_or_nan), constants are exact.
  auto hbits = [](float x) { return half_bits_or_nan(x); };
  auto pack = [](const uint16_t* e, int first) {
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = static_cast<uint32_t>(e[first + 2 * t]) | (static_cast<uint32_t>(e[first + 2 * t + 1]) << 16);
    return w;
  };
  auto put_row = [&](uint16_t* dst, const uint16_t* e) {
    u32x4* o = reinterpret_cast<u32x4*>(dst + (n * kH + h) * 16);
    o[0] = pack(e, 0);
    o[1] = pack(e, 8);
  };
  const uint16_t one = 0x3C00u;   // half 1.0
  const uint16_t ninf = 0xFC00u;  // half -inf (padding)
  if (n < ops.npq) {
    uint16_t qa[16] = {}, da[16] = {};
    qa[10] = one;
    if (n < N) {
      const int64_t r = n * kH + h;
      const u32x4 qw = *reinterpret_cast<const u32x4*>(q + r * kD);
      const u32x4 dw = *reinterpret_cast<const u32x4*>(dout + r * kD);
      const float4 o0 = *reinterpret_cast<const float4*>(out + r * kD);
      const float4 o1 = *reinterpret_cast<const float4*>(out + r * kD + 4);
      const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
      float delta = 0.f;
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        const int wi = d >> 1;
        const float qf = (d & 1) ? bf16_hi(qw[wi]) : bf16_lo(qw[wi]);
        const float df = (d & 1) ? bf16_hi(dw[wi]) : bf16_lo(dw[wi]);
        delta = fmaf(df, ov[d], delta);
        qa[d] = hbits(qf);
        da[d] = hbits(df);
      }
      const float L = lse[r] * sqrtf(static_cast<float>(kD));
      const _Float16 lh = to_half_or_nan(L);
      qa[8] = hbits(-static_cast<float>(lh));
      qa[9] = hbits(-(L - static_cast<float>(lh)));
      const _Float16 dh = to_half_or_nan(delta);
      da[8] = hbits(-static_cast<float>(dh));
      da[9] = hbits(-(delta - static_cast<float>(dh)));
    } else {
      qa[8] = ninf;
    }
    put_row(ops.qa, qa);
    put_row(ops.doa, da);
  }
  if (n < ops.npk) {
    uint16_t ka[16] = {}, va[16] = {};
    ka[8] = one;
    ka[9] = one;
    va[8] = one;
    va[9] = one;
    if (n < Nk) {
      const int64_t r = n * kH + h;
      const u32x4 kw = *reinterpret_cast<const u32x4*>(k + r * kD);
      const u32x4 vw = *reinterpret_cast<const u32x4*>(v + r * kD);
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        const int wi = d >> 1;
        ka[d] = hbits((d & 1) ? bf16_hi(kw[wi]) : bf16_lo(kw[wi]));
        va[d] = hbits((d & 1) ? bf16_hi(vw[wi]) : bf16_lo(vw[wi]));
      }
    } else {
      ka[10] = ninf;
    }
    put_row(ops.ka, ka);
    put_row(ops.va, va);
#pragma unroll
    for (int d = 0; d < kD; ++d) ops.kt[(static_cast<int64_t>(h) * kD + d) * ops.npk + n] = ka[d];
  }
}

constexpr int kBwdWaves = 4;              // waves per backward workgroup: 4 x 32 nodes, one head pair
constexpr int kKvTable = 64;              // key-outer table entries (codes clamped to NB-1 <= 63)
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kFusedWaves = 8;            // waves per one-pass workgroup: 8 x (1 or 2) x 32 keys, one head pair
constexpr int kFusedThreads = 64 * kFusedWaves;

constexpr int kFusedMaxSets = 2;          // 32-key sets per one-pass wave: 1 or 2 (fused_sets)
constexpr int kFusedMaxBlocks = kFusedWaves * kFusedMaxSets;  // 32-key blocks per one-pass workgroup, at most

// 32-key blocks of dtable partial rows, padded to whole one-pass workgroups of either size
// (a multiple of 16, so of the 4-wave kernels' blocks too); every key-outer kernel covers
// them all, a wave past the last key writing zero rows, so each row is defined whichever ran.
__host__ __device__ constexpr int64_t kv_row_blocks(int64_t npad32) {
  return (npad32 + kFusedMaxBlocks - 1) / kFusedMaxBlocks * kFusedMaxBlocks;
}

// One 32-node tile of backward operands of a head pair, staged into LDS: two
// augmented-row tiles, and for the query-outer kernel a transposed k tile. Each tile is
// 32 rows of 64 bytes (4 chunks of 16 bytes):
//   augmented:  row = slot s holding node a(s) (the MFMA row order), chunk = 2*head + half
//   transposed: row = 8*head + d, chunk = 8-node group
// Chunk k of row r is stored at chunk position k ^ ((r >> 1) & 3), so that the eight
// lanes of one LDS cycle, which read rows 0..7 (or 8..15, ...) at one chunk index,
// hit 8 distinct 16-byte bank groups instead of two.
// The global source is cut into 16-byte chunks x: [0,128) first augmented, [128,256)
// second augmented, [256,320) the transposed tile; thread t moves chunks t, t + 256.
// The key-outer kernels stage the two augmented tiles only and read Q^T and dO^T from
// them transposed (tr_aug_op).
constexpr int kAugHalves = 32 * 32;             // one augmented tile, halves
constexpr int kTrHalves = 2 * kD * 32;          // one transposed tile [2 heads][8][32], halves
constexpr int kStageHalves = 2 * kAugHalves + kTrHalves;  // one buffer of the query-outer's double buffer

struct StageSrc {
  const uint16_t* row0;  // first augmented rows (qa or ka) at node 0, head h0
  const uint16_t* row1;  // second augmented rows (doa or va) at node 0, head h0
  const uint16_t* tr;    // transposed copy at head h0, d 0, node 0 (null when none is staged)
};

// global chunk c of an augmented tile: node = c >> 2, chunk = c & 3 (head = bit 1, half = bit 0)
__device__ __forceinline__ const uint16_t* aug_chunk(const uint16_t* base, int64_t n0, int c) {
  return base + ((n0 + (c >> 2)) * kH + ((c >> 1) & 1)) * 16 + 8 * (c & 1);
}
// global chunk c of a transposed tile: row = c >> 2 (head = c >> 5, d = (c >> 2) & 7), 8 nodes from 8*(c & 3)
__device__ __forceinline__ const uint16_t* tr_chunk(const uint16_t* base, int64_t npad, int64_t n0, int c) {
  return base + ((c >> 5) * kD + ((c >> 2) & 7)) * npad + n0 + 8 * (c & 3);
}
__device__ __forceinline__ const uint16_t* stage_chunk(const StageSrc& s, int64_t npad, int64_t n0, int x) {
  if (x < 128) return aug_chunk(s.row0, n0, x);
  if (x < 256) return aug_chunk(s.row1, n0, x - 128);
  return tr_chunk(s.tr, npad, n0, x - 256);
}
// LDS position (halves) of global chunk x within one stage buffer
__device__ __forceinline__ int stage_pos(int x) {
  if (x < 256) {
    const int c = x & 127;
    return (x >> 7) * kAugHalves + swz(slot_of_node(c >> 2), c & 3);
  }
  const int c = x - 256;  // the transposed tile (chunks 256..319)
  return 2 * kAugHalves + swz(c >> 2, c & 3);
}

template <int kChunks>
constexpr int stage_per_thread() { return (kChunks + kBwdThreads - 1) / kBwdThreads; }

// Per-thread global sources of the staged chunks, one tile after another: the mapping
// from chunk to address (which depends on the chunk's kind) is worked out once, and each
// tile's loads then only advance a pointer (32 nodes: 32*H*16 halves along augmented
// rows, 32 halves along transposed rows).
template <int kChunks>
struct StageCursor {
  const uint16_t* p[stage_per_thread<kChunks>()];
  int64_t step[stage_per_thread<kChunks>()];
  __device__ __forceinline__ void init(const StageSrc& s, int64_t npad, int tid) {
#pragma unroll
    for (int u = 0; u < stage_per_thread<kChunks>(); ++u) {
      const int x = tid + u * kBwdThreads;
      p[u] = x < kChunks ? stage_chunk(s, npad, 0, x) : nullptr;
      step[u] = x < 256 ? 32 * kH * 16 : 32;
    }
  }
  // the next tile's chunks into r
  __device__ __forceinline__ void load_next(s16x8 (&r)[stage_per_thread<kChunks>()], int tid) {
#pragma unroll
    for (int u = 0; u < stage_per_thread<kChunks>(); ++u) {
      if (tid + u * kBwdThreads < kChunks) {
        r[u] = load_h8(p[u]);
        p[u] += step[u];
      }
    }
  }
};

template <int kChunks>
__device__ __forceinline__ void stage_store(uint16_t* buf, const s16x8 (&r)[stage_per_thread<kChunks>()],
                                            int tid) {
#pragma unroll
  for (int u = 0; u < stage_per_thread<kChunks>(); ++u) {
    const int x = tid + u * kBwdThreads;
    if (x < kChunks) *reinterpret_cast<s16x8*>(buf + stage_pos(x)) = r[u];
  }
}

// Staged augmented operand of MFMA row c (node a(c)): head hl, half hp.
__device__ __forceinline__ s16x8 staged_aug(const uint16_t* aug, int c, int hl, int hp) {
  return *reinterpret_cast<const s16x8*>(aug + swz(c, 2 * hl + hp));
}
// Staged transposed operand: head hl, d = m & 7, nodes 8g .. 8g+7.
__device__ __forceinline__ s16x8 staged_tr(const uint16_t* tr, int hl, int m, int g) {
  return *reinterpret_cast<const s16x8*>(tr + swz(hl * kD + (m & 7), g));
}

constexpr int kAugStageHalves = 2 * kAugHalves;  // a stage buffer of the two augmented row tiles only

// Transposed read of an augmented row tile (32 slots x [2 heads][16 halves], swz): in a
// 16-lane group, ds_read_b64_tr_b16 gives lane j element j % 4 of the 8-byte pieces that
// lanes 4e + j / 4 address (e = 0..3). Lane 4e + r addresses node n0 + e, head hl,
// columns 4r .. 4r+3 of the node's 16-half row, so lane j receives nodes n0 .. n0+3 of
// column j: for j < 8 that is d = j, the MFMA row of lane c = j; columns 8..15 (the
// augmented terms) and lanes 16..31 (which repeat lanes 0..15) only feed accumulator rows
// 8..31, which are never stored. n0 = 16 hp + 8 k1 + 4 half; the slot term
// 512 k1 + 256 half is left out here, and with swz's swizzle the rest depends on hl only.
__device__ __forceinline__ int tr_aug_base(int lane, int hl) {
  const int hp = lane >> 5, e = (lane >> 2) & 3, r = lane & 3;
  return 128 * hp + 32 * e + 8 * (2 * (hl ^ hp) + ((r >> 1) ^ (e >> 1))) + 4 * (r & 1);
}
// 8 consecutive nodes 16 hp + 8 k1 .. +7 at the lane's d (rows 0..7), as an MFMA operand
__device__ __forceinline__ s16x8 tr_aug_op(const uint16_t* aug, int base, int k1) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(aug + 512 * k1 + base));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(aug + 512 * k1 + 256 + base));
  return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The same read for a 16x16x32 MFMA whose rows are (key half u, d) = 8u + d and whose
// contraction index is k = 8G + p for lane group G = lane / 16 (nodes 16 (G / 2) + 8 k1 + p):
// that operand is block-diagonal, node k pairing with keys of half G % 2 only. Lane 4e + r of
// group G addresses columns 4 (r % 2) .. +3 of node 4e' + e's row (as above) when r / 2 = G % 2,
// so lanes j = 8u + d of the group receive column d for u = G % 2; otherwise it addresses
// columns 12..15, which are zero in every augmented row (the extra terms sit in columns
// 8..10), so the lanes of the other key half receive zeros.
__device__ __forceinline__ int tr_aug_base16(int lane, int hl) {
  const int G = lane >> 4, hp = lane >> 5, e = (lane >> 2) & 3, r = lane & 3;
  const bool data = (r >> 1) == (G & 1);
  const int hb = data ? 0 : 1, off = data ? 4 * (r & 1) : 4;
  return 128 * hp + 32 * e + 8 * (2 * (hl ^ hp) + (hb ^ (e >> 1))) + off;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_h16x16(s16x8 a, s16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// Backward, step 2 (key-outer). A workgroup is 4 waves = 128 keys x one head pair;
// each wave owns 32 keys (lane c keeps key c for the whole sweep) and all waves share
// each staged query tile (augmented q and dout rows) in LDS, double-buffered. Codes
// come along rows of the transposed code matrix.
// S = Q K^T - lse and dP - delta = dO V^T - delta come out of two augmented MFMAs with
// rows = queries (order a(r)) and columns = keys, so a lane's accumulator entries
// are queries 16*hp + 0..15; then P = exp2(S log2e / sqrt(D)) and dS = P (dP - delta)
// take one multiply each. dV^T += dO^T P and dK^T += Q^T dS contract over those
// queries, Q^T and dO^T read from the staged rows with ds_read_b64_tr_b16. Bucket sums
// of dS go to per-lane LDS bins laid out [bucket][lane][head]
// (no two lanes share an address, so a plain read-add-write suffices; one 8-byte
// read-add-write updates both heads), reduced in a fixed order at the end.
template <bool kAligned>
__global__ __launch_bounds__(kBwdThreads) void bwd_kv_mfma_d8_kernel(
    const uint8_t* __restrict__ spd_t, const float* __restrict__ table, BwdOps ops, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ partial, int64_t N, int64_t Nk, int64_t ldt, int NB, int acc,
    int64_t qchunk, int64_t gstride, int64_t pstride, const uint32_t* __restrict__ gate) {
  // As a rerun of the fused pass (gate given) it returns at once unless that pass met a
  // code beyond its private bins.
  if (gate != nullptr && *gate == 0u) return;
  extern __shared__ __align__(16) unsigned char smem[];
  // workgroup row y of a split launch: queries [y*qchunk, min(N, (y+1)*qchunk)), partial
  // dK, dV at + y*gstride and bucket partials at + y*pstride
  const int64_t ib = static_cast<int64_t>(blockIdx.y) * qchunk;
  N = N - ib < qchunk ? N - ib : qchunk;
  ops.qa += ib * kH * 16;
  ops.doa += ib * kH * 16;
  dk += blockIdx.y * gstride;
  dv += blockIdx.y * gstride;
  partial += blockIdx.y * pstride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float* bins = reinterpret_cast<float*>(smem) + w * (2 * NB * 64);      // [NB][64 lanes][2 heads] per wave
  float2* tb = reinterpret_cast<float2*>(reinterpret_cast<float*>(smem) + kBwdWaves * 2 * NB * 64);  // [64] by code
  uint16_t* stage = reinterpret_cast<uint16_t*>(tb + kKvTable);           // [2][kAugStageHalves]

  const int nkb = static_cast<int>(kv_row_blocks(ops.npk / 32) / kBwdWaves);
  int kb, hpair;
  xcd_map(blockIdx.x, nkb, kb, hpair);
  if (kb < 0) return;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * hpair;
  const int64_t jw = static_cast<int64_t>(kb) * (32 * kBwdWaves) + 32 * w;  // this wave's first key
  const int64_t j = jw + c;
  const bool wave_live = jw < ops.npk;
  const int64_t jj = wave_live ? j : 0;
  const int64_t npad = ops.npq;  // staged tiles are query tiles
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < kKvTable; b += kBwdThreads) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * kLog2e, table[(h0 + 1) * NB + c] * kLog2e);
  }
  for (int x = lane; x < 2 * NB * 64; x += 64) bins[x] = 0.f;
  const s16x8 kb0 = load_h8(ops.ka + (jj * kH + h0) * 16 + 8 * hp);
  const s16x8 kb1 = load_h8(ops.ka + (jj * kH + h0 + 1) * 16 + 8 * hp);
  const s16x8 vb0 = load_h8(ops.va + (jj * kH + h0) * 16 + 8 * hp);
  const s16x8 vb1 = load_h8(ops.va + (jj * kH + h0 + 1) * 16 + 8 * hp);
  f32x16 dv0 = {}, dv1 = {}, dk0 = {}, dk1 = {};
  const uint32_t nbm1 = static_cast<uint32_t>(NB - 1);
  float2* mybins = reinterpret_cast<float2*>(bins) + lane;
  const uint8_t* crow = spd_t + (j < Nk ? j : Nk - 1) * ldt + ib;
  const int64_t cc = 16 * hp;  // this lane's first code column within a tile

  StageSrc src;
  src.row0 = ops.qa + h0 * 16;
  src.row1 = ops.doa + h0 * 16;
  src.tr = nullptr;  // Q^T and dO^T are read transposed from the row tiles
  const int tb_h0 = tr_aug_base(lane, 0), tb_h1 = tr_aug_base(lane, 1);
  const int64_t ntiles = (N + 31) / 32, nfull = N / 32;
  constexpr int kCh = 256;  // qa, doa
  s16x8 sr[stage_per_thread<kCh>()];
  StageCursor<kCh> cursor;
  cursor.init(src, npad, tid);
  cursor.load_next(sr, tid);
  stage_store<kCh>(stage, sr, tid);
  u32x4 cw = nfull > 0 ? codes_at<false, kAligned>(crow, cc, N) : codes_at<true, kAligned>(crow, cc, N);
  wait_vm0();
  __syncthreads();

  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t i0 = t * 32;
    const uint16_t* cur = stage + (t & 1) * kAugStageHalves;
    u32x4 cwn = cw;
    if (t + 1 < ntiles) {
      cursor.load_next(sr, tid);
      cwn = (t + 1 < nfull) ? codes_at<false, kAligned>(crow, i0 + 32 + cc, N)
                            : codes_at<true, kAligned>(crow, i0 + 32 + cc, N);
    }
    if (wave_live) {
      const uint16_t* qa_t = cur;
      const uint16_t* doa_t = cur + kAugHalves;
      uint32_t code[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) code[e] = min(code_byte(cw, e), nbm1);
      // Every LDS read of the tile (bias, then the dK/dV operands) precedes the bin
      // updates in program order: the bins share the LDS array with the table and the
      // stage, so a read placed after a bin store would wait behind it.
      float2 tv[16];  // both heads' log2e-scaled bias, the FMA addends
#pragma unroll
      for (int e = 0; e < 16; ++e) tv[e] = tb[code[e]];
      f32x16 s0 = mfma_h16(staged_aug(qa_t, c, 0, hp), kb0, f32x16{});
      f32x16 s1 = mfma_h16(staged_aug(qa_t, c, 1, hp), kb1, f32x16{});
      f32x16 p0 = mfma_h16(staged_aug(doa_t, c, 0, hp), vb0, f32x16{});
      f32x16 p1 = mfma_h16(staged_aug(doa_t, c, 1, hp), vb1, f32x16{});
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pa = __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, tv[e].x));
        const float pb = __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, tv[e].y));
        s0[e] = pa;
        s1[e] = pb;
        p0[e] *= pa;
        p1[e] *= pb;
      }
#pragma unroll
      for (int k1 = 0; k1 < 2; ++k1) {
        dv0 = mfma_h16(tr_aug_op(doa_t, tb_h0, k1), pack_f16x8(s0, 8 * k1), dv0);
        dv1 = mfma_h16(tr_aug_op(doa_t, tb_h1, k1), pack_f16x8(s1, 8 * k1), dv1);
        dk0 = mfma_h16(tr_aug_op(qa_t, tb_h0, k1), pack_f16x8(p0, 8 * k1), dk0);
        dk1 = mfma_h16(tr_aug_op(qa_t, tb_h1, k1), pack_f16x8(p1, 8 * k1), dk1);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float2 bin = mybins[code[e] * 64];
        bin.x += p0[e];
        bin.y += p1[e];
        mybins[code[e] * 64] = bin;
      }
    }
    if (t + 1 < ntiles) stage_store<kCh>(stage + ((t + 1) & 1) * kAugStageHalves, sr, tid);
    cw = cwn;
    __syncthreads();
  }
  if (wave_live && j < Nk) {
    const float rs = 1.f / sqd;
    float* kp = dk + j * kHD + h0 * kD + 4 * hp;
    float* vp = dv + j * kHD + h0 * kD + 4 * hp;
    store4(kp, make_float4(dk0[0] * rs, dk0[1] * rs, dk0[2] * rs, dk0[3] * rs), acc);
    store4(kp + kD, make_float4(dk1[0] * rs, dk1[1] * rs, dk1[2] * rs, dk1[3] * rs), acc);
    store4(vp, make_float4(dv0[0], dv0[1], dv0[2], dv0[3]), acc);
    store4(vp + kD, make_float4(dv1[0], dv1[1], dv1[2], dv1[3]), acc);
  }
  // per-wave bins -> one partial row per 32-key block and head; a wave past the last
  // key block writes its (zero) bins too, so every partial row is defined
  for (int x = lane; x < 2 * NB; x += 64) {
    const int hl = x / NB, b = x - hl * NB;
    const float* srcb = bins + b * 128 + hl;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains, fixed order
#pragma unroll
    for (int l = 0; l < 64; l += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) s4[u] += srcb[2 * (l + u)];
    }
    const float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    partial[((jw / 32) * kH + h0 + hl) * NB + b] = sum;
  }
}

// Backward in one pass (key-outer with dQ): the key-outer kernel's work and, from the
// same probabilities, the queries' gradient, so the query-outer pass (a third sweep
// over the codes with a third exp per entry) is not needed. The dK/dV contractions are
// those of bwd_kv_mfma_d8_kernel, with 8-wave workgroups of one head pair, one workgroup per
// CU: each wave owns kSets sets of 32 keys and runs them one after the other on every staged
// query tile (two sets, 512 keys per workgroup, once those workgroups alone fill the GPU;
// one set, 256 keys, below: fused_sets). The tile, its barrier and the cross-wave dQ sum
// then serve 2 or 4 times the keys of a 4-wave, one-set workgroup, and each workgroup's dQ
// partial covers all its keys (0.54 GB of partials at N = 32768 instead of 2.1 GB at 128
// keys). dK and dV contract on 16x16x32 MFMAs, which leaves the registers for a second set.
// Only the two augmented row tiles are staged (4 KB per tile): the dK^T and dV^T
// contractions read Q^T and dO^T from them with ds_read_b64_tr_b16 (tr_aug_base16). Per
// 32-query tile each of a wave's sets also:
//  * writes its packed dS (f16, both heads, 32 keys x 32 queries) row by row into the
//    wave's LDS buffer [head][key][query] and reads it back transposed with ds_read_b64_tr_b16:
//    lane l of a 16-lane group receives element l%4 of the 8-byte chunks that lanes
//    4e + l/4 address (e = 0..3), so each lane's address names a 4-query chunk of one key
//    row and its result holds 4 keys of one query;
//  * contracts those over its 32 keys against K^T (held in registers for the whole
//    sweep: the wave's keys do not change), dQ^T[d][query] += K^T[d][key] dS^T[key][query];
//  * adds its result to the wave's, which goes to LDS beside the other waves' (summed in a
//    fixed order), and the workgroup writes
//    one dQ partial row per query for its 512 keys; the backward's last kernel sums the
//    partials of all key blocks in order, so the result stays bitwise reproducible.
// dtable bins are lane-private for codes 0..15 only (8 KB per wave): a lane that meets a
// larger code raises *flag (cleared by the prep kernel), and the three-pass kernels,
// launched after this one with that flag as their gate, then redo the backward.
constexpr int kFusedBins = 16;

constexpr int kDsHalves = 2 * 32 * 32;            // one wave's dS buffer: [head][key][query]
constexpr int kRedRow = 20;                       // floats per query of a dQ slot (16 used)
constexpr int kRedFloats = kFusedWaves * 32 * kRedRow;  // [wave][query][head][d] dQ contributions

// Position (halves) of queries 8k..8k+7 of key row r in a dS buffer: 64-byte rows whose
// 16-byte chunks are XOR-swizzled by (r >> 1) & 3, so that the eight lanes of one write
// cycle (rows r..r+7 at one chunk) and the sixteen 8-byte transposed reads of one lane
// group (rows r0..r0+3, r0 a multiple of 4, at four chunk offsets) hit distinct banks.
__device__ __forceinline__ int ds_pos(int r, int k) { return r * 32 + 8 * (k ^ ((r >> 1) & 3)); }

// One 32-key set of a one-pass wave: its keys' operands, its dK/dV accumulators and its
// code row (the keys stay the wave's for the whole sweep).
struct FusedSet {
  s16x8 kb0, kb1, vb0, vb1;  // augmented k and v rows of both heads (score MFMA operands)
  s16x8 kt[2];               // K^T operands of the dQ contractions (16-key halves)
  f32x4 dv0, dv1, dk0, dk1;  // dV^T and dK^T of both heads (tr_aug_base16 layout)
  const uint8_t* crow;       // this lane's code row (its key, the launch's query range)
  u32x4 cw, cwn;             // codes of the current and the next query tile
};

template <bool kAligned, int kSets>
__global__ __launch_bounds__(kFusedThreads) void bwd_fused_mfma_d8_kernel(
    const uint8_t* __restrict__ spd_t, const float* __restrict__ table, BwdOps ops, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ partial, float* __restrict__ dqpart, int64_t N, int64_t Nk,
    int64_t ldt, int NB, int64_t qchunk, int64_t gstride, int64_t pstride, int64_t dqstride,
    uint32_t* __restrict__ flag) {
  // Five separate LDS arrays (144.5 KB): as distinct objects the compiler knows that
  // accesses to different ones never overlap, so it may interleave the bin updates with
  // the other arrays' reads and writes instead of keeping all of them in program order.
  __shared__ __align__(16) float2 bins[kFusedWaves * kFusedBins * 64];  // [wave][code][lane]
  __shared__ __align__(16) float2 tb[kKvTable];                         // by code
  __shared__ __align__(16) uint16_t stage[2 * kAugStageHalves];         // [2][kAugStageHalves]
  __shared__ __align__(16) uint16_t dsbuf[kFusedWaves * kDsHalves];     // [wave][kDsHalves]
  __shared__ __align__(16) float red[2 * kRedFloats];                   // [2][kRedFloats]
  const int64_t ib = static_cast<int64_t>(blockIdx.y) * qchunk;
  N = N - ib < qchunk ? N - ib : qchunk;
  ops.qa += ib * kH * 16;
  ops.doa += ib * kH * 16;
  dk += blockIdx.y * gstride;
  dv += blockIdx.y * gstride;
  partial += blockIdx.y * pstride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float2* mybins = bins + w * (kFusedBins * 64) + lane;
  uint16_t* mydst = dsbuf + w * kDsHalves;

  constexpr int kBlocks = kFusedWaves * kSets;  // 32-key blocks per workgroup
  const int nkb = static_cast<int>(kv_row_blocks(ops.npk / 32) / kBlocks);
  int kb, hpair;
  xcd_map(blockIdx.x, nkb, kb, hpair);
  if (kb < 0) return;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * hpair;
  // the wave's keys: set s (s < kSets) holds the 32 keys from jw + 32 s
  const int64_t jw = static_cast<int64_t>(kb) * (32 * kBlocks) + 32 * kSets * w;
  const int nlive = kSets == 2 && jw + 32 < ops.npk ? 2 : (jw < ops.npk ? 1 : 0);  // live sets (wave-uniform)
  const int64_t npad = ops.npq;
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < kKvTable; b += kFusedThreads) {
    const int cb = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + cb] * kLog2e, table[(h0 + 1) * NB + cb] * kLog2e);
  }
  for (int b = 0; b < kFusedBins; ++b) mybins[b * 64] = make_float2(0.f, 0.f);
  // dQ contractions on 16x16x32 MFMAs: rows m = (head m / 8, d m % 8) of both heads,
  // columns 16 queries, k = 8G + p for lane group G = lane / 16: head G / 2 and key
  // 16u + 8 (G % 2) + p of the set (u = 0, 1: its two 16-key halves). The K^T operand is
  // zero where a row's head is not the k-group's, and is the same every tile.
  const int G = lane >> 4, m16 = lane & 15;
  const int64_t cc = 16 * hp;
  FusedSet set[kSets];
#pragma unroll
  for (int si = 0; si < kSets; ++si) {
    FusedSet& st = set[si];
    const int64_t js = jw + 32 * si;
    const bool live = js < ops.npk;
    const int64_t jj = live ? js + c : 0, jsl = live ? js : 0;
    st.kb0 = load_h8(ops.ka + (jj * kH + h0) * 16 + 8 * hp);
    st.kb1 = load_h8(ops.ka + (jj * kH + h0 + 1) * 16 + 8 * hp);
    st.vb0 = load_h8(ops.va + (jj * kH + h0) * 16 + 8 * hp);
    st.vb1 = load_h8(ops.va + (jj * kH + h0 + 1) * 16 + 8 * hp);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      st.kt[u] = (m16 >> 3) == (G >> 1)
                     ? load_h8(ops.kt + (static_cast<int64_t>(h0 + (m16 >> 3)) * kD + (m16 & 7)) * ops.npk + jsl +
                               16 * u + 8 * (G & 1))
                     : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    st.dv0 = st.dv1 = st.dk0 = st.dk1 = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t j = js + c;
    st.crow = spd_t + (j < Nk ? j : Nk - 1) * ldt + ib;
  }
  const uint32_t bound = static_cast<uint32_t>(min(NB - 1, kFusedBins - 1));
  uint32_t over = 0u;
  // transposed-read address of this lane (group G, e4 = (lane % 16) / 4, j4 = lane % 4),
  // for query half qh, key half u and read s: head G / 2, key row r = 16u + 8 (G % 2) + 4s
  // + e4, queries 16 qh + 4 j4 .. +3; a lane of group G then receives 4 keys of head G / 2.
  // With ds_pos's swizzle ((r >> 1) & 3 = 2s + e4 / 2) that is tr_base + 512u + 128s +
  // 16 (qh ^ s) halves.
  const int e4 = (lane & 15) >> 2, j4 = lane & 3;
  const int tr_base = (G >> 1) * 32 * 32 + (8 * (G & 1) + e4) * 32 + 8 * ((j4 >> 1) ^ (e4 >> 1)) + 4 * (j4 & 1);
  // this thread's share of the workgroup's dQ sum: one value of [query][head][d]
  const int rq = tid >> 4, rh = (tid >> 3) & 1, rd = tid & 7;

  StageSrc src;
  src.row0 = ops.qa + h0 * 16;
  src.row1 = ops.doa + h0 * 16;
  src.tr = nullptr;  // no transposed tile is staged
  const int tb_h0 = tr_aug_base16(lane, 0), tb_h1 = tr_aug_base16(lane, 1);
  const int64_t ntiles = (N + 31) / 32, nfull = N / 32;
  constexpr int kCh = 256;  // qa, doa
  s16x8 sr[stage_per_thread<kCh>()];
  // The sweep starts at query tile rot and wraps around. Code rows are N bytes apart, so
  // the code lines that the key blocks of one XCD read at one time all sat at the same
  // column offset, in the same few L2 sets, and were fetched again and again. Those key
  // blocks (kb = 8i + xcd) now start 4 tiles (one 128-byte line) apart, i mod 8: their
  // lines fall in different sets, while the staged query rows they read stay within a
  // window of 32 tiles that L2 holds for all of them. The 4 head pairs of a key block share
  // its rotation, and its code lines.
  const int64_t rot = static_cast<int64_t>(((kb / kXcds) % 8) * 4) % ntiles;
  auto wrap = [&](int64_t x) { return x < ntiles ? x : x - ntiles; };
  const uint16_t* sp0 = tid < kCh ? stage_chunk(src, npad, 0, tid) : nullptr;  // this thread's staged chunk
  auto stage_load = [&](int64_t tt) {
    if (tid < kCh) sr[0] = load_h8(sp0 + tt * (32 * kH * 16));
  };
  auto codes_of = [&](const FusedSet& st, int64_t tt) {
    return tt < nfull ? codes_at<false, kAligned>(st.crow, tt * 32 + cc, N) : codes_at<true, kAligned>(st.crow, tt * 32 + cc, N);
  };
  stage_load(rot);
  stage_store<kCh>(stage, sr, tid);
#pragma unroll
  for (int si = 0; si < kSets; ++si) set[si].cw = codes_of(set[si], rot);
  float* dqw = dqpart + static_cast<int64_t>(kb) * dqstride + (ib + rq) * kHD + (h0 + rh) * kD + rd;
  // the workgroup's dQ for tile tt (iteration t) from the eight waves' contributions, in wave order
  auto reduce_dq = [&](int64_t tt, int64_t t) {
    const float* slot = red + (t & 1) * kRedFloats + rq * kRedRow + rh * 8 + rd;
    float acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < kFusedWaves; ++ww) acc += slot[ww * (32 * kRedRow)];
    const float rs = 1.f / sqd;  // dQ = dS K / sqrt(D)
    if (tt * 32 + rq < N) dqw[tt * 32 * kHD] = acc * rs;
  };
  wait_vm0();
  __syncthreads();

  // One 32-key set's work on the staged query tile: scores, P and dS, the dtable bins, the
  // dK/dV contractions, and its share of the tile's dQ^T (added to dq).
  auto set_tile = [&](FusedSet& st, const uint16_t* cur, f32x4(&dq)[2]) __attribute__((always_inline)) {
    const uint16_t* qa_t = cur;
    const uint16_t* doa_t = cur + kAugHalves;
    const u32x4 cw = st.cw;
    over |= (cw[0] | cw[1] | cw[2] | cw[3]) & 0xF0F0F0F0u;
    uint32_t code[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) code[e] = min(code_byte(cw, e), bound);
    // All 16 bias reads are issued together, before the bin updates: one LDS round trip
    // for the tile's exp arguments instead of one per entry.
    float2 tv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) tv[e] = tb[code[e]];
    f32x16 s0 = mfma_h16(staged_aug(qa_t, c, 0, hp), st.kb0, f32x16{});
    f32x16 s1 = mfma_h16(staged_aug(qa_t, c, 1, hp), st.kb1, f32x16{});
    f32x16 p0 = mfma_h16(staged_aug(doa_t, c, 0, hp), st.vb0, f32x16{});
    f32x16 p1 = mfma_h16(staged_aug(doa_t, c, 1, hp), st.vb1, f32x16{});
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pa = __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, tv[e].x));
      const float pb = __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, tv[e].y));
      s0[e] = pa;
      s1[e] = pb;
      p0[e] *= pa;
      p1[e] *= pb;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float2 bin = mybins[code[e] * 64];
      bin.x += p0[e];
      bin.y += p1[e];
      mybins[code[e] * 64] = bin;
    }
    const s16x8 d0a = pack_f16x8(p0, 0), d0b = pack_f16x8(p0, 8);
    const s16x8 d1a = pack_f16x8(p1, 0), d1b = pack_f16x8(p1, 8);
    // dS rows of this lane's key: queries 16hp .. 16hp+15 of both heads (the wave's next
    // set reuses the buffer: the LDS operations of one wave complete in order)
    *reinterpret_cast<s16x8*>(mydst + ds_pos(c, 2 * hp)) = d0a;
    *reinterpret_cast<s16x8*>(mydst + ds_pos(c, 2 * hp + 1)) = d0b;
    *reinterpret_cast<s16x8*>(mydst + 32 * 32 + ds_pos(c, 2 * hp)) = d1a;
    *reinterpret_cast<s16x8*>(mydst + 32 * 32 + ds_pos(c, 2 * hp + 1)) = d1b;
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1) {
      st.dv0 = mfma_h16x16(tr_aug_op(doa_t, tb_h0, k1), pack_f16x8(s0, 8 * k1), st.dv0);
      st.dv1 = mfma_h16x16(tr_aug_op(doa_t, tb_h1, k1), pack_f16x8(s1, 8 * k1), st.dv1);
      st.dk0 = mfma_h16x16(tr_aug_op(qa_t, tb_h0, k1), k1 ? d0b : d0a, st.dk0);
      st.dk1 = mfma_h16x16(tr_aug_op(qa_t, tb_h1, k1), k1 ? d1b : d1a, st.dk1);
    }
    // dS^T operands: lane (query 16qh + m16, group G) gets keys 16u + 8 (G % 2) .. +7 of
    // head G / 2, from two transposed reads of 4 keys each
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lds4;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t* rb = mydst + tr_base + 512 * u;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(rb + 16 * qh));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(rb + 128 + 16 * (qh ^ 1)));
        const s16x8 bop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dq[qh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, st.kt[u]),
                                                        __builtin_bit_cast(f16x8, bop), dq[qh], 0, 0, 0);
      }
    }
  };

  // The query sweep of a wave with kLive live sets (2, 1 or 0: only the last workgroup's
  // waves can have fewer than 2); the sets' work on a tile runs one after the other.
  auto sweep = [&](auto live_tag) __attribute__((always_inline)) {
    constexpr int kLive = decltype(live_tag)::value;
    for (int64_t t = 0; t < ntiles; ++t) {
      const int64_t tt = wrap(t + rot), tn = wrap(t + 1 + rot);  // this tile and the next
      const uint16_t* cur = stage + (t & 1) * kAugStageHalves;
      if (t + 1 < ntiles) {
        stage_load(tn);
#pragma unroll
        for (int si = 0; si < kLive; ++si) set[si].cwn = codes_of(set[si], tn);
      }
      // rows 4G .. 4G+3 = head G / 2, d 4 (G % 2) .. +3 of query 16qh + m16: this lane's dQ^T
      f32x4 dq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int si = 0; si < kLive; ++si) set_tile(set[si], cur, dq);
      // the workgroup's dQ for this tile: every wave's contribution, summed in wave order.
      // The contributions of tile t go to buffer t & 1 and one barrier per tile orders
      // everything: after it, tile t's contributions and tile t+1's stage are complete, and
      // the buffers written next (contributions of t+1, stage of t+2) were last read before it.
      float* myred = red + (t & 1) * kRedFloats + w * (32 * kRedRow) + m16 * kRedRow + 8 * (G >> 1) + 4 * (G & 1);
      *reinterpret_cast<float4*>(myred) = make_float4(dq[0][0], dq[0][1], dq[0][2], dq[0][3]);
      *reinterpret_cast<float4*>(myred + 16 * kRedRow) = make_float4(dq[1][0], dq[1][1], dq[1][2], dq[1][3]);
      if (t + 1 < ntiles) stage_store<kCh>(stage + ((t + 1) & 1) * kAugStageHalves, sr, tid);
#pragma unroll
      for (int si = 0; si < kLive; ++si) set[si].cw = set[si].cwn;
      __syncthreads();
      reduce_dq(tt, t);
    }
  };
  if (kSets == 2 && nlive == 2)
    sweep(std::integral_constant<int, kSets>{});
  else if (nlive >= 1)
    sweep(std::integral_constant<int, 1>{});
  else
    sweep(std::integral_constant<int, 0>{});

  const float rs = 1.f / sqd;
  const int dg = 4 * ((lane >> 4) & 1);
#pragma unroll
  for (int si = 0; si < kSets; ++si) {
    const FusedSet& st = set[si];
    const int64_t jo = jw + 32 * si + 16 * hp + (lane & 15);  // this lane's key of the set's dK/dV
    if (si < nlive && jo < Nk) {
      float* kp = dk + jo * kHD + h0 * kD + dg;
      float* vp = dv + jo * kHD + h0 * kD + dg;
      store4(kp, make_float4(st.dk0[0] * rs, st.dk0[1] * rs, st.dk0[2] * rs, st.dk0[3] * rs), 0);
      store4(kp + kD, make_float4(st.dk1[0] * rs, st.dk1[1] * rs, st.dk1[2] * rs, st.dk1[3] * rs), 0);
      store4(vp, make_float4(st.dv0[0], st.dv0[1], st.dv0[2], st.dv0[3]), 0);
      store4(vp + kD, make_float4(st.dv1[0], st.dv1[1], st.dv1[2], st.dv1[3]), 0);
    }
  }
  if (NB > kFusedBins && over != 0u) *flag = 1u;  // every writer stores the same value
  // the wave's bins cover all its 32-key blocks: their sum goes to the first block's
  // partial row, zeros to the second's (two sets)
  for (int x = lane; x < 2 * NB; x += 64) {
    const int hl = x / NB, b = x - hl * NB;
    float sum = 0.f;
    if (b < kFusedBins) {
      const float* srcb = reinterpret_cast<const float*>(bins + w * (kFusedBins * 64)) + b * 128 + hl;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains, fixed order
#pragma unroll
      for (int l = 0; l < 64; l += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s4[u] += srcb[2 * (l + u)];
      }
      sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    partial[((jw / 32) * kH + h0 + hl) * NB + b] = sum;
    if (kSets == 2) partial[((jw / 32 + 1) * kH + h0 + hl) * NB + b] = 0.f;
  }
}

// Backward, step 3 (query-outer). A workgroup is 4 waves = 128 queries x one head
// pair (lane c keeps query c); all waves share each staged key tile (augmented k and
// v rows, transposed k) in LDS, double-buffered. S^T - lse and dP^T - delta come from
// the augmented MFMAs and dQ^T += K^T dS^T per key tile.
template <bool kAligned>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_mfma_d8_kernel(const uint8_t* __restrict__ spd,
                                                                      const float* __restrict__ table,
                                                                      BwdOps ops, float* __restrict__ dq,
                                                                      int64_t N, int64_t Nk, int64_t ldc, int NB,
                                                                      int acc, int64_t kchunk, int64_t gstride,
                                                                      const uint32_t* __restrict__ gate) {
  if (gate != nullptr && *gate == 0u) return;  // rerun of the fused pass, not needed
  __shared__ float2 tb[256];  // both heads' bias for each byte value
  __shared__ __align__(16) uint16_t stage[2 * kStageHalves];
  // workgroup row y of a split launch: keys [y*kchunk, min(Nk, (y+1)*kchunk)), partial dQ
  // at dq + y*gstride
  const int64_t jb = static_cast<int64_t>(blockIdx.y) * kchunk;
  Nk = Nk - jb < kchunk ? Nk - jb : kchunk;
  ops.ka += jb * kH * 16;
  ops.va += jb * kH * 16;
  ops.kt += jb;
  spd += jb;
  dq += blockIdx.y * gstride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int npad32 = static_cast<int>(ops.npq / 32);
  const int nqb = (npad32 + kBwdWaves - 1) / kBwdWaves;
  int qb, hpair;
  xcd_map(blockIdx.x, nqb, qb, hpair);
  if (qb < 0) return;
  const int c = lane & 31, hp = lane >> 5;
  const int h0 = 2 * hpair;
  const int64_t iw = static_cast<int64_t>(qb) * (32 * kBwdWaves) + 32 * w;
  const int64_t i = iw + c;
  const bool wave_live = iw < ops.npq;
  const int64_t ii = wave_live ? i : 0;
  const bool qvalid = i < N;
  const int64_t npad = ops.npk;  // staged tiles are key tiles
  const float sqd = sqrtf(static_cast<float>(kD));
  const float sc2 = kLog2e / sqd;

  for (int b = tid; b < 256; b += kBwdThreads) {
    const int c = min(b, NB - 1);
    tb[b] = make_float2(table[h0 * NB + c] * kLog2e, table[(h0 + 1) * NB + c] * kLog2e);
  }
  const s16x8 qb0 = load_h8(ops.qa + (ii * kH + h0) * 16 + 8 * hp);
  const s16x8 qb1 = load_h8(ops.qa + (ii * kH + h0 + 1) * 16 + 8 * hp);
  const s16x8 ob0 = load_h8(ops.doa + (ii * kH + h0) * 16 + 8 * hp);
  const s16x8 ob1 = load_h8(ops.doa + (ii * kH + h0 + 1) * 16 + 8 * hp);
  f32x16 dq0 = {}, dq1 = {};
  const uint8_t* srow = spd + (qvalid ? i : N - 1) * ldc;
  const int64_t cc = 16 * hp;

  StageSrc src;
  src.row0 = ops.ka + h0 * 16;
  src.row1 = ops.va + h0 * 16;
  src.tr = ops.kt + static_cast<int64_t>(h0) * kD * npad;
  const int64_t ntiles = (Nk + 31) / 32, nfull = Nk / 32;
  constexpr int kCh = 320;  // ka, va, k^T
  s16x8 sr[stage_per_thread<kCh>()];
  StageCursor<kCh> cursor;
  cursor.init(src, npad, tid);
  cursor.load_next(sr, tid);
  stage_store<kCh>(stage, sr, tid);
  u32x4 cw = nfull > 0 ? codes_at<false, kAligned>(srow, cc, Nk) : codes_at<true, kAligned>(srow, cc, Nk);
  wait_vm0();
  __syncthreads();

  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t j0 = t * 32;
    const uint16_t* cur = stage + (t & 1) * kStageHalves;
    u32x4 cwn = cw;
    if (t + 1 < ntiles) {
      cursor.load_next(sr, tid);
      cwn = (t + 1 < nfull) ? codes_at<false, kAligned>(srow, j0 + 32 + cc, Nk)
                            : codes_at<true, kAligned>(srow, j0 + 32 + cc, Nk);
    }
    if (wave_live) {
      const uint16_t* ka_t = cur;
      const uint16_t* va_t = cur + kAugHalves;
      const uint16_t* kt_t = cur + 2 * kAugHalves;
      f32x16 s0 = mfma_h16(staged_aug(ka_t, c, 0, hp), qb0, f32x16{});
      f32x16 s1 = mfma_h16(staged_aug(ka_t, c, 1, hp), qb1, f32x16{});
      f32x16 p0 = mfma_h16(staged_aug(va_t, c, 0, hp), ob0, f32x16{});
      f32x16 p1 = mfma_h16(staged_aug(va_t, c, 1, hp), ob1, f32x16{});
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float2 t = tb[code_byte(cw, e)];  // both heads' log2e-scaled bias: the FMA addends
        p0[e] *= __builtin_amdgcn_exp2f(fmaf(s0[e], sc2, t.x));
        p1[e] *= __builtin_amdgcn_exp2f(fmaf(s1[e], sc2, t.y));
      }
#pragma unroll
      for (int k1 = 0; k1 < 2; ++k1) {
        const int g = 2 * hp + k1;
        dq0 = mfma_h16(staged_tr(kt_t, 0, c, g), pack_f16x8(p0, 8 * k1), dq0);
        dq1 = mfma_h16(staged_tr(kt_t, 1, c, g), pack_f16x8(p1, 8 * k1), dq1);
      }
    }
    if (t + 1 < ntiles) stage_store<kCh>(stage + ((t + 1) & 1) * kStageHalves, sr, tid);
    cw = cwn;
    __syncthreads();
  }
  if (wave_live && qvalid) {
    const float rs = 1.f / sqd;
    float* qp = dq + i * kHD + h0 * kD + 4 * hp;
    store4(qp, make_float4(dq0[0] * rs, dq0[1] * rs, dq0[2] * rs, dq0[3] * rs), acc);
    store4(qp + kD, make_float4(dq1[0] * rs, dq1[1] * rs, dq1[2] * rs, dq1[3] * rs), acc);
  }
}

size_t kv_mfma_lds(int NB) {
  return 4ull * kBwdWaves * 2 * NB * 64 + sizeof(float2) * kKvTable + 2ull * 2 * kAugStageHalves;
}

}  // namespace

bool mfma_supported(int H, int D, int dtype) { return H == kH && (D == 8 || D == 32) && dtype == 1; }

int64_t mfma_npad(int64_t N) { return (N + 31) / 32 * 32; }

// dtable partial rows: one per 32-key block (padded to whole one-pass workgroups)
int64_t mfma_kv_blocks(int64_t Nk) { return kv_row_blocks(mfma_npad(Nk) / 32); }

// 32-key sets per wave of the one-pass backward: two once the 512-key workgroups alone fill
// the GPU (64 key blocks x 4 head pairs = 256 CUs), one below, where workgroups of 256 keys
// give the launch twice as many workgroups for the same query split.
int fused_sets(int64_t Nk) { return (mfma_npad(Nk) + 511) / 512 >= 64 ? 2 : 1; }

// dQ partials of the one-pass backward: one per workgroup (256 or 512 keys)
int64_t mfma_fused_dq_parts(int64_t Nk) { return mfma_kv_blocks(Nk) / (kFusedWaves * fused_sets(Nk)); }

size_t mfma_ops_bytes(int64_t N, int64_t Nk) {
  const size_t npq = static_cast<size_t>(mfma_npad(N)), npk = static_cast<size_t>(mfma_npad(Nk));
  return 2 * (npq + npk) * kH * 16 * 2 + npk * kH * kD * 2;
}

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t s) {
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
  const dim3 grid(static_cast<unsigned>(xcd_grid(static_cast<int>((a.N + 32 * kFwdWaves - 1) / (32 * kFwdWaves)))),
                  static_cast<unsigned>(sp.S));
  trace_begin(kTraceFwd, s);
  if (codes_aligned(a.spd, a.ld))
    hipLaunchKernelGGL(fwd_mfma_d8_kernel<true>, grid, dim3(64 * kFwdWaves), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table, out,
                       lse, a.N, a.Nk, a.ld, a.NB, sp.chunk, rows * kD, rows);
  else
    hipLaunchKernelGGL(fwd_mfma_d8_kernel<false>, grid, dim3(64 * kFwdWaves), 0, s, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.spd, a.table, out,
                       lse, a.N, a.Nk, a.ld, a.NB, sp.chunk, rows * kD, rows);
  const hipError_t e = hipGetLastError();
  trace_end(kTraceFwd, s);
  if (e != hipSuccess || !part) return e;
  return launch_merge_splits(out, lse, sp.S, a.out, a.lse, rows, kD, a.acc, s);
}

hipError_t launch_bwd_mfma(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  float* partial = reinterpret_cast<float*>(ws + w.partial_off);
  BwdOps ops;
  ops.npq = mfma_npad(a.N);
  ops.npk = mfma_npad(a.Nk);
  const size_t hq = static_cast<size_t>(ops.npq) * kH, hk = static_cast<size_t>(ops.npk) * kH;
  uint16_t* base = reinterpret_cast<uint16_t*>(ws + w.ops_off);
  ops.qa = base;
  ops.doa = ops.qa + hq * 16;
  ops.ka = ops.doa + hq * 16;
  ops.va = ops.ka + hk * 16;
  ops.kt = ops.va + hk * 16;

  uint32_t* flag = reinterpret_cast<uint32_t*>(ws + w.flag_off);
  trace_begin(kTraceBwdDelta, s);
  const int64_t nmax = std::max(ops.npq, ops.npk);
  hipLaunchKernelGGL(bwd_prep_mfma_d8_kernel, dim3(static_cast<unsigned>((nmax * kH + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.out, static_cast<const uint16_t*>(a.dout), a.lse, ops,
                     a.N, a.Nk, flag);
  hipError_t e = hipGetLastError();
  trace_end(kTraceBwdDelta, s);
  if (e != hipSuccess) return e;

  // key-outer: split over query ranges writes partial dK, dV ([2][S][Nk*H*D] in the
  // workspace) that are summed afterwards; unsplit it writes (or adds) directly
  const dim3 block(kBwdThreads);
  const int64_t nk_el = a.Nk * kHD, nq_el = a.N * kHD;
  const bool kv_split = w.kv.S > 1;
  float* dkp = kv_split ? reinterpret_cast<float*>(ws + w.dkv_off) : a.dk;
  float* dvp = kv_split ? dkp + static_cast<size_t>(w.kv.S) * nk_el : a.dv;
  const int kv_acc = kv_split ? 0 : (a.acc & kAccDkv);
  const int64_t pstride = w.n_kv_blocks * kH * a.NB;
  const int nkb = static_cast<int>(mfma_kv_blocks(a.Nk) / kBwdWaves);
  const dim3 kgrid(static_cast<unsigned>(xcd_grid(nkb)), static_cast<unsigned>(w.kv.S));
  const bool kv_aligned = codes_aligned(a.spd_t, a.ld_t);
  const SumSplits none{nullptr, nullptr, 0, 0, 0};
  const int dkv = a.acc & kAccDkv;
  const SumSplits sk = kv_split ? SumSplits{dkp, a.dk, nk_el, w.kv.S, dkv} : none;
  const SumSplits sv = kv_split ? SumSplits{dvp, a.dv, nk_el, w.kv.S, dkv} : none;

  // One pass when every output is overwritten: dK, dV, dtable partials and per-key-block
  // dQ partials, then one launch that sums the partials in order. If a code fell outside
  // the pass's private bins, the three-pass kernels after it (gated on the flag) redo the
  // backward; with NB <= kFusedBins no code can, and they are not launched.
  const bool fused = w.fused && a.acc == 0;
  const uint32_t* gate = nullptr;
  if (fused) {
    float* dqpart = reinterpret_cast<float*>(ws + w.dqf_off);
    const int nfb = static_cast<int>(mfma_fused_dq_parts(a.Nk));
    const dim3 fgrid(static_cast<unsigned>(xcd_grid(nfb)), static_cast<unsigned>(w.kv.S));
    trace_begin(kTraceBwdFused, s);
    auto fused_kernel = fused_sets(a.Nk) == 2
                            ? (kv_aligned ? bwd_fused_mfma_d8_kernel<true, 2> : bwd_fused_mfma_d8_kernel<false, 2>)
                            : (kv_aligned ? bwd_fused_mfma_d8_kernel<true, 1> : bwd_fused_mfma_d8_kernel<false, 1>);
    hipLaunchKernelGGL(fused_kernel, fgrid, dim3(kFusedThreads), 0, s, a.spd_t, a.table, ops, dkp, dvp, partial,
                       dqpart, a.N, a.Nk, a.ld_t, a.NB, w.kv.chunk, nk_el, pstride, nq_el, flag);
    e = hipGetLastError();
    trace_end(kTraceBwdFused, s);
    if (e != hipSuccess) return e;
    const SumSplits sqf{dqpart, a.dq, nq_el, nfb, 0};
    e = launch_bwd_finish(sk, sv, sqf, partial, a.dtable, w.kv.S * w.n_kv_blocks, kH * a.NB, 0, s);
    if (e != hipSuccess || a.NB <= kFusedBins) return e;
    gate = flag;
  }

  const size_t lds = kv_mfma_lds(a.NB);
  e = allow_lds_mfma(bwd_kv_mfma_d8_kernel<true>, lds);
  if (e == hipSuccess) e = allow_lds_mfma(bwd_kv_mfma_d8_kernel<false>, lds);
  if (e != hipSuccess) return e;
  trace_begin(kTraceBwdKv, s);
  if (kv_aligned)
    hipLaunchKernelGGL(bwd_kv_mfma_d8_kernel<true>, kgrid, block, lds, s, a.spd_t, a.table, ops, dkp, dvp, partial,
                       a.N, a.Nk, a.ld_t, a.NB, kv_acc, w.kv.chunk, nk_el, pstride, gate);
  else
    hipLaunchKernelGGL(bwd_kv_mfma_d8_kernel<false>, kgrid, block, lds, s, a.spd_t, a.table, ops, dkp, dvp, partial,
                       a.N, a.Nk, a.ld_t, a.NB, kv_acc, w.kv.chunk, nk_el, pstride, gate);
  e = hipGetLastError();
  trace_end(kTraceBwdKv, s);
  if (e != hipSuccess) return e;

  const bool q_split = w.q.S > 1;
  float* dqp = q_split ? reinterpret_cast<float*>(ws + w.dq_off) : a.dq;
  const int q_acc = q_split ? 0 : (a.acc & kAccDq);
  const int nqb = static_cast<int>((ops.npq / 32 + kBwdWaves - 1) / kBwdWaves);
  const dim3 qgrid(static_cast<unsigned>(xcd_grid(nqb)), static_cast<unsigned>(w.q.S));
  trace_begin(kTraceBwdQ, s);
  if (codes_aligned(a.spd, a.ld))
    hipLaunchKernelGGL(bwd_q_mfma_d8_kernel<true>, qgrid, block, 0, s, a.spd, a.table, ops, dqp, a.N, a.Nk, a.ld,
                       a.NB, q_acc, w.q.chunk, nq_el, gate);
  else
    hipLaunchKernelGGL(bwd_q_mfma_d8_kernel<false>, qgrid, block, 0, s, a.spd, a.table, ops, dqp, a.N, a.Nk, a.ld,
                       a.NB, q_acc, w.q.chunk, nq_el, gate);
  e = hipGetLastError();
  trace_end(kTraceBwdQ, s);
  if (e != hipSuccess) return e;
  if (!kv_split && !q_split && gate == nullptr)
    return launch_dtable_reduce(partial, a.dtable, w.n_kv_blocks, kH * a.NB, a.acc & kAccDtable, s);
  const SumSplits sq = q_split ? SumSplits{dqp, a.dq, nq_el, w.q.S, a.acc & kAccDq} : none;
  return launch_bwd_finish(sk, sv, sq, partial, a.dtable, w.kv.S * w.n_kv_blocks, kH * a.NB, a.acc & kAccDtable, s,
                           gate);
}

}  // namespace gt
