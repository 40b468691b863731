// Clipped hop-distance codes on the GPU: breadth-first search from every node at once,
// level by level, 64 sources per 64-bit mask.
//
// The graph is undirected, so dist(s, v) = dist(v, s) and the codes of the 64 sources
// of a batch, seen from node v, are the 64 consecutive bytes spd[v, s0 .. s0+63] of row
// v. A group of G batches (G * 64 sources) is searched together; per node and batch
// the search keeps the sources that have reached the node (visited) and those that
// reached it at the previous level (frontier). One level is one launch over all
// (node, batch) pairs: a node ORs its neighbours' frontier masks (a "pull" step), keeps
// the bits it had not seen and writes the level as the code of those pairs. The level
// launches stop doing work once a level discovers nothing (a flag per level); after
// level C-2 every pair still unseen is at distance >= C-1 in the same connected
// component (code C-1) or in another component (code C), told apart by component
// labels computed on the host.
//
// Layout of the masks: [node][batch], so the lanes of a wave are consecutive batches
// of one node and a neighbour's masks are read as one contiguous run.
#include "gt_internal.h"

#include <algorithm>

namespace gt {
namespace {

constexpr int kSpdThreads = 256;

struct SpdGroup {
  const int64_t* indptr;
  const int32_t* indices;
  const int32_t* comp;
  uint64_t* visited;
  uint8_t* spd;
  int64_t N;
  int64_t g0;  // first batch of the group
  int G;       // batches in the group
};

__device__ __forceinline__ uint64_t batch_mask(int64_t N, int64_t batch) {
  const int64_t ns = N - batch * 64;
  return ns >= 64 ? ~0ull : ((1ull << ns) - 1);
}

// visited = frontier = the batch's own source bit for each source node; its diagonal
// code is 0. Also clears the per-level flags.
__global__ __launch_bounds__(kSpdThreads) void spd_init_kernel(SpdGroup p, uint64_t* frontier, int* flags,
                                                               int nflags) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kSpdThreads + threadIdx.x;
  if (x < nflags) flags[x] = 0;
  if (x >= p.N * p.G) return;
  const int64_t v = x / p.G;
  const int b = static_cast<int>(x - v * p.G);
  const int64_t s0 = (p.g0 + b) * 64;
  const uint64_t m = (v >= s0 && v < s0 + 64) ? 1ull << (v - s0) : 0ull;
  p.visited[x] = m;
  frontier[x] = m;
  if (m) p.spd[v * p.N + v] = 0;
}

// One level: fresh = (OR of the neighbours' frontier masks) minus visited; the newly
// reached (node, source) pairs get code `level`. Does nothing once the previous level
// found no new pair (*prev_any == 0).
__global__ __launch_bounds__(kSpdThreads) void spd_level_kernel(SpdGroup p, const uint64_t* __restrict__ frontier,
                                                                uint64_t* __restrict__ fresh, int level,
                                                                const int* prev_any, int* any) {
  if (prev_any != nullptr && *prev_any == 0) return;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kSpdThreads + threadIdx.x;
  if (x >= p.N * p.G) return;
  const int64_t v = x / p.G;
  const int b = static_cast<int>(x - v * p.G);
  const uint64_t all = batch_mask(p.N, p.g0 + b);
  const uint64_t vis = p.visited[x];
  uint64_t m = 0;
  if (vis != all) {
    const int64_t e1 = p.indptr[v + 1];
    for (int64_t e = p.indptr[v]; e < e1; ++e) m |= frontier[static_cast<int64_t>(p.indices[e]) * p.G + b];
    m &= ~vis;
  }
  fresh[x] = m;
  if (m) {
    p.visited[x] = vis | m;
    *any = 1;  // every writer stores the same value
    uint8_t* row = p.spd + v * p.N + (p.g0 + b) * 64;
    const uint8_t code = static_cast<uint8_t>(level);
    for (uint64_t r = m; r; r &= r - 1) row[__builtin_ctzll(r)] = code;
  }
}

// Pairs never reached by level C-2: code C-1 within a component, C across components.
__global__ __launch_bounds__(kSpdThreads) void spd_final_kernel(SpdGroup p, int C) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kSpdThreads + threadIdx.x;
  if (x >= p.N * p.G) return;
  const int64_t v = x / p.G;
  const int b = static_cast<int>(x - v * p.G);
  const int64_t s0 = (p.g0 + b) * 64;
  const uint64_t rest = ~p.visited[x] & batch_mask(p.N, p.g0 + b);
  if (!rest) return;
  uint8_t* row = p.spd + v * p.N + s0;
  const int32_t cv = p.comp[v];
  const uint8_t far_code = static_cast<uint8_t>(C - 1), unreachable = static_cast<uint8_t>(C);
  for (uint64_t r = rest; r; r &= r - 1) {
    const int kk = __builtin_ctzll(r);
    row[kk] = p.comp[s0 + kk] == cv ? far_code : unreachable;
  }
}

}  // namespace

SpdDeviceLayout spd_device_layout(int64_t N, int64_t nnz) {
  SpdDeviceLayout l{};
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int64_t nb = (N + 63) / 64;
  const int64_t fit = static_cast<int64_t>(kSpdMaskBudget / (3 * 8 * static_cast<size_t>(N)));
  l.G = static_cast<int>(std::min<int64_t>(nb, std::max<int64_t>(1, fit)));
  size_t o = 0;
  l.indptr_off = o;
  o += up(static_cast<size_t>(N + 1) * 8);
  l.indices_off = o;
  o += up(static_cast<size_t>(nnz) * 4);
  l.comp_off = o;
  o += up(static_cast<size_t>(N) * 4);
  l.flags_off = o;
  o += up(256 * 4);
  l.masks_off = o;
  o += 3 * up(static_cast<size_t>(N) * l.G * 8);
  l.bytes = o;
  return l;
}

hipError_t launch_spd_device(void* workspace, const SpdDeviceLayout& l, int64_t N, int32_t C, uint8_t* spd,
                             hipStream_t s) {
  char* base = static_cast<char*>(workspace);
  const size_t mask_bytes = ((static_cast<size_t>(N) * l.G * 8) + 255) & ~static_cast<size_t>(255);
  uint64_t* bufs[3] = {reinterpret_cast<uint64_t*>(base + l.masks_off),
                       reinterpret_cast<uint64_t*>(base + l.masks_off + mask_bytes),
                       reinterpret_cast<uint64_t*>(base + l.masks_off + 2 * mask_bytes)};
  int* flags = reinterpret_cast<int*>(base + l.flags_off);
  SpdGroup p;
  p.indptr = reinterpret_cast<const int64_t*>(base + l.indptr_off);
  p.indices = reinterpret_cast<const int32_t*>(base + l.indices_off);
  p.comp = reinterpret_cast<const int32_t*>(base + l.comp_off);
  p.visited = bufs[0];
  p.spd = spd;
  p.N = N;
  const int64_t nb = (N + 63) / 64;
  trace_begin(kTraceSpd, s);
  for (int64_t g0 = 0; g0 < nb; g0 += l.G) {
    p.g0 = g0;
    p.G = static_cast<int>(std::min<int64_t>(l.G, nb - g0));
    const int64_t pairs = N * p.G;
    const unsigned grid = static_cast<unsigned>((std::max<int64_t>(pairs, 256) + kSpdThreads - 1) / kSpdThreads);
    uint64_t* frontier = bufs[1];
    uint64_t* fresh = bufs[2];
    hipLaunchKernelGGL(spd_init_kernel, dim3(grid), dim3(kSpdThreads), 0, s, p, frontier, flags, 256);
    for (int level = 1; level <= C - 2; ++level) {
      hipLaunchKernelGGL(spd_level_kernel, dim3(grid), dim3(kSpdThreads), 0, s, p,
                         static_cast<const uint64_t*>(frontier), fresh, level,
                         static_cast<const int*>(level > 1 ? flags + level - 1 : nullptr), flags + level);
      std::swap(frontier, fresh);
    }
    hipLaunchKernelGGL(spd_final_kernel, dim3(grid), dim3(kSpdThreads), 0, s, p, C);
  }
  const hipError_t e = hipGetLastError();
  trace_end(kTraceSpd, s);
  return e;
}

}  // namespace gt
