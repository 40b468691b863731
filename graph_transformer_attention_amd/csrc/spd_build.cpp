// Clipped hop-distance codes for every node pair, on the host.
//
// Breadth-first search from 64 sources at once: each node keeps a 64-bit mask of
// the sources that have reached it, and one level of the search is a pass over the
// adjacency that ORs the neighbours' frontier masks (a "pull" step). On an
// undirected graph dist(s, v) = dist(v, s), so the codes of the 64 sources are
// written as 64 contiguous bytes of row v. The search stops after level C-2; every
// pair still unreached is then either at distance >= C-1 (same connected component,
// code C-1) or unreachable (code C).
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

namespace gt {

std::string spd_validate(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C);
void spd_fill(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C, uint8_t* spd,
              int nthreads);
std::vector<int64_t> components(const int64_t* indptr, const int32_t* indices, int64_t N);

// Connected-component label of every node (the smallest node index in its component),
// by union-find over the edges.
std::vector<int64_t> components(const int64_t* indptr, const int32_t* indices, int64_t N) {
  std::vector<int64_t> parent(N);
  for (int64_t x = 0; x < N; ++x) parent[x] = x;
  auto find = [&](int64_t x) {
    while (parent[x] != x) {
      parent[x] = parent[parent[x]];
      x = parent[x];
    }
    return x;
  };
  for (int64_t u = 0; u < N; ++u)
    for (int64_t e = indptr[u]; e < indptr[u + 1]; ++e) {
      const int64_t a = find(u), b = find(indices[e]);
      if (a != b) parent[std::max(a, b)] = std::min(a, b);
    }
  for (int64_t x = 0; x < N; ++x) parent[x] = find(x);
  return parent;
}

std::string spd_validate(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C) {
  if (C < 1 || C > 254) return "C must lie in [1, 254] (codes 0..C fit in uint8)";
  if (N < 1) return "N must be >= 1";
  if (indptr[0] != 0) return "indptr[0] must be 0";
  for (int64_t u = 0; u < N; ++u)
    if (indptr[u + 1] < indptr[u]) return "indptr must be non-decreasing";
  const int64_t nnz = indptr[N];
  if (nnz > 0 && indices == nullptr) return "indices is null";
  for (int64_t e = 0; e < nnz; ++e)
    if (indices[e] < 0 || indices[e] >= N) return "indices out of range [0, N)";
  // the adjacency must be symmetric: u -> w implies w -> u
  std::vector<int32_t> sorted(indices, indices + nnz);
  for (int64_t u = 0; u < N; ++u) std::sort(sorted.begin() + indptr[u], sorted.begin() + indptr[u + 1]);
  for (int64_t u = 0; u < N; ++u)
    for (int64_t e = indptr[u]; e < indptr[u + 1]; ++e) {
      const int32_t w = sorted[e];
      if (!std::binary_search(sorted.begin() + indptr[w], sorted.begin() + indptr[w + 1],
                              static_cast<int32_t>(u)))
        return "adjacency is not symmetric (the graph must be undirected)";
    }
  return std::string();
}

void spd_fill(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C, uint8_t* spd,
              int nthreads) {
  const std::vector<int64_t> comp = components(indptr, indices, N);
  const int64_t nblocks = (N + 63) / 64;
  if (nthreads <= 0) nthreads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  nthreads = static_cast<int>(std::min<int64_t>(nthreads, nblocks));
  std::atomic<int64_t> next_block{0};
  const uint8_t far_code = static_cast<uint8_t>(C - 1);
  const uint8_t unreachable = static_cast<uint8_t>(C);

  auto worker = [&]() {
    std::vector<uint64_t> visited(N), frontier(N), fresh(N);
    for (;;) {
      const int64_t b = next_block.fetch_add(1);
      if (b >= nblocks) break;
      const int64_t s0 = b * 64;
      const int ns = static_cast<int>(std::min<int64_t>(64, N - s0));
      const uint64_t all = ns == 64 ? ~0ull : ((1ull << ns) - 1);
      std::fill(visited.begin(), visited.end(), 0ull);
      std::fill(frontier.begin(), frontier.end(), 0ull);
      for (int kk = 0; kk < ns; ++kk) {
        visited[s0 + kk] = frontier[s0 + kk] = 1ull << kk;
        spd[(s0 + kk) * N + s0 + kk] = 0;
      }
      for (int32_t level = 1; level <= C - 2; ++level) {
        bool any = false;
        for (int64_t v = 0; v < N; ++v) {
          uint64_t m = 0;
          if (visited[v] != all)
            for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e) m |= frontier[indices[e]];
          m &= ~visited[v];
          fresh[v] = m;
          if (m) {
            any = true;
            uint8_t* row = spd + v * N + s0;
            for (uint64_t x = m; x; x &= x - 1) row[__builtin_ctzll(x)] = static_cast<uint8_t>(level);
          }
        }
        if (!any) break;
        for (int64_t v = 0; v < N; ++v) visited[v] |= fresh[v];
        frontier.swap(fresh);
      }
      for (int64_t v = 0; v < N; ++v) {
        const uint64_t rest = ~visited[v] & all;
        if (!rest) continue;
        uint8_t* row = spd + v * N + s0;
        for (uint64_t x = rest; x; x &= x - 1) {
          const int kk = __builtin_ctzll(x);
          row[kk] = comp[v] == comp[s0 + kk] ? far_code : unreachable;
        }
      }
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace gt
