// Expert-parallel load balancing: the placement plan (host) and the routing
// of token slots to expert copies (device).
//
// "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
// "Routing imbalance": hot experts get redundant copies on less-loaded GPUs,
// hot and cold experts share GPUs, and the busiest GPU's token count over
// the mean is the imbalance factor the plan lowers.  The steps (copies,
// heaviest-first placement on the least-loaded rank, numbering) and their
// tie rules are stated with moe_eplb_plan in moe.h.
#include <algorithm>
#include <vector>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

int eplb_plan(const int64_t* load, int E, int G, int R, int32_t* replicas, int32_t* phys_to_log,
              int32_t* log_to_phys, double* rank_load) {
  const int P = E + R, S = P / G;
  std::vector<int32_t> rep(E, 1);
  // 1. copies: the largest load per copy (exact: a/b > c/d <=> a*d > c*b,
  //    loads < 2^40 and copies <= 512 keep the products below 2^50)
  for (int n = 0; n < R; ++n) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (rep[e] >= G) continue;
      if (best < 0 || load[e] * (int64_t)rep[best] > load[best] * (int64_t)rep[e]) best = e;
    }
    rep[best] += 1;
  }
  // 2. placement, heaviest copy first
  struct Copy {
    double w;
    int e, j;
  };
  std::vector<Copy> copies;
  copies.reserve(P);
  for (int e = 0; e < E; ++e)
    for (int j = 0; j < rep[e]; ++j) copies.push_back({(double)load[e] / (double)rep[e], e, j});
  std::sort(copies.begin(), copies.end(), [](const Copy& a, const Copy& b) {
    if (a.w != b.w) return a.w > b.w;
    if (a.e != b.e) return a.e < b.e;
    return a.j < b.j;
  });
  std::vector<double> rl(G, 0.0);
  std::vector<int> used(G, 0);
  std::vector<uint8_t> holds((size_t)G * E, 0);
  std::vector<int> rank_of_copy(P);  // indexed like `copies`
  for (int c = 0; c < P; ++c) {
    const int e = copies[c].e;
    int best = -1;
    for (int pass = 0; pass < 2 && best < 0; ++pass) {
      for (int g = 0; g < G; ++g) {
        if (used[g] >= S) continue;
        if (pass == 0 && holds[(size_t)g * E + e]) continue;
        if (best < 0 || rl[g] < rl[best]) best = g;
      }
    }
    rank_of_copy[c] = best;
    used[best] += 1;
    holds[(size_t)best * E + e] = 1;
    rl[best] += copies[c].w;
  }
  // 3. numbering: rank g's slots in increasing (expert, copy)
  std::vector<std::vector<std::pair<int, int>>> on_rank(G);
  for (int c = 0; c < P; ++c) on_rank[rank_of_copy[c]].push_back({copies[c].e, copies[c].j});
  for (int g = 0; g < G; ++g) {
    std::sort(on_rank[g].begin(), on_rank[g].end());
    for (int q = 0; q < S; ++q) phys_to_log[g * S + q] = on_rank[g][q].first;
  }
  std::vector<int> seen(E, 0);
  for (size_t i = 0; i < (size_t)E * G; ++i) log_to_phys[i] = -1;
  for (int p = 0; p < P; ++p) {
    const int e = phys_to_log[p];
    log_to_phys[(size_t)e * G + seen[e]++] = p;
  }
  for (int e = 0; e < E; ++e) replicas[e] = rep[e];
  if (rank_load)
    for (int g = 0; g < G; ++g) rank_load[g] = rl[g];
  return 0;
}

namespace {

// One thread per slot; the tables are small and stay in L2.
__global__ __launch_bounds__(256) void eplb_remap_kernel(const int32_t* __restrict__ topk_idx,
                                                         const int32_t* __restrict__ replicas,
                                                         const int32_t* __restrict__ log_to_phys,
                                                         int32_t* __restrict__ topk_phys, int k,
                                                         int E, int G, long long S) {
  const long long s = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int t = (int)(s / k);
  const int e = topk_idx[s];
  int p = -1;
  if (e >= 0 && e < E) {
    const int r = replicas[e];
    if (r >= 1 && r <= G) p = log_to_phys[(long long)e * G + t % r];
  }
  topk_phys[s] = p;
}

}  // namespace

hipError_t eplb_remap(int T, int k, int E, int G, const int32_t* topk_idx,
                      const int32_t* replicas, const int32_t* log_to_phys, int32_t* topk_phys,
                      hipStream_t st) {
  const long long S = (long long)T * k;
  const unsigned blocks = (unsigned)((S + 255) / 256);
  hipLaunchKernelGGL(eplb_remap_kernel, dim3(blocks), dim3(256), 0, st, topk_idx, replicas,
                     log_to_phys, topk_phys, k, E, G, S);
  return hipGetLastError();
}

}  // namespace moe
