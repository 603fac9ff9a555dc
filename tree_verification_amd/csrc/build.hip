// Draft-tree construction on the GPU, for gfx950: the best-first search over
// cumulative draft log-probability that grows the tree to its budget.
//
// The SpecExec page ("Approach") builds the draft tree deterministically from
// the continuations of highest cumulative probability with a parallel
// shortest-path search: each step runs the drafter on a batch of nodes and
// keeps the best candidates.  This file turns that into rounds that reproduce
// the sequential best-first order exactly.  Node n's drafter logits are row n
// of `draft` (the drafter's output at the node that received id n), node ids
// follow the order in which the sequential search would take the nodes, and
// ties go to the smaller (parent, token).
//
// After n nodes are in the tree (ids 0 .. n - 1), every child of those nodes
// is a candidate, scored cum[parent] + log_softmax(row[parent] / tau)[token].
// The nodes already taken are the best n - 1 candidates, so sorting the best
// T - 1 candidates puts the next ones at positions n - 1 .. T - 2.  A
// sequential search would take candidate j (which would get id n + j) next
// exactly when no earlier candidate i's best child scores higher; that child
// scores cum_i - lse(row n + i) (its log-probability is the row's largest,
// -lse after the max is taken out), so the round takes the longest prefix of
// candidates for which cum_j >= max_{i<j} (cum_i - lse(row n + i)), at least
// one.  (On equal scores the candidate wins: its parent id is below n.)
//
// A round is one pre-selection of the best T - 1 + margin candidates in
// float32 (the expansion step's kernels, over the n rows taken so far), then
// one workgroup that recomputes their scores in float64 (the order the
// search is defined by), sorts them by (score descending, parent, token),
// checks that the first n - 1 are the nodes already taken, finds the prefix
// and appends it.  Per-row float64 max and log-sum-exp are formed once for
// all rows.  The margin makes the float32 pre-selection safe unless more than
// `margin` candidates lie within float32 rounding of the cut; the prefix
// check reports it if that ever happens.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace sdtree {

constexpr int kBuildThreads = 1024;
constexpr int kBuildSort = kMaxExpandK;   // sort slots (a power of two)

// Row statistics in float64 for every row of the drafter table: the max of
// z = l / tau and L = log(sum exp(z - max)).
template <typename LT>
__global__ void __launch_bounds__(256) build_row_stats_kernel(BuildArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const LT* row = reinterpret_cast<const LT*>(a.logits) + (size_t)r * a.V;
  __shared__ double red[4];
  double m = -INFINITY;
  for (int x = tid; x < a.V; x += 256) m = fmax(m, (double)Elem<LT>::load(row, x) / (double)a.tau);
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double s = 0.0;
  for (int x = tid; x < a.V; x += 256) s += exp((double)Elem<LT>::load(row, x) / (double)a.tau - m);
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    a.rmax[r] = m;
    a.rlse[r] = log((red[0] + red[1]) + (red[2] + red[3]));
  }
}

// The root: id 0, parent -1, the given token, cumulative log-probability 0.
__global__ void build_init_kernel(BuildArgs a) {
  if (threadIdx.x == 0) {
    a.parent[0] = -1;
    a.token[0] = a.root_token;
    a.cum[0] = 0.0;
    a.cum32[0] = 0.f;
    *a.n_dev = 1;
  }
}

// (score descending, then parent, then token): true when (s1, k1) sorts first
__device__ __forceinline__ bool build_before(double s1, unsigned long long k1, double s2,
                                             unsigned long long k2) {
  return s1 > s2 || (s1 == s2 && k1 < k2);
}

// One round, one workgroup.  kc pre-selected candidates (row = parent id,
// token) are rescored in float64 and sorted; n nodes are in the tree.
template <typename LT>
__global__ void __launch_bounds__(kBuildThreads) build_round_kernel(BuildArgs a, int n, int kc) {
  __shared__ double s_sc[kBuildSort];
  __shared__ unsigned long long s_key[kBuildSort];   // parent << 32 | token
  __shared__ double s_scan[kBuildSort];
  __shared__ int s_m, s_bad;
  const int tid = threadIdx.x;
  const int T = a.T;
  // candidates after the n - 1 taken ones (fewer than T - n when the n rows
  // have fewer children in all than the budget asks for)
  const int M = min(T - n, kc - (n - 1));
  // the round's candidates fit the sort and cover the nodes already taken
  SD_DCHECK(kc <= kBuildSort && n >= 1 && n < T && kc >= n - 1, a.status);
  if (tid == 0) {
    s_m = M;
    s_bad = 0;
  }
  for (int i = tid; i < kBuildSort; i += kBuildThreads) {
    double sc = -INFINITY;
    unsigned long long key = ~0ull;
    if (i < kc) {
      const int e = a.cand_row[i], x = a.cand_token[i];
      const LT* row = reinterpret_cast<const LT*>(a.logits) + (size_t)e * a.V;
      const double z = (double)Elem<LT>::load(row, x) / (double)a.tau;
      sc = a.cum[e] + ((z - a.rmax[e]) - a.rlse[e]);
      key = ((unsigned long long)(unsigned)e << 32) | (unsigned)x;
    }
    s_sc[i] = sc;
    s_key[i] = key;
  }
  __syncthreads();
  // bitonic sort of kBuildSort slots into (score desc, parent, token) order
  for (int size = 2; size <= kBuildSort; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kBuildSort / 2; i += kBuildThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const double sl = s_sc[lo], sh = s_sc[hi];
        const unsigned long long kl = s_key[lo], kh = s_key[hi];
        if (build_before(sh, kh, sl, kl) == up) {
          s_sc[lo] = sh;
          s_sc[hi] = sl;
          s_key[lo] = kh;
          s_key[hi] = kl;
        }
      }
      __syncthreads();
    }
  }
  // the first n - 1 must be the nodes already in the tree, in id order
  for (int i = tid; i < n - 1; i += kBuildThreads) {
    const unsigned long long want =
        ((unsigned long long)(unsigned)a.parent[i + 1] << 32) | (unsigned)a.token[i + 1];
    if (s_key[i] != want) s_bad = 1;
  }
  // candidate j (position n - 1 + j, would-be id n + j): its best child's score
  for (int j = tid; j < kBuildSort; j += kBuildThreads)
    s_scan[j] = j < M ? s_sc[n - 1 + j] - a.rlse[n + j] : -INFINITY;
  __syncthreads();
  // inclusive prefix max (Hillis-Steele, double-buffered through registers)
  for (int off = 1; off < kBuildSort; off <<= 1) {
    double v[kBuildSort / kBuildThreads];
#pragma unroll
    for (int u = 0; u < kBuildSort / kBuildThreads; ++u) {
      const int j = tid + u * kBuildThreads;
      v[u] = j >= off ? fmax(s_scan[j], s_scan[j - off]) : s_scan[j];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBuildSort / kBuildThreads; ++u) s_scan[tid + u * kBuildThreads] = v[u];
    __syncthreads();
  }
  // the prefix ends at the first j >= 1 whose score falls below an earlier
  // candidate's best child
  for (int j = 1 + tid; j < M; j += kBuildThreads)
    if (s_sc[n - 1 + j] < s_scan[j - 1]) atomicMin(&s_m, j);
  __syncthreads();
  if (s_bad) {
    if (tid == 0) {
      set_status(a.status, SD_ERR_BUILD);
      *a.n_dev = n;   // no progress: the host stops
    }
    return;
  }
  const int m = s_m;
  for (int j = tid; j < m; j += kBuildThreads) {
    const unsigned long long key = s_key[n - 1 + j];
    const double sc = s_sc[n - 1 + j];
    a.parent[n + j] = (int)(key >> 32);
    a.token[n + j] = (int)(unsigned)key;
    a.cum[n + j] = sc;
    a.cum32[n + j] = (float)sc;
  }
  if (tid == 0) *a.n_dev = n + m;
}

hipError_t run_tree_build(const BuildArgs& a, const ExpandArgs& ex0, bool f32, hipStream_t st,
                          int* rounds) {
  auto stats = f32 ? reinterpret_cast<const void*>(build_row_stats_kernel<float>)
                   : reinterpret_cast<const void*>(build_row_stats_kernel<bf16_bits>);
  auto round = f32 ? reinterpret_cast<const void*>(build_round_kernel<float>)
                   : reinterpret_cast<const void*>(build_round_kernel<bf16_bits>);
  BuildArgs ac = a;
  hipLaunchKernelGGL(build_init_kernel, dim3(1), dim3(64), 0, st, ac);
  {
    void* args[] = {&ac};
    hipError_t e = hipLaunchKernel(stats, dim3(a.T), dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
  }
  int n = 1, r = 0;
  while (n < a.T) {
    ExpandArgs ex = ex0;
    ex.E = n;
    ex.k = (int)std::min<long long>((long long)a.T - 1 + a.margin, (long long)n * a.V);
    hipError_t e = launch_expand(ex, f32, st);
    if (e != hipSuccess) return e;
    int kc = ex.k;
    void* args[] = {&ac, &n, &kc};
    e = hipLaunchKernel(round, dim3(1), dim3(kBuildThreads), args, 0, st);
    if (e != hipSuccess) return e;
    int n_new = n;
    e = hipMemcpyAsync(&n_new, a.n_dev, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return e;
    ++r;
    if (n_new <= n) break;   // a data error stopped the round (status bit set)
    n = n_new;
  }
  if (rounds) *rounds = r;
  return hipGetLastError();
}

}  // namespace sdtree
