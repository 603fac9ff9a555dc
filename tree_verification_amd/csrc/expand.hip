// One batched expansion step of the draft-tree search, for gfx950.
//
// The SpecExec page ("Approach") grows the draft tree from the continuations
// of highest cumulative probability, by a batched shortest-path search with
// the draft model.  The data-parallel step: every token x after an expanded
// node e (draft logits l_e over the vocabulary) is a candidate child scored
//   s(e, x) = cum[e] + log_softmax(l_e / tau)[x],
// and the k best are kept, best first, ties to the smaller (e, x).
//
// Kernels (float32 throughout, no contraction, so every pass forms the same
// score bits):
//   expand_lse_kernel      per row: off[e] = cum[e] - log sum_x exp(l / tau)
//                          (max first); also clears the histograms
//   expand_hist_kernel<P>  pass P of an exact radix select over a unique
//                          64-bit key per candidate (the score's order bits,
//                          then the inverted flat index e * V + x, so larger
//                          keys are better candidates and no two are equal):
//                          each workgroup first re-derives the digits chosen
//                          by passes < P from their histograms, then counts
//                          digit P of the candidates that still match
//   expand_collect_kernel  the k candidates whose key is >= the k-th key
//   expand_sort_kernel     bitonic sort of the k keys (one workgroup), decoded
//                          into (row, token, score)
#include "common.h"

#pragma clang fp contract(off)

namespace sdtree {

constexpr int kExpTok = 8;                 // tokens per thread per chunk (one 16-byte bf16 load)
constexpr int kExpChunk = 256 * kExpTok;   // tokens per workgroup per row and step
// Large batches take IT = 4 steps per workgroup, so each workgroup forms the
// prefix (and flushes its histogram) once per 4 chunks; small ones one step,
// for more workgroups.

__device__ __forceinline__ float exp_score(float off, float l, float inv_tau) {
  return __fadd_rn(off, __fmul_rn(l, inv_tau));
}
__device__ __forceinline__ uint32_t exp_order_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float exp_from_order_bits(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ unsigned long long exp_key(float s, uint32_t flat) {
  return ((unsigned long long)exp_order_bits(s) << 32) | (unsigned long long)(0xFFFFFFFFu - flat);
}

template <typename LT>
__device__ __forceinline__ void exp_load8(const LT* row, int x0, int V, float* v) {
  if constexpr (sizeof(LT) == 2) {
    if (x0 + 8 <= V && (V & 7) == 0) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + x0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = x0 + e < V ? bf16_to_f32(row[x0 + e]) : 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = x0 + e < V ? row[x0 + e] : 0.f;
  }
}

// Row offsets; workgroup 0 also clears the 8 x 256 histograms.
template <typename LT>
__global__ void __launch_bounds__(256) expand_lse_kernel(ExpandArgs a) {
  const int e = blockIdx.x, tid = threadIdx.x;
  if (e == 0)
    for (int i = tid; i < 8 * 256; i += 256) a.hist[i] = 0u;
  const LT* row = reinterpret_cast<const LT*>(a.logits) + (size_t)e * a.V;
  __shared__ float red[4];
  float m = -INFINITY;
  for (int x0 = tid * 8; x0 < a.V; x0 += 256 * 8) {
    float v[8];
    exp_load8<LT>(row, x0, a.V, v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (x0 + j < a.V) m = fmaxf(m, __fmul_rn(v[j], a.inv_tau));
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float s = 0.f;
  for (int x0 = tid * 8; x0 < a.V; x0 += 256 * 8) {
    float v[8];
    exp_load8<LT>(row, x0, a.V, v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (x0 + j < a.V) s += __expf(__fmul_rn(v[j], a.inv_tau) - m);
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    a.off[e] = a.cum[e] - (m + __logf(tot));
  }
}

// The digits chosen by passes < P (from their histograms): the key prefix and
// its mask.  Cooperative (256 threads): every histogram is loaded into LDS at
// once, then each pass's digit is the bin where the count of candidates at or
// above it first reaches the number still to take (a parallel suffix scan).
// When that bin holds exactly the candidates still to take, the k best are
// the keys at or above the prefix (its lower digits zero): the selection is
// `closed`, later passes have nothing to split and are skipped.
struct ExpPrefix {
  uint32_t hs[8][256];
  uint32_t suf[257];
  uint32_t wsum[4];
  int d;
  uint32_t above;
  uint32_t at;
};
template <int P>
__device__ __forceinline__ void exp_prefix(const uint32_t* hist, int k, ExpPrefix& sh, unsigned long long& prefix,
                                           unsigned long long& mask, bool& closed) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int p = 0; p < P; ++p) sh.hs[p][tid] = hist[p * 256 + tid];
  if (tid == 0) sh.suf[256] = 0u;
  __syncthreads();
  prefix = 0ull;
  mask = 0ull;
  closed = false;
  uint32_t k_rem = (uint32_t)k;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    // suf[d] = candidates in bins >= d: an inclusive scan over the bins taken
    // from the top (thread t holds bin 255 - t)
    uint32_t v = sh.hs[p][255 - tid];
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(v, o);
      if (lane >= o) v += y;
    }
    if (lane == 63) sh.wsum[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += sh.wsum[w];
    sh.suf[255 - tid] = v;
    __syncthreads();
    if (sh.suf[tid] >= k_rem && sh.suf[tid + 1] < k_rem) {
      sh.d = tid;
      sh.above = sh.suf[tid + 1];
      sh.at = sh.suf[tid];
    }
    __syncthreads();
    const int d = sh.d;
    const bool whole = sh.at == k_rem;
    k_rem -= sh.above;
    const int shift = 56 - 8 * p;
    prefix |= (unsigned long long)d << shift;
    mask |= 0xFFull << shift;
    __syncthreads();
    if (whole) {
      closed = true;
      break;
    }
  }
}

template <typename LT, int P, int IT>
__global__ void __launch_bounds__(256) expand_hist_kernel(ExpandArgs a) {
  __shared__ uint32_t h[4][256];     // one histogram per wavefront
  __shared__ ExpPrefix sh;
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int w = 0; w < 4; ++w) h[w][tid] = 0u;
  unsigned long long prefix, mask;
  bool closed;
  exp_prefix<P>(a.hist, a.k, sh, prefix, mask, closed);
  if (closed) return;
  const int e = blockIdx.y;
  const LT* row = reinterpret_cast<const LT*>(a.logits) + (size_t)e * a.V;
  const float off = a.off[e];
  constexpr int shift = 56 - 8 * P;
  float v[IT][8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x0 = (blockIdx.x * IT + it) * kExpChunk + tid * kExpTok;
    if (x0 < a.V) exp_load8<LT>(row, x0, a.V, v[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x0 = (blockIdx.x * IT + it) * kExpChunk + tid * kExpTok;
    if (x0 >= a.V) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (x0 + j >= a.V) break;
      const unsigned long long key = exp_key(exp_score(off, v[it][j], a.inv_tau), (uint32_t)e * (uint32_t)a.V + x0 + j);
      if ((key & mask) == prefix) atomicAdd(&h[wave][(key >> shift) & 0xFF], 1u);
    }
  }
  __syncthreads();
  const uint32_t c = h[0][tid] + h[1][tid] + h[2][tid] + h[3][tid];
  if (c) atomicAdd(a.hist + P * 256 + tid, c);
}

template <typename LT, int IT>
__global__ void __launch_bounds__(256) expand_collect_kernel(ExpandArgs a) {
  __shared__ ExpPrefix sh;
  const int tid = threadIdx.x;
  unsigned long long thr, mask;
  bool closed;
  // the k-th largest key itself, or the prefix at which the selection closed
  exp_prefix<8>(a.hist, a.k, sh, thr, mask, closed);
  const int e = blockIdx.y;
  const LT* row = reinterpret_cast<const LT*>(a.logits) + (size_t)e * a.V;
  const float off = a.off[e];
  float v[IT][8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x0 = (blockIdx.x * IT + it) * kExpChunk + tid * kExpTok;
    if (x0 < a.V) exp_load8<LT>(row, x0, a.V, v[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x0 = (blockIdx.x * IT + it) * kExpChunk + tid * kExpTok;
    if (x0 >= a.V) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (x0 + j >= a.V) break;
      const unsigned long long key = exp_key(exp_score(off, v[it][j], a.inv_tau), (uint32_t)e * (uint32_t)a.V + x0 + j);
      if (key >= thr) {
        const uint32_t slot = atomicAdd(a.count, 1u);
        if (slot < (uint32_t)a.k) a.keys[slot] = key;
      }
    }
  }
}

// Bitonic sort of the k keys, descending, in one workgroup (k <= kMaxExpandK),
// then decoded; resets the collection counter for the next call.
__global__ void __launch_bounds__(1024) expand_sort_kernel(ExpandArgs a) {
  __shared__ unsigned long long s[kMaxExpandK];
  const int tid = threadIdx.x;
  int n = 1;
  while (n < a.k) n <<= 1;
  for (int i = tid; i < n; i += 1024) s[i] = i < a.k ? a.keys[i] : 0ull;
  __syncthreads();
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const unsigned long long x = s[i], y = s[j];
          if (desc ? (x < y) : (x > y)) {
            s[i] = y;
            s[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.k; i += 1024) {
    const unsigned long long key = s[i];
    const uint32_t flat = 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
    a.out_row[i] = (int32_t)(flat / (uint32_t)a.V);
    a.out_token[i] = (int32_t)(flat % (uint32_t)a.V);
    a.out_score[i] = exp_from_order_bits((uint32_t)(key >> 32));
  }
  if (tid == 0) *a.count = 0u;
}

template <typename LT, int IT>
static void launch_passes(const ExpandArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.V + kExpChunk * IT - 1) / (kExpChunk * IT)), (unsigned)a.E);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 0, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 1, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 2, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 3, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 4, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 5, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 6, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_hist_kernel<LT, 7, IT>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((expand_collect_kernel<LT, IT>), grid, dim3(256), 0, st, a);
}

template <typename LT>
static hipError_t launch_expand_t(const ExpandArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((expand_lse_kernel<LT>), dim3(a.E), dim3(256), 0, st, a);
  const long long chunks = (long long)a.E * ((a.V + kExpChunk - 1) / kExpChunk);
  if (chunks >= 4096) launch_passes<LT, 4>(a, st);
  else launch_passes<LT, 1>(a, st);
  hipLaunchKernelGGL(expand_sort_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs& a, bool f32, hipStream_t st) {
  return f32 ? launch_expand_t<float>(a, st) : launch_expand_t<bf16_bits>(a, st);
}

}  // namespace sdtree
