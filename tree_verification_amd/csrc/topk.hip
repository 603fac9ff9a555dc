// Top-k KV-block selection for sparse verification, for gfx950.
//
// The sparse-verification page ("Methodology", attention sparsity) keeps only
// the top-k key/value blocks per query, chosen by a cheap relevance score.  The
// score of block n for query (b, i, h) is q . mean(K of the block's valid
// tokens).  Selections must be reproducible bit for bit, so the float32
// arithmetic order is fixed and no multiply-add is contracted:
//   mean   sequential sum over the block's tokens in position order, then one
//          IEEE division by the valid count            (block_mean_kernel)
//   score  products q[d] * mean[d], then a halving tree: d + D/2 into d,
//          then d + D/4, ..., then d + 1               (block_score_kernel)
//   select the k largest scores, lower block first on ties, emitted in
//          ascending block order, -1 padded            (block_select_kernel)
#include "common.h"

#pragma clang fp contract(off)

namespace sdtree {

// One wavefront per (b, block, KV head): lane l owns D / 64 consecutive dims.
template <typename E, int D>
__global__ void __launch_bounds__(256) block_mean_kernel(TopkArgs a) {
#pragma clang fp contract(off)
  constexpr int DPL = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long unit = (long long)blockIdx.x * 4 + wave;
  const long long nunits = (long long)a.B * a.nbmax * a.Hkv;
  if (unit >= nunits) return;
  const int g = (int)(unit % a.Hkv);
  const int n = (int)((unit / a.Hkv) % a.nbmax);
  const int b = (int)(unit / ((long long)a.Hkv * a.nbmax));
  const int ctx = a.ctx[b];
  if (ctx < 0 || (long long)ctx > (long long)a.max_blocks * a.bs) {
    if (n == 0 && g == 0 && lane == 0) set_status(a.status, SD_ERR_CAPACITY);
    return;
  }
  const int nblk = (ctx + a.bs - 1) / a.bs;
  if (n >= nblk) return;
  const int blk = a.table[(size_t)b * a.max_blocks + n];
  float* out = a.means + (((size_t)b * a.nbmax + n) * a.Hkv + g) * D + lane * DPL;
  if (blk < 0 || blk >= a.num_blocks) {
    if (lane == 0) set_status(a.status, SD_ERR_BLOCK);
    for (int e = 0; e < DPL; ++e) out[e] = 0.f;
    return;
  }
  const int valid = min(a.bs, ctx - n * a.bs);
  const E* base = reinterpret_cast<const E*>(a.k) + (((size_t)blk * a.Hkv + g) * a.bs) * D + lane * DPL;
  float s[DPL];
  for (int e = 0; e < DPL; ++e) s[e] = 0.f;
  int t = 0;
  for (; t + 8 <= valid; t += 8) {
    float x[8][DPL];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < DPL; ++e) x[u][e] = Elem<E>::load(base, (size_t)(t + u) * D + e);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < DPL; ++e) s[e] = s[e] + x[u][e];
  }
  for (; t < valid; ++t)
    for (int e = 0; e < DPL; ++e) s[e] = s[e] + Elem<E>::load(base, (size_t)t * D + e);
  const float fv = (float)valid;
  for (int e = 0; e < DPL; ++e) out[e] = __fdiv_rn(s[e], fv);
}

// Workgroup per (b, g, chunk of 64 blocks).  Each group of 16 lanes computes
// one score: lane d' holds dims d' + 16 e, folds them in-lane down to width 16,
// then four xor steps finish the halving tree (bit-identical to it, since the
// two operands of every addition are the same).
template <typename E, int D>
__global__ void __launch_bounds__(256) block_score_kernel(TopkArgs a) {
#pragma clang fp contract(off)
  constexpr int EL = D / 16;
  constexpr int NBC = 64;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int ctx = a.ctx[b];
  if (ctx < 0 || (long long)ctx > (long long)a.max_blocks * a.bs) return;
  const int nblk = (ctx + a.bs - 1) / a.bs;
  const int n0 = chunk * NBC;
  if (n0 >= nblk) return;
  const int tid = threadIdx.x;
  const int grp = tid >> 4, dl = tid & 15;
  const int R = a.T * a.G;  // query rows of this KV group
  for (int nn = grp; nn < NBC; nn += 16) {
    const int n = n0 + nn;
    if (n >= nblk) break;
    const float* mrow = a.means + (((size_t)b * a.nbmax + n) * a.Hkv + g) * D;
    float m[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) m[e] = mrow[dl + 16 * e];
    for (int r = 0; r < R; ++r) {
      const int i = r / a.G, h = g * a.G + r % a.G;
      const size_t qrow = ((size_t)b * a.T + i) * a.Hq + h;
      const E* qp = reinterpret_cast<const E*>(a.q) + qrow * D;
      float v[EL];
#pragma unroll
      for (int e = 0; e < EL; ++e) v[e] = Elem<E>::load(qp, dl + 16 * e) * m[e];
#pragma unroll
      for (int hw = EL / 2; hw >= 1; hw >>= 1)
#pragma unroll
        for (int e = 0; e < hw; ++e) v[e] = v[e] + v[e + hw];
      float s = v[0];
      s = s + __shfl_xor(s, 8);
      s = s + __shfl_xor(s, 4);
      s = s + __shfl_xor(s, 2);
      s = s + __shfl_xor(s, 1);
      if (dl == 0) a.scores[qrow * a.nbmax + n] = s;
    }
  }
}

// Order-preserving key of a float score (-0 counts as +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per query row: radix-select the k-th largest key, then emit
// every block above it plus the lowest-indexed blocks equal to it.
__global__ void __launch_bounds__(256) block_select_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_krem;
  __shared__ int wcnt_eq[4], wcnt_sel[4];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = (int)(row / ((long long)a.T * a.Hq));
  int32_t* out = a.sel + row * a.topk;
  const int ctx = a.ctx[b];
  const bool ok = ctx >= 0 && (long long)ctx <= (long long)a.max_blocks * a.bs;
  const int nb = ok ? (ctx + a.bs - 1) / a.bs : 0;
  const float* sc = a.scores + row * a.nbmax;
  if (nb <= a.topk) {
    for (int e = tid; e < a.topk; e += 256) out[e] = e < nb ? e : -1;
    return;
  }
  uint32_t prefix = 0, mask = 0, krem = a.topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int y = tid; y < nb; y += 256) {
      const uint32_t u = score_key(sc[y]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= krem) break;
        above += hist[d];
      }
      s_prefix = prefix | ((uint32_t)d << shift);
      s_krem = krem - above;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is now the k-th largest key; take everything above it and the first
  // krem blocks equal to it, in ascending block order.
  int eq_before = 0, sel_before = 0;
  for (int base = 0; base < nb; base += 256) {
    const int y = base + tid;
    const uint32_t u = y < nb ? score_key(sc[y]) : 0u;
    const bool eq = y < nb && u == prefix;
    const unsigned long long beq = __ballot(eq);
    if (lane == 0) wcnt_eq[wave] = __popcll(beq);
    __syncthreads();
    int eq_rank = eq_before + __popcll(beq & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) eq_rank += wcnt_eq[w];
    const bool take = y < nb && (u > prefix || (eq && eq_rank < (int)krem));
    const unsigned long long bsel = __ballot(take);
    if (lane == 0) wcnt_sel[wave] = __popcll(bsel);
    __syncthreads();
    int pos = sel_before + __popcll(bsel & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) pos += wcnt_sel[w];
    if (take && pos < a.topk) out[pos] = y;
    for (int w = 0; w < 4; ++w) {
      eq_before += wcnt_eq[w];
      sel_before += wcnt_sel[w];
    }
    __syncthreads();
  }
  for (int e = sel_before + tid; e < a.topk; e += 256) out[e] = -1;
}

template <typename E, int D>
static hipError_t launch_topk_t(const TopkArgs& a, hipStream_t st) {
  const long long units = (long long)a.B * a.nbmax * a.Hkv;
  hipLaunchKernelGGL((block_mean_kernel<E, D>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((a.nbmax + 63) / 64, a.Hkv, a.B);
  hipLaunchKernelGGL((block_score_kernel<E, D>), g2, dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_select_kernel, dim3((unsigned)((long long)a.B * a.T * a.Hq)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, bool f32, hipStream_t st) {
  if (f32) return a.D == 64 ? launch_topk_t<float, 64>(a, st) : launch_topk_t<float, 128>(a, st);
  return a.D == 64 ? launch_topk_t<bf16_bits, 64>(a, st) : launch_topk_t<bf16_bits, 128>(a, st);
}

}  // namespace sdtree
