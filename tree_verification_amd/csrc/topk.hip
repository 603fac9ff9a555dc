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
// Cached selection keeps the sums (the numerators of the means) per physical
// block: built once from K, extended in position order by the positions each
// commit appends (block_sums_append_kernel), and divided at selection time,
// so its means are the same float32 values without reading K.
// Shared selection (one list per sequence and KV group, reused by all the
// group's nodes and heads) scores each block against the group's pooled
// query, the sequential float32 sum of its rows (group_score_kernel), and
// selects with one workgroup per list (group_select_kernel).
#include "common.h"

#pragma clang fp contract(off)

namespace sdtree {

// Block means.  A (b, block, KV head) unit is served by LPU lanes, each
// owning one 16-byte column chunk (EPL consecutive dims) of the block's rows:
// it walks the block's valid tokens in position order, 16 rows in flight, so
// every dim's sum is the sequential one.  A wavefront serves 64 / LPU units.
// MODE 0 writes the means; MODE 1 writes the sums to the kept block sums of
// the physical block instead; MODE 2 reads the sums from there (no K walk)
// and writes the means.
constexpr int kMeansFromK = 0, kSumsFromK = 1, kMeansFromSums = 2;
template <typename E, int D, int MODE>
__global__ void __launch_bounds__(256) block_mean_kernel(TopkArgs a) {
#pragma clang fp contract(off)
  constexpr int EPL = 16 / (int)sizeof(E);      // dims per lane
  constexpr int LPU = D / EPL;                   // lanes per unit
  constexpr int UPW = 64 / LPU;                  // units per wavefront
  static_assert(LPU * EPL == D && UPW * LPU == 64, "lane split");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / LPU, col = lane % LPU;
  const long long unit = ((long long)blockIdx.x * 4 + wave) * UPW + sub;
  const long long nunits = (long long)a.B * a.nbmax * a.Hkv;
  if (unit >= nunits) return;
  const int g = (int)(unit % a.Hkv);
  const int n = (int)((unit / a.Hkv) % a.nbmax);
  const int b = (int)(unit / ((long long)a.Hkv * a.nbmax));
  const int ctx = a.ctx[b];
  if (ctx < 0 || (long long)ctx > (long long)a.max_blocks * a.bs) {
    if (n == 0 && g == 0 && col == 0) set_status(a.status, SD_ERR_CAPACITY);
    return;
  }
  const int nblk = (ctx + a.bs - 1) / a.bs;
  if (n >= nblk) return;
  const int blk = a.table[(size_t)b * a.max_blocks + n];
  float* out = MODE == kSumsFromK ? nullptr : a.means + (((size_t)b * a.nbmax + n) * a.Hkv + g) * D + col * EPL;
  if (blk < 0 || blk >= a.num_blocks) {
    if (col == 0) set_status(a.status, SD_ERR_BLOCK);
    if constexpr (MODE != kSumsFromK)
      for (int e = 0; e < EPL; ++e) out[e] = 0.f;
    return;
  }
  const int valid = min(a.bs, ctx - n * a.bs);
  float* kept = MODE == kMeansFromK ? nullptr : a.sums + ((size_t)blk * a.Hkv + g) * D + col * EPL;
  float s[EPL];
  if constexpr (MODE == kMeansFromSums) {
    const float4 u = reinterpret_cast<const float4*>(kept)[0];
    s[0] = u.x; s[1] = u.y; s[2] = u.z; s[3] = u.w;
    if constexpr (EPL == 8) {
      const float4 w = reinterpret_cast<const float4*>(kept)[1];
      s[4] = w.x; s[5] = w.y; s[6] = w.z; s[7] = w.w;
    }
  } else {
    const uint4* base = reinterpret_cast<const uint4*>(
        reinterpret_cast<const E*>(a.k) + (((size_t)blk * a.Hkv + g) * a.bs) * D) + col;
    constexpr int RS = D * (int)sizeof(E) / 16;    // uint4 per row
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = 0.f;
    auto add = [&](const uint4& u) {
      if constexpr (sizeof(E) == 2) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < EPL; ++e) s[e] = s[e] + bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
      } else {
        s[0] = s[0] + __uint_as_float(u.x);
        s[1] = s[1] + __uint_as_float(u.y);
        s[2] = s[2] + __uint_as_float(u.z);
        s[3] = s[3] + __uint_as_float(u.w);
      }
    };
    constexpr int RIF = 16;   // rows in flight
    int t = 0;
    for (; t + RIF <= valid; t += RIF) {
      uint4 x[RIF];
#pragma unroll
      for (int u = 0; u < RIF; ++u) x[u] = base[(size_t)(t + u) * RS];
#pragma unroll
      for (int u = 0; u < RIF; ++u) add(x[u]);
    }
    for (; t < valid; ++t) add(base[(size_t)t * RS]);
  }
  if constexpr (MODE == kSumsFromK) {
    reinterpret_cast<float4*>(kept)[0] = make_float4(s[0], s[1], s[2], s[3]);
    if constexpr (EPL == 8) reinterpret_cast<float4*>(kept)[1] = make_float4(s[4], s[5], s[6], s[7]);
    return;
  }
  const float fv = (float)valid;
  float r[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) r[e] = __fdiv_rn(s[e], fv);
  if constexpr (EPL == 8) {
    reinterpret_cast<float4*>(out)[0] = make_float4(r[0], r[1], r[2], r[3]);
    reinterpret_cast<float4*>(out)[1] = make_float4(r[4], r[5], r[6], r[7]);
  } else {
    reinterpret_cast<float4*>(out)[0] = make_float4(r[0], r[1], r[2], r[3]);
  }
}

// Scores.  Workgroup per (b, g, chunk of 64 blocks); the query rows of the KV
// group are staged in LDS 32 at a time, lane d' of a 16-lane group finding
// its dims d' + 16 e contiguous.  Each group takes one block at a time: lane
// d' holds the block mean's dims d' + 16 e, forms the products with a row and
// folds them in-lane down to width 16; four row rotations (by 8, 4, 2, 1
// lanes) then finish the halving tree for lane 0, which adds exactly the
// operands the tree pairs.  Scores are staged in LDS and written as
// contiguous row segments.
__device__ __forceinline__ float row_ror_add(float v, int n) {
  // lane i of each 16-lane row receives lane (i + n) % 16
  int r;
  switch (n) {
    case 8: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, false); break;
  }
  return v + __int_as_float(r);
}
template <typename E, int D>
__global__ void __launch_bounds__(256) block_score_kernel(TopkArgs a) {
#pragma clang fp contract(off)
  constexpr int EL = D / 16;
  constexpr int NBC = 64;
  constexpr int RC = 32;                     // query rows per LDS stage
  __shared__ __align__(16) float qs[RC][D];   // [row][lane d'][e] = q[row][d' + 16 e]
  __shared__ float ss[RC][NBC + 1];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int ctx = a.ctx[b];
  if (ctx < 0 || (long long)ctx > (long long)a.max_blocks * a.bs) return;
  const int nblk = (ctx + a.bs - 1) / a.bs;
  const int n0 = chunk * NBC;
  if (n0 >= nblk) return;
  const int nbc = min(NBC, nblk - n0);
  const int tid = threadIdx.x;
  const int grp = tid >> 4, dl = tid & 15;
  const int R = a.T * a.G;  // query rows of this KV group
  // the score rows hold every block of the context
  SD_DCHECK(nblk <= a.nbmax, a.status);
  for (int r0 = 0; r0 < R; r0 += RC) {
    const int rc = min(RC, R - r0);
    __syncthreads();
    // 8-dim chunks, all of a thread's loads issued before any is used
    constexpr int NCH = RC * D / 8 / 256;     // chunks per thread
    float qv8[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + 256 * c;
      const int rr = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
      const int r = r0 + min(rr, rc - 1);
      const int i = r / a.G, h = g * a.G + r % a.G;
      const E* src = reinterpret_cast<const E*>(a.q) + (((size_t)b * a.T + i) * a.Hq + h) * D + d0;
      if constexpr (sizeof(E) == 2) {
        const uint4 u = *reinterpret_cast<const uint4*>(src);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qv8[c][e] = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
      } else {
        const float4 u0 = reinterpret_cast<const float4*>(src)[0], u1 = reinterpret_cast<const float4*>(src)[1];
        qv8[c][0] = u0.x; qv8[c][1] = u0.y; qv8[c][2] = u0.z; qv8[c][3] = u0.w;
        qv8[c][4] = u1.x; qv8[c][5] = u1.y; qv8[c][6] = u1.z; qv8[c][7] = u1.w;
      }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + 256 * c;
      const int rr = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
      if (rr < rc)
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[rr][((d0 + e) % 16) * EL + (d0 + e) / 16] = qv8[c][e];
    }
    __syncthreads();
    // this group's NBG blocks (grp, grp + 16, ...) against two rows at a time:
    // 2 NBG independent dot products in flight per lane
    constexpr int NBG = NBC / 16;
    float m[NBG][EL];
#pragma unroll
    for (int j = 0; j < NBG; ++j) {
      const int nn = grp + 16 * j;
      const float* mrow = a.means + (((size_t)b * a.nbmax + n0 + min(nn, nbc - 1)) * a.Hkv + g) * D;
#pragma unroll
      for (int e = 0; e < EL; ++e) m[j][e] = mrow[dl + 16 * e];
    }
    for (int rr0 = 0; rr0 < rc; rr0 += 2) {
      float q[2][EL];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4* qv = reinterpret_cast<const float4*>(&qs[min(rr0 + u, rc - 1)][dl * EL]);
#pragma unroll
        for (int e4 = 0; e4 < EL / 4; ++e4) {
          const float4 q4 = qv[e4];
          q[u][4 * e4 + 0] = q4.x;
          q[u][4 * e4 + 1] = q4.y;
          q[u][4 * e4 + 2] = q4.z;
          q[u][4 * e4 + 3] = q4.w;
        }
      }
      float sc[NBG][2];
#pragma unroll
      for (int j = 0; j < NBG; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float v[EL];
#pragma unroll
          for (int e = 0; e < EL; ++e) v[e] = q[u][e] * m[j][e];
#pragma unroll
          for (int hw = EL / 2; hw >= 1; hw >>= 1)
#pragma unroll
            for (int e = 0; e < hw; ++e) v[e] = v[e] + v[e + hw];
          sc[j][u] = v[0];
        }
#pragma unroll
      for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
        for (int j = 0; j < NBG; ++j)
#pragma unroll
          for (int u = 0; u < 2; ++u) sc[j][u] = row_ror_add(sc[j][u], n);
      if (dl == 0)
#pragma unroll
        for (int j = 0; j < NBG; ++j)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (grp + 16 * j < nbc && rr0 + u < rc) ss[rr0 + u][grp + 16 * j] = sc[j][u];
    }
    __syncthreads();
    for (int idx = tid; idx < rc * NBC; idx += 256) {
      const int rr = idx / NBC, nn = idx % NBC;
      if (nn >= nbc) continue;
      const int r = r0 + rr;
      const int i = r / a.G, h = g * a.G + r % a.G;
      const size_t qrow = ((size_t)b * a.T + i) * a.Hq + h;
      a.scores[qrow * a.nbmax + n0 + nn] = ss[rr][nn];
    }
  }
}

// Order-preserving key of a float score (-0 counts as +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selection: one wavefront per query row.  A radix select over 8-bit digits
// finds the k-th largest key (per-wavefront histogram in LDS, suffix sums by a
// lane scan); then every block above it and the first blocks equal to it are
// emitted in ascending block order (ballot compaction).
constexpr int kSelStage = 2048;  // scores per row staged in LDS (longer rows read global memory)

__global__ void __launch_bounds__(256) block_select_kernel(TopkArgs a) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t keys[4][kSelStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wave;
  const long long nrows = (long long)a.B * a.T * a.Hq;
  if (row >= nrows) return;
  const int b = (int)(row / ((long long)a.T * a.Hq));
  int32_t* out = a.sel + row * a.topk;
  const int ctx = a.ctx[b];
  const bool ok = ctx >= 0 && (long long)ctx <= (long long)a.max_blocks * a.bs;
  const int nb = ok ? (ctx + a.bs - 1) / a.bs : 0;
  const float* sc = a.scores + row * a.nbmax;
  SD_DCHECK(nb <= a.nbmax, a.status);
  if (nb <= a.topk) {
    for (int e = lane; e < a.topk; e += 64) out[e] = e < nb ? e : -1;
    return;
  }
  uint32_t* h = hist[wave];
  // the row's keys, staged once when they fit
  const bool staged = nb <= kSelStage;
  uint32_t* kw = keys[wave];
  if (staged) {
    // 16 loads per lane in flight at a time
    for (int y0 = 0; y0 < nb; y0 += 64 * 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int y = y0 + lane + 64 * u;
        v[u] = sc[y < nb ? y : 0];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int y = y0 + lane + 64 * u;
        if (y < nb) kw[y] = score_key(v[u]);
      }
    }
  }
  auto key_of = [&](int y) -> uint32_t { return staged ? kw[y] : score_key(sc[y]); };
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)a.topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) h[lane * 4 + i] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int y = lane; y < nb; y += 64) {
      const uint32_t u = key_of(y);
      if ((u & mask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    // lane l holds bins 4l .. 4l + 3; x = count of keys in bins >= 4l
    uint32_t hb[4], lt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hb[i] = h[lane * 4 + i];
      lt += hb[i];
    }
    uint32_t x = lt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(x, off);
      if (lane + off < 64) x += y;
    }
    // bin d = 4 lane + i holds the k-th largest when the keys in bins above
    // it number fewer than krem and with it at least krem
    uint32_t above = x - lt;
    int dsel = -1;
    uint32_t asel = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (dsel < 0 && above < krem && above + hb[i] >= krem) {
        dsel = lane * 4 + i;
        asel = above;
      }
      above += hb[i];
    }
    const unsigned long long bal = __ballot(dsel >= 0);
    const int src = __ffsll((long long)bal) - 1;
    const int d = __shfl(dsel, src);
    const uint32_t ab = __shfl(asel, src);
    prefix |= (uint32_t)d << shift;
    mask |= 255u << shift;
    krem -= ab;
    __builtin_amdgcn_wave_barrier();
  }
  // prefix is the k-th largest key; krem of the keys equal to it are taken,
  // lowest block first.
  int eq_before = 0, sel_before = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int base = 0; base < nb; base += 64) {
    const int y = base + lane;
    const uint32_t u = y < nb ? key_of(y) : 0u;
    const bool eq = y < nb && u == prefix;
    const unsigned long long beq = __ballot(eq);
    const int eq_rank = eq_before + __popcll(beq & below);
    const bool take = y < nb && (u > prefix || (eq && eq_rank < (int)krem));
    const unsigned long long bsel = __ballot(take);
    const int pos = sel_before + __popcll(bsel & below);
    if (take && pos < a.topk) out[pos] = y;
    eq_before += __popcll(beq);
    sel_before += __popcll(bsel);
  }
  for (int e = sel_before + lane; e < a.topk; e += 64) out[e] = -1;
}

// Shared selection, scores: one workgroup per (64 blocks, KV group,
// sequence).  The workgroup first forms the group's pooled query -- the
// sequential float32 sum from +0 of its T * G rows, node by node and head by
// head -- staging 32 rows at a time in LDS, one thread per dim.  Each block's
// mean is then read (MEANS) or formed from the kept sum with one IEEE
// division (SUMS), and scored against the pooled query with the products and
// halving tree of block_score_kernel (same lane layout, same pairs).  A block
// id out of range scores with a zero mean and sets the block bit, as in
// block_mean_kernel.
template <typename E, int D, bool SUMS>
__global__ void __launch_bounds__(256) group_score_kernel(TopkArgs a) {
#pragma clang fp contract(off)
  constexpr int EL = D / 16;
  constexpr int NBC = 64;
  constexpr int RS = 32;                                  // rows per LDS stage
  constexpr int CPR = D * (int)sizeof(E) / 16;            // 16-byte chunks per row
  constexpr int CPT = RS * CPR / 256;                     // chunks per thread per stage
  static_assert(CPT * 256 == RS * CPR, "stage split");
  __shared__ __align__(16) uint4 stage[RS * CPR];
  __shared__ __align__(16) float qs[D];                   // [lane d'][e] = pooled[d' + 16 e]
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int ctx = a.ctx[b];
  if (ctx < 0 || (long long)ctx > (long long)a.max_blocks * a.bs) {
    if (SUMS && chunk == 0 && g == 0 && tid == 0) set_status(a.status, SD_ERR_CAPACITY);
    return;
  }
  const int nblk = (ctx + a.bs - 1) / a.bs;
  const int n0 = chunk * NBC;
  if (n0 >= nblk) return;
  const int nbc = min(NBC, nblk - n0);
  const int grp = tid >> 4, dl = tid & 15;
  constexpr int NBG = NBC / 16;
  float m[NBG][EL];
  bool bad[NBG];
  if constexpr (SUMS) {
    // block ids, then every sum load issued before the pooled query's loads;
    // the means are formed after it
    int blk[NBG];
#pragma unroll
    for (int j = 0; j < NBG; ++j) blk[j] = a.table[(size_t)b * a.max_blocks + n0 + min(grp + 16 * j, nbc - 1)];
#pragma unroll
    for (int j = 0; j < NBG; ++j) {
      bad[j] = blk[j] < 0 || blk[j] >= a.num_blocks;
      const float* srow = a.sums + ((size_t)(bad[j] ? 0 : blk[j]) * a.Hkv + g) * D + dl;
#pragma unroll
      for (int e = 0; e < EL; ++e) m[j][e] = srow[16 * e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NBG; ++j) {
      const float* mrow = a.means + (((size_t)b * a.nbmax + n0 + min(grp + 16 * j, nbc - 1)) * a.Hkv + g) * D;
#pragma unroll
      for (int e = 0; e < EL; ++e) m[j][e] = mrow[dl + 16 * e];
    }
  }
  // pooled query
  const int R = a.T * a.G;
  float acc = 0.f;
  for (int r0 = 0; r0 < R; r0 += RS) {
    const int rc = min(RS, R - r0);
    uint4 v[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + 256 * c, rr = min(idx / CPR, rc - 1), col = idx % CPR;
      const int r = r0 + rr, i = r / a.G, h = g * a.G + r % a.G;
      v[c] = reinterpret_cast<const uint4*>(reinterpret_cast<const E*>(a.q) +
                                            (((size_t)b * a.T + i) * a.Hq + h) * D)[col];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) stage[tid + 256 * c] = v[c];
    __syncthreads();
    if (tid < D) {
      const E* st = reinterpret_cast<const E*>(stage);
      for (int rr = 0; rr < rc; ++rr) {
        const E x = st[rr * D + tid];
        if constexpr (sizeof(E) == 2) acc = acc + bf16_to_f32((bf16_bits)x);
        else acc = acc + x;
      }
    }
  }
  if (tid < D) qs[(tid % 16) * EL + tid / 16] = acc;
  __syncthreads();
  float q[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) q[e] = qs[dl * EL + e];
  if constexpr (SUMS) {
#pragma unroll
    for (int j = 0; j < NBG; ++j) {
      const int n = n0 + min(grp + 16 * j, nbc - 1);
      if (bad[j] && dl == 0 && grp + 16 * j < nbc) set_status(a.status, SD_ERR_BLOCK);
      const float fv = (float)min(a.bs, ctx - n * a.bs);
#pragma unroll
      for (int e = 0; e < EL; ++e) m[j][e] = bad[j] ? 0.f : __fdiv_rn(m[j][e], fv);
    }
  }
  float sc[NBG];
#pragma unroll
  for (int j = 0; j < NBG; ++j) {
    float v[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) v[e] = q[e] * m[j][e];
#pragma unroll
    for (int hw = EL / 2; hw >= 1; hw >>= 1)
#pragma unroll
      for (int e = 0; e < hw; ++e) v[e] = v[e] + v[e + hw];
    sc[j] = v[0];
  }
#pragma unroll
  for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
    for (int j = 0; j < NBG; ++j) sc[j] = row_ror_add(sc[j], n);
  if (dl == 0)
#pragma unroll
    for (int j = 0; j < NBG; ++j)
      if (grp + 16 * j < nbc) a.scores[((size_t)b * a.Hkv + g) * a.nbmax + n0 + grp + 16 * j] = sc[j];
}

// Shared selection, select: one workgroup per (sequence, KV group).  The
// same radix select as block_select_kernel, spread over four wavefronts (one
// histogram copy each, bins scanned by all 256 threads), then an ordered
// block-wide compaction.  The list is gathered in LDS and written to every
// row of the group by all threads.
constexpr int kGroupStage = 8192;   // scores staged in LDS (longer rows read global memory)
constexpr int kGroupList = 4096;    // longer lists are written to the rows as they are found

__global__ void __launch_bounds__(256) group_select_kernel(TopkArgs a) {
  __shared__ uint32_t keys[kGroupStage];
  __shared__ int32_t slist[kGroupList];
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t wtot[4], ceq[4], csel[4];
  __shared__ int s_d;
  __shared__ uint32_t s_ab;
  const int row = blockIdx.x, b = row / a.Hkv, g = row % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ctx = a.ctx[b];
  const bool ok = ctx >= 0 && (long long)ctx <= (long long)a.max_blocks * a.bs;
  const int nb = ok ? (ctx + a.bs - 1) / a.bs : 0;
  const int R = a.rep_T * a.rep_G;
  auto row_ptr = [&](int r) -> int32_t* {
    const int i = r / a.rep_G, j = r % a.rep_G;
    return a.rep + (((size_t)b * a.rep_T + i) * a.rep_Hq + (size_t)g * a.rep_G + j) * a.topk;
  };
  if (nb <= a.topk) {
    for (long long idx = tid; idx < (long long)R * a.topk; idx += 256) {
      const int r = (int)(idx / a.topk), e = (int)(idx % a.topk);
      row_ptr(r)[e] = e < nb ? e : -1;
    }
    return;
  }
  const float* sc = a.scores + (size_t)row * a.nbmax;
  const bool staged = nb <= kGroupStage;
  if (staged) {
    for (int y0 = 0; y0 < nb; y0 += 256 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int y = y0 + tid + 256 * u;
        v[u] = sc[y < nb ? y : 0];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int y = y0 + tid + 256 * u;
        if (y < nb) keys[y] = score_key(v[u]);
      }
    }
  }
  __syncthreads();
  auto key_of = [&](int y) -> uint32_t { return staged ? keys[y] : score_key(sc[y]); };
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)a.topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[wave][lane] = 0u; hist[wave][lane + 64] = 0u; hist[wave][lane + 128] = 0u; hist[wave][lane + 192] = 0u;
    __syncthreads();
    for (int y = tid; y < nb; y += 256) {
      const uint32_t u = key_of(y);
      if ((u & mask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t owns bin t; x = keys in bins t .. (wave end), then wave totals
    const uint32_t c = hist[0][tid] + hist[1][tid] + hist[2][tid] + hist[3][tid];
    uint32_t x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(x, off);
      if (lane + off < 64) x += y;
    }
    if (lane == 0) wtot[wave] = x;
    __syncthreads();
    uint32_t above = x - c;
    for (int w = wave + 1; w < 4; ++w) above += wtot[w];
    if (above < krem && above + c >= krem) {
      s_d = tid;
      s_ab = above;
    }
    __syncthreads();
    prefix |= (uint32_t)s_d << shift;
    mask |= 255u << shift;
    krem -= s_ab;
    __syncthreads();
  }
  // every key above prefix, and the first krem keys equal to it, lowest block first
  const bool gather = a.topk <= kGroupList;
  const unsigned long long below = (1ull << lane) - 1ull;
  int eq_base = 0, sel_base = 0;
  for (int base = 0; base < nb; base += 256) {
    const int y = base + tid;
    const uint32_t u = y < nb ? key_of(y) : 0u;
    const bool eq = y < nb && u == prefix;
    const unsigned long long beq = __ballot(eq);
    if (lane == 0) ceq[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    int eq_rank = eq_base + __popcll(beq & below);
    for (int w = 0; w < wave; ++w) eq_rank += (int)ceq[w];
    const bool take = y < nb && (u > prefix || (eq && eq_rank < (int)krem));
    const unsigned long long bsel = __ballot(take);
    if (lane == 0) csel[wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    int pos = sel_base + __popcll(bsel & below);
    for (int w = 0; w < wave; ++w) pos += (int)csel[w];
    if (take && pos < a.topk) {
      if (gather) slist[pos] = y;
      else
        for (int r = 0; r < R; ++r) row_ptr(r)[pos] = y;
    }
    for (int w = 0; w < 4; ++w) {
      eq_base += (int)ceq[w];
      sel_base += (int)csel[w];
    }
    __syncthreads();
  }
  const int nsel = min(sel_base, a.topk);
  if (gather) {
    for (long long idx = tid; idx < (long long)R * a.topk; idx += 256) {
      const int r = (int)(idx / a.topk), e = (int)(idx % a.topk);
      row_ptr(r)[e] = e < nsel ? slist[e] : -1;
    }
  } else {
    for (long long idx = tid; idx < (long long)R * (a.topk - nsel); idx += 256) {
      const int r = (int)(idx / (a.topk - nsel)), e = nsel + (int)(idx % (a.topk - nsel));
      row_ptr(r)[e] = -1;
    }
  }
}

// Kept block sums after a commit: the positions [ctx_b - n_b, ctx_b) it
// appended (ctx_lens after the commit, n_b = path_len[b]) are added, in
// position order, to their blocks' sums; a block whose first position is
// among them starts from +0, so every sum stays the sequential one.  One
// wavefront per (b, KV head), D / 64 dims per lane; the touched blocks are
// validated before anything is written.
template <typename E, int D>
__global__ void __launch_bounds__(256) block_sums_append_kernel(TopkArgs a, const int32_t* __restrict__ n_new) {
#pragma clang fp contract(off)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long unit = (long long)blockIdx.x * 4 + wave;
  if (unit >= (long long)a.B * a.Hkv) return;
  const int b = (int)(unit / a.Hkv), g = (int)(unit % a.Hkv);
  const int ctx = a.ctx[b], L = n_new[b];
  if (L < 0 || L > ctx || (long long)ctx > (long long)a.max_blocks * a.bs) {
    if (g == 0 && lane == 0) set_status(a.status, SD_ERR_CAPACITY);
    return;
  }
  if (L == 0) return;
  const int32_t* table = a.table + (size_t)b * a.max_blocks;
  for (int n = (ctx - L) / a.bs; n <= (ctx - 1) / a.bs; ++n) {
    const int blk = table[n];
    if (blk < 0 || blk >= a.num_blocks) {
      if (g == 0 && lane == 0) set_status(a.status, SD_ERR_BLOCK);
      return;
    }
  }
  const E* K = reinterpret_cast<const E*>(a.k);
  extend_head_sums<E, D>(
      a.bs, ctx - L, ctx, lane,
      [&](int n) { return K + (((size_t)table[n] * a.Hkv + g) * a.bs) * D; },
      [&](int n) { return a.sums + ((size_t)table[n] * a.Hkv + g) * D; });
}

template <typename E, int D, int MODE>
static hipError_t launch_means(const TopkArgs& a, hipStream_t st) {
  constexpr int UPW = 64 / (D / (16 / (int)sizeof(E)));
  const long long units = (long long)a.B * a.nbmax * a.Hkv;
  const long long per_wg = 4LL * UPW;
  hipLaunchKernelGGL((block_mean_kernel<E, D, MODE>), dim3((unsigned)((units + per_wg - 1) / per_wg)),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_topk_t(const TopkArgs& a, bool cached, hipStream_t st) {
  hipError_t e = cached ? launch_means<E, D, kMeansFromSums>(a, st) : launch_means<E, D, kMeansFromK>(a, st);
  if (e != hipSuccess) return e;
  dim3 g2((a.nbmax + 63) / 64, a.Hkv, a.B);
  hipLaunchKernelGGL((block_score_kernel<E, D>), g2, dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.B * a.T * a.Hq;
  hipLaunchKernelGGL(block_select_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Shared selection: block means from K first when there are no kept sums,
// then the group scores and the group select.
template <typename E, int D>
static hipError_t launch_topk_shared_t(const TopkArgs& a, bool cached, hipStream_t st) {
  hipError_t e = hipSuccess;
  const dim3 grid((a.nbmax + 63) / 64, a.Hkv, a.B);
  if (cached) {
    hipLaunchKernelGGL((group_score_kernel<E, D, true>), grid, dim3(256), 0, st, a);
  } else {
    e = launch_means<E, D, kMeansFromK>(a, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((group_score_kernel<E, D, false>), grid, dim3(256), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TopkArgs p = a;
  p.rep = a.sel; p.rep_T = a.T; p.rep_Hq = a.Hq; p.rep_G = a.G;
  hipLaunchKernelGGL(group_select_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_topk_shared(const TopkArgs& a, bool f32, bool cached, hipStream_t st) {
  if (f32)
    return a.D == 64 ? launch_topk_shared_t<float, 64>(a, cached, st) : launch_topk_shared_t<float, 128>(a, cached, st);
  return a.D == 64 ? launch_topk_shared_t<bf16_bits, 64>(a, cached, st)
                   : launch_topk_shared_t<bf16_bits, 128>(a, cached, st);
}

hipError_t launch_topk(const TopkArgs& a, bool f32, bool cached, hipStream_t st) {
  if (f32) return a.D == 64 ? launch_topk_t<float, 64>(a, cached, st) : launch_topk_t<float, 128>(a, cached, st);
  return a.D == 64 ? launch_topk_t<bf16_bits, 64>(a, cached, st) : launch_topk_t<bf16_bits, 128>(a, cached, st);
}

hipError_t launch_block_sums(const TopkArgs& a, bool f32, hipStream_t st) {
  if (f32)
    return a.D == 64 ? launch_means<float, 64, kSumsFromK>(a, st) : launch_means<float, 128, kSumsFromK>(a, st);
  return a.D == 64 ? launch_means<bf16_bits, 64, kSumsFromK>(a, st) : launch_means<bf16_bits, 128, kSumsFromK>(a, st);
}

hipError_t launch_block_sums_append(const TopkArgs& a, const int32_t* n_new, bool f32, hipStream_t st) {
  const dim3 grid((unsigned)(((long long)a.B * a.Hkv + 3) / 4));
  if (f32) {
    if (a.D == 64) hipLaunchKernelGGL((block_sums_append_kernel<float, 64>), grid, dim3(256), 0, st, a, n_new);
    else hipLaunchKernelGGL((block_sums_append_kernel<float, 128>), grid, dim3(256), 0, st, a, n_new);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((block_sums_append_kernel<bf16_bits, 64>), grid, dim3(256), 0, st, a, n_new);
    else hipLaunchKernelGGL((block_sums_append_kernel<bf16_bits, 128>), grid, dim3(256), 0, st, a, n_new);
  }
  return hipGetLastError();
}

}  // namespace sdtree
