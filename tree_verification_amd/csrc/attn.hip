// Tree-masked grouped-query attention over a paged KV cache, for gfx950.
//
// Every draft-tree node attends to the committed context plus its own
// ancestors, so the whole tree is verified in one target pass (SpecExec page,
// "Approach"; EasySpec page, "+tree" baseline).  The sparse variant keeps only
// the context blocks each query selected (sparse-verification page,
// "Methodology", attention sparsity).
//
// Kernels:
//   anc_mask_kernel     ancestor bitmask per node, anc(i) = anc(parent(i)) | bit(i)
//   attn_valu_kernel    one wavefront per query row, float32 math (fp32 inputs)
//   attn_mfma_kernel    bf16 MFMA flash-style kernel: K / V^T tiles staged in LDS
//                       and shared by every query row of a KV group, online
//                       softmax in registers, split context with partials
//   attn_combine_kernel merges split partials into the normalised output
#include "common.h"

namespace sdtree {

// ---------------------------------------------------------------------------
// Ancestor bitmasks.  anc[(tree * T + i) * W64 + w] holds bits j - 64 w of the
// inclusive ancestor set of node i.  Parents are validated on the way up.
__global__ void __launch_bounds__(256) anc_mask_kernel(const int32_t* __restrict__ parent, int T,
                                                       int W64, uint64_t* __restrict__ anc,
                                                       uint32_t* status) {
  const int tree = blockIdx.y;
  const int32_t* par = parent + (size_t)tree * T;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < T; i += gridDim.x * blockDim.x) {
    uint64_t* row = anc + ((size_t)tree * T + i) * W64;
    for (int w = 0; w < W64; ++w) row[w] = 0;
    int cur_w = i >> 6;
    uint64_t acc = 0;
    bool bad = false;
    int n = i;
    while (n >= 0) {
      const int w = n >> 6;
      if (w != cur_w) {
        row[cur_w] = acc;
        cur_w = w;
        acc = 0;
      }
      acc |= 1ull << (n & 63);
      const int p = par[n];
      if (n == 0) {
        bad = (p != -1);
        break;
      }
      if (p >= n || p < -1) {
        bad = true;
        break;
      }
      n = p;  // p == -1 on a non-root node ends the chain (a forest is allowed)
    }
    row[cur_w] = acc;
    if (bad) set_status(status, SD_ERR_PARENT);
  }
}

// ---------------------------------------------------------------------------
// float32 attention, one wavefront per query row (b, i, h).  Keys are walked
// 64 at a time in a virtual order: dense = positions [0, ctx) then the tree
// slots ctx + j; sparse = the ksel * bs slots of the row's selected blocks,
// then the tree slots.  Tree slot j is visible when j is an ancestor of i.
template <typename E, int D>
__global__ void __launch_bounds__(256) attn_valu_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + wave;
  const long long nrows = (long long)a.B * a.T * a.Hq;
  if (row >= nrows) return;
  const int h = (int)(row % a.Hq);
  const int i = (int)((row / a.Hq) % a.T);
  const int b = (int)(row / ((long long)a.Hq * a.T));
  const int g = h / a.G;
  const E* q = reinterpret_cast<const E*>(a.q) + row * D;
  const E* K = reinterpret_cast<const E*>(a.k);
  const E* V = reinterpret_cast<const E*>(a.v);
  E* out = reinterpret_cast<E*>(a.out);
  const int ctx = a.ctx[b];
  constexpr int DL = D / 64;
  if (ctx < 0 || (long long)ctx + a.T > (long long)a.max_blocks * a.bs) {
    if (lane == 0) set_status(a.status, SD_ERR_CAPACITY);
    for (int k = 0; k < DL; ++k) Elem<E>::store(out, row * D + lane + 64 * k, 0.f);
    return;
  }
  const int bt = a.tree_stride ? b : 0;
  const uint64_t* anc = a.anc + ((size_t)bt * a.T + i) * a.W64;
  const int32_t* sel = a.sel ? a.sel + row * a.ksel : nullptr;
  const int nblk_ctx = (ctx + a.bs - 1) / a.bs;
  const long long n_ctx_keys = sel ? (long long)a.ksel * a.bs : ctx;
  const long long n_keys = n_ctx_keys + a.T;
  float m = -1e30f, l = 0.f, o[DL];
  for (int k = 0; k < DL; ++k) o[k] = 0.f;
  for (long long c0 = 0; c0 < n_keys; c0 += 64) {
    // lane <-> key c0 + lane: position, visibility, score
    const long long kidx = c0 + lane;
    long long pos = -1;
    if (kidx < n_ctx_keys) {
      if (sel) {
        const int e = (int)(kidx / a.bs);
        const int n = sel[e];
        const bool dup = (e > 0 && n >= 0 && sel[e - 1] >= n);
        if (n >= nblk_ctx || dup) set_status(a.status, SD_ERR_SELECTION);
        const long long p = (long long)n * a.bs + kidx % a.bs;
        if (n >= 0 && n < nblk_ctx && !dup && p < ctx) pos = p;
      } else {
        pos = kidx;
      }
    } else if (kidx < n_keys) {
      const int j = (int)(kidx - n_ctx_keys);
      if ((anc[j >> 6] >> (j & 63)) & 1ull) pos = ctx + j;
    }
    float s = -1e30f;
    long long vbase = -1;
    if (pos >= 0) {
      const int blk = a.table[(size_t)b * a.max_blocks + pos / a.bs];
      if (blk < 0 || blk >= a.num_blocks) {
        set_status(a.status, SD_ERR_BLOCK);
      } else {
        const int off = (int)(pos % a.bs);
        const E* kr = K + (((size_t)blk * a.Hkv + g) * a.bs + off) * D;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += Elem<E>::load(q, d) * Elem<E>::load(kr, d);
        s = acc * a.scale_log2;
        vbase = ((long long)blk * a.Hkv + g) * D * a.bs + off;
      }
    }
    float cm = s;
    for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float mn = fmaxf(m, cm);
    const float alpha = exp2f(m - mn);
    const float p = (vbase >= 0) ? exp2f(s - mn) : 0.f;
    float ps = p;
    for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
    m = mn;
    for (int k = 0; k < DL; ++k) o[k] *= alpha;
    // lanes now own output dims: accumulate the 64 keys' values
    const int vlo = (int)(vbase & 0xffffffffll), vhi = (int)(vbase >> 32);
    for (int kk = 0; kk < 64; ++kk) {
      const float w = __shfl(p, kk);
      const long long base = ((long long)__shfl(vhi, kk) << 32) | (unsigned)__shfl(vlo, kk);
      if (base >= 0) {
        for (int k = 0; k < DL; ++k) o[k] += w * Elem<E>::load(V, base + (size_t)(lane + 64 * k) * a.bs);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int k = 0; k < DL; ++k) Elem<E>::store(out, row * D + lane + 64 * k, o[k] * inv);
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention.
//
// Work unit (one workgroup of 4 wavefronts): sequence b, KV head g, a tile of
// ROWS query rows of that group (row r = node r / G, head g * G + r % G) and a
// contiguous range of key tiles (one context split).  Waves are arranged WQ x
// WK: WQ waves cover different query rows and share every key; WK waves take
// disjoint key slices of each tile and merge their softmax states at the end.
//
// Per tile of NK keys: K rows [NK][D] and V^T rows [D][NK] are loaded with
// 16-byte global loads into registers (prefetched one tile ahead), stored to
// one of two LDS buffers and read by every wave.  S^T = K Q^T is formed with
// v_mfma_f32_16x16x32_bf16 with Q^T held in registers; the K rows fed to the
// two 16-row halves of each 32-key group are interleaved so that the
// accumulator layout of S^T is directly the B operand of O^T = V^T P^T.
// Each lane therefore owns one query column, and the online-softmax scale is a
// per-lane scalar; the row max needs two cross-lane steps.
template <int D, int QW, int WQ, int WK, int KW>
__global__ void __launch_bounds__(256, 1) attn_mfma_kernel(AttnArgs a) {
  constexpr int NK = KW * WK;
  constexpr int ROWS = WQ * QW;
  constexpr int QB = QW / 16;
  constexpr int DS = D / 32;
  constexpr int DB = D / 16;
  constexpr int KG = KW / 32;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = NK + 8;
  constexpr int KCH = D / 8;
  constexpr int K_ITEMS = NK * KCH / 256;
  constexpr int V_ITEMS = D * (NK / 8) / 256;
  static_assert(K_ITEMS * 256 == NK * KCH && V_ITEMS * 256 == D * (NK / 8), "tile split");
  static_assert(WQ * WK == 4, "four wavefronts");

  // K rows 16 apart fall on the same LDS banks with a 17-chunk stride; the
  // 16-byte chunk index is XOR-ed with 4 on rows whose bit 4 is set.
  auto kswz = [](int row) { return ((row >> 4) & 1) << 2; };
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_bits* Ks = reinterpret_cast<bf16_bits*>(smem);
  bf16_bits* Vs = Ks + 2 * NK * KSTR;
  unsigned char* tflag = reinterpret_cast<unsigned char*>(Vs + 2 * D * VSTR);
  uint32_t* ubits = reinterpret_cast<uint32_t*>(tflag + 128);
  __shared__ int s_nU;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % WQ;
  const int wk = wave / WQ;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // Workgroup id -> (b, g, split, qtile).  Workgroups are dispatched round-robin
  // over the 8 XCDs; consecutive logical ids are placed on the same XCD so the
  // query tiles that read the same KV share that XCD's L2.
  const int nwg = gridDim.x;
  int L = blockIdx.x;
  if ((nwg & 7) == 0) L = (L & 7) * (nwg >> 3) + (L >> 3);
  const int qtile = L % a.n_qtiles;
  L /= a.n_qtiles;
  const int split = L % a.n_splits;
  L /= a.n_splits;
  const int g = L % a.Hkv;
  const int b = L / a.Hkv;

  const int T = a.T, G = a.G, M = a.M, bs = a.bs;
  const bf16_bits* __restrict__ Kp = reinterpret_cast<const bf16_bits*>(a.k);
  const bf16_bits* __restrict__ Vp = reinterpret_cast<const bf16_bits*>(a.v);
  const int32_t* __restrict__ table = a.table + (size_t)b * a.max_blocks;
  const int ctx = a.ctx[b];
  const bool cap_ok = ctx >= 0 && (long long)ctx + T <= (long long)a.max_blocks * bs;
  const int bt = a.tree_stride ? b : 0;
  const int row0 = qtile * ROWS;
  const int rowbase = row0 + wq * QW;
  const bool sparse = a.sel != nullptr;

  // ---- query fragments (B operand of S^T = K Q^T) -------------------------
  bf16x8 qf[QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = rowbase + qb * 16 + l16;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < M) {
        const int i = r / G, h = g * G + r % G;
        v = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_bits*>(a.q) +
                                            (((size_t)b * T + i) * a.Hq + h) * D + ds * 32 + lg * 8);
      }
      qf[qb][ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tree tiles touched by any row of this workgroup -------------------
  const int n_tt = (T + NK - 1) / NK;
  if (tid < 128) tflag[tid] = 0;
  __syncthreads();
  {
    const int r_hi = min(row0 + ROWS, M);
    if (row0 < r_hi) {
      const int i_lo = row0 / G, i_hi = (r_hi - 1) / G;
      const int cnt = (i_hi - i_lo + 1) * a.W64;
      for (int idx = tid; idx < cnt; idx += 256) {
        const int i = i_lo + idx / a.W64, w = idx % a.W64;
        if (a.anc[((size_t)bt * T + i) * a.W64 + w] != 0ull) tflag[(w * 64) / NK] = 1;
      }
    }
  }

  // ---- sparse: union of the blocks selected by this workgroup's rows -----
  const int nblk_ctx = cap_ok ? (ctx + bs - 1) / bs : 0;
  const int UW = (a.u_max + 31) >> 5;
  const int BW = (nblk_ctx + 31) >> 5;
  uint32_t* upre = ubits + ((a.max_blocks + 31) >> 5);
  int* U = reinterpret_cast<int*>(upre + ((a.max_blocks + 31) >> 5));
  uint32_t* rowbits = reinterpret_cast<uint32_t*>(U + a.u_max);
  int nU = 0;
  if (sparse) {
    const int r_hi = min(row0 + ROWS, M);
    for (int w = tid; w < BW; w += 256) ubits[w] = 0;
    for (int w = tid; w < ROWS * UW; w += 256) rowbits[w] = 0;
    __syncthreads();
    const int nsel = max(r_hi - row0, 0) * a.ksel;
    if (cap_ok) {
      for (int idx = tid; idx < nsel; idx += 256) {
        const int r = row0 + idx / a.ksel, e = idx % a.ksel;
        const int i = r / G, h = g * G + r % G;
        const int32_t* sr = a.sel + (((size_t)b * T + i) * a.Hq + h) * a.ksel;
        const int n = sr[e];
        if (n < 0) continue;
        if (n >= nblk_ctx || (e > 0 && sr[e - 1] >= n)) {
          set_status(a.status, SD_ERR_SELECTION);
          continue;
        }
        atomicOr(&ubits[n >> 5], 1u << (n & 31));
      }
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int w = 0; w < BW; ++w) {
        upre[w] = acc;
        acc += __popc(ubits[w]);
      }
      s_nU = acc;
    }
    __syncthreads();
    nU = s_nU;
    for (int w = tid; w < BW; w += 256) {
      uint32_t bits = ubits[w];
      int o = upre[w];
      while (bits) {
        const int bpos = __ffs(bits) - 1;
        bits &= bits - 1;
        U[o++] = w * 32 + bpos;
      }
    }
    if (cap_ok) {
      for (int idx = tid; idx < nsel; idx += 256) {
        const int rl = idx / a.ksel, e = idx % a.ksel;
        const int r = row0 + rl;
        const int i = r / G, h = g * G + r % G;
        const int32_t* sr = a.sel + (((size_t)b * T + i) * a.Hq + h) * a.ksel;
        const int n = sr[e];
        if (n < 0 || n >= nblk_ctx || (e > 0 && sr[e - 1] >= n)) continue;
        const int u = upre[n >> 5] + __popc(ubits[n >> 5] & ((1u << (n & 31)) - 1u));
        atomicOr(&rowbits[rl * UW + (u >> 5)], 1u << (u & 31));
      }
    }
  }
  __syncthreads();

  // ---- tile range of this split ------------------------------------------
  const int nct = !cap_ok ? 0 : (sparse ? (nU * bs + NK - 1) / NK : (ctx + NK - 1) / NK);
  const int ntot = cap_ok ? nct + n_tt : 0;
  const int t_lo = split * a.tps;
  const int t_hi = min(t_lo + a.tps, ntot);
  auto usable = [&](int t) { return t < nct || tflag[t - nct]; };
  auto next_tile = [&](int t) {
    ++t;
    while (t < t_hi && !usable(t)) ++t;
    return t;
  };

  // Logical position of key k of tile t, or -1.
  auto key_pos = [&](int t, int k) -> int {
    if (t < nct) {
      if (!sparse) {
        const int p = t * NK + k;
        return p < ctx ? p : -1;
      }
      const int vi = t * NK + k;
      const int e = vi / bs;
      if (e >= nU) return -1;
      const int p = U[e] * bs + vi % bs;
      return p < ctx ? p : -1;
    }
    const int j = (t - nct) * NK + k;
    return j < T ? ctx + j : -1;
  };
  auto block_of = [&](int pos) -> int {
    const int blk = table[pos / bs];
    if (blk < 0 || blk >= a.num_blocks) {
      set_status(a.status, SD_ERR_BLOCK);
      return -1;
    }
    return blk;
  };

  uint4 kreg[K_ITEMS], vreg[V_ITEMS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int n = 0; n < K_ITEMS; ++n) {
      const int it = tid + 256 * n;
      const int row = it / KCH, ch = it % KCH;
      const int pos = key_pos(t, row);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos >= 0) {
        const int blk = block_of(pos);
        if (blk >= 0)
          v = *reinterpret_cast<const uint4*>(Kp + (((size_t)blk * a.Hkv + g) * bs + pos % bs) * D +
                                              ch * 8);
      }
      kreg[n] = v;
    }
#pragma unroll
    for (int n = 0; n < V_ITEMS; ++n) {
      const int it = tid + 256 * n;
      const int d = it / (NK / 8), kc = it % (NK / 8);
      const int p0 = key_pos(t, kc * 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (p0 >= 0 && (p0 & 7) == 0 && key_pos(t, kc * 8 + 7) == p0 + 7) {
        const int blk = block_of(p0);
        if (blk >= 0)
          v = *reinterpret_cast<const uint4*>(Vp + (((size_t)blk * a.Hkv + g) * D + d) * bs + p0 % bs);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (int e = 0; e < 8; ++e) {
          const int p = key_pos(t, kc * 8 + e);
          if (p < 0) continue;
          const int blk = block_of(p);
          if (blk < 0) continue;
          const uint32_t x = Vp[(((size_t)blk * a.Hkv + g) * D + d) * bs + p % bs];
          w[e >> 1] |= x << (16 * (e & 1));
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      vreg[n] = v;
    }
  };
  auto store_tile = [&](int buf) {
    bf16_bits* Kt = Ks + buf * NK * KSTR;
    bf16_bits* Vt = Vs + buf * D * VSTR;
#pragma unroll
    for (int n = 0; n < K_ITEMS; ++n) {
      const int it = tid + 256 * n;
      const int row = it / KCH, ch = it % KCH;
      *reinterpret_cast<uint4*>(Kt + row * KSTR + ((ch ^ kswz(row)) * 8)) = kreg[n];
    }
#pragma unroll
    for (int n = 0; n < V_ITEMS; ++n) {
      const int it = tid + 256 * n;
      const int d = it / (NK / 8), kc = it % (NK / 8);
      *reinterpret_cast<uint4*>(Vt + d * VSTR + kc * 8) = vreg[n];
    }
  };

  // ---- per-lane softmax state ----------------------------------------------
  float m_run[QB], l_run[QB];
  f32x4 o[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // node of each of this lane's query columns (or -1 past M)
  int node[QB];
  int rloc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = rowbase + qb * 16 + l16;
    node[qb] = r < M ? r / G : -1;
    rloc[qb] = r - row0;
  }
  const int kbase = wk * KW;

  auto compute_tile = [&](int buf, int t) {
    const bf16_bits* Kt = Ks + buf * NK * KSTR;
    const bf16_bits* Vt = Vs + buf * D * VSTR;
    f32x4 s[QB][2 * KG];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = kbase + 32 * kg + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][2 * kg + half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8 ka =
              *reinterpret_cast<const bf16x8*>(Kt + key * KSTR + (((ds * 4 + lg) ^ kswz(key)) * 8));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][2 * kg + half] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][ds], s[qb][2 * kg + half], 0, 0, 0);
        }
      }
    }
    // visibility of this lane's 8 keys per 32-key group
    uint32_t vis[QB][KG];
    const bool full_ctx = (t < nct) && !sparse && (t * NK + NK <= ctx);
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int k0 = kbase + 32 * kg + 8 * lg;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint32_t bits = 0xFFu;
        if (!full_ctx) {
          if (t < nct) {
            if (!sparse) {
              const int p = t * NK + k0;
              bits = p >= ctx ? 0u : (p + 8 <= ctx ? 0xFFu : ((1u << (ctx - p)) - 1u));
            } else {
              const int vi = t * NK + k0;
              const int e = vi / bs;
              bits = 0u;
              if (e < nU && node[qb] >= 0 &&
                  ((rowbits[rloc[qb] * UW + (e >> 5)] >> (e & 31)) & 1u)) {
                const int p = U[e] * bs + vi % bs;
                bits = p >= ctx ? 0u : (p + 8 <= ctx ? 0xFFu : ((1u << (ctx - p)) - 1u));
              }
            }
          } else {
            const int j0 = (t - nct) * NK + k0;
            bits = 0u;
            if (node[qb] >= 0 && j0 < T) {
              const uint64_t word = a.anc[((size_t)bt * T + node[qb]) * a.W64 + (j0 >> 6)];
              bits = (uint32_t)(word >> (j0 & 63)) & 0xFFu;
            }
          }
        }
        vis[qb][kg] = bits;
      }
    }
    // online softmax, P^T operands
    bf16x8 pf[QB][KG];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -1e30f;
#pragma unroll
      for (int kg = 0; kg < KG; ++kg)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v = s[qb][2 * kg + half][j] * a.scale_log2;
            if (!((vis[qb][kg] >> (4 * half + j)) & 1u)) v = -1e30f;
            s[qb][2 * kg + half][j] = v;
            mx = fmaxf(mx, v);
          }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_run[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mn);
      m_run[qb] = mn;
      float lsum = 0.f;
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        bf16x8 pk;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = s[qb][2 * kg + half][j];
            const float p = v > -1e29f ? __builtin_amdgcn_exp2f(v - mn) : 0.f;
            const bf16_bits pb = f32_to_bf16(p);
            lsum += bf16_to_f32(pb);
            pk[4 * half + j] = __builtin_bit_cast(__bf16, pb);
          }
        pf[qb][kg] = pk;
      }
      l_run[qb] = l_run[qb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(Vt + (db * 16 + l16) * VSTR + kbase + 32 * kg + 8 * lg);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[qb][kg], o[qb][db], 0, 0, 0);
      }
    }
  };

  // ---- main loop: double-buffered LDS, register prefetch one tile ahead ---
  int t = t_lo;
  while (t < t_hi && !usable(t)) ++t;
  if (t < t_hi) {
    load_tile(t);
    store_tile(0);
  }
  __syncthreads();
  int tn = t < t_hi ? next_tile(t) : t_hi;
  if (tn < t_hi) load_tile(tn);
  int buf = 0;
  while (t < t_hi) {
    compute_tile(buf, t);
    if (tn < t_hi) store_tile(buf ^ 1);
    __syncthreads();
    t = tn;
    buf ^= 1;
    if (t < t_hi) {
      tn = next_tile(t);
      if (tn < t_hi) load_tile(tn);
    }
  }

  // ---- finish: per-column sums, merge key-sliced waves, write -------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  if constexpr (WK > 1) {
    __syncthreads();
    float* xm = reinterpret_cast<float*>(smem);  // [4][QW]
    float* xl = xm + 4 * QW;                     // [4][QW]
    float* xo = xl + 4 * QW;                     // [4][QW][D]
    if (wk > 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qc = qb * 16 + l16;
        if (lg == 0) {
          xm[wave * QW + qc] = m_run[qb];
          xl[wave * QW + qc] = l_run[qb];
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) xo[(wave * QW + qc) * D + db * 16 + 4 * lg + j] = o[qb][db][j];
      }
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int kw = 1; kw < WK; ++kw) {
        const int ow = wq + WQ * kw;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qc = qb * 16 + l16;
          const float mo = xm[ow * QW + qc], lo = xl[ow * QW + qc];
          const float mn = fmaxf(m_run[qb], mo);
          const float fs = __builtin_amdgcn_exp2f(m_run[qb] - mn);
          const float fo = __builtin_amdgcn_exp2f(mo - mn);
          m_run[qb] = mn;
          l_run[qb] = l_run[qb] * fs + lo * fo;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              o[qb][db][j] = o[qb][db][j] * fs + xo[(ow * QW + qc) * D + db * 16 + 4 * lg + j] * fo;
        }
      }
    }
  }
  if (wk != 0) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = rowbase + qb * 16 + l16;
    if (r >= M) continue;
    const int i = r / G, h = g * G + r % G;
    const size_t orow = ((size_t)b * T + i) * a.Hq + h;
    if (a.n_splits == 1) {
      const float inv = l_run[qb] > 0.f ? 1.f / l_run[qb] : 0.f;
      bf16_bits* out = reinterpret_cast<bf16_bits*>(a.out) + orow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t lo = f32_to_bf16(o[qb][db][0] * inv) | ((uint32_t)f32_to_bf16(o[qb][db][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16(o[qb][db][2] * inv) | ((uint32_t)f32_to_bf16(o[qb][db][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + db * 16 + 4 * lg) = make_uint2(lo, hi);
      }
    } else {
      const size_t pr = orow * a.n_splits + split;
      float* po = a.part_o + pr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(po + db * 16 + 4 * lg) = o[qb][db];
      if (lg == 0) {
        a.part_ml[pr * 2 + 0] = m_run[qb];
        a.part_ml[pr * 2 + 1] = l_run[qb];
      }
    }
  }
  if (!cap_ok && tid == 0 && split == 0 && qtile == 0) set_status(a.status, SD_ERR_CAPACITY);
}

// ---------------------------------------------------------------------------
// Merge split partials: out = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           bf16_bits* __restrict__ out,
                                                           long long nrows, int S) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + wave;
  if (row >= nrows) return;
  const float* ml = part_ml + row * S * 2;
  float m = -1e30f;
  for (int s = 0; s < S; ++s) m = fmaxf(m, ml[2 * s]);
  constexpr int DL = D / 64;
  float acc[DL], l = 0.f;
  for (int k = 0; k < DL; ++k) acc[k] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - m);
    l += w * ml[2 * s + 1];
    const float* po = part_o + (row * S + s) * D;
    for (int k = 0; k < DL; ++k) acc[k] += w * po[lane + 64 * k];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int k = 0; k < DL; ++k) out[row * D + lane + 64 * k] = f32_to_bf16(acc[k] * inv);
}

// ---------------------------------------------------------------------------
// Host-side launchers.

hipError_t launch_anc_mask(const int32_t* parent, int T, int W64, int n_trees, uint64_t* anc,
                           uint32_t* status, hipStream_t st) {
  dim3 grid((T + 255) / 256, n_trees);
  hipLaunchKernelGGL(anc_mask_kernel, grid, dim3(256), 0, st, parent, T, W64, anc, status);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_valu_d(const AttnArgs& a, bool f32, hipStream_t st) {
  const long long nrows = (long long)a.B * a.T * a.Hq;
  dim3 grid((unsigned)((nrows + 3) / 4));
  if (f32)
    hipLaunchKernelGGL((attn_valu_kernel<float, D>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_valu_kernel<bf16_bits, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_valu(const AttnArgs& a, bool f32, hipStream_t st) {
  return a.D == 64 ? launch_valu_d<64>(a, f32, st) : launch_valu_d<128>(a, f32, st);
}

template <int D, int QW, int WQ, int WK, int KW>
static hipError_t launch_mfma_cfg(const AttnArgs& a, size_t lds, hipStream_t st) {
  auto fn = attn_mfma_kernel<D, QW, WQ, WK, KW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned nwg = (unsigned)a.B * a.Hkv * a.n_qtiles * a.n_splits;
  hipLaunchKernelGGL(fn, dim3(nwg), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  if (p.WQ == 1) return launch_mfma_cfg<D, 32, 1, 4, 32>(a, p.lds_bytes, st);
  if (p.WQ == 2) return launch_mfma_cfg<D, 32, 2, 2, 32>(a, p.lds_bytes, st);
  return launch_mfma_cfg<D, 32, 4, 1, 64>(a, p.lds_bytes, st);
}

hipError_t launch_attn_mfma(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  hipError_t e = a.D == 64 ? launch_mfma_d<64>(a, p, st) : launch_mfma_d<128>(a, p, st);
  if (e != hipSuccess || a.n_splits == 1) return e;
  const long long nrows = (long long)a.B * a.T * a.Hq;
  dim3 grid((unsigned)((nrows + 3) / 4));
  bf16_bits* out = reinterpret_cast<bf16_bits*>(a.out);
  if (a.D == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, st, a.part_o, a.part_ml, out, nrows,
                       a.n_splits);
  else
    hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, st, a.part_o, a.part_ml, out, nrows,
                       a.n_splits);
  return hipGetLastError();
}

}  // namespace sdtree
