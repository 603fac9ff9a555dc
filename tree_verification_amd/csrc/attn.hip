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
//   attn_valu_kernel    one workgroup per query row, float32 math (fp32 inputs)
//   attn_mfma_kernel    bf16 MFMA flash-style kernel: K / V tiles staged in LDS
//                       and shared by every query row of a KV group, online
//                       softmax in registers, split context with partials
//   attn_combine_kernel merges split partials into the normalised output
#include <type_traits>
#include <utility>

#include <hip/hip_ext.h>

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
// float32 attention, one workgroup per query row (b, i, h).  Keys are walked
// 64 at a time in a virtual order: dense = positions [0, ctx) then the tree
// slots ctx + j; sparse = the ksel * bs slots of the row's selected blocks,
// then the tree slots.  Tree slot j is visible when j is an ancestor of i.
// The four wavefronts take every fourth 64-key chunk, each with its own
// online softmax, and merge their (max, sum, output) states at the end.
template <typename E, int D>
__global__ void __launch_bounds__(256) attn_valu_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long row = blockIdx.x;
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
  const int32_t* sel = a.sel ? a.sel + (size_t)row * a.ksel : nullptr;
  const int nblk_ctx = (ctx + a.bs - 1) / a.bs;
  const long long n_ctx_keys = sel ? (long long)a.ksel * a.bs : ctx;
  const long long n_keys = n_ctx_keys + a.T;
  float m = -1e30f, l = 0.f, o[DL];
  for (int k = 0; k < DL; ++k) o[k] = 0.f;
  for (long long c0 = 64LL * wave; c0 < n_keys; c0 += 256) {
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
        vbase = (((long long)blk * a.Hkv + g) * a.bs + off) * D;
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
    // lanes now own output dims: accumulate the 64 keys' values, eight keys'
    // loads in flight at a time (a key that is not visible reads element 0
    // and contributes zero)
    const int vlo = (int)(vbase & 0xffffffffll), vhi = (int)(vbase >> 32);
    for (int k0 = 0; k0 < 64; k0 += 8) {
      float w[8], v[8][DL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const long long base = ((long long)__shfl(vhi, k0 + u) << 32) | (unsigned)__shfl(vlo, k0 + u);
        const bool vis = base >= 0;
        w[u] = vis ? __shfl(p, k0 + u) : 0.f;
        const long long bb = vis ? base : 0;
#pragma unroll
        for (int k = 0; k < DL; ++k) {
          const float x = Elem<E>::load(V, bb + lane + 64 * k);
          v[u][k] = vis ? x : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int k = 0; k < DL; ++k) o[k] += w[u] * v[u][k];
    }
  }
  __shared__ float xm[4], xl[4], xo[4][D];
  if (lane == 0) {
    xm[wave] = m;
    xl[wave] = l;
  }
  for (int k = 0; k < DL; ++k) xo[wave][lane + 64 * k] = o[k];
  __syncthreads();
  if (wave != 0) return;
  float mt = xm[0];
  for (int w = 1; w < 4; ++w) mt = fmaxf(mt, xm[w]);
  float lt = 0.f, ot[DL];
  for (int k = 0; k < DL; ++k) ot[k] = 0.f;
  for (int w = 0; w < 4; ++w) {
    const float f = exp2f(xm[w] - mt);
    lt += xl[w] * f;
    for (int k = 0; k < DL; ++k) ot[k] += xo[w][lane + 64 * k] * f;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  for (int k = 0; k < DL; ++k) Elem<E>::store(out, row * D + lane + 64 * k, ot[k] * inv);
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
// Key tiles of NK keys stream through an S-stage LDS ring: each K row [D] and
// each V row [D] is brought in with 16-byte direct global-to-LDS loads
// (global_load_lds_dwordx4), issued S - 1 tiles ahead and waited for with an
// explicit vmcnt before the tile's barrier, so up to S - 1 tiles are in flight
// while one is computed.  LDS rows are unpadded; the 16-byte chunk a lane
// writes is chosen (XOR swizzle) so that the rows read by one MFMA operand
// fetch fall on distinct banks.  Keys that do not exist (past a context or
// tree edge) read a zero page.  The V^T operand of P V is formed from the V
// rows by the LDS transposing reads (ds_read_b64_tr_b16).
//
// S^T = K Q^T is formed with v_mfma_f32_16x16x32_bf16 with Q^T held in
// registers; the K rows fed to the two 16-row halves of each 32-key group are
// interleaved so that the accumulator layout of S^T is directly the B operand
// of O^T = V^T P^T.  Each lane therefore owns one query column, the
// online-softmax scale is a per-lane scalar and the row max needs two
// cross-lane steps.
// Reference-max slack of the online softmax, in log2 units: probabilities are
// formed relative to a running max that may lag the true one by up to this.
constexpr float kLazy = 8.0f;

// Calls f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N - 1>).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

template <int D, int QW, int WQ, int WK, int KW, int S>
__global__ void __launch_bounds__(WQ * WK * 64) attn_mfma_kernel(AttnArgs a) {
  constexpr int NWAVE = WQ * WK;
  constexpr int NT = NWAVE * 64;
  constexpr int NK = KW * WK;
  constexpr int ROWS = WQ * QW;
  constexpr int QB = QW / 16;
  constexpr int DS = D / 32;
  constexpr int DB = D / 16;
  constexpr int KG = KW / 32;
  constexpr int CK = D / 8;                      // 16-byte chunks per K or V row
  constexpr int K_BYTES = NK * D * 2;
  constexpr int V_BYTES = NK * D * 2;
  constexpr int K_OPS = K_BYTES / (NT * 16);     // DMA instructions per thread per tile
  constexpr int V_OPS = K_OPS;                   // (a V row is laid out as a K row)
  constexpr int OPS = K_OPS + V_OPS;
  static_assert(K_OPS * NT * 16 == K_BYTES, "tile split");
  static_assert(NWAVE == 4 || NWAVE == 8, "four or eight wavefronts");
  static_assert(S >= 2 && (S - 1) * OPS <= 63, "vmcnt range");

  // K tile: chunk c of K row r sits at position c ^ kswz(r) of the row (one
  // K operand read takes 16-byte chunks of the 16 K rows {8a + 4h + b} of a
  // 32-key group).
  // V tile: stored in 256-byte slabs of 8 keys x 16 dims.  Key
  // 16 m + 8 e + 4 h + k (e, h in {0, 1}, k < 4), dims 16 d .. 16 d + 15, lie
  // at byte m * 32 D + h * 16 D + d * 256 + (4 e + k) * 32.  One V operand
  // read is a pair of transposing 8-byte reads (h = 0, 1) in which the 32
  // lanes of a half wavefront cover one slab exactly, so they meet no bank
  // twice, and a lane's address differs between fragments by constants only.
  auto kswz = [](int r) -> int {
    return CK == 16 ? ((r & 3) | ((r >> 1) & 12)) : (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
  };

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* Kst = smem;                                 // [S][K_BYTES]  (NK rows of D)
  unsigned char* Vst = smem + S * K_BYTES;                   // [S][V_BYTES]  (NK rows of D)
  unsigned char* tflag = Vst + S * V_BYTES;                  // [128]
  int* tlist = reinterpret_cast<int*>(tflag + 128);          // [128]
  // element offset of (block, head g) for this split's context blocks / the tree blocks
  long long* ctab = reinterpret_cast<long long*>(tlist + 128);
  long long* ttab = ctab + a.ct_max;
  uint64_t* ancL = reinterpret_cast<uint64_t*>(ttab + a.tt_max);
  uint32_t* ubits = reinterpret_cast<uint32_t*>(ancL + a.anc_lds_words);
  __shared__ int s_nU, s_err, s_ntree;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so indexes built from it stay scalar
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
  const int bsh = a.bs_shift, bsm = bs - 1;
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

  // ---- ancestors of this workgroup's nodes; tree tiles any of them touch ---
  const int n_tt = (T + NK - 1) / NK;
  const int r_hi = min(row0 + ROWS, M);
  const int i_lo = row0 / G;
  const int i_hi = row0 < r_hi ? (r_hi - 1) / G : i_lo - 1;
  // The parents of nodes 0..i_hi are staged in the still idle K/V ring; each of
  // the tile's nodes then collects its inclusive ancestor set by walking up to
  // a root, validating the parents on the way (a parent precedes its child; a
  // non-root node may have parent -1, a forest).  ancL is sized by the plan for
  // every node of the tile.
  int* s_par = reinterpret_cast<int*>(smem);
  static_assert(2 * (K_BYTES + V_BYTES) >= 4 * kMaxTreeNodes, "parents fit the ring");
  const int nn = i_hi - i_lo + 1;
  SD_DCHECK(nn <= 0 || (long long)nn * a.W64 <= a.anc_lds_words, a.status);
  SD_DCHECK(n_tt <= 128, a.status);
  // flag the tree tiles (NK nodes each) that a nonzero ancestor word touches
  auto flag_word = [&](int w, uint64_t acc) {
    if constexpr (NK >= 64) {
      tflag[(w * 64) / NK] = 1;
    } else {
#pragma unroll
      for (int h = 0; h < 64 / NK; ++h)
        if ((acc >> (h * NK)) & ((1ull << NK) - 1ull)) tflag[(w * 64) / NK + h] = 1;
    }
  };
  if (tid < 128) tflag[tid] = 0;
  if (tid == 0) s_err = 0;
  // (loads batched so that a thread's loads are in flight together: a plain
  // loop waits for each load before the next iteration's)
  constexpr int LB = 4;
  for (int j0 = 0; j0 <= i_hi; j0 += LB * NT) {
    int pv[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = j0 + u * NT + tid;
      pv[u] = j <= i_hi ? a.parent[(size_t)bt * T + j] : 0;
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = j0 + u * NT + tid;
      if (j <= i_hi) s_par[j] = pv[u];
    }
  }
  for (int idx = tid; idx < nn * a.W64; idx += NT) ancL[idx] = 0ull;
  __syncthreads();
  int err = 0;
  for (int idx = tid; idx < nn; idx += NT) {
    uint64_t* row = ancL + idx * a.W64;
    int n = i_lo + idx, cur_w = n >> 6;
    uint64_t acc = 0;
    while (true) {
      const int w = n >> 6;
      if (w != cur_w) {
        row[cur_w] = acc;
        flag_word(cur_w, acc);
        cur_w = w;
        acc = 0;
      }
      acc |= 1ull << (n & 63);
      const int par = s_par[n];
      if (n == 0 ? par != -1 : (par >= n || par < -1)) err |= SD_ERR_PARENT;
      if (n == 0 || par >= n || par < 0) break;
      n = par;
    }
    row[cur_w] = acc;
    flag_word(cur_w, acc);
  }

  // ---- sparse: union of the blocks selected by this workgroup's rows -----
  const int nblk_ctx = cap_ok ? (ctx + bs - 1) >> bsh : 0;
  const int UW = (a.u_max + 31) >> 5;
  const int BW = (nblk_ctx + 31) >> 5;
  uint32_t* upre = ubits + ((a.max_blocks + 31) >> 5);
  int* U = reinterpret_cast<int*>(upre + ((a.max_blocks + 31) >> 5));
  int* Uphys = U + a.u_max;
  uint32_t* rowbits = reinterpret_cast<uint32_t*>(Uphys + a.u_max);
  int nU = 0;
  if (sparse) {
    for (int w = tid; w < BW; w += NT) ubits[w] = 0;
    for (int w = tid; w < ROWS * UW; w += NT) rowbits[w] = 0;
    __syncthreads();
    const int nsel = max(r_hi - row0, 0) * a.ksel;
    // Selection entries idx = base + u * NT + tid (u < LB) of this
    // workgroup's rows: the entry n[u] and its row predecessor np[u] (-1 for
    // a row's first entry), all loads in flight together.
    auto sel_batch = [&](int base, int (&n)[LB], int (&np)[LB]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int idx = base + u * NT + tid;
        n[u] = -1;
        np[u] = -1;
        if (idx < nsel) {
          const int rl = idx / a.ksel, e = idx - rl * a.ksel;
          const int r = row0 + rl;
          const int i = r / G, h = g * G + r % G;
          const int32_t* sr = a.sel + (((size_t)b * T + i) * a.Hq + h) * a.ksel;
          n[u] = sr[e];
          if (e > 0) np[u] = sr[e - 1];
        }
      }
    };
    if (cap_ok) {
      for (int base = 0; base < nsel; base += LB * NT) {
        int n[LB], np[LB];
        sel_batch(base, n, np);
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          if (n[u] < 0) continue;
          if (n[u] >= nblk_ctx || np[u] >= n[u]) {
            err |= SD_ERR_SELECTION;
            continue;
          }
          atomicOr(&ubits[n[u] >> 5], 1u << (n[u] & 31));
        }
      }
    }
    __syncthreads();
    // exclusive prefix of the words' bit counts: wavefront 0, 64 words a step
    if (tid < 64) {
      int carry = 0;
      for (int w0 = 0; w0 < BW; w0 += 64) {
        const int w = w0 + tid;
        const int c = w < BW ? __popc(ubits[w]) : 0;
        int x = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off);
          if (tid >= off) x += y;
        }
        if (w < BW) upre[w] = carry + x - c;
        carry += __shfl(x, 63);
      }
      if (tid == 0) s_nU = carry;
    }
    __syncthreads();
    nU = s_nU;
    SD_DCHECK(nU <= a.u_max, a.status);
    for (int w = tid; w < BW; w += NT) {
      uint32_t bits = ubits[w];
      int o = upre[w];
      while (bits) {
        const int bpos = __ffs(bits) - 1;
        bits &= bits - 1;
        U[o++] = w * 32 + bpos;
      }
    }
    __syncthreads();
    // physical ids of the union's blocks, all loads in flight together
    for (int o0 = 0; o0 < nU; o0 += LB * NT) {
      int phys[LB];
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int o = o0 + u * NT + tid;
        phys[u] = o < nU ? table[U[o]] : 0;
      }
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int o = o0 + u * NT + tid;
        if (o >= nU) continue;
        if (phys[u] < 0 || phys[u] >= a.num_blocks) {
          err |= SD_ERR_BLOCK;
          phys[u] = 0;
        }
        Uphys[o] = phys[u];
      }
    }
    if (cap_ok) {
      for (int base = 0; base < nsel; base += LB * NT) {
        int n[LB], np[LB];
        sel_batch(base, n, np);
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          if (n[u] < 0 || n[u] >= nblk_ctx || np[u] >= n[u]) continue;
          const int rl = (base + u * NT + tid) / a.ksel;
          const int uu = upre[n[u] >> 5] + __popc(ubits[n[u] >> 5] & ((1u << (n[u] & 31)) - 1u));
          atomicOr(&rowbits[rl * UW + (uu >> 5)], 1u << (uu & 31));
        }
      }
    }
  }
  __syncthreads();

  // ---- tile range of this split, usable tiles ------------------------------
  const int nct = !cap_ok ? 0 : (sparse ? ((nU << bsh) + NK - 1) / NK : (ctx + NK - 1) / NK);
  const int ntot = cap_ok ? nct + n_tt : 0;
  // The sequence's actual tiles are spread evenly over the splits (the plan's
  // tiles per split bound this share, so the LDS block tables still fit).
  const int tps_here = (ntot + a.n_splits - 1) / a.n_splits;
  const int t_lo = split * tps_here;
  const int t_hi = min(t_lo + tps_here, ntot);
  const int n_ctx_here = max(0, min(t_hi, nct) - t_lo);
  // the flagged tree tiles of this split, in order (wavefront 0 compacts 64
  // tiles at a time with a ballot)
  if (wave == 0) {
    int n = 0;
    for (int t0 = max(t_lo, nct); t0 < t_hi; t0 += 64) {
      const int t = t0 + lane;
      const bool f = t < t_hi && tflag[t - nct];
      const unsigned long long bal = __ballot(f);
      if (f) tlist[n + __popcll(bal & ((1ull << lane) - 1ull))] = t;
      n += __popcll(bal);
    }
    if (lane == 0) s_ntree = n;
  }

  // Physical block ids this split reads, staged once: dense context blocks
  // [cb0, cb0 + ccount) and the blocks holding the tree slots [tb0, tb0 + tcount).
  const int cb0 = (t_lo * NK) >> bsh;
  const int ccount = (!sparse && n_ctx_here > 0)
                         ? min((min(t_hi, nct) * NK - 1) >> bsh, (ctx - 1) >> bsh) - cb0 + 1 : 0;
  const int tb0 = ctx >> bsh;
  const int tcount = (cap_ok && t_hi > nct) ? ((ctx + T - 1) >> bsh) - tb0 + 1 : 0;
  SD_DCHECK(ccount <= a.ct_max && tcount <= a.tt_max, a.status);
  SD_DCHECK(split < a.n_splits && t_hi - t_lo <= a.tps, a.status);
  const long long blk_elems = (long long)a.Hkv * bs * D;
  const long long head_off = (long long)g * bs * D;   // head g inside a K or a V block
  for (int j = tid; j < ccount + tcount; j += NT) {
    const int n = j < ccount ? cb0 + j : tb0 + (j - ccount);
    int phys = table[n];
    if (phys < 0 || phys >= a.num_blocks) {
      err |= SD_ERR_BLOCK;
      phys = 0;
    }
    const long long off = phys * blk_elems + head_off;
    if (j < ccount) ctab[j] = off;
    else ttab[j - ccount] = off;
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const int nuse = n_ctx_here + s_ntree;
  auto tile_at = [&](int k) { return k < n_ctx_here ? t_lo + k : tlist[k - n_ctx_here]; };

  // Logical position of key k of tile t (< 0: none) and the element offset of
  // its (block, head g).
  auto key_at = [&](int t, int k, long long& boff) __attribute__((always_inline)) -> int {
    if (t < nct) {
      if (!sparse) {
        const int p = t * NK + k;
        if (p >= ctx) return -1;
        boff = ctab[(p >> bsh) - cb0];
        return p;
      }
      const int vi = t * NK + k;
      const int e = vi >> bsh;
      if (e >= nU) return -1;
      const int p = (U[e] << bsh) + (vi & bsm);
      if (p >= ctx) return -1;
      boff = (long long)Uphys[e] * blk_elems + head_off;
      return p;
    }
    const int j = (t - nct) * NK + k;
    if (j >= T) return -1;
    const int p = ctx + j;
    boff = ttab[(p >> bsh) - tb0];
    return p;
  };
  const bf16_bits* zeros = reinterpret_cast<const bf16_bits*>(a.zeros);

  // Per-thread DMA geometry (loop invariant).  DMA n of a tile writes the
  // 16-byte slot s = lane + 64 (wave + NWAVE n).  K: row s / CK (a key),
  // position s % CK, holding global chunk (s % CK) ^ kswz(row).  V: byte 16 s
  // of the slab layout, i.e. key v_key and element offset v_col of its row.
  int k_row[K_OPS], k_col[K_OPS], v_key[V_OPS], v_col[V_OPS];
#pragma unroll
  for (int n = 0; n < K_OPS; ++n) {
    const int sl = lane + 64 * (wave + NWAVE * n);
    k_row[n] = sl / CK;
    k_col[n] = ((sl % CK) ^ kswz(sl / CK)) * 8;
    const int o = sl * 16;                      // byte in the V tile
    const int m = o / (32 * D), h = (o / (16 * D)) & 1, d = (o >> 8) & (DB - 1);
    const int j = (o >> 5) & 7, half = (o >> 4) & 1;
    v_key[n] = 16 * m + 8 * (j >> 2) + 4 * h + (j & 3);
    v_col[n] = (2 * d + half) * 8;
  }

  // Issue the loads of tile t's K (issue_k) or V (issue_v) into the ring slot
  // at `kst` / `vst`.  Every thread issues the same number of DMA operations.  The LDS
  // DMA builtin is always given a named pointer variable: handed an array
  // element directly, the host compilation pass silently drops the kernel's
  // launch stub (the link check in the build catches that).
  auto dense_full = [&](int t) { return t < nct && !sparse && t * NK + NK <= ctx; };
  auto issue_k = [&](int t, unsigned char* kst) __attribute__((always_inline)) {
    if (dense_full(t)) {
#pragma unroll
      for (int n = 0; n < K_OPS; ++n) {
        const int p = t * NK + k_row[n];
        const bf16_bits* src = Kp + ctab[(p >> bsh) - cb0] + (long long)((p & bsm) * D + k_col[n]);
        __builtin_amdgcn_global_load_lds(src, kst + (wave + NWAVE * n) * 1024, 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < K_OPS; ++n) {
      long long boff = 0;
      const int p = key_at(t, k_row[n], boff);
      const bf16_bits* src = p >= 0 ? Kp + boff + (long long)((p & bsm) * D + k_col[n]) : zeros;
      __builtin_amdgcn_global_load_lds(src, kst + (wave + NWAVE * n) * 1024, 16, 0, 0);
    }
  };
  auto issue_v = [&](int t, unsigned char* vst) __attribute__((always_inline)) {
    if (dense_full(t)) {
#pragma unroll
      for (int n = 0; n < V_OPS; ++n) {
        const int p = t * NK + v_key[n];
        const bf16_bits* src = Vp + ctab[(p >> bsh) - cb0] + (long long)((p & bsm) * D + v_col[n]);
        __builtin_amdgcn_global_load_lds(src, vst + (wave + NWAVE * n) * 1024, 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < V_OPS; ++n) {
      long long boff = 0;
      const int p = key_at(t, v_key[n], boff);
      const bf16_bits* src = p >= 0 ? Vp + boff + (long long)((p & bsm) * D + v_col[n]) : zeros;
      __builtin_amdgcn_global_load_lds(src, vst + (wave + NWAVE * n) * 1024, 16, 0, 0);
    }
  };

  // ---- per-lane softmax state ----------------------------------------------
  // l_run: this lane's share of its column's sum of p (summed over the four
  // lanes of the column at the end).
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
  typedef f32x4 STile[QB][2 * KG];
  typedef bf16x8 PTile[QB][KG];

  // S^T = K Q^T for this wave's keys of the K tile at Kt.
  auto qk = [&](const unsigned char* Kt, STile& s) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = kbase + 32 * kg + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][2 * kg + half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
              Kt + key * (D * 2) + (((ds * 4 + lg) ^ kswz(key)) * 16));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][2 * kg + half] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][ds], s[qb][2 * kg + half], 0, 0, 0);
        }
      }
    }
  };

  typedef bf16x8 KFrag[KG][2][DS];
  auto load_k = [&](const unsigned char* Kt, KFrag& kf) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = kbase + 32 * kg + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          kf[kg][half][ds] = *reinterpret_cast<const bf16x8*>(
              Kt + key * (D * 2) + (((ds * 4 + lg) ^ kswz(key)) * 16));
      }
  };
  // (halves: a bit mask of the 16-row key halves to compute)
  auto qk_regs = [&](const KFrag& kf, STile& s, int halves = 3) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (!((halves >> half) & 1)) continue;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][2 * kg + half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][2 * kg + half] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kg][half][ds], qf[qb][ds], s[qb][2 * kg + half], 0, 0, 0);
      }
  };

  // Masks the scores of tile t that a query column may not see.
  auto mask_tile = [&](int t, STile& s) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int k0 = kbase + 32 * kg + 8 * lg;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint32_t bits;
        if (t < nct) {
          if (!sparse) {
            const int p = t * NK + k0;
            bits = p >= ctx ? 0u : (p + 8 <= ctx ? 0xFFu : ((1u << (ctx - p)) - 1u));
          } else {
            const int vi = t * NK + k0;
            const int e = vi >> bsh;
            bits = 0u;
            if (e < nU && node[qb] >= 0 &&
                ((rowbits[rloc[qb] * UW + (e >> 5)] >> (e & 31)) & 1u)) {
              const int p = (U[e] << bsh) + (vi & bsm);
              bits = p >= ctx ? 0u : (p + 8 <= ctx ? 0xFFu : ((1u << (ctx - p)) - 1u));
            }
          }
        } else {
          const int j0 = (t - nct) * NK + k0;
          bits = 0u;
          if (node[qb] >= 0 && j0 < T) {
            const uint64_t word = ancL[(node[qb] - i_lo) * a.W64 + (j0 >> 6)];
            bits = (uint32_t)(word >> (j0 & 63)) & 0xFFu;
          }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (!((bits >> (4 * half + j)) & 1u)) s[qb][2 * kg + half][j] = -INFINITY;
      }
    }
  };

  // Online softmax of one tile's (masked) scores; the scale is folded into the
  // exponent.  The reference max m_run is only raised when a score exceeds it
  // by more than 2^kLazy, so p <= 2^kLazy and the accumulators are rarely
  // rescaled.
  const float c = a.scale_log2;
  // The reference max m_run of a query column only has to bound the column's
  // scores to within 2^kLazy.  Each lane checks its own scores; only when some
  // lane exceeds the bound is the exact column max formed (across the four
  // lanes holding the column) and m_run raised, rescaling o and l.
  auto softmax_bound = [&](const STile& s) __attribute__((always_inline)) {
    float lm[QB];
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 2 * KG; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[qb][e][j]);
      lm[qb] = mx;
      any |= mx * c > m_run[qb] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = lm[qb];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * c;
        const bool raise = ms > m_run[qb] + kLazy;
        const float mn = raise ? ms : m_run[qb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mn);
        m_run[qb] = mn;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
      }
    }
  };
  auto exp_tile = [&](const STile& s, PTile& pf) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        bf16x8 pk;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][2 * kg + half][j], c, nm));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][2 * kg + half][j + 1], c, nm));
            l_run[qb] += p0 + p1;
            const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
            pk[4 * half + j] = pp[0];
            pk[4 * half + j + 1] = pp[1];
          }
        pf[qb][kg] = pk;
      }
    }
  };
  // O^T += V^T P^T: the V^T fragments of the tile in ring slot `slot` are
  // read into registers (load_v), then multiplied (pv_regs).  Fragment
  // (kg, db) of lane (lg, l16) is V^T[db * 16 + l16][8 keys from
  // kbase + 32 kg + 8 lg]: two transposing reads, each giving 4 consecutive
  // keys of dim l16.  For such a read the lanes of a 16-lane group each name
  // one 8-byte piece of a 4-key x 16-dim block, lane 4 k + c the piece
  // (key k, dims 4c .. 4c + 3), and lane n receives dim n of the 4 keys.
  typedef bf16x8 VFrag[KG][DB];
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lds_v4p;
  // this lane's byte in the slab layout for key kbase + 8 lg + (l16 >> 2),
  // dims 4 (l16 & 3) .. + 3; fragments add kg, h and d terms
  const int v_lane = ((kbase >> 4) + (lg >> 1)) * (32 * D) + (4 * (lg & 1) + (l16 >> 2)) * 32 + (l16 & 3) * 8;
  // (fragments db0 <= db < db1 only: a step can split the reads in batches
  // that keep the LDS counter's waits exact)
  auto load_v = [&](const unsigned char* Vs, VFrag& vf, int db0 = 0, int db1 = D / 16)
      __attribute__((always_inline)) {
    const unsigned char* Vt = Vs + v_lane;
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db < db0 || db >= db1) continue;
        v4i16 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const unsigned char* at = Vt + kg * (64 * D) + hh * (16 * D) + db * 256;
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(at));
        }
        const v4i16 lo = h[0], hi = h[1];
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        vf[kg][db] = __builtin_bit_cast(bf16x8, w);
      }
  };
  auto pv_regs = [&](const VFrag& vf, const PTile& pf) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kg][db], pf[qb][kg], o[qb][db], 0, 0, 0);
  };
  auto pv = [&](const unsigned char* Vs, const PTile& pf) __attribute__((always_inline)) {
    VFrag vf;
    load_v(Vs, vf);
    pv_regs(vf, pf);
  };

  auto sync_tiles = [&](bool exact) __attribute__((always_inline)) {
    if (exact) __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * OPS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- main loop --------------------------------------------------------------
  // K and V have rings of S slots each.  Tile k's scores are computed one
  // iteration ahead, so iteration k reads K(k + 1) and V(k): it runs the score
  // MFMAs of tile k + 1 beside the softmax of tile k, then tile k's P V.  It
  // then issues K(k + S) into K(k)'s slot (last read in iteration k - 1) and
  // V(k + S - 1) into V(k - 1)'s slot.  Every thread issues the same DMA
  // operations, so K(k + 1) and V(k), issued together in iteration
  // k + 1 - S, have landed once at most the (S - 2) later iterations'
  // operations are outstanding; near the end that count is not exact and
  // everything is drained instead.  The leading whole dense context tiles run
  // in a tight loop (an even number of iterations whose prefetches are whole
  // dense tiles too); the rest (context tail, tree tiles, sparse tiles) in the
  // general loop.  The set-up loads are drained first.
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (k < nuse) {
      issue_k(tile_at(k), Kst + k * K_BYTES);
      issue_v(tile_at(k), Vst + k * V_BYTES);
    }
  if (S - 1 < nuse) issue_k(tile_at(S - 1), Kst + (S - 1) * K_BYTES);
  STile sa, sb;
  PTile pf;
  if (nuse > 0) {
    // K(0) has landed once at most the (S - 1) * OPS operations issued after
    // it (V(0), tiles 1 .. S - 2, K(S - 1)) are outstanding; with fewer than S
    // usable tiles that count is not exact and everything is drained.  Only
    // K(0) is waited for: the rest of the first tiles land while tile 0's
    // scores are formed.
    if (nuse >= S) __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * OPS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    qk(Kst, sa);
  }
  // Whole tiles: dense context tiles inside ctx; sparse tiles made only of
  // whole selected blocks (the union is ascending, so only its last block can
  // be the partial block at the end of the context).
  int n_full;
  if (!sparse) {
    n_full = max(0, min(t_hi, ctx / NK) - t_lo);
  } else {
    const int n_whole = nU - ((nU > 0 && U[nU - 1] == nblk_ctx - 1 && (ctx & bsm) != 0) ? 1 : 0);
    n_full = max(0, min(t_hi, (int)(((long long)n_whole << bsh) / NK)) - t_lo);
  }
  // (a multiple of TU, the tight loop's unroll.  With the 8-stage ring it is
  // a whole ring turn, so every step's ring slots are constants and its
  // fragment reads and DMA destinations fixed offsets from loop-invariant
  // addresses; the other configurations unroll by a pair of score tiles and
  // form the slots at run time, since the invariant addresses would not fit
  // their registers.)
  constexpr bool kConstSlots = S == 8;
  constexpr int TU = kConstSlots ? S : 2;
  const int n_tight = max(0, n_full - S) / TU * TU;
  // DMA sources of K(tk) and V(tk - 1) for a tight step, formed one step
  // ahead so the block-table reads are off the issue path.
  // The 64 / CK K rows one wave-operation copies lie in one page, so that
  // operation's page base is wave-uniform: dense tiles read it from the page
  // offsets the prologue staged and validated in LDS, so a step forms it with
  // one LDS read and no block-table load or 64-bit multiply on the scalar
  // unit, which the CU's wavefronts share; each lane adds a fixed byte offset.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[K_OPS];
#pragma unroll
  for (int n = 0; n < K_OPS; ++n) {
    const int r0 = (64 * (wave_u + NWAVE * n)) / CK;
    koff[n] = (uint32_t)(((k_row[n] - r0) * D + k_col[n]) * 2);
  }
  const unsigned char* kpage[K_OPS];
  const bf16_bits* vsrc[V_OPS];
  // A wave-operation's V bytes (slab layout) and its K rows fall in the same
  // 16-key group of the tile, so with pages of 16 keys or more the V
  // operation reads the page its K operation read one tile earlier: V's page
  // base is that K base, kept from the previous step, plus a fixed per-lane
  // offset, and no per-lane block-table read is needed.
  const bool v_from_k = bs >= 16;
  int vlane[V_OPS];
#pragma unroll
  for (int n = 0; n < V_OPS; ++n) vlane[n] = (v_key[n] & bsm) * D + v_col[n];
  long long kb[K_OPS];  // page element offsets of the K operations of the last tile formed
  // (sparse tiles index the union of selected blocks: virtual key vi lies in
  // union block vi >> bsh, whose validated physical id is Uphys[vi >> bsh])
  auto page_of = [&](auto sp_tag, int p0) __attribute__((always_inline)) -> long long {
    if constexpr (!decltype(sp_tag)::value) {
      // the page's element offset as staged (and validated) in LDS
      const uint64_t bu = (uint64_t)ctab[(p0 >> bsh) - cb0];
      return (long long)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu));
    } else {
      const int phys = __builtin_amdgcn_readfirstlane(Uphys[p0 >> bsh]);
      return phys * blk_elems + head_off;
    }
  };
  auto tight_sources = [&](auto sp_tag, int tk, bool first) __attribute__((always_inline)) {
    constexpr bool SP = decltype(sp_tag)::value;
    if (v_from_k) {
      if (first)
#pragma unroll
        for (int n = 0; n < K_OPS; ++n) kb[n] = page_of(sp_tag, (tk - 1) * NK + (64 * (wave_u + NWAVE * n)) / CK);
      const long long u = (long long)((((tk - 1) * NK) & bsm) * D);
#pragma unroll
      for (int n = 0; n < V_OPS; ++n) vsrc[n] = Vp + (kb[n] + u) + vlane[n];
    } else {
#pragma unroll
      for (int n = 0; n < V_OPS; ++n) {
        const int p = (tk - 1) * NK + v_key[n];
        const long long boff = SP ? (long long)Uphys[p >> bsh] * blk_elems + head_off : ctab[(p >> bsh) - cb0];
        vsrc[n] = Vp + boff + (long long)((p & bsm) * D + v_col[n]);
      }
    }
#pragma unroll
    for (int n = 0; n < K_OPS; ++n) {
      const int p0 = tk * NK + (64 * (wave_u + NWAVE * n)) / CK;
      kb[n] = page_of(sp_tag, p0);
      kpage[n] = reinterpret_cast<const unsigned char*>(Kp + (kb[n] + (long long)((p0 & bsm) * D)));
    }
  };
  // Mask of a whole sparse tile: a row sees an 8-key chunk when it selected
  // the chunk's block.
  auto sparse_mask = [&](int t, STile& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int e = (t * NK + kbase + 32 * kg + 8 * lg) >> bsh;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool vis = node[qb] >= 0 && ((rowbits[rloc[qb] * UW + (e >> 5)] >> (e & 31)) & 1u);
        if (!vis)
#pragma unroll
          for (int half = 0; half < 2; ++half) sc[qb][2 * kg + half] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
  };
  // A step's DMA destinations (kdst, vdst) and the tiles it reads (krd,
  // vrd) are distinct ring slots, and the reads' own DMA was waited for by
  // sync_tiles; the restrict qualifiers say so to the compiler, which would
  // otherwise drain every DMA in flight before the transposing reads.
  auto tight_body = [&](auto sp_tag, int k, STile& sc, STile& sn, unsigned char* __restrict__ kdst,
                        unsigned char* __restrict__ vdst, const unsigned char* __restrict__ krd,
                        const unsigned char* __restrict__ vrd) __attribute__((always_inline)) {
    constexpr bool SP = decltype(sp_tag)::value;
#pragma unroll
    for (int n = 0; n < K_OPS; ++n)
    {
      const unsigned char* src = kpage[n] + koff[n];  // (a named pointer: see issue_k)
      __builtin_amdgcn_global_load_lds(src, kdst + (wave + NWAVE * n) * 1024, 16, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < V_OPS; ++n)
    {
      const bf16_bits* src = vsrc[n];  // (a named pointer: see issue_k)
      __builtin_amdgcn_global_load_lds(src, vdst + (wave + NWAVE * n) * 1024, 16, 0, 0);
    }
    if (k + 1 < n_tight) tight_sources(sp_tag, t_lo + k + 1 + S, false);
    if constexpr (SP) sparse_mask(t_lo + k, sc);
    softmax_bound(sc);
    // The K fragments of tile k + 1 are read before any MFMA and the V^T
    // fragments of tile k ahead of their MFMAs, so their LDS latency is
    // covered; the scheduling barriers keep the compiler from sinking the
    // reads to their first use.  The next step's block-table reads (scalar
    // loads, which return out of order, and LDS reads) are waited for here,
    // leaving only the in-order fragment reads pending.  At most 15 of those
    // are outstanding at a time (the counter's range), so each MFMA waits for
    // just its own operands.
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    KFrag kf;
    load_k(krd, kf);
    __builtin_amdgcn_sched_barrier(0);
    qk_regs(kf, sn, 1);
    // the V^T fragments take two transposing reads each: half of them before
    // the second key half's score MFMAs, half after, so at most 15 LDS reads
    // are outstanding when an MFMA waits for its operands
    VFrag vf;
    load_v(vrd, vf, 0, DB / 2);
    __builtin_amdgcn_sched_barrier(0);
    qk_regs(kf, sn, 2);
    load_v(vrd, vf, DB / 2, DB);
    __builtin_amdgcn_sched_barrier(0);
    exp_tile(sc, pf);
    pv_regs(vf, pf);
  };
  // Step k = k0 + J of the tight loop (k0 a multiple of TU).
  auto tight_step = [&](auto sp_tag, auto j_tag, int k, STile& sc, STile& sn) __attribute__((always_inline)) {
    sync_tiles(true);
    if constexpr (kConstSlots) {
      constexpr int J = decltype(j_tag)::value;
      tight_body(sp_tag, k, sc, sn, Kst + (J % S) * K_BYTES, Vst + ((J + S - 1) % S) * V_BYTES,
                 Kst + ((J + 1) % S) * K_BYTES, Vst + (J % S) * V_BYTES);
    } else {
      tight_body(sp_tag, k, sc, sn, Kst + (k % S) * K_BYTES, Vst + ((k + S - 1) % S) * V_BYTES,
                 Kst + ((k + 1) % S) * K_BYTES, Vst + (k % S) * V_BYTES);
    }
  };
  auto tight_turn = [&](auto sp_tag, int k0) __attribute__((always_inline)) {
    static_for<TU>([&](auto j_tag) __attribute__((always_inline)) {
      constexpr int J = decltype(j_tag)::value;
      if constexpr (J % 2 == 0) tight_step(sp_tag, j_tag, k0 + J, sa, sb);
      else tight_step(sp_tag, j_tag, k0 + J, sb, sa);
    });
  };
  auto general_body = [&](int k, STile& sc, STile& sn, unsigned char* __restrict__ kdst,
                          unsigned char* __restrict__ vdst, const unsigned char* __restrict__ krd,
                          const unsigned char* __restrict__ vrd) __attribute__((always_inline)) {
    if (k + S < nuse) issue_k(tile_at(k + S), kdst);
    if (k + S - 1 < nuse) issue_v(tile_at(k + S - 1), vdst);
    const int t = tile_at(k);
    if (!dense_full(t)) mask_tile(t, sc);
    softmax_bound(sc);
    if (k + 1 < nuse) qk(krd, sn);
    exp_tile(sc, pf);
    pv(vrd, pf);
  };
  auto general_step = [&](int k, STile& sc, STile& sn) __attribute__((always_inline)) {
    sync_tiles(k + S - 1 < nuse);
    general_body(k, sc, sn, Kst + (k % S) * K_BYTES, Vst + ((k + S - 1) % S) * V_BYTES,
                 Kst + ((k + 1) % S) * K_BYTES, Vst + (k % S) * V_BYTES);
  };
  int k = 0;
  // (two copies of the loop: dense and sparse, each specialised)
  if (!sparse) {
    const std::integral_constant<bool, false> dense_tag;
    if (n_tight > 0) tight_sources(dense_tag, t_lo + S, true);
    for (; k < n_tight; k += TU) tight_turn(dense_tag, k);
  } else {
    const std::integral_constant<bool, true> sparse_tag;
    if (n_tight > 0) tight_sources(sparse_tag, t_lo + S, true);
    for (; k < n_tight; k += TU) tight_turn(sparse_tag, k);
  }
  for (; k < nuse; k += 2) {
    general_step(k, sa, sb);
    if (k + 1 < nuse) general_step(k + 1, sb, sa);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- finish: per-column sums, merge key-sliced waves, write -------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  if constexpr (WK > 1) {
    // The key-slice partners of a query slice pass (m, l, o) through the
    // idle ring in the lanes' own layout, so every access is a conflict-free
    // 16-byte (or 4-byte) one: partner slot sl = (wk - 1) * WQ + wq holds
    // o[qb][db] of lane l at f32x4 index ((sl * QB + qb) * DB + db) * 64 + l
    // and m, l of qb at float index (sl * QB + qb) * 64 + l.  (The partner
    // lane holds the same query column and dims.)
    constexpr int NSL = (WK - 1) * WQ;
    f32x4* xo = reinterpret_cast<f32x4*>(smem);                        // [NSL][QB][DB][64]
    float* xm = reinterpret_cast<float*>(xo + NSL * QB * DB * 64);     // [NSL][QB][64]
    float* xl = xm + NSL * QB * 64;                                    // [NSL][QB][64]
    if (wk > 0) {
      const int sl = (wk - 1) * WQ + wq;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        xm[(sl * QB + qb) * 64 + lane] = m_run[qb];
        xl[(sl * QB + qb) * 64 + lane] = l_run[qb];
#pragma unroll
        for (int db = 0; db < DB; ++db) xo[((sl * QB + qb) * DB + db) * 64 + lane] = o[qb][db];
      }
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int kw = 1; kw < WK; ++kw) {
        const int sl = (kw - 1) * WQ + wq;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float mo = xm[(sl * QB + qb) * 64 + lane], lo = xl[(sl * QB + qb) * 64 + lane];
          const float mn = fmaxf(m_run[qb], mo);
          const float fs = __builtin_amdgcn_exp2f(m_run[qb] - mn);
          const float fo = __builtin_amdgcn_exp2f(mo - mn);
          m_run[qb] = mn;
          l_run[qb] = l_run[qb] * fs + lo * fo;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] = o[qb][db] * fs + xo[((sl * QB + qb) * DB + db) * 64 + lane] * fo;
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
  if (tid == 0) {
    if (!cap_ok && split == 0 && qtile == 0) set_status(a.status, SD_ERR_CAPACITY);
    if (s_err) set_status(a.status, (uint32_t)s_err);
  }
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
// Host-side launchers.  A kernel given a start or stop event is launched with
// hipExtLaunchKernelGGL, which records the events at the kernel's own start
// and end.

template <typename F, typename... Args>
static void launch_ev(F fn, dim3 grid, dim3 block, size_t lds, hipStream_t st, hipEvent_t e0,
                      hipEvent_t e1, Args... args) {
  if (e0 || e1) hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)lds, st, e0, e1, 0u, args...);
  else hipLaunchKernelGGL(fn, grid, block, lds, st, args...);
}

hipError_t launch_anc_mask(const int32_t* parent, int T, int W64, int n_trees, uint64_t* anc,
                           uint32_t* status, hipStream_t st, hipEvent_t start) {
  dim3 grid((T + 255) / 256, n_trees);
  launch_ev(anc_mask_kernel, grid, dim3(256), 0, st, start, nullptr, parent, T, W64, anc, status);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_valu_d(const AttnArgs& a, bool f32, hipStream_t st, CallEvents ev) {
  const long long nrows = (long long)a.B * a.T * a.Hq;
  dim3 grid((unsigned)nrows);
  if (f32)
    launch_ev(attn_valu_kernel<float, D>, grid, dim3(256), 0, st, ev.start, ev.stop, a);
  else
    launch_ev(attn_valu_kernel<bf16_bits, D>, grid, dim3(256), 0, st, ev.start, ev.stop, a);
  return hipGetLastError();
}

hipError_t launch_attn_valu(const AttnArgs& a, bool f32, hipStream_t st, CallEvents ev) {
  return a.D == 64 ? launch_valu_d<64>(a, f32, st, ev) : launch_valu_d<128>(a, f32, st, ev);
}

template <int D, int QW, int WQ, int WK, int KW, int S>
static hipError_t launch_mfma_cfg(const AttnArgs& a, size_t lds, hipStream_t st, CallEvents ev) {
  auto fn = attn_mfma_kernel<D, QW, WQ, WK, KW, S>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned nwg = (unsigned)a.B * a.Hkv * a.n_qtiles * a.n_splits;
  launch_ev(fn, dim3(nwg), dim3(WQ * WK * 64), lds, st, ev.start, ev.stop, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const AttnArgs& a, const AttnPlan& p, hipStream_t st, CallEvents ev) {
  if constexpr (D == 128) {
    if (p.WQ == 8) {
      if (p.stages == 8) return launch_mfma_cfg<D, 32, 8, 1, 32, 8>(a, p.lds_bytes, st, ev);
      return launch_mfma_cfg<D, 32, 8, 1, 32, 4>(a, p.lds_bytes, st, ev);
    }
  }
  if (p.WQ == 1) return launch_mfma_cfg<D, 32, 1, 4, 32, 2>(a, p.lds_bytes, st, ev);
  if (p.WQ == 2) {
    if (p.stages == 4) return launch_mfma_cfg<D, 32, 2, 2, 32, 4>(a, p.lds_bytes, st, ev);
    return launch_mfma_cfg<D, 32, 2, 2, 32, 2>(a, p.lds_bytes, st, ev);
  }
  if (p.stages == 4) return launch_mfma_cfg<D, 32, 4, 2, 32, 4>(a, p.lds_bytes, st, ev);
  if (p.stages == 3) return launch_mfma_cfg<D, 32, 4, 2, 32, 3>(a, p.lds_bytes, st, ev);
  return launch_mfma_cfg<D, 32, 4, 2, 32, 2>(a, p.lds_bytes, st, ev);
}

hipError_t launch_attn_mfma(const AttnArgs& a, const AttnPlan& p, hipStream_t st, CallEvents ev) {
  // with a split context the merge kernel is the call's last
  const CallEvents main_ev{ev.start, a.n_splits == 1 ? ev.stop : nullptr};
  hipError_t e = a.D == 64 ? launch_mfma_d<64>(a, p, st, main_ev) : launch_mfma_d<128>(a, p, st, main_ev);
  if (e != hipSuccess || a.n_splits == 1) return e;
  const long long nrows = (long long)a.B * a.T * a.Hq;
  dim3 grid((unsigned)((nrows + 3) / 4));
  bf16_bits* out = reinterpret_cast<bf16_bits*>(a.out);
  if (a.D == 64)
    launch_ev(attn_combine_kernel<64>, grid, dim3(256), 0, st, nullptr, ev.stop, (const float*)a.part_o,
              (const float*)a.part_ml, out, nrows, a.n_splits);
  else
    launch_ev(attn_combine_kernel<128>, grid, dim3(256), 0, st, nullptr, ev.stop, (const float*)a.part_o,
              (const float*)a.part_ml, out, nrows, a.n_splits);
  return hipGetLastError();
}

}  // namespace sdtree
