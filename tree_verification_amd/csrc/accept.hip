// Acceptance walk over a verified draft tree, for gfx950.
//
// At each visited node the walk reads that node's target logits row (V
// values):
//   greedy      one argmax pass (lowest id on ties);
//   rejection   one statistics pass (max and normaliser), one residual pass
//   sampling    per rejected sibling, then an inverse-CDF draw if every sibling
//               is rejected (standard speculative sampling applied sibling by
//               sibling: SpecExec page, "Builds on");
//   target      one statistics pass, then an inverse-CDF draw from
//   sampling    softmax(l / tau), which stays equivalent to sequential
//               sampling from the target and is therefore safe for
//               deterministic trees (SpecExec page, "Approach").
//
// A sequence is walked by P workgroups of 256 threads; workgroup w owns the
// vocabulary slice [w * SL, (w + 1) * SL), read in chunks of 2048 tokens with
// one 16-byte load per thread per chunk (a bf16 slice stays in registers for
// the whole step).  After each pass the P workgroups exchange a two-value
// partial through barrier-tagged atomic slots in the workspace (bounded spin;
// B * P <= 256 workgroups, one per CU, are all resident); every workgroup then
// reduces the P partials in the same order and takes the same decision.  At
// each node the loads that the walk will need are issued together: the test
// scalars of the children, the draft row and, after the statistics exchange,
// the first child's logits (the likeliest next node).  An inverse-CDF draw
// picks the slice holding the crossing point from the per-slice masses and
// only that workgroup rescans its slice.  Sums are float64; the probability a
// test is taken on is recomputed in float64.  Over register-cached rows, the
// statistics (argmaxes; drawn tokens) of a whole first-child chain (the
// likely path) are formed and exchanged in one round, so a chain node whose
// first child is accepted takes no pass and no exchange.
#include <mutex>
#include <type_traits>

#include "common.h"

namespace sdtree {

constexpr int kAT = 256;              // threads per workgroup
constexpr int kAW = kAT / 64;         // wavefronts per workgroup
constexpr int kChunk = kAT * 8;       // tokens per chunk
constexpr int kMaxCh = 4;             // chunks kept in registers
constexpr int kMaxT = kMaxTreeNodes;
constexpr int kMaxP = 16;             // (the slice butterflies span 16 lanes)
constexpr int kMaxKid = 64;          // children whose test scalars are prefetched
constexpr int kCKRegs = 4;           // commit: 16-byte K (and V) chunks per thread per group
constexpr int kMaxCBlk = kMaxT / 8 + 2;  // commit: blocks of the tree slots (bs >= 8)
constexpr unsigned kSpinLimit = 1u << 20;
constexpr int kSeg = 6;              // nodes of a first-child chain whose statistics are formed together
constexpr int kXW = 2 * kSeg;        // exchanged 32-bit words per workgroup, at most
static_assert(2 * kMaxP * kXW * 8 + 8 <= (int)kAccSeqBytes, "exchange slots exceed a sequence's sync bytes");
static_assert(kMaxP * kXW <= kAT, "one polling thread per exchanged word");

// Workgroup barrier for data exchanged through LDS.  __syncthreads() would
// also wait for every outstanding global load (on this architecture a
// workgroup release waits for vmcnt(0)), serialising the row prefetches into
// the first barrier after them.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Cross-lane moves through DPP (no LDS round trip).  dpp_*<CTRL, ROWS>(old, v)
// returns v of the lane CTRL selects, or `old` in rows outside ROWS.
// Row-local reductions use: swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), mirror within 8 lanes, mirror within 16 lanes -- after
// these a 16-lane row holds its total in every lane, and since each step
// combines a pair of values in either order, every lane holds the same bits.
// Broadcasting lane 15 of each row into the next row (rows 1, 3) and lane 31
// into rows 2, 3 then leaves the wavefront's total in lane 63.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double old, double v) {
  const long long o = __double_as_longlong(old), x = __double_as_longlong(v);
  const int lo = dpp_i<CTRL, ROWS>((int)o, (int)x);
  const int hi = dpp_i<CTRL, ROWS>((int)(o >> 32), (int)(x >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
// Reduce a value of type X over each 16-lane row with comb(a, b) (commutative);
// with WAVE, go on to leave the wavefront's total in lane 63 (`id` is the
// identity of comb, taken by lanes outside the broadcast rows).
template <bool WAVE, typename X, typename Mv, typename Comb>
__device__ __forceinline__ X dpp_reduce(X v, X id, Mv mv, Comb comb) {
  v = comb(v, mv(std::integral_constant<int, kDppXor1>(), std::integral_constant<int, 0xF>(), id, v));
  v = comb(v, mv(std::integral_constant<int, kDppXor2>(), std::integral_constant<int, 0xF>(), id, v));
  v = comb(v, mv(std::integral_constant<int, kDppHalfMirror>(), std::integral_constant<int, 0xF>(), id, v));
  v = comb(v, mv(std::integral_constant<int, kDppMirror>(), std::integral_constant<int, 0xF>(), id, v));
  if constexpr (WAVE) {
    v = comb(v, mv(std::integral_constant<int, kDppBcast15>(), std::integral_constant<int, 0xA>(), id, v));
    v = comb(v, mv(std::integral_constant<int, kDppBcast31>(), std::integral_constant<int, 0xC>(), id, v));
  }
  return v;
}

// float64 sum over the wavefront, in lane 63
__device__ __forceinline__ double wave_sum_d(double v) {
  auto mv = [](auto c, auto r, double old, double x) { return dpp_d<decltype(c)::value, decltype(r)::value>(old, x); };
  return dpp_reduce<true>(v, 0.0, mv, [](double x, double y) { return x + y; });
  return v;
}

__device__ __forceinline__ void store_d(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), (unsigned long long)__double_as_longlong(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_d(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<double*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT));
}

// 8 consecutive values starting at y0 (a multiple of 8); `pad` past V.
template <typename E>
__device__ __forceinline__ void load8(const E* row, int y0, int V, bool vec, float pad, float* out) {
  if constexpr (sizeof(E) == 2) {
    if (vec && y0 + 8 <= V) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + y0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
      return;
    }
  } else {
    if (vec && y0 + 8 <= V) {
      const float4 u = *reinterpret_cast<const float4*>(row + y0);
      const float4 v = *reinterpret_cast<const float4*>(row + y0 + 4);
      out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
      out[4] = v.x; out[5] = v.y; out[6] = v.z; out[7] = v.w;
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = y0 + e < V ? Elem<E>::load(row, y0 + e) : pad;
}

// Loop over this workgroup's chunks; with CACHED the loop is unrolled so the
// register cache is indexed statically.
#define FOR_CHUNKS(c, ...)                                 \
  if constexpr (CACHED) {                                  \
    _Pragma("unroll") for (int c = 0; c < kMaxCh; ++c) {   \
      if (c < NC) { __VA_ARGS__ }                          \
    }                                                      \
  } else {                                                 \
    for (int c = 0; c < NC; ++c) { __VA_ARGS__ }           \
  }

enum AcceptMode { kGreedy = 0, kRejection = 1, kTarget = 2 };

// One kernel per (logit type, register cache, rule), so each holds only the
// code of its rule.
template <typename LT, bool CACHED, int MODE>
__global__ void __launch_bounds__(kAT) accept_kernel(AcceptArgs a) {
  constexpr bool kBF = sizeof(LT) == 2;
  static_assert(!CACHED || kBF, "only bf16 rows are cached");
  __shared__ int s_par[kMaxT];
  __shared__ int s_tok[kMaxT];
  __shared__ int kids[kMaxT];
  __shared__ float kid_l[kMaxKid], kid_q[kMaxKid], kid_u[kMaxKid];
  __shared__ int wcnt[kAW];
  __shared__ double red_d[kAW];
  __shared__ double red4[kAW][4];
  __shared__ float red_f[kAW];
  __shared__ int red_i[kAW];
  __shared__ double mass[kMaxP];    // per-slice mass of the distribution to draw from
  // reciprocals of the residual normalisers of the siblings rejected so far
  // at the current node (0 where the mass was 0); a node has fewer than T
  // children, so the history never overflows
  __shared__ double zinv[MODE == kRejection ? kMaxT : 1];
  __shared__ __align__(8) uint32_t xv[kMaxP][2];
  // First-child chains (cached rows, every rule): the first child of every
  // node, the chain's nodes, each node's first-child test scalars (rejection
  // sampling) and draw uniform, and the P workgroups' statistics (argmax,
  // or drawn token) of every chain node.
  constexpr bool kSegOn = CACHED;
  __shared__ int fk[kSegOn ? kMaxT : 1];
  __shared__ int s_seg[kSeg];
  __shared__ int s_seglen;
  __shared__ float seg_l[kSeg], seg_q[kSeg], seg_u[kSeg], seg_ud[kSeg];
  __shared__ float sred_f[kSegOn ? kSeg : 1][kAW];
  __shared__ double sred_d[kSegOn ? kSeg : 1][kAW];
  __shared__ int sred_i[kSegOn ? kSeg : 1][kAW];
  __shared__ int seg_x[kSeg];
  __shared__ __align__(8) uint32_t xs[kMaxP][kSegOn ? kXW : 2];
  __shared__ int s_flag, s_to, s_first, s_last, s_x;

  const int P = a.P;
  // Workgroups are dispatched round-robin over the 8 XCDs; when the grid
  // allows, the P workgroups of a sequence are placed on one XCD so their
  // exchanges meet in one L2.
  int L = blockIdx.x;
  {
    const int G = gridDim.x, n = G >> 3;
    if ((G & 7) == 0 && n % P == 0) L = (L & 7) * n + (L >> 3);
  }
  const int b = L / P, wg = L % P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;
  const int bt = a.tree_stride ? b : 0;
  int32_t* path = a.path + (size_t)b * T;
  // Exchange slots of this sequence: [2 parities][P workgroups][kXW values],
  // each a 64-bit word (barrier number << 32 | 32-bit value), then the exit
  // counter.
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(a.sync + (size_t)b * kAccSeqBytes);
  unsigned* done = reinterpret_cast<unsigned*>(slots + 2 * kMaxP * kXW);

  const int sl0 = min(wg * a.SL, V), sl1 = min(sl0 + a.SL, V);
  const int NC = a.NC;
  // the P slices cover the vocabulary and each slice its chunks; a
  // register-cached slice has at most kMaxCh chunks
  SD_DCHECK(P >= 1 && P <= kMaxP && (long long)P * a.SL >= V && NC * kChunk >= a.SL, a.status);
  SD_DCHECK(!CACHED || NC <= kMaxCh, a.status);
  const bool vec = (V & 7) == 0;
  constexpr bool mss = MODE == kRejection;
  const float c2 = a.tau > 0.f ? 1.4426950408889634f / a.tau : 0.f;
  const double invtau_d = a.tau > 0.f ? 1.0 / (double)a.tau : 0.0;
  auto y0_of = [&](int c) { return sl0 + c * kChunk + tid * 8; };
  auto row_of = [&](int node) {
    return reinterpret_cast<const LT*>(a.logits) + ((size_t)b * T + node) * V;
  };

  // Row caches (CACHED): the current node's logits, the first child's logits
  // (prefetched in case it is accepted) and, for rejection sampling, the
  // current node's draft probabilities.
  uint4 lc[kMaxCh], pfc[kMaxCh];
  float qc[kMaxCh][8];
  const LT* row = row_of(0);
  const float* qrow = nullptr;
  // CACHED kernels run only when V % 8 == 0, so a chunk starting inside the
  // slice is whole.  Every cached chunk is loaded unconditionally (a chunk
  // outside the slice reads the row's first 8 values, which are never used):
  // a branch around the load would make its merge wait for the data at once.
  auto cached_y = [&](int c) {
    const int y0 = y0_of(c);
    return (c < NC && y0 < sl1) ? y0 : 0;
  };
  auto load_row = [&](const LT* r, uint4* dst) {
    if constexpr (CACHED) {
#pragma unroll
      for (int c = 0; c < kMaxCh; ++c) dst[c] = *reinterpret_cast<const uint4*>(r + cached_y(c));
    }
  };
  // With a commit: the context length, and the block ids of the tree slots
  // [ctx, ctx + T) staged and validated now, alongside the tree (the commit
  // runs after the walk; see below).
  const bool commit = a.cctx != nullptr;
  const int c_ctx = commit ? a.cctx[b] : 0;
  __shared__ int s_cblk[kMaxCBlk];
  __shared__ int s_cerr;
  uint32_t cbad = 0;
  // This thread's first tree entry and first tree-slot block id are loaded
  // before the root's row, so that waiting for them does not wait for the row
  // (vector loads complete in order); the walk starts at the root, whose row
  // is known before the tree is read, and its latency overlaps the set-up.
  const int32_t* tpar = a.parent + (size_t)bt * T;
  const int32_t* ttok = a.token + (size_t)bt * T;
  const int p_first = tid < T ? tpar[tid] : 0;
  const int t_first = tid < T ? ttok[tid] : 0;
  const bool c_ok = commit && c_ctx >= 0 && (long long)c_ctx + T <= (long long)a.cmax_blocks * a.cbs;
  const int c_lo = c_ok ? c_ctx / a.cbs : 0;
  const int c_nblk = c_ok ? (c_ctx + T - 1) / a.cbs - c_lo + 1 : 0;
  SD_DCHECK(c_nblk <= kMaxCBlk, a.status);
  const int32_t* ctable = commit ? a.ctable + (size_t)b * a.cmax_blocks + c_lo : nullptr;
  const int blk_first = tid < c_nblk ? ctable[tid] : 0;
  load_row(row_of(0), lc);
  if (commit && !c_ok) cbad = SD_ERR_CAPACITY;
  for (int n = tid; n < c_nblk; n += kAT) {
    const int blk = n == tid ? blk_first : ctable[n];
    if (blk < 0 || blk >= a.cnum_blocks) cbad |= SD_ERR_BLOCK;
    s_cblk[n] = blk;
  }
  // The tree (kept in LDS) must be topologically ordered with valid tokens.
  int bad = 0;
  auto check_node = [&](int n, int p, int t) {
    if (n == 0 ? p != -1 : (p < 0 || p >= n)) bad |= SD_ERR_PARENT;
    if (t < 0 || t >= V) bad |= SD_ERR_TOKEN;
    s_par[n] = p;
    s_tok[n] = t;
  };
  if (tid < T) check_node(tid, p_first, t_first);
  // the rest of a larger tree, four nodes per thread with their loads in
  // flight together (a plain loop would wait for each node's loads in turn)
  for (int n0 = kAT; n0 < T; n0 += 4 * kAT) {
    int pv[4], tv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + u * kAT + tid;
      pv[u] = n < T ? tpar[n] : 0;
      tv[u] = n < T ? ttok[n] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + u * kAT + tid;
      if (n < T) check_node(n, pv[u], tv[u]);
    }
  }
  if (tid == 0) {
    s_flag = 0;
    s_to = 0;
    s_cerr = 0;
  }
  lds_sync();
  if (bad) atomicOr(&s_flag, bad);
  if (cbad) atomicOr(&s_cerr, (int)cbad);
  lds_sync();
  const uint32_t cerr = (uint32_t)s_cerr;
  if (wg == 0)
    for (int n = tid; n < T; n += kAT) path[n] = -1;
  // ---- commit of the accepted path (when asked for) --------------------------
  // As a commit after the walk: positions ctx + j take the K/V of ctx + path[j]
  // for j < plen, every KV head, then ctx grows by plen.  Validation as the
  // commit (done above): the slots [ctx, ctx + T) must fit the table and their
  // blocks be valid, else the sequence is left untouched and a sticky bit is
  // set.
  // Copies the path's entries of this workgroup's KV heads (g = wg, wg + P,
  // ...) in groups: every thread loads its share of a group (16-byte chunks of
  // the K and V rows), the workgroup waits for all of them, then stores.  Since
  // path[j] >= j and the path increases, a group's destinations never overlap
  // a later group's sources, so the copy is safe in place.  kids[] holds the
  // path and s_cblk[] the block ids of slots [ctx, ctx + T).
  auto commit_copy = [&](int L) {
    const int D = a.cD, esize = a.cesize, bs = a.cbs, lo = c_ctx / bs;
    const int rowb = D * esize;
    const int kch = rowb / 16;                      // 16-byte chunks per row
    const int kstep = kAT / kch;
    const int kcol = tid % kch, ku0 = tid / kch;
    const int JG = kCKRegs * kstep;
    const long long blk_bytes = (long long)a.cHkv * bs * rowb;
    unsigned char* K = static_cast<unsigned char*>(a.ck);
    unsigned char* Vb = static_cast<unsigned char*>(a.cv);
    const long long c_off = (long long)kcol * 16;
    for (int g = wg; g < a.cHkv; g += P) {
      const long long head = (long long)g * bs * rowb;
      auto row_at = [&](int pos) {
        return (long long)s_cblk[pos / bs - lo] * blk_bytes + head + (long long)(pos % bs) * rowb;
      };
      for (int j0 = 0; j0 < L; j0 += JG) {
        const int nj = min(JG, L - j0);
        uint4 kr[kCKRegs], vr[kCKRegs];
#pragma unroll
        for (int r = 0; r < kCKRegs; ++r) {
          const int jj = ku0 + r * kstep;
          kr[r] = make_uint4(0, 0, 0, 0);
          vr[r] = make_uint4(0, 0, 0, 0);
          if (jj < nj && kids[j0 + jj] != j0 + jj) {
            const long long src = row_at(c_ctx + kids[j0 + jj]) + c_off;
            kr[r] = *reinterpret_cast<const uint4*>(K + src);
            vr[r] = *reinterpret_cast<const uint4*>(Vb + src);
          }
        }
        __syncthreads();   // every load of the group has landed before any store
#pragma unroll
        for (int r = 0; r < kCKRegs; ++r) {
          const int jj = ku0 + r * kstep;
          if (jj < nj && kids[j0 + jj] != j0 + jj) {
            const long long dst = row_at(c_ctx + j0 + jj) + c_off;
            *reinterpret_cast<uint4*>(K + dst) = kr[r];
            *reinterpret_cast<uint4*>(Vb + dst) = vr[r];
          }
        }
        __syncthreads();
      }
      // kept block key sums: this head's, extended over the committed
      // positions [ctx, ctx + L) (the rows written above are visible to the
      // workgroup after the last barrier)
      if (a.csums && wave == 0)
        extend_head_sums_rt(
            esize, D, bs, c_ctx, c_ctx + L, lane,
            [&](int n) { return K + (long long)s_cblk[n - lo] * blk_bytes + head; },
            [&](int n) { return a.csums + ((size_t)s_cblk[n - lo] * a.cHkv + g) * D; });
    }
  };
  if (s_flag) {
    if (wg == 0 && tid == 0) {
      set_status(a.status, (uint32_t)s_flag | cerr);
      a.path_len[b] = 0;
      a.bonus[b] = -1;
    }
    return;
  }
  if constexpr (kSegOn) {
    // the first (lowest-index) child of every node; T where there is none
    for (int n = tid; n < T; n += kAT) fk[n] = T;
    lds_sync();
    // (fk only decreases, so a node that reads a smaller value already is not
    // its parent's first child and skips the atomic: a node with many
    // children, such as the root of a best-first tree, then takes one
    // contended atomic per child of the first 256 nodes only)
    for (int n = 1 + tid; n < T; n += kAT) {
      const int p = s_par[n];
      if (fk[p] > n) atomicMin(&fk[p], n);
    }
    lds_sync();
  }

  // ---- cross-workgroup exchange ---------------------------------------------
  // exchange(v0, v1): every workgroup of the sequence publishes two 32-bit
  // values tagged with the barrier number; lanes j < P of wave 0 poll slot j
  // until it carries this barrier's number (bounded), and the P pairs land in
  // xv[] for the whole workgroup.  Slots alternate between two parities, so a
  // workgroup can never overwrite a value another one has not read yet.  No
  // fences are needed: each value travels in a single atomic word.
  int nbar = 0;
  auto exchange = [&](uint32_t v0, uint32_t v1) {
    lds_sync();
    ++nbar;
    if (P == 1) {
      if (tid == 0) {
        xv[0][0] = v0;
        xv[0][1] = v1;
      }
    } else {
      unsigned long long* sl = slots + (size_t)(nbar & 1) * kMaxP * kXW;
      const unsigned long long tag = (unsigned long long)(unsigned)nbar << 32;
      if (tid == 0) {
        __hip_atomic_store(sl + wg * kXW + 0, tag | v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sl + wg * kXW + 1, tag | v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (tid < P) {
        unsigned long long w0, w1;
        unsigned spins = 0;
        for (;;) {
          w0 = __hip_atomic_load(sl + tid * kXW + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          w1 = __hip_atomic_load(sl + tid * kXW + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((w0 >> 32) == (unsigned)nbar && (w1 >> 32) == (unsigned)nbar) break;
          if (++spins > kSpinLimit) {
            s_to = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        xv[tid][0] = (uint32_t)w0;
        xv[tid][1] = (uint32_t)w1;
      }
    }
    lds_sync();
  };
  // exchange_words(nw, w): as exchange, with nw <= kXW words per workgroup
  // (thread t < nw publishes word t, w); thread j * nw + k polls word k of
  // workgroup j, and the P * nw words land in xs[j][k].
  auto exchange_words = [&](int nw, uint32_t w) {
    lds_sync();
    ++nbar;
    if (P == 1) {
      if (tid < nw) xs[0][tid] = w;
    } else {
      unsigned long long* sl = slots + (size_t)(nbar & 1) * kMaxP * kXW;
      const unsigned long long tag = (unsigned long long)(unsigned)nbar << 32;
      if (tid < nw) __hip_atomic_store(sl + wg * kXW + tid, tag | w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid < P * nw) {
        const int j = tid / nw, k = tid - j * nw;
        unsigned long long x;
        unsigned spins = 0;
        for (;;) {
          x = __hip_atomic_load(sl + j * kXW + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((x >> 32) == (unsigned)nbar) break;
          if (++spins > kSpinLimit) {
            s_to = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        xs[j][k] = (uint32_t)x;
      }
    }
    lds_sync();
  };
  auto xf = [&](int j, int k) { return __uint_as_float(xv[j][k]); };
  // All P exchanged pairs read into registers together (one LDS wait rather
  // than one per slot); slots j >= P read as (fill0, fill1).
  auto read_pairs = [&](uint32_t* x0, uint32_t* x1, uint32_t fill0, uint32_t fill1) {
#pragma unroll
    for (int j = 0; j < kMaxP; ++j) {
      const uint2 w = *reinterpret_cast<const uint2*>(&xv[j][0]);
      x0[j] = j < P ? w.x : fill0;
      x1[j] = j < P ? w.y : fill1;
    }
  };

  // ---- workgroup reduction of a float64 sum -------------------------------------
  auto wg_sum = [&](double v) -> double {
    v = wave_sum_d(v);
    lds_sync();
    if (lane == 63) red_d[wave] = v;
    lds_sync();
    double t = 0.0;
    for (int w = 0; w < kAW; ++w) t += red_d[w];
    return t;
  };

  // children of `cur` in ascending index order -> kids[0..return)
  auto gather_children = [&](int cur) -> int {
    int nk = 0;
    for (int base = 0; base < T; base += kAT) {
      const int n = base + tid;
      const bool f = n < T && s_par[n] == cur;
      const unsigned long long bal = __ballot(f);
      if (lane == 0) wcnt[wave] = __popcll(bal);
      lds_sync();
      int off = nk;
      for (int w = 0; w < wave; ++w) off += wcnt[w];
      if (f) kids[off + __popcll(bal & ((1ull << lane) - 1ull))] = n;
      int tot = 0;
      for (int w = 0; w < kAW; ++w) tot += wcnt[w];
      lds_sync();
      nk += tot;
    }
    return nk;
  };

  auto logits8 = [&](int c, float* v) {
    const int y0 = y0_of(c);
    if (y0 >= sl1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = -INFINITY;
      return;
    }
    if constexpr (CACHED) {
      // (the empty asm keeps each conversion where it is written: the
      // compiler would otherwise hoist the residual passes' conversions out
      // of the test loop, in front of the first test)
      // (V % 8 == 0 here, so a chunk starting inside the slice is whole)
      uint4 u = lc[c];
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
    } else {
      load8<LT>(row, y0, V, vec, -INFINITY, v);
    }
  };
  auto q8_of = [&](int c, float* q8) {
    if constexpr (CACHED) {
      // (the empty asm keeps each use where it is written: hoisted out of
      // the test loop, the use would wait for the draft row before the first
      // test)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float q = qc[c][e];
        asm volatile("" : "+v"(q));
        q8[e] = q;
      }
    } else {
      const int y0 = y0_of(c);
      if (y0 < sl1) {
        load8<float>(qrow, y0, V, vec, 0.f, q8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) q8[e] = 0.f;
      }
    }
  };

  // Statistics of this thread's part of a cached row `rw` (its kMaxCh
  // chunks): the wavefront's max first (a float reduction), then every weight
  // relative to it at once, so no step of the sum waits on a rescale.  The
  // wavefront's (max, mass) are left in lane 63.
  auto row_stats = [&](const uint4* rw, float& mt, double& st) {
    float v[kMaxCh][8];
    float cm[kMaxCh];
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c) {
      if (c < NC && y0_of(c) < sl1) {
        uint4 u = rw[c];
        asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] = -INFINITY;
      }
      cm[c] = fmaxf(fmaxf(fmaxf(v[c][0], v[c][1]), fmaxf(v[c][2], v[c][3])),
                    fmaxf(fmaxf(v[c][4], v[c][5]), fmaxf(v[c][6], v[c][7])));
    }
    float lm = cm[0];
#pragma unroll
    for (int c = 1; c < kMaxCh; ++c) lm = fmaxf(lm, cm[c]);
    auto mvf = [](auto c, auto r, float old, float x) { return dpp_f<decltype(c)::value, decltype(r)::value>(old, x); };
    lm = dpp_reduce<true>(lm, -INFINITY, mvf, [](float x, float y) { return fmaxf(x, y); });
    mt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm), 63));   // (the reduction ends in lane 63)
    double ls = 0.0;
    if (mt > -INFINITY) {
      double cs[kMaxCh];
#pragma unroll
      for (int c = 0; c < kMaxCh; ++c) {
        double w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (double)__builtin_amdgcn_exp2f((v[c][e] - mt) * c2);
        cs[c] = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
      }
      ls = cs[0];
#pragma unroll
      for (int c = 1; c < kMaxCh; ++c) ls += cs[c];
    }
    st = wave_sum_d(ls);
  };
  // Argmax (lowest id among equal maxima) of this thread's part of a cached
  // row, reduced over the wavefront into lane 63.
  auto row_argmax = [&](const uint4* rw, float& bv, int& bi) {
    bv = -INFINITY;
    bi = V;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c) {
      const int y0 = y0_of(c);
      if (c < NC && y0 < sl1) {
        const uint4 u = rw[c];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1))));
          if (v > bv) {
            bv = v;
            bi = y0 + e;
          }
        }
      }
    }
    struct VI { float v; int i; };
    auto mv = [&](auto c, auto r, VI old, VI x) {
      return VI{dpp_f<decltype(c)::value, decltype(r)::value>(old.v, x.v),
                dpp_i<decltype(c)::value, decltype(r)::value>(old.i, x.i)};
    };
    auto comb = [](VI x, VI y) { return (y.v > x.v || (y.v == x.v && y.i < x.i)) ? y : x; };
    const VI t = dpp_reduce<true>(VI{bv, bi}, VI{-INFINITY, V}, mv, comb);
    bv = t.v;
    bi = t.i;
  };
  // The workgroup's (max, mass) from its wavefronts' (in wf[], wd[]), as a
  // two-value exchange carries it.
  auto wg_stats = [&](const float* wf, const double* wd, float& mw, double& sw) {
    mw = wf[0];
    for (int w = 1; w < kAW; ++w) mw = fmaxf(mw, wf[w]);
    sw = 0.0;
    if (mw > -INFINITY)
      for (int w = 0; w < kAW; ++w)
        if (wf[w] > -INFINITY) sw += wd[w] * (double)__builtin_amdgcn_exp2f((wf[w] - mw) * c2);
  };
  // Inverse-CDF draw: slices' masses in mass[0..P); threshold u * total.  The
  // workgroup owning the crossing finds it in its slice, four chunks at a
  // time: each thread sums its 8 weights `wf(c, w8)` of each chunk, a scan over
  // (chunk, thread) positions gives each thread the mass before its
  // elements, the first thread whose range passes the threshold scans its 8
  // weights.  Other workgroups return -1.
  auto draw = [&](float u, auto wf) -> int {
    lds_sync();
    double tot = 0.0;
    for (int j = 0; j < P; ++j) tot += mass[j];
    const double thr = (double)u * tot;
    int pick = -1, last_pos = -1;
    double run = 0.0, before = 0.0;
    for (int j = 0; j < P; ++j) {
      if (mass[j] > 0.0) last_pos = j;
      if (pick < 0 && run + mass[j] > thr) {
        pick = j;
        before = run;
      }
      run += mass[j];
    }
    if (pick < 0) {
      pick = last_pos;
      before = 0.0;
      for (int j = 0; j < pick; ++j) before += mass[j];
    }
    if (wg != pick) return -1;
    if (tid == 0) s_last = -1;
    // weights of chunk c; with CACHED the chunk index must be a constant for
    // the register cache, so c is matched against the unrolled candidates
    auto wfc = [&](int c, double* w8) {
      if constexpr (CACHED) {
#pragma unroll
        for (int j = 0; j < kMaxCh; ++j)
          if (j == c) wf(j, w8);
      } else {
        wf(c, w8);
      }
    };
    double rn = before;
    // CACHED slices have at most four chunks: one group
    for (int c0 = 0; c0 < (CACHED ? 1 : NC); c0 += 4) {
      double t[4], inc[4];
      int lp_pos = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t[j] = 0.0;
        if (c0 + j < NC) {
          double w8[8];
          if constexpr (CACHED) wf(j, w8);
          else wf(c0 + j, w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            t[j] += w8[e];
            if (w8[e] > 0.0) lp_pos = y0_of(c0 + j) + e;
          }
        }
        inc[j] = t[j];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double o = __shfl_up(inc[j], off);
          if (lane >= off) inc[j] += o;
        }
      if (lane == 63)
#pragma unroll
        for (int j = 0; j < 4; ++j) red4[wave][j] = inc[j];
      if (tid == 0) s_first = 1 << 30;
      for (int off = 32; off >= 1; off >>= 1) lp_pos = max(lp_pos, __shfl_xor(lp_pos, off));
      if (lane == 0 && lp_pos >= 0) atomicMax(&s_last, lp_pos);
      lds_sync();
      double gtot = 0.0, cum = rn;
      int key = 1 << 30;
      double excl_hit = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double woff = 0.0, ctot = 0.0;
        for (int w = 0; w < kAW; ++w) {
          if (w < wave) woff += red4[w][j];
          ctot += red4[w][j];
        }
        const double excl = cum + woff + inc[j] - t[j];
        if (key == (1 << 30) && t[j] > 0.0 && excl + t[j] > thr) {
          key = j * kAT + tid;
          excl_hit = excl;
        }
        cum += ctot;
        gtot += ctot;
      }
      int kmin = key;
      for (int off = 32; off >= 1; off >>= 1) kmin = min(kmin, __shfl_xor(kmin, off));
      if (lane == 0 && kmin < (1 << 30)) atomicMin(&s_first, kmin);
      lds_sync();
      const int first = s_first;
      if (first < (1 << 30)) {
        if (key == first) {
          const int c = c0 + first / kAT;
          double w8[8];
          wfc(c, w8);
          double r2 = excl_hit;
          int pk = -1, lp = -1;
          for (int e = 0; e < 8; ++e) {
            if (w8[e] > 0.0) lp = e;
            r2 += w8[e];
            if (pk < 0 && w8[e] > 0.0 && r2 > thr) pk = e;
          }
          s_x = y0_of(c) + (pk >= 0 ? pk : lp);
        }
        lds_sync();
        return s_x;
      }
      rn += gtot;
    }
    lds_sync();
    return s_last;
  };

  // Slice j's (max, mass) sits in lane j % 16 of every wavefront (mj, sj);
  // the global max m and the masses' sum z0 are formed by butterflies over
  // those 16 lanes, which leave the same value in every lane (each step adds
  // a pair of values in either order).  mass_j: this lane's slice's mass
  // relative to m.
  auto slice_bfly = [&](float mj, float sj, float& m, double& z0, double& mass_j) {
    auto mvf = [](auto c, auto r, float old, float x) { return dpp_f<decltype(c)::value, decltype(r)::value>(old, x); };
    auto mvd = [](auto c, auto r, double old, double x) { return dpp_d<decltype(c)::value, decltype(r)::value>(old, x); };
    m = dpp_reduce<false>(mj, -INFINITY, mvf, [](float x, float y) { return fmaxf(x, y); });
    mass_j = mj == -INFINITY ? 0.0 : (double)sj * (double)__builtin_amdgcn_exp2f((mj - m) * c2);
    z0 = dpp_reduce<false>(mass_j, 0.0, mvd, [](double x, double y) { return x + y; });
  };
  // Statistics of a first-child chain (cached rows).  In the seeded trees
  // the walk accepts a node's first child nine times in ten, so the chain
  // from `start` (up to kSeg nodes: start, its first child, that child's
  // first child, ...) is likely the path ahead.  Its rows are loaded
  // together, every node's (max, mass) -- or argmax -- formed as the
  // per-node pass would form it, and all of them exchanged at once; so is
  // each node's first-child test scalars and draw uniform.  With target
  // sampling every chain node's draw is then made from its row (the draw
  // depends only on the node) and the drawn tokens exchanged in a second
  // round.  A node of the chain needs no pass and no exchange of its own.
  auto seg_build = [&](int start, bool start_row) {   // start_row: lc holds start's row
    if (tid == 0) {
      int n = start, len = 0;
      for (;;) {
        s_seg[len++] = n;
        if (len == kSeg) break;
        const int f = fk[n];
        if (f >= T) break;
        n = f;
      }
      s_seglen = len;
    }
    lds_sync();
    const int len = s_seglen;
    LT gl = LT(0);
    float gq = 0.f, gu = 0.f, gud = 0.f;
    if (tid < len) {
      const int n = s_seg[tid];
      if constexpr (mss) {
        const int f = fk[n];
        const int fn = f < T ? f : n;   // (a leaf reads its own values, unused)
        const int x = s_tok[fn];
        gl = row_of(n)[x];
        gq = a.draft[((size_t)b * T + n) * V + x];
        gu = a.unif[((size_t)b * T + fn) * 2 + 0];
      }
      if constexpr (MODE != kGreedy) gud = a.unif[((size_t)b * T + n) * 2 + 1];
    }
    uint4 sr[kSeg][kMaxCh];
#pragma unroll
    for (int j = 0; j < kSeg; ++j)
      if (j < len) {
        if (j == 0 && start_row) {
#pragma unroll
          for (int c = 0; c < kMaxCh; ++c) sr[0][c] = lc[c];
        } else {
          load_row(row_of(s_seg[j]), sr[j]);
        }
      }
#pragma unroll
    for (int j = 0; j < kSeg; ++j)
      if (j < len) {
        if constexpr (MODE == kGreedy) {
          float bv;
          int bi;
          row_argmax(sr[j], bv, bi);
          if (lane == 63) {
            sred_f[j][wave] = bv;
            sred_i[j][wave] = bi;
          }
        } else {
          float mt;
          double st;
          row_stats(sr[j], mt, st);
          if (lane == 63) {
            sred_f[j][wave] = mt;
            sred_d[j][wave] = st;
          }
        }
      }
    if (tid < len) {
      if constexpr (mss) {
        seg_l[tid] = bf16_to_f32(gl);
        seg_q[tid] = gq;
        seg_u[tid] = gu;
      }
      if constexpr (MODE != kGreedy) seg_ud[tid] = gud;
    }
    lds_sync();
    uint32_t w = 0;
    if (tid < 2 * len) {
      const int j = tid >> 1;
      if constexpr (MODE == kGreedy) {
        // the workgroup's argmax, combined over its wavefronts in order
        float bv = sred_f[j][0];
        int bi = sred_i[j][0];
        for (int w2 = 1; w2 < kAW; ++w2)
          if (sred_f[j][w2] > bv || (sred_f[j][w2] == bv && sred_i[j][w2] < bi)) {
            bv = sred_f[j][w2];
            bi = sred_i[j][w2];
          }
        w = (tid & 1) ? (uint32_t)bi : __float_as_uint(bv);
      } else {
        float mw;
        double sw;
        wg_stats(sred_f[j], sred_d[j], mw, sw);
        w = (tid & 1) ? __float_as_uint((float)sw) : __float_as_uint(mw);
      }
    }
    exchange_words(2 * len, w);
    if constexpr (MODE == kTarget) {
      // each chain node's draw, as the per-node step would make it; only the
      // workgroup holding the crossing point gets the token
#pragma unroll
      for (int j = 0; j < kSeg; ++j)
        if (j < len) {
          float m;
          double z0, mass_j;
          {
            const int jj = lane & 15;
            const float mj = jj < P ? __uint_as_float(xs[jj][2 * j + 0]) : -INFINITY;
            const float sj = jj < P ? __uint_as_float(xs[jj][2 * j + 1]) : 0.f;
            slice_bfly(mj, sj, m, z0, mass_j);
          }
          // (a workgroup not holding the last crossing returns from the draw
          // right after reading mass[]: every wavefront is past those reads
          // before mass[] changes)
          lds_sync();
          if (tid < P) mass[tid] = mass_j;
          auto ewj = [&](int c, double* w8) {
            if (y0_of(c) >= sl1) {
#pragma unroll
              for (int e = 0; e < 8; ++e) w8[e] = 0.0;
              return;
            }
            const uint4 u = sr[j][c];
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = bf16_to_f32((bf16_bits)(wd[e >> 1] >> (16 * (e & 1))));
              w8[e] = v == -INFINITY ? 0.0 : (double)__builtin_amdgcn_exp2f((v - m) * c2);
            }
          };
          const int x = draw(seg_ud[j], ewj);
          if (tid == 0) seg_x[j] = x;
        }
      lds_sync();
      exchange_words(len, tid < len ? (uint32_t)(seg_x[tid] + 1) : 0u);   // xs[j][k]: token + 1 of chain node k from slice j, or 0
    }
  };

  int cur = 0, plen = 1;
  bool have_row = true;    // lc already holds the current node's row (the root's since the start)
  int seg_len = 0, seg_i = 0;   // the current chain's length and cur's place in it
  int lc_node = 0;              // (chains) the node whose row lc holds
  if (wg == 0 && tid == 0) path[0] = 0;
  for (int step = 0; step < T; ++step) {
    if constexpr (kSegOn) {
      if (seg_i >= seg_len) {
        seg_build(cur, lc_node == cur);
        seg_len = s_seglen;
        seg_i = 0;
      }
    }
    // (a chain node lists its children only once its first child is rejected)
    int nk;
    if constexpr (kSegOn) nk = fk[cur] < T ? 1 : 0;
    else nk = gather_children(cur);
    row = row_of(cur);
    // Issue this node's loads together: the scalars of the child tests, the
    // row (unless prefetched), the draft row, and the first child's row.
    // (the logit is kept as loaded and converted only when it is stored, so
    // nothing waits for these loads before the statistics pass)
    // (every thread loads, lanes past the children reading node 0's values:
    // a branch around the loads would make its merge wait for them)
    LT kl_raw = LT(0);
    float kq = 0.f, ku = 0.f;
    const bool kid_lane = mss && !kSegOn && tid < min(nk, kMaxKid);
    if constexpr (mss && !kSegOn) {
      const int kid = kids[tid < kMaxKid ? tid : 0];
      const int node = kid_lane ? kid : 0;
      const int x = s_tok[node];
      kl_raw = row[x];
      kq = a.draft[((size_t)b * T + cur) * V + x];
      ku = a.unif[((size_t)b * T + node) * 2 + 0];
    }
    // (a chain node's row is loaded only when a rejection or a draw needs it)
    if constexpr (!kSegOn) {
      if (!have_row) load_row(row, lc);
    }
    // the uniform of this node's draw, loaded with the rest so that the draw
    // does not wait for it
    float u_draw;
    if constexpr (kSegOn && mss) u_draw = seg_ud[seg_i];
    else u_draw = a.unif[((size_t)b * T + cur) * 2 + 1];
    auto need_row = [&]() {
      if constexpr (kSegOn) {
        if (lc_node != cur) {
          load_row(row, lc);
          lc_node = cur;
        }
      }
    };
    if constexpr (mss) qrow = a.draft + ((size_t)b * T + cur) * V;
    // (greedy prefetches the first child's row now; the other rules after
    // the statistics exchange, whose polling loads would otherwise wait for
    // it: vector loads return in order)
    if constexpr (MODE == kGreedy && !kSegOn) {
      if (nk > 0) load_row(row_of(kids[0]), pfc);
    }
    int nxt = -1;
    bool stop = false;
    if constexpr (MODE == kGreedy) {
      // argmax, lowest id among equal maxima (a chain node has its slices'
      // argmaxes from its chain's exchange)
      float gv = -INFINITY;
      int gi = V;
      if constexpr (kSegOn) {
#pragma unroll
        for (int j = 0; j < kMaxP; ++j) {
          const float v = j < P ? __uint_as_float(xs[j][2 * seg_i + 0]) : -INFINITY;
          const int i = j < P ? (int)xs[j][2 * seg_i + 1] : V;
          if (v > gv || (v == gv && i < gi)) {
            gv = v;
            gi = i;
          }
        }
      } else {
        float bv = -INFINITY;
        int bi = V;
        FOR_CHUNKS(c,
          float v[8];
          logits8(c, v);
          const int y0 = y0_of(c);
          _Pragma("unroll")
          for (int e = 0; e < 8; ++e)
            if (v[e] > bv) {
              bv = v[e];
              bi = y0 + e;
            }
        )
        {
          struct VI { float v; int i; };
          auto mv = [&](auto c, auto r, VI old, VI x) {
            return VI{dpp_f<decltype(c)::value, decltype(r)::value>(old.v, x.v),
                      dpp_i<decltype(c)::value, decltype(r)::value>(old.i, x.i)};
          };
          auto comb = [](VI x, VI y) { return (y.v > x.v || (y.v == x.v && y.i < x.i)) ? y : x; };
          const VI t = dpp_reduce<true>(VI{bv, bi}, VI{-INFINITY, V}, mv, comb);
          bv = t.v;
          bi = t.i;
        }
        lds_sync();
        if (lane == 63) {
          red_f[wave] = bv;
          red_i[wave] = bi;
        }
        lds_sync();
        bv = red_f[0];
        bi = red_i[0];
        for (int w = 1; w < kAW; ++w)
          if (red_f[w] > bv || (red_f[w] == bv && red_i[w] < bi)) {
            bv = red_f[w];
            bi = red_i[w];
          }
        exchange(__float_as_uint(bv), (uint32_t)bi);
        {
          uint32_t x0[kMaxP], x1[kMaxP];
          read_pairs(x0, x1, __float_as_uint(-INFINITY), (uint32_t)V);
  #pragma unroll
          for (int j = 0; j < kMaxP; ++j) {
            const float v = __uint_as_float(x0[j]);
            const int i = (int)x1[j];
            if (v > gv || (v == gv && i < gi)) {
              gv = v;
              gi = i;
            }
          }
        }
      }
      if constexpr (kSegOn) {
        // the first child first; the others are listed only when it misses
        if (nk > 0 && s_tok[fk[cur]] == gi) {
          nxt = 0;
        } else if (nk > 0) {
          nk = gather_children(cur);
          for (int c = 1; c < nk; ++c)
            if (s_tok[kids[c]] == gi) {
              nxt = c;
              break;
            }
        }
      } else {
        for (int c = 0; c < nk; ++c)
          if (s_tok[kids[c]] == gi) {
            nxt = c;
            break;
          }
      }
      if (nxt < 0) {
        if (wg == 0 && tid == 0) a.bonus[b] = gi;
        stop = true;
      }
    } else if constexpr (kSegOn && !mss) {
      // target sampling on a chain: the node's token was drawn with its chain
      int xd = -1;
#pragma unroll
      for (int j = 0; j < kMaxP; ++j)
        if (j < P) xd = max(xd, (int)xs[j][seg_i] - 1);
      if (nk > 0 && s_tok[fk[cur]] == xd) {
        nxt = 0;
      } else if (nk > 0) {
        nk = gather_children(cur);
        for (int c = 1; c < nk; ++c)
          if (s_tok[kids[c]] == xd) {
            nxt = c;
            break;
          }
      }
      if (nxt < 0) {
        if (wg == 0 && tid == 0) a.bonus[b] = xd;
        stop = true;
      }
    } else {
      // statistics of this slice: its max and the mass relative to it,
      // merged across lanes and waves (in lane 63 of each wave); a chain
      // node has them from its chain's exchange
      if constexpr (!kSegOn) {
      float mt = -INFINITY;
      double st = 0.0;
      if constexpr (CACHED) {
        row_stats(lc, mt, st);   // the slice is in registers
      } else {
      FOR_CHUNKS(c,
        float v[8];
        logits8(c, v);
        float cm = v[0];
        _Pragma("unroll")
        for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[e]);
        if (cm > -INFINITY) {
          const float mn = fmaxf(mt, cm);
          double w[8];
          _Pragma("unroll")
          for (int e = 0; e < 8; ++e) w[e] = (double)__builtin_amdgcn_exp2f((v[e] - mn) * c2);
          const double add = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
          st = (mt == -INFINITY ? 0.0 : st * (double)__builtin_amdgcn_exp2f((mt - mn) * c2)) + add;
          mt = mn;
        }
      )
      {
        struct MS { float m; double s; };
        auto mv = [&](auto c, auto r, MS old, MS x) {
          return MS{dpp_f<decltype(c)::value, decltype(r)::value>(old.m, x.m),
                    dpp_d<decltype(c)::value, decltype(r)::value>(old.s, x.s)};
        };
        auto comb = [&](MS x, MS y) {
          const float mn = fmaxf(x.m, y.m);
          if (mn == -INFINITY) return MS{mn, 0.0};
          return MS{mn, (x.m == -INFINITY ? 0.0 : x.s * (double)__builtin_amdgcn_exp2f((x.m - mn) * c2)) +
                            (y.m == -INFINITY ? 0.0 : y.s * (double)__builtin_amdgcn_exp2f((y.m - mn) * c2))};
        };
        const MS t = dpp_reduce<true>(MS{mt, st}, MS{-INFINITY, 0.0}, mv, comb);
        mt = t.m;
        st = t.s;
      }
      }
      lds_sync();
      if (lane == 63) {
        red_f[wave] = mt;
        red_d[wave] = st;
      }
      lds_sync();
      float mw;
      double sw;
      wg_stats(red_f, red_d, mw, sw);
      // the children's test scalars reach LDS only now: their loads were in
      // flight during the statistics pass and the exchange's wait
      if (kid_lane) {
        if constexpr (kBF) kid_l[tid] = bf16_to_f32(kl_raw);
        else kid_l[tid] = kl_raw;
        kid_q[tid] = kq;
        kid_u[tid] = ku;
      }
      exchange(__float_as_uint(mw), __float_as_uint((float)sw));
      if (nk > 0) load_row(row_of(kids[0]), pfc);
      }
      // the P slices' (max, mass) combined (slice_bfly); mass[] is read only
      // by the draw
      float m;
      double z0;
      {
        const int j = lane & 15;
        float mj = -INFINITY, sj = 0.f;
        if (j < P) {
          if constexpr (kSegOn) {
            mj = __uint_as_float(xs[j][2 * seg_i + 0]);
            sj = __uint_as_float(xs[j][2 * seg_i + 1]);
          } else {
            mj = xf(j, 0);
            sj = xf(j, 1);
          }
        }
        double mass_j;
        slice_bfly(mj, sj, m, z0, mass_j);
        if (tid < P) mass[tid] = mass_j;
      }
      auto ew8 = [&](int c, double* w8) {
        float v[8];
        logits8(c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w8[e] = v[e] == -INFINITY ? 0.0 : (double)__builtin_amdgcn_exp2f((v[e] - m) * c2);
      };
      if constexpr (!mss) {
        const float u = u_draw;
        const int x = draw(u, ew8);
        exchange((uint32_t)(x + 1), 0u);   // only the drawing workgroup has x >= 0
        int xs = -1;
        {
          uint32_t x0[kMaxP], x1[kMaxP];
          read_pairs(x0, x1, 0u, 0u);
#pragma unroll
          for (int j = 0; j < kMaxP; ++j) xs = max(xs, (int)x0[j] - 1);
        }
        for (int c = 0; c < nk; ++c)
          if (s_tok[kids[c]] == xs) {
            nxt = c;
            break;
          }
        if (nxt < 0) {
          if (wg == 0 && tid == 0) a.bonus[b] = xs;
          stop = true;
        }
      } else {
        int nrej = 0;
        // the normaliser of the last rejection whose residual mass was
        // positive (the statistics pass's if none was): the unit of mass[]
        double units = z0;
        // Residual after `upto` rejections for one token: r <- max(r - q, 0) /
        // Z_j for each rejection j whose mass Z_j was positive (zero mass
        // leaves r unchanged), multiplying by the reciprocals zinv[j].  The
        // cached path below applies the same operations element by element.
        auto resid = [&](double r0, double qy, int upto) -> double {
          double r = r0;
          for (int j = 0; j < upto; ++j)
            if (zinv[j] > 0.0) r = fmax(r - qy, 0.0) * zinv[j];
          return r;
        };
        const double iz0 = 1.0 / z0;
        // p(y) / z0 in the arithmetic the tests use: fp32 exp2 of the scaled
        // difference, then float64
        auto p_of = [&](float l) -> double {
          return l == -INFINITY ? 0.0 : (double)__builtin_amdgcn_exp2f((l - m) * c2) * iz0;
        };
        // CACHED: this thread's elements of the current residual, in float64,
        // formed at the first rejection (a first child accepted at once never
        // needs them)
        double rr[CACHED ? kMaxCh : 1][8];
        auto init_rr = [&]() {
          if constexpr (CACHED) {
            FOR_CHUNKS(cc,
              float v[8];
              logits8(cc, v);
              _Pragma("unroll")
              for (int e = 0; e < 8; ++e) rr[cc][e] = p_of(v[e]);
            )
          }
        };
        for (int c = 0; c < nk; ++c) {
          if ((c > 0 && c % kMaxKid == 0) || (kSegOn && c == 1)) {
            // the next batch of children's test scalars (wide nodes, and a
            // chain node once its first child is rejected); these loads are
            // waited for here, off the common path
            lds_sync();
            const int cc = c - c % kMaxKid + tid;
            if (tid < kMaxKid && cc < nk) {
              const int node = kids[cc];
              const int x = s_tok[node];
              kid_l[tid] = Elem<LT>::load(row, x);
              kid_q[tid] = qrow[x];
              kid_u[tid] = a.unif[((size_t)b * T + node) * 2];
            }
            lds_sync();
          }
          const int ci = c % kMaxKid;
          float lx;
          double qx, u;
          if (kSegOn && c == 0) {
            lx = seg_l[seg_i];
            qx = (double)seg_q[seg_i];
            u = (double)seg_u[seg_i];
          } else {
            lx = kid_l[ci];
            qx = (double)kid_q[ci];
            u = (double)kid_u[ci];
          }
          const double rx = resid(p_of(lx), qx, nrej);
          if (u * qx < rx) {
            nxt = c;
            break;
          }
          // rejected: this slice's mass of max(r - q, 0), exchanged in full
          // float64 precision
          double pz = 0.0;
          if constexpr (CACHED) {
            if (nrej == 0) {
              need_row();
              // The draft row's slice is read only now: a first child accepted
              // at once never needs it, and it is two thirds of a node's bytes
              // (float32 against bf16 logits), which all sequences' walks
              // share the memory for.  (Chunks outside the slice hold unused
              // draft values; every use there meets a zero residual.)
#pragma unroll
              for (int c = 0; c < kMaxCh; ++c) {
                const int yq = cached_y(c);
                const float4 u0 = *reinterpret_cast<const float4*>(qrow + yq);
                const float4 u1 = *reinterpret_cast<const float4*>(qrow + yq + 4);
                qc[c][0] = u0.x; qc[c][1] = u0.y; qc[c][2] = u0.z; qc[c][3] = u0.w;
                qc[c][4] = u1.x; qc[c][5] = u1.y; qc[c][6] = u1.z; qc[c][7] = u1.w;
              }
              init_rr();
            }
            FOR_CHUNKS(cc,
              float q8[8];
              q8_of(cc, q8);
              _Pragma("unroll")
              for (int e = 0; e < 8; ++e) pz += fmax(rr[cc][e] - (double)q8[e], 0.0);
            )
          } else {
            FOR_CHUNKS(cc,
              float v[8];
              float q8[8];
              logits8(cc, v);
              q8_of(cc, q8);
              _Pragma("unroll")
              for (int e = 0; e < 8; ++e) {
                const double qy = (double)q8[e];
                pz += fmax(resid(p_of(v[e]), qy, nrej) - qy, 0.0);
              }
            )
          }
          pz = wg_sum(pz);
          const unsigned long long pzb = (unsigned long long)__double_as_longlong(pz);
          exchange((uint32_t)pzb, (uint32_t)(pzb >> 32));
          double z;
          {
            // butterfly over the 16 slices, as for z0
            const int j = lane & 15;
            z = j < P ? __longlong_as_double((long long)(((unsigned long long)xv[j][1] << 32) | xv[j][0])) : 0.0;
            auto mvd = [](auto c, auto r, double old, double x) { return dpp_d<decltype(c)::value, decltype(r)::value>(old, x); };
            z = dpp_reduce<false>(z, 0.0, mvd, [](double x, double y) { return x + y; });
          }
          if (z > 0.0 && tid < P)
            mass[tid] = __longlong_as_double((long long)(((unsigned long long)xv[tid][1] << 32) | xv[tid][0]));
          const double zi = z > 0.0 ? 1.0 / z : 0.0;
          if (z > 0.0) units = z;
          if (tid == 0) zinv[nrej] = zi;
          if constexpr (CACHED) {
            if (z > 0.0) {
              FOR_CHUNKS(cc,
                float q8[8];
                q8_of(cc, q8);
                _Pragma("unroll")
                for (int e = 0; e < 8; ++e) rr[cc][e] = fmax(rr[cc][e] - (double)q8[e], 0.0) * zi;
              )
            }
          }
          lds_sync();
          ++nrej;
          if (kSegOn && c == 0) nk = gather_children(cur);
        }
        if (nxt < 0) {
          if (nrej == 0) {
            need_row();
            init_rr();   // a leaf: the draw is from p itself
          }
          const float u = u_draw;
          const int nr = nrej;
          // weights in the units of mass[]: the residual times `units`
          auto rw8 = [&](int c, double* w8) {
            if constexpr (CACHED) {
#pragma unroll
              for (int e = 0; e < 8; ++e) w8[e] = rr[c][e] * units;
            } else {
              float v[8];
              float q8[8];
              logits8(c, v);
              q8_of(c, q8);
#pragma unroll
              for (int e = 0; e < 8; ++e) w8[e] = resid(p_of(v[e]), (double)q8[e], nr) * units;
            }
          };
          const int x = draw(u, rw8);
          if (x >= 0 && tid == 0) a.bonus[b] = x;
          stop = true;
        }
      }
    }
    if (stop) break;
    const int nnode = (kSegOn && nxt == 0) ? fk[cur] : kids[nxt];
    if (wg == 0 && tid == 0) path[plen] = nnode;
    ++plen;
    cur = nnode;
    have_row = false;
    if constexpr (kSegOn) {
      // the first child is the chain's next node; any other starts a chain
      if (nxt == 0 && seg_i + 1 < seg_len) ++seg_i;
      else seg_len = 0;
    } else if constexpr (CACHED) {
      if (nxt == 0) {
#pragma unroll
        for (int c = 0; c < kMaxCh; ++c) lc[c] = pfc[c];
        have_row = true;
      }
    }
    lds_sync();
  }
  if (wg == 0 && tid == 0) a.path_len[b] = plen;
  SD_DCHECK(plen >= 1 && plen <= T, a.status);
  if (commit) {
    if (cerr) {
      if (wg == 0 && tid == 0) set_status(a.status, cerr);
    } else {
      // the path, rebuilt from its last node through the parents, in kids[]
      lds_sync();
      if (tid == 0) {
        int n = cur;
        for (int j = plen - 1; j >= 0; --j) {
          kids[j] = n;
          n = s_par[n];
        }
      }
      lds_sync();
      commit_copy(plen);
    }
  }
  if (P > 1) {
    // the last workgroup of the sequence to leave clears the slots, so the
    // next call starts from barrier number 1 again; with a commit it also
    // writes the new context length (every workgroup read the old one first)
    lds_sync();
    if (tid == 0) s_flag = atomicAdd(done, 1u) == (unsigned)P - 1;
    lds_sync();
    if (s_flag) {
      for (int j = tid; j < 2 * kMaxP * kXW; j += kAT)
        __hip_atomic_store(slots + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) {
        if (commit && !cerr) a.cctx[b] = c_ctx + plen;
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else if (commit && !cerr && tid == 0) {
    a.cctx[b] = c_ctx + plen;
  }
  if (tid == 0 && s_to) set_status(a.status, SD_ERR_TIMEOUT);
}

int accept_wgs(int B, int V) {
  int P = 256 / (B > 0 ? B : 1);
  P = P < kMaxP ? P : kMaxP;
  const int by_v = (V + kChunk - 1) / kChunk;
  P = P < by_v ? P : by_v;
  return P > 1 ? P : 1;
}

template <int MODE>
static const void* accept_fn(const AcceptArgs& a) {
  if (a.logits_f32) return reinterpret_cast<const void*>(accept_kernel<float, false, MODE>);
  if (a.NC <= kMaxCh && (a.V & 7) == 0)
    return reinterpret_cast<const void*>(accept_kernel<bf16_bits, true, MODE>);
  return reinterpret_cast<const void*>(accept_kernel<bf16_bits, false, MODE>);
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  const void* fn = a.tau == 0.f ? accept_fn<kGreedy>(a)
                   : a.draft != nullptr ? accept_fn<kRejection>(a)
                                        : accept_fn<kTarget>(a);
  const dim3 grid((unsigned)a.B * a.P), block(kAT);
  // B * P <= 256: with one workgroup per CU every workgroup of the grid is
  // resident at once, which the cross-workgroup waits rely on (they are
  // bounded in any case).
  AcceptArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(fn, grid, block, args, 0, st);
}

// ---- the allocation-free variant ------------------------------------------
// Exchange slots of up to kNoAllocMaxSeqs sequences in a device array owned by
// the library (one copy per GPU, alive until the process ends).  Host code
// never uses the array's name as an address: the device address is looked up
// once per device and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[(size_t)kNoAllocMaxSeqs * kAccSeqBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call there).
static hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Zero-fill of n 16-byte words (a kernel rather than a memset node, so the
// call stays safe to capture in a graph).
__global__ void __launch_bounds__(256) zero16_kernel(uint4* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_accept_noalloc(AcceptArgs a, hipStream_t st) {
  if (a.P > 1 && a.B > kNoAllocMaxSeqs) return hipErrorInvalidValue;   // (the caller checks first)
  void* sp = nullptr;
  hipError_t e = scratch_on_current_device(&sp);
  if (e != hipSuccess) return e;
  a.sync = static_cast<unsigned char*>(sp);   // (read only when P > 1)
  if (a.P > 1) {
    // the slots of the sequences this call uses start from zero whatever an
    // earlier call (on any stream of this device) left there
    const int n16 = (int)((size_t)a.B * kAccSeqBytes / 16);
    hipLaunchKernelGGL(zero16_kernel, dim3((n16 + 255) / 256), dim3(256), 0, st,
                       static_cast<uint4*>(sp), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_accept(a, st);
}

}  // namespace sdtree
