// Internal definitions shared by the sdtree kernels and the host layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "sdtree.h"

namespace sdtree {

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Workspace header: the sticky status word and small counters live in the
// first 256 bytes; call-specific regions follow.
constexpr size_t kWsHeader = 256;
// 64 bytes inside the header that no kernel writes: a zero source for loads
// of keys that do not exist.
constexpr size_t kWsZeros = 128;

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_bits>(u >> 16);
}

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory /
// n LDS-or-scalar operations are outstanding, leaving the other counters free.
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | ((n >> 4) << 14) | (7u << 4) | (15u << 8); }
constexpr unsigned lgkmcnt_imm(unsigned n) { return 15u | (3u << 14) | (7u << 4) | ((n & 15u) << 8); }

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// Device-side consistency checks of the debug build (compiled with
// -DSDTREE_DEBUG into libsdtree_debug.so): invariants that the host's plan and
// the kernels must agree on, which no argument reaching a kernel can break.
// A failed check sets SD_ERR_DEBUG in the call's status word and the kernel
// goes on (no trap); the release build compiles them away.
#ifdef SDTREE_DEBUG
#define SD_DCHECK(cond, status)                                       \
  do {                                                                \
    if (!(cond)) ::sdtree::set_status((status), SD_ERR_DEBUG);        \
  } while (0)
#else
#define SD_DCHECK(cond, status) \
  do {                          \
  } while (0)
#endif

// Element loads for the two storage types.
template <typename E> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_bits> {
  static __device__ __forceinline__ float load(const bf16_bits* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(bf16_bits* p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// ---------------------------------------------------------------------------
// Kept block key sums (float32 [num_blocks][Hkv][D], per physical block):
// extend one KV head's sums over positions [t0, t1) of a sequence, in
// position order, each block continuing from its current sum, or from +0 for
// a block whose first position is among them -- the sequential sum the block
// selection divides.  One wavefront: lane owns dims lane * D / 64 ...
// krow(n): the K rows of logical block n, head g (row 0); sum_at(n): its sums.
template <typename E, int D, typename KRow, typename SumAt>
__device__ __forceinline__ void extend_head_sums(int bs, int t0, int t1, int lane, KRow krow, SumAt sum_at) {
  constexpr int DPL = D / 64;
  const int d0 = lane * DPL;
  for (int t = t0; t < t1;) {
    const int n = t / bs, off = t - n * bs;
    const int tn = min((n + 1) * bs, t1);
    float* kept = sum_at(n) + d0;
    const E* row = krow(n) + d0;
    float s[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) s[e] = off == 0 ? 0.f : kept[e];
    // rows loaded RIF at a time, all in flight, then added in position order
    constexpr int RIF = 16;
    const int end = off + (tn - t);
    for (int u0 = off; u0 < end; u0 += RIF) {
      float x[RIF][DPL];
#pragma unroll
      for (int r = 0; r < RIF; ++r) {
        const int u = min(u0 + r, end - 1);     // (past the end: a valid row, not added)
        if constexpr (sizeof(E) == 2) {
          if constexpr (DPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(row + (size_t)u * D);
            x[r][0] = bf16_to_f32((bf16_bits)(w & 0xFFFFu));
            x[r][1] = bf16_to_f32((bf16_bits)(w >> 16));
          } else {
            x[r][0] = bf16_to_f32(row[(size_t)u * D]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < DPL; ++e) x[r][e] = row[(size_t)u * D + e];
        }
      }
#pragma unroll
      for (int r = 0; r < RIF; ++r)
        if (u0 + r < end)
#pragma unroll
          for (int e = 0; e < DPL; ++e) s[e] = s[e] + x[r][e];
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) kept[e] = s[e];
    t = tn;
  }
}

// extend_head_sums for the element type and head dim known at run time
// (D in {64, 128}, esize 2 = bf16 or 4 = float32).
template <typename KRow, typename SumAt>
__device__ __forceinline__ void extend_head_sums_rt(int esize, int D, int bs, int t0, int t1, int lane,
                                                    KRow krow_bytes, SumAt sum_at) {
  if (esize == 2) {
    auto kr = [&](int n) { return reinterpret_cast<const bf16_bits*>(krow_bytes(n)); };
    if (D == 128) extend_head_sums<bf16_bits, 128>(bs, t0, t1, lane, kr, sum_at);
    else extend_head_sums<bf16_bits, 64>(bs, t0, t1, lane, kr, sum_at);
  } else {
    auto kr = [&](int n) { return reinterpret_cast<const float*>(krow_bytes(n)); };
    if (D == 128) extend_head_sums<float, 128>(bs, t0, t1, lane, kr, sum_at);
    else extend_head_sums<float, 64>(bs, t0, t1, lane, kr, sum_at);
  }
}

// ---------------------------------------------------------------------------
// Attention launch plan (host side; depends on the shape only).
struct AttnPlan {
  int variant;          // 0: VALU (fp32 or tiny), 1: MFMA bf16
  int D;
  int WQ, WK, QW, KW;   // waves across query rows / across keys; rows and keys per wave
  int NK;               // keys per LDS tile = KW * WK
  int rows;             // query rows per workgroup = WQ * QW
  int n_qtiles, n_splits, tps;
  int n_ct_max;         // context tiles, upper bound
  int n_tt;             // tree tiles
  int W64;              // 64-bit ancestor words per node
  int T_tree;           // number of distinct trees (1 or B)
  int u_max;            // sparse: max distinct blocks per workgroup
  int ct_max, tt_max;   // LDS block-id table sizes (context tiles of one split, tree slots)
  int stages;           // LDS ring depth
  int anc_lds_words;
  size_t lds_bytes;
  size_t anc_off, part_o_off, part_ml_off, total;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* ctx;
  const int32_t* parent;
  const uint64_t* anc;
  const int32_t* sel;
  int32_t ksel;
  void* out;
  float* part_o;
  float* part_ml;
  uint32_t* status;
  int B, T, Hq, Hkv, G, M, D, bs, max_blocks, num_blocks, tree_stride;
  float scale_log2;
  int n_qtiles, n_splits, tps, W64, u_max;
  int bs_shift;         // log2(bs)
  int ct_max, tt_max;   // LDS entries for context / tree block ids
  int anc_lds_words;    // ancestor words the kernel may stage in LDS
  const void* zeros;    // >= 16 zero bytes in device memory
};

// Per-sequence synchronisation scratch of the acceptance walk: barrier
// counter, exit counter, a broadcast slot, then [2][P][2] float64 partials.
constexpr size_t kAccSeqBytes = 8192;

struct AcceptArgs {
  const void* logits;
  int logits_f32;
  const float* draft;
  const int32_t* parent;
  const int32_t* token;
  const float* unif;
  float tau;
  int B, T, V, tree_stride;
  int32_t* path;
  int32_t* path_len;
  int32_t* bonus;
  uint32_t* status;
  unsigned char* sync;  // B * kAccSeqBytes, zero before the first call (P > 1 only)
  int P, SL, NC;        // workgroups per sequence, tokens per workgroup, 2048-token chunks
  // commit of the accepted paths in the same launch (cctx == nullptr: none)
  void* ck;
  void* cv;
  const int32_t* ctable;
  int32_t* cctx;
  float* csums;         // kept block key sums to extend with the commit (NULL: none)
  int cHkv, cD, cbs, cmax_blocks, cnum_blocks, cesize;
};

int accept_wgs(int B, int V);

constexpr int kMaxTreeNodes = 4096;  // largest tree (T) any call accepts
constexpr int kMaxCommitT = kMaxTreeNodes;

struct CommitArgs {
  void* k;
  void* v;
  const int32_t* table;
  int32_t* ctx;
  const int32_t* path;
  const int32_t* path_len;
  uint32_t* status;
  unsigned* counters;   // one per sequence, zero between calls
  float* sums;          // kept block key sums to extend (NULL: none)
  int B, T, Hkv, D, bs, max_blocks, num_blocks, esize;
};

struct TopkArgs {
  const void* q;
  const void* k;
  const int32_t* table;
  const int32_t* ctx;
  int32_t* sel;
  float* means;    // [B][nbmax][Hkv][D]
  float* scores;   // [B*T*Hq][nbmax]
  float* sums;     // kept block key sums [num_blocks][Hkv][D] (cached selection)
  int32_t* rep;    // shared selection: each (b, group) list goes to all the group's rows
  int rep_T, rep_Hq, rep_G;
  uint32_t* status;
  int B, T, Hq, Hkv, G, D, bs, max_blocks, num_blocks, topk, nbmax;
};

// One batched expansion step of the draft-tree search.
constexpr int kMaxExpandK = 4096;
struct ExpandArgs {
  const void* logits;   // [E][V]
  const float* cum;     // [E]
  float inv_tau;
  int E, V, k;
  float* off;           // [E] workspace
  uint32_t* hist;       // [8][256] workspace
  uint32_t* count;      // workspace, zero between calls
  unsigned long long* keys;  // [k] workspace
  int32_t* out_row;
  int32_t* out_token;
  float* out_score;
};

// Best-first construction of a draft tree on the GPU.
struct BuildArgs {
  const void* logits;   // [T][V] drafter logits, row n = node n's
  int T, V;
  float tau;
  int root_token;
  int margin;           // extra candidates of the float32 pre-selection
  int32_t* parent;      // [T] out
  int32_t* token;       // [T] out
  double* cum;          // [T] out: cumulative log-probability
  float* cum32;         // [T] workspace: float32 copy for the pre-selection
  double* rmax;         // [T] workspace: row max of l / tau
  double* rlse;         // [T] workspace: row log-sum-exp after the max
  int32_t* cand_row;    // [k] workspace: pre-selected candidates
  int32_t* cand_token;
  int* n_dev;           // nodes in the tree
  uint32_t* status;
};

// Events a call's first kernel records at its start and its last kernel at
// its end (either may be null).
struct CallEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (one per kernel family).
hipError_t launch_expand(const ExpandArgs& a, bool f32, hipStream_t st);
hipError_t run_tree_build(const BuildArgs& a, const ExpandArgs& ex0, bool f32, hipStream_t st,
                          int* rounds);
hipError_t launch_anc_mask(const int32_t* parent, int T, int W64, int n_trees, uint64_t* anc,
                           uint32_t* status, hipStream_t st, hipEvent_t start = nullptr);
hipError_t launch_attn_valu(const AttnArgs& a, bool f32, hipStream_t st, CallEvents ev = {});
hipError_t launch_attn_mfma(const AttnArgs& a, const AttnPlan& p, hipStream_t st, CallEvents ev = {});
hipError_t launch_accept(const AcceptArgs& a, hipStream_t st);
// The acceptance walk with its exchange slots in the library's own device
// array (no workspace argument): at most kNoAllocMaxSeqs sequences when a
// sequence spans several workgroups.
constexpr int kNoAllocMaxSeqs = 128;
hipError_t launch_accept_noalloc(AcceptArgs a, hipStream_t st);
hipError_t launch_commit(const CommitArgs& a, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, bool f32, bool cached, hipStream_t st);
hipError_t launch_topk_shared(const TopkArgs& a, bool f32, bool cached, hipStream_t st);
hipError_t launch_block_sums(const TopkArgs& a, bool f32, hipStream_t st);
hipError_t launch_block_sums_append(const TopkArgs& a, const int32_t* n_new, bool f32, hipStream_t st);

}  // namespace sdtree
