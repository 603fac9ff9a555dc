// Host side of the sdtree C ABI: argument validation (always before any HIP
// call), launch planning, workspace carving, kernel launches.
#include <math.h>
#include <string.h>

#include <algorithm>

#include <limits.h>

#include "common.h"

namespace sdtree {

constexpr int kMaxKsel = 1 << 16;   // widest sparse selection (blocks per query row)
constexpr size_t kLdsLimit = 160 * 1024;

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static sd_status check_shape(const sd_shape* s) {
  if (!s) return SD_INVALID_ARG;
  if (s->B < 1 || s->T < 1 || s->Hq < 1 || s->Hkv < 1 || s->D < 1 || s->bs < 1 ||
      s->max_blocks < 1 || s->num_blocks < 1)
    return SD_BAD_SHAPE;
  if (s->Hq % s->Hkv != 0) return SD_BAD_SHAPE;
  if (s->tree_stride != 0 && s->tree_stride != s->T) return SD_BAD_SHAPE;
  if (s->dtype != SD_F32 && s->dtype != SD_BF16) return SD_BAD_DTYPE;
  if (s->D != 64 && s->D != 128) return SD_UNSUPPORTED;
  if (s->bs < 8 || (s->bs & (s->bs - 1)) != 0) return SD_UNSUPPORTED;
  if (s->T > kMaxTreeNodes) return SD_UNSUPPORTED;
  // query rows, and so every per-row index, fit an int
  if ((long long)s->B * s->T > INT_MAX || (long long)s->B * s->T * s->Hq > INT_MAX) return SD_UNSUPPORTED;
  if ((long long)s->max_blocks * s->bs > (1ll << 30)) return SD_UNSUPPORTED;
  // (in double: the product of four ints can pass 2^63)
  if ((double)s->num_blocks * s->Hkv * s->bs * s->D > (double)(1ll << 40)) return SD_UNSUPPORTED;
  if (!(s->scale >= 0.f) || isinf(s->scale)) return SD_INVALID_ARG;
  return SD_OK;
}

// The plan depends on the shape only, so workspace sizing and launch agree.
static AttnPlan plan_attn(const sd_shape* s, int ksel, bool sparse) {
  AttnPlan p;
  memset(&p, 0, sizeof(p));
  const int G = s->Hq / s->Hkv;
  const int M = s->T * G;
  p.D = s->D;
  p.W64 = (s->T + 63) / 64;
  p.T_tree = s->tree_stride ? s->B : 1;
  p.anc_off = kWsHeader;
  // precomputed ancestor masks, read by the per-row float32 kernel only
  const size_t anc_bytes = s->dtype == SD_F32 ? (size_t)p.T_tree * s->T * p.W64 * 8 : 0;
  p.part_o_off = align_up(p.anc_off + anc_bytes, 256);
  if (s->dtype == SD_F32) {
    p.variant = 0;
    p.n_splits = 1;
    p.part_ml_off = p.part_o_off;
    p.total = p.part_o_off;
    return p;
  }
  p.variant = 1;
  if (M <= 32) {
    p.WQ = 1; p.WK = 4; p.QW = 32; p.KW = 32;
  } else if (M <= 64) {
    p.WQ = 2; p.WK = 2; p.QW = 32; p.KW = 32;
  } else if (M <= 128 || p.D != 128 || (long long)s->B * s->Hkv * ((M + 255) / 256) < 256) {
    // eight wavefronts: four 32-row query slices x two 32-key slices, two
    // wavefronts per SIMD so one's MFMAs overlap the other's softmax
    p.WQ = 4; p.WK = 2; p.QW = 32; p.KW = 32;
  } else {
    // eight wavefronts of 32 query rows each over 32-key tiles: one workgroup
    // streams a (sequence, KV head)'s keys once for 256 query rows, halving
    // the L2-to-LDS traffic of many query tiles.  Taken when it fills the
    // chip without splitting the context (a split's partials and their merge
    // cost more than the halved traffic saves), and for D = 128 (a 32-key K
    // tile is then one 16-byte load per thread).
    p.WQ = 8; p.WK = 1; p.QW = 32; p.KW = 32;
  }
  p.NK = p.KW * p.WK;
  p.rows = p.WQ * p.QW;
  p.n_qtiles = (M + p.rows - 1) / p.rows;
  p.n_tt = (s->T + p.NK - 1) / p.NK;
  const long long cap = (long long)s->max_blocks * s->bs;
  if (sparse) {
    p.u_max = (int)std::min<long long>(s->max_blocks, (long long)p.rows * ksel);
    p.n_ct_max = (int)(((long long)p.u_max * s->bs + p.NK - 1) / p.NK);
  } else {
    const long long ctx_max = std::max<long long>(cap - s->T, 0);
    p.n_ct_max = (int)((ctx_max + p.NK - 1) / p.NK);
  }
  const int ntiles = p.n_ct_max + p.n_tt;
  const long long base = (long long)s->B * s->Hkv * p.n_qtiles;
  // At least one workgroup per CU (256 CUs) when the context allows, with at
  // least 8 tiles per split, and at most 2048 context block ids per split.
  const long long want = 256;
  int splits = (int)std::max<long long>(1, (want + base - 1) / base);
  splits = std::min(splits, std::max(1, ntiles / 8));
  const int per_tile = std::max(1, p.NK / s->bs);
  splits = std::max(splits, (ntiles * per_tile + 2047) / 2048);
  p.tps = (ntiles + splits - 1) / splits;
  p.n_splits = (ntiles + p.tps - 1) / p.tps;
  p.ct_max = (int)(((long long)p.tps * p.NK + s->bs - 1) / s->bs) + 2;
  p.tt_max = (s->T + s->bs - 1) / s->bs + 2;
  // LDS: the K / V ring, tree-tile flags and list, block-id tables, staged
  // ancestor words, sparse tables.  The key-slice merge reuses the ring.
  const size_t stage = (size_t)p.NK * p.D * 2 * 2;
  const int nnodes = (p.rows + G - 1) / G + 1;
  const size_t anc_need = (size_t)nnodes * p.W64;
  size_t extras = 128 + 4 * 128 + 8 * (size_t)(p.ct_max + p.tt_max);
  if (sparse) {
    const size_t bw = (size_t)(s->max_blocks + 31) / 32;
    extras += 4 * bw * 2 + 8 * (size_t)p.u_max + 4 * (size_t)p.rows * ((p.u_max + 31) / 32);
  }
  p.anc_lds_words = (int)anc_need;
  extras += 8 * anc_need;
  // deepest ring that fits: 4, 3 or 2 stages for the wide tile, 4 or 2 for
  // two key slices, 2 for four key slices
  const int cand[5] = {8, 4, 3, 2, 0};
  p.stages = 0;
  for (int c : cand) {
    if (c == 0) break;
    if (p.WQ == 8 ? (c != 8 && c != 4) : c == 8) continue;
    if (p.WQ == 1 && c != 2) continue;
    if (p.WQ == 2 && c == 3) continue;
    const size_t merge = p.WK > 1 ? (size_t)p.WQ * p.WK * (p.QW * p.D + 2 * p.QW) * 4 : 0;
    if (std::max(c * stage, merge) + extras <= kLdsLimit) {
      p.stages = c;
      break;
    }
  }
  if (p.stages == 0) p.stages = p.WQ == 8 ? 4 : 2;   // reported as SD_UNSUPPORTED by the LDS check
  const size_t merge = p.WK > 1 ? (size_t)p.WQ * p.WK * (p.QW * p.D + 2 * p.QW) * 4 : 0;
  size_t lds = std::max(p.stages * stage, merge) + extras;
  p.lds_bytes = align_up(lds, 16);
  const size_t nrows = (size_t)s->B * s->T * s->Hq;
  if (p.n_splits > 1) {
    p.part_ml_off = align_up(p.part_o_off + nrows * p.n_splits * p.D * 4, 256);
    p.total = align_up(p.part_ml_off + nrows * p.n_splits * 2 * 4, 256);
  } else {
    p.part_ml_off = p.part_o_off;
    p.total = p.part_o_off;
  }
  return p;
}

// Commit scratch: the status header and one completion counter per sequence.
static size_t commit_ws(const sd_shape* s) { return kWsHeader + align_up((size_t)s->B * 4, 256); }

// Expansion scratch: row offsets, 8 x 256 histograms, a counter, k keys.
// The counter and the histograms sit at offsets that do not depend on the
// shape, so a workspace that was zero-filled once stays valid for calls of any
// shape (the sort kernel clears the counter, the first kernel the histograms).
static size_t expand_ws(const sd_expand_shape* s, int32_t k, size_t* off, size_t* hist, size_t* cnt,
                        size_t* keys) {
  const size_t c = kWsHeader;
  const size_t h = align_up(c + 4, 256);
  const size_t o = h + 8 * 256 * 4;
  const size_t kk = align_up(o + (size_t)s->E * 4, 256);
  if (off) *off = o;
  if (hist) *hist = h;
  if (cnt) *cnt = c;
  if (keys) *keys = kk;
  return align_up(kk + (size_t)k * 8, 256);
}

constexpr int kBuildMargin = 256;

static sd_status check_build(const sd_build_shape* s) {
  if (!s) return SD_INVALID_ARG;
  if (s->T < 1 || s->V < 1) return SD_BAD_SHAPE;
  if (s->logit_dtype != SD_F32 && s->logit_dtype != SD_BF16) return SD_BAD_DTYPE;
  if ((long long)s->T * s->V >= 0xFFFFFFFFll) return SD_UNSUPPORTED;
  if ((long long)s->T - 1 + kBuildMargin > kMaxExpandK) return SD_UNSUPPORTED;
  return SD_OK;
}

// Build scratch: the expansion step's scratch for T rows and the round's
// candidate count, then per-row float64 statistics, the float32 copy of the
// cumulative log-probabilities, the candidates and the node counter.
struct BuildLayout {
  size_t exp_off, exp_hist, exp_cnt, exp_keys, rmax, rlse, cum32, crow, ctok, cscore, ndev, total;
};
static BuildLayout build_layout(const sd_build_shape* s) {
  BuildLayout L;
  sd_expand_shape es{s->T, s->V, s->logit_dtype};
  const int kc = s->T - 1 + kBuildMargin;
  const size_t e = expand_ws(&es, kc, &L.exp_off, &L.exp_hist, &L.exp_cnt, &L.exp_keys);
  L.rmax = align_up(e, 256);
  L.rlse = align_up(L.rmax + (size_t)s->T * 8, 256);
  L.cum32 = align_up(L.rlse + (size_t)s->T * 8, 256);
  L.crow = align_up(L.cum32 + (size_t)s->T * 4, 256);
  L.ctok = align_up(L.crow + (size_t)kc * 4, 256);
  L.cscore = align_up(L.ctok + (size_t)kc * 4, 256);
  L.ndev = align_up(L.cscore + (size_t)kc * 4, 256);
  L.total = L.ndev + 256;
  return L;
}

static sd_status check_expand(const sd_expand_shape* s, int32_t k) {
  if (!s) return SD_INVALID_ARG;
  if (s->E < 1 || s->V < 1) return SD_BAD_SHAPE;
  if (s->logit_dtype != SD_F32 && s->logit_dtype != SD_BF16) return SD_BAD_DTYPE;
  if ((long long)s->E * s->V >= 0xFFFFFFFFll || s->E > 65535) return SD_UNSUPPORTED;
  if (k < 1 || (long long)k > (long long)s->E * s->V) return SD_INVALID_ARG;
  if (k > kMaxExpandK) return SD_UNSUPPORTED;
  return SD_OK;
}

static size_t topk_ws(const sd_shape* s, size_t* means_off, size_t* scores_off) {
  const size_t nbmax = (size_t)s->max_blocks;
  const size_t mo = kWsHeader;
  const size_t so = align_up(mo + (size_t)s->B * nbmax * s->Hkv * s->D * 4, 256);
  if (means_off) *means_off = mo;
  if (scores_off) *scores_off = so;
  return align_up(so + (size_t)s->B * s->T * s->Hq * nbmax * 4, 256);
}

// Acceptance scratch: the status header, plus per-sequence barrier state when
// a sequence is split over several workgroups.
static size_t accept_ws(const sd_accept_shape* s) {
  const int P = accept_wgs(s->B, s->V);
  return kWsHeader + (P > 1 ? (size_t)s->B * kAccSeqBytes : 0);
}

static sd_status hip_status(hipError_t e) { return e == hipSuccess ? SD_OK : SD_HIP_ERROR; }

}  // namespace sdtree

using namespace sdtree;

extern "C" {

const char* sd_status_str(int32_t code) {
  // (an int, not the enum: any value a caller passes is a defined input)
  switch (code) {
    case SD_OK: return "ok";
    case SD_INVALID_ARG: return "invalid argument";
    case SD_BAD_SHAPE: return "bad shape";
    case SD_BAD_DTYPE: return "bad dtype";
    case SD_UNSUPPORTED: return "unsupported";
    case SD_CAPACITY: return "workspace too small";
    case SD_HIP_ERROR: return "HIP error";
    case SD_DEVICE_DATA_ERROR: return "device data error";
  }
  return "unknown status";
}

size_t sd_workspace_bytes(int32_t call_id, const void* shape, int32_t extra) {
  if (!shape) return 0;
  if (call_id == SD_CALL_ATTN) {
    const sd_shape* s = static_cast<const sd_shape*>(shape);
    if (check_shape(s) != SD_OK) return 0;
    if (extra < 0 || extra > kMaxKsel) return 0;
    return plan_attn(s, extra, extra > 0).total;
  }
  if (call_id == SD_CALL_ACCEPT) {
    const sd_accept_shape* s = static_cast<const sd_accept_shape*>(shape);
    if (s->B < 1 || s->T < 1 || s->V < 1) return 0;
    return accept_ws(s);
  }
  if (call_id == SD_CALL_COMMIT) {
    const sd_shape* s = static_cast<const sd_shape*>(shape);
    return check_shape(s) == SD_OK ? commit_ws(s) : 0;
  }
  if (call_id == SD_CALL_EXPAND) {
    const sd_expand_shape* s = static_cast<const sd_expand_shape*>(shape);
    return check_expand(s, extra) == SD_OK ? expand_ws(s, extra, nullptr, nullptr, nullptr, nullptr) : 0;
  }
  if (call_id == SD_CALL_BUILD) {
    const sd_build_shape* s = static_cast<const sd_build_shape*>(shape);
    return check_build(s) == SD_OK ? build_layout(s).total : 0;
  }
  if (call_id == SD_CALL_BLOCK_SUMS) {
    const sd_shape* s = static_cast<const sd_shape*>(shape);
    return check_shape(s) == SD_OK ? kWsHeader : 0;
  }
  if (call_id == SD_CALL_TOPK) {
    const sd_shape* s = static_cast<const sd_shape*>(shape);
    if (check_shape(s) != SD_OK || extra < 1) return 0;
    return topk_ws(s, nullptr, nullptr);
  }
  return 0;
}

// Timing events for this host thread's next attention call.
static thread_local CallEvents t_attn_events;

sd_status sd_attn_timing_events(void* start_event, void* stop_event) {
  t_attn_events.start = static_cast<hipEvent_t>(start_event);
  t_attn_events.stop = static_cast<hipEvent_t>(stop_event);
  return SD_OK;
}

sd_status sd_tree_verify_attn(const sd_shape* shape, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table,
                              const int32_t* ctx_lens, const int32_t* tree_parent,
                              const int32_t* sel_blocks, int32_t k_sel, void* out, void* ws,
                              size_t ws_bytes, void* stream) {
  const CallEvents ev = t_attn_events;
  t_attn_events = CallEvents{};
  sd_status st = check_shape(shape);
  if (st != SD_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !ctx_lens || !tree_parent || !out || !ws)
    return SD_INVALID_ARG;
  const bool sparse = sel_blocks != nullptr;
  if (sparse && k_sel < 1) return SD_INVALID_ARG;
  if (sparse && k_sel > kMaxKsel) return SD_UNSUPPORTED;
  if (!sparse && k_sel != 0) return SD_INVALID_ARG;
  const sd_shape& s = *shape;
  const AttnPlan p = plan_attn(&s, k_sel, sparse);
  if (ws_bytes < p.total) return SD_CAPACITY;
  if (p.variant == 1 && p.lds_bytes > kLdsLimit) return SD_UNSUPPORTED;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint32_t* status = reinterpret_cast<uint32_t*>(w);
  uint64_t* anc = reinterpret_cast<uint64_t*>(w + p.anc_off);
  if (p.variant == 0) {
    // the per-row kernel reads precomputed ancestor masks; the MFMA kernel
    // walks the tree itself
    hipError_t e = launch_anc_mask(tree_parent, s.T, p.W64, p.T_tree, anc, status, hs, ev.start);
    if (e != hipSuccess) return SD_HIP_ERROR;
  }

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k_pages; a.v = v_pages; a.table = block_table; a.ctx = ctx_lens;
  a.parent = tree_parent; a.anc = anc; a.sel = sel_blocks; a.ksel = k_sel; a.out = out;
  a.part_o = reinterpret_cast<float*>(w + p.part_o_off);
  a.part_ml = reinterpret_cast<float*>(w + p.part_ml_off);
  a.status = status;
  a.B = s.B; a.T = s.T; a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.Hq / s.Hkv; a.M = s.T * a.G;
  a.D = s.D; a.bs = s.bs; a.max_blocks = s.max_blocks; a.num_blocks = s.num_blocks;
  a.tree_stride = s.tree_stride;
  const float scale = s.scale > 0.f ? s.scale : 1.f / sqrtf((float)s.D);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.n_qtiles = p.n_qtiles; a.n_splits = p.n_splits; a.tps = p.tps; a.W64 = p.W64; a.u_max = p.u_max;
  a.bs_shift = __builtin_ctz((unsigned)s.bs);
  a.ct_max = p.ct_max; a.tt_max = p.tt_max;
  a.anc_lds_words = p.anc_lds_words;
  a.zeros = w + kWsZeros;
  if (p.variant == 0) return hip_status(launch_attn_valu(a, s.dtype == SD_F32, hs, CallEvents{nullptr, ev.stop}));
  return hip_status(launch_attn_mfma(a, p, hs, ev));
}

// Checks the arguments of an acceptance call and fills its kernel arguments
// (no commit, no scratch: the callers place the status word and the exchange
// slots).
static sd_status accept_args(const sd_accept_shape* shape, const void* target_logits,
                             const float* draft_probs, const int32_t* tree_parent,
                             const int32_t* tree_token, const float* uniforms, float temperature,
                             int32_t* path, int32_t* path_len, int32_t* bonus, AcceptArgs* out) {
  if (!shape) return SD_INVALID_ARG;
  const sd_accept_shape& s = *shape;
  if (s.B < 1 || s.T < 1 || s.V < 1) return SD_BAD_SHAPE;
  if (s.tree_stride != 0 && s.tree_stride != s.T) return SD_BAD_SHAPE;
  if (s.logit_dtype != SD_F32 && s.logit_dtype != SD_BF16) return SD_BAD_DTYPE;
  if (s.T > kMaxTreeNodes) return SD_UNSUPPORTED;
  if (!(temperature >= 0.f) || isinf(temperature)) return SD_INVALID_ARG;
  if (!target_logits || !tree_parent || !tree_token || !path || !path_len || !bonus)
    return SD_INVALID_ARG;
  if (temperature > 0.f && !uniforms) return SD_INVALID_ARG;
  AcceptArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = target_logits;
  a.logits_f32 = s.logit_dtype == SD_F32;
  a.draft = temperature > 0.f ? draft_probs : nullptr;
  a.parent = tree_parent; a.token = tree_token; a.unif = uniforms; a.tau = temperature;
  a.B = s.B; a.T = s.T; a.V = s.V; a.tree_stride = s.tree_stride;
  a.path = path; a.path_len = path_len; a.bonus = bonus;
  a.P = accept_wgs(s.B, s.V);
  a.SL = (((s.V + a.P - 1) / a.P) + 7) / 8 * 8;
  a.NC = (a.SL + 2047) / 2048;
  *out = a;
  return SD_OK;
}

// The status word and exchange slots of a call with a caller workspace.
static sd_status accept_ws_args(const sd_accept_shape* shape, void* ws, size_t ws_bytes,
                                AcceptArgs* a) {
  if (!ws) return SD_INVALID_ARG;
  if (ws_bytes < accept_ws(shape)) return SD_CAPACITY;
  a->status = static_cast<uint32_t*>(ws);
  a->sync = static_cast<unsigned char*>(ws) + kWsHeader;
  return SD_OK;
}

// The commit half of an acceptance call that also commits its paths.
static sd_status accept_commit_args(const sd_accept_shape* shape, const sd_shape* kv_shape,
                                    void* k_pages, void* v_pages, const int32_t* block_table,
                                    int32_t* ctx_lens, float* block_sums, AcceptArgs* a) {
  if (!shape || !kv_shape) return SD_INVALID_ARG;
  const sd_status st = check_shape(kv_shape);
  if (st != SD_OK) return st;
  if (kv_shape->B != shape->B || kv_shape->T != shape->T) return SD_BAD_SHAPE;
  if (!k_pages || !v_pages || !block_table || !ctx_lens) return SD_INVALID_ARG;
  a->ck = k_pages; a->cv = v_pages; a->ctable = block_table; a->cctx = ctx_lens;
  a->csums = block_sums;
  a->cHkv = kv_shape->Hkv; a->cD = kv_shape->D; a->cbs = kv_shape->bs;
  a->cmax_blocks = kv_shape->max_blocks; a->cnum_blocks = kv_shape->num_blocks;
  a->cesize = kv_shape->dtype == SD_F32 ? 4 : 2;
  return SD_OK;
}

sd_status sd_accept(const sd_accept_shape* shape, const void* target_logits,
                    const float* draft_probs, const int32_t* tree_parent,
                    const int32_t* tree_token, const float* uniforms, float temperature,
                    int32_t* path, int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes,
                    void* stream) {
  AcceptArgs a;
  sd_status st = accept_args(shape, target_logits, draft_probs, tree_parent, tree_token,
                             uniforms, temperature, path, path_len, bonus, &a);
  if (st != SD_OK) return st;
  st = accept_ws_args(shape, ws, ws_bytes, &a);
  if (st != SD_OK) return st;
  return hip_status(launch_accept(a, static_cast<hipStream_t>(stream)));
}

sd_status sd_accept_commit(const sd_accept_shape* shape, const sd_shape* kv_shape,
                           const void* target_logits, const float* draft_probs,
                           const int32_t* tree_parent, const int32_t* tree_token,
                           const float* uniforms, float temperature, int32_t* path,
                           int32_t* path_len, int32_t* bonus, void* k_pages, void* v_pages,
                           const int32_t* block_table, int32_t* ctx_lens, float* block_sums,
                           void* ws, size_t ws_bytes, void* stream) {
  AcceptArgs a;
  sd_status st = accept_args(shape, target_logits, draft_probs, tree_parent, tree_token, uniforms,
                             temperature, path, path_len, bonus, &a);
  if (st != SD_OK) return st;
  st = accept_commit_args(shape, kv_shape, k_pages, v_pages, block_table, ctx_lens, block_sums, &a);
  if (st != SD_OK) return st;
  st = accept_ws_args(shape, ws, ws_bytes, &a);
  if (st != SD_OK) return st;
  return hip_status(launch_accept(a, static_cast<hipStream_t>(stream)));
}

sd_status sd_accept_commit_noalloc(const sd_accept_shape* shape, const sd_shape* kv_shape,
                                   const void* target_logits, const float* draft_probs,
                                   const int32_t* tree_parent, const int32_t* tree_token,
                                   const float* uniforms, float temperature, int32_t* path,
                                   int32_t* path_len, int32_t* bonus, void* k_pages,
                                   void* v_pages, const int32_t* block_table, int32_t* ctx_lens,
                                   float* block_sums, uint32_t* status, void* stream) {
  AcceptArgs a;
  sd_status st = accept_args(shape, target_logits, draft_probs, tree_parent, tree_token, uniforms,
                             temperature, path, path_len, bonus, &a);
  if (st != SD_OK) return st;
  st = accept_commit_args(shape, kv_shape, k_pages, v_pages, block_table, ctx_lens, block_sums, &a);
  if (st != SD_OK) return st;
  if (!status) return SD_INVALID_ARG;
  // the library's exchange slots hold kNoAllocMaxSeqs sequences
  if (a.P > 1 && a.B > kNoAllocMaxSeqs) return SD_CAPACITY;
  a.status = status;
  return hip_status(launch_accept_noalloc(a, static_cast<hipStream_t>(stream)));
}

sd_status sd_kv_commit(const sd_shape* shape, void* k_pages, void* v_pages,
                       const int32_t* block_table, int32_t* ctx_lens, float* block_sums,
                       const int32_t* path, const int32_t* path_len, void* ws, size_t ws_bytes,
                       void* stream) {
  sd_status st = check_shape(shape);
  if (st != SD_OK) return st;
  if (!k_pages || !v_pages || !block_table || !ctx_lens || !path || !path_len || !ws)
    return SD_INVALID_ARG;
  if (ws_bytes < commit_ws(shape)) return SD_CAPACITY;
  CommitArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k_pages; a.v = v_pages; a.table = block_table; a.ctx = ctx_lens; a.path = path;
  a.path_len = path_len; a.sums = block_sums;
  a.B = shape->B; a.T = shape->T; a.Hkv = shape->Hkv; a.D = shape->D; a.bs = shape->bs;
  a.max_blocks = shape->max_blocks; a.num_blocks = shape->num_blocks;
  a.esize = shape->dtype == SD_F32 ? 4 : 2;
  a.status = static_cast<uint32_t*>(ws);
  a.counters = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(ws) + kWsHeader);
  return hip_status(launch_commit(a, static_cast<hipStream_t>(stream)));
}

static TopkArgs topk_args(const sd_shape* shape, const int32_t* block_table, const int32_t* ctx_lens,
                          void* ws) {
  TopkArgs a;
  memset(&a, 0, sizeof(a));
  a.table = block_table; a.ctx = ctx_lens;
  a.status = static_cast<uint32_t*>(ws);
  a.B = shape->B; a.T = shape->T; a.Hq = shape->Hq; a.Hkv = shape->Hkv;
  a.G = shape->Hq / shape->Hkv; a.D = shape->D; a.bs = shape->bs;
  a.max_blocks = shape->max_blocks; a.num_blocks = shape->num_blocks;
  a.nbmax = shape->max_blocks;
  return a;
}

// Top-k from K (block_sums == nullptr) or from kept block sums, per query
// row or shared by each KV group's rows.
static sd_status topk_common(const sd_shape* shape, const void* q, const void* k_pages,
                             const float* block_sums, const int32_t* block_table,
                             const int32_t* ctx_lens, int32_t k, int32_t* sel_blocks, void* ws,
                             size_t ws_bytes, void* stream, bool shared = false) {
  sd_status st = check_shape(shape);
  if (st != SD_OK) return st;
  if (!q || (!k_pages && !block_sums) || !block_table || !ctx_lens || !sel_blocks || !ws)
    return SD_INVALID_ARG;
  if (k < 1) return SD_INVALID_ARG;
  size_t mo, so;
  const size_t need = topk_ws(shape, &mo, &so);
  if (ws_bytes < need) return SD_CAPACITY;
  unsigned char* w = static_cast<unsigned char*>(ws);
  TopkArgs a = topk_args(shape, block_table, ctx_lens, ws);
  a.q = q; a.k = k_pages; a.sel = sel_blocks; a.topk = k;
  a.sums = const_cast<float*>(block_sums);
  a.means = reinterpret_cast<float*>(w + mo);
  a.scores = reinterpret_cast<float*>(w + so);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool f32 = shape->dtype == SD_F32, cached = block_sums != nullptr;
  return hip_status(shared ? launch_topk_shared(a, f32, cached, hs) : launch_topk(a, f32, cached, hs));
}

sd_status sd_topk_blocks(const sd_shape* shape, const void* q, const void* k_pages,
                         const int32_t* block_table, const int32_t* ctx_lens, int32_t k,
                         int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream) {
  if (!k_pages) return SD_INVALID_ARG;
  return topk_common(shape, q, k_pages, nullptr, block_table, ctx_lens, k, sel_blocks, ws, ws_bytes,
                     stream);
}

sd_status sd_topk_blocks_cached(const sd_shape* shape, const void* q, const float* block_sums,
                                const int32_t* block_table, const int32_t* ctx_lens, int32_t k,
                                int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream) {
  if (!block_sums) return SD_INVALID_ARG;
  return topk_common(shape, q, nullptr, block_sums, block_table, ctx_lens, k, sel_blocks, ws,
                     ws_bytes, stream);
}

sd_status sd_topk_blocks_shared(const sd_shape* shape, const void* q, const void* k_pages,
                                const float* block_sums, const int32_t* block_table,
                                const int32_t* ctx_lens, int32_t k, int32_t* sel_blocks, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!k_pages && !block_sums) return SD_INVALID_ARG;
  return topk_common(shape, q, block_sums ? nullptr : k_pages, block_sums, block_table, ctx_lens, k,
                     sel_blocks, ws, ws_bytes, stream, true);
}

sd_status sd_block_sums(const sd_shape* shape, const void* k_pages, const int32_t* block_table,
                        const int32_t* ctx_lens, float* block_sums, void* ws, size_t ws_bytes,
                        void* stream) {
  sd_status st = check_shape(shape);
  if (st != SD_OK) return st;
  if (!k_pages || !block_table || !ctx_lens || !block_sums || !ws) return SD_INVALID_ARG;
  if (ws_bytes < kWsHeader) return SD_CAPACITY;
  TopkArgs a = topk_args(shape, block_table, ctx_lens, ws);
  a.k = k_pages; a.sums = block_sums;
  return hip_status(launch_block_sums(a, shape->dtype == SD_F32, static_cast<hipStream_t>(stream)));
}

sd_status sd_block_sums_append(const sd_shape* shape, const void* k_pages,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               const int32_t* n_new, float* block_sums, void* ws, size_t ws_bytes,
                               void* stream) {
  sd_status st = check_shape(shape);
  if (st != SD_OK) return st;
  if (!k_pages || !block_table || !ctx_lens || !n_new || !block_sums || !ws) return SD_INVALID_ARG;
  if (ws_bytes < kWsHeader) return SD_CAPACITY;
  TopkArgs a = topk_args(shape, block_table, ctx_lens, ws);
  a.k = k_pages; a.sums = block_sums;
  return hip_status(launch_block_sums_append(a, n_new, shape->dtype == SD_F32,
                                             static_cast<hipStream_t>(stream)));
}

sd_status sd_tree_expand(const sd_expand_shape* shape, const void* draft_logits,
                         const float* cum_logp, float temperature, int32_t k, int32_t* out_row,
                         int32_t* out_token, float* out_score, void* ws, size_t ws_bytes,
                         void* stream) {
  const sd_status st = check_expand(shape, k);
  if (st != SD_OK) return st;
  if (!(temperature > 0.f) || isinf(temperature)) return SD_INVALID_ARG;
  if (!draft_logits || !cum_logp || !out_row || !out_token || !out_score || !ws) return SD_INVALID_ARG;
  size_t o, h, c, kk;
  if (ws_bytes < expand_ws(shape, k, &o, &h, &c, &kk)) return SD_CAPACITY;
  unsigned char* w = static_cast<unsigned char*>(ws);
  ExpandArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = draft_logits; a.cum = cum_logp; a.inv_tau = 1.f / temperature;
  a.E = shape->E; a.V = shape->V; a.k = k;
  a.off = reinterpret_cast<float*>(w + o);
  a.hist = reinterpret_cast<uint32_t*>(w + h);
  a.count = reinterpret_cast<uint32_t*>(w + c);
  a.keys = reinterpret_cast<unsigned long long*>(w + kk);
  a.out_row = out_row; a.out_token = out_token; a.out_score = out_score;
  return hip_status(launch_expand(a, shape->logit_dtype == SD_F32, static_cast<hipStream_t>(stream)));
}

sd_status sd_tree_build(const sd_build_shape* shape, const void* draft_logits, float temperature,
                        int32_t root_token, int32_t* parent, int32_t* token, double* cum_logp,
                        int32_t* rounds, void* ws, size_t ws_bytes, void* stream) {
  const sd_status st = check_build(shape);
  if (st != SD_OK) return st;
  if (!(temperature > 0.f) || isinf(temperature)) return SD_INVALID_ARG;
  if (root_token < 0 || root_token >= shape->V) return SD_INVALID_ARG;
  if (!draft_logits || !parent || !token || !cum_logp || !ws) return SD_INVALID_ARG;
  const BuildLayout L = build_layout(shape);
  if (ws_bytes < L.total) return SD_CAPACITY;
  unsigned char* w = static_cast<unsigned char*>(ws);
  BuildArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = draft_logits; a.T = shape->T; a.V = shape->V; a.tau = temperature;
  a.root_token = root_token; a.margin = kBuildMargin;
  a.parent = parent; a.token = token; a.cum = cum_logp;
  a.cum32 = reinterpret_cast<float*>(w + L.cum32);
  a.rmax = reinterpret_cast<double*>(w + L.rmax);
  a.rlse = reinterpret_cast<double*>(w + L.rlse);
  a.cand_row = reinterpret_cast<int32_t*>(w + L.crow);
  a.cand_token = reinterpret_cast<int32_t*>(w + L.ctok);
  a.n_dev = reinterpret_cast<int*>(w + L.ndev);
  a.status = reinterpret_cast<uint32_t*>(w);
  ExpandArgs ex;
  memset(&ex, 0, sizeof(ex));
  ex.logits = draft_logits; ex.cum = a.cum32; ex.inv_tau = 1.f / temperature;
  ex.V = shape->V;
  ex.off = reinterpret_cast<float*>(w + L.exp_off);
  ex.hist = reinterpret_cast<uint32_t*>(w + L.exp_hist);
  ex.count = reinterpret_cast<uint32_t*>(w + L.exp_cnt);
  ex.keys = reinterpret_cast<unsigned long long*>(w + L.exp_keys);
  ex.out_row = a.cand_row; ex.out_token = a.cand_token;
  ex.out_score = reinterpret_cast<float*>(w + L.cscore);
  int r = 0;
  const hipError_t e = run_tree_build(a, ex, shape->logit_dtype == SD_F32, static_cast<hipStream_t>(stream), &r);
  if (rounds) *rounds = r;
  return hip_status(e);
}

sd_status sd_device_status(void* ws, void* stream, uint32_t* bits) {
  if (!ws) return SD_INVALID_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(hs) != hipSuccess) return SD_HIP_ERROR;
  uint32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SD_HIP_ERROR;
  if (v) {
    const uint32_t zero = 0;
    if (hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return SD_HIP_ERROR;
  }
  if (bits) *bits = v;
  return v ? SD_DEVICE_DATA_ERROR : SD_OK;
}

}  // extern "C"
