/* Host-side checks of libsdtree under AddressSanitizer and
 * UndefinedBehaviorSanitizer: workspace sizing over a seeded sweep of shapes
 * (edge and extreme values of every field, for every call id and selection
 * width), status strings, and the argument checks of every entry point that
 * return before any HIP call.  Exits 0 when every call returned; a sanitizer
 * report aborts the run. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "sdtree.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  /* xorshift64* */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}

static const int32_t kVals[] = {INT_MIN, -7, -1, 0, 1, 2, 3, 5, 7, 8, 15, 16, 31, 32, 64, 100, 127, 128,
                                255, 256, 1000, 2047, 2048, 3841, 3842, 4096, 4097, 32000, 65536, 65537,
                                128256, 1 << 20, 1 << 27, 1 << 30, INT_MAX};
#define NV ((int)(sizeof(kVals) / sizeof(kVals[0])))
static int32_t pick(void) { return kVals[next_u32() % NV]; }

int main(void) {
  size_t sink = 0;
  for (int code = -2; code < 12; ++code) sink += sd_status_str(code) != NULL;
  for (int it = 0; it < 200000; ++it) {
    sd_shape s = {pick(), pick(), pick(), pick(), pick(), pick(), pick(), pick(),
                  (int32_t)(next_u32() % 3), 0, 0.0f};
    s.tree_stride = (next_u32() & 1) ? s.T : 0;
    const int32_t extra = pick();
    sink += sd_workspace_bytes(SD_CALL_ATTN, &s, extra);
    sink += sd_workspace_bytes(SD_CALL_ATTN, &s, 0);
    sink += sd_workspace_bytes(SD_CALL_TOPK, &s, extra);
    sink += sd_workspace_bytes(SD_CALL_COMMIT, &s, 0);
    sink += sd_workspace_bytes(SD_CALL_BLOCK_SUMS, &s, 0);
    sd_accept_shape as = {pick(), pick(), pick(), (int32_t)(next_u32() % 3), pick()};
    sink += sd_workspace_bytes(SD_CALL_ACCEPT, &as, 0);
    sd_expand_shape es = {pick(), pick(), (int32_t)(next_u32() % 3)};
    sink += sd_workspace_bytes(SD_CALL_EXPAND, &es, extra);
    sd_build_shape bs = {pick(), pick(), (int32_t)(next_u32() % 3)};
    sink += sd_workspace_bytes(SD_CALL_BUILD, &bs, 0);
    sink += sd_workspace_bytes(next_u32() % 12, &s, extra);
  }
  sink += sd_workspace_bytes(SD_CALL_ATTN, NULL, 0);
  /* shapes that pass the checks, so the planners' arithmetic runs: every
     field in its accepted range, up to its extremes */
  static const int32_t kD[] = {64, 128}, kBs[] = {8, 16, 64, 256, 1 << 12}, kG[] = {1, 2, 4, 8, 64};
  static const int32_t kHkv[] = {1, 2, 8, 64}, kK[] = {0, 1, 32, 64, 65, 256, 4096, 65536};
  for (int it = 0; it < 200000; ++it) {
    const int32_t Hkv = kHkv[next_u32() % 4], G = kG[next_u32() % 5];
    const int32_t T = 1 + (int32_t)(next_u32() % (it & 1 ? 4096 : 80));
    const int32_t bs = kBs[next_u32() % 5];
    const int32_t mb = 1 + (int32_t)(next_u32() % ((1u << 30) / (uint32_t)bs));
    int32_t B = 1 + (int32_t)(next_u32() % (it & 2 ? 4096 : 64));
    sd_shape s = {B, T, Hkv * G, Hkv, kD[next_u32() & 1], bs, mb, 1 + (int32_t)(next_u32() % (1u << 28)),
                  (int32_t)(next_u32() & 1), (next_u32() & 1) ? T : 0, 0.0f};
    const int32_t k = kK[next_u32() % 8];
    sink += sd_workspace_bytes(SD_CALL_ATTN, &s, k);
    sink += sd_workspace_bytes(SD_CALL_TOPK, &s, k);
    sink += sd_workspace_bytes(SD_CALL_COMMIT, &s, 0);
    sink += sd_workspace_bytes(SD_CALL_BLOCK_SUMS, &s, 0);
    sd_accept_shape as = {B, T, 1 + (int32_t)(next_u32() % 300000), (int32_t)(next_u32() % 2), T};
    sink += sd_workspace_bytes(SD_CALL_ACCEPT, &as, 0);
    sd_expand_shape es = {T, as.V, (int32_t)(next_u32() % 2)};
    sink += sd_workspace_bytes(SD_CALL_EXPAND, &es, k);
    sd_build_shape bsh = {T, as.V, (int32_t)(next_u32() % 2)};
    sink += sd_workspace_bytes(SD_CALL_BUILD, &bsh, 0);
  }

  /* argument checks (null or out-of-range arguments: every call returns an
     error code before touching a device) */
  void* F = (void*)0x1000;
  sd_shape good = {16, 64, 32, 8, 128, 16, 260, 4160, SD_BF16, 64, 0.0f};
  int bad = 0;
  bad |= sd_tree_verify_attn(&good, NULL, F, F, F, F, F, NULL, 0, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_tree_verify_attn(NULL, F, F, F, F, F, F, NULL, 0, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_tree_verify_attn(&good, F, F, F, F, F, F, F, 0, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_tree_verify_attn(&good, F, F, F, F, F, F, F, 70000, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_tree_verify_attn(&good, F, F, F, F, F, F, NULL, 0, F, F, 0, NULL) == SD_OK;
  sd_accept_shape ag = {2, 8, 100, 1, 8};
  bad |= sd_accept(&ag, F, F, F, F, NULL, 0.8f, F, F, F, F, 256, NULL) == SD_OK;
  bad |= sd_accept(NULL, F, F, F, F, F, 0.8f, F, F, F, F, 256, NULL) == SD_OK;
  bad |= sd_accept(&ag, F, F, F, F, F, -1.0f, F, F, F, F, 256, NULL) == SD_OK;
  sd_shape kv = {2, 8, 8, 8, 128, 16, 260, 4160, SD_BF16, 8, 0.0f};
  bad |= sd_accept_commit(&ag, NULL, F, F, F, F, F, 0.8f, F, F, F, F, F, F, F, NULL, F, 256, NULL) == SD_OK;
  bad |= sd_accept_commit(&ag, &kv, F, F, F, F, F, 0.8f, F, F, F, NULL, F, F, F, NULL, F, 256, NULL) == SD_OK;
  bad |= sd_accept_commit_noalloc(&ag, &kv, F, F, F, F, F, 0.8f, F, F, F, F, F, F, F, NULL, NULL, NULL) ==
         SD_OK;
  bad |= sd_kv_commit(&good, F, F, F, F, NULL, F, F, NULL, 256, NULL) == SD_OK;
  bad |= sd_topk_blocks(&good, F, F, F, F, 0, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_topk_blocks_cached(&good, F, NULL, F, F, 4, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_topk_blocks_shared(&good, F, NULL, NULL, F, F, 4, F, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_block_sums(&good, F, F, F, NULL, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_block_sums_append(&good, F, F, F, NULL, F, F, 1u << 30, NULL) == SD_OK;
  sd_expand_shape eg = {4, 100, SD_BF16};
  bad |= sd_tree_expand(&eg, F, F, 0.8f, 0, F, F, F, F, 1u << 20, NULL) == SD_OK;
  sd_build_shape bg = {64, 100, SD_F32};
  bad |= sd_tree_build(&bg, F, 0.0f, 0, F, F, F, NULL, F, 1u << 30, NULL) == SD_OK;
  bad |= sd_device_status(NULL, NULL, NULL) == SD_OK;
  printf("checked %zu\n", sink);
  return bad ? 2 : 0;
}
