// Commit the accepted root path into the paged KV cache, for gfx950.
//
// After acceptance the accepted nodes become committed context in path order:
// position ctx_b + j takes the K/V held at ctx_b + path[j], then ctx_b grows by
// the path length.  One workgroup per (sequence, KV head) copies the path in
// groups of JG entries: every thread first loads its share of the group (16-byte
// chunks of the K and V rows) into registers, the workgroup synchronises, then
// the stores are issued.  The path is increasing with path[j] >= j, so a
// group's destinations (positions < ctx + j0 + JG) never overlap the sources of
// a later group (positions >= ctx + j0 + JG): the copy is safe in place.
// With kept block key sums, the workgroup then extends its head's sums over
// the committed positions (the same sequential float32 sums as
// sd_block_sums_append).  The sequence's last workgroup to finish (a counter
// per sequence in the workspace) writes the new context length; every
// workgroup has read the old one before it counts itself.
#include "common.h"

namespace sdtree {

constexpr int kCommitThreads = 256;
constexpr int kKRegs = 4;        // 16-byte chunks of K (and of V) per thread per group
constexpr int kMaxCommitBlocks = kMaxCommitT / 8 + 2;  // blocks of slots [ctx, ctx + T), bs >= 8

__global__ void __launch_bounds__(kCommitThreads) commit_kernel(CommitArgs a) {
  __shared__ int s_err;
  __shared__ int s_path[kMaxCommitT];
  __shared__ int s_blk[kMaxCommitBlocks];
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv, tid = threadIdx.x;
  const int32_t* path = a.path + (size_t)b * a.T;
  const int32_t* table = a.table + (size_t)b * a.max_blocks;
  // Validate with every thread: the path (staged in LDS) starts at the root
  // and increases within [0, T); the blocks of slots [ctx, ctx + T) (staged in
  // LDS) are valid.
  const int ctx = a.ctx[b], L = a.path_len[b];
  if (tid == 0) s_err = 0;
  uint32_t err = 0;
  if (ctx < 0 || (long long)ctx + a.T > (long long)a.max_blocks * a.bs) err |= SD_ERR_CAPACITY;
  if (L < 0 || L > a.T) err |= SD_ERR_PARENT;
  const bool shape_ok = err == 0;
  const int lo = shape_ok ? ctx / a.bs : 0;
  const int nblk = shape_ok ? (ctx + a.T - 1) / a.bs - lo + 1 : 0;
  // the path and the tree slots' block ids fit their LDS copies
  SD_DCHECK(a.T <= kMaxCommitT && nblk <= kMaxCommitBlocks, a.status);
  if (shape_ok) {
    for (int j = tid; j < L; j += kCommitThreads) s_path[j] = path[j];
    for (int n = tid; n < nblk; n += kCommitThreads) {
      const int blk = table[lo + n];
      if (blk < 0 || blk >= a.num_blocks) err |= SD_ERR_BLOCK;
      s_blk[n] = blk;
    }
  }
  __syncthreads();
  if (shape_ok)
    for (int j = tid; j < L; j += kCommitThreads) {
      const int pj = s_path[j];
      if (j == 0 ? pj != 0 : (pj <= s_path[j - 1] || pj >= a.T)) err |= SD_ERR_PARENT;
    }
  if (err) atomicOr(&s_err, (int)err);
  __syncthreads();
  if (s_err) {
    if (g == 0 && tid == 0) set_status(a.status, (uint32_t)s_err);
    return;
  }

  // Threads own a fixed 16-byte column chunk (kch per row) of the K and V
  // rows of an entry.
  const int kch = a.D * a.esize / 16;                 // 16-byte chunks per row (power of 2)
  const int rowb = a.D * a.esize;
  unsigned char* K = reinterpret_cast<unsigned char*>(a.k);
  unsigned char* V = reinterpret_cast<unsigned char*>(a.v);
  const int kstep = kCommitThreads / kch;
  const int kcol = tid % kch, ku0 = tid / kch;
  const int JG = kKRegs * kstep;
  const long long blk_bytes = (long long)a.Hkv * a.bs * rowb;
  const long long head = (long long)g * a.bs * rowb;
  // byte offset of slot p's row (head g), K and V alike
  auto row_at = [&](int p) -> long long {
    return (long long)s_blk[p / a.bs - lo] * blk_bytes + head + (long long)(p % a.bs) * rowb;
  };
  const long long c_off = (long long)kcol * 16;
  for (int j0 = 0; j0 < L; j0 += JG) {
    const int nj = min(JG, L - j0);
    uint4 kr[kKRegs], vr[kKRegs];
#pragma unroll
    for (int r = 0; r < kKRegs; ++r) {
      const int jj = ku0 + r * kstep;
      kr[r] = make_uint4(0, 0, 0, 0);
      vr[r] = make_uint4(0, 0, 0, 0);
      if (jj < nj && s_path[j0 + jj] != j0 + jj) {
        const long long src = row_at(ctx + s_path[j0 + jj]) + c_off;
        kr[r] = *reinterpret_cast<const uint4*>(K + src);
        vr[r] = *reinterpret_cast<const uint4*>(V + src);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kKRegs; ++r) {
      const int jj = ku0 + r * kstep;
      if (jj < nj && s_path[j0 + jj] != j0 + jj) {
        const long long dst = row_at(ctx + j0 + jj) + c_off;
        *reinterpret_cast<uint4*>(K + dst) = kr[r];
        *reinterpret_cast<uint4*>(V + dst) = vr[r];
      }
    }
    __syncthreads();
  }
  // With kept block key sums: extend this head's sums over the committed
  // positions [ctx, ctx + L) (the rows the workgroup just wrote are visible
  // to it after the copy's last barrier); the blocks are those validated
  // above.
  if (a.sums && (tid >> 6) == 0)
    extend_head_sums_rt(
        a.esize, a.D, a.bs, ctx, ctx + L, tid & 63,
        [&](int n) { return K + (long long)s_blk[n - lo] * blk_bytes + head; },
        [&](int n) { return a.sums + ((size_t)s_blk[n - lo] * a.Hkv + g) * a.D; });
  if (tid == 0) {
    const unsigned done = atomicAdd(a.counters + b, 1u);
    if (done == (unsigned)a.Hkv - 1) {
      a.ctx[b] = ctx + L;
      __hip_atomic_store(a.counters + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3((unsigned)a.B * a.Hkv), dim3(kCommitThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdtree
