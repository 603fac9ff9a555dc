// Commit the accepted root path into the paged KV cache, for gfx950.
//
// After acceptance the accepted nodes become committed context in path order:
// position ctx_b + j takes the K/V held at ctx_b + path[j], then ctx_b grows by
// the path length.  One workgroup per (sequence, KV head) copies the path in
// groups of JG entries: every thread first loads its share of the group (16-byte
// K chunks and V^T elements) into registers, the workgroup synchronises, then
// the stores are issued.  The path is increasing with path[j] >= j, so a
// group's destinations (positions < ctx + j0 + JG) never overlap the sources of
// a later group (positions >= ctx + j0 + JG): the copy is safe in place.
// The sequence's last workgroup to finish (a counter per sequence in the
// workspace) writes the new context length; every workgroup has read the old
// one before it counts itself.
#include "common.h"

namespace sdtree {

constexpr int kCommitThreads = 256;
constexpr int kKRegs = 4;        // 16-byte K chunks per thread per group
constexpr int kVRegs = 24;       // V^T elements per thread per group
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

  // Threads own fixed columns of an entry: a 16-byte K chunk (kch per row) or
  // one V^T element (D per column).
  const int kch = a.D * a.esize / 16;                 // 16-byte chunks per K row (power of 2)
  const int rowb = a.D * a.esize;
  unsigned char* K = reinterpret_cast<unsigned char*>(a.k);
  unsigned char* V = reinterpret_cast<unsigned char*>(a.v);
  const int kstep = kCommitThreads / kch, vstep = kCommitThreads / a.D;
  const int kcol = tid % kch, ku0 = tid / kch;
  const int vcol = tid % a.D, vu0 = tid / a.D;
  const int JG = min(kKRegs * kstep, kVRegs * vstep);
  const long long blk_bytes = (long long)a.Hkv * a.bs * rowb;
  const long long head_k = (long long)g * a.bs * rowb;
  const long long head_v = (long long)g * a.D * a.bs * a.esize;
  // byte offsets of slot p's K row and V^T column (head g)
  auto k_at = [&](int p) -> long long {
    return (long long)s_blk[p / a.bs - lo] * blk_bytes + head_k + (long long)(p % a.bs) * rowb;
  };
  auto v_at = [&](int p) -> long long {
    return (long long)s_blk[p / a.bs - lo] * blk_bytes + head_v + (long long)(p % a.bs) * a.esize;
  };
  const long long kc_off = (long long)kcol * 16;
  const long long vc_off = (long long)vcol * a.bs * a.esize;
  for (int j0 = 0; j0 < L; j0 += JG) {
    const int nj = min(JG, L - j0);
    uint4 kr[kKRegs];
    uint32_t vr[kVRegs];
#pragma unroll
    for (int r = 0; r < kKRegs; ++r) {
      const int jj = ku0 + r * kstep;
      kr[r] = make_uint4(0, 0, 0, 0);
      if (jj < nj && s_path[j0 + jj] != j0 + jj)
        kr[r] = *reinterpret_cast<const uint4*>(K + k_at(ctx + s_path[j0 + jj]) + kc_off);
    }
#pragma unroll
    for (int r = 0; r < kVRegs; ++r) {
      const int jj = vu0 + r * vstep;
      vr[r] = 0;
      if (jj < nj && s_path[j0 + jj] != j0 + jj) {
        const unsigned char* src = V + v_at(ctx + s_path[j0 + jj]) + vc_off;
        vr[r] = a.esize == 2 ? *reinterpret_cast<const uint16_t*>(src) : *reinterpret_cast<const uint32_t*>(src);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kKRegs; ++r) {
      const int jj = ku0 + r * kstep;
      if (jj < nj && s_path[j0 + jj] != j0 + jj)
        *reinterpret_cast<uint4*>(K + k_at(ctx + j0 + jj) + kc_off) = kr[r];
    }
#pragma unroll
    for (int r = 0; r < kVRegs; ++r) {
      const int jj = vu0 + r * vstep;
      if (jj < nj && s_path[j0 + jj] != j0 + jj) {
        unsigned char* dst = V + v_at(ctx + j0 + jj) + vc_off;
        if (a.esize == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)vr[r];
        else *reinterpret_cast<uint32_t*>(dst) = vr[r];
      }
    }
    __syncthreads();
  }
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
