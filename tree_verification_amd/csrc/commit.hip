// Commit the accepted root path into the paged KV cache, for gfx950.
//
// After acceptance the accepted nodes become committed context in path order:
// position ctx_b + j takes the K/V held at ctx_b + path[j], then ctx_b grows by
// the path length.  One workgroup per sequence; each thread owns one 16-byte
// chunk of a K row or one V element column of one KV head and copies it for
// j = 0, 1, ... in order.  Because the path is increasing with path[j] >= j,
// a source slot is always read before any write can reach it, so the copy is
// safe in place.
#include "common.h"

namespace sdtree {

__global__ void __launch_bounds__(256) commit_kernel(CommitArgs a) {
  __shared__ int s_ok, s_ctx, s_len;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* path = a.path + (size_t)b * a.T;
  const int32_t* table = a.table + (size_t)b * a.max_blocks;
  if (tid == 0) {
    const int ctx = a.ctx[b], L = a.path_len[b];
    uint32_t err = 0;
    if (ctx < 0 || (long long)ctx + a.T > (long long)a.max_blocks * a.bs) err |= SD_ERR_CAPACITY;
    if (L < 0 || L > a.T) err |= SD_ERR_PARENT;
    if (!err && L > 0) {
      if (path[0] != 0) err |= SD_ERR_PARENT;
      for (int j = 1; j < L; ++j)
        if (path[j] <= path[j - 1] || path[j] >= a.T) err |= SD_ERR_PARENT;
      const int lo = ctx / a.bs, hi = (ctx + a.T - 1) / a.bs;
      for (int n = lo; n <= hi; ++n)
        if (table[n] < 0 || table[n] >= a.num_blocks) err |= SD_ERR_BLOCK;
    }
    if (err) set_status(a.status, err);
    s_ok = !err;
    s_ctx = ctx;
    s_len = L;
  }
  __syncthreads();
  if (!s_ok) return;
  const int ctx = s_ctx, L = s_len;
  const int kchunks = a.D * a.esize / 16;             // 16-byte chunks per K row
  const int items = a.Hkv * (kchunks + a.D);          // K chunks, then V columns
  unsigned char* K = reinterpret_cast<unsigned char*>(a.k);
  unsigned char* V = reinterpret_cast<unsigned char*>(a.v);
  for (int it = tid; it < items; it += blockDim.x) {
    const int g = it / (kchunks + a.D);
    const int r = it % (kchunks + a.D);
    for (int j = 0; j < L; ++j) {
      const int src = ctx + path[j], dst = ctx + j;
      if (src == dst) continue;
      const size_t sb = (size_t)table[src / a.bs], so = src % a.bs;
      const size_t db = (size_t)table[dst / a.bs], dof = dst % a.bs;
      if (r < kchunks) {
        const size_t row = (size_t)a.D * a.esize;
        const uint4 x = *reinterpret_cast<const uint4*>(K + ((sb * a.Hkv + g) * a.bs + so) * row + r * 16);
        *reinterpret_cast<uint4*>(K + ((db * a.Hkv + g) * a.bs + dof) * row + r * 16) = x;
      } else {
        const int d = r - kchunks;
        const size_t s_off = (((sb * a.Hkv + g) * a.D + d) * a.bs + so) * a.esize;
        const size_t d_off = (((db * a.Hkv + g) * a.D + d) * a.bs + dof) * a.esize;
        if (a.esize == 2)
          *reinterpret_cast<uint16_t*>(V + d_off) = *reinterpret_cast<const uint16_t*>(V + s_off);
        else
          *reinterpret_cast<uint32_t*>(V + d_off) = *reinterpret_cast<const uint32_t*>(V + s_off);
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.ctx[b] = ctx + L;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdtree
