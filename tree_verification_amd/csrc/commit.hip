// Commit the accepted root path into the paged KV cache, for gfx950.
//
// After acceptance the accepted nodes become committed context in path order:
// position ctx_b + j takes the K/V held at ctx_b + path[j], then ctx_b grows by
// the path length.  One workgroup per sequence copies the path in groups of
// JG entries: every thread first loads its share of the group (16-byte K
// chunks and V^T elements, all heads) into registers, the workgroup
// synchronises, then the stores are issued.  The path is increasing with
// path[j] >= j, so a group's destinations (positions < ctx + j0 + JG) never
// overlap the sources of a later group (positions >= ctx + j0 + JG): the copy
// is safe in place.  Shapes whose group does not fit the registers copy one
// entry at a time (source and destination of one entry never overlap).
#include "common.h"

namespace sdtree {

constexpr int kCommitThreads = 256;
constexpr int kKRegs = 4;        // 16-byte K chunks per thread per group
constexpr int kVRegs = 24;       // V^T elements per thread per group
constexpr int kCommitGroup = 16; // path entries per group
constexpr int kCommitUnits = 256; // (entry, KV head) units per group

__global__ void __launch_bounds__(kCommitThreads) commit_kernel(CommitArgs a) {
  __shared__ int s_ok, s_ctx, s_len;
  __shared__ int s_path[kMaxCommitT];
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
  for (int j = tid; j < L; j += kCommitThreads) s_path[j] = path[j];
  __syncthreads();

  // A unit is (path entry, KV head).  Threads own fixed columns of a unit: a
  // 16-byte K chunk (kch per row) or one V^T element (D per column); their
  // byte offsets live in LDS, so the copy loops do no index arithmetic.
  const int kch = a.D * a.esize / 16;                 // 16-byte chunks per K row (power of 2)
  const int rowb = a.D * a.esize;
  unsigned char* K = reinterpret_cast<unsigned char*>(a.k);
  unsigned char* V = reinterpret_cast<unsigned char*>(a.v);
  const int kstep = kCommitThreads / kch, vstep = kCommitThreads / a.D;
  const int kcol = tid % kch, ku0 = tid / kch;
  const int vcol = tid % a.D, vu0 = tid / a.D;
  int JG = min(kCommitUnits, min(kKRegs * kstep, kVRegs * vstep)) / a.Hkv;
  JG = min(JG, kCommitGroup);
  __shared__ long long s_ks[kCommitUnits], s_kd[kCommitUnits], s_vs[kCommitUnits], s_vd[kCommitUnits];
  const long long blk_bytes = (long long)a.Hkv * a.bs * rowb;
  const long long head_k = (long long)a.bs * rowb;
  const long long head_v = (long long)a.D * a.bs * a.esize;
  const long long kc_off = (long long)kcol * 16;
  const long long vc_off = (long long)vcol * a.bs * a.esize;
  // offsets of units [0, nj * Hkv) for path entries j0 .. j0 + nj - 1
  auto stage = [&](int j0, int nj) {
    for (int u = tid; u < nj * a.Hkv; u += kCommitThreads) {
      const int jj = u / a.Hkv, g = u % a.Hkv;
      const int src = ctx + s_path[j0 + jj], dst = ctx + j0 + jj;
      const long long sb = (long long)table[src / a.bs] * blk_bytes;
      const long long db = (long long)table[dst / a.bs] * blk_bytes;
      const bool same = s_path[j0 + jj] == j0 + jj;
      s_ks[u] = sb + g * head_k + (long long)(src % a.bs) * rowb;
      s_kd[u] = same ? -1 : db + g * head_k + (long long)(dst % a.bs) * rowb;
      s_vs[u] = sb + g * head_v + (long long)(src % a.bs) * a.esize;
      s_vd[u] = same ? -1 : db + g * head_v + (long long)(dst % a.bs) * a.esize;
    }
    __syncthreads();
  };

  if (JG >= 1) {
    for (int j0 = 0; j0 < L; j0 += JG) {
      const int nj = min(JG, L - j0);
      const int nu = nj * a.Hkv;
      stage(j0, nj);
      uint4 kr[kKRegs];
      uint32_t vr[kVRegs];
#pragma unroll
      for (int r = 0; r < kKRegs; ++r) {
        const int u = ku0 + r * kstep;
        kr[r] = u < nu ? *reinterpret_cast<const uint4*>(K + s_ks[u] + kc_off) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < kVRegs; ++r) {
        const int u = vu0 + r * vstep;
        vr[r] = 0;
        if (u < nu)
          vr[r] = a.esize == 2 ? *reinterpret_cast<const uint16_t*>(V + s_vs[u] + vc_off)
                               : *reinterpret_cast<const uint32_t*>(V + s_vs[u] + vc_off);
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kKRegs; ++r) {
        const int u = ku0 + r * kstep;
        if (u < nu && s_kd[u] >= 0) *reinterpret_cast<uint4*>(K + s_kd[u] + kc_off) = kr[r];
      }
#pragma unroll
      for (int r = 0; r < kVRegs; ++r) {
        const int u = vu0 + r * vstep;
        if (u < nu && s_vd[u] >= 0) {
          if (a.esize == 2) *reinterpret_cast<uint16_t*>(V + s_vd[u] + vc_off) = (uint16_t)vr[r];
          else *reinterpret_cast<uint32_t*>(V + s_vd[u] + vc_off) = vr[r];
        }
      }
      __syncthreads();
    }
  } else {
    // one entry at a time: its source and destination never overlap
    for (int j = 0; j < L; ++j) {
      for (int g0 = 0; g0 < a.Hkv; g0 += kCommitUnits) {
        const int ng = min(kCommitUnits, a.Hkv - g0);
        for (int u = tid; u < ng; u += kCommitThreads) {
          const int src = ctx + s_path[j], dst = ctx + j, g = g0 + u;
          const long long sb = (long long)table[src / a.bs] * blk_bytes;
          const long long db = (long long)table[dst / a.bs] * blk_bytes;
          s_ks[u] = sb + g * head_k + (long long)(src % a.bs) * rowb;
          s_kd[u] = db + g * head_k + (long long)(dst % a.bs) * rowb;
          s_vs[u] = sb + g * head_v + (long long)(src % a.bs) * a.esize;
          s_vd[u] = db + g * head_v + (long long)(dst % a.bs) * a.esize;
        }
        __syncthreads();
        if (s_path[j] != j) {
          for (int u = ku0; u < ng; u += kstep)
            *reinterpret_cast<uint4*>(K + s_kd[u] + kc_off) = *reinterpret_cast<const uint4*>(K + s_ks[u] + kc_off);
          for (int u = vu0; u < ng; u += vstep) {
            if (a.esize == 2)
              *reinterpret_cast<uint16_t*>(V + s_vd[u] + vc_off) = *reinterpret_cast<const uint16_t*>(V + s_vs[u] + vc_off);
            else
              *reinterpret_cast<uint32_t*>(V + s_vd[u] + vc_off) = *reinterpret_cast<const uint32_t*>(V + s_vs[u] + vc_off);
          }
        }
        __syncthreads();
      }
    }
  }
  if (tid == 0) a.ctx[b] = ctx + L;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(a.B), dim3(kCommitThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdtree
