// Acceptance walk over a verified draft tree, for gfx950.
//
// One workgroup of 1024 threads walks one sequence from the root.  Each step
// reads the current node's target logits row (V values) a few times:
//   greedy      one argmax pass (lowest id on ties);
//   rejection   max pass, normaliser pass, one residual pass per rejected
//   sampling    sibling, and a sampling pass if every sibling is rejected
//               (standard speculative sampling applied sibling by sibling:
//               SpecExec page, "Builds on");
//   target      max pass, then a sampling pass from softmax(l / tau)
//   sampling    (stays equivalent to sequential sampling from the target, so it
//               is safe for deterministic trees: SpecExec page, "Approach").
// Wavefront w owns a contiguous slice of the vocabulary and its lanes read it
// 64 consecutive tokens at a time, so every pass is coalesced and the
// inverse-CDF search can finish inside one slice.  Sums are accumulated in
// float64; the probability a decision is taken on is recomputed in float64.
#include "common.h"

namespace sdtree {

constexpr int kAccThreads = 1024;
constexpr int kAccWaves = kAccThreads / 64;
constexpr int kMaxT = 4096;
constexpr int kMaxRej = 64;

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ void __launch_bounds__(kAccThreads) accept_kernel(AcceptArgs a) {
  __shared__ int kids[kMaxT];
  __shared__ int wcnt[kAccWaves];
  __shared__ double wsum[kAccWaves];
  __shared__ float wmax[kAccWaves];
  __shared__ int widx[kAccWaves];
  __shared__ double zrej[kMaxRej];
  __shared__ int s_flag, s_x;
  __shared__ double s_thr, s_before;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;
  const int bt = a.tree_stride ? b : 0;
  const int32_t* par = a.parent + (size_t)bt * T;
  const int32_t* tok = a.token + (size_t)bt * T;
  int32_t* path = a.path + (size_t)b * T;

  // The tree must be topologically ordered with valid tokens.
  int bad = 0;
  for (int n = tid; n < T; n += kAccThreads) {
    const int p = par[n];
    if (n == 0 ? p != -1 : (p < 0 || p >= n)) bad |= SD_ERR_PARENT;
    const int t = tok[n];
    if (t < 0 || t >= V) bad |= SD_ERR_TOKEN;
  }
  if (tid == 0) s_flag = 0;
  __syncthreads();
  if (bad) atomicOr(&s_flag, bad);
  __syncthreads();
  for (int n = tid; n < T; n += kAccThreads) path[n] = -1;
  if (s_flag) {
    if (tid == 0) {
      set_status(a.status, (uint32_t)s_flag);
      a.path_len[b] = 0;
      a.bonus[b] = -1;
    }
    return;
  }

  // Vocabulary slice of this wavefront: [seg0, seg1), read 64 tokens at a time.
  const int seg = ((V + kAccWaves * 64 - 1) / (kAccWaves * 64)) * 64;
  const int seg0 = min(wave * seg, V), seg1 = min(seg0 + seg, V);
  const float invtau = a.tau > 0.f ? 1.f / a.tau : 0.f;
  const float c2 = invtau * 1.4426950408889634f;
  const double invtau_d = a.tau > 0.f ? 1.0 / (double)a.tau : 0.0;

  auto row_ptr = [&](int node) { return (size_t)b * T + node; };
  auto logit = [&](size_t rowbase, int y) -> float {
    return a.logits_f32 ? reinterpret_cast<const float*>(a.logits)[rowbase + y]
                        : bf16_to_f32(reinterpret_cast<const bf16_bits*>(a.logits)[rowbase + y]);
  };

  // block-wide reductions through the per-wave slots
  auto block_sum = [&](double v) -> double {
    v = wave_sum_d(v);
    __syncthreads();
    if (lane == 0) wsum[wave] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kAccWaves; ++w) t += wsum[w];
    return t;
  };

  // Inverse CDF: smallest y with sum_{y' <= y} w(y') > u * sum(w), else the last
  // y with w(y) > 0.  `wf(rowbase, y)` gives the unnormalised weight (double).
  auto sample = [&](size_t rowbase, float u, auto wf) -> int {
    double part = 0.0;
    for (int y = seg0 + lane; y < seg1; y += 64) part += wf(rowbase, y);
    part = wave_sum_d(part);
    __syncthreads();
    if (lane == 0) wsum[wave] = part;
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int w = 0; w < kAccWaves; ++w) tot += wsum[w];
      const double thr = (double)u * tot;
      double run = 0.0;
      int pick = -1, last_pos = -1;
      for (int w = 0; w < kAccWaves; ++w) {
        if (wsum[w] > 0.0) last_pos = w;
        if (pick < 0 && run + wsum[w] > thr) pick = w;
        run += wsum[w];
      }
      widx[0] = pick >= 0 ? pick : last_pos;
      s_thr = thr;
      // mass before the chosen slice
      double before = 0.0;
      for (int w = 0; w < widx[0]; ++w) before += wsum[w];
      s_before = before;
      s_x = -1;
    }
    __syncthreads();
    const int wsel = widx[0];
    if (wave == wsel) {
      const double thr = s_thr;
      double run = s_before;
      int found = -1, lastpos = -1;
      for (int y0 = seg0; y0 < seg1 && found < 0; y0 += 64) {
        const int y = y0 + lane;
        const double w = y < seg1 ? wf(rowbase, y) : 0.0;
        double inc = w;
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(inc, off);
          if (lane >= off) inc += o;
        }
        const bool cross = (run + inc > thr) && w > 0.0;
        const unsigned long long bal = __ballot(cross);
        const unsigned long long posb = __ballot(w > 0.0);
        if (bal) found = y0 + __ffsll((long long)bal) - 1;
        if (posb) lastpos = y0 + 63 - __clzll((long long)posb);
        run += __shfl(inc, 63);
      }
      if (lane == 0) s_x = found >= 0 ? found : lastpos;
    }
    __syncthreads();
    return s_x;
  };

  // children of `cur` in ascending index order -> kids[0..return)
  auto gather_children = [&](int cur) -> int {
    int nk = 0;
    for (int base = 0; base < T; base += kAccThreads) {
      const int n = base + tid;
      const bool f = n < T && par[n] == cur;
      const unsigned long long bal = __ballot(f);
      if (lane == 0) wcnt[wave] = __popcll(bal);
      __syncthreads();
      int off = nk;
      for (int w = 0; w < wave; ++w) off += wcnt[w];
      if (f) kids[off + __popcll(bal & ((1ull << lane) - 1ull))] = n;
      int tot = 0;
      for (int w = 0; w < kAccWaves; ++w) tot += wcnt[w];
      __syncthreads();
      nk += tot;
    }
    return nk;
  };

  int cur = 0, plen = 1, bonus = -1;
  if (tid == 0) path[0] = 0;
  for (int step = 0; step < T; ++step) {
    const int nk = gather_children(cur);
    const size_t rb = row_ptr(cur) * (size_t)V;
    int nxt = -1;
    if (a.tau == 0.f) {
      // argmax, lowest id among equal maxima
      float bv = -INFINITY;
      int bi = V;
      for (int y = seg0 + lane; y < seg1; y += 64) {
        const float v = logit(rb, y);
        if (v > bv) { bv = v; bi = y; }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      __syncthreads();
      if (lane == 0) { wmax[wave] = bv; widx[wave] = bi; }
      __syncthreads();
      float gv = wmax[0];
      int gi = widx[0];
      for (int w = 1; w < kAccWaves; ++w)
        if (wmax[w] > gv || (wmax[w] == gv && widx[w] < gi)) { gv = wmax[w]; gi = widx[w]; }
      for (int c = 0; c < nk; ++c)
        if (tok[kids[c]] == gi) { nxt = kids[c]; break; }
      if (nxt < 0) bonus = gi;
    } else {
      // max of the row
      float mx = -INFINITY;
      for (int y = seg0 + lane; y < seg1; y += 64) mx = fmaxf(mx, logit(rb, y));
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      __syncthreads();
      if (lane == 0) wmax[wave] = mx;
      __syncthreads();
      float m = wmax[0];
      for (int w = 1; w < kAccWaves; ++w) m = fmaxf(m, wmax[w]);
      auto ew = [&](size_t r, int y) -> double {
        return (double)__builtin_amdgcn_exp2f((logit(r, y) - m) * c2);
      };
      if (a.draft == nullptr) {
        const float u = a.unif[row_ptr(cur) * 2 + 1];
        const int x = sample(rb, u, ew);
        for (int c = 0; c < nk; ++c)
          if (tok[kids[c]] == x) { nxt = kids[c]; break; }
        if (nxt < 0) bonus = x;
      } else {
        double part = 0.0;
        for (int y = seg0 + lane; y < seg1; y += 64) part += ew(rb, y);
        const double z0 = block_sum(part);
        const float* q = a.draft + rb;
        int nrej = 0;
        // residual after j rejections, elementwise; zrej[j] is the j-th normaliser
        auto resid = [&](double r0, double qy, int upto) -> double {
          double r = r0;
          for (int j = 0; j < upto; ++j)
            if (zrej[j] > 0.0) r = fmax(r - qy, 0.0) / zrej[j];  // zero mass: unchanged
          return r;
        };
        for (int c = 0; c < nk && nrej < kMaxRej; ++c) {
          const int node = kids[c];
          const int x = tok[node];
          const double rx0 = exp(((double)logit(rb, x) - (double)m) * invtau_d) / z0;
          const double qx = (double)q[x];
          const double rx = resid(rx0, qx, nrej);
          const double u = (double)a.unif[row_ptr(node) * 2 + 0];
          if (u * qx < rx) { nxt = node; break; }
          // rejected: normaliser of max(r - q, 0)
          double pz = 0.0;
          for (int y = seg0 + lane; y < seg1; y += 64) {
            const double r = resid(ew(rb, y) / z0, (double)q[y], nrej);
            pz += fmax(r - (double)q[y], 0.0);
          }
          const double z = block_sum(pz);
          __syncthreads();
          if (tid == 0) zrej[nrej] = z;
          __syncthreads();
          ++nrej;
        }
        if (nxt < 0) {
          const float u = a.unif[row_ptr(cur) * 2 + 1];
          const int nr = nrej;
          auto rw = [&](size_t r, int y) -> double { return resid(ew(r, y) / z0, (double)q[y], nr); };
          bonus = sample(rb, u, rw);
        }
      }
    }
    __syncthreads();
    if (nxt < 0) break;
    if (tid == 0) path[plen] = nxt;
    ++plen;
    cur = nxt;
  }
  if (tid == 0) {
    a.path_len[b] = plen;
    a.bonus[b] = bonus;
  }
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(a.B), dim3(kAccThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdtree
