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
// the whole step).  After each pass the P workgroups publish a two-value
// partial to the workspace and meet at a barrier (an atomic counter with a
// bounded spin; the launch is cooperative, so all P are resident); every
// workgroup then reduces the P partials in the same order and takes the same
// decision.  An inverse-CDF draw picks the slice holding the crossing point
// from the per-slice masses and only that workgroup rescans its slice.  Sums
// are float64; the probability a test is taken on is recomputed in float64.
#include "common.h"

namespace sdtree {

constexpr int kAT = 256;              // threads per workgroup
constexpr int kAW = kAT / 64;         // wavefronts per workgroup
constexpr int kChunk = kAT * 8;       // tokens per chunk
constexpr int kMaxCh = 4;             // chunks kept in registers
constexpr int kMaxT = 4096;
constexpr int kMaxRej = 64;
constexpr int kMaxP = 16;
constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
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

template <typename LT, bool CACHED>
__global__ void __launch_bounds__(kAT) accept_kernel(AcceptArgs a) {
  constexpr bool kBF = sizeof(LT) == 2;
  static_assert(!CACHED || kBF, "only bf16 rows are cached");
  __shared__ int kids[kMaxT];
  __shared__ int wcnt[kAW];
  __shared__ double red_d[kAW];
  __shared__ float red_f[kAW];
  __shared__ int red_i[kAW];
  __shared__ double mass[kMaxP];    // per-slice mass of the distribution to draw from
  __shared__ double zrej[kMaxRej];  // residual normalisers at the current node
  __shared__ double s_part[2];
  __shared__ int s_flag, s_to, s_first, s_last, s_x;

  const int P = a.P;
  const int b = blockIdx.x / P, wg = blockIdx.x % P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;
  const int bt = a.tree_stride ? b : 0;
  const int32_t* par = a.parent + (size_t)bt * T;
  const int32_t* tok = a.token + (size_t)bt * T;
  int32_t* path = a.path + (size_t)b * T;
  unsigned char* seq = a.sync + (size_t)b * kAccSeqBytes;
  unsigned* ctr = reinterpret_cast<unsigned*>(seq);
  unsigned* done = ctr + 1;
  int* xslot = reinterpret_cast<int*>(ctr + 2);
  double* part = reinterpret_cast<double*>(seq + 64);  // [2][P][2]

  // The tree must be topologically ordered with valid tokens.
  int bad = 0;
  for (int n = tid; n < T; n += kAT) {
    const int p = par[n];
    if (n == 0 ? p != -1 : (p < 0 || p >= n)) bad |= SD_ERR_PARENT;
    const int t = tok[n];
    if (t < 0 || t >= V) bad |= SD_ERR_TOKEN;
  }
  if (tid == 0) {
    s_flag = 0;
    s_to = 0;
  }
  __syncthreads();
  if (bad) atomicOr(&s_flag, bad);
  __syncthreads();
  if (wg == 0)
    for (int n = tid; n < T; n += kAT) path[n] = -1;
  if (s_flag) {
    if (wg == 0 && tid == 0) {
      set_status(a.status, (uint32_t)s_flag);
      a.path_len[b] = 0;
      a.bonus[b] = -1;
    }
    return;
  }

  const int sl0 = min(wg * a.SL, V), sl1 = min(sl0 + a.SL, V);
  const int NC = a.NC;
  const bool vec = (V & 7) == 0;
  const float c2 = a.tau > 0.f ? 1.4426950408889634f / a.tau : 0.f;
  const double invtau_d = a.tau > 0.f ? 1.0 / (double)a.tau : 0.0;
  auto y0_of = [&](int c) { return sl0 + c * kChunk + tid * 8; };

  // ---- cross-workgroup exchange ---------------------------------------------
  int nbar = 0;
  auto barrier = [&]() {
    __syncthreads();
    if (P > 1) {
      ++nbar;
      if (tid == 0) {
        __threadfence();
        atomicAdd(ctr, 1u);
        const unsigned target = (unsigned)nbar * (unsigned)P;
        if (!s_to) {
          unsigned spins = 0;
          while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kSpinLimit) {
              s_to = 1;
              break;
            }
          }
        }
        __threadfence();
      }
      __syncthreads();
    }
  };
  auto publish = [&](double v0, double v1) {
    if (tid == 0) {
      if (P > 1) {
        double* p = part + (((nbar + 1) & 1) * P + wg) * 2;
        store_d(p, v0);
        store_d(p + 1, v1);
      } else {
        s_part[0] = v0;
        s_part[1] = v1;
      }
    }
  };
  auto fetch = [&](int j, int k) -> double {
    return P == 1 ? s_part[k] : load_d(part + ((nbar & 1) * P + j) * 2 + k);
  };

  // ---- workgroup reductions ---------------------------------------------------
  auto wg_sum = [&](double v) -> double {
    v = wave_sum_d(v);
    __syncthreads();
    if (lane == 0) red_d[wave] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kAW; ++w) t += red_d[w];
    return t;
  };
  auto wg_max = [&](float v) -> float {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    __syncthreads();
    if (lane == 0) red_f[wave] = v;
    __syncthreads();
    float t = red_f[0];
    for (int w = 1; w < kAW; ++w) t = fmaxf(t, red_f[w]);
    return t;
  };

  // children of `cur` in ascending index order -> kids[0..return)
  auto gather_children = [&](int cur) -> int {
    int nk = 0;
    for (int base = 0; base < T; base += kAT) {
      const int n = base + tid;
      const bool f = n < T && par[n] == cur;
      const unsigned long long bal = __ballot(f);
      if (lane == 0) wcnt[wave] = __popcll(bal);
      __syncthreads();
      int off = nk;
      for (int w = 0; w < wave; ++w) off += wcnt[w];
      if (f) kids[off + __popcll(bal & ((1ull << lane) - 1ull))] = n;
      int tot = 0;
      for (int w = 0; w < kAW; ++w) tot += wcnt[w];
      __syncthreads();
      nk += tot;
    }
    return nk;
  };

  uint4 lc[kMaxCh];  // this thread's bf16 logits (when `cache`)
  const LT* row = nullptr;
  auto logits8 = [&](int c, float* v) {
    const int y0 = y0_of(c);
    if (y0 >= sl1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = -INFINITY;
      return;
    }
    if constexpr (CACHED) {
      const uint4 u = lc[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = y0 + e < V ? bf16_to_f32((bf16_bits)(w[e >> 1] >> (16 * (e & 1)))) : -INFINITY;
    } else {
      load8<LT>(row, y0, V, vec, -INFINITY, v);
    }
  };

  // Inverse-CDF draw: slices' masses in mass[0..P); threshold u * total.  The
  // workgroup owning the crossing rescans its slice with `wf(c, w8)` and
  // returns the token (other workgroups return -1).
  auto draw = [&](float u, auto wf) -> int {
    __syncthreads();
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
    if (tid == 0) {
      s_x = -1;
      s_last = -1;
    }
    double rn = before;
    FOR_CHUNKS(c,
      double w8[8];
      wf(c, w8);
      double ls = 0.0;
_Pragma("unroll")
      for (int e = 0; e < 8; ++e) ls += w8[e];
      double inc = ls;
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
      }
      __syncthreads();
      if (lane == 63) red_d[wave] = inc;
      if (tid == 0) s_first = kAT;
      __syncthreads();
      double woff = 0.0, ctot = 0.0;
      for (int w = 0; w < kAW; ++w) {
        if (w < wave) woff += red_d[w];
        ctot += red_d[w];
      }
      const double excl = rn + woff + inc - ls;
      if (ls > 0.0 && excl + ls > thr) atomicMin(&s_first, tid);
      if (ls > 0.0) {
        int lp = 0;
        for (int e = 0; e < 8; ++e)
          if (w8[e] > 0.0) lp = e;
        atomicMax(&s_last, y0_of(c) + lp);
      }
      __syncthreads();
      const int first = s_first;
      if (first < kAT) {
        if (tid == first) {
          double r2 = excl;
          int pk = -1, lp = -1;
          for (int e = 0; e < 8; ++e) {
            if (w8[e] > 0.0) lp = e;
            r2 += w8[e];
            if (pk < 0 && w8[e] > 0.0 && r2 > thr) pk = e;
          }
          s_x = y0_of(c) + (pk >= 0 ? pk : lp);
        }
        __syncthreads();
        return s_x;
      }
      rn += ctot;
    )
    __syncthreads();
    return s_last;
  };

  int cur = 0, plen = 1;
  if (wg == 0 && tid == 0) path[0] = 0;
  for (int step = 0; step < T; ++step) {
    const int nk = gather_children(cur);
    row = reinterpret_cast<const LT*>(a.logits) + ((size_t)b * T + cur) * V;
    if constexpr (CACHED) {
      {
#pragma unroll
        for (int c = 0; c < kMaxCh; ++c) {
          const int y0 = y0_of(c);
          if (c < NC && y0 < sl1) {
            if (vec && y0 + 8 <= V) {
              lc[c] = *reinterpret_cast<const uint4*>(row + y0);
            } else {
              uint32_t w[4] = {0, 0, 0, 0};
              for (int e = 0; e < 8; ++e)
                if (y0 + e < V) w[e >> 1] |= (uint32_t)row[y0 + e] << (16 * (e & 1));
              lc[c] = make_uint4(w[0], w[1], w[2], w[3]);
            }
          }
        }
      }
    }
    int nxt = -1;
    bool stop = false;
    if (a.tau == 0.f) {
      // argmax, lowest id among equal maxima
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
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      __syncthreads();
      if (lane == 0) {
        red_f[wave] = bv;
        red_i[wave] = bi;
      }
      __syncthreads();
      bv = red_f[0];
      bi = red_i[0];
      for (int w = 1; w < kAW; ++w)
        if (red_f[w] > bv || (red_f[w] == bv && red_i[w] < bi)) {
          bv = red_f[w];
          bi = red_i[w];
        }
      publish((double)bv, (double)bi);
      barrier();
      double gv = -INFINITY;
      int gi = V;
      for (int j = 0; j < P; ++j) {
        const double v = fetch(j, 0);
        const int i = (int)fetch(j, 1);
        if (v > gv || (v == gv && i < gi)) {
          gv = v;
          gi = i;
        }
      }
      for (int c = 0; c < nk; ++c)
        if (tok[kids[c]] == gi) {
          nxt = kids[c];
          break;
        }
      if (nxt < 0) {
        if (wg == 0 && tid == 0) a.bonus[b] = gi;
        stop = true;
      }
    } else {
      // statistics of this slice: max, then mass relative to that max
      float mw = -INFINITY;
      FOR_CHUNKS(c,
        float v[8];
        logits8(c, v);
_Pragma("unroll")
        for (int e = 0; e < 8; ++e) mw = fmaxf(mw, v[e]);
      )
      mw = wg_max(mw);
      double sw = 0.0;
      if (mw != -INFINITY) {
        FOR_CHUNKS(c,
          float v[8];
          logits8(c, v);
_Pragma("unroll")
          for (int e = 0; e < 8; ++e) sw += (double)__builtin_amdgcn_exp2f((v[e] - mw) * c2);
        )
      }
      sw = wg_sum(sw);
      publish((double)mw, sw);
      barrier();
      float m = -INFINITY;
      for (int j = 0; j < P; ++j) m = fmaxf(m, (float)fetch(j, 0));
      if (tid < P) {
        const float mj = (float)fetch(tid, 0);
        mass[tid] = mj == -INFINITY ? 0.0 : fetch(tid, 1) * (double)__builtin_amdgcn_exp2f((mj - m) * c2);
      }
      __syncthreads();
      double z0 = 0.0;
      for (int j = 0; j < P; ++j) z0 += mass[j];
      auto ew8 = [&](int c, double* w8) {
        float v[8];
        logits8(c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w8[e] = v[e] == -INFINITY ? 0.0 : (double)__builtin_amdgcn_exp2f((v[e] - m) * c2);
      };
      const float* qrow = a.draft ? a.draft + ((size_t)b * T + cur) * V : nullptr;
      if (qrow == nullptr) {
        const float u = a.unif[((size_t)b * T + cur) * 2 + 1];
        const int x = draw(u, ew8);
        if (x >= 0 && tid == 0) {
          if (P > 1) __hip_atomic_store(xslot, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else s_x = x;
        }
        barrier();
        const int xs = P > 1 ? __hip_atomic_load(xslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : s_x;
        for (int c = 0; c < nk; ++c)
          if (tok[kids[c]] == xs) {
            nxt = kids[c];
            break;
          }
        if (nxt < 0) {
          if (wg == 0 && tid == 0) a.bonus[b] = xs;
          stop = true;
        }
      } else {
        int nrej = 0;
        // residual after `upto` rejections, elementwise; zrej[j] is the j-th normaliser
        auto resid = [&](double r0, double qy, int upto) -> double {
          double r = r0;
          for (int j = 0; j < upto; ++j)
            if (zrej[j] > 0.0) r = fmax(r - qy, 0.0) / zrej[j];  // zero mass: unchanged
          return r;
        };
        auto q8_of = [&](int c, float* q8) {
          const int y0 = y0_of(c);
          if (y0 < sl1) {
            load8<float>(qrow, y0, V, vec, 0.f, q8);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) q8[e] = 0.f;
          }
        };
        for (int c = 0; c < nk && nrej < kMaxRej; ++c) {
          const int node = kids[c];
          const int x = tok[node];
          const double lx = (double)Elem<LT>::load(row, x);
          const double rx0 = exp((lx - (double)m) * invtau_d) / z0;
          const double qx = (double)qrow[x];
          const double rx = resid(rx0, qx, nrej);
          const double u = (double)a.unif[((size_t)b * T + node) * 2 + 0];
          if (u * qx < rx) {
            nxt = node;
            break;
          }
          // rejected: this slice's mass of max(r - q, 0)
          double pz = 0.0;
          if constexpr (CACHED) {
            float q8[kMaxCh][8];
#pragma unroll
            for (int k = 0; k < kMaxCh; ++k)
              if (k < NC) q8_of(k, q8[k]);
#pragma unroll
            for (int k = 0; k < kMaxCh; ++k) {
              if (k < NC) {
                double w8[8];
                ew8(k, w8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const double qy = (double)q8[k][e];
                  pz += fmax(resid(w8[e] / z0, qy, nrej) - qy, 0.0);
                }
              }
            }
          } else {
            for (int c = 0; c < NC; ++c) {
              float q8[8];
              double w8[8];
              q8_of(c, q8);
              ew8(c, w8);
              for (int e = 0; e < 8; ++e) {
                const double qy = (double)q8[e];
                pz += fmax(resid(w8[e] / z0, qy, nrej) - qy, 0.0);
              }
            }
          }
          pz = wg_sum(pz);
          publish(pz, 0.0);
          barrier();
          double z = 0.0;
          for (int j = 0; j < P; ++j) z += fetch(j, 0);
          if (z > 0.0 && tid < P) mass[tid] = fetch(tid, 0);
          if (tid == 0) zrej[nrej] = z;
          __syncthreads();
          ++nrej;
        }
        if (nxt < 0) {
          const float u = a.unif[((size_t)b * T + cur) * 2 + 1];
          const int nr = nrej;
          // weights in the units of mass[]: the residual times the normaliser of
          // the last pass that changed it (the statistics pass if none did)
          double units = z0;
          for (int j = 0; j < nr; ++j)
            if (zrej[j] > 0.0) units = zrej[j];
          auto rw8 = [&](int c, double* w8) {
            float q8[8];
            q8_of(c, q8);
            ew8(c, w8);
#pragma unroll
            for (int e = 0; e < 8; ++e) w8[e] = resid(w8[e] / z0, (double)q8[e], nr) * units;
          };
          const int x = draw(u, rw8);
          if (x >= 0 && tid == 0) a.bonus[b] = x;
          stop = true;
        }
      }
    }
    if (stop) break;
    if (wg == 0 && tid == 0) path[plen] = nxt;
    ++plen;
    cur = nxt;
  }
  if (wg == 0 && tid == 0) a.path_len[b] = plen;
  if (P > 1 && tid == 0) {
    // the last workgroup of the sequence to leave resets the counters
    __threadfence();
    if (atomicAdd(done, 1u) == (unsigned)P - 1) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  const void* fn = a.logits_f32 ? reinterpret_cast<const void*>(accept_kernel<float, false>)
                   : a.NC <= kMaxCh ? reinterpret_cast<const void*>(accept_kernel<bf16_bits, true>)
                                    : reinterpret_cast<const void*>(accept_kernel<bf16_bits, false>);
  const dim3 grid((unsigned)a.B * a.P), block(kAT);
  AcceptArgs copy = a;
  void* args[] = {&copy};
  if (a.P == 1) return hipLaunchKernel(fn, grid, block, args, 0, st);
  return hipLaunchCooperativeKernel(fn, grid, block, args, 0, st);
}

}  // namespace sdtree
