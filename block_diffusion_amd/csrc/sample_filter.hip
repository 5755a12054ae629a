// Top-k / top-p filtered sampling from stored logits, gfx950.
//
// The pages' SamplingParams carry topk and topp besides the temperature
// (JetEngine README usage examples), and the developer notes found a
// separate sampler after the logits faster than a fused one ("Ruled-Out
// Optimizations").  Here the LM head stores the listed rows' logits
// (lmhead_tile_kernel, store mode) and this kernel draws each row's token:
//   * tokens other than the mask token are ranked by logit, higher first,
//     the lower id first among equal logits;
//   * top_k > 0 keeps the first top_k; top_p < 1 then keeps the shortest
//     leading run of those whose running sum of exp((l - m)/T) reaches
//     top_p of their total (at least one token);
//   * the token is drawn from softmax(l/T) over the kept set with the same
//     block draw as the fused sampler (Philox4x32-10, counter (chunk, row,
//     step, 0); per 16-column block an inverse-CDF candidate and a Gumbel
//     value at the block's log-sum-exp; the largest Gumbel wins), the other
//     tokens having zero weight; the confidence is the drawn token's
//     probability at temperature 1.
// One workgroup of 1024 threads per listed row.  The ranking is never
// sorted: a radix select over the order-preserving 32-bit image of the
// logits finds the top-k boundary (counts per 8-bit digit, four passes over
// the row) and the top-p boundary (sums of exp((l - m)/T) per digit), and a
// pass in id order settles ties at a boundary value.  Each pass re-reads the
// row (L2 / HBM); passes that a filter does not need are skipped.
#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

constexpr int kSfThreads = 1024;

__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // larger float -> larger key
}

// the same Philox4x32-10 and uniforms as the fused sampler
__device__ __forceinline__ void sf_philox(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                          uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}
__device__ __forceinline__ float sf_uniform(uint32_t w) {
  return (float)(((w >> 9) << 1) | 1u) * (1.0f / 16777216.0f);
}

// block-wide reductions over 1024 threads (16 waves) through LDS
template <typename T, typename F>
__device__ T block_reduce(T v, F op, T* s_tmp) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    v = op(v, __shfl_xor(v, off, 64));
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  T r = s_tmp[0];
  for (int w = 1; w < kSfThreads / 64; ++w) r = op(r, s_tmp[w]);
  return r;
}

}  // namespace

__global__ __launch_bounds__(1024) void sample_filtered_kernel(SampleArgs a) {
  __shared__ float s_f[16];
  __shared__ int s_i[16];
  __shared__ uint32_t s_hist[256];
  __shared__ float s_mass[256];
  __shared__ int s_sel[2];
  __shared__ float s_rem;
  __shared__ float s_gbest[16];
  __shared__ int s_cbest[16];
  __shared__ float s_lbest[16];
  __shared__ int s_cnt[kSfThreads];     // per-thread tie counts / masses in id order
  __shared__ float s_ms[kSfThreads];

  const int r = blockIdx.x;
  if (r >= *a.num_rows) return;
  const int tid = threadIdx.x;
  const int V = a.V, mask = a.mask_id;
  const float* l = a.logits + (size_t)r * V;
  const uint32_t rid = (uint32_t)(a.row_index ? a.row_index[r] : r);
  const float invT = a.inv_temp;

  // every logit of the row once, 16 bytes per load when rows are 16-byte
  // aligned (V % 4 == 0), else one at a time
  auto each = [&](auto fn) {
    if ((V & 3) == 0) {
      const f32x4* l4 = reinterpret_cast<const f32x4*>(l);
      for (int q = tid; q < (V >> 2); q += kSfThreads) {
        const f32x4 x = l4[q];
        fn(4 * q, x.x); fn(4 * q + 1, x.y); fn(4 * q + 2, x.z); fn(4 * q + 3, x.w);
      }
    } else {
      for (int v = tid; v < V; v += kSfThreads) fn(v, l[v]);
    }
  };

  // ---- one pass: max logit m, sum exp(l - m) (temperature 1) and
  // sum exp((l - m)/T), online per thread, then merged over the workgroup
  float mt = -INFINITY, s1t = 0.f, sTt = 0.f;
  each([&](int v, float x) {
    if (v == mask) return;
    if (x > mt) {
      const float d = mt - x;                 // -inf on the first value
      s1t = s1t * __expf(d);
      sTt = sTt * __expf(d * invT);
      mt = x;
    }
    s1t += __expf(x - mt);
    sTt += __expf((x - mt) * invT);
  });
  const float m = block_reduce(mt, [](float x, float y) { return fmaxf(x, y); }, s_f);
  const float wt = mt == -INFINITY ? 0.f : 1.f;
  const float S1 = block_reduce(wt * s1t * __expf(mt - m), [](float x, float y) { return x + y; }, s_f);
  const float ST = block_reduce(wt * sTt * __expf((mt - m) * invT), [](float x, float y) { return x + y; }, s_f);

  // kept-set test: key above the boundary key, or equal to it with id at
  // most the boundary id; bk = 0 with bid = V keeps everything
  uint32_t kk = 0u;     // top-k boundary key
  int kid = V;          // top-k boundary id among keys == kk
  const int nval = V - 1;
  const bool use_k = a.top_k > 0 && a.top_k < nval;
  auto keep_k = [&](int v, uint32_t key) { return v != mask && (key > kk || (key == kk && v <= kid)); };

  // radix select of the rank-`need` element (1-based, from the top) among
  // the elements `in` admits; counts (MASS false) or mass (MASS true)
  auto radix = [&](auto in, bool use_mass, float need_f, int need_i, uint32_t& key_out,
                   int& id_out) {
    uint32_t prefix = 0u, pmask = 0u;
    float rem_f = need_f;
    int rem_i = need_i;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSfThreads) {
        s_hist[i] = 0u;
        s_mass[i] = 0.f;
      }
      __syncthreads();
      each([&](int v, float x) {
        const uint32_t key = okey(x);
        if (!in(v, key) || (key & pmask) != prefix) return;
        const int d = (key >> shift) & 255;
        if (use_mass) atomicAdd(&s_mass[d], __expf((x - m) * invT));
        else atomicAdd(&s_hist[d], 1u);
      });
      __syncthreads();
      if (tid == 0) {
        // from the largest digit down: the digit where the running total
        // first reaches the remaining need (the last non-empty digit if
        // rounding leaves it short)
        float cf = 0.f;
        int ci = 0, pick = -1, last = -1;
        for (int d = 255; d >= 0; --d) {
          const bool ne = use_mass ? s_mass[d] > 0.f : s_hist[d] > 0u;
          if (!ne) continue;
          last = d;
          if (use_mass) {
            if (cf + s_mass[d] >= rem_f) { pick = d; break; }
            cf += s_mass[d];
          } else {
            if (ci + (int)s_hist[d] >= rem_i) { pick = d; break; }
            ci += (int)s_hist[d];
          }
        }
        if (pick < 0) {
          pick = last < 0 ? 0 : last;
          // remove the digits above the last one from the need
          cf = 0.f; ci = 0;
          for (int d = 255; d > last; --d) { cf += s_mass[d]; ci += (int)s_hist[d]; }
        }
        s_sel[0] = pick;
        s_sel[1] = rem_i - ci;
        s_rem = rem_f - cf;
      }
      __syncthreads();
      const int pick = s_sel[0];
      rem_i = s_sel[1];
      rem_f = s_rem;
      prefix |= (uint32_t)pick << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    // ties at the boundary key, in id order: the id where the running count
    // (mass) of tied elements reaches the remaining need
    const int per = (V + kSfThreads - 1) / kSfThreads;
    const int v0 = tid * per, v1 = min(V, v0 + per);
    int cnt = 0;
    float ms = 0.f;
    for (int v = v0; v < v1; ++v) {
      const float x = l[v];
      const uint32_t key = okey(x);
      if (in(v, key) && key == prefix) {
        ++cnt;
        if (use_mass) ms += __expf((x - m) * invT);
      }
    }
    // the thread (in id order) where the running count (mass) reaches it
    s_cnt[tid] = cnt;
    s_ms[tid] = ms;
    __syncthreads();
    if (tid == 0) {
      int c = 0, t = 0;
      float f = 0.f;
      for (t = 0; t < kSfThreads; ++t) {
        const bool reach = use_mass ? (f + s_ms[t] >= rem_f) : (c + s_cnt[t] >= rem_i);
        if (reach && s_cnt[t] > 0) break;
        c += s_cnt[t];
        f += s_ms[t];
      }
      if (t == kSfThreads) {        // rounding left it short: the last tie
        for (t = kSfThreads - 1; t > 0 && s_cnt[t] == 0; --t) {}
        c = 0; f = 0.f;
        for (int u = 0; u < t; ++u) { c += s_cnt[u]; f += s_ms[u]; }
      }
      s_sel[0] = t;
      s_sel[1] = rem_i - c;
      s_rem = rem_f - f;
    }
    __syncthreads();
    int idc = V;
    if (tid == s_sel[0]) {
      int need2 = s_sel[1];
      float rf = s_rem;
      int lastv = v0;
      for (int v = v0; v < v1; ++v) {
        const float x = l[v];
        const uint32_t key = okey(x);
        if (!(in(v, key) && key == prefix)) continue;
        lastv = v;
        if (use_mass) {
          const float w = __expf((x - m) * invT);
          if (w >= rf) { idc = v; break; }
          rf -= w;
        } else {
          if (need2 <= 1) { idc = v; break; }
          --need2;
        }
      }
      if (idc == V) idc = lastv;
      s_sel[0] = idc;
    }
    __syncthreads();
    key_out = prefix;
    id_out = s_sel[0];
    __syncthreads();
  };

  if (use_k) {
    radix([&](int v, uint32_t) { return v != mask; }, false, 0.f, a.top_k, kk, kid);
  }
  uint32_t pk = 0u;
  int pid = V;
  if (a.top_p < 1.f) {
    // total mass of the top-k set at temperature T (all tokens: ST)
    float Z = ST;
    if (use_k) {
      float z = 0.f;
      each([&](int v, float x) {
        if (keep_k(v, okey(x))) z += __expf((x - m) * invT);
      });
      Z = block_reduce(z, [](float x, float y) { return x + y; }, s_f);
    }
    radix([&](int v, uint32_t key) { return keep_k(v, key); }, true, a.top_p * Z, 0, pk, pid);
  }
  auto keep = [&](int v, uint32_t key) {
    return keep_k(v, key) && (key > pk || (key == pk && v <= pid));
  };

  // ---- the block draw over the kept set (log2 units as the fused sampler)
  float gbest = -INFINITY, lbest = 0.f;
  int cbest = 0x7fffffff;
  const int nchunk = (V + 31) / 32;
  for (int c = tid; c < nchunk; c += kSfThreads) {
    uint32_t w0 = (uint32_t)c, w1 = rid, w2 = a.step, w3 = 0u;
    sf_philox(w0, w1, w2, w3, a.key0, a.key1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v0 = 32 * c + 8 * q + 4 * h;
        float lv[4];
        if ((V & 3) == 0 && v0 + 4 <= V) {
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(l + v0);
          lv[0] = x4.x; lv[1] = x4.y; lv[2] = x4.z; lv[3] = x4.w;
        } else {
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2) lv[r2] = v0 + r2 < V ? l[v0 + r2] : -INFINITY;
        }
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const int v = v0 + r2;
          const float xv = (v < V && keep(v, okey(lv[r2]))) ? lv[r2] * kLog2e : -INFINITY;
          x[4 * q + r2] = xv;
          bm = fmaxf(bm, xv);
        }
      }
      if (bm == -INFINITY) continue;
      const float u = sf_uniform(h ? w2 : w0);
      const float eg = sf_uniform(h ? w3 : w1);
      const float bmT = bm * invT;
      float e[16], S = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e[i] = fast_exp2(fmaf(x[i], invT, -bmT));
        S += e[i];
      }
      const float target = u * S;
      float cum = 0.f;
      int ci = -1, last = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        cum += e[i];
        last = e[i] > 0.f ? i : last;
        ci = (ci < 0 && e[i] > 0.f && cum >= target) ? i : ci;
      }
      ci = ci < 0 ? last : ci;
      float xc = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) xc = (i == ci) ? x[i] : xc;
      const float G = bmT + __log2f(S) - __log2f(-__log2f(eg));
      const int cand = 32 * c + 8 * (ci >> 2) + 4 * h + (ci & 3);
      if (G > gbest || (G == gbest && cand < cbest)) {
        gbest = G; cbest = cand; lbest = xc * (1.0f / kLog2e);
      }
    }
  }
  // argmax of (G, lower candidate) over the workgroup
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float g2 = __shfl_xor(gbest, off, 64);
    const int c2 = __shfl_xor(cbest, off, 64);
    const float l2 = __shfl_xor(lbest, off, 64);
    if (g2 > gbest || (g2 == gbest && c2 < cbest)) { gbest = g2; cbest = c2; lbest = l2; }
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) {
    s_gbest[wave] = gbest;
    s_cbest[wave] = cbest;
    s_lbest[wave] = lbest;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSfThreads / 64; ++w)
      if (s_gbest[w] > gbest || (s_gbest[w] == gbest && s_cbest[w] < cbest)) {
        gbest = s_gbest[w]; cbest = s_cbest[w]; lbest = s_lbest[w];
      }
    a.token[rid] = cbest;
    a.conf[rid] = __expf(lbest - m) / S1;
  }
}

hipError_t sample_filtered_launch(const SampleArgs& a, hipStream_t st) {
  sample_filtered_kernel<<<a.max_rows, kSfThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
