// Top-k / top-p filtered sampling from stored logits, gfx950.
//
// The pages' SamplingParams carry topk and topp besides the temperature
// (JetEngine README usage examples), and the developer notes found a
// separate sampler after the logits faster than a fused one ("Ruled-Out
// Optimizations").  Here the LM head stores the listed rows' logits
// (lmhead_tile_kernel, store mode) and this kernel draws each row's token:
//   * candidates are the finite logits other than the mask token's, ranked
//     by logit, higher first, the lower id first among equal logits;
//   * top_k > 0 keeps the first top_k; top_p < 1 then keeps the shortest
//     leading run of those whose running sum of exp((l - m)/T) reaches
//     top_p of their total (at least one token);
//   * the token is drawn from softmax(l/T) over the kept set with the same
//     block draw as the fused sampler (Philox4x32-10, counter (chunk, row,
//     step, 0); per 16-column block an inverse-CDF candidate and a Gumbel
//     value at the block's log-sum-exp; the largest Gumbel wins), the other
//     tokens having zero weight; the confidence is the drawn token's
//     probability at temperature 1.  A row without a candidate gets the
//     mask token with confidence 0.
//
// One workgroup of 1024 threads per listed row; the ranking is never
// sorted as a whole.  Passes over the row (16-byte loads, several in flight
// per thread):
//   1. the row maximum m (read from the LM head's partial row maxima when
//      the caller passes them: the round does);
//   2. (filters only) a histogram over 4096 value bins below m, bin =
//      floor((m - l) log2(e) / T * 32) (the last bin takes everything
//      further down), with per bin the candidate count (top-k) and the sum
//      of exp((l - m)/T) in 2^-40 fixed point (top-p: integer sums, so the
//      boundary does not depend on the order of the atomic adds).  The bin
//      is a monotone function of the logit, so every bin holds a run of
//      the ranking;
//   3. a scan over the bins finds the bin holding a boundary (the top_k-th
//      candidate, or the first candidate whose running mass reaches top_p
//      of the kept total); one more pass gathers that bin's candidates
//      into LDS as (key, ~id), a bitonic sort puts them in ranking order
//      and a scan over them gives the boundary candidate.  A bin of more
//      than 2048 candidates (long runs of equal logits, extreme
//      temperatures) is resolved instead by a radix select over the
//      order-preserving 32-bit image of its logits (8-bit digits, four
//      passes, then a pass in id order for ties);
//   4. the block draw over the kept set, which also sums exp(l - m) for
//      the confidence.
// Without a filter only passes 1 and 4 run.
#include <climits>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

constexpr int kSfThreads = 1024;
constexpr int kSfWaves = kSfThreads / 64;
constexpr int kSfBins = 4096;             // value bins below the row maximum
constexpr float kSfBinsPerLog2 = 32.f;    // bins per unit of (m - l) log2(e) / T
constexpr int kSfCap = 2048;              // candidates of one bin sorted in LDS
constexpr float kSfFix = 1099511627776.f; // 2^40: fixed-point scale of the masses

__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // larger float -> larger key
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src_lane) {
  const uint32_t lo = __shfl((uint32_t)v, src_lane, 64), hi = __shfl((uint32_t)(v >> 32), src_lane, 64);
  return ((uint64_t)hi << 32) | lo;
}

// block-wide reduction over 1024 threads (16 waves) through LDS
template <typename F>
__device__ float block_reduce(float v, F op, float* s_tmp) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = s_tmp[0];
  for (int w = 1; w < kSfWaves; ++w) r = op(r, s_tmp[w]);
  return r;
}

}  // namespace

__global__ __launch_bounds__(1024) void sample_filtered_kernel(SampleArgs a) {
  __shared__ uint32_t s_bc[kSfBins];     // candidates per bin
  __shared__ uint64_t s_bm[kSfBins];     // fixed-point mass per bin
  __shared__ uint64_t s_g[kSfCap];       // one bin's candidates, (key << 32) | ~id
  __shared__ uint64_t s_w[kSfWaves];
  __shared__ float s_f[kSfWaves];
  __shared__ int s_n, s_first, s_ndef;
  __shared__ uint64_t s_before;
  __shared__ int s_sel;
  __shared__ float s_gbest[kSfWaves];
  __shared__ int s_cbest[kSfWaves];
  // radix-select scratch on top of s_g: it runs only when a bin did not fit
  uint64_t* const s_h64 = s_g;                                        // [256]
  int* const s_cnt = reinterpret_cast<int*>(s_g + 256);               // [1024]
  static_assert(256 * 8 + kSfThreads * 4 <= kSfCap * 8, "radix scratch must fit in the gather buffer");

  const int r = blockIdx.x;
  if (r >= *a.num_rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, mask = a.mask_id;
  const float* l = a.logits + (size_t)r * V;
  const uint32_t rid = (uint32_t)(a.row_index ? a.row_index[r] : r);
  const float invT = a.inv_temp;

  auto cand = [&](int v, float x) { return (v != mask) & (fabsf(x) <= 3.402823466e38f); };

  // every logit of the row once; with 16-byte aligned rows (V % 4 == 0)
  // each thread keeps four 16-byte loads in flight
  auto each = [&](auto fn) {
    if ((V & 3) == 0) {
      const f32x4* l4 = reinterpret_cast<const f32x4*>(l);
      const int n4 = V >> 2;
      auto fn4 = [&](int q, const f32x4& x) {
        fn(4 * q, x.x); fn(4 * q + 1, x.y); fn(4 * q + 2, x.z); fn(4 * q + 3, x.w);
      };
      int q = tid;
      for (; q + 3 * kSfThreads < n4; q += 4 * kSfThreads) {
        const f32x4 x0 = l4[q], x1 = l4[q + kSfThreads], x2 = l4[q + 2 * kSfThreads],
                    x3 = l4[q + 3 * kSfThreads];
        fn4(q, x0); fn4(q + kSfThreads, x1); fn4(q + 2 * kSfThreads, x2); fn4(q + 3 * kSfThreads, x3);
      }
      for (; q < n4; q += kSfThreads) fn4(q, l4[q]);
    } else {
      for (int v = tid; v < V; v += kSfThreads) fn(v, l[v]);
    }
  };

  // ---- pass 1: the maximum candidate logit, or the maximum of the LM
  // head's partial row maxima when it left them (the same fp32 values)
  float mt = -INFINITY;
  if (a.pmax != nullptr) {
    const int nteam = kLmGrid / lm_team_size(*a.num_rows);
    for (int t = tid; t < nteam; t += kSfThreads)
      mt = fmaxf(mt, fmaxf(a.pmax[(size_t)r * nteam + t], a.pmax2[(size_t)r * nteam + t]));
  } else {
    each([&](int v, float x) {
      if (cand(v, x)) mt = fmaxf(mt, x);
    });
  }
  const float m = block_reduce(mt, [](float x, float y) { return fmaxf(x, y); }, s_f);
  if (m == -INFINITY) {
    if (tid == 0) {
      a.token[rid] = mask;
      a.conf[rid] = 0.f;
    }
    return;
  }

  const float c2 = invT * kLog2e;               // exp((l - m)/T) = 2^((l - m) c2)
  const float c3 = c2 * kSfBinsPerLog2;
  auto bin_of = [&](float x) -> int {
    const float d = fmaxf((m - x) * c3, 0.f);   // >= 0 (m is the maximum), monotone in x
    return d < (float)(kSfBins - 1) ? (int)d : kSfBins - 1;
  };
  auto mass_of = [&](float x) -> uint64_t {
    return (uint64_t)(fast_exp2((x - m) * c2) * kSfFix);
  };

  // exclusive prefix over the workgroup (thread order) of a 64-bit value;
  // `total` = the sum over all threads
  auto block_scan = [&](uint64_t v, uint64_t& total) -> uint64_t {
    uint64_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t y = shfl_u64(x, lane >= off ? lane - off : lane);
      x += lane >= off ? y : 0ull;
    }
    __syncthreads();
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    uint64_t run = 0ull, tot = 0ull;
    for (int w = 0; w < kSfWaves; ++w) {
      const uint64_t t = s_w[w];
      run += w < wave ? t : 0ull;
      tot += t;
    }
    total = tot;
    return run + x - v;
  };

  // first slot s of [0, n) (four per thread, thread-major) with val(s) > 0
  // whose inclusive running sum reaches tgt, or -1; `before` = the running
  // sum ahead of it, `total` = the sum of all slots
  auto find_first = [&](auto val, int n, uint64_t tgt, uint64_t& before, uint64_t& total) -> int {
    uint64_t v[4], sum = 0ull;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * tid + j;
      v[j] = s < n ? val(s) : 0ull;
      sum += v[j];
    }
    if (tid == 0) s_first = INT_MAX;
    uint64_t run = block_scan(sum, total);
    int mine = -1;
    uint64_t mb = 0ull;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (mine < 0 && v[j] > 0ull && run + v[j] >= tgt) {
        mine = 4 * tid + j;
        mb = run;
      }
      run += v[j];
    }
    if (mine >= 0) atomicMin(&s_first, mine);
    __syncthreads();
    const int f = s_first;
    if (mine >= 0 && mine == f) s_before = mb;
    __syncthreads();
    before = s_before;
    __syncthreads();
    return f == INT_MAX ? -1 : f;
  };

  // s_g[0, n) (n <= kSfCap) into ranking order by a bitonic sort
  auto sort_list = [&](int n) {
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = n + tid; i < n2; i += kSfThreads) s_g[i] = 0ull;   // below every candidate
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kSfThreads) {
          const int p = i ^ j;
          if (p > i) {
            const uint64_t x = s_g[i], y = s_g[p];
            if ((i & k) == 0 ? x < y : x > y) {
              s_g[i] = y;
              s_g[p] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  };
  // the candidates of bin b that pred admits, into s_g in ranking order
  // (descending (key, ~id)); returns their number, > kSfCap if they did not
  // fit (s_g then holds no list)
  auto gather_sort = [&](int b, auto pred) -> int {
    // every thread has read any earlier value of s_n (the merged draw's
    // count, say) before thread 0 clears it
    __syncthreads();
    if (tid == 0) s_n = 0;
    __syncthreads();
    each([&](int v, float x) {
      if (!cand(v, x) || bin_of(x) != b || !pred(v, x)) return;
      const int i = atomicAdd(&s_n, 1);
      if (i < kSfCap) s_g[i] = ((uint64_t)okey(x) << 32) | (uint32_t)~(uint32_t)v;
    });
    __syncthreads();
    const int n = s_n;
    if (n > kSfCap) return n;
    sort_list(n);
    return n;
  };
  auto entry_key = [&](int i) { return (uint32_t)(s_g[i] >> 32); };
  auto entry_id = [&](int i) { return (int)~(uint32_t)s_g[i]; };

  // radix select among the candidates `in` admits: the first, in ranking
  // order, whose running count (use_mass false) or fixed-point mass reaches
  // `need`.  Four passes of 8-bit digits of the order-preserving key, then
  // the tied candidates (key == the selected key) share one value, so the
  // boundary is the c-th of them in id order, c = need left / their mass
  // (rounded up); a pass counts them per thread over contiguous id ranges.
  auto radix = [&](auto in, bool use_mass, uint64_t need, uint32_t& key_out, int& id_out) {
    uint32_t prefix = 0u, pmask = 0u;
    uint64_t rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSfThreads) s_h64[i] = 0ull;
      __syncthreads();
      each([&](int v, float x) {
        const uint32_t key = okey(x);
        if (!in(v, x) || (key & pmask) != prefix) return;
        atomicAdd(reinterpret_cast<unsigned long long*>(&s_h64[(key >> shift) & 255]),
                  (unsigned long long)(use_mass ? mass_of(x) : 1ull));
      });
      __syncthreads();
      uint64_t before, total;
      // slot i = digit 255 - i: from the largest digit down
      int sl = find_first([&](int i) { return s_h64[255 - i]; }, 256, rem, before, total);
      if (sl < 0) {      // not reachable: the need is within the admitted total
        sl = 0;
        before = 0ull;
      }
      rem -= before;
      prefix |= (uint32_t)(255 - sl) << shift;
      pmask |= 255u << shift;
    }
    const uint64_t w = use_mass ? mass_of(key_float(prefix)) : 1ull;
    uint64_t c = w == 0ull ? 1ull : (rem + w - 1ull) / w;
    c = c < 1ull ? 1ull : c;
    const int per = (V + kSfThreads - 1) / kSfThreads;
    const int v0 = tid * per, v1 = min(V, v0 + per);
    int cnt = 0;
    for (int v = v0; v < v1; ++v) {
      const float x = l[v];
      cnt += (in(v, x) && okey(x) == prefix) ? 1 : 0;
    }
    s_cnt[tid] = cnt;
    __syncthreads();
    uint64_t before, total;
    int t = find_first([&](int i) { return (uint64_t)s_cnt[i]; }, kSfThreads, c, before, total);
    if (t < 0) {       // fewer ties than c (not reachable): the last tie
      t = find_first([&](int i) { return (uint64_t)s_cnt[i]; }, kSfThreads, total, before, total);
      c = total;
    }
    if (tid == t) {
      uint64_t k = c - before;
      int idc = v0;
      for (int v = v0; v < v1; ++v) {
        const float x = l[v];
        if (!(in(v, x) && okey(x) == prefix)) continue;
        idc = v;
        if (--k == 0ull) break;
      }
      s_sel = idc;
    }
    __syncthreads();
    key_out = prefix;
    id_out = s_sel;
    __syncthreads();
  };

  // the top-p boundary among the n sorted candidates of its bin: the first
  // whose running mass reaches rem
  auto select_sorted = [&](int n, uint64_t rem, uint32_t& key_out, int& id_out) {
    uint64_t b2, t2;
    int e = find_first([&](int i) { return mass_of(key_float(entry_key(i))); }, n, rem, b2, t2);
    e = e < 0 ? max(n - 1, 0) : e;      // n >= 1: the bin has mass
    key_out = entry_key(e);
    id_out = entry_id(e);
  };

  // kept-set tests: key above the boundary key, or equal to it with id at
  // most the boundary id; key 0 with id V keeps everything
  uint32_t kk = 0u, pk = 0u;
  int kid = V, pid = V;
  auto keep_k = [&](int v, uint32_t key) { return v != mask && (key > kk || (key == kk && v <= kid)); };
  const bool use_k = a.top_k > 0 && a.top_k < V - 1;
  const bool use_p = a.top_p < 1.f;
  // one filter alone: its boundary bin and the mass (top-p) or the rank
  // (top-k) needed inside it, resolved during the draw pass (-1: not used)
  int mbin = -1, mrank = 0;
  uint64_t mrem = 0ull;

  if (use_k || use_p) {
    // ---- pass 2: the value-bin histogram
    for (int i = tid; i < kSfBins; i += kSfThreads) {
      s_bc[i] = 0u;
      s_bm[i] = 0ull;
    }
    __syncthreads();
    each([&](int v, float x) {
      if (!cand(v, x)) return;
      const int b = bin_of(x);
      if (use_k) atomicAdd(&s_bc[b], 1u);
      if (use_p) atomicAdd(reinterpret_cast<unsigned long long*>(&s_bm[b]),
                           (unsigned long long)mass_of(x));
    });
    __syncthreads();

    int bk = kSfBins, rk = 0, listed = -1;     // top-k boundary bin, rank in it, sorted bin
    if (use_k) {
      uint64_t before, total;
      const int b = find_first([&](int s) { return (uint64_t)s_bc[s]; }, kSfBins, (uint64_t)a.top_k,
                               before, total);
      if (b >= 0) {                            // else fewer candidates than top_k: keep all
        bk = b;
        rk = a.top_k - (int)before;
        if (!use_p) {
          mbin = bk;
          mrank = rk;
        } else {
        const int n = gather_sort(bk, [](int, float) { return true; });
        if (n <= kSfCap) {
          kk = entry_key(rk - 1);
          kid = entry_id(rk - 1);
          listed = bk;
        } else {
          radix([&](int v, float x) { return cand(v, x) && bin_of(x) == bk; }, false, (uint64_t)rk, kk,
                kid);
        }
        }
      }
    }
    if (use_p) {
      // mass of the kept part of the top-k boundary bin
      uint64_t massk = 0ull;
      if (bk < kSfBins) {
        uint64_t part = 0ull;
        if (listed == bk) {
          for (int i = tid; i < rk; i += kSfThreads) part += mass_of(key_float(entry_key(i)));
        } else {
          each([&](int v, float x) {
            if (cand(v, x) && bin_of(x) == bk && keep_k(v, okey(x))) part += mass_of(x);
          });
        }
        block_scan(part, massk);
      }
      auto pval = [&](int s) -> uint64_t { return s < bk ? s_bm[s] : (s == bk ? massk : 0ull); };
      uint64_t before, Z;
      find_first(pval, kSfBins, ~0ull, before, Z);          // the kept total
      uint64_t tgt = 0ull;
      if (a.top_p > 0.f) {
        const double t = ceil((double)a.top_p * (double)Z);
        tgt = t >= (double)Z ? Z : (uint64_t)t;
      }
      // >= 0: the maximum is kept and has mass 2^40
      const int bp = find_first(pval, kSfBins, tgt, before, Z);
      const uint64_t rem = tgt - before;
      int n = kSfCap + 1;
      if (!use_k) {
        mbin = bp;
        mrem = rem;
      } else {
      if (bp == bk && listed == bk) n = rk;                  // the sorted top-k part
      else if (bp != bk) n = gather_sort(bp, [](int, float) { return true; });
      if (n <= kSfCap) {
        select_sorted(n, rem, pk, pid);
      } else {
        radix([&](int v, float x) { return cand(v, x) && bin_of(x) == bp && keep_k(v, okey(x)); },
              true, rem, pk, pid);
      }
      }
    }
  }
  // both kept-set tests compare (key, id) in ranking order (higher key,
  // then lower id); as (key << 32 | ~id) that order is the unsigned one, so
  // the two tests are one 64-bit comparison with the larger boundary pair
  uint64_t thr = 0ull;
  auto set_thr = [&]() {
    thr = max(((uint64_t)kk << 32) | (uint32_t)~(uint32_t)kid,
              ((uint64_t)pk << 32) | (uint32_t)~(uint32_t)pid);
  };
  set_thr();
  auto keep = [&](int v, float x) {
    return cand(v, x) & ((((uint64_t)okey(x) << 32) | (uint32_t)~(uint32_t)v) >= thr);
  };

  // ---- pass 4: the block draw over the kept set (log2 units as the fused
  // sampler), and sum exp(l - m) over the candidates for the confidence
  float gbest = -INFINITY, s1 = 0.f;
  int cbest = 0x7fffffff;
  const int nchunk = (V + 31) / 32;

  // one 16-token half block of chunk c: x = its members' logits in log2
  // units, -inf where not kept; wu, we = its two Philox words
  auto draw_half = [&](const float (&x)[16], uint32_t wu, uint32_t we, int c, int h) {
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) bm = fmaxf(bm, x[i]);
    if (bm == -INFINITY) return;
    const float u = sf_uniform(wu);
    const float eg = sf_uniform(we);
    const float bmT = bm * invT;
    float e[16], S = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      e[i] = fast_exp2(fmaf(x[i], invT, -bmT));
      S += e[i];
    }
    // the running sums never decrease and target > 0, so the members whose
    // sum is below it are a prefix and the first member past it has weight;
    // if rounding leaves none past it, the last member with weight
    const float target = u * S;
    float cum = 0.f;
    int below = 0, last = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cum += e[i];
      below += cum < target ? 1 : 0;
      last = e[i] > 0.f ? i : last;
    }
    const int ci = below < 16 ? below : last;
    const float G = bmT + __log2f(S) - __log2f(-__log2f(eg));
    const int cnd = 32 * c + 8 * (ci >> 2) + 4 * h + (ci & 3);
    if (G > gbest || (G == gbest && cnd < cbest)) {
      gbest = G; cbest = cnd;
    }
  };

  // merged (one filter alone): the boundary bin mbin is not resolved yet.  Bins
  // are monotone in the logit, so members of lower bins are kept and members
  // of higher bins are not, as the final test will say; members of mbin go
  // into s_g, and a half block holding one is deferred to s_def until the
  // boundary inside mbin is known.
  uint32_t* const s_def = s_bc;                 // the count histogram is dead here
  auto draw = [&](bool merged) {
    for (int c = tid; c < nchunk; c += kSfThreads) {
      float lv[32];
      if ((V & 3) == 0 && 32 * c + 32 <= V) {
        const f32x4* p4 = reinterpret_cast<const f32x4*>(l + 32 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 x4 = p4[i];
          lv[4 * i] = x4.x; lv[4 * i + 1] = x4.y; lv[4 * i + 2] = x4.z; lv[4 * i + 3] = x4.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) lv[i] = 32 * c + i < V ? l[32 * c + i] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) s1 += cand(32 * c + i, lv[i]) ? fast_exp2((lv[i] - m) * kLog2e) : 0.f;
      uint32_t w0 = (uint32_t)c, w1 = rid, w2 = a.step, w3 = 0u;
      sf_philox(w0, w1, w2, w3, a.key0, a.key1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // half h: columns 32c + 8q + 4h + r'
        float x[16];
        bool pend = false;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2) {
            const int i = 8 * q + 4 * h + r2, v = 32 * c + i;
            bool kept;
            if (merged) {
              const bool cd = cand(v, lv[i]);
              const int bn = bin_of(lv[i]);
              kept = cd & (bn < mbin);
              if (cd & (bn == mbin)) {
                pend = true;
                const int k = atomicAdd(&s_n, 1);
                if (k < kSfCap) s_g[k] = ((uint64_t)okey(lv[i]) << 32) | (uint32_t)~(uint32_t)v;
              }
            } else {
              kept = keep(v, lv[i]);
            }
            x[4 * q + r2] = kept ? lv[i] * kLog2e : -INFINITY;
          }
        if (pend) {
          const int k = atomicAdd(&s_ndef, 1);
          if (k < kSfBins) s_def[k] = (uint32_t)(2 * c + h);
          continue;
        }
        draw_half(x, h ? w2 : w0, h ? w3 : w1, c, h);
      }
    }
  };

  if (mbin < 0) {
    draw(false);
  } else {
    if (tid == 0) {
      s_n = 0;
      s_ndef = 0;
    }
    __syncthreads();
    draw(true);
    __syncthreads();
    const int n = s_n, nd = s_ndef;
    if (n <= kSfCap && nd <= kSfBins) {
      sort_list(n);
      if (use_k) {                              // n >= mrank: the bin holds the top_k-th
        const int e = max(min(mrank, n) - 1, 0);
        kk = entry_key(e);
        kid = entry_id(e);
      } else {
        select_sorted(n, mrem, pk, pid);
      }
      set_thr();
      for (int j = tid; j < nd; j += kSfThreads) {
        const int c = (int)(s_def[j] >> 1), h = (int)(s_def[j] & 1u);
        uint32_t w0 = (uint32_t)c, w1 = rid, w2 = a.step, w3 = 0u;
        sf_philox(w0, w1, w2, w3, a.key0, a.key1);
        float x[16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2) {
            const int v = 32 * c + 8 * q + 4 * h + r2;
            const float xv = v < V ? l[v] : -INFINITY;
            x[4 * q + r2] = keep(v, xv) ? xv * kLog2e : -INFINITY;
          }
        draw_half(x, h ? w2 : w0, h ? w3 : w1, c, h);
      }
    } else {
      // the boundary bin did not fit in LDS: resolve it as with top-k and
      // draw the row again
      const int n2 = gather_sort(mbin, [](int, float) { return true; });
      if (use_k) {
        if (n2 <= kSfCap) {
          const int e = max(min(mrank, n2) - 1, 0);
          kk = entry_key(e);
          kid = entry_id(e);
        } else {
          radix([&](int v, float x) { return cand(v, x) && bin_of(x) == mbin; }, false, (uint64_t)mrank, kk,
                kid);
        }
      } else if (n2 <= kSfCap) {
        select_sorted(n2, mrem, pk, pid);
      } else {
        radix([&](int v, float x) { return cand(v, x) && bin_of(x) == mbin; }, true, mrem, pk, pid);
      }
      set_thr();
      gbest = -INFINITY;
      cbest = 0x7fffffff;
      s1 = 0.f;
      draw(false);
    }
  }
  const float S1 = block_reduce(s1, [](float x, float y) { return x + y; }, s_f);
  // argmax of (G, lower candidate) over the workgroup
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float g2 = __shfl_xor(gbest, off, 64);
    const int c2i = __shfl_xor(cbest, off, 64);
    if (g2 > gbest || (g2 == gbest && c2i < cbest)) { gbest = g2; cbest = c2i; }
  }
  if (lane == 0) {
    s_gbest[wave] = gbest;
    s_cbest[wave] = cbest;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSfWaves; ++w)
      if (s_gbest[w] > gbest || (s_gbest[w] == gbest && s_cbest[w] < cbest)) {
        gbest = s_gbest[w]; cbest = s_cbest[w];
      }
    // the drawn token's own logit (a kept token always exists: the kept
    // set holds at least the row maximum)
    const float lb = cbest < V ? l[cbest] : -INFINITY;
    a.token[rid] = cbest;
    a.conf[rid] = __expf(lb - m) / S1;
  }
}

hipError_t sample_filtered_launch(const SampleArgs& a, hipStream_t st) {
  sample_filtered_kernel<<<a.max_rows, kSfThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
