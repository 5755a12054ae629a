// Top-k / top-p filtered sampling from stored logits, gfx950.
//
// The pages' SamplingParams carry topk and topp besides the temperature
// (JetEngine README usage examples), and the developer notes found a
// separate sampler after the logits faster than a fused one ("Ruled-Out
// Optimizations").  Here the LM head stores the listed rows' logits
// (lmhead_tile_kernel, store mode) and this kernel draws each row's token:
//   * candidates are the finite logits other than the mask token's, ranked
//     by logit, higher first, the lower id first among equal logits (-0 and
//     +0 are equal);
//   * top_k > 0 keeps the first top_k; top_p < 1 then keeps the shortest
//     leading run of those whose running sum of exp((l - m)/T) reaches
//     top_p of their total (at least one token);
//   * the token is drawn from softmax(l/T) over the kept set with the same
//     block draw as the fused sampler (Philox4x32-10, counter (chunk, row,
//     step, 0); per 16-column block an inverse-CDF candidate and a Gumbel
//     value at the block's log-sum-exp; the largest Gumbel wins, the lower
//     candidate on equal values), the other tokens having zero weight; the
//     confidence is the drawn token's probability at temperature 1.  A row
//     without a candidate gets the mask token with confidence 0.
//
// One workgroup of 512 threads per listed row, two workgroups per CU, so
// that one row's scans and barriers overlap another row's streaming.
// Passes over the row:
//   1. the row maximum m (read from the LM head's partial row maxima when
//      the caller passes them: the round does);
//   2. (filters only) a histogram over 4096 value bins below m: with
//      d = (m - x) log2(e) / T * 128, bin = floor(d), the last bin
//      taking everything further down (below 2^-32 of the maximum's mass;
//      its members are summed in registers, so they do not all queue on
//      one LDS address).  Per bin: the candidate count (top-k), and the sum
//      of the members' masses exp((x - m)/T) in units of 2^-31 of the bin's
//      upper edge, floor(2^(31 - frac(d)/128)) each (top-p).  The sums are
//      integers, so they do not depend on the order of the atomic adds; a
//      bin's mass relative to the maximum's is its sum times
//      2^(-31 - bin/128), and the scans add those in float64 in a fixed
//      order.  The pass also sums exp(x - m) for the confidence;
//   3. a scan over the bins finds the bin holding a boundary (the top_k-th
//      candidate, or the first candidate whose running mass reaches top_p
//      of the kept total).  With one filter alone the boundary inside that
//      bin is found during the draw (below); with both, one more pass
//      gathers the bin's candidates into LDS as (key, ~id), a bitonic sort
//      puts them in ranking order and a scan over them gives the boundary.
//      A bin of more than 2048 candidates (long runs of equal logits,
//      extreme temperatures) is resolved by a radix select over the
//      order-preserving 32-bit image of its logits (8-bit digits, four
//      passes, then a pass in id order for ties);
//   4. the draw, one 32-token chunk (both of its blocks) per thread at a
//      time: per block S = the sum over its kept members of
//      exp((x - m)/T) (the row maximum as the common reference, so no block
//      maximum is needed) and G = log2 S + a Gumbel variable from the
//      block's Philox word; the largest G wins (the lower block on equal
//      values), and only the winning block's inverse CDF is evaluated, at
//      the end.  With one filter alone a block holding a member of the
//      boundary bin is deferred (per-wave lists, one ballot per block, the
//      block's 16 logits staged in LDS while there is room); after the pass
//      the bin's members are gathered from the deferred blocks into LDS,
//      sorted, the boundary found, and the deferred blocks drawn.  Without
//      a filter this pass also sums exp(x - m) for the confidence.
// Without a filter only passes 1 and 4 run.
#include <climits>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

constexpr int kSfThreads = 512;
constexpr int kSfWaves = kSfThreads / 64;
constexpr int kSfBins = 4096;                  // value bins below the row maximum
constexpr int kSfPer = kSfBins / kSfThreads;   // scan slots per thread
constexpr float kSfBinsPerLog2 = 128.f;        // bins per unit of (m - l) log2(e) / T: the
                                               // bins reach 2^-32 of the maximum's mass
constexpr int kSfCap = 2048;                   // candidates of one bin sorted in LDS
constexpr int kSfWaveDef = kSfBins / kSfWaves; // a wave's deferred blocks
constexpr int kSfWaveStage = kSfBins * 2 / 16 / kSfWaves;   // of those, kept in LDS (64)
constexpr float kSfUnitLog2 = 31.f;            // a member's mass: 2^31 at its bin's upper edge
constexpr float kFltMax = 3.402823466e38f;

template <bool B>
struct Tag {
  static constexpr bool value = B;
};

// order-preserving image of a float (-0 taken as +0)
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t b = __float_as_uint(f + 0.f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // larger float -> larger key
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t rank_pair(float x, int v) {
  return ((uint64_t)okey(x) << 32) | (uint32_t)~(uint32_t)v;
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
__device__ __forceinline__ uint64_t to_bits(uint64_t v) { return v; }
__device__ __forceinline__ uint64_t to_bits(double v) { return (uint64_t)__double_as_longlong(v); }
__device__ __forceinline__ void from_bits(uint64_t b, uint64_t& v) { v = b; }
__device__ __forceinline__ void from_bits(uint64_t b, double& v) { v = __longlong_as_double((long long)b); }

// lanes below this one with a set bit in `bal`
__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// block-wide reduction over the workgroup through LDS
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

// the 16 members of block h of a chunk's 32 logits, in member order j
// (offset 8(j/4) + 4h + j%4 in the chunk)
__device__ __forceinline__ void half_of(const float (&lv)[32], int h, float (&x)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * q + r] = lv[8 * q + 4 * h + r];
}

}  // namespace

__global__ __launch_bounds__(kSfThreads, 4) void sample_filtered_kernel(SampleArgs a) {
  __shared__ uint32_t s_bc[kSfBins];     // candidates per bin; then the deferred blocks
  __shared__ uint64_t s_bm[kSfBins];     // mass per bin in its own units
  __shared__ uint64_t s_g[kSfCap];       // one bin's candidates, (key << 32) | ~id
  __shared__ uint64_t s_w[kSfWaves];
  __shared__ float s_f[kSfWaves];
  __shared__ int s_n, s_first, s_sel, s_last;
  __shared__ uint64_t s_before;
  __shared__ float s_gbest[kSfWaves];
  __shared__ int s_kbest[kSfWaves], s_wd[kSfWaves];
  // radix-select scratch on top of s_g: it runs only when a bin did not fit
  uint64_t* const s_h64 = s_g;                                        // [256]
  int* const s_cnt = reinterpret_cast<int*>(s_g + 256);               // [kSfThreads]
  static_assert(256 * 8 + kSfThreads * 4 <= kSfCap * 8, "radix scratch must fit in the gather buffer");
  uint32_t* const s_def = s_bc;          // the count histogram is dead by the draw
  float* const s_stage = reinterpret_cast<float*>(s_bm);   // so are the masses: deferred blocks

  const int r = blockIdx.x;
  if (r >= *a.num_rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, mask = a.mask_id;
  const float* l = a.logits + (size_t)r * V;
  const uint32_t rid = (uint32_t)(a.row_index ? a.row_index[r] : r);
  const float invT = a.inv_temp;
  const bool vec = (V & 3) == 0;         // rows 16-byte aligned
  auto fin = [](float x) { return fabsf(x) <= kFltMax; };

  // every logit of the row once, the mask token's as NaN (no candidate);
  // with 16-byte aligned rows each thread keeps eight 16-byte loads in
  // flight, the next four issued before the current four are used.  With
  // rev the row is walked from its end: the histogram pass does, so that it
  // starts on what the pass before it read last (still in the caches)
  auto each = [&](auto fn, bool rev = false) {
    if (vec) {
      const f32x4* l4 = reinterpret_cast<const f32x4*>(l);
      const int n4 = V >> 2, qm = mask >> 2, jm = mask & 3;
      auto fn4 = [&](int q, f32x4 x) {
        if (q == qm) {
          x.x = jm == 0 ? NAN : x.x;
          x.y = jm == 1 ? NAN : x.y;
          x.z = jm == 2 ? NAN : x.z;
          x.w = jm == 3 ? NAN : x.w;
        }
        fn(4 * q, x.x); fn(4 * q + 1, x.y); fn(4 * q + 2, x.z); fn(4 * q + 3, x.w);
      };
      constexpr int U = 4;
      int q = tid;
      f32x4 cur[U];
      bool full = q + (U - 1) * kSfThreads < n4;
      if (full) {
#pragma unroll
        for (int j = 0; j < U; ++j) cur[j] = l4[rev ? n4 - 1 - (q + j * kSfThreads) : q + j * kSfThreads];
      }
      while (full) {
        const int qn = q + U * kSfThreads;
        const bool nfull = qn + (U - 1) * kSfThreads < n4;
        f32x4 nx[U];
        if (nfull) {
#pragma unroll
          for (int j = 0; j < U; ++j) nx[j] = l4[rev ? n4 - 1 - (qn + j * kSfThreads) : qn + j * kSfThreads];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) fn4(rev ? n4 - 1 - (q + j * kSfThreads) : q + j * kSfThreads, cur[j]);
#pragma unroll
        for (int j = 0; j < U; ++j) cur[j] = nx[j];
        q = qn;
        full = nfull;
      }
      for (; q < n4; q += kSfThreads) fn4(rev ? n4 - 1 - q : q, l4[rev ? n4 - 1 - q : q]);
    } else {
      for (int v = tid; v < V; v += kSfThreads) {
        const float x = l[v];
        fn(v, v == mask ? NAN : x);
      }
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
    each([&](int, float x) {
      if (fin(x)) mt = fmaxf(mt, x);
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

  const float c2 = invT * kLog2e;               // exp((l - m)/T) = 2^(l c2 - m c2)
  const float c3 = c2 * kSfBinsPerLog2;
  const float mc2 = m * c2, ml = m * kLog2e;
  auto bin_d = [&](float x) { return fmaxf((m - x) * c3, 0.f); };        // monotone in x, +inf at -inf
  auto bin_of = [&](float x) -> int { return (int)fminf(floorf(bin_d(x)), (float)(kSfBins - 1)); };
  // a candidate's mass in units of 2^-31 of its bin's upper edge
  auto mass_in_bin = [&](float x) -> uint32_t {
    const float d = bin_d(x);
    const float bf = fminf(floorf(d), (float)(kSfBins - 1));
    return (uint32_t)fast_exp2(fmaf(d - bf, -1.f / kSfBinsPerLog2, kSfUnitLog2));
  };
  // one unit of bin b relative to the maximum's mass
  auto bin_scale = [](int b) -> double {
    return exp2(-(double)b / (double)kSfBinsPerLog2 - (double)kSfUnitLog2);
  };
  // the largest finite float whose bin is at least b (FLT_MAX when every
  // one is): bin_of(x) < b exactly when x is above it
  auto bin_floor = [&](int b) -> float {
    if (bin_of(kFltMax) >= b) return kFltMax;
    uint32_t lo = okey(-kFltMax), hi = okey(kFltMax);
    while (hi - lo > 1u) {                    // bin_of(key_float(lo)) >= b > bin_of(key_float(hi))
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (bin_of(key_float(mid)) >= b) lo = mid;
      else hi = mid;
    }
    return key_float(lo);
  };

  // exclusive prefix over the workgroup (thread order) of a value held per
  // thread, uint64_t or double; `total` = the sum over all threads.  The
  // additions run in a fixed order, so double sums are the same on every run.
  auto block_scan = [&](auto v, auto& total) {
    using T = decltype(v);
    T x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      T y;
      from_bits(shfl_u64(to_bits(x), lane >= off ? lane - off : lane), y);
      if (lane >= off) x += y;
    }
    T excl;
    from_bits(shfl_u64(to_bits(x), lane > 0 ? lane - 1 : 0), excl);
    if (lane == 0) excl = T(0);
    __syncthreads();
    if (lane == 63) s_w[wave] = to_bits(x);
    __syncthreads();
    T run = T(0), tot = T(0);
    for (int w = 0; w < kSfWaves; ++w) {
      T t;
      from_bits(s_w[w], t);
      if (w < wave) run += t;
      tot += t;
    }
    total = tot;
    return run + excl;
  };

  // first slot s of [0, n) (kSfPer per thread, thread-major) with val(s) > 0
  // whose inclusive running sum reaches tgt, or -1; `before` = the running
  // sum ahead of it, `total` = the sum of all slots
  auto find_first = [&](auto val, int n, auto tgt, auto& before, auto& total) -> int {
    using T = decltype(tgt);
    T v[kSfPer], sum = T(0);
#pragma unroll
    for (int j = 0; j < kSfPer; ++j) {
      const int s = kSfPer * tid + j;
      v[j] = s < n ? val(s) : T(0);
      sum += v[j];
    }
    if (tid == 0) s_first = INT_MAX;
    T run = block_scan(sum, total);
    int mine = -1;
    T mb = T(0);
#pragma unroll
    for (int j = 0; j < kSfPer; ++j) {
      if (mine < 0 && v[j] > T(0) && run + v[j] >= tgt) {
        mine = kSfPer * tid + j;
        mb = run;
      }
      run += v[j];
    }
    if (mine >= 0) atomicMin(&s_first, mine);
    __syncthreads();
    const int f = s_first;
    if (mine >= 0 && mine == f) s_before = to_bits(mb);
    __syncthreads();
    from_bits(s_before, before);
    __syncthreads();
    return f == INT_MAX ? -1 : f;
  };

  // list[0, n) (n <= kSfCap) into ranking order (descending pairs) by a
  // bitonic sort
  auto sort_list = [&](uint64_t* list, int n) {
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = n + tid; i < n2; i += kSfThreads) list[i] = 0ull;   // below every candidate
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kSfThreads) {
          const int p = i ^ j;
          if (p > i) {
            const uint64_t x = list[i], y = list[p];
            if ((i & k) == 0 ? x < y : x > y) {
              list[i] = y;
              list[p] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  };
  // the candidates of bin b that pred admits, into s_g in ranking order;
  // returns their number, > kSfCap if they did not fit (s_g then holds no
  // list)
  auto gather_sort = [&](int b, auto pred) -> int {
    // every thread has read any earlier value of s_n before thread 0
    // clears it
    __syncthreads();
    if (tid == 0) s_n = 0;
    __syncthreads();
    each([&](int v, float x) {
      if (!fin(x) || bin_of(x) != b || !pred(v, x)) return;
      const int i = atomicAdd(&s_n, 1);
      if (i < kSfCap) s_g[i] = rank_pair(x, v);
    });
    __syncthreads();
    const int n = s_n;
    if (n > kSfCap) return n;
    sort_list(s_g, n);
    return n;
  };
  auto entry_key = [&](int i) { return (uint32_t)(s_g[i] >> 32); };
  auto entry_id = [&](int i) { return (int)~(uint32_t)s_g[i]; };

  // radix select among the candidates `in` admits (all in one bin): the
  // first, in ranking order, whose running count (use_mass false) or mass in
  // the bin's units reaches `need`.  Four passes of 8-bit digits of the
  // order-preserving key, then the tied candidates (key == the selected key)
  // share one value, so the boundary is the c-th of them in id order,
  // c = need left / their mass (rounded up); a pass counts them per thread
  // over contiguous id ranges.
  auto radix = [&](auto in, bool use_mass, uint64_t need, uint32_t& key_out, int& id_out) {
    uint32_t prefix = 0u, pmask = 0u;
    uint64_t rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSfThreads) s_h64[i] = 0ull;
      __syncthreads();
      each([&](int v, float x) {
        if (!fin(x)) return;
        const uint32_t key = okey(x);
        if (!in(v, x) || (key & pmask) != prefix) return;
        atomicAdd(reinterpret_cast<unsigned long long*>(&s_h64[(key >> shift) & 255]),
                  (unsigned long long)(use_mass ? mass_in_bin(x) : 1u));
      });
      __syncthreads();
      uint64_t before, total;
      // slot i = digit 255 - i: from the largest digit down
      int sl = find_first([&](int i) -> uint64_t { return s_h64[255 - i]; }, 256, rem, before, total);
      if (sl < 0) {      // not reachable: the need is within the admitted total
        sl = 0;
        before = 0ull;
      }
      rem -= before;
      prefix |= (uint32_t)(255 - sl) << shift;
      pmask |= 255u << shift;
    }
    const uint64_t w = use_mass ? mass_in_bin(key_float(prefix)) : 1ull;
    uint64_t c = w == 0ull ? 1ull : (rem + w - 1ull) / w;
    c = c < 1ull ? 1ull : c;
    const int per = (V + kSfThreads - 1) / kSfThreads;
    const int v0 = tid * per, v1 = min(V, v0 + per);
    auto tie = [&](int v) {
      const float x = l[v];
      return v != mask && fin(x) && in(v, x) && okey(x) == prefix;
    };
    int cnt = 0;
    for (int v = v0; v < v1; ++v) cnt += tie(v) ? 1 : 0;
    s_cnt[tid] = cnt;
    __syncthreads();
    uint64_t before, total;
    int t = find_first([&](int i) -> uint64_t { return (uint64_t)s_cnt[i]; }, kSfThreads, c, before, total);
    if (t < 0) {       // fewer ties than c (not reachable): the last tie
      t = find_first([&](int i) -> uint64_t { return (uint64_t)s_cnt[i]; }, kSfThreads, total, before, total);
      c = total;
    }
    if (tid == t) {
      uint64_t k = c - before;
      int idc = v0;
      for (int v = v0; v < v1; ++v) {
        if (!tie(v)) continue;
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

  // the boundary among the n sorted candidates of one bin: the first whose
  // running mass (in the bin's units) reaches need
  auto select_sorted = [&](int n, uint64_t need, uint32_t& key_out, int& id_out) {
    uint64_t b2, t2;
    int e = find_first([&](int i) -> uint64_t { return mass_in_bin(key_float(entry_key(i))); }, n, need, b2,
                       t2);
    e = e < 0 ? max(n - 1, 0) : e;      // n >= 1: the bin has mass
    key_out = entry_key(e);
    id_out = entry_id(e);
  };

  // boundary pairs (key, id) of each filter: a candidate is kept when its
  // pair is at least the boundary's in ranking order; key 0 keeps all
  uint32_t kk = 0u, pk = 0u;
  int kid = V, pid = V;
  auto keep_k = [&](int v, float x) {
    const uint32_t key = okey(x);
    return key > kk || (key == kk && v <= kid);
  };
  const bool use_k = a.top_k > 0 && a.top_k < V - 1;
  const bool use_p = a.top_p < 1.f;
  // one filter alone: its boundary bin and the rank (top-k) or the mass in
  // the bin's units (top-p) needed inside it, resolved during the draw pass
  // (-1: not used)
  int mbin = -1, mrank = 0;
  uint64_t mrem = 0ull;
  float s1 = 0.f;                        // sum over the candidates of exp(l - m)

  if (use_k || use_p) {
    // ---- pass 2: the value-bin histogram, and the confidence's sum
    for (int i = tid; i < kSfBins; i += kSfThreads) {
      s_bc[i] = 0u;
      s_bm[i] = 0ull;
    }
    __syncthreads();
    // a non-candidate enters as -inf: no exp(x - m), no mass, no count.  The
    // last bin (everything further down) can hold most of a row: its
    // members are summed in registers and added once per thread, so they
    // do not all queue on one LDS address.
    auto hist = [&](auto with_k, auto with_p) {
      uint32_t tail_n = 0u;
      uint64_t tail_m = 0ull;
      each([&](int, float x) {
        const bool cd = fin(x);
        const float xs = cd ? x : -INFINITY;
        s1 += fast_exp2(fmaf(xs, kLog2e, -ml));
        const float d = bin_d(xs);
        const float bf = fminf(floorf(d), (float)(kSfBins - 1));
        const int b = (int)bf;
        const uint32_t u = (uint32_t)fast_exp2(fmaf(d - bf, -1.f / kSfBinsPerLog2, kSfUnitLog2));
        if (b < kSfBins - 1) {
          if constexpr (decltype(with_k)::value) atomicAdd(&s_bc[b], cd ? 1u : 0u);
          if constexpr (decltype(with_p)::value)
            atomicAdd(reinterpret_cast<unsigned long long*>(&s_bm[b]), (unsigned long long)u);
        } else {
          tail_n += cd ? 1u : 0u;
          tail_m += u;
        }
      }, true);
      if constexpr (decltype(with_k)::value)
        if (tail_n) atomicAdd(&s_bc[kSfBins - 1], tail_n);
      if constexpr (decltype(with_p)::value)
        if (tail_m) atomicAdd(reinterpret_cast<unsigned long long*>(&s_bm[kSfBins - 1]), (unsigned long long)tail_m);
    };
    if (use_k && use_p) hist(Tag<true>{}, Tag<true>{});
    else if (use_k) hist(Tag<true>{}, Tag<false>{});
    else hist(Tag<false>{}, Tag<true>{});
    __syncthreads();

    int bk = kSfBins, rk = 0, listed = -1;     // top-k boundary bin, rank in it, sorted bin
    if (use_k) {
      uint64_t before, total;
      const int b = find_first([&](int s) -> uint64_t { return s_bc[s]; }, kSfBins, (uint64_t)a.top_k, before,
                               total);
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
            radix([&](int, float x) { return bin_of(x) == bk; }, false, (uint64_t)rk, kk, kid);
          }
        }
      }
    }
    if (use_p) {
      // mass of the kept part of the top-k boundary bin, in its units
      uint64_t massk = 0ull;
      if (bk < kSfBins) {
        uint64_t part = 0ull;
        if (listed == bk) {
          for (int i = tid; i < rk; i += kSfThreads) part += mass_in_bin(key_float(entry_key(i)));
        } else {
          each([&](int v, float x) {
            if (fin(x) && bin_of(x) == bk && keep_k(v, x)) part += mass_in_bin(x);
          });
        }
        block_scan(part, massk);
      }
      auto units = [&](int s) -> uint64_t { return s < bk ? s_bm[s] : (s == bk ? massk : 0ull); };
      auto pval = [&](int s) -> double { return (double)units(s) * bin_scale(s); };
      double before, Z;
      find_first(pval, kSfBins, (double)INFINITY, before, Z);      // the kept total
      const double tgt = a.top_p > 0.f ? fmin((double)a.top_p * Z, Z) : 0.0;
      int bp = find_first(pval, kSfBins, tgt, before, Z);
      uint64_t rem;
      if (bp >= 0) {
        const uint64_t u = units(bp);
        const double need = ceil((tgt - before) / bin_scale(bp));
        rem = need < 1.0 ? 1ull : (need >= (double)u ? u : (uint64_t)need);
      } else {
        // the running sums fell short of a target equal to the total by
        // rounding: the boundary is the last candidate with mass
        if (tid == 0) s_last = -1;
        __syncthreads();
        int lastb = -1;
        for (int s = tid; s < kSfBins; s += kSfThreads)
          if (units(s) > 0ull) lastb = s;
        if (lastb >= 0) atomicMax(&s_last, lastb);
        __syncthreads();
        bp = max(s_last, 0);                   // >= 0: the maximum has mass
        rem = units(bp);
        __syncthreads();
      }
      if (!use_k) {
        mbin = bp;
        mrem = rem;
      } else {
        int n = kSfCap + 1;
        if (bp == bk && listed == bk) n = rk;                  // the sorted top-k part
        else if (bp != bk) n = gather_sort(bp, [](int, float) { return true; });
        if (n <= kSfCap) {
          select_sorted(n, rem, pk, pid);
        } else {
          radix([&](int v, float x) { return bin_of(x) == bp && keep_k(v, x); }, true, rem, pk, pid);
        }
      }
    }
  }

  // ---- pass 4: the block draw
  const bool s1_in_draw = !(use_k || use_p);
  float gbest = -INFINITY;
  int kbest = INT_MAX;                   // 2c + h of the best block
  // the final kept test: both boundaries are lower bounds in ranking order,
  // so the larger pair decides, compared as a float with the id breaking
  // ties
  // Outside the chunk holding the boundary's id the test is one compare:
  // ties at xb are all kept (ids below the boundary's) or all dropped
  // (above), and x >= xb is x > xb_below, the float just below xb.
  float xb = -INFINITY, xb_below = -INFINITY;
  int idb = -1;
  auto set_final = [&]() {
    const uint64_t thr = max(((uint64_t)kk << 32) | (uint32_t)~(uint32_t)kid,
                             ((uint64_t)pk << 32) | (uint32_t)~(uint32_t)pid);
    if ((thr >> 32) == 0ull) {           // no boundary: every candidate
      xb = -INFINITY;
      xb_below = -INFINITY;
      idb = -1;
    } else {
      xb = key_float((uint32_t)(thr >> 32));
      const uint32_t u = __float_as_uint(xb);
      xb_below = __uint_as_float(u == 0u ? 0x80000001u : (xb > 0.f ? u - 1u : u + 1u));
      idb = (int)~(uint32_t)thr;
    }
  };
  set_final();
  // merged: members of bins below mbin are kept, those of bins above it are
  // not, as the final test will say; bin_of(x) < mbin exactly when x > t_lo,
  // bin_of(x) <= mbin exactly when x > t_hi
  float t_lo = kFltMax, t_hi = -INFINITY;
  if (mbin >= 0) {
    t_lo = bin_floor(mbin);
    t_hi = mbin + 1 < kSfBins ? bin_floor(mbin + 1) : -INFINITY;
  }

  const int nchunk = (V + 31) >> 5;
  const int cmask = mask >> 5, imask = mask & 31;
  auto philox_chunk = [&](int c, uint32_t (&w)[4]) {
    w[0] = (uint32_t)c; w[1] = rid; w[2] = a.step; w[3] = 0u;
    sf_philox(w[0], w[1], w[2], w[3], a.key0, a.key1);
  };
  // the final kept test for member x at offset i of its chunk, dv = idb - 32c
  auto kept_final = [&](float x, int i, int dv) {
    return fin(x) & ((x > xb) | ((x == xb) & (i <= dv)));
  };
  // S of block (c, h) under the final test, its 16 members x in member
  // order j (token 32c + 8(j/4) + 4h + j%4), summed in that order
  auto half_sum16 = [&](const float (&x)[16], int c, int h) {
    const int dv = idb - 32 * c;
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = 8 * (j >> 2) + 4 * h + (j & 3);
      S += kept_final(x[j], i, dv) ? fast_exp2(fmaf(x[j], c2, -mc2)) : 0.f;
    }
    return S;
  };
  auto gumbel = [&](float S, uint32_t we) {
    return __log2f(S) - __log2f(-__log2f(sf_uniform(we)));
  };
  auto consider = [&](float S, uint32_t we, int k) {
    if (S > 0.f) {
      const float G = gumbel(S, we);
      if (G > gbest || (G == gbest && k < kbest)) {
        gbest = G;
        kbest = k;
      }
    }
  };
  // one chunk's 32 logits from memory (NaN past the row's end: no candidate)
  auto load_chunk = [&](int c, float (&lv)[32]) {
    if (vec && 32 * c + 32 <= V) {
      const f32x4* p4 = reinterpret_cast<const f32x4*>(l + 32 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 x4 = p4[i];
        lv[4 * i] = x4.x; lv[4 * i + 1] = x4.y; lv[4 * i + 2] = x4.z; lv[4 * i + 3] = x4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) lv[i] = 32 * c + i < V ? l[32 * c + i] : NAN;
    }
  };
  // the mask token is no candidate
  auto unmask = [&](int c, float (&lv)[32]) {
    if (c == cmask) {
#pragma unroll
      for (int i = 0; i < 32; ++i) lv[i] = i == imask ? NAN : lv[i];
    }
  };

  int wd = 0;                            // this wave's deferred blocks
  auto draw_chunk = [&](auto merged, int c, float (&lv)[32]) {
    unmask(c, lv);
    // candidates only: everything else as -inf (weight 0, never kept)
#pragma unroll
    for (int i = 0; i < 32; ++i) lv[i] = fin(lv[i]) ? lv[i] : -INFINITY;
    if (s1_in_draw) {
#pragma unroll
      for (int i = 0; i < 32; ++i) s1 += fast_exp2(fmaf(lv[i], kLog2e, -ml));
    }
    uint32_t w[4];
    philox_chunk(c, w);
    const int dv = idb - 32 * c;
    const bool mixed = dv >= 0 && dv < 31;         // ties on both sides of the boundary id
    const float thr = dv < 0 ? xb : xb_below;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float S = 0.f;
      bool pend = false;
      if constexpr (decltype(merged)::value) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2) {
            const int i = 8 * q + 4 * h + r2;
            const float x = lv[i];
            const bool kept = x > t_lo;
            pend |= !kept & (x > t_hi);
            S += kept ? fast_exp2(fmaf(x, c2, -mc2)) : 0.f;
          }
        const uint64_t dbal = __ballot(pend);
        if (dbal != 0ull) {
          if (pend) {
            const int slot = wd + lanes_below(dbal);
            if (slot < kSfWaveDef) s_def[wave * kSfWaveDef + slot] = (uint32_t)(2 * c + h);
            if (slot < kSfWaveStage) {
              float x16[16];
              half_of(lv, h, x16);
              f32x4* st = reinterpret_cast<f32x4*>(s_stage + (wave * kSfWaveStage + slot) * 16);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                st[q] = f32x4{x16[4 * q], x16[4 * q + 1], x16[4 * q + 2], x16[4 * q + 3]};
            }
          }
          wd += (int)__popcll(dbal);
        }
        if (pend) continue;
      } else {
        if (mixed) {
          float x16[16];
          half_of(lv, h, x16);
          S = half_sum16(x16, c, h);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
              const float x = lv[8 * q + 4 * h + r2];
              S += x > thr ? fast_exp2(fmaf(x, c2, -mc2)) : 0.f;
            }
        }
      }
      consider(S, h ? w[3] : w[1], 2 * c + h);
    }
  };
  // every chunk once, one per thread at a time
  auto draw = [&](auto merged) {
    for (int c = tid; c < nchunk; c += kSfThreads) {
      float lv[32];
      load_chunk(c, lv);
      draw_chunk(merged, c, lv);
    }
  };
  // the 16 members of block (c, h) in member order, as the draw sees them
  // (NaN past the row's end and at the mask token)
  auto load_half = [&](int c, int h, float (&x)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v0 = 32 * c + 8 * q + 4 * h;
      if (vec && v0 + 4 <= V) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(l + v0);
        x[4 * q] = x4.x; x[4 * q + 1] = x4.y; x[4 * q + 2] = x4.z; x[4 * q + 3] = x4.w;
      } else {
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) x[4 * q + r2] = v0 + r2 < V ? l[v0 + r2] : NAN;
      }
#pragma unroll
      for (int r2 = 0; r2 < 4; ++r2) x[4 * q + r2] = v0 + r2 == mask ? NAN : x[4 * q + r2];
    }
  };
  // deferred block j of wave w: from LDS when it was staged
  auto deferred_half = [&](int w, int j, int c, int h, float (&x)[16]) {
    if (j < kSfWaveStage) {
      const f32x4* st = reinterpret_cast<const f32x4*>(s_stage + (w * kSfWaveStage + j) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = st[q];
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
      }
    } else {
      load_half(c, h, x);
    }
  };
  // a deferred block, or one evaluated again, under the final test
  auto half_G_final = [&](int c, int h, float& S) {
    float x[16];
    load_half(c, h, x);
    uint32_t w[4];
    philox_chunk(c, w);
    S = half_sum16(x, c, h);
    return h ? w[3] : w[1];
  };

  // fn(w, j) for every deferred block, the waves' lists taken as one list
  // of which each thread takes every kSfThreads-th entry
  auto for_deferred = [&](auto fn) {
    int pre[kSfWaves + 1];
    pre[0] = 0;
#pragma unroll
    for (int w = 0; w < kSfWaves; ++w) pre[w + 1] = pre[w] + s_wd[w];
    for (int f = tid; f < pre[kSfWaves]; f += kSfThreads) {
      int w = 0, j = f;
#pragma unroll
      for (int ww = 1; ww < kSfWaves; ++ww)
        if (f >= pre[ww]) {
          w = ww;
          j = f - pre[ww];
        }
      fn(w, j);
    }
  };

  if (mbin < 0) {
    draw(Tag<false>{});
  } else {
    // the histogram's arrays become the deferred list and the staging
    // area: every thread is done reading them
    __syncthreads();
    draw(Tag<true>{});
    if (lane == 0) s_wd[wave] = wd;
    __syncthreads();
    bool ovf = false;
    for (int w = 0; w < kSfWaves; ++w) ovf |= s_wd[w] > kSfWaveDef;
    if (!ovf) {
      // every member of the boundary bin lies in a deferred block: gather
      // them from those blocks' re-read logits, then ranking order
      if (tid == 0) s_n = 0;
      __syncthreads();
      for_deferred([&](int w, int j) {
        const uint32_t k = s_def[w * kSfWaveDef + j];
        const int c = (int)(k >> 1), h = (int)(k & 1u);
        float x16[16];
        deferred_half(w, j, c, h, x16);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float x = x16[jj];
          if (fin(x) && !(x > t_lo) && x > t_hi) {
            const int e = atomicAdd(&s_n, 1);
            if (e < kSfCap) s_g[e] = rank_pair(x, 32 * c + 8 * (jj >> 2) + 4 * h + (jj & 3));
          }
        }
      });
      __syncthreads();
      const int n = s_n;
      if (n <= kSfThreads) {
        // ranking order by counting: each entry's position is the number of
        // entries above it (the pairs are distinct)
        uint64_t mine = 0ull;
        int rank = 0;
        if (tid < n) {
          mine = s_g[tid];
          for (int j = 0; j < n; ++j) rank += s_g[j] > mine ? 1 : 0;
        }
        __syncthreads();
        if (tid < n) s_g[rank] = mine;
        __syncthreads();
      } else if (n <= kSfCap) {
        sort_list(s_g, n);
      }
      if (n <= kSfCap) {
        if (use_k) {                            // n >= mrank: the bin holds the top_k-th
          const int e = max(min(mrank, n) - 1, 0);
          kk = entry_key(e);
          kid = entry_id(e);
        } else {
          select_sorted(n, mrem, pk, pid);
        }
      } else if (use_k) {
        radix([&](int, float x) { return bin_of(x) == mbin; }, false, (uint64_t)mrank, kk, kid);
      } else {
        radix([&](int, float x) { return bin_of(x) == mbin; }, true, mrem, pk, pid);
      }
      set_final();
      // the deferred blocks under the final test
      for_deferred([&](int w, int j) {
        const uint32_t k = s_def[w * kSfWaveDef + j];
        const int c = (int)(k >> 1), h = (int)(k & 1u);
        float x16[16];
        deferred_half(w, j, c, h, x16);
        uint32_t wr[4];
        philox_chunk(c, wr);
        consider(half_sum16(x16, c, h), h ? wr[3] : wr[1], (int)k);
      });
    } else {
      // too many deferred blocks to list: resolve the boundary bin from the
      // whole row and draw the row again
      const int n2 = gather_sort(mbin, [](int, float) { return true; });
      if (use_k) {
        if (n2 <= kSfCap) {
          const int e = max(min(mrank, n2) - 1, 0);
          kk = entry_key(e);
          kid = entry_id(e);
        } else {
          radix([&](int, float x) { return bin_of(x) == mbin; }, false, (uint64_t)mrank, kk, kid);
        }
      } else if (n2 <= kSfCap) {
        select_sorted(n2, mrem, pk, pid);
      } else {
        radix([&](int, float x) { return bin_of(x) == mbin; }, true, mrem, pk, pid);
      }
      set_final();
      gbest = -INFINITY;
      kbest = INT_MAX;
      draw(Tag<false>{});
    }
  }

  const float S1 = block_reduce(s1, [](float x, float y) { return x + y; }, s_f);
  // the best (G, lower block index) over the workgroup
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float g2 = __shfl_xor(gbest, off, 64);
    const int k2 = __shfl_xor(kbest, off, 64);
    if (g2 > gbest || (g2 == gbest && k2 < kbest)) { gbest = g2; kbest = k2; }
  }
  if (lane == 0) {
    s_gbest[wave] = gbest;
    s_kbest[wave] = kbest;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSfWaves; ++w)
      if (s_gbest[w] > gbest || (s_gbest[w] == gbest && s_kbest[w] < kbest)) {
        gbest = s_gbest[w]; kbest = s_kbest[w];
      }
    // a kept token always exists (the kept set holds at least the row
    // maximum, with weight 1), so the best block is set; the guard keeps
    // every read inside the row regardless
    if (kbest < 0 || kbest >= 2 * nchunk) {
      a.token[rid] = mask;
      a.conf[rid] = 0.f;
      return;
    }
    const int c = kbest >> 1, h = kbest & 1;
    // the winning chunk once: both blocks' members, as the draw saw them
    float lv[32];
    load_chunk(c, lv);
    unmask(c, lv);
#pragma unroll
    for (int i = 0; i < 32; ++i) lv[i] = fin(lv[i]) ? lv[i] : -INFINITY;
    float x0[16], x1[16];
    half_of(lv, 0, x0);
    half_of(lv, 1, x1);
    uint32_t w[4];
    philox_chunk(c, w);
    // the inverse CDF inside block hh of the chunk: the first member whose
    // running sum reaches u S (the sums never decrease and u S > 0, so the
    // members below it are a prefix and the first past it has weight); if
    // rounding leaves none past it, the last member with weight.  Returns
    // the member index.
    auto icdf = [&](const float (&x)[16], int hh, uint32_t wu) {
      const int dv = idb - 32 * c;
      float e[16], S = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = 8 * (j >> 2) + 4 * hh + (j & 3);
        e[j] = kept_final(x[j], i, dv) ? fast_exp2(fmaf(x[j], c2, -mc2)) : 0.f;
        S += e[j];
      }
      const float target = sf_uniform(wu) * S;
      float cum = 0.f;
      int below = 0, last = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        cum += e[j];
        below += cum < target ? 1 : 0;
        last = e[j] > 0.f ? j : last;
      }
      return below < 16 ? below : last;
    };
    const int j0 = icdf(h ? x1 : x0, h, h ? w[2] : w[0]);
    int tok = 32 * c + 8 * (j0 >> 2) + 4 * h + (j0 & 3);
    float lt = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) lt = j == j0 ? (h ? x1[j] : x0[j]) : lt;
    if (h == 0) {
      // the chunk's other block at an equal G: the lower candidate wins
      const float S1b = half_sum16(x1, c, 1);
      if (S1b > 0.f && gumbel(S1b, w[3]) == gbest) {
        const int j1 = icdf(x1, 1, w[2]);
        const int tok1 = 32 * c + 8 * (j1 >> 2) + 4 + (j1 & 3);
        if (tok1 < tok) {
          tok = tok1;
#pragma unroll
          for (int j = 0; j < 16; ++j) lt = j == j1 ? x1[j] : lt;
        }
      }
    }
    a.token[rid] = tok;
    a.conf[rid] = __expf(lt - m) / S1;
  }
}

hipError_t sample_filtered_launch(const SampleArgs& a, hipStream_t st) {
  sample_filtered_kernel<<<a.max_rows, kSfThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
