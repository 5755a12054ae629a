// Selective LM head fused with the softmax, gfx950.
//
// The LM head runs only for still-masked positions of DENOISING sequences
// (JetEngine README, "Selective Logits"; developer notes, "Optimization
// History": sparse logits on masked positions only), and greedy decoding
// needs only each row's best token and its probability (SDAR page:
// generate.py runs greedy generation).  No logit is ever stored: a tile of
// logits lives in MFMA accumulators and is reduced there.
//
// lmhead_tile_kernel (persistent, kLmGrid workgroups of four waves, one per
// CU): C^T[v][m] = W[v][:] . h[m][:] with v_mfma_f32_32x32x16_bf16, each wave
// owning a 128 (vocab) x 128 (row) block.  The workgroup tile adapts to the
// row count M read on the device, so W streams from HBM exactly once while
// every wave has work:  M <= 128: 512 vocab x 128 rows;  M <= 256: 256 x 256;
// otherwise 128 x 512 (and row tiles of 512 in turn past 512 rows).  W and
// the gathered hidden rows stream in k-stages of 32 straight from global
// memory into four LDS buffers (16-byte chunks XOR-swizzled by row, so the
// fragment reads are bank-conflict free); stages k+1..k+3 are in flight
// while stage k is multiplied.  Each workgroup owns a contiguous vocabulary
// range (32-column blocks split evenly), tiled NT columns at a time.  After each tile a wave reduces its accumulators per row
// -- the largest logit (mask id and columns past V excluded), the lowest id
// reaching it, sum(exp(l - max)) in fp32 -- and folds that into a running
// (max, id, sum) per row; at the end the waves sharing rows fold through LDS
// and the workgroup writes one partial per row.
//
// lmhead_merge_kernel: one wave per row folds the kLmGrid partials,
// (m,a,s) + (m',a',s') = (max, id of the larger max or the lower id on equal
// maxima, s*e^(m-max) + s'*e^(m'-max)), in a fixed order, and writes the
// greedy token and the confidence 1/s = exp(max - logsumexp).
#include <type_traits>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {
constexpr int TK = 32;           // k depth of one stage
constexpr int MAXR = 640;        // rows of the largest stage (128 + 512)

// Physical 16-byte slot of logical k-chunk kc of a 64-byte LDS row: XOR with
// ((row>>1) ^ (row>>3)) & 3, so that the 32 rows one fragment read touches
// fall in distinct slots of every 128-byte and every 256-byte bank window.
__device__ __forceinline__ int slot_xor(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int swz(int row, int kc) {
  return row * TK + ((kc ^ slot_xor(row)) << 3);
}

struct Part {
  float m;
  int a;
  float s;
};

__device__ __forceinline__ void fold(Part& x, float m2, int a2, float s2) {
  if (m2 == -INFINITY) return;
  if (x.m == -INFINITY) {
    x.m = m2; x.a = a2; x.s = s2;
    return;
  }
  const float M = fmaxf(x.m, m2);
  const int a = (m2 > x.m || (m2 == x.m && a2 < x.a)) ? a2 : x.a;
  x.s = x.s * fast_exp2((x.m - M) * kLog2e) + s2 * fast_exp2((m2 - M) * kLog2e);
  x.m = M;
  x.a = a;
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// vmcnt(n) and lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the release fence of __syncthreads(): that fence
// would also wait for every load still streaming into LDS.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One workgroup's share of the vocabulary for row tile mt, with tile shape
// NT (vocab) x MT (rows); WN x WM waves of 128 x 128.  Stages of TK=32 go
// straight from global memory into LDS (global_load_lds_dwordx4: lane l of
// a wave instruction fills bytes 16*l of a 1 KB block, i.e. 16 rows of 64 B),
// four buffers deep, so stages k+1..k+3 stream in while stage k is multiplied.
template <int NT, int MT>
__device__ __forceinline__ void lm_rowtile(const LmArgs& a, int M, int mt, uint16_t* B0,
                                           uint16_t* B1, uint16_t* B2, uint16_t* B3) {
  constexpr int WN = NT / 128;
  constexpr int CHW = (NT + MT) / 64;   // 1 KB wave loads per stage per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases in SGPRs
  const int wn = wave % WN, wm = wave / WN;
  const int m0 = mt * MT;
  const int nk = a.Hd / TK;
  // this workgroup's contiguous vocabulary range [v_lo, v_hi), in 32-column
  // blocks split evenly over the grid, so every workgroup streams the same
  // share of W whatever the tile count
  const int nblk = (a.V + 31) / 32;
  const int v_lo = min(a.V, (int)(((long)blockIdx.x * nblk) / gridDim.x) * 32);
  const int v_hi = min(a.V, (int)(((long)(blockIdx.x + 1) * nblk) / gridDim.x) * 32);

  // Each wave fills WPW 1 KB blocks of W rows and HPW of gathered hidden
  // rows per stage (a block = 16 rows of 64 B).  Lane l writes row R + l/4,
  // LDS slot l%4, which must hold logical k-chunk (l%4) ^ slot_xor(row).
  constexpr int WPW = NT / 64, HPW = MT / 64;
  const int lrow = lane >> 2;
  const int hdb = a.Hd * 2;                                  // row bytes
  uint32_t hoffb[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int r = 16 * (wave * HPW + j) + lrow;              // row within the hidden part
    const int m = m0 + r;
    const int hr = m < M ? (a.row_index ? a.row_index[m] : m) : 0;  // rows past M: any valid row
    hoffb[j] = (uint32_t)hr * (uint32_t)hdb + (((lane & 3) ^ slot_xor(NT + r)) << 4);
  }
  uint32_t woffb[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int r = 16 * (wave * WPW + i) + lrow;
    woffb[i] = (uint32_t)(((lane & 3) ^ slot_xor(r)) << 4);
  }

  int mbv = (M - (m0 + wm * 128) + 31) >> 5;  // valid 32-row blocks of this wave
  mbv = mbv < 0 ? 0 : (mbv > 4 ? 4 : mbv);

  Part run[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) run[mb] = Part{-INFINITY, 0x7fffffff, 0.f};

  for (int n0 = v_lo; n0 < v_hi; n0 += NT) {
    // W rows past the range re-read one of the tile's first 16 rows (their
    // products are never used): spread over 16 rows rather than all on the
    // last one, so that a ragged tile does not hammer one cache line
    const int vlim = v_hi - 1 - n0;
    auto dma = [&](uint16_t* buf, int kt) {
      const char* wbase = reinterpret_cast<const char*>(a.w + (size_t)n0 * a.Hd + kt * TK);
      const char* hbase = reinterpret_cast<const char*>(a.hidden + kt * TK);
#pragma unroll
      for (int i = 0; i < WPW; ++i) {
        const int q = wave * WPW + i;                        // LDS block (16 rows)
        const int r0 = 16 * q + lrow;
        const int row = r0 <= vlim ? r0 : min(r0 & 15, vlim);
        __builtin_amdgcn_global_load_lds((const void*)(wbase + (uint32_t)(row * hdb) + woffb[i]),
                                         LDS_PTR(buf + q * 512), 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int q = NT / 16 + wave * HPW + j;
        __builtin_amdgcn_global_load_lds((const void*)(hbase + hoffb[j]),
                                         LDS_PTR(buf + q * 512), 16, 0, 0);
      }
    };

    // Accumulators start at 0, or at -inf on columns that are not candidates
    // (the mask id, columns past this workgroup's range): MFMA accumulation
    // keeps them at -inf, so the reduction below needs no per-value test.
    const int vbase = n0 + wn * 128;
    const bool plain = (vbase + 128 <= v_hi) && (a.mask_id < vbase || a.mask_id >= vbase + 128);
    f32x16 acc[4][4];
    if (plain) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x16 b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = vbase + nb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          b[i] = (v < v_hi && v != a.mask_id) ? 0.f : -INFINITY;
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = b;
      }
    }

    // fragments of one k-step (16): A = 4 blocks of W rows, B = 4 of hidden rows
    auto read_frags = [&](const uint16_t* buf, int kk, bf16x8* af, bf16x8* bfr) {
      const int kc = kk * 2 + (lane >> 5);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        af[nb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&buf[swz(wn * 128 + nb * 32 + (lane & 31), kc)]));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bfr[mb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&buf[swz(NT + wm * 128 + mb * 32 + (lane & 31), kc)]));
    };
    auto mfmas = [&](const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bfr[mb], acc[nb][mb], 0, 0, 0);
    };
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    // Stage kt (buffer `cur`, first k-step already in fa0/fb0): start the
    // load of stage kt+3 into `nxt3` (read in stage kt-1, released by that
    // stage's barrier), read the second k-step while the first multiplies,
    // then wait for stage kt+1, sync in the middle of the stage, and read its
    // first k-step while the second multiplies.  Every stage is the same code:
    // past the last stage the loads repeat the last stage into the idle
    // buffer and the final fragment read is unused.  Fragment reads complete
    // (lgkmcnt 0) before each barrier, so a buffer is never refilled under a
    // read still in flight.
    auto step = [&](int kt, const uint16_t* cur, const uint16_t* nxt, uint16_t* nxt3) {
      dma(nxt3, min(kt + 3, nk - 1));
      read_frags(cur, 1, fa1, fb1);
      mfmas(fa0, fb0);
      wait_vm_lgkm0<2 * CHW>();
      barrier_only();
      read_frags(nxt, 0, fa0, fb0);
      mfmas(fa1, fb1);
    };

    // nk is a multiple of 4 (Hd % 128 == 0), so the loop body is straight-line
    dma(B0, 0);
    dma(B1, 1);
    dma(B2, 2);
    wait_vm_lgkm0<2 * CHW>();
    barrier_only();
    read_frags(B0, 0, fa0, fb0);
    for (int kt = 0; kt < nk; kt += 4) {
      step(kt, B0, B1, B3);
      step(kt + 1, B1, B2, B0);
      step(kt + 2, B2, B3, B1);
      step(kt + 3, B3, B0, B2);
    }
    // the next tile's first loads must not overtake this tile's last reads
    wait_vm_lgkm0<0>();
    barrier_only();

    // reduce this tile: lane holds column (lane & 31) = one row per mb and
    // vocab rows 8*(i/4) + 4*(lane/32) + (i%4) of each 32-block nb.
    if (vbase < v_hi) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // Block-online reduction of the lane's 64 values of this row, 16 at a
        // time (one 32x32 block nb): block max, lowest id reaching it, and
        // sum(2^(x - m)) rescaled once per block.  Values are in log2 units;
        // non-candidates are -inf and contribute 0.
        float m = -INFINITY, sum = 0.f;
        int idx = 0x7fffffff;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          __builtin_amdgcn_sched_barrier(0);
          const int vb0 = vbase + nb * 32 + 4 * (lane >> 5);
          float x[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // read the accumulator from its AGPR here, not in one burst at the
            // loop exit (which would need all 256 values in VGPRs at once)
            float r;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(acc[nb][mb][i]));
            x[i] = r * kLog2e;
          }
          float bm = x[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) bm = fmaxf(bm, x[i]);
          int bi = 0x7fffffff;   // lowest id reaching the block max (ids grow with i)
#pragma unroll
          for (int i = 15; i >= 0; --i) bi = (x[i] == bm) ? vb0 + 8 * (i >> 2) + (i & 3) : bi;
          const float mn = fmaxf(m, bm);
          float sb = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sb += fast_exp2(x[i] - mn);
          sb = (mn == -INFINITY) ? 0.f : sb;            // all -inf so far: -inf - -inf
          const float scale = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
          sum = fmaf(sum, scale, sb);
          idx = (bm > m) ? bi : idx;   // equal maxima keep the earlier, lower id
          m = mn;
        }
        __builtin_amdgcn_sched_barrier(0);
        // combine with the lane holding the other half of the row's values
        const float pm = shfl_xor_f(m, 32);
        const int pi = shfl_xor_i(idx, 32);
        const float ps = shfl_xor_f(sum, 32);
        const float mx = fmaxf(m, pm);
        const float w1 = m == -INFINITY ? 0.f : fast_exp2(m - mx);
        const float w2 = pm == -INFINITY ? 0.f : fast_exp2(pm - mx);
        sum = sum * w1 + ps * w2;
        idx = (pm > m || (pm == m && pi < idx)) ? pi : idx;
        fold(run[mb], mx * (1.0f / kLog2e), idx, sum);
      }
    }
  }

  // fold the waves that share rows, then one partial per row (the row
  // partials use the first stage buffer, idle after the last barrier)
  Part* s_part = reinterpret_cast<Part*>(B0);
  if (WN > 1) {
    if (lane < 32) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) s_part[(wave * 4 + mb) * 32 + lane] = run[mb];
    }
    __syncthreads();
    if (wn == 0 && lane < 32) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        for (int o = 1; o < WN; ++o) {
          const Part p = s_part[((wave + o) * 4 + mb) * 32 + lane];
          fold(run[mb], p.m, p.a, p.s);
        }
    }
    __syncthreads();
  }
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + lane;
      if (m < M) {
        const size_t o = (size_t)m * kLmGrid + blockIdx.x;
        a.pm[o] = run[mb].m;
        a.pa[o] = run[mb].a;
        a.ps[o] = run[mb].s;
      }
    }
  }
}
}  // namespace

// One kernel per tile shape; each exits unless the row count on the device
// selects its shape, so the launch sequence stays fixed for graph capture.
template <int NT, int MT>
__global__ __launch_bounds__(256, 1) void lmhead_tile_kernel(LmArgs a) {
  __shared__ __align__(16) uint16_t B0[MAXR * TK];
  __shared__ __align__(16) uint16_t B1[MAXR * TK];
  __shared__ __align__(16) uint16_t B2[MAXR * TK];
  __shared__ __align__(16) uint16_t B3[MAXR * TK];
  const int M = *a.num_rows;
  const int want = M <= 0 ? 0 : (M <= 128 ? 512 : (M <= 256 ? 256 : 128));
  if (want != NT) return;
  const int n_mt = (M + MT - 1) / MT;
  for (int mt = 0; mt < n_mt; ++mt) {
    lm_rowtile<NT, MT>(a, M, mt, B0, B1, B2, B3);
    __syncthreads();   // row partials in B0 are read before the next row tile loads
  }
}

__global__ __launch_bounds__(256) void lmhead_merge_kernel(LmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const int M = *a.num_rows;
  if (r >= M) return;
  constexpr int PER = kLmGrid / 64;
  const size_t base = (size_t)r * kLmGrid;
  float pm[PER], ps[PER];
  int pa[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    pm[j] = a.pm[base + lane + 64 * j];
    pa[j] = a.pa[base + lane + 64 * j];
    ps[j] = a.ps[base + lane + 64 * j];
  }
  Part x{-INFINITY, 0x7fffffff, 0.f};
#pragma unroll
  for (int j = 0; j < PER; ++j) fold(x, pm[j], pa[j], ps[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = shfl_xor_f(x.m, off);
    const int a2 = shfl_xor_i(x.a, off);
    const float s2 = shfl_xor_f(x.s, off);
    fold(x, m2, a2, s2);
  }
  if (lane == 0) {
    const int row = a.row_index ? a.row_index[r] : r;
    a.argmax_tok[row] = x.a;
    a.conf[row] = 1.f / x.s;
  }
}

size_t lmhead_ws_bytes(int max_rows, int V) {
  (void)V;
  const size_t one = ((size_t)max_rows * kLmGrid * 4 + 255) & ~(size_t)255;
  return 3 * one;
}

hipError_t lmhead_launch(const LmArgs& a, hipStream_t st) {
  lmhead_tile_kernel<512, 128><<<kLmGrid, 256, 0, st>>>(a);
  lmhead_tile_kernel<256, 256><<<kLmGrid, 256, 0, st>>>(a);
  lmhead_tile_kernel<128, 512><<<kLmGrid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lmhead_merge_kernel<<<(a.max_rows + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
