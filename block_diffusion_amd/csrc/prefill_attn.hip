// Block-causal prefill attention over packed prompts, gfx950.
//
// A prompt is prefilled with the block pattern a block-diffusion model
// decodes with (JetEngine developer notes, "ModelRunner": prefill has its
// own attention pattern; "Layers": a block-sparse varlen attention serves
// it, and a store kernel writes the prompt's K/V into the paged cache):
// token i of a prompt attends to token j iff floor(j/B) <= floor(i/B) --
// every earlier block, and its own block in both directions.
//
// Unlike the denoise step, this is a dense contraction: every key tile is
// used by many query rows, so its roofline is the MFMA peak; at this tiling
// the softmax's VALU work per score is about as long as the MFMA work, so
// both matter.  Work item = (prompt s, kv head g, tile of 64*PF_RT query
// rows); a row is (token t, head gi) with row = t*G + gi, so the G query
// heads of a kv head share every key tile.  Four waves of 16*PF_RT rows
// share a PF_NS-stage LDS ring of 32-key K/V tiles that the waves fill with
// direct-to-LDS loads (global_load_lds_dwordx4, 16-byte chunks XOR-permuted
// by row); three workgroups fit on a CU.  Per run of 32 keys a wave
// computes S^T = K Q^T in two 16-key halves, an online softmax in fp32
// (base 2), and O^T += V^T P^T, all with v_mfma_f32_16x16x32_bf16 (the
// K = 32 form runs at twice the rate of the K = 16 one on gfx950), V^T read
// by ds_read_b64_tr_b16.  A wave raises its priority for the two MFMA
// phases, so that among the waves of a SIMD the one with matrix work issues
// first.  The block-causal mask is a per-row key bound,
// min(L, (floor(t/B)+1)*B); runs past a wave's largest bound are skipped,
// and the runs below its smallest bound (most of them) go through a loop of
// their own without the per-score test.  Row sums add the fp32
// probabilities (the P V product takes them rounded to bf16).  The running
// maximum is only moved when some row's new maximum exceeds it by more than
// 2^8 (probabilities up to 2^8 are exact in the fp32 sums), which leaves
// most runs without the rescale of the accumulators.
//
// Tiles of one prompt are handed out last first (the late, long rows), and
// the workgroup of a tile also copies that tile's tokens' K/V of head g into
// the paged cache when one is given (positions 0 .. L-1).
#include <type_traits>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

#ifndef PF_KT
#define PF_KT 32
#endif
#ifndef PF_NS
#define PF_NS 2
#endif
#ifndef PF_RT
#define PF_RT 2
#endif
#ifndef PF_OCC
#define PF_OCC 3
#endif
#ifndef PF_SUM_ROUNDED
#define PF_SUM_ROUNDED 0   // row sums over the fp32 probabilities
#endif
constexpr int kPfKT = PF_KT;               // keys per stage
constexpr int kPfNS = PF_NS;               // ring stages
constexpr int kPfRT = PF_RT;               // 16-row MFMA tiles per wave
constexpr int kPfWaveRows = 16 * kPfRT;    // 64
constexpr int kPfRows = 4 * kPfWaveRows;   // query rows per workgroup

template <int D>
__device__ __forceinline__ int pswz(int r) {
  return D == 128 ? (r & 15) : (((r >> 1) ^ ((r & 1) << 2)) & 7);
}
template <int D>
__device__ __forceinline__ int poff(int r, int c) {
  return r * D + ((c ^ pswz<D>(r)) << 3);
}

// One 1 KB direct-to-LDS load (lane l: 16 bytes at base + off to lds +
// 16*l).  s_nop 4: the five wait states a VMEM instruction needs after a
// VALU write of an SGPR it reads (the base pair may come from v_readlane;
// the compiler adds no wait states for inline-assembly operands), which
// also cover the one a fresh M0 needs.
__device__ __forceinline__ void pf_dma16(const void* base, uint32_t off, const lds_u16* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
}
template <int N>
__device__ __forceinline__ void pf_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void pf_wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void pf_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ int pf_ldc(const int32_t* p, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

}  // namespace

// plan[s] = sum over s' < s of ceil(L_s' * G / kPfRows); plan[S] = the total
__global__ __launch_bounds__(1024) void prefill_plan_kernel(PrefillArgs a) {
  __shared__ int s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;
  const int per = (S + 1023) / 1024;
  const int b0 = tid * per;
  auto tiles = [&](int s) {
    const int L = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
    return (L * a.G + kPfRows - 1) / kPfRows;
  };
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (b0 + j < S) local += tiles(b0 + j);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_wsum[w];
  run += incl - local;
  for (int j = 0; j < per; ++j)
    if (b0 + j < S) {
      a.plan[b0 + j] = run;
      run += tiles(b0 + j);
    }
  if (tid == 1023) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += s_wsum[w];
    a.plan[S] = tot;
  }
}

template <int D>
__global__ __launch_bounds__(256, PF_OCC) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int RT = kPfRT, KT = kPfKT, NS = kPfNS;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int KVE = KT * D;              // elements of one K (or V) stage
  constexpr int LPR = D / 8;               // 16-byte chunks per row
  constexpr int RPI = 64 / LPR;            // rows per 1 KB load
  constexpr int NLD = 2 * KT / RPI / 4;    // 1 KB loads per wave per stage (K and V)
  static_assert(NLD >= 1 && (2 * KT / RPI) % 4 == 0, "stage split over four waves");
  static_assert(KT % 32 == 0, "runs of 32 keys");
  __shared__ __align__(16) uint16_t ring_[NS * 2 * KVE];
  lds_u16* const ring = (lds_u16*)ring_;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int x = blockIdx.x;
  const int g = x % a.Hkv, idx = x / a.Hkv;
  if (idx >= pf_ldc(a.plan, a.S)) return;
  // prompt s: the largest with plan[s] <= idx (plan is non-decreasing)
  int lo = 0, hi = a.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pf_ldc(a.plan, mid) <= idx) lo = mid;
    else hi = mid;
  }
  const int s = lo;
  const int t0s = pf_ldc(a.cu_seqlens, s);
  const int L = pf_ldc(a.cu_seqlens, s + 1) - t0s;
  const int G = a.G, Bk = a.B;
  const int ntile = pf_ldc(a.plan, s + 1) - pf_ldc(a.plan, s);
  const int tile = ntile - 1 - (idx - pf_ldc(a.plan, s));   // last tiles first
  const int R = L * G;
  const int row_wg = tile * kPfRows;
  const int row0 = row_wg + wave * kPfWaveRows;             // this wave's first row

  // the tile's tokens' K/V of head g into the paged cache
  if (a.k_cache_out != nullptr) {
    const int tlo = row_wg / G, thi = min(L, (row_wg + kPfRows) / G);
    const int nchunk = (thi - tlo) * LPR;
    for (int c = tid; c < nchunk; c += 256) {
      const int t = tlo + c / LPR, ch = c % LPR;
      const int pidx = t / a.P;
      if (pidx >= a.max_pages) continue;
      const int page = a.page_table[(size_t)s * a.max_pages + pidx];
      if (page < 0 || page >= a.num_pages) continue;
      const size_t src = ((size_t)(t0s + t) * a.Hkv + g) * D + ch * 8;
      const size_t dst = (((size_t)page * a.Hkv + g) * a.P + t % a.P) * D + ch * 8;
      *reinterpret_cast<u32x4*>(a.k_cache_out + dst) = *reinterpret_cast<const u32x4*>(a.k + src);
      *reinterpret_cast<u32x4*>(a.v_cache_out + dst) = *reinterpret_cast<const u32x4*>(a.v + src);
    }
  }

  // key bounds: the workgroup streams keys [0, kend); this wave needs keys
  // below kend_w, and keys below kfree_w are visible to all of its rows
  const int tmax_wg = (min(R, row_wg + kPfRows) - 1) / G;
  const int kend = min(L, (tmax_wg / Bk + 1) * Bk);
  const bool wave_live = row0 < R;
  const int tmax_w = (min(R, row0 + kPfWaveRows) - 1) / G;
  const int kend_w = wave_live ? min(L, (tmax_w / Bk + 1) * Bk) : 0;
  const int kfree_w = wave_live ? min(L, ((row0 / G) / Bk) * Bk) : 0;

  // per-lane rows: row = row0 + rt*16 + lr; its key bound
  int klim[RT];
  bf16x8 qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + lr;
    const int rr = min(row, R - 1);
    const int t = rr / G, gi = rr % G;
    klim[rt] = min(L, (t / Bk + 1) * Bk);
    const uint16_t* qp = a.q + ((size_t)(t0s + t) * a.Hq + g * G + gi) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = ld_bf16x8(qp + (4 * ks + lg) * 8);
  }

  // stage st (keys st*KT ..): this wave's NLD loads, rows past L re-read
  // row L-1 (their scores are masked)
  const int nstage = (kend + KT - 1) / KT;
  const uint32_t rowb = (uint32_t)a.Hkv * D * 2;           // bytes between token rows
  const char* kbase = reinterpret_cast<const char*>(a.k + ((size_t)t0s * a.Hkv + g) * D);
  const char* vbase = reinterpret_cast<const char*>(a.v + ((size_t)t0s * a.Hkv + g) * D);
  // load i of this wave fills stage row r = r0 + lane/LPR (r0 from the wave
  // and i), physical chunk lane%LPR with logical chunk lc; loff[i] is the
  // lane's byte offset from the stage's first key, the same in every stage
  uint32_t loff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ii = wave * NLD + i;                         // 0 .. 2*KT/RPI-1
    const int r0 = (ii >= KT / RPI ? ii - KT / RPI : ii) * RPI;
    const int r = r0 + lane / LPR;
    loff[i] = (uint32_t)r * rowb + (uint32_t)((lane % LPR) ^ pswz<D>(r)) * 16;
  }
  auto issue = [&](int st) {
    const int stc = st < nstage ? st : nstage - 1;         // past the end: repeat the last
    lds_u16* slot = ring + (st % NS) * 2 * KVE;
    if ((stc + 1) * KT <= L) {
      // every key of the stage is real: only the scalar base moves
      const size_t sb = (size_t)stc * KT * rowb;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int ii = wave * NLD + i;
        const bool isv = ii >= KT / RPI;
        const int r0 = (isv ? ii - KT / RPI : ii) * RPI;
        pf_dma16((isv ? vbase : kbase) + sb, loff[i], slot + (isv ? KVE : 0) + r0 * D);
      }
    } else {
      // the prompt's last stage: rows past L re-read row L-1
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int ii = wave * NLD + i;
        const bool isv = ii >= KT / RPI;
        const int r0 = (isv ? ii - KT / RPI : ii) * RPI;
        const int r = r0 + lane / LPR;
        const int lc = (lane % LPR) ^ pswz<D>(r);
        const int key = min(stc * KT + r, L - 1);
        pf_dma16(isv ? vbase : kbase, (uint32_t)key * rowb + (uint32_t)lc * 16,
                 slot + (isv ? KVE : 0) + r0 * D);
      }
    }
  };

  float m_run[RT], l_run[RT];
  f32x4 acc[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one run of 16 keys starting at key j0 from LDS rows kt16 / vt16
  // one run of 32 keys starting at key j0 from LDS rows kt32 / vt32: two
  // 16-key halves for S^T, one softmax step, and P V with K = 32 MFMAs whose
  // k slots 8*lg .. 8*lg+7 hold keys 4*lg .. 4*lg+3 of the first half, then
  // of the second (the same order in both operands)
  // (MASKED: some of the 32 keys lie past some row's bound; the other runs,
  // most of them, skip the per-score test)
  auto run32 = [&](auto masked_c, const lds_u16* kt32, const lds_u16* vt32, int j0) {
    constexpr bool masked = decltype(masked_c)::value;
    f32x4 sc[2][RT];
    __builtin_amdgcn_s_setprio(1);     // the MFMA phases first, the softmax of other waves after
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(kt32 + hh * 16 * D + poff<D>(lr, lg + 4 * ks)));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        sc[hh][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[hh][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[rt][ks], sc[hh][rt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    float xs[RT][8], tmax[RT];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      tmax[rt] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = j0 + 16 * (i >> 2) + 4 * lg + (i & 3);
        const float sv = sc[i >> 2][rt][i & 3];
        xs[rt][i] = (!masked || j < klim[rt]) ? sv : -INFINITY;   // raw scores
        tmax[rt] = fmaxf(tmax[rt], xs[rt][i]);
      }
      tmax[rt] *= a.scale_log2;
      tmax[rt] = max_xor32(max_xor16(tmax[rt]));
      grow |= tmax[rt] > m_run[rt] + 8.f;
    }
    // move the running maxima (and rescale) only when one has grown by more
    // than 2^8; otherwise probabilities are taken against the old maxima
    if (__ballot(grow) != 0ull) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float m_new = fmaxf(m_run[rt], tmax[rt]);
        const float alpha = m_run[rt] == -INFINITY ? 0.f : fast_exp2(m_run[rt] - m_new);
        m_run[rt] = m_new;
        l_run[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      }
    }
    bf16x8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float psum = 0.f;
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float e0 = fast_exp2(fmaf(xs[rt][i], a.scale_log2, -m_run[rt]));
        const float e1 = fast_exp2(fmaf(xs[rt][i + 1], a.scale_log2, -m_run[rt]));
        const uint32_t w = pack_bf16x2(e0, e1);
#if PF_SUM_ROUNDED
        psum += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
#else
        psum += e0 + e1;
#endif
        pw[i >> 1] = w;
      }
      pb[rt] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      l_run[rt] += psum;
    }
    // O^T[d][row] += V^T[d][key] P^T[key][row]; in each half, lane w of
    // 16-lane group lg reads V[4*lg + w/4][16*dt + 4*(w%4) .. +3] by
    // transpose reads and receives V[4*lg .. 4*lg+3][16*dt + w]
    const int vrow = 4 * lg + (lr >> 2), vsub = 4 * (lr & 1), vch = (lr & 3) >> 1;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vt32 + poff<D>(vrow, 2 * dt + vch) + vsub));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vt32 + 16 * D + poff<D>(vrow, 2 * dt + vch) + vsub));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 v8 = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], acc[rt][dt], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ring: stages 0 .. NS-2 up front; at stage st, after the barrier, load
  // stage st+NS-1 into the slot every wave finished reading at stage st-1
  if (nstage > 0) {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st);
  }
  // stage st: wait for it, then load stage st+NS-1; the stages below the
  // wave's first masked key (kfree_w) run without the per-score bound test,
  // in a loop of their own (two instances of the run in one loop body would
  // cost registers); every wave passes the same number of barriers
  auto stage = [&](int st, auto masked_c) {
    pf_wait_vm<NLD * (NS - 2)>();
    pf_wait_lgkm0();
    pf_barrier();
    issue(st + NS - 1);
    const lds_u16* slot = ring + (st % NS) * 2 * KVE;
#pragma unroll
    for (int hh = 0; hh < KT / 32; ++hh) {
      const int j0 = st * KT + 32 * hh;
      if (j0 < kend_w) run32(masked_c, slot + hh * 32 * D, slot + KVE + hh * 32 * D, j0);
    }
  };
  const int nfree = min(nstage, kfree_w / KT);
  for (int st = 0; st < nfree; ++st) stage(st, std::false_type{});
  for (int st = nfree; st < nstage; ++st) stage(st, std::true_type{});
  pf_wait_vm<0>();   // no load may land in LDS after the workgroup is gone

  // out rows: O^T columns; lane holds d = 16*dt + 4*lg .. +3 of row lr
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = l_run[rt];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    const int row = row0 + rt * 16 + lr;
    if (row < R) {
      const float inv = 1.f / l;
      const int t = row / G, gi = row % G;
      uint16_t* op = a.out + ((size_t)(t0s + t) * a.Hq + g * G + gi) * D + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2 v;
        v.x = pack_bf16x2(acc[rt][dt].x * inv, acc[rt][dt].y * inv);
        v.y = pack_bf16x2(acc[rt][dt].z * inv, acc[rt][dt].w * inv);
        *reinterpret_cast<u32x2*>(op + 16 * dt) = v;
      }
    }
  }
}

int prefill_rows_per_wg() { return kPfRows; }

size_t prefill_ws_bytes(int S) { return ((size_t)(S + 1) * sizeof(int32_t) + 255) & ~(size_t)255; }

int prefill_grid(int S, int T_total, int Hkv, int G) {
  const long tiles = ((long)T_total * G + kPfRows - 1) / kPfRows + S;
  return (int)(tiles * Hkv);
}

hipError_t prefill_launch(const PrefillArgs& a, int D, hipStream_t st) {
  prefill_plan_kernel<<<1, 1024, 0, st>>>(a);
  const int grid = prefill_grid(a.S, a.T_total, a.Hkv, a.G);
  if (D == 128) prefill_attn_kernel<128><<<grid, 256, 0, st>>>(a);
  else prefill_attn_kernel<64><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
