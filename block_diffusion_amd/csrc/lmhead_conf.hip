// Selective LM head fused with the softmax, gfx950.
//
// The LM head runs only for still-masked positions of DENOISING sequences
// (JetEngine README, "Selective Logits"; developer notes, "Optimization
// History": sparse logits on masked positions only), and greedy decoding
// needs only each row's best token and its probability (SDAR page:
// generate.py runs greedy generation).  No logit is ever stored: a tile of
// logits lives in MFMA accumulators and is reduced there.
//
// lmhead_tile_kernel: persistent, one workgroup of four waves per CU.  The M
// rows (read on the device) are split among the G members of a *team* of
// workgroups that sit on the same XCD (workgroup b runs on XCD b % 8), with
// G = 1, 2 or 4 for M <= 256, 512 or 1024 (larger M loops over passes of
// 1024 rows).  Each team owns a contiguous range of the vocabulary; each
// member streams that range of W against its own <= 256 rows.  The members
// read the same W tile at about the same time, so W comes from HBM once per
// XCD and from L2 for the other members.
//
// A tile is 256 vocabulary columns x R <= 256 rows, four waves of 128 x R/2
// computing C^T[v][m] = W[v].h[m] with v_mfma_f32_32x32x16_bf16.  A team's
// range rarely ends on a tile boundary: in its partial last tile of nbl
// 32-column blocks the two waves that share rows take ceil(nbl/2) blocks
// each instead of 4 and 0..4, so the tile costs what its columns need
// (12% off the LM head at 256 rows, whose ranges of 2.3 tiles used to take
// three full tiles).  K streams
// in stages of 64 (one 128-byte line per row) straight from global memory
// into LDS (global_load_lds_dwordx4; 16-byte chunks XOR-permuted by row so
// fragment reads are bank-conflict free):
//   * waves 0-1 load W into a 3-slot ring, two stages ahead (HBM latency),
//   * waves 2-3 load hidden rows into a 2-slot ring, one stage ahead (L2),
// each with its own vmcnt, so a slow W line never holds up a hidden stage.
// Stages run back to back across tiles.  Within a stage, the fragment reads
// of k-step j+1 are interleaved with the MFMAs of k-step j.  After a tile,
// each wave reduces its accumulators per row -- the largest logit (mask id
// and columns past the range excluded), the lowest id reaching it, and
// sum(exp(l - max)) -- and folds that into a running (max, id, sum) per row;
// at the end the two waves sharing rows fold through LDS and the workgroup
// writes one partial per (row, team).
//
// Sampling (SMP instances): the token is drawn from softmax(l / T) instead
// of taken as the argmax, exactly and without any extra pass.  Each block of
// 16 vocabulary columns that a lane holds for a row (chunk c = 32 aligned
// columns, half h: columns 32c + 8q + 4h + r) draws two uniforms from
// Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2,
// 3"; counter (c, row id, step, 0), key = the 64-bit seed): one picks a
// column inside the block by inverse CDF of exp(l/T), the other a Gumbel
// variable located at the block's log-sum-exp.  The block with the largest
// Gumbel value wins (the Gumbel-max trick over blocks), so the token has
// probability exp(l_v/T) / sum exp(l/T).  The confidence stays the model's
// probability of that token at temperature 1.
//
// lmhead_merge_kernel: one wave per row folds the partials of all teams,
// (m,a,s) + (m',a',s') = (max, id of the larger max or the lower id on equal
// maxima, s*e^(m-max) + s'*e^(m'-max)), in a fixed order, and writes the
// greedy token and the confidence 1/s = exp(max - logsumexp).
#include <type_traits>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int TK = 64;               // k per stage: one 128-byte line per row
constexpr int NT = 256;              // vocabulary columns per tile
constexpr int RMAX = 256;            // hidden rows per workgroup per pass
constexpr int WSLOT = NT * TK;       // elements of one W stage (32 KB)
constexpr int HSLOT = RMAX * TK;     // elements of one hidden stage (32 KB)
constexpr int NWS = 3;               // W ring slots (two stages in flight)
constexpr int NHS = 2;               // hidden ring slots (one stage in flight)
constexpr int WPW = NT / 8 / 2;      // 1 KB W loads per W wave per stage

// chunk permutation of LDS row r: rows 2i and 2i+1 (one 256-byte bank window)
// and any 8 consecutive rows (one 128-byte window per row) use distinct slots
__device__ __forceinline__ int rswz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// Running reduction of a row's logits l over the columns seen so far, in
// natural units: m = max l, a = lowest id reaching m, s = sum e^(l-m),
// t = sum e^(l-m) (l-m).  The softmax entropy is ln s - t/s.
struct Part {
  float m;
  int a;
  float s;
  float t;
};

// (m,a,s,t) + (m2,a2,s2,t2): rescale both to M = max(m, m2):
// s -> s e^(m-M), t -> e^(m-M) (t + (m-M) s).
__device__ __forceinline__ void fold(Part& x, float m2, int a2, float s2, float t2) {
  if (m2 == -INFINITY) return;
  if (x.m == -INFINITY) {
    x.m = m2; x.a = a2; x.s = s2; x.t = t2;
    return;
  }
  const float M = fmaxf(x.m, m2);
  const int a = (m2 > x.m || (m2 == x.m && a2 < x.a)) ? a2 : x.a;
  const float w1 = fast_exp2((x.m - M) * kLog2e), w2 = fast_exp2((m2 - M) * kLog2e);
  x.t = w1 * fmaf(x.m - M, x.s, x.t) + w2 * fmaf(m2 - M, s2, t2);
  x.s = x.s * w1 + s2 * w2;
  x.m = M;
  x.a = a;
}

// Sampling draw of one block or of a set of blocks: the largest Gumbel value
// so far (log2 units), the candidate column of that block, and its logit at
// temperature 1 (natural units).  Lower candidate on equal values.
struct Pick {
  float g;
  int c;
  float l;
};

__device__ __forceinline__ void pick_fold(Pick& x, float g2, int c2, float l2) {
  if (g2 > x.g || (g2 == x.g && c2 < x.c)) {
    x.g = g2; x.c = c2; x.l = l2;
  }
}

// Philox4x32-10: ten rounds of two 32x32->64 products of words 0 and 2,
// their halves mixed with words 1 and 3 and the key, the key bumped by the
// Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
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

// ((w >> 9) + 0.5) / 2^23 in (0, 1), exact in float32
__device__ __forceinline__ float uniform01(uint32_t w) {
  return (float)(((w >> 9) << 1) | 1u) * (1.0f / 16777216.0f);
}

// One 1 KB direct-to-LDS load: lane l copies the 16 bytes at base + off to
// lds + 16*l.  Inline assembly, so that the compiler neither adds its own
// vmcnt waits for the LDS it writes nor moves LDS accesses across it; the
// rings are paced by explicit waits.  M0 carries the LDS address; the s_nop
// is the one wait state a freshly written M0 needs.  A VMEM instruction also
// needs five wait states after a VALU instruction wrote an SGPR it reads,
// and the compiler inserts none for an operand of inline assembly: if it
// ever materialised the base pair with v_readlane (an SGPR spill reload)
// right before this, the load would use a stale base.  The build scans the
// linked assembly for that pattern and refuses the library (isa_check.py);
// five wait states in every instance would cost 1-2% of the kernel.  FIVE
// selects them for the store-mode instance, whose partial-maximum
// bookkeeping leaves the compiler short of SGPRs.
template <bool FIVE, bool NT = false>
__device__ __forceinline__ void dma16(const void* base, uint32_t off, const lds_u16* lds) {
  if constexpr (FIVE && NT)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(off), "s"(base), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
  else if constexpr (FIVE)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
  else if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(off), "s"(base), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
}
#ifndef LM_W_NT
#define LM_W_NT 0
#endif

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int team_size(int M) { return lm_team_size(M); }

// One pass of one workgroup: rows [m_base, m_end) of the compact row list
// (R = 64*MB row slots, two waves of 32*MB rows) against vocabulary columns
// [v_lo, v_hi), as seen by one wave; WL: this wave streams W (else hidden
// rows); MODE bit 0 (ENT): also accumulate sum e^(l-m)(l-m) for the
// entropy; bit 1 (SMP): draw a sampled token instead of the argmax.  Writes
// one partial per valid row into slot `team`.  MODE 4 (STO): store the
// logits themselves (mask column -inf) instead of reducing them.
template <int MB, bool WL, int MODE>
__device__ __forceinline__ void lm_pass(const LmArgs& a, int m_base, int m_end, int v_lo, int v_hi,
                                        int team, int nteam, lds_u16* Wr, lds_u16* Hr) {
  constexpr bool ENT = (MODE & 1) != 0, SMP = (MODE & 2) != 0, STO = (MODE & 4) != 0;
  constexpr int R = 64 * MB, RH = 32 * MB;
  constexpr int HPW = R / 16;                  // 1 KB hidden loads per hidden wave per stage
  constexpr int NLD = WL ? WPW : HPW;          // this wave's loads per stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int nk = a.Hd / TK;
  const int ntile = (v_hi - v_lo + NT - 1) / NT;
  // Tile order.  The store mode's epilogue writes each tile's logits, and
  // workgroups that finish tiles together queue on HBM writes together: odd
  // teams take their partial last tile first, which offsets their
  // epilogues from the even teams' by that tile's (shorter) time.  Every
  // other mode keeps the plain order.
#ifndef LM_ROT
#define LM_ROT 1
#endif
  const bool rot = STO && LM_ROT != 0 && (team & 1) != 0 && ntile > 1;
  auto tmap = [&](int t) { return rot ? (t == 0 ? ntile - 1 : t - 1) : t; };
  const uint32_t hdb = (uint32_t)a.Hd * 2;     // row bytes

  // Lane l of a 1 KB load fills LDS row 8*blk + l/8, physical chunk l%8,
  // which holds logical chunk (l%8) ^ rswz(row).  off[i]: byte offset of the
  // lane's 16 bytes for this wave's i-th load, relative to the stage's
  // first W row (W waves) or to the hidden matrix (hidden waves).
  const int lr = lane >> 3;
  uint32_t off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int blk = wn * NLD + i;
    const int row = 8 * blk + lr;                       // LDS row
    const uint32_t ch = (uint32_t)(((lane & 7) ^ rswz(row)) << 4);
    if (WL) {
      off[i] = (uint32_t)row * hdb + ch;
    } else {
      const int m = m_base + row;
      const int mm = m < m_end ? m : m_base;            // rows past the list: any listed row
      const int hr = a.row_index ? a.row_index[mm] : mm;
      off[i] = (uint32_t)hr * hdb + ch;
    }
  }

  // Issue cursor: the next stage this wave loads (tile it_t, k-stage it_k);
  // past the last stage it keeps loading the last one (never used).
  int it_t = 0, it_k = 0;
  // loads [I0, I1) of this wave's share of the cursor's stage into `slot`
  auto issue_part = [&](lds_u16* slot, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
    const char* kb = reinterpret_cast<const char*>(WL ? a.w : a.hidden) + (size_t)it_k * (TK * 2);
    if (WL) {
      const int n0 = v_lo + tmap(min(it_t, ntile - 1)) * NT;
      const char* tb = kb + (size_t)n0 * hdb;
      const int lim = v_hi - n0;                       // valid rows of this tile
      // rows past the range re-read a row of the tile's first 8
      const uint32_t back = (uint32_t)min(lr, lim - 1) * hdb;
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const int row = 8 * (wn * NLD + i) + lr;
        const uint32_t o = row < lim ? off[i] : back + (off[i] & 0x70);
        dma16<STO, LM_W_NT != 0>(tb, o, slot + (wn * NLD + i) * 512);
      }
    } else {
#pragma unroll
      for (int i = I0; i < I1; ++i) dma16<STO>(kb, off[i], slot + (wn * NLD + i) * 512);
    }
  };
  auto advance = [&]() {
    if (it_t < ntile) {
      if (++it_k == nk) {
        it_k = 0;
        if (it_t + 1 < ntile) ++it_t;
        else it_k = nk - 1, it_t = ntile;              // hold at the last stage
      }
    }
  };
  auto issue = [&](lds_u16* slot) {
    issue_part(slot, std::integral_constant<int, 0>{}, std::integral_constant<int, NLD>{});
    advance();
  };
  // the stage about to be read has landed for this wave's stream, and this
  // wave's fragment reads are done; then the whole workgroup syncs
  auto sync = [&]() {
    wait_vm<WL ? WPW * (NWS - 2) : HPW * (NHS - 2)>();
    wait_lgkm0();
    barrier_only();
  };

  // fragment reads: lane row (lane & 31) of a 32-row block, logical chunk
  // 2j + lane/32 of k-step j; the permutation depends on the row mod 16 only,
  // so blocks 32 rows apart share it
  const int fr = lane & 31;
  int chk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) chk[j] = ((2 * j + (lane >> 5)) ^ rswz(fr)) << 3;
  const lds_u16* wfr = Wr + (wn * 128 + fr) * TK;    // this wave's first W row; set per tile
  const lds_u16* const hfr = Hr + (wm * RH + fr) * TK;
  auto read_frags = [&](int ws, int hs, int j, bf16x8* af, bf16x8* bfr) {
    const lds_u16* w = wfr + ws * WSLOT + chk[j];
    const lds_u16* h = hfr + hs * HSLOT + chk[j];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      af[nb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(w + nb * 32 * TK));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      bfr[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(h + mb * 32 * TK));
  };

  f32x16 acc[4][MB];
  // NBW: the 32-column blocks this wave computes in the current tile
  auto mfma_rows = [&](auto nbw_c, const bf16x8* af, const bf16x8* bfr, int mb) {
    constexpr int NBW = decltype(nbw_c)::value;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bfr[mb], acc[nb][mb], 0, 0, 0);
  };
  // one k-step's MFMAs with the next step's fragment reads interleaved,
  // fenced so that nothing else is scheduled into it
  auto step = [&](auto nbw_c, const bf16x8* af, const bf16x8* bfr, int ws, int hs, int jn, bf16x8* an,
                  bf16x8* bn) {
    constexpr int NBW = decltype(nbw_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    read_frags(ws, hs, jn, an, bn);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mfma_rows(nbw_c, af, bfr, mb);
    constexpr int NPAIR = NBW * MB < 4 + MB ? NBW * MB : 4 + MB;
#pragma unroll
    for (int r = 0; r < NPAIR; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    if (NBW * MB > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NBW * MB - NPAIR, 0);
    if (4 + MB > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, 4 + MB - NPAIR, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  Part run[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) run[mb] = Part{-INFINITY, 0x7fffffff, 0.f, 0.f};
  // sampling: running draw and the row id (s*B + position) of each row the
  // lane holds; rows past the list use a listed row (never written)
  Pick pick[MB];
  uint32_t rid[MB];
  if constexpr (SMP) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      pick[mb] = Pick{-INFINITY, 0x7fffffff, 0.f};
      const int m = m_base + wm * RH + mb * 32 + (lane & 31);
      const int mm = m < m_end ? m : m_base;
      rid[mb] = (uint32_t)(a.row_index ? a.row_index[mm] : mm);
    }
  }

  // Accumulators start at 0, or at -inf on columns that are not candidates
  // (the mask id, columns past the range): MFMA accumulation keeps them at
  // -inf, so the reduction needs no per-value test.
  auto init_acc = [&](int n0, int wofs) {
    const int vbase = n0 + wofs;
    const bool plain = (vbase + 128 <= v_hi) && (a.mask_id < vbase || a.mask_id >= vbase + 128);
    if (plain) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};
    } else {
      // column vbase + loff + c of value c: compare the lane part against
      // uniform bounds so that no per-value column index is kept in registers
      const int loff = 4 * (lane >> 5), lim = v_hi - vbase, mk = a.mask_id - vbase;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x16 b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = nb * 32 + 8 * (i >> 2) + (i & 3);
          b[i] = (loff < lim - c && loff != mk - c) ? 0.f : -INFINITY;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = b;
      }
    }
  };

  // Sampling draw of one block: the lane's 16 values x (log2 units, -inf
  // for non-candidates) of row block mb in 32-column chunk nb, columns
  // vb0 + 8*(i/4) + (i%4), block maximum bm.
  auto sample_block = [&](const float* x, float bm, int vb0, int nb, int mb) {
    // the lanes of this block and of the other half of the chunk draw the
    // same four words; half h uses words 2h and 2h+1
    uint32_t w0 = (uint32_t)((vb0 - 4 * (lane >> 5)) >> 5), w1 = rid[mb], w2 = a.step, w3 = 0u;
    philox4x32_10(w0, w1, w2, w3, a.key0, a.key1);
    const bool h = (lane >> 5) != 0;
    const float u = uniform01(h ? w2 : w0);
    const float eg = uniform01(h ? w3 : w1);
    if (bm == -INFINITY) return;                      // no candidate in this block
    const float bmT = bm * a.inv_temp;
    float e[16], S = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      e[i] = fast_exp2(fmaf(x[i], a.inv_temp, -bmT));
      S += e[i];
    }
    // inverse CDF: the first member whose running sum reaches u*S (the last
    // member with weight if rounding leaves none)
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
    // Gumbel at the block's log-sum-exp, log2 units (a constant shift of
    // m + ln S - ln(-ln e) in natural units)
    const float G = bmT + __log2f(S) - __log2f(-__log2f(eg));
    pick_fold(pick[mb], G, vb0 + 8 * (ci >> 2) + (ci & 3), xc * (1.0f / kLog2e));
    (void)nb;
  };

  // store a finished tile's logits: lane holds row (lane & 31) of each row
  // block mb and vocabulary rows vb0 + 8*(i/4) + (i%4) of each 32-block nb
  // store mode with pm given: the row maximum over the wave's columns of
  // the pass, kept in memory rather than in a register (the tile loop has
  // none to spare): slot (row, team) of pm for the wave with wn = 0, of pa
  // (as floats) for wn = 1, read, raised and written back by the one lane
  // that owns it after every tile (-inf written at the first)
  auto tile_max = [&](int mb, float tmx, bool first) {
    tmx = fmaxf(tmx, shfl_xor_f(tmx, 32));
    const int m = m_base + wm * RH + mb * 32 + lane;
    if (a.pm != nullptr && lane < 32 && m < m_end) {
      float* slot = (wn ? reinterpret_cast<float*>(a.pa) : a.pm) + (size_t)m * nteam + team;
      *slot = first ? tmx : fmaxf(*slot, tmx);
    }
  };
  auto store_tile = [&](auto nbw_c, int n0, int wofs, bool first) {
    constexpr int NBW = decltype(nbw_c)::value;
    const int vbase = n0 + wofs;
    if (vbase >= v_hi) {
      if (first)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) tile_max(mb, -INFINITY, true);
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m_base + wm * RH + mb * 32 + (lane & 31);
      float* lrow = a.logits + (size_t)(m < m_end ? m : m_base) * a.V;
      float tmx = -INFINITY;   // columns that are not candidates hold -inf
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
        const int vb0 = vbase + nb * 32 + 4 * (lane >> 5);
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float r;
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(acc[nb][mb][i]));
          x[i] = r;
        }
        if (m < m_end) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int v0 = vb0 + 8 * q;
            if (((a.V & 3) == 0) && v0 + 4 <= v_hi) {
              *reinterpret_cast<f32x4*>(lrow + v0) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (v0 + r < v_hi) lrow[v0 + r] = x[4 * q + r];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tmx = fmaxf(tmx, x[i]);
      }
      tile_max(mb, tmx, first);
    }
  };

  // reduce a finished tile: lane holds row (lane & 31) of each row block mb
  // and vocabulary rows 8*(i/4) + 4*(lane/32) + (i%4) of each 32-block nb
  auto reduce_tile = [&](auto nbw_c, int n0, int wofs) {
    constexpr int NBW = decltype(nbw_c)::value;
    const int vbase = n0 + wofs;
    if (vbase >= v_hi) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // block-online reduction of the lane's 16*NBW values of this row, 16
      // at a time: block max, lowest id reaching it, sum(2^(x - m)) rescaled
      // once per block.  Values are in log2 units; non-candidates are -inf.
      float m = -INFINITY, sum = 0.f, tt = 0.f;   // tt: sum 2^(x-m) (x-m)
      int idx = 0x7fffffff;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
        const int vb0 = vbase + nb * 32 + 4 * (lane >> 5);
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // read the accumulator from its AGPR here, not in one burst at the
          // loop exit (which would need all of them in VGPRs at once)
          float r;
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(acc[nb][mb][i]));
          x[i] = r * kLog2e;
        }
        float bm = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) bm = fmaxf(bm, x[i]);
        int bi = 0;   // offset of the lowest id reaching the block max (ids grow with i)
#pragma unroll
        for (int i = 15; i >= 0; --i) bi = (x[i] == bm) ? 8 * (i >> 2) + (i & 3) : bi;
        bi += vb0;
        if constexpr (SMP) sample_block(x, bm, vb0, nb, mb);
        const float mn = fmaxf(m, bm);
        float sb = 0.f, tb = 0.f;
        if (ENT) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // d >= -200: 2^d is then 0 in fp32 and d*2^d too (also for -inf)
            const float d = fmaxf(x[i] - mn, -200.f);
            const float e = fast_exp2(d);
            sb += e;
            tb = fmaf(e, d, tb);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) sb += fast_exp2(x[i] - mn);
        }
        sb = (mn == -INFINITY) ? 0.f : sb;            // all -inf so far: -inf - -inf
        tb = (mn == -INFINITY) ? 0.f : tb;
        const float scale = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
        if (ENT) tt = (m == -INFINITY) ? tb : fmaf(scale, fmaf(m - mn, sum, tt), tb);
        sum = fmaf(sum, scale, sb);
        idx = (bm > m) ? bi : idx;   // equal maxima keep the earlier, lower id
        m = mn;
      }
      __builtin_amdgcn_sched_barrier(0);
      // combine with the lane holding the other half of the row's values
      const float pm = shfl_xor_f(m, 32);
      const int pi = shfl_xor_i(idx, 32);
      const float ps = shfl_xor_f(sum, 32);
      const float pt = ENT ? shfl_xor_f(tt, 32) : 0.f;
      const float mx = fmaxf(m, pm);
      const float w1 = m == -INFINITY ? 0.f : fast_exp2(m - mx);
      const float w2 = pm == -INFINITY ? 0.f : fast_exp2(pm - mx);
      const float t1 = (!ENT || m == -INFINITY) ? 0.f : w1 * fmaf(m - mx, sum, tt);
      const float t2 = (!ENT || pm == -INFINITY) ? 0.f : w2 * fmaf(pm - mx, ps, pt);
      sum = sum * w1 + ps * w2;
      tt = t1 + t2;
      idx = (pm > m || (pm == m && pi < idx)) ? pi : idx;
      // to natural units: t = tt * ln 2
      fold(run[mb], mx * (1.0f / kLog2e), idx, sum, tt * (1.0f / kLog2e));
      if constexpr (SMP) {
        // the other half of each chunk
        const float g2 = shfl_xor_f(pick[mb].g, 32);
        const int c2 = shfl_xor_i(pick[mb].c, 32);
        const float l2 = shfl_xor_f(pick[mb].l, 32);
        pick_fold(pick[mb], g2, c2, l2);
      }
    }
  };

  // Ring schedule.  W waves: stages 0 and 1 up front; during stage s they
  // load stage s+2 into the slot released by the sync before stage s, a
  // quarter at the start of each k-step.  Hidden waves: stage 0 up front,
  // then right after the sync that ends stage s, stage s+2 into the slot of
  // stage s (a whole stage to land; the hidden rows are L2 hits).
  using I = std::integral_constant<int, 0>;
  if (WL) {
    issue(Wr);
    issue(Wr + WSLOT);
  } else {
    issue(Hr);
  }
  sync();
  if (!WL) issue(Hr + HSLOT);
  int ws = 0, hs = 0;      // ring slots of the stage being computed
  bf16x8 fa0[4], fb0[MB], fa1[4], fb1[MB];
  // Tile geometry of this wave: a full tile gives each of the two waves
  // sharing rows 128 columns (four 32-column blocks); a partial last tile of
  // nbl blocks gives each ceil(nbl/2) of them, so that both waves' MFMA
  // work shrinks with the tile (the sampling modes keep full-width tiles,
  // whose register budget has no room for more variants).  wofs: the
  // wave's first W row in the slot.
  auto tile_geom = [&](int t, int& wofs, int& nbw) {
    const int wt = min(NT, v_hi - (v_lo + tmap(t) * NT));
    const int h = wt >= NT ? 4 : ((wt + 31) / 32 + 1) / 2;
    wofs = wn * 32 * h;
    nbw = h;
  };
  int wofs_n = wn * 128, nbw_n = 4;   // geometry of the tile whose fragments are read next
  if constexpr (!SMP) {
    tile_geom(0, wofs_n, nbw_n);
    wfr = Wr + (wofs_n + fr) * TK;
  }
  read_frags(ws, hs, 0, fa0, fb0);

  for (int tile = 0; tile < ntile; ++tile) {
    const int n0 = v_lo + tmap(tile) * NT;
    const int wofs = wofs_n, nbw = nbw_n;
    if constexpr (!SMP) {
      if (tile + 1 < ntile) tile_geom(tile + 1, wofs_n, nbw_n);
    }
    auto run_tile = [&](auto nbw_c) {
      constexpr int NBW = decltype(nbw_c)::value;
      init_acc(n0, wofs);
      for (int kt = 0; kt < nk; ++kt) {
        lds_u16* const wt = Wr + (ws == 0 ? NWS - 1 : ws - 1) * WSLOT;
        constexpr int Q = WPW / 4;
        if (WL) issue_part(wt, I{}, std::integral_constant<int, Q>{});
        step(nbw_c, fa0, fb0, ws, hs, 1, fa1, fb1);
        if (WL) issue_part(wt, std::integral_constant<int, Q>{}, std::integral_constant<int, 2 * Q>{});
        step(nbw_c, fa1, fb1, ws, hs, 2, fa0, fb0);
        if (WL) issue_part(wt, std::integral_constant<int, 2 * Q>{}, std::integral_constant<int, 3 * Q>{});
        step(nbw_c, fa0, fb0, ws, hs, 3, fa1, fb1);
        if (WL) {
          issue_part(wt, std::integral_constant<int, 3 * Q>{}, std::integral_constant<int, 4 * Q>{});
          advance();
        }
        // k-step 3: half its MFMAs, the sync for the next stage, the hidden
        // loads, and the other half under the next stage's first fragments
        // (of the next tile after the last stage)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB / 2; ++mb) mfma_rows(nbw_c, fa1, fb1, mb);
        __builtin_amdgcn_sched_barrier(0);
        sync();
        if (!WL) issue(Hr + hs * HSLOT);
        ws = ws == NWS - 1 ? 0 : ws + 1;
        hs = hs == NHS - 1 ? 0 : hs + 1;
        if constexpr (!SMP) {
          if (kt == nk - 1) wfr = Wr + (wofs_n + fr) * TK;
        }
        __builtin_amdgcn_sched_barrier(0);
        read_frags(ws, hs, 0, fa0, fb0);
#pragma unroll
        for (int mb = MB / 2; mb < MB; ++mb) mfma_rows(nbw_c, fa1, fb1, mb);
        constexpr int NM2 = NBW * (MB - MB / 2), NP2 = NM2 < 4 + MB ? NM2 : 4 + MB;
#pragma unroll
        for (int r = 0; r < NP2; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        }
        if (4 + MB > NP2) __builtin_amdgcn_sched_group_barrier(0x100, 4 + MB - NP2, 0);
        if (NM2 > NP2) __builtin_amdgcn_sched_group_barrier(0x008, NM2 - NP2, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (STO) store_tile(nbw_c, n0, wofs, tile == 0);
      else reduce_tile(nbw_c, n0, wofs);
    };
    if constexpr (SMP) {
      run_tile(std::integral_constant<int, 4>{});
    } else {
      switch (nbw) {
        case 1: run_tile(std::integral_constant<int, 1>{}); break;
        case 2: run_tile(std::integral_constant<int, 2>{}); break;
        case 3: run_tile(std::integral_constant<int, 3>{}); break;
        default: run_tile(std::integral_constant<int, 4>{}); break;
      }
    }
  }

  // all loads have landed and every wave is past its last fragment read
  wait_vm<0>();
  wait_lgkm0();
  barrier_only();

  // fold the two waves that share rows, then one partial per row
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) int lds_i32;
  if constexpr (STO) return;
  lds_f32* const s_m = (lds_f32*)Hr;
  lds_i32* const s_a = (lds_i32*)(Hr + 2 * 256);
  lds_f32* const s_s = (lds_f32*)(Hr + 4 * 256);
  lds_f32* const s_t = (lds_f32*)(Hr + 6 * 256);
  lds_f32* const s_g = (lds_f32*)(Hr + 8 * 256);
  lds_i32* const s_c = (lds_i32*)(Hr + 10 * 256);
  lds_f32* const s_l = (lds_f32*)(Hr + 12 * 256);
  if (wn == 1 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int k = (wm * MB + mb) * 32 + lane;
      s_m[k] = run[mb].m;
      s_a[k] = run[mb].a;
      s_s[k] = run[mb].s;
      s_t[k] = run[mb].t;
      if constexpr (SMP) {
        s_g[k] = pick[mb].g;
        s_c[k] = pick[mb].c;
        s_l[k] = pick[mb].l;
      }
    }
  }
  __syncthreads();
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int k = (wm * MB + mb) * 32 + lane;
      fold(run[mb], s_m[k], s_a[k], s_s[k], s_t[k]);
      if constexpr (SMP) pick_fold(pick[mb], s_g[k], s_c[k], s_l[k]);
      const int m = m_base + wm * RH + mb * 32 + lane;
      if (m < m_end) {
        const size_t o = (size_t)m * nteam + team;
        a.pm[o] = run[mb].m;
        a.pa[o] = SMP ? pick[mb].c : run[mb].a;
        a.ps[o] = run[mb].s;
        if (ENT) a.pt[o] = run[mb].t;
        if constexpr (SMP) {
          a.pg[o] = pick[mb].g;
          a.pl[o] = pick[mb].l;
        }
      }
    }
  }
  __syncthreads();   // the partial scratch is read before the next pass loads
}

template <int MB, int MODE>
__device__ __forceinline__ void lm_pass_any(const LmArgs& a, int m_base, int m_end, int v_lo, int v_hi,
                                            int team, int nteam, lds_u16* Wr, lds_u16* Hr) {
  if (v_hi <= v_lo) {
    if (MODE & 4) {
      // store mode: nothing to store; neutral partial maxima if asked
      if (a.pm != nullptr)
        for (int m = m_base + (int)threadIdx.x; m < m_end; m += blockDim.x) {
          a.pm[(size_t)m * nteam + team] = -INFINITY;
          reinterpret_cast<float*>(a.pa)[(size_t)m * nteam + team] = -INFINITY;
        }
      return;
    }
    // an empty vocabulary range still leaves a neutral partial for its rows
    for (int m = m_base + (int)threadIdx.x; m < m_end; m += blockDim.x) {
      const size_t o = (size_t)m * nteam + team;
      a.pm[o] = -INFINITY;
      a.pa[o] = 0x7fffffff;
      a.ps[o] = 0.f;
      a.pt[o] = 0.f;
      if (MODE & 2) {
        a.pg[o] = -INFINITY;
        a.pl[o] = 0.f;
      }
    }
    return;
  }
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 2)
    lm_pass<MB, true, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr);
  else
    lm_pass<MB, false, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr);
}
}  // namespace

template <int MODE>
__global__ __launch_bounds__(256, 1) void lmhead_tile_kernel(LmArgs a) {
  __shared__ __align__(16) uint16_t Wr_[NWS * WSLOT];
  __shared__ __align__(16) uint16_t Hr_[NHS * HSLOT];
  lds_u16* const Wr = (lds_u16*)Wr_;
  lds_u16* const Hr = (lds_u16*)Hr_;
  const int M = *a.num_rows;
  if (M <= 0) return;
  const int G = team_size(M), nteam = kLmGrid / G;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;       // 32 workgroups per XCD
  const int member = local % G, team = xcd * (32 / G) + local / G;
  const int nblk = (a.V + 31) / 32;
  const int v_lo = min(a.V, (int)(((long)team * nblk) / nteam) * 32);
  const int v_hi = min(a.V, (int)(((long)(team + 1) * nblk) / nteam) * 32);
  const int pass_rows = RMAX * G;
  for (int p0 = 0; p0 < M; p0 += pass_rows) {
    const int Mp = min(pass_rows, M - p0);
    const int R = min(RMAX, (((Mp + G - 1) / G) + 63) / 64 * 64);
    const int m_base = p0 + member * R;
    const int m_end = min(m_base + R, p0 + Mp);
    if (m_base >= m_end) continue;
    switch (R / 64) {
      case 1: lm_pass_any<1, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr); break;
      case 2: lm_pass_any<2, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr); break;
      case 3: lm_pass_any<3, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr); break;
      default: lm_pass_any<4, MODE>(a, m_base, m_end, v_lo, v_hi, team, nteam, Wr, Hr); break;
    }
  }
}

__global__ __launch_bounds__(256) void lmhead_merge_kernel(LmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const int M = *a.num_rows;
  if (r >= M) return;
  const int nteam = kLmGrid / team_size(M);
  const size_t base = (size_t)r * nteam;
  Part x{-INFINITY, 0x7fffffff, 0.f, 0.f};
  Pick pk{-INFINITY, 0x7fffffff, 0.f};
  const bool ent = a.entropy != nullptr, smp = a.sample != 0;
  for (int t = lane; t < nteam; t += 64) {
    fold(x, a.pm[base + t], a.pa[base + t], a.ps[base + t], ent ? a.pt[base + t] : 0.f);
    if (smp) pick_fold(pk, a.pg[base + t], a.pa[base + t], a.pl[base + t]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = shfl_xor_f(x.m, off);
    const int a2 = shfl_xor_i(x.a, off);
    const float s2 = shfl_xor_f(x.s, off);
    const float t2 = shfl_xor_f(x.t, off);
    fold(x, m2, a2, s2, t2);
    const float g2 = shfl_xor_f(pk.g, off);
    const int c2 = shfl_xor_i(pk.c, off);
    const float l2 = shfl_xor_f(pk.l, off);
    pick_fold(pk, g2, c2, l2);
  }
  if (lane == 0) {
    const int row = a.row_index ? a.row_index[r] : r;
    if (x.m == -INFINITY) {
      // no candidate (every logit but the mask's is -inf): no distribution;
      // the mask token with confidence 0 and entropy +inf
      a.argmax_tok[row] = a.mask_id;
      a.conf[row] = 0.f;
      if (a.entropy) a.entropy[row] = INFINITY;
    } else {
      if (smp) {
        // the drawn token and its probability at temperature 1
        a.argmax_tok[row] = pk.c;
        a.conf[row] = __expf(pk.l - x.m) / x.s;
      } else {
        a.argmax_tok[row] = x.a;
        a.conf[row] = 1.f / x.s;
      }
      if (a.entropy) a.entropy[row] = __logf(x.s) - x.t / x.s;
    }
  }
}

size_t lmhead_ws_bytes(int max_rows, int V) {
  (void)V;
  const size_t one = ((size_t)max_rows * kLmGrid * 4 + 255) & ~(size_t)255;
  return kLmPartArrays * one;
}

hipError_t lmhead_launch(const LmArgs& a, hipStream_t st) {
  // the entropy sums only when a caller wants the entropy, the draw only
  // when sampling
  if (a.logits) {
    // the logits themselves: no partials, no merge
    lmhead_tile_kernel<4><<<kLmGrid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const int mode = (a.entropy ? 1 : 0) | (a.sample ? 2 : 0);
  if (mode == 0) lmhead_tile_kernel<0><<<kLmGrid, 256, 0, st>>>(a);
  else if (mode == 1) lmhead_tile_kernel<1><<<kLmGrid, 256, 0, st>>>(a);
  else if (mode == 2) lmhead_tile_kernel<2><<<kLmGrid, 256, 0, st>>>(a);
  else lmhead_tile_kernel<3><<<kLmGrid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lmhead_merge_kernel<<<(a.max_rows + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
