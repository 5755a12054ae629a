// Block-diffusion attention over a paged KV cache, gfx950.
//
// The denoise step's attention (JetEngine developer notes, "ModelRunner" and
// "Layers"; README architecture tree, "Paged KV Cache"): each query of a
// sequence's block attends to all of that sequence's prefix tokens, found
// through its page table, and to every token of its own block, with no mask
// inside the block.  Grouped-query heads: the G = Hq/Hkv query heads of kv
// head g share its keys and values; their G*B query rows form MFMA tiles of
// 16 rows (RT tiles per row group).
//
// Work decomposition.  A segment is (sequence s, kv head g, row group rg); it
// owns ceil(L_s/kKT) prefix tiles of kKT keys plus ceil(B/kKT) tiles of the
// block's own keys.  All segments, in order, form one global tile stream,
// which is cut into equal contiguous ranges, one per single-wave workgroup
// (at least kMinTilesPerWave tiles each): every wave streams the same number
// of tiles whatever the prefix lengths.  A wave finishes each segment it
// touches with (max, sum, unnormalised output); a segment split over several
// waves leaves fp32 partials that attn_combine_kernel merges, one that fits
// in one wave is written directly.  A wave's range cuts at most two segments
// (at its two ends), so the partials take two slots per wave; every piece
// records its segment's piece count and first slot for the combine launch.
// Each wave first turns the prefix lengths into tile prefix sums itself: a
// separate planning launch would cost more than the few loads it saves.
//
// Per wave, tiles go straight from global memory into a ring of NR LDS
// slots (global_load_lds_dwordx4, non-temporal: kKT keys of K and of V in
// runs of 16 that never cross a page), NR-1 tiles in flight while one is
// computed.  NR is 2 (four waves per CU), or 3 for 16-row segments in a
// launch whose page tables can hold kDeepRingTiles tiles or more (two waves
// per CU, two tiles in flight each: a long stream per wave takes fewer
// pauses; a short one pays more for filling the deeper ring).  A 16-row segment's query rows ride along in a small region of
// its first tile's slot and go from there into the MFMA operand registers
// (a load from global memory at that point would drain the ring: the
// compiler's wait for it counts every load before it); larger row groups
// load them from global memory, so their slots hold K and V only and the
// waves per CU do not shrink with the rows per segment.  Rows are stored with
// their 16-byte chunks XOR-permuted by row so fragment reads hit distinct
// banks.  Per run of 32 keys:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 for each 16-key half
//     (lane: query row, 4 keys of each half);
//   * online softmax in fp32, base 2 (scores pre-scaled by scale*log2 e),
//     probabilities rounded to bf16 for the MFMA, the row sum taken over the
//     rounded values; the running maximum moves only when it grows by more
//     than 2^8, so most runs skip the accumulator rescale;
//   * the two halves' score accumulators together are the B operand of
//     O^T += V^T P^T with the K = 32 MFMA (v_mfma_f32_16x16x32_bf16, twice
//     the rate of the K = 16 form); the V^T operand comes straight from the
//     row-major V rows with the LDS transpose read ds_read_b64_tr_b16.
// Keys past the end of a prefix or block are masked to -inf; their loads
// re-read a valid key, so nothing past a page or buffer is touched.
//
// Gate: with AttnArgs::gate set, all three kernels return at once when the
// device count it points to is 0 -- a round of a device-side block loop
// that has nothing left to denoise.
//
// SAVING forward (the SAVE instances): the forward over a finished block
// also stores the block's keys and values into the sequence's pages at
// positions prefix_len + j (JetEngine developer notes, "Important
// Patterns": the SAVING forward writes the final block into the KV cache;
// "Optimization History": one kernel both writes the cache and attends).
// The wave that consumes a block tile of row group 0 copies the tile's
// valid rows from LDS to the cache after computing on it.  Nothing in the
// same launch reads those slots: prefix reads stop below prefix_len.
#include <algorithm>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#define INL __attribute__((always_inline))

#ifndef ATTN_RING
#define ATTN_RING 2
#endif
#ifndef ATTN_WAVES
#define ATTN_WAVES 4
#endif
#ifndef ATTN_KT
#define ATTN_KT 32
#endif
#ifndef ATTN_NT
#define ATTN_NT 1
#endif
constexpr int kKT = ATTN_KT;   // keys per tile (a multiple of 32)
static_assert(kKT % 32 == 0, "runs of 32 keys");
constexpr int kRing = ATTN_RING;       // ring slots per wave (the deep ring: kRing + 1)
constexpr int kDeepRingTiles = 65536;
constexpr int kMaxWavesPerCU = ATTN_WAVES;
constexpr int kCUs = 256;      // MI355X compute units
constexpr int kLdsPerCU = 160 * 1024;
constexpr int kSavingState = 3;   // sequence state SAVING
// a wave streams at least this many tiles (a small launch uses fewer waves
// rather than many waves with a handful of tiles each)
constexpr int kMinTilesPerWave = 16;

// chunk permutation of row r (D=128: 16 chunks per row; D=64: 8)
template <int D>
__device__ __forceinline__ int rswz(int r) {
  return D == 128 ? (r & 15) : (((r >> 1) ^ ((r & 1) << 2)) & 7);
}
// element offset of logical 16-byte chunk c of row r
template <int D>
__device__ __forceinline__ int eoff(int r, int c) {
  return r * D + ((c ^ rswz<D>(r)) << 3);
}

#ifndef ATTN_QLDS
#define ATTN_QLDS 1
#endif

template <int D, int RT>
struct Geo {
  static constexpr int ROWS = 16 * RT;
  static constexpr int KS = D / 32;
  static constexpr int DT = D / 16;
  static constexpr int KV = kKT * D;                // elements of one K (or V) tile
  // 16-row segments also stage their query rows in the slot of their first
  // tile (a 4 KB region at D = 128), so that a segment start reads them from
  // LDS instead of global memory; larger row groups keep the slots small
  // (four waves per CU) and load their query rows from global memory
  static constexpr bool QLDS = ATTN_QLDS != 0 && RT == 1;
  static constexpr int QE = QLDS ? ROWS * D : 0;    // elements of the query region
  static constexpr int SLOT = 2 * KV + QE;          // K, V, query rows
  static constexpr int LPR = D / 8;                 // lanes per row in a 1 KB load
  static constexpr int RPI = 64 / LPR;              // rows per 1 KB load
};

// LDS bytes of one ring slot (the plan sizes the launch with it)
inline int attn_slot_bytes(int D, int RT) {
  const bool q = ATTN_QLDS != 0 && RT == 1;
  return (2 * kKT * D + (q ? 16 * RT * D : 0)) * 2;
}

// One direct-to-LDS load: lane l copies 16 bytes from its own global address
// to lds + 16*l.  Issued as inline assembly so that the compiler neither
// pairs it with its own vmcnt bookkeeping nor moves LDS accesses across it
// (the memory clobber); the ring's waits are explicit (wait_vm).  M0 carries
// the LDS base; the s_nop is the wait state a fresh M0 needs before an LDS
// DMA reads it.  The loads are non-temporal (nt): every prefix key and value
// is read once per launch, and streaming them past the caches raised a plain
// read of this shape from 5.7 to 6.7-7.0 TB/s on the device.
__device__ __forceinline__ void dma16(const void* g, const lds_u16* lds) {
#if ATTN_NT
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(g), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
#else
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "{m0}"((uint32_t)(uintptr_t)lds) : "memory");
#endif
}

// Copy 16 rows (row i from src0 + min(i, nvalid-1)*stride) into a region of
// the ring, permuting chunks; lane l of each 1 KB load fills row
// r0 + l/LPR, physical chunk l%LPR.
template <int D, int RT>
__device__ __forceinline__ void dma_rows16(lds_u16* dst, const uint16_t* src0, int stride,
                                           int nvalid, int lane) {
  using Gm = Geo<D, RT>;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += Gm::RPI) {
    const int row = r0 + lane / Gm::LPR;
    const int lc = (lane % Gm::LPR) ^ rswz<D>(row);
    const int srow = min(row, nvalid - 1);
    dma16(src0 + (size_t)srow * stride + lc * 8, dst + r0 * D);
  }
}

// Uniform loads of read-only metadata through the scalar cache (constant
// address space), so they never join the vector-memory counter that paces
// the LDS ring.
__device__ __forceinline__ int ldc(const int32_t* p, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// s_waitcnt vmcnt(n), also a compiler barrier for memory accesses
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// all of this wave's LDS reads (and scalar loads) have returned
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// state of sequence s through the scalar cache: the aligned dword holding
// byte s (the state array is 16-byte aligned, so that dword never crosses
// the end of the page holding byte s)
__device__ __forceinline__ int state_of(const uint8_t* st, int s) {
  const uint32_t w = (uint32_t)ldc(reinterpret_cast<const int32_t*>(st), (size_t)(s >> 2));
  return (int)((w >> (8 * (s & 3))) & 0xFFu);
}

struct Dec {      // a position in the tile stream
  int s, hg, j;   // sequence, segment within the sequence, tile within the segment
  int L, nP, tiles;
  int p;          // tiles of all sequences before s
};

}  // namespace

template <int D, int RT, int NR, bool SAVE>
__global__ __launch_bounds__(64) void attn_stream_kernel(AttnArgs a) {
  using Gm = Geo<D, RT>;
  constexpr int ROWS = Gm::ROWS, KS = Gm::KS, DT = Gm::DT, KV = Gm::KV;
  __shared__ __align__(16) uint16_t ring_[NR * Gm::SLOT];
  lds_u16* const ring = (lds_u16*)ring_;

  if (a.gate != nullptr && ldc(a.gate, 0) <= 0) return;
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int S = a.S, NHG = a.Hkv * a.n_rg, nB = (a.B + kKT - 1) / kKT;
  const int R = a.G * a.B;
  // tile prefix sums plan(s) = tiles of the sequences before s (each has
  // ceil(L/kKT) + nB >= 1 tiles): lane l sums sequences [l*c, l*c + c)
  const int c = (S + 63) / 64;
  int mine = 0;
  for (int i = 0; i < c; ++i) {
    const int s = lane * c + i;
    if (s < S) mine += (a.prefix_len[s] + kKT - 1) / kKT + nB;
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int start = incl - mine;                                    // plan(l*c)
  const long T = (long)NHG * __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  const long NWe = min((long)a.grid, max(1L, T / kMinTilesPerWave));
  const long w = blockIdx.x;
  if (w >= NWe) return;
  const long t0 = w * T / NWe, t1 = (w + 1) * T / NWe;
  const int n = (int)(t1 - t0);
  if (n <= 0) return;

  // locate t0: the largest s with NHG*plan(s) <= t0 -- the lane whose
  // sequences hold it (lane 0 always qualifies: plan(0) = 0), then a walk
  // through that lane's at most c sequences
  const unsigned long long bal = __ballot(lane * c < S && (long)NHG * start <= t0);
  const int k = 63 - __clzll(bal);
  int s_lo = __builtin_amdgcn_readfirstlane(k * c);
  int p_lo = __builtin_amdgcn_readfirstlane(__shfl(start, k, 64));
  for (int i = 1; i < c && s_lo + 1 < S; ++i) {
    const int tl = (ldc(a.prefix_len, s_lo) + kKT - 1) / kKT + nB;
    if ((long)NHG * (p_lo + tl) > t0) break;
    ++s_lo;
    p_lo += tl;
  }
  auto load_seq = [&](Dec& d) INL {
    d.L = ldc(a.prefix_len, d.s);
    d.nP = (d.L + kKT - 1) / kKT;
    d.tiles = d.nP + nB;
  };
  Dec dc;
  dc.s = s_lo;
  dc.p = p_lo;
  load_seq(dc);
  {
    const long rem = t0 - (long)NHG * p_lo;
    dc.hg = (int)(rem / dc.tiles);
    dc.j = (int)(rem % dc.tiles);
  }
  Dec dd = dc;                 // stream position of the next tile to load
  auto advance = [&](Dec& d) INL {
    if (++d.j == d.tiles) {
      d.j = 0;
      if (++d.hg == NHG) {
        d.hg = 0;
        d.p += d.tiles;
        if (++d.s < S) load_seq(d);
      }
    }
  };

  // load tile `d` into `slot` (with_q: also the segment's query rows)
  auto dma_tile = [&](lds_u16* slot, const Dec& d, bool with_q) INL {
    wait_lgkm0();   // the slot's previous tile has been read out
    const int g = d.hg / a.n_rg, rg = d.hg % a.n_rg;
    if constexpr (Gm::QLDS) {
      if (with_q) {
        // query row r of the row group: rr = rg*ROWS + r -> (pos, gi) =
        // (rr / G, rr % G); rows past G*B re-read the last real row (never
        // written out); chunks permuted by row as in the K/V tiles
#pragma unroll
        for (int r0 = 0; r0 < ROWS; r0 += Gm::RPI) {
          const int row = r0 + lane / Gm::LPR;
          const int rr = min(rg * ROWS + row, R - 1);
          const int pos = rr / a.G, gi = rr % a.G;
          const int lc = (lane % Gm::LPR) ^ rswz<D>(row);
          dma16(a.q + ((size_t)(d.s * a.B + pos) * a.Hq + g * a.G + gi) * D + lc * 8, slot + 2 * KV + r0 * D);
        }
      }
    }
    // kKT/16 runs of 16 keys; a run never crosses a page (the page size is a
    // multiple of 16).  A run wholly past the end re-reads the tile's first
    // key (its scores are masked).
#pragma unroll
    for (int hh = 0; hh < kKT / 16; ++hh) {
      const uint16_t* sk;
      const uint16_t* sv;
      int stride, nvalid;
      if (d.j < d.nP) {
        int key0 = kKT * d.j + 16 * hh;
        nvalid = min(16, d.L - key0);
        if (nvalid <= 0) key0 = kKT * d.j, nvalid = 1;
        const int page = ldc(a.page_table, (size_t)d.s * a.max_pages + key0 / a.P);
        const size_t base = (((size_t)page * a.Hkv + g) * a.P + key0 % a.P) * D;
        sk = a.k_cache + base;
        sv = a.v_cache + base;
        stride = D;
      } else {
        int key0 = kKT * (d.j - d.nP) + 16 * hh;
        nvalid = min(16, a.B - key0);
        if (nvalid <= 0) key0 = kKT * (d.j - d.nP), nvalid = 1;
        const size_t base = ((size_t)(d.s * a.B + key0) * a.Hkv + g) * D;
        sk = a.k_blk + base;
        sv = a.v_blk + base;
        stride = a.Hkv * D;
      }
      dma_rows16<D, RT>(slot + hh * 16 * D, sk, stride, nvalid, lane);
      dma_rows16<D, RT>(slot + KV + hh * 16 * D, sv, stride, nvalid, lane);
    }
  };

  // per-segment state
  bf16x8 qf[RT][KS];
  float m_run[RT], l_run[RT];
  f32x4 acc[RT][DT];

  auto finalize = [&](const Dec& d) INL {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      l_run[rt] += shfl_xor_f(l_run[rt], 16);
      l_run[rt] += shfl_xor_f(l_run[rt], 32);
    }
    const int g = d.hg / a.n_rg, rg = d.hg % a.n_rg;
    const long ts = (long)NHG * d.p + (long)d.hg * d.tiles;
    const long w0 = ((ts + 1) * NWe - 1) / T;
    const long w1 = ((ts + d.tiles) * NWe - 1) / T;
    // A wave's range splits at most two segments: the one holding its first
    // tile (partial slot 2w) and the one holding its last (slot 2w + 1).
    // Every piece of a segment records the same word: its piece count, its
    // first wave, and which of that wave's slots the first piece took (the
    // others always take slot 2w), so the combine reads one word.
    const int side0 = ts == w0 * T / NWe ? 0 : 1;
    if (lane == 0) a.seg_np[d.s * NHG + d.hg] = (int)(w1 - w0 + 1) | (side0 << 11) | ((int)w0 << 12);
    if (w0 == w1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int rr = rg * ROWS + rt * 16 + lr;
        if (rr < R) {
          const float inv = 1.f / l_run[rt];
          const int pos = rr / a.G, gi = rr % a.G;
          uint16_t* op = a.out + ((size_t)(d.s * a.B + pos) * a.Hq + g * a.G + gi) * D + 4 * lg;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            u32x2 v;
            v.x = pack_bf16x2(acc[rt][dt].x * inv, acc[rt][dt].y * inv);
            v.y = pack_bf16x2(acc[rt][dt].z * inv, acc[rt][dt].w * inv);
            *reinterpret_cast<u32x2*>(op + 16 * dt) = v;
          }
        }
      }
    } else {
      const size_t slot = (size_t)(2 * w + (ts <= t0 ? 0 : 1)) * ROWS;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const size_t row = slot + rt * 16 + lr;
        float* po = a.part_o + row * D + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = acc[rt][dt];
        if (lg == 0) a.part_ml[row] = make_float2(m_run[rt], l_run[rt]);
      }
    }
  };

  // SAVING forward: copy the valid rows of block tile dc (K and V, in LDS)
  // to the cache at positions L + key; lane l moves 16-byte chunks l,
  // l+64, ... of each run of 16 rows
  auto save_tile = [&](const lds_u16* slot) {
    const int g = dc.hg / a.n_rg;
    const int kb = kKT * (dc.j - dc.nP);
#pragma unroll
    for (int hh = 0; hh < kKT / 16; ++hh) {
      const int nvalid = min(16, a.B - (kb + 16 * hh));
#pragma unroll
      for (int i = lane; i < 16 * Gm::LPR; i += 64) {
        const int r = i / Gm::LPR, c = i % Gm::LPR;
        if (r >= nvalid) continue;
        const int pos = dc.L + kb + 16 * hh + r;
        const int pidx = pos / a.P;
        if (pidx >= a.max_pages) continue;
        const int page = a.page_table[(size_t)dc.s * a.max_pages + pidx];
        if (page < 0 || page >= a.num_pages) continue;
        const size_t dst = (((size_t)page * a.Hkv + g) * a.P + pos % a.P) * D + c * 8;
        const int src = hh * 16 * D + eoff<D>(r, c);
        *reinterpret_cast<u32x4*>(a.k_cache_out + dst) = *(const lds_u32x4*)(slot + src);
        *reinterpret_cast<u32x4*>(a.v_cache_out + dst) = *(const lds_u32x4*)(slot + KV + src);
      }
    }
  };

  auto consume = [&](const lds_u16* slot, int k) INL {
    // every tile issues at least 2*D/32 loads (K and V) and NR-1 tiles were
    // issued after this one: waiting down to that many leaves this slot done
    wait_vm<(NR - 1) * 2 * Gm::KV / 512>();
    if (k > 0 && dc.j == 0) {
      // the previous tile closed a segment
      Dec prev = dc;
      if (prev.hg == 0) {
        --prev.s;
        load_seq(prev);
        prev.p -= prev.tiles;
        prev.hg = NHG - 1;
      } else {
        --prev.hg;
      }
      finalize(prev);
    }
    if (k == 0 || dc.j == 0) {
      // the segment's query rows into the MFMA operand registers: from the
      // slot's query region (16-row segments), else straight from global
      // memory: row r = rg*ROWS + i -> (pos, gi) = (r / G, r % G); rows past
      // G*B re-read the last real row (never written out)
      const int g = dc.hg / a.n_rg, rg = dc.hg % a.n_rg;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (Gm::QLDS) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qf[rt][ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(slot + 2 * KV + eoff<D>(lr, lg + 4 * ks)));
        } else {
          const int rr = min(rg * ROWS + rt * 16 + lr, R - 1);
          const int pos = rr / a.G, gi = rr % a.G;
          const uint16_t* qp = a.q + ((size_t)(dc.s * a.B + pos) * a.Hq + g * a.G + gi) * D;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = ld_bf16x8(qp + (lg + 4 * ks) * 8);
        }
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const int nvalid_t = dc.j < dc.nP ? dc.L - kKT * dc.j : a.B - kKT * (dc.j - dc.nP);
    // runs of 32 keys: S^T for two 16-key halves, one softmax step, and
    // O^T += V^T P^T with K = 32 MFMAs whose k slots 8*lg .. 8*lg+7 hold keys
    // 4*lg .. 4*lg+3 of the first half, then of the second (the same order
    // in both operands).  Keys past the valid count are -inf.
#pragma unroll
    for (int h2 = 0; h2 < kKT / 32; ++h2) {
      f32x4 sc[2][RT];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const lds_u16* kt16 = slot + (2 * h2 + hh) * 16 * D;
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(kt16 + eoff<D>(lr, lg + 4 * ks)));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          sc[hh][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            sc[hh][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[rt][ks], sc[hh][rt], 0, 0, 0);
        }
      }
      const int nv0 = nvalid_t - 32 * h2;        // valid keys from this run's first (may be <= 0)
      float xs[RT][8], tmax[RT];
      bool grow = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        tmax[rt] = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = 16 * (i >> 2) + 4 * lg + (i & 3);
          xs[rt][i] = key < nv0 ? sc[i >> 2][rt][i & 3] * a.scale_log2 : -INFINITY;
          tmax[rt] = fmaxf(tmax[rt], xs[rt][i]);
        }
        tmax[rt] = max_xor32(max_xor16(tmax[rt]));
        grow |= tmax[rt] > m_run[rt] + 8.f;
      }
      // the running maxima (and the rescale) move only when some row's
      // maximum grows by more than 2^8; below that, probabilities up to 2^8
      // against the old maxima are exact in the fp32 sums.  A run with no
      // valid key leaves everything as it is.
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
          const uint32_t w = pack_bf16x2(fast_exp2(xs[rt][i] - m_run[rt]),
                                         fast_exp2(xs[rt][i + 1] - m_run[rt]));
          psum += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
          pw[i >> 1] = w;
        }
        pb[rt] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        l_run[rt] += psum;
      }
      // O^T[d][row] += V^T[d][key] P^T[key][row]: in each half, lane w of
      // 16-lane group lg needs V[keys 4*lg .. 4*lg+3][d = 16*dt + w].
      // ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of
      // the 8-byte words read by lanes i/4 + 4k (k = 0..3) of its group, so
      // lane w of group lg reads V[4*lg + w/4][16*dt + 4*(w%4) .. +3].
      const lds_u16* vt = slot + KV + 2 * h2 * 16 * D;
      const int vrow = 4 * lg + (lr >> 2), vsub = 4 * (lr & 1), vch = (lr & 3) >> 1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vt + eoff<D>(vrow, 2 * dt + vch) + vsub));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vt + 16 * D + eoff<D>(vrow, 2 * dt + vch) + vsub));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v8 = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], acc[rt][dt], 0, 0, 0);
      }
    }
    if constexpr (SAVE) {
      if (dc.j >= dc.nP && dc.hg % a.n_rg == 0 && state_of(a.save_state, dc.s) == kSavingState) save_tile(slot);
    }
  };

  // the stream: tiles 0..n-1; loads run NR-1 tiles ahead (past the end
  // they repeat the last tile into the idle slot)
  // a tile carries its segment's query rows when it starts the segment or
  // the wave's range (the first tile, kt = 0, may start mid-segment)
  auto next_dma = [&](lds_u16* slot, int kt) INL {
    dma_tile(slot, dd, kt == 0 || dd.j == 0);
    if (kt + 1 < n) advance(dd);
  };
#pragma unroll
  for (int u = 0; u + 1 < NR; ++u) next_dma(ring + u * Gm::SLOT, u);
  for (int k = 0; k < n; k += NR) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      next_dma(ring + ((u + NR - 1) % NR) * Gm::SLOT, k + u + NR - 1);
      if (u == 0 || k + u < n) {
        consume(ring + u * Gm::SLOT, k + u);
        advance(dc);
      }
    }
  }
  // close the last segment: dc now points one past the last tile
  {
    Dec prev = dc;
    if (prev.j == 0) {
      if (prev.hg == 0) {
        --prev.s;
        load_seq(prev);
        prev.p -= prev.tiles;
        prev.hg = NHG - 1;
      } else {
        --prev.hg;
      }
      prev.j = prev.tiles - 1;
    } else {
      --prev.j;
    }
    finalize(prev);
  }
  wait_vm<0>();   // no load may land in LDS after the wave is gone
}

// Merge the partials of segments split over several waves.  One workgroup
// per segment; the stream kernel recorded each segment's piece count, and
// segments in one piece (written directly) return at once.
constexpr int kCombineThreads = 128;

template <int D, int RT>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int ROWS = 16 * RT;
  if (a.gate != nullptr && *a.gate <= 0) return;
  const int NHG = a.Hkv * a.n_rg;
  const int seg = blockIdx.x;
  const int rec = a.seg_np[seg];
  const int pieces = rec & 0x7FF;
  if (pieces <= 1) return;
  const int side0 = (rec >> 11) & 1, w0 = rec >> 12;
  // piece p came from wave w0 + p, slot 2(w0 + p) (+1 for the first piece
  // when it was its wave's second split segment)
  auto pslot = [&](int p) { return (size_t)(2 * (w0 + p) + (p == 0 ? side0 : 0)); };
  const int s = seg / NHG, hg = seg % NHG;
  const int g = hg / a.n_rg, rg = hg % a.n_rg;
  const int R = a.G * a.B;
  for (int idx = threadIdx.x; idx < ROWS * (D / 8); idx += kCombineThreads) {
    const int row = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
    const int rr = rg * ROWS + row;
    if (rr >= R) continue;
    // the first kCombineFirst pieces' (m, l) and partial rows are loaded
    // together (one round trip for the usual two pieces); any further piece
    // is read in the loops.  The sums run in piece order either way.
    constexpr int kCombineFirst = 4;
    float2 mlf[kCombineFirst];
    f32x4 lof[kCombineFirst], hif[kCombineFirst];
#pragma unroll
    for (int p = 0; p < kCombineFirst; ++p) {
      if (p < pieces) {
        mlf[p] = a.part_ml[pslot(p) * ROWS + row];
        const float* po = a.part_o + (pslot(p) * ROWS + row) * D + d0;
        lof[p] = *reinterpret_cast<const f32x4*>(po);
        hif[p] = *reinterpret_cast<const f32x4*>(po + 4);
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kCombineFirst; ++p)
      if (p < pieces) M = fmaxf(M, mlf[p].x);
    for (int p = kCombineFirst; p < pieces; ++p) M = fmaxf(M, a.part_ml[pslot(p) * ROWS + row].x);
    float Ls = 0.f, o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
    auto add_piece = [&](float2 ml, f32x4 lo4, f32x4 hi4) {
      const float wgt = fast_exp2(ml.x - M);
      Ls += ml.y * wgt;
      o[0] += wgt * lo4.x; o[1] += wgt * lo4.y; o[2] += wgt * lo4.z; o[3] += wgt * lo4.w;
      o[4] += wgt * hi4.x; o[5] += wgt * hi4.y; o[6] += wgt * hi4.z; o[7] += wgt * hi4.w;
    };
#pragma unroll
    for (int p = 0; p < kCombineFirst; ++p)
      if (p < pieces) add_piece(mlf[p], lof[p], hif[p]);
    for (int p = kCombineFirst; p < pieces; ++p) {
      const float* po = a.part_o + (pslot(p) * ROWS + row) * D + d0;
      add_piece(a.part_ml[pslot(p) * ROWS + row], *reinterpret_cast<const f32x4*>(po),
                *reinterpret_cast<const f32x4*>(po + 4));
    }
    const float inv = 1.f / Ls;
    const int pos = rr / a.G, gi = rr % a.G;
    uint16_t* op = a.out + ((size_t)(s * a.B + pos) * a.Hq + g * a.G + gi) * D + d0;
    u32x4 packed;
    packed.x = pack_bf16x2(o[0] * inv, o[1] * inv);
    packed.y = pack_bf16x2(o[2] * inv, o[3] * inv);
    packed.z = pack_bf16x2(o[4] * inv, o[5] * inv);
    packed.w = pack_bf16x2(o[6] * inv, o[7] * inv);
    *reinterpret_cast<u32x4*>(op) = packed;
  }
}

AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int D, int page_size, int max_pages) {
  AttnPlan p{};
  p.D = D;
  const int G = Hq / Hkv;
  const int R = G * B;
  p.RT = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  p.n_rg = (R + 16 * p.RT - 1) / (16 * p.RT);
  const int slot_bytes = attn_slot_bytes(D, p.RT);
  // tiles the page tables can hold: an upper bound of the launch's stream
  const size_t tiles_cap = (size_t)S * Hkv * p.n_rg *
                           ((size_t)max_pages * page_size / kKT + (B + kKT - 1) / kKT);
  p.ring = (p.RT == 1 && tiles_cap >= (size_t)kDeepRingTiles) ? kRing + 1 : kRing;
  const int waves_per_cu = std::max(1, std::min(kMaxWavesPerCU, kLdsPerCU / (p.ring * slot_bytes)));
  p.grid = kCUs * waves_per_cu;
  // two partial slots per wave (the segments its range cuts at either end)
  const size_t slots = (size_t)2 * p.grid * 16 * p.RT;
  p.o_bytes = (slots * D * sizeof(float) + 255) & ~(size_t)255;
  p.ml_bytes = (slots * sizeof(float2) + 255) & ~(size_t)255;
  p.ws_bytes = p.o_bytes + p.ml_bytes + (size_t)S * Hkv * p.n_rg * sizeof(int32_t);
  return p;
}

template <int D, int RT>
static hipError_t launch_dr(const AttnPlan& p, const AttnArgs& a, hipStream_t st) {
  const bool deep = RT == 1 && p.ring != kRing;
  if constexpr (RT == 1) {
    if (deep) {
      if (a.save_state != nullptr)
        attn_stream_kernel<D, RT, kRing + 1, true><<<p.grid, 64, 0, st>>>(a);
      else
        attn_stream_kernel<D, RT, kRing + 1, false><<<p.grid, 64, 0, st>>>(a);
    }
  }
  if (!deep) {
    if (a.save_state != nullptr)
      attn_stream_kernel<D, RT, kRing, true><<<p.grid, 64, 0, st>>>(a);
    else
      attn_stream_kernel<D, RT, kRing, false><<<p.grid, 64, 0, st>>>(a);
  }
  attn_combine_kernel<D, RT><<<a.S * a.Hkv * p.n_rg, kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnPlan& p, const AttnArgs& a, hipStream_t st) {
  if (p.D == 128) {
    if (p.RT == 1) return launch_dr<128, 1>(p, a, st);
    if (p.RT == 2) return launch_dr<128, 2>(p, a, st);
    return launch_dr<128, 4>(p, a, st);
  }
  if (p.RT == 1) return launch_dr<64, 1>(p, a, st);
  if (p.RT == 2) return launch_dr<64, 2>(p, a, st);
  return launch_dr<64, 4>(p, a, st);
}

}  // namespace dbd
