// Block-diffusion attention over a paged KV cache, gfx950.
//
// The denoise step's attention (JetEngine developer notes, "ModelRunner" and
// "Layers"; README architecture tree, "Paged KV Cache"): each query of a
// sequence's block attends to all of that sequence's prefix tokens, found
// through its page table, and to every token of its own block, with no mask
// inside the block.  Grouped-query heads: the G = Hq/Hkv query heads of kv
// head g share its keys and values.
//
// Work decomposition (split-KV): one workgroup per (prefix chunk, kv head,
// row group, sequence).  The G*B query rows of a kv head form MFMA tiles of
// 16 rows (RT tiles per row group).  Chunk 0 also takes the block's own keys.
// The four waves of a workgroup stream disjoint 16-key tiles of the chunk
// without workgroup barriers:
//   * K tile: each lane loads 16 contiguous bytes of one key row straight
//     into the A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16);
//   * V tile: coalesced 16-byte loads into a wave-private LDS tile, read back
//     transposed as the A operand of O^T += V^T P^T (16x16x16 bf16 MFMA);
//   * the score tile's accumulator layout (lane = query row, 4 keys) is
//     exactly the B operand layout of the PV product, so probabilities go
//     from the softmax to the MFMA without a shuffle;
//   * online softmax in fp32 with base-2 exponentials (scores pre-scaled by
//     scale*log2(e)); probabilities are rounded to bf16 for the MFMA and the
//     row sum uses the rounded values.
// Loads of the wave's next tile are issued before the current tile's math.
// At the end the four waves merge (max, sum, acc) through LDS; a sequence
// with one chunk writes bf16 output directly, otherwise the chunk writes an
// fp32 partial and attn_combine_kernel merges the chunks.
#include <algorithm>

#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {

template <int D>
struct TileRegs {
  static constexpr int KS = D / 32;          // 16-byte K pieces per lane
  static constexpr int VN = (16 * D / 8) / 64; // 16-byte V pieces per lane
  bf16x8 k[KS];
  u32x4 v[VN];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const AttnArgs& a,
                                          int s, int g, int t, int n_ptiles,
                                          int kbeg, int kend, int lane,
                                          int& nvalid) {
  const uint16_t* kb;
  const uint16_t* vb;
  int stride;
  if (t < n_ptiles) {
    const int j0 = kbeg + 16 * t;
    const int page = a.page_table[(size_t)s * a.max_pages + j0 / a.P];
    const size_t base = ((size_t)(page * a.Hkv + g) * a.P + (j0 % a.P)) * D;
    kb = a.k_cache + base;
    vb = a.v_cache + base;
    stride = D;
    nvalid = min(16, kend - j0);
  } else {
    const int j0 = 16 * (t - n_ptiles);
    const size_t base = ((size_t)(s * a.B + j0) * a.Hkv + g) * D;
    kb = a.k_blk + base;
    vb = a.v_blk + base;
    stride = a.Hkv * D;
    nvalid = min(16, a.B - j0);
  }
  const int lr = lane & 15, lg = lane >> 4;
  const int kr = min(lr, nvalid - 1);  // clamp: never read past the tile
#pragma unroll
  for (int ks = 0; ks < TileRegs<D>::KS; ++ks)
    r.k[ks] = ld_bf16x8(kb + (size_t)kr * stride + 8 * lg + 32 * ks);
#pragma unroll
  for (int i = 0; i < TileRegs<D>::VN; ++i) {
    const int c = lane + 64 * i;
    const int key = c / (D / 8), dch = c % (D / 8);
    const int kc = min(key, nvalid - 1);
    u32x4 v = ld_u32x4(vb + (size_t)kc * stride + dch * 8);
    if (key >= nvalid) v = u32x4{0u, 0u, 0u, 0u};
    r.v[i] = v;
  }
}

}  // namespace

template <int D, int RT>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a) {
  constexpr int ROWS = 16 * RT;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int VSTR = D + 4;  // bf16 elements per V row in LDS (bank spread)
  constexpr int MSTR = D + 4;  // floats per row of the merge buffer

  __shared__ __align__(16) uint16_t s_v[4][16 * VSTR];
  __shared__ __align__(16) float s_o[4][16 * MSTR];
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];

  const int s = blockIdx.z;
  const int gy = blockIdx.y;
  const int g = gy / a.n_rg, rg = gy % a.n_rg;
  const int c = blockIdx.x;
  const int L = a.prefix_len[s];
  const int n_chunks = max(1, (L + a.chunk_keys - 1) / a.chunk_keys);
  if (c >= n_chunks) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int R = a.G * a.B;

  // Q^T as the B operand: lane holds query row lr, dims 8*lg + 32*ks.
  bf16x8 qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rg * ROWS + rt * 16 + lr;
    if (r < R) {
      const int pos = r / a.G, gi = r % a.G;
      const uint16_t* qp = a.q + ((size_t)(s * a.B + pos) * a.Hq + g * a.G + gi) * D + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = ld_bf16x8(qp + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = bf16x8{};
    }
  }

  float m_run[RT], l_run[RT];
  f32x4 acc[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kbeg = c * a.chunk_keys;
  const int kend = min(L, kbeg + a.chunk_keys);
  const int n_ptiles = kend > kbeg ? (kend - kbeg + 15) / 16 : 0;
  const int n_btiles = c == 0 ? (a.B + 15) / 16 : 0;
  const int n_tiles = n_ptiles + n_btiles;

  uint16_t* vt = s_v[wave];
  TileRegs<D> nxt;
  int nv_next = 0;
  if (wave < n_tiles) load_tile<D>(nxt, a, s, g, wave, n_ptiles, kbeg, kend, lane, nv_next);

  for (int t = wave; t < n_tiles; t += 4) {
    TileRegs<D> cur = nxt;
    const int nvalid = nv_next;
    if (t + 4 < n_tiles) load_tile<D>(nxt, a, s, g, t + 4, n_ptiles, kbeg, kend, lane, nv_next);

    // V tile -> wave-private LDS, row-major [key][d]
#pragma unroll
    for (int i = 0; i < TileRegs<D>::VN; ++i) {
      const int cidx = lane + 64 * i;
      const int key = cidx / (D / 8), dch = cidx % (D / 8);
      u32x2* dst = reinterpret_cast<u32x2*>(vt + key * VSTR + dch * 8);
      dst[0] = u32x2{cur.v[i].x, cur.v[i].y};
      dst[1] = u32x2{cur.v[i].z, cur.v[i].w};
    }

    // scores S^T[key][row] (lane: row lr, keys 4*lg+i)
    f32x4 sc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[ks], qf[rt][ks], sc[rt], 0, 0, 0);
    }

    i16x4 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (4 * lg + i < nvalid) ? sc[rt][i] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[i]);
      }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run[rt], tmax);
      const float alpha = fast_exp2(m_run[rt] - m_new);
      m_run[rt] = m_new;
      float psum = 0.f;
      short pbits[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t b = f2bf(fast_exp2(x[i] - m_new));
        pbits[i] = (short)b;
        psum += bf2f(b);
      }
      pb[rt] = i16x4{pbits[0], pbits[1], pbits[2], pbits[3]};
      l_run[rt] = l_run[rt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
    }

    wave_lds_sync();
    // O^T[d][row] += V^T[d][key] P^T[key][row]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vp = vt + (4 * lg) * VSTR + 16 * dt + lr;
      const i16x4 va = i16x4{(short)vp[0], (short)vp[VSTR], (short)vp[2 * VSTR], (short)vp[3 * VSTR]};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[rt], acc[rt][dt], 0, 0, 0);
    }
    wave_lds_sync();
  }

  // row sums: the four lanes of a row each hold part of it
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += shfl_xor_f(l_run[rt], 16);
    l_run[rt] += shfl_xor_f(l_run[rt], 32);
  }

  const size_t pbase = ((size_t)(s * (a.Hkv * a.n_rg) + gy) * a.n_chunk_max + c) * ROWS;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    __syncthreads();
    if (lg == 0) {
      s_m[wave][lr] = m_run[rt];
      s_l[wave][lr] = l_run[rt];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(&s_o[wave][lr * MSTR + 16 * dt + 4 * lg]) = acc[rt][dt];
    __syncthreads();
    for (int idx = tid; idx < 16 * (D / 8); idx += 256) {
      const int row = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
      const int r = rg * ROWS + rt * 16 + row;
      if (r >= R) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][row]);
      float wgt[4], Ls = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wgt[w] = fast_exp2(s_m[w][row] - M);
        Ls += s_l[w][row] * wgt[w];
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&s_o[w][row * MSTR + d0]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&s_o[w][row * MSTR + d0 + 4]);
        o[0] += wgt[w] * lo.x; o[1] += wgt[w] * lo.y; o[2] += wgt[w] * lo.z; o[3] += wgt[w] * lo.w;
        o[4] += wgt[w] * hi.x; o[5] += wgt[w] * hi.y; o[6] += wgt[w] * hi.z; o[7] += wgt[w] * hi.w;
      }
      if (n_chunks == 1) {
        const float inv = 1.f / Ls;
        const int pos = r / a.G, gi = r % a.G;
        uint16_t* op = a.out + ((size_t)(s * a.B + pos) * a.Hq + g * a.G + gi) * D + d0;
        u32x4 packed;
        packed.x = (uint32_t)f2bf(o[0] * inv) | ((uint32_t)f2bf(o[1] * inv) << 16);
        packed.y = (uint32_t)f2bf(o[2] * inv) | ((uint32_t)f2bf(o[3] * inv) << 16);
        packed.z = (uint32_t)f2bf(o[4] * inv) | ((uint32_t)f2bf(o[5] * inv) << 16);
        packed.w = (uint32_t)f2bf(o[6] * inv) | ((uint32_t)f2bf(o[7] * inv) << 16);
        *reinterpret_cast<u32x4*>(op) = packed;
      } else {
        float* po = a.part_o + (pbase + rt * 16 + row) * D + d0;
        *reinterpret_cast<f32x4*>(po) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(po + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if (d0 == 0) a.part_ml[pbase + rt * 16 + row] = make_float2(M, Ls);
      }
    }
  }
}

// Merge the chunk partials of one (sequence, kv head, row group).
template <int D, int RT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int ROWS = 16 * RT;
  const int s = blockIdx.y, gy = blockIdx.x;
  const int g = gy / a.n_rg, rg = gy % a.n_rg;
  const int L = a.prefix_len[s];
  const int n_chunks = max(1, (L + a.chunk_keys - 1) / a.chunk_keys);
  if (n_chunks == 1) return;
  const int R = a.G * a.B;
  const size_t base0 = (size_t)(s * (a.Hkv * a.n_rg) + gy) * a.n_chunk_max;
  for (int idx = threadIdx.x; idx < ROWS * (D / 8); idx += 256) {
    const int row = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
    const int r = rg * ROWS + row;
    if (r >= R) continue;
    float M = -INFINITY;
    for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, a.part_ml[(base0 + c) * ROWS + row].x);
    float Ls = 0.f, o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
      const float2 ml = a.part_ml[(base0 + c) * ROWS + row];
      const float w = fast_exp2(ml.x - M);
      Ls += ml.y * w;
      const float* po = a.part_o + ((base0 + c) * ROWS + row) * D + d0;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(po);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(po + 4);
      o[0] += w * lo.x; o[1] += w * lo.y; o[2] += w * lo.z; o[3] += w * lo.w;
      o[4] += w * hi.x; o[5] += w * hi.y; o[6] += w * hi.z; o[7] += w * hi.w;
    }
    const float inv = 1.f / Ls;
    const int pos = r / a.G, gi = r % a.G;
    uint16_t* op = a.out + ((size_t)(s * a.B + pos) * a.Hq + g * a.G + gi) * D + d0;
    u32x4 packed;
    packed.x = (uint32_t)f2bf(o[0] * inv) | ((uint32_t)f2bf(o[1] * inv) << 16);
    packed.y = (uint32_t)f2bf(o[2] * inv) | ((uint32_t)f2bf(o[3] * inv) << 16);
    packed.z = (uint32_t)f2bf(o[4] * inv) | ((uint32_t)f2bf(o[5] * inv) << 16);
    packed.w = (uint32_t)f2bf(o[6] * inv) | ((uint32_t)f2bf(o[7] * inv) << 16);
    *reinterpret_cast<u32x4*>(op) = packed;
  }
}

AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int D, int page_size,
                   int max_pages) {
  AttnPlan p{};
  p.D = D;
  const int G = Hq / Hkv;
  const int R = G * B;
  p.RT = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  p.n_rg = (R + 16 * p.RT - 1) / (16 * p.RT);
  p.chunk_keys = p.RT >= 4 ? 1024 : 512;
  const long max_prefix = (long)max_pages * page_size;
  p.n_chunk_max = (int)std::max<long>(1, (max_prefix + p.chunk_keys - 1) / p.chunk_keys);
  if (p.n_chunk_max > 1) {
    const size_t slots = (size_t)S * Hkv * p.n_rg * p.n_chunk_max * 16 * p.RT;
    const size_t o_bytes = (slots * D * sizeof(float) + 255) & ~(size_t)255;
    p.ws_bytes = o_bytes + slots * sizeof(float2);
  } else {
    p.ws_bytes = 0;
  }
  return p;
}

template <int D, int RT>
static hipError_t launch_dr(const AttnPlan& p, const AttnArgs& a, hipStream_t st) {
  dim3 grid(p.n_chunk_max, a.Hkv * p.n_rg, a.S);
  attn_chunk_kernel<D, RT><<<grid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_chunk_max == 1) return e;
  dim3 g2(a.Hkv * p.n_rg, a.S);
  attn_combine_kernel<D, RT><<<g2, 256, 0, st>>>(a);
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
