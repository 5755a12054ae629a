// Selective LM head fused with the softmax, gfx950.
//
// The LM head runs only for still-masked positions of DENOISING sequences
// (JetEngine README, "Selective Logits"; developer notes, "Optimization
// History": sparse logits on masked positions only), and greedy decoding
// needs only each row's best token and its probability (SDAR page:
// generate.py runs greedy generation).  The full logits row is never
// stored: it lives in MFMA accumulators for one 256x256 tile and is reduced
// there.
//
// lmhead_tile_kernel: C^T[v][m] = W[v][:] . h[m][:] over a 256 (vocab) x 256
// (row) tile with v_mfma_f32_32x32x16_bf16; four waves each own 128x128.
// W and the gathered hidden rows stream through a double-buffered LDS stage
// of depth 64 (16-byte chunks XOR-swizzled by row so the fragment reads are
// bank-conflict free).  Workgroup ids are mapped so that the row tiles of one
// vocabulary tile land on the same XCD back to back: the second reads W from
// that XCD's L2.  Epilogue per row and per 128-column vocabulary tile: the
// largest logit (mask id and columns past V excluded), the lowest id that
// reaches it, and sum(exp(l - max)) in fp32.
//
// lmhead_merge_kernel: one wave per row folds the row's tile partials,
// (m,a,s) + (m',a',s') = (max, id of the larger max or the lower id on equal
// maxima, s*e^(m-max) + s'*e^(m'-max)), in a fixed order, and writes the
// greedy token and the confidence 1/s = exp(max - logsumexp).
#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

namespace {
constexpr int TN = 256;  // vocabulary columns per workgroup tile
constexpr int TM = 256;  // hidden rows per workgroup tile
constexpr int TK = 64;   // depth of one LDS stage
constexpr int NXCD = 8;

__device__ __forceinline__ int swz(int row, int kc) {
  return row * TK + ((kc ^ (row & 7)) << 3);
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
}  // namespace

__global__ __launch_bounds__(256) void lmhead_tile_kernel(LmArgs a, int n_tiles_v, int n_tiles_m) {
  __shared__ __align__(16) uint16_t sW[2][TN * TK];
  __shared__ __align__(16) uint16_t sH[2][TM * TK];

  const int id = blockIdx.x;
  const int xcd = id % NXCD, slot = id / NXCD;
  const int mt = slot % n_tiles_m;
  const int vt = (slot / n_tiles_m) * NXCD + xcd;
  if (vt >= n_tiles_v) return;
  const int M = *a.num_rows;
  const int m0 = mt * TM;
  if (m0 >= M) return;
  const int n0 = vt * TN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wm = wave >> 1;

  // global -> LDS assignment: chunk c = tid + 256*i is (row c/8, k-chunk c%8)
  int woff[8], hoff[8], loff[8];
  bool wok[8], hok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, kc = c & 7;
    const int v = n0 + row;
    wok[i] = v < a.V;
    woff[i] = (wok[i] ? v : 0) * a.Hd + kc * 8;
    const int mr = m0 + row;
    hok[i] = mr < M;
    const int hr = hok[i] ? (a.row_index ? a.row_index[mr] : mr) : 0;
    hoff[i] = hr * a.Hd + kc * 8;
    loff[i] = swz(row, kc);
  }

  u32x4 rw[8], rh[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rw[i] = wok[i] ? ld_u32x4(a.w + woff[i] + k0) : u32x4{0u, 0u, 0u, 0u};
      rh[i] = hok[i] ? ld_u32x4(a.hidden + hoff[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(&sW[buf][loff[i]]) = rw[i];
      *reinterpret_cast<u32x4*>(&sH[buf][loff[i]]) = rh[i];
    }
  };

  int mb_valid = (M - (m0 + wm * 128) + 31) / 32;
  mb_valid = mb_valid < 0 ? 0 : (mb_valid > 4 ? 4 : mb_valid);

  f32x16 acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};

  const int nk = a.Hd / TK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * TK);
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = wn * 128 + nb * 32 + (lane & 31);
        af[nb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sW[buf][swz(row, kc)]));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = wm * 128 + mb * 32 + (lane & 31);
        bfr[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sH[buf][swz(row, kc)]));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < mb_valid) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bfr[mb], acc[nb][mb], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) = a
  // hidden row, and vocab rows 8*(i/4) + 4*(lane/32) + (i%4), i = 0..15.
  const int vbase = n0 + wn * 128;
  if (vbase >= a.V) return;
  const int nt = vbase / 128;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb >= mb_valid) break;
    const int mrow = m0 + wm * 128 + mb * 32 + (lane & 31);
    float best = -INFINITY;
    int bidx = 0x7fffffff;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = vbase + nb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float x = acc[nb][mb][i];
        if (v < a.V && v != a.mask_id && x > best) {
          best = x;
          bidx = v;
        }
      }
    const float pbst = shfl_xor_f(best, 32);
    const int pidx = shfl_xor_i(bidx, 32);
    if (pbst > best || (pbst == best && pidx < bidx)) {
      best = pbst;
      bidx = pidx;
    }
    float sum = 0.f;
    if (best != -INFINITY) {
      const float mb2 = best * kLog2e;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = vbase + nb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (v < a.V && v != a.mask_id) sum += fast_exp2(fmaf(acc[nb][mb][i], kLog2e, -mb2));
        }
    }
    sum += shfl_xor_f(sum, 32);
    if (lane < 32 && mrow < M) {
      const size_t o = (size_t)mrow * a.n_vt + nt;
      a.pm[o] = best;
      a.pa[o] = bidx;
      a.ps[o] = sum;
    }
  }
}

__global__ __launch_bounds__(256) void lmhead_merge_kernel(LmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const int M = *a.num_rows;
  if (r >= M) return;
  Part x{-INFINITY, 0x7fffffff, 0.f};
  const size_t base = (size_t)r * a.n_vt;
  for (int t = lane; t < a.n_vt; t += 64) fold(x, a.pm[base + t], a.pa[base + t], a.ps[base + t]);
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
  const size_t n_vt = (size_t)(V + 127) / 128;
  const size_t one = ((size_t)max_rows * n_vt * 4 + 255) & ~(size_t)255;
  return 3 * one;
}

hipError_t lmhead_launch(const LmArgs& a, hipStream_t st) {
  const int n_tiles_v = (a.V + TN - 1) / TN;
  const int n_tiles_m = (a.max_rows + TM - 1) / TM;
  const int n_groups = (n_tiles_v + NXCD - 1) / NXCD;
  const int grid = n_groups * n_tiles_m * NXCD;
  lmhead_tile_kernel<<<grid, 256, 0, st>>>(a, n_tiles_v, n_tiles_m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lmhead_merge_kernel<<<(a.max_rows + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
