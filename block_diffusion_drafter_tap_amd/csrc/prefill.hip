// Prefill staging: many context rows at once (a request's whole window), where
// fc and the per-layer K/V projections are dense contractions (thousands of
// rows) rather than weight streams. bf16 or INT4 (g64) weights.
//
//   tap_gather_kernel  X[m][t*H + j] = bf16(mean over the hc streams of tap t)
//                      (the same arithmetic as the skinny GEMM's tap staging:
//                      hc_mean8_bf16)
//   gemm_tile_kernel   Y[M][N] = X[M][K] . W[N][K]^T, fp32 accumulate, fp32 or
//                      bf16 out. 128 x BN tiles per workgroup of 4 waves (2 x 2,
//                      64 x BN/2 per wave, MFMA 16x16x32 bf16); K in stages of 64
//                      double-buffered through LDS (rows padded by 8 elements so
//                      the 16 rows of a fragment read fall in different banks),
//                      each stage's global loads issued two stages ahead. Tiles
//                      are numbered in groups of 8 row blocks, column-major
//                      inside a group, and dealt out XCD-major (workgroup i runs
//                      on XCD i % 8): the tiles resident on one XCD form an
//                      8 x 8 block that shares X rows and W columns in its L2.
#include <string.h>

#include "device.h"
#include "kernels.h"

namespace {

constexpr int PF_BM = 128, PF_BK = 64, PF_LDK = PF_BK + 8, PF_GM = 8;

__global__ __launch_bounds__(256) void tap_gather_kernel(const TapGather g) {
  const int m = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 8;   // first of 8 columns of the gathered row
  if (e >= g.n_taps * g.tap_hidden) return;
  const int t = e / g.tap_hidden, col = e - t * g.tap_hidden;
  const float* tp = g.taps[0];
#pragma unroll
  for (int i = 1; i < MAX_TAPS; ++i)
    if (t == i) tp = g.taps[i];
  const int src = g.src_row ? g.src_row[m] : m;
  *(u32x4*)(g.out + (size_t)m * g.n_taps * g.tap_hidden + e) =
      hc_mean8_bf16(tp + (size_t)src * g.tap_stride + col, (size_t)g.tap_hidden, g.hc);
}

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_HEADS = 2 };

// OUT_HEADS: the tile's columns are whole context K heads (k RMSNorm over the
// head, RoPE at the row's position, rows into the K ring) or V heads (into the
// transposed V ring, 64 consecutive rows of one dimension per wave store).
// INT4 weights (Q4): a K stage of 64 is one quantization group. Its packed words
// are unpacked into the LDS W tile as bf16 (128 + u) pairs (one and-or per pair;
// bf16's ulp at 128 is 1), the group scale of every W row goes to LDS, and the X
// staging also leaves each row's sum of the stage's bf16 values. The stage's
// MFMAs accumulate t = sum x * (u + 128) from zero and the stage adds
// s * (t - 136 * sum x) = s * sum x * q.
// BM rows x BN columns per workgroup of BM / 32 waves (a 2-column grid of 64-row
// x BN/2-column wave tiles). 128-row tiles run two workgroups per CU; a 256-row
// tile (bf16 only) takes a CU alone and loads a quarter fewer operand bytes per
// flop, which is what bounds these tiles (operand reads from L2 at the CU's
// load rate). Every output's MFMA chain over the K stages is the same for both.
template <int BM, int BN, int OUT, int Q4>
__global__ __launch_bounds__(BM * 2, Q4 || BM > 128 ? 1 : 2)   // INT4 holds per-group accumulators too
void gemm_tile_kernel(const TileArgs a, const GemmArgs h) {
  constexpr int NTH = BM * 2, NWV = NTH / 64, RB = BM / 64;
  static_assert(!Q4 || BM == 128, "INT4 tiles are 128 rows");
  constexpr int WN = BN / 2;        // columns per wave
  constexpr int NJ = WN / 16;       // 16-column MFMA tiles per wave
  constexpr int XP = BM * PF_BK / 8 / NTH;   // 16-byte X pieces per thread per stage
  constexpr int WP = Q4 ? 1 : BN * PF_BK / 8 / NTH;   // W pieces (bf16)
  constexpr int TPR = 256 / BN;     // INT4: threads per W row, each with 4 / TPR of its word pairs
  constexpr int JPT = 4 / TPR;
  constexpr int XS_BYTES = 2 * BM * PF_LDK * 2, WS_BYTES = 2 * BN * PF_LDK * 2;
  constexpr int TILE_BYTES = OUT == OUT_HEADS ? BM * (BN + 1) * 4 : 0;
  constexpr int SMEM = XS_BYTES + WS_BYTES > TILE_BYTES ? XS_BYTES + WS_BYTES : TILE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  auto xs = (uint16_t(*)[BM][PF_LDK])smem;
  auto ws = (uint16_t(*)[BN][PF_LDK])(smem + XS_BYTES);
  __shared__ float s_xsum[Q4 ? 2 : 1][Q4 ? PF_BM : 1], s_sc[Q4 ? 2 : 1][Q4 ? BN : 1];

  const int mt = (a.M + BM - 1) / BM, nt = a.N / BN, tiles = mt * nt;
  const int per_xcd = (tiles + 7) / 8;
  const int seq = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (seq >= tiles) return;
  // the tile sequence runs through groups of PF_GM row blocks, column-major inside
  // a group: the 64 tiles resident on one XCD span 8 row blocks x 8 column blocks,
  // so each X row block and each W column block is re-read from that XCD's L2
  const int grp = seq / (PF_GM * nt), first = grp * PF_GM;
  const int gm = min(PF_GM, mt - first);
  const int r = seq - grp * PF_GM * nt;
  const int m0 = (first + r % gm) * BM, n0 = (r / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nst = a.K / PF_BK;

  // two register sets: stage s + 2 is loaded while stage s computes and is
  // stored to LDS after stage s + 1 computes (two stages of latency cover)
  u32x4 xr[2][XP], wr[2][WP];
  u32x2 qr[2][JPT];   // INT4: the stage's two words of each word pair j of this thread's row
  uint32_t sr[2];     // INT4: the row's fp16 group scale
  const int wrow = tid / TPR, jt = (tid % TPR) * JPT;
  auto load = [&](int s, int q) {
    const int k0 = s * PF_BK;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * NTH, row = p / 8, seg = p % 8;
      xr[q][i] = ld16(a.x + (size_t)min(m0 + row, a.M - 1) * a.ldx + k0 + 8 * seg);
    }
    if constexpr (Q4) {
      // 128-wide chunk s/2, half s%2: words 4j + 2(s%2) and 4j + 2(s%2) + 1 hold
      // the stage's k-values 32i + 8j + e (i = 0, 1)
      const uint8_t* rp = (const uint8_t*)a.w + (size_t)(n0 + wrow) * (a.K / 2) + (s / 2) * 64 + (s % 2) * 8;
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) qr[q][jj] = *(const u32x2*)(rp + 16 * (jt + jj));
      sr[q] = a.wscale[(size_t)(n0 + wrow) * (a.K / 64) + s];
    } else {
#pragma unroll
      for (int i = 0; i < WP; ++i) {
        const int p = tid + i * NTH, row = p / 8, seg = p % 8;
        wr[q][i] = ld16((const uint16_t*)a.w + (size_t)(n0 + row) * a.K + k0 + 8 * seg);
      }
    }
  };
  auto store = [&](int b, int q) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * NTH;
      *(u32x4*)&xs[b][p / 8][8 * (p % 8)] = xr[q][i];
      if constexpr (Q4) {
        // the row's 8 pieces sit on 8 consecutive lanes
        float t = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) t += __uint_as_float(xr[q][i][u] << 16) + __uint_as_float(xr[q][i][u] & 0xffff0000u);
        t += __shfl_xor(t, 1, 64);
        t += __shfl_xor(t, 2, 64);
        t += __shfl_xor(t, 4, 64);
        if (p % 8 == 0) s_xsum[b][p / 8] = t;
      }
    }
    if constexpr (Q4) {
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t w = qr[q][jj][i];
          u32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = ((w >> (4 * t)) & 0x000F000Fu) | 0x43004300u;
          *(u32x4*)&ws[b][wrow][32 * i + 8 * (jt + jj)] = v;
        }
      if (tid % TPR == 0) s_sc[b][wrow] = (float)__builtin_bit_cast(_Float16, (uint16_t)sr[q]);
    } else {
#pragma unroll
      for (int i = 0; i < WP; ++i) {
        const int p = tid + i * NTH;
        *(u32x4*)&ws[b][p / 8][8 * (p % 8)] = wr[q][i];
      }
    }
  };

  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int b) {
    f32x4 t[Q4 ? 4 : 1][Q4 ? NJ : 1];
    if constexpr (Q4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) t[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < PF_BK; kk += 32) {
      u32x4 af[4], bf[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const u32x4*)&xs[b][wm * 64 + 16 * i + lr][kk + 8 * lg];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *(const u32x4*)&ws[b][wn * WN + 16 * j + lr][kk + 8 * lg];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (Q4) t[i][j] = mfma16x16x32(as_bf16x8(af[i]), as_bf16x8(bf[j]), t[i][j]);
          else acc[i][j] = mfma16x16x32(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
        }
    }
    if constexpr (Q4) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float sc = s_sc[b][wn * WN + 16 * j + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 xg = *(const f32x4*)&s_xsum[b][wm * 64 + 16 * i + 4 * lg];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, fmaf(-136.0f, xg[r], t[i][j][r]), acc[i][j][r]);
        }
      }
    }
  };
  // stage s lives in LDS buffer s & 1 and register set s & 1; the stage count
  // is even (K a multiple of 128). No load sits behind a branch (the last two
  // steps re-read the last stage), so each store waits only for its own set.
  load(0, 0);
  load(1, 1);
  store(0, 0);
  __syncthreads();
  for (int s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      load(min(s0 + q + 2, nst - 1), q);
      compute(q);
      store(q ^ 1, q ^ 1);
      __syncthreads();
    }
  }

  // lane holds C[4*lg + r][lr] of each 16 x 16 tile
  if constexpr (OUT != OUT_HEADS) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + 16 * i + 4 * lg + r;
        if (m >= a.M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = n0 + wn * WN + 16 * j + lr;
          if (OUT == OUT_BF16) ((uint16_t*)a.out)[(size_t)m * a.ldo + n] = f2bfbits(acc[i][j][r]);
          else ((float*)a.out)[(size_t)m * a.ldo + n] = acc[i][j][r];
        }
      }
  } else {
    // the stage buffers are free after the loop's last barrier
    __shared__ int s_req[BM], s_pos[BM];
    auto tile = (float(*)[BN + 1])smem;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) tile[wm * 64 + 16 * i + 4 * lg + r][wn * WN + 16 * j + lr] = acc[i][j][r];
    const int rows = min(BM, a.M - m0);
    for (int r = tid; r < rows; r += NTH) {
      int req;
      long long p, rp;
      const unsigned bad = ring_row(h, m0 + r, &req, &p, &rp);
      if (bad) set_error(h.err, bad);
      s_req[r] = req;
      s_pos[r] = p < 0 ? -1 : (int)p;
    }
    __syncthreads();
    const int hd = h.hd, half = hd / 2, nh = BN / hd;
    if (n0 < h.nkv * hd) {
      // K heads: one wave per (row, head), lane d < hd/2 owns the pair (d, d + hd/2)
      const bool on = lane < half;
      const float g1 = on ? bfbits2f(h.k_gain[lane]) : 0.f, g2 = on ? bfbits2f(h.k_gain[lane + half]) : 0.f;
      const double freq = rope_freq(on ? lane : 0, hd, h.log2_theta);
      for (int it = wave; it < rows * nh; it += NWV) {
        const int r = it / nh, hh = it % nh;
        const int p = s_pos[r];
        if (p < 0) continue;
        const float x1 = on ? tile[r][hh * hd + lane] : 0.f;
        const float x2 = on ? tile[r][hh * hd + lane + half] : 0.f;
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float inv = 1.0f / sqrtf(ss / (float)hd + h.eps);
        if (!on) continue;
        const float y1 = x1 * inv * g1, y2 = x2 * inv * g2;
        float c, sn;
        rope_cs(p, freq, &c, &sn);
        uint16_t* o = h.ring_k + (((size_t)s_req[r] * h.nkv + n0 / hd + hh) * h.C + p % h.C) * hd;
        o[lane] = f2bfbits(y1 * c - y2 * sn);
        o[lane + half] = f2bfbits(y2 * c + y1 * sn);
      }
    } else {
      // V heads: one wave per (dimension, 64-row block); lane = row
      for (int it = wave; it < nh * hd * RB; it += NWV) {
        const int hh = it / (RB * hd), d = (it / RB) % hd, r = (it % RB) * 64 + lane;
        if (r >= rows) continue;
        const int p = s_pos[r];
        if (p < 0) continue;
        const int gv = (n0 - h.nkv * hd) / hd + hh;
        h.ring_v[(((size_t)s_req[r] * h.nkv + gv) * hd + d) * h.C + p % h.C] = f2bfbits(tile[r][hh * hd + d]);
      }
    }
  }
}

template <int BN, int Q4>
hipError_t launch_tile_q(const TileArgs& a, const GemmArgs& h, int out, hipStream_t st) {
  const int tiles = ((a.M + PF_BM - 1) / PF_BM) * (a.N / BN);
  const dim3 grid(8 * ((tiles + 7) / 8));
  if (out == OUT_BF16) hipLaunchKernelGGL((gemm_tile_kernel<PF_BM, BN, OUT_BF16, Q4>), grid, dim3(256), 0, st, a, h);
  else if (out == OUT_F32) hipLaunchKernelGGL((gemm_tile_kernel<PF_BM, BN, OUT_F32, Q4>), grid, dim3(256), 0, st, a, h);
  else hipLaunchKernelGGL((gemm_tile_kernel<PF_BM, BN, OUT_HEADS, Q4>), grid, dim3(256), 0, st, a, h);
  return hipGetLastError();
}

template <int BN>
hipError_t launch_tile(const TileArgs& a, const GemmArgs& h, int out, hipStream_t st) {
  if (a.wscale) return launch_tile_q<BN, 1>(a, h, out, st);
  return launch_tile_q<BN, 0>(a, h, out, st);
}

}  // namespace

hipError_t launch_tap_gather(const TapGather& g, int M, hipStream_t st) {
  const int width = g.n_taps * g.tap_hidden;
  if (M < 1 || width % 8 || g.tap_hidden % 8 || g.hc < 1 || g.n_taps > MAX_TAPS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tap_gather_kernel, dim3((width / 8 + 255) / 256, M), dim3(256), 0, st, g);
  return hipGetLastError();
}

int tile_bn(int M, int N, int n_cu) {
  // the column tile with the shorter estimated time over rounds of workgroups
  // (2 per CU); 128 when equal. A 128-wide tile takes about 1.2x the time of a
  // 64-wide one (measured at fc 4096 x 2560 x 12800: 0.93 -> 0.84 ms for the
  // prefill stage with 128), since both are bound by operand reads from L2.
  const int mt = (M + PF_BM - 1) / PF_BM, slots = 2 * n_cu;
  if (N % 128) return N % 64 ? 0 : 64;
  const long long t128 = (long long)mt * (N / 128), t64 = (long long)mt * (N / 64);
  const double c128 = (double)((t128 + slots - 1) / slots) * 1.25;
  const double c64 = (double)((t64 + slots - 1) / slots);
  return c64 < c128 ? 64 : 128;
}

hipError_t launch_gemm_tile(const TileArgs& a, int bn, int out_bf16, hipStream_t st) {
  if (a.M < 1 || a.K % (2 * PF_BK) || (bn != 64 && bn != 128) || a.N % bn) return hipErrorInvalidValue;
  GemmArgs none;
  memset(&none, 0, sizeof none);
  const int out = out_bf16 ? OUT_BF16 : OUT_F32;
  return bn == 128 ? launch_tile<128>(a, none, out, st) : launch_tile<64>(a, none, out, st);
}

hipError_t launch_gemm_tile_heads(const TileArgs& a, const GemmArgs& h, int n_cu, hipStream_t st) {
  // whole heads per tile: 128 columns (1 head of 128 or 2 of 64)
  if (a.M < 1 || a.K % (2 * PF_BK) || h.hd < 2 || h.hd > 128 || h.hd % 2 || 128 % h.hd || a.N != 2 * h.nkv * h.hd ||
      (h.nkv * h.hd) % 128)
    return hipErrorInvalidValue;
  // bf16 weights with at least one 256-row tile per CU: the larger tile
  if (!a.wscale && n_cu > 0 && (long long)(a.M / 256) * (a.N / 128) >= n_cu) {
    const int tiles = ((a.M + 255) / 256) * (a.N / 128);
    hipLaunchKernelGGL((gemm_tile_kernel<256, 128, OUT_HEADS, 0>), dim3(8 * ((tiles + 7) / 8)), dim3(512), 0, st, a, h);
    return hipGetLastError();
  }
  return launch_tile<128>(a, h, OUT_HEADS, st);
}
