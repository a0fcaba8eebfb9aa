// Prefill staging: many context rows at once (a request's whole window), where
// fc and the per-layer K/V projections are dense contractions (thousands of
// rows) rather than weight streams. bf16 weights only; INT4 weights stage
// through the split-K path.
//
//   tap_gather_kernel  X[m][t*H + j] = bf16(mean over the hc streams of tap t)
//                      (the same arithmetic as the skinny GEMM's tap staging)
//   gemm_tile_kernel   Y[M][N] = X[M][K] . W[N][K]^T, fp32 accumulate, fp32 or
//                      bf16 out. 128 x BN tiles per workgroup of 4 waves (2 x 2,
//                      64 x BN/2 per wave, MFMA 16x16x32 bf16); K in stages of 64
//                      double-buffered through LDS (rows padded by 8 elements so
//                      the 16 rows of a fragment read fall in different banks),
//                      each stage's global loads issued one stage ahead. Tiles
//                      are numbered row-major and dealt out XCD-major (workgroup
//                      i runs on XCD i % 8), so the tiles resident on one XCD
//                      share X rows in its L2.
#include "device.h"
#include "kernels.h"

namespace {

constexpr int PF_BM = 128, PF_BK = 64, PF_LDK = PF_BK + 8;

__global__ __launch_bounds__(256) void tap_gather_kernel(const TapGather g) {
  const int m = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 8;   // first of 8 columns of the gathered row
  if (e >= g.n_taps * g.tap_hidden) return;
  const int t = e / g.tap_hidden, col = e - t * g.tap_hidden;
  const float* tp = g.taps[0];
#pragma unroll
  for (int i = 1; i < MAX_TAPS; ++i)
    if (t == i) tp = g.taps[i];
  const float* p = tp + (size_t)m * g.tap_stride + col;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < g.hc; ++st) {
    s0 += *(const f32x4*)(p + (size_t)st * g.tap_hidden);
    s1 += *(const f32x4*)(p + (size_t)st * g.tap_hidden + 4);
  }
  const float hinv = 1.0f / (float)g.hc;
  s0 *= hinv;
  s1 *= hinv;
  u32x4 r;
  r[0] = pack_bf16x2(s0[0], s0[1]);
  r[1] = pack_bf16x2(s0[2], s0[3]);
  r[2] = pack_bf16x2(s1[0], s1[1]);
  r[3] = pack_bf16x2(s1[2], s1[3]);
  *(u32x4*)(g.out + (size_t)m * g.n_taps * g.tap_hidden + e) = r;
}

template <int BN, int OUT_BF16>
__global__ __launch_bounds__(256, 2) void gemm_tile_kernel(const TileArgs a) {
  constexpr int WN = BN / 2;        // columns per wave
  constexpr int NJ = WN / 16;       // 16-column MFMA tiles per wave
  constexpr int XP = PF_BM * PF_BK / 8 / 256;   // 16-byte X pieces per thread per stage
  constexpr int WP = BN * PF_BK / 8 / 256;      // W pieces
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][PF_BM][PF_LDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN][PF_LDK];

  const int mt = (a.M + PF_BM - 1) / PF_BM, nt = a.N / BN, tiles = mt * nt;
  const int per_xcd = (tiles + 7) / 8;
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= tiles) return;
  const int m0 = (tile / nt) * PF_BM, n0 = (tile % nt) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nst = a.K / PF_BK;

  u32x4 xr[XP], wr[WP];
  auto load = [&](int s) {
    const int k0 = s * PF_BK;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * 256, row = p / 8, seg = p % 8;
      xr[i] = ld16(a.x + (size_t)min(m0 + row, a.M - 1) * a.ldx + k0 + 8 * seg);
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int p = tid + i * 256, row = p / 8, seg = p % 8;
      wr[i] = ld16(a.w + (size_t)(n0 + row) * a.K + k0 + 8 * seg);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * 256;
      *(u32x4*)&xs[b][p / 8][8 * (p % 8)] = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int p = tid + i * 256;
      *(u32x4*)&ws[b][p / 8][8 * (p % 8)] = wr[i];
    }
  };

  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  if (nst > 1) load(1);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int b = s & 1;
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
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
    }
    if (s + 1 < nst) store(b ^ 1);
    if (s + 2 < nst) load(s + 2);
    __syncthreads();
  }

  // lane holds C[4*lg + r][lr] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + 16 * i + 4 * lg + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WN + 16 * j + lr;
        if (OUT_BF16) ((uint16_t*)a.out)[(size_t)m * a.ldo + n] = f2bfbits(acc[i][j][r]);
        else ((float*)a.out)[(size_t)m * a.ldo + n] = acc[i][j][r];
      }
    }
}

template <int BN>
hipError_t launch_tile(const TileArgs& a, int out_bf16, hipStream_t st) {
  const int tiles = ((a.M + PF_BM - 1) / PF_BM) * (a.N / BN);
  const dim3 grid(8 * ((tiles + 7) / 8));
  if (out_bf16) hipLaunchKernelGGL((gemm_tile_kernel<BN, 1>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((gemm_tile_kernel<BN, 0>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tap_gather(const TapGather& g, int M, hipStream_t st) {
  const int width = g.n_taps * g.tap_hidden;
  if (M < 1 || width % 8 || g.tap_hidden % 8 || g.hc < 1 || g.n_taps > MAX_TAPS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tap_gather_kernel, dim3((width / 8 + 255) / 256, M), dim3(256), 0, st, g);
  return hipGetLastError();
}

int tile_bn(int M, int N, int n_cu) {
  // the column tile that leaves the fewest idle slots in the last round of
  // workgroups (2 per CU); 128 when equal
  const int mt = (M + PF_BM - 1) / PF_BM, slots = 2 * n_cu;
  if (N % 128) return N % 64 ? 0 : 64;
  const long long t128 = (long long)mt * (N / 128), t64 = (long long)mt * (N / 64);
  const double c128 = (double)((t128 + slots - 1) / slots) * 2.0;   // a 128-wide tile costs two 64-wide ones
  const double c64 = (double)((t64 + slots - 1) / slots);
  return c64 < c128 ? 64 : 128;
}

hipError_t launch_gemm_tile(const TileArgs& a, int bn, int out_bf16, hipStream_t st) {
  if (a.M < 1 || a.K % PF_BK || (bn != 64 && bn != 128) || a.N % bn) return hipErrorInvalidValue;
  return bn == 128 ? launch_tile<128>(a, out_bf16, st) : launch_tile<64>(a, out_bf16, st);
}
