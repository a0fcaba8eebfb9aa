// Second halves of the split-K projections. The GEMM stored S partial tiles
// P[s][m][n] (fp32); these kernels sum them in split order, so every result is
// deterministic, and apply the projection's epilogue. Each output element's S
// loads are independent and issued in batches of 8.
#include "device.h"
#include "kernels.h"

namespace {

// sum_s P[s * stride + off], s = 0..S-1, in order, padded with +0 terms to a
// multiple of 8 (the padding is part of the fixed addition sequence). Up to 32
// splits, every load is issued before the first add: one L2 round trip.
template <int N>
DEV float sum_splits_n(const float* P, int S, size_t stride, size_t off) {
  float v[N];
#pragma unroll
  for (int u = 0; u < N; ++u) v[u] = u < S ? P[(size_t)u * stride + off] : 0.f;
  float t = 0.f;
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (u < ((S + 7) & ~7)) t += v[u];
  return t;
}
DEV float sum_splits(const float* P, int S, size_t stride, size_t off) {
  if (S <= 8) return sum_splits_n<8>(P, S, stride, off);
  if (S <= 16) return sum_splits_n<16>(P, S, stride, off);
  if (S <= 32) return sum_splits_n<32>(P, S, stride, off);
  float t = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s0 + u < S ? P[(size_t)(s0 + u) * stride + off] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  return t;
}

// h += Y for one row and one 128-column group; the group's sum of squares of
// the new h goes to ssq_out[group * ssq_ld + row] (the next RMSNorm's input).
__global__ __launch_bounds__(128) void finish_resid_kernel(const float* P, int S, int M, int N, float* h, int ldh,
                                                           float* ssq_out, int ssq_ld) {
  __shared__ float red[2];
  const int grp = blockIdx.x, m = blockIdx.y;
  const int n = grp * 128 + threadIdx.x;
  float v = 0.f;
  if (n < N) {
    const float y = sum_splits(P, S, (size_t)M * N, (size_t)m * N + n);
    float* hp = h + (size_t)m * ldh + n;
    v = *hp + y;
    *hp = v;
  }
  float ss = wave_sum(v * v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0 && ssq_out) ssq_out[(size_t)grp * ssq_ld + m] = red[0] + red[1];
}

__global__ __launch_bounds__(256) void finish_silu_kernel(const float* P, int S, int M, int N, uint16_t* act,
                                                          int ldo) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const size_t stride = (size_t)M * 2 * N;
  const float g = sum_splits(P, S, stride, (size_t)m * 2 * N + n);
  const float u = sum_splits(P, S, stride, (size_t)m * 2 * N + N + n);
  act[(size_t)m * ldo + n] = f2bfbits(g / (1.0f + expf(-g)) * u);
}

__global__ __launch_bounds__(256) void finish_store_kernel(const float* P, int S, int M, int N, void* out, int ldo,
                                                           int bf16) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const float y = sum_splits(P, S, (size_t)M * N, (size_t)m * N + n);
  if (bf16) ((uint16_t*)out)[(size_t)m * ldo + n] = f2bfbits(y);
  else ((float*)out)[(size_t)m * ldo + n] = y;
}

// One wave per (row, head) of the projection: q/k heads get RMSNorm over
// head_dim with their gain and rotate-half RoPE at the row's position; Q goes
// to the block buffer (bf16), K to the ring at slot position % C, V (no norm)
// to the transposed V ring. Lane d owns the rotation pair (d, d + hd/2).
__global__ __launch_bounds__(256) void finish_head_kernel(const GemmArgs a, const float* __restrict__ P0, int S, int ld,
                                                          int n_heads) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nl = a.nb > 0 ? a.nb : 1;
  if (item >= nl * a.M * n_heads) return;
  const int layer = item / (a.M * n_heads);
  const int m = item % (a.M * n_heads) / n_heads, hl = item % n_heads;
  uint16_t* ring_k = a.nb > 0 ? pick(a.rkb, layer) : a.ring_k;
  uint16_t* ring_v = a.nb > 0 ? pick(a.rvb, layer) : a.ring_v;
  const uint16_t* k_gain = a.nb > 0 ? pick(a.kgb, layer) : a.k_gain;
  const float* P = P0 + (size_t)layer * S * a.M * ld;
  const int head = a.head_base + hl;
  const int hd = a.hd, half = hd / 2;
  // the partial sums do not depend on the row's position: their loads go out
  // first, together with the position lookups
  const bool on = lane < half;
  const size_t stride = (size_t)a.M * ld, base = (size_t)m * ld + (size_t)hl * hd;
  const float s1 = sum_splits(P, S, stride, base + (on ? lane : 0));
  const float s2 = sum_splits(P, S, stride, base + (on ? lane + half : 0));
  const float x1 = on ? s1 : 0.f, x2 = on ? s2 : 0.f;
  int req;
  long long p, rp;
  const unsigned bad = ring_row(a, m, &req, &p, &rp);
  if (bad) {
    if (lane == 0) set_error(a.err, bad);
    return;
  }
  const bool is_q = head < a.nq, is_k = !is_q && head < a.nq + a.nkv;
  if (is_q || is_k) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float inv = 1.0f / sqrtf(ss / (float)hd + a.eps);
    if (!on) return;
    const uint16_t* g = is_q ? a.q_gain : k_gain;
    const float y1 = x1 * inv * bfbits2f(g[lane]);
    const float y2 = x2 * inv * bfbits2f(g[lane + half]);
    float c, s;
    rope_cos_sin(rp, lane, hd, a.log2_theta, &c, &s);
    uint16_t* o = is_q ? a.q_out + (size_t)m * a.nq * hd + (size_t)head * hd
                       : ring_k + (((size_t)req * a.nkv + (head - a.nq)) * a.C + p % a.C) * hd;
    o[lane] = f2bfbits(y1 * c - y2 * s);
    o[lane + half] = f2bfbits(y2 * c + y1 * s);
  } else {
    if (!on) return;
    uint16_t* o = ring_v + ((size_t)req * a.nkv + (head - a.nq - a.nkv)) * (size_t)hd * a.C + p % a.C;
    o[(size_t)lane * a.C] = f2bfbits(x1);
    o[(size_t)(lane + half) * a.C] = f2bfbits(x2);
  }
}

// Head finish of many staged rows from one fp32 product P[M][ld] holding the K
// and V heads of the rows (head_dim HD, 64 or 128): a workgroup takes 32 rows
// of one head. Every load goes out at once (each thread up to 4
// 16-byte pieces of the 32 x hd block, the first 32 threads one row's slot),
// the block lands in LDS, and then:
//   K heads  a wave per row, lane d < hd/2 owning the rotation pair (d, d + hd/2),
//            with finish_head_kernel's arithmetic; each row is contiguous;
//   V heads  each store instruction writes two dimensions of the 32 rows, which
//            sit at consecutive ring slots when their positions do (64
//            contiguous bytes of V^T each).
// Measured for 4096 rows x 16 heads of 128: 64-row blocks took the staging
// 0.607 ms, 32-row blocks 0.589-0.597, 16-row blocks 0.591 (the waves' chains
// of rows are shorter).
constexpr int KV_ROWS = 32;
constexpr int KV_NP = KV_ROWS * 32 / 256;   // 16-byte pieces of a 32 x 128 block per thread
template <int HD>
__global__ __launch_bounds__(256) void finish_kv_rows_kernel(const GemmArgs a, const float* __restrict__ P, int ld) {
  __shared__ float tile[KV_ROWS][129];
  __shared__ long long s_off[KV_ROWS];   // the row's K or V^T offset in its ring, or -1
  __shared__ long long s_rp[KV_ROWS];    // its RoPE position
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * KV_ROWS, hl = blockIdx.y;
  const int rows = min(KV_ROWS, a.M - m0);
  constexpr int hd = HD, half = HD / 2, pr = HD / 4;   // pr: pieces per row
  const int head = a.head_base + hl;
  const bool is_k = head < a.nq + a.nkv;
  f32x4 v[KV_NP];   // piece e = threadIdx.x + 256 u: row e / pr, columns 4 (e % pr) .. + 3
#pragma unroll
  for (int u = 0; u < KV_NP; ++u) {
    const int e = min((int)threadIdx.x + 256 * u, rows * pr - 1);
    v[u] = *(const f32x4*)(P + (size_t)(m0 + e / pr) * ld + (size_t)hl * hd + 4 * (e % pr));
  }
  if (threadIdx.x < KV_ROWS) {
    long long off = -1, rpos = 0;
    if ((int)threadIdx.x < rows) {
      int req;
      long long p, rp;
      const unsigned bad = ring_row(a, m0 + (int)threadIdx.x, &req, &p, &rp);
      if (bad) {
        set_error(a.err, bad);
      } else if (is_k) {
        off = (((long long)req * a.nkv + (head - a.nq)) * a.C + p % a.C) * hd;
        rpos = rp;
      } else {
        off = (((long long)req * a.nkv + (head - a.nq - a.nkv)) * hd) * a.C + p % a.C;
      }
    }
    s_off[threadIdx.x] = off;
    s_rp[threadIdx.x] = rpos;
  }
#pragma unroll
  for (int u = 0; u < KV_NP; ++u) {
    const int e = (int)threadIdx.x + 256 * u;
    if (e < rows * pr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[e / pr][4 * (e % pr) + i] = v[u][i];
    }
  }
  __syncthreads();
  if (is_k) {
    const bool on = lane < half;
    const float g1 = on ? bfbits2f(a.k_gain[lane]) : 0.f, g2 = on ? bfbits2f(a.k_gain[lane + half]) : 0.f;
    const double freq = rope_freq(on ? lane : 0, hd, a.log2_theta);   // once per lane, not per row
    for (int r = wave; r < rows; r += 4) {
      const long long off = s_off[r];
      if (off < 0) continue;
      const float x1 = on ? tile[r][lane] : 0.f, x2 = on ? tile[r][lane + half] : 0.f;
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float inv = 1.0f / sqrtf(ss / (float)hd + a.eps);
      if (!on) continue;
      const float y1 = x1 * inv * g1;
      const float y2 = x2 * inv * g2;
      float c, s;
      rope_cs(s_rp[r], freq, &c, &s);
      a.ring_k[off + lane] = f2bfbits(y1 * c - y2 * s);
      a.ring_k[off + lane + half] = f2bfbits(y2 * c + y1 * s);
    }
    return;
  }
  // V^T: thread t stores row t % KV_ROWS of dimensions t / KV_ROWS + 256 / KV_ROWS * j
  const int vr = threadIdx.x % KV_ROWS;
  const long long off = s_off[vr];
  if (off >= 0 && vr < rows)
    for (int d = threadIdx.x / KV_ROWS; d < hd; d += 256 / KV_ROWS)
      a.ring_v[off + (long long)d * a.C] = f2bfbits(tile[vr][d]);
}

}  // namespace

hipError_t launch_finish_kv_rows(const GemmArgs& a, const float* P, int ld, hipStream_t st) {
  if ((a.hd != 64 && a.hd != 128) || a.nb > 0 || a.M < 1 || a.head_base != a.nq || ld < 2 * a.nkv * a.hd || ld % 4)
    return hipErrorInvalidValue;
  const dim3 grid((a.M + KV_ROWS - 1) / KV_ROWS, 2 * a.nkv);
  if (a.hd == 128) hipLaunchKernelGGL(finish_kv_rows_kernel<128>, grid, dim3(256), 0, st, a, P, ld);
  else hipLaunchKernelGGL(finish_kv_rows_kernel<64>, grid, dim3(256), 0, st, a, P, ld);
  return hipGetLastError();
}

hipError_t launch_finish_resid(const float* P, int S, int M, int N, float* h, int ldh, float* ssq_out, int ssq_ld,
                               hipStream_t st) {
  hipLaunchKernelGGL(finish_resid_kernel, dim3((N + 127) / 128, M), dim3(128), 0, st, P, S, M, N, h, ldh, ssq_out,
                     ssq_ld);
  return hipGetLastError();
}

hipError_t launch_finish_silu(const float* P, int S, int M, int N, uint16_t* act, int ldo, hipStream_t st) {
  hipLaunchKernelGGL(finish_silu_kernel, dim3((N + 255) / 256, M), dim3(256), 0, st, P, S, M, N, act, ldo);
  return hipGetLastError();
}

hipError_t launch_finish_store(const float* P, int S, int M, int N, void* out, int ldo, int bf16, hipStream_t st) {
  hipLaunchKernelGGL(finish_store_kernel, dim3((N + 255) / 256, M), dim3(256), 0, st, P, S, M, N, out, ldo, bf16);
  return hipGetLastError();
}

hipError_t launch_finish_head(const GemmArgs& a, const float* P, int S, int ld, int n_heads, hipStream_t st) {
  if (a.hd > 128 || a.hd % 2) return hipErrorInvalidValue;
  if (a.nb > MAX_BATCH) return hipErrorInvalidValue;
  const int items = (a.nb > 0 ? a.nb : 1) * a.M * n_heads;
  hipLaunchKernelGGL(finish_head_kernel, dim3((items + 3) / 4), dim3(256), 0, st, a, P, S, ld, n_heads);
  return hipGetLastError();
}
