// Shared LM head with fused top-k for gfx950.
//
// logits = W_lm z for every block row, z = RMSNorm(h; final gain) as bf16,
// followed by per-row top-k over the vocabulary. Persistent: workgroup w
// handles column groups w, w + P, ... of 128 vocabulary rows; the normed X is
// staged in LDS once (or read from L2 when it does not fit). Each row belongs
// to one wave, which keeps the row's running top-k in registers (lanes 0..k-1,
// best first):
//   k = 1   a wave reduction per group;
//   k = 16  the first group is sorted by a bitonic network on registers and
//           shuffles (two values per lane), later groups only insert the values
//           that beat the current k-th entry (ballot, then a shifted insert).
// Weight loads run four 128-wide chunks ahead, across group boundaries, so the
// next group's first chunks are in flight during the selection.
// Output: per workgroup and mask row, its k best (value, id), best first.

#include "device.h"
#include "kernels.h"

namespace {

constexpr size_t LM_XL_MAX_BYTES = 96 * 1024;   // stage the normed rows in LDS up to this size

// 8 consecutive values (k..k+7) of row `row` of the final RMSNorm as bf16x8:
// z = h * inv * g, h the fp32 residual stream, inv the row's 1/rms.
DEV u32x4 norm_x8(const GemmArgs& a, int row, int k, float inv) {
  const float* p = a.xf + (size_t)row * a.ldx + k;
  const f32x4 h0 = *(const f32x4*)p, h1 = *(const f32x4*)(p + 4);
  const u32x4 g = ld16(a.xgain + k);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x4 h = i ? h1 : h0;
    r[2 * i] = pack_bf16x2(h[0] * inv * __uint_as_float(g[2 * i] << 16),
                           h[1] * inv * __uint_as_float(g[2 * i] & 0xffff0000u));
    r[2 * i + 1] = pack_bf16x2(h[2] * inv * __uint_as_float(g[2 * i + 1] << 16),
                               h[3] * inv * __uint_as_float(g[2 * i + 1] & 0xffff0000u));
  }
  return r;
}

// Sort 128 (value, id) pairs held as lane + 64*u, u = 0, 1, best first.
DEV void wave_sort128(float (&v)[2], int (&id)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 128; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = lane + 64 * u;
        float ov;
        int oi;
        if (j == 64) {
          ov = v[u ^ 1];
          oi = id[u ^ 1];
        } else {
          ov = __shfl_xor(v[u], j, 64);
          oi = __shfl_xor(id[u], j, 64);
        }
        const bool lo = (i & j) == 0, first = (i & k) == 0;
        const bool take_other = (lo == first) ? better(ov, oi, v[u], id[u]) : better(v[u], id[u], ov, oi);
        if (j == 64) {
          // both halves of the pair live in this lane: resolve once (u == 0)
          if (u == 0 && take_other) {
            const float tv = v[0]; const int ti = id[0];
            v[0] = v[1]; id[0] = id[1];
            v[1] = tv; id[1] = ti;
          }
        } else if (take_other) {
          v[u] = ov;
          id[u] = oi;
        }
      }
    }
  }
}

// Insert (cv, ci) into a sorted list held by lanes 0..K-1 (if it belongs).
template <int K>
DEV void wave_insert(float& rv, int& ri, float cv, int ci) {
  const int lane = threadIdx.x & 63;
  const unsigned long long ahead = __ballot(lane < K && better(rv, ri, cv, ci));
  const int pos = __popcll(ahead);
  const float up_v = __shfl_up(rv, 1, 64);
  const int up_i = __shfl_up(ri, 1, 64);
  if (pos < K && lane < K && lane >= pos) {
    if (lane == pos) { rv = cv; ri = ci; }
    else { rv = up_v; ri = up_i; }
  }
}

template <int MT, int XL, int KK, int D>
__global__ __launch_bounds__(512) void lmhead_kernel(const GemmArgs a, int n_groups) {
  constexpr int NW = 8, GC = 128, ROWS = MT * 16, RPW = ROWS / NW;   // rows per wave
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_inv[ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, nchunks = K / 128, ldl = K + 8;
  uint16_t* xs = (uint16_t*)smem;
  float(*tile)[GC + 1] = (float(*)[GC + 1])(smem + (XL ? (size_t)ROWS * ldl * 2 : 0));
  const int rows = min(ROWS, a.M);

  for (int r = threadIdx.x; r < ROWS; r += blockDim.x) {
    const int m = min(r, a.M - 1);
    float ss = 0.f;
    for (int b = 0; b < a.n_ssq; ++b) ss += a.ssq_in[(size_t)b * a.ssq_ld + m];
    s_inv[r] = 1.0f / sqrtf(ss / (float)K + a.eps);
  }
  __syncthreads();
  // running lists: row wave + NW*t lives in lanes 0..KK-1 of rv[t], ri[t]
  float rv[RPW];
  int ri[RPW];
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    rv[t] = -INFINITY;
    ri[t] = 0x7fffffff - (t * 64 + lane);   // distinct placeholder ids
  }

  // W chunks of 128 k-values stream D deep: chunk c of a group lives in buffer
  // c % D (D divides the chunk count), and the last D buffers of a group are
  // refilled with the next group's first chunks, so loads stay in flight
  // through the top-k selection.
  int g = blockIdx.x;
  auto rowp = [&](int gg) {
    return (const uint16_t*)a.w + (size_t)min(gg * GC + wave * 16 + lr, a.N - 1) * K + 8 * lg;
  };
  u32x4 wbuf[D][4];
  auto load_w = [&](const uint16_t* base, int c, u32x4 (&w)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = ld16(base + 128 * c + 32 * s);
  };
  const uint16_t* wcur = rowp(min(g, n_groups - 1));
  if (g < n_groups) {
#pragma unroll
    for (int j = 0; j < D; ++j) load_w(wcur, j, wbuf[j]);
  }
  if (XL) {
    const int per_row = K / 8;
    for (int e = threadIdx.x; e < ROWS * per_row; e += blockDim.x) {
      const int r = e / per_row, c = e % per_row;
      *(u32x4*)(xs + r * ldl + 8 * c) = norm_x8(a, min(r, a.M - 1), 8 * c, s_inv[r]);
    }
    __syncthreads();
  }
  auto xfrag = [&](int mt, int k) -> u32x4 {
    if (XL) return *(const u32x4*)(xs + (mt * 16 + lr) * ldl + k + 8 * lg);
    return norm_x8(a, min(mt * 16 + lr, a.M - 1), k + 8 * lg, s_inv[mt * 16 + lr]);
  };

  bool first = true;
  for (; g < n_groups; g += gridDim.x) {
    const int gnext = g + gridDim.x;
    const bool has_next = gnext < n_groups;
    const uint16_t* wnext = has_next ? rowp(gnext) : wcur;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nchunks; c0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int c = c0 + j;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = mfma16x16x32(as_bf16x8(xfrag(mt, 128 * c + 32 * s)), as_bf16x8(wbuf[j][s]), acc[mt]);
        const int nc = c + D;
        if (nc < nchunks) load_w(wcur, nc, wbuf[j]);
        else if (has_next) load_w(wnext, nc - nchunks, wbuf[j]);
      }
    }
    wcur = wnext;
    __syncthreads();   // every wave is done reading the previous group's tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[mt * 16 + 4 * lg + i][wave * 16 + lr] = acc[mt][i];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int r = wave + NW * t;
      float v[2];
      int id[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = lane + 64 * u, n = g * GC + c;
        id[u] = n;
        const bool ok = r < rows && n < a.N;
        v[u] = ok ? tile[r][c] : -INFINITY;
        if (ok && a.logits) {
          const int i = r % a.B;
          if (i) a.logits[(size_t)((r / a.B) * (a.B - 1) + i - 1) * a.N + n] = v[u];
        }
      }
      if constexpr (KK == 1) {
        float bv = v[0];
        int bi = id[0];
        if (better(v[1], id[1], bv, bi)) { bv = v[1]; bi = id[1]; }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (better(bv, bi, rv[t], ri[t])) { rv[t] = bv; ri[t] = bi; }
      } else if (first) {
        wave_sort128(v, id);
        rv[t] = v[0];   // lanes 0..15 hold the group's 16 best
        ri[t] = id[0];
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float thv = __shfl(rv[t], KK - 1, 64);
          int thi = __shfl(ri[t], KK - 1, 64);
          unsigned long long mask = __ballot(better(v[u], id[u], thv, thi));
          while (mask) {
            const int b = __builtin_ctzll(mask);
            mask &= mask - 1;
            const float cv = __shfl(v[u], b, 64);
            const int ci = __shfl(id[u], b, 64);
            if (!better(cv, ci, thv, thi)) continue;   // threshold rose meanwhile
            wave_insert<KK>(rv[t], ri[t], cv, ci);
            thv = __shfl(rv[t], KK - 1, 64);
            thi = __shfl(ri[t], KK - 1, 64);
          }
        }
      }
    }
    first = false;
  }
  const int n_out = (a.M / a.B) * (a.B - 1);
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int r = wave + NW * t, i = r % a.B;
    if (r >= rows || i == 0 || lane >= KK) continue;
    const size_t o = ((size_t)blockIdx.x * n_out + (r / a.B) * (a.B - 1) + i - 1) * KK + lane;
    a.cand_val[o] = rv[t];
    a.cand_idx[o] = ri[t];
  }
}

template <int MT, int XL, int D>
void launch_lm_d(const GemmArgs& a, int groups, int P, size_t lds, hipStream_t st) {
  if (a.topk == 1) hipLaunchKernelGGL((lmhead_kernel<MT, XL, 1, D>), dim3(P), dim3(512), lds, st, a, groups);
  else hipLaunchKernelGGL((lmhead_kernel<MT, XL, 16, D>), dim3(P), dim3(512), lds, st, a, groups);
}

// pipeline depth: the largest of 4, 2, 1 that divides the chunk count
template <int MT, int XL>
hipError_t launch_lm(const GemmArgs& a, int groups, int P, size_t lds, hipStream_t st) {
  const int nchunks = a.K / 128;
  if (nchunks % 4 == 0) launch_lm_d<MT, XL, 4>(a, groups, P, lds, st);
  else if (nchunks % 2 == 0) launch_lm_d<MT, XL, 2>(a, groups, P, lds, st);
  else launch_lm_d<MT, XL, 1>(a, groups, P, lds, st);
  return hipGetLastError();
}

}  // namespace

LmPlan plan_lmhead(int M, int V, int K, int n_cu) {
  LmPlan p;
  p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.groups = (V + 127) / 128;
  const int per = (p.groups + n_cu - 1) / n_cu;
  p.P = (p.groups + per - 1) / per;
  const int rows = 16 * p.MT;
  const size_t xbytes = (size_t)rows * (K + 8) * 2;
  p.XL = xbytes <= LM_XL_MAX_BYTES;
  p.lds = (p.XL ? xbytes : 0) + (size_t)rows * 129 * 4;
  return p;
}

hipError_t launch_lmhead(const GemmArgs& a, const LmPlan& p, hipStream_t st) {
  if (a.topk != 1 && a.topk != 16) return hipErrorInvalidValue;
#define LM(MT) return p.XL ? launch_lm<MT, 1>(a, p.groups, p.P, p.lds, st) : launch_lm<MT, 0>(a, p.groups, p.P, p.lds, st);
  switch (p.MT) {
    case 1: LM(1)
    case 2: LM(2)
    case 4: LM(4)
    default: return hipErrorInvalidValue;
  }
#undef LM
}
