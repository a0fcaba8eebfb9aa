// Skinny (weight-streaming) GEMM for gfx950: Y[M, N] = X[M, K] . W[N, K]^T with
// M a few block rows and N, K in the thousands. Every weight byte is read once
// per call, so the kernel is HBM-bound; MFMA 16x16x32 bf16 does the arithmetic
// (16 rows x 16 columns per instruction) so the VALU is free to issue loads.
//
// Work split
//   grid.x  column groups of GC = 4 waves * NT tiles * 16 columns
//   grid.y  K splits (S); partial sums are reduced by the last-arriving
//           workgroup of each column group in fixed split order (deterministic)
//   grid.z  row chunks of 16*MT rows
// Each wave streams its NT weight tiles (16 rows of W each) over its K range
// with one 128-wide K chunk of loads in flight ahead of the MFMAs; X fragments
// come straight from L2 (X is small and shared by every workgroup).
//
// MFMA operand layout used here (v_mfma_f32_16x16x32_bf16): lane l supplies
// A[l%16][8 k-values] and B[8 k-values][l%16], the k-values of lane group
// l/16 being k0 + 8*(l/16) + 0..7 in both operands; the result lands as
// C[4*(l/16) + i][l%16], i = 0..3.
//
// Epilogues run on a [16*MT][GC] fp32 tile in LDS after the reduction:
//   E_BF16 / E_F32  store; E_RESID  h += Y (fp32 residual stream);
//   E_SILU  SiLU(gate) * up -> bf16 (gate and up tiles of one workgroup pair up);
//   E_HEAD  one head per workgroup: q/k RMSNorm over head_dim, RoPE at the row's
//           position, Q to the block buffer, K / V into the context ring;
//   E_TOPK  LM head: per-row top-k (or argmax) of the group's columns for mask
//           rows, written as candidates for topk_merge.
#include "device.h"
#include "kernels.h"

namespace {

template <int NT, bool PAIR>
DEV int tile_col(int wave, int t) {
  if constexpr (PAIR) {
    constexpr int HALF = NT / 2;
    constexpr int GC = GEMM_WAVES * NT * 16;
    return (t < HALF ? 0 : GC / 2) + wave * HALF * 16 + (t % HALF) * 16;
  } else {
    return wave * NT * 16 + t * 16;
  }
}

DEV const float* tap_ptr(const GemmArgs& a, int t) {
  const float* p = a.taps[0];
#pragma unroll
  for (int i = 1; i < MAX_TAPS; ++i)
    if (t == i) p = a.taps[i];
  return p;
}

template <int XK>
DEV u32x4 load_x(const GemmArgs& a, int row, int k) {
  if (XK == X_BF16) {
    return ld16(a.x + (size_t)row * a.ldx + k);
  } else {
    const int t = k / a.tap_hidden;
    const int col = k - t * a.tap_hidden;
    const float* p = tap_ptr(a, t) + (size_t)row * a.tap_stride + col;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < a.hc; ++st) {
      s0 += *(const f32x4*)(p + (size_t)st * a.tap_hidden);
      s1 += *(const f32x4*)(p + (size_t)st * a.tap_hidden + 4);
    }
    const float inv = 1.0f / (float)a.hc;
    s0 *= inv;
    s1 *= inv;
    u32x4 r;
    r[0] = pack_bf16x2(s0[0], s0[1]);
    r[1] = pack_bf16x2(s0[2], s0[3]);
    r[2] = pack_bf16x2(s1[0], s1[1]);
    r[3] = pack_bf16x2(s1[2], s1[3]);
    return r;
  }
}

// Row -> (request, absolute position) for E_HEAD.
DEV void row_info(const GemmArgs& a, int m, int* req, long long* p) {
  int r = a.req_of_row ? a.req_of_row[m] : m / a.rows_per_req;
  *req = r;
  if (r < 0 || r >= a.Rmax) {
    *p = -1;
    return;
  }
  *p = a.pos_of_row ? (long long)a.pos_of_row[m] : (long long)a.pos[r] + m % a.rows_per_req;
}

template <int ROWS, int GC>
DEV void epi_head(const GemmArgs& a, float (*tile)[GC + 1], int m0, int rows, int head) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hd = a.hd, half = hd / 2;
  const bool is_q = head < a.nq, is_k = !is_q && head < a.nq + a.nkv;
  for (int r = wave; r < rows; r += GEMM_WAVES) {
    const int m = m0 + r;
    int req;
    long long p;
    row_info(a, m, &req, &p);
    if (p < 0) {
      if (lane == 0) set_error(a.err, req < 0 || req >= a.Rmax ? 4u : 8u);
      continue;
    }
    if (is_q || is_k) {
      float ss = 0.f;
      for (int d = lane; d < hd; d += 64) ss += tile[r][d] * tile[r][d];
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)hd + a.eps);
      const uint16_t* g = is_q ? a.q_gain : a.k_gain;
      for (int d = lane; d < half; d += 64) {
        const float x1 = tile[r][d] * inv * bfbits2f(g[d]);
        const float x2 = tile[r][d + half] * inv * bfbits2f(g[d + half]);
        float c, s;
        rope_cos_sin(p, d, hd, a.log2_theta, &c, &s);
        const uint16_t y1 = f2bfbits(x1 * c - x2 * s);
        const uint16_t y2 = f2bfbits(x2 * c + x1 * s);
        if (is_q) {
          uint16_t* o = a.q_out + (size_t)m * a.nq * hd + (size_t)head * hd;
          o[d] = y1;
          o[d + half] = y2;
        } else {
          const int gk = head - a.nq;
          const long long slot = p % a.C;
          uint16_t* o = a.ring_k + (((size_t)req * a.nkv + gk) * a.C + slot) * hd;
          o[d] = y1;
          o[d + half] = y2;
        }
      }
    } else {
      const int gv = head - a.nq - a.nkv;
      const long long slot = p % a.C;
      uint16_t* o = a.ring_v + ((size_t)req * a.nkv + gv) * (size_t)hd * a.C + slot;
      for (int d = lane; d < hd; d += 64) o[(size_t)d * a.C] = f2bfbits(tile[r][d]);
    }
  }
}

template <int ROWS, int GC>
DEV void epi_topk(const GemmArgs& a, float (*tile)[GC + 1], int m0, int rows, int group) {
  constexpr int PER = GC / 64;  // values per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_out = (a.M / a.B) * (a.B - 1);
  for (int r = wave; r < rows; r += GEMM_WAVES) {
    const int m = m0 + r;
    const int req = m / a.B, i = m % a.B;
    if (i == 0) continue;
    const int orow = req * (a.B - 1) + (i - 1);
    float v[PER];
    int id[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = lane + 64 * u;
      id[u] = group * GC + c;
      v[u] = id[u] < a.N ? tile[r][c] : -INFINITY;
      if (a.logits && id[u] < a.N) a.logits[(size_t)orow * a.N + id[u]] = v[u];
    }
    unsigned live = (1u << PER) - 1u;
    float* cv = a.cand_val + ((size_t)group * n_out + orow) * a.topk;
    int* ci = a.cand_idx + ((size_t)group * n_out + orow) * a.topk;
    for (int j = 0; j < a.topk; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff, bu = -1;
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if ((live >> u) & 1u)
          if (bu < 0 || better(v[u], id[u], bv, bi)) { bv = v[u]; bi = id[u]; bu = u; }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if (id[u] == bi) live &= ~(1u << u);
      if (lane == 0) {
        cv[j] = bv;
        ci[j] = bi;
      }
    }
  }
}

template <int MT, int NT, int XK, int EPI, int WF>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  constexpr int ROWS = MT * 16;
  constexpr int GC = GEMM_WAVES * NT * 16;
  constexpr bool PAIR = (EPI == E_SILU);
  static_assert(!PAIR || NT % 2 == 0, "gate/up pairing needs an even tile count");
  static_assert(WF == WF_BF16, "INT4 weights take the int4 kernel");

  __shared__ float tile[ROWS][GC + 1];
  __shared__ int last_flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int group = blockIdx.x, split = blockIdx.y, mz = blockIdx.z;
  const int m0 = mz * ROWS;
  const int kbeg = split * a.ks;
  const int kend = min(a.K, kbeg + a.ks);
  const int nchunks = (kend - kbeg) / 128;

  const uint16_t* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row;
    if constexpr (PAIR) {
      constexpr int HALF = NT / 2;
      int logical = group * (GC / 2) + wave * HALF * 16 + (t % HALF) * 16 + lr;
      logical = min(logical, a.N - 1);
      row = logical + (t >= HALF ? a.pair_off : 0);
    } else {
      row = min(group * GC + wave * NT * 16 + t * 16 + lr, a.N - 1);
    }
    wrow[t] = (const uint16_t*)a.w + (size_t)row * a.K + 8 * lg;
  }
  int xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xrow[mt] = min(m0 + mt * 16 + lr, a.M - 1);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Two register stages of one 128-wide K chunk each: loads for chunk c+1 are in
  // flight while chunk c feeds the MFMAs.
  u32x4 wA[4][NT], wB[4][NT], xA[4][MT], xB[4][MT];
  auto load = [&](int c, u32x4 (&w)[4][NT], u32x4 (&x)[4][MT]) {
    const int k = kbeg + 128 * min(c, nchunks - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) x[s][mt] = load_x<XK>(a, xrow[mt], k + 32 * s + 8 * lg);
#pragma unroll
      for (int t = 0; t < NT; ++t) w[s][t] = ld_nt16(wrow[t] + k + 32 * s);
    }
  };
  auto compute = [&](int c, const u32x4 (&w)[4][NT], const u32x4 (&x)[4][MT]) {
    const bool ok = c < nchunks;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 xv = ok ? x[s][mt] : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = mfma16x16x32(as_bf16x8(xv), as_bf16x8(w[s][t]), acc[mt][t]);
      }
  };
  if (nchunks > 0) {
    load(0, wA, xA);
    for (int c = 0; c < nchunks; c += 2) {
      load(c + 1, wB, xB);
      compute(c, wA, xA);
      if (c + 2 < nchunks) load(c + 2, wA, xA);
      compute(c + 1, wB, xB);
    }
  }

  const int rows = min(ROWS, a.M - m0);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = tile_col<NT, PAIR>(wave, t) + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[mt * 16 + 4 * lg + i][col] = acc[mt][t][i];
    }
  __syncthreads();

  if (a.S > 1) {
    // Split-K: publish this split's tile, the last workgroup of the group sums
    // all splits in order s = 0..S-1.
    const size_t wg = (size_t)mz * gridDim.x + group;
    float* mine = a.partials + (wg * a.S + split) * (size_t)(ROWS * GC);
    for (int e = threadIdx.x; e < rows * GC; e += blockDim.x) mine[e] = tile[e / GC][e % GC];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev = atomicAdd(&a.counters[wg], 1u);
      const int last = (prev == (unsigned)(a.S - 1));
      if (last) atomicExch(&a.counters[wg], 0u);
      last_flag = last;
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    const float* base = a.partials + wg * a.S * (size_t)(ROWS * GC);
    for (int e = threadIdx.x; e < rows * GC; e += blockDim.x) {
      float s = 0.f;
      for (int sp = 0; sp < a.S; ++sp) s += __builtin_nontemporal_load(base + (size_t)sp * ROWS * GC + e);
      tile[e / GC][e % GC] = s;
    }
    __syncthreads();
  }

  // ---- epilogue on tile[0:rows][0:GC]
  if (EPI == E_BF16 || EPI == E_F32 || EPI == E_RESID) {
    for (int e = threadIdx.x; e < rows * GC; e += blockDim.x) {
      const int r = e / GC, c = e % GC;
      const int n = group * GC + c;
      if (n >= a.N) continue;
      const size_t o = (size_t)(m0 + r) * a.ldo + n;
      if (EPI == E_BF16) ((uint16_t*)a.out)[o] = f2bfbits(tile[r][c]);
      else if (EPI == E_F32) ((float*)a.out)[o] = tile[r][c];
      else ((float*)a.out)[o] += tile[r][c];
    }
  } else if (EPI == E_SILU) {
    constexpr int LC = GC / 2;
    for (int e = threadIdx.x; e < rows * LC; e += blockDim.x) {
      const int r = e / LC, c = e % LC;
      const int n = group * LC + c;
      if (n >= a.N) continue;
      const float g = tile[r][c], u = tile[r][LC + c];
      const float act = g / (1.0f + expf(-g)) * u;
      ((uint16_t*)a.out)[(size_t)(m0 + r) * a.ldo + n] = f2bfbits(act);
    }
  } else if (EPI == E_HEAD) {
    epi_head<ROWS, GC>(a, tile, m0, rows, a.head_base + group);
  } else if (EPI == E_TOPK) {
    epi_topk<ROWS, GC>(a, tile, m0, rows, group);
  }
}

template <int MT, int NT, int XK, int WF>
hipError_t launch_epi(const GemmArgs& a, dim3 grid, int epi, hipStream_t st) {
  switch (epi) {
    case E_BF16: hipLaunchKernelGGL((gemm_kernel<MT, NT, XK, E_BF16, WF>), grid, dim3(256), 0, st, a); break;
    case E_F32: hipLaunchKernelGGL((gemm_kernel<MT, NT, XK, E_F32, WF>), grid, dim3(256), 0, st, a); break;
    case E_RESID:
      if (XK != X_BF16) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_kernel<MT, NT, X_BF16, E_RESID, WF>), grid, dim3(256), 0, st, a); break;
    case E_SILU:
      if (XK != X_BF16 || NT % 2) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_kernel<MT, (NT % 2 ? 2 : NT), X_BF16, E_SILU, WF>), grid, dim3(256), 0, st, a); break;
    case E_HEAD:
      if (XK != X_BF16) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_kernel<MT, NT, X_BF16, E_HEAD, WF>), grid, dim3(256), 0, st, a); break;
    case E_TOPK:
      if (XK != X_BF16) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_kernel<MT, NT, X_BF16, E_TOPK, WF>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MT, int NT>
hipError_t launch_x(const GemmArgs& a, dim3 grid, int xk, int epi, int wf, hipStream_t st) {
  if (wf != WF_BF16) return hipErrorInvalidValue;
  if (xk == X_TAPS) {
    if (epi != E_BF16 && epi != E_F32) return hipErrorInvalidValue;
    if (epi == E_BF16)
      hipLaunchKernelGGL((gemm_kernel<MT, NT, X_TAPS, E_BF16, WF_BF16>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((gemm_kernel<MT, NT, X_TAPS, E_F32, WF_BF16>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return launch_epi<MT, NT, X_BF16, WF_BF16>(a, grid, epi, st);
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K, int gc, int pair, int cu_target) {
  GemmPlan p;
  p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.NT = gc / (GEMM_WAVES * 16);
  const int cols_per_group = pair ? gc / 2 : gc;
  p.groups = (N + cols_per_group - 1) / cols_per_group;
  p.mz = (M + 16 * p.MT - 1) / (16 * p.MT);
  const int kchunks = K / 128;
  int S = 1;
  const long long base = (long long)p.groups * p.mz;
  if (base < cu_target) S = (int)((cu_target + base - 1) / base);
  S = S > kchunks ? kchunks : S;
  S = S < 1 ? 1 : S;
  const int chunks_per = (kchunks + S - 1) / S;
  p.ks = chunks_per * 128;
  p.S = (K + p.ks - 1) / p.ks;
  return p;
}

size_t gemm_partial_floats(const GemmPlan& p, int gc) {
  if (p.S <= 1) return 0;
  return (size_t)p.mz * p.groups * p.S * (16 * p.MT) * gc;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int xk, int epi, int wf, hipStream_t st) {
  const dim3 grid(p.groups, p.S, p.mz);
  GemmArgs b = a;
  b.ks = p.ks;
  b.S = p.S;
#define DISPATCH_NT(MT)                                                   \
  switch (p.NT) {                                                         \
    case 1: return launch_x<MT, 1>(b, grid, xk, epi, wf, st);             \
    case 2: return launch_x<MT, 2>(b, grid, xk, epi, wf, st);             \
    default: return hipErrorInvalidValue;                                 \
  }
  switch (p.MT) {
    case 1: DISPATCH_NT(1)
    case 2: DISPATCH_NT(2)
    case 4: DISPATCH_NT(4)
    default: return hipErrorInvalidValue;
  }
#undef DISPATCH_NT
}
