// Skinny (weight-streaming) GEMM for gfx950: Y[M, N] = X[M, K] . W[N, K]^T with
// M a few block rows and N, K in the thousands. Every weight byte is read once
// per call, so the kernel is HBM-bound; MFMA 16x16x32 bf16 does the arithmetic
// (16 rows x 16 columns per instruction) so the VALU is free to issue loads.
//
// Work split
//   grid.x  column groups of GC = NW waves * 16 columns (one 16-row W tile per wave)
//   grid.y  K splits (S)
//   grid.z  row chunks of 16*MT rows
// The workgroup first stages its X slice [16*MT rows][K range] in LDS (for tap
// inputs the hc-stream mean and the bf16 cast happen here, once per element);
// then every wave streams its W tile over the K range, several 128-wide chunks
// of loads in flight ahead of the MFMAs. Plain (cached) loads measured faster than
// non-temporal ones for this pattern.
//
// Split-K (S > 1): each split stores its partial tile straight from the MFMA
// accumulators (E_PART, E_PARTP) and the workgroup ends; a finish kernel sums
// the splits in split order (deterministic) and applies the epilogue. An
// in-kernel "last split reduces" scheme was measured slower: its publish /
// count / re-read chain is three dependent device-scope round trips at the
// tail of every projection, while the kernel boundary costs well under 1 us.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l supplies A[l%16][8
// k-values] and B[8 k-values][l%16], the k-values of lane group l/16 being
// k0 + 8*(l/16) + 0..7 in both operands; the result lands as
// C[4*(l/16) + i][l%16], i = 0..3.
//
// INT4 weights (symmetric, groups of 64 along K, fp16 scales): in the 128-wide
// chunk c of a row, 32-bit word 4*j + s of the packed row holds the eight values
// k = 128c + 32s + 8j + e (e = 0..7) as u = q + 8, value e in nibble e/2 (even
// e) or 4 + (e-1)/2 (odd e). Lane group lg therefore gets all its k-values of
// the chunk's four MFMA steps with one 16-byte load (words 4lg..4lg+3), and the
// nibble pair (e, e+1) of a word w becomes the bf16 pair (128 + u_e, 128 + u_e+1)
// in two ops: ((w >> 2e) & 0x000F000F) | 0x43004300 (0x4300 is bf16 128.0, whose
// ulp is 1). The MFMAs of one 64-group accumulate t = sum x * (u + 128) from
// zero; with xs = sum x over the group (row sums of the bf16 X values, computed
// once while X is staged) the group adds s * (t - 136 * xs) = s * sum x * q.
//
// Epilogues run on a [16*MT][GC] fp32 tile in LDS:
//   E_BF16 / E_F32  store; E_RESID  h += Y (fp32 residual stream);
//   E_SILU  SiLU(gate) * up -> bf16 (the first half of the waves stream gate
//           rows, the second half the matching up rows);
//   E_HEAD  one head per workgroup: q/k RMSNorm over head_dim, RoPE at the row's
//           position, Q to the block buffer, K / V into the context ring;
// these need the whole K range in one workgroup (S = 1).

#include "device.h"
#include "kernels.h"

namespace {

DEV const float* tap_ptr(const GemmArgs& a, int t) {
  const float* p = a.taps[0];
#pragma unroll
  for (int i = 1; i < MAX_TAPS; ++i)
    if (t == i) p = a.taps[i];
  return p;
}

// 8 consecutive X values (k..k+7) of row `row` as bf16x8 (`inv`: the row's
// 1/rms for X_NORM).
template <int XK>
DEV u32x4 load_x(const GemmArgs& a, int row, int k, float inv) {
  if constexpr (XK == X_BF16) {
    return ld16(a.x + (size_t)row * a.ldx + k);
  } else if constexpr (XK == X_NORM) {
    const float* p = a.xf + (size_t)row * a.ldx + k;
    return norm8(*(const f32x4*)p, *(const f32x4*)(p + 4), ld16(a.xgain + k), inv);
  } else {
    const int t = k / a.tap_hidden;
    const int col = k - t * a.tap_hidden;
    const int src = a.src_row ? a.src_row[row] : row;
    return hc_mean8_bf16(tap_ptr(a, t) + (size_t)src * a.tap_stride + col, (size_t)a.tap_hidden, a.hc);
  }
}

template <int GC, int NW>
DEV void epi_head(const GemmArgs& a, float (*tile)[GC + 1], int m0, int rows, int head) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hd = a.hd, half = hd / 2;
  const bool is_q = head < a.nq, is_k = !is_q && head < a.nq + a.nkv;
  for (int r = wave; r < rows; r += NW) {
    const int m = m0 + r;
    int req;
    long long p, rp;
    const unsigned bad = ring_row(a, m, &req, &p, &rp);
    if (bad) {
      if (lane == 0) set_error(a.err, bad);
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
        rope_cos_sin(rp, d, hd, a.log2_theta, &c, &s);
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


// Per-row sums over 64-wide K groups of the bf16 X values, [klen/64][ROWS] floats
// after the X slice (or at the start of LDS when X is not staged).
template <int ROWS>
DEV size_t xsum_offset(int XL, int ks) {
  return XL ? (((size_t)ROWS * (ks + 8) * 2 + 15) & ~(size_t)15) : 0;
}

template <int MT, int NW, int XK, int XL, int EPI, int D, int WF>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const GemmArgs a) {
  constexpr int ROWS = MT * 16;
  constexpr int GC = NW * 16;
  constexpr bool PAIR = (EPI == E_SILU || EPI == E_PARTP);
  constexpr bool Q4 = WF == WF_INT4;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n_mz = (a.M + ROWS - 1) / ROWS;
  const int group = blockIdx.x, split = blockIdx.y, mz = blockIdx.z % n_mz, layer = blockIdx.z / n_mz;
  const int m0 = mz * ROWS;
  const void* wbase = a.nb > 0 ? pick(a.wb, layer) : a.w;
  const int kbeg = split * a.ks;
  const int kend = min(a.K, kbeg + a.ks);
  const int klen = kend - kbeg;
  const int nchunks = klen / 128;
  const int ldl = a.ks + 8;   // LDS row pitch of the X slice (elements)
  uint16_t* xs = (uint16_t*)smem;

  // this wave's W rows (16 per tile); for gate/up the first half of the waves
  // take gate rows, the second half the up rows of the same columns
  int wrow_i, tcol;
  if constexpr (PAIR) {
    constexpr int HALF = NW / 2;
    const int logical = min(group * (GC / 2) + (wave % HALF) * 16 + lr, a.N - 1);
    wrow_i = logical + (wave >= HALF ? a.pair_off : 0);
    tcol = (wave >= HALF ? GC / 2 : 0) + (wave % HALF) * 16;
  } else {
    wrow_i = min(group * GC + wave * 16 + lr, a.N - 1);
    tcol = wave * 16;
  }
  const uint16_t* wrow = (const uint16_t*)wbase + (size_t)wrow_i * a.K + kbeg + 8 * lg;
  const uint8_t* qrow = (const uint8_t*)wbase + (size_t)wrow_i * (a.K / 2) + kbeg / 2 + 16 * lg;
  const uint16_t* srow = nullptr;
  if constexpr (Q4) srow = (a.nb > 0 ? pick(a.wsb, layer) : a.wscale) + (size_t)wrow_i * (a.K / 64) + kbeg / 64;

  // D 128-wide chunks of W loads stay in flight (chunk c in buffer c % D); the
  // first D are issued before the X slice is staged, so they stream meanwhile.
  // bf16: four 16-byte loads per chunk; INT4: one 16-byte load of packed words
  // plus the chunk's two fp16 group scales.
  u32x4 wbuf[D][Q4 ? 1 : 4];
  uint32_t sbuf[D];
  auto load_w = [&](int c, int j) {
    if constexpr (Q4) {
      wbuf[j][0] = ld16(qrow + 64 * c);
      sbuf[j] = *(const uint32_t*)(srow + 2 * c);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) wbuf[j][s] = ld16(wrow + 128 * c + 32 * s);
    }
  };
  // Loads are never behind a branch (a chunk past the end re-reads the last
  // one): the compiler then counts outstanding loads exactly and waits only for
  // the buffer it needs, instead of draining every load at each branch.
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nchunks) load_w(j, j);

  __shared__ float s_inv[ROWS];
  if constexpr (XK == X_NORM) {
    // 1/rms of each row from the producer's per-column-group sums of squares
    // (summed in group order; the loads of 8 groups are in flight together)
    for (int r = threadIdx.x; r < ROWS; r += blockDim.x) {
      const int m = min(m0 + r, a.M - 1);
      float ss = 0.f;
      for (int b0 = 0; b0 < a.n_ssq; b0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = a.ssq_in[(size_t)min(b0 + u, a.n_ssq - 1) * a.ssq_ld + m];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (b0 + u < a.n_ssq) ss += v[u];
      }
      s_inv[r] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    }
    __syncthreads();
  }
  auto row_inv = [&](int r) -> float {
    if constexpr (XK == X_NORM) return s_inv[r];
    return 1.0f;
  };
  float* xsum = (float*)(smem + xsum_offset<ROWS>(XL, a.ks));
  if (XL || Q4) {
    // one pass over the X slice: stage it (XL) and, for INT4, sum each row's
    // bf16 values per 64-group (8 lanes hold the 8 pieces of one group: the
    // per-row count klen/8 is a multiple of 16, so groups never straddle rows
    // and all 8 lanes of a group are active together)
    // Only the rows below M are loaded (an 8-row block would otherwise read its
    // X twice); the tile's padding rows are zeros. The loop bound is a multiple
    // of 16 pieces, so the 8 lanes of a group are active together.
    const int per_row = klen / 8;
    const int rows_x = min(ROWS, a.M - m0);
    for (int e = threadIdx.x; e < (ROWS - rows_x) * per_row; e += blockDim.x) {
      const int r = rows_x + e / per_row, c = e % per_row;
      if (XL) *(u32x4*)(xs + r * ldl + 8 * c) = (u32x4){0u, 0u, 0u, 0u};
      if (Q4 && (c & 7) == 0) xsum[(c >> 3) * ROWS + r] = 0.f;
    }
    for (int e = threadIdx.x; e < rows_x * per_row; e += blockDim.x) {
      const int r = e / per_row, c = e % per_row;
      const u32x4 v = load_x<XK>(a, m0 + r, kbeg + 8 * c, row_inv(r));
      if (XL) *(u32x4*)(xs + r * ldl + 8 * c) = v;
      if constexpr (Q4) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) t += __uint_as_float(v[i] << 16) + __uint_as_float(v[i] & 0xffff0000u);
        t += __shfl_xor(t, 1, 64);
        t += __shfl_xor(t, 2, 64);
        t += __shfl_xor(t, 4, 64);
        if ((c & 7) == 0) xsum[(c >> 3) * ROWS + r] = t;
      }
    }
    __syncthreads();
  }
  auto xfrag = [&](int mt, int kk) -> u32x4 {   // kk: offset inside the K range
    if (XL) return *(const u32x4*)(xs + (mt * 16 + lr) * ldl + kk + 8 * lg);
    return load_x<XK>(a, min(m0 + mt * 16 + lr, a.M - 1), kbeg + kk + 8 * lg, row_inv(mt * 16 + lr));
  };

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint32_t q4_mask = 0, q4_bias = 0;
  if constexpr (Q4) int4_unpack_consts(q4_mask, q4_bias);
  auto compute = [&](int c, int j) {
    if constexpr (Q4) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float sc = half_bits_to_float(gi ? sbuf[j] >> 16 : sbuf[j] & 0xffffu);
        f32x4 t[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 2 * gi; s < 2 * gi + 2; ++s) {
          const bf16x8 b = as_bf16x8(int4_biased_bf16(wbuf[j][0][s], q4_mask, q4_bias));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) t[mt] = mfma16x16x32(as_bf16x8(xfrag(mt, 128 * c + 32 * s)), b, t[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 xg = *(const f32x4*)(xsum + (2 * c + gi) * ROWS + mt * 16 + 4 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(sc, fmaf(-136.0f, xg[i], t[mt][i]), acc[mt][i]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = mfma16x16x32(as_bf16x8(xfrag(mt, 128 * c + 32 * s)), as_bf16x8(wbuf[j][s]), acc[mt]);
    }
  };
  for (int c0 = 0; c0 < nchunks; c0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int c = c0 + j;
      if (c < nchunks) {
        compute(c, j);
        if (c + D < nchunks) load_w(c + D, j);
      }
    }
  }

  if constexpr (EPI == E_PART || EPI == E_PARTP) {
    // partial tile of this split: lane holds C[4*lg + i][lr] of each row tile
    int n;
    bool ok;
    if constexpr (PAIR) {
      constexpr int HALF = NW / 2;
      const int logical = group * (GC / 2) + (wave % HALF) * 16 + lr;
      ok = logical < a.N;
      n = logical + (wave >= HALF ? a.N : 0);
    } else {
      n = group * GC + wave * 16 + lr;
      ok = n < a.N;
    }
    const int ntot = PAIR ? 2 * a.N : a.N;
    float* dst = a.partials + ((size_t)layer * a.S + split) * a.M * ntot + n;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mt * 16 + 4 * lg + i;
        if (ok && m < a.M) dst[(size_t)m * ntot] = acc[mt][i];
      }
    return;
  }

  // ---- result tile in LDS (aliases the X slice, which is dead now)
  __syncthreads();
  float(*tile)[GC + 1] = (float(*)[GC + 1])smem;
  const int rows = min(ROWS, a.M - m0);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[mt * 16 + 4 * lg + i][tcol + lr] = acc[mt][i];
  __syncthreads();

  // ---- epilogue on tile[0:rows][0:GC]
  if constexpr (EPI == E_BF16 || EPI == E_F32) {
    for (int e = threadIdx.x; e < rows * GC; e += blockDim.x) {
      const int r = e / GC, c = e % GC;
      const int n = group * GC + c;
      if (n >= a.N) continue;
      const size_t o = (size_t)(m0 + r) * a.ldo + n;
      if (EPI == E_BF16) ((uint16_t*)a.out)[o] = f2bfbits(tile[r][c]);
      else ((float*)a.out)[o] = tile[r][c];
    }
  } else if constexpr (EPI == E_RESID) {
    // h += Y; the updated values stay in the tile for the row sums of squares
    for (int e = threadIdx.x; e < rows * GC; e += blockDim.x) {
      const int r = e / GC, c = e % GC;
      const int n = group * GC + c;
      float hv = 0.f;
      if (n < a.N) {
        float* hp = (float*)a.out + (size_t)(m0 + r) * a.ldo + n;
        hv = *hp + tile[r][c];
        *hp = hv;
      }
      tile[r][c] = hv;
    }
    if (a.ssq_out) {
      __syncthreads();
      for (int r = wave; r < rows; r += NW) {
        float ss = 0.f;
        for (int c = lane; c < GC; c += 64) ss += tile[r][c] * tile[r][c];
        ss = wave_sum(ss);
        if (lane == 0) a.ssq_out[(size_t)group * a.ssq_ld + m0 + r] = ss;
      }
    }
  } else if constexpr (EPI == E_SILU) {
    constexpr int LC = GC / 2;
    for (int e = threadIdx.x; e < rows * LC; e += blockDim.x) {
      const int r = e / LC, c = e % LC;
      const int n = group * LC + c;
      if (n >= a.N) continue;
      const float g = tile[r][c], u = tile[r][LC + c];
      const float act = g / (1.0f + expf(-g)) * u;
      ((uint16_t*)a.out)[(size_t)(m0 + r) * a.ldo + n] = f2bfbits(act);
    }
  } else if constexpr (EPI == E_HEAD) {
    epi_head<GC, NW>(a, tile, m0, rows, a.head_base + group);
  }
}

// bf16 W chunks in flight per wave. Measured at the qwen3-4b shape, 16 rows: 4 lets
// every chunk of a 4-chunk split go out before the X staging (gate/up 28.9 ->
// 28.2 us per layer with the finish, fc 21.5 -> 21.2 us); with more row tiles
// the registers of 3 are enough.
constexpr int gemm_depth(int MT) { return MT == 1 ? 4 : 3; }
constexpr int GEMM_DEPTH_Q4 = 8;   // INT4 chunks are a quarter of the bytes
// with X fragments read from L2 (no LDS slice) the deeper INT4 pipeline spills
constexpr int GEMM_DEPTH_Q4_NOXL = 4;

template <int MT, int NW, int XK, int XL, int EPI>
void launch_one(const GemmArgs& a, dim3 grid, size_t lds, int wf, hipStream_t st) {
  constexpr int DQ = XL ? GEMM_DEPTH_Q4 : GEMM_DEPTH_Q4_NOXL;
  if (wf == WF_INT4)
    hipLaunchKernelGGL((gemm_kernel<MT, NW, XK, XL, EPI, DQ, WF_INT4>), grid, dim3(NW * 64), lds, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<MT, NW, XK, XL, EPI, gemm_depth(MT), WF_BF16>), grid, dim3(NW * 64), lds, st, a);
}

template <int MT, int NW, int XL>
hipError_t launch_x(const GemmArgs& a, dim3 grid, size_t lds, int xk, int epi, int wf, hipStream_t st) {
  if (xk == X_TAPS) {
    if (epi == E_BF16) launch_one<MT, NW, X_TAPS, XL, E_BF16>(a, grid, lds, wf, st);
    else if (epi == E_F32) launch_one<MT, NW, X_TAPS, XL, E_F32>(a, grid, lds, wf, st);
    else if (epi == E_PART) launch_one<MT, NW, X_TAPS, XL, E_PART>(a, grid, lds, wf, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (xk == X_NORM) {
    switch (epi) {
      case E_SILU: launch_one<MT, NW, X_NORM, XL, E_SILU>(a, grid, lds, wf, st); break;
      case E_HEAD: launch_one<MT, NW, X_NORM, XL, E_HEAD>(a, grid, lds, wf, st); break;
      case E_PART: launch_one<MT, NW, X_NORM, XL, E_PART>(a, grid, lds, wf, st); break;
      case E_PARTP: launch_one<MT, NW, X_NORM, XL, E_PARTP>(a, grid, lds, wf, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case E_BF16: launch_one<MT, NW, X_BF16, XL, E_BF16>(a, grid, lds, wf, st); break;
    case E_F32: launch_one<MT, NW, X_BF16, XL, E_F32>(a, grid, lds, wf, st); break;
    case E_RESID: launch_one<MT, NW, X_BF16, XL, E_RESID>(a, grid, lds, wf, st); break;
    case E_SILU: launch_one<MT, NW, X_BF16, XL, E_SILU>(a, grid, lds, wf, st); break;
    case E_HEAD: launch_one<MT, NW, X_BF16, XL, E_HEAD>(a, grid, lds, wf, st); break;
    case E_PART: launch_one<MT, NW, X_BF16, XL, E_PART>(a, grid, lds, wf, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MT, int NW>
hipError_t launch_xl(const GemmArgs& a, dim3 grid, size_t lds, int xl, int xk, int epi, int wf, hipStream_t st) {
  return xl ? launch_x<MT, NW, 1>(a, grid, lds, xk, epi, wf, st) : launch_x<MT, NW, 0>(a, grid, lds, xk, epi, wf, st);
}

constexpr size_t XL_MAX_BYTES = 96 * 1024;
constexpr size_t GEMM_LDS_MAX = 160 * 1024;   // LDS per workgroup on gfx950


}  // namespace

GemmPlan plan_gemm(int M, int N, int K, int gc, int pair, int cps, int wf) {
  GemmPlan p;
  p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.NT = 1;
  p.NW = gc / 16;
  const int cols_per_group = pair ? gc / 2 : gc;
  p.groups = (N + cols_per_group - 1) / cols_per_group;
  p.mz = (M + 16 * p.MT - 1) / (16 * p.MT);
  const int kchunks = K / 128;
  // enough column-group x row-chunk workgroups already (prefill): no split;
  // otherwise about cps chunks of K per split
  const long long base = (long long)p.groups * p.mz;
  int S = base >= 256 ? 1 : (kchunks + cps - 1) / cps;
  // partial tiles stay within the workspace budget
  const long long per_split = (long long)M * (pair ? 2 * N : N);
  const long long cap = GEMM_PARTIAL_BUDGET / (per_split > 0 ? per_split : 1);
  if (S > cap) S = (int)cap;
  S = S < 1 ? 1 : S;
  const int chunks_per = (kchunks + S - 1) / S;
  const int rows = 16 * p.MT;
  p.ks = chunks_per * 128;
  p.S = (K + p.ks - 1) / p.ks;
  // INT4: per-row sums of X over each 64-group of the K range
  const size_t sbytes = wf == WF_INT4 ? (size_t)rows * (p.ks / 64) * 4 : 0;
  const size_t xl_bytes = (((size_t)rows * (p.ks + 8) * 2 + 15) & ~(size_t)15) + sbytes;
  // stage X through LDS when the slice fits; otherwise fragments come from L2
  p.XL = xl_bytes <= XL_MAX_BYTES;
  const size_t xbytes = p.XL ? xl_bytes : sbytes;
  const size_t tbytes = (size_t)rows * (gc + 1) * 4;   // result tile
  p.lds = xbytes > tbytes ? xbytes : tbytes;
  return p;
}

size_t gemm_partial_floats(const GemmPlan& p, int M, int N, int pair) {
  if (p.S <= 1) return 0;
  return (size_t)p.S * M * (pair ? 2 * N : N);
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int xk, int epi, int wf, hipStream_t st) {
  if (wf != WF_BF16 && wf != WF_INT4) return hipErrorInvalidValue;
  if (wf == WF_INT4 && (a.K % 128 || (a.nb > 0 ? !a.wsb[0] : !a.wscale))) return hipErrorInvalidValue;
  if (p.lds > GEMM_LDS_MAX) return hipErrorInvalidValue;
  // a complete epilogue needs the whole K range in one workgroup
  if (p.S > 1 && epi != E_PART && epi != E_PARTP) return hipErrorInvalidValue;
  if (a.nb > MAX_BATCH || (a.nb > 0 && epi != E_PART)) return hipErrorInvalidValue;
  const dim3 grid(p.groups, p.S, p.mz * (a.nb > 0 ? a.nb : 1));
  GemmArgs b = a;
  b.ks = p.ks;
  b.S = p.S;
#define DISPATCH_NW(MT)                                                         \
  switch (p.NW) {                                                               \
    case 4: return launch_xl<MT, 4>(b, grid, p.lds, p.XL, xk, epi, wf, st);      \
    case 8: return launch_xl<MT, 8>(b, grid, p.lds, p.XL, xk, epi, wf, st);      \
    default: return hipErrorInvalidValue;                                       \
  }
  switch (p.MT) {
    case 1: DISPATCH_NW(1)
    case 2: DISPATCH_NW(2)
    case 4: DISPATCH_NW(4)
    default: return hipErrorInvalidValue;
  }
#undef DISPATCH_NW
}
