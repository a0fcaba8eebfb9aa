// Staging of ROWS (16, 32 or 64) RMS-normed rows, or columns [k0, k0 + kw) of
// them, in LDS (bf16 [ROWS][kw + 8]) by a workgroup of NT threads, for kernels that also stream
// weights straight into LDS: the RMSNorm of the layer input before the gate/up
// projection and the final norm before the LM head (x = h * rsqrt(ss / K + eps) * gain, ss the sum
// over the producer's 128-column groups of h^2, added in group order).
//
// Two calls around the kernel's own weight prologue:
//   norm_rows_issue  the gains of the columns (straight to LDS), then for this
//                    thread's row (NT / ROWS threads per row) its share of the
//                    producer's sums of squares (the whole row's) and its X
//                    pieces (8 fp32 values each, pieces t % TPR + TPR u of the
//                    columns) into registers;
//   norm_rows_store  one wait covers every load issued so far; the row's sums
//                    pass through LDS, each thread adds its row's in group order
//                    to form 1/rms and stores its pieces, reading the gains of
//                    half its pieces at a time.
// The compiler makes any register use or LDS access wait for every
// direct-to-LDS load in flight, so all loads go out before the first use (a
// scheduling barrier keeps them there) and the sums of squares are loaded
// unconditionally (clamped to the last group). The arithmetic is norm8's, and the
// sums are added in the same order, so the staged bits equal those of every
// other path that normalizes these rows.
#pragma once
#include "device.h"
#include "kernels.h"

typedef __attribute__((address_space(3))) void lds_void;

constexpr int NORM_SSQ_MAX = 32;   // producer column groups per row: K / 128 <= 32

// LDS bytes of kw staged columns of `rows` rows, then of their gains (whole KB)
__host__ __device__ inline size_t norm_rows_bytes(int kw, int rows = 16) {
  return ((size_t)rows * (kw + 8) * 2 + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t norm_gain_bytes(int kw) { return ((size_t)kw * 2 + 1023) & ~(size_t)1023; }
// whether NT threads with XP pieces each cover kw columns of `rows` rows of K
__host__ __device__ inline bool norm_rows_fit(int K, int kw, int NT, int XP, int rows = 16) {
  return K % 128 == 0 && kw % 128 == 0 && kw <= K && K / 128 <= NORM_SSQ_MAX && kw / 8 <= XP * (NT / rows);
}

// static LDS of norm_rows_store: each row's sums of squares as its threads loaded them
__host__ __device__ inline size_t norm_sq_bytes(int NT, int rows) {
  const int tpr = NT / rows, sqp = (NORM_SSQ_MAX + tpr - 1) / tpr;
  return (size_t)rows * tpr * sqp * 4;
}

// per thread: SQP of the row's sums of squares (groups t % TPR + TPR j) and XP
// pieces of its columns
template <int XP, int SQP>
struct NormRowsLoads {
  float sq[SQP];
  f32x4 h0[XP], h1[XP];
};
template <int NT, int ROWS>
constexpr int norm_sqp() { return (NORM_SSQ_MAX + NT / ROWS - 1) / (NT / ROWS); }

template <int NT, int XP, int ROWS = 16>
DEV void norm_rows_issue(const GemmArgs& a, int k0, int kw, uint16_t* gains,
                         NormRowsLoads<XP, norm_sqp<NT, ROWS>()>& L) {
  constexpr int TPR = NT / ROWS, SQP = norm_sqp<NT, ROWS>();
  const int per_row = kw / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = threadIdx.x / TPR, pc0 = threadIdx.x % TPR;
  const int m = min(row, a.M - 1);
  for (int i = wave; i < (int)(norm_gain_bytes(kw) / 1024); i += NT / 64)   // 1 KB of gains per instruction
    __builtin_amdgcn_global_load_lds((const void*)(a.xgain + k0 + min(512 * i + 8 * lane, kw - 8)),
                                     (lds_void*)(gains + 512 * i), 16, 0, 0);
#pragma unroll
  for (int j = 0; j < SQP; ++j) L.sq[j] = a.ssq_in[(size_t)min(pc0 + TPR * j, a.n_ssq - 1) * a.ssq_ld + m];
  // rows at or past M are the tile's padding: zeros, not a second copy of a row
  const float* hrow = a.xf + (size_t)m * a.ldx + k0;
  const bool real = row < a.M;
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int pc = pc0 + TPR * u;
    if (pc < per_row && real) {
      L.h0[u] = *(const f32x4*)(hrow + 8 * pc);
      L.h1[u] = *(const f32x4*)(hrow + 8 * pc + 4);
    } else {
      L.h0[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      L.h1[u] = L.h0[u];
    }
  }
}

// With XSUM, also each row's sums over the 64-column groups of the staged bf16
// values, xsum[g][ROWS] (the INT4 weights' correction term): each 8-value piece
// summed in order, then the 8 pieces of a group in a butterfly over the 8
// consecutive lanes that hold them (TPR is a multiple of 8, so a group never
// straddles rows or lane groups).
template <int NT, int XP, int ROWS = 16, bool XSUM = false>
DEV void norm_rows_store(const GemmArgs& a, int kw, const uint16_t* gains, uint16_t* xs, int ldl,
                         NormRowsLoads<XP, norm_sqp<NT, ROWS>()>& L, float* xsum = nullptr) {
  static_assert(XP % 2 == 0, "gains are read for half the pieces at a time");
  constexpr int TPR = NT / ROWS, GB = XP / 2, SQP = norm_sqp<NT, ROWS>();
  static_assert(!XSUM || TPR % 8 == 0, "a group's 8 pieces in 8 lanes of one row");
  __builtin_amdgcn_sched_barrier(0);
  const int K = a.K, per_row = kw / 8;
  const int row = threadIdx.x / TPR, pc0 = threadIdx.x % TPR;
  __shared__ float s_sq[ROWS][TPR * SQP];
#pragma unroll
  for (int j = 0; j < SQP; ++j) s_sq[row][pc0 + TPR * j] = L.sq[j];
  __syncthreads();   // the gains and the sums of squares are in LDS
  float ss = 0.f;
  for (int b = 0; b < a.n_ssq; ++b) ss += s_sq[row][b];
  const float inv = 1.0f / sqrtf(ss / (float)K + a.eps);
#pragma unroll
  for (int u0 = 0; u0 < XP; u0 += GB) {
    u32x4 g[GB];
#pragma unroll
    for (int j = 0; j < GB; ++j) g[j] = *(const u32x4*)(gains + 8 * min(pc0 + TPR * (u0 + j), per_row - 1));
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int pc = pc0 + TPR * (u0 + j);
      const u32x4 v = norm8(L.h0[u0 + j], L.h1[u0 + j], g[j], inv);
      if (pc < per_row) *(u32x4*)(xs + row * ldl + 8 * pc) = v;
      if constexpr (XSUM) {   // every lane takes part; per_row is a multiple of 8
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) t += __uint_as_float(v[i] << 16) + __uint_as_float(v[i] & 0xffff0000u);
        t += __shfl_xor(t, 1, 64);
        t += __shfl_xor(t, 2, 64);
        t += __shfl_xor(t, 4, 64);
        if (pc < per_row && (pc & 7) == 0) xsum[(pc >> 3) * ROWS + row] = t;
      }
    }
  }
  __syncthreads();
}
