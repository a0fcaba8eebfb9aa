// Staging of up to 16 RMS-normed rows, whole, in LDS (bf16 [16][K + 8]) by a
// workgroup of NT threads, for kernels that also stream weights straight into
// LDS: the RMSNorm of the layer input before the gate/up projection and the
// final norm before the LM head (x = h * rsqrt(ss / K + eps) * gain, ss the sum
// over the producer's 128-column groups of h^2, added in group order).
//
// Two calls around the kernel's own weight prologue:
//   norm_rows_issue  the gains (straight to LDS), then for this thread's row
//                    (NT / 16 threads per row) the producer's sums of squares
//                    and this thread's X pieces (8 fp32 values each, pieces
//                    t % TPR + TPR u of the row) into registers;
//   norm_rows_store  one wait covers every load issued so far; the thread forms
//                    its row's 1/rms in registers and stores its pieces, reading
//                    the gains of half its pieces at a time.
// The compiler makes any register use or LDS access wait for every
// direct-to-LDS load in flight, so all loads go out before the first use (a
// scheduling barrier keeps them there) and the sums of squares are loaded
// unconditionally (clamped to the last group). The arithmetic is norm8's, so the
// staged bits equal those of every other path that normalizes these rows.
#pragma once
#include "device.h"
#include "kernels.h"

typedef __attribute__((address_space(3))) void lds_void;

constexpr int NORM_SSQ_MAX = 24;   // producer column groups per row: K / 128 <= 24

// LDS bytes of the staged rows, then of the gains (whole KB)
__host__ __device__ inline size_t norm_rows_bytes(int K) { return ((size_t)16 * (K + 8) * 2 + 15) & ~(size_t)15; }
__host__ __device__ inline size_t norm_gain_bytes(int K) { return ((size_t)K * 2 + 1023) & ~(size_t)1023; }
// whether NT threads with XP pieces each cover the rows (and the sums of squares fit)
__host__ __device__ inline bool norm_rows_fit(int K, int NT, int XP) {
  return K % 128 == 0 && K / 128 <= NORM_SSQ_MAX && K / 8 <= XP * (NT / 16);
}

template <int XP>
struct NormRowsLoads {
  float sq[NORM_SSQ_MAX];
  f32x4 h0[XP], h1[XP];
};

template <int NT, int XP>
DEV void norm_rows_issue(const GemmArgs& a, uint16_t* gains, NormRowsLoads<XP>& L) {
  constexpr int TPR = NT / 16;
  const int K = a.K, per_row = K / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = threadIdx.x / TPR, pc0 = threadIdx.x % TPR;
  const int m = min(row, a.M - 1);
  for (int i = wave; i < (int)(norm_gain_bytes(K) / 1024); i += NT / 64)   // 1 KB of gains per instruction
    __builtin_amdgcn_global_load_lds((const void*)(a.xgain + min(512 * i + 8 * lane, K - 8)),
                                     (lds_void*)(gains + 512 * i), 16, 0, 0);
#pragma unroll
  for (int b = 0; b < NORM_SSQ_MAX; ++b) L.sq[b] = a.ssq_in[(size_t)min(b, a.n_ssq - 1) * a.ssq_ld + m];
  const float* hrow = a.xf + (size_t)m * a.ldx;
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int pc = pc0 + TPR * u;
    if (pc < per_row) {
      L.h0[u] = *(const f32x4*)(hrow + 8 * pc);
      L.h1[u] = *(const f32x4*)(hrow + 8 * pc + 4);
    }
  }
}

template <int NT, int XP>
DEV void norm_rows_store(const GemmArgs& a, const uint16_t* gains, uint16_t* xs, int ldl, NormRowsLoads<XP>& L) {
  static_assert(XP % 2 == 0, "gains are read for half the pieces at a time");
  constexpr int TPR = NT / 16, GB = XP / 2;
  __builtin_amdgcn_sched_barrier(0);
  const int K = a.K, per_row = K / 8;
  const int row = threadIdx.x / TPR, pc0 = threadIdx.x % TPR;
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < NORM_SSQ_MAX; ++b)
    if (b < a.n_ssq) ss += L.sq[b];
  const float inv = 1.0f / sqrtf(ss / (float)K + a.eps);
  __syncthreads();   // the gains have landed in every wave
#pragma unroll
  for (int u0 = 0; u0 < XP; u0 += GB) {
    u32x4 g[GB];
#pragma unroll
    for (int j = 0; j < GB; ++j) g[j] = *(const u32x4*)(gains + 8 * min(pc0 + TPR * (u0 + j), per_row - 1));
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int pc = pc0 + TPR * (u0 + j);
      if (pc < per_row) *(u32x4*)(xs + row * ldl + 8 * pc) = norm8(L.h0[u0 + j], L.h1[u0 + j], g[j], inv);
    }
  }
  __syncthreads();
}
