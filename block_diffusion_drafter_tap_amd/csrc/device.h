// Device-side helpers shared by the gfx950 kernels of the drafter round.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

// bf16 <-> fp32. The fp32 -> bf16 conversion rounds to nearest even (gfx950 has
// a hardware conversion; the compiler emits it for this cast).
DEV float bf2f(__bf16 v) { return (float)v; }
DEV float bfbits2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
DEV __bf16 f2bf(float v) { return (__bf16)v; }
DEV uint16_t f2bfbits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// Two values as a bf16 pair (lo in the low half), rounded to nearest even: one
// v_cvt_pk_bf16_f32, the same conversion f2bfbits makes for each value alone.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// RMSNorm of 8 consecutive values: bf16x8 of (h * inv) * g, with h the fp32
// values in h0, h1, inv the row's 1/rms and g their 8 bf16 gains. Every path
// that stages normed rows uses this, so a row's bf16 operand is the same bits
// whichever kernel stages it.
DEV u32x4 norm8(f32x4 h0, f32x4 h1, u32x4 g, float inv) {
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

// fp64 -> bf16 rounded to nearest even in one step: fp64 -> fp32 toward zero
// with the sticky bit ORed into the last fp32 bit (round to odd), then the
// fp32 -> bf16 conversion (nearest even). fp32 keeps 16 more significand bits
// than bf16, so the two steps round exactly like a single one.
DEV uint16_t f64_to_bf16bits(double x) {
  float t = __double2float_rz(x);
  if ((double)t != x) t = __uint_as_float(__float_as_uint(t) | 1u);
  return f2bfbits(t);
}

// Eight consecutive values of the per-token mean over hc hyper-connection
// streams, as bf16x8: p points at stream 0's first value, streams are `ld`
// floats apart. With one stream the value is the tap itself. Otherwise the
// streams are summed in fp64 (exact for fp32 inputs of similar magnitude),
// divided by hc in fp64 and rounded once to bf16, so the result is the
// correctly rounded mean; an fp32 sum would round first and flip a share of
// the bf16 casts that follow.
DEV u32x4 hc_mean8_bf16(const float* p, size_t ld, int hc) {
  u32x4 r;
  if (hc == 1) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    r[0] = pack_bf16x2(a[0], a[1]);
    r[1] = pack_bf16x2(a[2], a[3]);
    r[2] = pack_bf16x2(b[0], b[1]);
    r[3] = pack_bf16x2(b[2], b[3]);
    return r;
  }
  double s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0;
  for (int st = 0; st < hc; ++st) {
    const f32x4 a = *(const f32x4*)(p + (size_t)st * ld), b = *(const f32x4*)(p + (size_t)st * ld + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] += (double)a[i];
      s[4 + i] += (double)b[i];
    }
  }
  if ((hc & (hc - 1)) == 0) {
    // a power of two: 1/hc is exact, so the product is the quotient
    const double inv = 1.0 / (double)hc;
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] *= inv;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] /= (double)hc;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (uint32_t)f64_to_bf16bits(s[2 * i]) | ((uint32_t)f64_to_bf16bits(s[2 * i + 1]) << 16);
  return r;
}

// 16-byte loads. Weights stream through once per round: non-temporal so they do
// not evict activations, partial sums and the context ring from L2/MALL.
DEV u32x4 ld_nt16(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
DEV u32x4 ld16(const void* p) { return *(const u32x4*)p; }
DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

DEV f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// arr[i] for a block-uniform i < N, without dynamic indexing of a kernel argument
template <class T, int N>
DEV T pick(const T (&arr)[N], int i) {
  T r = arr[0];
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (i == j) r = arr[j];
  return r;
}

// Bits of the sticky device error word (the values of include/dflash.h).
constexpr unsigned ERR_BAD_TOKEN = 1u, ERR_BAD_WINDOW = 2u, ERR_BAD_ROW = 4u, ERR_BAD_POSITION = 8u,
                   ERR_RING_CAPACITY = 16u;

DEV void set_error(unsigned* err, unsigned bit) {
  if (err) atomicOr(err, bit);
}

// Request and absolute position of row m of a call that writes K/V rows into
// the ring (a tap stage, or a block's own rows): the request is req_of_row[m]
// or m / rows_per_req, the position pos_of_row[m] or pos[req] + m %
// rows_per_req. Returns 0, or the error bit of a row that must be skipped: a
// request outside [0, Rmax), a negative position, or a position whose ring
// slot holds another live row of the request. The live positions are the
// window and the block, [pos - W, pos + B) with C >= W + B, so a row at p may
// use slot p mod C only for p in [pos + B - C, pos + C - W).
// *rp is the position RoPE uses: the row's own, or pos[req] + rope_off[m] for a
// tree row, whose ring slot follows its row index but whose position is pos +
// its depth.
template <class A>
DEV unsigned ring_row(const A& a, int m, int* req, long long* p, long long* rp) {
  const int r = a.req_of_row ? a.req_of_row[m] : m / a.rows_per_req;
  *req = r;
  *p = -1;
  *rp = -1;
  if (r < 0 || r >= a.Rmax) return ERR_BAD_ROW;
  const long long base = a.pos[r];
  const long long q = a.pos_of_row ? (long long)a.pos_of_row[m] : base + m % a.rows_per_req;
  if (q < 0) return ERR_BAD_POSITION;
  if (q < base + a.B - a.C || q >= base + a.C - a.win) return ERR_RING_CAPACITY;
  *p = q;
  *rp = a.rope_off ? base + a.rope_off[m] : q;
  return 0u;
}

// INT4 weights (symmetric, groups of 64 along K, fp16 scales; the packing is
// described in gemm.hip): (128 + u_e, 128 + u_e+1) for the nibble pairs of one
// packed word.
// mask = 0x000F000F and bias = 0x43004300 come in registers (int4_unpack_consts):
// gfx950's three-operand v_and_or_b32 cannot encode two literals, so with the
// constants folded in the compiler spends an AND and an OR per pair.
DEV u32x4 int4_biased_bf16(uint32_t w, uint32_t mask, uint32_t bias) {
  u32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) r[t] = ((w >> (4 * t)) & mask) | bias;
  return r;
}
// the two constants of int4_biased_bf16 as register values the compiler cannot fold
DEV void int4_unpack_consts(uint32_t& mask, uint32_t& bias) {
  asm("v_mov_b32 %0, 0x000F000F" : "=v"(mask));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
}

DEV float half_bits_to_float(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }

// RoPE. The frequency of pair d, theta^(-2d/hd), is computed in fp64, and so is
// the angle p * freq; the angle is reduced to [-pi, pi] in fp64 (exact to
// ~1e-12 for positions in the millions) and its sine and cosine taken in fp32,
// which keeps them within about one fp32 ulp of the exact values.
DEV double rope_freq(int d, int hd, double log2_theta) { return exp2(-(double)(2 * d) / (double)hd * log2_theta); }
DEV void rope_cs(long long p, double freq, float* c, float* s) {
  const double a = (double)p * freq;
  const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
  sincosf((float)r, s, c);
}
DEV void rope_cos_sin(long long p, int d, int hd, double log2_theta, float* c, float* s) {
  rope_cs(p, rope_freq(d, hd, log2_theta), c, s);
}
