// Gate/up projection of the MLP sublayer in one launch for up to 16 rows:
// act = SiLU(x W_gate^T) * (x W_up^T), x the RMS-normed rows (bf16), act bf16.
// The drafter layer's MLP is the Qwen3 one (ExecuTorch PR #20840, "[RFC] DFlash",
// landing criteria, item 2: the draft layer reuses the Qwen3 RMSNorm and MLP).
//
// One workgroup of 2 NP waves per 16 NP output columns: waves 0..NP-1 stream
// the gate rows of W, waves NP..2NP-1 the matching up rows, each wave 16 rows
// over the whole of K. The normed rows are staged once in LDS (16 x K bf16); the weights
// go from HBM straight into a per-wave LDS ring of D slots of 4 KB, one
// 16-row x 128-column chunk per slot, with nontemporal direct-to-LDS loads of
// 4 rows x 256 B per instruction (whole 128-byte lines). The ring layout is
// swizzled through the piece each lane fetches (row r's 16-byte piece b at
// (r/4)*64 + (r%4)*16 + (b+r)%16), so the 16 lanes that read one piece index of
// 16 rows for an MFMA B fragment hit 16 different bank groups.
//
// A single workgroup per CU streams about 30-35 GB/s this way, so the ~200
// workgroups of a qwen3-sized gate/up move its weights about as fast as the
// split-K GEMM's 760, without the split partials' round trip through memory
// and the separate SiLU kernel.
//
// Rounding: the sums are formed exactly as the split-K GEMM and its finish
// kernel form them for the same split plan (ks columns per split): each split's
// chunks accumulate in one MFMA chain from zero, the split sums are added in
// split order starting from +0, and SiLU(g) * u is evaluated with the same
// expression. A row's result is therefore bit-identical on both paths, so it
// does not depend on how many rows share the call.
#include "norm_stage.h"

namespace {

// 3 wave pairs: ~200 workgroups at a qwen3-sized ffn keep more CUs streaming than
// 4 pairs' ~150 (measured 1.5-2 us faster per launch); a deeper ring measured no
// faster
constexpr int GU_PAIRS = 3;   // gate/up wave pairs per workgroup
constexpr int GU_DEPTH = 2;   // ring slots per wave
constexpr int GU_XP = 16;     // staged X pieces per thread
constexpr size_t GU_LDS_TOTAL = 160 * 1024;   // a workgroup's LDS, dynamic and static

template <int D>
DEV void wait_chunk_ring() {   // vmcnt <= 4 (D - 1): the oldest chunk has landed
  constexpr int n = 4 * (D - 1);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
DEV void wait_all_loads() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }   // vmcnt(0)

// LDS: the staged rows [16][K + 8] bf16, the gains (whole KB), then the rings
__host__ __device__ inline size_t gu_x_bytes(int K) { return norm_rows_bytes(K) + norm_gain_bytes(K); }

template <int NP, int D, int XP>
__global__ __launch_bounds__(128 * NP) void gateup_lds_kernel(const GemmArgs a) {
  constexpr int COLS = 16 * NP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, nchunks = K / 128, ldl = K + 8;
  const int split_chunks = a.ks / 128;
  uint16_t* xs = (uint16_t*)smem;
  const size_t ring_off = gu_x_bytes(K);
  char* ring = smem + ring_off + (size_t)wave * D * 4096;
  const uint16_t* W = (const uint16_t*)a.w;
  const bool is_up = wave >= NP;
  const int col0 = blockIdx.x * COLS + (wave - (is_up ? NP : 0)) * 16;   // this wave's first logical column
  const size_t row_add = is_up ? (size_t)a.pair_off : 0;

  // chunk c of this wave's 16 rows into ring slot `slot`: instruction s loads
  // rows 4s..4s+3, lane l taking piece (l - row) & 15 of row 4s + l/16
  auto issue = [&](int c, int slot) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = 4 * s + lg, kb = (lane - row) & 15;
      const uint16_t* src = W + ((size_t)min(col0 + row, a.N - 1) + row_add) * K + c * 128 + kb * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(ring + slot * 4096 + s * 1024), 16, 0, 2);
    }
  };
  // Prologue: the ring's first D chunks, then the normed rows' loads; one wait
  // covers all of them, about one HBM latency after the start.
#pragma unroll
  for (int j = 0; j < D; ++j) issue(j, j);
  uint16_t* gains = (uint16_t*)(smem + norm_rows_bytes(K));
  NormRowsLoads<XP, norm_sqp<128 * NP, 16>()> L;
  norm_rows_issue<128 * NP, XP>(a, 0, K, gains, L);
  norm_rows_store<128 * NP, XP>(a, K, gains, xs, ldl, L);

  // stream: chunk c's slot is read as 4 MFMA B fragments and refilled with
  // chunk c + D before they are used; a split's chain is added to the running
  // sum when it ends
  f32x4 tot = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f};
  int slot = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (c + D <= nchunks) wait_chunk_ring<D>();
    else wait_all_loads();
    const char* sl = ring + slot * 4096;
    u32x4 f[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int b = 4 * s2 + lg;
      f[s2] = *(const u32x4*)(sl + ((lr >> 2) * 64 + (lr & 3) * 16 + ((b + lr) & 15)) * 16);
    }
    // the slot's fragments are in registers: refill it before the MFMAs
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    if (c + D < nchunks) issue(c + D, slot);
    slot = slot + 1 == D ? 0 : slot + 1;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      acc = mfma16x16x32(as_bf16x8(*(const u32x4*)(xs + lr * ldl + 128 * c + 32 * s2 + 8 * lg)), as_bf16x8(f[s2]),
                         acc);
    if ((c + 1) % split_chunks == 0 || c + 1 == nchunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] = tot[i] + acc[i];
      acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }

  // lane holds C[4 lg + i][lr] of its wave's 16 columns; the up waves hand
  // theirs to the gate waves through LDS (the ring is dead once every wave
  // has passed the barrier: its last chunks waited for every load)
  __syncthreads();
  float* up = (float*)(smem + ring_off);   // [16][COLS]
  if (is_up) {
#pragma unroll
    for (int i = 0; i < 4; ++i) up[(4 * lg + i) * COLS + (wave - NP) * 16 + lr] = tot[i];
  }
  __syncthreads();
  if (!is_up) {
    const int n = col0 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * lg + i;
      if (m < a.M && n < a.N) {
        const float g = tot[i], u = up[m * COLS + wave * 16 + lr];
        ((uint16_t*)a.out)[(size_t)m * a.ldo + n] = f2bfbits(g / (1.0f + expf(-g)) * u);
      }
    }
  }
}

// The same one-launch gate/up with INT4 weights (symmetric, groups of 64
// along K, fp16 scales, packed as described in gemm.hip), for up to 16 rows.
// A wave's ring slot holds two 128-column chunks of its 16 rows: 16 x 128 B of
// packed values, loaded as whole 128-byte lines (two instructions of 8 rows),
// then the rows' 4 group scales (one 4-byte direct-to-LDS load). Row r's 16-byte
// piece p (chunk p / 4, lane group p % 4) sits at piece (r / 8) * 64 + (r % 8) * 8
// + (p + r + r / 8) % 8 of the slot, so the 16 lanes that read one piece index
// of 16 rows hit 16 different bank groups. With INT4 weights the normed rows
// are about as many bytes as a workgroup's weights, so only the rows below M
// are staged: 8 rows when M <= 8 (the A operand's rows 8..15 then repeat rows
// 0..7, and their results are never stored).
//
// Rounding: the split GEMM's, step for step. Each 64-group's two MFMAs start
// from zero (t = sum x (128 + u)), the group adds s * (t - 136 xs) with xs the
// group's sum of the staged bf16 values (each 8-value piece summed in order,
// then the 8 pieces of a group in a butterfly), each split (ks columns) starts
// its sum from zero, the split sums are added in split order from +0, and
// SiLU(g) * u is the finish kernel's expression: bit-identical results.
constexpr int GQ_PAIRS = 3;
constexpr int GQ_DEPTH = 5;                  // ring slots (2 chunks each) per wave: 10 KB in flight
constexpr int GQ_SLOT = 2048 + 256;          // packed values, then the scales
constexpr int GQ_PRO = 2;                    // units issued before the rows are staged
constexpr int gq_xp(int rx) { return rx == 8 ? 12 : 14; }   // staged X pieces per thread

// LDS: the staged rows [rx][K + 8] bf16, the gains, the group sums [K/64][rx], then the rings
__host__ __device__ inline size_t gq_xsum_offset(int K, int rx) { return norm_rows_bytes(K, rx) + norm_gain_bytes(K); }
__host__ __device__ inline size_t gq_ring_offset(int K, int rx) {
  return (gq_xsum_offset(K, rx) + (size_t)(K / 64) * rx * 4 + 15) & ~(size_t)15;
}

template <int n>
DEV void wait_vm_n() {   // vmcnt <= n
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int NP, int D, int RX, int XP>
__global__ __launch_bounds__(128 * NP) void gateup_q4_kernel(const GemmArgs a) {
  constexpr int COLS = 16 * NP, NT = 128 * NP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, nchunks = K / 128, nunits = nchunks / 2, ldl = K + 8;
  const int split_chunks = a.ks / 128;
  uint16_t* xs = (uint16_t*)smem;
  uint16_t* gains = (uint16_t*)(smem + norm_rows_bytes(K, RX));
  float* xsum = (float*)(smem + gq_xsum_offset(K, RX));
  const size_t ring_off = gq_ring_offset(K, RX);
  char* ring = smem + ring_off + (size_t)wave * D * GQ_SLOT;
  const bool is_up = wave >= NP;
  const int col0 = blockIdx.x * COLS + (wave - (is_up ? NP : 0)) * 16;   // this wave's first logical column
  const size_t row_add = is_up ? (size_t)a.pair_off : 0;
  const uint8_t* Wq = (const uint8_t*)a.w;
  const size_t rowb = (size_t)K / 2, rows_s = (size_t)K / 64;   // packed bytes, scales per W row

  // slot unit v (chunks 2v, 2v + 1) into ring slot `slot`: instruction t loads
  // rows 8t..8t+7, lane l fetching piece (l % 8 - r - t) % 8 of row 8t + l / 8;
  // lane l of the scale load takes the two scales of chunk 2v + l % 2 of row
  // (l / 2) % 16 (lanes 32..63 repeat 0..31)
  auto issue = [&](int v, int slot) {
    char* sb = ring + slot * GQ_SLOT;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 8 * t + (lane >> 3);
      const int pc = ((lane & 7) - r - t) & 7;
      const uint8_t* src = Wq + ((size_t)min(col0 + r, a.N - 1) + row_add) * rowb + (size_t)v * 128 + pc * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(sb + t * 1024), 16, 0, 2);
    }
    const int rs = (lane >> 1) & 15;
    const uint16_t* ssrc = a.wscale + ((size_t)min(col0 + rs, a.N - 1) + row_add) * rows_s + 4 * v + 2 * (lane & 1);
    __builtin_amdgcn_global_load_lds((const void*)ssrc, (lds_void*)(sb + 2048), 4, 0, 2);
  };
  // Prologue: the ring's first GQ_PRO units, then the normed rows' loads (one
  // wait covers all of them: the compiler waits for every direct-to-LDS load
  // before a register load's value is used), then the rest of the ring, which
  // lands while the first units are processed. A smaller first burst lands sooner.
#pragma unroll
  for (int j = 0; j < GQ_PRO; ++j) issue(j, j);
  NormRowsLoads<XP, norm_sqp<NT, RX>()> L;
  norm_rows_issue<NT, XP, RX>(a, 0, K, gains, L);
  norm_rows_store<NT, XP, RX, true>(a, K, gains, xs, ldl, L, xsum);   // with the rows' 64-group sums
#pragma unroll
  for (int j = GQ_PRO; j < D; ++j) issue(j, j);

  uint32_t q4_mask, q4_bias;
  int4_unpack_consts(q4_mask, q4_bias);
  const int xrow = RX == 8 ? (lr & 7) : lr;   // A-operand row (rows 8..15 repeat 0..7 when 8 are staged)
  const int xg_row = (4 * lg) & (RX - 1);
  f32x4 tot = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f};
  int slot = 0;
  for (int v = 0; v < nunits; ++v) {
    if (v + D <= nunits) wait_vm_n<3 * (D - 1)>();
    else wait_vm_n<0>();
    const char* sb = ring + slot * GQ_SLOT;
    u32x4 wq[2];
    uint32_t scw[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int pc = 4 * cc + lg;
      wq[cc] = *(const u32x4*)(sb + ((lr >> 3) * 64 + (lr & 7) * 8 + ((pc + lr + (lr >> 3)) & 7)) * 16);
      scw[cc] = *(const uint32_t*)(sb + 2048 + (2 * lr + cc) * 4);
    }
    // the slot's values are in registers: refill it before the math
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    if (v + D < nunits) issue(v + D, slot);
    slot = slot + 1 == D ? 0 : slot + 1;
    // the unit's A operands and group sums in one LDS round trip, then the four
    // groups' MFMA pairs as independent chains, then the groups folded into the
    // running sum in order
    u32x4 xf[2][4];
    f32x4 xg[2][2], t[2][2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        xf[cc][s2] = *(const u32x4*)(xs + xrow * ldl + 128 * (2 * v + cc) + 32 * s2 + 8 * lg);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) xg[cc][gi] = *(const f32x4*)(xsum + (2 * (2 * v + cc) + gi) * RX + xg_row);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int s2 = 2 * gi + h;
          t[cc][gi] = mfma16x16x32(as_bf16x8(xf[cc][s2]), as_bf16x8(int4_biased_bf16(wq[cc][s2], q4_mask, q4_bias)),
                                   h ? t[cc][gi] : (f32x4){0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = 2 * v + cc;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float sc = half_bits_to_float(gi ? scw[cc] >> 16 : scw[cc] & 0xffffu);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, fmaf(-136.0f, xg[cc][gi][i], t[cc][gi][i]), acc[i]);
      }
      if ((c + 1) % split_chunks == 0 || c + 1 == nchunks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = tot[i] + acc[i];
        acc = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // the up waves hand their sums to the gate waves through LDS (the ring is
  // dead: the last units waited for every load)
  __syncthreads();
  float* up = (float*)(smem + ring_off);   // [16][COLS]
  if (is_up) {
#pragma unroll
    for (int i = 0; i < 4; ++i) up[(4 * lg + i) * COLS + (wave - NP) * 16 + lr] = tot[i];
  }
  __syncthreads();
  if (!is_up) {
    const int n = col0 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * lg + i;
      if (m < a.M && n < a.N) {
        const float g = tot[i], u = up[m * COLS + wave * 16 + lr];
        ((uint16_t*)a.out)[(size_t)m * a.ldo + n] = f2bfbits(g / (1.0f + expf(-g)) * u);
      }
    }
  }
}

}  // namespace

size_t gateup_lds_bytes(int M, int K) {
  // rows, whole chunks, a full ring, and one producer sum of squares per thread
  if (M < 1 || M > 16 || K / 128 < GU_DEPTH || !norm_rows_fit(K, K, 128 * GU_PAIRS, GU_XP)) return 0;
  const size_t b = gu_x_bytes(K) + (size_t)2 * GU_PAIRS * GU_DEPTH * 4096;
  return b + norm_sq_bytes(128 * GU_PAIRS, 16) <= GU_LDS_TOTAL ? b : 0;
}

hipError_t launch_gateup_lds(const GemmArgs& a, int ks, hipStream_t st) {
  const size_t lds = gateup_lds_bytes(a.M, a.K);
  if (!lds || ks < 128 || ks % 128 || a.pair_off < a.N || a.N < 1 || a.n_ssq < 1 || a.n_ssq > NORM_SSQ_MAX)
    return hipErrorInvalidValue;
  GemmArgs b = a;
  b.ks = ks;
  constexpr int cols = 16 * GU_PAIRS;
  hipLaunchKernelGGL((gateup_lds_kernel<GU_PAIRS, GU_DEPTH, GU_XP>), dim3((a.N + cols - 1) / cols), dim3(128 * GU_PAIRS), lds,
                     st, b);
  return hipGetLastError();
}

size_t gateup_q4_bytes(int M, int K) {
  // rows below M (8 or 16 staged), whole slot units, a full ring, one producer
  // sum of squares per thread
  if (M < 1 || M > 16 || K % 256 || K / 256 < GQ_DEPTH) return 0;
  const int rx = M <= 8 ? 8 : 16;
  if (!norm_rows_fit(K, K, 128 * GQ_PAIRS, gq_xp(rx), rx)) return 0;
  const size_t b = gq_ring_offset(K, rx) + (size_t)2 * GQ_PAIRS * GQ_DEPTH * GQ_SLOT;
  return b + norm_sq_bytes(128 * GQ_PAIRS, rx) <= GU_LDS_TOTAL ? b : 0;
}

hipError_t launch_gateup_q4(const GemmArgs& a, int ks, hipStream_t st) {
  const size_t lds = gateup_q4_bytes(a.M, a.K);
  if (!lds || ks < 128 || ks % 128 || a.pair_off < a.N || a.N < 1 || a.n_ssq < 1 || a.n_ssq > NORM_SSQ_MAX ||
      !a.wscale)
    return hipErrorInvalidValue;
  GemmArgs b = a;
  b.ks = ks;
  constexpr int cols = 16 * GQ_PAIRS;
  const dim3 grid((a.N + cols - 1) / cols);
  if (a.M <= 8)
    hipLaunchKernelGGL((gateup_q4_kernel<GQ_PAIRS, GQ_DEPTH, 8, gq_xp(8)>), grid, dim3(128 * GQ_PAIRS), lds, st, b);
  else
    hipLaunchKernelGGL((gateup_q4_kernel<GQ_PAIRS, GQ_DEPTH, 16, gq_xp(16)>), grid, dim3(128 * GQ_PAIRS), lds, st, b);
  return hipGetLastError();
}
