// Shared LM head for gfx950: logits of the block's mask rows, then top-k.
//
// lm_logits_kernel: logits = W_lm z for every block row, z = RMSNorm(h; final
// gain) rounded to bf16. Persistent: workgroup w streams column groups w,
// w + P, ... of 128 vocabulary rows with 8 waves (one 16-row W tile each).
// The normed rows are staged in LDS once (all loads of a batch in flight
// together), W chunks of 128 k-values run D deep across group boundaries, and
// there is no barrier in the streaming loop. Each wave's fp32 tiles wait in LDS
// and are stored after its last weight load has been issued (as many groups as
// the LDS left over holds).
//
// The logits kernel also writes, per mask row, the max of every 16-column group.
// topk_rows_kernel: per row, an exact radix select picks the k best groups by
// their max, and the k best of those groups' logits are ranked directly.
// Selecting after streaming keeps the dependent cross-lane work of a running
// top-k out of the weight stream, where it stalled the loads.

#include <algorithm>

#include "norm_stage.h"

namespace {

// stage the normed rows in LDS up to this size (one persistent workgroup per
// CU, so nearly all of the 160 KB of a gfx950 CU)
constexpr size_t LM_XL_MAX_BYTES = 159 * 1024;
constexpr size_t LM_LDS_TOTAL = 160 * 1024;   // a workgroup's LDS, dynamic and static

// The final-normed rows as bf16 for the path that does not stage them in LDS,
// with the staging's arithmetic (sums of squares added in column-group order,
// the same normalize-and-round per 8 values), so a row's logits do not depend
// on how many rows share the launch.
__global__ __launch_bounds__(256) void lm_norm_rows_kernel(const GemmArgs a, uint16_t* z) {
  __shared__ float s_inv;
  const int m = blockIdx.x;
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int g = 0; g < a.n_ssq; ++g) ss += a.ssq_in[(size_t)g * a.ssq_ld + m];
    s_inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
  }
  __syncthreads();
  const float inv = s_inv;
  for (int c = threadIdx.x; c < a.K / 8; c += blockDim.x) {
    const float* p = a.xf + (size_t)m * a.ldx + 8 * c;
    *(u32x4*)(z + (size_t)m * a.K + 8 * c) =
        norm8(*(const f32x4*)p, *(const f32x4*)(p + 4), ld16(a.xgain + 8 * c), inv);
  }
}

// Logits: the caller's layout [R*(B-1)][N] (mask rows only), or the transposed
// scratch layout [N][16*MT] (every row), where a wave's 16 columns x 16 rows of a
// tile are one contiguous 1 KB store. The 16 lanes of a lane group also reduce
// their row's max over the wave's 16 columns (one entry per 16-column group, for
// the top-k filter).
template <int MT>
DEV void lm_epilogue(const GemmArgs& a, int grp16, const f32x4 (&ac)[MT], float* logits, int transposed,
                     float* gmax) {
  constexpr int ROWS = MT * 16;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n = grp16 * 16 + lr;   // this wave's 16 columns are grp16's
  const int ng = (a.N + 15) / 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (transposed && n < a.N) *(f32x4*)(logits + (size_t)n * ROWS + mt * 16 + 4 * lg) = ac[mt];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * lg + i;
      const int bi = m % a.B, r0 = a.lm_first_row;
      const bool row_ok = m < a.M && bi >= r0;
      const size_t orow = (size_t)((m / a.B) * (a.B - r0) + bi - r0);
      if (!transposed && row_ok && n < a.N) logits[orow * a.N + n] = ac[mt][i];
      float v = n < a.N ? ac[mt][i] : -INFINITY;
      v = fmaxf(v, __shfl_xor(v, 1, 64));
      v = fmaxf(v, __shfl_xor(v, 2, 64));
      v = fmaxf(v, __shfl_xor(v, 4, 64));
      v = fmaxf(v, __shfl_xor(v, 8, 64));
      if (row_ok && lr == 0 && grp16 < ng) gmax[orow * ng + grp16] = v;
    }
  }
}

template <int MT, int XL, int D>
__global__ __launch_bounds__(512) void lm_logits_kernel(const GemmArgs a, int n_groups, float* logits, int transposed,
                                                        float* gmax, int nslots, int defer_off) {
  constexpr int NW = 8, GC = 128, ROWS = MT * 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_inv[ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, nchunks = K / 128, ldl = K + 8;
  uint16_t* xs = (uint16_t*)smem;
  // accumulator fragments of this workgroup's first nslots groups, [slot][wave][mt][lane]
  f32x4* dslot = (f32x4*)(smem + defer_off);

  // W chunks stream D deep: chunk c of a group lives in buffer c % D (D divides
  // the chunk count); the last D buffers of a group are refilled with the next
  // group's first chunks
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

  for (int r = threadIdx.x; r < (XL == 1 ? ROWS : 0); r += blockDim.x) {
    const int m = min(r, a.M - 1);
    float ss = 0.f;
    for (int b0 = 0; b0 < a.n_ssq; b0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.ssq_in[(size_t)min(b0 + u, a.n_ssq - 1) * a.ssq_ld + m];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < a.n_ssq) ss += v[u];
    }
    s_inv[r] = 1.0f / sqrtf(ss / (float)K + a.eps);
  }
  __syncthreads();
  if (XL == 1) {
    // 8 vectors of a thread in flight per batch
    const int per_row = K / 8, total = ROWS * per_row;
    for (int e0 = threadIdx.x; e0 < total; e0 += 8 * blockDim.x) {
      f32x4 h0[8], h1[8];
      u32x4 gg[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = min(e0 + u * (int)blockDim.x, total - 1);
        const int r = e / per_row, c = e % per_row;
        const float* p = a.xf + (size_t)min(r, a.M - 1) * a.ldx + 8 * c;
        h0[u] = *(const f32x4*)p;
        h1[u] = *(const f32x4*)(p + 4);
        gg[u] = ld16(a.xgain + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * (int)blockDim.x;
        if (e < total) {
          const int r = e / per_row, c = e % per_row;
          *(u32x4*)(xs + r * ldl + 8 * c) = norm8(h0[u], h1[u], gg[u], s_inv[r]);
        }
      }
    }
    __syncthreads();
  }
  // XL == 2: the normed bf16 rows (a.x, written beforehand) pass through LDS in
  // windows of D chunks, double-buffered: the 8 waves share one copy, the next
  // window's loads are in flight while the current one is used, and one barrier
  // per window separates them (D divides the chunk count)
  constexpr int WK = 128 * D, WLD = WK + 8;
  constexpr int WPT = XL == 2 ? ROWS * WK / 8 / 512 : 1;   // 16-byte pieces per thread per window
  static_assert(XL != 2 || (WPT >= 1 && ROWS * WK / 8 == WPT * 512), "a window is whole pieces of every thread");
  const int nwin = nchunks / D;
  u32x4 xr[WPT];
  auto wload = [&](int w) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int p = threadIdx.x + i * 512, r = p / (WK / 8), c = p % (WK / 8);
      xr[i] = ld16(a.x + (size_t)min(r, a.M - 1) * a.ldx + w * WK + 8 * c);
    }
  };
  auto wstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int p = threadIdx.x + i * 512, r = p / (WK / 8), c = p % (WK / 8);
      *(u32x4*)(xs + ((size_t)b * ROWS + r) * WLD + 8 * c) = xr[i];
    }
  };
  int wb = 0;   // LDS buffer of the current window
  if constexpr (XL == 2) {
    wload(0);
    wstore(0);
    __syncthreads();
  }
  // kk: offset inside the K range; kl: offset inside the current window
  auto xfrag = [&](int mt, int kk, int kl) -> u32x4 {
    if constexpr (XL == 1) return *(const u32x4*)(xs + (mt * 16 + lr) * ldl + kk + 8 * lg);
    if constexpr (XL == 2) return *(const u32x4*)(xs + ((size_t)wb * ROWS + mt * 16 + lr) * WLD + kl + 8 * lg);
    // rows too many for LDS and K not a multiple of the window: straight from L2
    return ld16(a.x + (size_t)min(mt * 16 + lr, a.M - 1) * a.ldx + kk + 8 * lg);
  };

  auto epilogue = [&](int gg, const f32x4 (&ac)[MT]) {
    lm_epilogue<MT>(a, gg * (GC / 16) + wave, ac, logits, transposed, gmax);
  };

  for (; g < n_groups; g += gridDim.x) {
    const int gnext = g + gridDim.x;
    const bool has_next = gnext < n_groups;
    const uint16_t* wnext = has_next ? rowp(gnext) : wcur;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nchunks; c0 += D) {
      if constexpr (XL == 2) wload((c0 / D + 1) % nwin);   // the next window (window 0 of the next group at the end)
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int c = c0 + j;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = mfma16x16x32(as_bf16x8(xfrag(mt, 128 * c + 32 * s, 128 * j + 32 * s)), as_bf16x8(wbuf[j][s]),
                                   acc[mt]);
        const int nc = c + D;
        if (nc < nchunks) load_w(wcur, nc, wbuf[j]);
        else if (has_next) load_w(wnext, nc - nchunks, wbuf[j]);
      }
      if constexpr (XL == 2) {
        wstore(wb ^ 1);
        __syncthreads();
        wb ^= 1;
      }
    }
    wcur = wnext;
    // A store here would hold up the next group's weight loads: vector loads and
    // stores share one in-order counter, so every later load wait would include
    // the store's write acknowledgement. The first nslots groups therefore park
    // their fragments in LDS, and their epilogues run after the last load.
    const int gi = (g - (int)blockIdx.x) / (int)gridDim.x;
    if (gi < nslots) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) dslot[((size_t)(gi * NW + wave) * MT + mt) * 64 + lane] = acc[mt];
    } else {
      epilogue(g, acc);
    }
  }
  for (int gi = 0; gi < nslots; ++gi) {
    const int gg = (int)blockIdx.x + gi * (int)gridDim.x;
    if (gg >= n_groups) break;
    f32x4 ac[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ac[mt] = dslot[((size_t)(gi * NW + wave) * MT + mt) * 64 + lane];
    epilogue(gg, ac);
  }
}

// W through LDS (one tile of up to 16 rows, the normed rows staged in LDS whole
// or a phase of K columns at a time; 8 staged rows when the call has at most 8,
// so that a wider hidden size still fits in one phase; more than 16 rows go to
// lm_logits_dma_kernel): every weight load is a
// direct-to-LDS, nontemporal 16-byte load, and one load instruction covers 4
// whole W rows x 256 bytes, so the 128-byte lines of the stream are each read
// by one instruction. (The MFMA operand pattern, 16 rows x 64 bytes per
// instruction, leaves every line to two instructions; read nontemporally it
// fell to 4.8 TB/s against 7.0 for whole lines, in a bare-load probe on this
// grid.) A wave's 16-row x 128-k chunk is one 4 KB LDS slot, D slots per wave.
// In the slot, W row r's k-block b (8 values) sits at piece
// (r / 4) * 64 + (r % 4) * 16 + ((b + r) % 16): load instruction s fills pieces
// 64s .. 64s + 63 with rows 4s .. 4s + 3, and the MFMA B fragment of step s2
// (lane L: row L % 16, k-block 4 s2 + L / 16) reads 16 lanes' pieces from 16
// distinct bank groups. The loads write LDS behind the compiler's back, so
// the wait for a slot is an explicit vmcnt: the only vector memory operations
// in the streaming loop are these loads (4 per chunk), with D chunks in flight
// (after the last group's last refill, a wait is for every load).
// Work is dealt out in 16-row tiles of W (T of them), wave w of workgroup b (of
// P) taking tiles base + i * stride below an end, so the 8 waves of a workgroup
// are always on 128 adjacent rows:
//   by 128-row groups  base 8 b + w, stride 8 P, end T: groups b, b + P, ...,
//                      every wave of a workgroup the same count of tiles;
//   contiguous         base b T / P + w, stride 8, end (b + 1) T / P: one
//                      workgroup per CU, each CU 37 or 38 tiles of the qwen3
//                      vocabulary where groups give 238 CUs 40 and the rest none.
// Measured on the qwen3 vocabulary: with 5 KB rows (hidden 2560) groups are
// faster (127.5 against 129.7 us; the waves' unequal counts leave a tail), with
// 8 KB rows (hidden 4096) the contiguous ranges (214.8 -> 206.6 us).
// Each wave's accumulators of its (at most lm_lds_max_groups) tiles stay in
// registers until the last load is out, so no store interleaves with the
// stream. A tile's MFMA inputs and their order equal lm_logits_kernel's, so the
// logits are the same bit for bit.
constexpr int LM_LDS_MAX_GROUPS = 8;
// groups per workgroup the LDS kernel parks in registers: fewer with more row tiles
constexpr int lm_lds_max_groups(int MT) { return MT == 1 ? LM_LDS_MAX_GROUPS : 5; }
constexpr int LM_LDS_DEPTH = 2;   // W chunks in flight per wave (measured in the probe: 2 as fast as 3 or 4)
constexpr int LM_LDS_XP = 10;     // staged X pieces per thread

template <int D>
DEV void wait_w_chunk() {   // vmcnt <= 4 (D - 1); expcnt and lgkmcnt not waited for
  constexpr int n = 4 * (D - 1);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, int KPH, int RX>
__global__ __launch_bounds__(512) void lm_logits_lds_kernel(const GemmArgs a, int n_tiles, int contig,
                                                            float* logits, int transposed, float* gmax, int w_off) {
  // one 16-row tile, of which RX rows (8 or 16) are staged: with 8, the A
  // operand's rows 8..15 repeat rows 0..7 and their logits are never read
  constexpr int MT = 1, ROWS = RX, kph = KPH, MAXG = lm_lds_max_groups(MT);
  static_assert(RX == 8 || RX == 16, "8 or 16 staged rows");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, kw = K / kph, npc = kw / 128, ldl = kw + 8;
  uint16_t* xs = (uint16_t*)smem;
  uint16_t* gains = (uint16_t*)(smem + norm_rows_bytes(kw, ROWS));
  char* wring = smem + w_off + (size_t)wave * D * 4096;
  const uint16_t* W = (const uint16_t*)a.w;
  auto issue = [&](int t, int c, int slot) {   // chunk c of tile t (W rows 16 t .. 16 t + 15)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = 4 * s + lg, kb = (lane - row) & 15;
      const uint16_t* src = W + (size_t)min(t * 16 + row, a.N - 1) * K + c * 128 + kb * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(wring + slot * 4096 + s * 1024), 16, 0, 2);
    }
  };
  // this wave's tiles: t0, t0 + step, ... below t_end
  const int P = gridDim.x, b = blockIdx.x;
  const int step = contig ? 8 : 8 * P;
  const int t0 = (contig ? (int)((long long)b * n_tiles / P) : 8 * b) + wave;
  const int t_end = contig ? (int)((long long)(b + 1) * n_tiles / P) : n_tiles;
  f32x4 park[MAXG][MT];
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) park[gi][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // K in kph phases of kw columns: each phase stages its columns of the normed
  // rows and streams every group's chunks of those columns; a group's chain of
  // MFMAs runs over the chunks in order across the phases, and a row's chain does
  // not depend on the other row tiles, so its logits are the same bits for any MT
#pragma unroll
  for (int ph = 0; ph < kph; ++ph) {
    const int cb = ph * npc;   // first chunk of the phase
    // the first group's first D chunks of the phase, then the rows' loads; one
    // wait covers all of them (the previous phase ended with every load landed,
    // and the staging's first barrier follows every wave's last read of xs)
    if (t0 < t_end) {
#pragma unroll
      for (int j = 0; j < D; ++j) issue(t0, cb + j, j);
    }
    NormRowsLoads<LM_LDS_XP, norm_sqp<512, ROWS>()> L;
    norm_rows_issue<512, LM_LDS_XP, ROWS>(a, ph * kw, kw, gains, L);
    norm_rows_store<512, LM_LDS_XP, ROWS>(a, kw, gains, xs, ldl, L);
    int slot = 0;
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi) {
      const int g = t0 + gi * step;
      if (g < t_end) {
        const int gn = g + step;
        const bool last = gn >= t_end;   // no refills past its end: its last D - 1 chunks wait for every load
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = park[gi][mt];
        for (int c = 0; c < npc; ++c) {
          if (last && c > npc - D) __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
          else wait_w_chunk<D>();
          const char* sl = wring + slot * 4096;
          u32x4 f[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const int b = 4 * s2 + lg;
            f[s2] = *(const u32x4*)(sl + ((lr >> 2) * 64 + (lr & 3) * 16 + ((b + lr) & 15)) * 16);
          }
          // the slot's fragments are in registers: refill it before the MFMAs, so
          // a slot turns over in one load latency, not that plus the chunk's math
          __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
          const int nc = c + D;
          if (nc < npc) issue(g, cb + nc, slot);
          else if (!last) issue(gn, cb + nc - npc, slot);
          slot = slot + 1 == D ? 0 : slot + 1;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt] = mfma16x16x32(as_bf16x8(*(const u32x4*)(xs + (lr & (RX - 1)) * ldl + 128 * c + 32 * s2 + 8 * lg)),
                                     as_bf16x8(f[s2]), acc[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) park[gi][mt] = acc[mt];
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = t0 + gi * step;
    if (g < t_end) lm_epilogue<MT>(a, g, park[gi], logits, transposed, gmax);
  }
}

template <int n>
DEV void wait_vm() {   // vmcnt <= n (n < 64); expcnt and lgkmcnt not waited for
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
// A workgroup barrier without the fence of __syncthreads, whose release waits
// for every direct-to-LDS load in flight (here: the W ring's next chunks). The
// caller has waited for the loads whose LDS data the other waves read after it,
// and its own LDS reads before it have completed (their values were used). The
// memory clobber keeps the compiler from moving memory accesses across it.
DEV void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// W through LDS as above, for 17..64 rows (MT = 2 or 4 row tiles). The rows are
// the final-normed bf16 rows z (written beforehand by lm_norm_rows_kernel, whose
// bits equal the staging's), and go from L2 straight into LDS as well, in MFMA
// operand order: K is taken in phases of NPC chunks, and a phase's rows are 4 MT
// NPC fragments of 1 KB, fragment (c * 4 + s2) * MT + mt holding rows mt * 16 +
// (0..15) x columns 32 s2 + (0..31) of chunk c with lane L's 16 bytes at 16 L
// (row L % 16, columns 8 (L / 16) + (0..7)), so an A-operand read is one linear
// 1 KB read per wave. Two phase buffers: the next phase's rows are loaded while
// this phase streams, and each wave's W ring runs on across the phase
// boundaries, where the workgroup only meets at a barrier. Every wave's
// sequence of W chunks runs over (phase, group, chunk); the rows of phase p + 1
// are issued at the first chunk of phase p, just before that chunk's refill,
// so the wait of the next chunk allows for them. A row's chain of MFMAs runs
// over the chunks in order, with the same inputs as the 16-row kernels, so its
// logits are the same bits for any number of rows.
template <int MT, int NPC>
__global__ __launch_bounds__(512) void lm_logits_dma_kernel(const GemmArgs a, int n_groups, float* logits,
                                                            int transposed, float* gmax) {
  constexpr int D = 2, GC = 128, NF = 4 * MT * NPC, NXW = NF / 8, MAXG = lm_lds_max_groups(MT);
  static_assert(NF % 8 == 0 && NPC >= D, "whole fragments per wave; a group spans at least D chunks per phase");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, nph = K / (128 * NPC);
  char* wring = smem + 2 * NF * 1024 + (size_t)wave * D * 4096;
  const uint16_t* W = (const uint16_t*)a.w;
  auto issue_w = [&](int gg, int c, int slot) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = 4 * s + lg, kb = (lane - row) & 15;
      const uint16_t* src = W + (size_t)min(gg * GC + wave * 16 + row, a.N - 1) * K + c * 128 + kb * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(wring + slot * 4096 + s * 1024), 16, 0, 2);
    }
  };
  auto issue_x = [&](int ph, int b) {   // this wave's NXW fragments of phase ph into buffer b
#pragma unroll
    for (int j = 0; j < NXW; ++j) {
      const int f = wave * NXW + j;
      const int mt = f % MT, s2 = (f / MT) % 4, cl = f / (4 * MT);
      const uint16_t* src = a.x + (size_t)min(mt * 16 + lr, a.M - 1) * a.ldx + 128 * (ph * NPC + cl) + 32 * s2 + 8 * lg;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(smem + ((size_t)b * NF + f) * 1024), 16, 0, 0);
    }
  };
  const int g0 = blockIdx.x, P = gridDim.x;
  f32x4 park[MAXG][MT];
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) park[gi][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // phase 0's rows, then the first D chunks; the rows land first
  issue_x(0, 0);
#pragma unroll
  for (int j = 0; j < D; ++j) issue_w(g0, j, j);
  wait_vm<4 * D>();
  barrier_no_fence();
  int slot = 0;
  for (int ph = 0; ph < nph; ++ph) {
    const bool more = ph + 1 < nph;
    const char* xb = smem + (size_t)(ph & 1) * NF * 1024;
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi) {
      const int g = g0 + gi * P;
      if (g < n_groups) {
        const bool gnext = g + P < n_groups;
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = park[gi][mt];
#pragma unroll
        for (int c = 0; c < NPC; ++c) {
          // this chunk's loads were followed by the next chunk's (if any) and,
          // at the second chunk of a phase, by the next phase's rows
          if (!more && !gnext && c == NPC - 1) wait_vm<0>();
          else if (more && gi == 0 && c == 1) wait_vm<4 + NXW>();
          else wait_vm<4>();
          const char* sl = wring + slot * 4096;
          u32x4 f[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const int b = 4 * s2 + lg;
            f[s2] = *(const u32x4*)(sl + ((lr >> 2) * 64 + (lr & 3) * 16 + ((b + lr) & 15)) * 16);
          }
          __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0): the slot is free
          if (more && gi == 0 && c == 0) issue_x(ph + 1, (ph + 1) & 1);
          // the chunk D steps on: this group's, the next group's, or the next phase's first group's
          if (c + D < NPC) issue_w(g, ph * NPC + c + D, slot);
          else if (gnext) issue_w(g + P, ph * NPC + c + D - NPC, slot);
          else if (more) issue_w(g0, (ph + 1) * NPC + c + D - NPC, slot);
          slot ^= 1;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt] = mfma16x16x32(as_bf16x8(*(const u32x4*)(xb + (((c * 4 + s2) * MT + mt) * 64 + lane) * 16)),
                                     as_bf16x8(f[s2]), acc[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) park[gi][mt] = acc[mt];
      }
    }
    if (more) {
      // the next phase's rows were followed by at least one refill (4 loads):
      // they have landed; after the barrier no wave reads this phase's buffer
      wait_vm<4>();
      barrier_no_fence();
    }
  }
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = g0 + gi * P;
    if (g < n_groups) lm_epilogue<MT>(a, g * (GC / 16) + wave, park[gi], logits, transposed, gmax);
  }
}

// Order-preserving key of an fp32 value (larger value -> larger key; -0 maps to
// +0; NaN ordered above +inf, never produced by the logits).
DEV unsigned fkey(float v) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;   // -0 and +0 compare equal (ties go by index)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact top-k (k <= 16) by (key desc, index asc) over the block's values: thread t
// holds the PER keys of indices [t*PER, t*PER + cnt) (contiguous, in index
// order). Radix select on 8-bit digits finds the k-th key P; every key above P is
// taken, and of the keys equal to P the lowest indices fill the rest. Writes the k
// selected (key, index) pairs to sel_key/sel_idx (unordered). 256 threads.
template <int PER>
DEV void block_select(const unsigned (&key)[PER], int cnt, int base_idx, int k, unsigned* sel_key, int* sel_idx,
                      unsigned* hist, int* scratch) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  unsigned prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (j < cnt && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l; an inclusive scan over lanes counts
      // the keys at or above each lane's lowest digit
      unsigned c[4], s4 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        s4 += c[q];
      }
      unsigned incl = s4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
      }
      const unsigned long long hit = __ballot(incl >= (unsigned)need);
      const int L = (int)__builtin_ctzll(hit);   // first lane reaching need (exists: need <= count)
      if (lane == L) {
        unsigned above = incl - s4;
        int d = 255 - 4 * lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + c[q] >= (unsigned)need) { d = 255 - 4 * lane - q; break; }
          above += c[q];
        }
        scratch[0] = d;
        scratch[1] = (int)above;
      }
    }
    __syncthreads();
    const int d = scratch[0];
    need -= scratch[1];
    prefix |= (unsigned)d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // keys above P: k - need of them, any order
  if (t == 0) scratch[2] = 0;
  int eq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) eq += (j < cnt && key[j] == prefix) ? 1 : 0;
  // exclusive scan of the per-thread counts of keys equal to P (index order)
  int incl = eq;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) scratch[4 + wave] = incl;
  __syncthreads();
  int before = incl - eq;
  for (int w = 0; w < wave; ++w) before += scratch[4 + w];
  const int n_above = k - need;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j >= cnt) continue;
    if (key[j] > prefix) {
      const int slot = atomicAdd(&scratch[2], 1);
      sel_key[slot] = key[j];
      sel_idx[slot] = base_idx + j;
    } else if (key[j] == prefix) {
      if (before < need) {
        sel_key[n_above + before] = key[j];
        sel_idx[n_above + before] = base_idx + j;
      }
      ++before;
    }
  }
  __syncthreads();
}

// Within one wave: the k-th largest (1 <= k <= number of valid entries) of up
// to 256 keys, four per lane (entry lane + 64q). Bitwise radix select with
// ballots: at each bit, the keys that match the decided high bits and have the
// bit set are counted; if they are enough the k-th largest has the bit set,
// else they all rank above it.
DEV unsigned wave_kth_largest(const unsigned (&key)[4], const bool (&valid)[4], int k) {
  unsigned prefix = 0;
  int need = k;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned cand = prefix | (1u << bit);
    const unsigned hi = ~((1u << bit) - 1u);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt += __popcll(__ballot(valid[q] && (key[q] & hi) == cand));
    if (cnt >= need) prefix = cand;
    else need -= cnt;
  }
  return prefix;
}

// Per mask row: T = the k-th best per-thread maximum of the 16-column group
// maxima (a wave radix select); every group reaching T is a candidate, a
// superset of the k best groups, since at least k groups reach T. A top-k logit
// always lies in a top-k group under (max desc, group asc), because groups are
// contiguous index ranges. The candidates' logits (at most 512; otherwise the
// exact top-k groups from a block radix select) are ranked by counting. Output
// sorted by (value desc, index asc). The row's group maxima are staged in
// dynamic LDS.
// logits element (row r, column n): caller layout logits[r * N + n], or the
// transposed scratch logits[n * cs + srow], srow = req*B + i for r = req*(B-r0) + i - r0
// (output rows are the block rows i >= r0: the mask rows for drafts, r0 = 1;
// every row for a verify pass, r0 = 0).
template <int PER>
__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ logits, long long cs, int B, int r0,
                                                        int transposed, const float* __restrict__ gmax, int N, int k,
                                                        int* ids, float* vals) {
  extern __shared__ __attribute__((aligned(16))) float s_g[];   // [ng]
  __shared__ unsigned hist[256];
  __shared__ int scratch[8];
  __shared__ unsigned sel_key[16];
  __shared__ int sel_idx[16];
  __shared__ unsigned cand_k[256];
  __shared__ int cand_i[256];
  __shared__ unsigned s_tmax[256];
  // candidate logits as (key << 32 | ~index): one unsigned compare orders them
  // by (value desc, index asc)
  __shared__ __attribute__((aligned(16))) unsigned long long cb[512];
  __shared__ unsigned long long cf[512];   // the candidates at or above T
  __shared__ int s_nf;                      // their count
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ng = (N + 15) / 16;
  const float* gm = gmax + (size_t)row * ng;
  if (t == 0) {
    scratch[3] = 0;
    s_nf = 0;
  }
  // thread t owns groups t + 256*j: coalesced loads, all in flight together
  float gv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) gv[j] = gm[min(t + 256 * j, ng - 1)];
  unsigned key[PER];
  unsigned tmax = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    key[j] = t + 256 * j < ng ? fkey(gv[j]) : 0u;
    tmax = key[j] > tmax ? key[j] : tmax;
  }
  s_tmax[t] = tmax;
  __syncthreads();
  const int kg = min(k, ng);   // fewer groups than k: all of them
  // T = the kg-th best per-thread maximum: at least kg groups reach it, so every
  // top-kg group does
  if (wave == 0) {
    unsigned q4[4];
    bool v4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      q4[q] = s_tmax[lane + 64 * q];
      v4[q] = true;
    }
    const unsigned T = wave_kth_largest(q4, v4, kg);
    if (lane == 0) scratch[2] = (int)T;
  }
  __syncthreads();
  const unsigned T = (unsigned)scratch[2];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (t + 256 * j < ng && key[j] >= T) {
      const int slot = atomicAdd(&scratch[3], 1);
      if (slot < 256) {
        cand_k[slot] = key[j];
        cand_i[slot] = t + 256 * j;
      }
    }
  }
  __syncthreads();
  const int n_cand = scratch[3];
  // candidate groups: all groups reaching T when their logits fit (a superset
  // of the top-kg groups), else exactly the top-kg groups (radix select)
  int n_groups_c;
  const int* gsel;
  if (n_cand * 16 <= 512) {
    n_groups_c = n_cand;
    gsel = cand_i;
  } else {
    // ties defeat the filter: exact radix select over contiguous group ranges
    // (thread t owns groups [t*PER, t*PER + cnt)), staged through LDS
    for (int j0 = t; j0 < ng; j0 += 256) s_g[j0] = gm[j0];
    __syncthreads();
    const int g0 = t * PER;
    const int cnt = max(0, min(PER, ng - g0));
    unsigned kc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) kc[j] = j < cnt ? fkey(s_g[min(g0 + j, ng - 1)]) : 0u;
    block_select<PER>(kc, cnt, g0, kg, sel_key, sel_idx, hist, scratch);
    n_groups_c = kg;
    gsel = sel_idx;
  }
  // stage B: the logits of the candidate groups, ranked by counting
  const int nc = 16 * n_groups_c;
  const size_t srow = transposed ? (size_t)(row / (B - r0) * B + row % (B - r0) + r0) : (size_t)row;
  for (int e = t; e < nc; e += 256) {
    const int n = 16 * gsel[e / 16] + (e % 16);
    const int nn = min(n, N - 1);
    const float v = transposed ? logits[(size_t)nn * cs + srow] : logits[srow * N + nn];
    // past the vocabulary: key 0 (below every logit's key), distinct per slot
    cb[e] = n < N ? ((unsigned long long)fkey(v) << 32) | (unsigned)~n : (unsigned long long)e;
  }
  __syncthreads();
  // Every top-k logit's key reaches T (at least k logits, the group maxima that
  // made T, do), so only the candidates at or above T are ranked: ranks counted
  // within that set are the exact ranks of its best k. With fewer groups than k
  // every candidate is ranked. The set's order in LDS depends on the atomics;
  // the ranks do not.
  const unsigned Tf = kg < k ? 0u : T;
  for (int e = t; e < nc; e += 256) {
    const unsigned long long c = cb[e];
    if ((unsigned)(c >> 32) >= Tf) cf[atomicAdd(&s_nf, 1)] = c;
  }
  __syncthreads();
  const int nf = s_nf;
  for (int e = t; e < nf; e += 256) {
    const unsigned long long c = cf[e];
    int rank = 0;
    for (int j = 0; j < nf; ++j) rank += cf[j] > c ? 1 : 0;
    if (rank < k) {
      ids[(size_t)row * k + rank] = (int)~(unsigned)c;
      if (vals) {
        const unsigned kk = (unsigned)(c >> 32);
        const unsigned u = (kk & 0x80000000u) ? (kk & 0x7fffffffu) : ~kk;   // inverse of fkey
        vals[(size_t)row * k + rank] = __uint_as_float(u);
      }
    }
  }
}

template <int MT, int XL>
hipError_t launch_lm(const GemmArgs& a, const LmPlan& p, float* logits, int tr, float* gmax, hipStream_t st) {
  const int groups = p.groups, P = p.P, ns = p.slots, doff = p.defer_off;
  const size_t lds = p.lds;
  const int nchunks = a.K / 128;
  if constexpr (XL == 2) {   // windows of 4 chunks
    if (nchunks % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((lm_logits_kernel<MT, XL, 4>), dim3(P), dim3(512), lds, st, a, groups, logits, tr, gmax, ns,
                         doff);
  } else {
    if (nchunks % 4 == 0)
      hipLaunchKernelGGL((lm_logits_kernel<MT, XL, 4>), dim3(P), dim3(512), lds, st, a, groups, logits, tr, gmax, ns,
                         doff);
    else if (nchunks % 2 == 0)
      hipLaunchKernelGGL((lm_logits_kernel<MT, XL, 2>), dim3(P), dim3(512), lds, st, a, groups, logits, tr, gmax, ns,
                         doff);
    else
      hipLaunchKernelGGL((lm_logits_kernel<MT, XL, 1>), dim3(P), dim3(512), lds, st, a, groups, logits, tr, gmax, ns,
                         doff);
  }
  return hipGetLastError();
}

}  // namespace

LmPlan plan_lmhead(int M, int B, int V, int K, int n_cu) {
  LmPlan p;
  p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.groups = (V + 127) / 128;
  const int per = (p.groups + n_cu - 1) / n_cu;
  p.P = (p.groups + per - 1) / per;
  const int rows = 16 * p.MT;
  const size_t xbytes = (size_t)rows * (K + 8) * 2;            // the whole normed rows
  const size_t wbytes = (size_t)2 * rows * (4 * 128 + 8) * 2;  // two windows of 4 chunks
  p.XL = xbytes <= LM_XL_MAX_BYTES ? 1 : (K % 512 == 0 && wbytes <= LM_XL_MAX_BYTES ? 2 : 0);
  // 17..64 rows: normed bf16 rows and W both straight into LDS (XL 4), in phases
  // of npc chunks (the largest that divides K / 128, at most 48 KB of rows each)
  if (p.MT > 1 && K % 128 == 0 && per <= lm_lds_max_groups(p.MT)) {
    const int nch = K / 128;
    for (int npc = p.MT == 4 ? 2 : 5; npc >= (p.MT == 4 ? 2 : 4); --npc)
      if (nch % npc == 0) {
        p.XL = 4;
        p.kph = nch / npc;
        p.slots = 0;
        p.defer_off = 0;
        p.lds = (size_t)2 * 4 * p.MT * npc * 1024 + (size_t)8 * LM_LDS_DEPTH * 4096;
        return p;
      }
  }
  // one row tile (8 of its rows staged when the call has at most 8) with its
  // gains in 1 or 2 phases of K, with room for the W slots: W through LDS (XL 3)
  const int rx = M <= 8 ? 8 : 16;
  // 16-row W tiles dealt by 128-row groups (P as above), or as contiguous ranges
  // of one workgroup per CU when W rows are 8 KB or longer (measured)
  const int tiles = (V + 15) / 16, contig = K >= 4096 ? 1 : 0;
  const int pt = contig ? std::min(n_cu, tiles) : p.P;
  for (int kph = 1; p.MT == 1 && kph <= 2 && tiles <= 8 * pt * lm_lds_max_groups(1); kph *= 2) {
    if (K % kph) break;
    const int kw = K / kph;
    const size_t xoff = norm_rows_bytes(kw, rx) + norm_gain_bytes(kw);
    if (norm_rows_fit(K, kw, 512, LM_LDS_XP, rx) && kw / 128 >= LM_LDS_DEPTH &&
        xoff + (size_t)8 * LM_LDS_DEPTH * 4096 + norm_sq_bytes(512, rx) <= LM_LDS_TOTAL) {
      p.XL = 3;
      p.P = pt;
      p.contig = contig;
      p.rx = rx;
      p.kph = kph;
      p.defer_off = (int)xoff;   // the W slots
      p.slots = 0;
      p.lds = xoff + (size_t)8 * LM_LDS_DEPTH * 4096;
      return p;
    }
  }
  p.lds = p.XL == 1 ? xbytes : (p.XL == 2 ? wbytes : 0);
  // LDS left over holds the deferred accumulator fragments (8 waves x MT x 1 KB per group)
  p.defer_off = (int)((p.lds + 15) & ~(size_t)15);
  const size_t slot_bytes = (size_t)8 * p.MT * 64 * 16;
  const size_t room = LM_XL_MAX_BYTES > (size_t)p.defer_off ? LM_XL_MAX_BYTES - p.defer_off : 0;
  p.slots = (int)std::min<size_t>((size_t)per, room / slot_bytes);
  if (p.slots > 0) p.lds = p.defer_off + p.slots * slot_bytes;
  return p;
}

hipError_t launch_lm_norm_rows(const GemmArgs& a, uint16_t* z, hipStream_t st) {
  if (a.K % 8 || a.M < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lm_norm_rows_kernel, dim3(a.M), dim3(256), 0, st, a, z);
  return hipGetLastError();
}

hipError_t launch_lm_logits(const GemmArgs& a, const LmPlan& p, float* logits, int transposed, float* gmax,
                            hipStream_t st) {
  if (a.lm_first_row < 0 || a.lm_first_row > 1 || a.B < a.lm_first_row + 1) return hipErrorInvalidValue;
  if (p.XL == 3) {
    if (p.MT != 1 || (p.rx != 8 && p.rx != 16) || p.kph < 1 || a.K % p.kph ||
        !norm_rows_fit(a.K, a.K / p.kph, 512, LM_LDS_XP, p.rx) || a.K / p.kph / 128 < LM_LDS_DEPTH ||
        a.M > p.rx || a.n_ssq < 1 || a.n_ssq > NORM_SSQ_MAX || p.P < 1 ||
        (long long)8 * p.P * lm_lds_max_groups(1) < (a.N + 15) / 16)
      return hipErrorInvalidValue;
#define LMLDS(KPH, RX)                                                                                      \
  hipLaunchKernelGGL((lm_logits_lds_kernel<LM_LDS_DEPTH, KPH, RX>), dim3(p.P), dim3(512), p.lds, st, a, \
                     (a.N + 15) / 16, p.contig, logits, transposed, gmax, p.defer_off)
    if (p.kph == 1 && p.rx == 16) LMLDS(1, 16);
    else if (p.kph == 2 && p.rx == 16) LMLDS(2, 16);
    else if (p.kph == 1 && p.rx == 8) LMLDS(1, 8);
    else if (p.kph == 2 && p.rx == 8) LMLDS(2, 8);
    else return hipErrorInvalidValue;
#undef LMLDS
    return hipGetLastError();
  }
  if (p.XL == 4) {
    const int nch = a.K / 128, npc = p.kph > 0 ? nch / p.kph : 0;
    if (a.K % 128 || p.kph < 1 || nch % p.kph || a.M > 16 * p.MT || a.M < 1 || !a.x || a.ldx < a.K ||
        (long long)p.P * lm_lds_max_groups(p.MT) < p.groups)
      return hipErrorInvalidValue;
#define LMDMA(MT, NPC)                                                                                          \
  hipLaunchKernelGGL((lm_logits_dma_kernel<MT, NPC>), dim3(p.P), dim3(512), p.lds, st, a, p.groups, logits, \
                     transposed, gmax)
    if (p.MT == 4 && npc == 2) LMDMA(4, 2);
    else if (p.MT == 2 && npc == 4) LMDMA(2, 4);
    else if (p.MT == 2 && npc == 5) LMDMA(2, 5);
    else return hipErrorInvalidValue;
#undef LMDMA
    return hipGetLastError();
  }
  hipError_t e;
#define LM(MT)                                                                              \
  e = p.XL == 1   ? launch_lm<MT, 1>(a, p, logits, transposed, gmax, st) \
      : p.XL == 2 ? launch_lm<MT, 2>(a, p, logits, transposed, gmax, st) \
                  : launch_lm<MT, 0>(a, p, logits, transposed, gmax, st);
  switch (p.MT) {
    case 1: LM(1) break;
    case 2: LM(2) break;
    case 4: LM(4) break;
    default: return hipErrorInvalidValue;
  }
#undef LM
  return e;
}

hipError_t launch_lm_topk(const GemmArgs& a, const LmPlan& p, const float* logits, int transposed,
                          const float* gmax, int* ids, float* vals, hipStream_t st) {
  const int r0 = a.lm_first_row;
  if (a.topk < 1 || a.topk > 16 || r0 < 0 || r0 > 1 || a.B < r0 + 1) return hipErrorInvalidValue;
  const int rows = (a.M / a.B) * (a.B - r0);
  const int ng = (a.N + 15) / 16;
  if (ng > 256 * 64) return hipErrorInvalidValue;   // at most 64 groups per thread
  const long long cs = 16ll * p.MT;   // transposed scratch: [N][16*MT]
  const size_t lds = (size_t)ng * sizeof(float);
#define TK(PER) hipLaunchKernelGGL((topk_rows_kernel<PER>), dim3(rows), dim3(256), lds, st, logits, cs, a.B, r0, transposed, gmax, a.N, a.topk, ids, vals)
  if (ng <= 256 * 8) TK(8);
  else if (ng <= 256 * 16) TK(16);
  else if (ng <= 256 * 40) TK(40);
  else TK(64);
#undef TK
  return hipGetLastError();
}
