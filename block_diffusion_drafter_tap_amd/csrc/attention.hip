// Block attention for gfx950: every block query attends to the context window
// [lo, pos) and to all B block rows [pos, pos+B), with no mask inside (the block
// is bidirectional; a causal target's verify pass sets `causal`, and block row i
// then sees block rows j <= i only; a tree pass, causal = 2, lets row i see the
// block rows that are its ancestors in the candidate tree, itself included). Keys and values of both live in the per-request ring (the
// block's own K/V were written to slots pos..pos+B-1 by the QKV epilogue), so a
// query sees one contiguous position range [lo, pos+B).
//
// Workgroup = (key chunk, kv head, request, query-slot part) with HD/16 waves
// and 32 keys per wave (256-key chunks at head_dim 128). The G*B query slots of
// a kv head are split over `hs` workgroups when there would otherwise be fewer
// than 256 workgroups (each then stages only its slots' Q and P in LDS; the
// chunk's K/V are read by each part, from L2 after the first). Two phases with
// an exact softmax inside the chunk:
//  1. wave w takes the chunk's 32-key sub-tile w and computes S^T = K Q^T for
//     all G*B queries of the kv head's query-head group (MFMA, keys x queries,
//     Q staged once in LDS: the waves share it instead of each loading it).
//     The chunk max of every query comes from an LDS exchange between the
//     waves; the wave then forms P = 2^(S - M) in registers and parks it in
//     LDS as two bf16 terms (hi + lo keep ~16 significant bits).
//  2. wave w owns head_dim tile w: it accumulates O^T = V^T P^T over all the
//     chunk's sub-tiles (MFMA, head_dim x queries) and writes its rows of the
//     chunk partial straight from the accumulators.
// A wave's K loads are issued first and its V loads once its scores are formed
// (K lands sooner without V competing for HBM; V streams in during the
// softmax), and no wave holds more than one head_dim tile of O.
// The ring keeps V transposed ([hd][C]) so that both MFMA operands are 16-byte
// loads. Keys of the two 16-row S^T tiles are permuted so that after the first
// MFMA each lane group already holds the 8 consecutive keys the second MFMA
// needs as its k-values (no cross-lane shuffles between the two products).
//
// A second kernel combines the chunk partials in chunk order, so results do not
// depend on scheduling. Both kernels use a 1-D grid whose workgroup id is
// (chunk * hs + part) * (R*nkv) + (request, head): workgroups are dealt to the 8
// XCDs round robin, so with R*nkv a multiple of 8 every chunk and part of one
// head lands on the same XCD, and the combine reads its partials from that
// XCD's L2.
#include "device.h"
#include "kernels.h"

namespace {

struct Range {
  int lo, hi, base, n_ch, pos;
};

// [lo, hi): keys a block query sees; chunks of a.kc keys start at base = lo
// rounded down to 32.
DEV Range key_range(const AttnArgs& a, int r, bool report) {
  const int pos = a.pos[r];
  int vf = a.valid_from[r];
  if (vf > pos) {
    if (report) set_error(a.err, ERR_BAD_WINDOW);
    vf = pos;
  }
  int lo = pos - a.W;
  lo = lo > vf ? lo : vf;
  lo = lo > 0 ? lo : 0;
  Range g;
  g.pos = pos;
  g.lo = lo;
  g.hi = pos + a.B;
  g.base = lo & ~31;
  g.n_ch = (g.hi - g.base + a.kc - 1) / a.kc;
  return g;
}

template <int HD, int QT, int NWA>
__global__ __launch_bounds__(64 * NWA) void attn_kernel(const AttnArgs a) {
  constexpr int ATT_WAVES = NWA;
  constexpr int ATT_KC = 32 * NWA;         // keys per chunk
  constexpr int QS = HD / 32;              // MFMA k-steps along head_dim
  constexpr int HTW = HD / 16 / ATT_WAVES; // O^T head_dim tiles per wave
  constexpr int NSL = QT * 16;             // query slots (padded to whole tiles)
  static_assert(HTW >= 1, "at most HD/16 waves");
  __shared__ __attribute__((aligned(16))) uint16_t s_q[NSL][HD + 8];
  __shared__ float s_mx[ATT_WAVES][NSL], s_l[ATT_WAVES][NSL];
  // P of every sub-tile (hi and lo bf16 terms), up to 64 KB: dynamic LDS
  extern __shared__ __attribute__((aligned(16))) u32x4 s_pdyn[];
  u32x4 (*s_p)[QT][2][64] = (u32x4 (*)[QT][2][64])s_pdyn;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int RN = a.R * a.nkv;
  const int lrg = blockIdx.x % RN, rest = blockIdx.x / RN;
  const int hs = rest % a.hs, chunk = rest / a.hs;
  const int r = lrg / a.nkv, g = lrg % a.nkv;
  const int G = a.nq / a.nkv;
  const int slots = G * a.B;
  const int s0 = hs * NSL;                 // this workgroup's first query slot
  const int nsl = min(NSL, slots - s0);    // its query slots

  const Range kr = key_range(a, r, threadIdx.x == 0 && chunk == 0 && g == 0);
  if (chunk >= kr.n_ch) return;
  const int kb = kr.base + chunk * ATT_KC;

  const uint16_t* rk = a.ring_k + (size_t)lrg * a.C * HD;
  const uint16_t* rv = a.ring_v + (size_t)lrg * HD * a.C;

  // this wave's K loads first
  const int k0 = kb + 32 * wave;
  const bool live = k0 < kr.hi;
  u32x4 kf[2][QS];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = k0 + 8 * (lr >> 2) + 4 * kt + (lr & 3);
    const uint16_t* kp = rk + (size_t)(key % a.C) * HD + 8 * lg;
#pragma unroll
    for (int s = 0; s < QS; ++s) kf[kt][s] = live ? ld16(kp + 32 * s) : (u32x4){0u, 0u, 0u, 0u};
  }

  // Q of this workgroup's query slots (slot = h_local * B + i); zero rows pad the last tile
  for (int e = threadIdx.x; e < NSL * (HD / 8); e += blockDim.x) {
    const int ls = e / (HD / 8), c = e % (HD / 8);
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (ls < nsl) {
      const int slot = s0 + ls;
      const int hq = slot / a.B, iq = slot % a.B;
      v = ld16(a.q + ((size_t)r * a.B + iq) * a.nq * HD + (size_t)(g * G + hq) * HD + 8 * c);
    }
    *(u32x4*)&s_q[ls][8 * c] = v;
  }
  __syncthreads();

  // phase 1: scores of sub-tile `wave`; lane holds, for query slot qt*16 + lr,
  // keys k0 + 8*lg + e (e = 4*kt + i)
  float p[QT][8];
  // a tree pass: the ancestor mask of each of this lane's query rows
  unsigned long long anc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    anc[qt] = a.causal == 2 ? a.anc[(size_t)r * a.B + (s0 + qt * 16 + lr) % a.B] : 0ull;
  // no per-key mask needed: the sub-tile lies inside the window (and, for a
  // causal pass, before the block)
  const bool interior = k0 >= kr.lo && k0 + 32 <= (a.causal ? kr.pos : kr.hi);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int iq = (s0 + qt * 16 + lr) % a.B;   // block row of this lane's query slot
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s)
        acc = mfma16x16x32(as_bf16x8(kf[kt][s]), as_bf16x8(*(const u32x4*)&s_q[qt * 16 + lr][32 * s + 8 * lg]),
                           acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 8 * lg + 4 * kt + i;
        bool ok = interior || (key >= kr.lo && key < kr.hi);
        if (!interior && key >= kr.pos) {
          if (a.causal == 1) ok = ok && key <= kr.pos + iq;
          else if (a.causal == 2) ok = ok && ((anc[qt] >> (key - kr.pos)) & 1ull);
        }
        p[qt][4 * kt + i] = ok ? acc[i] * a.scale_log2 : -INFINITY;
      }
    }
    float mx = p[qt][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, p[qt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lg == 0) s_mx[wave][qt * 16 + lr] = mx;
  }
  // V only now, once this wave's K has landed: every workgroup issues its K and V
  // at the same moment, so K alone lands sooner and V streams in during the
  // softmax
  u32x4 vf[ATT_WAVES][HTW];
#pragma unroll
  for (int sb = 0; sb < ATT_WAVES; ++sb) {
    const int ks = kb + 32 * sb;
    const int vslot = (ks + 8 * lg) % a.C;
#pragma unroll
    for (int tt = 0; tt < HTW; ++tt) {
      const int t = wave * HTW + tt;
      vf[sb][tt] = ks < kr.hi ? ld16(rv + (size_t)(16 * t + lr) * a.C + vslot) : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int sl = qt * 16 + lr;
    float M = s_mx[0][sl];
#pragma unroll
    for (int w = 1; w < ATT_WAVES; ++w) M = fmaxf(M, s_mx[w][sl]);
    const float m_use = M == -INFINITY ? 0.f : M;
    float psum = 0.f;
    u32x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = exp2f(p[qt][2 * e] - m_use), p1 = exp2f(p[qt][2 * e + 1] - m_use);
      psum += p0 + p1;
      const float h0 = bf2f(f2bf(p0)), h1 = bf2f(f2bf(p1));
      ph[e] = pack_bf16x2(h0, h1);
      pl[e] = pack_bf16x2(p0 - h0, p1 - h1);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (lg == 0) s_l[wave][sl] = psum;
    s_p[wave][qt][0][lane] = ph;
    s_p[wave][qt][1][lane] = pl;
  }
  __syncthreads();

  // phase 2: O^T tiles of this wave's head_dim rows over the chunk's sub-tiles
  f32x4 o[QT][HTW];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int tt = 0; tt < HTW; ++tt) o[qt][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sb = 0; sb < ATT_WAVES; ++sb) {
    if (kb + 32 * sb >= kr.hi) break;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const bf16x8 ph = as_bf16x8(s_p[sb][qt][0][lane]), pl = as_bf16x8(s_p[sb][qt][1][lane]);
#pragma unroll
      for (int tt = 0; tt < HTW; ++tt) {
        o[qt][tt] = mfma16x16x32(as_bf16x8(vf[sb][tt]), ph, o[qt][tt]);
        o[qt][tt] = mfma16x16x32(as_bf16x8(vf[sb][tt]), pl, o[qt][tt]);
      }
    }
  }

  // chunk partial: O (relative to the chunk max M), M, L
  const size_t cbase = ((size_t)lrg * a.n_chunks + chunk) * slots + s0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int sl = qt * 16 + lr;
    if (sl < nsl) {
#pragma unroll
      for (int tt = 0; tt < HTW; ++tt)
        *(f32x4*)(a.part_o + (cbase + sl) * HD + 16 * (wave * HTW + tt) + 4 * lg) = o[qt][tt];
    }
  }
  for (int sl = threadIdx.x; sl < nsl; sl += blockDim.x) {
    float M = s_mx[0][sl], L = s_l[0][sl];
#pragma unroll
    for (int w = 1; w < ATT_WAVES; ++w) {
      M = fmaxf(M, s_mx[w][sl]);
      L += s_l[w][sl];
    }
    a.part_ml[(cbase + sl) * 2] = M;
    a.part_ml[(cbase + sl) * 2 + 1] = L;
  }
}

// Combine the chunk partials of one (request, kv head): O = sum_c w_c O_c with
// w_c = 2^(m_c - M) / sum_c 2^(m_c - M) l_c, in chunk order (up to 24 chunks
// from one batch of loads, more in batches of 8, with the same sums). Each thread owns
// four consecutive head_dim values of one query slot; workgroup id =
// part * (R*nkv) + (request, head), so each head's combine runs on the XCD that
// ran its chunks.
template <int HD>
__global__ __launch_bounds__(64) void attn_combine_kernel(const AttnArgs a) {
  constexpr int CB = 24;   // chunks combined from one batch of loads
  const int RN = a.R * a.nkv;
  const int lrg = blockIdx.x % RN, part = blockIdx.x / RN;
  const int r = lrg / a.nkv, g = lrg % a.nkv;
  const int G = a.nq / a.nkv, slots = G * a.B;
  const int e = part * 64 + threadIdx.x;   // float4 index within [slots][HD/4]
  if (e >= slots * HD / 4) return;
  const int s = e / (HD / 4), d4 = e % (HD / 4);
  const int n_ch = key_range(a, r, false).n_ch;
  const size_t c0 = (size_t)lrg * a.n_chunks * slots;
  const float2* ml = (const float2*)a.part_ml;
  float M = -INFINITY;
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (n_ch <= CB) {
    // every chunk's loads in one batch: one L2 round trip. The sums run in chunk
    // order over n_ch rounded up to 8 terms (zero-weight padding), the same
    // sequence as the batched loop below.
    float2 v[CB];
    f32x4 ov[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {   // a chunk index past the end re-reads the last chunk
      const size_t cs = c0 + (size_t)min(u, n_ch - 1) * slots + s;
      v[u] = ml[cs];
      ov[u] = *(const f32x4*)(a.part_o + cs * HD + 4 * d4);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (u >= n_ch) {
        v[u] = make_float2(-INFINITY, 0.f);
        ov[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int u = 0; u < CB; ++u) M = fmaxf(M, v[u].x);
    const int terms = (n_ch + 7) & ~7;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (u < terms) {
        const float wgt = v[u].x == -INFINITY ? 0.f : exp2f(v[u].x - M);
        L += wgt * v[u].y;
        acc += wgt * ov[u];
      }
    }
  } else {
    for (int c0i = 0; c0i < n_ch; c0i += 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = c0i + u < n_ch ? ml[c0 + (size_t)(c0i + u) * slots + s] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, v[u].x);
    }
    for (int c0i = 0; c0i < n_ch; c0i += 8) {
      float2 v[8];
      f32x4 ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = c0i + u < n_ch;
        const size_t cs = c0 + (size_t)(c0i + u) * slots + s;
        v[u] = ok ? ml[cs] : make_float2(-INFINITY, 0.f);
        ov[u] = ok ? *(const f32x4*)(a.part_o + cs * HD + 4 * d4) : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = v[u].x == -INFINITY ? 0.f : exp2f(v[u].x - M);
        L += wgt * v[u].y;
        acc += wgt * ov[u];
      }
    }
  }
  const float inv = 1.0f / L;
  const int hq = s / a.B, iq = s % a.B;
  uint16_t* op = a.out + ((size_t)r * a.B + iq) * a.nq * HD + (size_t)(g * G + hq) * HD + 4 * d4;
  u32x2 w;
  w[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)op = w;
}

template <int HD, int QT>
void launch_hd(const AttnArgs& a, hipStream_t st) {
  constexpr int NWA = HD / 16;   // one head_dim tile of O per wave in the P.V phase
  const int RN = a.R * a.nkv;
  const int slots = attn_slots(a.nq, a.nkv, a.B);
  const int parts = (slots * HD / 4 + 63) / 64;
  const size_t lds = (size_t)NWA * QT * 2 * 64 * sizeof(u32x4);
  hipLaunchKernelGGL((attn_kernel<HD, QT, NWA>), dim3(a.n_chunks * a.hs * RN), dim3(64 * NWA), lds, st, a);
  hipLaunchKernelGGL((attn_combine_kernel<HD>), dim3(parts * RN), dim3(64), 0, st, a);
}

}  // namespace

int attn_slots(int nq, int nkv, int B) { return (nq / nkv) * B; }
int attn_chunk_keys(int hd) { return 32 * (hd / 16); }

hipError_t launch_attention(const AttnArgs& args, int R, hipStream_t st) {
  AttnArgs a = args;
  a.R = R;
  const int slots = attn_slots(a.nq, a.nkv, a.B);
  const int qt_all = (slots + 15) / 16;
  // query-slot split: few (chunk, kv head) workgroups leave CUs idle and every
  // wave reads all of a workgroup's Q and P from LDS, so split the query tiles
  // over up to qt_all workgroups until there are at least 256 (measured: 512 is slower)
  int hs = 1;
  while (hs < qt_all && (long long)a.n_chunks * R * a.nkv * hs < 256) hs *= 2;
  if (hs > qt_all) hs = qt_all;
  a.hs = hs;
  const int qt = (qt_all + hs - 1) / hs;
  if (qt > 4 || a.kc != attn_chunk_keys(a.hd)) return hipErrorInvalidValue;   // <= 64 query slots per kv head
#define QTS(HD)                                  \
  switch (qt) {                                  \
    case 1: launch_hd<HD, 1>(a, st); break;   \
    case 2: launch_hd<HD, 2>(a, st); break;   \
    case 3: launch_hd<HD, 3>(a, st); break;   \
    default: launch_hd<HD, 4>(a, st); break;  \
  }
  if (a.hd == 128) { QTS(128) }
  else if (a.hd == 64) { QTS(64) }
  else return hipErrorInvalidValue;
#undef QTS
  return hipGetLastError();
}
