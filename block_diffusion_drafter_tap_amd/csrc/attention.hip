// Block attention for gfx950: every block query attends to the context window
// [lo, pos) and to all B block rows [pos, pos+B), with no mask inside (the block
// is bidirectional). Keys and values of both live in the per-request ring (the
// block's own K/V were written to slots pos..pos+B-1 by the QKV epilogue), so a
// query sees one contiguous position range [lo, pos+B).
//
// Workgroup = (key chunk, kv head, request). Its waves hold the G*B queries of
// the kv head's query-head group, 16 per wave (one MFMA tile). Per 32-key
// sub-tile a wave computes S^T = K Q^T (MFMA, keys x queries), runs the online
// softmax in registers, and accumulates O^T = V^T P^T (MFMA, head_dim x queries,
// with P split into two bf16 terms).
// The ring keeps V transposed ([hd][C]) so that both MFMA operands are 16-byte
// loads. Keys of the two 16-row S^T tiles are permuted so that after the first
// MFMA each lane group already holds the 8 consecutive keys the second MFMA
// needs as its k-values (no cross-lane shuffles between the two products).
//
// Chunks of one (request, kv head) write partial (max, sum, O) to scratch and a
// second kernel combines them in chunk order, so results do not depend on
// scheduling.
#include "device.h"
#include "kernels.h"

namespace {

constexpr int HD_MAX = 128;

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int HT = HD / 16;   // O^T tiles along head_dim
  constexpr int QS = HD / 32;   // MFMA k-steps along head_dim

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int chunk = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int nwaves = blockDim.x >> 6;
  const int G = a.nq / a.nkv;
  const int slots = G * a.B;

  int pos = a.pos[r], vf = a.valid_from[r];
  if (vf > pos) {
    if (threadIdx.x == 0 && chunk == 0 && g == 0) set_error(a.err, 2u);
    vf = pos;
  }
  int lo = pos - a.W;
  lo = lo > vf ? lo : vf;
  lo = lo > 0 ? lo : 0;
  const int hi = pos + a.B;
  const int base = lo & ~31;
  const int n_ch = (hi - base + a.kc - 1) / a.kc;
  if (chunk >= n_ch) return;
  const int kb = base + chunk * a.kc;
  const int ke = min(kb + a.kc, hi);

  const size_t lrg = (size_t)r * a.nkv + g;
  const uint16_t* rk = a.ring_k + lrg * (size_t)a.C * HD;
  const uint16_t* rv = a.ring_v + lrg * (size_t)HD * a.C;

  // this wave's 16 query slots; slot = h_local * B + i
  const int slot = wave * 16 + lr;
  const bool qvalid = slot < slots;
  const int hq = qvalid ? slot / a.B : 0, iq = qvalid ? slot % a.B : 0;
  const uint16_t* qrow = a.q + ((size_t)r * a.B + iq) * a.nq * HD + (size_t)(g * G + hq) * HD;
  bf16x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    u32x4 v = ld16(qrow + 32 * s + 8 * lg);
    if (!qvalid) v = (u32x4){0u, 0u, 0u, 0u};
    qf[s] = as_bf16x8(v);
  }

  f32x4 o[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) o[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // K / V fragments of one 32-key sub-tile; the next sub-tile's are loaded
  // while the current one is computed.
  u32x4 kA[2][QS], vA[HT], kB[2][QS], vB[HT];
  auto load = [&](int k0, u32x4 (&kf)[2][QS], u32x4 (&vf)[HT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = k0 + 8 * (lr >> 2) + 4 * kt + (lr & 3);
      const uint16_t* kp = rk + (size_t)(key % a.C) * HD + 8 * lg;
#pragma unroll
      for (int s = 0; s < QS; ++s) kf[kt][s] = ld16(kp + 32 * s);
    }
    const int vslot = (k0 + 8 * lg) % a.C;
#pragma unroll
    for (int t = 0; t < HT; ++t) vf[t] = ld16(rv + (size_t)(16 * t + lr) * a.C + vslot);
  };
  auto compute = [&](int k0, const u32x4 (&kf)[2][QS], const u32x4 (&vf)[HT]) {
    // S^T for keys k0 + 8*(rr/4) + 4*kt + rr%4 (rr = row of the tile)
    f32x4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s) acc = mfma16x16x32(as_bf16x8(kf[kt][s]), qf[s], acc);
      sc[kt] = acc;
    }
    // lane holds, for query lr, keys k0 + 8*lg + e (e = 4*kt + i)
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 8 * lg + 4 * kt + i;
        const bool ok = key >= lo && key < hi;
        const float v = ok ? sc[kt][i] * a.scale_log2 : -INFINITY;
        p[4 * kt + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(p[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P enters the MFMA as two bf16 terms, P = hi + lo (about 16 significant
    // bits), so the probabilities are not rounded to 8 bits.
    u32x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h0 = bf2f(f2bf(p[2 * e])), h1 = bf2f(f2bf(p[2 * e + 1]));
      ph[e] = pack_bf16x2(h0, h1);
      pl[e] = pack_bf16x2(p[2 * e] - h0, p[2 * e + 1] - h1);
    }
    const bf16x8 pf_hi = as_bf16x8(ph), pf_lo = as_bf16x8(pl);
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      o[t] *= alpha;
      o[t] = mfma16x16x32(as_bf16x8(vf[t]), pf_hi, o[t]);
      o[t] = mfma16x16x32(as_bf16x8(vf[t]), pf_lo, o[t]);
    }
  };
  load(kb, kA, vA);
  for (int k0 = kb; k0 < ke; k0 += 64) {
    const bool more = k0 + 32 < ke;
    if (more) load(k0 + 32, kB, vB);
    compute(k0, kA, vA);
    if (!more) break;
    if (k0 + 64 < ke) load(k0 + 64, kA, vA);
    compute(k0 + 32, kB, vB);
  }
  // full softmax denominator of query lr: sum over the four lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // partial state of this chunk: o[t][i] = O^T[hd = 16t + 4*lg + i][query lr]
  const size_t cbase = (lrg * a.n_chunks + chunk) * (size_t)slots;
  if (qvalid) {
    float* po = a.part_o + (cbase + slot) * HD;
#pragma unroll
    for (int t = 0; t < HT; ++t) *(f32x4*)(po + 16 * t + 4 * lg) = o[t];
    if (lg == 0) {
      a.part_ml[(cbase + slot) * 2] = m_run;
      a.part_ml[(cbase + slot) * 2 + 1] = l_run;
    }
  }
  (void)nwaves;
}

// Combine the chunk partials of one (request, kv head): O = sum_c w_c O_c with
// w_c = 2^(m_c - M) / sum_c 2^(m_c - M) l_c, in chunk order. Each thread owns
// four consecutive head_dim values of one query slot.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  const int lrg = blockIdx.x;
  const int r = lrg / a.nkv, g = lrg % a.nkv;
  const int G = a.nq / a.nkv, slots = G * a.B;
  const int e = blockIdx.y * blockDim.x + threadIdx.x;   // float4 index within [slots][HD/4]
  if (e >= slots * HD / 4) return;
  const int s = e / (HD / 4), d4 = e % (HD / 4);
  int pos = a.pos[r], vf = a.valid_from[r];
  vf = vf > pos ? pos : vf;
  int lo = pos - a.W;
  lo = lo > vf ? lo : vf;
  lo = lo > 0 ? lo : 0;
  const int base = lo & ~31;
  const int n_ch = (pos + a.B - base + a.kc - 1) / a.kc;
  const size_t c0 = (size_t)lrg * a.n_chunks * slots;
  const float2* ml = (const float2*)a.part_ml;
  float M = -INFINITY;
  for (int c0i = 0; c0i < n_ch; c0i += 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0i + u < n_ch ? ml[c0 + (size_t)(c0i + u) * slots + s] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, v[u].x);
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
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
      const float wgt = exp2f(v[u].x - M);
      L += wgt * v[u].y;
      acc += wgt * ov[u];
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

}  // namespace

int attn_slots(int nq, int nkv, int B) { return (nq / nkv) * B; }

hipError_t launch_attention(const AttnArgs& a, int R, hipStream_t st) {
  const int slots = attn_slots(a.nq, a.nkv, a.B);
  const int waves = (slots + 15) / 16;
  if (waves > 4 || a.kc % 64) return hipErrorInvalidValue;   // <= 64 query slots per kv head
  const dim3 grid(a.n_chunks, a.nkv, R), block(64 * waves);
  const dim3 cgrid(R * a.nkv, (slots * a.hd / 4 + 255) / 256);
  if (a.hd == 128) {
    hipLaunchKernelGGL((attn_kernel<128>), grid, block, 0, st, a);
    hipLaunchKernelGGL((attn_combine_kernel<128>), cgrid, dim3(256), 0, st, a);
  } else if (a.hd == 64) {
    hipLaunchKernelGGL((attn_kernel<64>), grid, block, 0, st, a);
    hipLaunchKernelGGL((attn_combine_kernel<64>), cgrid, dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
