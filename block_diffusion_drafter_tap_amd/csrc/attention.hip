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
// Chunks of one (request, kv head) write partial (max, sum, O) to scratch; the
// last one to finish combines them in chunk order, so results do not depend on
// scheduling.
#include "device.h"
#include "kernels.h"

namespace {

constexpr int HD_MAX = 128;

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int HT = HD / 16;   // O^T tiles along head_dim
  constexpr int QS = HD / 32;   // MFMA k-steps along head_dim
  __shared__ float s_m[64], s_l[64];
  __shared__ int last_flag;

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

  for (int k0 = kb; k0 < ke; k0 += 32) {
    // S^T for keys k0 + 8*(rr/4) + 4*kt + rr%4 (rr = row of the tile)
    f32x4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = k0 + 8 * (lr >> 2) + 4 * kt + (lr & 3);
      const uint16_t* kp = rk + (size_t)(key % a.C) * HD + 8 * lg;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s) acc = mfma16x16x32(as_bf16x8(ld16(kp + 32 * s)), qf[s], acc);
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
    // bits): a single bf16 rounding of the probabilities would move the output
    // by far more than every other rounding of the layer together.
    u32x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h0 = bf2f(f2bf(p[2 * e])), h1 = bf2f(f2bf(p[2 * e + 1]));
      ph[e] = pack_bf16x2(h0, h1);
      pl[e] = pack_bf16x2(p[2 * e] - h0, p[2 * e + 1] - h1);
    }
    const bf16x8 pf_hi = as_bf16x8(ph), pf_lo = as_bf16x8(pl);
    const int vslot = (k0 + 8 * lg) % a.C;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      o[t] *= alpha;
      const bf16x8 vf8 = as_bf16x8(ld16(rv + (size_t)(16 * t + lr) * a.C + vslot));
      o[t] = mfma16x16x32(vf8, pf_hi, o[t]);
      o[t] = mfma16x16x32(vf8, pf_lo, o[t]);
    }
  }
  // full softmax denominator of query lr: sum over the four lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // o[t][i] = O^T[hd = 16t + 4*lg + i][query lr]
  if (n_ch == 1) {
    if (qvalid) {
      const float inv = 1.0f / l_run;
      uint16_t* op = a.out + ((size_t)r * a.B + iq) * a.nq * HD + (size_t)(g * G + hq) * HD;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        u32x2 v;
        v[0] = pack_bf16x2(o[t][0] * inv, o[t][1] * inv);
        v[1] = pack_bf16x2(o[t][2] * inv, o[t][3] * inv);
        *(u32x2*)(op + 16 * t + 4 * lg) = v;
      }
    }
    return;
  }

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
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counters[lrg], 1u);
    const int last = prev == (unsigned)(n_ch - 1);
    if (last) atomicExch(&a.counters[lrg], 0u);
    last_flag = last;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  const size_t c0 = lrg * a.n_chunks * (size_t)slots;
  for (int s = threadIdx.x; s < slots; s += blockDim.x) {
    float M = -INFINITY;
    for (int c = 0; c < n_ch; ++c) M = fmaxf(M, __builtin_nontemporal_load(a.part_ml + (c0 + (size_t)c * slots + s) * 2));
    float L = 0.f;
    for (int c = 0; c < n_ch; ++c) {
      const float mc = __builtin_nontemporal_load(a.part_ml + (c0 + (size_t)c * slots + s) * 2);
      const float lc = __builtin_nontemporal_load(a.part_ml + (c0 + (size_t)c * slots + s) * 2 + 1);
      L += exp2f(mc - M) * lc;
    }
    s_m[s] = M;
    s_l[s] = 1.0f / L;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < slots * HD; e += blockDim.x) {
    const int s = e / HD, d = e % HD;
    const float M = s_m[s];
    float acc = 0.f;
    for (int c = 0; c < n_ch; ++c) {
      const size_t cs = c0 + (size_t)c * slots + s;
      const float mc = __builtin_nontemporal_load(a.part_ml + cs * 2);
      acc += exp2f(mc - M) * __builtin_nontemporal_load(a.part_o + cs * HD + d);
    }
    const int hq2 = s / a.B, iq2 = s % a.B;
    a.out[((size_t)r * a.B + iq2) * a.nq * HD + (size_t)(g * G + hq2) * HD + d] = f2bfbits(acc * s_l[s]);
  }
  (void)nwaves;
}

}  // namespace

int attn_slots(int nq, int nkv, int B) { return (nq / nkv) * B; }

hipError_t launch_attention(const AttnArgs& a, int R, hipStream_t st) {
  const int slots = attn_slots(a.nq, a.nkv, a.B);
  const int waves = (slots + 15) / 16;
  if (waves > 4) return hipErrorInvalidValue;   // <= 64 query slots per kv head
  const dim3 grid(a.n_chunks, a.nkv, R), block(64 * waves);
  if (a.hd == 128) hipLaunchKernelGGL((attn_kernel<128>), grid, block, 0, st, a);
  else if (a.hd == 64) hipLaunchKernelGGL((attn_kernel<64>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
