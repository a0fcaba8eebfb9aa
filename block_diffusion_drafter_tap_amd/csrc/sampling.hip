// Sampling-mode acceptance: typical acceptance of the drafts against the
// target's verify logits and card sampling (temperature, top-k, top-p) of the
// token after the accepted drafts, with a counter-based uniform draw. The pages
// run the drafter this way ("dflash: the chain verify builds pipelined ...",
// mlx-serve PR #937, "Measured": typical acceptance 0.2, T 1.0, top-p 0.95,
// top-k 20, a fixed seed) without formulas; the rule here:
//   p = softmax(z / T), H = -sum p log p over the vocabulary of a verify row;
//   the row's draft token d is accepted iff p(d) > min(eps, delta exp(-H));
//   acceptance stops at the first rejected row a (a = b - 1 if none);
//   the next token comes from row a: its top_k logits (value desc, index asc),
//   q = softmax(x) with x = z / T (fp64), the shortest prefix whose q sum
//   reaches top_p, and the first of them whose running q sum exceeds u times
//   the prefix's sum, u from Philox4x32-10 (Salmon et al., "Parallel random
//   numbers: as easy as 1, 2, 3", SC 2011) with key = seed, counter =
//   (round, request, a, 0), u = (word 0 >> 8) * 2^-24.
#include "device.h"
#include "kernels.h"

namespace {

// Order-preserving key of an fp32 value (-0 and +0 equal).
DEV unsigned order_key(float v) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

DEV float key_value(unsigned k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

DEV void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = (uint64_t)M0 * c[0], p1 = (uint64_t)M1 * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
  }
}

constexpr int TPB = 256;
constexpr int MAXK = 64;

// Top-K (K <= 64) of n keyed elements held in LDS, in (key desc, position asc)
// order: radix select of the K-th largest key over four 8-bit digits, then every
// key above it and the first `need` positions among the keys equal to it, then a
// rank by comparison. key(e) is the order key of element e, id(e) its token id;
// callers order positions so that equal keys come by ascending token id.
// Results: out_key[0..K), out_id[0..K) in LDS. Every thread of the block calls it.
template <class KeyF, class IdF>
DEV void block_topk(int n, int K, KeyF key, IdF id, unsigned* hist, int* sc, unsigned* cand_key, int* cand_id,
                    unsigned* out_key, int* out_id) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  unsigned prefix = 0, pmask = 0;
  int need = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
    for (int e = t; e < n; e += TPB) {
      const unsigned k = key(e);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255-4l .. 252-4l; inclusive scan from the top digit
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
      const int L = (int)__builtin_ctzll(hit);
      if (lane == L) {
        unsigned above = incl - s4;
        int dg = 255 - 4 * lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + c[q] >= (unsigned)need) {
            dg = 255 - 4 * lane - q;
            break;
          }
          above += c[q];
        }
        sc[0] = dg;
        sc[1] = (int)above;
      }
    }
    __syncthreads();
    prefix |= (unsigned)sc[0] << shift;
    pmask |= 255u << shift;
    need -= sc[1];
    __syncthreads();
  }
  // the last digit pass counted the keys equal to the K-th (hist[prefix & 255])
  const int n_above = K - need;
  const int n_eq = (int)hist[prefix & 255u];
  if (t == 0) sc[2] = 0;
  __syncthreads();
  if (n_eq == need) {
    for (int e = t; e < n; e += TPB) {
      const unsigned k = key(e);
      if (k >= prefix) {
        const int slot = atomicAdd(&sc[2], 1);
        cand_key[slot] = k;
        cand_id[slot] = id(e);
      }
    }
  } else {
    // more equal keys than places: thread t scans the positions [t*per, (t+1)*per)
    // and a prefix count over threads keeps the first `need` of them
    const int per = (n + TPB - 1) / TPB;
    const int e0 = min(n, t * per), e1 = min(n, e0 + per);
    int eq = 0;
    for (int e = e0; e < e1; ++e) eq += key(e) == prefix ? 1 : 0;
    int incl = eq;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    if (lane == 63) sc[4 + wave] = incl;
    __syncthreads();
    int before = incl - eq;
    for (int w = 0; w < wave; ++w) before += sc[4 + w];
    for (int e = e0; e < e1; ++e) {
      const unsigned k = key(e);
      if (k > prefix) {
        const int slot = atomicAdd(&sc[2], 1);
        cand_key[slot] = k;
        cand_id[slot] = id(e);
      } else if (k == prefix) {
        if (before < need) {
          cand_key[n_above + before] = k;
          cand_id[n_above + before] = id(e);
        }
        ++before;
      }
    }
  }
  __syncthreads();
  if (t < K) {
    const unsigned kt = cand_key[t];
    const int it = cand_id[t];
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += (cand_key[j] > kt || (cand_key[j] == kt && cand_id[j] < it)) ? 1 : 0;
    out_key[rank] = kt;
    out_id[rank] = it;
  }
  __syncthreads();
}

// Stage 1, one workgroup per (chunk c, row i, request r): the chunk of
// SAMPLE_CHUNK logits goes to LDS once; its max m_c, Z_c = sum exp(x), S_c =
// sum exp(x) x with x = (z - m_c) / T, and its top-K in (value desc, index asc).
__global__ __launch_bounds__(TPB) void sample_chunks_kernel(const SampleArgs a) {
  __shared__ float s_z[SAMPLE_CHUNK];
  __shared__ unsigned hist[256];
  __shared__ int s_sc[4 + TPB / 64];
  __shared__ unsigned s_ck[MAXK], s_ok[MAXK];
  __shared__ int s_ci[MAXK], s_oi[MAXK];
  __shared__ float s_red[TPB / 64];
  __shared__ double s_dred[2][TPB / 64];
  const int c = blockIdx.x, i = blockIdx.y, r = blockIdx.z, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V, S = a.n_chunks;
  const int e0 = c * SAMPLE_CHUNK, n = min(SAMPLE_CHUNK, V - e0);
  const size_t row = (size_t)r * a.b + i;
  const float* z = a.logits + row * V + e0;
  float mx = -INFINITY;
  for (int e = t; e < n; e += TPB) {
    const float v = z[e];
    s_z[e] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = s_red[0];
  for (int w = 1; w < TPB / 64; ++w) mx = fmaxf(mx, s_red[w]);
  const double invT = 1.0 / (double)a.T;
  double sz = 0.0, sx = 0.0;
  for (int e = t; e < n; e += TPB) {
    const float x = (float)(((double)s_z[e] - (double)mx) * invT);
    const float ex = expf(x);
    sz += (double)ex;
    sx += (double)ex * (double)x;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sz += __shfl_xor(sz, o, 64);
    sx += __shfl_xor(sx, o, 64);
  }
  if (lane == 0) {
    s_dred[0][wave] = sz;
    s_dred[1][wave] = sx;
  }
  const int K = min(a.top_k, n);
  block_topk(
      n, K, [&](int e) { return order_key(s_z[e]); }, [&](int e) { return e0 + e; }, hist, s_sc, s_ck, s_ci, s_ok,
      s_oi);
  const size_t part = row * S + c;
  if (t < K) {
    a.part_key[part * MAXK + t] = s_ok[t];
    a.part_idx[part * MAXK + t] = s_oi[t];
  }
  if (t == 0) {
    double Z = 0.0, Sx = 0.0;
    for (int w = 0; w < TPB / 64; ++w) {
      Z += s_dred[0][w];
      Sx += s_dred[1][w];
    }
    a.part_m[part] = mx;
    a.part_z[part] = Z;
    a.part_s[part] = Sx;
  }
}

// Stage 2, one workgroup per (row i, request r): the chunks' statistics merged
// at the row max M (Z = sum_c Z_c e^{(m_c - M)/T}, S = sum_c e^{(m_c - M)/T}
// (S_c + Z_c (m_c - M)/T), H = log Z - S / Z), the acceptance test of the row's
// draft token (rows i < b - 1), and the row's top-K from the chunks' lists (the
// lists are laid out by chunk, each in (value desc, index asc) order, so equal
// values come by ascending index).
__global__ __launch_bounds__(TPB) void sample_rows_kernel(const SampleArgs a) {
  __shared__ unsigned s_key[SAMPLE_MAX_CHUNKS * MAXK];
  __shared__ int s_idx[SAMPLE_MAX_CHUNKS * MAXK];
  __shared__ unsigned hist[256];
  __shared__ int s_sc[4 + TPB / 64];
  __shared__ unsigned s_ck[MAXK], s_ok[MAXK];
  __shared__ int s_ci[MAXK], s_oi[MAXK];
  const int i = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  const int V = a.V, S = a.n_chunks, K = min(a.top_k, V);
  const size_t row = (size_t)r * a.b + i;
  // every chunk but the last holds SAMPLE_CHUNK > 64 >= top_k logits, so chunk c's
  // list starts at c * top_k; the last one has min(top_k, its size) entries
  const int kc = a.top_k;
  const int n = (S - 1) * kc + min(kc, V - (S - 1) * SAMPLE_CHUNK);
  for (int e = t; e < n; e += TPB) {
    const int c = e / kc;
    const size_t src = (row * S + c) * MAXK + (e - c * kc);
    s_key[e] = a.part_key[src];
    s_idx[e] = a.part_idx[src];
  }
  if (t == 0 && i < a.b - 1) {
    float M = -INFINITY;
    for (int c = 0; c < S; ++c) M = fmaxf(M, a.part_m[row * S + c]);
    const double invT = 1.0 / (double)a.T;
    double Z = 0.0, Sx = 0.0;
    for (int c = 0; c < S; ++c) {
      const double sh = ((double)a.part_m[row * S + c] - (double)M) * invT;
      const double w = exp(sh), zc = a.part_z[row * S + c];
      Z += w * zc;
      Sx += w * (a.part_s[row * S + c] + zc * sh);
    }
    const double H = log(Z) - Sx / Z;
    const int d = a.draft[((size_t)r * (a.b - 1) + i) * a.draft_stride];
    int ok = 0;
    if (d >= 0 && d < V) {
      const double pd = exp(((double)a.logits[row * V + d] - (double)M) * invT) / Z;
      const double delta = a.delta > 0.f ? (double)a.delta : sqrt((double)a.eps);
      const double thr = fmin((double)a.eps, delta * exp(-H));
      ok = pd > thr ? 1 : 0;
    }
    a.row_ok[row] = ok;
  }
  __syncthreads();
  block_topk(
      n, K, [&](int e) { return s_key[e]; }, [&](int e) { return s_idx[e]; }, hist, s_sc, s_ck, s_ci, s_ok, s_oi);
  if (t < K) {
    a.cand_idx[row * MAXK + t] = s_oi[t];
    a.cand_val[row * MAXK + t] = key_value(s_ok[t]);
  }
}

// One wave per request: the first rejected row, the card sample there, the
// emitted tokens with the EOS / budget clamps, pos += n_emit, statistics.
__global__ __launch_bounds__(64) void sample_accept_kernel(const SampleArgs a) {
  __shared__ int s_tok;
  const int r = blockIdx.x, lane = threadIdx.x;
  const int Bm1 = a.b - 1;
  const int ok = lane < Bm1 ? a.row_ok[(size_t)r * a.b + lane] : 1;
  const unsigned long long rej = __ballot(lane < Bm1 && !ok);
  const int acc = rej ? (int)__builtin_ctzll(rej) : Bm1;
  if (lane == 0) {
    uint32_t c[4] = {a.round, (uint32_t)r, (uint32_t)acc, 0u};
    philox4x32_10(c, a.seed_lo, a.seed_hi);
    const double u = (double)(c[0] >> 8) * (1.0 / 16777216.0);
    const int K = min(a.top_k, a.V);
    const float* cv = a.cand_val + ((size_t)r * a.b + acc) * MAXK;
    const int* ci = a.cand_idx + ((size_t)r * a.b + acc) * MAXK;
    const double T = (double)a.T;
    const double x0 = (double)cv[0] / T;
    double q[MAXK], tot = 0.0;
    for (int j = 0; j < K; ++j) {
      q[j] = exp((double)cv[j] / T - x0);
      tot += q[j];
    }
    int keep = K;
    double c1 = 0.0;
    for (int j = 0; j < K; ++j) {
      q[j] /= tot;
      c1 += q[j];
      if (c1 >= (double)a.top_p) {
        keep = j + 1;
        break;
      }
    }
    for (int j = keep; j < K; ++j) q[j] /= tot;
    double cp = 0.0;
    for (int j = 0; j < keep; ++j) cp += q[j];
    const double target = u * cp;
    double run = 0.0;
    int pick = keep - 1;
    for (int j = 0; j < keep; ++j) {
      run += q[j];
      if (run > target) {
        pick = j;
        break;
      }
    }
    s_tok = ci[pick];
  }
  __syncthreads();
  const int x = s_tok;
  const int d = lane < Bm1 ? a.draft[((size_t)r * Bm1 + lane) * a.draft_stride] : -1;
  const int tok = lane < acc ? d : x;
  int n = acc + 1;
  if (a.eos >= 0) {
    const unsigned long long hit = __ballot(lane < n && tok == a.eos);
    if (hit) n = (int)__builtin_ctzll(hit) + 1;
  }
  if (a.budget) {
    int bg = a.budget[r];
    bg = bg < 1 ? 1 : bg;
    n = n < bg ? n : bg;
  }
  const int acc_c = acc < n - 1 ? acc : n - 1;
  if (lane < a.b) a.emitted[(size_t)r * a.b + lane] = lane < n ? tok : -1;
  const int last = __shfl(tok, n - 1, 64);
  if (a.next_tokens && lane < a.b) a.next_tokens[(size_t)r * a.b + lane] = lane == 0 ? last : a.mask_id;
  if (lane == 0) {
    a.accept_len[r] = acc_c;
    a.n_emit[r] = n;
    a.pos[r] += n;
    if (a.stats) {
      atomicAdd(&a.stats[0], 1ull);
      atomicAdd(&a.stats[a.stats_b + 1], (unsigned long long)n);
    }
  }
  if (a.stats && lane < acc_c) atomicAdd(&a.stats[1 + lane], 1ull);
}

}  // namespace

hipError_t launch_sampled_accept(const SampleArgs& a, hipStream_t st) {
  if (a.b < 1 || a.b > 64 || a.R < 1 || a.V < 1 || a.top_k < 1 || a.top_k > MAXK || !(a.T > 0.f))
    return hipErrorInvalidValue;
  if (a.n_chunks != (a.V + SAMPLE_CHUNK - 1) / SAMPLE_CHUNK || a.n_chunks > SAMPLE_MAX_CHUNKS)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_chunks_kernel, dim3(a.n_chunks, a.b, a.R), dim3(TPB), 0, st, a);
  hipLaunchKernelGGL(sample_rows_kernel, dim3(a.b, a.R), dim3(TPB), 0, st, a);
  hipLaunchKernelGGL(sample_accept_kernel, dim3(a.R), dim3(64), 0, st, a);
  return hipGetLastError();
}
