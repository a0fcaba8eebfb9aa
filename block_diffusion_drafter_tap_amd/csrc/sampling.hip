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

// The K-th largest order key among the n elements whose key is >= floor (at
// least K of them must be): radix select over four 8-bit digits with an LDS
// histogram. Returns the key; *need_out = how many elements equal to it belong
// to the top K. The floor only prunes the histogram updates (elements below it
// cannot be among the top K), which keeps the LDS atomics off the crowded low
// bins. Every thread of the block calls it.
template <class KeyF>
DEV unsigned radix_kth(int n, int K, unsigned floor, KeyF key, unsigned* hist, int* sc, int* need_out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  unsigned prefix = 0, pmask = 0;
  int need = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
    for (int e = t; e < n; e += TPB) {
      const unsigned k = key(e);
      if (k >= floor && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
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
  *need_out = need;
  return prefix;
}

// Top-K (K <= 64) of n keyed elements, in (key desc, position asc) order: the
// K-th largest key, then every key above it and the first `need` positions
// among the keys equal to it, then a rank by comparison. key(e) is the order key
// of element e, id(e) its token id; callers order positions so that equal keys
// come by ascending token id, and pass a floor with at least K keys >= it.
// Results: out_key[0..K), out_id[0..K) in LDS. Every thread of the block calls it.
template <class KeyF, class IdF>
DEV void block_topk(int n, int K, unsigned floor, KeyF key, IdF id, unsigned* hist, int* sc, unsigned* cand_key,
                    int* cand_id, unsigned* out_key, int* out_id) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int need;
  const unsigned prefix = radix_kth(n, K, floor, key, hist, sc, &need);
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

// Top-K of C <= TPB candidates (key, id) held in LDS, ids distinct: each thread
// ranks its candidate by (key desc, id asc) against all C and the K best land
// in out_key / out_id. Every thread of the block calls it.
DEV void rank_select(int C, int K, const unsigned* ck, const int* ci, unsigned* out_key, int* out_id) {
  const int t = threadIdx.x;
  if (t < C) {
    const unsigned kt = ck[t];
    const int it = ci[t];
    int rank = 0;
    for (int j = 0; j < C; ++j) rank += (ck[j] > kt || (ck[j] == kt && ci[j] < it)) ? 1 : 0;
    if (rank < K) {
      out_key[rank] = kt;
      out_id[rank] = it;
    }
  }
  __syncthreads();
}

DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The m-th largest (m in 1..64) of the wave's 64 keys: a bitwise search, each
// step a ballot count of the keys at or above a candidate.
DEV unsigned wave_mth_key(unsigned key, int m) {
  unsigned ans = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned cand = ans | (1u << bit);
    if (__popcll(__ballot(key >= cand)) >= m) ans = cand;
  }
  return ans;
}

// Top-K of C <= 64 candidates, one (key, id) per lane of the calling wave (ids
// distinct): each lane's rank by (key desc, id asc) from the others' pairs,
// broadcast one lane at a time; the lane of rank r < K writes entry r.
DEV void wave_rank_select(unsigned key, int id, int C, int K, int lane, unsigned* out_key, int* out_id) {
  int rank = 0;
  for (int m = 0; m < C; ++m) {
    const unsigned mk = (unsigned)__builtin_amdgcn_readlane((int)key, m);
    const int mi = __builtin_amdgcn_readlane(id, m);
    rank += (mk > key || (mk == key && mi < id)) ? 1 : 0;
  }
  if (lane < C && rank < K) {
    out_key[rank] = key;
    out_id[rank] = id;
  }
}

// Top-K (K <= 64) of the C candidates compacted in LDS (ids distinct), written
// with stride 1 to out_key / out_id in global memory: ranked by one wave when
// C <= 64, else by every thread.
DEV void select_candidates(int C, int K, const unsigned* ck, const int* ci, unsigned* ok_lds, int* oi_lds,
                           unsigned* out_key, int* out_id) {
  const int t = threadIdx.x;
  if (C <= 64) {
    if (t < 64) wave_rank_select(t < C ? ck[t] : 0u, t < C ? ci[t] : 0x7fffffff, C, K, t, out_key, out_id);
  } else {
    rank_select(C, K, ck, ci, ok_lds, oi_lds);
    if (t < K) {
      out_key[t] = ok_lds[t];
      out_id[t] = oi_lds[t];
    }
  }
}

// Stage 1, one workgroup per (chunk c, row i, request r) over SAMPLE_CHUNK
// logits (16 a thread, in registers): the chunk max m_c, Z_c = sum exp(x),
// S_c = sum exp(x) x with x = (z - m_c) / T, and the chunk's top-K in (value
// desc, index asc). The selection starts from a floor that at least K logits
// reach: each wave's ceil(K/4)-th largest thread maximum, the least of the four.
// The logits at or above it (typically a few dozen) are compacted and ranked;
// a chunk with more than TPB of them (flat rows) takes a radix select instead.
__global__ __launch_bounds__(TPB) void sample_chunks_kernel(const SampleArgs a) {
  __shared__ unsigned s_cand_k[TPB];
  __shared__ int s_cand_i[TPB];
  __shared__ unsigned hist[256];
  __shared__ int s_sc[4 + TPB / 64];
  __shared__ unsigned s_ck[MAXK], s_ok[MAXK];
  __shared__ int s_ci[MAXK], s_oi[MAXK];
  __shared__ float s_red[TPB / 64];
  __shared__ unsigned s_fl[TPB / 64];
  __shared__ double s_dred[2][TPB / 64];
  const int c = blockIdx.x, i = blockIdx.y, r = blockIdx.z, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V, S = a.n_chunks;
  const int e0 = c * SAMPLE_CHUNK, n = min(SAMPLE_CHUNK, V - e0);
  const size_t row = (size_t)r * a.b + i;
  const float* z = a.logits + row * V + e0;
  constexpr int PER = SAMPLE_CHUNK / TPB;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = t + j * TPB < n ? z[t + j * TPB] : -INFINITY;
  float tmx = -INFINITY;
  unsigned tkey = 0;   // a thread without logits keeps key 0, below every real one
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (t + j * TPB < n) {
      tmx = fmaxf(tmx, v[j]);
      tkey = max(tkey, order_key(v[j]));
    }
  }
  const int K = min(a.top_k, n);
  const unsigned fw = wave_mth_key(tkey, (K + 3) / 4);
  float mx = wave_max(tmx);
  if (lane == 0) {
    s_red[wave] = mx;
    s_fl[wave] = fw;
  }
  if (t == 0) s_sc[2] = 0;
  __syncthreads();
  mx = s_red[0];
  unsigned floor = s_fl[0];
  for (int w = 1; w < TPB / 64; ++w) {
    mx = fmaxf(mx, s_red[w]);
    floor = min(floor, s_fl[w]);
  }
  // the logits at or above the floor, compacted (their order does not matter:
  // the selection orders by id)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = t + j * TPB;
    if (e < n) {
      const unsigned k = order_key(v[j]);
      if (k >= floor) {
        const int slot = atomicAdd(&s_sc[2], 1);
        if (slot < TPB) {
          s_cand_k[slot] = k;
          s_cand_i[slot] = e0 + e;
        }
      }
    }
  }
  // x in fp32, exp from the hardware exp2 (relative error ~2e-7 over the
  // range that carries weight), the sums in fp64
  const float invT = 1.0f / a.T;
  double sz = 0.0, sx = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (t + j * TPB < n) {
      const float x = (v[j] - mx) * invT;
      const float ex = __expf(x);
      sz += (double)ex;
      sx = fma((double)ex, (double)x, sx);
    }
  }
  sz = wave_sum_d(sz);
  sx = wave_sum_d(sx);
  if (lane == 0) {
    s_dred[0][wave] = sz;
    s_dred[1][wave] = sx;
  }
  __syncthreads();
  const int C = s_sc[2];
  const size_t part = row * S + c;
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
  unsigned* out_key = a.part_key + part * MAXK;
  int* out_id = a.part_idx + part * MAXK;
  if (C <= TPB) {
    select_candidates(C, K, s_cand_k, s_cand_i, s_ok, s_oi, out_key, out_id);
  } else {
    // flat rows: radix select over the chunk, re-read from global memory
    __syncthreads();
    block_topk(
        n, K, floor, [&](int e) { return order_key(z[e]); }, [&](int e) { return e0 + e; }, hist, s_sc, s_ck,
        s_ci, s_ok, s_oi);
    if (t < K) {
      out_key[t] = s_ok[t];
      out_id[t] = s_oi[t];
    }
  }
}

// Stage 2, one workgroup per (row i, request r): the chunks' statistics merged
// at the row max M (Z = sum_c Z_c e^{(m_c - M)/T}, S = sum_c e^{(m_c - M)/T}
// (S_c + Z_c (m_c - M)/T), H = log Z - S / Z), the acceptance test of the row's
// draft token (rows i < b - 1), and the row's top-K from the chunks' lists
// (each in (value desc, index asc) order). The floor is the larger of the
// largest K-th entry of a full list (that list alone holds K keys at or above
// it) and the K-th largest chunk maximum (K lists reach it); the entries at or
// above it are compacted and ranked, or, past TPB of them, radix-selected (the
// lists laid out by chunk keep equal values by ascending index there).
__global__ __launch_bounds__(TPB) void sample_rows_kernel(const SampleArgs a) {
  __shared__ unsigned s_key[SAMPLE_MAX_CHUNKS * MAXK];
  __shared__ int s_idx[SAMPLE_MAX_CHUNKS * MAXK];
  __shared__ unsigned s_cand_k[TPB];
  __shared__ int s_cand_i[TPB];
  __shared__ unsigned hist[256];
  __shared__ int s_sc[4 + TPB / 64];
  __shared__ unsigned s_ck[MAXK], s_ok[MAXK];
  __shared__ int s_ci[MAXK], s_oi[MAXK];
  __shared__ float s_red[TPB / 64];
  __shared__ unsigned s_floor[TPB / 64];
  __shared__ double s_dred[2][TPB / 64];
  __shared__ float s_zd;
  __shared__ int s_d;
  const int i = blockIdx.x, r = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V, S = a.n_chunks, K = min(a.top_k, V);
  const size_t row = (size_t)r * a.b + i;
  // every chunk but the last holds SAMPLE_CHUNK > 64 >= top_k logits, so chunk c's
  // list starts at c * top_k; the last one has min(top_k, its size) entries
  const int kc = a.top_k;
  const int n = (S - 1) * kc + min(kc, V - (S - 1) * SAMPLE_CHUNK);
  // every global read first: the draft token's logit (the last thread), the
  // lists, and thread c < S the statistics and K-th entry of chunk c
  if (t == TPB - 1 && i < a.b - 1) {
    const int d = a.draft[((size_t)r * (a.b - 1) + i) * a.draft_stride];
    s_d = d;
    s_zd = (d >= 0 && d < V) ? a.logits[row * V + d] : 0.f;
  }
  constexpr int PER = SAMPLE_MAX_CHUNKS * MAXK / TPB;
  unsigned lk[PER];
  int li[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = t + j * TPB;
    if (e < n) {
      const int c = e / kc;
      const size_t src = (row * S + c) * MAXK + (e - c * kc);
      lk[j] = a.part_key[src];
      li[j] = a.part_idx[src];
    }
  }
  const bool has = t < S;
  const bool full = has && (t < S - 1 || V - (S - 1) * SAMPLE_CHUNK >= kc);
  const float mc = has ? a.part_m[row * S + t] : -INFINITY;
  const double zz = has ? a.part_z[row * S + t] : 0.0, ss = has ? a.part_s[row * S + t] : 0.0;
  unsigned fl = full ? a.part_key[(row * S + t) * MAXK + kc - 1] : 0u;
  const unsigned top = has ? a.part_key[(row * S + t) * MAXK] : 0u;
  float M = wave_max(mc);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) fl = max(fl, (unsigned)__shfl_xor((int)fl, o, 64));
  // the K-th largest chunk maximum: K chunks reach it, one entry each (0 when
  // there are fewer than K chunks); S <= 64, so wave 0 holds every chunk
  fl = max(fl, wave_mth_key(top, K));
  if (lane == 0) {
    s_red[wave] = M;
    s_floor[wave] = fl;
  }
  if (t == 0) s_sc[2] = 0;
  __syncthreads();
  M = s_red[0];
  unsigned floor = s_floor[0];
  for (int w = 1; w < TPB / 64; ++w) {
    M = fmaxf(M, s_red[w]);
    floor = max(floor, s_floor[w]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = t + j * TPB;
    if (e < n && lk[j] >= floor) {
      const int slot = atomicAdd(&s_sc[2], 1);
      if (slot < TPB) {
        s_cand_k[slot] = lk[j];
        s_cand_i[slot] = li[j];
      }
    }
  }
  const double invT = 1.0 / (double)a.T;
  double zc = 0.0, sc = 0.0;
  if (has) {
    const double sh = ((double)mc - (double)M) * invT;
    const double w = exp(sh);
    zc = w * zz;
    sc = w * (ss + zz * sh);
  }
  zc = wave_sum_d(zc);
  sc = wave_sum_d(sc);
  if (lane == 0) {
    s_dred[0][wave] = zc;
    s_dred[1][wave] = sc;
  }
  __syncthreads();
  const int C = s_sc[2];
  if (t == 0 && i < a.b - 1) {
    double Z = 0.0, Sx = 0.0;
    for (int w = 0; w < TPB / 64; ++w) {
      Z += s_dred[0][w];
      Sx += s_dred[1][w];
    }
    const double H = log(Z) - Sx / Z;
    const int d = s_d;
    int ok = 0;
    if (d >= 0 && d < V) {
      const double pd = exp(((double)s_zd - (double)M) * invT) / Z;
      const double delta = a.delta > 0.f ? (double)a.delta : sqrt((double)a.eps);
      const double thr = fmin((double)a.eps, delta * exp(-H));
      ok = pd > thr ? 1 : 0;
    }
    a.row_ok[row] = ok;
  }
  unsigned* out_key = a.cand_key + row * MAXK;
  int* out_id = a.cand_idx + row * MAXK;
  if (C <= TPB) {
    select_candidates(C, K, s_cand_k, s_cand_i, s_ok, s_oi, out_key, out_id);
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = t + j * TPB;
      if (e < n) {
        s_key[e] = lk[j];
        s_idx[e] = li[j];
      }
    }
    __syncthreads();
    block_topk(
        n, K, floor, [&](int e) { return s_key[e]; }, [&](int e) { return s_idx[e]; }, hist, s_sc, s_ck, s_ci, s_ok,
        s_oi);
    if (t < K) {
      out_key[t] = s_ok[t];
      out_id[t] = s_oi[t];
    }
  }
}

// One wave per request: the first rejected row a, the card sample there (lane
// j holds the j-th candidate: q_j = exp(x_j - x_0) / sum, then running sums
// over lanes), the emitted tokens with the EOS / budget clamps, pos += n_emit,
// statistics.
__global__ __launch_bounds__(64) void sample_accept_kernel(const SampleArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int Bm1 = a.b - 1;
  const int ok = lane < Bm1 ? a.row_ok[(size_t)r * a.b + lane] : 1;
  const unsigned long long rej = __ballot(lane < Bm1 && !ok);
  const int acc = rej ? (int)__builtin_ctzll(rej) : Bm1;
  const int K = min(a.top_k, a.V);
  const size_t cb = ((size_t)r * a.b + acc) * MAXK;
  const double T = (double)a.T;
  const unsigned* ckey = a.cand_key + cb;
  const double x0 = (double)key_value(ckey[0]) / T;
  const double qj = lane < K ? exp((double)key_value(ckey[lane]) / T - x0) : 0.0;
  const double q = qj / wave_sum_d(qj);
  double run = q;   // inclusive running sum over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double up = __shfl_up(run, o, 64);
    if (lane >= o) run += up;
  }
  // keep the shortest prefix reaching top_p (all K if rounding keeps the total below it)
  const unsigned long long reach = __ballot(lane < K && run >= (double)a.top_p);
  const int keep = reach ? (int)__builtin_ctzll(reach) + 1 : K;
  const double cp = __shfl(run, keep - 1, 64);
  uint32_t ctr[4] = {a.round, (uint32_t)r, (uint32_t)acc, 0u};
  philox4x32_10(ctr, a.seed_lo, a.seed_hi);
  const double u = (double)(ctr[0] >> 8) * (1.0 / 16777216.0);
  const unsigned long long over = __ballot(lane < keep && run > u * cp);
  const int pick = over ? (int)__builtin_ctzll(over) : keep - 1;
  const int x = a.cand_idx[cb + pick];
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
