// Latency-bound kernels of the drafter round: state fill, embedding gather with
// the first RMSNorm, RMSNorm, position set, top-k merge and first-mismatch accept.
#include "device.h"
#include "kernels.h"

namespace {

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Block-wide sum over 256 threads.
DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

// One workgroup per row: h = E[token] (fp32), a = bf16(RMSNorm(h) * gain).
__global__ __launch_bounds__(256) void embed_norm_kernel(const int* tokens, const uint16_t* embed,
                                                         const uint16_t* gain, float* h,
                                                         uint16_t* a, int H, int V, float eps,
                                                         unsigned* err) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) set_error(err, 1u);
    tok = 0;
  }
  const uint16_t* e = embed + (size_t)tok * H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += blockDim.x) {
    const float v = bfbits2f(e[k]);
    h[(size_t)m * H + k] = v;
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    a[(size_t)m * H + k] = f2bfbits(bfbits2f(e[k]) * inv * bfbits2f(gain[k]));
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, const uint16_t* gain,
                                                      uint16_t* a, int H, float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const float* x = h + (size_t)m * H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += blockDim.x) ss += x[k] * x[k];
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    a[(size_t)m * H + k] = f2bfbits(x[k] * inv * bfbits2f(gain[k]));
}

__global__ void set_pos_kernel(int* pos, int* valid_from, int req, int vf, int p) {
  if (threadIdx.x == 0) {
    pos[req] = p;
    valid_from[req] = vf;
  }
}

// Merge per-group candidate lists (each sorted best-first) into the top-k of a
// row, ordered by (value desc, index asc). One workgroup per row; each thread
// keeps a sorted private list over a strided subset of groups (stopping inside
// a group at the first candidate that cannot enter its list), then the 256
// lists are merged pairwise in shared memory.
constexpr int KMAX = 16;

template <int K>
__global__ __launch_bounds__(256) void topk_merge_kernel(const float* cand_val, const int* cand_idx,
                                                         int groups, int rows, int* ids, float* vals) {
  __shared__ float sv[256][K];
  __shared__ int si[256][K];
  const int row = blockIdx.x;
  float lv[K];
  int li[K];
#pragma unroll
  for (int j = 0; j < K; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  for (int gr = threadIdx.x; gr < groups; gr += blockDim.x) {
    const float* cv = cand_val + ((size_t)gr * rows + row) * K;
    const int* ci = cand_idx + ((size_t)gr * rows + row) * K;
    for (int j = 0; j < K; ++j) {
      float v = cv[j];
      int id = ci[j];
      if (!better(v, id, lv[K - 1], li[K - 1])) break;
#pragma unroll
      for (int q = 0; q < K; ++q) {
        if (better(v, id, lv[q], li[q])) {
          const float tv = lv[q];
          const int ti = li[q];
          lv[q] = v; li[q] = id;
          v = tv; id = ti;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) { sv[threadIdx.x][j] = lv[j]; si[threadIdx.x][j] = li[j]; }
  __syncthreads();
  for (int width = 128; width >= 1; width >>= 1) {
    if ((int)threadIdx.x < width) {
      const int a = threadIdx.x, b = threadIdx.x + width;
      float ov[K];
      int oi[K];
      int ia = 0, ib = 0;
      for (int j = 0; j < K; ++j) {
        const bool ta = better(sv[a][ia], si[a][ia], sv[b][ib], si[b][ib]);
        ov[j] = ta ? sv[a][ia] : sv[b][ib];
        oi[j] = ta ? si[a][ia] : si[b][ib];
        if (ta) ++ia; else ++ib;
      }
      for (int j = 0; j < K; ++j) { sv[a][j] = ov[j]; si[a][j] = oi[j]; }
    }
    __syncthreads();
  }
  if ((int)threadIdx.x < K) {
    ids[(size_t)row * K + threadIdx.x] = si[0][threadIdx.x];
    if (vals) vals[(size_t)row * K + threadIdx.x] = sv[0][threadIdx.x];
  }
}

// First-mismatch accept, one wave per request (B <= 64): a ballot over the
// lanes j < B-1 whose draft differs from the verify id gives the accept length
// as the index of its lowest set bit.
__global__ __launch_bounds__(64) void accept_kernel(const int* draft, int draft_stride,
                                                    const int* verify, int B, int eos,
                                                    const int* budget, int mask_id,
                                                    int* accept_len, int* emitted, int* n_emit,
                                                    int* next_tokens, int* pos,
                                                    unsigned long long* stats) {
  const int r = blockIdx.x, j = threadIdx.x;
  const int Bm1 = B - 1;
  const int d = j < Bm1 ? draft[((size_t)r * Bm1 + j) * draft_stride] : -1;
  const int v = j < B ? verify[(size_t)r * B + j] : -1;
  const unsigned long long mis = __ballot(j < Bm1 && d != v);
  int acc = mis ? (int)__builtin_ctzll(mis) : Bm1;
  // emitted[j] = draft[j] for j < acc, verify[acc] at j == acc
  const int tok = j < acc ? d : v;
  int n = acc + 1;
  if (eos >= 0) {
    const unsigned long long hit = __ballot(j < n && tok == eos);
    if (hit) n = (int)__builtin_ctzll(hit) + 1;
  }
  if (budget) {
    int b = budget[r];
    b = b < 1 ? 1 : b;
    n = n < b ? n : b;
  }
  acc = acc < n - 1 ? acc : n - 1;
  if (j < B) emitted[(size_t)r * B + j] = j < n ? tok : -1;
  const int last = __shfl(tok, n - 1, 64);
  if (next_tokens && j < B) next_tokens[(size_t)r * B + j] = j == 0 ? last : mask_id;
  if (j == 0) {
    accept_len[r] = acc;
    n_emit[r] = n;
    pos[r] += n;
    if (stats) {
      atomicAdd(&stats[0], 1ull);
      atomicAdd(&stats[B + 1], (unsigned long long)n);
    }
  }
  if (stats && j < acc) atomicAdd(&stats[1 + j], 1ull);
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, words);
  return hipGetLastError();
}

hipError_t launch_embed_norm(const int* tokens, const uint16_t* embed, const uint16_t* gain, float* h,
                             uint16_t* a, int M, int H, int V, float eps, unsigned* err, hipStream_t st) {
  hipLaunchKernelGGL(embed_norm_kernel, dim3(M), dim3(256), 0, st, tokens, embed, gain, h, a, H, V, eps, err);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, const uint16_t* gain, uint16_t* a, int M, int H, float eps,
                          hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, st, h, gain, a, H, eps);
  return hipGetLastError();
}

hipError_t launch_set_pos(int* pos, int* valid_from, int req, int vf, int p, hipStream_t st) {
  hipLaunchKernelGGL(set_pos_kernel, dim3(1), dim3(64), 0, st, pos, valid_from, req, vf, p);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const float* cand_val, const int* cand_idx, int groups, int rows, int k,
                             int* ids, float* vals, hipStream_t st) {
  if (k == 1) hipLaunchKernelGGL((topk_merge_kernel<1>), dim3(rows), dim3(256), 0, st, cand_val, cand_idx, groups, rows, ids, vals);
  else if (k == 16) hipLaunchKernelGGL((topk_merge_kernel<16>), dim3(rows), dim3(256), 0, st, cand_val, cand_idx, groups, rows, ids, vals);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_accept(const int* draft, int draft_stride, const int* verify, int R, int B, int eos,
                         const int* budget, int mask_id, int* accept_len, int* emitted, int* n_emit,
                         int* next_tokens, int* pos, unsigned long long* stats, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(R), dim3(64), 0, st, draft, draft_stride, verify, B, eos,
                     budget, mask_id, accept_len, emitted, n_emit, next_tokens, pos, stats);
  return hipGetLastError();
}
