// Latency-bound kernels of the drafter round: state fill, embedding gather with
// the first RMSNorm, RMSNorm, position set and first-mismatch accept.
#include "device.h"
#include "kernels.h"

namespace {

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Streaming read of `n16` 16-byte vectors (the HBM read reference of the
// measurements): 256 workgroups x 256 threads, eight independent nontemporal
// 16-byte loads per thread in flight (the fastest plain read measured on
// MI355X over the shapes tried: grids of 256-4096 workgroups, 256 or 512
// threads, 4 or 8 loads in flight, temporal or nontemporal), an XOR of
// everything read per workgroup into sink[blockIdx.x] so that no load is dead.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t n16, unsigned* sink) {
  __shared__ unsigned red[4];
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld_nt16(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  for (; i < n16; i += stride) x ^= src[i];
  unsigned v = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
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

// One workgroup per row: h = E[token] (fp32) and the row's sum of squares,
// which the first QKV projection turns into its input RMSNorm. The row goes in
// 16-byte pieces (8 values), up to EMBED_PIECES per thread all loaded before the
// first is used: with one value per load, the stores to h between the loads kept
// every load waiting for the one before (6 us for a 2560-wide row).
constexpr int EMBED_PIECES = 4;
__global__ __launch_bounds__(256) void embed_kernel(const int* tokens, const uint16_t* embed, float* h,
                                                    float* ssq, int H, int V, unsigned* err) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) set_error(err, ERR_BAD_TOKEN);
    tok = 0;
  }
  const uint16_t* e = embed + (size_t)tok * H;
  float* hr = h + (size_t)m * H;
  const int np = H / 8;   // H is a multiple of 128
  float ss = 0.f;
  for (int i0 = 0; i0 < np; i0 += 256 * EMBED_PIECES) {
    u32x4 v[EMBED_PIECES];
#pragma unroll
    for (int u = 0; u < EMBED_PIECES; ++u) v[u] = ld16(e + 8 * min(i0 + (int)threadIdx.x + 256 * u, np - 1));
#pragma unroll
    for (int u = 0; u < EMBED_PIECES; ++u) {
      const int i = i0 + (int)threadIdx.x + 256 * u;
      if (i >= np) continue;
      f32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        lo[2 * j] = __uint_as_float(v[u][j] << 16);
        lo[2 * j + 1] = __uint_as_float(v[u][j] & 0xffff0000u);
        hi[2 * j] = __uint_as_float(v[u][2 + j] << 16);
        hi[2 * j + 1] = __uint_as_float(v[u][2 + j] & 0xffff0000u);
      }
      *(f32x4*)(hr + 8 * i) = lo;
      *(f32x4*)(hr + 8 * i + 4) = hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss += lo[j] * lo[j] + hi[j] * hi[j];
    }
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) ssq[m] = ss;
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

// First-mismatch accept, one wave per request (B <= 64): a ballot over the
// lanes j < B-1 whose draft differs from the verify id gives the accept length
// as the index of its lowest set bit.
__global__ __launch_bounds__(64) void accept_kernel(const int* draft, int draft_stride,
                                                    const int* verify, int B, int stats_b, int eos,
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
      atomicAdd(&stats[stats_b + 1], (unsigned long long)n);   // slots laid out for the configured block
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

hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* sink, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(STREAM_READ_BLOCKS), dim3(256), 0, st, (const u32x4*)src, bytes / 16,
                     sink);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_rows_kernel(const float* h, int H, float* dst, long long ld) {
  const int m = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c < H) *(f32x4*)(dst + (size_t)m * ld + c) = *(const f32x4*)(h + (size_t)m * H + c);
}

__global__ void advance_kernel(int* pos, const int* n_emit, int n_req) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n_req) pos[r] += n_emit[r];
}

hipError_t launch_copy_rows(const float* h, int M, int H, float* dst, long long ld, hipStream_t st) {
  if (H % 4 || ld % 4 || M < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((H / 4 + 255) / 256, M), dim3(256), 0, st, h, H, dst, ld);
  return hipGetLastError();
}

hipError_t launch_advance(int* pos, const int* n_emit, int n_req, hipStream_t st) {
  hipLaunchKernelGGL(advance_kernel, dim3((n_req + 63) / 64), dim3(64), 0, st, pos, n_emit, n_req);
  return hipGetLastError();
}

hipError_t launch_embed(const int* tokens, const uint16_t* embed, float* h, float* ssq, int M, int H, int V,
                        unsigned* err, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(256), 0, st, tokens, embed, h, ssq, H, V, err);
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

hipError_t launch_accept(const int* draft, int draft_stride, const int* verify, int R, int B, int stats_b, int eos,
                         const int* budget, int mask_id, int* accept_len, int* emitted, int* n_emit,
                         int* next_tokens, int* pos, unsigned long long* stats, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(R), dim3(64), 0, st, draft, draft_stride, verify, B, stats_b, eos,
                     budget, mask_id, accept_len, emitted, n_emit, next_tokens, pos, stats);
  return hipGetLastError();
}
