// Candidate trees from the drafter's top-k lists, and the kernels around a
// tree-masked verify pass. The pages keep top-16 candidates per draft position
// for a path selector ("feat: DFlash2 block-diffusion drafter for Qwen 3.8",
// Mference PR #22, "What's here") without stating its rule; the rule here:
//   - node 0 is the root (the block's known token); a node at depth d holds one
//     of the k candidates of draft position d, and its children are the k
//     candidates of position d + 1;
//   - candidate j of position d has log-probability
//     lp = (v[j] - v[0]) - log(sum_j' exp(v[j'] - v[0])) (fp64, list order), a
//     node's score is the sum of lp along its path (added in depth order);
//   - the tree is the root, the top-1 chain, then best first the highest
//     scoring child of any node in the tree, ties to the smaller depth, then
//     the smaller parent index, then the smaller rank.
// Within a list lp does not increase with the rank, so the best child of a
// node not yet taken is its lowest untaken rank: every node offers exactly one
// candidate, and a step of the best-first loop is an argmax over at most 64
// nodes, one per lane of a wave.
#include "device.h"
#include "kernels.h"

namespace {

// Whole-wave lane shifts (DPP wave_shl:1 / wave_shr:1): dst[l] = src[l + 1] and
// dst[l] = src[l - 1]; the lane without a source keeps `old`.
DEV int wave_shl1(int old, int v) { return __builtin_amdgcn_update_dpp(old, v, 0x130, 0xF, 0xF, false); }
DEV int wave_shr1(int old, int v) { return __builtin_amdgcn_update_dpp(old, v, 0x138, 0xF, 0xF, false); }

DEV int lo32(double x) { return (int)(uint32_t)__double_as_longlong(x); }
DEV int hi32(double x) { return (int)(uint32_t)((unsigned long long)__double_as_longlong(x) >> 32); }
DEV double mk64(int lo, int hi) {
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
DEV double lane_d(double x, int l) {
  return mk64(__builtin_amdgcn_readlane(lo32(x), l), __builtin_amdgcn_readlane(hi32(x), l));
}

// An offer: the score of the child and a packed (depth << 16 | parent << 8 |
// rank). Ordered by (score desc, depth asc, parent asc); a node has at most one
// offer outstanding, so (depth, parent) never ties.
DEV bool offer_beats(double sa, int pa, double sb, int pb) { return sa > sb || (sa == sb && pa < pb); }

// The offers outstanding, best first, one per lane (lanes past the last hold
// (-inf, INT_MAX)); insert keeps the order: the lanes before the new offer's
// place keep theirs, the rest shift up by one lane.
struct OfferQueue {
  double s;
  int p;
  DEV void pop() {
    const int lo = wave_shl1(lo32(-INFINITY), lo32(s)), hi = wave_shl1(hi32(-INFINITY), hi32(s));
    s = mk64(lo, hi);
    p = wave_shl1(0x7fffffff, p);
  }
  DEV void insert(double xs, int xp, int lane) {
    const int at = __popcll(__ballot(offer_beats(s, p, xs, xp)));
    const double us = mk64(wave_shr1(lo32(s), lo32(s)), wave_shr1(hi32(s), hi32(s)));
    const int up = wave_shr1(p, p);
    if (lane == at) {
      s = xs;
      p = xp;
    } else if (lane > at) {
      s = us;
      p = up;
    }
  }
};

// One wave per request: lane i holds node i.
__global__ __launch_bounds__(64) void tree_build_kernel(const int* block_tokens, int B, const int* ids,
                                                        const float* vals, int k, int n, int* out_tok,
                                                        int* out_par, int* out_dep) {
  __shared__ double s_lp[64][16];
  __shared__ double s_qs[64];
  __shared__ int s_qp[64];
  const int r = blockIdx.x, lane = threadIdx.x;
  const int Dm = B - 1;
  const int* rid = ids + (size_t)r * Dm * k;
  const float* rval = vals + (size_t)r * Dm * k;
  // list log-probabilities of position d = lane + 1
  if (lane < Dm) {
    const float* v = rval + (size_t)lane * k;
    float vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) vv[j] = j < k ? v[j] : 0.f;
    const double v0 = (double)vv[0];
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) s += exp((double)vv[j] - v0);
    const double lse = log(s);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) s_lp[lane][j] = ((double)vv[j] - v0) - lse;
  }
  __syncthreads();
  // root and the top-1 chain (nodes 1..dc at depths 1..dc)
  const int dc = min(Dm, n - 1);
  int tok = -1, par = -1, dep = 0, src = -1;
  double score = 0.0;
  if (lane == 0) {
    tok = block_tokens[(size_t)r * B];
  } else if (lane <= dc) {
    tok = rid[(size_t)(lane - 1) * k];
    par = lane - 1;
    dep = lane;
    for (int e = 0; e < lane; ++e) score += s_lp[e][0];   // depth order, as the scores add up along the path
  }
  // the chain's outstanding offers: rank 1 below every chain node but the last,
  // rank 0 below the last (when it may have children)
  const int orank = lane < dc ? 1 : 0;
  const bool offers = lane <= dc && dep < Dm && orank < k;
  const double os = offers ? score + s_lp[dep][orank] : -INFINITY;
  const int opk = offers ? ((dep + 1) << 16 | lane << 8 | orank) : 0x7fffffff;
  int place = 0;
  for (int m = 0; m <= dc; ++m) {
    const double ms = lane_d(os, m);
    const int mp = __builtin_amdgcn_readlane(opk, m);
    place += (m != lane && offer_beats(ms, mp, os, opk)) ? 1 : 0;
  }
  s_qs[lane] = -INFINITY;
  s_qp[lane] = 0x7fffffff;
  __syncthreads();
  if (offers) {
    s_qs[place] = os;
    s_qp[place] = opk;
  }
  __syncthreads();
  OfferQueue q{s_qs[lane], s_qp[lane]};
  // best first: pop the best offer as node cnt, then queue its parent's next
  // rank and its own first child
  for (int cnt = dc + 1; cnt < n; ++cnt) {
    const double ts = lane_d(q.s, 0);
    const int tp = __builtin_amdgcn_readlane(q.p, 0);   // the host guarantees an offer remains
    const int od = tp >> 16, op = (tp >> 8) & 255, j = tp & 255;
    q.pop();
    if (lane == cnt) {
      src = (od - 1) * k + j;   // the token is read after the loop, off its critical path
      par = op;
      dep = od;
      score = ts;
    }
    if (j + 1 < k) q.insert(lane_d(score, op) + s_lp[od - 1][j + 1], od << 16 | op << 8 | (j + 1), lane);
    if (od < Dm) q.insert(ts + s_lp[od][0], (od + 1) << 16 | cnt << 8, lane);
  }
  if (src >= 0) tok = rid[src];
  if (lane < n) {
    out_tok[(size_t)r * n + lane] = tok;
    out_par[(size_t)r * n + lane] = par;
    out_dep[(size_t)r * n + lane] = dep;
  }
}

// Tree accept, one wave per request (lane i holds node i; n <= 64): walk from
// the root along the child whose token is the target's token at the current
// node; emit the walked tokens and the target's token at the end; EOS and
// budget clamps; pos += n_emit. The committed nodes (root first) give the tap
// rows to stage next: stage_rows = r * n + node, stage_pos = old pos + depth,
// padded past n_emit with the last committed node at the following positions.
__global__ __launch_bounds__(64) void tree_accept_kernel(const int* tok, const int* par, int n, const int* verify,
                                                         int B, int stats_b, int eos, const int* budget, int mask_id,
                                                         int* accept_len, int* emitted, int* n_emit, int* next_tokens,
                                                         int* path_nodes, int* stage_rows, int* stage_pos, int* pos,
                                                         unsigned long long* stats) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int t = lane < n ? tok[(size_t)r * n + lane] : -1;
  const int p = lane < n ? par[(size_t)r * n + lane] : -2;
  const int v = lane < n ? verify[(size_t)r * n + lane] : -1;
  int cur = 0, depth = 0;
  int my_depth_node = lane == 0 ? 0 : -1;   // lane d: the walked node at depth d
  for (int step = 0; step < B - 1; ++step) {
    const int want = __shfl(v, cur, 64);
    const unsigned long long hit = __ballot(lane < n && p == cur && t == want);
    if (!hit) break;
    cur = (int)__builtin_ctzll(hit);
    ++depth;
    if (lane == depth) my_depth_node = cur;
  }
  // emitted[j] = token of the walked node at depth j + 1 (j < depth), then the bonus
  const int node_j1 = __shfl(my_depth_node, min(lane + 1, 63), 64);
  const int tok_j1 = __shfl(t, max(node_j1, 0), 64);
  const int bonus = __shfl(v, cur, 64);
  const int e_tok = lane < depth ? tok_j1 : bonus;
  int ne = depth + 1;
  if (eos >= 0) {
    const unsigned long long hit = __ballot(lane < ne && e_tok == eos);
    if (hit) ne = (int)__builtin_ctzll(hit) + 1;
  }
  if (budget) {
    int b = budget[r];
    b = b < 1 ? 1 : b;
    ne = ne < b ? ne : b;
  }
  const int acc = depth < ne - 1 ? depth : ne - 1;
  const int old_pos = pos[r];
  const int last = __shfl(e_tok, ne - 1, 64);
  const int last_node = __shfl(my_depth_node, ne - 1, 64);
  if (lane < B) {
    emitted[(size_t)r * B + lane] = lane < ne ? e_tok : -1;
    if (next_tokens) next_tokens[(size_t)r * B + lane] = lane == 0 ? last : mask_id;
    const int node = lane < ne ? my_depth_node : last_node;
    path_nodes[(size_t)r * B + lane] = node;
    stage_rows[(size_t)r * B + lane] = r * n + node;
    stage_pos[(size_t)r * B + lane] = old_pos + lane;
  }
  if (lane == 0) {
    accept_len[r] = acc;
    n_emit[r] = ne;
    pos[r] = old_pos + ne;
    if (stats) {
      atomicAdd(&stats[0], 1ull);
      atomicAdd(&stats[stats_b + 1], (unsigned long long)ne);
    }
  }
  if (stats && lane < acc) atomicAdd(&stats[1 + lane], 1ull);
}

// Ancestor masks of the tree rows (bit j of row i: node j is an ancestor of node
// i, itself included), one wave per request; rows past n are plain chain rows.
__global__ __launch_bounds__(64) void tree_anc_kernel(const int* par, int n, int rows, unsigned long long* anc) {
  const int r = blockIdx.x, lane = threadIdx.x;
  if (lane >= rows) return;
  unsigned long long m = 0ull;
  int i = lane;
  for (int s = 0; s < 64 && i >= 0 && i < 64; ++s) {   // a parent array that is not a tree ends the walk
    m |= 1ull << i;
    i = i < n ? par[(size_t)r * n + i] : i - 1;
  }
  anc[(size_t)r * rows + lane] = m;
}

// Commit of a target's tree pass: the K rows and V columns of the committed
// nodes (ring slots pos + node) move to slots pos + d, d < n_emit, for every
// layer and kv head; one workgroup per (layer, request, kv head). All sources
// are read before any slot is written (a destination slot can be another
// depth's source).
template <int HD>
__global__ __launch_bounds__(256) void tree_commit_kernel(uint16_t* ring_k, uint16_t* ring_v, size_t layer_elems,
                                                          int R, int nkv, int C, const int* pos,
                                                          const int* path_nodes, int path_ld, const int* n_emit) {
  constexpr int MAXB = 64;
  __shared__ uint16_t s_k[MAXB][HD], s_v[HD][MAXB];
  const int lg = blockIdx.x % nkv, rest = blockIdx.x / nkv;
  const int r = rest % R, l = rest / R;   // ring offsets use the state's own request stride (layer_elems)
  const int ne = max(0, min(n_emit[r], path_ld));
  const int p0 = pos[r];
  uint16_t* rk = ring_k + l * layer_elems + ((size_t)r * nkv + lg) * C * HD;
  uint16_t* rv = ring_v + l * layer_elems + ((size_t)r * nkv + lg) * HD * C;
  for (int e = threadIdx.x; e < ne * HD; e += blockDim.x) {
    const int d = e / HD, c = e % HD;
    const int node = max(0, min(path_nodes[(size_t)r * path_ld + d], MAXB - 1));
    const int src = (p0 + node) % C;
    s_k[d][c] = rk[(size_t)src * HD + c];
    s_v[c][d] = rv[(size_t)c * C + src];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ne * HD; e += blockDim.x) {
    const int d = e / HD, c = e % HD;
    const int dst = (p0 + d) % C;
    rk[(size_t)dst * HD + c] = s_k[d][c];
    rv[(size_t)c * C + dst] = s_v[c][d];
  }
}

}  // namespace

hipError_t launch_tree_build(const int* block_tokens, int B, const int* ids, const float* vals, int k, int R, int n,
                             int* tok, int* par, int* dep, hipStream_t st) {
  if (B < 2 || B > 64 || k < 1 || k > 16 || n < 1 || n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_build_kernel, dim3(R), dim3(64), 0, st, block_tokens, B, ids, vals, k, n, tok, par, dep);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const int* tok, const int* par, int n, const int* verify, int R, int B, int stats_b,
                              int eos, const int* budget, int mask_id, int* accept_len, int* emitted, int* n_emit,
                              int* next_tokens, int* path_nodes, int* stage_rows, int* stage_pos, int* pos,
                              unsigned long long* stats, hipStream_t st) {
  if (n < 1 || n > 64 || B < 1 || B > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_accept_kernel, dim3(R), dim3(64), 0, st, tok, par, n, verify, B, stats_b, eos, budget,
                     mask_id, accept_len, emitted, n_emit, next_tokens, path_nodes, stage_rows, stage_pos, pos, stats);
  return hipGetLastError();
}

hipError_t launch_tree_anc(const int* par, int n, int rows, int R, unsigned long long* anc, hipStream_t st) {
  if (rows < 1 || rows > 64 || n > rows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_anc_kernel, dim3(R), dim3(64), 0, st, par, n, rows, anc);
  return hipGetLastError();
}

hipError_t launch_tree_commit(uint16_t* ring_k, uint16_t* ring_v, size_t layer_elems, int L, int R, int nkv, int hd,
                              int C, const int* pos, const int* path_nodes, int path_ld, const int* n_emit,
                              hipStream_t st) {
  if (R < 1 || path_ld < 1 || path_ld > 64) return hipErrorInvalidValue;
  const dim3 grid(L * R * nkv);
  if (hd == 128)
    hipLaunchKernelGGL((tree_commit_kernel<128>), grid, dim3(256), 0, st, ring_k, ring_v, layer_elems, R, nkv, C,
                       pos, path_nodes, path_ld, n_emit);
  else if (hd == 64)
    hipLaunchKernelGGL((tree_commit_kernel<64>), grid, dim3(256), 0, st, ring_k, ring_v, layer_elems, R, nkv, C, pos,
                       path_nodes, path_ld, n_emit);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
