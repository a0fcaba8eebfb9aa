// Internal interface between the host library (api.hip) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum XKind { X_BF16 = 0, X_TAPS = 1, X_NORM = 2 };
// E_PART / E_PARTP: split-K partial tiles to partials[split][M][Ntot] (fp32), Ntot = N,
// or 2N for a gate/up pair (gate columns first, then up); a finish kernel sums them.
enum EpiKind { E_BF16 = 0, E_F32 = 1, E_RESID = 2, E_SILU = 3, E_HEAD = 4, E_PART = 5, E_PARTP = 6 };
enum WFmt { WF_BF16 = 0, WF_INT4 = 1 };

constexpr int MAX_TAPS = 8;
constexpr int MAX_BATCH = 8;   // layers per batched stage K/V launch
constexpr int GEMM_WAVES = 4;

// Arguments of the skinny GEMM Y[M, N] = X[M, K] . W[N, K]^T with a fused epilogue.
struct GemmArgs {
  // X operand: bf16 rows (X_BF16), fp32 tap rows reduced on the fly (X_TAPS),
  // or the fp32 residual normalized on the fly (X_NORM: x = h * rsqrt(ss/K + eps) * g,
  // ss = sum over the n_ssq column blocks of ssq_in[block * ssq_ld + row])
  const uint16_t* x;
  long long ldx;
  const float* xf;
  const uint16_t* xgain;
  const float* ssq_in;
  int n_ssq;
  int ssq_ld;
  float* ssq_out;   // E_RESID: per-row sum of squares of the updated h, one entry per column group
  const float* taps[MAX_TAPS];
  long long tap_stride;
  int n_taps, hc, tap_hidden;
  // W operand: bf16 [N][K] or packed INT4 [N][K/2] + fp16 scales [N][K/64]
  const void* w;
  const uint16_t* wscale;
  int M, N, K;     // N counts output columns (gate/up pairs count once)
  int ks, S;       // K per split, number of splits (grid.y)
  int pair_off;    // W row offset of the "up" rows (E_SILU)
  // plain epilogues
  void* out;
  long long ldo;
  // split-K partial tiles (E_PART / E_PARTP)
  float* partials;
  // layer batch (nb > 0): grid.z also runs over nb layers; layer b uses W wb[b],
  // rings rkb[b] / rvb[b], k gain kgb[b] and partials + b * S * M * N
  int nb;
  const void* wb[MAX_BATCH];
  const uint16_t* wsb[MAX_BATCH];   // INT4 scales of layer b
  uint16_t* rkb[MAX_BATCH];
  uint16_t* rvb[MAX_BATCH];
  const uint16_t* kgb[MAX_BATCH];
  // E_HEAD: per-head q/k RMSNorm + RoPE, Q to q_out, K/V to the ring
  int head_base, nq, nkv, hd;
  float eps;
  double log2_theta;
  const uint16_t* q_gain;
  const uint16_t* k_gain;
  uint16_t* q_out;
  uint16_t* ring_k;   // this layer's [Rmax][nkv][C][hd]
  uint16_t* ring_v;   // this layer's [Rmax][nkv][hd][C]
  int C, Rmax;
  int win;                // window W: staged rows are checked against the ring's live range
  const int* pos;         // state pos[]
  const int* req_of_row;  // NULL -> row / rows_per_req
  const int* pos_of_row;  // NULL -> pos[req] + row % rows_per_req
  int rows_per_req;
  const int* rope_off;    // NULL, or per row: RoPE at pos[req] + rope_off[row] (a tree row's depth), ring slot unchanged
  const int* src_row;     // NULL, or per row: the tap row X_TAPS reads for it
  unsigned* err;
  // B: the configured block (the ring's live range is [pos - win, pos + B)),
  // except for the LM head, where it is the call's block length. LM head: rows
  // m = r*B + i; rows i >= lm_first_row produce logits (1: the mask rows of a
  // draft; 0: every row of a verify pass)
  int B, topk, lm_first_row;
};

struct GemmPlan {
  int MT, NT, NW, XL, S, ks, groups, mz;
  size_t lds;   // dynamic LDS bytes per workgroup
};

// cps: target K chunks (of 128) per split when the grid needs splitting; the
// S partial tiles of one launch never exceed GEMM_PARTIAL_BUDGET floats.
// wf: weight format (INT4 adds per-group row sums of X to the LDS budget).
constexpr long long GEMM_PARTIAL_BUDGET = 8ll << 20;
GemmPlan plan_gemm(int M, int N, int K, int gc, int pair, int cps, int wf);
hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int xk, int epi, int wf,
                       hipStream_t st);
size_t gemm_partial_floats(const GemmPlan& p, int M, int N, int pair);

// Gate/up of the MLP in one launch for up to 16 rows (bf16 weights [2N][K], the
// up rows at pair_off = N; X_NORM fields of GemmArgs): act = SiLU(gate) * up as
// bf16 to out [M][ldo]. The sums are formed as the split-K GEMM with `ks`
// columns per split and its finish form them, so the bits match that path.
// gateup_lds_bytes: dynamic LDS of a launch, 0 when the shape does not fit.
size_t gateup_lds_bytes(int M, int K);
hipError_t launch_gateup_lds(const GemmArgs& a, int ks, hipStream_t st);
// The same with INT4 weights (packed [2N][K/2] + fp16 scales [2N][K/64] in
// wscale), matching the INT4 split-K GEMM and its finish bit for bit.
size_t gateup_q4_bytes(int M, int K);
hipError_t launch_gateup_q4(const GemmArgs& a, int ks, hipStream_t st);

// LM head: persistent logits GEMM over the block rows (GemmArgs X_NORM fields
// xf, xgain, ssq_*, w = W_lm, M = R*B, N = vocab, K, B, topk; when the plan does
// not stage the rows in LDS (XL = 0), x / ldx instead hold the final-normed rows
// as bf16, written by the caller beforehand): fp32 logits to
// the caller's logits[R*(B-1)][N] (mask rows), or transposed to a scratch
// [N][16*MT] (all rows; coalesced), and per-16-column maxima of the mask rows to
// gmax[R*(B-1)][ceil(N/16)]; then the exact per-row top-k to ids/vals
// [R*(B-1)][topk] (topk <= 16).
struct LmPlan {
  int MT, XL, groups, P;   // XL: 1 rows staged in LDS, 2 LDS windows of bf16 rows, 0 rows from L2,
                           // 3 rows staged and W through LDS (direct loads); P workgroups
  int slots, defer_off;    // groups per workgroup whose epilogue waits for the last load; their LDS
                           // offset (XL 3: the offset of the W slots)
  size_t lds;
  int kph = 1;             // XL 3/4: phases of K (XL 3: each stages K / kph columns of the rows)
  int rx = 16;             // XL 3: rows staged (8 when the call has at most 8)
  int contig = 0;          // XL 3: W's 16-row tiles in contiguous ranges per workgroup, not by groups
};
LmPlan plan_lmhead(int M, int B, int V, int K, int n_cu);
// the final-normed rows as bf16 z[M][K] (for plans with XL = 0), from the same
// X_NORM fields, with the LDS staging's arithmetic
hipError_t launch_lm_norm_rows(const GemmArgs& a, uint16_t* z, hipStream_t st);
hipError_t launch_lm_logits(const GemmArgs& a, const LmPlan& p, float* logits, int transposed, float* gmax,
                            hipStream_t st);
hipError_t launch_lm_topk(const GemmArgs& a, const LmPlan& p, const float* logits, int transposed,
                          const float* gmax, int* ids, float* vals, hipStream_t st);

// Attention over [context window | block] per (request, kv head), split over key chunks.
struct AttnArgs {
  const uint16_t* q;       // [R*B][nq*hd]
  const uint16_t* ring_k;  // layer base [Rmax][nkv][C][hd]
  const uint16_t* ring_v;  // layer base [Rmax][nkv][hd][C]
  uint16_t* out;           // [R*B][nq*hd]
  const int* pos;
  const int* valid_from;
  int B, W, C, nq, nkv, hd, kc, n_chunks;
  int causal;              // 1: block query i sees block keys j <= i only (a target verify pass);
                           // 2: block query i sees block key j iff bit j of anc[r * B + i] is set (a tree pass)
  const unsigned long long* anc;   // [R][B] ancestor masks of the tree rows (causal == 2)
  int R;                   // requests of this launch (set by launch_attention)
  int hs;                  // query-slot parts per (chunk, kv head) (set by launch_attention)
  float scale_log2;        // log2(e) / sqrt(hd)
  float* part_o;           // [R*nkv][n_chunks][slots][hd]
  float* part_ml;          // [R*nkv][n_chunks][slots][2]
  unsigned* err;
};
hipError_t launch_attention(const AttnArgs& a, int R, hipStream_t st);
int attn_slots(int nq, int nkv, int B);
int attn_chunk_keys(int hd);   // keys per attention chunk

// Second halves of split-K projections: sum the S partial tiles [S][M][ld] in
// split order, then apply the epilogue.
//   resid: h += Y; ssq_out[g * ssq_ld + m] = sum over 128-column group g of h^2
//   silu:  act = SiLU(gate) * up (bf16); gate at column n, up at N + n
//   head:  q/k head RMSNorm + RoPE, Q to q_out, K/V to the ring (GemmArgs head
//          fields), n_heads heads starting at a.head_base, rows a.M
//   store: Y to bf16 or fp32
hipError_t launch_finish_resid(const float* P, int S, int M, int N, float* h, int ldh, float* ssq_out, int ssq_ld,
                               hipStream_t st);
hipError_t launch_finish_silu(const float* P, int S, int M, int N, uint16_t* act, int ldo, hipStream_t st);
hipError_t launch_finish_head(const GemmArgs& a, const float* P, int S, int ld, int n_heads, hipStream_t st);
// the K and V heads of many staged rows (head_dim 64 or 128) from one
// fp32 product P[M][ld] (K heads then V heads): 32 rows of one head per workgroup
hipError_t launch_finish_kv_rows(const GemmArgs& a, const float* P, int ld, hipStream_t st);
hipError_t launch_finish_store(const float* P, int S, int M, int N, void* out, int ldo, int bf16, hipStream_t st);

// Prefill staging (many rows, bf16 weights): the gathered tap rows as bf16, and
// a tiled GEMM Y[M][N] = X[M][K] . W[N][K]^T (K a multiple of 64, N of the
// column tile bn in {64, 128}; fp32 or bf16 out, row pitch ldo).
struct TapGather {
  const float* taps[MAX_TAPS];
  long long tap_stride;
  const int* src_row;   // NULL, or the tap row to read for each output row
  int n_taps, hc, tap_hidden;
  uint16_t* out;   // [M][n_taps * tap_hidden]
};
struct TileArgs {
  const uint16_t* x;
  long long ldx;
  const void* w;             // bf16 [N][K], or packed INT4 [N][K/2] when wscale is set
  int M, N, K;
  void* out;
  long long ldo;
  const uint16_t* wscale;    // INT4 fp16 group scales [N][K/64], or NULL for bf16 weights
};
hipError_t launch_tap_gather(const TapGather& g, int M, hipStream_t st);
int tile_bn(int M, int N, int n_cu);   // 0: N fits neither tile
hipError_t launch_gemm_tile(const TileArgs& a, int bn, int out_bf16, hipStream_t st);
// Y[M][N] = X[M][K] . W[N][K]^T through hipBLASLt (bf16 in, fp32 accumulation,
// bf16 or fp32 out); hipErrorNotSupported when the current device has no handle
// (blaslt_prepare creates it: once per process and device) or the library offers
// no algorithm that needs no workspace (the caller then runs launch_gemm_tile).
hipError_t blaslt_prepare();
hipError_t blaslt_gemm_nt(const uint16_t* x, long long ldx, const uint16_t* w, int M, int N, int K, void* out,
                          long long ldo, int out_f32, hipStream_t st);
// Context K/V projection (N = 2 * nkv * hd, 128-column tiles of whole heads)
// straight into the rings: GemmArgs head fields as for the head finish.
// (n_cu: the device's compute units, which decide the row tile: 256 rows when
// every CU gets at least one such tile, else 128)
hipError_t launch_gemm_tile_heads(const TileArgs& a, const GemmArgs& h, int n_cu, hipStream_t st);

// Verify pass of a causal target: copy the residual rows h [M][H] of a tapped
// layer to a tap buffer with row pitch ld; add n_emit to the positions.
hipError_t launch_copy_rows(const float* h, int M, int H, float* dst, long long ld, hipStream_t st);

// Sampling-mode acceptance (sampling.hip): typical acceptance of the drafts
// against the target's verify logits, card sampling of the next token.
struct SampleArgs {
  const float* logits;     // [R][b][V] target logits of the verify rows
  const int* draft;        // element (r, j) at draft[(r * (b-1) + j) * draft_stride]
  int draft_stride;
  int R, b, V, stats_b, mask_id, eos;
  float T, top_p, eps, delta;   // delta <= 0: sqrt(eps)
  int top_k;                    // 1..64
  uint32_t seed_lo, seed_hi, round;
  const int* budget;
  int *accept_len, *emitted, *n_emit, *next_tokens, *pos;
  unsigned long long* stats;
  int* row_ok;             // workspace [R][b]
  int* cand_idx;           // workspace [R][b][64]
  unsigned* cand_key;      // workspace [R][b][64]: order keys of the row's top-k logits
  int n_chunks;            // ceil(V / SAMPLE_CHUNK)
  unsigned* part_key;      // workspace [R][b][n_chunks][64]: each chunk's top-k (order keys)
  int* part_idx;           //   and ids
  float* part_m;           // workspace [R][b][n_chunks]: chunk max
  double *part_z, *part_s; //   sum exp(x), sum exp(x) x at the chunk max
};
constexpr int SAMPLE_CHUNK = 4096;        // logits per stage-1 workgroup (16 KiB of LDS)
constexpr int SAMPLE_MAX_CHUNKS = 64;     // vocabularies up to 262144
inline int sample_chunks(int V) { return (V + SAMPLE_CHUNK - 1) / SAMPLE_CHUNK; }
hipError_t launch_sampled_accept(const SampleArgs& a, hipStream_t st);

// Candidate trees (tree.hip): build from top-k lists, accept, ancestor masks of
// the tree rows, and the commit of a target's tree pass (K/V of the committed
// nodes to consecutive ring slots).
hipError_t launch_tree_build(const int* block_tokens, int B, const int* ids, const float* vals, int k, int R, int n,
                             int* tok, int* par, int* dep, hipStream_t st);
hipError_t launch_tree_accept(const int* tok, const int* par, int n, const int* verify, int R, int B, int stats_b,
                              int eos, const int* budget, int mask_id, int* accept_len, int* emitted, int* n_emit,
                              int* next_tokens, int* path_nodes, int* stage_rows, int* stage_pos, int* pos,
                              unsigned long long* stats, hipStream_t st);
hipError_t launch_tree_anc(const int* par, int n, int rows, int R, unsigned long long* anc, hipStream_t st);
hipError_t launch_tree_commit(uint16_t* ring_k, uint16_t* ring_v, size_t layer_elems, int L, int R, int nkv, int hd,
                              int C, const int* pos, const int* path_nodes, int path_ld, const int* n_emit,
                              hipStream_t st);
hipError_t launch_advance(int* pos, const int* n_emit, int n_req, hipStream_t st);

// Small kernels.
constexpr int STREAM_READ_BLOCKS = 256;
hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* sink, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_embed(const int* tokens, const uint16_t* embed, float* h, float* ssq, int M, int H,
                        int V, unsigned* err, hipStream_t st);
hipError_t launch_rmsnorm(const float* h, const uint16_t* gain, uint16_t* a, int M, int H,
                          float eps, hipStream_t st);
hipError_t launch_set_pos(int* pos, int* valid_from, int req, int vf, int p, hipStream_t st);
hipError_t launch_accept(const int* draft, int draft_stride, const int* verify, int R, int B, int stats_b,
                         int eos, const int* budget, int mask_id, int* accept_len,
                         int* emitted, int* n_emit, int* next_tokens, int* pos,
                         unsigned long long* stats, hipStream_t st);
