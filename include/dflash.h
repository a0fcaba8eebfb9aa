/*
 * dflash.h - C ABI of the MI355X (gfx950) DFlash block-diffusion drafter round.
 *
 * One draft round is four steps (the method of "[RFC] DFlash", ExecuTorch PR
 * #20840, "DFlash Overview" and "Key Implementation Details", and of "feat:
 * DFlash2 block-diffusion drafter for Qwen 3.8", Mference PR #22, "What's here"):
 *   1. dflash_tap_stage   - gather the target's hidden rows at its tapped layers
 *                           (optionally the per-token mean of hc hyper-connection
 *                           streams, "dflash: the chain verify builds pipelined
 *                           ...", mlx-serve PR #937, hc commit), concatenate,
 *                           fc-project to the draft hidden size and write every
 *                           draft layer's context K/V into a per-request ring.
 *   2/3. dflash_draft_block - a masked block of B tokens through every draft
 *                           layer in one forward (attention over [sliding context
 *                           window | bidirectional block]), the shared LM head,
 *                           then argmax or top-16 per mask position.
 *   4. dflash_accept      - first-mismatch acceptance against the target's verify
 *                           argmaxes plus the bonus token, EOS/budget clamps, and
 *                           the context position update (rollback is implicit:
 *                           only rows below pos are ever read).
 *
 * Conventions
 *   - Every pointer argument is a DEVICE pointer unless marked "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call below except dflash_check enqueues asynchronously on it and never
 *     synchronizes, allocates or frees; callers may capture rounds in a HIP graph
 *     (nothing in a round uses hipMemsetAsync).
 *   - The library allocates no device memory. Weights, taps, state, workspace and
 *     outputs belong to the caller (e.g. PyTorch tensors) and must outlive the
 *     handle. The handle stores the config and borrowed pointers only.
 *     One exception: a staging call of at least 256 rows with bf16 weights runs
 *     its fc and context K/V products through hipBLASLt. dflash_bind of such a
 *     drafter creates the device's hipBLASLt handle (once per process and device:
 *     the library's own internal buffers), and hipBLASLt loads its kernels the
 *     first time a staging shape runs. Nothing in a draft round (draft, accept, reset, check, staging of
 *     fewer than 256 rows) allocates.
 *   - One handle = one state + one workspace; calls on one handle must be ordered
 *     (one stream, or events between streams). Two handles never share a workspace.
 *   - Errors: host-side validation runs before any launch and returns a negative
 *     dflash_status; dflash_last_error() gives a message (thread-local). Values
 *     that live on the device (tokens, positions) are checked in the kernels: a bad
 *     value is skipped or clamped and sets a sticky bit in the device error word,
 *     which dflash_check() returns as DFLASH_E_DEVICE.
 *   - Layouts are row-major. Linear weights are [out, in] (torch Linear).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_ARG = -1,         /* null/invalid argument                              */
  DFLASH_E_CONFIG = -2,      /* inconsistent configuration (checked at create)     */
  DFLASH_E_SHAPE = -3,       /* call shape outside what the config allows          */
  DFLASH_E_CAPACITY = -4,    /* more rows/requests than state/workspace can hold   */
  DFLASH_E_UNSUPPORTED = -5, /* a valid request this build does not implement      */
  DFLASH_E_HIP = -6,         /* a HIP runtime call failed                          */
  DFLASH_E_DEVICE = -7,      /* the device error word is non-zero (dflash_check)   */
  DFLASH_E_STATE = -8        /* handle not bound to state/workspace                */
} dflash_status;

/* Weight format of fc and the per-layer projections (embedding and LM head are bf16). */
typedef enum { DFLASH_W_BF16 = 0, DFLASH_W_INT4_G64 = 1 } dflash_wfmt;

/* Device error word bits (sticky until dflash_bind or dflash_clear_error). */
enum {
  DFLASH_DEV_BAD_TOKEN = 1,      /* a block token outside [0, vocab): row 0 of embed used */
  DFLASH_DEV_BAD_WINDOW = 2,     /* valid_from > pos: the context is treated as empty      */
  DFLASH_DEV_BAD_ROW = 4,        /* a staged row names a request outside [0, max_requests) */
  DFLASH_DEV_BAD_POSITION = 8,   /* a negative position: the row is skipped                */
  /* A K/V row (staged, or a block's own) whose ring slot belongs to another live
   * row of its request: the live positions are the window and the block,
   * [pos - window, pos + block), so a row at p is written only if
   * pos + block - ring_capacity <= p < pos + ring_capacity - window (pos = the
   * request's state position at the time of the call). Outside that range the
   * row is skipped and the ring is left as it was. The capacity bound is a hard
   * bound ("[RFC] DFlash", ExecuTorch PR #20840, author's reply on the draft
   * cache's capacity). */
  DFLASH_DEV_RING_CAPACITY = 16
};

/*
 * Drafter configuration (host struct, copied at create).
 *   n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab:
 *       Qwen3-shaped draft layers ("[RFC] DFlash" review threads: the drafter
 *       reuses Qwen3 attention / RMSNorm / MLP / rotary embedding).
 *   n_taps, hc_streams, tap_hidden:
 *       tapped target layers; each tap row is hc_streams*tap_hidden fp32 values,
 *       stream-major; fc input width = n_taps*tap_hidden. tap_hidden must equal
 *       hidden: the drafter shares the target's embedding and LM head, and the
 *       guard that validates the hidden size before any buffer is built is the
 *       one the Mference PR adds (hidden_size guard commit).
 *   block:         B, tokens per draft block (1..64); row 0 is the known token.
 *   window:        W, context rows attended (sliding window over committed rows).
 *   ring_capacity: C, ring slots per request and layer; C >= W + B, C % 32 == 0.
 *   max_requests:  R_max, requests the state holds.
 *   mask_id:       token id of the mask positions (used by dflash_accept).
 *   rope_theta, rms_eps: RoPE base and RMSNorm epsilon.
 *   ctx_norm:      1 = RMSNorm (gain weights.ctx_norm) after fc; 0 = none.
 *   wfmt:          dflash_wfmt.
 *   max_stage_rows: most rows one dflash_tap_stage call may stage (sizes workspace).
 */
typedef struct {
  int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int n_taps, hc_streams, tap_hidden;
  int block, window, ring_capacity, max_requests, mask_id;
  float rope_theta, rms_eps;
  int ctx_norm;
  int wfmt;
  int max_stage_rows;
} dflash_config;

/*
 * Weights: device pointers, borrowed. Per-layer fields are HOST arrays of
 * n_layers device pointers.
 *   embed, lm_head: bf16 [vocab, hidden] (the target's; may be the same pointer).
 *   fc:             [hidden, n_taps*tap_hidden]
 *   wqkv[l]:        [(n_q_heads + 2*n_kv_heads)*head_dim, hidden] = [Wq; Wk; Wv]
 *   wo[l]:          [hidden, n_q_heads*head_dim]
 *   wgu[l]:         [2*ffn, hidden] = [Wgate; Wup]
 *   wd[l]:          [hidden, ffn]
 *   For DFLASH_W_BF16 these are bf16. For DFLASH_W_INT4_G64 they are packed INT4
 *   (uint8 [rows, in/2], `in` a multiple of 128) with fp16 scales *_scales
 *   [rows, in/64]. Packing: per row, in 128-wide chunks c, little-endian 32-bit
 *   word 4*j + s (j, s = 0..3) holds the values k = 128c + 32s + 8j + e, e = 0..7,
 *   as u = q + 8 in [0, 15]; value e sits in nibble e/2 (e even) or 4 + (e-1)/2
 *   (e odd). The weight is q * scale.
 *   ln_in[l], ln_post[l]: bf16 [hidden]; q_norm[l], k_norm[l]: bf16 [head_dim];
 *   final_norm: bf16 [hidden]; ctx_norm: bf16 [hidden] (read only if cfg.ctx_norm).
 *   Every pointer is 16-byte aligned (the kernels read in 16-byte pieces;
 *   dflash_create refuses others with DFLASH_E_ARG).
 */
typedef struct {
  const void* embed;
  const void* lm_head;
  const void* fc;
  const void* fc_scales;
  const void* ctx_norm;
  const void* final_norm;
  const void* const* wqkv;
  const void* const* wqkv_scales;
  const void* const* wo;
  const void* const* wo_scales;
  const void* const* wgu;
  const void* const* wgu_scales;
  const void* const* wd;
  const void* const* wd_scales;
  const void* const* ln_in;
  const void* const* ln_post;
  const void* const* q_norm;
  const void* const* k_norm;
} dflash_weights;

/* Byte offsets of the state sections (for inspection by tests and tools). */
typedef struct {
  size_t pos;         /* int32 [max_requests]: absolute position of block token 0  */
  size_t valid_from;  /* int32 [max_requests]: first valid context position        */
  size_t error;       /* uint32: device error word                                 */
  size_t stats;       /* uint64 [block + 2]: [0] rounds, [1+i] rounds with accept  */
                      /*   length > i (i = 0..block-1), [block+1] tokens emitted    */
  size_t ring_k;      /* bf16 [n_layers][max_requests][n_kv_heads][C][head_dim]    */
  size_t ring_v;      /* bf16 [n_layers][max_requests][n_kv_heads][head_dim][C]    */
  size_t total;
} dflash_state_layout;

typedef struct dflash_ctx dflash_ctx;

/* Validate `cfg` (and the non-null pointers of `w`) and make a handle. No device calls. */
int dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_ctx** out);
void dflash_destroy(dflash_ctx* ctx);

/* Sizes the caller allocates (any alignment >= 256 bytes). 0 on an invalid config. */
size_t dflash_state_bytes(const dflash_config* cfg);
size_t dflash_workspace_bytes(const dflash_config* cfg);
int dflash_get_state_layout(const dflash_config* cfg, dflash_state_layout* out);

/* Attach state and workspace; zero-fills both on `stream` (a kernel, no memset). */
int dflash_bind(dflash_ctx* ctx, void* state, void* workspace, void* stream);

/* Continuity break / prefill start for request `req`: valid_from = `valid_from`,
 * pos = `pos` (the Mference PR resets the drafter with realigned positions on
 * plain-decode gaps and rewinds). Requires 0 <= valid_from <= pos. */
int dflash_reset(dflash_ctx* ctx, void* stream, int req, int valid_from, int pos);

/*
 * Stage n_rows tap rows: x = concat_t mean_s taps[t][row, s*tap_hidden : ...]
 * (bf16), c = fc(x) (+ ctx RMSNorm), and for every layer K = RoPE(k_norm(W_k c),
 * position), V = W_v c written to ring slot position % C of the row's request.
 *   taps:        HOST array [n_taps] of device pointers; taps[t] + row*tap_row_stride
 *                is row `row` (fp32, hc_streams*tap_hidden values).
 *   tap_row_stride: elements between rows (>= hc_streams*tap_hidden, % 4 == 0).
 *   req_of_row:  [n_rows] int32 or NULL (then request = row / rows_per_req).
 *   pos_of_row:  [n_rows] int32 or NULL (then position = pos[request] +
 *                row % rows_per_req, read from the state on the device).
 *   rows_per_req: used only where the arrays above are NULL (>= 1).
 * The verify rows of a round are staged at [pos, pos+B) before dflash_accept;
 * rows the accept does not commit are overwritten later and never read.
 */
int dflash_tap_stage(dflash_ctx* ctx, void* stream, const float* const* taps,
                     long long tap_row_stride, int n_rows, const int* req_of_row,
                     const int* pos_of_row, int rows_per_req);

/*
 * Draft one block per request r < n_req from block_tokens [n_req, B] (int32;
 * token 0 known, the rest mask ids) at positions pos[r] + i, attending to the
 * context rows [max(valid_from[r], pos[r] - W), pos[r]) and to all B block rows.
 *   logits:    NULL or fp32 [n_req, B-1, vocab] (rows 1..B-1)
 *   topk_ids:  int32 [n_req, B-1, k], ordered by (logit desc, id asc)
 *   topk_vals: NULL or fp32 [n_req, B-1, k]
 *   k:         1 (argmax) or 16.
 * The block's own K/V are written to ring slots [pos, pos+B) (slots the next
 * stage overwrites), so the ring must not be read there by anyone else.
 */
int dflash_draft_block(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req,
                       float* logits, int* topk_ids, float* topk_vals, int k);

/*
 * dflash_draft_block with a per-call block length b = block_len in [1, cfg.block]
 * in place of cfg.block: every shape above uses b (block_tokens [n_req, b], b-1
 * drafted rows). For the shrunk last rounds of a generation: the block length
 * of a round is min(block size, tokens still to generate, sequence capacity
 * left) ("[RFC] DFlash", ExecuTorch PR #20840: the review item on a dynamic
 * block length and the author's reply). b = 1 drafts nothing (a target-only
 * step).
 */
int dflash_draft_block_n(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req,
                         int block_len, float* logits, int* topk_ids, float* topk_vals, int k);

/*
 * dflash_draft_block for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same arguments and the same kernels, but the call's scratch (residual rows,
 * split-K partials, attention chunk partials, the LM head's logits hand-off)
 * lives in a static device array of the library, DFLASH_STATIC_SCRATCH_BYTES
 * (64 MiB) on each GPU the library runs on, held until the process ends,
 * instead of the bound workspace. The call allocates and frees nothing.
 *   - A configuration whose draft needs more scratch than that
 *     (dflash_draft_scratch_bytes) is refused with DFLASH_E_CAPACITY before any
 *     launch. The state (ring, positions) is still the handle's bound state.
 *   - Every call on one GPU, from any handle, uses that GPU's one array, which
 *     keeps the last call's contents; nothing in it needs to start at zero
 *     (each section a call reads is written earlier in the same call). Calls
 *     that overlap on one GPU (two streams, two threads) race on the array:
 *     order them.
 * The device address of the array is looked up once per device, on the
 * device's first call.
 */
#define DFLASH_STATIC_SCRATCH_BYTES (64u << 20)
int dflash_draft_block_noalloc(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req,
                               float* logits, int* topk_ids, float* topk_vals, int k);
/* Scratch bytes dflash_draft_block_noalloc needs for `cfg` (0 on an invalid config). */
size_t dflash_draft_scratch_bytes(const dflash_config* cfg);

/*
 * First-mismatch accept for requests r < n_req.
 *   draft_ids:   element (r, j) at draft_ids[(r*(B-1) + j)*draft_stride], j < B-1
 *                (pass topk_ids with draft_stride = k).
 *   verify_ids:  int32 [n_req, B], the target's argmax at each verify row.
 *   eos_id:      < 0 disables EOS truncation.
 *   budget:      NULL or int32 [n_req]: most tokens to emit (values < 1 act as 1).
 * Outputs: accept_len [n_req], emitted [n_req, B] (padded with -1), n_emit [n_req];
 * next_tokens (NULL or [n_req, B]) = [last emitted, mask_id, ...]. The state's
 * pos[r] advances by n_emit[r]; accept-profile counters are updated.
 */
int dflash_accept(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride,
                  const int* verify_ids, int n_req, int eos_id, const int* budget,
                  int* accept_len, int* emitted, int* n_emit, int* next_tokens);

/*
 * dflash_accept for a round drafted with block length b = block_len in
 * [1, cfg.block] (dflash_draft_block_n): draft_ids hold b-1 drafts per request,
 * verify_ids [n_req, b], emitted and next_tokens [n_req, b]. b = 1 emits the
 * target's token verify_ids[r][0]. The accept-profile counters keep the layout
 * of the configured block.
 */
int dflash_accept_n(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride,
                    const int* verify_ids, int n_req, int block_len, int eos_id, const int* budget,
                    int* accept_len, int* emitted, int* n_emit, int* next_tokens);

/*
 * Sampling-mode acceptance (the pages run the drafter with "typical 0.2" and
 * card sampling T 1.0, top-p 0.95, top-k 20: "dflash: the chain verify builds
 * pipelined ...", mlx-serve PR #937, "Measured"; the pages give no formulas).
 * For request r and verify row i (target logits z = target_logits[r][i][:],
 * fp32, e.g. dflash_verify_block's logits output): p = softmax(z / T), H =
 * -sum p log p; draft token i is accepted iff p(draft) > min(eps, delta *
 * exp(-H)) (delta <= 0 means sqrt(eps)), and acceptance stops at the first
 * rejected row a (a = b-1 if none). The next token is drawn from row a: its
 * top_k logits (value desc, index asc), q = softmax(z / T) over them (fp64),
 * the shortest prefix whose q sum reaches top_p, and in it the first token
 * whose running q sum exceeds u * the prefix's sum, with u = (word 0 >> 8) *
 * 2^-24 of Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as
 * 1, 2, 3", SC 2011) at key = seed, counter = (round, r, a, 0). Emitted =
 * accepted drafts + that token; EOS, budget, pos, next_tokens and the
 * statistics as in dflash_accept_n. Decisions within about 1e-6 (relative) of
 * the acceptance threshold may differ from an fp64 evaluation: the row sums
 * are fp32 exponentials added in fp64.
 */
typedef struct {
  float temperature;     /* > 0 */
  int top_k;             /* 1..64 */
  float top_p;           /* (0, 1] */
  float typical_eps;     /* >= 0; 0 accepts every draft */
  float typical_delta;   /* <= 0: sqrt(typical_eps) */
} dflash_sampling;

int dflash_accept_sampled(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride,
                          const float* target_logits, int n_req, int block_len, const dflash_sampling* params,
                          unsigned long long seed, unsigned round, int eos_id, const int* budget,
                          int* accept_len, int* emitted, int* n_emit, int* next_tokens);

/*
 * Adaptive block length (the round policy of "dflash: the chain verify builds
 * pipelined ...", mlx-serve PR #937, hyper-connection-stream commit, whose rule
 * the pages do not give). Host-side, one per request: an exponential average m
 * of the accepted drafts, m <- (1 - weight) m + weight * accepted, starting at
 * block - 1; the next round's block length is clamp(floor(m + 1/2) + 2, 2,
 * block), for dflash_draft_block_n / dflash_accept_n. A serving loop reads each
 * round's accept lengths anyway (it streams the emitted tokens), so the policy
 * needs no extra synchronization.
 */
typedef struct {
  int block;
  double weight;
  double mean;
} dflash_block_policy;
void dflash_policy_init(dflash_block_policy* p, int block, double weight);
int dflash_policy_next(const dflash_block_policy* p);
void dflash_policy_update(dflash_block_policy* p, int accepted);

/*
 * Causal target (the verify side of the loop). A target handle is created from
 * the same config and weight structs (fc, fc_scales and ctx_norm are not used):
 * a Qwen3-shaped causal decoder whose own per-layer K/V live in the ring of its
 * state, at slot position mod ring_capacity, over the window of the config.
 * The verify pass runs the B rows of the round (the last emitted token and the
 * drafts) through every layer with block row i attending to ring rows
 * [max(valid_from, pos - window), pos) and to block rows j <= i (a target with
 * full attention sets window >= its longest sequence), writes the block's K/V to ring slots [pos, pos+B), returns
 * the argmax (lowest id on ties) of every row, and copies the residual rows
 * after the tapped layers, which are the drafter's taps ("[RFC] DFlash",
 * ExecuTorch PR #20840, "Key Implementation Details": the target returns its
 * selected layers' hidden rows with the verify logits; "feat: DFlash2", Mference
 * PR #22, the commit on verify staging tap rows for the drafter). Rows the
 * accept does not commit are overwritten by the next pass (rollback is moving
 * pos: dflash_advance adds the accept's n_emit, dflash_reset restarts).
 */
int dflash_create_target(const dflash_config* cfg, const dflash_weights* w, dflash_ctx** out);

/*
 * Verify pass of a target handle for requests r < n_req at positions pos[r] + i,
 * i < b = block_len in [1, cfg.block].
 *   block_tokens: int32 [n_req, b].
 *   tap_layers:   NULL or HOST int[n_tap_out], layer indices in [0, n_layers):
 *                 tap t receives the residual after layer tap_layers[t].
 *   tap_out:      NULL or HOST array of n_tap_out device pointers, each fp32
 *                 [n_req * b] rows of pitch tap_ld (>= hidden, % 4 == 0),
 *                 16-byte aligned; row r*b + i is block row i of request r.
 *   logits:       NULL or fp32 [n_req, b, vocab].
 *   ids:          int32 [n_req, b], argmax of every row.
 */
int dflash_verify_block(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req, int block_len,
                        const int* tap_layers, int n_tap_out, float* const* tap_out, long long tap_ld,
                        float* logits, int* ids);

/*
 * Candidate trees from the drafter's top-k lists (tree speculation). The pages
 * keep top-16 candidates per draft position and hand them to a path selector
 * ("feat: DFlash2 block-diffusion drafter for Qwen 3.8", Mference PR #22,
 * "What's here" and the Metal-port commit; a tree verify round appears in
 * "dflash: the chain verify builds pipelined ...", mlx-serve PR #937) without
 * giving its rule. The rule here: node 0 is the root (block token 0 of the
 * request); a node at depth d holds one of the k candidates of draft position
 * d and its children are the candidates of position d + 1; candidate j of a
 * list has log-probability lp = (v[j] - v[0]) - log(sum_j' exp(v[j'] - v[0]))
 * (fp64, list order) and a node's score is the sum of lp along its path. The
 * tree is the root, the top-1 chain (up to depth min(block - 1, n_nodes - 1)),
 * then, best first, the highest-scoring child of any node in the tree, ties
 * to the smaller depth, then the smaller parent index, then the smaller rank;
 * nodes are numbered in that order (a parent precedes its children).
 *   block_tokens: [n_req, block]; topk_ids / topk_vals: [n_req, block-1, k], as
 *                 dflash_draft_block writes them (k in [1, 16]);
 *   n_nodes:      1..64, at most the number of nodes the lists offer;
 *   tree_tokens, tree_parent (-1 for the root), tree_depth: int32 [n_req, n_nodes].
 */
int dflash_tree_build(dflash_ctx* ctx, void* stream, const int* block_tokens, const int* topk_ids,
                      const float* topk_vals, int k, int n_req, int n_nodes, int* tree_tokens,
                      int* tree_parent, int* tree_depth);

/*
 * Tree-masked verify pass of a target handle: node i of request r is a row at
 * position pos[r] + tree_depth[r][i] that attends to the window and to its own
 * ancestors (itself included); its K/V go to ring slot pos[r] + i. Outputs as
 * dflash_verify_block with block_len = n_nodes (n_nodes <= cfg.block): ids
 * [n_req, n_nodes] = the target's greedy next token after each node's path,
 * tap rows [n_req * n_nodes] (pitch tap_ld), optional logits. Follow with
 * dflash_tree_commit once the accept is known.
 */
int dflash_verify_tree(dflash_ctx* ctx, void* stream, const int* tree_tokens, const int* tree_parent,
                       const int* tree_depth, int n_req, int n_nodes, const int* tap_layers, int n_tap_out,
                       float* const* tap_out, long long tap_ld, float* logits, int* ids);

/*
 * Tree accept on a drafter handle: from the root, move to the child whose
 * token equals the target's token at the current node (verify_ids [n_req,
 * n_nodes] from dflash_verify_tree), while one exists; emitted = the walked
 * tokens then the target's token at the last node; EOS/budget clamps as in
 * dflash_accept; pos[r] += n_emit[r]. Outputs (int32, [n_req, cfg.block] unless
 * noted): accept_len [n_req], emitted (padded with -1), n_emit [n_req],
 * next_tokens (nullable) = [last emitted, mask_id, ...], path_nodes = the
 * committed nodes (root first; entries past n_emit repeat the last one),
 * stage_rows = r * n_nodes + path_nodes (the verify tap rows to stage) and
 * stage_pos = the old pos[r] + d: the arguments of dflash_tap_stage_rows for
 * the committed rows (entries past n_emit stage at positions the next round
 * overwrites, as the chain's rejected verify rows are).
 */
int dflash_tree_accept(dflash_ctx* ctx, void* stream, const int* tree_tokens, const int* tree_parent, int n_nodes,
                       const int* verify_ids, int n_req, int eos_id, const int* budget, int* accept_len,
                       int* emitted, int* n_emit, int* next_tokens, int* path_nodes, int* stage_rows,
                       int* stage_pos);

/*
 * Commit of a target's tree pass: for every layer, the K/V of node
 * path_nodes[r][d] (ring slot pos + node) moves to slot pos + d, d < n_emit[r];
 * then pos[r] += n_emit[r]. path_nodes: [n_req, path_ld] (dflash_tree_accept's,
 * path_ld = the drafter's block).
 */
int dflash_tree_commit(dflash_ctx* ctx, void* stream, const int* path_nodes, int path_ld, const int* n_emit,
                       int n_req);

/*
 * dflash_tap_stage where row m of the call reads tap row src_row[m] (device
 * int32 [n_rows]) of the tap buffers: stages a subset of a verify pass's rows,
 * e.g. the committed nodes of a tree pass (dflash_tree_accept's stage_rows with
 * pos_of_row = its stage_pos and rows_per_req = the drafter's block).
 */
int dflash_tap_stage_rows(dflash_ctx* ctx, void* stream, const float* const* taps, long long tap_row_stride,
                          int n_rows, const int* src_row, const int* req_of_row, const int* pos_of_row,
                          int rows_per_req);

/* pos[r] += n_emit[r] for r < n_req (n_emit: device int32 [n_req], e.g. the
 * drafter's dflash_accept output), enqueued on `stream`: commits a target's
 * accepted rows. */
int dflash_advance(dflash_ctx* ctx, void* stream, const int* n_emit, int n_req);

/* Synchronize `stream`, read the device error word into *word (host, may be NULL);
 * returns DFLASH_E_DEVICE if it is non-zero. */
int dflash_check(dflash_ctx* ctx, void* stream, unsigned* word);
/* Clear the device error word (enqueued on `stream`). */
int dflash_clear_error(dflash_ctx* ctx, void* stream);

/* Kernel classes for timing. */
enum {
  DFLASH_K_LMHEAD = 0, DFLASH_K_QKV = 1, DFLASH_K_O = 2, DFLASH_K_GATEUP = 3,
  DFLASH_K_DOWN = 4, DFLASH_K_ATTN = 5, DFLASH_K_FC = 6, DFLASH_K_STAGE_KV = 7,
  DFLASH_K_COUNT = 8
};
/* Record caller-created hipEvents (passed as void*) around every later launch of
 * kernel class `kclass`: launch number i uses pair i % n. n = 0 turns it off.
 * `before`/`after` are HOST arrays of n events, borrowed until turned off. */
int dflash_set_timing_events(dflash_ctx* ctx, int kclass, void* const* before,
                             void* const* after, int n);

/* Measurement reference, not part of the round: read `bytes` (a multiple of 16)
 * of device memory at `src` (16-byte aligned) once with a plain streaming-read
 * kernel of this library (256 workgroups, eight nontemporal 16-byte loads in
 * flight per thread), enqueued on `stream`; its duration against `bytes` is
 * the HBM read rate the round's kernels are compared with beside the vendor
 * peak. `sink`: device uint32[1024] (the first 256 are written) that receives
 * an XOR of what each workgroup read (contents meaningless; it keeps the loads live). */
int dflash_stream_read(const void* src, size_t bytes, unsigned* sink, void* stream);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
