// Host side of the C ABI declared in include/dflash.h: configuration guards,
// state/workspace layout and the per-call launch sequences. No device memory is
// allocated here; every launch goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// K chunks (of 128) per split of each projection, measured best on MI355X at the
// qwen3-4b shape with 16 rows: about 2-4 chunks keeps a few hundred workgroups
// streaming while the partial tiles stay small.
enum Proj { P_QKV, P_O, P_GATEUP, P_DOWN, P_FC, P_STAGE_KV };
constexpr int CPS_BF16[] = {2, 3, 4, 3, 4, 2};
// INT4 chunks carry a quarter of the bytes; measured best at the qwen3-8b
// shape with 8 rows (hidden 4096, ffn 12288)
constexpr int CPS_INT4[] = {6, 4, 8, 4, 4, 2};
constexpr int GC_DEFAULT = 128;

int wf_of(const dflash_config& c) { return c.wfmt == DFLASH_W_INT4_G64 ? WF_INT4 : WF_BF16; }
GemmPlan plan_for(const dflash_config& c, int M, int N, int K, int gc, int pair, Proj pj) {
  const int cps = c.wfmt == DFLASH_W_INT4_G64 ? CPS_INT4[pj] : CPS_BF16[pj];
  return plan_gemm(M, N, K, gc, pair, cps, wf_of(c));
}

// Rows [row, ...) of a projection matrix [N][K]: bf16 rows of K elements, or
// packed INT4 rows of K/2 bytes with fp16 scale rows of K/64.
const void* w_rows(const dflash_config& c, const uint16_t* w, size_t row, int K) {
  if (c.wfmt == DFLASH_W_INT4_G64) return (const uint8_t*)w + row * (size_t)(K / 2);
  return w + row * (size_t)K;
}
const uint16_t* s_rows(const uint16_t* s, size_t row, int K) { return s ? s + row * (size_t)(K / 64) : nullptr; }

// Staging calls of at least this many rows take the prefill path: tap gather,
// then tiled GEMMs for fc and each layer's context K/V.
constexpr int PREFILL_MIN_ROWS = 256;
bool prefill_enabled(const dflash_config& c) {
  // fc in 64- or 128-column tiles; context K/V in 128-column tiles of whole heads
  return c.max_stage_rows >= PREFILL_MIN_ROWS && tile_bn(PREFILL_MIN_ROWS, c.hidden, 256) != 0 &&
         (c.n_kv_heads * c.head_dim) % 128 == 0 && 128 % c.head_dim == 0;
}

int attn_nchunks(const dflash_config& c) {
  const int kc = attn_chunk_keys(c.head_dim);
  return (c.window + c.block + 31 + kc - 1) / kc;
}

struct WsLayout {
  size_t h, ssq, q, o, act, z, c32, c, xg, partials, attn_o, attn_ml, logits, gmax, anc, row_ok, cand_idx,
      cand_key, part_key, part_idx, part_m, part_z, part_s, total;
};

struct GemmShape {
  int N, K, gc, pair;
  Proj pj;
};

// Layers per stage K/V launch: split-K launches batch up to MAX_BATCH layers
// while their partial tiles fit the budget.
int stage_batch(const GemmPlan& p, int M, int N, int n_layers) {
  if (p.S <= 1) return 1;
  const long long one = (long long)gemm_partial_floats(p, M, N, 0);
  int b = n_layers < MAX_BATCH ? n_layers : MAX_BATCH;
  while (b > 1 && one * b > GEMM_PARTIAL_BUDGET) --b;
  return b;
}

// Largest split-K partial buffer over every GEMM a call may launch (with
// draft_only, over the block forward's projections alone).
size_t gemm_scratch(const dflash_config& c, bool draft_only = false) {
  const int H = c.hidden, hd = c.head_dim;
  const GemmShape draft[] = {{(c.n_q_heads + 2 * c.n_kv_heads) * hd, H, hd, 0, P_QKV},
                             {H, c.n_q_heads * hd, GC_DEFAULT, 0, P_O},
                             {c.ffn, H, GC_DEFAULT, 1, P_GATEUP},
                             {H, c.ffn, GC_DEFAULT, 0, P_DOWN}};
  const GemmShape stage[] = {{H, c.n_taps * c.tap_hidden, GC_DEFAULT, 0, P_FC},
                             {2 * c.n_kv_heads * hd, H, hd, 0, P_STAGE_KV}};
  size_t pf = 0;
  auto visit = [&](int M, const GemmShape& s, bool batched) {
    GemmPlan p = plan_for(c, M, s.N, s.K, s.gc, s.pair, s.pj);
    const int layers = batched ? stage_batch(p, M, s.N, c.n_layers) : 1;
    size_t f = gemm_partial_floats(p, M, s.N, s.pair) * layers;
    if (f > pf) pf = f;
  };
  for (int R = 1; R <= c.max_requests; ++R)
    for (const auto& s : draft) visit(R * c.block, s, false);
  for (int M = 1; M <= (draft_only ? 0 : c.max_stage_rows); ++M) {
    visit(M, stage[0], false);
    visit(M, stage[1], true);
  }
  return pf;
}

// Workspace sections. With draft_only, only what a block forward (draft or
// verify pass) uses: the staging sections (c, c32, xg) are empty and the
// split-K partials cover the block forward's projections alone.
WsLayout ws_layout(const dflash_config& c, bool draft_only = false) {
  WsLayout L;
  const size_t Mmax = (size_t)c.max_requests * c.block;
  const size_t S = draft_only ? 0 : (size_t)c.max_stage_rows;
  const size_t qw = (size_t)c.n_q_heads * c.head_dim;
  const size_t pf = gemm_scratch(c, draft_only);
  const size_t slots = (size_t)attn_slots(c.n_q_heads, c.n_kv_heads, c.block);
  const size_t lrg = (size_t)c.max_requests * c.n_kv_heads;
  const size_t nch = (size_t)attn_nchunks(c);
  const size_t out_rows = Mmax;   // LM-head output rows: the mask rows of a draft, every row of a verify pass
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.h = take(Mmax * c.hidden * 4);
  L.ssq = take((size_t)(c.hidden / GC_DEFAULT) * Mmax * 4);
  L.q = take(Mmax * qw * 2);
  L.o = take(Mmax * qw * 2);
  L.act = take(Mmax * c.ffn * 2);
  L.z = take(Mmax * c.hidden * 2);   // final-normed rows (LM head without LDS staging)
  L.c32 = take(c.ctx_norm ? S * c.hidden * 4 : 0);
  L.c = take(S * c.hidden * 2);
  // gathered tap rows as bf16: the prefill path, and every staging call when
  // the taps carry several hyper-connection streams
  L.xg = take(!draft_only && (prefill_enabled(c) || c.hc_streams > 1) ? S * c.n_taps * c.tap_hidden * 2 : 0);
  L.partials = take((pf ? pf : 1) * 4);
  L.attn_o = take(lrg * nch * slots * c.head_dim * 4);
  L.attn_ml = take(lrg * nch * slots * 2 * 4);
  const size_t lm_rows = Mmax <= 16 ? 16 : (Mmax <= 32 ? 32 : 64 * ((Mmax + 63) / 64));
  L.logits = take(lm_rows * c.vocab * 4);           // transposed logits when the caller passes none
  L.gmax = take(out_rows * ((c.vocab + 15) / 16) * 4);   // per-16-column maxima of the logits
  L.anc = take(Mmax * 8);                                  // ancestor masks of a tree pass's rows
  L.row_ok = take(Mmax * 4);                               // sampled accept: per-row test of the draft
  L.cand_idx = take(Mmax * 64 * 4);                        // sampled accept: each row's top-k ids
  L.cand_key = take(Mmax * 64 * 4);                        // and their logits (order keys)
  const size_t sch = (size_t)sample_chunks(c.vocab);       // sampled accept, per chunk of the vocabulary:
  L.part_key = take(Mmax * sch * 64 * 4);                  //   the chunk's top-k keys
  L.part_idx = take(Mmax * sch * 64 * 4);                  //   and ids,
  L.part_m = take(Mmax * sch * 4);                         //   its max,
  L.part_z = take(Mmax * sch * 8);                         //   sum of exp
  L.part_s = take(Mmax * sch * 8);                         //   and sum of exp * x
  L.total = off;
  return L;
}

dflash_state_layout st_layout(const dflash_config& c) {
  dflash_state_layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.pos = take((size_t)c.max_requests * 4);
  L.valid_from = take((size_t)c.max_requests * 4);
  L.error = take(4);
  L.stats = take((size_t)(c.block + 2) * 8);
  const size_t ring = (size_t)c.n_layers * c.max_requests * c.n_kv_heads * c.ring_capacity * c.head_dim * 2;
  L.ring_k = take(ring);
  L.ring_v = take(ring);
  L.total = off;
  return L;
}

int validate_config(const dflash_config* c) {
  if (!c) return fail(DFLASH_E_ARG, "config is NULL");
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->ffn < 1 || c->vocab < 2)
    return fail(DFLASH_E_CONFIG, "layer/width/vocab sizes must be positive (vocab >= 2)");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(DFLASH_E_CONFIG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  if (c->head_dim % 2) return fail(DFLASH_E_CONFIG, "head_dim must be even for RoPE");
  if (c->n_taps < 1 || c->n_taps > MAX_TAPS || c->hc_streams < 1 || c->tap_hidden < 1)
    return fail(DFLASH_E_CONFIG, "n_taps must be in [1, %d], hc_streams and tap_hidden positive", MAX_TAPS);
  if (c->tap_hidden != c->hidden)
    return fail(DFLASH_E_CONFIG, "tap_hidden (%d) must equal hidden (%d): the drafter shares the target's "
                "embedding and LM head and reads its hidden rows", c->tap_hidden, c->hidden);
  if (c->block < 1 || c->block > 64) return fail(DFLASH_E_CONFIG, "block must be in [1, 64]");
  if (c->window < 0) return fail(DFLASH_E_CONFIG, "window must be >= 0");
  if (c->ring_capacity < c->window + c->block || c->ring_capacity % 32)
    return fail(DFLASH_E_CONFIG, "ring_capacity (%d) must be >= window + block (%d) and a multiple of 32",
                c->ring_capacity, c->window + c->block);
  if (c->max_requests < 1) return fail(DFLASH_E_CONFIG, "max_requests must be >= 1");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(DFLASH_E_CONFIG, "mask_id outside [0, vocab)");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(DFLASH_E_CONFIG, "rope_theta > 0 and rms_eps >= 0 required");
  if (c->max_stage_rows < 1) return fail(DFLASH_E_CONFIG, "max_stage_rows must be >= 1");
  if (c->wfmt != DFLASH_W_BF16 && c->wfmt != DFLASH_W_INT4_G64) return fail(DFLASH_E_CONFIG, "unknown weight format %d", c->wfmt);
  // shapes the kernels are built for
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_E_UNSUPPORTED, "head_dim %d: kernels are built for 64 and 128", c->head_dim);
  if (c->hidden % 128 || c->ffn % 128 || (c->n_q_heads * c->head_dim) % 128)
    return fail(DFLASH_E_UNSUPPORTED, "hidden, ffn and n_q_heads*head_dim must be multiples of 128");
  if (c->max_requests * c->block > 64)
    return fail(DFLASH_E_UNSUPPORTED, "max_requests * block = %d block rows; the LM-head kernel holds at most 64",
                c->max_requests * c->block);
  if (attn_slots(c->n_q_heads, c->n_kv_heads, c->block) > 64)
    return fail(DFLASH_E_UNSUPPORTED, "(n_q_heads/n_kv_heads)*block = %d query rows per kv head; at most 64",
                attn_slots(c->n_q_heads, c->n_kv_heads, c->block));
  if (c->vocab > 256 * 64 * 16)
    return fail(DFLASH_E_UNSUPPORTED, "vocab %d exceeds the top-k selection capacity (%d)", c->vocab, 256 * 64 * 16);
  return DFLASH_OK;
}

struct Timing {
  std::vector<hipEvent_t> before, after;
  unsigned long long count = 0;
};

}  // namespace

struct dflash_ctx {
  dflash_config cfg;
  const uint16_t *embed, *lm_head, *fc, *ctx_norm, *final_norm;
  const uint16_t* fc_s;
  std::vector<const uint16_t*> wqkv, wo, wgu, wd, ln_in, ln_post, q_norm, k_norm;
  std::vector<const uint16_t*> wqkv_s, wo_s, wgu_s, wd_s;
  char* state = nullptr;
  char* ws = nullptr;
  dflash_state_layout sl;
  WsLayout wl;
  bool target = false;   // a causal target (dflash_create_target): verify passes only
  int n_cu = 256;   // compute units of the bound device (read at bind)
  Timing timing[DFLASH_K_COUNT];
  // INT4 scales of layer l's matrix (NULL for bf16 weights)
  static const uint16_t* sc(const std::vector<const uint16_t*>& v, int l) { return v.empty() ? nullptr : v[l]; }
};

namespace {

struct Timed {
  dflash_ctx* ctx;
  int k;
  hipStream_t st;
  bool on;
  unsigned long long idx;
  Timed(dflash_ctx* c, int kclass, hipStream_t s) : ctx(c), k(kclass), st(s) {
    Timing& t = ctx->timing[k];
    on = !t.before.empty();
    if (on) {
      idx = t.count % t.before.size();
      hipEventRecord(t.before[idx], st);
    }
  }
  ~Timed() {
    if (on) {
      Timing& t = ctx->timing[k];
      hipEventRecord(t.after[idx], st);
      ++t.count;
    }
  }
};

int hip_fail(hipError_t e, const char* what) {
  return fail(DFLASH_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

template <class T>
T* at(char* base, size_t off) { return (T*)(base + off); }

GemmArgs base_args(const dflash_ctx* c) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  const dflash_config& g = c->cfg;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.hd = g.head_dim;
  a.eps = g.rms_eps;
  a.log2_theta = log2((double)g.rope_theta);
  a.C = g.ring_capacity;
  a.win = g.window;
  a.Rmax = g.max_requests;
  a.pos = at<int>(c->state, c->sl.pos);
  a.err = at<unsigned>(c->state, c->sl.error);
  a.partials = at<float>(c->ws, c->wl.partials);
  a.B = g.block;
  return a;
}

size_t ring_layer_elems(const dflash_config& g) {
  return (size_t)g.max_requests * g.n_kv_heads * g.ring_capacity * g.head_dim;
}

// Many staged rows at once: gather the taps once as bf16, then fc and every
// layer's context K/V as tiled GEMMs (the K/V tiles end in the head epilogue:
// k RMSNorm, RoPE at each row's position, K and V into the rings).
int stage_prefill(dflash_ctx* ctx, hipStream_t st, const float* const* taps, long long tap_row_stride, int n_rows,
                  const int* src_row, const int* req_of_row, const int* pos_of_row, int rows_per_req) {
  const dflash_config& g = ctx->cfg;
  const int H = g.hidden, hd = g.head_dim, TW = g.n_taps * g.tap_hidden;
  const int nkv_w = 2 * g.n_kv_heads * hd;
  hipError_t e;
  uint16_t* xg = at<uint16_t>(ctx->ws, ctx->wl.xg);
  uint16_t* c_bf = at<uint16_t>(ctx->ws, ctx->wl.c);
  {
    Timed tm(ctx, DFLASH_K_FC, st);
    TapGather tg;
    memset(&tg, 0, sizeof tg);
    for (int t = 0; t < g.n_taps; ++t) tg.taps[t] = taps[t];
    tg.tap_stride = tap_row_stride;
    tg.src_row = src_row;
    tg.n_taps = g.n_taps;
    tg.hc = g.hc_streams;
    tg.tap_hidden = g.tap_hidden;
    tg.out = xg;
    e = launch_tap_gather(tg, n_rows, st);
    if (e == hipSuccess) {
      TileArgs ta{xg, TW, ctx->fc, n_rows, H, TW,
                  g.ctx_norm ? (void*)at<float>(ctx->ws, ctx->wl.c32) : (void*)c_bf, H, ctx->fc_s};
      // bf16 weights: a plain product, through hipBLASLt when it has a kernel for the shape
      e = ctx->fc_s ? hipErrorNotSupported
                    : blaslt_gemm_nt(xg, TW, (const uint16_t*)ctx->fc, n_rows, H, TW, ta.out, H, g.ctx_norm, st);
      if (e == hipErrorNotSupported) e = launch_gemm_tile(ta, tile_bn(n_rows, H, ctx->n_cu), !g.ctx_norm, st);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "prefill fc");
  if (g.ctx_norm) {
    e = launch_rmsnorm(at<float>(ctx->ws, ctx->wl.c32), ctx->ctx_norm, c_bf, n_rows, H, g.rms_eps, st);
    if (e != hipSuccess) return hip_fail(e, "prefill ctx norm");
  }
  const size_t rl = ring_layer_elems(g);
  // bf16 weights: each layer's K/V product through hipBLASLt as fp32 rows into the
  // gathered tap rows' buffer (dead once the fc has read it), then the head finish
  // (k RMSNorm, RoPE, K rows and V^T columns into the rings); otherwise, or when
  // hipBLASLt has no kernel for the shape, the tile GEMM with that epilogue fused
  float* kv32 = at<float>(ctx->ws, ctx->wl.xg);
  const bool kv_lt = (hd == 64 || hd == 128) && (size_t)n_rows * nkv_w * 4 <= (size_t)g.max_stage_rows * TW * 2;
  for (int l = 0; l < g.n_layers; ++l) {
    Timed tm(ctx, DFLASH_K_STAGE_KV, st);
    const size_t kv_row0 = (size_t)g.n_q_heads * hd;   // the K and V rows of the fused QKV matrix
    const uint16_t* wscale = s_rows(dflash_ctx::sc(ctx->wqkv_s, l), kv_row0, H);
    TileArgs ta{c_bf, H, w_rows(g, ctx->wqkv[l], kv_row0, H), n_rows, nkv_w, H, nullptr, 0, wscale};
    GemmArgs b = base_args(ctx);
    b.M = n_rows;
    b.k_gain = ctx->k_norm[l];
    b.ring_k = at<uint16_t>(ctx->state, ctx->sl.ring_k) + l * rl;
    b.ring_v = at<uint16_t>(ctx->state, ctx->sl.ring_v) + l * rl;
    b.req_of_row = req_of_row;
    b.pos_of_row = pos_of_row;
    b.rows_per_req = rows_per_req < 1 ? 1 : rows_per_req;
    e = hipErrorNotSupported;
    if (!wscale && kv_lt) {
      e = blaslt_gemm_nt(c_bf, H, (const uint16_t*)ta.w, n_rows, nkv_w, H, kv32, nkv_w, 1, st);
      if (e == hipSuccess) {
        b.head_base = g.n_q_heads;
        b.q_gain = ctx->q_norm[l];
        e = launch_finish_kv_rows(b, kv32, nkv_w, st);
      }
    }
    if (e == hipErrorNotSupported) e = launch_gemm_tile_heads(ta, b, ctx->n_cu, st);
    if (e != hipSuccess) return hip_fail(e, "prefill kv");
  }
  return DFLASH_OK;
}

int forward_block(dflash_ctx* ctx, char* ws, const WsLayout& wl, hipStream_t st, const int* block_tokens, int n_req,
                  int block_len, int causal, const int* tap_layers, int n_tap_out, float* const* tap_out,
                  long long tap_ld, int first_row, float* logits, int* topk_ids, float* topk_vals, int k,
                  const int* rope_off = nullptr);

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_err; }

size_t dflash_state_bytes(const dflash_config* cfg) {
  if (validate_config(cfg) != DFLASH_OK) return 0;
  return st_layout(*cfg).total;
}

size_t dflash_workspace_bytes(const dflash_config* cfg) {
  if (validate_config(cfg) != DFLASH_OK) return 0;
  return ws_layout(*cfg).total;
}

int dflash_get_state_layout(const dflash_config* cfg, dflash_state_layout* out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!out) return fail(DFLASH_E_ARG, "out is NULL");
  *out = st_layout(*cfg);
  return DFLASH_OK;
}

static int create_impl(const dflash_config* cfg, const dflash_weights* w, dflash_ctx** out, bool target) {
  g_err[0] = 0;
  if (!out) return fail(DFLASH_E_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!w) return fail(DFLASH_E_ARG, "weights is NULL");
  const dflash_config& c = *cfg;
  const bool q4 = c.wfmt == DFLASH_W_INT4_G64;
  if (!w->embed || !w->lm_head || (!target && !w->fc) || !w->final_norm)
    return fail(DFLASH_E_ARG, target ? "embed, lm_head and final_norm are required"
                                     : "embed, lm_head, fc and final_norm are required");
  if (!target && c.ctx_norm && !w->ctx_norm) return fail(DFLASH_E_ARG, "ctx_norm gain required when cfg.ctx_norm = 1");
  if (!target && q4 && !w->fc_scales) return fail(DFLASH_E_ARG, "fc_scales required for INT4 weights");
  const void* const* arrays[] = {w->wqkv, w->wo, w->wgu, w->wd, w->ln_in, w->ln_post, w->q_norm, w->k_norm};
  const char* names[] = {"wqkv", "wo", "wgu", "wd", "ln_in", "ln_post", "q_norm", "k_norm"};
  for (int i = 0; i < 8; ++i) {
    if (!arrays[i]) return fail(DFLASH_E_ARG, "%s array is NULL", names[i]);
    for (int l = 0; l < c.n_layers; ++l)
      if (!arrays[i][l]) return fail(DFLASH_E_ARG, "%s[%d] is NULL", names[i], l);
  }
  if (q4) {
    const void* const* sarr[] = {w->wqkv_scales, w->wo_scales, w->wgu_scales, w->wd_scales};
    for (int i = 0; i < 4; ++i) {
      if (!sarr[i]) return fail(DFLASH_E_ARG, "INT4 scale array %d is NULL", i);
      for (int l = 0; l < c.n_layers; ++l)
        if (!sarr[i][l]) return fail(DFLASH_E_ARG, "INT4 scale array %d[%d] is NULL", i, l);
    }
  }
  // every kernel reads weights, gains and scales in 16-byte pieces
  auto misaligned = [](const void* p) { return ((uintptr_t)p & 15) != 0; };
  if (misaligned(w->embed) || misaligned(w->lm_head) || misaligned(w->fc) || misaligned(w->final_norm) ||
      misaligned(w->ctx_norm) || misaligned(w->fc_scales))
    return fail(DFLASH_E_ARG, "embed, lm_head, fc, final_norm, ctx_norm and fc_scales must be 16-byte aligned");
  for (int i = 0; i < 8; ++i)
    for (int l = 0; l < c.n_layers; ++l)
      if (misaligned(arrays[i][l])) return fail(DFLASH_E_ARG, "%s[%d] must be 16-byte aligned", names[i], l);
  if (q4) {
    const void* const* sarr[] = {w->wqkv_scales, w->wo_scales, w->wgu_scales, w->wd_scales};
    for (int i = 0; i < 4; ++i)
      for (int l = 0; l < c.n_layers; ++l)
        if (misaligned(sarr[i][l])) return fail(DFLASH_E_ARG, "INT4 scale array %d[%d] must be 16-byte aligned", i, l);
  }
  dflash_ctx* x = new dflash_ctx;
  x->cfg = c;
  x->embed = (const uint16_t*)w->embed;
  x->lm_head = (const uint16_t*)w->lm_head;
  x->fc = (const uint16_t*)w->fc;
  x->fc_s = (const uint16_t*)w->fc_scales;
  x->ctx_norm = (const uint16_t*)w->ctx_norm;
  x->final_norm = (const uint16_t*)w->final_norm;
  for (int l = 0; l < c.n_layers; ++l) {
    x->wqkv.push_back((const uint16_t*)w->wqkv[l]);
    x->wo.push_back((const uint16_t*)w->wo[l]);
    x->wgu.push_back((const uint16_t*)w->wgu[l]);
    x->wd.push_back((const uint16_t*)w->wd[l]);
    x->ln_in.push_back((const uint16_t*)w->ln_in[l]);
    x->ln_post.push_back((const uint16_t*)w->ln_post[l]);
    x->q_norm.push_back((const uint16_t*)w->q_norm[l]);
    x->k_norm.push_back((const uint16_t*)w->k_norm[l]);
    if (q4) {
      x->wqkv_s.push_back((const uint16_t*)w->wqkv_scales[l]);
      x->wo_s.push_back((const uint16_t*)w->wo_scales[l]);
      x->wgu_s.push_back((const uint16_t*)w->wgu_scales[l]);
      x->wd_s.push_back((const uint16_t*)w->wd_scales[l]);
    }
  }
  x->sl = st_layout(c);
  x->wl = ws_layout(c);
  x->target = target;
  *out = x;
  return DFLASH_OK;
}

int dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_ctx** out) {
  return create_impl(cfg, w, out, false);
}

int dflash_create_target(const dflash_config* cfg, const dflash_weights* w, dflash_ctx** out) {
  return create_impl(cfg, w, out, true);
}

void dflash_destroy(dflash_ctx* ctx) { delete ctx; }

int dflash_bind(dflash_ctx* ctx, void* state, void* workspace, void* stream) {
  if (!ctx || !state || !workspace) return fail(DFLASH_E_ARG, "ctx, state and workspace are required");
  if (((uintptr_t)state | (uintptr_t)workspace) & 255)
    return fail(DFLASH_E_ARG, "state and workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  ctx->state = (char*)state;
  ctx->ws = (char*)workspace;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
    ctx->n_cu = ncu;
  hipError_t e = launch_fill_zero(state, ctx->sl.total, st);
  if (e == hipSuccess) e = launch_fill_zero(workspace, ctx->wl.total, st);
  if (e != hipSuccess) return hip_fail(e, "bind fill");
  // staging calls that take the prefill path run a bf16 fc through hipBLASLt:
  // its handle for this device is created here, not in a stream call (without
  // one, staging runs the tile kernel)
  if (!ctx->target && ctx->cfg.wfmt == DFLASH_W_BF16 && prefill_enabled(ctx->cfg)) blaslt_prepare();
  return DFLASH_OK;
}

int dflash_reset(dflash_ctx* ctx, void* stream, int req, int valid_from, int pos) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (req < 0 || req >= ctx->cfg.max_requests) return fail(DFLASH_E_SHAPE, "req %d outside [0, %d)", req, ctx->cfg.max_requests);
  if (valid_from < 0 || valid_from > pos) return fail(DFLASH_E_ARG, "need 0 <= valid_from (%d) <= pos (%d)", valid_from, pos);
  hipError_t e = launch_set_pos(at<int>(ctx->state, ctx->sl.pos), at<int>(ctx->state, ctx->sl.valid_from), req,
                                valid_from, pos, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reset");
  return DFLASH_OK;
}

}  // extern "C"

namespace {

int tap_stage_impl(dflash_ctx* ctx, void* stream, const float* const* taps, long long tap_row_stride, int n_rows,
                   const int* src_row, const int* req_of_row, const int* pos_of_row, int rows_per_req) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  const dflash_config& g = ctx->cfg;
  if (!taps) return fail(DFLASH_E_ARG, "taps array is NULL");
  for (int t = 0; t < g.n_taps; ++t)
    if (!taps[t]) return fail(DFLASH_E_ARG, "taps[%d] is NULL", t);
  if (n_rows < 1) return fail(DFLASH_E_SHAPE, "n_rows must be >= 1");
  if (n_rows > g.max_stage_rows)
    return fail(DFLASH_E_CAPACITY, "n_rows %d exceeds max_stage_rows %d", n_rows, g.max_stage_rows);
  if (tap_row_stride < (long long)g.hc_streams * g.tap_hidden || tap_row_stride % 4)
    return fail(DFLASH_E_ARG, "tap_row_stride %lld must be >= hc_streams*tap_hidden and a multiple of 4", tap_row_stride);
  if ((!req_of_row || !pos_of_row) && rows_per_req < 1)
    return fail(DFLASH_E_ARG, "rows_per_req must be >= 1 when req_of_row or pos_of_row is NULL");
  if (!req_of_row && (n_rows + rows_per_req - 1) / rows_per_req > g.max_requests)
    return fail(DFLASH_E_CAPACITY, "n_rows / rows_per_req names more than max_requests requests");
  for (int t = 0; t < g.n_taps; ++t)
    if ((uintptr_t)taps[t] & 15) return fail(DFLASH_E_ARG, "taps[%d] must be 16-byte aligned", t);
  hipStream_t st = (hipStream_t)stream;
  const int H = g.hidden, hd = g.head_dim;
  hipError_t e;
  if (n_rows >= PREFILL_MIN_ROWS && prefill_enabled(g))
    return stage_prefill(ctx, st, taps, tap_row_stride, n_rows, src_row, req_of_row, pos_of_row, rows_per_req);

  // fc over the gathered taps
  GemmArgs a = base_args(ctx);
  for (int t = 0; t < g.n_taps; ++t) a.taps[t] = taps[t];
  a.tap_stride = tap_row_stride;
  a.src_row = src_row;
  a.n_taps = g.n_taps;
  a.hc = g.hc_streams;
  a.tap_hidden = g.tap_hidden;
  a.w = ctx->fc;
  a.wscale = ctx->fc_s;
  a.M = n_rows;
  a.N = H;
  a.K = g.n_taps * g.tap_hidden;
  const int wf = wf_of(g);
  uint16_t* c_bf = at<uint16_t>(ctx->ws, ctx->wl.c);
  a.out = g.ctx_norm ? (void*)at<float>(ctx->ws, ctx->wl.c32) : (void*)c_bf;
  a.ldo = H;
  {
    GemmPlan p = plan_for(g, n_rows, H, a.K, GC_DEFAULT, 0, P_FC);
    Timed tm(ctx, DFLASH_K_FC, st);
    int xk = X_TAPS;
    e = hipSuccess;
    if (g.hc_streams > 1) {
      // Several streams: their mean (summed in fp64, one rounding to bf16) is
      // taken once per element by the gather kernel, not by every column group
      // of the projection that stages the same X slice; the projection then
      // reads the bf16 rows. The values are those the tap staging would form.
      TapGather tg;
      memset(&tg, 0, sizeof tg);
      for (int t = 0; t < g.n_taps; ++t) tg.taps[t] = taps[t];
      tg.tap_stride = tap_row_stride;
      tg.src_row = src_row;
      tg.n_taps = g.n_taps;
      tg.hc = g.hc_streams;
      tg.tap_hidden = g.tap_hidden;
      tg.out = at<uint16_t>(ctx->ws, ctx->wl.xg);
      e = launch_tap_gather(tg, n_rows, st);
      a.x = tg.out;
      a.ldx = a.K;
      xk = X_BF16;
    }
    if (e == hipSuccess) {
      if (p.S > 1) {
        e = launch_gemm(a, p, xk, E_PART, wf, st);
        if (e == hipSuccess) e = launch_finish_store(a.partials, p.S, n_rows, H, a.out, H, !g.ctx_norm, st);
      } else {
        e = launch_gemm(a, p, xk, g.ctx_norm ? E_F32 : E_BF16, wf, st);
      }
    }
  }
  if (e != hipSuccess) return hip_fail(e, "stage fc");
  if (g.ctx_norm) {
    e = launch_rmsnorm(at<float>(ctx->ws, ctx->wl.c32), ctx->ctx_norm, c_bf, n_rows, H, g.rms_eps, st);
    if (e != hipSuccess) return hip_fail(e, "stage ctx norm");
  }
  // per layer: K/V of the staged rows into the ring
  const size_t rl = ring_layer_elems(g);
  GemmPlan p = plan_for(g, n_rows, 2 * g.n_kv_heads * hd, H, hd, 0, P_STAGE_KV);
  const size_t kv_row0 = (size_t)g.n_q_heads * hd;   // the K and V rows of the fused QKV matrix
  // split-K (a few rows per round): up to MAX_BATCH layers share one launch of the
  // projection and one of the head finish; S = 1 (prefill) runs one launch per layer
  const int step = stage_batch(p, n_rows, 2 * g.n_kv_heads * hd, g.n_layers);
  for (int l0 = 0; l0 < g.n_layers; l0 += step) {
    const int nl = g.n_layers - l0 < step ? g.n_layers - l0 : step;
    GemmArgs b = base_args(ctx);
    b.x = c_bf;
    b.ldx = H;
    b.w = w_rows(g, ctx->wqkv[l0], kv_row0, H);
    b.wscale = s_rows(dflash_ctx::sc(ctx->wqkv_s, l0), kv_row0, H);
    b.M = n_rows;
    b.N = 2 * g.n_kv_heads * hd;
    b.K = H;
    b.head_base = g.n_q_heads;
    b.k_gain = ctx->k_norm[l0];
    b.q_gain = ctx->q_norm[l0];
    b.ring_k = at<uint16_t>(ctx->state, ctx->sl.ring_k) + l0 * rl;
    b.ring_v = at<uint16_t>(ctx->state, ctx->sl.ring_v) + l0 * rl;
    b.req_of_row = req_of_row;
    b.pos_of_row = pos_of_row;
    b.rows_per_req = rows_per_req < 1 ? 1 : rows_per_req;
    Timed tm(ctx, DFLASH_K_STAGE_KV, st);
    if (p.S > 1) {
      b.nb = step > 1 ? nl : 0;
      for (int i = 0; i < nl; ++i) {
        b.wb[i] = w_rows(g, ctx->wqkv[l0 + i], kv_row0, H);
        b.wsb[i] = s_rows(dflash_ctx::sc(ctx->wqkv_s, l0 + i), kv_row0, H);
        b.rkb[i] = at<uint16_t>(ctx->state, ctx->sl.ring_k) + (l0 + i) * rl;
        b.rvb[i] = at<uint16_t>(ctx->state, ctx->sl.ring_v) + (l0 + i) * rl;
        b.kgb[i] = ctx->k_norm[l0 + i];
      }
      e = launch_gemm(b, p, X_BF16, E_PART, wf, st);
      if (e == hipSuccess) e = launch_finish_head(b, b.partials, p.S, b.N, 2 * g.n_kv_heads, st);
    } else {
      e = launch_gemm(b, p, X_BF16, E_HEAD, wf, st);
    }
    if (e != hipSuccess) return hip_fail(e, "stage kv");
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_tap_stage(dflash_ctx* ctx, void* stream, const float* const* taps, long long tap_row_stride,
                     int n_rows, const int* req_of_row, const int* pos_of_row, int rows_per_req) {
  return tap_stage_impl(ctx, stream, taps, tap_row_stride, n_rows, nullptr, req_of_row, pos_of_row, rows_per_req);
}

int dflash_tap_stage_rows(dflash_ctx* ctx, void* stream, const float* const* taps, long long tap_row_stride,
                          int n_rows, const int* src_row, const int* req_of_row, const int* pos_of_row,
                          int rows_per_req) {
  if (!src_row) return fail(DFLASH_E_ARG, "src_row is required");
  return tap_stage_impl(ctx, stream, taps, tap_row_stride, n_rows, src_row, req_of_row, pos_of_row, rows_per_req);
}

int dflash_draft_block(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req, float* logits,
                       int* topk_ids, float* topk_vals, int k) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  return dflash_draft_block_n(ctx, stream, block_tokens, n_req, ctx->cfg.block, logits, topk_ids, topk_vals, k);
}

int dflash_draft_block_n(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req, int block_len,
                         float* logits, int* topk_ids, float* topk_vals, int k) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (ctx->target) return fail(DFLASH_E_STATE, "a target handle runs verify passes, not drafts");
  const dflash_config& g = ctx->cfg;
  if (!block_tokens || !topk_ids) return fail(DFLASH_E_ARG, "block_tokens and topk_ids are required");
  if (n_req < 1 || n_req > g.max_requests)
    return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (block_len < 1 || block_len > g.block)
    return fail(DFLASH_E_SHAPE, "block_len %d outside [1, %d]", block_len, g.block);
  if (k != 1 && k != 16) return fail(DFLASH_E_ARG, "k must be 1 or 16 (got %d)", k);
  if (k > g.vocab) return fail(DFLASH_E_ARG, "k exceeds vocab");
  if (block_len == 1) return DFLASH_OK;   // no mask rows: nothing to draft
  return forward_block(ctx, ctx->ws, ctx->wl, (hipStream_t)stream, block_tokens, n_req, block_len, 0, nullptr, 0,
                       nullptr, 0, 1, logits, topk_ids, topk_vals, k);
}

}  // extern "C"

namespace {

// Scratch of the allocation-free draft entry point: one copy on every GPU the
// library runs on, held until the process ends. Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress, once
// per device, and is kept in g_scratch_ptr.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)DFLASH_STATIC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[MAX_DEVICES];

// The current device's copy of `scratch` (looked up on its first use).
int static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DFLASH_E_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_draft_scratch_bytes(const dflash_config* cfg) {
  if (validate_config(cfg) != DFLASH_OK) return 0;
  return ws_layout(*cfg, true).total;
}

int dflash_draft_block_noalloc(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req, float* logits,
                               int* topk_ids, float* topk_vals, int k) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (ctx->target) return fail(DFLASH_E_STATE, "a target handle runs verify passes, not drafts");
  const dflash_config& g = ctx->cfg;
  if (!block_tokens || !topk_ids) return fail(DFLASH_E_ARG, "block_tokens and topk_ids are required");
  if (n_req < 1 || n_req > g.max_requests)
    return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (k != 1 && k != 16) return fail(DFLASH_E_ARG, "k must be 1 or 16 (got %d)", k);
  if (k > g.vocab) return fail(DFLASH_E_ARG, "k exceeds vocab");
  const WsLayout L = ws_layout(g, true);
  if (L.total > STATIC_SCRATCH_BYTES)
    return fail(DFLASH_E_CAPACITY, "this configuration's draft needs %zu bytes of scratch; the static scratch holds %zu",
                L.total, STATIC_SCRATCH_BYTES);
  if (g.block == 1) return DFLASH_OK;   // no mask rows: nothing to draft
  char* ws = nullptr;
  const int rc = static_scratch(&ws);
  if (rc) return rc;
  return forward_block(ctx, ws, L, (hipStream_t)stream, block_tokens, n_req, g.block, 0, nullptr, 0, nullptr, 0, 1,
                       logits, topk_ids, topk_vals, k);
}

int dflash_verify_block(dflash_ctx* ctx, void* stream, const int* block_tokens, int n_req, int block_len,
                        const int* tap_layers, int n_tap_out, float* const* tap_out, long long tap_ld, float* logits,
                        int* ids) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (!ctx->target) return fail(DFLASH_E_STATE, "verify passes need a target handle (dflash_create_target)");
  const dflash_config& g = ctx->cfg;
  if (!block_tokens || !ids) return fail(DFLASH_E_ARG, "block_tokens and ids are required");
  if (n_req < 1 || n_req > g.max_requests)
    return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (block_len < 1 || block_len > g.block)
    return fail(DFLASH_E_SHAPE, "block_len %d outside [1, %d]", block_len, g.block);
  if (n_tap_out < 0 || n_tap_out > MAX_TAPS || (n_tap_out > 0 && (!tap_layers || !tap_out)))
    return fail(DFLASH_E_ARG, "n_tap_out must be in [0, %d] with tap_layers and tap_out given", MAX_TAPS);
  for (int t = 0; t < n_tap_out; ++t) {
    if (tap_layers[t] < 0 || tap_layers[t] >= g.n_layers)
      return fail(DFLASH_E_ARG, "tap_layers[%d] = %d outside [0, %d)", t, tap_layers[t], g.n_layers);
    if (!tap_out[t] || ((uintptr_t)tap_out[t] & 15)) return fail(DFLASH_E_ARG, "tap_out[%d] must be 16-byte aligned", t);
  }
  if (n_tap_out > 0 && (tap_ld < g.hidden || tap_ld % 4)) return fail(DFLASH_E_ARG, "tap_ld must be >= hidden, % 4 == 0");
  return forward_block(ctx, ctx->ws, ctx->wl, (hipStream_t)stream, block_tokens, n_req, block_len, 1, tap_layers,
                       n_tap_out, tap_out, tap_ld, 0, logits, ids, nullptr, 1);
}

int dflash_tree_build(dflash_ctx* ctx, void* stream, const int* block_tokens, const int* topk_ids,
                      const float* topk_vals, int k, int n_req, int n_nodes, int* tree_tokens, int* tree_parent,
                      int* tree_depth) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  const dflash_config& g = ctx->cfg;
  if (!block_tokens || !topk_ids || !topk_vals || !tree_tokens || !tree_parent || !tree_depth)
    return fail(DFLASH_E_ARG, "block_tokens, topk_ids, topk_vals and the three tree outputs are required");
  if (n_req < 1 || n_req > g.max_requests) return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (g.block < 2) return fail(DFLASH_E_SHAPE, "a tree needs draft positions (block >= 2)");
  if (k < 1 || k > 16) return fail(DFLASH_E_ARG, "k must be in [1, 16] (got %d)", k);
  if (n_nodes < 1 || n_nodes > 64) return fail(DFLASH_E_SHAPE, "n_nodes %d outside [1, 64]", n_nodes);
  // nodes available: 1 + k + k^2 + ... + k^(B-1), saturated
  long long avail = 1, level = 1;
  for (int d = 1; d < g.block && avail < n_nodes; ++d) {
    level = level * k > 64 ? 64 : level * k;
    avail += level;
  }
  if (n_nodes > avail) return fail(DFLASH_E_SHAPE, "n_nodes %d exceeds the %lld nodes the lists offer", n_nodes, avail);
  hipError_t e = launch_tree_build(block_tokens, g.block, topk_ids, topk_vals, k, n_req, n_nodes, tree_tokens,
                                   tree_parent, tree_depth, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree build");
  return DFLASH_OK;
}

int dflash_verify_tree(dflash_ctx* ctx, void* stream, const int* tree_tokens, const int* tree_parent,
                       const int* tree_depth, int n_req, int n_nodes, const int* tap_layers, int n_tap_out,
                       float* const* tap_out, long long tap_ld, float* logits, int* ids) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (!ctx->target) return fail(DFLASH_E_STATE, "verify passes need a target handle (dflash_create_target)");
  const dflash_config& g = ctx->cfg;
  if (!tree_tokens || !tree_parent || !tree_depth || !ids)
    return fail(DFLASH_E_ARG, "tree_tokens, tree_parent, tree_depth and ids are required");
  if (n_req < 1 || n_req > g.max_requests) return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (n_nodes < 1 || n_nodes > g.block || n_nodes > 64)
    return fail(DFLASH_E_SHAPE, "n_nodes %d outside [1, min(block %d, 64)]", n_nodes, g.block);
  if (n_tap_out < 0 || n_tap_out > MAX_TAPS || (n_tap_out > 0 && (!tap_layers || !tap_out)))
    return fail(DFLASH_E_ARG, "n_tap_out must be in [0, %d] with tap_layers and tap_out given", MAX_TAPS);
  for (int t = 0; t < n_tap_out; ++t) {
    if (tap_layers[t] < 0 || tap_layers[t] >= g.n_layers)
      return fail(DFLASH_E_ARG, "tap_layers[%d] = %d outside [0, %d)", t, tap_layers[t], g.n_layers);
    if (!tap_out[t] || ((uintptr_t)tap_out[t] & 15)) return fail(DFLASH_E_ARG, "tap_out[%d] must be 16-byte aligned", t);
  }
  if (n_tap_out > 0 && (tap_ld < g.hidden || tap_ld % 4)) return fail(DFLASH_E_ARG, "tap_ld must be >= hidden, % 4 == 0");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_tree_anc(tree_parent, n_nodes, n_nodes, n_req, at<unsigned long long>(ctx->ws, ctx->wl.anc), st);
  if (e != hipSuccess) return hip_fail(e, "tree masks");
  return forward_block(ctx, ctx->ws, ctx->wl, st, tree_tokens, n_req, n_nodes, 2, tap_layers, n_tap_out, tap_out,
                       tap_ld, 0, logits, ids, nullptr, 1, tree_depth);
}

int dflash_tree_accept(dflash_ctx* ctx, void* stream, const int* tree_tokens, const int* tree_parent, int n_nodes,
                       const int* verify_ids, int n_req, int eos_id, const int* budget, int* accept_len, int* emitted,
                       int* n_emit, int* next_tokens, int* path_nodes, int* stage_rows, int* stage_pos) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  const dflash_config& g = ctx->cfg;
  if (!tree_tokens || !tree_parent || !verify_ids || !accept_len || !emitted || !n_emit || !path_nodes ||
      !stage_rows || !stage_pos)
    return fail(DFLASH_E_ARG, "the tree, verify_ids and every output except next_tokens are required");
  if (n_req < 1 || n_req > g.max_requests) return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (n_nodes < 1 || n_nodes > 64) return fail(DFLASH_E_SHAPE, "n_nodes %d outside [1, 64]", n_nodes);
  hipError_t e = launch_tree_accept(tree_tokens, tree_parent, n_nodes, verify_ids, n_req, g.block, g.block, eos_id,
                                    budget, g.mask_id, accept_len, emitted, n_emit, next_tokens, path_nodes,
                                    stage_rows, stage_pos, at<int>(ctx->state, ctx->sl.pos),
                                    at<unsigned long long>(ctx->state, ctx->sl.stats), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree accept");
  return DFLASH_OK;
}

int dflash_tree_commit(dflash_ctx* ctx, void* stream, const int* path_nodes, int path_ld, const int* n_emit,
                       int n_req) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (!ctx->target) return fail(DFLASH_E_STATE, "only a target handle commits a tree pass");
  const dflash_config& g = ctx->cfg;
  if (!path_nodes || !n_emit) return fail(DFLASH_E_ARG, "path_nodes and n_emit are required");
  if (n_req < 1 || n_req > g.max_requests) return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (path_ld < 1 || path_ld > 64) return fail(DFLASH_E_ARG, "path_ld %d outside [1, 64]", path_ld);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_tree_commit(at<uint16_t>(ctx->state, ctx->sl.ring_k), at<uint16_t>(ctx->state, ctx->sl.ring_v),
                                    ring_layer_elems(g), g.n_layers, n_req, g.n_kv_heads, g.head_dim,
                                    g.ring_capacity, at<int>(ctx->state, ctx->sl.pos), path_nodes, path_ld, n_emit, st);
  if (e == hipSuccess) e = launch_advance(at<int>(ctx->state, ctx->sl.pos), n_emit, n_req, st);
  if (e != hipSuccess) return hip_fail(e, "tree commit");
  return DFLASH_OK;
}

int dflash_advance(dflash_ctx* ctx, void* stream, const int* n_emit, int n_req) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  if (!n_emit) return fail(DFLASH_E_ARG, "n_emit is required");
  if (n_req < 1 || n_req > ctx->cfg.max_requests)
    return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, ctx->cfg.max_requests);
  hipError_t e = launch_advance(at<int>(ctx->state, ctx->sl.pos), n_emit, n_req, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "advance");
  return DFLASH_OK;
}

}  // extern "C"

namespace {

// One block forward of every request r < n_req at positions pos[r] + i: the
// drafter's masked block (bidirectional, the mask rows' top-k) or a causal
// target's verify pass (block row i sees rows <= i, argmax of every row, the
// residual rows after the tapped layers copied out).
int forward_block(dflash_ctx* ctx, char* ws, const WsLayout& wl, hipStream_t st, const int* block_tokens, int n_req,
                  int block_len, int causal, const int* tap_layers, int n_tap_out, float* const* tap_out,
                  long long tap_ld, int first_row, float* logits, int* topk_ids, float* topk_vals, int k,
                  const int* rope_off) {
  const dflash_config& g = ctx->cfg;
  // GEMM arguments with this call's split-K partial buffer
  auto base = [&]() {
    GemmArgs a = base_args(ctx);
    a.partials = at<float>(ws, wl.partials);
    return a;
  };
  const int H = g.hidden, hd = g.head_dim, B = block_len;
  const int M = n_req * B;
  const int qw = g.n_q_heads * hd;
  float* h = at<float>(ws, wl.h);
  float* ssq = at<float>(ws, wl.ssq);
  uint16_t* q = at<uint16_t>(ws, wl.q);
  uint16_t* o = at<uint16_t>(ws, wl.o);
  uint16_t* act = at<uint16_t>(ws, wl.act);
  unsigned* err = at<unsigned>(ctx->state, ctx->sl.error);
  const int ssq_ld = g.max_requests * g.block;   // row pitch of the ssq buffer
  const int h_blocks = H / GC_DEFAULT;
  const int wf = wf_of(g);
  // every RMSNorm is applied by the GEMM that consumes it (X_NORM), from h and
  // the per-row sums of squares its producer left in ssq
  auto norm_input = [&](GemmArgs& a, const uint16_t* gain, int n_blocks) {
    a.xf = h;
    a.ldx = H;
    a.xgain = gain;
    a.ssq_in = ssq;
    a.n_ssq = n_blocks;
    a.ssq_ld = ssq_ld;
  };
  hipError_t e = launch_embed(block_tokens, ctx->embed, h, ssq, M, H, g.vocab, err, st);
  if (e != hipSuccess) return hip_fail(e, "embed");
  const size_t rl = ring_layer_elems(g);
  for (int l = 0; l < g.n_layers; ++l) {
    uint16_t* rk = at<uint16_t>(ctx->state, ctx->sl.ring_k) + l * rl;
    uint16_t* rv = at<uint16_t>(ctx->state, ctx->sl.ring_v) + l * rl;
    {  // RMSNorm + QKV + q/k head norm + RoPE; the block's K/V go to ring slots [pos, pos+B)
      GemmArgs a = base();
      norm_input(a, ctx->ln_in[l], l == 0 ? 1 : h_blocks);
      a.w = ctx->wqkv[l];
      a.wscale = dflash_ctx::sc(ctx->wqkv_s, l);
      a.M = M;
      a.N = (g.n_q_heads + 2 * g.n_kv_heads) * hd;
      a.K = H;
      a.head_base = 0;
      a.q_gain = ctx->q_norm[l];
      a.k_gain = ctx->k_norm[l];
      a.q_out = q;
      a.ring_k = rk;
      a.ring_v = rv;
      a.rows_per_req = B;
      a.rope_off = rope_off;
      GemmPlan p = plan_for(g, M, a.N, H, hd, 0, P_QKV);
      Timed tm(ctx, DFLASH_K_QKV, st);
      if (p.S > 1) {
        e = launch_gemm(a, p, X_NORM, E_PART, wf, st);
        if (e == hipSuccess) e = launch_finish_head(a, a.partials, p.S, a.N, g.n_q_heads + 2 * g.n_kv_heads, st);
      } else {
        e = launch_gemm(a, p, X_NORM, E_HEAD, wf, st);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv");
    }
    {  // attention over [context window | block]
      AttnArgs t;
      memset(&t, 0, sizeof t);
      t.q = q;
      t.ring_k = rk;
      t.ring_v = rv;
      t.out = o;
      t.pos = at<int>(ctx->state, ctx->sl.pos);
      t.valid_from = at<int>(ctx->state, ctx->sl.valid_from);
      t.B = B;
      t.W = g.window;
      t.C = g.ring_capacity;
      t.nq = g.n_q_heads;
      t.nkv = g.n_kv_heads;
      t.hd = hd;
      t.kc = attn_chunk_keys(hd);
      t.n_chunks = attn_nchunks(g);
      t.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
      t.part_o = at<float>(ws, wl.attn_o);
      t.part_ml = at<float>(ws, wl.attn_ml);
      t.err = err;
      t.causal = causal;
      t.anc = causal == 2 ? at<unsigned long long>(ws, wl.anc) : nullptr;
      Timed tm(ctx, DFLASH_K_ATTN, st);
      e = launch_attention(t, n_req, st);
      if (e != hipSuccess) return hip_fail(e, "attention");
    }
    {  // o projection, residual add, row sums of squares for the post-attention norm
      GemmArgs a = base();
      a.x = o;
      a.ldx = qw;
      a.w = ctx->wo[l];
      a.wscale = dflash_ctx::sc(ctx->wo_s, l);
      a.M = M;
      a.N = H;
      a.K = qw;
      a.out = h;
      a.ldo = H;
      a.ssq_out = ssq;
      a.ssq_ld = ssq_ld;
      GemmPlan p = plan_for(g, M, H, qw, GC_DEFAULT, 0, P_O);
      Timed tm(ctx, DFLASH_K_O, st);
      if (p.S > 1) {
        e = launch_gemm(a, p, X_BF16, E_PART, wf, st);
        if (e == hipSuccess) e = launch_finish_resid(a.partials, p.S, M, H, h, H, ssq, ssq_ld, st);
      } else {
        e = launch_gemm(a, p, X_BF16, E_RESID, wf, st);
      }
      if (e != hipSuccess) return hip_fail(e, "o proj");
    }
    {  // RMSNorm + gate/up with SiLU(gate) * up
      GemmArgs a = base();
      norm_input(a, ctx->ln_post[l], h_blocks);
      a.w = ctx->wgu[l];
      a.wscale = dflash_ctx::sc(ctx->wgu_s, l);
      a.M = M;
      a.N = g.ffn;
      a.K = H;
      a.pair_off = g.ffn;
      a.out = act;
      a.ldo = g.ffn;
      GemmPlan p = plan_for(g, M, g.ffn, H, GC_DEFAULT, 1, P_GATEUP);
      Timed tm(ctx, DFLASH_K_GATEUP, st);
      if (wf == WF_BF16 && gateup_lds_bytes(M, H)) {
        e = launch_gateup_lds(a, p.ks, st);   // same sums as the split plan p, one launch
      } else if (wf == WF_INT4 && gateup_q4_bytes(M, H)) {
        e = launch_gateup_q4(a, p.ks, st);
      } else if (p.S > 1) {
        e = launch_gemm(a, p, X_NORM, E_PARTP, wf, st);
        if (e == hipSuccess) e = launch_finish_silu(a.partials, p.S, M, g.ffn, act, g.ffn, st);
      } else {
        e = launch_gemm(a, p, X_NORM, E_SILU, wf, st);
      }
      if (e != hipSuccess) return hip_fail(e, "gate/up");
    }
    {  // down projection, residual add, row sums of squares for the next norm
      GemmArgs a = base();
      a.x = act;
      a.ldx = g.ffn;
      a.w = ctx->wd[l];
      a.wscale = dflash_ctx::sc(ctx->wd_s, l);
      a.M = M;
      a.N = H;
      a.K = g.ffn;
      a.out = h;
      a.ldo = H;
      a.ssq_out = ssq;
      a.ssq_ld = ssq_ld;
      GemmPlan p = plan_for(g, M, H, g.ffn, GC_DEFAULT, 0, P_DOWN);
      Timed tm(ctx, DFLASH_K_DOWN, st);
      if (p.S > 1) {
        e = launch_gemm(a, p, X_BF16, E_PART, wf, st);
        if (e == hipSuccess) e = launch_finish_resid(a.partials, p.S, M, H, h, H, ssq, ssq_ld, st);
      } else {
        e = launch_gemm(a, p, X_BF16, E_RESID, wf, st);
      }
      if (e != hipSuccess) return hip_fail(e, "down proj");
    }
    for (int t = 0; t < n_tap_out; ++t)   // the residual after this layer, for the drafter's taps
      if (tap_layers[t] == l) {
        e = launch_copy_rows(h, M, H, tap_out[t], tap_ld, st);
        if (e != hipSuccess) return hip_fail(e, "tap copy");
      }
  }
  {  // shared LM head: mask-row logits, then per-row top-k
    GemmArgs a = base();
    norm_input(a, ctx->final_norm, h_blocks);
    a.w = ctx->lm_head;
    a.M = M;
    a.N = g.vocab;
    a.K = H;
    a.B = B;   // this call's block length
    a.lm_first_row = first_row;
    a.topk = k;
    LmPlan p = plan_lmhead(M, B, g.vocab, H, ctx->n_cu);
    if (p.XL == 0 || p.XL == 2 || p.XL == 4) {
      // more than one row tile: the final RMSNorm once into bf16 rows, which the
      // head loads straight into LDS (or streams through LDS windows, or reads
      // from L2)
      uint16_t* z = at<uint16_t>(ws, wl.z);
      e = launch_lm_norm_rows(a, z, st);
      if (e != hipSuccess) return hip_fail(e, "final norm");
      a.x = z;
    }
    float* lg = logits ? logits : at<float>(ws, wl.logits);
    const int tr = logits ? 0 : 1;
    float* gm = at<float>(ws, wl.gmax);
    {
      Timed tm(ctx, DFLASH_K_LMHEAD, st);
      e = launch_lm_logits(a, p, lg, tr, gm, st);
    }
    if (e != hipSuccess) return hip_fail(e, "lm head");
    e = launch_lm_topk(a, p, lg, tr, gm, topk_ids, topk_vals, st);
    if (e != hipSuccess) return hip_fail(e, "top-k");
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_accept(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride, const int* verify_ids,
                  int n_req, int eos_id, const int* budget, int* accept_len, int* emitted, int* n_emit,
                  int* next_tokens) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  return dflash_accept_n(ctx, stream, draft_ids, draft_stride, verify_ids, n_req, ctx->cfg.block, eos_id, budget,
                         accept_len, emitted, n_emit, next_tokens);
}

int dflash_accept_n(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride, const int* verify_ids,
                    int n_req, int block_len, int eos_id, const int* budget, int* accept_len, int* emitted,
                    int* n_emit, int* next_tokens) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  const dflash_config& g = ctx->cfg;
  if (block_len < 1 || block_len > g.block)
    return fail(DFLASH_E_SHAPE, "block_len %d outside [1, %d]", block_len, g.block);
  if ((!draft_ids && block_len > 1) || !verify_ids || !accept_len || !emitted || !n_emit)
    return fail(DFLASH_E_ARG, "draft_ids, verify_ids, accept_len, emitted and n_emit are required");
  if (n_req < 1 || n_req > g.max_requests)
    return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (draft_stride < 1) return fail(DFLASH_E_ARG, "draft_stride must be >= 1");
  hipError_t e = launch_accept(draft_ids, draft_stride, verify_ids, n_req, block_len, g.block, eos_id, budget,
                               g.mask_id, accept_len, emitted, n_emit, next_tokens, at<int>(ctx->state, ctx->sl.pos),
                               at<unsigned long long>(ctx->state, ctx->sl.stats), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "accept");
  return DFLASH_OK;
}

int dflash_accept_sampled(dflash_ctx* ctx, void* stream, const int* draft_ids, int draft_stride,
                          const float* target_logits, int n_req, int block_len, const dflash_sampling* params,
                          unsigned long long seed, unsigned round, int eos_id, const int* budget, int* accept_len,
                          int* emitted, int* n_emit, int* next_tokens) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  const dflash_config& g = ctx->cfg;
  if (block_len < 1 || block_len > g.block)
    return fail(DFLASH_E_SHAPE, "block_len %d outside [1, %d]", block_len, g.block);
  if ((!draft_ids && block_len > 1) || !target_logits || !params || !accept_len || !emitted || !n_emit)
    return fail(DFLASH_E_ARG, "draft_ids, target_logits, params, accept_len, emitted and n_emit are required");
  if (n_req < 1 || n_req > g.max_requests) return fail(DFLASH_E_SHAPE, "n_req %d outside [1, %d]", n_req, g.max_requests);
  if (draft_stride < 1) return fail(DFLASH_E_ARG, "draft_stride must be >= 1");
  if (!(params->temperature > 0.f) || params->top_k < 1 || params->top_k > 64 || !(params->top_p > 0.f) ||
      params->top_p > 1.f || !(params->typical_eps >= 0.f))
    return fail(DFLASH_E_ARG, "need temperature > 0, top_k in [1, 64], top_p in (0, 1], typical_eps >= 0");
  SampleArgs a;
  memset(&a, 0, sizeof a);
  a.logits = target_logits;
  a.draft = draft_ids;
  a.draft_stride = draft_stride;
  a.R = n_req;
  a.b = block_len;
  a.V = g.vocab;
  a.stats_b = g.block;
  a.mask_id = g.mask_id;
  a.eos = eos_id;
  a.T = params->temperature;
  a.top_p = params->top_p;
  a.eps = params->typical_eps;
  a.delta = params->typical_delta;
  a.top_k = params->top_k;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.round = round;
  a.budget = budget;
  a.accept_len = accept_len;
  a.emitted = emitted;
  a.n_emit = n_emit;
  a.next_tokens = next_tokens;
  a.pos = at<int>(ctx->state, ctx->sl.pos);
  a.stats = at<unsigned long long>(ctx->state, ctx->sl.stats);
  a.row_ok = at<int>(ctx->ws, ctx->wl.row_ok);
  a.cand_idx = at<int>(ctx->ws, ctx->wl.cand_idx);
  a.cand_key = at<unsigned>(ctx->ws, ctx->wl.cand_key);
  a.n_chunks = sample_chunks(g.vocab);
  a.part_key = at<unsigned>(ctx->ws, ctx->wl.part_key);
  a.part_idx = at<int>(ctx->ws, ctx->wl.part_idx);
  a.part_m = at<float>(ctx->ws, ctx->wl.part_m);
  a.part_z = at<double>(ctx->ws, ctx->wl.part_z);
  a.part_s = at<double>(ctx->ws, ctx->wl.part_s);
  if (a.n_chunks > SAMPLE_MAX_CHUNKS)
    return fail(DFLASH_E_SHAPE, "sampled accept supports vocabularies up to %d (got %d)",
                SAMPLE_CHUNK * SAMPLE_MAX_CHUNKS, g.vocab);
  hipError_t e = launch_sampled_accept(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sampled accept");
  return DFLASH_OK;
}

void dflash_policy_init(dflash_block_policy* p, int block, double weight) {
  if (!p) return;
  p->block = block;
  p->weight = weight;
  p->mean = (double)(block - 1);
}

int dflash_policy_next(const dflash_block_policy* p) {
  if (!p) return 0;
  const int hi = p->block, lo = hi < 2 ? hi : 2;
  const double b = floor(p->mean + 0.5) + 2.0;   // compared in fp64: no int conversion of an unbounded mean
  if (!(b > (double)lo)) return lo;               // a NaN mean too
  if (b >= (double)hi) return hi;
  return (int)b;
}

void dflash_policy_update(dflash_block_policy* p, int accepted) {
  if (!p) return;
  p->mean = (1.0 - p->weight) * p->mean + p->weight * (double)accepted;
}

int dflash_check(dflash_ctx* ctx, void* stream, unsigned* word) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  hipStream_t st = (hipStream_t)stream;
  unsigned w = 0;
  hipError_t e = hipMemcpyAsync(&w, ctx->state + ctx->sl.error, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "check");
  if (word) *word = w;
  if (w) return fail(DFLASH_E_DEVICE, "device error word 0x%x", w);
  return DFLASH_OK;
}

int dflash_clear_error(dflash_ctx* ctx, void* stream) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!ctx->state) return fail(DFLASH_E_STATE, "handle not bound");
  hipError_t e = launch_fill_zero(ctx->state + ctx->sl.error, 4, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "clear error");
  return DFLASH_OK;
}

int dflash_stream_read(const void* src, size_t bytes, unsigned* sink, void* stream) {
  if (!src || !sink) return fail(DFLASH_E_ARG, "src and sink are required");
  if (bytes % 16 || ((uintptr_t)src & 15)) return fail(DFLASH_E_ARG, "src must be 16-byte aligned and bytes a multiple of 16");
  hipError_t e = launch_stream_read(src, bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream read");
  return DFLASH_OK;
}

int dflash_set_timing_events(dflash_ctx* ctx, int kclass, void* const* before, void* const* after, int n) {
  if (!ctx) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (kclass < 0 || kclass >= DFLASH_K_COUNT) return fail(DFLASH_E_ARG, "unknown kernel class %d", kclass);
  if (n < 0 || (n > 0 && (!before || !after))) return fail(DFLASH_E_ARG, "bad event arrays");
  Timing& t = ctx->timing[kclass];
  t.before.clear();
  t.after.clear();
  t.count = 0;
  for (int i = 0; i < n; ++i) {
    t.before.push_back((hipEvent_t)before[i]);
    t.after.push_back((hipEvent_t)after[i]);
  }
  return DFLASH_OK;
}

}  // extern "C"
