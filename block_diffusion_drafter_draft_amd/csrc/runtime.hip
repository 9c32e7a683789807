// C ABI of libdbd.so: argument validation (host, before any launch), workspace carving and the
// launch sequence of draft_block, verify_greedy and select_streak.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dbd.h"
#include "dbd_internal.h"

using namespace dbd;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                               \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess)                                                           \
      return fail(DBD_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));             \
  } while (0)

// Launch the expression on stream `st`, bracketed by timing events when timing is enabled.
#define HIP_STAGE(stage, st, expr)                                                  \
  do {                                                                              \
    Timing::Pair* tp_ = g_timing.begin(stage, st);                                  \
    HIP_TRY(expr);                                                                  \
    if (tp_) g_timing.end(tp_, st);                                                 \
  } while (0)

// Per-stage kernel timing (benchmarks only): event pairs recorded around every launch.
struct Timing {
  struct Pair {
    hipEvent_t a, b;
    int stage;
  };
  bool on = false;
  std::vector<Pair> pool;     // created once, reused after reset
  size_t used = 0;
  Pair* begin(int stage, hipStream_t st) {
    if (!on) return nullptr;
    if (used == pool.size()) {
      Pair p{};
      if (hipEventCreate(&p.a) != hipSuccess || hipEventCreate(&p.b) != hipSuccess) return nullptr;
      pool.push_back(p);
    }
    Pair* p = &pool[used++];
    p->stage = stage;
    if (hipEventRecord(p->a, st) != hipSuccess) { --used; return nullptr; }
    return p;
  }
  void end(Pair* p, hipStream_t st) { (void)hipEventRecord(p->b, st); }
};
Timing g_timing;

constexpr size_t kAlign = 256;

// Bump allocator over the caller's workspace; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  size_t last = 0;            // offset of the most recent take
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    last = off;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

int elem_size(int dtype) { return dtype == DBD_BF16 ? 2 : 4; }

// Attention tuning overrides (dbd_attn_override): workgroups and chunks loaded ahead of the
// bf16 kernel, 0 = the library's choice.
static int g_attn_workgroups = 0, g_attn_depth = 0;

// Workgroups of the bf16 attention: two per CU of the 256, which is what its registers (two
// register sets of staged keys and values) and its two 32 KB LDS slots allow.
static int attn_workgroups() { return g_attn_workgroups > 0 ? g_attn_workgroups : kAttnWorkgroups; }
static int attn_depth() { return g_attn_depth > 0 ? g_attn_depth : kAttnDepth; }

// Keys per split of the fp32 attention (one workgroup per (split, kv head, sequence), each key
// of a split its own thread): the largest of 256, 128 and 64 that still gives the launch at least
// 512 workgroups over the capacity.
static int attn_split_f32(int cap, int kvh, int batch) {
  int s = 256;
  while (s > 64 && (int64_t)ceil_div(cap, s) * kvh * batch < 512) s /= 2;
  return s;
}

// Attention partials (rows of hd floats) to reserve for up to `batch` sequences.  bf16: one
// 64-row slot per (workgroup, segment) piece, at most workgroups + segments.  fp32: R rows per
// (sequence, split, kv head); the split shrinks with the batch, so the maximum over 1 .. batch
// keeps a workspace sized for a batch enough for every smaller one.
static int64_t attn_partial_rows(int dtype, int cap, int kvh, int batch, int R, bool at_most) {
  if (dtype == DBD_BF16)
    return attn_partial_slots(attn_workgroups(), (int64_t)batch * kvh * attn_row_blocks(R)) *
           kAttnRows;
  int64_t m = 0;
  for (int n = at_most ? 1 : batch; n <= batch; ++n)
    m = std::max(m, (int64_t)n * ceil_div(cap, attn_split_f32(cap, kvh, n)));
  return m * kvh * R;
}

// Per-stage GEMM tile / split overrides (dbd_gemm_override), indexed by DBD_STAGE_*: -1 / 0 =
// the library's choice.
static int g_ov_cfg[DBD_STAGE_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
static int g_ov_split[DBD_STAGE_COUNT] = {};
static bool bad_split(int32_t split) { return split < 0 || split > kMaxGemmSplit; }

struct DraftBufs {
  RowMeta meta;
  void* ctxfeat;
  float* fcout;         // fully connected fusion output before its RMSNorm [T, H] fp32
  float* x;
  size_t x_off;         // byte offset of x in the workspace
  void* xn;
  void* q;
  void* q_lo;           // low part of the rotated queries' bf16 pair (bf16 drafters)
  void* attn;
  void* act;
  void* xn_lo;          // low parts of the bf16 pairs (act_pairs only, else null)
  void* attn_lo;
  void* act_lo;
  float* part_o;
  float2* part_ml;
  AttnPlan* attn_plan;  // bf16 attention schedule (see launch_attn_plan)
  int32_t* attn_pref;
  int64_t* attn_total;
  float* lm_pv;
  int32_t* lm_pi;
  float* logits;
  float* vpv;
  int32_t* vpi;
  int32_t* vflag;
  uint64_t* zpart;
  float* row_max;
  int32_t* row_arg;
  int s_max;
  int split;
  int ntiles;
  float* gemm_part;
  size_t gemm_part_bytes;
};

// Asks a residual projection for the RMSNorm of its updated rows (see EpiArgs).
static void set_norm(EpiArgs* e, const void* g, void* out, void* out_lo, float eps) {
  e->norm_g = g;
  e->norm_out = out;
  e->norm_out_lo = out_lo;
  e->norm_eps = eps;
}

// Split-K partial bytes of one step's GEMMs with n sequences of block length B (the block
// projections and the LM head) and t ingested rows (the context K/V projection and the fully
// connected fusion; t = 0: none), kept apart because they depend on different sizes.  *lm_bn is
// the LM head tile's width.
static void step_gemm_parts(const dbd_model_desc& d, int n, int B, int n_anchor, int t,
                            float temperature, size_t* block_part, size_t* ingest_part,
                            int* lm_bn) {
  const bool pr = d.dtype == DBD_BF16 && d.act_pairs;
  const int kd = d.n_kv_heads * d.head_dim, qd = d.n_q_heads * d.head_dim;
  const int M = n * B, Md = n * (B - n_anchor);
  auto need = [](const GemmPlan& p) { return p.split > 1 ? p.part_bytes : (size_t)0; };
  size_t bp = 0, ip = 0;
  if (n > 0) {
    // O and down ask for the following RMSNorm (down: not after the last layer), which can
    // change their tiles
    const bool nf = resid_norm_fits(d.hidden, d.hidden);
    const GemmPlan pl[6] = {
        plan_gemm(d.dtype, EPI_QKV, g_ov_cfg[DBD_STAGE_GEMM_QKV], M, qd + 2 * kd, d.hidden, 1,
                  0, 0, pr, true, g_ov_split[DBD_STAGE_GEMM_QKV]),
        plan_gemm(d.dtype, EPI_RESID, g_ov_cfg[DBD_STAGE_GEMM_O], M, d.hidden, qd, 1, 0, 0, pr,
                  true, g_ov_split[DBD_STAGE_GEMM_O], nf),
        plan_gemm(d.dtype, EPI_SWIGLU, g_ov_cfg[DBD_STAGE_GEMM_GATEUP], M, 2 * d.ffn, d.hidden,
                  1, 1, d.ffn, pr, true, g_ov_split[DBD_STAGE_GEMM_GATEUP]),
        plan_gemm(d.dtype, EPI_RESID, g_ov_cfg[DBD_STAGE_GEMM_DOWN], M, d.hidden, d.ffn, 1, 0, 0,
                  pr, true, g_ov_split[DBD_STAGE_GEMM_DOWN], nf),
        plan_gemm(d.dtype, EPI_RESID, g_ov_cfg[DBD_STAGE_GEMM_DOWN], M, d.hidden, d.ffn, 1, 0, 0,
                  pr, true, g_ov_split[DBD_STAGE_GEMM_DOWN], false),
        plan_gemm(d.dtype, temperature > 0.f ? EPI_STORE_F32 : EPI_ARGMAX,
                  g_ov_cfg[DBD_STAGE_GEMM_LMHEAD], Md, d.vocab, d.hidden, 1, 0, 0, pr, true,
                  g_ov_split[DBD_STAGE_GEMM_LMHEAD])};
    for (const GemmPlan& p : pl) bp = std::max(bp, need(p));
    if (lm_bn) *lm_bn = pl[5].bn;
  }
  if (d.n_target_layers > 0 && t > 0) {
    ip = need(plan_gemm(d.dtype, EPI_CTXKV, g_ov_cfg[DBD_STAGE_GEMM_CTXKV], t, 2 * kd, d.hidden,
                        d.n_layers, 0, 0, d.dtype == DBD_BF16, true,
                        g_ov_split[DBD_STAGE_GEMM_CTXKV]));
    if (d.ctx_fusion)
      ip = std::max(ip, need(plan_gemm(d.dtype, EPI_STORE_F32, -1, t, d.hidden,
                                       d.n_target_layers * d.hidden, 1, 0, 0, false, true)));
  }
  *block_part = bp;
  *ingest_part = ip;
}

// Rows of ingest up to which the workspace query takes the split-K need at every row count (the
// planner splits K only while a problem has too few tiles to fill the chip, far below this).
constexpr int kExactIngestRows = 4096;

// Workspace layout of one draft_block call; returns its size.  With at_most, the split-partial
// regions (attention and split-K) take their largest size over every batch 1 .. N and every
// ingest 1 .. T (exactly up to kExactIngestRows rows, and at T): both depend on the sizes
// through the tile and split choices and are not monotone, while every other buffer is.
size_t carve_draft(const dbd_model_desc& d, int N, int B, int n_anchor, int T, int K,
                   float temperature, int cap, char* base, DraftBufs* b, bool at_most) {
  Carver c{base};
  DraftBufs t{};
  const int es = elem_size(d.dtype);
  const int64_t M = (int64_t)N * B, Md = (int64_t)N * (B - n_anchor);
  const int half = d.head_dim / 2;
  const int qd = d.n_q_heads * d.head_dim;
  const int grp = d.n_q_heads / d.n_kv_heads;
  const int R = B * grp;
  const int Tn = T > 0 ? T : 1;
  t.meta.blk_pos = c.take<int32_t>(M);
  t.meta.ctx_seq = c.take<int32_t>(Tn);
  t.meta.ctx_pos = c.take<int32_t>(Tn);
  t.meta.seq_keys = c.take<int32_t>(N);
  t.meta.rope_blk = c.take<float2>(M * half);
  t.meta.rope_ctx = c.take<float2>((int64_t)Tn * half);
  // context features; bf16 keeps the (high, low) pair so the K/V projection sees ~16 bits
  // (one shared feature with the fully connected fusion, one per draft layer with mixing)
  const int nparts = d.dtype == DBD_BF16 ? 2 : 1;
  const int nfeat = d.ctx_fusion ? 1 : d.n_layers;
  t.ctxfeat = d.n_target_layers > 0
                  ? (void*)c.take<char>((int64_t)nparts * nfeat * Tn * d.hidden * es)
                  : nullptr;
  t.fcout = d.n_target_layers > 0 && d.ctx_fusion ? c.take<float>((int64_t)Tn * d.hidden)
                                                  : nullptr;
  t.x = c.take<float>(M * d.hidden);
  t.x_off = c.last;
  t.xn = c.take<char>(M * d.hidden * es);
  t.q = c.take<char>(M * qd * es);
  t.q_lo = d.dtype == DBD_BF16 ? (void*)c.take<char>(M * qd * es) : nullptr;
  t.attn = c.take<char>(M * qd * es);
  t.act = c.take<char>(M * d.ffn * es);
  if (d.dtype == DBD_BF16 && d.act_pairs) {
    t.xn_lo = c.take<char>(M * d.hidden * es);
    t.attn_lo = c.take<char>(M * qd * es);
    t.act_lo = c.take<char>(M * d.ffn * es);
  }
  t.split = attn_split_f32(cap, d.n_kv_heads, N);
  t.s_max = ceil_div(cap, t.split);
  const int64_t prow = attn_partial_rows(d.dtype, cap, d.n_kv_heads, N, R, at_most);
  t.part_o = c.take<float>(prow * d.head_dim);
  t.part_ml = c.take<float2>(prow);
  if (d.dtype == DBD_BF16) {
    t.attn_plan = c.take<AttnPlan>(attn_workgroups());
    t.attn_pref = c.take<int32_t>((int64_t)N + 1);
    t.attn_total = c.take<int64_t>(2);
  }
  // split-K partials: the largest need over the step's GEMMs
  {
    size_t bp = 0, ip = 0;
    int lm_bn = 128;
    step_gemm_parts(d, N, B, n_anchor, T, temperature, &bp, &ip, &lm_bn);
    t.ntiles = ceil_div(d.vocab, lm_bn);
    if (at_most) {
      for (int n = 1; n < N; ++n) {
        size_t x, y;
        step_gemm_parts(d, n, B, n_anchor, 0, temperature, &x, &y, nullptr);
        bp = std::max(bp, x);
      }
      for (int r = 1; r < T && r <= kExactIngestRows; ++r) {
        size_t x, y;
        step_gemm_parts(d, 0, B, n_anchor, r, temperature, &x, &y, nullptr);
        ip = std::max(ip, y);
      }
    }
    const size_t part = std::max(bp, ip);
    t.gemm_part = part ? (float*)c.take<char>((int64_t)part) : nullptr;
    t.gemm_part_bytes = part;
  }
  const int64_t max_tiles = ceil_div(d.vocab, 128);          // any configuration fits
  t.lm_pv = c.take<float>(Md * max_tiles);
  t.lm_pi = c.take<int32_t>(Md * max_tiles);
  if (temperature > 0.f) {
    const int nch = ceil_div(d.vocab, vocab_chunk());
    t.logits = c.take<float>(Md * d.vocab);
    t.vpv = c.take<float>(Md * nch);
    t.vpi = c.take<int32_t>(Md * nch);
    t.vflag = c.take<int32_t>(Md * nch);
    t.zpart = c.take<uint64_t>(Md * nch);
    t.row_max = c.take<float>(Md);
    t.row_arg = c.take<int32_t>(Md);
  }
  (void)K;
  if (b) *b = t;
  return (c.off + kAlign - 1) / kAlign * kAlign;
}

int check_desc(const dbd_model_desc* d) {
  if (!d) return fail(DBD_ERR_ARG, "desc is NULL");
  if (d->dtype != DBD_F32 && d->dtype != DBD_BF16)
    return fail(DBD_ERR_ARG, "dtype %d is neither DBD_F32 nor DBD_BF16", d->dtype);
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->ffn <= 0 ||
      d->n_layers <= 0 || d->vocab < 2 || d->n_target_layers < 0)
    return fail(DBD_ERR_ARG, "non-positive model dimension");
  if (d->vocab >= (1 << 18)) return fail(DBD_ERR_SHAPE, "vocab %d >= 2^18", d->vocab);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DBD_ERR_SHAPE, "head_dim %d: only 64 and 128 are supported", d->head_dim);
  if (d->n_q_heads % d->n_kv_heads)
    return fail(DBD_ERR_SHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads,
                d->n_kv_heads);
  const int qd = d->n_q_heads * d->head_dim, kd = d->n_kv_heads * d->head_dim;
  if (qd % 128 || kd % 128)
    return fail(DBD_ERR_SHAPE, "q_heads*head_dim (%d) and kv_heads*head_dim (%d) must be "
                "multiples of 128", qd, kd);
  if (d->hidden % 8) return fail(DBD_ERR_SHAPE, "hidden %d not a multiple of 8", d->hidden);
  if (d->dtype == DBD_BF16) {
    if (d->hidden % 64 || d->ffn % 64)
      return fail(DBD_ERR_SHAPE, "bf16 path needs hidden (%d) and ffn (%d) multiples of 64",
                  d->hidden, d->ffn);
    if (d->hidden > 8192) return fail(DBD_ERR_UNSUPPORTED, "hidden %d > 8192", d->hidden);
  } else if (d->hidden > 4096) {
    return fail(DBD_ERR_UNSUPPORTED, "fp32 path: hidden %d > 4096", d->hidden);
  }
  if (d->n_target_layers > 16)
    return fail(DBD_ERR_UNSUPPORTED, "n_target_layers %d > 16", d->n_target_layers);
  if ((d->ctx_fusion != 0 && d->ctx_fusion != 1) || (d->mix_raw != 0 && d->mix_raw != 1) ||
      (d->ctx_shared_kv != 0 && d->ctx_shared_kv != 1))
    return fail(DBD_ERR_ARG, "ctx_fusion, mix_raw and ctx_shared_kv must be 0 or 1");
  if (d->ctx_fusion && d->mix_raw)
    return fail(DBD_ERR_ARG, "mix_raw applies to the mixing path only (ctx_fusion == 0)");
  if (d->act_pairs != 0 && d->act_pairs != 1)
    return fail(DBD_ERR_ARG, "act_pairs must be 0 or 1");
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.0))
    return fail(DBD_ERR_ARG, "rms_eps must be >= 0 and rope_theta > 0");
  return DBD_OK;
}

int check_draft_shape(const dbd_model_desc* d, int N, int B, int n_anchor, int T, int K,
                      float temperature, int cap) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (N < 1) return fail(DBD_ERR_ARG, "batch %d < 1", N);
  if (n_anchor != 0 && n_anchor != 1) return fail(DBD_ERR_ARG, "n_anchor must be 0 or 1");
  if (B < 1 + n_anchor || B > 64) return fail(DBD_ERR_SHAPE, "block_len %d out of range", B);
  if (T < 0) return fail(DBD_ERR_ARG, "n_new_total %d < 0", T);
  if (d->n_target_layers == 0 && T > 0)
    return fail(DBD_ERR_ARG, "n_new_total must be 0 for a drafter without target mixing");
  if (K < 1 || K > 64) return fail(DBD_ERR_ARG, "n_drafts %d out of [1, 64]", K);
  if (!(temperature > 0.f) && K != 1)
    return fail(DBD_ERR_ARG, "argmax drafting (temperature <= 0) needs n_drafts == 1");
  if (!std::isfinite(temperature)) return fail(DBD_ERR_ARG, "temperature is not finite");
  if (cap < B || cap % 64) return fail(DBD_ERR_CAPACITY, "ctx_capacity %d must be >= block_len "
                                       "and a multiple of 64", cap);
  return DBD_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

const char* dbd_last_error(void) { return g_err.c_str(); }

int dbd_gemm_override(int32_t stage, int32_t tile_cfg, int32_t split) {
  g_err.clear();
  const bool gemm = stage == DBD_STAGE_GEMM_CTXKV || stage == DBD_STAGE_GEMM_QKV ||
                    stage == DBD_STAGE_GEMM_O || stage == DBD_STAGE_GEMM_GATEUP ||
                    stage == DBD_STAGE_GEMM_DOWN || stage == DBD_STAGE_GEMM_LMHEAD;
  if (!gemm) return fail(DBD_ERR_ARG, "stage %d is not a GEMM stage", stage);
  if (tile_cfg < -1 || tile_cfg > kMaxGemmCfg)
    return fail(DBD_ERR_ARG, "tile_cfg %d out of [-1, %d]", tile_cfg, kMaxGemmCfg);
  if (bad_split(split))
    return fail(DBD_ERR_ARG, "split %d out of [0, %d]", split, kMaxGemmSplit);
  g_ov_cfg[stage] = tile_cfg;
  g_ov_split[stage] = split;
  return DBD_OK;
}

int dbd_attn_override(int32_t workgroups, int32_t depth) {
  g_err.clear();
  if (workgroups < 0 || workgroups > kAttnMaxWorkgroups)
    return fail(DBD_ERR_ARG, "workgroups %d out of [0, %d]", workgroups, kAttnMaxWorkgroups);
  if (depth < 0 || depth > 2) return fail(DBD_ERR_ARG, "depth %d out of [0, 2]", depth);
  g_attn_workgroups = workgroups;
  g_attn_depth = depth;
  return DBD_OK;
}

int dbd_timing_enable(int on) {
  g_err.clear();
  g_timing.on = on != 0;
  return DBD_OK;
}

int dbd_timing_reset(void) {
  g_err.clear();
  g_timing.used = 0;
  return DBD_OK;
}

int dbd_timing_read(int stage, double* total_ms, int64_t* launches) {
  g_err.clear();
  if (!total_ms || !launches) return fail(DBD_ERR_ARG, "output pointer is NULL");
  if (stage < 0 || stage >= DBD_STAGE_COUNT) return fail(DBD_ERR_ARG, "bad stage %d", stage);
  double ms = 0.0;
  int64_t n = 0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    Timing::Pair& p = g_timing.pool[i];
    if (p.stage != stage) continue;
    HIP_TRY(hipEventSynchronize(p.b));
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, p.a, p.b));
    ms += t;
    ++n;
  }
  *total_ms = ms;
  *launches = n;
  return DBD_OK;
}

int dbd_draft_workspace_bytes(const dbd_model_desc* desc, int32_t max_batch, int32_t block_len,
                              int32_t n_anchor, int32_t max_new_tokens, int32_t n_drafts,
                              float temperature, int32_t ctx_capacity, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  int rc = check_draft_shape(desc, max_batch, block_len, n_anchor, max_new_tokens, n_drafts,
                             temperature, ctx_capacity);
  if (rc) return rc;
  *bytes = carve_draft(*desc, max_batch, block_len, n_anchor, max_new_tokens, n_drafts,
                       temperature, ctx_capacity, nullptr, nullptr, true);
  return DBD_OK;
}

int dbd_draft_residual_offset(const dbd_model_desc* desc, int32_t batch, int32_t block_len,
                              int32_t n_anchor, int32_t n_new_total, int32_t n_drafts,
                              float temperature, int32_t ctx_capacity, size_t* offset) {
  g_err.clear();
  if (!offset) return fail(DBD_ERR_ARG, "offset is NULL");
  int rc = check_draft_shape(desc, batch, block_len, n_anchor, n_new_total, n_drafts,
                             temperature, ctx_capacity);
  if (rc) return rc;
  DraftBufs b;
  carve_draft(*desc, batch, block_len, n_anchor, n_new_total, n_drafts, temperature,
              ctx_capacity, nullptr, &b, false);
  *offset = b.x_off;
  return DBD_OK;
}

int draft_block(const dbd_model_desc* desc, const dbd_weights* w, int32_t batch,
                int32_t block_len, int32_t n_anchor, const int32_t* block_tokens,
                const void* target_hidden_new, int64_t hid_token_stride,
                int64_t hid_layer_stride, int32_t n_new_total, const int32_t* new_offsets,
                const int32_t* ctx_len, void* kv_k, void* kv_v, int32_t ctx_capacity,
                int32_t n_drafts, float temperature, uint64_t seed, int32_t* draft_tokens,
                float* logits_out, int32_t* seq_status, void* workspace, size_t workspace_bytes,
                void* stream) {
  g_err.clear();
  int rc = check_draft_shape(desc, batch, block_len, n_anchor, n_new_total, n_drafts,
                             temperature, ctx_capacity);
  if (rc) return rc;
  const dbd_model_desc& d = *desc;
  if (!w) return fail(DBD_ERR_ARG, "weights is NULL");
  if (!block_tokens || !new_offsets || !ctx_len || !kv_k || !kv_v || !draft_tokens)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (!w->attn_norm_w || !w->wq || !w->wk_draft || !w->wv_draft || !w->wo || !w->mlp_norm_w ||
      !w->w_gate || !w->w_up || !w->w_down || !w->final_norm_w || !w->embed || !w->lm_head)
    return fail(DBD_ERR_ARG, "a required weight pointer is NULL");
  // the kernels read weights with 8- and 16-byte vector loads
  for (const void* p : {(const void*)w->mix_logits, w->mix_norm_w, w->wk_ctx, w->wv_ctx,
                        w->attn_norm_w, w->wq, w->wk_draft, w->wv_draft, w->wo, w->mlp_norm_w,
                        w->w_gate, w->w_up, w->w_down, w->final_norm_w, w->embed, w->lm_head,
                        w->fc_w, w->fc_norm_w})
    if (p && !aligned16(p)) return fail(DBD_ERR_SHAPE, "weight pointer %p is not 16-byte aligned", p);
  const int es = elem_size(d.dtype);
  const int vec = 16 / es;
  if (d.n_target_layers > 0) {
    if (d.ctx_fusion ? (!w->fc_w || !w->fc_norm_w) : (!w->mix_logits || !w->mix_norm_w))
      return fail(DBD_ERR_ARG, "context fusion weights are NULL but n_target_layers > 0");
    if (!d.ctx_shared_kv && (!w->wk_ctx || !w->wv_ctx))
      return fail(DBD_ERR_ARG, "context K/V weights are NULL but n_target_layers > 0");
    if (n_new_total > 0) {
      if (!target_hidden_new) return fail(DBD_ERR_ARG, "target_hidden_new is NULL");
      if (!aligned16(target_hidden_new) || hid_token_stride % vec || hid_layer_stride % vec)
        return fail(DBD_ERR_SHAPE, "target_hidden_new must be 16-byte aligned with strides "
                    "that are multiples of %d elements", vec);
      if (hid_token_stride <= 0 || hid_layer_stride <= 0)
        return fail(DBD_ERR_ARG, "hidden strides must be positive");
      if (d.ctx_fusion && (hid_layer_stride != d.hidden ||
                           hid_token_stride < (int64_t)d.n_target_layers * d.hidden))
        return fail(DBD_ERR_SHAPE, "fully connected fusion reads each token's target layers as "
                    "one concatenated row: hid_layer_stride must be H and hid_token_stride >= "
                    "L_t * H");
    }
  }
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const size_t need = carve_draft(d, batch, block_len, n_anchor, n_new_total, n_drafts,
                                  temperature, ctx_capacity, nullptr, nullptr, false);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  DraftBufs b;
  carve_draft(d, batch, block_len, n_anchor, n_new_total, n_drafts, temperature, ctx_capacity,
              (char*)workspace, &b, false);
  hipStream_t st = (hipStream_t)stream;

  const int N = batch, B = block_len, T = n_new_total;
  const int H = d.hidden, hd = d.head_dim, kvh = d.n_kv_heads;
  const int qd = d.n_q_heads * hd, kd = kvh * hd, F = d.ffn, V = d.vocab;
  const int M = N * B, D = B - n_anchor, Md = N * D;
  const int64_t layer_elems = (int64_t)N * kvh * ctx_capacity * hd;

  // rotary inverse frequencies theta^(-2i/hd), fp64
  double inv_freq[64];
  for (int i = 0; i < hd / 2; ++i) inv_freq[i] = std::pow(d.rope_theta, -2.0 * i / hd);
  HIP_STAGE(DBD_STAGE_PREP, st, launch_prep(ctx_len, new_offsets, N, B, T, ctx_capacity, hd, inv_freq, b.meta,
                      seq_status, st));
  if (d.dtype == DBD_BF16)
    HIP_STAGE(DBD_STAGE_PREP, st, launch_attn_plan(b.meta.seq_keys, N, hd, kvh, B * (d.n_q_heads / kvh),
                                                   attn_workgroups(), b.attn_plan, b.attn_pref,
                                                   b.attn_total, st));

  // 1. ingest: mix + RMSNorm, then context K/V for every draft layer (batched over layers)
  if (d.n_target_layers > 0 && T > 0) {
    const int nfeat = d.ctx_fusion ? 1 : d.n_layers;
    void* ctx_lo = d.dtype == DBD_BF16
                       ? (void*)((char*)b.ctxfeat + (int64_t)nfeat * T * H * es)
                       : nullptr;
    if (d.ctx_fusion) {
      // c = RMSNorm(fc_w . [h_0; ...; h_{L_t-1}]) * fc_norm_w, one feature for every layer
      GemmArgs f{};
      f.part = b.gemm_part;
      f.part_cap = b.gemm_part_bytes;
      f.A = target_hidden_new;
      f.lda = hid_token_stride;
      f.seg[0] = BSeg{w->fc_w, 0, H};
      f.nseg = 1;
      f.ldb = (int64_t)d.n_target_layers * H;
      f.M = T;
      f.N = H;
      f.K = d.n_target_layers * H;
      EpiArgs fe{};
      fe.kind = EPI_STORE_F32;
      fe.C = b.fcout;
      fe.ldc = H;
      HIP_STAGE(DBD_STAGE_MIX, st, launch_gemm(d.dtype, f, fe, 1, st));
      HIP_STAGE(DBD_STAGE_MIX, st, launch_rmsnorm(d.dtype, b.fcout, w->fc_norm_w, b.ctxfeat,
                                                  ctx_lo, T, H, d.rms_eps, 0, 0, st));
    } else {
      HIP_STAGE(DBD_STAGE_MIX, st, launch_mix_rmsnorm(d.dtype, target_hidden_new,
                                                      hid_token_stride, hid_layer_stride, T, H,
                                                      d.n_target_layers, d.n_layers,
                                                      w->mix_logits, d.mix_raw, w->mix_norm_w,
                                                      b.ctxfeat, ctx_lo, d.rms_eps, st));
    }
    GemmArgs g{};
    g.part = b.gemm_part;
    g.part_cap = b.gemm_part_bytes;
    g.A = b.ctxfeat;
    g.A2 = ctx_lo;
    g.lda = H;
    g.a_bs = d.ctx_fusion ? 0 : (int64_t)T * H;
    g.seg[0] = BSeg{d.ctx_shared_kv ? w->wk_draft : w->wk_ctx, 0, kd};
    g.seg[1] = BSeg{d.ctx_shared_kv ? w->wv_draft : w->wv_ctx, kd, 2 * kd};
    g.nseg = 2;
    g.ldb = H;
    g.b_bs = (int64_t)kd * H;
    g.M = T;
    g.N = 2 * kd;
    g.K = H;
    EpiArgs e{};
    e.kind = EPI_CTXKV;
    e.kv_k = kv_k;
    e.kv_v = kv_v;
    e.layer_stride = layer_elems;
    e.qd = qd;
    e.kd = kd;
    e.hd = hd;
    e.kvh = kvh;
    e.block_len = B;
    e.batch = N;
    e.cap = ctx_capacity;
    e.row_seq = b.meta.ctx_seq;
    e.row_pos = b.meta.ctx_pos;
    e.rope = b.meta.rope_ctx;
    HIP_STAGE(DBD_STAGE_GEMM_CTXKV, st, launch_gemm(d.dtype, g, e, d.n_layers, st, g_ov_cfg[DBD_STAGE_GEMM_CTXKV],
                                                  g_ov_split[DBD_STAGE_GEMM_CTXKV]));
  }

  // 2. block forward
  // the embedding gather also writes the first layer's attention norm when it can
  bool normed = false;        // the previous kernel already wrote this layer's norm
  HIP_STAGE(DBD_STAGE_ROWNORM, st, launch_embed(d.dtype, block_tokens, w->embed, M, H, V, b.x,
                                                w->attn_norm_w, b.xn, b.xn_lo, d.rms_eps, st,
                                                &normed));
  const char* cw = nullptr;
  for (int l = 0; l < d.n_layers; ++l) {
    auto lw = [&](const void* p, int64_t per_layer) {
      return (const void*)((const char*)p + (int64_t)l * per_layer * es);
    };
    if (!normed)
      HIP_STAGE(DBD_STAGE_ROWNORM, st, launch_rmsnorm(d.dtype, b.x, lw(w->attn_norm_w, H), b.xn,
                                                       b.xn_lo, M, H, d.rms_eps, B, 0, st));
    normed = false;
    {
      GemmArgs g{};
      g.part = b.gemm_part;
      g.part_cap = b.gemm_part_bytes;
      g.A = b.xn;
      g.A2 = b.xn_lo;
      g.lda = H;
      g.seg[0] = BSeg{lw(w->wq, (int64_t)qd * H), 0, qd};
      g.seg[1] = BSeg{lw(w->wk_draft, (int64_t)kd * H), qd, qd + kd};
      g.seg[2] = BSeg{lw(w->wv_draft, (int64_t)kd * H), qd + kd, qd + 2 * kd};
      g.nseg = 3;
      g.ldb = H;
      g.M = M;
      g.N = qd + 2 * kd;
      g.K = H;
      EpiArgs e{};
      e.kind = EPI_QKV;
      e.q_out = b.q;
      e.q_out_lo = b.q_lo;
      e.kv_k = kv_k;
      e.kv_v = kv_v;
      e.layer_off_k = (int64_t)l * layer_elems;
      e.qd = qd;
      e.kd = kd;
      e.hd = hd;
      e.kvh = kvh;
      e.block_len = B;
      e.batch = N;
      e.cap = ctx_capacity;
      e.row_pos = b.meta.blk_pos;
      e.rope = b.meta.rope_blk;
      HIP_STAGE(DBD_STAGE_GEMM_QKV, st, launch_gemm(d.dtype, g, e, 1, st, g_ov_cfg[DBD_STAGE_GEMM_QKV],
                                                  g_ov_split[DBD_STAGE_GEMM_QKV]));
    }
    {
      AttnArgs a{};
      a.q = b.q;
      a.q_lo = b.q_lo;
      a.kv_k = (const char*)kv_k + (int64_t)l * layer_elems * es;
      a.kv_v = (const char*)kv_v + (int64_t)l * layer_elems * es;
      a.seq_keys = b.meta.seq_keys;
      a.out = b.attn;
      a.out_lo = b.attn_lo;
      a.part_o = b.part_o;
      a.part_ml = b.part_ml;
      a.batch = N;
      a.kvh = kvh;
      a.grp = d.n_q_heads / kvh;
      a.block_len = B;
      a.cap = ctx_capacity;
      a.qd = qd;
      a.s_max = b.s_max;
      a.split = b.split;
      a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
      a.plan = b.attn_plan;
      a.plan_pref = b.attn_pref;
      a.plan_total = b.attn_total;
      a.workgroups = attn_workgroups();
      a.depth = attn_depth();
      HIP_STAGE(DBD_STAGE_ATTN, st, launch_attention(d.dtype, hd, a, st));
    }
    {
      GemmArgs g{};
      g.part = b.gemm_part;
      g.part_cap = b.gemm_part_bytes;
      g.A = b.attn;
      g.A2 = b.attn_lo;
      g.lda = qd;
      g.seg[0] = BSeg{lw(w->wo, (int64_t)H * qd), 0, H};
      g.nseg = 1;
      g.ldb = qd;
      g.M = M;
      g.N = H;
      g.K = qd;
      EpiArgs e{};
      e.kind = EPI_RESID;
      e.C = b.x;
      e.ldc = H;
      set_norm(&e, lw(w->mlp_norm_w, H), b.xn, b.xn_lo, d.rms_eps);
      HIP_STAGE(DBD_STAGE_GEMM_O, st, launch_gemm(d.dtype, g, e, 1, st, g_ov_cfg[DBD_STAGE_GEMM_O],
                                                  g_ov_split[DBD_STAGE_GEMM_O], &normed));
    }
    if (!normed)
      HIP_STAGE(DBD_STAGE_ROWNORM, st, launch_rmsnorm(d.dtype, b.x, lw(w->mlp_norm_w, H), b.xn,
                                                       b.xn_lo, M, H, d.rms_eps, B, 0, st));
    normed = false;
    {
      GemmArgs g{};
      g.part = b.gemm_part;
      g.part_cap = b.gemm_part_bytes;
      g.A = b.xn;
      g.A2 = b.xn_lo;
      g.lda = H;
      g.seg[0] = BSeg{lw(w->w_gate, (int64_t)F * H), 0, F};
      g.seg[1] = BSeg{lw(w->w_up, (int64_t)F * H), 0, F};
      g.nseg = 2;
      g.gateup = 1;
      g.ldb = H;
      g.M = M;
      g.N = 2 * F;                      // padded to whole gate|up column tiles by the launcher
      g.K = H;
      EpiArgs e{};
      e.kind = EPI_SWIGLU;
      e.act = b.act;
      e.act_lo = b.act_lo;
      e.F = F;
      HIP_STAGE(DBD_STAGE_GEMM_GATEUP, st, launch_gemm(d.dtype, g, e, 1, st, g_ov_cfg[DBD_STAGE_GEMM_GATEUP],
                                                  g_ov_split[DBD_STAGE_GEMM_GATEUP]));
    }
    {
      GemmArgs g{};
      g.part = b.gemm_part;
      g.part_cap = b.gemm_part_bytes;
      g.A = b.act;
      g.A2 = b.act_lo;
      g.lda = F;
      g.seg[0] = BSeg{lw(w->w_down, (int64_t)H * F), 0, H};
      g.nseg = 1;
      g.ldb = F;
      g.M = M;
      g.N = H;
      g.K = F;
      EpiArgs e{};
      e.kind = EPI_RESID;
      e.C = b.x;
      e.ldc = H;
      // the next layer's attention norm, or after the last layer the final norm of the mask
      // rows, written compactly for the LM head
      if (l + 1 < d.n_layers) {
        set_norm(&e, (const char*)w->attn_norm_w + (int64_t)(l + 1) * H * es, b.xn, b.xn_lo,
                 d.rms_eps);
      } else {
        set_norm(&e, w->final_norm_w, b.xn, b.xn_lo, d.rms_eps);
        e.norm_block_len = B;
        e.norm_n_anchor = n_anchor;
      }
      HIP_STAGE(DBD_STAGE_GEMM_DOWN, st, launch_gemm(d.dtype, g, e, 1, st, g_ov_cfg[DBD_STAGE_GEMM_DOWN],
                                                  g_ov_split[DBD_STAGE_GEMM_DOWN], &normed));
    }
  }
  (void)cw;

  // 3. final norm on the mask rows (unless the last down projection wrote it), LM head
  if (!normed)
    HIP_STAGE(DBD_STAGE_ROWNORM, st, launch_rmsnorm(d.dtype, b.x, w->final_norm_w, b.xn, b.xn_lo,
                                                     Md, H, d.rms_eps, B, n_anchor, st));
  const bool sampling = temperature > 0.f;
  float* logits = logits_out ? logits_out : (sampling ? b.logits : nullptr);
  {
    GemmArgs g{};
    g.part = b.gemm_part;
    g.part_cap = b.gemm_part_bytes;
    g.A = b.xn;
    g.A2 = b.xn_lo;
    g.lda = H;
    g.seg[0] = BSeg{w->lm_head, 0, V};
    g.nseg = 1;
    g.ldb = H;
    g.M = Md;
    g.N = V;
    g.K = H;
    EpiArgs e{};
    if (sampling) {
      e.kind = EPI_STORE_F32;
      e.C = logits;
      e.ldc = V;
    } else {
      e.kind = EPI_ARGMAX;
      e.part_val = b.lm_pv;
      e.part_idx = b.lm_pi;
      e.ntiles = b.ntiles;
      e.logits = logits;
      e.ldc = V;
    }
    HIP_STAGE(DBD_STAGE_GEMM_LMHEAD, st, launch_gemm(d.dtype, g, e, 1, st, g_ov_cfg[DBD_STAGE_GEMM_LMHEAD],
                                                  g_ov_split[DBD_STAGE_GEMM_LMHEAD]));
  }
  // 4. drafts
  if (!sampling) {
    HIP_STAGE(DBD_STAGE_DRAFT, st, launch_lm_argmax_final(b.lm_pv, b.lm_pi, Md, b.ntiles, b.meta.blk_pos, B, n_anchor,
                                   D, draft_tokens, st));
  } else {
    const int ch = vocab_chunk();
    const float inv_t = (float)(1.0 / (double)temperature);
    HIP_STAGE(DBD_STAGE_DRAFT, st, launch_argmax_partial(logits, Md, V, ch, b.vpv, b.vpi,
                                                         b.vflag, st));
    HIP_STAGE(DBD_STAGE_DRAFT, st, launch_zsum_partial(logits, Md, V, ch, b.vpv, b.vpi, inv_t, b.zpart, b.row_max,
                                b.row_arg, st));
    HIP_STAGE(DBD_STAGE_DRAFT, st, launch_sample_pick(logits, Md, V, ch, b.zpart, b.row_max, inv_t, D, n_drafts, seed,
                               b.meta.blk_pos, B, n_anchor, nullptr, draft_tokens, st));
  }
  return DBD_OK;
}

// ------------------------------------------------------------------ verify / select
static size_t carve_verify(int rows, int vocab, char* base, float** pv, int32_t** pi,
                           int32_t** pf) {
  Carver c{base};
  const int nch = ceil_div(vocab, vocab_chunk());
  float* a = c.take<float>((int64_t)rows * nch);
  int32_t* b = c.take<int32_t>((int64_t)rows * nch);
  int32_t* f = c.take<int32_t>((int64_t)rows * nch);
  if (pv) { *pv = a; *pi = b; *pf = f; }
  return (c.off + kAlign - 1) / kAlign * kAlign;
}

int dbd_verify_workspace_bytes(int32_t batch, int32_t n_rows, int32_t vocab, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_rows < 1 || vocab < 2) return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_verify(batch * n_rows, vocab, nullptr, nullptr, nullptr, nullptr);
  return DBD_OK;
}

static int check_verify_args(const float* target_logits, const int32_t* draft_tokens,
                             int32_t draft_stride, int32_t batch, int32_t n_draft,
                             int32_t n_rows, int32_t vocab, const int32_t* n_accepted,
                             const int32_t* bonus, const int32_t* committed) {
  if (!target_logits || !draft_tokens || !n_accepted || !bonus || !committed)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2 || vocab >= (1 << 18))
    return fail(DBD_ERR_ARG, "bad dimensions (batch %d, n_draft %d, vocab %d)", batch, n_draft,
                vocab);
  if (n_draft > 64) return fail(DBD_ERR_UNSUPPORTED, "n_draft %d > 64", n_draft);
  if (n_rows != n_draft && n_rows != n_draft + 1)
    return fail(DBD_ERR_SHAPE, "n_rows %d must be n_draft or n_draft + 1", n_rows);
  if (draft_stride < n_draft) return fail(DBD_ERR_SHAPE, "draft_stride < n_draft");
  return DBD_OK;
}

// The launches of verify_greedy on a scratch region of at least carve_verify() bytes.  Every
// partial the finalize kernel reads is written first by the argmax kernel of the same call, so
// the region needs no clearing.
static int run_verify_greedy(const float* target_logits, const int32_t* draft_tokens,
                             int32_t draft_stride, int32_t batch, int32_t n_draft,
                             int32_t n_rows, int32_t vocab, int32_t* n_accepted, int32_t* bonus,
                             int32_t* committed, int32_t* row_flags, void* scratch_mem,
                             hipStream_t st) {
  const int rows = batch * n_rows;
  float* pv;
  int32_t *pi, *pf;
  carve_verify(rows, vocab, (char*)scratch_mem, &pv, &pi, &pf);
  const int ch = vocab_chunk();
  HIP_STAGE(DBD_STAGE_VERIFY, st, launch_argmax_partial(target_logits, rows, vocab, ch, pv, pi,
                                                        pf, st));
  HIP_STAGE(DBD_STAGE_VERIFY, st, launch_verify_finalize(pv, pi, pf, ceil_div(vocab, ch), draft_tokens, draft_stride,
                                 batch, n_draft, n_rows, n_accepted, bonus, committed, row_flags,
                                 st));
  return DBD_OK;
}

int verify_greedy(const float* target_logits, const int32_t* draft_tokens, int32_t draft_stride,
                  int32_t batch, int32_t n_draft, int32_t n_rows, int32_t vocab,
                  int32_t* n_accepted, int32_t* bonus, int32_t* committed, int32_t* row_flags,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int rc = check_verify_args(target_logits, draft_tokens, draft_stride, batch, n_draft, n_rows,
                             vocab, n_accepted, bonus, committed);
  if (rc) return rc;
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const size_t need = carve_verify(batch * n_rows, vocab, nullptr, nullptr, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  return run_verify_greedy(target_logits, draft_tokens, draft_stride, batch, n_draft, n_rows,
                           vocab, n_accepted, bonus, committed, row_flags, workspace,
                           (hipStream_t)stream);
}

// Workspace of verify_sample: argmax partials, integer weight sums, row max / argmax of the
// target rows [batch * n_rows] and of the draft rows [batch * n_draft]; per sequence the accept
// result and the residual chunk sums (128-bit).
struct VsampleWs {
  float *pv_t, *pv_d, *rm_t, *rm_d;
  int32_t *pi_t, *pi_d, *pf_t, *pf_d, *ra_t, *ra_d;
  uint64_t *zp_t, *zp_d;
  int64_t* spec;
  void* wpart;
};
static size_t carve_vsample(int batch, int n_draft, int n_rows, int vocab, char* base,
                            VsampleWs* w) {
  Carver c{base};
  const int nch = ceil_div(vocab, vocab_chunk());
  const int64_t rt = (int64_t)batch * n_rows, rd = (int64_t)batch * n_draft;
  VsampleWs t;
  t.pv_t = c.take<float>(rt * nch);
  t.pi_t = c.take<int32_t>(rt * nch);
  t.pf_t = c.take<int32_t>(rt * nch);
  t.zp_t = c.take<uint64_t>(rt * nch);
  t.rm_t = c.take<float>(rt);
  t.ra_t = c.take<int32_t>(rt);
  t.pv_d = c.take<float>(rd * nch);
  t.pi_d = c.take<int32_t>(rd * nch);
  t.pf_d = c.take<int32_t>(rd * nch);
  t.zp_d = c.take<uint64_t>(rd * nch);
  t.rm_d = c.take<float>(rd);
  t.ra_d = c.take<int32_t>(rd);
  t.spec = c.take<int64_t>((int64_t)batch * 4);
  t.wpart = c.take<char>((int64_t)batch * nch * 16);
  if (w) *w = t;
  return (c.off + kAlign - 1) / kAlign * kAlign;
}

int dbd_verify_sample_workspace_bytes(int32_t batch, int32_t n_draft, int32_t n_rows,
                                      int32_t vocab, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_draft < 1 || n_rows < 1 || vocab < 2) return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_vsample(batch, n_draft, n_rows, vocab, nullptr, nullptr);
  return DBD_OK;
}

int verify_sample(const float* target_logits, const float* draft_logits,
                  const int32_t* draft_tokens, int32_t draft_stride, int32_t batch,
                  int32_t n_draft, int32_t n_rows, int32_t vocab, float t_target, float t_draft,
                  uint64_t seed, int32_t* n_accepted, int32_t* bonus, int32_t* committed,
                  int32_t* row_flags, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!target_logits || !draft_logits || !draft_tokens || !n_accepted || !bonus || !committed)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2 || vocab >= (1 << 18))
    return fail(DBD_ERR_ARG, "bad dimensions (batch %d, n_draft %d, vocab %d)", batch, n_draft,
                vocab);
  if (!(t_target > 0.f) || !(t_draft > 0.f) || !std::isfinite(t_target) ||
      !std::isfinite(t_draft))
    return fail(DBD_ERR_ARG, "temperatures must be finite and > 0 (%g, %g)", t_target, t_draft);
  if (n_draft > 64) return fail(DBD_ERR_UNSUPPORTED, "n_draft %d > 64", n_draft);
  if (n_rows != n_draft && n_rows != n_draft + 1)
    return fail(DBD_ERR_SHAPE, "n_rows %d must be n_draft or n_draft + 1", n_rows);
  if (draft_stride < n_draft) return fail(DBD_ERR_SHAPE, "draft_stride < n_draft");
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const size_t need = carve_vsample(batch, n_draft, n_rows, vocab, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  VsampleWs w;
  carve_vsample(batch, n_draft, n_rows, vocab, (char*)workspace, &w);
  hipStream_t st = (hipStream_t)stream;
  const int ch = vocab_chunk();
  const int rt = batch * n_rows, rd = batch * n_draft;
  const float inv_p = (float)(1.0 / (double)t_target), inv_q = (float)(1.0 / (double)t_draft);
  HIP_STAGE(DBD_STAGE_VERIFY, st,
            launch_argmax_partial(target_logits, rt, vocab, ch, w.pv_t, w.pi_t, w.pf_t, st));
  HIP_STAGE(DBD_STAGE_VERIFY, st,
            launch_argmax_partial(draft_logits, rd, vocab, ch, w.pv_d, w.pi_d, w.pf_d, st));
  HIP_STAGE(DBD_STAGE_VERIFY, st,
            launch_zsum_partial(target_logits, rt, vocab, ch, w.pv_t, w.pi_t, inv_p, w.zp_t,
                                w.rm_t, w.ra_t, st));
  HIP_STAGE(DBD_STAGE_VERIFY, st,
            launch_zsum_partial(draft_logits, rd, vocab, ch, w.pv_d, w.pi_d, inv_q, w.zp_d,
                                w.rm_d, w.ra_d, st));
  HIP_STAGE(DBD_STAGE_VERIFY, st,
            launch_verify_sample(target_logits, draft_logits, draft_tokens, draft_stride, batch,
                                 n_draft, n_rows, vocab, ch, w.zp_t, w.rm_t, w.zp_d, w.rm_d,
                                 w.pf_t, w.pf_d, inv_p, inv_q, seed, w.spec, w.wpart,
                                 n_accepted, bonus, committed, row_flags, st));
  return DBD_OK;
}

static size_t carve_select(int rows, int vocab, char* base, float** pv, int32_t** pi,
                           int32_t** pf, uint64_t** zp, float** rm, int32_t** ra) {
  Carver c{base};
  const int nch = ceil_div(vocab, vocab_chunk());
  float* a = c.take<float>((int64_t)rows * nch);
  int32_t* b = c.take<int32_t>((int64_t)rows * nch);
  int32_t* f = c.take<int32_t>((int64_t)rows * nch);
  uint64_t* z = c.take<uint64_t>((int64_t)rows * nch);
  float* m = c.take<float>(rows);
  int32_t* r = c.take<int32_t>(rows);
  if (pv) { *pv = a; *pi = b; *pf = f; *zp = z; *rm = m; *ra = r; }
  return (c.off + kAlign - 1) / kAlign * kAlign;
}

int dbd_select_workspace_bytes(int32_t batch, int32_t n_drafts, int32_t n_rows, int32_t vocab,
                               size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_drafts < 1 || n_rows < 1 || vocab < 2)
    return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_select(batch * n_drafts * n_rows, vocab, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr);
  return DBD_OK;
}

int select_streak(const float* verifier_logits, const int32_t* drafts, int32_t batch,
                  int32_t n_drafts, int32_t gamma, int32_t n_rows, int32_t vocab,
                  int32_t* selected, double* scores, int32_t* n_accepted, int32_t* bonus,
                  int32_t* committed, int32_t* row_flags, void* workspace,
                  size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!verifier_logits || !drafts || !selected || !n_accepted || !bonus || !committed)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (batch < 1 || n_drafts < 1 || gamma < 1 || vocab < 2 || vocab >= (1 << 18))
    return fail(DBD_ERR_ARG, "bad dimensions");
  if (n_drafts > 64) return fail(DBD_ERR_UNSUPPORTED, "n_drafts %d > 64", n_drafts);
  if (gamma > 64) return fail(DBD_ERR_UNSUPPORTED, "gamma %d > 64", gamma);
  if (n_rows != gamma && n_rows != gamma + 1)
    return fail(DBD_ERR_SHAPE, "n_rows %d must be gamma or gamma + 1", n_rows);
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const int rows = batch * n_drafts * n_rows;
  const size_t need = carve_select(rows, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  float *pv, *rm;
  int32_t *pi, *pf, *ra;
  uint64_t* zp;
  carve_select(rows, vocab, (char*)workspace, &pv, &pi, &pf, &zp, &rm, &ra);
  hipStream_t st = (hipStream_t)stream;
  const int ch = vocab_chunk();
  HIP_STAGE(DBD_STAGE_SELECT, st, launch_argmax_partial(verifier_logits, rows, vocab, ch, pv, pi,
                                                        pf, st));
  HIP_STAGE(DBD_STAGE_SELECT, st, launch_zsum_partial(verifier_logits, rows, vocab, ch, pv, pi,
                                                      1.0f, zp, rm, ra, st));
  HIP_STAGE(DBD_STAGE_SELECT, st, launch_select_finalize(verifier_logits, vocab, ch, zp, rm, ra, pf, drafts, batch,
                                 n_drafts, gamma, n_rows, selected, scores, n_accepted, bonus,
                                 committed, row_flags, st));
  return DBD_OK;
}

// ------------------------------------------------------------------ test hooks
static size_t carve_sample(int rows, int vocab, char* base, float** pv, int32_t** pi,
                           int32_t** pf, uint64_t** zp, float** rm, int32_t** ra) {
  return carve_select(rows, vocab, base, pv, pi, pf, zp, rm, ra);
}

int dbd_sample_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2) return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_sample(batch * n_draft, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr);
  return DBD_OK;
}

int dbd_sample_from_logits(const float* logits, int32_t batch, int32_t n_draft, int32_t vocab,
                           int32_t n_drafts, float temperature, uint64_t seed, int32_t* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!logits || !out) return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2 || vocab >= (1 << 18))
    return fail(DBD_ERR_ARG, "bad dimensions");
  if (n_drafts < 1 || n_drafts > 64) return fail(DBD_ERR_ARG, "n_drafts out of [1, 64]");
  if (!(temperature > 0.f) && n_drafts != 1)
    return fail(DBD_ERR_ARG, "argmax drafting (temperature <= 0) needs n_drafts == 1");
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const int rows = batch * n_draft;
  const size_t need = carve_sample(rows, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  float *pv, *rm;
  int32_t *pi, *pf, *ra;
  uint64_t* zp;
  carve_sample(rows, vocab, (char*)workspace, &pv, &pi, &pf, &zp, &rm, &ra);
  hipStream_t st = (hipStream_t)stream;
  const int ch = vocab_chunk();
  HIP_TRY(launch_argmax_partial(logits, rows, vocab, ch, pv, pi, pf, st));
  if (!(temperature > 0.f)) {
    HIP_TRY(launch_argmax_final(pv, pi, rows, ceil_div(vocab, ch), out, nullptr, st));
    return DBD_OK;
  }
  const float inv_t = (float)(1.0 / (double)temperature);
  HIP_TRY(launch_zsum_partial(logits, rows, vocab, ch, pv, pi, inv_t, zp, rm, ra, st));
  HIP_TRY(launch_sample_pick(logits, rows, vocab, ch, zp, rm, inv_t, n_draft, n_drafts, seed,
                             nullptr, 0, 0, nullptr, out, st));
  return DBD_OK;
}

// Top-p sampling workspace: the sampler's buffers, then the nucleus state, per-chunk digit
// histograms, tie counts and nucleus chunk sums.
struct ToppWs {
  int64_t* st;
  uint64_t *hist, *above, *keys, *rz;
  int32_t* cnt;
};

static size_t carve_top_p(int rows, int vocab, char* base, ToppWs* t) {
  const size_t s0 = carve_sample(rows, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr);
  Carver c{base ? base + s0 : nullptr};
  const int ch = vocab_chunk();
  const int64_t nch = ceil_div(vocab, ch);
  ToppWs w;
  w.st = c.take<int64_t>((int64_t)rows * 4);
  w.hist = c.take<uint64_t>((int64_t)rows * top_p_spans(vocab, ch) * top_p_bins());
  w.above = c.take<uint64_t>((int64_t)rows * nch);
  w.rz = c.take<uint64_t>((int64_t)rows * nch);
  w.cnt = c.take<int32_t>((int64_t)rows * nch);
  w.keys = c.take<uint64_t>((int64_t)rows * nch * top_p_cap());
  if (t) *t = w;
  return s0 + (c.off + kAlign - 1) / kAlign * kAlign;
}

int dbd_sample_top_p_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab,
                                     size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2) return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_top_p(batch * n_draft, vocab, nullptr, nullptr);
  return DBD_OK;
}

int dbd_sample_top_p(const float* logits, int32_t batch, int32_t n_draft, int32_t vocab,
                     int32_t n_drafts, float temperature, float top_p, uint64_t seed,
                     int32_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!logits || !out) return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2 || vocab >= (1 << 18))
    return fail(DBD_ERR_ARG, "bad dimensions");
  if (n_drafts < 1 || n_drafts > 64) return fail(DBD_ERR_ARG, "n_drafts out of [1, 64]");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DBD_ERR_ARG, "top-p sampling needs a finite temperature > 0");
  if (!(top_p > 0.f) || !std::isfinite(top_p))
    return fail(DBD_ERR_ARG, "top_p must be finite and > 0");
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const int rows = batch * n_draft;
  const size_t need = carve_top_p(rows, vocab, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  float *pv, *rm;
  int32_t *pi, *pf, *ra;
  uint64_t* zp;
  ToppWs tw;
  carve_sample(rows, vocab, (char*)workspace, &pv, &pi, &pf, &zp, &rm, &ra);
  carve_top_p(rows, vocab, (char*)workspace, &tw);
  hipStream_t st = (hipStream_t)stream;
  const int ch = vocab_chunk();
  const float inv_t = (float)(1.0 / (double)temperature);
  HIP_TRY(launch_argmax_partial(logits, rows, vocab, ch, pv, pi, pf, st));
  if (top_p >= 1.f) {
    HIP_TRY(launch_zsum_partial(logits, rows, vocab, ch, pv, pi, inv_t, zp, rm, ra, st));
    HIP_TRY(launch_sample_pick(logits, rows, vocab, ch, zp, rm, inv_t, n_draft, n_drafts, seed,
                               nullptr, 0, 0, nullptr, out, st));
    return DBD_OK;
  }
  // p = mp / 2^sp exactly: the float's 24-bit significand and its binary exponent
  int e = 0;
  const float m = std::frexp(top_p, &e);              // top_p = m * 2^e, m in [0.5, 1)
  const uint64_t mp = (uint64_t)std::ldexp((double)m, 24);
  const int sp = 24 - e;
  HIP_TRY(launch_top_p(logits, rows, vocab, ch, pv, pi, inv_t, mp, sp, rm, tw.st, tw.hist,
                       tw.above, tw.cnt, tw.keys, tw.rz, st));
  HIP_TRY(launch_sample_pick(logits, rows, vocab, ch, tw.rz, rm, inv_t, n_draft, n_drafts, seed,
                             nullptr, 0, 0, tw.st, out, st));
  return DBD_OK;
}

int dbd_refine_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (batch < 1 || n_draft < 1 || vocab < 2) return fail(DBD_ERR_ARG, "bad dimensions");
  *bytes = carve_sample(batch * n_draft, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr);
  return DBD_OK;
}

int refine_block(const float* logits, int32_t batch, int32_t block_len, int32_t n_anchor,
                 int32_t vocab, int32_t mask_id, int32_t n_remask, int32_t* block_tokens,
                 uint64_t* conf, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!logits || !block_tokens || !conf)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (n_anchor != 0 && n_anchor != 1) return fail(DBD_ERR_ARG, "n_anchor must be 0 or 1");
  if (batch < 1 || block_len < 1 + n_anchor || block_len > 64)
    return fail(DBD_ERR_SHAPE, "batch %d / block_len %d out of range", batch, block_len);
  if (vocab < 2 || vocab >= (1 << 18)) return fail(DBD_ERR_SHAPE, "vocab %d out of range", vocab);
  const int D = block_len - n_anchor;
  if (mask_id < 0 || mask_id >= vocab) return fail(DBD_ERR_ARG, "mask_id %d not in the vocabulary", mask_id);
  if (n_remask < 0 || n_remask > D)
    return fail(DBD_ERR_ARG, "n_remask %d out of [0, %d]", n_remask, D);
  if (!workspace || ((uintptr_t)workspace % kAlign))
    return fail(DBD_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
  const int rows = batch * D;
  const size_t need = carve_sample(rows, vocab, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  float *pv, *rm;
  int32_t *pi, *pf, *ra;
  uint64_t* zp;
  carve_sample(rows, vocab, (char*)workspace, &pv, &pi, &pf, &zp, &rm, &ra);
  hipStream_t st = (hipStream_t)stream;
  const int ch = vocab_chunk();
  HIP_TRY(launch_argmax_partial(logits, rows, vocab, ch, pv, pi, pf, st));
  HIP_TRY(launch_zsum_partial(logits, rows, vocab, ch, pv, pi, 1.0f, zp, rm, ra, st));
  HIP_TRY(launch_refine(ra, zp, batch, vocab, ch, D, block_len, n_anchor, mask_id, n_remask,
                        block_tokens, conf, st));
  return DBD_OK;
}

int dbd_mix_rmsnorm(const dbd_model_desc* desc, const float* mix_logits, const void* mix_norm_w,
                    const void* hidden, int64_t hid_token_stride, int64_t hid_layer_stride,
                    int32_t n_tokens, void* out, void* stream) {
  g_err.clear();
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->n_target_layers < 1) return fail(DBD_ERR_ARG, "n_target_layers must be >= 1");
  if (!mix_logits || !mix_norm_w || !hidden || !out)
    return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  const int vec = 16 / elem_size(desc->dtype);
  if (!aligned16(hidden) || hid_token_stride % vec || hid_layer_stride % vec || n_tokens < 0)
    return fail(DBD_ERR_SHAPE, "hidden must be 16-byte aligned with strides multiple of %d",
                vec);
  HIP_TRY(launch_mix_rmsnorm(desc->dtype, hidden, hid_token_stride, hid_layer_stride, n_tokens,
                             desc->hidden, desc->n_target_layers, desc->n_layers, mix_logits,
                             desc->mix_raw,
                             mix_norm_w, out, nullptr, desc->rms_eps, (hipStream_t)stream));
  return DBD_OK;
}

static size_t gemm_ws_bytes(int dtype, int M, int N, int K, int cfg, int split) {
  const GemmPlan p = plan_gemm(dtype, EPI_STORE_F32, cfg, M, N, K, 1, 0, 0, false, true, split);
  return p.split > 1 ? p.part_bytes : 0;
}

int dbd_gemm_workspace_bytes(int32_t dtype, int32_t M, int32_t N, int32_t K, int32_t tile_cfg,
                             int32_t split, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DBD_ERR_ARG, "bytes is NULL");
  if (dtype != DBD_F32 && dtype != DBD_BF16) return fail(DBD_ERR_ARG, "bad dtype");
  if (M < 0 || N < 0 || K < 1) return fail(DBD_ERR_SHAPE, "bad GEMM dimensions");
  if (tile_cfg < -1 || tile_cfg > kMaxGemmCfg)
    return fail(DBD_ERR_ARG, "tile_cfg %d out of [-1, %d]", tile_cfg, kMaxGemmCfg);
  if (bad_split(split))
    return fail(DBD_ERR_ARG, "split %d out of [0, %d]", split, kMaxGemmSplit);
  *bytes = M > 0 && N > 0 ? gemm_ws_bytes(dtype, M, N, K, tile_cfg, split) : 0;
  return DBD_OK;
}

int dbd_gemm_nt(int32_t dtype, const void* A, const void* Bm, float* C, int32_t M, int32_t N,
                int32_t K, int64_t lda, int64_t ldb, int64_t ldc, int32_t tile_cfg,
                int32_t split, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (dtype != DBD_F32 && dtype != DBD_BF16) return fail(DBD_ERR_ARG, "bad dtype");
  if (!A || !Bm || !C) return fail(DBD_ERR_ARG, "a required device pointer is NULL");
  if (M < 0 || N < 0 || K < 1 || lda < K || ldb < K || ldc < N)
    return fail(DBD_ERR_SHAPE, "bad GEMM dimensions");
  if (dtype == DBD_BF16 && (K % 64 || lda % 8 || ldb % 8 || !aligned16(A) || !aligned16(Bm)))
    return fail(DBD_ERR_SHAPE, "bf16 GEMM needs K % 64 == 0, 16-byte aligned rows");
  if (tile_cfg < -1 || tile_cfg > kMaxGemmCfg)
    return fail(DBD_ERR_ARG, "tile_cfg %d out of [-1, %d]", tile_cfg, kMaxGemmCfg);
  if (bad_split(split))
    return fail(DBD_ERR_ARG, "split %d out of [0, %d]", split, kMaxGemmSplit);
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.seg[0] = BSeg{Bm, 0, N};
  g.nseg = 1;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  EpiArgs e{};
  e.kind = EPI_STORE_F32;
  e.C = C;
  e.ldc = ldc;
  hipStream_t st = (hipStream_t)stream;
  if (workspace && M > 0 && N > 0) {
    const size_t need = gemm_ws_bytes(dtype, M, N, K, tile_cfg, split);
    if ((uintptr_t)workspace % kAlign)
      return fail(DBD_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(DBD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                  need);
    g.part = (float*)workspace;
    g.part_cap = workspace_bytes;
  }
  HIP_TRY(launch_gemm(dtype, g, e, 1, st, tile_cfg, split));
  return DBD_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ verify without a workspace
// verify_greedy_noalloc keeps its argmax partials in this file-scope device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: kernels get the address
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kStaticScratchBytes = DBD_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];      // per device: the array's device address

// The current device's scratch address; `stream` must belong to the current device.
int static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(DBD_ERR_UNSUPPORTED, "device %d: static scratch tracks devices 0..%d", dev,
                kMaxScratchDevices - 1);
  if (stream) {
    hipDevice_t sdev = -1;
    HIP_TRY(hipStreamGetDevice(stream, &sdev));
    if (sdev != dev)
      return fail(DBD_ERR_ARG, "stream belongs to device %d but device %d is current", sdev,
                  dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || ((uintptr_t)p % kAlign))
      return fail(DBD_ERR_HIP, "static scratch address %p is not 256-byte aligned", p);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DBD_OK;
}
}  // namespace

extern "C" {

int verify_greedy_noalloc(const float* target_logits, const int32_t* draft_tokens,
                          int32_t draft_stride, int32_t batch, int32_t n_draft, int32_t n_rows,
                          int32_t vocab, int32_t* n_accepted, int32_t* bonus, int32_t* committed,
                          int32_t* row_flags, void* stream) {
  g_err.clear();
  int rc = check_verify_args(target_logits, draft_tokens, draft_stride, batch, n_draft, n_rows,
                             vocab, n_accepted, bonus, committed);
  if (rc) return rc;
  const size_t need = carve_verify(batch * n_rows, vocab, nullptr, nullptr, nullptr, nullptr);
  if (need > kStaticScratchBytes)
    return fail(DBD_ERR_WORKSPACE, "verify_greedy_noalloc: %d rows over vocab %d need %zu bytes "
                "of scratch, above the static limit of %zu bytes (use verify_greedy with a "
                "workspace)", batch * n_rows, vocab, need, kStaticScratchBytes);
  void* mem = nullptr;
  rc = static_scratch((hipStream_t)stream, &mem);
  if (rc) return rc;
  return run_verify_greedy(target_logits, draft_tokens, draft_stride, batch, n_draft, n_rows,
                           vocab, n_accepted, bonus, committed, row_flags, mem,
                           (hipStream_t)stream);
}

}  // extern "C"
