/*
 * dbd.h - C ABI of libdbd.so: the data-parallel hot path of block-diffusion speculative drafting
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (the pages the library is built from):
 *   [DFlare]     "DFlare: Scaling Up Draft Capacity for Block Diffusion Speculative Decoding", as
 *                summarised on the iplexlaw blog page on DFlare block-diffusion drafting.
 *   [SpecDiff-2] "SpecDiff-2: Scaling Diffusion Drafter Alignment For Faster Speculative
 *                Decoding", MLSys 2026 talk notes.
 *   [DFlash]     "DFlash: Block Diffusion for Flash Speculative Decoding", Qiita article.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and allocates every
 *     buffer, including the workspace; the library allocates and frees nothing and keeps no
 *     device state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  Calls return after
 *     enqueueing; they never synchronise the device.
 *   - Arguments are validated on the host before any launch; a non-zero return means nothing was
 *     enqueued.  dbd_last_error() gives a message for the last failure on the calling thread.
 *   - Dense tensors are row-major and contiguous unless a stride is given; "Linear" weights are
 *     [out_features, in_features] (y = x W^T).
 *   - Integer outputs (token ids, accepted lengths, selected drafts) are a pure function of the
 *     inputs; ties in an argmax go to the lowest token index, ties between drafts to the lowest
 *     draft index.
 *   - Calls on different streams with disjoint output buffers are independent.
 */
#ifndef DBD_H
#define DBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  DBD_OK = 0,
  DBD_ERR_ARG = -1,          /* a required pointer is NULL or a scalar is out of range */
  DBD_ERR_SHAPE = -2,        /* dimensions inconsistent or not supported by the kernels */
  DBD_ERR_CAPACITY = -3,     /* KV-cache capacity too small for the requested work */
  DBD_ERR_WORKSPACE = -4,    /* workspace NULL, misaligned (256 B) or smaller than required */
  DBD_ERR_UNSUPPORTED = -5,  /* valid request outside what the library implements */
  DBD_ERR_HIP = -6           /* a HIP runtime call failed (message has the HIP error) */
};

/* Element type of weights, target hidden states, KV cache and internal activations. */
enum { DBD_F32 = 0, DBD_BF16 = 1 };

/* Per-sequence status bits written by draft_block (seq_status) and the verify calls
 * (row_flags). */
enum {
  DBD_SEQ_NONFINITE = 1,     /* a non-finite logit was seen in this sequence's rows */
  DBD_SEQ_BAD_LENGTH = 2     /* ctx_len / new_offsets inconsistent or beyond capacity: the
                                sequence was skipped and its outputs are -1 */
};

/* Drafter architecture (host struct).
 * [DFlare], sections on per-draft-layer mixing and on splitting K/V projections by source:
 * every draft layer mixes n_target_layers target hidden states with its own softmax weights and
 * RMS-normalises the mix; context features and draft-block features have separate K/V
 * projections; queries come from the draft block.  The block is one forward pass, attention is
 * bidirectional inside the block and reaches the whole context ([DFlare] section on parallel
 * drafting; [DFlash] section on writing a block in one forward pass).  The embedding and LM head
 * are the target's, shared.  Layer form: pre-norm, RMSNorm y = x / sqrt(mean(x^2) + rms_eps) * g,
 * rotate-half RoPE with base rope_theta on Q and on both kinds of K, SwiGLU MLP, no biases.
 * n_target_layers = 0 describes a drafter with no target mixing ([SpecDiff-2] section 4: a
 * standalone diffusion drafter) whose context K/V the caller supplies in the cache. */
typedef struct {
  int32_t hidden;            /* H */
  int32_t n_q_heads;         /* qh */
  int32_t n_kv_heads;        /* kvh; qh % kvh == 0 */
  int32_t head_dim;          /* hd: 64 or 128 */
  int32_t ffn;               /* F, SwiGLU inner size */
  int32_t n_layers;          /* L_d, draft layers */
  int32_t n_target_layers;   /* L_t, mixed target layers (0..16); 0 = context K/V in the cache */
  int32_t vocab;             /* V < 2^18 */
  int32_t mask_token_id;     /* id of [MASK] (informational: block_tokens carry the ids) */
  int32_t dtype;             /* DBD_F32 or DBD_BF16 */
  float rms_eps;             /* e.g. 1e-6 */
  int32_t act_pairs;         /* bf16 only: 1 = feed every projection GEMM its activation as a
                                bf16 (high, low) pair, ~16 significant bits, at twice the MFMA
                                work; 0 = plain bf16 activations.  The mixed context features
                                always use the pair. */
  double rope_theta;         /* e.g. 1e6 */
  /* Context-feature path ([DFlare] sections on per-layer mixing and on splitting K/V by source;
   * its ablations; [DFlash] fusion of the target features).  All 0 = the mixing drafter. */
  int32_t ctx_fusion;        /* 0: per-draft-layer softmax mixing of the L_t target layers, then
                                RMSNorm * mix_norm_w[l]; 1: one fully connected fusion of the
                                concatenated target layers, RMSNorm(fc_w . [h_0; ...; h_{L_t-1}])
                                * fc_norm_w, shared by every draft layer (needs
                                hid_layer_stride == H) */
  int32_t mix_raw;           /* ctx_fusion 0 only: 1 = mixing coefficients used as given, no
                                softmax */
  int32_t ctx_shared_kv;     /* 1 = the context K/V are projected with the draft block's
                                wk_draft / wv_draft (no K/V split; wk_ctx / wv_ctx unused) */
} dbd_model_desc;

/* Drafter weights (device pointers, element type desc.dtype unless noted, each 16-byte aligned:
 * draft_block returns DBD_ERR_SHAPE otherwise).  Per-layer tensors are stacked over the L_d
 * draft layers. */
typedef struct {
  const float* mix_logits;   /* [L_d, L_t] fp32 mixing logits (unused if L_t == 0) */
  const void* mix_norm_w;    /* [L_d, H] RMSNorm gain after mixing (unused if L_t == 0) */
  const void* wk_ctx;        /* [L_d, kvh*hd, H] context K projection (unused if L_t == 0) */
  const void* wv_ctx;        /* [L_d, kvh*hd, H] context V projection (unused if L_t == 0) */
  const void* attn_norm_w;   /* [L_d, H] */
  const void* wq;            /* [L_d, qh*hd, H] */
  const void* wk_draft;      /* [L_d, kvh*hd, H] draft-block K projection */
  const void* wv_draft;      /* [L_d, kvh*hd, H] draft-block V projection */
  const void* wo;            /* [L_d, H, qh*hd] */
  const void* mlp_norm_w;    /* [L_d, H] */
  const void* w_gate;        /* [L_d, F, H] */
  const void* w_up;          /* [L_d, F, H] */
  const void* w_down;        /* [L_d, H, F] */
  const void* final_norm_w;  /* [H] */
  const void* embed;         /* [V, H] shared token embedding */
  const void* lm_head;       /* [V, H] shared LM head (may alias embed) */
  const void* fc_w;          /* [H, L_t*H] fully connected context fusion (ctx_fusion == 1) */
  const void* fc_norm_w;     /* [H] RMSNorm gain after the fusion (ctx_fusion == 1) */
} dbd_weights;

/* KV-cache layout (device, element type desc.dtype, caller-owned, persistent across calls):
 *   kv_k: [L_d, N, kvh, ctx_capacity, hd]        rotated keys, one row of hd per position;
 *   kv_v: [L_d, N, kvh, ctx_capacity/8, hd, 8]   values in blocks of 8 positions: value (p, d)
 *         sits at [p/8][d][p%8], so the attention's P.V product reads 8 consecutive positions
 *         of one dimension as one 16-byte vector and a 64-position chunk is contiguous.
 * ctx_capacity must be a multiple of 64. */

/* Workspace size (host) for draft_block with at most `max_batch` sequences, block length
 * `block_len`, `n_anchor` anchors, at most `max_new_tokens` ingested rows in total, `n_drafts`
 * drafts per block, the given temperature (> 0: sampling) and cache capacity. */
int dbd_draft_workspace_bytes(const dbd_model_desc* desc, int32_t max_batch, int32_t block_len,
                              int32_t n_anchor, int32_t max_new_tokens, int32_t n_drafts,
                              float temperature, int32_t ctx_capacity,
                              size_t* bytes /* host out */);

/* draft_block: one forward pass of the block-diffusion drafter for a batch of sequences,
 * followed by drafting from its single-step marginals.
 *
 * Steps ([DFlare] mixing / K-V split / parallel drafting sections; [SpecDiff-2] sections 4
 * and 5.2):
 *   1. ingest: for the n_new[n] = new_offsets[n+1] - new_offsets[n] newly committed positions of
 *      each sequence (rows new_offsets[n] .. new_offsets[n+1]-1 of target_hidden_new, positions
 *      ctx_len[n] .. ctx_len[n]+n_new[n]-1), every draft layer l mixes the L_t target hidden
 *      states with softmax(mix_logits[l]), applies RMSNorm * mix_norm_w[l], projects with
 *      wk_ctx[l] / wv_ctx[l], rotates K and appends both to the cache;
 *   2. block: x = embed[block_tokens] at positions P+b, P = ctx_len[n] + n_new[n]; each layer:
 *      RMSNorm, Q/K/V from the block with wq/wk_draft/wv_draft (Q and K rotated); the block's K/V
 *      are written into the cache at positions P .. P+B-1 (scratch: the next call's ingest
 *      overwrites them); attention of every block row over cache positions 0 .. P+B-1 with no
 *      mask; output projection and residual; RMSNorm, SwiGLU MLP and residual;
 *   3. head: final RMSNorm and LM head on the D = B - n_anchor mask rows;
 *   4. drafts: temperature <= 0 -> per-row argmax (n_drafts must be 1); temperature > 0 ->
 *      n_drafts independent joint drafts, each position sampled from softmax(logits / T) with the
 *      library's integer-exact sampler (counter RNG seeded by `seed`).
 *
 * block_tokens      [N, B] int32 (device): [anchor, MASK, ...] (n_anchor = 1) or all masks (0).
 * target_hidden_new device, element type desc.dtype: row t, target layer i starts at element
 *                   t*hid_token_stride + i*hid_layer_stride; H contiguous.  May be NULL when
 *                   n_new_total == 0.  Ignored when L_t == 0.
 * n_new_total       (host) total ingested rows = new_offsets[N] - new_offsets[0]; must be 0 when
 *                   L_t == 0.
 * new_offsets       [N+1] int32 (device), non-decreasing.
 * ctx_len           [N] int32 (device): cached positions before this call.  Not modified; the
 *                   caller advances it by n_new[n] after the call.
 * kv_k, kv_v        the cache (layout above), read and written.
 * draft_tokens      [N, n_drafts, D] int32 (device) out.
 * logits_out        [N, D, V] fp32 (device) out, optional (NULL): the LM-head logits.
 * seq_status        [N] int32 (device) out, optional: DBD_SEQ_* bits.
 * workspace         device, 256-byte aligned, >= dbd_draft_workspace_bytes(...).
 *
 * Sequences whose lengths do not fit the capacity (P + B > ctx_capacity) are detected on the
 * device: they get DBD_SEQ_BAD_LENGTH, their drafts are -1 and the cache is not touched for
 * them. */
int draft_block(const dbd_model_desc* desc, const dbd_weights* weights, int32_t batch,
                int32_t block_len, int32_t n_anchor, const int32_t* block_tokens,
                const void* target_hidden_new, int64_t hid_token_stride,
                int64_t hid_layer_stride, int32_t n_new_total, const int32_t* new_offsets,
                const int32_t* ctx_len, void* kv_k, void* kv_v, int32_t ctx_capacity,
                int32_t n_drafts, float temperature, uint64_t seed, int32_t* draft_tokens,
                float* logits_out, int32_t* seq_status, void* workspace, size_t workspace_bytes,
                void* stream);

/* Workspace size (host) for verify_greedy. */
int dbd_verify_workspace_bytes(int32_t batch, int32_t n_rows, int32_t vocab,
                               size_t* bytes /* host out */);

/* verify_greedy: greedy verification of one draft per sequence ([DFlare] section on parallel
 * drafting and acceptance by the target: under greedy decoding the prefix up to the first
 * mismatch is accepted and the target's next token is appended).
 *
 * target_logits [N, n_rows, V] fp32: row j is the target's distribution for draft position j;
 *               n_rows is D or D+1 (the last row scores the token after a full accept).
 * draft_tokens  [N, D] int32, row stride `draft_stride` elements (>= D).
 * With t_j = argmax(row j): n_accepted[n] = first j with draft[j] != t_j (D if none);
 * bonus[n] = t_{n_acc} if n_acc < n_rows else -1; committed[n] = draft[0..n_acc-1] followed by
 * the bonus, padded with -1 to D+1 entries.  row_flags[n] (optional) gets DBD_SEQ_NONFINITE if a
 * non-finite logit was seen (the argmax then ignores NaNs). */
int verify_greedy(const float* target_logits, const int32_t* draft_tokens, int32_t draft_stride,
                  int32_t batch, int32_t n_draft, int32_t n_rows, int32_t vocab,
                  int32_t* n_accepted, int32_t* bonus, int32_t* committed, int32_t* row_flags,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's static device scratch (see verify_greedy_noalloc). */
#define DBD_STATIC_SCRATCH_BYTES ((size_t)4 << 20)

/* verify_greedy_noalloc: verify_greedy with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and validation as verify_greedy; the argmax
 * partials live in a static device array of DBD_STATIC_SCRATCH_BYTES that each GPU holds from
 * the library's first use on it until the process ends.  The call allocates nothing.
 *
 * Limit: batch * n_rows * ceil(vocab / 4096) row-chunk partials of 12 bytes (each of the three
 * arrays rounded up to 256 bytes) must fit the array, e.g. 512 rows over a 151,936-token vocab
 * (233 KB); larger calls return DBD_ERR_WORKSPACE.  The stream must belong to the current device
 * (DBD_ERR_ARG otherwise).  Every call on one GPU uses the same array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must be serialised by the caller.  No
 * part of the array needs to start cleared: a call writes every partial it reads. */
int verify_greedy_noalloc(const float* target_logits, const int32_t* draft_tokens,
                          int32_t draft_stride, int32_t batch, int32_t n_draft, int32_t n_rows,
                          int32_t vocab, int32_t* n_accepted, int32_t* bonus, int32_t* committed,
                          int32_t* row_flags, void* stream);

/* Workspace size (host) for verify_sample. */
int dbd_verify_sample_workspace_bytes(int32_t batch, int32_t n_draft, int32_t n_rows,
                                      int32_t vocab, size_t* bytes /* host out */);

/* verify_sample: lossless stochastic verification of one draft per sequence ([SpecDiff-2]
 * section 4: the verifier applies a lossless acceptance rule left to right; section 5.1: its
 * per-position accept rate is sum_x min(P, Q)).  The rule is the speculative-sampling rule
 * (Leviathan et al., 2023) in the library's integer arithmetic: P_j = the integer weights of
 * target row j at t_target, Q_j = those of draft row j at t_draft (as in the sampler of
 * draft_block), each a pure function of the fp32 logits.
 *
 * For j = 0 .. D-1: draft token x_j is accepted iff u * q_Q(x_j) * Z_P < q_P(x_j) * Z_Q * 2^32
 * (probability min(1, P_j(x_j) / Q_j(x_j))), u the 32-bit draw (seed, n, stream 0, j); a token
 * outside [0, V) is rejected.  At the first rejection j the replacement token is drawn (stream 1,
 * position j) from the weights max(0, q_P(v) Z_Q - q_Q(v) Z_P) (from q_P when those are all 0)
 * and verification stops; after a full accept a bonus token is drawn from target row D (stream
 * 1, position D) when n_rows = D + 1, else there is none (-1).  The committed tokens are thus
 * distributed as the target's P.
 *
 * target_logits [N, n_rows, V] fp32 (device), n_rows = D or D+1.
 * draft_logits  [N, D, V] fp32 (device): the drafter's logits the drafts were sampled from (the
 *               logits_out of draft_block).
 * draft_tokens  [N, D] int32 (device), row stride `draft_stride` (>= D).
 * t_target, t_draft  temperatures (> 0, finite) of P and Q.
 * Outputs as verify_greedy: n_accepted[n], bonus[n] (the replacement or bonus token, -1 if
 * none), committed[n][0 .. D] (accepted drafts, then bonus, padded with -1), row_flags[n]
 * (optional) DBD_SEQ_NONFINITE if a non-finite logit was seen in the sequence's target or draft
 * rows (the results are then unspecified). */
int verify_sample(const float* target_logits, const float* draft_logits,
                  const int32_t* draft_tokens, int32_t draft_stride, int32_t batch,
                  int32_t n_draft, int32_t n_rows, int32_t vocab, float t_target, float t_draft,
                  uint64_t seed, int32_t* n_accepted, int32_t* bonus, int32_t* committed,
                  int32_t* row_flags, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace size (host) for select_streak. */
int dbd_select_workspace_bytes(int32_t batch, int32_t n_drafts, int32_t n_rows, int32_t vocab,
                               size_t* bytes /* host out */);

/* select_streak: self-selection among K joint drafts by expected streak, then greedy acceptance
 * on the chosen draft ([SpecDiff-2] section 5.2, with the streak equation of section 5.1).
 *
 * verifier_logits [N, K, n_rows, V] fp32: row (n, k, j) is the verifier's distribution for
 *                 position j of draft k given that draft's prefix; n_rows is G or G+1.
 * drafts          [N, K, G] int32.
 * p_{k,j} = q(x_j) / Z of row (n,k,j) with the library's integer weights (temperature 1);
 * S_k = sum_{m=1..G} prod_{j<=m} p_{k,j} accumulated in fp64 in position order;
 * selected[n] = argmax_k S_k (lowest k on ties); scores [N, K] fp64 (optional);
 * n_accepted / bonus / committed [N, G+1] / row_flags as in verify_greedy on rows (n, k*, .). */
int select_streak(const float* verifier_logits, const int32_t* drafts, int32_t batch,
                  int32_t n_drafts, int32_t gamma, int32_t n_rows, int32_t vocab,
                  int32_t* selected, double* scores, int32_t* n_accepted, int32_t* bonus,
                  int32_t* committed, int32_t* row_flags, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Workspace size (host) for refine_block. */
int dbd_refine_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab,
                               size_t* bytes /* host out */);

/* refine_block: one update of iterative block refinement between two draft_block passes.  The
 * DFlash article (section on writing a whole block in one forward pass) says the block is
 * refined when needed and gives no rule; the library reads it as Mask-Predict (Ghazvininejad,
 * Levy, Liu and Zettlemoyer, EMNLP 2019): T passes, the first drafts every position, before pass
 * t the floor(D (T - t) / T) least confident positions are masked again and re-drafted.
 *
 * logits       [N, D, V] fp32 (device): the D drafted rows of the forward that read block_tokens
 *              (draft_block's logits_out).
 * block_tokens [N, B] int32 (device, in/out): the block of that forward -> the block of the next.
 * conf         [N, D] uint64 (device, in/out): 0 marks a position masked in that forward; other
 *              values are confidences kept from earlier passes.  Start with all zeros.
 * For every position with conf 0: token = the row's argmax (lowest index on ties), conf = Z of
 * the row's integer weights at temperature 1 (its argmax probability is 2^40 / Z).  Then the
 * n_remask positions with the largest conf (lower index first on ties) get mask_id and conf 0;
 * n_remask = 0 after the last pass leaves the final tokens in block_tokens.
 * Anchors (n_anchor = 1: column 0) are never touched.  Results for rows with non-finite logits
 * are unspecified. */
int refine_block(const float* logits, int32_t batch, int32_t block_len, int32_t n_anchor,
                 int32_t vocab, int32_t mask_id, int32_t n_remask, int32_t* block_tokens,
                 uint64_t* conf, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Test hooks: exported for parity tests of single stages; not part of the drafting API ---- */

/* Workspace size (host) for dbd_sample_from_logits. */
int dbd_sample_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab, size_t* bytes);

/* The drafting stage of draft_block on given fp32 logits [N, D, V]: argmax (temperature <= 0,
 * n_drafts == 1) or n_drafts samples per position; out [N, n_drafts, D] int32. */
int dbd_sample_from_logits(const float* logits, int32_t batch, int32_t n_draft, int32_t vocab,
                           int32_t n_drafts, float temperature, uint64_t seed, int32_t* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace size (host) for dbd_sample_top_p. */
int dbd_sample_top_p_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab,
                                     size_t* bytes /* host out */);

/* Top-p (nucleus) drafting from fp32 logits [N, D, V] (device): the drafting stage of
 * draft_block with each position's draw restricted to its nucleus.  The pages name no nucleus
 * rule; in the library's integer arithmetic: with the weights q_v of the row at `temperature`
 * and Z = sum q_v, the nucleus is the shortest run of tokens, in order of decreasing weight with
 * ties by increasing index, whose mass reaches ceil(p * Z), p the float value of top_p (a dyadic
 * rational, so the ceiling is exact); the n_drafts draws are the sampler's (same counter draws)
 * on the weights restricted to it.  top_p >= 1 is plain sampling.  out [N, n_drafts, D] int32.
 * temperature must be finite and > 0, top_p finite and > 0. */
int dbd_sample_top_p(const float* logits, int32_t batch, int32_t n_draft, int32_t vocab,
                     int32_t n_drafts, float temperature, float top_p, uint64_t seed,
                     int32_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* The ingest mixing stage of draft_block ([DFlare] section on per-draft-layer mixing):
 * out[l, t, :] = RMSNorm(sum_i softmax(mix_logits[l])_i * hidden[t, i, :]) * mix_norm_w[l],
 * out [L_d, n_tokens, H] in desc.dtype. */
int dbd_mix_rmsnorm(const dbd_model_desc* desc, const float* mix_logits, const void* mix_norm_w,
                    const void* hidden, int64_t hid_token_stride, int64_t hid_layer_stride,
                    int32_t n_tokens, void* out, void* stream);

/* Byte offset (host out) inside the workspace of a draft_block call with these arguments of
 * the block's fp32 residual stream x [batch * block_len, H] (row n * block_len + b is block
 * position b of sequence n).  After the call it holds the residual after the last draft layer,
 * before the final RMSNorm.  Called with a desc whose n_layers is truncated to l + 1 (the
 * stacked per-layer weights, the mixing rows and the cache layers 0 .. l are prefixes of the
 * full drafter's) it exposes the residual after layer l, for per-layer parity tests. */
int dbd_draft_residual_offset(const dbd_model_desc* desc, int32_t batch, int32_t block_len,
                              int32_t n_anchor, int32_t n_new_total, int32_t n_drafts,
                              float temperature, int32_t ctx_capacity,
                              size_t* offset /* host out */);

/* Workspace size (host) for dbd_gemm_nt with the same dtype, shape, tile_cfg and split: the
 * split-K partials of the configuration (0 when it does not split K). */
int dbd_gemm_workspace_bytes(int32_t dtype, int32_t M, int32_t N, int32_t K, int32_t tile_cfg,
                             int32_t split, size_t* bytes);

/* The GEMM used for every projection: C[M, N] (fp32) = A[M, K] . B[N, K]^T with A, B in
 * `dtype`; row strides lda, ldb, ldc in elements.  bf16 needs K % 64 == 0 and 16-byte aligned
 * rows.  tile_cfg selects the bf16 block tile (BM x BN): 0-7 a ring of 64-wide k tiles
 * (0: 256x256/2 stages, 1: 256x128/3, 2: 128x128/3, 3: 64x128/4, 4: 128x128/2, 5: 64x128/3,
 * 6: 256x128/2, 7: 128x256/2); 8-13 a deep ring of 32-wide k stages (4 waves: 8: 256x128/3,
 * 9: 128x256/3, 10: 128x128/4; 8 waves, 64-wide k stages: 11: 256x256/2, 12: 256x192/2,
 * 13: 256x128/3) which splits K over several workgroups when `workspace` is given (NULL: no
 * split); 14-16 the 8-wave tiles 256x256, 256x192, 256x128 staged through registers instead of
 * global->LDS DMA; 17, 18 the skinny tiles 64x128, 32x128 for M <= 64 (every weight element
 * read once) (14-18: same split rule; Q/K/V and context K/V take
 * 256x128 for 14-16); -1: the library's choice.  split (deep-ring tiles with a
 * workspace only; in [0, 16]): 0 the library's choice, 1 no split, S > 1 K split over S
 * workgroups per output tile whose fp32 partials a second kernel adds, in split order, with
 * several workgroups per tile; a split is capped at K / 64.  The workspace
 * (dbd_gemm_workspace_bytes, 256-byte aligned) is used only by this call. */
int dbd_gemm_nt(int32_t dtype, const void* A, const void* B, float* C, int32_t M, int32_t N,
                int32_t K, int64_t lda, int64_t ldb, int64_t ldc, int32_t tile_cfg,
                int32_t split, void* workspace, size_t workspace_bytes, void* stream);

/* Per-stage timing for benchmarks.  While enabled, every kernel launch of the library is
 * bracketed by a pair of hipEvents recorded on the launch's stream and accounted to its stage
 * (DBD_STAGE_*).  Enabling creates the events (hipEventCreate); it is not meant for production
 * calls.  dbd_timing_read synchronises on the recorded events and returns, for one stage, the
 * summed kernel milliseconds and the number of launches since the last reset. */
enum {
  DBD_STAGE_PREP = 0,        /* row metadata and rotary tables */
  DBD_STAGE_MIX = 1,         /* ingest mix + RMSNorm */
  DBD_STAGE_GEMM_CTXKV = 2,  /* context K/V projection + cache append */
  DBD_STAGE_ROWNORM = 3,     /* embedding gather and RMSNorm */
  DBD_STAGE_GEMM_QKV = 4,
  DBD_STAGE_ATTN = 5,        /* attention + split combine */
  DBD_STAGE_GEMM_O = 6,
  DBD_STAGE_GEMM_GATEUP = 7,
  DBD_STAGE_GEMM_DOWN = 8,
  DBD_STAGE_GEMM_LMHEAD = 9,
  DBD_STAGE_DRAFT = 10,      /* argmax reduction or sampling of the drafts */
  DBD_STAGE_VERIFY = 11,     /* verify_greedy */
  DBD_STAGE_SELECT = 12,     /* select_streak */
  DBD_STAGE_COUNT = 13
};
int dbd_timing_enable(int on);
int dbd_timing_reset(void);
int dbd_timing_read(int stage, double* total_ms /* host out */, int64_t* launches /* host out */);

/* Tile tuning: replaces the library's choice of bf16 block tile and split-K (tile_cfg and split
 * as in dbd_gemm_nt; -1 and 0 restore the library's choice) for one GEMM stage of draft_block
 * (DBD_STAGE_GEMM_*), process-wide.  dbd_draft_workspace_bytes sizes the split partials from
 * the same choice, so set it before sizing a workspace; a workspace sized before the change may
 * run the stage unsplit.  Not thread-safe; meant for benchmarks.  Returns DBD_ERR_ARG for a
 * stage that is not a GEMM or an out-of-range tile_cfg / split. */
int dbd_gemm_override(int32_t stage, int32_t tile_cfg, int32_t split);

/* Attention tuning of the bf16 kernel, process-wide: the number of workgroups that share the
 * key chunks of every (sequence, kv head, 64-row query block) equally (1 .. 8192) and the chunks
 * each loads ahead (1 or 2); 0 and 0 restore the library's choice (512 and 1).
 * dbd_draft_workspace_bytes sizes the attention partials from the same choice, so set it before
 * sizing a workspace.  Not thread-safe; meant for benchmarks.  Returns DBD_ERR_ARG for values
 * out of range. */
int dbd_attn_override(int32_t workgroups, int32_t depth);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* dbd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DBD_H */
