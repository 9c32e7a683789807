// Internal declarations shared by the translation units of libdbd.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_rules.h"

namespace dbd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte copies
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- element conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------- wave64 reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// (value, index) maximum; ties and NaN-free equal values go to the lower index; NaN never wins.
__device__ __forceinline__ void argmax_combine(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    argmax_combine(v, i, ov, oi);
  }
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// ---------------------------------------------------------------- argument structs
// Per-row metadata produced at the start of draft_block (all device pointers into workspace).
struct RowMeta {
  int32_t* blk_pos;     // [N*B]   position of block row, -1 if its sequence is invalid
  int32_t* ctx_seq;     // [T_new] sequence of ingest row, -1 if invalid
  int32_t* ctx_pos;     // [T_new] position of ingest row, -1 if invalid
  int32_t* seq_keys;    // [N]     keys the block attends to (P + B), 0 if invalid
  float2* rope_blk;     // [N*B][hd/2] (cos, sin)
  float2* rope_ctx;     // [T_new][hd/2]
};

// GEMM: C = A[M,K] . Bv[N,K]^T where the virtual B rows come from up to three weight tensors
// (concatenated along N) or, in gate/up mode, from two tensors interleaved per column tile.
struct BSeg {
  const void* ptr;
  int n0, n1;           // virtual columns [n0, n1) read rows 0 .. n1-n0-1 of ptr
};
struct GemmArgs {
  const void* A;
  const void* A2;       // optional low part of A (bf16 pair split; same strides as A)
  int64_t lda, a_bs;    // row stride, batch (grid.z) stride, in elements
  BSeg seg[3];
  int nseg;
  int64_t ldb, b_bs;
  int gateup;           // 1: tile t holds gate rows [t*BN/2, +BN/2) then up rows; seg0 = gate,
                        //    seg1 = up, both with n1 - n0 = F
  int M, N, K;          // N = virtual columns
  // split-K (deep-ring tiles only): `split` workgroups share one output tile, each over its
  // share of K, and write fp32 partials to part[(tile*split + s) * BM*BN] (fragment order); a
  // second kernel adds them in split order and runs the epilogue.  part_cap: bytes available; a
  // split that does not fit runs unsplit.
  int split;
  float* part;
  size_t part_cap;
};

// Epilogue selectors and their parameters.
enum EpiKind { EPI_STORE_F32 = 0, EPI_RESID = 1, EPI_QKV = 2, EPI_CTXKV = 3, EPI_SWIGLU = 4,
               EPI_ARGMAX = 5 };
struct EpiArgs {
  int kind;
  // store / residual / argmax-logits
  void* C;              // EPI_STORE_F32: float*; EPI_RESID: float* residual (x += acc)
  int64_t ldc, c_bs;
  // attention projections
  void* q_out;          // [M, qd] element T
  void* q_out_lo;       // optional [M, qd] low part of the bf16 pair of the rotated queries
  void* kv_k;           // cache (element T)
  void* kv_v;
  int64_t layer_off_k;  // element offset of this layer's block in the cache (QKV epilogue)
  int64_t layer_stride; // elements per layer in the cache (CTXKV epilogue: layer = grid.z)
  int qd, kd, hd, kvh, block_len, batch, cap;
  const int32_t* row_seq;   // CTXKV: ctx_seq
  const int32_t* row_pos;   // QKV: blk_pos; CTXKV: ctx_pos
  const float2* rope;       // rope table for the rows
  // SwiGLU
  void* act;            // [M, F] element T
  void* act_lo;         // optional low part of the bf16 pair of act
  int F;
  // LM-head argmax
  float* part_val;      // [M, ntiles]
  int32_t* part_idx;
  int ntiles;
  float* logits;        // optional [M, N] fp32
  // EPI_RESID: the RMSNorm of the updated residual rows, norm_out = T(x / rms(x) * norm_g) (and
  // the low part of the bf16 pair); done in the split-K reduction of the tiles that can
  // (gemm_fuses_norm), else left to the caller (launch_gemm reports which).  norm_g null: no
  // norm.  norm_n_anchor > 0: only the mask rows of each block of norm_block_len rows are
  // normalised, written compactly (row n * B + b to n * (B - n_anchor) + b - n_anchor).
  const void* norm_g;
  void* norm_out;
  void* norm_out_lo;
  float norm_eps;
  int norm_block_len;
  int norm_n_anchor;
};

// Attention over the cache: every block row of sequence n, head h, attends to cache positions
// 0 .. seq_keys[n]-1 of kv head h / grp.
// One launched bf16 attention workgroup's share: its range j and chunks [lo, hi) (lo == hi: no
// work), and at lo the sequence, segment of the sequence (kv head * row blocks + row block),
// chunk inside the segment and the sequence's keys.
struct AttnPlan {
  int32_t n, seg, chunk, keys, j, pad;
  int64_t lo, hi;
};

struct AttnArgs {
  const void* q;        // [N*B, qd]
  const void* q_lo;     // optional [N*B, qd]: low part of the bf16 pair of q (bf16 kernel)
  const void* kv_k;     // layer base: [N, kvh, cap, hd]
  const void* kv_v;     // layer base: [N, kvh, hd, cap]
  const int32_t* seq_keys;
  void* out;            // [N*B, qd]
  void* out_lo;         // optional low part of the bf16 pair of out
  // partials: fp32 kernel [N, kvh, S_max, R, hd] and [N, kvh, S_max, R]; bf16 kernel
  // [slots, 64, hd] and [slots, 64] with slots = workgroups + N * kvh * row blocks
  float* part_o;
  float2* part_ml;      // (running max in log2 units, sum)
  int batch, kvh, grp, block_len, cap, qd, s_max, split;   // s_max, split: fp32 kernel
  float scale_log2;     // log2(e) / sqrt(hd)
  // bf16 kernel: the chunk schedule written by launch_attn_plan once per step
  const AttnPlan* plan;         // [workgroups], indexed by blockIdx.x
  const int32_t* plan_pref;     // [N + 1] chunks of the sequences before n
  const int64_t* plan_total;    // [2]: chunks over every segment, workgroups with chunks
  int workgroups;               // workgroups of the bf16 kernel
  int depth;                    // chunks loaded ahead (1 or 2)
};

// ---------------------------------------------------------------- launchers (one per TU)
hipError_t launch_prep(const int32_t* ctx_len, const int32_t* new_offsets, int batch,
                       int block_len, int n_new_total, int cap, int hd, const double* inv_freq,
                       RowMeta meta, int32_t* seq_status, hipStream_t s);
// raw: the mixing coefficients are used as given (no softmax over the target layers)
hipError_t launch_mix_rmsnorm(int dtype, const void* hid, int64_t ts, int64_t ls, int n_tok,
                              int H, int Lt, int Ld, const float* mix_logits, int raw,
                              const void* g, void* out, void* out_lo, float eps, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
hipError_t launch_embed(int dtype, const int32_t* tokens, const void* E, int rows, int H,
                        int V, float* x, const void* g, void* out, void* out_lo, float eps,
                        hipStream_t s, bool* normed);
hipError_t launch_rmsnorm(int dtype, const float* x, const void* g, void* out, void* out_lo,
                          int rows, int H, float eps, int block_len, int n_anchor, hipStream_t s);
// cfg: bf16 block-tile configuration index (see dbd_gemm_nt in dbd.h), -1 = pick for the shape
// *norm_done (optional) tells whether an EPI_RESID launch with e.norm_g also wrote the norm.
hipError_t launch_gemm(int dtype, const GemmArgs& a, const EpiArgs& e, int batch,
                       hipStream_t s, int cfg = -1, int split = 0, bool* norm_done = nullptr);
// What launch_gemm does for a problem: the tile configuration (-1 on the fp32 path), its column
// tile width, the split-K factor (1 unless split_ok: a partial buffer and counters are given),
// the output tiles over the batch and the partial-buffer bytes.  pair = the A operand comes as a
// bf16 pair.  The workspace sizing and the launch both use it, so they agree.
// split_req: 0 = the library's choice, 1 = no split, S > 1 = S-way split.
struct GemmPlan {
  int cfg, bn, split, tiles;
  size_t part_bytes;
};
// norm: a residual projection whose caller asks for the RMSNorm of the updated rows (EpiArgs
// norm_g set, rows that resid_norm_fits); the tile choice then counts the norm's own launch
// against the tiles whose split-K reduction can write it (gemm_fuses_norm).
GemmPlan plan_gemm(int dtype, int kind, int cfg, int M, int N, int K, int batch, int gateup,
                   int F, bool pair, bool split_ok, int split_req = 0, bool norm = false);
// Whether a residual projection planned as p, with (pair) or without a bf16-pair A operand,
// runs the following RMSNorm in its split-K reduction (resid_norm_kernel): the skinny tiles, the
// register-staged 256-row tiles without pair rows and the deep-ring four-wave tiles, split, one
// batch entry.
bool gemm_fuses_norm(const GemmPlan& p, bool pair, int batch);
constexpr int kMaxGemmCfg = 18;
constexpr int kMaxGemmSplit = 16;
hipError_t launch_attention(int dtype, int hd, const AttnArgs& a, hipStream_t s);
// Chunk schedule of the bf16 attention for one step (the keys per sequence are the same in
// every layer): plan [workgroups], pref [batch + 1], total [2].
hipError_t launch_attn_plan(const int32_t* seq_keys, int batch, int hd, int kvh, int rows,
                            int workgroups, AttnPlan* plan, int32_t* pref, int64_t* total,
                            hipStream_t s);
hipError_t launch_lm_argmax_final(const float* part_val, const int32_t* part_idx, int rows,
                                  int ntiles, const int32_t* blk_pos, int block_len,
                                  int n_anchor, int n_draft, int32_t* out, hipStream_t s);
hipError_t launch_argmax_partial(const float* x, int rows, int vocab, int chunk, float* pv,
                                 int32_t* pi, int32_t* pflag, hipStream_t s);
hipError_t launch_argmax_final(const float* pv, const int32_t* pi, int rows, int nch,
                               int32_t* out_idx, float* out_max, hipStream_t s);
hipError_t launch_zsum_partial(const float* x, int rows, int vocab, int chunk, const float* pv,
                               const int32_t* pi, float inv_t, uint64_t* zpart, float* row_max,
                               int32_t* row_arg, hipStream_t s);
// topp: optional per-row nucleus state of launch_top_p ({q*, -, v_cut, -}); zpart then holds
// the nucleus chunk sums (rz of launch_top_p)
hipError_t launch_sample_pick(const float* x, int rows, int vocab, int chunk,
                              const uint64_t* zpart, const float* row_max, float inv_t,
                              int n_draft, int n_drafts, uint64_t seed,
                              const int32_t* row_valid_pos, int block_len, int n_anchor,
                              const int64_t* topp, int32_t* out, hipStream_t s);
// Top-p nucleus of each row after launch_argmax_partial (pv, pi): p = mp / 2^sp exactly.  Writes
// row_max [rows]; st [rows * 4] int64; hist [rows * top_p_spans * top_p_bins] uint64;
// above, rz [rows * chunks] uint64 (rz: the nucleus chunk sums); cnt [rows * chunks] int32;
// keys [rows * chunks * top_p_cap] uint64.  chunks <= 64.
int top_p_spans(int vocab, int chunk);
int top_p_bins();
int top_p_cap();
hipError_t launch_top_p(const float* x, int rows, int vocab, int chunk, const float* pv,
                        const int32_t* pi, float inv_t, uint64_t mp, int sp, float* row_max,
                        int64_t* st, uint64_t* hist, uint64_t* above, int32_t* cnt,
                        uint64_t* keys, uint64_t* rz, hipStream_t s);
// One Mask-Predict update per sequence from row_arg / zpart of launch_zsum_partial at
// temperature 1 over the N * D rows: tokens [N, B] and conf [N, D] in/out.
hipError_t launch_refine(const int32_t* row_arg, const uint64_t* zpart, int batch, int vocab,
                         int chunk, int D, int B, int n_anchor, int mask_id, int n_remask,
                         int32_t* tokens, uint64_t* conf, hipStream_t s);
hipError_t launch_verify_finalize(const float* pv, const int32_t* pi, const int32_t* pflag,
                                  int nch, const int32_t* drafts, int draft_stride, int batch,
                                  int n_draft, int n_rows, int32_t* n_acc, int32_t* bonus,
                                  int32_t* committed, int32_t* row_flags, hipStream_t s);
// Lossless stochastic verification after the argmax partials (pf_*) and integer weight sums
// (zp_*, rm_*) of the target rows [batch * R] and draft rows [batch * D]; spec: [batch * 4]
// int64 scratch, wpart: [batch * chunks] 16-byte (128-bit) scratch.
hipError_t launch_verify_sample(const float* tl, const float* dl, const int32_t* drafts,
                                int stride, int batch, int D, int R, int V, int chunk,
                                const uint64_t* zp_t, const float* rm_t, const uint64_t* zp_d,
                                const float* rm_d, const int32_t* pf_t, const int32_t* pf_d,
                                float inv_p, float inv_q, uint64_t seed, int64_t* spec,
                                void* wpart, int32_t* n_acc, int32_t* bonus,
                                int32_t* committed, int32_t* row_flags, hipStream_t s);
hipError_t launch_select_finalize(const float* x, int vocab, int chunk, const uint64_t* zpart,
                                  const float* row_max, const int32_t* row_arg,
                                  const int32_t* pflag, const int32_t* drafts, int batch,
                                  int n_drafts, int gamma, int n_rows, int32_t* selected,
                                  double* scores, int32_t* n_acc, int32_t* bonus,
                                  int32_t* committed, int32_t* row_flags, hipStream_t s);

inline int vocab_chunk() { return 4096; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dbd
