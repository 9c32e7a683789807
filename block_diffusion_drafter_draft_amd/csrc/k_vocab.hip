// Vocabulary-wide kernels: row argmax, integer-exact sampling weights, drafting by sampling,
// greedy verification and streak-score self-selection.
//
// Greedy verification: DFlare page, section on drafting in parallel and accepting with the target
// (keep the prefix up to the first mismatch, append the target's token).  Sampling K joint
// drafts from the single-step marginals and choosing the one with the largest expected streak:
// SpecDiff-2 notes, sections 5.1 and 5.2.
//
// Integer results must not depend on the order of parallel reductions, so probabilities are
// built from integers: per row, M = max logit; e_v = exp_i((l_v - M) * invT) in fp32 with every
// multiply and add rounded separately; q_v = floor(e_v * 2^40); Z = sum q_v (exact in uint64).
// exp_i is Cody-Waite range reduction by ln 2 (Cody & Waite, 1980) followed by the degree-7
// Taylor polynomial of e^r, scaled by 2^k.  Draws come from the SplitMix64 output function
// (Steele, Lea & Flood, OOPSLA 2014) keyed by (seed, sequence, draft, position).
// This translation unit is compiled with -ffp-contract=off and uses explicit _rn operations.
#include "dbd_internal.h"

namespace dbd {

// ------------------------------------------------------------------ integer-exact exp
// log2(e), fp32 nearest
#define EXPI_LOG2E 0x1.715476p+0f
// ln 2 rounded to fp32 with its 8 low mantissa bits cleared (16 significant bits, so that
// k * HI is exact for |k| <= 128), and the fp32 nearest to the remainder ln 2 - HI
#define EXPI_LN2_HI 0x1.62e4p-1f
#define EXPI_LN2_LO 0x1.7f7d1cp-20f

__device__ __forceinline__ float exp_i(float x) {
  // 1/i! for i = 7 .. 2 (fp32 nearest), then 1, 1
  const float c7 = 1.0f / 5040.0f, c6 = 1.0f / 720.0f, c5 = 1.0f / 120.0f, c4 = 1.0f / 24.0f,
              c3 = 1.0f / 6.0f, c2 = 0.5f;
  const float t = __fmul_rn(x, EXPI_LOG2E);
  if (t < -64.0f) return 0.0f;
  const float k = rintf(t);
  float r = __fsub_rn(x, __fmul_rn(k, EXPI_LN2_HI));
  r = __fsub_rn(r, __fmul_rn(k, EXPI_LN2_LO));
  float p = c7;
  p = __fadd_rn(__fmul_rn(p, r), c6);
  p = __fadd_rn(__fmul_rn(p, r), c5);
  p = __fadd_rn(__fmul_rn(p, r), c4);
  p = __fadd_rn(__fmul_rn(p, r), c3);
  p = __fadd_rn(__fmul_rn(p, r), c2);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  return ldexpf(p, (int)k);
}

__device__ __forceinline__ uint64_t weight_q(float l, float M, float inv_t) {
  const float e = exp_i(__fmul_rn(__fsub_rn(l, M), inv_t));
  return (uint64_t)floorf(ldexpf(e, 40));
}

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ------------------------------------------------------------------ block reductions
template <int NT>
__device__ __forceinline__ void block_argmax(float& v, int& i, float* sv, int* si) {
  wave_argmax(v, i);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < NT / 64; ++k) argmax_combine(sv[0], si[0], sv[k], si[k]);
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
}

// ------------------------------------------------------------------ argmax partials
// grid (chunks, rows): (max, lowest argmax) of logits[row, chunk]; flag = non-finite seen.
__global__ __launch_bounds__(256) void argmax_partial_kernel(const float* __restrict__ x, int V,
                                                             int chunk, int nch,
                                                             float* __restrict__ pv,
                                                             int32_t* __restrict__ pi,
                                                             int32_t* __restrict__ pflag) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int sflag;
  const int c = blockIdx.x, row = blockIdx.y;
  const int64_t rbase = (int64_t)row * V;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  if (threadIdx.x == 0) sflag = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  int bad = 0;
  const float* xr = x + rbase;
  if (((rbase & 3) == 0) && ((v0 & 3) == 0)) {
    const int nv = (v1 - v0) >> 2;
    for (int k = threadIdx.x; k < nv; k += 256) {
      const float4 q = *reinterpret_cast<const float4*>(xr + v0 + 4 * k);
      const int b = v0 + 4 * k;
      bad |= !isfinite(q.x) | !isfinite(q.y) | !isfinite(q.z) | !isfinite(q.w);
      argmax_combine(bv, bi, q.x, b);
      argmax_combine(bv, bi, q.y, b + 1);
      argmax_combine(bv, bi, q.z, b + 2);
      argmax_combine(bv, bi, q.w, b + 3);
    }
    for (int v = v0 + 4 * nv + threadIdx.x; v < v1; v += 256) {
      const float q = xr[v];
      bad |= !isfinite(q);
      argmax_combine(bv, bi, q, v);
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) {
      const float q = xr[v];
      bad |= !isfinite(q);
      argmax_combine(bv, bi, q, v);
    }
  }
  __syncthreads();
  if (bad) atomicOr(&sflag, 1);
  block_argmax<256>(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    pv[(int64_t)row * nch + c] = bv;
    pi[(int64_t)row * nch + c] = bi == 0x7fffffff ? v0 : bi;     // all-NaN chunk: first index
    pflag[(int64_t)row * nch + c] = sflag;
  }
}

hipError_t launch_argmax_partial(const float* x, int rows, int vocab, int chunk, float* pv,
                                 int32_t* pi, int32_t* pflag, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nch = ceil_div(vocab, chunk);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nch, rows), dim3(256), 0, s, x, vocab, chunk,
                     nch, pv, pi, pflag);
  return hipGetLastError();
}

// One wave per row: reduce the chunk partials.
__device__ __forceinline__ void reduce_partials(const float* pv, const int32_t* pi, int64_t row,
                                                int nch, float& bv, int& bi) {
  bv = -INFINITY;
  bi = 0x7fffffff;
  for (int c = threadIdx.x & 63; c < nch; c += 64)
    argmax_combine(bv, bi, pv[row * nch + c], pi[row * nch + c]);
  wave_argmax(bv, bi);
}

__global__ __launch_bounds__(64) void argmax_final_kernel(const float* pv, const int32_t* pi,
                                                          int nch, int32_t* out_idx,
                                                          float* out_max) {
  const int row = blockIdx.x;
  float bv;
  int bi;
  reduce_partials(pv, pi, row, nch, bv, bi);
  if (threadIdx.x == 0) {
    out_idx[row] = bi;
    if (out_max) out_max[row] = bv;
  }
}

hipError_t launch_argmax_final(const float* pv, const int32_t* pi, int rows, int nch,
                               int32_t* out_idx, float* out_max, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(64), 0, s, pv, pi, nch, out_idx,
                     out_max);
  return hipGetLastError();
}

// LM-head argmax: reduce the per-column-tile partials of the GEMM epilogue; rows of invalid
// sequences give -1.
__global__ __launch_bounds__(64) void lm_argmax_final_kernel(const float* pv, const int32_t* pi,
                                                             int ntiles, const int32_t* blk_pos,
                                                             int block_len, int n_anchor,
                                                             int n_draft, int32_t* out) {
  const int row = blockIdx.x;
  float bv;
  int bi;
  reduce_partials(pv, pi, row, ntiles, bv, bi);
  if (threadIdx.x == 0) {
    const int n = row / n_draft, j = row % n_draft;
    const bool ok = blk_pos[n * block_len + n_anchor + j] >= 0;
    out[row] = ok ? bi : -1;
  }
}

hipError_t launch_lm_argmax_final(const float* part_val, const int32_t* part_idx, int rows,
                                  int ntiles, const int32_t* blk_pos, int block_len,
                                  int n_anchor, int n_draft, int32_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lm_argmax_final_kernel, dim3(rows), dim3(64), 0, s, part_val, part_idx,
                     ntiles, blk_pos, block_len, n_anchor, n_draft, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ integer weight sums
// grid (chunks, rows).  Every workgroup reduces the row's argmax partials to M itself (same
// inputs, same result), then sums q_v over its chunk.  Chunk 0 also stores M and the argmax.
__global__ __launch_bounds__(256) void zsum_partial_kernel(
    const float* __restrict__ x, int V, int chunk, int nch, const float* __restrict__ pv,
    const int32_t* __restrict__ pi, float inv_t, uint64_t* __restrict__ zpart,
    float* __restrict__ row_max, int32_t* __restrict__ row_arg) {
  __shared__ float sM;
  __shared__ uint64_t red[4];
  const int c = blockIdx.x, row = blockIdx.y;
  if (threadIdx.x < 64) {
    float bv;
    int bi;
    reduce_partials(pv, pi, row, nch, bv, bi);
    if (threadIdx.x == 0) {
      sM = bv;
      if (c == 0) {
        row_max[row] = bv;
        row_arg[row] = bi;
      }
    }
  }
  __syncthreads();
  const float M = sM;
  const float* xr = x + (int64_t)row * V;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  uint64_t acc = 0;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) acc += weight_q(xr[v], M, inv_t);
  acc = wave_sum_u64(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) zpart[(int64_t)row * nch + c] = red[0] + red[1] + red[2] + red[3];
}

hipError_t launch_zsum_partial(const float* x, int rows, int vocab, int chunk, const float* pv,
                               const int32_t* pi, float inv_t, uint64_t* zpart, float* row_max,
                               int32_t* row_arg, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nch = ceil_div(vocab, chunk);
  hipLaunchKernelGGL(zsum_partial_kernel, dim3(nch, rows), dim3(256), 0, s, x, vocab, chunk, nch,
                     pv, pi, inv_t, zpart, row_max, row_arg);
  return hipGetLastError();
}

// ------------------------------------------------------------------ sampling
// grid (K, rows).  thr = (u * Z) >> 32; the chunk holding the threshold is found from the chunk
// sums, then one block-wide exclusive scan over that chunk finds the first token whose
// inclusive prefix exceeds thr.
__global__ __launch_bounds__(256) void sample_pick_kernel(
    const float* __restrict__ x, int V, int chunk, int nch, const uint64_t* __restrict__ zpart,
    const float* __restrict__ row_max, float inv_t, int n_draft, int n_drafts, uint64_t seed,
    const int32_t* __restrict__ blk_pos, int block_len, int n_anchor, int32_t* __restrict__ out) {
  __shared__ uint64_t s_thr;
  __shared__ int s_chunk;
  __shared__ uint64_t wsum[4];
  const int k = blockIdx.x, row = blockIdx.y;
  const int n = row / n_draft, j = row % n_draft;
  const int64_t oidx = ((int64_t)n * n_drafts + k) * n_draft + j;
  if (blk_pos && blk_pos[n * block_len + n_anchor + j] < 0) {
    if (threadIdx.x == 0) out[oidx] = -1;
    return;
  }
  if (threadIdx.x == 0) {
    uint64_t Z = 0;
    for (int c = 0; c < nch; ++c) Z += zpart[(int64_t)row * nch + c];
    const uint64_t idx = ((uint64_t)n * n_drafts + k) * n_draft + j;
    const uint64_t u = splitmix_mix(splitmix_mix(seed) + (idx + 1) * 0x9E3779B97F4A7C15ull) >> 32;
    // (u * Z) >> 32 with the full 128-bit product
    const uint64_t lo = u * Z, hi = __umul64hi(u, Z);
    uint64_t thr = (hi << 32) | (lo >> 32);
    int cc = 0;
    uint64_t cum = 0;
    for (; cc < nch; ++cc) {
      const uint64_t zc = zpart[(int64_t)row * nch + cc];
      if (cum + zc > thr) break;
      cum += zc;
    }
    s_chunk = cc < nch ? cc : nch - 1;
    s_thr = thr - cum;                       // threshold relative to the chunk start
  }
  __syncthreads();
  const int c = s_chunk;
  const uint64_t thr = s_thr;
  const float M = row_max[row];
  const float* xr = x + (int64_t)row * V;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  const int per = (chunk + 255) / 256;         // contiguous segment per thread
  const int a0 = v0 + threadIdx.x * per, a1 = min(v1, a0 + per);
  uint64_t mine = 0;
  for (int v = a0; v < a1; ++v) mine += weight_q(xr[v], M, inv_t);
  // exclusive scan of the 256 segment sums: wave scan then wave offsets
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)incl, o, 64);
    const uint32_t hi = __shfl_up((uint32_t)(incl >> 32), o, 64);
    if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint64_t excl = incl - mine;
  for (int q = 0; q < w; ++q) excl += wsum[q];
  if (excl <= thr && thr < excl + mine) {
    uint64_t run = excl;
    for (int v = a0; v < a1; ++v) {
      run += weight_q(xr[v], M, inv_t);
      if (run > thr) {
        out[oidx] = v;
        break;
      }
    }
  }
}

hipError_t launch_sample_pick(const float* x, int rows, int vocab, int chunk,
                              const uint64_t* zpart, const float* row_max, float inv_t,
                              int n_draft, int n_drafts, uint64_t seed,
                              const int32_t* row_valid_pos, int block_len, int n_anchor,
                              int32_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nch = ceil_div(vocab, chunk);
  hipLaunchKernelGGL(sample_pick_kernel, dim3(n_drafts, rows), dim3(256), 0, s, x, vocab, chunk,
                     nch, zpart, row_max, inv_t, n_draft, n_drafts, seed, row_valid_pos,
                     block_len, n_anchor, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ greedy acceptance
// One wave per sequence.  t_j = argmax of row j; mismatch mask by ballot; first set bit is the
// accepted length.
__device__ void greedy_accept(const int32_t* t_s, const int32_t* draft, int D, int R,
                              int32_t* n_acc, int32_t* bonus, int32_t* committed) {
  const int lane = threadIdx.x & 63;
  int first = D;
  for (int j0 = 0; j0 < D; j0 += 64) {
    const int j = j0 + lane;
    const bool mism = j < D && draft[j] != t_s[j];
    const uint64_t mask = __ballot(mism);
    if (mask) {
      first = j0 + __ffsll((unsigned long long)mask) - 1;
      break;
    }
  }
  const int b = first < R ? t_s[first] : -1;
  if (lane == 0) {
    *n_acc = first;
    *bonus = b;
  }
  for (int j = lane; j <= D; j += 64)
    committed[j] = j < first ? draft[j] : (j == first ? b : -1);
}

// One workgroup per sequence; wave w reduces rows w, w + VF_WAVES, ... (the rows' partial
// reductions are independent, so they overlap instead of queueing behind each other's loads),
// then wave 0 runs the acceptance.
constexpr int VF_WAVES = 16;
__global__ __launch_bounds__(64 * VF_WAVES) void verify_finalize_kernel(
    const float* pv, const int32_t* pi, const int32_t* pflag, int nch, const int32_t* drafts,
    int draft_stride, int n_draft, int n_rows, int32_t* n_acc, int32_t* bonus,
    int32_t* committed, int32_t* row_flags) {
  __shared__ int32_t t_s[128];
  __shared__ int s_bad;
  const int n = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  for (int j = wave; j < n_rows; j += VF_WAVES) {
    float bv;
    int bi;
    const int64_t row = (int64_t)n * n_rows + j;
    reduce_partials(pv, pi, row, nch, bv, bi);
    for (int c = lane; c < nch; c += 64) bad |= pflag[row * nch + c];
    if (lane == 0) t_s[j] = bi;
  }
  if (__ballot(bad != 0) && lane == 0) atomicOr(&s_bad, 1);
  __syncthreads();
  if (wave != 0) return;
  greedy_accept(t_s, drafts + (int64_t)n * draft_stride, n_draft, n_rows, n_acc + n, bonus + n,
                committed + (int64_t)n * (n_draft + 1));
  if (row_flags && lane == 0) row_flags[n] = s_bad ? 1 : 0;
}

hipError_t launch_verify_finalize(const float* pv, const int32_t* pi, const int32_t* pflag,
                                  int nch, const int32_t* drafts, int draft_stride, int batch,
                                  int n_draft, int n_rows, int32_t* n_acc, int32_t* bonus,
                                  int32_t* committed, int32_t* row_flags, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_finalize_kernel, dim3(batch), dim3(64 * VF_WAVES), 0, s, pv, pi,
                     pflag, nch, drafts, draft_stride, n_draft, n_rows, n_acc, bonus, committed,
                     row_flags);
  return hipGetLastError();
}

// ------------------------------------------------------------------ streak selection
// One wave per sequence; lane k scores draft k: p_j = double(q_x) / double(Z) for the draft's
// token x in row (n, k, j); S = sum_m prod_{j<=m} p_j in fp64, in position order.
__global__ __launch_bounds__(64) void select_finalize_kernel(
    const float* __restrict__ x, int V, int nch, const uint64_t* __restrict__ zpart,
    const float* __restrict__ row_max, const int32_t* __restrict__ row_arg,
    const int32_t* __restrict__ pflag, const int32_t* __restrict__ drafts, int K, int G, int R,
    int32_t* selected, double* scores, int32_t* n_acc, int32_t* bonus, int32_t* committed,
    int32_t* row_flags) {
  __shared__ double s_score[64];
  __shared__ int32_t t_s[128];
  __shared__ int s_best;
  const int n = blockIdx.x;
  const int lane = threadIdx.x;
  for (int k = lane; k < K; k += 64) {
    double P = 1.0, S = 0.0;
    for (int j = 0; j < G; ++j) {
      const int64_t row = ((int64_t)n * K + k) * R + j;
      uint64_t Z = 0;
      for (int c = 0; c < nch; ++c) Z += zpart[row * nch + c];
      const int tok = drafts[((int64_t)n * K + k) * G + j];
      const uint64_t q = (tok >= 0 && tok < V) ? weight_q(x[row * V + tok], row_max[row], 1.0f)
                                               : 0;
      const double p = __ddiv_rn((double)q, (double)Z);
      P = __dmul_rn(P, p);
      S = __dadd_rn(S, P);
    }
    s_score[k] = S;
    if (scores) scores[(int64_t)n * K + k] = S;
  }
  __syncthreads();
  if (lane == 0) {
    int best = 0;
    for (int k = 1; k < K; ++k)
      if (s_score[k] > s_score[best]) best = k;
    s_best = best;
    selected[n] = best;
  }
  __syncthreads();
  const int best = s_best;
  for (int j = lane; j < R; j += 64) t_s[j] = row_arg[((int64_t)n * K + best) * R + j];
  int bad = 0;
  for (int r = 0; r < K * R; ++r)
    for (int c = lane; c < nch; c += 64) bad |= pflag[((int64_t)n * K * R + r) * nch + c];
  __syncthreads();
  greedy_accept(t_s, drafts + ((int64_t)n * K + best) * G, G, R, n_acc + n, bonus + n,
                committed + (int64_t)n * (G + 1));
  if (row_flags) {
    const uint64_t m = __ballot(bad != 0);
    if (lane == 0) row_flags[n] = m ? 1 : 0;
  }
}

hipError_t launch_select_finalize(const float* x, int vocab, int chunk, const uint64_t* zpart,
                                  const float* row_max, const int32_t* row_arg,
                                  const int32_t* pflag, const int32_t* drafts, int batch,
                                  int n_drafts, int gamma, int n_rows, int32_t* selected,
                                  double* scores, int32_t* n_acc, int32_t* bonus,
                                  int32_t* committed, int32_t* row_flags, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int nch = ceil_div(vocab, chunk);
  hipLaunchKernelGGL(select_finalize_kernel, dim3(batch), dim3(64), 0, s, x, vocab, nch, zpart,
                     row_max, row_arg, pflag, drafts, n_drafts, gamma, n_rows, selected, scores,
                     n_acc, bonus, committed, row_flags);
  return hipGetLastError();
}

}  // namespace dbd
