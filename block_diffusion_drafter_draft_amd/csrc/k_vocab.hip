// Vocabulary-wide kernels: row argmax, integer-exact sampling weights, drafting by sampling,
// greedy verification and streak-score self-selection.
//
// Block refinement: the DFlash article's section on writing a whole block in one forward pass (the
// block is refined when needed), read as Mask-Predict (Ghazvininejad et al., EMNLP 2019).
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
  // Branch-free: inputs with t < -64 are computed too and replaced by 0 at the end.  The clamp
  // leaves every t >= -64 unchanged and keeps k's conversion to int in range for the others.
  const float k = rintf(fmaxf(t, -65.0f));
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
  const float v = ldexpf(p, (int)k);
  return t < -64.0f ? 0.0f : v;
}

// q = floor(e * 2^40) for e in [0, 1]: f = e * 2^40 < 2^41 is exact, hi = floor(f / 2^32) and
// lo = f - hi * 2^32 in [0, 2^32) are exact, and converting lo truncates, which is its floor.
__device__ __forceinline__ uint64_t weight_q(float l, float M, float inv_t) {
  const float e = exp_i(__fmul_rn(__fsub_rn(l, M), inv_t));
  const float f = ldexpf(e, 40);
  const float hi = floorf(__fmul_rn(f, 0x1p-32f));
  const float lo = fmaf(hi, -0x1p32f, f);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Logits per thread in the pick kernels' chunk scans (256 threads per chunk): chunks are at most
// 256 * PICK_SEG wide.
constexpr int PICK_SEG = 16;

typedef unsigned __int128 u128;

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
  if (((uintptr_t)(xr + v0) & 15) == 0) {
    const int nv = (v1 - v0) >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(xr + v0);
    auto take = [&](const float4& q, int b) __attribute__((always_inline)) {
      bad |= !isfinite(q.x) | !isfinite(q.y) | !isfinite(q.z) | !isfinite(q.w);
      argmax_combine(bv, bi, q.x, b);
      argmax_combine(bv, bi, q.y, b + 1);
      argmax_combine(bv, bi, q.z, b + 2);
      argmax_combine(bv, bi, q.w, b + 3);
    };
    // four float4 loads in flight per thread before any is combined (a 4096-wide chunk is
    // exactly one such round); the combine is order-independent (max, lowest index on ties)
    int k = threadIdx.x;
    for (; k + 3 * 256 < nv; k += 4 * 256) {
      float4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = x4[k + u * 256];
#pragma unroll
      for (int u = 0; u < 4; ++u) take(q[u], v0 + 4 * (k + u * 256));
    }
    for (; k < nv; k += 256) take(x4[k], v0 + 4 * k);
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
  const int lane = threadIdx.x & 63;
  // eight partials per lane loaded before any is combined (the combine is order-independent)
  int c = lane;
  for (; c + 7 * 64 < nch; c += 8 * 64) {
    float v[8];
    int ix[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = pv[row * nch + c + 64 * u];
      ix[u] = pi[row * nch + c + 64 * u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) argmax_combine(bv, bi, v[u], ix[u]);
  }
  for (; c < nch; c += 64) argmax_combine(bv, bi, pv[row * nch + c], pi[row * nch + c]);
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
  if (((uintptr_t)(xr + v0) & 15) == 0) {
    // four float4 loads in flight per thread before their weights are computed
    const int nv = (v1 - v0) >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(xr + v0);
    int k = threadIdx.x;
    for (; k + 3 * 256 < nv; k += 4 * 256) {
      float4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = x4[k + u * 256];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc += weight_q(q[u].x, M, inv_t) + weight_q(q[u].y, M, inv_t) +
               weight_q(q[u].z, M, inv_t) + weight_q(q[u].w, M, inv_t);
    }
    for (; k < nv; k += 256) {
      const float4 q = x4[k];
      acc += weight_q(q.x, M, inv_t) + weight_q(q.y, M, inv_t) + weight_q(q.z, M, inv_t) +
             weight_q(q.w, M, inv_t);
    }
    for (int v = v0 + 4 * nv + threadIdx.x; v < v1; v += 256) acc += weight_q(xr[v], M, inv_t);
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) acc += weight_q(xr[v], M, inv_t);
  }
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
    const int32_t* __restrict__ blk_pos, int block_len, int n_anchor,
    const int64_t* __restrict__ topp, int32_t* __restrict__ out) {
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
  if (threadIdx.x < 64) {
    // chunk sums in one wave (nch <= 64): inclusive scan, Z, the first chunk whose inclusive
    // sum exceeds the threshold
    const int lane = threadIdx.x;
    const uint64_t zc = lane < nch ? zpart[(int64_t)row * nch + lane] : 0;
    uint64_t incl = zc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t lo = __shfl_up((uint32_t)incl, o, 64);
      const uint32_t hi = __shfl_up((uint32_t)(incl >> 32), o, 64);
      if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
    }
    const uint64_t Z = ((uint64_t)__shfl((uint32_t)(incl >> 32), 63, 64) << 32) |
                       __shfl((uint32_t)incl, 63, 64);
    const uint64_t idx = ((uint64_t)n * n_drafts + k) * n_draft + j;
    const uint64_t u = splitmix_mix(splitmix_mix(seed) + (idx + 1) * 0x9E3779B97F4A7C15ull) >> 32;
    // (u * Z) >> 32 with the full 128-bit product
    const uint64_t lo = u * Z, hi = __umul64hi(u, Z);
    const uint64_t thr = (hi << 32) | (lo >> 32);
    const uint64_t past = __ballot(lane < nch && incl > thr);
    const int cc = past ? __ffsll((unsigned long long)past) - 1 : nch - 1;
    const uint64_t ex = incl - zc;
    const uint64_t cum = ((uint64_t)__shfl((uint32_t)(ex >> 32), cc, 64) << 32) |
                         __shfl((uint32_t)ex, cc, 64);
    if (lane == 0) {
      s_chunk = cc;
      s_thr = past ? thr - cum : 0;            // relative to the chunk start
    }
  }
  __syncthreads();
  const int c = s_chunk;
  const uint64_t thr = s_thr;
  const float M = row_max[row];
  const float* xr = x + (int64_t)row * V;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  const int per = (chunk + 255) / 256;         // contiguous segment per thread, loaded once
  const int a0 = v0 + threadIdx.x * per, a1 = min(v1, a0 + per);
  // top-p: only the nucleus (weight above q*, or equal to it up to index v_cut) keeps its weight
  const uint64_t qs = topp ? (uint64_t)topp[(int64_t)row * 4] : 0;
  const int vcut = topp ? (int)topp[(int64_t)row * 4 + 2] : 0;
  auto wq = [&](float l, int v) __attribute__((always_inline)) -> uint64_t {
    const uint64_t q = weight_q(l, M, inv_t);
    return (!topp || q > qs || (q == qs && v <= vcut)) ? q : 0;
  };
  float lx[PICK_SEG];
#pragma unroll
  for (int e = 0; e < PICK_SEG; ++e) lx[e] = a0 + e < a1 ? xr[a0 + e] : 0.f;
  uint64_t mine = 0;
#pragma unroll
  for (int e = 0; e < PICK_SEG; ++e)
    if (a0 + e < a1) mine += wq(lx[e], a0 + e);
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
    int tok = -1;
#pragma unroll
    for (int e = 0; e < PICK_SEG; ++e) {
      if (tok < 0 && a0 + e < a1) {
        run += wq(lx[e], a0 + e);
        if (run > thr) tok = a0 + e;
      }
    }
    if (tok >= 0) out[oidx] = tok;
  }
}

hipError_t launch_sample_pick(const float* x, int rows, int vocab, int chunk,
                              const uint64_t* zpart, const float* row_max, float inv_t,
                              int n_draft, int n_drafts, uint64_t seed,
                              const int32_t* row_valid_pos, int block_len, int n_anchor,
                              const int64_t* topp, int32_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (chunk > 256 * PICK_SEG || ceil_div(vocab, chunk) > 64) return hipErrorInvalidValue;
  const int nch = ceil_div(vocab, chunk);
  hipLaunchKernelGGL(sample_pick_kernel, dim3(n_drafts, rows), dim3(256), 0, s, x, vocab, chunk,
                     nch, zpart, row_max, inv_t, n_draft, n_drafts, seed, row_valid_pos,
                     block_len, n_anchor, topp, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-p nucleus
// The nucleus of a row is the shortest run of tokens, in order of decreasing integer weight
// with ties by increasing index, whose mass reaches Tp = ceil(p * Z) (p = mp / 2^sp exactly).
// Tokens are ordered by the 59-bit key (q << 18) | (2^18 - 1 - v), unique per token, so the
// nucleus is every token whose key is at least the boundary key K*.
//  1. topp_hist_kernel: per span of the row, the mass of the weights in logarithmic bins
//     (octave of q, then its next 5 bits: monotone in q, at most 3.2 % wide).
//  2. topp_bin_kernel: Z, Tp and the bin b* that holds the boundary (mass above < Tp <= mass
//     above + its own), with R = Tp - mass above.
//  3. topp_collect_kernel: per chunk, the mass of the bins above b* and the keys of the tokens
//     in b* (at most TOPP_CAP per chunk are stored; the count is exact).
//  4. topp_resolve_kernel: one workgroup per row finds K* by a mass-weighted radix select over
//     the keys in b* (from LDS, or by rescanning the row when the stored keys overflow) and
//     writes the nucleus chunk sums and {q*, -, v_cut, b*} for the sampler.
constexpr int TOPP_SUB = 5;                       // bits below the octave in a bin
constexpr int TOPP_BINS = 41 << TOPP_SUB;         // q <= 2^40
constexpr int TOPP_SPAN = 8;                      // chunks per histogram workgroup
constexpr int TOPP_CAP = 256;                     // keys stored per chunk
constexpr int TOPP_LDS_CAP = 6144;                // keys resolved from LDS
constexpr uint64_t TOPP_VMASK = (1u << 18) - 1;
static_assert(TOPP_BINS <= 6 * 256, "bins per thread in topp_bin_kernel");

__device__ __forceinline__ int topp_bin(uint64_t q) {     // q > 0
  const int msb = 63 - __clzll((long long)q);
  const uint32_t sub = msb >= TOPP_SUB ? (uint32_t)(q >> (msb - TOPP_SUB))
                                       : (uint32_t)q << (TOPP_SUB - msb);
  return (msb << TOPP_SUB) | (int)(sub & ((1u << TOPP_SUB) - 1));
}

// f(logit, index) over [v0, v1) of a row, NT threads: unaligned head, then float4 loads four in
// flight per thread, then the tail.
template <int NT, typename F>
__device__ __forceinline__ void for_logits(const float* __restrict__ xr, int v0, int v1, F&& f) {
  const int head = min(v1 - v0, (int)((4 - (((uintptr_t)(xr + v0) >> 2) & 3)) & 3));
  if ((int)threadIdx.x < head) f(xr[v0 + threadIdx.x], v0 + (int)threadIdx.x);
  const int a0 = v0 + head;
  const int nv = (v1 - a0) >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(xr + a0);
  int k = threadIdx.x;
  for (; k + 3 * NT < nv; k += 4 * NT) {
    float4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = x4[k + u * NT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = a0 + 4 * (k + u * NT);
      f(q[u].x, b);
      f(q[u].y, b + 1);
      f(q[u].z, b + 2);
      f(q[u].w, b + 3);
    }
  }
  for (; k < nv; k += NT) {
    const float4 q = x4[k];
    const int b = a0 + 4 * k;
    f(q.x, b);
    f(q.y, b + 1);
    f(q.z, b + 2);
    f(q.w, b + 3);
  }
  for (int v = a0 + 4 * nv + threadIdx.x; v < v1; v += NT) f(xr[v], v);
}

// grid (spans, rows): M from the argmax partials (span 0 stores it), then the bin masses of the
// span's weights.
__global__ __launch_bounds__(256) void topp_hist_kernel(
    const float* __restrict__ x, int V, int chunk, int nch, int nsp,
    const float* __restrict__ pv, const int32_t* __restrict__ pi, float inv_t,
    float* __restrict__ row_max, uint64_t* __restrict__ hist) {
  __shared__ unsigned long long lh[TOPP_BINS];
  __shared__ float sM;
  const int s = blockIdx.x, row = blockIdx.y;
  for (int b = threadIdx.x; b < TOPP_BINS; b += 256) lh[b] = 0;
  if (threadIdx.x < 64) {
    float bv;
    int bi;
    reduce_partials(pv, pi, row, nch, bv, bi);
    if (threadIdx.x == 0) {
      sM = bv;
      if (s == 0) row_max[row] = bv;
    }
  }
  __syncthreads();
  const float M = sM;
  const int v0 = s * TOPP_SPAN * chunk, v1 = min(V, v0 + TOPP_SPAN * chunk);
  for_logits<256>(x + (int64_t)row * V, v0, v1, [&](float l, int) {
    const uint64_t q = weight_q(l, M, inv_t);
    if (q) atomicAdd(&lh[topp_bin(q)], (unsigned long long)q);
  });
  __syncthreads();
  uint64_t* h = hist + ((int64_t)row * nsp + s) * TOPP_BINS;
  for (int b = threadIdx.x; b < TOPP_BINS; b += 256) h[b] = lh[b];
}

// one workgroup per row: thread t owns bins [6t, 6t + 6); suffix sums over the threads give the
// mass above each bin, Z is the total.  st = {-, R, -, b*}; b* = -1 if no bin qualifies
// (non-finite logits), which makes the nucleus every token of positive weight.
__global__ __launch_bounds__(256) void topp_bin_kernel(const uint64_t* __restrict__ hist,
                                                       int nsp, uint64_t mp, int sp,
                                                       int64_t* __restrict__ st) {
  __shared__ uint64_t wtot[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  uint64_t m[6], tot = 0;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const int b = 6 * tid + k;
    m[k] = 0;
    if (b < TOPP_BINS)
      for (int s = 0; s < nsp; ++s) m[k] += hist[((int64_t)row * nsp + s) * TOPP_BINS + b];
    tot += m[k];
  }
  // inclusive suffix sum over threads
  const int lane = tid & 63, w = tid >> 6;
  uint64_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_down((uint32_t)incl, o, 64);
    const uint32_t hi = __shfl_down((uint32_t)(incl >> 32), o, 64);
    if (lane + o < 64) incl += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 0) wtot[w] = incl;
  if (tid == 0) {
    st[(int64_t)row * 4 + 1] = 0;
    st[(int64_t)row * 4 + 3] = -1;
  }
  __syncthreads();
  for (int q = w + 1; q < 4; ++q) incl += wtot[q];
  const uint64_t Z = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  // Tp = ceil(mp * Z / 2^sp); mp < 2^24 and Z < 2^58, so mp * Z < 2^82
  const u128 prod = (u128)mp * Z;
  const uint64_t tp = sp >= 82 ? (prod ? 1 : 0)
                               : (uint64_t)((prod + (((u128)1 << sp) - 1)) >> sp);
  uint64_t above = incl - tot;
#pragma unroll
  for (int k = 5; k >= 0; --k) {
    if (m[k] && above < tp && tp <= above + m[k]) {
      st[(int64_t)row * 4 + 1] = (int64_t)(tp - above);
      st[(int64_t)row * 4 + 3] = 6 * tid + k;
    }
    above += m[k];
  }
}

// grid (chunks, rows): mass of the bins above b* and the keys of the tokens in b*.
__global__ __launch_bounds__(256) void topp_collect_kernel(
    const float* __restrict__ x, int V, int chunk, int nch, const float* __restrict__ row_max,
    float inv_t, const int64_t* __restrict__ st, uint64_t* __restrict__ above,
    int32_t* __restrict__ cnt, uint64_t* __restrict__ keys) {
  __shared__ uint64_t red[4];
  __shared__ int s_n;
  const int c = blockIdx.x, row = blockIdx.y;
  const int bs = (int)st[(int64_t)row * 4 + 3];
  const float M = row_max[row];
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  uint64_t* kk = keys + ((int64_t)row * nch + c) * TOPP_CAP;
  uint64_t acc = 0;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  for_logits<256>(x + (int64_t)row * V, v0, v1, [&](float l, int v) {
    const uint64_t q = weight_q(l, M, inv_t);
    if (!q) return;
    const int b = topp_bin(q);
    if (b > bs) {
      acc += q;
    } else if (b == bs) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < TOPP_CAP) kk[slot] = (q << 18) | (TOPP_VMASK - (uint64_t)v);
    }
  });
  acc = wave_sum_u64(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    above[(int64_t)row * nch + c] = red[0] + red[1] + red[2] + red[3];
    cnt[(int64_t)row * nch + c] = s_n;
  }
}

// one workgroup per row (nch <= 64).  The keys of bin b* come from LDS when every chunk kept all
// of its keys and they fit, otherwise every pass rescans the row.  Radix select from the top
// digit: per digit, the mass of each digit value among the keys matching the prefix, and the
// digit where the mass above reaches the remaining target.
__global__ __launch_bounds__(256) void topp_resolve_kernel(
    const float* __restrict__ x, int V, int chunk, int nch, const float* __restrict__ row_max,
    float inv_t, const uint64_t* __restrict__ above, const int32_t* __restrict__ cnt,
    const uint64_t* __restrict__ keys, int64_t* __restrict__ st, uint64_t* __restrict__ rz) {
  __shared__ uint64_t lk[TOPP_LDS_CAP];
  __shared__ unsigned long long lh[256];
  __shared__ unsigned long long ts[64];
  __shared__ int off[65];
  __shared__ int s_fast;
  __shared__ uint64_t s_pre, s_R, wtot[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int bs = (int)st[(int64_t)row * 4 + 3];
  if (tid < 64) {
    // offsets of the chunks' stored keys: one wave scan (nch <= 64)
    const int k = tid < nch ? cnt[(int64_t)row * nch + tid] : 0;
    const int kept = min(k, TOPP_CAP);
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (tid >= o) incl += t;
    }
    if (tid < nch) off[tid] = incl - kept;
    const int total = __shfl(incl, 63, 64);
    const bool over = __ballot(k > TOPP_CAP) != 0;
    if (tid == 0) {
      off[nch] = total;
      s_fast = !over && total <= TOPP_LDS_CAP;
      s_pre = 0;
      s_R = (uint64_t)st[(int64_t)row * 4 + 1];
    }
  }
  if (tid < 64) ts[tid] = 0;
  __syncthreads();
  const bool fast = s_fast;
  const int n = off[nch];
  if (fast) {
    const int lane = tid & 63;
    for (int c = tid >> 6; c < nch; c += 4) {
      const uint64_t* kk = keys + ((int64_t)row * nch + c) * TOPP_CAP;
      for (int j = lane; j < off[c + 1] - off[c]; j += 64) lk[off[c] + j] = kk[j];
    }
  }
  __syncthreads();
  const float M = row_max[row];
  const float* xr = x + (int64_t)row * V;
  // g(key) over the keys of bin b*
  auto each_key = [&](auto&& g) __attribute__((always_inline)) {
    if (fast) {
      for (int i = tid; i < n; i += 256) g(lk[i]);
    } else {
      for_logits<256>(xr, 0, V, [&](float l, int v) {
        const uint64_t q = weight_q(l, M, inv_t);
        if (q && topp_bin(q) == bs) g((q << 18) | (TOPP_VMASK - (uint64_t)v));
      });
    }
  };
  const int lane = tid & 63, w = tid >> 6;
  for (int d = 0; d < 8; ++d) {
    const int shift = d < 7 ? 51 - 8 * d : 0, width = d < 7 ? 8 : 3;
    lh[tid] = 0;
    __syncthreads();
    const uint64_t hp = s_pre >> (shift + width);
    const uint32_t mask = (1u << width) - 1;
    each_key([&](uint64_t k) {
      if ((k >> (shift + width)) == hp)
        atomicAdd(&lh[(k >> shift) & mask], (unsigned long long)(k >> 18));
    });
    __syncthreads();
    const uint64_t m = lh[tid];
    uint64_t incl = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t lo = __shfl_down((uint32_t)incl, o, 64);
      const uint32_t hi = __shfl_down((uint32_t)(incl >> 32), o, 64);
      if (lane + o < 64) incl += ((uint64_t)hi << 32) | lo;
    }
    if (lane == 0) wtot[w] = incl;
    __syncthreads();
    for (int q = w + 1; q < 4; ++q) incl += wtot[q];
    const uint64_t ab = incl - m, R = s_R;
    __syncthreads();
    if (tid <= (int)mask && m && ab < R && R <= ab + m) {
      s_pre |= (uint64_t)tid << shift;
      s_R = R - ab;
    }
    __syncthreads();
  }
  const uint64_t ks = s_pre;
  each_key([&](uint64_t k) {
    if (k >= ks) atomicAdd(&ts[(int)(TOPP_VMASK - (k & TOPP_VMASK)) / chunk],
                           (unsigned long long)(k >> 18));
  });
  __syncthreads();
  if (tid < nch) rz[(int64_t)row * nch + tid] = above[(int64_t)row * nch + tid] + ts[tid];
  if (tid == 0) {
    st[(int64_t)row * 4] = (int64_t)(ks >> 18);
    st[(int64_t)row * 4 + 2] = (int64_t)(TOPP_VMASK - (ks & TOPP_VMASK));
  }
}

int top_p_spans(int vocab, int chunk) { return ceil_div(ceil_div(vocab, chunk), TOPP_SPAN); }
int top_p_bins() { return TOPP_BINS; }
int top_p_cap() { return TOPP_CAP; }

hipError_t launch_top_p(const float* x, int rows, int vocab, int chunk, const float* pv,
                        const int32_t* pi, float inv_t, uint64_t mp, int sp, float* row_max,
                        int64_t* st, uint64_t* hist, uint64_t* above, int32_t* cnt,
                        uint64_t* keys, uint64_t* rz, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nch = ceil_div(vocab, chunk), nsp = top_p_spans(vocab, chunk);
  if (nch > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topp_hist_kernel, dim3(nsp, rows), dim3(256), 0, s, x, vocab, chunk, nch,
                     nsp, pv, pi, inv_t, row_max, hist);
  hipLaunchKernelGGL(topp_bin_kernel, dim3(rows), dim3(256), 0, s, hist, nsp, mp, sp, st);
  hipLaunchKernelGGL(topp_collect_kernel, dim3(nch, rows), dim3(256), 0, s, x, vocab, chunk, nch,
                     row_max, inv_t, st, above, cnt, keys);
  hipLaunchKernelGGL(topp_resolve_kernel, dim3(rows), dim3(256), 0, s, x, vocab, chunk, nch,
                     row_max, inv_t, above, cnt, keys, st, rz);
  return hipGetLastError();
}

// ------------------------------------------------------------------ block refinement
// One wave per sequence (D <= 64), after the argmax and weight sums of the D rows at temperature
// 1.  A position masked in the forward that produced the logits (conf 0) takes its row's argmax
// and Z; the argmax weight is 2^40, so its probability 2^40 / Z orders like 1 / Z.  Then the
// n_remask positions of largest Z, the lower index first on ties, are masked again (block token
// mask_id, conf 0) for the next forward.
__global__ __launch_bounds__(64) void refine_kernel(const int32_t* __restrict__ row_arg,
                                                    const uint64_t* __restrict__ zpart, int nch,
                                                    int D, int B, int n_anchor, int mask_id,
                                                    int n_remask, int32_t* __restrict__ tokens,
                                                    uint64_t* __restrict__ conf) {
  const int n = blockIdx.x, j = threadIdx.x;
  uint64_t z = 0;
  int tok = 0;
  if (j < D) {
    const int64_t row = (int64_t)n * D + j;
    z = conf[row];
    tok = tokens[(int64_t)n * B + n_anchor + j];
    if (z == 0) {
      for (int c = 0; c < nch; ++c) z += zpart[row * nch + c];
      tok = row_arg[row];
    }
  }
  int rank = 0;                                // positions less confident than this one
  for (int k = 0; k < D; ++k) {
    const uint64_t zk = ((uint64_t)__shfl((uint32_t)(z >> 32), k, 64) << 32) |
                        __shfl((uint32_t)z, k, 64);
    rank += zk > z || (zk == z && k < j);
  }
  if (j < D) {
    const bool re = rank < n_remask;
    tokens[(int64_t)n * B + n_anchor + j] = re ? mask_id : tok;
    conf[(int64_t)n * D + j] = re ? 0 : z;
  }
}

hipError_t launch_refine(const int32_t* row_arg, const uint64_t* zpart, int batch, int vocab,
                         int chunk, int D, int B, int n_anchor, int mask_id, int n_remask,
                         int32_t* tokens, uint64_t* conf, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (D > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(refine_kernel, dim3(batch), dim3(64), 0, s, row_arg, zpart,
                     ceil_div(vocab, chunk), D, B, n_anchor, mask_id, n_remask, tokens, conf);
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

// ------------------------------------------------------------------ lossless stochastic verify
// SpecDiff-2 notes, section 4 (the verifier accepts left to right with a lossless rule) and
// section 5.1 (its per-position accept rate is sum_x min(P, Q)).  The rule is the
// speculative-sampling rule (Leviathan et al., 2023) on the integer weights: with P(x) = qP_x/ZP
// (target row, temperature t_target) and Q(x) = qQ_x/ZQ (draft row, t_draft), draft token x is
// accepted iff u * qQ_x * ZP < qP_x * ZQ * 2^32 for the 32-bit draw u of (n, stream 0, j); at the
// first rejection the replacement is drawn (stream 1) from w_v = max(0, qP_v ZQ - qQ_v ZP), or
// from qP when every w_v is 0; after a full accept the bonus is drawn from target row D if it
// exists.  Draws: the SplitMix64 counter with 2 streams over D + 1 positions.  The two sides of
// the accept test reach 130 bits and are compared as (high 128, low 64) pairs; residual weights
// are below 2^98 and their sums below 2^116.

__device__ __forceinline__ uint64_t spec_draw(uint64_t seed, int n, int stream, int j, int D) {
  const uint64_t idx = ((uint64_t)n * 2 + stream) * (uint64_t)(D + 1) + j;
  return splitmix_mix(splitmix_mix(seed) + (idx + 1) * 0x9E3779B97F4A7C15ull) >> 32;
}

// u * qq * zp < qp * zq * 2^32, exactly
__device__ __forceinline__ bool spec_accept(uint64_t u, uint64_t qq, uint64_t zp, uint64_t qp,
                                            uint64_t zq) {
  const u128 a = (u128)qq * zp, b = (u128)qp * zq;
  const u128 pl = (u128)u * (uint64_t)a;
  const u128 lhi = (u128)u * (uint64_t)(a >> 64) + (pl >> 64);
  const uint64_t llo = (uint64_t)pl;
  const u128 rhi = b >> 32;
  const uint64_t rlo = (uint64_t)b << 32;
  return lhi < rhi || (lhi == rhi && llo < rlo);
}

// (u * W) >> 32 for W < 2^116
__device__ __forceinline__ u128 spec_threshold(uint64_t u, u128 W) {
  return (((u128)u * (uint64_t)(W >> 64)) << 32) + (((u128)u * (uint64_t)W) >> 32);
}

__device__ __forceinline__ u128 shfl_xor_u128(u128 v, int o) {
  const uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
  const uint64_t l = ((uint64_t)__shfl_xor((uint32_t)(lo >> 32), o, 64) << 32) |
                     __shfl_xor((uint32_t)lo, o, 64);
  const uint64_t h = ((uint64_t)__shfl_xor((uint32_t)(hi >> 32), o, 64) << 32) |
                     __shfl_xor((uint32_t)hi, o, 64);
  return ((u128)h << 64) | l;
}
__device__ __forceinline__ u128 shfl_up_u128(u128 v, int o) {
  const uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
  const uint64_t l = ((uint64_t)__shfl_up((uint32_t)(lo >> 32), o, 64) << 32) |
                     __shfl_up((uint32_t)lo, o, 64);
  const uint64_t h = ((uint64_t)__shfl_up((uint32_t)(hi >> 32), o, 64) << 32) |
                     __shfl_up((uint32_t)hi, o, 64);
  return ((u128)h << 64) | l;
}

__device__ __forceinline__ u128 shfl_idx_u128(u128 v, int src) {
  const uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
  const uint64_t l = ((uint64_t)__shfl((uint32_t)(lo >> 32), src, 64) << 32) |
                     __shfl((uint32_t)lo, src, 64);
  const uint64_t h = ((uint64_t)__shfl((uint32_t)(hi >> 32), src, 64) << 32) |
                     __shfl((uint32_t)hi, src, 64);
  return ((u128)h << 64) | l;
}

// residual weight of token v at a rejected position (mode 1) or P's weight (otherwise)
__device__ __forceinline__ u128 spec_weight(const float* tr, const float* dr, int v, float Mp,
                                            float Mq, float inv_p, float inv_q, uint64_t zp,
                                            uint64_t zq, bool resid) {
  const uint64_t qp = weight_q(tr[v], Mp, inv_p);
  if (!resid) return qp;
  const u128 a = (u128)qp * zq, b = (u128)weight_q(dr[v], Mq, inv_q) * zp;
  return a > b ? a - b : 0;
}

// One workgroup per sequence.  Wave w sums the chunk partials of positions w, w + 4, ... (lane c
// takes chunk c), its lane 0 runs the position's accept test; the first rejection (lowest
// rejected position) ends the accepted prefix.  spec[n] = {mode, position, ZP, ZQ}: mode 1
// residual draw at the rejected position, 2 bonus draw from target row D, 0 no draw.
__global__ __launch_bounds__(256) void spec_accept_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl, const int32_t* __restrict__ drafts,
    int stride, int D, int R, int V, int nch, const uint64_t* __restrict__ zp_t,
    const float* __restrict__ rm_t, const uint64_t* __restrict__ zp_d,
    const float* __restrict__ rm_d, float inv_p, float inv_q, uint64_t seed,
    int32_t* __restrict__ n_acc, int64_t* __restrict__ spec) {
  __shared__ uint64_t s_zp[65], s_zq[65];
  __shared__ int s_first;
  const int n = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_first = D;
  __syncthreads();
  for (int j = wave; j <= D; j += 4) {
    if (j == D && R == D) break;
    const int64_t rt = (int64_t)n * R + j, rd = (int64_t)n * D + j;
    uint64_t zp = 0, zq = 0;
    for (int c = lane; c < nch; c += 64) {
      zp += zp_t[rt * nch + c];
      if (j < D) zq += zp_d[rd * nch + c];
    }
    zp = wave_sum_u64(zp);
    zq = wave_sum_u64(zq);
    if (lane == 0) {
      s_zp[j] = zp;
      s_zq[j] = zq;
      if (j < D) {
        const int x = drafts[(int64_t)n * stride + j];
        const bool in = x >= 0 && x < V;
        const uint64_t qp = in ? weight_q(tl[rt * V + x], rm_t[rt], inv_p) : 0;
        const uint64_t qq = in ? weight_q(dl[rd * V + x], rm_d[rd], inv_q) : 0;
        if (!spec_accept(spec_draw(seed, n, 0, j, D), qq, zp, qp, zq)) atomicMin(&s_first, j);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int first = s_first;
    int64_t* sp = spec + (int64_t)n * 4;
    n_acc[n] = first;
    sp[0] = first < D ? 1 : (R > D ? 2 : 0);
    sp[1] = first;
    sp[2] = first < D || R > D ? (int64_t)s_zp[first] : 0;
    sp[3] = first < D ? (int64_t)s_zq[first] : 0;
  }
}

// grid (chunks, N): chunk sums of the residual weights of a rejected position (mode 1 only).
__global__ __launch_bounds__(256) void spec_resid_partial_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl, int D, int R, int V, int chunk,
    int nch, const float* __restrict__ rm_t, const float* __restrict__ rm_d, float inv_p,
    float inv_q, const int64_t* __restrict__ spec, u128* __restrict__ wpart) {
  __shared__ u128 red[4];
  const int c = blockIdx.x, n = blockIdx.y;
  const int64_t* sp = spec + (int64_t)n * 4;
  if (sp[0] != 1) return;
  const int j = (int)sp[1];
  const uint64_t zp = (uint64_t)sp[2], zq = (uint64_t)sp[3];
  const int64_t rt = (int64_t)n * R + j, rd = (int64_t)n * D + j;
  const float* tr = tl + rt * V;
  const float* dr = dl + rd * V;
  const float Mp = rm_t[rt], Mq = rm_d[rd];
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);
  u128 acc = 0;
  auto w1 = [&](float a, float b) __attribute__((always_inline)) -> u128 {
    const u128 x = (u128)weight_q(a, Mp, inv_p) * zq, y = (u128)weight_q(b, Mq, inv_q) * zp;
    return x > y ? x - y : 0;
  };
  if ((((uintptr_t)(tr + v0) | (uintptr_t)(dr + v0)) & 15) == 0) {
    const int nv = (v1 - v0) >> 2;
    const float4* t4 = reinterpret_cast<const float4*>(tr + v0);
    const float4* d4 = reinterpret_cast<const float4*>(dr + v0);
    int k = threadIdx.x;
    for (; k + 256 < nv; k += 2 * 256) {
      const float4 a0 = t4[k], b0 = d4[k], a1 = t4[k + 256], b1 = d4[k + 256];
      acc += w1(a0.x, b0.x) + w1(a0.y, b0.y) + w1(a0.z, b0.z) + w1(a0.w, b0.w);
      acc += w1(a1.x, b1.x) + w1(a1.y, b1.y) + w1(a1.z, b1.z) + w1(a1.w, b1.w);
    }
    for (; k < nv; k += 256) {
      const float4 a = t4[k], b = d4[k];
      acc += w1(a.x, b.x) + w1(a.y, b.y) + w1(a.z, b.z) + w1(a.w, b.w);
    }
    for (int v = v0 + 4 * nv + threadIdx.x; v < v1; v += 256) acc += w1(tr[v], dr[v]);
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) acc += w1(tr[v], dr[v]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += shfl_xor_u128(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) wpart[(int64_t)n * nch + c] = red[0] + red[1] + red[2] + red[3];
}

// One workgroup per sequence: the replacement / bonus token by threshold search (chunk from the
// chunk sums, then a block-wide exclusive scan over that chunk), the committed tokens and the
// non-finite flag of the sequence's rows.
__global__ __launch_bounds__(256) void spec_pick_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl,
    const int32_t* __restrict__ drafts, int stride, int D, int R, int V, int chunk, int nch,
    const uint64_t* __restrict__ zp_t, const float* __restrict__ rm_t,
    const float* __restrict__ rm_d, const int32_t* __restrict__ pf_t,
    const int32_t* __restrict__ pf_d, float inv_p, float inv_q, uint64_t seed,
    const int64_t* __restrict__ spec, const u128* __restrict__ wpart,
    const int32_t* __restrict__ n_acc, int32_t* __restrict__ bonus,
    int32_t* __restrict__ committed, int32_t* __restrict__ row_flags) {
  __shared__ u128 s_thr;
  __shared__ int s_chunk, s_resid, s_tok, s_bad;
  __shared__ u128 wsum[4];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t* sp = spec + (int64_t)n * 4;
  const int mode = (int)sp[0], j = (int)sp[1];
  const uint64_t zp = (uint64_t)sp[2], zq = (uint64_t)sp[3];
  const int64_t rt = (int64_t)n * R + j, rd = (int64_t)n * D + (j < D ? j : 0);
  if (tid == 0) {
    s_tok = -1;
    s_bad = 0;
  }
  if (mode != 0 && tid < 64) {
    // wave 0: chunk sums (lane c holds chunks c, c + 64, ...), total, threshold, then the first
    // chunk whose inclusive prefix exceeds it by a wave-wide scan per 64-chunk group
    const int lane = tid;
    bool resid = mode == 1;
    u128 W = 0;
    if (resid) {
      for (int c = lane; c < nch; c += 64) W += wpart[(int64_t)n * nch + c];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) W += shfl_xor_u128(W, o);
      if (W == 0) resid = false;                // P <= Q everywhere: draw from P
    }
    if (!resid) {
      uint64_t z = 0;
      for (int c = lane; c < nch; c += 64) z += zp_t[rt * nch + c];
      W = wave_sum_u64(z);
    }
    const u128 thr = spec_threshold(spec_draw(seed, n, 1, j, D), W);
    u128 base = 0;
    int found = -1;
    u128 below = 0;
    for (int c0 = 0; c0 < nch && found < 0; c0 += 64) {
      const int c = c0 + lane;
      const u128 wc = c < nch ? (resid ? wpart[(int64_t)n * nch + c] : (u128)zp_t[rt * nch + c])
                              : (u128)0;
      u128 incl = wc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u128 t = shfl_up_u128(incl, o);
        if (lane >= o) incl += t;
      }
      const uint64_t hit = __ballot(c < nch && base + incl > thr);
      if (hit) {
        found = c0 + __ffsll((unsigned long long)hit) - 1;
        const int src = found - c0;
        const u128 ex = shfl_idx_u128(incl - wc, src);
        below = base + ex;
      } else {
        base += shfl_idx_u128(incl, 63);
      }
    }
    if (lane == 0) {
      if (found < 0) {                           // threshold beyond the sums: last chunk
        found = nch - 1;
        below = base - (resid ? wpart[(int64_t)n * nch + found] : (u128)zp_t[rt * nch + found]);
      }
      s_chunk = found;
      s_thr = thr - below;
      s_resid = resid;
    }
  }
  __syncthreads();
  int bad = 0;
  for (int q = tid; q < R * nch; q += 256) bad |= pf_t[(int64_t)n * R * nch + q];
  for (int q = tid; q < D * nch; q += 256) bad |= pf_d[(int64_t)n * D * nch + q];
  if (bad) atomicOr(&s_bad, 1);
  if (mode != 0) {
    const bool resid = s_resid;
    const int c = s_chunk;
    const u128 thr = s_thr;
    const float* tr = tl + rt * V;
    const float* dr = dl + rd * V;
    const float Mp = rm_t[rt], Mq = resid ? rm_d[rd] : 0.f;
    const int v0 = c * chunk, v1 = min(V, v0 + chunk);
    // the thread's contiguous segment of the chunk, loaded once (all loads in flight together)
    const int per = (chunk + 255) / 256;
    const int a0 = v0 + tid * per, a1 = min(v1, a0 + per);
    float lt[PICK_SEG], ld[PICK_SEG];
#pragma unroll
    for (int e = 0; e < PICK_SEG; ++e) {
      const int v = a0 + e;
      lt[e] = v < a1 ? tr[v] : 0.f;
      ld[e] = v < a1 && resid ? dr[v] : 0.f;
    }
    auto wgt = [&](int e) __attribute__((always_inline)) -> u128 {
      const uint64_t qp = weight_q(lt[e], Mp, inv_p);
      if (!resid) return qp;
      const u128 a = (u128)qp * zq, b = (u128)weight_q(ld[e], Mq, inv_q) * zp;
      return a > b ? a - b : 0;
    };
    u128 mine = 0;
#pragma unroll
    for (int e = 0; e < PICK_SEG; ++e)
      if (a0 + e < a1) mine += wgt(e);
    const int lane = tid & 63, w = tid >> 6;
    u128 incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u128 t = shfl_up_u128(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    u128 excl = incl - mine;
    for (int q = 0; q < w; ++q) excl += wsum[q];
    if (excl <= thr && thr < excl + mine) {
      u128 run = excl;
      int tok = -1;
#pragma unroll
      for (int e = 0; e < PICK_SEG; ++e) {
        if (tok < 0 && a0 + e < a1) {
          run += wgt(e);
          if (run > thr) tok = a0 + e;
        }
      }
      s_tok = tok;
    }
  }
  __syncthreads();
  const int a = n_acc[n], b = s_tok;
  for (int q = tid; q <= D; q += 256)
    committed[(int64_t)n * (D + 1) + q] =
        q < a ? drafts[(int64_t)n * stride + q] : (q == a ? b : -1);
  if (tid == 0) {
    bonus[n] = b;
    if (row_flags) row_flags[n] = s_bad ? 1 : 0;
  }
}

hipError_t launch_verify_sample(const float* tl, const float* dl, const int32_t* drafts,
                                int stride, int batch, int D, int R, int V, int chunk,
                                const uint64_t* zp_t, const float* rm_t, const uint64_t* zp_d,
                                const float* rm_d, const int32_t* pf_t, const int32_t* pf_d,
                                float inv_p, float inv_q, uint64_t seed, int64_t* spec,
                                void* wpart, int32_t* n_acc, int32_t* bonus,
                                int32_t* committed, int32_t* row_flags, hipStream_t s) {
  if (chunk > 256 * PICK_SEG) return hipErrorInvalidValue;
  const int nch = ceil_div(V, chunk);
  hipLaunchKernelGGL(spec_accept_kernel, dim3(batch), dim3(256), 0, s, tl, dl, drafts, stride, D,
                     R, V, nch, zp_t, rm_t, zp_d, rm_d, inv_p, inv_q, seed, n_acc, spec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_resid_partial_kernel, dim3(nch, batch), dim3(256), 0, s, tl, dl, D, R,
                     V, chunk, nch, rm_t, rm_d, inv_p, inv_q, spec, (u128*)wpart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_pick_kernel, dim3(batch), dim3(256), 0, s, tl, dl, drafts, stride, D, R,
                     V, chunk, nch, zp_t, rm_t, rm_d, pf_t, pf_d, inv_p, inv_q, seed, spec,
                     (const u128*)wpart, n_acc, bonus, committed, row_flags);
  return hipGetLastError();
}

// ------------------------------------------------------------------ streak selection
// One workgroup per sequence.  Its threads take the K x G (draft, position) rows in parallel:
// Z from the row's chunk sums, the draft token's integer weight q, p = double(q) / double(Z)
// correctly rounded, kept in LDS; then thread k scores draft k, S = sum_m prod_{j<=m} p_j in
// fp64 in position order (the same operations in the same order as one thread per draft doing
// everything, so the scores are unchanged).  K, G <= 64.
constexpr int SF_THREADS = 1024;
constexpr int SF_TPR = 4;                 // threads per (draft, row): the chunk sums split 4 ways
__global__ __launch_bounds__(SF_THREADS) void select_finalize_kernel(
    const float* __restrict__ x, int V, int nch, const uint64_t* __restrict__ zpart,
    const float* __restrict__ row_max, const int32_t* __restrict__ row_arg,
    const int32_t* __restrict__ pflag, const int32_t* __restrict__ drafts, int K, int G, int R,
    int32_t* selected, double* scores, int32_t* n_acc, int32_t* bonus, int32_t* committed,
    int32_t* row_flags) {
  __shared__ double s_p[64 * 64];
  __shared__ double s_score[64];
  __shared__ int32_t t_s[128];
  __shared__ int s_best, s_bad;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // Z of each (draft k, row j): SF_TPR neighbouring lanes add every SF_TPR-th chunk, then
  // combine (integer sums: the order does not change them)
  for (int r0 = 0; r0 < K * G; r0 += SF_THREADS / SF_TPR) {
    const int r = r0 + tid / SF_TPR, part = tid % SF_TPR;
    const bool live = r < K * G;
    const int k = live ? r / G : 0, j = live ? r % G : 0;
    const int64_t row = ((int64_t)n * K + k) * R + j;
    uint64_t q = 0;
    if (live && part == 0) {
      const int tok = drafts[((int64_t)n * K + k) * G + j];
      if (tok >= 0 && tok < V) q = weight_q(x[row * V + tok], row_max[row], 1.0f);
    }
    uint64_t Z = 0;
    if (live)
      for (int c = part; c < nch; c += SF_TPR) Z += zpart[row * nch + c];
#pragma unroll
    for (int o = 1; o < SF_TPR; o <<= 1) Z += __shfl_xor(Z, o, 64);
    if (live && part == 0) s_p[r] = __ddiv_rn((double)q, (double)Z);
  }
  // non-finite flags of every row of the sequence (K x R rows)
  int bad = 0;
  const int64_t f0 = (int64_t)n * K * R * nch;
  for (int i = tid; i < K * R * nch; i += SF_THREADS) bad |= pflag[f0 + i];
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  for (int k = tid; k < K; k += SF_THREADS) {
    double P = 1.0, S = 0.0;
    for (int j = 0; j < G; ++j) {
      P = __dmul_rn(P, s_p[k * G + j]);
      S = __dadd_rn(S, P);
    }
    s_score[k] = S;
    if (scores) scores[(int64_t)n * K + k] = S;
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int k = 1; k < K; ++k)
      if (s_score[k] > s_score[best]) best = k;
    s_best = best;
    selected[n] = best;
  }
  __syncthreads();
  const int best = s_best;
  for (int j = tid; j < R; j += SF_THREADS) t_s[j] = row_arg[((int64_t)n * K + best) * R + j];
  __syncthreads();
  if (tid < 64) {
    greedy_accept(t_s, drafts + ((int64_t)n * K + best) * G, G, R, n_acc + n, bonus + n,
                  committed + (int64_t)n * (G + 1));
    if (row_flags && tid == 0) row_flags[n] = s_bad ? 1 : 0;
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
  hipLaunchKernelGGL(select_finalize_kernel, dim3(batch), dim3(SF_THREADS), 0, s, x, vocab, nch,
                     zpart,
                     row_max, row_arg, pflag, drafts, n_drafts, gamma, n_rows, selected, scores,
                     n_acc, bonus, committed, row_flags);
  return hipGetLastError();
}

}  // namespace dbd
