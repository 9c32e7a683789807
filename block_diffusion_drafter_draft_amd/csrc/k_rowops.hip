// Row kernels of draft_block: per-row metadata and rotary tables, the ingest mix + RMSNorm
// (DFlare page, section on per-draft-layer mixing), the embedding gather and RMSNorm.
#include "dbd_internal.h"

namespace dbd {

// ------------------------------------------------------------------ prep
// One thread per (row, frequency pair).  Rows 0 .. N*B-1 are block rows, then the ingest rows.
// A sequence is valid when its offsets are ordered, lie in [0, n_new_total] and its block fits
// the cache: ctx_len + n_new + B <= cap.  Invalid sequences get position -1 everywhere.
struct Freqs {
  double v[64];
};

__device__ __forceinline__ bool seq_ok(const int32_t* ctx_len, const int32_t* off, int n,
                                       int block_len, int n_new_total, int cap, int* P) {
  int c = ctx_len[n], a = off[n], b = off[n + 1];
  bool ok = c >= 0 && a >= 0 && b >= a && b <= n_new_total &&
            (int64_t)c + (b - a) + block_len <= cap;
  *P = c + (b - a);
  return ok;
}

__global__ void prep_kernel(const int32_t* __restrict__ ctx_len,
                            const int32_t* __restrict__ off, int batch, int block_len,
                            int n_new_total, int cap, int half, Freqs fq, RowMeta meta,
                            int32_t* seq_status) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nblk = batch * block_len;
  const int64_t total = (int64_t)(nblk + n_new_total) * half;
  if (gid < batch) {
    int P;
    bool ok = seq_ok(ctx_len, off, (int)gid, block_len, n_new_total, cap, &P);
    meta.seq_keys[gid] = ok ? P + block_len : 0;
    if (seq_status) seq_status[gid] = ok ? 0 : 2;
  }
  if (gid >= total) return;
  const int row = (int)(gid / half);
  const int i = (int)(gid % half);
  int pos;
  if (row < nblk) {
    const int n = row / block_len, b = row % block_len;
    int P;
    bool ok = seq_ok(ctx_len, off, n, block_len, n_new_total, cap, &P);
    pos = ok ? P + b : -1;
    if (i == 0) meta.blk_pos[row] = pos;
  } else {
    const int t = row - nblk;
    // sequence of ingest row t: the last n with off[n] <= t (offsets are non-decreasing)
    int lo = 0, hi = batch - 1, n = -1;
    while (lo <= hi) {
      int mid = (lo + hi) >> 1;
      if (off[mid] <= t) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    pos = -1;
    if (n >= 0 && t < off[n + 1]) {
      int P;
      if (seq_ok(ctx_len, off, n, block_len, n_new_total, cap, &P)) pos = ctx_len[n] + (t - off[n]);
    }
    if (i == 0) {
      meta.ctx_seq[t] = pos >= 0 ? n : -1;
      meta.ctx_pos[t] = pos;
    }
  }
  // rotation angle pos * theta^(-2i/hd) in fp64, stored as fp32 (cos, sin)
  double ang = (double)(pos < 0 ? 0 : pos) * fq.v[i];
  double sn, cs;
  sincos(ang, &sn, &cs);
  float2 r = make_float2((float)cs, (float)sn);
  if (row < nblk) meta.rope_blk[(int64_t)row * half + i] = r;
  else meta.rope_ctx[(int64_t)(row - nblk) * half + i] = r;
}

hipError_t launch_prep(const int32_t* ctx_len, const int32_t* new_offsets, int batch,
                       int block_len, int n_new_total, int cap, int hd, const double* inv_freq,
                       RowMeta meta, int32_t* seq_status, hipStream_t s) {
  Freqs fq;
  const int half = hd / 2;
  for (int i = 0; i < 64; ++i) fq.v[i] = i < half ? inv_freq[i] : 0.0;
  int64_t total = (int64_t)(batch * block_len + n_new_total) * half;
  if (total < batch) total = batch;
  const int threads = 256;
  const int blocks = (int)ceil_div64(total, threads);
  hipLaunchKernelGGL(prep_kernel, dim3(blocks), dim3(threads), 0, s, ctx_len, new_offsets, batch,
                     block_len, n_new_total, cap, half, fq, meta, seq_status);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// ------------------------------------------------------------------ mix + RMSNorm
// One workgroup of NT threads per (ingested token, group of LG draft layers): the L_d outputs
// of a token are independent given its L_t target rows, so each workgroup reads the token's L_t
// rows (16-byte coalesced loads) once and writes the normalised rows of its LG layers.  LG = 8
// reads every target row once for all layers (many tokens: a cold ingest, a large batch);
// LG = 1 spreads a few tokens over L_d times more workgroups.  Each thread owns CPT chunks of
// VEC consecutive hidden elements; with one chunk per thread every target layer's chunk and the
// gain chunks are loaded at once, before the mixing weights are ready, with more, target layer
// i + 1 is loaded while layer i is mixed.
constexpr int kMaxLt = 16;

template <typename T> struct Vec16;
template <> struct Vec16<bf16> { static constexpr int n = 8; };
template <> struct Vec16<float> { static constexpr int n = 4; };

template <typename T, int CPT, int NT, int LG>
__global__ __launch_bounds__(NT) void mix_rmsnorm_kernel(
    const T* __restrict__ hid, int64_t ts, int64_t ls, int n_tok, int H, int Lt, int Ld,
    const float* __restrict__ mix_logits, int raw, const T* __restrict__ g, T* __restrict__ out,
    T* __restrict__ out_lo, float eps) {
  constexpr int VEC = Vec16<T>::n, NW = NT / 64;
  constexpr bool ALL = CPT == 1;                 // every layer's chunk in flight at once
  __shared__ float w[LG * kMaxLt];
  __shared__ float red[LG][NW];
  const int t = blockIdx.x, l0 = blockIdx.y * LG;
  const int nl = min(LG, Ld - l0);              // layers of this workgroup
  const int tid = threadIdx.x;
  const int nch = H / VEC;
  const T* base = hid + (int64_t)t * ts;
  u32x4 hv[ALL ? kMaxLt : 1], gv[ALL ? LG : 1][CPT];
  if constexpr (ALL) {
    if (tid < nch) {
#pragma unroll
      for (int i = 0; i < kMaxLt; ++i)
        if (i < Lt) hv[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)i * ls + tid * VEC);
#pragma unroll
      for (int j = 0; j < LG; ++j)
        if (j < nl) gv[j][0] = *reinterpret_cast<const u32x4*>(g + (int64_t)(l0 + j) * H + tid * VEC);
    }
  }
  if (tid < nl) {
    // softmax over the target layers of draft layer l0 + tid's mixing logits (raw: the logits)
    const float* lg = mix_logits + (l0 + tid) * Lt;
    float m = -INFINITY;
    for (int i = 0; i < Lt; ++i) m = fmaxf(m, lg[i]);
    float sum = 0.f;
    for (int i = 0; i < Lt; ++i) sum += expf(lg[i] - m);
    for (int i = 0; i < Lt; ++i) w[tid * Lt + i] = raw ? lg[i] : expf(lg[i] - m) / sum;
  }
  __syncthreads();
  float acc[LG][CPT * VEC];
#pragma unroll
  for (int j = 0; j < LG; ++j)
#pragma unroll
    for (int e = 0; e < CPT * VEC; ++e) acc[j][e] = 0.f;
  auto mix = [&](const u32x4* r, int i) __attribute__((always_inline)) {
    float wl[LG];
#pragma unroll
    for (int j = 0; j < LG; ++j) wl[j] = j < nl ? w[j * Lt + i] : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        T v[VEC];
        *reinterpret_cast<u32x4*>(v) = r[c];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float x = to_f(v[e]);
#pragma unroll
          for (int j = 0; j < LG; ++j) acc[j][c * VEC + e] += wl[j] * x;
        }
      }
    }
  };
  if constexpr (ALL) {
#pragma unroll
    for (int i = 0; i < kMaxLt; ++i)
      if (i < Lt) mix(&hv[i], i);
  } else {
    u32x4 cur[CPT], nxt[CPT];
    auto load = [&](u32x4* r, int i) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = tid + c * NT;
        if (ch < nch) r[c] = *reinterpret_cast<const u32x4*>(base + (int64_t)i * ls + ch * VEC);
      }
    };
    load(cur, 0);
    for (int i = 0; i < Lt; ++i) {
      if (i + 1 < Lt) load(nxt, i + 1);
      mix(cur, i);
#pragma unroll
      for (int c = 0; c < CPT; ++c) cur[c] = nxt[c];
    }
  }
  float ss[LG];
#pragma unroll
  for (int j = 0; j < LG; ++j) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < CPT * VEC; ++e) s += acc[j][e] * acc[j][e];
    ss[j] = wave_sum(s);
  }
  if ((tid & 63) == 0)
#pragma unroll
    for (int j = 0; j < LG; ++j) red[j][tid >> 6] = ss[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < LG; ++j) {
    if (j >= nl) break;
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) tot += red[j][q];
    const float inv = rsqrtf(tot / (float)H + eps);
    const int l = l0 + j;
    T* o = out + ((int64_t)l * n_tok + t) * H;
    T* ol = out_lo ? out_lo + ((int64_t)l * n_tok + t) * H : nullptr;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        T gr[VEC], ov[VEC], lv[VEC];
        if constexpr (ALL) *reinterpret_cast<u32x4*>(gr) = gv[j][0];
        else *reinterpret_cast<u32x4*>(gr) = *reinterpret_cast<const u32x4*>(g + (int64_t)l * H + ch * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float y = acc[j][c * VEC + e] * inv * to_f(gr[e]);
          ov[e] = from_f<T>(y);
          lv[e] = from_f<T>(y - to_f(ov[e]));     // low part of the bf16 pair
        }
        *reinterpret_cast<u32x4*>(o + ch * VEC) = *reinterpret_cast<u32x4*>(ov);
        if (ol) *reinterpret_cast<u32x4*>(ol + ch * VEC) = *reinterpret_cast<u32x4*>(lv);
      }
    }
  }
}

// Fewer tokens than kMixSpreadTokens: one draft layer per workgroup (measured on MI355X: 7
// tokens of the Qwen3-4B shape 0.016 -> 0.009 ms; at 215 tokens of the Qwen3-8B shape one
// workgroup per token stays faster, 0.021 against 0.025 ms, as the target rows are read once).
constexpr int kMixSpreadTokens = 128;

template <typename T>
static hipError_t mix_dispatch(const void* hid, int64_t ts, int64_t ls, int n_tok, int H, int Lt,
                               int Ld, const float* ml, int raw, const void* g, void* out,
                               void* out_lo, float eps, hipStream_t s) {
  constexpr int VEC = Vec16<T>::n;
  const int nch = H / VEC;
  const T* h = (const T*)hid;
  if (n_tok == 0 || Ld == 0) return hipSuccess;
  const bool spread = n_tok < kMixSpreadTokens;
#define DBD_MIX(CPT, NT, LG)                                                                   \
  hipLaunchKernelGGL((mix_rmsnorm_kernel<T, CPT, NT, LG>), dim3(n_tok, (Ld + LG - 1) / LG),   \
                     dim3(NT), 0, s, h, ts, ls, n_tok, H, Lt, Ld, ml, raw, (const T*)g, (T*)out, \
                     (T*)out_lo, eps)
#define DBD_MIX_LG(CPT, NT) \
  do { if (spread) DBD_MIX(CPT, NT, 1); else DBD_MIX(CPT, NT, 8); } while (0)
  if (nch <= 256) DBD_MIX_LG(1, 256);
  else if (nch <= 512) DBD_MIX_LG(1, 512);
  else if (nch <= 1024) DBD_MIX_LG(2, 512);      // bf16 rows up to 8192, fp32 up to 4096
  else return hipErrorInvalidValue;
#undef DBD_MIX_LG
#undef DBD_MIX
  return hipGetLastError();
}

hipError_t launch_mix_rmsnorm(int dtype, const void* hid, int64_t ts, int64_t ls, int n_tok,
                              int H, int Lt, int Ld, const float* mix_logits, int raw,
                              const void* g, void* out, void* out_lo, float eps, hipStream_t s) {
  return dtype == 1 ? mix_dispatch<bf16>(hid, ts, ls, n_tok, H, Lt, Ld, mix_logits, raw, g, out,
                                         out_lo, eps, s)
                    : mix_dispatch<float>(hid, ts, ls, n_tok, H, Lt, Ld, mix_logits, raw, g, out,
                                          nullptr, eps, s);
}

// ------------------------------------------------------------------ embedding gather
// One workgroup per block row: the row's token embedding (ids clamped to the vocabulary) becomes
// the fp32 residual row x.  With a gain g the kernel also writes the first layer's attention
// RMSNorm of the row, which it holds in registers, as rmsnorm_kernel would (out, and the bf16
// low part in out_lo).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok,
                                                    const T* __restrict__ E, int H, int V,
                                                    float* __restrict__ x,
                                                    const T* __restrict__ g,
                                                    T* __restrict__ out, T* __restrict__ out_lo,
                                                    float eps) {
  constexpr int VEC = 16 / (int)sizeof(T);             // elements per 16-byte load
  constexpr int MAXC = 8192 / (256 * VEC);              // chunks per thread at H = 8192
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  int id = tok[r];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);       // out-of-range ids are clamped
  const T* e = E + (int64_t)id * H;
  float* o = x + (int64_t)r * H;
  if (H % VEC != 0 || ((((uintptr_t)e | (uintptr_t)o) & 15) != 0)) {
    for (int i = tid; i < H; i += 256) o[i] = to_f(e[i]);   // (never with a norm: see launch)
    return;
  }
  // 16-byte loads, all of a thread's chunks (and the gain's) in flight at once
  u32x4 raw[MAXC], gr[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int i = (tid + c * 256) * VEC;
    if (i < H) {
      raw[c] = *reinterpret_cast<const u32x4*>(e + i);
      if (g) gr[c] = *reinterpret_cast<const u32x4*>(g + i);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int i = (tid + c * 256) * VEC;
    if (i >= H) continue;
    const T* v = reinterpret_cast<const T*>(&raw[c]);
#pragma unroll
    for (int q = 0; q < VEC; q += 4) {
      const f32x4 f = f32x4{to_f(v[q]), to_f(v[q + 1]), to_f(v[q + 2]), to_f(v[q + 3])};
      *reinterpret_cast<f32x4*>(o + i + q) = f;
      ss += f[0] * f[0] + f[1] * f[1] + f[2] * f[2] + f[3] * f[3];
    }
  }
  if (!g) return;
  // the first layer's attention RMSNorm of the row (as rmsnorm_kernel computes it)
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  T* no = out + (int64_t)r * H;
  T* nl = out_lo ? out_lo + (int64_t)r * H : nullptr;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int i = (tid + c * 256) * VEC;
    if (i >= H) continue;
    const T* v = reinterpret_cast<const T*>(&raw[c]);
    const T* gv = reinterpret_cast<const T*>(&gr[c]);
    T hi[VEC], lo[VEC];
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      const float y = to_f(v[q]) * inv * to_f(gv[q]);
      hi[q] = from_f<T>(y);
      lo[q] = from_f<T>(y - to_f(hi[q]));
    }
    *reinterpret_cast<u32x4*>(no + i) = *reinterpret_cast<const u32x4*>(hi);
    if (nl) *reinterpret_cast<u32x4*>(nl + i) = *reinterpret_cast<const u32x4*>(lo);
  }
}

// With g set (and H a multiple of the 16-byte vector, 16-byte aligned rows) the kernel also
// writes the row's RMSNorm with gain g to out (and its bf16 low part to out_lo) and *normed is
// set; otherwise the caller runs the norm itself.
hipError_t launch_embed(int dtype, const int32_t* tokens, const void* E, int rows, int H, int V,
                        float* x, const void* g, void* out, void* out_lo, float eps,
                        hipStream_t s, bool* normed) {
  const int es = dtype == 1 ? 2 : 4;
  const bool fuse = g && H % (16 / es) == 0 && H <= 8192 && ((uintptr_t)E & 15) == 0 &&
                    ((uintptr_t)x & 15) == 0 && ((uintptr_t)g & 15) == 0 &&
                    ((uintptr_t)out & 15) == 0 && ((uintptr_t)out_lo & 15) == 0 &&
                    (int64_t)H * es % 16 == 0;
  if (!fuse) g = out = out_lo = nullptr;
  if (dtype == 1)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(rows), dim3(256), 0, s, tokens, (const bf16*)E,
                       H, V, x, (const bf16*)g, (bf16*)out, (bf16*)out_lo, eps);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, s, tokens,
                       (const float*)E, H, V, x, (const float*)g, (float*)out, nullptr, eps);
  if (normed) *normed = fuse;
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// out[r'] = T(x[r] / sqrt(mean(x[r]^2) + eps) * g), and with out_lo the low part of the bf16
// pair.  With n_anchor > 0 only the mask rows of each block are normalised and written
// compactly (r' = n*(B - n_anchor) + b - n_anchor).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const T* __restrict__ g,
                                                      T* __restrict__ out, T* __restrict__ out_lo,
                                                      int H, float eps, int block_len,
                                                      int n_anchor) {
  // thread t owns the groups of 4 columns t, t + 256, ... (coalesced); the row stays in registers
  // between the sum of squares and the scaling (H <= 8192)
  constexpr int MAXG = 8;
  __shared__ float red[4];
  const int ro = blockIdx.x;
  int ri = ro;
  if (n_anchor > 0) {
    const int D = block_len - n_anchor;
    ri = (ro / D) * block_len + n_anchor + ro % D;
  }
  const float* xr = x + (int64_t)ri * H;
  float4 v[MAXG];
  T gv[MAXG][4];                                  // the gain, loaded with the row
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int i = (threadIdx.x + q * 256) * 4;
    if (i < H) {
      v[q] = *reinterpret_cast<const float4*>(xr + i);
      if constexpr (sizeof(T) == 2)
        *reinterpret_cast<uint2*>(gv[q]) = *reinterpret_cast<const uint2*>(g + i);
      else
        *reinterpret_cast<float4*>(gv[q]) = *reinterpret_cast<const float4*>(g + i);
      s += v[q].x * v[q].x + v[q].y * v[q].y + v[q].z * v[q].z + v[q].w * v[q].w;
    }
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  T* o = out + (int64_t)ro * H;
  T* ol = out_lo ? out_lo + (int64_t)ro * H : nullptr;
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int i = (threadIdx.x + q * 256) * 4;
    if (i >= H) continue;
    T hi[4], lo[4];
    const float y[4] = {v[q].x * inv * to_f(gv[q][0]), v[q].y * inv * to_f(gv[q][1]),
                        v[q].z * inv * to_f(gv[q][2]), v[q].w * inv * to_f(gv[q][3])};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = from_f<T>(y[e]);
      lo[e] = from_f<T>(y[e] - to_f(hi[e]));
    }
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint2*>(o + i) = *reinterpret_cast<uint2*>(hi);
      if (ol) *reinterpret_cast<uint2*>(ol + i) = *reinterpret_cast<uint2*>(lo);
    } else {
      *reinterpret_cast<float4*>(o + i) = *reinterpret_cast<float4*>(hi);
    }
  }
}

hipError_t launch_rmsnorm(int dtype, const float* x, const void* g, void* out, void* out_lo,
                          int rows, int H, float eps, int block_len, int n_anchor, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(rows), dim3(256), 0, s, x, (const bf16*)g,
                       (bf16*)out, (bf16*)out_lo, H, eps, block_len, n_anchor);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(rows), dim3(256), 0, s, x, (const float*)g,
                       (float*)out, (float*)nullptr, H, eps, block_len, n_anchor);
  return hipGetLastError();
}

}  // namespace dbd
