// Block attention over the cache (DFlare page, section on parallel drafting: attention inside
// the block is bidirectional and the block sees the whole context).  No mask: every row of the
// block attends to all cache positions 0 .. P+B-1 of its sequence (context, then the block's own
// keys, which draft_block wrote into the cache first).
//
// Work item: (key split s, kv head g, sequence n); one wave per 16 query rows of the GQA group
// (rows r = b + B*h over block positions b and the group's heads h).  Per 64-key chunk the K rows
// and V (kept in the cache in blocks of 8 positions, [cap/8][hd][8]) are staged in LDS; each wave computes S^T = K.Q^T with the gfx950 MFMA
// 16x16x32 bf16, so that its lanes hold 8 consecutive keys of one query (keys are permuted inside
// the MFMA tiles), runs the online softmax in fp32 (exp2 domain) and feeds P^T straight from
// registers into O^T += V^T.P^T.  Splits of one (n, g) are merged by attn_combine_kernel.
#include <algorithm>

#include "dbd_internal.h"

namespace dbd {

constexpr int KCH = 64;        // keys per LDS chunk

// ------------------------------------------------------------------ helpers
template <int HD>
__device__ __forceinline__ int kswz(int row, int c) {
  // K tile row = HD*2 bytes.  The S^T operand reads rows {8(i/4) + i%4 (+4)}: spread them over
  // distinct 16-byte slots.
  if constexpr (HD == 128) return c ^ ((row & 3) | (((row >> 3) & 3) << 2));
  else return c ^ (((row >> 1) & 1) | (((row >> 3) & 3) << 1));
}
__device__ __forceinline__ int vswz(int row, int c) { return c ^ ((row >> 1) & 7); }

// NW waves (a power of two, >= the 16-row query tiles of the group); every thread stages
// 2 * KCH * HD * 2 / (64 * NW) bytes of the next chunk in registers while the current chunk is
// consumed from LDS.  QPAIR: the queries come as a bf16 (high, low) pair and every score is the
// sum of two MFMAs, K.Q_hi + K.Q_lo, so the scores see ~16 significant bits of the rotated
// query instead of 8 (the keys stay bf16 as stored in the cache).
template <int HD, int NW, bool QPAIR>
__global__ __launch_bounds__(64 * NW) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KC = HD / 8;                    // 16-byte chunks per K row
  constexpr int NT = 64 * NW;
  constexpr int KT = KCH * KC, VT = HD * (KCH / 8);   // 16-byte chunks of K and V per stage
  constexpr int KI = (KT + NT - 1) / NT;        // K chunks staged per thread
  constexpr int VI = (VT + NT - 1) / NT;        // V chunks staged per thread
  __shared__ __attribute__((aligned(16))) bf16 Ks[KCH * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[HD * KCH];
  // grid.y = kv head + kvh * row block: a group of more than 16 * NW query rows is spread over
  // several workgroups that read the same keys
  const int s = blockIdx.x, g = blockIdx.y % a.kvh, rb = blockIdx.y / a.kvh, n = blockIdx.z;
  const int L = a.seq_keys[n];
  const int k_begin = s * a.split;
  if (L <= 0 || k_begin >= L) return;
  const int k_end = min(L, k_begin + a.split);
  const int nsplit = (L + a.split - 1) / a.split;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.block_len * a.grp;
  const int r0 = rb * 16 * NW;

  const bf16* Kg = (const bf16*)a.kv_k + ((int64_t)n * a.kvh + g) * a.cap * HD;
  // V cache of (n, g): blocks of 8 positions, [cap/8][HD][8]
  const bf16* Vg = (const bf16*)a.kv_v + ((int64_t)n * a.kvh + g) * HD * a.cap;

  // this lane's query row (column of S^T / O^T)
  const int r = r0 + wave * 16 + (lane & 15);
  const bool rvalid = r < R;
  const bool wactive = r0 + wave * 16 < R;      // wave owns at least one query row
  const int b = rvalid ? r % a.block_len : 0, h = rvalid ? r / a.block_len : 0;
  const int64_t qrow = (int64_t)n * a.block_len + b;
  const int qcol = (g * a.grp + h) * HD;
  bf16x8 qf[HD / 32], qlf[QPAIR ? HD / 32 : 1];
  {
    const int64_t qo = qrow * a.qd + qcol + (lane >> 4) * 8;
    const bf16* qp = (const bf16*)a.q + qo;
    const bf16* qlp = QPAIR ? (const bf16*)a.q_lo + qo : nullptr;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
      if (rvalid) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
      else for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.f;
      if constexpr (QPAIR) {
        if (rvalid) qlf[ks] = *reinterpret_cast<const bf16x8*>(qlp + ks * 32);
        else for (int e = 0; e < 8; ++e) qlf[ks][e] = (bf16)0.f;
      }
    }
  }
  f32x4 acc[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // key rows of the two S^T tiles in a 32-key group: lane group G = lane/16 ends up holding
  // keys 8G .. 8G+7
  const int i16 = lane & 15;
  const int kr0 = 8 * (i16 >> 2) + (i16 & 3);
  const int kr1 = kr0 + 4;

  // A 64-key chunk of K ([cap][HD]) and of V ([cap/8][HD][8]) is one contiguous run of
  // KCH * HD * 2 bytes starting c0 * HD * 2 bytes into the (n, g) region, and chunk starts are
  // multiples of 64 inside a capacity that is a multiple of 64: 16-byte piece idx of a chunk
  // sits idx * 16 bytes in.  Buffer loads take that as one per-thread offset plus a uniform
  // one, so staging needs no per-load 64-bit addresses.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(Kg), (short)0, a.cap * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(Vg), (short)0, a.cap * HD * 2, 0x00020000);
  u32x4 kreg[KI], vreg[VI];
  auto load_chunk = [&](int c0) {
    const int base = c0 * HD * 2;
#pragma unroll
    for (int j = 0; j < KI; ++j)
      if (KT % NT == 0 || tid + j * NT < KT)
        kreg[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, tid * 16, base + j * NT * 16, 0);
#pragma unroll
    for (int j = 0; j < VI; ++j)
      if (VT % NT == 0 || tid + j * NT < VT)
        vreg[j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, tid * 16, base + j * NT * 16, 0);
  };
  auto store_chunk = [&](int c0) {
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int idx = tid + j * NT, row = idx / KC, c = idx % KC;
      if (KT % NT == 0 || idx < KT)
        *reinterpret_cast<u32x4*>(Ks + row * HD + kswz<HD>(row, c) * 8) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int idx = tid + j * NT, c = idx / HD, d = idx % HD;
      if (!(VT % NT == 0 || idx < VT)) continue;
      const int k0 = c0 + c * 8;
      u32x4 v = vreg[j];
      if (k0 + 8 > k_end) {               // positions past the end read as 0
        bf16* e = reinterpret_cast<bf16*>(&v);
        for (int q = 0; q < 8; ++q)
          if (k0 + q >= k_end) e[q] = (bf16)0.f;
      }
      *reinterpret_cast<u32x4*>(Vs + d * KCH + vswz(d, c) * 8) = v;
    }
  };

  load_chunk(k_begin);
  for (int c0 = k_begin; c0 < k_end; c0 += KCH) {
    store_chunk(c0);
    __syncthreads();
    if (c0 + KCH < k_end) load_chunk(c0 + KCH);     // in flight while this chunk is consumed
    if (wactive) {
#pragma unroll
      for (int sub = 0; sub < KCH / 32; ++sub) {
        const int key0 = c0 + sub * 32;
        if (key0 < k_end) {
          f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
          const int row0 = sub * 32 + kr0, row1 = sub * 32 + kr1;
#pragma unroll
          for (int ks = 0; ks < HD / 32; ++ks) {
            const int c = ks * 4 + (lane >> 4);
            bf16x8 k0v =
                *reinterpret_cast<const bf16x8*>(Ks + row0 * HD + kswz<HD>(row0, c) * 8);
            bf16x8 k1v =
                *reinterpret_cast<const bf16x8*>(Ks + row1 * HD + kswz<HD>(row1, c) * 8);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0v, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1v, qf[ks], s1, 0, 0, 0);
            if constexpr (QPAIR) {
              s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0v, qlf[ks], s0, 0, 0, 0);
              s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1v, qlf[ks], s1, 0, 0, 0);
            }
          }
          // lane holds S^T[key0 + 8*(lane/16) + e][query], e = 0..7
          float sv[8];
          const int kb = key0 + 8 * (lane >> 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[e] = kb + e < k_end ? s0[e] * a.scale_log2 : -INFINITY;
            sv[4 + e] = kb + 4 + e < k_end ? s1[e] * a.scale_log2 : -INFINITY;
          }
          float mx = sv[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float m_new = fmaxf(m_run, mx);
          const float alpha = exp2f(m_run - m_new);
          bf16x8 pb;
          float ps = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = exp2f(sv[e] - m_new);
            ps += p;
            pb[e] = (bf16)p;
          }
          l_run = l_run * alpha + ps;
          m_run = m_new;
#pragma unroll
          for (int dt = 0; dt < HD / 16; ++dt) {
            acc[dt] *= alpha;
            const int d = dt * 16 + (lane & 15);
            const int c = sub * 4 + (lane >> 4);
            bf16x8 vv = *reinterpret_cast<const bf16x8*>(Vs + d * KCH + vswz(d, c) * 8);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb, acc[dt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
  // per-lane partial sums of the 4 lane groups belong to the same query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!rvalid) return;
  // acc[dt][i] = O^T[d = dt*16 + 4*(lane/16) + i][query]
  if (nsplit == 1) {
    const float inv = 1.f / l_run;
    bf16* o = (bf16*)a.out + qrow * a.qd + qcol;
    bf16* ol = a.out_lo ? (bf16*)a.out_lo + qrow * a.qd + qcol : nullptr;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[dt][i] * inv;
        const bf16 hi = (bf16)y;
        o[dt * 16 + (lane >> 4) * 4 + i] = hi;
        if (ol) ol[dt * 16 + (lane >> 4) * 4 + i] = (bf16)(y - (float)hi);
      }
  } else {
    const int64_t pr = (((int64_t)n * a.kvh + g) * a.s_max + s) * R + r;
    float* po = a.part_o + pr * HD;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
      *reinterpret_cast<f32x4*>(po + dt * 16 + (lane >> 4) * 4) = acc[dt];
    if (lane < 16) a.part_ml[pr] = make_float2(m_run, l_run);
  }
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 attention for the fp32 drafter: one workgroup per (split, kv head, sequence), one
// query row at a time; scores one key per thread, values one dimension per thread.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a, int HD) {
  __shared__ float p[256];
  __shared__ float q[128];
  __shared__ float red[8];
  const int s = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
  const int L = a.seq_keys[n];
  const int k_begin = s * a.split;
  if (L <= 0 || k_begin >= L) return;
  const int k_end = min(L, k_begin + a.split);
  const int nk = k_end - k_begin;
  const int nsplit = (L + a.split - 1) / a.split;
  const int tid = threadIdx.x;
  const int R = a.block_len * a.grp;
  const float* Kg = (const float*)a.kv_k + ((int64_t)n * a.kvh + g) * a.cap * HD;
  const float* Vg = (const float*)a.kv_v + ((int64_t)n * a.kvh + g) * HD * a.cap;
  for (int r = 0; r < R; ++r) {
    const int b = r % a.block_len, h = r / a.block_len;
    const int64_t qrow = (int64_t)n * a.block_len + b;
    const int qcol = (g * a.grp + h) * HD;
    __syncthreads();
    if (tid < HD) q[tid] = ((const float*)a.q)[qrow * a.qd + qcol + tid];
    __syncthreads();
    float sc = -INFINITY;
    if (tid < nk) {
      const float* kr = Kg + (int64_t)(k_begin + tid) * HD;
      float acc = 0.f;
      for (int d = 0; d < HD; ++d) acc += q[d] * kr[d];
      sc = acc * a.scale_log2;
    }
    float m = wave_max(sc);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float e = tid < nk ? exp2f(sc - m) : 0.f;
    p[tid] = e;
    float l = wave_sum(e);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = l;
    __syncthreads();
    l = red[4] + red[5] + red[6] + red[7];
    if (tid < HD) {
      float o = 0.f;
      for (int k = 0; k < nk; ++k) {
        const int kk = k_begin + k;                 // blocks of 8 positions [cap/8][HD][8]
        o += p[k] * Vg[((int64_t)(kk >> 3) * HD + tid) * 8 + (kk & 7)];
      }
      if (nsplit == 1) {
        ((float*)a.out)[qrow * a.qd + qcol + tid] = o / l;
      } else {
        const int64_t pr = (((int64_t)n * a.kvh + g) * a.s_max + s) * R + r;
        a.part_o[pr * HD + tid] = o;
        if (tid == 0) a.part_ml[pr] = make_float2(m, l);
      }
    }
  }
}

// ------------------------------------------------------------------ combine splits
// grid (R / 4, kvh, N): each workgroup merges 4 query rows; thread = (row, 4 dimensions).  All
// partial loads of a thread are independent of each other, so they are in flight together.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a, int HD) {
  const int g = blockIdx.y, n = blockIdx.z;
  const int L = a.seq_keys[n];
  const int nsplit = (L + a.split - 1) / a.split;
  if (L <= 0 || nsplit <= 1) return;
  const int R = a.block_len * a.grp;
  const int dq = HD / 4;                                  // float4 groups per row
  const int r = blockIdx.x * 4 + threadIdx.x / dq;
  const int d4 = threadIdx.x % dq;
  if (r >= R || threadIdx.x >= 4 * dq) return;
  const int64_t base = ((int64_t)n * a.kvh + g) * a.s_max;
  constexpr int SU = 8;
  float m = -INFINITY;
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (nsplit <= SU) {
    // every split's (max, sum) and partial output in one round of loads
    float2 ml[SU];
    f32x4 po[SU];
#pragma unroll
    for (int q = 0; q < SU; ++q) {
      const bool ok = q < nsplit;
      const int64_t pr = (base + q) * R + r;
      ml[q] = ok ? a.part_ml[pr] : make_float2(-INFINITY, 0.f);
      po[q] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + pr * HD + 4 * d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < SU; ++q) m = fmaxf(m, ml[q].x);
#pragma unroll
    for (int q = 0; q < SU; ++q) {
      const float w = exp2f(ml[q].x - m);
      l += w * ml[q].y;
      o += w * po[q];
    }
  } else {
    for (int s0 = 0; s0 < nsplit; s0 += SU) {
      float2 ml[SU];
#pragma unroll
      for (int q = 0; q < SU; ++q)
        ml[q] = s0 + q < nsplit ? a.part_ml[(base + s0 + q) * R + r]
                                : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int q = 0; q < SU; ++q) m = fmaxf(m, ml[q].x);
    }
    for (int s0 = 0; s0 < nsplit; s0 += SU) {
      float2 ml[SU];
      f32x4 po[SU];
#pragma unroll
      for (int q = 0; q < SU; ++q) {
        const bool ok = s0 + q < nsplit;
        const int64_t pr = (base + s0 + q) * R + r;
        ml[q] = ok ? a.part_ml[pr] : make_float2(-INFINITY, 0.f);
        po[q] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + pr * HD + 4 * d4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int q = 0; q < SU; ++q) {
        const float w = exp2f(ml[q].x - m);
        l += w * ml[q].y;
        o += w * po[q];
      }
    }
  }
  const float inv = 1.f / l;
  const int b = r % a.block_len, h = r / a.block_len;
  const int64_t off = ((int64_t)n * a.block_len + b) * a.qd + (g * a.grp + h) * HD + 4 * d4;
  T* out = (T*)a.out + off;
  T* out_lo = a.out_lo ? (T*)a.out_lo + off : nullptr;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float y = o[q] * inv;
    const T hi = from_f<T>(y);
    out[q] = hi;
    if (out_lo) out_lo[q] = from_f<T>(y - to_f(hi));
  }
}

template <int HD, bool QP>
static void launch_bf16_q(const AttnArgs& a, dim3 grid, int nw, hipStream_t s) {
  if (nw <= 2) hipLaunchKernelGGL((attn_bf16_kernel<HD, 2, QP>), grid, dim3(128), 0, s, a);
  else if (nw <= 4) hipLaunchKernelGGL((attn_bf16_kernel<HD, 4, QP>), grid, dim3(256), 0, s, a);
  else if (nw <= 8) hipLaunchKernelGGL((attn_bf16_kernel<HD, 8, QP>), grid, dim3(512), 0, s, a);
  else hipLaunchKernelGGL((attn_bf16_kernel<HD, 16, QP>), grid, dim3(1024), 0, s, a);
}
template <int HD>
static void launch_bf16(const AttnArgs& a, dim3 grid, int nw, hipStream_t s) {
  if (a.q_lo) launch_bf16_q<HD, true>(a, grid, nw, s);
  else launch_bf16_q<HD, false>(a, grid, nw, s);
}

hipError_t launch_attention(int dtype, int hd, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.s_max, a.kvh, a.batch);
  const int R = a.block_len * a.grp;
  dim3 cgrid(ceil_div(R, 4), a.kvh, a.batch);
  if (dtype == 1) {
    // waves per workgroup: at most four (64 query rows) unless overridden; the kernel template
    // takes the next power of two, and the grid's row blocks use the same count
    const int need = ceil_div(R, 16);
    int nw = a.waves > 0 ? std::min(a.waves, need) : std::min(4, need);
    nw = nw <= 2 ? 2 : nw <= 4 ? 4 : nw <= 8 ? 8 : 16;
    grid.y = a.kvh * ceil_div(R, 16 * nw);
    if (hd == 128) launch_bf16<128>(a, grid, nw, s);
    else launch_bf16<64>(a, grid, nw, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(attn_combine_kernel<bf16>, cgrid, dim3(128), 0, s, a, hd);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 0, s, a, hd);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(attn_combine_kernel<float>, cgrid, dim3(128), 0, s, a, hd);
  }
  return hipGetLastError();
}

}  // namespace dbd
