// Projection GEMMs of the drafter: C = A[M,K] . W[N,K]^T (both operands K-contiguous), with the
// epilogues that consume the tile: plain store, residual add, Q/K/V with rotation and cache
// write, context K/V with rotation and cache append, SwiGLU, and the LM head's per-tile argmax.
//
// bf16 path: 128x128x64 block tile, 4 waves (2x2), each wave 64x64 = 4x4 tiles of the gfx950
// MFMA 16x16x32 bf16 instruction, fp32 accumulation, double-buffered LDS with an XOR swizzle of
// the 16-byte chunks, global loads for tile k+1 issued before the MFMAs of tile k.
// fp32 path: 64x128x16 block tile on the vector ALUs (exact fp32 products and sums).
// Both paths stage the finished tile in LDS as fp32 and run the same epilogue code over it.
#include "dbd_internal.h"

namespace dbd {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int CS_LD = BN + 4;                  // fp32 tile row stride in LDS
constexpr int FM = 64;                         // fp32 path block rows

// ------------------------------------------------------------------ B row addressing
// Virtual column v (< N) -> pointer to the K-contiguous weight row that produces it.  The
// segment base addresses are combined with integer arithmetic: a conditional choice between
// members of the by-value argument struct is turned by the compiler into a load through a
// selected address, which places the whole struct in private (scratch) memory.
struct BMap {
  uint64_t p0, d1, d2;   // base of segment 0, and offsets of segments 1, 2 from it (bytes)
  int n1, n2, nseg, gateup, F;
  int64_t ldb, b_bs;
};
__device__ __forceinline__ BMap make_bmap(const GemmArgs& a) {
  BMap m;
  m.p0 = (uint64_t)a.seg[0].ptr;
  m.d1 = (uint64_t)a.seg[1].ptr - m.p0;
  m.d2 = (uint64_t)a.seg[2].ptr - m.p0;
  m.n1 = a.seg[1].n0;
  m.n2 = a.seg[2].n0;
  m.nseg = a.nseg;
  m.gateup = a.gateup;
  m.F = a.seg[0].n1 - a.seg[0].n0;
  m.ldb = a.ldb;
  m.b_bs = a.b_bs;
  return m;
}
template <typename T>
__device__ __forceinline__ const T* brow_ptr(const BMap& m, int v, int z) {
  uint64_t s1, s2;
  int r;
  if (m.gateup) {
    const int t = v / BN, c = v % BN;
    const int f = t * (BN / 2) + (c % (BN / 2));
    r = f < m.F ? f : m.F - 1;
    s1 = c >= BN / 2;
    s2 = 0;
  } else {
    s2 = (m.nseg > 2 && v >= m.n2) ? 1 : 0;
    s1 = (!s2 && m.nseg > 1 && v >= m.n1) ? 1 : 0;
    r = v - (int)(s2 * m.n2 + s1 * m.n1);
  }
  const uint64_t base = m.p0 + s1 * m.d1 + s2 * m.d2;
  return (const T*)base + (int64_t)z * m.b_bs + (int64_t)r * m.ldb;
}

// ------------------------------------------------------------------ epilogues
// The finished tile sits in LDS as fp32 (row stride CS_LD).  Each thread owns a contiguous
// segment of one row (TPR threads per row, CPT columns each), issues all of its global loads
// before any store (a store could alias a later load, so the compiler cannot hoist loads across
// it), and stores 16-byte vectors where the layout is contiguous.
template <typename T>
__device__ __forceinline__ void store8(T* dst, const float* v) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(dst) = o;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// rotate-half RoPE of tile row `row` (LDS) at tile columns c .. c+7 (same head, same half);
// cs = the 8 (cos, sin) pairs of the head-local pair indices of those columns.
__device__ __forceinline__ void rope8(const float* row, int c, int hd, const float2* cs,
                                      float* out) {
  const int half = hd / 2, d = c % hd;
  if (d < half) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = row[c + e] * cs[e].x - row[c + e + half] * cs[e].y;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = row[c + e] * cs[e].x + row[c + e - half] * cs[e].y;
  }
}

template <typename T, int TM, int KIND>
__device__ __forceinline__ void run_epilogue(const EpiArgs& e, const float* Cs, int m0, int n0,
                                             int tn, int z, int M, int N) {
  constexpr int TPR = 256 / TM;                 // threads per tile row
  constexpr int CPT = BN / TPR;                 // columns per thread
  __shared__ int s_pos[TM], s_seq[TM];
  const int tid = threadIdx.x;
  const int rows = min(TM, M - m0);
  const int cols = min(BN, N - n0);
  const int r = tid / TPR, cb = (tid % TPR) * CPT;
  const int m = m0 + r;
  const bool rok = r < rows;
  const float* crow = Cs + r * CS_LD;

  if constexpr (KIND == EPI_STORE_F32 || KIND == EPI_RESID || KIND == EPI_ARGMAX) {
    float* C = KIND == EPI_ARGMAX ? e.logits : (float*)e.C + (int64_t)z * e.c_bs;
    if (C && rok) {
      float* dst = C + (int64_t)m * e.ldc + n0 + cb;
      const bool vec = (e.ldc & 3) == 0 && cb + CPT <= cols && ((uintptr_t)dst & 15) == 0;
      if (vec) {
        f32x4 v[CPT / 4];
        if constexpr (KIND == EPI_RESID) {
#pragma unroll
          for (int j = 0; j < CPT / 4; ++j) v[j] = *reinterpret_cast<const f32x4*>(dst + 4 * j);
        }
#pragma unroll
        for (int j = 0; j < CPT / 4; ++j) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(crow + cb + 4 * j);
          if constexpr (KIND == EPI_RESID) v[j] += a;
          else v[j] = a;
        }
#pragma unroll
        for (int j = 0; j < CPT / 4; ++j) *reinterpret_cast<f32x4*>(dst + 4 * j) = v[j];
      } else {
        for (int c = 0; c < CPT && cb + c < cols; ++c) {
          if constexpr (KIND == EPI_RESID) dst[c] += crow[cb + c];
          else dst[c] = crow[cb + c];
        }
      }
    }
    if constexpr (KIND == EPI_ARGMAX) {
      // TPR threads per row each scan their columns in increasing order, then combine
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      if (rok)
        for (int c = cb; c < cb + CPT && c < cols; ++c) argmax_combine(bv, bi, crow[c], n0 + c);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        argmax_combine(bv, bi, ov, oi);
      }
      if (rok && (tid % TPR) == 0) {
        e.part_val[(int64_t)m * e.ntiles + tn] = bv;
        e.part_idx[(int64_t)m * e.ntiles + tn] = bi;
      }
    }
  } else if constexpr (KIND == EPI_SWIGLU) {
    // tile columns [0, BN/2) are gate, [BN/2, BN) up, for f = tn*BN/2 + c
    constexpr int FPT = CPT / 2;
    const int f0 = tn * (BN / 2) + (tid % TPR) * FPT;
    const int fl = (tid % TPR) * FPT;
    if (rok) {
      T* dst = (T*)e.act + (int64_t)m * e.F + f0;
      if (f0 + FPT <= e.F && (e.F & 7) == 0) {
#pragma unroll
        for (int j = 0; j < FPT / 8; ++j) {
          float h[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float gt = crow[fl + 8 * j + q], up = crow[BN / 2 + fl + 8 * j + q];
            h[q] = gt / (1.f + __expf(-gt)) * up;
          }
          store8<T>(dst + 8 * j, h);
        }
      } else {
        for (int c = 0; c < FPT && f0 + c < e.F; ++c) {
          const float gt = crow[fl + c], up = crow[BN / 2 + fl + c];
          dst[c] = from_f<T>(gt / (1.f + __expf(-gt)) * up);
        }
      }
    }
  } else {
    // EPI_QKV (block rows) and EPI_CTXKV (ingest rows): row metadata staged in LDS once
    const bool ctx = KIND == EPI_CTXKV;
    if (tid < TM) {
      const int mm = m0 + tid;
      const bool ok = tid < rows;
      s_pos[tid] = ok ? e.row_pos[mm] : -1;
      s_seq[tid] = ok ? (ctx ? e.row_seq[mm] : mm / e.block_len) : -1;
    }
    __syncthreads();
    const int64_t lay = ctx ? (int64_t)z * e.layer_stride : e.layer_off_k;
    const int kbeg = ctx ? 0 : e.qd;                    // first virtual column of K
    const int vbeg = kbeg + e.kd;                       // first virtual column of V
    const int half = e.hd / 2;
    if (n0 < vbeg) {
      // queries or keys: rotate, then store rows of 8
      const bool isq = n0 < kbeg;
      const int pos = rok ? s_pos[r] : -1;
      const int n = rok ? s_seq[r] : 0;
      if (rok && (isq || pos >= 0)) {
#pragma unroll
        for (int c8 = 0; c8 < CPT; c8 += 16) {
          float2 cs[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int i = ((cb + c8 + q) % e.hd) % half;
            cs[q] = e.rope[(int64_t)m * half + i];
          }
#pragma unroll
          for (int h8 = 0; h8 < 16; h8 += 8) {
            const int c = cb + c8 + h8;
            if (c >= cols) continue;
            float v[8];
            rope8(crow, c, e.hd, cs + h8, v);
            if (isq) {
              store8<T>((T*)e.q_out + (int64_t)m * e.qd + n0 + c, v);
            } else {
              const int col = n0 - kbeg + c, g = col / e.hd, d = col % e.hd;
              store8<T>((T*)e.kv_k + lay + (((int64_t)n * e.kvh + g) * e.cap + pos) * e.hd + d,
                        v);
            }
          }
        }
      }
    } else {
      // values to the position-minor cache: thread = one column, a run of rows
      constexpr int RPT = TM * BN / 256;     // rows per thread: 256 threads cover BN columns
      const int c = tid % BN, rb = (tid / BN) * RPT;
      if (c < cols) {
        const int col = n0 - vbeg + c, g = col / e.hd, d = col % e.hd;
        T* vbase = (T*)e.kv_v + lay + (int64_t)g * e.hd * e.cap + (int64_t)d * e.cap;
        for (int q = 0; q < RPT; ++q) {
          const int rr = rb + q;
          if (rr >= rows) break;
          const int pos = s_pos[rr];
          if (pos < 0) continue;
          vbase[(int64_t)s_seq[rr] * e.kvh * e.hd * e.cap + pos] = from_f<T>(Cs[rr * CS_LD + c]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA mainloop
__device__ __forceinline__ int swz(int row, int kc) { return kc ^ ((row >> 1) & 7); }

// SPLITA: the A operand is given as two bf16 tensors, A (high part) and A2 = bf16(a - A) (low
// part), and every MFMA is issued for both, so that the product sees A to about 16 significant
// bits (the bf16 pair technique of Henry, Tang & Heinecke, "Leveraging the bfloat16 artificial
// intelligence datatype for higher-precision computations", ARITH 2019).
template <bool SPLITA>
constexpr int gemm_smem_bytes() {
  return SPLITA ? 3 * 2 * BM * BK * 2 : BM * CS_LD * 4;
}

template <int KIND, bool SPLITA>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a, EpiArgs e) {
  // LDS: two stages of the A (and A2) and B tiles, reused as the fp32 output tile (66 KB)
  __shared__ __attribute__((aligned(16))) char smem[gemm_smem_bytes<SPLITA>()];
  bf16* As = (bf16*)smem;                                   // [2][BM][BK]
  bf16* Bs = (bf16*)(smem + 2 * BM * BK * 2);              // [2][BN][BK]
  bf16* A2s = (bf16*)(smem + 4 * BM * BK * 2);             // [2][BM][BK] (SPLITA)
  float* Cs = (float*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = a.M, N = a.N, K = a.K;

  const BMap bm = make_bmap(a);
  const bf16* ap[4];
  const bf16* ap2[4];
  const bf16* bp[4];
  int so[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i, row = id >> 3, kc = id & 7;
    const int ar = min(m0 + row, M - 1);
    const int64_t aoff = (int64_t)z * a.a_bs + (int64_t)ar * a.lda + kc * 8;
    ap[i] = (const bf16*)a.A + aoff;
    ap2[i] = SPLITA ? (const bf16*)a.A2 + aoff : ap[i];
    bp[i] = brow_ptr<bf16>(bm, min(n0 + row, N - 1), z) + kc * 8;
    so[i] = row * BK + swz(row, kc) * 8;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4], ra2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const u32x4*>(ap[i]);
    rb[i] = *reinterpret_cast<const u32x4*>(bp[i]);
    if constexpr (SPLITA) ra2[i] = *reinterpret_cast<const u32x4*>(ap2[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<u32x4*>(As + so[i]) = ra[i];
    *reinterpret_cast<u32x4*>(Bs + so[i]) = rb[i];
    if constexpr (SPLITA) *reinterpret_cast<u32x4*>(A2s + so[i]) = ra2[i];
  }
  __syncthreads();

  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + koff);
        rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + koff);
        if constexpr (SPLITA) ra2[i] = *reinterpret_cast<const u32x4*>(ap2[i] + koff);
      }
    }
    const bf16* Ac = As + cur * BM * BK;
    const bf16* A2c = A2s + cur * BM * BK;
    const bf16* Bc = Bs + cur * BN * BK;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      bf16x8 af[4], bfr[4];
      const int kc = s * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_ = wm * 64 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8*>(Ac + ra_ * BK + swz(ra_, kc) * 8);
        const int rb_ = wn * 64 + i * 16 + (lane & 15);
        bfr[i] = *reinterpret_cast<const bf16x8*>(Bc + rb_ * BK + swz(rb_, kc) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      if constexpr (SPLITA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ra_ = wm * 64 + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const bf16x8*>(A2c + ra_ * BK + swz(ra_, kc) * 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) {
      bf16* An = As + (cur ^ 1) * BM * BK;
      bf16* Bn = Bs + (cur ^ 1) * BN * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(An + so[i]) = ra[i];
        *reinterpret_cast<u32x4*>(Bn + so[i]) = rb[i];
        if constexpr (SPLITA)
          *reinterpret_cast<u32x4*>(A2s + (cur ^ 1) * BM * BK + so[i]) = ra2[i];
      }
    }
    __syncthreads();
  }

  // accumulators -> fp32 tile in LDS.  MFMA 16x16 output: lane holds rows 4*(lane/16)+r, col
  // lane%16.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        const int col = wn * 64 + j * 16 + (lane & 15);
        Cs[row * CS_LD + col] = acc[i][j][r];
      }
  __syncthreads();
  run_epilogue<bf16, BM, KIND>(e, Cs, m0, n0, tn, z, M, N);
}

// ------------------------------------------------------------------ fp32 mainloop
constexpr int FK = 16;
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) float smem[FM * CS_LD];
  float* As = smem;                      // [FK][FM]
  float* Bs = smem + FK * FM;            // [FK][BN]
  float* Cs = smem;
  const int tid = threadIdx.x;
  const int z = blockIdx.z;
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int m0 = tm * FM, n0 = tn * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int ty = tid >> 4, tx = tid & 15;   // 16 x 16 threads, each 4 rows x 8 cols
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  const float* A = (const float*)a.A + (int64_t)z * a.a_bs;
  const BMap bm = make_bmap(a);
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int idx = tid; idx < FM * FK; idx += 256) {
      const int r = idx / FK, k = idx % FK;
      float v = 0.f;
      if (m0 + r < M && k0 + k < K) v = A[(int64_t)(m0 + r) * a.lda + k0 + k];
      As[k * FM + r] = v;
    }
    for (int idx = tid; idx < BN * FK; idx += 256) {
      const int r = idx / FK, k = idx % FK;
      float v = 0.f;
      if (n0 + r < N && k0 + k < K) v = brow_ptr<float>(bm, n0 + r, z)[k0 + k];
      Bs[k * BN + r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float av[4], bv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k * FM + ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = Bs[k * BN + tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) Cs[(ty * 4 + i) * CS_LD + tx + 16 * j] = acc[i][j];
  __syncthreads();
  run_epilogue<float, FM, KIND>(e, Cs, m0, n0, tn, z, M, N);
}

template <int KIND>
static void launch_kind(int dtype, const GemmArgs& a, const EpiArgs& e, int batch,
                        hipStream_t s) {
  if (dtype == 1) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM), batch);
    bool split = false;
    if constexpr (KIND == EPI_CTXKV) split = a.A2 != nullptr;   // only the context K/V GEMM
    if constexpr (KIND == EPI_CTXKV) {
      if (split) {
        hipLaunchKernelGGL((gemm_bf16_kernel<KIND, true>), grid, dim3(256), 0, s, a, e);
        return;
      }
    }
    hipLaunchKernelGGL((gemm_bf16_kernel<KIND, false>), grid, dim3(256), 0, s, a, e);
  } else {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, FM), batch);
    hipLaunchKernelGGL(gemm_f32_kernel<KIND>, grid, dim3(256), 0, s, a, e);
  }
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, const EpiArgs& e, int batch,
                       hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  switch (e.kind) {
    case EPI_STORE_F32: launch_kind<EPI_STORE_F32>(dtype, a, e, batch, s); break;
    case EPI_RESID: launch_kind<EPI_RESID>(dtype, a, e, batch, s); break;
    case EPI_QKV: launch_kind<EPI_QKV>(dtype, a, e, batch, s); break;
    case EPI_CTXKV: launch_kind<EPI_CTXKV>(dtype, a, e, batch, s); break;
    case EPI_SWIGLU: launch_kind<EPI_SWIGLU>(dtype, a, e, batch, s); break;
    case EPI_ARGMAX: launch_kind<EPI_ARGMAX>(dtype, a, e, batch, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dbd
