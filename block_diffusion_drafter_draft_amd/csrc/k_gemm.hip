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
template <typename T>
__device__ __forceinline__ float rot(const float* row, int c, int hd, float2 cs) {
  // rotate-half: pair (i, i + hd/2) of the head that column c belongs to
  const int d = c % hd, base = c - d, half = hd / 2, i = d % half;
  const float x1 = row[base + i], x2 = row[base + i + half];
  return d < half ? x1 * cs.x - x2 * cs.y : x2 * cs.x + x1 * cs.y;
}

template <typename T, int TM, int KIND>
__device__ __forceinline__ void run_epilogue(const EpiArgs& e, const float* Cs, int m0, int n0,
                                             int tn, int z, int M, int N) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int rows = min(TM, M - m0);
  const int cols = min(BN, N - n0);
  switch (KIND) {
    case EPI_STORE_F32: {
      float* C = (float*)e.C + (int64_t)z * e.c_bs;
      for (int idx = tid; idx < TM * BN; idx += nthr) {
        const int r = idx / BN, c = idx % BN;
        if (r < rows && c < cols) C[(int64_t)(m0 + r) * e.ldc + n0 + c] = Cs[r * CS_LD + c];
      }
      break;
    }
    case EPI_RESID: {
      float* C = (float*)e.C;
      for (int idx = tid; idx < TM * BN; idx += nthr) {
        const int r = idx / BN, c = idx % BN;
        if (r < rows && c < cols) C[(int64_t)(m0 + r) * e.ldc + n0 + c] += Cs[r * CS_LD + c];
      }
      break;
    }
    case EPI_QKV: {
      const int half = e.hd / 2;
      if (n0 < e.qd + e.kd) {
        // queries (rotated) to q_out, or block keys (rotated) to the cache rows of the block
        const bool isq = n0 < e.qd;
        for (int idx = tid; idx < TM * BN; idx += nthr) {
          const int r = idx / BN, c = idx % BN;
          if (r >= rows || c >= cols) continue;
          const int m = m0 + r;
          const int pos = e.row_pos[m];
          const int i = (c % e.hd) % half;
          const float v = rot<T>(Cs + r * CS_LD, c, e.hd, e.rope[(int64_t)m * half + i]);
          if (isq) {
            ((T*)e.q_out)[(int64_t)m * e.qd + n0 + c] = from_f<T>(v);
          } else if (pos >= 0) {
            const int col = n0 - e.qd + c, g = col / e.hd, d = col % e.hd;
            const int n = m / e.block_len;
            const int64_t off = e.layer_off_k +
                                (((int64_t)n * e.kvh + g) * e.cap + pos) * e.hd + d;
            ((T*)e.kv_k)[off] = from_f<T>(v);
          }
        }
      } else {
        // block values to the transposed cache: consecutive threads walk positions
        for (int idx = tid; idx < TM * BN; idx += nthr) {
          const int c = idx / TM, r = idx % TM;
          if (r >= rows || c >= cols) continue;
          const int m = m0 + r;
          const int pos = e.row_pos[m];
          if (pos < 0) continue;
          const int col = n0 - e.qd - e.kd + c, g = col / e.hd, d = col % e.hd;
          const int n = m / e.block_len;
          const int64_t off = e.layer_off_k +
                              (((int64_t)n * e.kvh + g) * e.hd + d) * e.cap + pos;
          ((T*)e.kv_v)[off] = from_f<T>(Cs[r * CS_LD + c]);
        }
      }
      break;
    }
    case EPI_CTXKV: {
      const int half = e.hd / 2;
      const int64_t lay = (int64_t)z * e.layer_stride;
      if (n0 < e.kd) {
        for (int idx = tid; idx < TM * BN; idx += nthr) {
          const int r = idx / BN, c = idx % BN;
          if (r >= rows || c >= cols) continue;
          const int t = m0 + r;
          const int pos = e.row_pos[t];
          if (pos < 0) continue;
          const int n = e.row_seq[t];
          const int i = (c % e.hd) % half;
          const float v = rot<T>(Cs + r * CS_LD, c, e.hd, e.rope[(int64_t)t * half + i]);
          const int col = n0 + c, g = col / e.hd, d = col % e.hd;
          ((T*)e.kv_k)[lay + (((int64_t)n * e.kvh + g) * e.cap + pos) * e.hd + d] = from_f<T>(v);
        }
      } else {
        for (int idx = tid; idx < TM * BN; idx += nthr) {
          const int c = idx / TM, r = idx % TM;
          if (r >= rows || c >= cols) continue;
          const int t = m0 + r;
          const int pos = e.row_pos[t];
          if (pos < 0) continue;
          const int n = e.row_seq[t];
          const int col = n0 - e.kd + c, g = col / e.hd, d = col % e.hd;
          ((T*)e.kv_v)[lay + (((int64_t)n * e.kvh + g) * e.hd + d) * e.cap + pos] =
              from_f<T>(Cs[r * CS_LD + c]);
        }
      }
      break;
    }
    case EPI_SWIGLU: {
      const int f0 = tn * (BN / 2);
      for (int idx = tid; idx < TM * (BN / 2); idx += nthr) {
        const int r = idx / (BN / 2), c = idx % (BN / 2);
        if (r >= rows || f0 + c >= e.F) continue;
        const float gt = Cs[r * CS_LD + c], up = Cs[r * CS_LD + BN / 2 + c];
        const float h = gt / (1.f + __expf(-gt)) * up;
        ((T*)e.act)[(int64_t)(m0 + r) * e.F + f0 + c] = from_f<T>(h);
      }
      break;
    }
    case EPI_ARGMAX: {
      if (e.logits) {
        for (int idx = tid; idx < TM * BN; idx += nthr) {
          const int r = idx / BN, c = idx % BN;
          if (r < rows && c < cols)
            e.logits[(int64_t)(m0 + r) * e.ldc + n0 + c] = Cs[r * CS_LD + c];
        }
      }
      // 2 threads per row, each scans half of the tile's columns in increasing order
      for (int pr = tid; pr < TM * 2; pr += nthr) {
        const int r = pr >> 1, h = pr & 1;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        if (r < rows) {
          for (int c = h * (BN / 2); c < (h + 1) * (BN / 2) && c < cols; ++c)
            argmax_combine(bv, bi, Cs[r * CS_LD + c], n0 + c);
        }
        const float ov = __shfl_xor(bv, 1, 64);
        const int oi = __shfl_xor(bi, 1, 64);
        argmax_combine(bv, bi, ov, oi);
        if (h == 0 && r < rows) {
          e.part_val[(int64_t)(m0 + r) * e.ntiles + tn] = bv;
          e.part_idx[(int64_t)(m0 + r) * e.ntiles + tn] = bi;
        }
      }
      break;
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
