// Projection GEMMs of the drafter: C = A[M,K] . W[N,K]^T (both operands K-contiguous), with the
// epilogues that consume the tile: plain store, residual add, Q/K/V with rotation and cache
// write, context K/V with rotation and cache append, SwiGLU, and the LM head's per-tile argmax.
//
// bf16 path (gfx950): block tile BM x BN x 64 for 4 waves in a 2 x 2 grid, each wave a
// (BM/2) x (BN/2) grid of 16x16x32 bf16 MFMA tiles with fp32 accumulation.  Tiles move from
// global memory straight into LDS (global_load_lds_dwordx4, no register staging) through an
// ST-stage ring; the 16-byte chunks of each 128-byte tile row are XOR-swizzled by choosing which
// global chunk each lane fetches.  One barrier per k-tile.  Tiles sharing a weight column tile
// are dispatched to the same XCD back to back so the weights come from HBM once.
// fp32 path: 64 x 128 x 16 block tile on the vector ALUs (exact fp32 products and sums).
// Both paths stage the finished tile in LDS as fp32 and run the same epilogue code over it.
#include "dbd_internal.h"

namespace dbd {

constexpr int BK = 64;

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
// Gate/up mode: column tile t of width BN holds gate rows [t*BN/2, (t+1)*BN/2) then the same up
// rows, so the SwiGLU epilogue finds both halves of every output in one tile.
template <typename T, int BN>
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
// The finished tile (or a chunk of TM of its rows) sits in LDS as fp32, row stride BN + 4.  Each thread owns a contiguous
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

template <typename T, int TM, int BN, int KIND>
__device__ __forceinline__ void run_epilogue(const EpiArgs& e, const float* Cs, int m0, int n0,
                                             int tn, int z, int M, int N) {
  constexpr int CS_LD = BN + 4;                 // fp32 tile row stride in LDS
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
      T* dlo = e.act_lo ? (T*)e.act_lo + (int64_t)m * e.F + f0 : nullptr;
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
          if (dlo) {
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] -= to_f(from_f<T>(h[q]));
            store8<T>(dlo + 8 * j, h);
          }
        }
      } else {
        for (int c = 0; c < FPT && f0 + c < e.F; ++c) {
          const float gt = crow[fl + c], up = crow[BN / 2 + fl + c];
          const float h = gt / (1.f + __expf(-gt)) * up;
          dst[c] = from_f<T>(h);
          if (dlo) dlo[c] = from_f<T>(h - to_f(from_f<T>(h)));
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
      // values to the cache, stored in blocks of 8 positions [cap/8][hd][8]: lanes take
      // consecutive dimensions, so one store instruction covers 1 KB of a block
      constexpr int RPT = TM * BN / 256;     // rows per thread: 256 threads cover BN columns
      const int c = tid % BN, rb = (tid / BN) * RPT;
      if (c < cols) {
        const int col = n0 - vbeg + c, g = col / e.hd, d = col % e.hd;
        T* vbase = (T*)e.kv_v + lay + (int64_t)g * e.cap * e.hd + (int64_t)d * 8;
        for (int q = 0; q < RPT; ++q) {
          const int rr = rb + q;
          if (rr >= rows) break;
          const int pos = s_pos[rr];
          if (pos < 0) continue;
          vbase[(int64_t)s_seq[rr] * e.kvh * e.cap * e.hd + (int64_t)(pos >> 3) * e.hd * 8 +
                (pos & 7)] = from_f<T>(Cs[rr * CS_LD + c]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA pipeline
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void lds_dma16(const void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_block, 16,
                                   0, 0);
}
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Linear workgroup id -> (m tile, n tile): workgroups are handed to the 8 XCDs round robin, so
// give each XCD a contiguous range of tiles, m fastest, and the m tiles of one weight column
// tile run on one XCD at about the same time.
__device__ __forceinline__ void tile_of(int bid, int total, int tiles_m, int* tm, int* tn) {
  const int q = total >> 3;
  const int t = bid < (q << 3) ? (bid & 7) * q + (bid >> 3) : bid;
  *tm = t % tiles_m;
  *tn = t / tiles_m;
}

// SPLITA: the A operand is given as two bf16 tensors, A (high part) and A2 = bf16(a - A) (low
// part), and every MFMA is issued for both, so that the product sees A to about 16 significant
// bits (the bf16 pair technique of Henry, Tang & Heinecke, "Leveraging the bfloat16 artificial
// intelligence datatype for higher-precision computations", ARITH 2019).
template <int BM, int BN, int ST, bool SPLITA>
struct PipeCfg {
  static constexpr int NA = SPLITA ? 2 : 1;
  static constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  static constexpr int STAGE = NA * ABYTES + BBYTES;
  static constexpr int LA = BM / 32, LB = BN / 32;     // 1 KB loads per wave per stage
  static constexpr int LPW = NA * LA + LB;
  static constexpr int WTM = BM / 2, WTN = BN / 2;     // wave tile
  static constexpr int MI = WTM / 16, NI = WTN / 16;
  static constexpr int CROWS = (BN == 128 && BM >= 128) ? 128 : 64;   // epilogue row chunk
  static constexpr int CBYTES = CROWS * (BN + 4) * 4;
  static constexpr int SMEM = ST * STAGE > CBYTES ? ST * STAGE : CBYTES;
};

template <int BM, int BN, int ST, int KIND, bool SPLITA>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a, EpiArgs e) {
  using C = PipeCfg<BM, BN, ST, SPLITA>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int M = a.M, N = a.N, K = a.K;
  const int tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Per-lane source of every 1 KB block this wave loads: block j of a tile holds rows
  // 8j .. 8j+7; lane l fills LDS slot (row 8j + l/8, chunk l%8), i.e. it fetches the global
  // chunk (l%8) ^ swz(row) of that row.
  const int rr = lane >> 3, slot = lane & 7;
  const BMap bm = make_bmap(a);
  const bf16* asrc[C::LA];
  const bf16* a2src[C::LA];
  const bf16* bsrc[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int row = (wave + 4 * i) * 8 + rr;
    const int64_t off = (int64_t)z * a.a_bs + (int64_t)min(m0 + row, M - 1) * a.lda +
                        (slot ^ swz(row)) * 8;
    asrc[i] = (const bf16*)a.A + off;
    a2src[i] = SPLITA ? (const bf16*)a.A2 + off : asrc[i];
  }
#pragma unroll
  for (int j = 0; j < C::LB; ++j) {
    const int row = (wave + 4 * j) * 8 + rr;
    bsrc[j] = brow_ptr<bf16, BN>(bm, min(n0 + row, N - 1), z) + (slot ^ swz(row)) * 8;
  }
  auto issue = [&](int st, int kt) {
    char* base = smem + st * C::STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) lds_dma16(asrc[i] + k0, base + (wave + 4 * i) * 1024);
    if constexpr (SPLITA) {
#pragma unroll
      for (int i = 0; i < C::LA; ++i)
        lds_dma16(a2src[i] + k0, base + C::ABYTES + (wave + 4 * i) * 1024);
    }
#pragma unroll
    for (int j = 0; j < C::LB; ++j)
      lds_dma16(bsrc[j] + k0, base + C::NA * C::ABYTES + (wave + 4 * j) * 1024);
  };

  f32x4 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
#pragma unroll
  for (int st = 0; st < ST - 1; ++st)
    if (st < nk) issue(st, st);

  for (int kt = 0; kt < nk; ++kt) {
    // k-tile kt has landed once at most min(ST-2, nk-1-kt) later stages are still in flight
    const int later = min(ST - 2, nk - 1 - kt);
    if (later >= 2) wait_vmcnt<2 * C::LPW>();
    else if (later == 1) wait_vmcnt<C::LPW>();
    else wait_vmcnt<0>();
    block_barrier();
    // the stage computed in the previous iteration is free again: refill it
    if (kt + ST - 1 < nk) issue((kt + ST - 1) % ST, kt + ST - 1);
    const bf16* As = (const bf16*)(smem + (kt % ST) * C::STAGE);
    const bf16* A2s = As + BM * BK;
    const bf16* Bs = As + C::NA * BM * BK;
    // All fragment reads of the stage (both k32 steps) are issued before its MFMAs, into
    // distinct registers, so the wave waits for LDS once per stage rather than once per
    // fragment; the scheduling barrier keeps the compiler from sinking the reads back.
    bf16x8 af[BK / 32][C::MI], bfr[BK / 32][C::NI], af2[SPLITA ? BK / 32 : 1][C::MI];
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int kc = s * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int row = wm * C::WTM + i * 16 + (lane & 15);
        af[s][i] = *reinterpret_cast<const bf16x8*>(As + row * BK + (kc ^ swz(row)) * 8);
        if constexpr (SPLITA)
          af2[s][i] = *reinterpret_cast<const bf16x8*>(A2s + row * BK + (kc ^ swz(row)) * 8);
      }
#pragma unroll
      for (int j = 0; j < C::NI; ++j) {
        const int row = wn * C::WTN + j * 16 + (lane & 15);
        bfr[s][j] = *reinterpret_cast<const bf16x8*>(Bs + row * BK + (kc ^ swz(row)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
      if constexpr (SPLITA) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af2[s][i], bfr[s][j], acc[i][j],
                                                                0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  block_barrier();       // every wave is done reading the ring: reuse it for the output tile

  // accumulators -> fp32 rows in LDS, CROWS rows at a time, then the epilogue on those rows.
  // MFMA 16x16 output: lane holds rows 4*(lane/16)+r, column lane%16 of its tile.
  float* Cs = (float*)smem;
  constexpr int CS_LD = BN + 4;
#pragma unroll
  for (int ch = 0; ch < BM / C::CROWS; ++ch) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int r0 = wm * C::WTM + i * 16;
      if (r0 / C::CROWS != ch) continue;
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 - ch * C::CROWS + (lane >> 4) * 4 + r;
          const int col = wn * C::WTN + j * 16 + (lane & 15);
          Cs[row * CS_LD + col] = acc[i][j][r];
        }
    }
    __syncthreads();
    run_epilogue<bf16, C::CROWS, BN, KIND>(e, Cs, m0 + ch * C::CROWS, n0, tn, z, M, N);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ fp32 mainloop
constexpr int FK = 16;
constexpr int FM = 64, FN = 128;               // fp32 path block tile
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, EpiArgs e) {
  constexpr int BN = FN, CS_LD = FN + 4;
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
      if (n0 + r < N && k0 + k < K) v = brow_ptr<float, FN>(bm, n0 + r, z)[k0 + k];
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
  run_epilogue<float, FM, FN, KIND>(e, Cs, m0, n0, tn, z, M, N);
}

// ------------------------------------------------------------------ launch
// Block tile configurations of the bf16 path: (BM, BN, pipeline stages).
constexpr int kNumCfg = 8;
static const int kCfgBM[kNumCfg] = {256, 256, 128, 64, 128, 64, 256, 128};
static const int kCfgBN[kNumCfg] = {256, 128, 128, 128, 128, 128, 128, 256};

// Choose the largest tile that still gives every CU work in whole rounds: a tile count of at
// least two per CU, else the configuration with the most tiles.
static int choose_cfg(int M, int N, int batch, int gateup, int F) {
  static const int order[4] = {0, 1, 4, 5};
  int best = 5, best_tiles = 0;
  for (int c : order) {
    const int n = gateup ? ceil_div(F, kCfgBN[c] / 2) * kCfgBN[c] : N;
    const int tiles = ceil_div(M, kCfgBM[c]) * ceil_div(n, kCfgBN[c]) * batch;
    if (tiles >= 512) return c;
    if (tiles > best_tiles) { best = c; best_tiles = tiles; }
  }
  return best;
}

template <int BM, int BN, int ST, int KIND, bool SPLITA>
static void launch_pipe(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, BN / 2) * BN;
  const int tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, ST, KIND, SPLITA>), dim3(tiles, 1, batch),
                     dim3(256), 0, s, a, e);
}

template <int KIND, bool SPLITA>
static void launch_cfg(int cfg, const GemmArgs& a, const EpiArgs& e, int batch, hipStream_t s) {
  if constexpr (SPLITA) {
    // the A2 stages double the A part of the ring: only the smaller tiles fit in LDS
    if (cfg == 3 || cfg == 5) launch_pipe<64, 128, 3, KIND, true>(a, e, batch, s);
    else launch_pipe<128, 128, 2, KIND, true>(a, e, batch, s);
  } else {
    switch (cfg) {
      case 0: launch_pipe<256, 256, 2, KIND, false>(a, e, batch, s); break;
      case 1: launch_pipe<256, 128, 3, KIND, false>(a, e, batch, s); break;
      case 2: launch_pipe<128, 128, 3, KIND, false>(a, e, batch, s); break;
      case 3: launch_pipe<64, 128, 4, KIND, false>(a, e, batch, s); break;
      case 4: launch_pipe<128, 128, 2, KIND, false>(a, e, batch, s); break;
      case 5: launch_pipe<64, 128, 3, KIND, false>(a, e, batch, s); break;
      case 6: launch_pipe<256, 128, 2, KIND, false>(a, e, batch, s); break;
      default: launch_pipe<128, 256, 2, KIND, false>(a, e, batch, s); break;
    }
  }
}

// The bf16 configuration a launch really uses: the requested one (or the shape's choice), with
// QKV / context K/V tiles kept at 128 columns (they must not straddle the Q/K/V segment
// boundaries, multiples of 128) and bf16-pair launches on the tiles whose ring fits in LDS.
static int resolve_cfg(int kind, int cfg, int M, int N, int batch, int gateup, int F,
                       bool split) {
  if (cfg < 0 || cfg >= kNumCfg) cfg = choose_cfg(M, N, batch, gateup, F);
  if ((kind == EPI_QKV || kind == EPI_CTXKV) && kCfgBN[cfg] != 128)
    cfg = kCfgBM[cfg] == 256 ? 1 : 4;
  if (split) cfg = (cfg == 3 || cfg == 5) ? 5 : 4;
  return cfg;
}

template <int KIND>
static void launch_kind(int dtype, int cfg, GemmArgs a, const EpiArgs& e, int batch,
                        hipStream_t s) {
  if (dtype == 1) {
    const int F = a.seg[0].n1 - a.seg[0].n0;
    cfg = resolve_cfg(KIND, cfg, a.M, a.N, batch, a.gateup, F, a.A2 != nullptr);
    if (a.A2) launch_cfg<KIND, true>(cfg, a, e, batch, s);
    else launch_cfg<KIND, false>(cfg, a, e, batch, s);
  } else {
    if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, FN / 2) * FN;
    dim3 grid(ceil_div(a.N, FN), ceil_div(a.M, FM), batch);
    hipLaunchKernelGGL(gemm_f32_kernel<KIND>, grid, dim3(256), 0, s, a, e);
  }
}

int gemm_ntiles(int dtype, int kind, int cfg, int M, int N, int batch, bool split) {
  if (dtype != 1) return ceil_div(N, FN);
  return ceil_div(N, kCfgBN[resolve_cfg(kind, cfg, M, N, batch, 0, 0, split)]);
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, const EpiArgs& e, int batch,
                       hipStream_t s, int cfg) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  switch (e.kind) {
    case EPI_STORE_F32: launch_kind<EPI_STORE_F32>(dtype, cfg, a, e, batch, s); break;
    case EPI_RESID: launch_kind<EPI_RESID>(dtype, cfg, a, e, batch, s); break;
    case EPI_QKV: launch_kind<EPI_QKV>(dtype, cfg, a, e, batch, s); break;
    case EPI_CTXKV: launch_kind<EPI_CTXKV>(dtype, cfg, a, e, batch, s); break;
    case EPI_SWIGLU: launch_kind<EPI_SWIGLU>(dtype, cfg, a, e, batch, s); break;
    case EPI_ARGMAX: launch_kind<EPI_ARGMAX>(dtype, cfg, a, e, batch, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dbd
