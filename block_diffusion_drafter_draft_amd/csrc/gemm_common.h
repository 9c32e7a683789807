// Shared parts of the projection GEMM kernels (included by k_gemm.hip and k_gemm_deep.hip):
// weight-row addressing for the virtual B operand, the epilogues that consume a finished tile
// (plain store, residual add, Q/K/V with rotation and cache write, context K/V with rotation and
// cache append, SwiGLU, the LM head's per-tile argmax), and the global->LDS DMA helpers.
#pragma once

#include "dbd_internal.h"

namespace dbd {

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

// A 16-byte load through a global (address space 1) pointer.  The weight-row pointers are built
// from integer arithmetic, so the compiler cannot prove them global and would emit a flat load,
// which also counts on lgkmcnt: every wait for an LDS read would then wait for the global
// prefetches as well.
__device__ __forceinline__ u32x4 load_global16(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4*)(p);
}
// the same load marked non-temporal (data read once)
__device__ __forceinline__ u32x4 load_global16_nt(const void* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(p));
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

// cs_pre / pos_pre (Q/K/V only, optional): this thread's rotation factors (CPT of them, for the
// columns it rotates) and, for threads tid < TM, its row's position, loaded by the caller ahead
// of time so that the epilogue does not wait on them.
template <typename T, int TM, int BN, int KIND, int NT = 256>
__device__ __forceinline__ void run_epilogue(const EpiArgs& e, const float* Cs, int m0, int n0,
                                             int tn, int z, int M, int N,
                                             const float2* cs_pre = nullptr,
                                             const int* pos_pre = nullptr) {
  constexpr int CS_LD = BN + 4;                 // fp32 tile row stride in LDS
  constexpr int TPR = NT / TM;                  // threads per tile row
  static_assert(NT % TM == 0 && BN % TPR == 0, "epilogue thread layout");
  constexpr int CPT = BN / TPR;                 // columns per thread
  // SwiGLU stores 8 outputs from 16 columns, the rotations work on 16 columns at a time
  static_assert((KIND != EPI_SWIGLU && KIND != EPI_QKV && KIND != EPI_CTXKV) || CPT % 16 == 0,
                "epilogue columns per thread");
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
      s_pos[tid] = ok ? (pos_pre ? *pos_pre : e.row_pos[mm]) : -1;
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
            cs[q] = cs_pre ? cs_pre[c8 + q] : e.rope[(int64_t)m * half + i];
          }
#pragma unroll
          for (int h8 = 0; h8 < 16; h8 += 8) {
            const int c = cb + c8 + h8;
            if (c >= cols) continue;
            float v[8];
            rope8(crow, c, e.hd, cs + h8, v);
            if (isq) {
              store8<T>((T*)e.q_out + (int64_t)m * e.qd + n0 + c, v);
              if (e.q_out_lo) {
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] -= to_f(from_f<T>(v[q]));
                store8<T>((T*)e.q_out_lo + (int64_t)m * e.qd + n0 + c, v);
              }
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
      constexpr int RPT = TM * BN / NT;      // rows per thread: NT threads cover BN columns
      static_assert(NT % BN == 0, "value-cache epilogue needs BN | NT");
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

// ------------------------------------------------------------------ bf16 MFMA pipeline, deep ring
// Block tile BM x BN (BM 128 or 256), k stages of 32, NS-deep LDS ring, 4 waves in a 2 x 2 grid
// (wave tile BM/2 x BN/2).  Per k stage each wave runs (BM/32) * (BN/32) MFMAs; the fragments of the next stage are
// read from LDS in between those MFMAs, and NS - 1 stages are in flight from global memory while a
// stage is computed.  Stage rows are 64 bytes (4 chunks of 8 bf16), chunk c of row r stored in
// slot swz32-permuted, which keeps both the DMA writes and the fragment reads free of bank
// conflicts.
template <int BM_, int BN, int NS, bool SPLITA>
struct BigCfg {
  static constexpr int BM = BM_, KS = 32;
  static constexpr int NA = SPLITA ? 2 : 1;
  static constexpr int ABYTES = BM * KS * 2, BBYTES = BN * KS * 2;
  static constexpr int STAGE = NA * ABYTES + BBYTES;
  static constexpr int LA = ABYTES / 4096, LB = BBYTES / 4096;   // 1 KB per wave and load
  static constexpr int LPW = NA * LA + LB;                        // loads per wave per stage
  static constexpr int WTM = BM / 2, WTN = BN / 2, MI = WTM / 16, NI = WTN / 16;
  static constexpr int CBYTES = 128 * (BN + 4) * 4;               // epilogue staging
  static constexpr int SMEM = NS * STAGE > CBYTES ? NS * STAGE : CBYTES;
  static_assert(BBYTES % 4096 == 0, "BN must be a multiple of 64");
  static_assert(LPW * (NS - 1) <= 63, "vmcnt range");
};
// 64-byte stage rows (4 chunks of 16 bytes): chunk c of row r sits in slot c ^ ((r >> 1) & 3).
// Measured on gfx950 with the SQ_LDS_BANK_CONFLICT counter: the 16 lanes reading rows 0-15 at
// one chunk (a fragment read) are then conflict-free, while a (r >> 2) & 3 swizzle costs about
// four conflict cycles per ds_read_b128.
__device__ __forceinline__ int swz32(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ void ds_read16(bf16x8& d, uint32_t lds_addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(lds_addr));
}

// s_waitcnt vmcnt(LPW * n) for a run-time n in [0, NS - 1]
template <int LPW, int NS>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (NS > 5) { if (n >= 5) { wait_vmcnt<LPW * 5>(); return; } }
  if constexpr (NS > 4) { if (n >= 4) { wait_vmcnt<LPW * 4>(); return; } }
  if constexpr (NS > 3) { if (n >= 3) { wait_vmcnt<LPW * 3>(); return; } }
  if constexpr (NS > 2) { if (n >= 2) { wait_vmcnt<LPW * 2>(); return; } }
  if (n >= 1) { wait_vmcnt<LPW>(); return; }
  wait_vmcnt<0>();
}

// Work unit -> (m tile, n tile, split): units go to the 8 XCDs round robin; each XCD takes a
// contiguous range of the order (split slowest, then n, then m), so the m tiles of a weight
// column tile run on one XCD close in time, and an XCD reads only its splits' part of the
// activation rows (with split 4 on 512 x 4096 x 12288, one quarter of the 12.6 MB activation
// per XCD instead of all of it: down 0.488 -> 0.482 ms per step, the SpecDiff-2 step 7.02 ->
// 6.95 ms, measured against split fastest).
__device__ __forceinline__ void unit_of(int bid, int total, int tiles_m, int split, int* tm,
                                        int* tn, int* sp) {
  const int q = total >> 3;
  const int t = bid < (q << 3) ? (bid & 7) * q + (bid >> 3) : bid;
  const int tiles = total / split;
  *sp = t / tiles;
  const int tile = t - *sp * tiles;
  *tm = tile % tiles_m;
  *tn = tile / tiles_m;
}

// Deep-ring bf16 kernels (k_gemm_deep.hip): launch configuration `cfg` (8 .. kMaxGemmCfg) of
// epilogue KIND; SPLITA = the A operand comes as a bf16 pair.
template <int KIND, bool SPLITA>
void launch_deep_cfg(int cfg, GemmArgs a, const EpiArgs& e, int batch, hipStream_t s);

}  // namespace dbd
