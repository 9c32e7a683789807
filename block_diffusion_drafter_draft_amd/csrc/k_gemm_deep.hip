// Deep-ring bf16 GEMM (gfx950): block tile BM x BN, k stages of 32 bf16, an NS-deep LDS ring
// filled by global->LDS DMA, 4 waves in a 2 x 2 grid, 16x16x32 bf16 MFMAs with fp32
// accumulation, optional split-K over several workgroups.  This translation unit is compiled
// with the MFMA accumulators in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form): the tiles here
// fit in the 256 architectural VGPRs, and the accumulator form keeps the software-pipelined
// loop free of accumulator copies.
#include "gemm_common.h"

namespace dbd {

template <int BM_, int BN, int NS, int KIND, bool SPLITA>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs a, EpiArgs e) {
  using C = BigCfg<BM_, BN, NS, SPLITA>;
  constexpr int BM = C::BM;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int M = a.M, N = a.N, K = a.K;
  const int S = a.split > 1 ? a.split : 1;
  const int tiles_m = (M + BM - 1) / BM;
  int tm, tn, sp;
  unit_of(blockIdx.x, gridDim.x, tiles_m, S, &tm, &tn, &sp);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk_all = K / C::KS;
  const int kb = (int)((int64_t)nk_all * sp / S), nk = (int)((int64_t)nk_all * (sp + 1) / S) - kb;

  // Per-lane source of each 1 KB load: load j of a tile covers rows 16j .. 16j+15; lane l fills
  // LDS slot (row 16j + l/4, chunk l%4) from global chunk (l%4) ^ swz32(row).
  const int rr = lane >> 2, slot = lane & 3;
  const BMap bm = make_bmap(a);
  const bf16* asrc[C::LA];
  const bf16* a2src[C::LA];
  const bf16* bsrc[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int row = (wave + 4 * i) * 16 + rr;
    const int64_t off = (int64_t)z * a.a_bs + (int64_t)min(m0 + row, M - 1) * a.lda +
                        kb * C::KS + (slot ^ swz32(row)) * 8;
    asrc[i] = (const bf16*)a.A + off;
    a2src[i] = SPLITA ? (const bf16*)a.A2 + off : asrc[i];
  }
#pragma unroll
  for (int j = 0; j < C::LB; ++j) {
    const int row = (wave + 4 * j) * 16 + rr;
    bsrc[j] = brow_ptr<bf16, BN>(bm, min(n0 + row, N - 1), z) + kb * C::KS +
              (slot ^ swz32(row)) * 8;
  }

  // Fragment reads.  Lane l reads row (l%16) of each 16-row group at chunk l/16.  The reads are
  // issued as inline ds_read_b128: a compiled LDS load after a global->LDS DMA makes the compiler
  // wait for every DMA in flight (it cannot tell the ring slots apart), which would drain the
  // ring each stage.  The kernel waits for the reads itself (lgkmcnt) and ties the fragment
  // registers to that wait, so no MFMA can be scheduled before it.
  const int fr = lane & 15, fk = lane >> 4;
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem +
      (uint32_t)((fr * C::KS + ((fk ^ swz32(fr)) * 8)) * 2);
  const uint32_t a_off = (uint32_t)(wm * C::WTM * C::KS * 2);
  const uint32_t b_off = (uint32_t)((C::NA * BM * C::KS + wn * C::WTN * C::KS) * 2);
  struct Frag {
    bf16x8 a[C::MI], a2[SPLITA ? C::MI : 1], b[C::NI];
  };
  constexpr int NRD = C::MI * (SPLITA ? 2 : 1) + C::NI;     // reads per stage
  // read r of the stage at LDS byte address `base`: A fragments, then A2, then B
  auto read_one = [&](Frag& f, uint32_t base, int r) __attribute__((always_inline)) {
    if (r < C::MI) {
      ds_read16(f.a[r], base + a_off + (uint32_t)(r * 16 * C::KS * 2));
    } else if (r < C::NA * C::MI) {
      if constexpr (SPLITA)
        ds_read16(f.a2[r - C::MI], base + a_off + (uint32_t)((BM + (r - C::MI) * 16) * C::KS * 2));
    } else {
      const int j = r - C::NA * C::MI;
      ds_read16(f.b[j], base + b_off + (uint32_t)(j * 16 * C::KS * 2));
    }
  };
  auto read_frags = [&](Frag& f, int st) __attribute__((always_inline)) {
    const uint32_t base = lds0 + (uint32_t)(st * C::STAGE);
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(f, base, r);
  };
  // wait for every issued fragment read, then make the fragments depend on that wait
  auto frags_ready = [&](Frag& f) __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(f.a[i]));
    if constexpr (SPLITA) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(f.a2[i]));
    }
#pragma unroll
    for (int j = 0; j < C::NI; ++j) asm volatile("" : "+v"(f.b[j]));
  };

  f32x4 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NMF = C::MI * C::NI * (SPLITA ? 2 : 1);      // MFMAs per stage
  auto mfma_one = [&](const Frag& f, int q) __attribute__((always_inline)) {
    const int h = SPLITA ? q & 1 : 0, ij = SPLITA ? q >> 1 : q;
    const int i = ij / C::NI, j = ij % C::NI;
    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h ? f.a2[i] : f.a[i], f.b[j], acc[i][j],
                                                        0, 0, 0);
  };
  // DMA load q of a stage (A, then A2, then B), into ring slot st from k stage kt
  auto issue_one = [&](int st, int kt, int q) __attribute__((always_inline)) {
    char* base = smem + st * C::STAGE;
    const int k0 = kt * C::KS;
    if (q < C::LA) {
      lds_dma16(asrc[q] + k0, base + (wave + 4 * q) * 1024);
    } else if (SPLITA && q < 2 * C::LA) {
      const int i = q - C::LA;
      lds_dma16(a2src[i] + k0, base + C::ABYTES + (wave + 4 * i) * 1024);
    } else {
      const int j = q - C::NA * C::LA;
      lds_dma16(bsrc[j] + k0, base + C::NA * C::ABYTES + (wave + 4 * j) * 1024);
    }
  };
  // One k stage.  Stage kt's fragments are in `cur`; after the vmcnt wait stage kt+1 has landed
  // for this wave, and after the barrier for every wave, and stage kt's slot is free (every wave
  // holds its fragments), so it is refilled with stage kt+NS.  The refill loads and the fragment
  // reads of stage kt+1 are spread over the MFMAs of stage kt in a fixed order.
  auto steady = [&](int kt, Frag& cur, Frag& nxt) __attribute__((always_inline)) {
    wait_vmcnt<C::LPW * (NS - 2)>();
    frags_ready(cur);
    block_barrier();
    const int sl = kt % NS;
    const uint32_t base = lds0 + (uint32_t)(((kt + 1) % NS) * C::STAGE);
    // MFMA q is followed by DMA load q (q < LPW), then by one fragment read after every other
    // MFMA; reads that do not fit go after the last MFMA
    constexpr int RSTEP = NMF - C::LPW >= 2 * NRD ? 2 : 1;
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      mfma_one(cur, q);
      if (q < C::LPW) issue_one(sl, kt + NS, q);
      if (q >= C::LPW && (q - C::LPW) % RSTEP == 0 && (q - C::LPW) / RSTEP < NRD)
        read_one(nxt, base, (q - C::LPW) / RSTEP);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = (NMF - C::LPW + RSTEP - 1) / RSTEP; r < NRD; ++r) read_one(nxt, base, r);
  };
  // the last stages: at most one left to issue
  auto tail = [&](int kt, Frag& cur, Frag& nxt) __attribute__((always_inline)) {
    wait_stages<C::LPW, NS>(min(NS - 2, nk - kt - 2));
    frags_ready(cur);
    block_barrier();
    if (kt + NS < nk) {
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) issue_one(kt % NS, kt + NS, q);
    }
    if (kt + 1 < nk) read_frags(nxt, (kt + 1) % NS);
#pragma unroll
    for (int q = 0; q < NMF; ++q) mfma_one(cur, q);
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nk) {
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) issue_one(st, st, q);
    }
  Frag f0, f1;
  if (nk > 0) {
    wait_stages<C::LPW, NS>(min(NS - 1, nk - 1));
    block_barrier();
    read_frags(f0, 0);
  }
  int kt = 0;
  for (; kt + 1 + NS < nk; kt += 2) {
    steady(kt, f0, f1);
    steady(kt + 1, f1, f0);
  }
  // at most NS + 1 stages remain, taken in pairs so the fragment sets keep alternating
  for (; kt < nk; kt += 2) {
    tail(kt, f0, f1);
    if (kt + 1 < nk) tail(kt + 1, f1, f0);
  }
  // no inline LDS read may still be in flight when the registers are reused below
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  // split-K: publish this unit's partial; gemm_reduce_kernel adds the partials and runs the
  // epilogue
  if (S > 1) {
    if constexpr (KIND == EPI_RESID) {
      if (e.norm_g) {
        // row-major partials [S][M][N] for resid_norm_kernel, which reduces whole rows and
        // writes the RMSNorm that follows the projection (a bf16-pair A is already summed)
        float* pr = reinterpret_cast<float*>(a.part) + (int64_t)sp * M * N;
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j) {
            const int col = n0 + wn * C::WTN + j * 16 + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * C::WTM + i * 16 + fk * 4 + r;
              if (row < M && col < N) pr[(int64_t)row * N + col] = acc[i][j][r];
            }
          }
        return;
      }
    }
    const int tiles_n = (N + BN - 1) / BN;
    const int tile = (z * tiles_n + tn) * tiles_m + tm;
    constexpr int FR = C::MI * C::NI * 64;                      // f32x4 per wave
    f32x4* mine = reinterpret_cast<f32x4*>(a.part) + (((int64_t)tile * S + sp) * 4 + wave) * FR +
                  lane;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j) mine[(i * C::NI + j) * 64] = acc[i][j];
    return;
  }

  // Output in rounds of 64 rows per wave row: round h stages accumulator rows [64h, 64h+64) of
  // both wave rows (tile rows wm*BM/2 + 64h + ...) in LDS as 128 fp32 rows, then runs the
  // epilogue over the two 64-row groups.  The accumulators a round uses are fixed at compile time.
  block_barrier();       // every wave is done reading the ring: reuse it for the output tile
  float* Cs = (float*)smem;
  constexpr int CS_LD = BN + 4;
#pragma unroll
  for (int h = 0; h < C::MI / 4; ++h) {
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * 64 + (i - 4 * h) * 16 + (lane >> 4) * 4 + r;
          const int col = wn * C::WTN + j * 16 + (lane & 15);
          Cs[row * CS_LD + col] = acc[i][j][r];
        }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      run_epilogue<bf16, 64, BN, KIND>(e, Cs + g * 64 * CS_LD, m0 + g * C::WTM + 64 * h, n0, tn,
                                       z, M, N);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ 8-wave ring
// Block tile 256 x BN, k stages of KS (32 or 64) bf16, NS-slot LDS ring filled by global->LDS
// DMA, 8 waves (two per SIMD) in a 2 x 4 grid: each wave owns a 128 x BN/4 sub-tile (8 x BN/64
// MFMA tiles) and one fragment set.  Per stage a wave waits for its own DMA of the stage, the
// workgroup synchronises once, the slot read in the previous stage is refilled, and the wave
// reads its fragments and runs its MFMAs one 32-wide k step at a time; the second wave on the
// SIMD runs MFMAs while the first waits for LDS.  With KS = 64 every DMA lane group reads whole
// 128-byte lines (8 rows x 128 bytes per 1 KB load), half the L2 requests of 64-byte rows.
// Stage rows are KS * 2 bytes; 16-byte chunk c of row r sits in slot c ^ swz(r) (swz32 for 64-byte
// rows, swz for 128-byte rows; both measured conflict-free for the fragment reads).
template <int BN, int NS, int KS_>
struct W8Cfg {
  static constexpr int BM = 256, KS = KS_, NT = 512, NW = 8;
  static constexpr int ROWB = KS * 2, CPR = KS / 8;       // bytes and 16-byte chunks per row
  static constexpr int RPL = 1024 / ROWB;                 // rows per 1 KB load
  static constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB;
  static constexpr int STAGE = ABYTES + BBYTES;
  static constexpr int NLA = ABYTES / 1024, NL = (ABYTES + BBYTES) / 1024;   // 1 KB loads / stage
  static constexpr int LPW = (NL + NW - 1) / NW;          // loads of waves 0 .. NL%NW-1 (or all)
  static constexpr int LPW_LO = NL % NW ? LPW - 1 : LPW;  // loads of the other waves
  static constexpr int WTM = 128, WTN = BN / 4, MI = 8, NI = WTN / 16;
  static constexpr int TM = BN == 192 ? 128 : 64;         // epilogue rows per round
  static constexpr int CBYTES = TM * (BN + 4) * 4;
  static constexpr int SMEM = NS * STAGE > CBYTES ? NS * STAGE : CBYTES;
  static_assert(KS == 32 || KS == 64, "stage depth");
  static_assert(BBYTES % 1024 == 0 && WTN % 16 == 0, "tile shape");
  static_assert(LPW * (NS - 1) <= 63, "vmcnt range");
  __device__ static int swizzle(int row) { return KS == 32 ? swz32(row) : swz(row); }
};

template <int BN, int NS, int KS, int KIND>
__global__ __launch_bounds__(512) void gemm_w8_kernel(GemmArgs a, EpiArgs e) {
  using C = W8Cfg<BN, NS, KS>;
  constexpr int BM = C::BM;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int z = blockIdx.z;
  const int M = a.M, N = a.N, K = a.K;
  const int S = a.split > 1 ? a.split : 1;
  const int tiles_m = (M + BM - 1) / BM;
  int tm, tn, sp;
  unit_of(blockIdx.x, gridDim.x, tiles_m, S, &tm, &tn, &sp);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk_all = K / KS;
  const int kb = (int)((int64_t)nk_all * sp / S), nk = (int)((int64_t)nk_all * (sp + 1) / S) - kb;

  // DMA load l of a stage (l < NL) fills LDS [l KB, l+1 KB) of the stage: tile rows RPL l' ..
  // RPL l' + RPL-1 of A (l' = l < NLA) or of B (l' = l - NLA); lane i fills row RPL l' + i/CPR,
  // slot i%CPR from global chunk (i%CPR) ^ swizzle(row).  Wave w issues loads w, w+8, w+16, ...
  const bool full = wave < (C::NL % C::NW ? C::NL % C::NW : C::NW);
  const int rr = lane / C::CPR, slot = lane % C::CPR;
  const BMap bm = make_bmap(a);
  const bf16* src[C::LPW];
#pragma unroll
  for (int q = 0; q < C::LPW; ++q) {
    int l = wave + C::NW * q;
    if (l >= C::NL) l = C::NL - 1;            // not issued (see issue); any valid address
    const bool isA = l < C::NLA;
    const int row = (isA ? l : l - C::NLA) * C::RPL + rr;
    const int chunk = (slot ^ C::swizzle(row)) * 8;
    src[q] = isA ? (const bf16*)a.A + (int64_t)z * a.a_bs + (int64_t)min(m0 + row, M - 1) * a.lda +
                       (int64_t)kb * KS + chunk
                 : brow_ptr<bf16, BN>(bm, min(n0 + row, N - 1), z) + (int64_t)kb * KS + chunk;
  }
  auto issue = [&](int st, int kt) __attribute__((always_inline)) {
    char* base = smem + st * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::LPW; ++q)
      if (q < C::LPW_LO || full) lds_dma16(src[q] + kt * KS, base + (wave + C::NW * q) * 1024);
  };
  // wait until at most n stages of this wave's loads are in flight (n in [0, NS - 2])
  auto wait_own = [&](int n) __attribute__((always_inline)) {
    if (full) wait_stages<C::LPW, NS>(n);
    else wait_stages<C::LPW_LO, NS>(n);
  };

  // fragment reads (inline ds_read_b128, see gemm_big_kernel): for k step s of a stage, lane l
  // reads row l%16 of each 16-row group at chunk 4s + l/16
  const int fr = lane & 15, fk = lane >> 4;
  const uint32_t smem0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  uint32_t lds_k[KS / 32];
#pragma unroll
  for (int s2 = 0; s2 < KS / 32; ++s2)
    lds_k[s2] = smem0 + (uint32_t)(fr * C::ROWB + (((4 * s2 + fk) ^ C::swizzle(fr)) * 16));
  const uint32_t a_off = (uint32_t)(wm * C::WTM * C::ROWB);
  const uint32_t b_off = (uint32_t)(C::ABYTES + wn * C::WTN * C::ROWB);
  bf16x8 fa[C::MI], fb[C::NI];

  f32x4 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st);
  for (int kt = 0; kt < nk; ++kt) {
    wait_own(min(NS - 2, nk - 1 - kt));
    block_barrier();
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
    const uint32_t stage = (uint32_t)((kt % NS) * C::STAGE);
#pragma unroll
    for (int s2 = 0; s2 < KS / 32; ++s2) {
      const uint32_t base = lds_k[s2] + stage;
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        ds_read16(fa[i], base + a_off + (uint32_t)(i * 16 * C::ROWB));
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
        ds_read16(fb[j], base + b_off + (uint32_t)(j * 16 * C::ROWB));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
      for (int j = 0; j < C::NI; ++j) asm volatile("" : "+v"(fb[j]));
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // Output: stage C::TM accumulator rows at a time in LDS as fp32, then the epilogue over them.
  // Round h holds tile rows [TM h, TM h + TM); the waves whose rows fall there write them.
  // `get(i, j)` yields accumulator tile (i, j) of this wave.
  auto store_tile = [&](auto get) __attribute__((always_inline)) {
    block_barrier();   // every wave is done reading the ring: reuse it for the output tile
    float* Cs = (float*)smem;
    constexpr int CS_LD = BN + 4;
#pragma unroll
    for (int h = 0; h < BM / C::TM; ++h) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int row0 = wm * C::WTM + i * 16;            // first tile row of acc tile (i, *)
        if (row0 / C::TM != h) continue;
#pragma unroll
        for (int j = 0; j < C::NI; ++j) {
          const f32x4 v = get(i, j);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row0 - h * C::TM + (lane >> 4) * 4 + r;
            const int col = wn * C::WTN + j * 16 + (lane & 15);
            Cs[row * CS_LD + col] = v[r];
          }
        }
      }
      __syncthreads();
      run_epilogue<bf16, C::TM, BN, KIND, C::NT>(e, Cs, m0 + h * C::TM, n0, tn, z, M, N);
      __syncthreads();
    }
  };

  if (S > 1) {
    // split-K: publish this unit's partial; gemm_reduce_kernel adds the partials and runs the
    // epilogue
    const int tiles_n = (N + BN - 1) / BN;
    const int tile = (z * tiles_n + tn) * tiles_m + tm;
    constexpr int FR = C::MI * C::NI * 64;                       // f32x4 per wave
    f32x4* mine = reinterpret_cast<f32x4*>(a.part) +
                  (((int64_t)tile * S + sp) * C::NW + wave) * FR + lane;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j) mine[(i * C::NI + j) * 64] = acc[i][j];
    return;
  }
  store_tile([&](int i, int j) { return acc[i][j]; });
}

// ------------------------------------------------------------------ 8-wave, register-staged
// The same 256 x BN tile, 8-wave grid, 64-wide k stages and epilogue as gemm_w8_kernel, but the
// tiles travel global -> VGPRs -> LDS (global_load_dwordx4, then ds_write_b128 into a two-slot
// ring) instead of global->LDS DMA: measured on gfx950, ordinary loads stream about 1.4x the
// bytes per CU that the DMA path does.  Two register sets alternate: stage kt+2 is loaded while
// stage kt is computed and stage kt+1 is written to LDS after it.  All LDS traffic is ordinary
// compiled code, so the compiler places every wait.
// WGM x (8 / WGM) wave grid: 2 x 4 gives each wave 128 x BN/4, 4 x 2 gives 64 x BN/2.  Every k
// stage each wave reads its A and B fragments from LDS, (WTM + WTN) rows of 128 bytes: the
// squarer 64 x BN/2 wave tile reads fewer bytes per MFMA (BN 128: 128 KB per stage for the
// workgroup instead of 160 KB).
template <int BN, int WGM = 2>
struct W8RCfg {
  static constexpr int BM = 256, KS = 64, NT = 512, NW = 8, ROWB = 128;
  static constexpr int WGN = NW / WGM;
  static constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB, STAGE = ABYTES + BBYTES;
  static constexpr int CH = STAGE / 16 / NT;              // 16-byte chunks per thread per stage
  static constexpr int WTM = BM / WGM, WTN = BN / WGN, MI = WTM / 16, NI = WTN / 16;
  static constexpr int TM = BN == 192 ? 128 : 64;
  static constexpr int CBYTES = TM * (BN + 4) * 4;
  static constexpr int SMEM = 2 * STAGE > CBYTES ? 2 * STAGE : CBYTES;
  static_assert(STAGE % (16 * NT) == 0 && WTN % 16 == 0, "tile shape");
};

// PR (pair rows, M <= 128 with a bf16-pair A operand): tile rows 0-127 are the rows of A's high
// part and rows 128-255 the same rows of its low part, so the waves of the lower half of the
// wave grid compute A_lo . B^T; the two halves are added per output row before the epilogue (and
// in the split-K reduction).  The pair then costs what a 256-row tile costs on 128 rows, with
// the tile's full arithmetic intensity on the weights.
template <int BN, int KIND, int WGM, bool PR>
__global__ __launch_bounds__(512) void gemm_w8r_kernel(GemmArgs a, EpiArgs e) {
  using C = W8RCfg<BN, WGM>;
  constexpr int BM = C::BM, KS = C::KS;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int z = blockIdx.z;
  const int M = a.M, N = a.N, K = a.K;
  const int S = a.split > 1 ? a.split : 1;
  const int tiles_m = (M + BM - 1) / BM;
  int tm, tn, sp;
  unit_of(blockIdx.x, gridDim.x, tiles_m, S, &tm, &tn, &sp);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk_all = K / KS;
  const int kb = (int)((int64_t)nk_all * sp / S), nk = (int)((int64_t)nk_all * (sp + 1) / S) - kb;

  // chunk c = tid + 512 q of a stage: tile row c / 8 (A rows first, then B rows), 16-byte chunk
  // c % 8 of the row's 128 bytes; eight consecutive threads read one 128-byte line.  It is
  // stored in LDS slot (c % 8) ^ swz(row) of the row.
  const BMap bm = make_bmap(a);
  const bf16* src[C::CH];
  uint32_t dst[C::CH];
#pragma unroll
  for (int q = 0; q < C::CH; ++q) {
    const int c = tid + C::NT * q, row = c >> 3, ch = c & 7;
    const bool isA = row < BM;
    const int r = isA ? row : row - BM;
    const bf16* arow;
    if constexpr (PR)
      arow = (const bf16*)(r < BM / 2 ? a.A : a.A2) + (int64_t)z * a.a_bs +
             (int64_t)min(r % (BM / 2), M - 1) * a.lda;
    else
      arow = (const bf16*)a.A + (int64_t)z * a.a_bs + (int64_t)min(m0 + r, M - 1) * a.lda;
    src[q] = (isA ? arow : brow_ptr<bf16, BN>(bm, min(n0 + r, N - 1), z)) + (int64_t)kb * KS +
             ch * 8;
    dst[q] = (uint32_t)(row * C::ROWB + ((ch ^ swz(row)) * 16));
  }
  u32x4 stA[C::CH], stB[C::CH];
  auto load = [&](u32x4* stg, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::CH; ++q) stg[q] = load_global16(src[q] + kt * KS);
  };
  auto store = [&](const u32x4* stg, int slot) __attribute__((always_inline)) {
    char* base = smem + slot * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::CH; ++q) *reinterpret_cast<u32x4*>(base + dst[q]) = stg[q];
  };

  const int fr = lane & 15, fk = lane >> 4;
  int rd[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) rd[s2] = fr * C::ROWB + (((4 * s2 + fk) ^ swz(fr)) * 16);
  const int a_off = wm * C::WTM * C::ROWB, b_off = C::ABYTES + wn * C::WTN * C::ROWB;

  f32x4 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) __attribute__((always_inline)) {
    const char* st = smem + slot * C::STAGE;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 fa[C::MI], fb[C::NI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off + rd[s2] + i * 16 * C::ROWB);
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(st + b_off + rd[s2] + j * 16 * C::ROWB);
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // Stage kt: slot kt&1 holds stage kt; the register set `nxt` holds stage kt+1 (loaded two
  // stages ago) and `fre` is free (its stage is in LDS).  Stage kt+2 is loaded into `fre`
  // first, so it has two stages of compute to land; after the MFMAs stage kt+1 goes from `nxt`
  // into the other slot, last read in stage kt-1 (before the barrier ending it).  Every step
  // loads and stores unconditionally (past the last stage it reloads and rewrites the last
  // one, which is never read again), so the order of the loads in flight is the same on every
  // path and the waits before the LDS writes cover only the older register set.
  auto step = [&](int kt, u32x4* nxt, u32x4* fre) __attribute__((always_inline)) {
    load(fre, min(kt + 2, nk - 1));
    compute(kt & 1);
    store(nxt, (kt + 1) & 1);
    __syncthreads();
  };

  load(stA, 0);
  store(stA, 0);
  load(stB, min(1, nk - 1));
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, stB, stA);
    step(kt + 1, stA, stB);
  }
  if (kt < nk) step(kt, stB, stA);

  auto store_tile = [&](auto get) __attribute__((always_inline)) {
    float* Cs = (float*)smem;
    constexpr int CS_LD = BN + 4;
    constexpr int OUT_ROWS = PR ? BM / 2 : BM;          // output rows of the tile
#pragma unroll
    for (int h = 0; h < OUT_ROWS / C::TM; ++h) {
      // with PR the waves holding low-part rows add onto the high part's rows after a barrier
#pragma unroll
      for (int part = 0; part < (PR ? 2 : 1); ++part) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const int row0 = wm * C::WTM + i * 16;
          if (PR && (row0 >= BM / 2) != (part == 1)) continue;
          const int orow0 = PR ? row0 % (BM / 2) : row0;
          if (orow0 / C::TM != h) continue;
#pragma unroll
          for (int j = 0; j < C::NI; ++j) {
            const f32x4 v = get(i, j);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = orow0 - h * C::TM + (lane >> 4) * 4 + r;
              const int col = wn * C::WTN + j * 16 + (lane & 15);
              if (part == 0) Cs[row * CS_LD + col] = v[r];
              else Cs[row * CS_LD + col] += v[r];
            }
          }
        }
        __syncthreads();
      }
      run_epilogue<bf16, C::TM, BN, KIND, C::NT>(e, Cs, m0 + h * C::TM, n0, tn, z, M, N);
      __syncthreads();
    }
  };

  if (S > 1) {
    if constexpr (KIND == EPI_RESID && !PR) {
      if (e.norm_g) {
        // row-major partials [S][M][N] for resid_norm_kernel, which reduces whole rows and
        // writes the RMSNorm that follows the projection
        float* pr = reinterpret_cast<float*>(a.part) + (int64_t)sp * M * N;
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j) {
            const int col = n0 + wn * C::WTN + j * 16 + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * C::WTM + i * 16 + fk * 4 + r;
              if (row < M && col < N) pr[(int64_t)row * N + col] = acc[i][j][r];
            }
          }
        return;
      }
    }
    // split-K: publish this unit's partial; gemm_reduce_kernel adds the partials and runs the
    // epilogue
    const int tiles_n = (N + BN - 1) / BN;
    const int tile = (z * tiles_n + tn) * tiles_m + tm;
    constexpr int FR = C::MI * C::NI * 64;                       // f32x4 per wave
    f32x4* mine = reinterpret_cast<f32x4*>(a.part) +
                  (((int64_t)tile * S + sp) * C::NW + wave) * FR + lane;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j) mine[(i * C::NI + j) * 64] = acc[i][j];
    return;
  }
  if constexpr (KIND == EPI_ARGMAX && !PR) {
    if (!e.logits) {
      // The argmax straight from the accumulators, without the tile's LDS round trip.  Lane
      // (fk, fr) holds rows wm*WTM + 16i + 4fk + r (k = 4i + r) at columns wn*WTN + 16j + fr.
      // Each lane first reduces its NI columns per row; then the 16 lanes of a row group
      // reduce by halving: at the step with lane offset o, a lane keeps half of its remaining
      // rows (the upper half if its bit o is set), sends the other half to lane ^ o and folds
      // in what it receives, so after four steps it holds the wave's result for KR / 16 rows
      // (two on the 2 x 4 wave grid, one on 4 x 2).  The WGN waves along N then meet in LDS.  Out-of-range columns never enter; the
      // lowest-index rule of argmax_combine makes the result independent of the order.
      constexpr int KR = C::MI * 4;                       // rows per lane
      static_assert(KR % 16 == 0, "rows per lane");
      float bv[KR];
      int bi[KR];
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bv[4 * i + r] = -INFINITY;
          bi[4 * i + r] = 0x7fffffff;
        }
#pragma unroll
      for (int j = 0; j < C::NI; ++j) {
        const int col = n0 + wn * C::WTN + j * 16 + fr;
        if (col < N) {
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) argmax_combine(bv[4 * i + r], bi[4 * i + r], acc[i][j][r], col);
        }
      }
#pragma unroll
      for (int o = 1, h = KR / 2; o < 16; o <<= 1, h >>= 1) {
        const bool up = (fr & o) != 0;
#pragma unroll
        for (int k = 0; k < h; ++k) {
          const float sv = up ? bv[k] : bv[k + h];
          const int si = up ? bi[k] : bi[k + h];
          const float ov = __shfl_xor(sv, o, 64);
          const int oi = __shfl_xor(si, o, 64);
          if (up) {
            bv[k] = bv[k + h];
            bi[k] = bi[k + h];
          }
          argmax_combine(bv[k], bi[k], ov, oi);
        }
      }
      // lane fr now holds the KR / 16 rows from k = kb on: the step at offset 2^s kept the
      // upper half (KR / 2^(s+1) rows further on) exactly when bit s of fr is set
      const int kb = (KR / 2) * (fr & 1) + (KR / 4) * ((fr >> 1) & 1) +
                     (KR / 8) * ((fr >> 2) & 1) + (KR / 16) * ((fr >> 3) & 1);
      float* sv = (float*)smem;                           // [WGN][BM]
      int* si = (int*)(smem + C::WGN * BM * 4);
#pragma unroll
      for (int q = 0; q < KR / 16; ++q) {
        const int k = kb + q, row = wm * C::WTM + 16 * (k >> 2) + 4 * fk + (k & 3);
        sv[wn * BM + row] = bv[q];
        si[wn * BM + row] = bi[q];
      }
      __syncthreads();
      if (tid < BM && m0 + tid < M) {
        float v = sv[tid];
        int ix = si[tid];
#pragma unroll
        for (int w = 1; w < C::WGN; ++w) argmax_combine(v, ix, sv[w * BM + tid], si[w * BM + tid]);
        e.part_val[(int64_t)(m0 + tid) * e.ntiles + tn] = v;
        e.part_idx[(int64_t)(m0 + tid) * e.ntiles + tn] = ix;
      }
      return;
    }
  }
  store_tile([&](int i, int j) { return acc[i][j]; });
}

// ------------------------------------------------------------------ skinny: M <= 64 rows
// For a handful of rows (a small block, few sequences) the projections stream their weights:
// one row tile covers all M rows (MT = 32 or 64), so every weight element is read exactly once.
// Block tile MT x 128, four waves in a 1 x 4 grid, each wave all MT rows and 32 columns.  Each
// wave loads its own 32 weight rows as whole 128-byte lines (eight lanes a line) into registers,
// two 64-wide k stages ahead in three register sets, and stages them through its own region of
// the two-slot LDS ring, from which it reads its MFMA fragments; A (and its low bf16 part with
// SPLITA) shares the ring.  Loading B fragments straight into registers instead (each load
// instruction then touches 16 half lines) streamed 8 % slower at 32 rows.  Split-K gives every
// CU work: units = column tiles x S.
template <int MT, bool SPLITA>
struct SkinnyCfg {
  static constexpr int BM = MT, BN = 128, KS = 64, NT = 256, NW = 4, ROWB = 128;
  static constexpr int NA = SPLITA ? 2 : 1;
  static constexpr int ABYTES = BM * ROWB;                  // one A part of a stage
  static constexpr int BBYTES = BN * ROWB;                  // 4 waves x 32 rows of B
  static constexpr int STAGE = NA * ABYTES + BBYTES;
  static constexpr int CH = (ABYTES + 16 * NT - 1) / (16 * NT);   // A chunks per thread
  static constexpr int WTN = BN / NW, MI = BM / 16, NI = WTN / 16;
  static constexpr int TM = MT > 32 ? 32 : MT;              // epilogue rows per pass
  static constexpr int CBYTES = TM * (BN + 4) * 4;
  static constexpr int SMEM = 2 * STAGE > CBYTES ? 2 * STAGE : CBYTES;
  static_assert(MI >= 1 && NI == 2, "tile shape");
};

template <int MT, int KIND, bool SPLITA>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a, EpiArgs e) {
  using C = SkinnyCfg<MT, SPLITA>;
  // The LM head streams its weights (hundreds of MB, each element read once) non-temporally:
  // Qwen3-4B shape, bs 1, 0.153 -> 0.141 ms per step.  The projections keep cached loads (down
  // measured slower non-temporal, gate/up and Q/K/V unchanged).
  constexpr bool kStreamB = KIND == EPI_ARGMAX || KIND == EPI_STORE_F32;
  constexpr int BM = C::BM, BN = C::BN, KS = C::KS, MI = C::MI, NI = C::NI;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z;
  const int M = a.M, N = a.N, K = a.K;
  const int S = a.split > 1 ? a.split : 1;
  const int tiles_m = (M + BM - 1) / BM;                    // 1 for M <= MT
  int tm, tn, sp;
  unit_of(blockIdx.x, gridDim.x, tiles_m, S, &tm, &tn, &sp);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk_all = K / KS;
  const int kb = (int)((int64_t)nk_all * sp / S), nk = (int)((int64_t)nk_all * (sp + 1) / S) - kb;

  // A: chunk c = tid + 256 q of a part is row c / 8, 16-byte chunk c % 8 (slot (c % 8) ^ swz(row))
  const bf16* asrc[C::CH];
  const bf16* a2src[C::CH];
  uint32_t adst[C::CH];
  bool aok[C::CH];
#pragma unroll
  for (int q = 0; q < C::CH; ++q) {
    const int c = tid + C::NT * q, row = c >> 3, ch = c & 7;
    aok[q] = row < BM;
    const int64_t off = (int64_t)z * a.a_bs + (int64_t)min(m0 + min(row, BM - 1), M - 1) * a.lda +
                        (int64_t)kb * KS + ch * 8;
    asrc[q] = (const bf16*)a.A + off;
    a2src[q] = SPLITA ? (const bf16*)a.A2 + off : asrc[q];
    adst[q] = (uint32_t)(min(row, BM - 1) * C::ROWB + ((ch ^ swz(row)) * 16));
  }
  // B: each wave's 32 weight rows (columns of C) as whole 128-byte lines, eight lanes a line: lane
  // l of load q is row 32 wave + 8 q + l / 8, chunk l % 8, stored in the wave's LDS region at
  // slot (l % 8) ^ swz(row); the fragments are read back like A's
  const int fr = lane & 15, fk = lane >> 4;
  const BMap bm = make_bmap(a);
  const bf16* bsrc[4];
  uint32_t bdst[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * q + (lane >> 3), ch = lane & 7;
    bsrc[q] = brow_ptr<bf16, BN>(bm, min(n0 + wave * C::WTN + row, N - 1), z) +
              (int64_t)kb * KS + ch * 8;
    bdst[q] = (uint32_t)(C::NA * C::ABYTES + wave * C::WTN * C::ROWB + row * C::ROWB +
                         ((ch ^ swz(row)) * 16));
  }
  u32x4 sa0[C::CH][2], sa1[C::CH][2], sa2[C::CH][2];
  u32x4 b0[NI][2], b1[NI][2], b2[NI][2];
  auto load = [&](u32x4 (*sa)[2], u32x4 (*bq)[2], int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bq[q / 2][q % 2] = kStreamB ? load_global16_nt(bsrc[q] + kt * KS)
                                  : load_global16(bsrc[q] + kt * KS);
#pragma unroll
    for (int q = 0; q < C::CH; ++q) {
      if (!aok[q]) continue;
      sa[q][0] = load_global16(asrc[q] + kt * KS);
      if constexpr (SPLITA) sa[q][1] = load_global16(a2src[q] + kt * KS);
    }
  };
  auto store = [&](u32x4 (*sa)[2], u32x4 (*bq)[2], int slot) __attribute__((always_inline)) {
    char* base = smem + slot * C::STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(base + bdst[q]) = bq[q / 2][q % 2];
#pragma unroll
    for (int q = 0; q < C::CH; ++q) {
      if (!aok[q]) continue;
      *reinterpret_cast<u32x4*>(base + adst[q]) = sa[q][0];
      if constexpr (SPLITA) *reinterpret_cast<u32x4*>(base + C::ABYTES + adst[q]) = sa[q][1];
    }
  };
  int rd[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) rd[s2] = fr * C::ROWB + (((4 * s2 + fk) ^ swz(fr)) * 16);

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) __attribute__((always_inline)) {
    const char* st = smem + slot * C::STAGE;
    const char* sb = st + C::NA * C::ABYTES + wave * C::WTN * C::ROWB;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 bq[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j)
        bq[j] = *reinterpret_cast<const bf16x8*>(sb + rd[s2] + j * 16 * C::ROWB);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 fa = *reinterpret_cast<const bf16x8*>(st + rd[s2] + i * 16 * C::ROWB);
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              fa, bq[j], acc[i][j], 0, 0, 0);
        if constexpr (SPLITA) {
          const bf16x8 fa2 =
              *reinterpret_cast<const bf16x8*>(st + C::ABYTES + rd[s2] + i * 16 * C::ROWB);
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fa2, bq[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  // Stage kt: LDS slot kt & 1 holds A of stage kt; register set `cur` B of stage kt, `nx1` A and
  // B of stage kt + 1, `nx2` free: stage kt + 2 is loaded into it, stage kt computed, A of stage
  // kt + 1 stored into the other slot (last read in stage kt - 1, before the barrier ending it).
  // Loads past the last stage reload the last one.
  auto step = [&](int kt, u32x4 (*anx1)[2], u32x4 (*bnx1)[2], u32x4 (*anx2)[2],
                  u32x4 (*bnx2)[2]) __attribute__((always_inline)) {
    load(anx2, bnx2, min(kt + 2, nk - 1));
    compute(kt & 1);
    store(anx1, bnx1, (kt + 1) & 1);
    __syncthreads();
  };

  load(sa0, b0, 0);
  store(sa0, b0, 0);
  load(sa1, b1, min(1, nk - 1));
  __syncthreads();
  int kt = 0;
  for (; kt + 2 < nk; kt += 3) {
    step(kt, sa1, b1, sa2, b2);
    step(kt + 1, sa2, b2, sa0, b0);
    step(kt + 2, sa0, b0, sa1, b1);
  }
  if (kt < nk) {
    step(kt, sa1, b1, sa2, b2);
    if (kt + 1 < nk) step(kt + 1, sa2, b2, sa0, b0);
  }

  if (S > 1) {
    if constexpr (KIND == EPI_RESID) {
      if (e.norm_g) {
        // row-major partials [S][M][N] for resid_norm_kernel, which reduces whole rows
        float* pr = reinterpret_cast<float*>(a.part) + (int64_t)sp * M * N;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int col = n0 + wave * C::WTN + j * 16 + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + i * 16 + fk * 4 + r;
              if (row < M && col < N) pr[(int64_t)row * N + col] = acc[i][j][r];
            }
          }
        return;
      }
    }
    const int tiles_n = (N + BN - 1) / BN;
    const int tile = (z * tiles_n + tn) * tiles_m + tm;
    constexpr int FR = MI * NI * 64;
    f32x4* mine = reinterpret_cast<f32x4*>(a.part) +
                  (((int64_t)tile * S + sp) * C::NW + wave) * FR + lane;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) mine[(i * NI + j) * 64] = acc[i][j];
    return;
  }
  float* Cs = (float*)smem;
  constexpr int CS_LD = BN + 4;
#pragma unroll
  for (int h = 0; h < BM / C::TM; ++h) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (i * 16 / C::TM != h) continue;
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Cs[(i * 16 - h * C::TM + fk * 4 + r) * CS_LD + wave * C::WTN + j * 16 + fr] =
              acc[i][j][r];
    }
    __syncthreads();
    run_epilogue<bf16, C::TM, BN, KIND, C::NT>(e, Cs, m0 + h * C::TM, n0, tn, z, M, N);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ split-K reduction
// Second kernel of a split-K GEMM (the units of the first only publish their partials): each
// workgroup adds, in split order, the S partials of TM rows x BN columns of one output tile and
// runs the epilogue over them, so the reduction of a tile is spread over BM / TM workgroups.
// Measured on gfx950 this is 2-3x faster than letting the last unit of each tile to finish add
// the partials (behind an atomic counter and a device-scope fence): that unit reads S tiles of
// fp32 alone while the rest of the chip idles.  The partials are in the main kernel's fragment
// order: per tile, per split, per wave of the WGM x WGN wave grid (wave = wm * WGN + wn), per
// 16 x 16 accumulator tile (i, j) of the wave, per lane one f32x4 holding rows 4 (lane / 16) ..
// + 3 of column lane % 16; 64 consecutive lanes read 1 KB.
template <int BN>
struct ReduceCfg {
  // the SwiGLU and rotation epilogues need 16 columns per thread: 192-wide tiles take 64 rows
  static constexpr int TM = BN == 192 ? 64 : 32, NT = 256, CS_LD = BN + 4;
};

// PR: the partials come from a pair-rows tile (gemm_w8r_kernel): output row r of the tile is the
// sum of tile rows r and r + BM/2, added here per split.
template <int BM, int BN, int WGM, int WGN, int KIND, bool PR = false>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a, EpiArgs e) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN, MI = WTM / 16, NI = WTN / 16;
  constexpr int NW = WGM * WGN, FR = MI * NI * 64;
  using R = ReduceCfg<BN>;
  constexpr int TM = R::TM, CS_LD = R::CS_LD;
  constexpr int UNITS = TM / 16 * WGN * NI * 64;            // f32x4 of one strip
  constexpr int UPT = UNITS / R::NT;
  static_assert(UNITS % R::NT == 0 && WTM % TM == 0, "reduction strip layout");
  __shared__ float Cs[TM * CS_LD];
  const int tid = threadIdx.x, z = blockIdx.z;
  const int M = a.M, N = a.N, S = a.split;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int strip = blockIdx.x % (BM / TM), t = blockIdx.x / (BM / TM);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN, r0 = strip * TM;
  if (m0 + r0 >= M) return;
  if (PR && r0 >= BM / 2) return;
  const int tile = (z * tiles_n + tn) * tiles_m + tm;
  const int wm = r0 / WTM, i0 = (r0 % WTM) / 16;
  const int wl = (r0 + BM / 2) / WTM, il = ((r0 + BM / 2) % WTM) / 16;   // PR: low-part rows
  const f32x4* part = reinterpret_cast<const f32x4*>(a.part) + (int64_t)tile * S * NW * FR;
  // Q/K/V: the epilogue's rotation factors and row positions are loaded now, with the
  // partials, instead of after them
  constexpr int ETPR = R::NT / TM, ECPT = BN / ETPR;     // run_epilogue's thread layout
  float2 cs_pre[KIND == EPI_QKV ? ECPT : 1];
  int pos_pre = -1;
  if constexpr (KIND == EPI_QKV) {
    const int em = m0 + r0 + tid / ETPR, ecb = (tid % ETPR) * ECPT, half = e.hd / 2;
    if (n0 < e.qd + e.kd && em < M) {
#pragma unroll
      for (int q = 0; q < ECPT; ++q) cs_pre[q] = e.rope[(int64_t)em * half + ((ecb + q) % e.hd) % half];
    }
    if (tid < TM && m0 + r0 + tid < M) pos_pre = e.row_pos[m0 + r0 + tid];
  }
  int off[UPT], offl[PR ? UPT : 1];
  f32x4 v[UPT];
#pragma unroll
  for (int q = 0; q < UPT; ++q) {
    const int u = tid + R::NT * q, lane = u & 63, rest = u >> 6;
    const int j = rest % NI, wn = (rest / NI) % WGN, di = rest / (NI * WGN);
    off[q] = (wm * WGN + wn) * FR + ((i0 + di) * NI + j) * 64 + lane;
    v[q] = part[off[q]];
    if constexpr (PR) {
      offl[q] = (wl * WGN + wn) * FR + ((il + di) * NI + j) * 64 + lane;
      v[q] += part[offl[q]];
    }
  }
  // the later splits in batches of RB, every load of a batch issued before any is added (the
  // additions keep split order); RB shrinks with the loads per split so the batch fits the
  // registers
  constexpr int LPS = UPT * (PR ? 2 : 1);                   // f32x4 loads per split
  constexpr int RB = LPS <= 4 ? 4 : (LPS <= 8 ? 2 : 1);
  for (int sp0 = 1; sp0 < S; sp0 += RB) {
    f32x4 w[RB][UPT], wl[PR ? RB : 1][PR ? UPT : 1];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (sp0 + b >= S) break;
      const f32x4* ps = part + (int64_t)(sp0 + b) * NW * FR;
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        w[b][q] = ps[off[q]];
        if constexpr (PR) wl[b][q] = ps[offl[q]];
      }
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (sp0 + b >= S) break;
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        v[q] += w[b][q];
        if constexpr (PR) v[q] += wl[b][q];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < UPT; ++q) {
    const int u = tid + R::NT * q, lane = u & 63, rest = u >> 6;
    const int j = rest % NI, wn = (rest / NI) % WGN, di = rest / (NI * WGN);
    const int col = wn * WTN + j * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) Cs[(di * 16 + (lane >> 4) * 4 + r) * CS_LD + col] = v[q][r];
  }
  __syncthreads();
  if constexpr (KIND == EPI_QKV)
    run_epilogue<bf16, TM, BN, KIND, R::NT>(e, Cs, m0 + r0, n0, tn, z, M, N, cs_pre, &pos_pre);
  else
    run_epilogue<bf16, TM, BN, KIND, R::NT>(e, Cs, m0 + r0, n0, tn, z, M, N);
}

// Split-K reduction of a residual projection fused with the RMSNorm that follows it (skinny
// tiles, register-staged 256-row tiles without pair rows, deep-ring four-wave tiles): one
// workgroup per row adds the row's S row-major partials in split order, adds the sum to the
// residual as the residual epilogue does, and writes the residual and the normalised bf16 row
// x / sqrt(mean(x^2) + eps) * g, with the low part of the bf16 pair when norm_out_lo is set.
// Thread t owns the groups of 4 columns t and t + 1024; the gain and the residual are loaded
// with the first RB splits' partials, and the normalised columns go out as 8-byte stores.
// RB splits' loads are in flight together: 4 keeps the kernel at 63 VGPRs, so two rows share a
// CU (512 rows in one round); 8 (95 VGPRs, one row per CU) halves the round trips when the rows
// fit on the CUs anyway.
template <int RB>
__global__ __launch_bounds__(1024) void resid_norm_kernel(GemmArgs a, EpiArgs e) {
  constexpr int NT = kResidNormThreads, MAXG = kResidNormVecsPerThread;
  static_assert(NT * MAXG * 4 == kResidNormMaxCols, "row coverage of resid_norm_fits");
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  __shared__ float red[NT / 64];
  const int row = blockIdx.x, tid = threadIdx.x, N = a.N, S = a.split;
  const float* part = reinterpret_cast<const float*>(a.part) + (int64_t)row * N;
  const int64_t ps = (int64_t)a.M * N;                  // one split's partials
  float* xr = reinterpret_cast<float*>(e.C) + (int64_t)row * N;
  const bf16* g = reinterpret_cast<const bf16*>(e.norm_g);
  f32x4 acc[MAXG], xv[MAXG];
  bf16x4 gv[MAXG];
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int i = (tid + q * NT) * 4;
    if (i < N) {
      xv[q] = *reinterpret_cast<const f32x4*>(xr + i);
      gv[q] = *reinterpret_cast<const bf16x4*>(g + i);
      acc[q] = *reinterpret_cast<const f32x4*>(part + i);
    }
  }
  for (int s0 = 1; s0 < S; s0 += RB) {
    f32x4 w[RB][MAXG];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int q = 0; q < MAXG; ++q) {
        const int i = (tid + q * NT) * 4;
        if (s0 + b < S && i < N)
          w[b][q] = *reinterpret_cast<const f32x4*>(part + (s0 + b) * ps + i);
      }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int q = 0; q < MAXG; ++q)
        if (s0 + b < S) acc[q] += w[b][q];
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int i = (tid + q * NT) * 4;
    if (i < N) {
      xv[q] += acc[q];
      *reinterpret_cast<f32x4*>(xr + i) = xv[q];
      ss += xv[q][0] * xv[q][0] + xv[q][1] * xv[q][1] + xv[q][2] * xv[q][2] + xv[q][3] * xv[q][3];
    }
  }
  // the normalised row's place: all rows, or the mask rows of each block, compacted
  int orow = row;
  if (e.norm_n_anchor > 0) {
    const int B = e.norm_block_len, b = row % B;
    if (b < e.norm_n_anchor) return;              // an anchor row: residual only (uniform)
    orow = (row / B) * (B - e.norm_n_anchor) + b - e.norm_n_anchor;
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) tot += red[w];
  const float inv = rsqrtf(tot / (float)N + e.norm_eps);
  bf16* o = reinterpret_cast<bf16*>(e.norm_out) + (int64_t)orow * N;
  bf16* ol = e.norm_out_lo ? reinterpret_cast<bf16*>(e.norm_out_lo) + (int64_t)orow * N : nullptr;
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int i = (tid + q * NT) * 4;
    if (i >= N) continue;
    bf16x4 hi, lo;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float y = xv[q][c] * inv * (float)gv[q][c];
      hi[c] = (bf16)y;
      lo[c] = (bf16)(y - (float)hi[c]);
    }
    *reinterpret_cast<bf16x4*>(o + i) = hi;
    if (ol) *reinterpret_cast<bf16x4*>(ol + i) = lo;
  }
}

static void launch_resid_norm(const GemmArgs& a, const EpiArgs& e, hipStream_t s) {
  if (a.M <= 256)
    hipLaunchKernelGGL(resid_norm_kernel<8>, dim3(a.M), dim3(kResidNormThreads), 0, s, a, e);
  else
    hipLaunchKernelGGL(resid_norm_kernel<4>, dim3(a.M), dim3(kResidNormThreads), 0, s, a, e);
}

template <int BM, int BN, int WGM, int WGN, int KIND, bool PR = false>
static void launch_reduce(const GemmArgs& a, const EpiArgs& e, int batch, hipStream_t s) {
  const int grid = ceil_div(a.M, BM) * ceil_div(a.N, BN) * (BM / ReduceCfg<BN>::TM);
  hipLaunchKernelGGL((gemm_reduce_kernel<BM, BN, WGM, WGN, KIND, PR>), dim3(grid, 1, batch),
                     dim3(ReduceCfg<BN>::NT), 0, s, a, e);
}

template <int BN, int KIND, int WGM, bool PR = false>
static void launch_w8r(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, BN / 2) * BN;
  const int S = a.split > 1 ? a.split : 1;
  const int units = ceil_div(a.M, 256) * ceil_div(a.N, BN) * S;
  hipLaunchKernelGGL((gemm_w8r_kernel<BN, KIND, WGM, PR>), dim3(units, 1, batch), dim3(512),
                     0, s, a, e);
  if (S > 1 && KIND == EPI_RESID && !PR && e.norm_g)
    launch_resid_norm(a, e, s);
  else if (S > 1)
    launch_reduce<256, BN, WGM, 8 / WGM, KIND, PR>(a, e, batch, s);
}

template <int MT, int KIND, bool SPLITA>
static void launch_skinny(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, 64) * 128;
  const int S = a.split > 1 ? a.split : 1;
  const int units = ceil_div(a.M, MT) * ceil_div(a.N, 128) * S;
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, KIND, SPLITA>), dim3(units, 1, batch), dim3(256), 0,
                     s, a, e);
  if (S > 1 && KIND == EPI_RESID && e.norm_g)
    launch_resid_norm(a, e, s);
  else if (S > 1)
    launch_reduce<MT, 128, 1, 4, KIND>(a, e, batch, s);
}

template <int BN, int NS, int KS, int KIND>
static void launch_w8(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, BN / 2) * BN;
  const int S = a.split > 1 ? a.split : 1;
  const int units = ceil_div(a.M, 256) * ceil_div(a.N, BN) * S;
  hipLaunchKernelGGL((gemm_w8_kernel<BN, NS, KS, KIND>), dim3(units, 1, batch), dim3(512), 0, s,
                     a, e);
  if (S > 1) launch_reduce<256, BN, 2, 4, KIND>(a, e, batch, s);
}

template <int BM, int BN, int NS, int KIND, bool SPLITA>
static void launch_deep(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, BN / 2) * BN;
  const int S = a.split > 1 ? a.split : 1;
  const int units = ceil_div(a.M, BM) * ceil_div(a.N, BN) * S;
  hipLaunchKernelGGL((gemm_big_kernel<BM, BN, NS, KIND, SPLITA>), dim3(units, 1, batch),
                     dim3(256), 0, s, a, e);
  if (S > 1 && KIND == EPI_RESID && e.norm_g)
    launch_resid_norm(a, e, s);
  else if (S > 1)
    launch_reduce<BM, BN, 2, 2, KIND>(a, e, batch, s);
}

// 8: 256 x 128 (3 stages), 9: 128 x 256 (3), 10: 128 x 128 (4): four waves, 32-wide k stages;
// 11: 256 x 256 (2), 12: 256 x 192 (2), 13: 256 x 128 (3): eight waves, 64-wide k stages;
// 14: 256 x 256, 15: 256 x 192, 16: 256 x 128: eight waves, register-staged two-slot ring;
// 17: 64 x 128, 18: 32 x 128: the skinny tile for M <= 64 (B straight into registers, bf16 pairs
// too).  The bf16-pair A operand doubles the A part
// of a stage and the A fragments: pairs always take the four-wave 128 x 128 tile with 6 stages.
// The value-cache epilogues (QKV, context K/V) need 128-column tiles.
template <int KIND, bool SPLITA>
void launch_deep_cfg(int cfg, GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (cfg == 17) {
    launch_skinny<64, KIND, SPLITA>(a, e, batch, s);
  } else if (cfg == 18) {
    launch_skinny<32, KIND, SPLITA>(a, e, batch, s);
  } else if constexpr (SPLITA) {
    // the register-staged tiles take a pair as rows (A high part, then low part) for M <= 128
    if (cfg >= 14 && cfg <= 16 && a.M <= 128) {
      if constexpr (KIND == EPI_QKV || KIND == EPI_CTXKV) {
        launch_w8r<128, KIND, 4, true>(a, e, batch, s);
      } else {
        switch (cfg) {
          case 14: launch_w8r<256, KIND, 2, true>(a, e, batch, s); break;
          case 15: launch_w8r<192, KIND, 4, true>(a, e, batch, s); break;
          default: launch_w8r<128, KIND, 4, true>(a, e, batch, s); break;
        }
      }
    } else {
      launch_deep<128, 128, 6, KIND, true>(a, e, batch, s);
    }
  } else if constexpr (KIND == EPI_QKV || KIND == EPI_CTXKV) {
    switch (cfg) {
      case 8: launch_deep<256, 128, 3, KIND, false>(a, e, batch, s); break;
      case 11: case 12: case 13: launch_w8<128, 3, 64, KIND>(a, e, batch, s); break;
      case 14: case 15: case 16: launch_w8r<128, KIND, 4>(a, e, batch, s); break;
      default: launch_deep<128, 128, 4, KIND, false>(a, e, batch, s); break;
    }
  } else {
    switch (cfg) {
      case 8: launch_deep<256, 128, 3, KIND, false>(a, e, batch, s); break;
      case 9: launch_deep<128, 256, 3, KIND, false>(a, e, batch, s); break;
      case 11: launch_w8<256, 2, 64, KIND>(a, e, batch, s); break;
      case 12: launch_w8<192, 2, 64, KIND>(a, e, batch, s); break;
      case 13: launch_w8<128, 3, 64, KIND>(a, e, batch, s); break;
      case 14: launch_w8r<256, KIND, 2>(a, e, batch, s); break;
      case 15: launch_w8r<192, KIND, 4>(a, e, batch, s); break;
      case 16: launch_w8r<128, KIND, 4>(a, e, batch, s); break;
      default: launch_deep<128, 128, 4, KIND, false>(a, e, batch, s); break;
    }
  }
}

#define DBD_DEEP(K)                                                                         \
  template void launch_deep_cfg<K, false>(int, GemmArgs, const EpiArgs&, int, hipStream_t); \
  template void launch_deep_cfg<K, true>(int, GemmArgs, const EpiArgs&, int, hipStream_t);
DBD_DEEP(EPI_STORE_F32)
DBD_DEEP(EPI_RESID)
DBD_DEEP(EPI_QKV)
DBD_DEEP(EPI_CTXKV)
DBD_DEEP(EPI_SWIGLU)
DBD_DEEP(EPI_ARGMAX)
#undef DBD_DEEP

}  // namespace dbd
