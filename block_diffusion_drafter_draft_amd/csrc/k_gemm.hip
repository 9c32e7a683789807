// Projection GEMMs of the drafter: C = A[M,K] . W[N,K]^T (both operands K-contiguous), with the
// epilogues that consume the tile (gemm_common.h), and the choice of kernel and tile per shape.
//
// bf16 pipelined path (gfx950): block tile BM x BN x 64 for 4 waves in a 2 x 2 grid, each wave a
// (BM/2) x (BN/2) grid of 16x16x32 bf16 MFMA tiles with fp32 accumulation.  Tiles move from
// global memory straight into LDS (global_load_lds_dwordx4, no register staging) through an
// ST-stage ring; the 16-byte chunks of each 128-byte tile row are XOR-swizzled by choosing which
// global chunk each lane fetches.  One barrier per k-tile.  Tiles sharing a weight column tile
// are dispatched to the same XCD back to back so the weights come from HBM once.  The deep-ring
// kernels (k_gemm_deep.hip) take the shapes where a deeper prefetch or split-K pays.
// fp32 path: 64 x 128 x 16 block tile on the vector ALUs (exact fp32 products and sums).
// All paths stage the finished tile in LDS as fp32 and run the same epilogue code over it.
#include <algorithm>
#include <cmath>

#include "gemm_common.h"

namespace dbd {

constexpr int BK = 64;


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
// Block tile configurations of the bf16 path: (BM, BN).  0-7: the pipelined ring of 64-wide k
// tiles (stages per configuration in launch_cfg); 8-13: the deep rings of 32-wide k stages with
// optional split-K (k_gemm_deep.hip; 8-10 four waves, 11-13 eight waves).
constexpr int kNumCfg = kMaxGemmCfg + 1;
static const int kCfgBM[kNumCfg] = {256, 256, 128, 64, 128, 64, 256, 128, 256, 128, 128,
                                    256, 256, 256, 256, 256, 256, 64, 32};
static const int kCfgBN[kNumCfg] = {256, 128, 128, 128, 128, 128, 128, 256, 128, 256, 128,
                                    256, 192, 128, 256, 192, 128, 128, 128};
// 17, 18: the skinny tiles (64 or 32 rows, every weight read once) for M <= 64
static bool is_skinny(int cfg) { return cfg == 17 || cfg == 18; }
static bool is_deep(int cfg) { return cfg >= 8; }

template <int BM, int BN, int ST, int KIND, bool SPLITA>
static void launch_pipe(GemmArgs a, const EpiArgs& e, int batch, hipStream_t s) {
  if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, BN / 2) * BN;
  const int tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, ST, KIND, SPLITA>), dim3(tiles, 1, batch),
                     dim3(256), 0, s, a, e);
}

template <int KIND, bool SPLITA>
static void launch_cfg(int cfg, const GemmArgs& a, const EpiArgs& e, int batch, hipStream_t s) {
  if (is_deep(cfg)) {
    launch_deep_cfg<KIND, SPLITA>(cfg, a, e, batch, s);
    return;
  }
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

// The register-staged 256-row tiles (14-16) take a bf16-pair A operand as 256 rows (high part,
// then low part) when M <= 128.
static bool pair_rows(int cfg, int M) { return cfg >= 14 && cfg <= 16 && M <= 128; }

// The configuration a bf16-pair launch of `cfg` really uses (the pair doubles the A operand's
// LDS and registers, so only the smaller tiles take it, or the 256-row tiles as pair rows).
static int pair_cfg(int cfg, int M) {
  if (is_skinny(cfg)) return cfg;                 // the skinny tiles take the pair themselves
  if (pair_rows(cfg, M)) return cfg;
  if (is_deep(cfg)) return 10;
  if (cfg == 3 || cfg == 5) return 5;
  return 4;
}

// Split-K factor for a deep-ring tile, from a time estimate: rounds of 256 workgroups times the
// time of one unit (a CU at about 1/256 of 1.9 PFLOP/s), plus the fp32 partials written and
// read back (at about 5 TB/s) and the reduction kernel's launch (about 4 us).  A unit keeps at
// least 4 k stages of 32.
static int choose_split(int cfg, int M, int Nv, int K, int batch) {
  const double BM = kCfgBM[cfg], BN = kCfgBN[cfg];
  const double tiles = (double)ceil_div(M, kCfgBM[cfg]) * ceil_div(Nv, kCfgBN[cfg]) * batch;
  const double cu_flops = 1.9e15 / 256, part_bw = 5e12, launch_s = 4e-6;
  static const int cand[6] = {1, 2, 3, 4, 6, 8};
  int best = 1;
  double best_t = 0;
  for (int S : cand) {
    if (S > 1 && K / 32 / S < 4) break;
    double t = std::ceil(tiles * S / 256.0) * 2.0 * BM * BN * ((double)K / S) / cu_flops;
    if (S > 1) t += tiles * S * BM * BN * 4.0 * 2.0 / part_bw + launch_s;
    if (S == 1 || t < best_t) { best = S; best_t = t; }
  }
  return best;
}

// Default tile for a problem, from timings of every configuration on the drafter's shapes with
// their own epilogues (MI355X, weights streamed from HBM):
//  - bf16-pair A operands, and the Q/K/V and context K/V epilogues (rotation, scattered cache
//    writes) when M >= 64: the four-wave deep 128 x 128 tile.  Two of its workgroups share a
//    CU, so one's epilogue overlaps the other's main loop (QKV 4096+2048 x 4096, M = 512:
//    58.8 us against 78.1 us for the pipelined 64 x 128 tile; context K/V with pairs: 147 us
//    against 230 us);
//  - the eight-wave 256-row tiles, register-staged, when one of them covers the problem in rounds
//    of 256 workgroups that are at least 85% full (gate/up, LM head).  The register-staged
//    256 x 192 tile runs gate/up 2-9 % faster per step than its DMA form on the boxes measured,
//    the 256 x 256 the LM head equally fast;
//  - M <= 128 with K >= 8192: the deep 128 x 128 tile, which may split K;
//  - else the pipelined 64 x 128 tile when it gives at most 320 tiles (small N); else the
//    largest pipelined tile that still gives every CU work in whole rounds (at least two tiles
//    per CU), or the one with the most tiles.
static int choose_cfg(int kind, int M, int N, int K, int batch, int gateup, int F, bool pair) {
  auto tiles_of = [&](int c) {
    const int n = gateup ? ceil_div(F, kCfgBN[c] / 2) * kCfgBN[c] : N;
    return ceil_div(M, kCfgBM[c]) * ceil_div(n, kCfgBN[c]) * batch;
  };
  // M <= 64 rows: the skinny tiles, which read every weight element once (measured on the
  // SpecDiff-2-shaped drafter at 32 and 64 rows, faster than every other tile for each
  // projection); 32-row tiles for Q/K/V even at 64 rows
  if (M <= 32 || (M <= 64 && (kind == EPI_QKV || kind == EPI_CTXKV))) return 18;
  if (M <= 64) return 17;
  // a bf16 pair on at most 128 rows: the register-staged 256 x 192 tile as pair rows for gate/up
  // (one round of 198 units at the SpecDiff-2 shape; 2.37 against 3.76 ms per call for the
  // 128 x 128 tile)
  if (pair && M <= 128 && gateup) return 15;
  // the LM head with a pair on at most 128 rows: the register-staged 256 x 128 tile as pair rows
  // (SpecDiff-2 shape, 128 rows, V = 152,064: 0.338 against 0.374 ms per step for the four-wave
  // 128 x 128 pair tile)
  if (pair && M <= 128 && (kind == EPI_ARGMAX || kind == EPI_STORE_F32) && N >= 65536) return 16;
  if (M >= 64 && (pair || kind == EPI_QKV || kind == EPI_CTXKV)) return 10;
  // at most 128 rows without a pair: 128-row tiles rather than half-empty 256-row ones
  // (GPT-OSS-20B shape, 128 and 112 rows: gate/up 0.418 -> 0.367 ms per step with the
  // four-wave 128 x 128 tile, LM head 0.360 -> 0.299 ms with the pipelined 128 x 128 tile)
  if (!pair && M <= 128 && gateup) return 10;
  if (!pair && M <= 128 && (kind == EPI_ARGMAX || kind == EPI_STORE_F32) && N >= 65536) return 4;
  if (!pair && kind != EPI_QKV && kind != EPI_CTXKV && M > 128) {
    // the register-staged forms of the 256 x 256 and 256 x 192 tiles (14, 15)
    int best = -1;
    double best_fill = 0.85;
    for (int c : {14, 15}) {
      const int t = tiles_of(c);
      const double fill = (double)t / (256.0 * ceil_div(t, 256));
      if (t >= 192 && fill > best_fill) { best = c; best_fill = fill; }
    }
    if (best >= 0) return best;
  }
  if (M <= 128 && K >= 8192) return 10;
  if (tiles_of(3) <= 320) return 3;
  static const int order[4] = {0, 1, 4, 5};
  int best = 5, best_tiles = 0;
  for (int c : order) {
    const int tiles = tiles_of(c);
    if (tiles >= 512) return c;
    if (tiles > best_tiles) { best = c; best_tiles = tiles; }
  }
  return best;
}

// Time (us) of a tile choice, a model fitted to measurements on MI355X of the drafter's shapes
// (M = 128 .. 512 rows, N = 2k .. 6k, K = 3.5k .. 19k, weights streamed from HBM, store and
// residual epilogues; within about 10% of the measured time).  A unit (one workgroup) costs a
// fixed start plus a time per k stage; the stage time is set by the bytes each CU pulls from L2
// per stage, and units beyond one per CU share it: in whole rounds for the one-per-CU tiles (3,
// 16), proportionally past 192 units for the 128 x 128 tile, two of which fit on a CU (with a
// bf16 pair one, in whole rounds).  A split adds the reduction kernel (its launch plus writing
// and reading the fp32 partials); without a split the rotation and cache-scatter epilogues run
// inside the main kernel (about 4.2 us per million outputs for Q/K/V, 1.3 for the context K/V).
//   3: pipelined 64 x 128, 64-wide stages: 6.7 + 0.455 per stage
//   10: four-wave 128 x 128, 32-wide stages: 5.3 + 0.356 per stage (x 1.5 with a bf16 pair A,
//       whose units then share no CU: whole rounds of 256)
//   16: register-staged eight-wave 256 x 128, 64-wide stages: 10.4 + 0.88 per stage
static double model_us(int kind, int cfg, int M, int Nv, int K, int batch, int S, bool pair,
                       bool norm) {
  const double units = (double)ceil_div(M, kCfgBM[cfg]) * ceil_div(Nv, kCfgBN[cfg]) * batch * S;
  double t;
  if (cfg == 10)
    // with a bf16 pair the tile's six-stage ring (144 KB of LDS) leaves one unit per CU
    t = 5.3 + 0.356 * (pair ? 1.5 : 1.0) * (K / 32.0 / S) *
              (pair ? std::ceil(units / 256.0) : std::max(1.0, units / 192.0));
  else if (cfg == 16)
    t = 10.4 + 0.88 * (K / 64.0 / S) * std::ceil(units / 256.0);
  else
    t = 6.7 + 0.455 * (K / 64.0) * std::ceil(units / 256.0);
  if (S > 1)
    t += 1.5 + 0.36e-6 * units * kCfgBM[cfg] * kCfgBN[cfg] * 4.0;
  else if (kind == EPI_QKV && is_deep(cfg))
    t += 4.2e-6 * (double)M * Nv * batch;
  else if (kind == EPI_CTXKV && is_deep(cfg))
    t += 1.3e-6 * (double)M * Nv * batch;
  // a requested residual norm: inside the split reduction it adds the normalised rows' writes;
  // otherwise it is a launch of its own that reads the residual back
  const bool fuses = S > 1 && ((cfg == 16 && !pair) || (cfg >= 8 && cfg <= 10));
  if (norm) t += fuses ? 0.5e-6 * M * Nv : 2.0 + 1.5e-6 * M * Nv;
  return t;
}

// The library's tile and split: the heuristic tile of choose_cfg, and where that is the 64 x 128
// or the 128 x 128 tile, the fastest under model_us of it and of the 128 x 128 and 256 x 128
// (M >= 192, no bf16 pair) tiles with splits of 2 .. 8 (each unit keeps at least 4 stages of
// 32, or 2 of 64).
struct TileChoice {
  int cfg, split;
};
static TileChoice choose_tile(int kind, int M, int N, int K, int batch, int gateup, int F,
                              bool pair, bool norm) {
  const int base = choose_cfg(kind, M, N, K, batch, gateup, F, pair);
  if (is_skinny(base)) {
    // split K in powers of two while there are fewer than 1024 units and each unit keeps at
    // least 7 k stages of 64 (measured at 32 and 64 rows: Q/K/V and O best at 8, down at 16,
    // gate/up at 4)
    const int nv = gateup ? ceil_div(F, 64) * 128 : N;
    const int tiles = ceil_div(M, kCfgBM[base]) * ceil_div(nv, 128) * batch;
    int S = 1;
    while (S < 16 && tiles * S < 1024 && K / 64 / (2 * S) >= 7) S *= 2;
    return {base, S};
  }
  if (gateup || (base != 3 && base != 10)) return {base, 1};
  TileChoice best{base, 1};
  double best_t = model_us(kind, base, M, N, K, batch, 1, pair, norm);
  static const int cand[6] = {1, 2, 3, 4, 6, 8};
  for (int cfg : {10, 16}) {
    // (the 256 x 128 tile as pair rows measured slower than the 128 x 128 tile with its split
    // on the SpecDiff-2 shape's Q/K/V, O and down projections: 0.97, 0.84, 1.79 ms per call
    // against 0.82, 0.73, 1.66)
    if (cfg == 16 && (pair || M < 192)) continue;
    for (int S : cand) {
      if (cfg == 10 ? K / 32 / S < 4 : K / 64 / S < 2) break;
      const double t = model_us(kind, cfg, M, N, K, batch, S, pair, norm);
      if (t < best_t) { best = {cfg, S}; best_t = t; }
    }
  }
  return best;
}

GemmPlan plan_gemm(int dtype, int kind, int cfg, int M, int N, int K, int batch, int gateup,
                   int F, bool pair, bool split_ok, int split_req, bool norm) {
  GemmPlan p{};
  p.split = 1;
  if (dtype != 1) {
    p.cfg = -1;
    p.bn = FN;
    return p;
  }
  // QKV / context K/V tiles stay at 128 columns: they must not straddle the Q/K/V segment
  // boundaries (multiples of 128)
  const bool n128 = kind == EPI_QKV || kind == EPI_CTXKV;
  const bool chosen = cfg >= 0 && cfg < kNumCfg;
  int lib_split = 1;
  if (!chosen) {
    const TileChoice c = choose_tile(kind, M, N, K, batch, gateup, F, pair,
                                     norm && kind == EPI_RESID && batch == 1);
    cfg = c.cfg;
    lib_split = c.split;
  }
  if (n128 && kCfgBN[cfg] != 128)
    cfg = cfg >= 14 ? 16 : cfg >= 11 ? 13 : is_deep(cfg) ? (kCfgBM[cfg] == 256 ? 8 : 10)
                                        : (kCfgBM[cfg] == 256 ? 1 : 4);
  if (pair) cfg = pair_cfg(cfg, M);
  auto nvirt = [&](int c) { return gateup ? ceil_div(F, kCfgBN[c] / 2) * kCfgBN[c] : N; };
  p.cfg = cfg;
  p.bn = kCfgBN[cfg];
  if (is_deep(cfg) && split_ok) {
    if (split_req > 1) {
      // a requested split keeps each unit at least one k stage
      p.split = std::min(split_req, std::max(1, K / 64));
    } else if (split_req == 0) {
      // the library's own tile comes with its split; a caller's tile gets the generic estimate
      p.split = chosen ? choose_split(cfg, M, nvirt(cfg), K, batch) : lib_split;
    }
  }
  p.tiles = ceil_div(M, kCfgBM[cfg]) * ceil_div(nvirt(cfg), kCfgBN[cfg]) * batch;
  p.part_bytes = p.split > 1 ? (size_t)p.tiles * p.split * kCfgBM[cfg] * kCfgBN[cfg] * 4 : 0;
  return p;
}

bool gemm_fuses_norm(const GemmPlan& p, bool pair, int batch) {
  if (p.cfg < 0 || p.split <= 1 || batch != 1) return false;
  // the skinny tiles, the register-staged 256-row tiles without pair rows, and the deep-ring
  // four-wave tiles (a bf16 pair there is a second A part, summed in the accumulators)
  return is_skinny(p.cfg) || (p.cfg >= 14 && p.cfg <= 16 && !pair) ||
         (p.cfg >= 8 && p.cfg <= 10);
}

template <int KIND>
static void launch_kind(int dtype, int cfg, int split, GemmArgs a, const EpiArgs& e, int batch,
                        hipStream_t s, bool* norm_done) {
  if (norm_done) *norm_done = false;
  if (dtype == 1) {
    const int F = a.seg[0].n1 - a.seg[0].n0;
    const bool want_norm = KIND == EPI_RESID && e.norm_g && resid_norm_fits(a.N, e.ldc);
    GemmPlan p = plan_gemm(dtype, KIND, cfg, a.M, a.N, a.K, batch, a.gateup, F,
                           a.A2 != nullptr, a.part != nullptr, split, want_norm);
    if (p.split > 1 && p.part_bytes > a.part_cap) p.split = 1;
    a.split = p.split;
    // the residual's norm rides on a split-K reduction that sees whole rows
    const bool fuse = want_norm && gemm_fuses_norm(p, a.A2 != nullptr, batch);
    EpiArgs ee = e;
    if (!fuse) ee.norm_g = nullptr;
    if (a.A2) launch_cfg<KIND, true>(p.cfg, a, ee, batch, s);
    else launch_cfg<KIND, false>(p.cfg, a, ee, batch, s);
    if (norm_done) *norm_done = fuse;
  } else {
    if (a.gateup) a.N = ceil_div(a.seg[0].n1 - a.seg[0].n0, FN / 2) * FN;
    dim3 grid(ceil_div(a.N, FN), ceil_div(a.M, FM), batch);
    hipLaunchKernelGGL(gemm_f32_kernel<KIND>, grid, dim3(256), 0, s, a, e);
  }
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, const EpiArgs& e, int batch,
                       hipStream_t s, int cfg, int split, bool* norm_done) {
  if (norm_done) *norm_done = false;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  bool* nd = norm_done;
  switch (e.kind) {
    case EPI_STORE_F32: launch_kind<EPI_STORE_F32>(dtype, cfg, split, a, e, batch, s, nd); break;
    case EPI_RESID: launch_kind<EPI_RESID>(dtype, cfg, split, a, e, batch, s, nd); break;
    case EPI_QKV: launch_kind<EPI_QKV>(dtype, cfg, split, a, e, batch, s, nd); break;
    case EPI_CTXKV: launch_kind<EPI_CTXKV>(dtype, cfg, split, a, e, batch, s, nd); break;
    case EPI_SWIGLU: launch_kind<EPI_SWIGLU>(dtype, cfg, split, a, e, batch, s, nd); break;
    case EPI_ARGMAX: launch_kind<EPI_ARGMAX>(dtype, cfg, split, a, e, batch, s, nd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dbd
