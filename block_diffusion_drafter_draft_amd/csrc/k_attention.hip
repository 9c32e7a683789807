// Block attention over the cache (DFlare page, section on parallel drafting: attention inside
// the block is bidirectional and the block sees the whole context).  No mask: every row of the
// block attends to all cache positions 0 .. P+B-1 of its sequence (context, then the block's own
// keys, which draft_block wrote into the cache first).
//
// bf16: a fixed number of workgroups share the (sequence, kv head, query row block) segments'
// key chunks equally (below); each wave holds 16 query rows of the GQA group (rows r = b + B*h
// over block positions b and the group's heads h).  Per chunk the K rows and V (kept in the cache
// in blocks of 8 positions, [cap/8][hd][8]) are staged in LDS; each wave computes S^T = K.Q^T
// with the gfx950 MFMA 16x16x32 bf16, so that its lanes hold 8 consecutive keys of one query
// (keys are permuted inside the MFMA tiles), runs the online softmax in fp32 (exp2 domain) and
// feeds P^T straight from registers into O^T += V^T.P^T.  fp32: one workgroup per (key split,
// kv head, sequence).  Pieces of a segment computed by several workgroups are merged by a
// combine kernel in chunk order.
#include <algorithm>

#include "dbd_internal.h"

namespace dbd {

// ------------------------------------------------------------------ helpers
template <int HD>
__device__ __forceinline__ int kswz(int row, int c) {
  // K tile row = HD*2 bytes.  The S^T operand reads rows {8(i/4) + i%4 (+4)}: spread them over
  // distinct 16-byte slots.
  if constexpr (HD == 128) return c ^ ((row & 3) | (((row >> 3) & 3) << 2));
  else return c ^ (((row >> 1) & 1) | (((row >> 3) & 3) << 1));
}
__device__ __forceinline__ int vswz(int row, int c) { return c ^ ((row >> 1) & 7); }

// Maximum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48): the gfx950 row
// swaps exchange rows 1 <-> 0 and 3 <-> 2 (16 lanes) and the two 32-lane halves.
__device__ __forceinline__ float group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ------------------------------------------------------------------ balanced bf16 attention
// Work is counted in chunks of KCH keys.  A segment is one (sequence n, kv head g, row block rb)
// with ceil(L_n / KCH) chunks; the segments lie end to end in (n, g, rb) order and their T
// chunks are cut into P equal ranges, one per workgroup, whatever the context lengths, so every
// workgroup streams the same number of bytes.  The part of a segment one range holds (a piece,
// the whole segment or a part of it) is published as a partial, its unnormalised output rows
// and (max, sum) per row, and attn_stream_combine_kernel merges the pieces of every segment and
// writes the output.
//
// Each workgroup is four waves of 16 query rows (one row block).  Chunk x of the range is
// staged global -> registers -> LDS slot x & 1; DEPTH chunks are loaded ahead (two register
// sets at DEPTH 2), so while chunk x is consumed from LDS the next DEPTH are in flight.  One
// barrier per chunk: slot x & 1 is rewritten two chunks later, after the barrier of chunk x + 1.
// QPAIR: the queries come as a bf16 (high, low) pair and every score is the sum of two MFMAs,
// K.Q_hi + K.Q_lo, so the scores see ~16 significant bits of the rotated query instead of 8
// (the keys stay bf16 as stored in the cache).
// cache policy of the K/V loads: non-temporal (read once per step)
constexpr int kNonTemporal = 2;

template <int HD>
struct AttnChunk {
  static constexpr int KCH = 8192 / HD;             // keys per chunk: 16 KB of K, 16 KB of V
  static constexpr int KC = HD / 8;                 // 16-byte pieces per K row
  static constexpr int NT = 256;
  static constexpr int KI = KCH * KC / NT;          // K pieces staged per thread
  static constexpr int VI = HD * (KCH / 8) / NT;    // V pieces staged per thread
  static_assert(KCH == attn_chunk_keys(HD) && KCH % 64 == 0 && KI == 4 && VI == 4, "chunk");
};

template <int HD, bool QPAIR, int DEPTH>
__global__ __launch_bounds__(256) void attn_stream_kernel(AttnArgs a) {
  using C = AttnChunk<HD>;
  constexpr int KCH = C::KCH, KC = C::KC, NT = C::NT, KI = C::KI, VI = C::VI;
  // K slot: [KCH][HD] rows; V slot: [KCH / 64][HD][64], i.e. 64-key halves with 128-byte rows
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KCH * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][HD * KCH];
  // one dependent load: this workgroup's share, written by the plan kernel
  const AttnPlan p0 = a.plan[blockIdx.x];
  const int64_t lo = p0.lo, hi = p0.hi;
  if (lo >= hi) return;
  const int j = p0.j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.block_len * a.grp;
  const int RB = attn_row_blocks(R);
  const int segs = a.kvh * RB;

  struct Cur {
    int n, seg, chunk, cn, L;
  };
  auto set_seq = [&](Cur& c) __attribute__((always_inline)) {
    c.L = __builtin_amdgcn_readfirstlane(a.seq_keys[c.n]);
    c.cn = c.L > 0 ? (c.L + KCH - 1) / KCH : 0;
  };
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    if (++c.chunk < c.cn) return;
    c.chunk = 0;
    if (++c.seg < segs) return;
    c.seg = 0;
    for (;;) {                                  // the next sequence with keys
      if (++c.n >= a.batch) {
        c.cn = 0;
        return;
      }
      set_seq(c);
      if (c.cn > 0) return;
    }
  };
  Cur cc;
  cc.n = __builtin_amdgcn_readfirstlane(p0.n);
  cc.seg = __builtin_amdgcn_readfirstlane(p0.seg);
  cc.chunk = __builtin_amdgcn_readfirstlane(p0.chunk);
  cc.L = __builtin_amdgcn_readfirstlane(p0.keys);
  cc.cn = (cc.L + KCH - 1) / KCH;
  Cur lc = cc;

  // queries of the current segment's row block: this lane's query row (column of S^T / O^T)
  bf16x8 qf[HD / 32], qlf[QPAIR ? HD / 32 : 1];
  int r = 0, b = 0, h = 0;
  bool rvalid = false, wactive = false;
  f32x4 acc[HD / 16];
  float m_run = -INFINITY, l_run = 0.f;
  auto begin = [&](const Cur& c) __attribute__((always_inline)) {
    const int g = c.seg / RB, rb = c.seg % RB;
    r = rb * kAttnRows + wave * 16 + (lane & 15);
    rvalid = r < R;
    wactive = rb * kAttnRows + wave * 16 < R;
    b = rvalid ? r % a.block_len : 0;
    h = rvalid ? r / a.block_len : 0;
    const int64_t qo = ((int64_t)c.n * a.block_len + b) * a.qd + (g * a.grp + h) * HD +
                       (lane >> 4) * 8;
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
    // wait for the queries here, at a piece's start: otherwise every later chunk's MFMAs would
    // wait behind the loads issued before the queries on some path, i.e. for the next chunk too
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // A chunk of K ([cap][HD] per (n, g)) and of V ([cap/8][HD][8]) is one contiguous run of
  // KCH * HD * 2 bytes starting chunk * KCH * HD * 2 bytes into the (n, g) region: 16-byte
  // piece idx sits idx * 16 bytes in, a per-thread offset plus a uniform one.  The buffer
  // resource spans the region, so a chunk running past the capacity reads zeros.  The loads are
  // non-temporal: K and V are read once per step (3-6 % faster than cached loads; walking each
  // chunk's 1 KB blocks in a per-workgroup order, against all workgroups reading the same
  // offsets of their 16 KB-aligned chunks at once, changed nothing).
  auto issue = [&](u32x4 (&kr)[KI], u32x4 (&vr)[VI], const Cur& c, bool real)
                   __attribute__((always_inline)) {
    const int64_t region = ((int64_t)c.n * a.kvh + c.seg / RB) * a.cap * HD;
    const int bytes = real ? a.cap * HD * 2 : 0;   // 0: every load is out of range, reads 0
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>((const bf16*)a.kv_k + region), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>((const bf16*)a.kv_v + region), (short)0, bytes, 0x00020000);
    const int base = c.chunk * KCH * HD * 2;
#pragma unroll
    for (int q = 0; q < KI; ++q)
      kr[q] = __builtin_amdgcn_raw_buffer_load_b128(krs, tid * 16, base + q * NT * 16,
                                                    kNonTemporal);
#pragma unroll
    for (int q = 0; q < VI; ++q)
      vr[q] = __builtin_amdgcn_raw_buffer_load_b128(vrs, tid * 16, base + q * NT * 16,
                                                    kNonTemporal);
  };
  // V piece idx = (8-key block c, dimension d); positions at or past the end read as 0 (their
  // probabilities are 0, but the cache beyond the keys may hold anything)
  auto store = [&](const u32x4 (&kr)[KI], const u32x4 (&vr)[VI], int slot, int c0, int k_end) {
    bf16* ks = Ks[slot];
    bf16* vs = Vs[slot];
#pragma unroll
    for (int q = 0; q < KI; ++q) {
      const int idx = tid + q * NT, row = idx / KC, c = idx % KC;
      *reinterpret_cast<u32x4*>(ks + row * HD + kswz<HD>(row, c) * 8) = kr[q];
    }
#pragma unroll
    for (int q = 0; q < VI; ++q) {
      const int idx = tid + q * NT, c = idx / HD, d = idx % HD;
      const int k0 = c0 + c * 8;
      u32x4 v = vr[q];
      if (k0 + 8 > k_end) {
        bf16* e = reinterpret_cast<bf16*>(&v);
        for (int t = 0; t < 8; ++t)
          if (k0 + t >= k_end) e[t] = (bf16)0.f;
      }
      *reinterpret_cast<u32x4*>(vs + (c >> 3) * HD * 64 + d * 64 + vswz(d, c & 7) * 8) = v;
    }
  };

  // key rows of the two S^T tiles in a 32-key group: lane group G = lane/16 ends up holding
  // keys 8G .. 8G+7
  const int i16 = lane & 15;
  const int kr0 = 8 * (i16 >> 2) + (i16 & 3);
  const int kr1 = kr0 + 4;
  // One chunk: the scores of all its keys first (two MFMA tiles of 16 keys per 32-key group),
  // one maximum and at most one rescale per chunk, then P^T into O^T.
  constexpr int NS = KCH / 32;                  // 32-key groups per chunk
  auto consume = [&](int slot, int c0, int k_end) __attribute__((always_inline)) {
    const bf16* ks = Ks[slot];
    const bf16* vs = Vs[slot];
    f32x4 sc[NS][2];
#pragma unroll
    for (int sub = 0; sub < NS; ++sub) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const int row0 = sub * 32 + kr0, row1 = sub * 32 + kr1;
#pragma unroll
      for (int ks_ = 0; ks_ < HD / 32; ++ks_) {
        const int c = ks_ * 4 + (lane >> 4);
        const bf16x8 k0v = *reinterpret_cast<const bf16x8*>(ks + row0 * HD + kswz<HD>(row0, c) * 8);
        const bf16x8 k1v = *reinterpret_cast<const bf16x8*>(ks + row1 * HD + kswz<HD>(row1, c) * 8);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0v, qf[ks_], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1v, qf[ks_], s1, 0, 0, 0);
        if constexpr (QPAIR) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0v, qlf[ks_], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1v, qlf[ks_], s1, 0, 0, 0);
        }
      }
      sc[sub][0] = s0;
      sc[sub][1] = s1;
    }
    // lane holds S^T[c0 + 32 sub + 8 (lane/16) + 4 t + e][query]; keys past the end -> -inf
    // (their K rows are whatever the cache holds there, their V rows were zeroed)
    if (c0 + KCH > k_end) {
#pragma unroll
      for (int sub = 0; sub < NS; ++sub) {
        const int kb = c0 + sub * 32 + 8 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb + 4 * t + e >= k_end) sc[sub][t][e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NS; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[sub][t][0], sc[sub][t][1]),
                             fmaxf(sc[sub][t][2], sc[sub][t][3])));
    mx = group_max4(mx);
    const float mxs = mx * a.scale_log2;
    // The running maximum m_run (log2 units) is raised only when a score passes it, and O and l
    // are rescaled only when some query of the wave needs it.  (A reference allowed to lag the
    // maximum by up to 8 skips more rescales but leaves the dominant probabilities rounded to
    // bf16 instead of exactly 1: logits rel-L2 1.69e-2 -> 1.73e-2 at the bench shape.)
    const bool raise = mxs > m_run;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mxs : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < NS; ++sub) {
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[sub][t][e], a.scale_log2, -m_run));
          ps += p;
          pb[4 * t + e] = (bf16)p;
        }
      const bf16* vh = vs + (sub >> 1) * HD * 64;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) {
        const int d = dt * 16 + (lane & 15);
        const int c = (sub & 1) * 4 + (lane >> 4);
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(vh + d * 64 + vswz(d, c) * 8);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb, acc[dt], 0, 0, 0);
      }
    }
    l_run += ps;
  };
  // End of a piece: its unnormalised O^T and (m, l) go to the piece's partial slot, rows in
  // order; the combine kernel merges the pieces of every segment and writes the output.
  auto publish = [&](const f32x4 (&o)[HD / 16], float m, float lsum, int n, int seg)
                     __attribute__((always_inline)) {
    // per-lane partial sums of the 4 lane groups belong to the same query
    float l = lsum + __shfl_xor(lsum, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int64_t slot = attn_partial_slot(j, (int64_t)n * segs + seg);
    float* po = a.part_o + (slot * kAttnRows + wave * 16 + (lane & 15)) * HD;
    // o[dt][i] = O^T[d = dt*16 + 4*(lane/16) + i][query]; rows past R are ignored
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
      *reinterpret_cast<f32x4*>(po + dt * 16 + (lane >> 4) * 4) = o[dt];
    if (lane < 16) a.part_ml[slot * kAttnRows + wave * 16 + lane] = make_float2(m, l);
  };
  // Stores count in vmcnt like the loads on gfx9: stores issued on some paths of the loop make
  // the compiler's waits on the following steps cover every load in flight.  So a piece that
  // ends before the range does is kept in registers (one such piece) and published after the
  // loop with the range's last piece; a second one in the same range is published at once and
  // followed by a full wait, which makes the counts exact again (at the bench shape a range
  // rarely holds more than one segment end).
  f32x4 stash[HD / 16];
  float stash_m = 0.f, stash_l = 0.f;
  int stash_n = -1, stash_seg = 0;

  u32x4 kra[KI], vra[VI], krb[KI], vrb[VI];
  // Every step issues one chunk's loads, so that the count of loads behind each register set is
  // the same on every path and the waits before the LDS stores cover only the chunk stored (a
  // conditional issue makes the compiler wait for every load in flight).  Past the range's last
  // chunk the loads go through a resource of size 0: they return zeros without a memory access
  // (reloading the last chunk instead re-read it from HBM, the loads being non-temporal).
  int64_t ln = lo;                              // next chunk to load, at the load cursor
  auto issue_next = [&](u32x4 (&kr)[KI], u32x4 (&vr)[VI]) __attribute__((always_inline)) {
    const bool real = ln < hi;
    issue(kr, vr, lc, real);
    if (real && ++ln < hi) advance(lc);
  };
  issue_next(kra, vra);
  if (DEPTH == 2) issue_next(krb, vrb);
  begin(cc);                                    // the queries load while the first chunks do
  int64_t x = lo;
  int last_n = cc.n, last_seg = cc.seg;         // segment of the chunk consumed last
  auto step = [&](auto par) __attribute__((always_inline)) {
    constexpr int S = decltype(par)::value;     // LDS slot and (DEPTH 2) register set
    auto& kr = (DEPTH == 2 && S == 1) ? krb : kra;
    auto& vr = (DEPTH == 2 && S == 1) ? vrb : vra;
    const int c0 = cc.chunk * KCH;
    store(kr, vr, S, c0, cc.L);
    issue_next(kr, vr);
    __syncthreads();
    if (wactive) consume(S, c0, cc.L);
    const bool seg_end = cc.chunk == cc.cn - 1;
    if (seg_end && x + 1 < hi) {                // a piece ending before the range does
      if (stash_n < 0) {
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) stash[dt] = acc[dt];
        stash_m = m_run;
        stash_l = l_run;
        stash_n = cc.n;
        stash_seg = cc.seg;
      } else {
        publish(acc, m_run, l_run, cc.n, cc.seg);
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
      }
    }
    last_n = cc.n;
    last_seg = cc.seg;
    advance(cc);
    ++x;
    if (seg_end && x < hi) begin(cc);
  };
  while (x + 1 < hi) {
    step(std::integral_constant<int, 0>());
    step(std::integral_constant<int, 1>());
  }
  if (x < hi) step(std::integral_constant<int, 0>());
  publish(acc, m_run, l_run, last_n, last_seg);
  if (stash_n >= 0) publish(stash, stash_m, stash_l, stash_n, stash_seg);
}

// Chunk schedule, one 1,024-thread workgroup: pref[n] = chunks of the sequences before n (every
// segment of a sequence has its chunk count), total = (T over all segments, active workgroups
// P), and for every launched workgroup its share: range j, chunks [lo, hi) and the (sequence,
// segment, chunk) at lo.
__device__ int block_excl_scan_1024(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = s_w[w];
      s_w[w] = run;
      run += t;
    }
    s_w[16] = run;
  }
  __syncthreads();
  const int ex = s_w[wave] + x - v;
  *total = s_w[16];
  __syncthreads();
  return ex;
}

// Sequences whose chunk prefix the plan kernel keeps in LDS for its search; larger batches walk
// the workgroups of each sequence instead.
constexpr int kPlanLdsSeqs = 8192;

__global__ __launch_bounds__(1024) void attn_plan_kernel(const int32_t* __restrict__ seq_keys,
                                                        int batch, int kch, int segs, int launched,
                                                        AttnPlan* __restrict__ plan,
                                                        int32_t* __restrict__ pref,
                                                        int64_t* __restrict__ total) {
  __shared__ int s_w[17];
  __shared__ int s_pref[kPlanLdsSeqs + 1];
  const int tid = threadIdx.x;
  const bool in_lds = batch <= kPlanLdsSeqs;
  int carry = 0;
  for (int base = 0; base < batch; base += 1024) {
    const int n = base + tid;
    const int L = n < batch ? seq_keys[n] : 0;
    const int c = L > 0 ? (L + kch - 1) / kch : 0;
    int tot;
    const int ex = block_excl_scan_1024(c, s_w, &tot);
    if (n < batch) {
      pref[n] = carry + ex;
      if (in_lds) s_pref[n] = carry + ex;
    }
    carry += tot;
  }
  const int64_t T = (int64_t)carry * segs;
  const int P = (int)attn_active_workgroups(launched, T);
  if (tid == 0) {
    pref[batch] = carry;
    total[0] = T;
    total[1] = P;
    if (in_lds) s_pref[batch] = carry;
  }
  // launched workgroups without a range (all of them when no sequence has keys) get an empty
  // share
  for (int bid = tid; bid < launched; bid += 1024)
    if (attn_range_of_bid(bid, launched, P) >= P) plan[bid] = AttnPlan{0, 0, 0, 0, 0, 0, 0, 0};
  if (T == 0) return;
  if (in_lds) {
    __syncthreads();
    // range j: its first chunk x, the first sequence whose chunks end past x, the offset
    for (int j = tid; j < P; j += 1024) {
      const int64_t x = attn_range_lo(j, T, P);
      const int n = attn_seq_of_chunk(s_pref, batch, segs, x);
      const int c = s_pref[n + 1] - s_pref[n];
      const int64_t off = x - (int64_t)s_pref[n] * segs;
      plan[attn_bid_of_range(j, launched, P)] =
          AttnPlan{n, (int)(off / c), (int)(off % c), seq_keys[n], j, 0, x,
                   attn_range_lo(j + 1, T, P)};
    }
    return;
  }
  carry = 0;
  for (int base = 0; base < batch; base += 1024) {
    const int n = base + tid;
    const int L = n < batch ? seq_keys[n] : 0;
    const int c = L > 0 ? (L + kch - 1) / kch : 0;
    int tot;
    const int ex = block_excl_scan_1024(c, s_w, &tot);
    if (c > 0) {
      // the ranges that begin inside this sequence's chunks
      const int64_t S = (int64_t)(carry + ex) * segs, E = S + (int64_t)c * segs;
      for (int64_t jj = attn_first_range_from(S, T, P); jj < attn_first_range_from(E, T, P); ++jj) {
        const int64_t x = attn_range_lo(jj, T, P), off = x - S;
        plan[attn_bid_of_range((int)jj, launched, P)] =
            AttnPlan{n, (int)(off / c), (int)(off % c), L, (int)jj, 0, x,
                     attn_range_lo(jj + 1, T, P)};
      }
    }
    carry += tot;
  }
}

// Merge of the partials of the segments that several workgroups share.  grid (64 / 4, kvh * row
// blocks, N); each workgroup merges 4 query rows of one segment, thread = (row, 4 dimensions).
// The pieces of segment s are those of the workgroups owning its first to last chunk, in chunk
// order.
__global__ __launch_bounds__(128) void attn_stream_combine_kernel(AttnArgs a, int HD) {
  const int seg = blockIdx.y, n = blockIdx.z;
  const int64_t T = a.plan_total[0];
  const int P = (int)a.plan_total[1];
  const int L = a.seq_keys[n];
  if (T <= 0 || L <= 0) return;
  const int kch = attn_chunk_keys(HD);
  const int cn = (L + kch - 1) / kch;
  const int R = a.block_len * a.grp;
  const int RB = attn_row_blocks(R);
  const int segs = a.kvh * RB;
  const int64_t start = (int64_t)a.plan_pref[n] * segs + (int64_t)seg * cn;
  const int64_t w0 = attn_range_owner(start, T, P), w1 = attn_range_owner(start + cn - 1, T, P);
  const int dq = HD / 4;                        // float4 groups per row
  const int rl = blockIdx.x * 4 + threadIdx.x / dq;
  const int d4 = threadIdx.x % dq;
  const int r = (seg % RB) * kAttnRows + rl;
  if (threadIdx.x >= 4 * dq || r >= R) return;
  const int64_t sidx = (int64_t)n * segs + seg;
  // one pass over the pieces, four loads in flight at a time (a segment rarely has more
  // pieces; the 52 VGPRs this leaves let every workgroup of the launch be resident at once),
  // rescaling the running sums to each batch's maximum
  float m = -INFINITY, l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  constexpr int SU = 4;
  for (int64_t w = w0; w <= w1; w += SU) {
    float2 ml[SU];
    f32x4 po[SU];
#pragma unroll
    for (int q = 0; q < SU; ++q) {
      const int64_t ww = w + q;
      const bool ok = ww <= w1;                 // every range holds a chunk: no empty pieces
      const int64_t pr = attn_partial_slot(ok ? ww : w0, sidx) * kAttnRows + rl;
      ml[q] = ok ? a.part_ml[pr] : make_float2(-INFINITY, 0.f);
      po[q] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + pr * HD + 4 * d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = m;
#pragma unroll
    for (int q = 0; q < SU; ++q) mb = fmaxf(mb, ml[q].x);
    const float sc = exp2f(m - mb);              // 0 while nothing is merged yet
    l *= sc;
    o *= sc;
#pragma unroll
    for (int q = 0; q < SU; ++q) {
      const float wgt = exp2f(ml[q].x - mb);
      l += wgt * ml[q].y;
      o += wgt * po[q];
    }
    m = mb;
  }
  const float inv = 1.f / l;
  const int b = r % a.block_len, h = r / a.block_len;
  const int64_t off = ((int64_t)n * a.block_len + b) * a.qd + (seg / RB * a.grp + h) * HD + 4 * d4;
  bf16* out = (bf16*)a.out + off;
  bf16* out_lo = a.out_lo ? (bf16*)a.out_lo + off : nullptr;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float y = o[q] * inv;
    const bf16 hi = (bf16)y;
    out[q] = hi;
    if (out_lo) out_lo[q] = (bf16)(y - (float)hi);
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
static void launch_stream_q(const AttnArgs& a, hipStream_t s) {
  if (a.depth == 1)
    hipLaunchKernelGGL((attn_stream_kernel<HD, QP, 1>), dim3(a.workgroups), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_stream_kernel<HD, QP, 2>), dim3(a.workgroups), dim3(256), 0, s, a);
}
template <int HD>
static void launch_stream(const AttnArgs& a, hipStream_t s) {
  if (a.q_lo) launch_stream_q<HD, true>(a, s);
  else launch_stream_q<HD, false>(a, s);
}

hipError_t launch_attn_plan(const int32_t* seq_keys, int batch, int hd, int kvh, int rows,
                            int workgroups, AttnPlan* plan, int32_t* pref, int64_t* total,
                            hipStream_t s) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, s, seq_keys, batch,
                     attn_chunk_keys(hd), kvh * attn_row_blocks(rows), workgroups, plan, pref,
                     total);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, int hd, const AttnArgs& a, hipStream_t s) {
  const int R = a.block_len * a.grp;
  if (dtype == 1) {
    if (hd == 128) launch_stream<128>(a, s);
    else launch_stream<64>(a, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(attn_stream_combine_kernel, dim3(kAttnRows / 4, a.kvh * attn_row_blocks(R),
                                                        a.batch),
                       dim3(128), 0, s, a, hd);
  } else {
    dim3 grid(a.s_max, a.kvh, a.batch);
    dim3 cgrid(ceil_div(R, 4), a.kvh, a.batch);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 0, s, a, hd);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(attn_combine_kernel<float>, cgrid, dim3(128), 0, s, a, hd);
  }
  return hipGetLastError();
}

}  // namespace dbd
