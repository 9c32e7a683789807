// Host-side shape rules shared by the launchers of libdbd.so.  Plain C++ (no HIP), so that host
// tests can compile and check them with an ordinary C++ compiler.
#pragma once

#include <stdint.h>

namespace dbd {

// resid_norm_kernel: one 1,024-thread workgroup per row, each thread holding up to two
// four-float vectors of the row, so a row has at most 2 * 1024 * 4 columns.
constexpr int kResidNormThreads = 1024;
constexpr int kResidNormVecsPerThread = 2;
constexpr int kResidNormMaxCols = kResidNormThreads * kResidNormVecsPerThread * 4;

// Whether the split-K reduction of a residual projection may also write the RMSNorm of its rows
// (resid_norm_kernel): the row must fit one workgroup, be made of whole 16-byte vectors (n_cols a
// multiple of 4 floats; the residual and the partials are 256-byte aligned buffers) and be
// stored densely (row stride ldc == n_cols, as the row-major partials are).
constexpr bool resid_norm_fits(int n_cols, int64_t ldc) {
  return n_cols > 0 && n_cols <= kResidNormMaxCols && n_cols % 4 == 0 && ldc == n_cols;
}

// ---------------------------------------------------------------- balanced bf16 attention
// Query rows per row block (four waves of 16 rows), keys per chunk (32 KB of K and V whatever
// the head size), and the workgroups and chunks loaded ahead unless overridden.
constexpr int kAttnRows = 64;
constexpr int kAttnWorkgroups = 512;
constexpr int kAttnMaxWorkgroups = 8192;
constexpr int kAttnDepth = 1;
constexpr int attn_chunk_keys(int hd) { return 8192 / hd; }
constexpr int attn_row_blocks(int rows) { return (rows + kAttnRows - 1) / kAttnRows; }

// A segment is one (sequence, kv head, row block) with ceil(keys / chunk) chunks; the segments
// are laid end to end in that order and the resulting T chunks are cut into P ranges, workgroup
// j taking [attn_range_lo(j), attn_range_lo(j + 1)).  P is the launch's workgroup count or T if
// that is smaller, so that no range is empty.
constexpr int64_t attn_active_workgroups(int64_t launched, int64_t T) {
  return launched < T ? launched : T;
}
constexpr int64_t attn_range_lo(int64_t j, int64_t T, int64_t P) { return j * T / P; }
// The workgroup whose range holds chunk x: the largest j with attn_range_lo(j) <= x.
constexpr int64_t attn_range_owner(int64_t x, int64_t T, int64_t P) {
  return ((x + 1) * P - 1) / T;
}
// The first workgroup whose range starts at chunk x or later: ceil(x P / T).
constexpr int64_t attn_first_range_from(int64_t x, int64_t T, int64_t P) {
  return (x * P + T - 1) / T;
}
// The sequence holding chunk x (0 <= x < T): the first n whose chunks end past x, found by
// bisection over pref (pref[n] = chunks per segment of the sequences before n, pref[batch] the
// total); sequences without keys end where they start and are never returned.
template <typename I>
constexpr int attn_seq_of_chunk(const I* pref, int batch, int64_t segs, int64_t x) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)pref[mid + 1] * segs > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}
// Workgroup j's range is computed by the launched workgroup whose blockIdx.x is
// attn_bid_of_range(j).  Consecutive workgroups go round-robin to the 8 XCDs: when every launched
// workgroup has a range (and their count is a multiple of 8), XCD x takes the contiguous run of
// ranges [x P / 8, (x + 1) P / 8), so that the row blocks of one (sequence, kv head), which read
// the same keys, share an L2; otherwise range j is blockIdx.x j.
constexpr bool attn_xcd_order(int launched, int64_t active) {
  return active == launched && launched % 8 == 0;
}
constexpr int attn_range_of_bid(int bid, int launched, int64_t active) {
  return attn_xcd_order(launched, active) ? (bid % 8) * (launched / 8) + bid / 8 : bid;
}
constexpr int attn_bid_of_range(int j, int launched, int64_t active) {
  return attn_xcd_order(launched, active) ? (j % (launched / 8)) * 8 + j / (launched / 8) : j;
}
// Partial slot of the piece of segment s that workgroup j computes.  Along the chunk axis every
// new piece advances j, s or both, so distinct pieces get distinct slots, all below P + the
// number of segments.
constexpr int64_t attn_partial_slot(int64_t j, int64_t s) { return j + s; }
constexpr int64_t attn_partial_slots(int64_t P, int64_t segments) { return P + segments; }

}  // namespace dbd
