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

}  // namespace dbd
