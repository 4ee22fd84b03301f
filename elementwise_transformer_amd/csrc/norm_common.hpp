// norm_common.hpp -- the row shape shared by the register-resident row
// kernels (RMSNorm, fused add+RMSNorm, LayerNorm): threads per row and
// vectors per thread from the row length alone, lane ownership, and the
// fixed-order row sum.
#pragma once

#include "et_common.hpp"

namespace et {
namespace {

// 16-byte vectors per thread in the register path: 4 for rows of 1024..4096
// vectors (256..1024 threads per row), 8 otherwise.
constexpr int kVPTMax = 8;
constexpr int kLargeTPR = 1024;  // threads per row in the two-pass path
// Issue the gain loads right after the row loads when a row spans several
// waves (its cross-wave reduction is long enough to hide them); for one-wave
// rows the extra registers cost more occupancy than they save.
constexpr int kWEarlyMinTPR = 128;
// Rows of at least this many vectors (up to 4096) take 4 vectors per thread.
constexpr int kVPT4MinVec = 1024;
// Threads per block when a row takes fewer (several rows per block).
constexpr int kNormBlock = 128;

template <int TPR>
struct NormShape {
  static constexpr int kBlock = TPR < kNormBlock ? kNormBlock : TPR;
  static constexpr int kRowsPerBlock = kBlock / TPR;
  static constexpr int kGroup = TPR < 64 ? TPR : 64;  // lanes of one row inside a wave
  static constexpr int kWavesPerRow = TPR > 64 ? TPR / 64 : 1;
};

// Reduce a per-thread partial over the TPR threads that own one row.
template <int TPR>
__device__ inline float row_sum(float part, float* lds, int row_in_block, int lane_in_row) {
  using Sh = NormShape<TPR>;
  float s = group_sum<Sh::kGroup>(part);
  if constexpr (Sh::kWavesPerRow > 1) {
    const int wave_in_row = lane_in_row / 64;
    if ((lane_in_row & 63) == 0) lds[row_in_block * Sh::kWavesPerRow + wave_in_row] = s;
    __syncthreads();
    s = 0.0f;
#pragma unroll
    for (int w = 0; w < Sh::kWavesPerRow; ++w) s += lds[row_in_block * Sh::kWavesPerRow + w];
  }
  return s;
}

// Vector slot k of thread t in its row.  Rows of one wave or less: slot k is
// the k-th TPR-vector stripe.  Longer rows: each wave owns a contiguous run of
// 64 * VPT vectors, slot k of lane l at k * 64 + l inside it.
template <int TPR, int VPT>
__device__ inline int own(int k, int t) {
  if constexpr (TPR > 64) {
    return (t / 64) * (64 * VPT) + k * 64 + (t % 64);
  } else {
    return k * TPR + t;
  }
}

// Launch shape from the row length alone: vectors per thread (4 for rows of
// 1024..4096 vectors, else 8) and threads per row (the smallest power of two
// with TPR * VPT >= number of vectors); TPR 0 selects the two-pass path.
inline void pick_shape(int64_t nvec, int* tpr_out, int* vpt_out) {
  const int vpt = (nvec >= kVPT4MinVec && nvec <= 4096) ? 4 : kVPTMax;
  int tpr = 1;
  while (static_cast<int64_t>(tpr) * vpt < nvec) {
    tpr <<= 1;
    if (tpr > 1024) {
      tpr = 0;
      break;
    }
  }
  *tpr_out = tpr;
  *vpt_out = vpt;
}

}  // namespace
}  // namespace et
