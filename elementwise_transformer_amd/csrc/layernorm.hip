// layernorm.hip -- LayerNorm over the last axis for gfx950.
//
// Definition: "Operations" 2 Normalization / LayerNorm; "ruDNN User Guide" 7
// (final axis, f32 statistics, optional bias, output in the input type):
//   mu = mean(x), var = mean((x - mu)^2), y = (x - mu) / sqrt(var + eps) * g + b.
//
// Design: the RMSNorm row shape (norm_common.hpp): a row per TPR-thread
// group, held in registers, read once and written once.  Two fixed-order
// reductions -- the sum for the mean, then the sum of squared deviations
// from it (the two-pass variance, as defined, not E[x^2] - mu^2) -- each a
// per-thread sum in slot order, a butterfly and wave partials in wave order,
// so a row's bits depend on d only.  Rows longer than the register path take
// a three-pass kernel (mean, variance, write) with 1024 threads per row.
// y may be x (in place): every element is read by the thread that writes it,
// before it writes it.
#include "et_common.hpp"
#include "norm_common.hpp"

namespace et {
namespace {

template <typename S, int TPR, int VPT, bool VEC, bool BIAS>
__global__ __launch_bounds__(NormShape<TPR>::kBlock) void layernorm_rows(
    const S* x, const S* __restrict__ w, const S* __restrict__ b, S* y, int64_t rows, int d,
    float eps) {
  using E = Elem<S>;
  using Sh = NormShape<TPR>;
  constexpr int V = E::V;
  __shared__ float lds_mean[Sh::kRowsPerBlock * Sh::kWavesPerRow];
  __shared__ float lds_var[Sh::kRowsPerBlock * Sh::kWavesPerRow];

  const int row_in_block = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * Sh::kRowsPerBlock + row_in_block;
  const bool live = row < rows;
  const int64_t base = (live ? row : rows - 1) * d;  // clamped: loaded, never stored
  const int nvec = (d + V - 1) / V;

  // The thread's elements in storage form (unpacked as used: for bf16 this
  // keeps half the registers); valid(k, e) marks those inside the row.
  u32x4 xr[VPT];
  u32x4 wr[VPT], br[VPT];
  // (With whole vectors, d % V == 0, so a vector is valid or not as a whole.)
  auto valid = [&](int k, int e) {
    return VEC ? own<TPR, VPT>(k, t) < nvec : own<TPR, VPT>(k, t) * V + e < d;
  };
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = own<TPR, VPT>(k, t);
      xr[k] = ld16(x, base + static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
    }
    if constexpr (TPR >= kWEarlyMinTPR) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j = own<TPR, VPT>(k, t);
        const int64_t off = static_cast<int64_t>(j < nvec ? j : nvec - 1) * V;
        wr[k] = ld16_keep(w, off);
        if constexpr (BIAS) br[k] = ld16_keep(b, off);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float a[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = own<TPR, VPT>(k, t) * V + e;
        a[e] = E::ld(x, base + (i < d ? i : d - 1));
      }
      xr[k] = E::pack(a);  // exact: the values are already in storage precision
    }
  }

  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) sum += valid(k, e) ? E::get(xr[k], e) : 0.0f;
  const float mu = row_sum<TPR>(sum, lds_mean, row_in_block, t) / static_cast<float>(d);
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float c = valid(k, e) ? E::get(xr[k], e) - mu : 0.0f;
      ss = __builtin_fmaf(c, c, ss);
    }
  }
  ss = row_sum<TPR>(ss, lds_var, row_in_block, t);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  if (!live) return;

  if constexpr (VEC) {
    // Outputs in groups of four vectors: for rows of one wave the gain and
    // bias load late, a group at a time (a scheduling barrier keeps the
    // compiler from hoisting every group's loads at once), so that gain, bias
    // and row together stay within the registers of four waves per SIMD.
    constexpr int kGroupV = VPT < 4 ? VPT : 4;
#pragma unroll
    for (int k0 = 0; k0 < VPT; k0 += kGroupV) {
      if constexpr (TPR < kWEarlyMinTPR) {
#pragma unroll
        for (int k = k0; k < k0 + kGroupV; ++k) {
          const int j = own<TPR, VPT>(k, t);
          const int64_t off = static_cast<int64_t>(j < nvec ? j : nvec - 1) * V;
          wr[k] = ld16_keep(w, off);
          if constexpr (BIAS) br[k] = ld16_keep(b, off);
        }
      }
#pragma unroll
      for (int k = k0; k < k0 + kGroupV; ++k) {
        const int j = own<TPR, VPT>(k, t);
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          o[e] = (E::get(xr[k], e) - mu) * inv * E::get(wr[k], e);
          if constexpr (BIAS) o[e] += E::get(br[k], e);
        }
        if (j < nvec) st16(y, base + static_cast<int64_t>(j) * V, E::pack(o));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = own<TPR, VPT>(k, t) * V + e;
        if (i >= d) continue;
        float o = (E::get(xr[k], e) - mu) * inv * E::ld(w, i);
        if constexpr (BIAS) o += E::ld(b, i);
        E::st(y, base + i, o);
      }
    }
  }
}

// Rows longer than the register path: thread t owns vectors t, t + 1024, ...
// in order.  Pass 1 sums, pass 2 re-reads and sums squared deviations, pass
// 3 re-reads and writes; pass 3 starts after the barrier inside the second
// row_sum, so no in-place write precedes a read.
template <typename S, bool VEC, bool BIAS>
__global__ __launch_bounds__(kLargeTPR) void layernorm_rows_large(const S* x,
                                                                  const S* __restrict__ w,
                                                                  const S* __restrict__ b, S* y,
                                                                  int d, float eps) {
  using E = Elem<S>;
  constexpr int V = E::V;
  __shared__ float lds_mean[kLargeTPR / 64];
  __shared__ float lds_var[kLargeTPR / 64];
  const int t = threadIdx.x;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * d;
  const int nvec = (d + V - 1) / V;
  auto load_vec = [&](int j, float (&a)[V]) {
    if constexpr (VEC) {
      E::unpack(ld16(x, base + static_cast<int64_t>(j) * V), a);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        a[e] = i < d ? E::ld(x, base + i) : 0.0f;
      }
    }
  };
  float sum = 0.0f;
  for (int j = t; j < nvec; j += kLargeTPR) {
    float a[V];
    load_vec(j, a);
#pragma unroll
    for (int e = 0; e < V; ++e) sum += a[e];
  }
  const float mu = row_sum<kLargeTPR>(sum, lds_mean, 0, t) / static_cast<float>(d);
  float ss = 0.0f;
  for (int j = t; j < nvec; j += kLargeTPR) {
    float a[V];
    load_vec(j, a);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float c = j * V + e < d ? a[e] - mu : 0.0f;
      ss = __builtin_fmaf(c, c, ss);
    }
  }
  ss = row_sum<kLargeTPR>(ss, lds_var, 0, t);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  for (int j = t; j < nvec; j += kLargeTPR) {
    float a[V];
    load_vec(j, a);
    if constexpr (VEC) {
      float g[V], o[V];
      E::unpack(ld16_keep(w, static_cast<int64_t>(j) * V), g);
      float bb[V];
      if constexpr (BIAS) E::unpack(ld16_keep(b, static_cast<int64_t>(j) * V), bb);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        o[e] = (a[e] - mu) * inv * g[e];
        if constexpr (BIAS) o[e] += bb[e];
      }
      st16(y, base + static_cast<int64_t>(j) * V, E::pack(o));
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        if (i >= d) continue;
        float o = (a[e] - mu) * inv * E::ld(w, i);
        if constexpr (BIAS) o += E::ld(b, i);
        E::st(y, base + i, o);
      }
    }
  }
}

template <typename S, int TPR, int VPT, bool VEC, bool BIAS>
void launch_ln(const S* x, const S* w, const S* b, S* y, int64_t rows, int d, float eps,
               hipStream_t s) {
  using Sh = NormShape<TPR>;
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid * Sh::kRowsPerBlock) {
    const int64_t n = rows - r0 < kMaxGrid * Sh::kRowsPerBlock ? rows - r0
                                                                : kMaxGrid * Sh::kRowsPerBlock;
    const unsigned grid = static_cast<unsigned>((n + Sh::kRowsPerBlock - 1) / Sh::kRowsPerBlock);
    layernorm_rows<S, TPR, VPT, VEC, BIAS><<<grid, Sh::kBlock, 0, s>>>(x + r0 * d, w, b, y + r0 * d,
                                                                      n, d, eps);
  }
}

template <typename S, bool VEC, bool BIAS>
void dispatch_ln(int tpr, int vpt, const S* x, const S* w, const S* b, S* y, int64_t rows, int d,
                 float eps, hipStream_t s) {
  switch (tpr) {
    case 1: launch_ln<S, 1, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 2: launch_ln<S, 2, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 4: launch_ln<S, 4, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 8: launch_ln<S, 8, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 16: launch_ln<S, 16, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 32: launch_ln<S, 32, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 64: launch_ln<S, 64, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 128: launch_ln<S, 128, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s); break;
    case 256:
      if (vpt == 4) launch_ln<S, 256, 4, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      else launch_ln<S, 256, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      break;
    case 512:
      if (vpt == 4) launch_ln<S, 512, 4, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      else launch_ln<S, 512, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      break;
    case 1024:
      if (vpt == 4) launch_ln<S, 1024, 4, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      else launch_ln<S, 1024, kVPTMax, VEC, BIAS>(x, w, b, y, rows, d, eps, s);
      break;
    default:
      for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
        const int64_t n = rows - r0 < kMaxGrid ? rows - r0 : kMaxGrid;
        layernorm_rows_large<S, VEC, BIAS><<<static_cast<unsigned>(n), kLargeTPR, 0, s>>>(
            x + r0 * d, w, b, y + r0 * d, d, eps);
      }
  }
}

template <typename S>
et_status layernorm_entry(const S* x, const S* w, const S* b, S* y, int64_t rows, int64_t d,
                          float eps, void* stream) {
  if (rows < 0 || d < 0) return ET_ERR_BAD_SIZE;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return ET_ERR_BAD_ARG;
  if (rows == 0) return ET_OK;
  if (d == 0 || d > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t n = 0, bytes = 0;
  if (!mul_ok(rows, d, &n) || !mul_ok(n, static_cast<int64_t>(sizeof(S)), &bytes))
    return ET_ERR_BAD_SIZE;
  if (!x || !w || !y) return ET_ERR_NULL_POINTER;
  const int64_t wbytes = d * static_cast<int64_t>(sizeof(S));
  if (!ranges_ok(y, bytes, x, bytes, true) || !ranges_ok(y, bytes, w, wbytes, false) ||
      !ranges_ok(y, bytes, b, wbytes, false))
    return ET_ERR_OVERLAP;
  constexpr int V = Elem<S>::V;
  const bool vec = (d % V) == 0 && aligned16(x) && aligned16(w) && aligned16(y) &&
                   (b == nullptr || aligned16(b));
  int tpr = 0, vpt = 0;
  pick_shape((d + V - 1) / V, &tpr, &vpt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int di = static_cast<int>(d);
  if (vec) {
    if (b) dispatch_ln<S, true, true>(tpr, vpt, x, w, b, y, rows, di, eps, s);
    else dispatch_ln<S, true, false>(tpr, vpt, x, w, b, y, rows, di, eps, s);
  } else {
    if (b) dispatch_ln<S, false, true>(tpr, vpt, x, w, b, y, rows, di, eps, s);
    else dispatch_ln<S, false, false>(tpr, vpt, x, w, b, y, rows, di, eps, s);
  }
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

et_status et_layernorm_f32(const float* x, const float* gamma, const float* beta, float* y,
                           int64_t rows, int64_t d, float eps, void* stream) {
  return et::layernorm_entry<float>(x, gamma, beta, y, rows, d, eps, stream);
}

et_status et_layernorm_bf16(const et_bf16* x, const et_bf16* gamma, const et_bf16* beta,
                            et_bf16* y, int64_t rows, int64_t d, float eps, void* stream) {
  return et::layernorm_entry<Bf16>(reinterpret_cast<const Bf16*>(x),
                                   reinterpret_cast<const Bf16*>(gamma),
                                   reinterpret_cast<const Bf16*>(beta), reinterpret_cast<Bf16*>(y),
                                   rows, d, eps, stream);
}

et_status et_layernorm_f16(const et_f16* x, const et_f16* gamma, const et_f16* beta,
                            et_f16* y, int64_t rows, int64_t d, float eps, void* stream) {
  return et::layernorm_entry<F16>(reinterpret_cast<const F16*>(x),
                                   reinterpret_cast<const F16*>(gamma),
                                   reinterpret_cast<const F16*>(beta), reinterpret_cast<F16*>(y),
                                   rows, d, eps, stream);
}

}  // extern "C"
