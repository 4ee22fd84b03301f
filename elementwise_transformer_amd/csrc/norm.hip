// norm.hip -- RMSNorm and fused residual-add + RMSNorm for gfx950.
//
// Definitions: "Operations" 2 Normalization / RmsNorm and 10 Fused ops
// (FusedSkipNorm); "Elementwise kernels in C ..." 2.1 RMSNorm.
//   y_i = x_i / sqrt(sum_i(x_i^2) / d + eps) * w_i   (eps inside the root)
//   fused: h = x + residual (rounded to storage), y = RMSNorm(h as stored).
//
// Design (HBM-bound; one read and one write per element):
//   * A row is owned by a group of TPR threads (TPR a power of two, 1..1024)
//     picked from d alone.  Thread t of the group owns 16-byte vectors
//     j = k*TPR + t, k = 0..VPT-1 (VPT 4 or 8, also from d alone), so
//     consecutive lanes touch consecutive 16 B.
//   * The whole row stays in registers: read once, reduced, scaled, written.
//   * Sum of squares: f32 FMA over the thread's elements in (k, element)
//     order, then an xor butterfly over min(TPR, 64) lanes, then (TPR > 64)
//     the per-wave partials added in wave order through LDS.  The order is a
//     function of d only, so a row's bits never depend on how many rows the
//     call holds.
//   * Rows longer than 8192 vectors fall back to a two-pass kernel (1024
//     threads per row, the row re-read for the write pass).
//   * Blocks of 128 threads (or one row of more): rows are independent.
//   * Unaligned buffers or d not a multiple of the vector width take the same
//     kernels with scalar loads (same ownership, same sums).
#include "et_common.hpp"
#include "norm_common.hpp"

namespace et {
namespace {

__device__ inline float inv_rms(float ss, int d, float eps) {
  return 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
}

// One row per TPR-thread group, row held in registers.  x/res carry no
// __restrict__: y may be x and h may be res (in place).  Every load of a
// thread is issued before its first store, and a thread touches only the
// elements it owns.
template <typename S, int TPR, int VPT, bool FUSED, bool VEC>
__global__ __launch_bounds__(NormShape<TPR>::kBlock) void rmsnorm_rows(
    const S* x, const S* res, const S* __restrict__ w, S* y, S* h, int64_t rows, int d,
    float eps) {
  using E = Elem<S>;
  using Sh = NormShape<TPR>;
  constexpr int V = E::V;
  __shared__ float lds[Sh::kRowsPerBlock * Sh::kWavesPerRow];

  const int row_in_block = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * Sh::kRowsPerBlock + row_in_block;
  const bool live = row < rows;
  // Loads are never guarded (a guarded load makes the compiler serialise
  // them): a thread past the last row reads the last row and stores nothing;
  // a vector slot past the end of the row reads the row's last vector and is
  // masked to 0.
  const int64_t base = (live ? row : rows - 1) * d;
  const int nvec = (d + V - 1) / V;
  // Vector stores go through resources based at the block's first row; the
  // byte offset of element e of this thread's row is (row_in_block * d + e)
  // times the element size, well below 2^31 for the register path.
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * Sh::kRowsPerBlock;
  const int64_t span = (rows - row0) * d * static_cast<int64_t>(sizeof(S));
  const int rel = row_in_block * d;

  // The row slice of this thread, packed in storage format (h when fused).
  u32x4 xr[VPT];
  u32x4 wr[VPT];
  if constexpr (VEC) {
    u32x4 rr[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = own<TPR, VPT>(k, t);
      const int64_t off = base + static_cast<int64_t>(j < nvec ? j : nvec - 1) * V;
      xr[k] = ld16(x, off);
      if constexpr (FUSED) rr[k] = ld16(res, off);
    }
    if constexpr (TPR >= kWEarlyMinTPR) {
      // The gain is cached (every row reads it); issuing its loads now hides
      // their latency behind the row loads and the reduction.
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j = own<TPR, VPT>(k, t);
        wr[k] = ld16_keep(w, static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
      }
    }
    if constexpr (FUSED) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j = own<TPR, VPT>(k, t);
        float a[V];
#pragma unroll
        for (int e = 0; e < V; ++e) a[e] = E::get(xr[k], e) + E::get(rr[k], e);
        xr[k] = E::pack(a);  // h rounded to storage, normalised as stored
        if (live && j < nvec)
          st16_buf(out_rsrc(h + row0 * d, span), (rel + j * V) * int(sizeof(S)), xr[k]);
      }
    }
  } else {
    float a[VPT][V];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = (own<TPR, VPT>(k, t)) * V + e;
        const int64_t off = base + (i < d ? i : d - 1);
        a[k][e] = E::ld(x, off);
        if constexpr (FUSED) a[k][e] = a[k][e] + E::ld(res, off);
      }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      xr[k] = E::pack(a[k]);
      if constexpr (FUSED) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int i = (own<TPR, VPT>(k, t)) * V + e;
          if (live && i < d) E::st(h, base + i, E::get(xr[k], e));
        }
      }
    }
  }

  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int i = (own<TPR, VPT>(k, t)) * V + e;
      const float a = i < d ? E::get(xr[k], e) : 0.0f;
      ss = __builtin_fmaf(a, a, ss);
    }
  }
  ss = row_sum<TPR>(ss, lds, row_in_block, t);
  const float inv = inv_rms(ss, d, eps);
  if (!live) return;

  if constexpr (VEC) {
    if constexpr (TPR < kWEarlyMinTPR) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j = own<TPR, VPT>(k, t);
        wr[k] = ld16_keep(w, static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
      }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = own<TPR, VPT>(k, t);
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = E::get(xr[k], e) * inv * E::get(wr[k], e);
      if (j < nvec)
        st16_buf(out_rsrc(y + row0 * d, span), (rel + j * V) * int(sizeof(S)), E::pack(o));
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = (own<TPR, VPT>(k, t)) * V + e;
        const float g = E::ld(w, i < d ? i : d - 1);
        if (i < d) E::st(y, base + i, E::get(xr[k], e) * inv * g);
      }
    }
  }
}

// Two-pass path for rows longer than the register path holds: thread t owns
// vectors t, t + 1024, ... in order; pass 1 sums, pass 2 re-reads, recomputes
// the same h bits and writes.  Pass 2 starts after the barrier inside
// row_sum, so no in-place write precedes a pass-1 read.
template <typename S, bool FUSED, bool VEC>
__global__ __launch_bounds__(kLargeTPR) void rmsnorm_rows_large(
    const S* x, const S* res, const S* __restrict__ w, S* y, S* h, int64_t rows, int d,
    float eps) {
  using E = Elem<S>;
  constexpr int V = E::V;
  __shared__ float lds[kLargeTPR / 64];
  const int t = threadIdx.x;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * d;
  const int nvec = (d + V - 1) / V;
  (void)rows;

  // The row's j-th vector as f32 values (h rounded to storage when fused);
  // scalar loads past the end of the row read 0.
  auto load_vec = [&](int j, float (&a)[V]) {
    if constexpr (VEC) {
      E::unpack(ld16(x, base + static_cast<int64_t>(j) * V), a);
      if constexpr (FUSED) {
        float b[V];
        E::unpack(ld16(res, base + static_cast<int64_t>(j) * V), b);
#pragma unroll
        for (int e = 0; e < V; ++e) a[e] = E::round(a[e] + b[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        a[e] = 0.0f;
        if (i < d) {
          a[e] = E::ld(x, base + i);
          if constexpr (FUSED) a[e] = E::round(a[e] + E::ld(res, base + i));
        }
      }
    }
  };

  float ss = 0.0f;
  for (int j = t; j < nvec; j += kLargeTPR) {
    float a[V];
    load_vec(j, a);
#pragma unroll
    for (int e = 0; e < V; ++e) ss = __builtin_fmaf(a[e], a[e], ss);
  }
  ss = row_sum<kLargeTPR>(ss, lds, 0, t);
  const float inv = inv_rms(ss, d, eps);
  for (int j = t; j < nvec; j += kLargeTPR) {
    float a[V];
    load_vec(j, a);
    if constexpr (VEC) {
      float g[V], o[V];
      if constexpr (FUSED) st16(h, base + static_cast<int64_t>(j) * V, E::pack(a));
      E::unpack(ld16_keep(w, static_cast<int64_t>(j) * V), g);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = a[e] * inv * g[e];
      st16(y, base + static_cast<int64_t>(j) * V, E::pack(o));
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        if (i >= d) continue;
        if constexpr (FUSED) E::st(h, base + i, a[e]);
        E::st(y, base + i, a[e] * inv * E::ld(w, i));
      }
    }
  }
}

template <typename S, int TPR, int VPT, bool FUSED, bool VEC>
void launch_rows(const S* x, const S* res, const S* w, S* y, S* h, int64_t rows, int d, float eps,
                 hipStream_t s) {
  using Sh = NormShape<TPR>;
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid * Sh::kRowsPerBlock) {
    const int64_t n = rows - r0 < kMaxGrid * Sh::kRowsPerBlock ? rows - r0
                                                                : kMaxGrid * Sh::kRowsPerBlock;
    const int64_t off = r0 * d;
    const unsigned grid = static_cast<unsigned>((n + Sh::kRowsPerBlock - 1) / Sh::kRowsPerBlock);
    rmsnorm_rows<S, TPR, VPT, FUSED, VEC><<<grid, Sh::kBlock, 0, s>>>(
        x + off, FUSED ? res + off : nullptr, w, y + off, FUSED ? h + off : nullptr, n, d, eps);
  }
}

template <typename S, bool FUSED, bool VEC>
void dispatch_tpr(int tpr, int vpt, const S* x, const S* res, const S* w, S* y, S* h, int64_t rows, int d,
                  float eps, hipStream_t s) {
  switch (tpr) {
    case 1: launch_rows<S, 1, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 2: launch_rows<S, 2, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 4: launch_rows<S, 4, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 8: launch_rows<S, 8, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 16: launch_rows<S, 16, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 32: launch_rows<S, 32, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 64: launch_rows<S, 64, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s); break;
    case 128:
      // (4 vectors per thread start at 1024 vectors, 256 threads)
      launch_rows<S, 128, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      break;
    case 256:
      if (vpt == 4) launch_rows<S, 256, 4, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      else launch_rows<S, 256, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      break;
    case 512:
      if (vpt == 4) launch_rows<S, 512, 4, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      else launch_rows<S, 512, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      break;
    case 1024:
      if (vpt == 4) launch_rows<S, 1024, 4, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      else launch_rows<S, 1024, kVPTMax, FUSED, VEC>(x, res, w, y, h, rows, d, eps, s);
      break;
    default: {
      for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
        const int64_t n = rows - r0 < kMaxGrid ? rows - r0 : kMaxGrid;
        const int64_t off = r0 * d;
        rmsnorm_rows_large<S, FUSED, VEC><<<static_cast<unsigned>(n), kLargeTPR, 0, s>>>(
            x + off, FUSED ? res + off : nullptr, w, y + off, FUSED ? h + off : nullptr, n, d,
            eps);
      }
    }
  }
}

template <typename S, bool FUSED>
et_status norm_entry(const S* x, const S* res, const S* w, S* y, S* h, int64_t rows, int64_t d,
                     float eps, void* stream) {
  if (rows < 0 || d < 0) return ET_ERR_BAD_SIZE;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return ET_ERR_BAD_ARG;
  if (rows == 0) return ET_OK;
  if (d == 0 || d > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t n = 0, bytes = 0;
  if (!mul_ok(rows, d, &n) || !mul_ok(n, static_cast<int64_t>(sizeof(S)), &bytes))
    return ET_ERR_BAD_SIZE;
  if (!x || !w || !y || (FUSED && (!res || !h))) return ET_ERR_NULL_POINTER;
  const int64_t wbytes = d * static_cast<int64_t>(sizeof(S));
  // Outputs against every other buffer: exact aliases only where allowed.
  if (!ranges_ok(y, bytes, x, bytes, true) || !ranges_ok(y, bytes, w, wbytes, false))
    return ET_ERR_OVERLAP;
  if (FUSED) {
    if (!ranges_ok(y, bytes, res, bytes, false) || !ranges_ok(y, bytes, h, bytes, false) ||
        !ranges_ok(h, bytes, res, bytes, true) || !ranges_ok(h, bytes, w, wbytes, false) ||
        !ranges_ok(h, bytes, x, bytes, y != x))
      return ET_ERR_OVERLAP;
  }
  constexpr int V = Elem<S>::V;
  const bool vec = (d % V) == 0 && aligned16(x) && aligned16(w) && aligned16(y) &&
                   (!FUSED || (aligned16(res) && aligned16(h)));
  int tpr = 0, vpt = 0;
  pick_shape((d + V - 1) / V, &tpr, &vpt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (vec)
    dispatch_tpr<S, FUSED, true>(tpr, vpt, x, res, w, y, h, rows, static_cast<int>(d), eps, s);
  else
    dispatch_tpr<S, FUSED, false>(tpr, vpt, x, res, w, y, h, rows, static_cast<int>(d), eps, s);
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

et_status et_rmsnorm_f32(const float* x, const float* w, float* y, int64_t rows, int64_t d,
                         float eps, void* stream) {
  return et::norm_entry<float, false>(x, nullptr, w, y, nullptr, rows, d, eps, stream);
}

et_status et_rmsnorm_bf16(const et_bf16* x, const et_bf16* w, et_bf16* y, int64_t rows,
                          int64_t d, float eps, void* stream) {
  return et::norm_entry<Bf16, false>(reinterpret_cast<const Bf16*>(x), nullptr,
                                     reinterpret_cast<const Bf16*>(w), reinterpret_cast<Bf16*>(y),
                                     nullptr, rows, d, eps, stream);
}

et_status et_rmsnorm_f16(const et_f16* x, const et_f16* w, et_f16* y, int64_t rows,
                          int64_t d, float eps, void* stream) {
  return et::norm_entry<F16, false>(reinterpret_cast<const F16*>(x), nullptr,
                                     reinterpret_cast<const F16*>(w), reinterpret_cast<F16*>(y),
                                     nullptr, rows, d, eps, stream);
}

et_status et_add_rmsnorm_f32(const float* x, const float* residual, const float* w, float* y,
                             float* h, int64_t rows, int64_t d, float eps, void* stream) {
  return et::norm_entry<float, true>(x, residual, w, y, h, rows, d, eps, stream);
}

et_status et_add_rmsnorm_bf16(const et_bf16* x, const et_bf16* residual, const et_bf16* w,
                              et_bf16* y, et_bf16* h, int64_t rows, int64_t d, float eps,
                              void* stream) {
  return et::norm_entry<Bf16, true>(
      reinterpret_cast<const Bf16*>(x), reinterpret_cast<const Bf16*>(residual),
      reinterpret_cast<const Bf16*>(w), reinterpret_cast<Bf16*>(y), reinterpret_cast<Bf16*>(h),
      rows, d, eps, stream);
}

et_status et_add_rmsnorm_f16(const et_f16* x, const et_f16* residual, const et_f16* w,
                              et_f16* y, et_f16* h, int64_t rows, int64_t d, float eps,
                              void* stream) {
  return et::norm_entry<F16, true>(
      reinterpret_cast<const F16*>(x), reinterpret_cast<const F16*>(residual),
      reinterpret_cast<const F16*>(w), reinterpret_cast<F16*>(y), reinterpret_cast<F16*>(h),
      rows, d, eps, stream);
}

}  // extern "C"
