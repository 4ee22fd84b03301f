// gather.hip -- embedding gather for gfx950.
//
// Definition: "Operations" 3 PosEmbed, TokenEmbed (y = W[id]);
// "Elementwise kernels in C ..." 2.4 (row ids[t] of a [V, d] table, starting
// at element ids[t] * d).  The pages leave checking ids to the caller; here an
// id outside [0, V) is never dereferenced and its output row is quiet NaN.
//
// Design: a pure copy.  Block b copies chunk (b % cpr) of output row
// (b / cpr); a chunk is kBlock * kU 16-byte vectors, so even a short decode
// batch spreads over many blocks.  Source offsets are 64-bit.
#include "et_common.hpp"

namespace et {
namespace {

constexpr int kBlock = 64;  // one wave per workgroup
constexpr int kU = 8;       // vectors per lane

template <typename S, bool VEC>
__global__ __launch_bounds__(kBlock) void embedding_kernel(const S* __restrict__ table,
                                                           int64_t vocab,
                                                           const int32_t* __restrict__ ids,
                                                           S* __restrict__ out, int d, int cpr) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int64_t t = blockIdx.x / cpr;
  const int c = blockIdx.x % cpr;
  const int32_t id = ids[t];
  const bool ok = id >= 0 && static_cast<int64_t>(id) < vocab;
  const int64_t dst = t * d;
  if constexpr (VEC) {
    const int nvec = d / V;
    const int first = c * (kBlock * kU) + threadIdx.x;
    // Stores through a resource based at this block's chunk of the row.
    const int64_t cbase = dst + static_cast<int64_t>(c) * (kBlock * kU) * V;
    const __amdgpu_buffer_rsrc_t ro =
        out_rsrc(out + cbase, (static_cast<int64_t>(nvec) - c * (kBlock * kU)) * 16);
    if (ok) {
      const int64_t src = static_cast<int64_t>(id) * d;
      u32x4 r[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = first + u * kBlock;
        r[u] = ld16(table, src + static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = first + u * kBlock;
        if (j < nvec) st16_buf(ro, (threadIdx.x + u * kBlock) * 16, r[u]);
      }
    } else {
      const u32x4 nan = u32x4{E::kQuietNaN, E::kQuietNaN, E::kQuietNaN, E::kQuietNaN};
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = first + u * kBlock;
        if (j < nvec) st16_buf(ro, (threadIdx.x + u * kBlock) * 16, nan);
      }
    }
  } else {
    constexpr int kPer = kU * 4;
    const int first = c * (kBlock * kPer) + threadIdx.x;
    const int64_t src = ok ? static_cast<int64_t>(id) * d : 0;
    S r[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = first + u * kBlock;
      if (ok) r[u] = table[src + (i < d ? i : d - 1)];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = first + u * kBlock;
      if (i >= d) continue;
      if (ok) {
        out[dst + i] = r[u];
      } else {
        E::st(out, dst + i, __uint_as_float(0x7FC00000u));
      }
    }
  }
}

template <typename S>
et_status embedding_entry(const S* table, int64_t vocab, const int32_t* ids, S* out, int64_t n,
                          int64_t d, void* stream) {
  if (vocab < 0 || n < 0 || d < 0) return ET_ERR_BAD_SIZE;
  if (n == 0 || d == 0) return ET_OK;
  if (d > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t nd = 0, obytes = 0, tbl = 0, tbytes = 0;
  if (!mul_ok(n, d, &nd) || !mul_ok(nd, static_cast<int64_t>(sizeof(S)), &obytes) ||
      !mul_ok(vocab, d, &tbl) || !mul_ok(tbl, static_cast<int64_t>(sizeof(S)), &tbytes))
    return ET_ERR_BAD_SIZE;
  if (!ids || !out || (vocab > 0 && !table)) return ET_ERR_NULL_POINTER;
  if (!ranges_ok(out, obytes, table, tbytes, false) ||
      !ranges_ok(out, obytes, ids, n * static_cast<int64_t>(sizeof(int32_t)), false))
    return ET_ERR_OVERLAP;
  constexpr int V = Elem<S>::V;
  const bool vec = (d % V) == 0 && aligned16(table) && aligned16(out);
  const int per_chunk = vec ? kBlock * kU * V : kBlock * kU * 4;
  const int64_t cpr = (d + per_chunk - 1) / per_chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t rows_per_launch = kMaxGrid / cpr;
  for (int64_t t0 = 0; t0 < n; t0 += rows_per_launch) {
    const int64_t m = n - t0 < rows_per_launch ? n - t0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * cpr);
    if (vec)
      embedding_kernel<S, true><<<grid, kBlock, 0, s>>>(
          table, vocab, ids + t0, out + t0 * d, static_cast<int>(d), static_cast<int>(cpr));
    else
      embedding_kernel<S, false><<<grid, kBlock, 0, s>>>(
          table, vocab, ids + t0, out + t0 * d, static_cast<int>(d), static_cast<int>(cpr));
  }
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

et_status et_embedding_f32(const float* table, int64_t V, const int32_t* ids, float* out,
                           int64_t n, int64_t d, void* stream) {
  return et::embedding_entry<float>(table, V, ids, out, n, d, stream);
}

et_status et_embedding_bf16(const et_bf16* table, int64_t V, const int32_t* ids, et_bf16* out,
                            int64_t n, int64_t d, void* stream) {
  return et::embedding_entry<Bf16>(reinterpret_cast<const Bf16*>(table), V, ids,
                                   reinterpret_cast<Bf16*>(out), n, d, stream);
}

et_status et_embedding_f16(const et_f16* table, int64_t V, const int32_t* ids, et_f16* out,
                            int64_t n, int64_t d, void* stream) {
  return et::embedding_entry<F16>(reinterpret_cast<const F16*>(table), V, ids,
                                   reinterpret_cast<F16*>(out), n, d, stream);
}

}  // extern "C"
