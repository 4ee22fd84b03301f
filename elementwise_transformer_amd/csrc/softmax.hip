// softmax.hip -- softmax over the last axis with a temperature, for gfx950.
//
// Definition: "Operations" 4 Activation / Softmax and 8 Sampling /
// Temperature; "ruDNN User Guide" 7 (statistics in f32, output in the input
// type).  Per row: z_i = x_i / t, m = max z, e_i = exp(z_i - m),
// y_i = e_i / sum e.  Special values follow the formula (a NaN anywhere, or a
// row whose max is +-inf, gives a NaN row).
//
// Design (HBM-bound):
//   * Rows of up to kRegMaxElems elements: one row per group of TPR threads
//     (VPT 16-byte vectors each, both from n alone), held in registers: read
//     once, max, sum of exponentials, scaled and written.  Reductions are
//     fixed trees (per-thread in slot order, xor butterfly, wave partials in
//     wave order), so a row's bits depend on n only.
//   * Longer rows: chunks of kChunkElems elements, each reduced by one
//     256-thread workgroup with one fixed tree to (m_c, s_c = sum exp(z-m_c)).
//     The row's statistics are M = max m_c and S = sum_c s_c exp(m_c - M),
//     the sum taken by the same fixed tree over c.  With a workspace, one
//     launch writes every (m_c, s_c) and a second reads them back, re-reads
//     its chunk and writes y -- both launches fill the chip.  Without one, a
//     single workgroup per row runs the same steps with the partials in LDS;
//     the bits are the same either way.
//   * f32 storage: IEEE division for z and for e / S, library expf.  bf16
//     storage: multiplication by 1/t and by 1/S and the hardware exp2 -- the
//     f32 result only has to be far inside half a bf16 ulp.
//   * y may be x (in place): every element is read before the thread that
//     owns it writes it, and a row's statistics are complete before any of
//     its outputs is written.
#include "et_common.hpp"

namespace et {
namespace {

constexpr int kChunkElems = 8192;     // elements per chunk (a multiple of V)
constexpr int kChunkThreads = 256;
constexpr int kRegMaxElems = 32768;   // register path up to this row length
constexpr int kRegBlock = 128;        // threads per block for short rows
constexpr int kMaxLdsChunks = 8000;   // partials a single-workgroup row keeps in LDS (64 KB)

template <int TPR>
struct SmShape {
  static constexpr int kBlock = TPR < kRegBlock ? kRegBlock : TPR;
  static constexpr int kRowsPerBlock = kBlock / TPR;
  static constexpr int kGroup = TPR < 64 ? TPR : 64;
  static constexpr int kWaves = TPR > 64 ? TPR / 64 : 1;
};

// Vector slot k of thread t: stripes of TPR vectors for rows of one wave or
// less; for longer rows each wave owns a contiguous run of 64 * VPT vectors.
template <int TPR, int VPT>
__device__ inline int slot(int k, int t) {
  if constexpr (TPR > 64) {
    return (t / 64) * (64 * VPT) + k * 64 + (t % 64);
  } else {
    return k * TPR + t;
  }
}

template <int W>
__device__ inline float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Max and sum over the TPR threads of one row.  The max is exact in any
// order; the sum is a fixed tree (butterfly, then wave partials in wave
// order).  lds holds kRowsPerBlock * kWaves floats.
template <int TPR>
__device__ inline float row_max(float v, float* lds, int row_in_block, int t) {
  using Sh = SmShape<TPR>;
  v = group_max<Sh::kGroup>(v);
  if constexpr (Sh::kWaves > 1) {
    __syncthreads();
    if ((t & 63) == 0) lds[row_in_block * Sh::kWaves + t / 64] = v;
    __syncthreads();
    v = lds[row_in_block * Sh::kWaves];
#pragma unroll
    for (int w = 1; w < Sh::kWaves; ++w) v = fmaxf(v, lds[row_in_block * Sh::kWaves + w]);
  }
  return v;
}

template <int TPR>
__device__ inline float row_sum(float v, float* lds, int row_in_block, int t) {
  using Sh = SmShape<TPR>;
  v = group_sum<Sh::kGroup>(v);
  if constexpr (Sh::kWaves > 1) {
    __syncthreads();
    if ((t & 63) == 0) lds[row_in_block * Sh::kWaves + t / 64] = v;
    __syncthreads();
    v = 0.0f;
#pragma unroll
    for (int w = 0; w < Sh::kWaves; ++w) v += lds[row_in_block * Sh::kWaves + w];
  }
  return v;
}

// z = x / t (f32) or x * (1/t) (bf16).
template <typename S>
__device__ inline float scaled(float x, float t, float inv_t) {
  if constexpr (sizeof(S) == 4) {
    return x / t;
  } else {
    return x * inv_t;
  }
}

// exp(d) for d = z - m <= 0 (or NaN).
template <typename S>
__device__ inline float expo(float d) {
  if constexpr (sizeof(S) == 4) {
    return expf(d);
  } else {
    return __builtin_amdgcn_exp2f(d * 1.44269504088896340736f);
  }
}

// e / s (f32) or e * (1/s) (bf16; inv_s = 1/s).
template <typename S>
__device__ inline float quot(float e, float s, float inv_s) {
  if constexpr (sizeof(S) == 4) {
    return e / s;
  } else {
    return e * inv_s;
  }
}

// Load the VPT slots of thread t covering vectors [v0, v0 + span) of a row
// whose first element is p and whose length is n; z values of slots past n
// are -inf (they add exp(-inf) = 0).  Loads are clamped, never guarded.
template <typename S, int TPR, int VPT, bool VEC>
__device__ inline void load_z(const S* p, int n, int v0, int t, float tt, float inv_t,
                              float (&z)[VPT][Elem<S>::V]) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int nvec = (n + V - 1) / V;
  if constexpr (VEC) {
    u32x4 r[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = v0 + slot<TPR, VPT>(k, t);
      r[k] = ld16(p, static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = v0 + slot<TPR, VPT>(k, t);
#pragma unroll
      for (int e = 0; e < V; ++e)
        z[k][e] = j < nvec ? scaled<S>(E::get(r[k], e), tt, inv_t) : -__builtin_inff();
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int j = v0 + slot<TPR, VPT>(k, t);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        const float xv = E::ld(p, i < n ? i : n - 1);
        z[k][e] = i < n ? scaled<S>(xv, tt, inv_t) : -__builtin_inff();
      }
    }
  }
}

// Write y = exp(z - m) / s for the thread's slots of vectors [v0, ...).
template <typename S, int TPR, int VPT, bool VEC>
__device__ inline void store_y(S* p, int n, int v0, int t, float m, float s,
                               const float (&z)[VPT][Elem<S>::V]) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int nvec = (n + V - 1) / V;
  const float inv_s = 1.0f / s;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int j = v0 + slot<TPR, VPT>(k, t);
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = quot<S>(expo<S>(z[k][e] - m), s, inv_s);
    if constexpr (VEC) {
      if (j < nvec) st16(p, static_cast<int64_t>(j) * V, E::pack(o));
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int i = j * V + e;
        if (i < n) E::st(p, i, o[e]);
      }
    }
  }
}

// Thread-local max and sum of exp(z - m) in slot order.
template <typename S, int VPT>
__device__ inline float local_max(const float (&z)[VPT][Elem<S>::V]) {
  float m = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < Elem<S>::V; ++e) m = fmaxf(m, z[k][e]);
  return m;
}

template <typename S, int VPT>
__device__ inline float local_sum(const float (&z)[VPT][Elem<S>::V], float m) {
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < Elem<S>::V; ++e) s += expo<S>(z[k][e] - m);
  return s;
}

// --------------------------------------------------------- register path

template <typename S, int TPR, int VPT, bool VEC>
__global__ __launch_bounds__(SmShape<TPR>::kBlock) void softmax_rows(const S* x, S* y,
                                                                     int64_t rows, int n, float tt,
                                                                     float inv_t) {
  using Sh = SmShape<TPR>;
  __shared__ float lds[Sh::kRowsPerBlock * Sh::kWaves];
  const int row_in_block = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * Sh::kRowsPerBlock + row_in_block;
  const bool live = row < rows;
  const int64_t base = (live ? row : rows - 1) * static_cast<int64_t>(n);
  float z[VPT][Elem<S>::V];
  load_z<S, TPR, VPT, VEC>(x + base, n, 0, t, tt, inv_t, z);
  const float m = row_max<TPR>(local_max<S, VPT>(z), lds, row_in_block, t);
  const float s = row_sum<TPR>(local_sum<S, VPT>(z, m), lds, row_in_block, t);
  if (live) store_y<S, TPR, VPT, VEC>(y + base, n, 0, t, m, s, z);
}

// ------------------------------------------------------------ chunk path

template <typename S>
struct Chunk {
  static constexpr int kVec = kChunkElems / Elem<S>::V;  // vectors per chunk
  static constexpr int kVPT = kVec / kChunkThreads;
};

// (m_c, s_c) of chunk c of the row at p; every thread gets the result.
template <typename S, bool VEC>
__device__ inline float2 chunk_stats(const S* p, int n, int c, float tt, float inv_t, float* lds) {
  constexpr int VPT = Chunk<S>::kVPT;
  float z[VPT][Elem<S>::V];
  load_z<S, kChunkThreads, VPT, VEC>(p, n, c * Chunk<S>::kVec, threadIdx.x, tt, inv_t, z);
  const float m = row_max<kChunkThreads>(local_max<S, VPT>(z), lds, 0, threadIdx.x);
  const float s = row_sum<kChunkThreads>(local_sum<S, VPT>(z, m), lds, 0, threadIdx.x);
  return float2{m, s};
}

// M = max m_c and S = sum_c s_c exp(m_c - M) over the row's chunks: thread t
// takes c = t, t + 256, ... in order, then the fixed block tree.
template <typename S, typename P>
__device__ inline float2 combine(const P* part, int chunks, float* lds) {
  float m = -__builtin_inff();
  for (int c = threadIdx.x; c < chunks; c += kChunkThreads) m = fmaxf(m, part[c].x);
  m = row_max<kChunkThreads>(m, lds, 0, threadIdx.x);
  float s = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += kChunkThreads) {
    const float2 pc = part[c];
    s += pc.y * expo<S>(pc.x - m);
  }
  s = row_sum<kChunkThreads>(s, lds, 0, threadIdx.x);
  return float2{m, s};
}

// Launch 1 of 2: block b writes the statistics of chunk (b % chunks) of row
// (b / chunks) to part[b].
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_chunk_stats(const S* x, int n, int chunks,
                                                                     float tt, float inv_t,
                                                                     float2* part) {
  __shared__ float lds[kChunkThreads / 64];
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const float2 st = chunk_stats<S, VEC>(x + row * n, n, c, tt, inv_t, lds);
  if (threadIdx.x == 0) part[blockIdx.x] = st;
}

// Launch 2 of 2: block b combines its row's partials and writes chunk
// (b % chunks) of row (b / chunks).
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_chunk_write(const S* x, S* y, int n,
                                                                     int chunks, float tt,
                                                                     float inv_t,
                                                                     const float2* part) {
  constexpr int VPT = Chunk<S>::kVPT;
  __shared__ float lds[kChunkThreads / 64];
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  float z[VPT][Elem<S>::V];
  load_z<S, kChunkThreads, VPT, VEC>(x + row * n, n, c * Chunk<S>::kVec, threadIdx.x, tt, inv_t,
                                     z);
  const float2 ms = combine<S>(part + row * chunks, chunks, lds);
  store_y<S, kChunkThreads, VPT, VEC>(y + row * n, n, c * Chunk<S>::kVec, threadIdx.x, ms.x, ms.y,
                                      z);
}

// Without a workspace: one block per row, the same chunk statistics kept in
// LDS, then the same combine and write.
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_row_blocks(const S* x, S* y, int n,
                                                                    int chunks, float tt,
                                                                    float inv_t) {
  constexpr int VPT = Chunk<S>::kVPT;
  extern __shared__ float2 part[];
  __shared__ float lds[kChunkThreads / 64];
  const S* px = x + static_cast<int64_t>(blockIdx.x) * n;
  S* py = y + static_cast<int64_t>(blockIdx.x) * n;
  for (int c = 0; c < chunks; ++c) {
    const float2 st = chunk_stats<S, VEC>(px, n, c, tt, inv_t, lds);
    if (threadIdx.x == 0) part[c] = st;
  }
  __syncthreads();
  const float2 ms = combine<S>(part, chunks, lds);
  for (int c = 0; c < chunks; ++c) {
    float z[VPT][Elem<S>::V];
    load_z<S, kChunkThreads, VPT, VEC>(px, n, c * Chunk<S>::kVec, threadIdx.x, tt, inv_t, z);
    store_y<S, kChunkThreads, VPT, VEC>(py, n, c * Chunk<S>::kVec, threadIdx.x, ms.x, ms.y, z);
  }
}

// ------------------------------------------------------------------ host

// Register-path shape from n alone: VPT 8 (f32) or 4/8 (bf16) vectors per
// thread and the smallest power-of-two TPR covering the row.
template <typename S>
void reg_shape(int64_t n, int* tpr, int* vpt) {
  constexpr int V = Elem<S>::V;
  const int64_t nvec = (n + V - 1) / V;
  const int vp = 8;
  int tp = 1;
  while (static_cast<int64_t>(tp) * vp < nvec) tp <<= 1;
  *tpr = tp;
  *vpt = vp;
}

template <typename S, int TPR, bool VEC>
void launch_rows(const S* x, S* y, int64_t rows, int n, float tt, float inv_t, hipStream_t s) {
  using Sh = SmShape<TPR>;
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid * Sh::kRowsPerBlock) {
    const int64_t m = rows - r0 < kMaxGrid * Sh::kRowsPerBlock ? rows - r0 : kMaxGrid * Sh::kRowsPerBlock;
    const unsigned grid = static_cast<unsigned>((m + Sh::kRowsPerBlock - 1) / Sh::kRowsPerBlock);
    softmax_rows<S, TPR, 8, VEC><<<grid, Sh::kBlock, 0, s>>>(x + r0 * n, y + r0 * n, m, n, tt,
                                                             inv_t);
  }
}

template <typename S, bool VEC>
void dispatch_rows(int tpr, const S* x, S* y, int64_t rows, int n, float tt, float inv_t,
                   hipStream_t s) {
  switch (tpr) {
    case 1: launch_rows<S, 1, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 2: launch_rows<S, 2, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 4: launch_rows<S, 4, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 8: launch_rows<S, 8, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 16: launch_rows<S, 16, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 32: launch_rows<S, 32, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 64: launch_rows<S, 64, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 128: launch_rows<S, 128, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 256: launch_rows<S, 256, VEC>(x, y, rows, n, tt, inv_t, s); break;
    case 512: launch_rows<S, 512, VEC>(x, y, rows, n, tt, inv_t, s); break;
    default: launch_rows<S, 1024, VEC>(x, y, rows, n, tt, inv_t, s); break;
  }
}

inline int64_t chunks_of(int64_t n) { return (n + kChunkElems - 1) / kChunkElems; }

template <typename S, bool VEC>
void launch_chunks(const S* x, S* y, int64_t rows, int n, float tt, float inv_t, float2* part,
                   hipStream_t s) {
  const int64_t chunks = chunks_of(n);
  const int64_t rows_per_launch = kMaxGrid / chunks;
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t m = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * chunks);
    softmax_chunk_stats<S, VEC><<<grid, kChunkThreads, 0, s>>>(x + r0 * n, n, static_cast<int>(chunks),
                                                               tt, inv_t, part);
    softmax_chunk_write<S, VEC><<<grid, kChunkThreads, 0, s>>>(
        x + r0 * n, y + r0 * n, n, static_cast<int>(chunks), tt, inv_t, part);
  }
}

template <typename S, bool VEC>
void launch_row_blocks(const S* x, S* y, int64_t rows, int n, float tt, float inv_t,
                       hipStream_t s) {
  const int64_t chunks = chunks_of(n);
  const size_t shmem = static_cast<size_t>(chunks) * sizeof(float2);
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
    const int64_t m = rows - r0 < kMaxGrid ? rows - r0 : kMaxGrid;
    softmax_row_blocks<S, VEC><<<static_cast<unsigned>(m), kChunkThreads, shmem, s>>>(
        x + r0 * n, y + r0 * n, n, static_cast<int>(chunks), tt, inv_t);
  }
}

template <typename S>
et_status softmax_entry(const S* x, S* y, int64_t rows, int64_t n, float temperature, void* ws,
                        size_t ws_bytes, void* stream) {
  if (rows < 0 || n < 0) return ET_ERR_BAD_SIZE;
  if (!(temperature > 0.0f) || !__builtin_isfinite(temperature)) return ET_ERR_BAD_ARG;
  if (rows == 0 || n == 0) return ET_OK;
  if (n > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t xn = 0, bytes = 0;
  if (!mul_ok(rows, n, &xn) || !mul_ok(xn, static_cast<int64_t>(sizeof(S)), &bytes))
    return ET_ERR_BAD_SIZE;
  if (!x || !y) return ET_ERR_NULL_POINTER;
  if (!ws && ws_bytes != 0) return ET_ERR_NULL_POINTER;
  if (!ranges_ok(y, bytes, x, bytes, true)) return ET_ERR_OVERLAP;
  constexpr int V = Elem<S>::V;
  const bool vec = (n % V) == 0 && aligned16(x) && aligned16(y);
  const float inv_t = 1.0f / temperature;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n <= kRegMaxElems) {
    int tpr = 0, vpt = 0;
    reg_shape<S>(n, &tpr, &vpt);
    if (vec) dispatch_rows<S, true>(tpr, x, y, rows, static_cast<int>(n), temperature, inv_t, s);
    else dispatch_rows<S, false>(tpr, x, y, rows, static_cast<int>(n), temperature, inv_t, s);
    return launch_status();
  }
  if (ws) {
    const size_t need = et_softmax_workspace_bytes(rows, n);
    if (ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 7u) != 0) return ET_ERR_WORKSPACE;
    if (!ranges_ok(ws, static_cast<int64_t>(ws_bytes), x, bytes, false) ||
        !ranges_ok(ws, static_cast<int64_t>(ws_bytes), y, bytes, false))
      return ET_ERR_OVERLAP;
    float2* part = static_cast<float2*>(ws);
    if (vec) launch_chunks<S, true>(x, y, rows, static_cast<int>(n), temperature, inv_t, part, s);
    else launch_chunks<S, false>(x, y, rows, static_cast<int>(n), temperature, inv_t, part, s);
    return launch_status();
  }
  if (chunks_of(n) > kMaxLdsChunks) return ET_ERR_WORKSPACE;
  if (vec) launch_row_blocks<S, true>(x, y, rows, static_cast<int>(n), temperature, inv_t, s);
  else launch_row_blocks<S, false>(x, y, rows, static_cast<int>(n), temperature, inv_t, s);
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;

extern "C" {

size_t et_softmax_workspace_bytes(int64_t rows, int64_t n) {
  if (rows <= 0 || n <= et::kRegMaxElems) return 0;
  int64_t cells = 0, bytes = 0;
  if (!et::mul_ok(rows, et::chunks_of(n), &cells) || !et::mul_ok(cells, 8, &bytes)) return SIZE_MAX;
  return static_cast<size_t>(bytes);
}

et_status et_softmax_f32(const float* x, float* y, int64_t rows, int64_t n, float temperature,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return et::softmax_entry<float>(x, y, rows, n, temperature, workspace, workspace_bytes, stream);
}

et_status et_softmax_bf16(const et_bf16* x, et_bf16* y, int64_t rows, int64_t n,
                          float temperature, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return et::softmax_entry<Bf16>(reinterpret_cast<const Bf16*>(x), reinterpret_cast<Bf16*>(y), rows,
                                 n, temperature, workspace, workspace_bytes, stream);
}

}  // extern "C"
