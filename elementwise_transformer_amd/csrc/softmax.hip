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
//     launch does it all: each workgroup keeps its chunk in registers,
//     publishes (m_c, s_c), waits (bounded) for the row's other chunks,
//     combines and writes -- one read and one write of every element.  A
//     row of more chunks than can be resident together (over 1024) takes
//     two launches instead: chunk statistics, then combine and write (two
//     reads, one write), so no workgroup waits for one that cannot start.
//     Without one, a single workgroup per row recomputes every chunk's
//     statistics itself and then writes (three reads); the bits are the same
//     either way, and also when a bounded wait gives up and the workgroup
//     falls back to computing the statistics itself.
//   * z = x * (1/t); exp(d) = hardware exp2(d * log2 e) for d = z - m <= 0;
//     the output is exp(z - m_c) * (exp(m_c - M) / S), one product per
//     element (the exponentials stay in registers between the passes).
//   * A chunk whose entries are all -inf (a masked stretch of logits) has
//     m_c = -inf; its exponentials are taken against 0 instead, so they are
//     exp(-inf) = 0 and s_c = +0, and the chunk adds nothing to the row (the
//     formula's exp(-inf - M) = 0 for a finite row max M).  A row of -inf
//     still gives M = -inf and a NaN row.
//   * y may be x (in place): every element is read before the thread that
//     owns it writes it, and a row's statistics are complete before any of
//     its outputs is written.  With a workspace, in-place calls take the
//     two-launch path, where a workgroup reads only its own chunk after the
//     statistics are complete: the one-launch exchange's fallback re-reads
//     the whole row, which other workgroups may already be overwriting.
#include "et_common.hpp"

namespace et {
namespace {

constexpr int kChunkElems = 8192;  // elements per chunk (256 threads x VPT vectors)
constexpr int kChunkThreads = 256;
constexpr int kRegMaxElems = 32768;   // register path up to this row length
constexpr int kRegBlock = 128;        // threads per block for short rows
// Chunks per row above which the workspace path takes two launches: the
// one-launch exchange needs a row's chunk blocks resident together, and 256
// CUs hold 2048 of them (eight each); half of that leaves room for other work.
constexpr int64_t kMaxExchangeChunks = 1024;
// Chunk kernels' reduction slots (kLdsSum floats each, one per wave): chunk
// max, chunk sum, then the row max and row sum of row_stats_self, so that
// no slot is written twice in a row without the other's barrier between.
constexpr int kLdsSum = kChunkThreads / 64;

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
// order).  Each takes its own LDS slots (kRowsPerBlock * kWaves floats) and
// one barrier: callers alternate max and sum, so a slot is rewritten only
// after every thread has passed the other reduction's barrier, which it
// reaches only after reading the slot.
template <int TPR>
__device__ inline float row_max(float v, float* lds, int row_in_block, int t) {
  using Sh = SmShape<TPR>;
  v = group_max<Sh::kGroup>(v);
  if constexpr (Sh::kWaves > 1) {
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
    if ((t & 63) == 0) lds[row_in_block * Sh::kWaves + t / 64] = v;
    __syncthreads();
    v = 0.0f;
#pragma unroll
    for (int w = 0; w < Sh::kWaves; ++w) v += lds[row_in_block * Sh::kWaves + w];
  }
  return v;
}

// z = x * (1/t): one more rounding than the quotient, and no division per
// element.
template <typename S>
__device__ inline float scaled(float x, float t, float inv_t) {
  (void)t;
  return x * inv_t;
}

// exp(d) for d = z - m <= 0 (or NaN): the hardware exp2 of d * log2(e).
// The product's rounding adds a relative error of about |d| 2^-24 to the
// result, the exp2 about one ulp; results below 2^-126 may come out as 0.
// (The library expf reduces the range and rescales first; for d <= 0 none
// of that is needed, and it would cost four times the instructions and
// registers in these fully unrolled loops.)
template <typename S>
__device__ inline float expo(float d) {
  return __builtin_amdgcn_exp2f(d * 1.44269504088896340736f);
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
      const int64_t off = static_cast<int64_t>(j < nvec ? j : nvec - 1) * V;
      r[k] = ld16(p, off);
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

// z of vector j of the row at p (length n), as load_z gives it.
template <typename S, bool VEC>
__device__ inline void load_one(const S* p, int n, int j, float tt, float inv_t,
                                float (&z)[Elem<S>::V]) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int nvec = (n + V - 1) / V;
  if constexpr (VEC) {
    const u32x4 r = ld16(p, static_cast<int64_t>(j < nvec ? j : nvec - 1) * V);
#pragma unroll
    for (int e = 0; e < V; ++e) z[e] = j < nvec ? scaled<S>(E::get(r, e), tt, inv_t) : -__builtin_inff();
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int i = j * V + e;
      const float xv = E::ld(p, i < n ? i : n - 1);
      z[e] = i < n ? scaled<S>(xv, tt, inv_t) : -__builtin_inff();
    }
  }
}

// Write y = e * g for the thread's slots of vectors [v0, ...), e the
// exponentials held in registers and g = exp(m_c - M) / S the chunk's scale.
template <typename S, int TPR, int VPT, bool VEC>
__device__ inline void store_y(S* p, int n, int v0, int t, float g,
                               const float (&ev)[VPT][Elem<S>::V]) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int nvec = (n + V - 1) / V;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int j = v0 + slot<TPR, VPT>(k, t);
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = ev[k][e] * g;
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

// The value a chunk's exponentials are taken against: its max, or 0 when
// every entry is -inf (then each is exp(-inf) = 0 rather than exp(NaN)).
__device__ inline float exp_base(float m) { return m == -__builtin_inff() ? 0.0f : m; }

// z <- exp(z - m) in place; returns their sum in slot order.
template <typename S, int VPT>
__device__ inline float exp_in_place(float (&z)[VPT][Elem<S>::V], float m) {
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < Elem<S>::V; ++e) {
      z[k][e] = expo<S>(z[k][e] - m);
      s += z[k][e];
    }
  return s;
}

// The output scale of a chunk whose max is mc, for row statistics (M, S).
template <typename S>
__device__ inline float out_scale(float mc, float2 ms) {
  return expo<S>(mc - ms.x) / ms.y;
}

// --------------------------------------------------------- register path

template <typename S, int TPR, int VPT, bool VEC>
__global__ __launch_bounds__(SmShape<TPR>::kBlock) void softmax_rows(const S* x, S* y,
                                                                     int64_t rows, int n, float tt,
                                                                     float inv_t) {
  using Sh = SmShape<TPR>;
  __shared__ float lds_m[Sh::kRowsPerBlock * Sh::kWaves];
  __shared__ float lds_s[Sh::kRowsPerBlock * Sh::kWaves];
  const int row_in_block = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * Sh::kRowsPerBlock + row_in_block;
  const bool live = row < rows;
  const int64_t base = (live ? row : rows - 1) * static_cast<int64_t>(n);
  float z[VPT][Elem<S>::V];
  load_z<S, TPR, VPT, VEC>(x + base, n, 0, t, tt, inv_t, z);
  const float m = row_max<TPR>(local_max<S, VPT>(z), lds_m, row_in_block, t);
  const float s = row_sum<TPR>(exp_in_place<S, VPT>(z, m), lds_s, row_in_block, t);
  if (live) store_y<S, TPR, VPT, VEC>(y + base, n, 0, t, out_scale<S>(m, float2{m, s}), z);
}

// ------------------------------------------------------------ chunk path

template <typename S>
struct Chunk {
  static constexpr int kVec = kChunkElems / Elem<S>::V;  // vectors per chunk
  static constexpr int kVPT = kVec / kChunkThreads;
};

// Chunk c of the row at p: its exponentials exp(z - m_c) in ev and
// (m_c, s_c) returned to every thread.
template <typename S, bool VEC>
__device__ inline float2 chunk_exp(const S* p, int n, int c, float tt, float inv_t, float* lds,
                                   float (&ev)[Chunk<S>::kVPT][Elem<S>::V]) {
  constexpr int VPT = Chunk<S>::kVPT;
  load_z<S, kChunkThreads, VPT, VEC>(p, n, c * Chunk<S>::kVec, threadIdx.x, tt, inv_t, ev);
  const float m = row_max<kChunkThreads>(local_max<S, VPT>(ev), lds, 0, threadIdx.x);
  const float s =
      row_sum<kChunkThreads>(exp_in_place<S, VPT>(ev, exp_base(m)), lds + kLdsSum, 0, threadIdx.x);
  return float2{m, s};
}

// The same (m_c, s_c) as chunk_exp, one vector at a time with two passes
// over the chunk (max, then the sum in the same (k, e) order), so that the
// self-computed statistics below hold no chunk in registers: they are the
// rare path of the kernels that do, and must not cost them occupancy.
template <typename S, bool VEC>
__device__ inline float2 chunk_stats(const S* p, int n, int c, float tt, float inv_t, float* lds) {
  constexpr int VPT = Chunk<S>::kVPT;
  constexpr int V = Elem<S>::V;
  const int v0 = c * Chunk<S>::kVec;
  const int t = threadIdx.x;
  float m = -__builtin_inff();
#pragma unroll 1
  for (int k = 0; k < VPT; ++k) {
    float z[V];
    load_one<S, VEC>(p, n, v0 + slot<kChunkThreads, VPT>(k, t), tt, inv_t, z);
#pragma unroll
    for (int e = 0; e < V; ++e) m = fmaxf(m, z[e]);
  }
  m = row_max<kChunkThreads>(m, lds, 0, t);
  const float mb = exp_base(m);
  float s = 0.0f;
#pragma unroll 1
  for (int k = 0; k < VPT; ++k) {
    float z[V];
    load_one<S, VEC>(p, n, v0 + slot<kChunkThreads, VPT>(k, t), tt, inv_t, z);
#pragma unroll
    for (int e = 0; e < V; ++e) s += expo<S>(z[e] - mb);
  }
  s = row_sum<kChunkThreads>(s, lds + kLdsSum, 0, t);
  return float2{m, s};
}

// M = max m_c and S = sum_c s_c exp(m_c - M) over the row's chunks: thread t
// folds c = t, t + 256, ... in increasing order, then the fixed block tree.
// get(c) returns (m_c, s_c).
template <typename S, typename Get>
__device__ inline float2 combine(Get get, int chunks, float* lds) {
  float m = -__builtin_inff();
  for (int c = threadIdx.x; c < chunks; c += kChunkThreads) m = fmaxf(m, get(c).x);
  m = row_max<kChunkThreads>(m, lds, 0, threadIdx.x);
  float s = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += kChunkThreads) {
    const float2 pc = get(c);
    s = __builtin_fmaf(pc.y, expo<S>(pc.x - m), s);
  }
  s = row_sum<kChunkThreads>(s, lds + kLdsSum, 0, threadIdx.x);
  return float2{m, s};
}

// combine() for chunks <= 64, in the first wave alone: lane t holds chunk
// t, the other three waves' contributions in combine() are -inf and +0, so
// the bits are the same with one barrier instead of two.  out2: 2 floats.
template <typename S, typename Get>
__device__ inline float2 combine_wave(Get get, int chunks, float* out2) {
  if (threadIdx.x < 64) {
    float2 pc{-__builtin_inff(), 0.0f};
    if (static_cast<int>(threadIdx.x) < chunks) pc = get(threadIdx.x);
    const float m = group_max<64>(fmaxf(-__builtin_inff(), pc.x));
    float s = 0.0f;
    if (static_cast<int>(threadIdx.x) < chunks) s = __builtin_fmaf(pc.y, expo<S>(pc.x - m), s);
    s = group_sum<64>(s);
    if (threadIdx.x == 0) {
      out2[0] = m;
      out2[1] = 0.0f + s;
    }
  }
  __syncthreads();
  return float2{out2[0], out2[1]};
}

// (lds: the four reduction slots; the chunk passes use the first two, M and
// S the last two.)
// The same (M, S) with every chunk's statistics recomputed by this block,
// chunk by chunk (two passes over the row, nothing stored): thread t folds
// the chunks c = t, t + 256, ... in the order combine() does, so the bits
// are the same.
template <typename S, bool VEC>
__device__ inline float2 row_stats_self(const S* p, int n, int chunks, float tt, float inv_t,
                                        float* lds) {
  float m = -__builtin_inff();
#pragma unroll 1
  for (int c = 0; c < chunks; ++c) {
    const float2 st = chunk_stats<S, VEC>(p, n, c, tt, inv_t, lds);
    if (c % kChunkThreads == static_cast<int>(threadIdx.x)) m = fmaxf(m, st.x);
  }
  m = row_max<kChunkThreads>(m, lds + 2 * kLdsSum, 0, threadIdx.x);
  float s = 0.0f;
#pragma unroll 1
  for (int c = 0; c < chunks; ++c) {
    const float2 st = chunk_stats<S, VEC>(p, n, c, tt, inv_t, lds);
    if (c % kChunkThreads == static_cast<int>(threadIdx.x))
      s = __builtin_fmaf(st.y, expo<S>(st.x - m), s);
  }
  s = row_sum<kChunkThreads>(s, lds + 3 * kLdsSum, 0, threadIdx.x);
  return float2{m, s};
}

// A published partial is one 64-bit word (m_c, s_c).  s_c >= 1 or NaN, or
// s_c = +0 with m_c = -inf (a chunk of -inf), so its bits are never 0 (a NaN
// is stored as the canonical quiet NaN): a zero-filled word means "not
// published yet", and the word itself is the flag -- no fence is needed
// between data and flag.
__device__ inline uint64_t partial_bits(float m, float s) {
  const float sc = s != s ? __uint_as_float(0x7FC00000u) : s;
  return __builtin_bit_cast(uint64_t, float2{m, sc});
}

__device__ inline uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One launch with a workspace: block b holds chunk (b % chunks) of row
// (b / chunks) in registers, publishes (m_c, s_c) with one device-scope
// 64-bit store, polls (bounded) until every partial of its row is there,
// combines and writes.  A block that has not seen every partial after
// spin_limit polls computes the row's statistics itself (row_stats_self,
// same bits) instead, so the kernel ends whatever order workgroups become
// resident in.  cnt[2 row] counts the blocks done reading; the last one
// zeroes the row's partials and the counter, leaving the workspace as it
// was found.
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_chunks(const S* x, S* y, int n, int chunks,
                                                               float tt, float inv_t,
                                                               uint64_t* part, uint32_t* cnt,
                                                               int spin_limit) {
  constexpr int VPT = Chunk<S>::kVPT;
  __shared__ float lds[4 * kLdsSum];
  __shared__ float res[2];
  __shared__ int missing;
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const S* px = x + row * n;
  float ev[VPT][Elem<S>::V];
  const float2 st = chunk_exp<S, VEC>(px, n, c, tt, inv_t, lds, ev);
  const float mc = st.x, sc = st.y;
  uint64_t* rp = part + row * chunks;
  if (threadIdx.x == 0) {
    __hip_atomic_store(rp + c, partial_bits(mc, sc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    missing = 0;
  }
  __syncthreads();
  // Thread t watches the partials t, t + 256, ...: each is polled until it
  // is nonzero, at most spin_limit times in all per thread.
  int polls = 0;
  bool seen = true;
  for (int k = threadIdx.x; k < chunks; k += kChunkThreads) {
    while (load_word(rp + k) == 0) {
      if (++polls > spin_limit) {
        seen = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!seen) break;
  }
  if (!seen) missing = 1;  // benign race: every writer writes 1
  __syncthreads();
  float2 ms;
  const auto get = [&](int k) { return __builtin_bit_cast(float2, load_word(rp + k)); };
  if (missing) {
    ms = row_stats_self<S, VEC>(px, n, chunks, tt, inv_t, lds);
  } else if (chunks <= 64) {
    ms = combine_wave<S>(get, chunks, res);
  } else {
    ms = combine<S>(get, chunks, lds);
  }
  store_y<S, kChunkThreads, VPT, VEC>(y + row * n, n, c * Chunk<S>::kVec, threadIdx.x,
                                      out_scale<S>(mc, ms), ev);
  __syncthreads();  // every thread has read what it needs of the partials
  if (threadIdx.x == 0) {
    if (atomicAdd(cnt + 2 * row, 1u) == static_cast<uint32_t>(chunks - 1)) {
      // The last block of the row to finish reading: reset for the next call.
      for (int k = 0; k < chunks; ++k)
        __hip_atomic_store(rp + k, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cnt + 2 * row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Rows of more chunks than can be resident at once (softmax_chunks needs
// every chunk of a row resident together to end without its fallback): two
// launches.  The first writes each chunk's (m_c, s_c) to the workspace; the
// second reloads each chunk, combines its row's partials (written by the
// previous launch, so plain loads see them) and writes -- two reads of the
// row and one write, and no block waits for another.  chunk_exp and combine
// are softmax_chunks', so the bits are the same.
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_chunk_stats(const S* x, int n, int chunks,
                                                                    float tt, float inv_t,
                                                                    uint64_t* part) {
  constexpr int VPT = Chunk<S>::kVPT;
  __shared__ float lds[4 * kLdsSum];
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  float ev[VPT][Elem<S>::V];
  const float2 st = chunk_exp<S, VEC>(x + row * n, n, c, tt, inv_t, lds, ev);
  if (threadIdx.x == 0) part[row * chunks + c] = partial_bits(st.x, st.y);
}

// The second launch.  cnt[2 row] counts the row's blocks done reading its
// partials; the last one zeroes them and the counter with all its threads,
// leaving the workspace as it was found.
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_chunk_write(const S* x, S* y, int n,
                                                                    int chunks, float tt,
                                                                    float inv_t, uint64_t* part,
                                                                    uint32_t* cnt) {
  constexpr int VPT = Chunk<S>::kVPT;
  __shared__ float lds[4 * kLdsSum];
  __shared__ float res[2];
  __shared__ int last;
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  float ev[VPT][Elem<S>::V];
  const float mc = chunk_exp<S, VEC>(x + row * n, n, c, tt, inv_t, lds, ev).x;
  uint64_t* rp = part + row * chunks;
  const auto get = [&](int k) { return __builtin_bit_cast(float2, rp[k]); };
  const float2 ms = chunks <= 64 ? combine_wave<S>(get, chunks, res) : combine<S>(get, chunks, lds);
  store_y<S, kChunkThreads, VPT, VEC>(y + row * n, n, c * Chunk<S>::kVec, threadIdx.x,
                                      out_scale<S>(mc, ms), ev);
  __syncthreads();  // every thread has read what it needs of the partials
  if (threadIdx.x == 0)
    last = atomicAdd(cnt + 2 * row, 1u) == static_cast<uint32_t>(chunks - 1) ? 1 : 0;
  __syncthreads();
  if (last) {
    for (int k = threadIdx.x; k < chunks; k += kChunkThreads) rp[k] = 0;
    if (threadIdx.x == 0) cnt[2 * row] = 0;
  }
}

// Without a workspace: one block per row computes the row's statistics
// itself (row_stats_self), then writes chunk by chunk -- three reads of the
// row, the same bits as the workspace path.
template <typename S, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void softmax_row_blocks(const S* x, S* y, int n,
                                                                    int chunks, float tt,
                                                                    float inv_t) {
  constexpr int VPT = Chunk<S>::kVPT;
  __shared__ float lds[4 * kLdsSum];
  const S* px = x + static_cast<int64_t>(blockIdx.x) * n;
  S* py = y + static_cast<int64_t>(blockIdx.x) * n;
  const float2 ms = row_stats_self<S, VEC>(px, n, chunks, tt, inv_t, lds);
#pragma unroll 1
  for (int c = 0; c < chunks; ++c) {
    float ev[VPT][Elem<S>::V];
    const float mc = chunk_exp<S, VEC>(px, n, c, tt, inv_t, lds, ev).x;
    store_y<S, kChunkThreads, VPT, VEC>(py, n, c * Chunk<S>::kVec, threadIdx.x,
                                        out_scale<S>(mc, ms), ev);
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

// Workspace of a call: per row a 32-bit counter (padded to 8 bytes), then
// (after 16-byte alignment) one 64-bit (m_c, s_c) word per chunk.
inline int64_t counter_bytes(int64_t rows) { return ((rows * 8 + 15) / 16) * 16; }

// Polls of a row's partials (per thread) before a workgroup computes the
// row's statistics itself.  Each poll is a device-coherent load plus a short
// sleep (well under a microsecond), so the bound is a few milliseconds; in
// a normal run every partial arrives within microseconds.  The entry points
// use kSpinLimit; et_softmax_wait_limit takes the bound as an argument, up
// to kSpinLimitMax (0 makes every workgroup take the self-computed path).
constexpr int kSpinLimit = 8192;
constexpr int kSpinLimitMax = 1 << 16;

template <typename S, bool VEC>
void launch_chunks(const S* x, S* y, int64_t rows, int n, float tt, float inv_t, void* ws,
                   int lim, hipStream_t s) {
  const int64_t chunks = chunks_of(n);
  const int64_t rows_per_launch = kMaxGrid / chunks;
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  uint64_t* part = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + counter_bytes(rows));
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t m = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * chunks);
    softmax_chunks<S, VEC><<<grid, kChunkThreads, 0, s>>>(x + r0 * n, y + r0 * n, n,
                                                          static_cast<int>(chunks), tt, inv_t,
                                                          part, cnt, lim);
  }
}

template <typename S, bool VEC>
void launch_two_pass(const S* x, S* y, int64_t rows, int n, float tt, float inv_t, void* ws,
                     hipStream_t s) {
  const int64_t chunks = chunks_of(n);
  const int64_t rows_per_launch = kMaxGrid / chunks;
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  uint64_t* part = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + counter_bytes(rows));
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t m = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * chunks);
    softmax_chunk_stats<S, VEC><<<grid, kChunkThreads, 0, s>>>(x + r0 * n, n,
                                                               static_cast<int>(chunks), tt, inv_t,
                                                               part + r0 * chunks);
    softmax_chunk_write<S, VEC><<<grid, kChunkThreads, 0, s>>>(
        x + r0 * n, y + r0 * n, n, static_cast<int>(chunks), tt, inv_t, part + r0 * chunks,
        cnt + 2 * r0);
  }
}

template <typename S, bool VEC>
void launch_row_blocks(const S* x, S* y, int64_t rows, int n, float tt, float inv_t,
                       hipStream_t s) {
  const int64_t chunks = chunks_of(n);
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
    const int64_t m = rows - r0 < kMaxGrid ? rows - r0 : kMaxGrid;
    softmax_row_blocks<S, VEC><<<static_cast<unsigned>(m), kChunkThreads, 0, s>>>(
        x + r0 * n, y + r0 * n, n, static_cast<int>(chunks), tt, inv_t);
  }
}

template <typename S>
et_status softmax_entry(const S* x, S* y, int64_t rows, int64_t n, float temperature, void* ws,
                        size_t ws_bytes, void* stream, int spin = kSpinLimit) {
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
    if (ws_bytes < need || !aligned16(ws)) return ET_ERR_WORKSPACE;
    if (!ranges_ok(ws, static_cast<int64_t>(ws_bytes), x, bytes, false) ||
        !ranges_ok(ws, static_cast<int64_t>(ws_bytes), y, bytes, false))
      return ET_ERR_OVERLAP;
    // In place, a workgroup must not read chunks other workgroups may
    // already be writing, which the one-launch fallback would: two launches.
    if (chunks_of(n) > kMaxExchangeChunks || static_cast<const void*>(x) == y) {
      if (vec) launch_two_pass<S, true>(x, y, rows, static_cast<int>(n), temperature, inv_t, ws, s);
      else launch_two_pass<S, false>(x, y, rows, static_cast<int>(n), temperature, inv_t, ws, s);
    } else if (vec) {
      launch_chunks<S, true>(x, y, rows, static_cast<int>(n), temperature, inv_t, ws, spin, s);
    } else {
      launch_chunks<S, false>(x, y, rows, static_cast<int>(n), temperature, inv_t, ws, spin, s);
    }
    return launch_status();
  }
  if (vec) launch_row_blocks<S, true>(x, y, rows, static_cast<int>(n), temperature, inv_t, s);
  else launch_row_blocks<S, false>(x, y, rows, static_cast<int>(n), temperature, inv_t, s);
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

size_t et_softmax_workspace_bytes(int64_t rows, int64_t n) {
  if (rows <= 0 || n <= et::kRegMaxElems) return 0;
  int64_t cells = 0, bytes = 0;
  if (!et::mul_ok(rows, et::chunks_of(n), &cells) || !et::mul_ok(cells, 8, &bytes)) return SIZE_MAX;
  return static_cast<size_t>(bytes + et::counter_bytes(rows));
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

et_status et_softmax_f16(const et_f16* x, et_f16* y, int64_t rows, int64_t n,
                          float temperature, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return et::softmax_entry<F16>(reinterpret_cast<const F16*>(x), reinterpret_cast<F16*>(y), rows,
                                 n, temperature, workspace, workspace_bytes, stream);
}

et_status et_softmax_wait_limit(int storage, const void* x, void* y, int64_t rows, int64_t n,
                                float temperature, void* workspace, size_t workspace_bytes,
                                int spin_limit, void* stream) {
  if (spin_limit < 0 || spin_limit > et::kSpinLimitMax) return ET_ERR_BAD_ARG;
  switch (storage) {
    case ET_STORAGE_F32:
      return et::softmax_entry<float>(static_cast<const float*>(x), static_cast<float*>(y), rows, n,
                                      temperature, workspace, workspace_bytes, stream, spin_limit);
    case ET_STORAGE_BF16:
      return et::softmax_entry<Bf16>(static_cast<const Bf16*>(x), static_cast<Bf16*>(y), rows, n,
                                     temperature, workspace, workspace_bytes, stream, spin_limit);
    case ET_STORAGE_F16:
      return et::softmax_entry<F16>(static_cast<const F16*>(x), static_cast<F16*>(y), rows, n,
                                    temperature, workspace, workspace_bytes, stream, spin_limit);
    default:
      return ET_ERR_BAD_ARG;
  }
}

}  // extern "C"
