// argmax.hip -- greedy argmax per row for gfx950.
//
// Definition: "Operations" 1 Argmax and 8 Sampling / Greedy;
// "Elementwise kernels in C ..." 2.4 and 4 (argmax_ties_nan_and_empty):
// the largest value, the lowest index among equal values, NaN skipped, -1
// when a row holds no number.
//
// Design (one read pass, HBM-bound):
//   * Each lane scans its elements in increasing index order keeping the
//     first strictly greater non-NaN value, so it holds the lowest index of
//     its own maximum.
//   * Partial results (value, index) are merged by "greater value, or equal
//     value and lower index; no-number loses".  That merge is associative and
//     commutative and -0 == +0, so the answer is the same for any split of
//     the row: the row is cut into chunks of whole 2048-element tiles, spread
//     over up to about a thousand workgroups (a single long row still gets
//     dozens); the
//     last workgroup of a row to finish merges the row's partials (one
//     launch in all).
//   * Without a workspace one workgroup scans a whole row in one launch.
#include "et_common.hpp"

namespace et {
namespace {

#ifndef ET_ARGMAX_BLOCK
#define ET_ARGMAX_BLOCK 256
#endif
constexpr int kBlock = ET_ARGMAX_BLOCK;
constexpr int kTile = 2048;         // elements per chunk granule
#ifndef ET_ARGMAX_TARGET
#define ET_ARGMAX_TARGET 1024
#endif
// Aim for this many workgroups.  Each one ends with two atomic round trips to
// the row's slot, so fewer, longer chunks measured faster than filling the
// chip several times over (1024: 23.3 us, 4096: 25.4 us, 8192: 30 us for
// 256 x 128256 f32).
constexpr int kTargetBlocks = ET_ARGMAX_TARGET;
#ifndef ET_ARGMAX_U
#define ET_ARGMAX_U 4
#endif
#ifndef ET_ARGMAX_KEY
#define ET_ARGMAX_KEY 1             // merge through a 64-bit key per row
#endif

struct Best {
  float v;
  int32_t i;  // -1: no number seen
};

__device__ inline Best better(Best a, Best b) {
  if (b.i < 0) return a;
  if (a.i < 0) return b;
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ inline void scan(Best& b, float v, int32_t i) {
  if (v == v && (b.i < 0 || v > b.v)) {  // v == v: not NaN
    b.v = v;
    b.i = i;
  }
}

__device__ inline Best wave_best(Best b) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    Best o;
    o.v = __shfl_xor(b.v, m, 64);
    o.i = __shfl_xor(b.i, m, 64);
    b = better(b, o);
  }
  return b;
}

__device__ inline Best block_best(Best b) {
  __shared__ float sv[kBlock / 64];
  __shared__ int32_t si[kBlock / 64];
  b = wave_best(b);
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = b.v;
    si[w] = b.i;
  }
  __syncthreads();
  Best r{0.0f, -1};
#pragma unroll
  for (int k = 0; k < kBlock / 64; ++k) r = better(r, Best{sv[k], si[k]});
  return r;
}

// Scan elements [lo, hi) of row `row`; the block's best of that range.
template <typename S, bool VEC>
__device__ inline Best scan_range(const S* __restrict__ x, int64_t row, int64_t n, int64_t lo,
                                  int64_t hi) {
  using E = Elem<S>;
  constexpr int V = E::V;
  constexpr int kU = ET_ARGMAX_U;
  Best b{0.0f, -1};
  const S* p = x + row * n;
  if constexpr (VEC) {
    // lo is a multiple of V; whole vectors first, then the scalar tail.
    const int64_t vlo = lo / V, vhi = hi / V;
    for (int64_t j0 = vlo; j0 < vhi; j0 += kBlock * kU) {
      u32x4 r[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t j = j0 + u * kBlock + threadIdx.x;
        r[u] = ld16(p, (j < vhi ? j : vhi - 1) * V);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t j = j0 + u * kBlock + threadIdx.x;
        if (j < vhi) {
#pragma unroll
          for (int e = 0; e < V; ++e) scan(b, E::get(r[u], e), static_cast<int32_t>(j * V + e));
        }
      }
    }
    const int64_t i = vhi * V + threadIdx.x;
    if (i < hi) scan(b, E::ld(p, i), static_cast<int32_t>(i));
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) scan(b, E::ld(p, i), static_cast<int32_t>(i));
  }
  return block_best(b);
}

// One block per (row, chunk): block b handles chunk b % chunks of row
// b / chunks.  With chunks == 1 the result goes straight to out.  Otherwise
// each block stores its (value, index) in the workspace and counts itself in
// the row's counter; the block that finds it was the last one merges the
// row's partials, writes out[row] and zeroes the row's cells and counter, so
// one launch does the whole row and the workspace is left zero-filled.
// Device-scope release/acquire fences make the partials written by blocks on
// other XCDs (other L2s) visible to the merging block.
template <typename S, bool VEC>
__global__ __launch_bounds__(kBlock) void argmax_chunks(const S* __restrict__ x, int64_t n,
                                                        int64_t chunk, int chunks, float* wv,
                                                        int32_t* wi, uint32_t* cnt,
                                                        int32_t* __restrict__ out) {
  __shared__ int last;
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const Best b = scan_range<S, VEC>(x, row, n, lo, hi);
  if (chunks == 1) {
    if (threadIdx.x == 0) out[row] = b.i;
    return;
  }
  if (threadIdx.x == 0) {
    wv[blockIdx.x] = b.v;
    wi[blockIdx.x] = b.i;
    __threadfence();                                  // release the partial
    last = atomicAdd(&cnt[row], 1u) == static_cast<uint32_t>(chunks - 1);
  }
  __syncthreads();
  if (!last) return;                                  // uniform per block
  __threadfence();                                    // acquire the others
  Best m{0.0f, -1};
  const int64_t first = row * chunks;
  for (int k = threadIdx.x; k < chunks; k += kBlock) {
    m = better(m, Best{__builtin_nontemporal_load(wv + first + k),
                       __builtin_nontemporal_load(wi + first + k)});
    wv[first + k] = 0.0f;                             // the row's cells back to zero
    wi[first + k] = 0;
  }
  m = block_best(m);
  if (threadIdx.x == 0) {
    out[row] = m.i;
    cnt[row] = 0u;                                    // ready for the next call
  }
}

// Same split, merged through one 64-bit key per row instead of a partial per
// chunk: key = (order-preserving bits of the value) << 32 | ~index, so the
// largest key is the largest value and, among equal values, the lowest index
// (-0 is folded into +0 first, so the two tie; 0 means "no number").  Each
// block atomically maxes its key into the row's slot, waits for that atomic
// to complete, then counts itself; the last block reads the slot, writes
// out[row] and zeroes the slot and the counter.  Workspace per row: the key
// (8 bytes) and the counter (4 bytes, padded to 8).
__device__ inline uint64_t best_key(Best b) {
  if (b.i < 0) return 0;
  uint32_t u = __float_as_uint(b.v);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 -> +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(b.i));
}

template <typename S, bool VEC>
__global__ __launch_bounds__(kBlock) void argmax_chunks_key(const S* __restrict__ x, int64_t n,
                                                            int64_t chunk, int chunks,
                                                            unsigned long long* slot, uint32_t* cnt,
                                                            int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const Best b = scan_range<S, VEC>(x, row, n, lo, hi);
  // Only thread 0 takes part in the merge: the other waves leave now instead
  // of idling through its atomics' round trips.
  if (threadIdx.x != 0) return;
  atomicMax(slot + row, static_cast<unsigned long long>(best_key(b)));
  // The max must be performed (acknowledged by the memory system) before
  // this block is counted; wait for every outstanding memory operation.
  __builtin_amdgcn_s_waitcnt(0);
  if (atomicAdd(&cnt[2 * row], 1u) == static_cast<uint32_t>(chunks - 1)) {
    const unsigned long long key = atomicMax(slot + row, 0ull);  // coherent read
    out[row] = key == 0 ? -1 : static_cast<int32_t>(~static_cast<uint32_t>(key));
    slot[row] = 0ull;
    cnt[2 * row] = 0u;
  }
}

__global__ void fill_minus_one(int32_t* out, int64_t rows) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r < rows) out[r] = -1;
}

// Chunk length (a multiple of kTile) and count for a split of rows x n.
inline void plan(int64_t rows, int64_t n, int64_t* chunk, int64_t* chunks) {
  const int64_t per_row = rows >= kTargetBlocks ? 1 : (kTargetBlocks + rows - 1) / rows;
  int64_t c = (n + per_row - 1) / per_row;
  c = ((c + kTile - 1) / kTile) * kTile;
  if (c < kTile) c = kTile;
  *chunk = c;
  *chunks = n > 0 ? (n + c - 1) / c : 1;
}

template <typename S>
et_status argmax_entry(const S* x, int64_t rows, int64_t n, int32_t* out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (rows < 0 || n < 0) return ET_ERR_BAD_SIZE;
  if (rows == 0) return ET_OK;
  if (n > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t xn = 0, xbytes = 0;
  if (!mul_ok(rows, n, &xn) || !mul_ok(xn, int64_t(sizeof(S)), &xbytes)) return ET_ERR_BAD_SIZE;
  if (!out || (n > 0 && !x)) return ET_ERR_NULL_POINTER;
  if (!ws && ws_bytes != 0) return ET_ERR_NULL_POINTER;
  const int64_t obytes = rows * int64_t(sizeof(int32_t));
  if (!ranges_ok(out, obytes, x, xbytes, false)) return ET_ERR_OVERLAP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid * kBlock) {
      const int64_t m = rows - r0 < kMaxGrid * kBlock ? rows - r0 : kMaxGrid * kBlock;
      fill_minus_one<<<static_cast<unsigned>((m + kBlock - 1) / kBlock), kBlock, 0, s>>>(out + r0, m);
    }
    return launch_status();
  }
  int64_t chunk = 0, chunks = 1;
  if (ws) {
    const size_t need = et_argmax_workspace_bytes(rows, n);
    if (ws_bytes < need) return ET_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return ET_ERR_WORKSPACE;
    if (need > 0) plan(rows, n, &chunk, &chunks);
    if (!ranges_ok(ws, static_cast<int64_t>(ws_bytes), x, xbytes, false) ||
        !ranges_ok(ws, static_cast<int64_t>(ws_bytes), out, obytes, false))
      return ET_ERR_OVERLAP;
  }
  if (chunks <= 1) {
    chunks = 1;
    chunk = n;
  }
  constexpr int V = Elem<S>::V;
  const bool vec = (n % V) == 0 && aligned16(x);
#if ET_ARGMAX_KEY
  unsigned long long* slot = static_cast<unsigned long long*>(ws);
  uint32_t* cnt = chunks > 1 ? reinterpret_cast<uint32_t*>(slot + rows) : nullptr;
#else
  float* wv = static_cast<float*>(ws);
  int32_t* wi = chunks > 1 ? reinterpret_cast<int32_t*>(wv + rows * chunks) : nullptr;
  uint32_t* cnt = chunks > 1 ? reinterpret_cast<uint32_t*>(wi + rows * chunks) : nullptr;
#endif
  const int64_t rows_per_launch = kMaxGrid / chunks;
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t m = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * chunks);
    const int ch = static_cast<int>(chunks);
#if ET_ARGMAX_KEY
    if (chunks > 1) {
      if (vec)
        argmax_chunks_key<S, true><<<grid, kBlock, 0, s>>>(x + r0 * n, n, chunk, ch, slot + r0,
                                                           cnt + 2 * r0, out + r0);
      else
        argmax_chunks_key<S, false><<<grid, kBlock, 0, s>>>(x + r0 * n, n, chunk, ch, slot + r0,
                                                            cnt + 2 * r0, out + r0);
      continue;
    }
    float* wvp = nullptr;
    int32_t* wip = nullptr;
    uint32_t* cp = nullptr;
#else
    float* wvp = chunks > 1 ? wv + r0 * chunks : nullptr;
    int32_t* wip = chunks > 1 ? wi + r0 * chunks : nullptr;
    uint32_t* cp = chunks > 1 ? cnt + r0 : nullptr;
#endif
    if (vec)
      argmax_chunks<S, true><<<grid, kBlock, 0, s>>>(x + r0 * n, n, chunk, ch, wvp, wip, cp,
                                                     out + r0);
    else
      argmax_chunks<S, false><<<grid, kBlock, 0, s>>>(x + r0 * n, n, chunk, ch, wvp, wip, cp,
                                                      out + r0);
  }
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

size_t et_argmax_workspace_bytes(int64_t rows, int64_t n) {
  if (rows <= 0 || n <= 0 || n > INT32_MAX) return 0;
  int64_t chunk = 0, chunks = 0;
  et::plan(rows, n, &chunk, &chunks);
  if (chunks <= 1) return 0;
  int64_t cells = 0;
  if (!et::mul_ok(rows, chunks, &cells)) return 0;
#if ET_ARGMAX_KEY
  (void)cells;
  return static_cast<size_t>(rows) * 16;  // key (8 bytes) + counter (4) + padding (4)
#else
  return static_cast<size_t>(cells) * (sizeof(float) + sizeof(int32_t)) +
         static_cast<size_t>(rows) * sizeof(uint32_t);
#endif
}

et_status et_argmax_f32(const float* x, int64_t rows, int64_t n, int32_t* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return et::argmax_entry<float>(x, rows, n, out, workspace, workspace_bytes, stream);
}

et_status et_argmax_bf16(const et_bf16* x, int64_t rows, int64_t n, int32_t* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return et::argmax_entry<Bf16>(reinterpret_cast<const Bf16*>(x), rows, n, out, workspace,
                                workspace_bytes, stream);
}

et_status et_argmax_f16(const et_f16* x, int64_t rows, int64_t n, int32_t* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return et::argmax_entry<F16>(reinterpret_cast<const F16*>(x), rows, n, out, workspace,
                                workspace_bytes, stream);
}

const char* et_status_string(et_status s) {
  switch (s) {
    case ET_OK: return "ok";
    case ET_ERR_NULL_POINTER: return "null pointer with a nonzero size";
    case ET_ERR_BAD_SIZE: return "bad size (negative, overflowing or past a limit)";
    case ET_ERR_BAD_ARG: return "bad argument (d_rot, layout, eps or attn_scaling)";
    case ET_ERR_OVERLAP: return "buffers overlap other than by an allowed exact alias";
    case ET_ERR_WORKSPACE: return "argmax workspace too small";
    case ET_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int et_abi_version(void) { return ET_ABI_VERSION; }

}  // extern "C"
