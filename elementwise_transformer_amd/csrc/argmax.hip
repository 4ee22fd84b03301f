// argmax.hip -- greedy argmax per row for gfx950.
//
// Definition: "Operations" 1 Argmax and 8 Sampling / Greedy;
// "Elementwise kernels in C ..." 2.4 and 4 (argmax_ties_nan_and_empty):
// the largest value, the lowest index among equal values, NaN skipped, -1
// when a row holds no number.
//
// Design (one read pass, HBM-bound):
//   * Each lane scans its 16-byte vectors in increasing index order keeping
//     the first strictly greater non-NaN value, so it holds the lowest index
//     of its own maximum.  Each wave owns a contiguous run of 64 * kU
//     vectors per step (slot u of lane l at u * 64 + l), every load of a
//     step issued before the first compare.
//   * Partial results (value, index) are merged by "greater value, or equal
//     value and lower index; no-number loses".  That merge is associative and
//     commutative and -0 == +0, so the answer is the same for any split.
//   * Workgroups of 256 threads, 4 vectors in flight per lane.  A call of at
//     least kFillBlocks rows gets one workgroup per row (no exchange, no
//     workspace).  Fewer rows, given a workspace, are cut into chunks of
//     whole granules so that about kFillBlocks workgroups run (four per
//     CU); each one atomically maxes a 64-bit key of its best into the row's
//     slot and counts itself, and the last one of the row writes the index
//     and re-zeroes the slot and the counter (one launch; the workspace is
//     left as it was found).
//   * Measured on [256, 128256] f32 over buffers rotated past the Infinity
//     Cache, against a plain read of the same bytes in the same process
//     (22.0 us on that GPU; this kernel 24.7 us): the scan's instruction
//     stream costs little (software pipelining, 2 or 4 accumulators, 8
//     vectors per lane, buffer loads: all within 1 % of one another), and
//     so does the chunk size (1 to 8 granules of 1024 vectors per
//     workgroup, or one 1024-thread workgroup per row); what the read does
//     not pay is the end of each workgroup: its reduction (DPP exchanges,
//     0.4 us faster than LDS-crossbar shuffles) and the merge's atomics
//     (about 1.1 us).  Publishing each chunk's key with a device-scope
//     store and having the last workgroup poll for them saves one round
//     trip on paper but ran no faster with 4 chunks a row and 2.7 us slower
//     with 16: such stores become visible later than atomics.
#include <mutex>

#include "et_common.hpp"

// Scratch of the entry point that allocates nothing (et_argmax_noalloc):
// the split path's per-row 64-bit key and counter (16 bytes per row) for up
// to kScratchRows rows.  The split path only runs for calls of fewer than
// kFillBlocks (1024) rows, so 1024 rows (16 KiB) cover every call.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name is only a stand-in: the device address comes from
// hipGetSymbolAddress, once per device.
constexpr int64_t kScratchRows = 1024;
static __device__ __align__(256) unsigned long long scratch[2 * kScratchRows];

namespace et {
namespace {

constexpr int kThreads = 256;        // threads per workgroup
constexpr int kU = 4;                 // vectors in flight per lane per step
constexpr int64_t kFillBlocks = 1024;  // workgroups a call aims at (four per CU)

// A candidate: value and index.  kNone marks "no number seen" (with value
// -inf); every real index is below it (n <= INT32_MAX).  Candidates never
// hold NaN: the scans skip it.
constexpr int32_t kNone = INT32_MAX;

struct Best {
  float v;
  int32_t i;
};

// The better of two candidates: the greater value, or of equal values the
// lower index.  No candidate holds NaN, so this is a total order on distinct
// indices, and a kNone candidate (-inf, INT32_MAX) loses to every real one.
__device__ inline Best better(Best a, Best b) {
  const bool take_b = b.v > a.v || (b.v == a.v && b.i < a.i);
  return take_b ? b : a;
}

template <int CTRL>
__device__ inline Best dpp_better(Best b) {
  const Best o{dpp::mov<CTRL>(b.v), __builtin_amdgcn_mov_dpp(b.i, CTRL, 0xF, 0xF, false)};
  return better(b, o);
}

__device__ inline Best lane_of(Best b, int lane) {
  return Best{__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b.v), lane)),
              __builtin_amdgcn_readlane(b.i, lane)};
}

// The best of a wave, the same in every lane: four DPP exchanges (partners
// 1 and 2 apart inside a quad, then the mirrored lane of the 8- and 16-lane
// half-row and row) leave every lane of each 16-lane row with that row's
// best; the four rows' results are then read out of lanes 0, 16, 32, 48.
// No step goes through the LDS crossbar.
__device__ inline Best wave_best(Best b) {
  b = dpp_better<dpp::kXor1>(b);
  b = dpp_better<dpp::kXor2>(b);
  b = dpp_better<dpp::kHalfMirror>(b);
  b = dpp_better<dpp::kMirror>(b);
  return better(better(lane_of(b, 0), lane_of(b, 16)), better(lane_of(b, 32), lane_of(b, 48)));
}

// The best of a T-thread workgroup, returned to every thread.
template <int T>
__device__ inline Best block_best(Best b) {
  __shared__ float sv[T / 64];
  __shared__ int32_t si[T / 64];
  b = wave_best(b);
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = b.v;
    si[w] = b.i;
  }
  __syncthreads();
  Best r{sv[0], si[0]};
#pragma unroll
  for (int k = 1; k < T / 64; ++k) r = better(r, Best{sv[k], si[k]});
  return r;
}

// A lane's running best in a scan of increasing indices: the largest value
// m greater than -inf seen so far and the position of its first occurrence
// (vector j, element e), or j = -1.  One compare and three selects per
// element: v > m is false for NaN (skipped) and for a value equal to m (the
// earlier index stays).  A value of -inf is never greater than the initial
// m, so a range holding nothing but -inf and NaN leaves j = -1 in every
// lane; first_number() then finds its answer.
struct Run {
  float m;
  int j;
  int e;
};

__device__ inline void run_update(Run& r, float v, int j, int e) {
  const bool gt = v > r.m;
  r.m = gt ? v : r.m;
  r.j = gt ? j : r.j;
  r.e = gt ? e : r.e;
}

// The lowest index in [lo, hi) of row p holding a number (not NaN), as a
// workgroup's Best (its value is then -inf, the largest value present), or
// kNone: the answer for a range where no value exceeds -inf.  Rare: only
// ranges of -inf and NaN get here.
template <typename S, int T>
__device__ __forceinline__ Best first_number(const S* p, int64_t lo, int64_t hi) {
  using E = Elem<S>;
  __syncthreads();  // every lane has read block_best's slots from the first pass
  Best b{-__builtin_inff(), kNone};
  for (int64_t i = lo + threadIdx.x; i < hi; i += T) {
    const float v = E::ld(p, i);
    if (v == v) {
      b = Best{v, static_cast<int32_t>(i)};
      break;
    }
  }
  return block_best<T>(b);
}

// Scan elements [lo, hi) of row `row` (lo a multiple of the vector width on
// the vector path); the workgroup's best of that range.
template <typename S, int T, bool VEC>
__device__ __forceinline__ Best scan_range(const S* __restrict__ x, int64_t row, int64_t n, int64_t lo,
                                  int64_t hi) {
  using E = Elem<S>;
  constexpr int V = E::V;
  constexpr int kTileVec = T * kU;
  const S* p = x + row * n;
  Run r{-__builtin_inff(), -1, 0};
  int32_t tail_i = kNone;  // the scalar tail's candidate (vector path)
  float tail_v = -__builtin_inff();
  if constexpr (VEC) {
    // Whole tiles without guards, then one clamped and guarded tile, then
    // the scalar tail (fewer than V elements).  Vector indices fit in int:
    // n <= INT32_MAX.
    const int vlo = static_cast<int>(lo / V), vhi = static_cast<int>(hi / V);
    const int own = static_cast<int>((threadIdx.x / 64) * (64 * kU) + (threadIdx.x % 64));
    int j0 = vlo;
    for (; j0 + kTileVec <= vhi; j0 += kTileVec) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = ld16(p, static_cast<int64_t>(j0 + own + u * 64) * V);
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) run_update(r, E::get(v[u], e), j0 + own + u * 64, e);
    }
    if (j0 < vhi) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = j0 + own + u * 64;
        v[u] = ld16(p, static_cast<int64_t>(j < vhi ? j : vhi - 1) * V);  // clamped, never guarded
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = j0 + own + u * 64;
        if (j < vhi) {
#pragma unroll
          for (int e = 0; e < V; ++e) run_update(r, E::get(v[u], e), j, e);
        }
      }
    }
    const int64_t i = static_cast<int64_t>(vhi) * V + threadIdx.x;
    if (i < hi) {
      const float v = E::ld(p, i);
      if (v > -__builtin_inff()) {  // a number above -inf (not NaN)
        tail_v = v;
        tail_i = static_cast<int32_t>(i);
      }
    }
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += T) run_update(r, E::ld(p, i), static_cast<int>(i), 0);
  }
  Best b{r.m, r.j < 0 ? kNone : (VEC ? r.j * V + r.e : r.j)};
  b = better(b, Best{tail_v, tail_i});
  b = block_best<T>(b);
  if (b.i == kNone) b = first_number<S, T>(p, lo, hi);  // (uniform: every lane holds the block's best)
  return b;
}

// One workgroup per row.
template <typename S, int T, bool VEC>
__global__ __launch_bounds__(T) void argmax_rows(const S* __restrict__ x, int64_t n,
                                                 int32_t* __restrict__ out) {
  const Best b = scan_range<S, T, VEC>(x, blockIdx.x, n, 0, n);
  if (threadIdx.x == 0) out[blockIdx.x] = b.i == kNone ? -1 : b.i;
}

// Rows split into chunks, merged through one 64-bit key per row: key =
// (order-preserving bits of the value) << 32 | ~index, so the largest key is
// the largest value and, among equal values, the lowest index (-0 is folded
// into +0 first, so the two tie; 0 means "no number").  Workspace per row:
// the key (8 bytes) and the counter (4 bytes, padded to 8).
__device__ inline uint64_t best_key(Best b) {
  if (b.i == kNone) return 0;
  uint32_t u = __float_as_uint(b.v);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 -> +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(b.i));
}

// Workgroup b scans chunk b % chunks of row b / chunks, atomically maxes its
// key into the row's slot, waits for that atomic to complete, then counts
// itself; the last one of the row reads the slot, writes out[row] and zeroes
// the slot and the counter.
template <typename S, int T, bool VEC>
__global__ __launch_bounds__(T) void argmax_split(const S* __restrict__ x, int64_t n, int64_t chunk,
                                                  int chunks, unsigned long long* slot,
                                                  uint32_t* cnt, int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const Best b = scan_range<S, T, VEC>(x, row, n, lo, hi);
  // Only thread 0 takes part in the merge: the other waves leave now instead
  // of idling through its atomics' round trips.
  if (threadIdx.x != 0) return;
  atomicMax(slot + row, static_cast<unsigned long long>(best_key(b)));
  // The max must be performed (acknowledged by the memory system) before
  // this workgroup is counted; wait for every outstanding memory operation.
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

// Chunk length and count of a split of rows x n (n >= 1): one chunk per row
// once the rows alone fill the chip, else chunks of whole granules (16
// elements per lane, a multiple of every vector width) aiming at about
// kFillBlocks workgroups.
inline void plan(int64_t rows, int64_t n, int64_t* chunk, int64_t* chunks) {
  *chunk = n;
  *chunks = 1;
  if (rows >= kFillBlocks) return;
  const int64_t gran = int64_t{16} * kThreads;
  const int64_t per_row = (kFillBlocks + rows - 1) / rows;
  int64_t c = (n + per_row - 1) / per_row;
  c = ((c + gran - 1) / gran) * gran;
  if (c >= n) return;
  *chunk = c;
  *chunks = (n + c - 1) / c;
}

template <typename S, int T, bool VEC>
void launch(const S* x, int64_t rows, int64_t n, int64_t chunk, int64_t chunks,
            unsigned long long* slot, uint32_t* cnt, int32_t* out, hipStream_t s) {
  const int64_t rows_per_launch = kMaxGrid / chunks;
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t m = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
    const unsigned grid = static_cast<unsigned>(m * chunks);
    if (chunks > 1)
      argmax_split<S, T, VEC><<<grid, T, 0, s>>>(x + r0 * n, n, chunk, static_cast<int>(chunks),
                                                 slot + r0, cnt + 2 * r0, out + r0);
    else
      argmax_rows<S, T, VEC><<<grid, T, 0, s>>>(x + r0 * n, n, out + r0);
  }
}

// check_only: validate the arguments and return, enqueueing nothing.
template <typename S>
et_status argmax_entry(const S* x, int64_t rows, int64_t n, int32_t* out, void* ws,
                       size_t ws_bytes, void* stream, bool check_only = false) {
  if (rows < 0 || n < 0) return ET_ERR_BAD_SIZE;
  if (rows == 0) return ET_OK;
  if (n > INT32_MAX) return ET_ERR_BAD_SIZE;
  int64_t xn = 0, xbytes = 0;
  if (!mul_ok(rows, n, &xn) || !mul_ok(xn, int64_t(sizeof(S)), &xbytes)) return ET_ERR_BAD_SIZE;
  if (!out || (n > 0 && !x)) return ET_ERR_NULL_POINTER;
  if (!ws && ws_bytes != 0) return ET_ERR_NULL_POINTER;
  const int64_t obytes = rows * int64_t(sizeof(int32_t));
  if (!ranges_ok(out, obytes, x, xbytes, false)) return ET_ERR_OVERLAP;
  if (check_only) return ET_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid * 256) {
      const int64_t m = rows - r0 < kMaxGrid * 256 ? rows - r0 : kMaxGrid * 256;
      fill_minus_one<<<static_cast<unsigned>((m + 255) / 256), 256, 0, s>>>(out + r0, m);
    }
    return launch_status();
  }
  int64_t chunk = n, chunks = 1;
  if (ws) {
    const size_t need = et_argmax_workspace_bytes(rows, n);
    if (ws_bytes < need) return ET_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return ET_ERR_WORKSPACE;
    if (!ranges_ok(ws, static_cast<int64_t>(ws_bytes), x, xbytes, false) ||
        !ranges_ok(ws, static_cast<int64_t>(ws_bytes), out, obytes, false))
      return ET_ERR_OVERLAP;
    if (need > 0) plan(rows, n, &chunk, &chunks);
  }
  unsigned long long* slot = static_cast<unsigned long long*>(ws);
  uint32_t* cnt = chunks > 1 ? reinterpret_cast<uint32_t*>(slot + rows) : nullptr;
  constexpr int V = Elem<S>::V;
  const bool vec = (n % V) == 0 && aligned16(x);
  if (vec) launch<S, kThreads, true>(x, rows, n, chunk, chunks, slot, cnt, out, s);
  else launch<S, kThreads, false>(x, rows, n, chunk, chunks, slot, cnt, out, s);
  return launch_status();
}

// Zero n 64-bit words: the scratch's keys and counters before a split call
// (a kernel on the caller's stream, so it is ordered before the call's own
// kernel and may be captured into a graph).
__global__ void zero_words(unsigned long long* p, int64_t n) {
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0ull;
}

// The device address of `scratch` on the current device, looked up once per
// device with that device current (hipGetSymbolAddress), then kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

et_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ET_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ET_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ET_OK;
}

template <typename S>
et_status argmax_noalloc(const S* x, int64_t rows, int64_t n, int32_t* out, void* stream) {
  // The arguments are checked exactly as et_argmax_* checks them, before the
  // scratch is touched; a call that needs no split passes no workspace.
  const size_t need = (rows > 0 && n > 0 && n <= INT32_MAX) ? et_argmax_workspace_bytes(rows, n) : 0;
  if (need == 0) return argmax_entry<S>(x, rows, n, out, nullptr, 0, stream);
  if (need > sizeof(scratch)) return ET_ERR_WORKSPACE;  // (the split path needs rows < 1024)
  if (const et_status st = argmax_entry<S>(x, rows, n, out, nullptr, 0, nullptr, true); st != ET_OK)
    return st;
  void* ws = nullptr;
  if (const et_status st = scratch_ptr(&ws); st != ET_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  zero_words<<<1, 256, 0, s>>>(static_cast<unsigned long long*>(ws),
                                static_cast<int64_t>(need / sizeof(unsigned long long)));
  if (hipGetLastError() != hipSuccess) return ET_ERR_HIP;
  return argmax_entry<S>(x, rows, n, out, ws, need, stream);
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
  return static_cast<size_t>(rows) * 16;  // key (8 bytes) + counter (4) + padding (4)
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

et_status et_argmax_noalloc(int storage, const void* x, int64_t rows, int64_t n, int32_t* out,
                            void* stream) {
  switch (storage) {
    case ET_STORAGE_F32:
      return et::argmax_noalloc<float>(static_cast<const float*>(x), rows, n, out, stream);
    case ET_STORAGE_BF16:
      return et::argmax_noalloc<Bf16>(static_cast<const Bf16*>(x), rows, n, out, stream);
    case ET_STORAGE_F16:
      return et::argmax_noalloc<F16>(static_cast<const F16*>(x), rows, n, out, stream);
    default:
      return ET_ERR_BAD_ARG;
  }
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
