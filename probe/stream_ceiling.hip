// stream_ceiling.hip -- plain HBM streams for gfx950: the yardstick the
// benchmark measures the library's kernels against.  It is built apart
// (probe/libet_probe.so) and computes nothing of the transformer ops.
//
// One launch streams n_read buffers in and n_write buffers out, each `bytes`
// long, with nothing between the loads and the stores: the output is the
// XOR (first output) and the sum (second) of the 16-byte words read, so no
// line written is all zeros (zero lines are written faster than data and
// would overstate the ceiling) and a pure read still has a data-dependent
// store the compiler cannot drop.  The access pattern is the library's:
// 16-byte buffer loads with the non-temporal cache policy and stores with
// the non-temporal one (the library's) or, as a yardstick, the device-scope
// one, 256 threads per workgroup, each wave
// owning 64 * U consecutive vectors (U = 4 or 8 per lane), every load index
// clamped below the vector count and every store guarded by it.
//
// Two grid shapes: one workgroup per 256 * U vectors (the library's
// kernels' shape), or a persistent grid of a given number of workgroups
// that step through the buffer by the grid's span (grid-stride), so the
// dispatch of workgroups is paid once per workgroup slot instead of once
// per tile.
//
// Also here: a hold kernel for the benchmark's timing of small kernels.  It
// keeps the stream busy for a given time, so the host can enqueue a whole
// batch of timed launches behind it; they then run back to back, and their
// events time the GPU, not the host's pace.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace etprobe {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kNonTemporal = 2;   // cache-policy bits of a buffer access: nt
constexpr int kDeviceScope = 16;  // sc1: device scope

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  // 0x00020000: the raw-buffer data format word of gfx9-class resources.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// One tile of kBlock * U vectors starting at vector t0.
template <int NR, int NW, int U, int POL>
__device__ inline void stream_tile(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                   __amdgpu_buffer_rsrc_t ry, __amdgpu_buffer_rsrc_t rh,
                                   int64_t t0, int64_t nvec) {
  const int64_t base = t0 + (threadIdx.x / 64) * (64 * U) + (threadIdx.x % 64);
  i32x4 va[U], vb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * 64;
    const int off = static_cast<int>((i < nvec ? i : nvec - 1) * 16);
    if constexpr (NR >= 1) va[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, kNonTemporal);
    else va[u] = i32x4{static_cast<int>(i), 0x5bd1e995, static_cast<int>(i >> 7), 0x1b873593};
    if constexpr (NR >= 2) vb[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, kNonTemporal);
    else vb[u] = i32x4{0x11, 0x22, 0x33, 0x44};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * 64;
    if (i >= nvec) continue;
    const int off = static_cast<int>(i * 16);
    const i32x4 v = va[u] ^ vb[u];
    if constexpr (NW >= 1) {
      __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, POL);
    } else if (v.x == 0x7fffffff && v.y == 0x7fffffff && v.z == 0x7fffffff && v.w == 0x7fffffff) {
      // pure read: a store no real data takes, so the loads stay
      __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, kNonTemporal);
    }
    if constexpr (NW >= 2) __builtin_amdgcn_raw_buffer_store_b128(va[u] + vb[u], rh, off, 0, POL);
  }
}

template <int NR, int NW, int U, int POL, bool PERSIST>
__global__ __launch_bounds__(kBlock) void stream_kernel(const void* a, const void* b, void* y,
                                                        void* h, int64_t nvec) {
  const uint32_t bytes = static_cast<uint32_t>(nvec * 16);
  const __amdgpu_buffer_rsrc_t ra = rsrc(a, bytes), rb = rsrc(b, bytes);
  const __amdgpu_buffer_rsrc_t ry = rsrc(y, bytes), rh = rsrc(h, bytes);
  constexpr int64_t kTile = int64_t{kBlock} * U;
  if constexpr (PERSIST) {
    // Every workgroup leaves the loop once its next tile starts past the end.
    for (int64_t t0 = blockIdx.x * kTile; t0 < nvec; t0 += int64_t{gridDim.x} * kTile)
      stream_tile<NR, NW, U, POL>(ra, rb, ry, rh, t0, nvec);
  } else {
    stream_tile<NR, NW, U, POL>(ra, rb, ry, rh, blockIdx.x * kTile, nvec);
  }
}

template <int NR, int NW, int U, bool PERSIST>
void launch(bool dev, unsigned grid, const void* a, const void* b, void* y, void* h, int64_t nvec,
            hipStream_t s) {
  if (dev) stream_kernel<NR, NW, U, kDeviceScope, PERSIST><<<grid, kBlock, 0, s>>>(a, b, y, h, nvec);
  else stream_kernel<NR, NW, U, kNonTemporal, PERSIST><<<grid, kBlock, 0, s>>>(a, b, y, h, nvec);
}

template <int NR, int NW>
void launch_u(int u, int persist_blocks, bool dev, const void* a, const void* b, void* y, void* h,
              int64_t nvec, hipStream_t s) {
  const int64_t tile = int64_t{kBlock} * u;
  const int64_t tiles = (nvec + tile - 1) / tile;
  if (persist_blocks > 0) {
    const unsigned grid = static_cast<unsigned>(persist_blocks < tiles ? persist_blocks : tiles);
    if (u == 8) launch<NR, NW, 8, true>(dev, grid, a, b, y, h, nvec, s);
    else launch<NR, NW, 4, true>(dev, grid, a, b, y, h, nvec, s);
  } else {
    const unsigned grid = static_cast<unsigned>(tiles);
    if (u == 8) launch<NR, NW, 8, false>(dev, grid, a, b, y, h, nvec, s);
    else launch<NR, NW, 4, false>(dev, grid, a, b, y, h, nvec, s);
  }
}

}  // namespace
}  // namespace etprobe

// One wave that waits until `ticks` of the constant-rate wall clock have
// passed since it started, then exits (the clock always advances, so every
// launch ends; the host caps the time at 100 ms).  Outside the probe's
// namespace, so profile summaries that match the library's and the probe's
// kernels by namespace skip it.
__global__ void probe_hold_kernel(long long ticks) {
  const long long t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(32);
}

extern "C" {

// Keeps `stream` busy for `microseconds` (1..100000) with one wave of
// probe_hold_kernel, counting the 100 MHz reference clock that wall_clock64()
// reads on this GPU family (the runtime's wall-clock-rate attribute gave a
// hold 60 times too long here, so it is not used).  Returns 0 on a launch, 1
// on a bad argument, 2 when the launch reports an error.
int et_probe_hold(int64_t microseconds, void* stream) {
  if (microseconds < 1 || microseconds > 100000) return 1;
  constexpr long long kTicksPerUs = 100;
  const long long ticks = static_cast<long long>(microseconds) * kTicksPerUs;
  (void)hipGetLastError();
  probe_hold_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(ticks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}


// Streams `n_read` buffers of `bytes` bytes in and `n_write` out in one
// launch on `stream`, (n_read, n_write) one of (0, 1), (1, 0), (1, 1),
// (2, 1), (2, 2), with `u` (4 or 8) vectors per lane, stores non-temporal
// (device_scope == 0) or device-scope (otherwise).  persist_blocks == 0
// launches one workgroup per 256 * u vectors; a value in 1..65536 launches
// that many workgroups (at most one per tile) stepping through the buffer
// by the grid's span.  a (read when n_read >= 1), b (n_read == 2), y
// (written when n_write >= 1; the guard store of a pure read targets it
// too, so it is always needed) and h (n_write == 2) are device pointers,
// 16-byte aligned, each `bytes` long; an unused a, b or h may be NULL.
// bytes must be a positive multiple of 16 below 2^31 (32-bit buffer
// offsets).  Returns 0 on a launch, 1 on bad arguments (nothing launched),
// 2 when the launch reports an error.
int et_probe_stream(const void* a, const void* b, void* y, void* h, int64_t bytes, int n_read,
                    int n_write, int u, int device_scope, int persist_blocks, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || bytes > INT32_MAX - 15) return 1;
  if (n_read < 0 || n_read > 2 || n_write < 0 || n_write > 2 || n_read + n_write == 0) return 1;
  if (u != 4 && u != 8) return 1;
  if (persist_blocks < 0 || persist_blocks > 65536) return 1;
  if ((n_read >= 1 && !a) || (n_read == 2 && !b) || !y || (n_write == 2 && !h)) return 1;
  for (const void* p : {a, b, static_cast<const void*>(y), static_cast<const void*>(h)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return 1;
  const int64_t nvec = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool dev = device_scope != 0;
  const int pb = persist_blocks;
  using etprobe::launch_u;
  if (n_read == 0 && n_write == 1) launch_u<0, 1>(u, pb, dev, a, b, y, h, nvec, s);
  else if (n_read == 1 && n_write == 0) launch_u<1, 0>(u, pb, dev, a, b, y, h, nvec, s);
  else if (n_read == 1 && n_write == 1) launch_u<1, 1>(u, pb, dev, a, b, y, h, nvec, s);
  else if (n_read == 2 && n_write == 1) launch_u<2, 1>(u, pb, dev, a, b, y, h, nvec, s);
  else if (n_read == 2 && n_write == 2) launch_u<2, 2>(u, pb, dev, a, b, y, h, nvec, s);
  else return 1;  // 0R2W, 1R2W, 2R0W: not offered
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
