// et_common.hpp -- shared pieces of the gfx950 kernels and their host-side
// launchers: storage types, 16-byte vector I/O, fixed-order wavefront
// reductions, exact integer division by run-time constants, and the argument
// checks every entry point runs before it enqueues anything.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "et.h"

namespace et {

// ---------------------------------------------------------------- storage
// Kernels are templated on the storage type: float (f32), Bf16 (raw
// bfloat16 bits) or F16 (raw IEEE binary16 bits).  Arithmetic is always f32.
struct Bf16 {
  uint16_t bits;
};
struct F16 {
  uint16_t bits;
};

// One 16-byte vector as a native clang vector (usable with the nontemporal
// builtins, unlike HIP's u32x4 struct).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename S>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int V = 4;  // elements per 16-byte vector
  __device__ static inline float ld(const float* p, int64_t i) { return p[i]; }
  __device__ static inline void st(float* p, int64_t i, float v) { p[i] = v; }
  __device__ static inline void unpack(const u32x4& u, float (&f)[4]) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static inline u32x4 pack(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
  __device__ static inline float round(float v) { return v; }  // to storage precision
  // Element e (compile-time after unrolling) of a packed vector.
  __device__ static inline float get(const u32x4& u, int e) { return __uint_as_float(u[e]); }
  static constexpr uint32_t kQuietNaN = 0x7FC00000u;
};

// bf16 -> f32 is exact (the bf16 bits are the high half of the f32 bits).
// f32 -> bf16 rounds to nearest even; on gfx950 the conversion below is the
// hardware v_cvt_pk_bf16_f32.
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16_pack2(float lo, float hi) {
  // One v_cvt_pk_bf16_f32 for the pair.
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <>
struct Elem<Bf16> {
  static constexpr int V = 8;
  __device__ static inline float ld(const Bf16* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i].bits) << 16);
  }
  __device__ static inline void st(Bf16* p, int64_t i, float v) {
    p[i].bits = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
  __device__ static inline void unpack(const u32x4& u, float (&f)[8]) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  __device__ static inline u32x4 pack(const float (&f)[8]) {
    return u32x4{bf16_pack2(f[0], f[1]), bf16_pack2(f[2], f[3]), bf16_pack2(f[4], f[5]),
                 bf16_pack2(f[6], f[7])};
  }
  __device__ static inline float round(float v) {  // to storage precision (RNE)
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)))
                           << 16);
  }
  __device__ static inline float get(const u32x4& u, int e) {
    return (e & 1) ? bf16_hi(u[e >> 1]) : bf16_lo(u[e >> 1]);
  }
  static constexpr uint32_t kQuietNaN = 0x7FC07FC0u;  // two bf16 quiet NaNs
  // The entries of one 32-bit word (entry 0 in the low half).
  __device__ static inline float lo(uint32_t w) { return bf16_lo(w); }
  __device__ static inline float hi(uint32_t w) { return bf16_hi(w); }
};

// f16 -> f32 is exact (every binary16 value, subnormals included, is an f32
// normal); f32 -> f16 rounds to nearest even (v_cvt_f16_f32), overflowing to
// infinity past 65504 and keeping subnormals.  An f32 result rounded once to
// f16 is the correctly rounded f16 of the exact result whenever the f32 one
// was, and for a sum or product of two f16 values it always is: f32 carries
// 24 >= 2 * 11 + 2 significant bits, so the double rounding is harmless.
__device__ inline float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ inline float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
__device__ inline uint32_t f16_bits(float v) {
  // The f32 value is formed first: left alone, the compiler may fold the last
  // multiply or multiply-add into a mixed-precision FMA that rounds straight
  // to f16 (v_fma_mixlo_f16) in one code path and not in another, so the
  // vector and scalar paths of a kernel could differ in the last bit.  The
  // empty asm makes v opaque; the conversion is then v_cvt_f16_f32 alone.
  __asm__("" : "+v"(v));
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v)));
}
__device__ inline uint32_t f16_pack2(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }

template <>
struct Elem<F16> {
  static constexpr int V = 8;
  __device__ static inline float ld(const F16* p, int64_t i) {
    return static_cast<float>(__builtin_bit_cast(_Float16, p[i].bits));
  }
  __device__ static inline void st(F16* p, int64_t i, float v) {
    p[i].bits = static_cast<uint16_t>(f16_bits(v));
  }
  __device__ static inline void unpack(const u32x4& u, float (&f)[8]) {
    f[0] = f16_lo(u.x); f[1] = f16_hi(u.x);
    f[2] = f16_lo(u.y); f[3] = f16_hi(u.y);
    f[4] = f16_lo(u.z); f[5] = f16_hi(u.z);
    f[6] = f16_lo(u.w); f[7] = f16_hi(u.w);
  }
  __device__ static inline u32x4 pack(const float (&f)[8]) {
    return u32x4{f16_pack2(f[0], f[1]), f16_pack2(f[2], f[3]), f16_pack2(f[4], f[5]),
                 f16_pack2(f[6], f[7])};
  }
  __device__ static inline float round(float v) {  // to storage precision (RNE)
    return static_cast<float>(static_cast<_Float16>(v));
  }
  __device__ static inline float get(const u32x4& u, int e) {
    return (e & 1) ? f16_hi(u[e >> 1]) : f16_lo(u[e >> 1]);
  }
  static constexpr uint32_t kQuietNaN = 0x7E007E00u;  // two f16 quiet NaNs
  __device__ static inline float lo(uint32_t w) { return f16_lo(w); }
  __device__ static inline float hi(uint32_t w) { return f16_hi(w); }
};

// 16-byte vector access; the caller guarantees 16-byte alignment.
// ld16/st16 are for data touched once (activations streamed through HBM):
// they carry the nontemporal hint, so the lines are not kept in the caches
// (this raised a 2-read/1-write stream from ~5.4 to ~6.1 TB/s on MI355X).
// ld16_keep is for small operands every row re-reads (gains).
template <typename S>
__device__ inline u32x4 ld16(const S* p, int64_t elem) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + elem));
}
template <typename S>
__device__ inline void st16(S* p, int64_t elem, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p + elem));
}
template <typename S>
__device__ inline u32x4 ld16_keep(const S* p, int64_t elem) {
  return *reinterpret_cast<const u32x4*>(p + elem);
}

// Output stores go through a buffer resource with the non-temporal bit set
// (cache policy nt = 2), so the line streams to HBM.  Device-scope
// write-through (sc1), which leaves the line in the 256 MB Infinity Cache to
// be written back behind later work, was used for outputs up to 64-128 MB
// and dropped: it made those kernels faster when timed alone over buffers
// rotated past the cache (an add writing 34 MB, 18.9 against 20.0 us;
// in-place RoPE writing 42 MB, 17.9 against 18.3 us) because each launch
// left part of its write-back to the next, and the kernels after it paid
// for that.  The whole prefill step (eight kernels, three interleaved
// rounds of 200 steps) ran 0.1621-0.1625 ms with non-temporal stores
// everywhere against 0.1637-0.1638 ms with device scope for add, SiLU-mul,
// GeGLU and RoPE.
constexpr int kStoreNT = 2;

// A resource for `bytes` bytes from `base` (a uniform pointer); stores at
// byte offsets beyond min(bytes, 2^31 - 1) are dropped by the hardware.
__device__ inline __amdgpu_buffer_rsrc_t out_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline void st16_buf(__amdgpu_buffer_rsrc_t r, int byte_off, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, byte_off, 0, kStoreNT);
}

// -------------------------------------------------------- wave reductions
// Sum over aligned groups of W lanes (W a power of two, W <= 64).  Within a
// 16-lane DPP row the partners come from DPP lane permutations (no LDS
// crossbar): quad_perm [1,0,3,2] and [2,3,0,1] pair lanes xor 1 and xor 2,
// row_half_mirror pairs each lane of a quad with a lane of the other quad of
// its 8-lane half, row_mirror pairs the two halves of the 16-lane row; groups
// of 32 and 64 add the partner 16 and 32 lanes away.  At every step a lane
// and its partner add the same two values (in swapped order, which IEEE
// addition does not see), so every lane of a group ends with the same bits,
// and the tree depends only on W.
namespace dpp {
constexpr int kXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror
constexpr int kMirror = 0x140;      // row_mirror
template <int CTRL>
__device__ inline float mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
}  // namespace dpp

template <int W>
__device__ inline float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two <= 64");
  if constexpr (W >= 2) v += dpp::mov<dpp::kXor1>(v);
  if constexpr (W >= 4) v += dpp::mov<dpp::kXor2>(v);
  if constexpr (W >= 8) v += dpp::mov<dpp::kHalfMirror>(v);
  if constexpr (W >= 16) v += dpp::mov<dpp::kMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// ------------------------------------------------- division by constants
// Exact n / d for 32-bit unsigned n and a run-time divisor d >= 1 fixed for
// the launch (multiply-high plus shift; Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994).
struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((uint64_t{1} << s) < d) ++s;  // s = ceil(log2 d)
  f.shift = s;
  f.magic = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << s) - d)) / d + 1);
  return f;
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
#ifdef __HIP_DEVICE_COMPILE__
  const uint64_t hi = __umulhi(n, f.magic);
#else
  const uint64_t hi = (static_cast<uint64_t>(n) * f.magic) >> 32;
#endif
  return static_cast<uint32_t>((hi + n) >> f.shift);
}

// ------------------------------------------------------------ host checks
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b with overflow detection; false if negative or overflowing.
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  return !__builtin_mul_overflow(a, b, out);
}

// Two byte ranges either coincide exactly (when `may_alias`) or are
// disjoint.  Empty ranges never overlap.
inline bool ranges_ok(const void* a, int64_t abytes, const void* b, int64_t bbytes,
                      bool may_alias) {
  if (abytes <= 0 || bbytes <= 0 || a == nullptr || b == nullptr) return true;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t a1 = a0 + static_cast<uintptr_t>(abytes);
  const uintptr_t b1 = b0 + static_cast<uintptr_t>(bbytes);
  if (a1 <= b0 || b1 <= a0) return true;
  return may_alias && a0 == b0 && abytes == bbytes;
}

inline et_status launch_status() {
  return hipGetLastError() == hipSuccess ? ET_OK : ET_ERR_HIP;
}

// Largest grid.x the launchers use per launch; longer work is split.
constexpr int64_t kMaxGrid = int64_t{1} << 30;

}  // namespace et
