// eltwise.hip -- residual add and SiLU-gated multiply for gfx950.
//
// Definitions: "Operations" 1 Add, 4 Activation / Silu, SwiGlu;
// "Elementwise kernels in C ..." 2.3 SiLU-mul, 2.4 add.
//   add:      y = a + b
//   silu_mul: y = g / (1 + exp(-g)) * u   (exp overflows to +inf for very
//             negative g, making the factor -0 rather than NaN)
//
// Design: three streams, each element read once and written once.  Each
// thread moves kU 16-byte vectors per input, all loads issued before any
// store (loads are clamped in range rather than guarded, so the compiler
// keeps them in flight together).  Elements past the last whole vector are
// done by the last block with scalar accesses.  Misaligned buffers use the
// scalar kernel.  y may equal a or b: every element is read by the thread
// that writes it, before it writes it.
#include "et_common.hpp"

namespace et {
namespace {

constexpr int kBlock = 256;
constexpr int kU = 4;  // vectors per thread per input

// Vector index of slot u of thread tid in block b.  A block covers
// kBlock * kU consecutive vectors and each wave owns a contiguous quarter of
// them (slot u of lane l at u * 64 + l).
__device__ inline int64_t slot_index(int64_t b, int tid, int u) {
  return b * (kBlock * kU) + (tid / 64) * (64 * kU) + u * 64 + (tid % 64);
}

enum Op { kAdd = 0, kSiluMul = 1, kGeluErfMul = 2, kGeluTanhMul = 3 };

// silu(g) = g / (1 + e^-g).  f32 storage: library expf and IEEE division.
// 2-byte storage (bf16, f16): the f32 value only has to be within ~1e-5
// relative before the final rounding to 8 or 11 significant bits, so the
// hardware exp2 and reciprocal (quarter-rate transcendental instructions,
// about 1 ulp of f32 each) replace the library calls -- at 2 bytes the op
// moves 6 bytes per element and the accurate sequence would make it
// ALU-bound.  The reciprocal flushes denormal results, so a 1 + e^-g above
// 2^64 is scaled by 2^-64 together with g (both exact); e^-g overflowing to
// +inf still gives g * 0 = -0 for very negative g.
template <typename S>
__device__ inline float silu(float g) {
  if constexpr (sizeof(S) == 4) {
    return g / (1.0f + expf(-g));
  } else {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896340736f);
    const float t = 1.0f + e;
    const float sc = t > 0x1p+64f ? 0x1p-64f : 1.0f;
    return (g * sc) * __builtin_amdgcn_rcpf(t * sc);
  }
}

// erfc, branch free: the Chebyshev-fitted form of Press, Teukolsky,
// Vetterling and Flannery, Numerical Recipes (2nd ed.), section 6.2: for
// a = |z|, t = 1 / (1 + a/2) and erfc(a) = t exp(-a^2 + P(t)), fractional
// error below 1.2e-7 for every a >= 0 with P of degree 9.  The library erfcf
// branches by range, so a wave of mixed arguments runs every branch: it made
// the bf16 GELU-gated multiply ALU-bound (103 us where 57 us moves the bytes).
// For 2-byte storage, whose results keep 8 or 11 significant bits, P has
// degree 5 instead, fitted here to log(erfc(a) e^(a^2) / t) over 0 <= a <= 12
// (Chebyshev nodes in t, weighted least squares iterated toward the minimax
// fit, coefficients rounded to f32): relative error below 1.3e-5 against
// scipy's erfc (1.2e-4 out to a = 20), four fused multiply-adds fewer in a
// kernel whose 2-byte form is close to ALU-bound.
//
// Both are evaluated in base 2 and at t8 = t / 8:
//   Phi(-|x|) = erfc(a) / 2 = t8 2^K,  K = P'(t8) - a'^2,
//   a' = a sqrt(log2 e),  t8 = 1 / (8 + (4 / sqrt(log2 e)) a'),
//   P'(t8) = (P(8 t8) + 2 ln 2) log2 e,
// so coefficient i of P' is P's times 8^i log2 e (the power of 8 is exact)
// and its constant term is (c0 + 2 ln 2) log2 e.  Since |x| t8 = |x| / (8 +
// 2 sqrt(2) |x|) < 2^-1.5, |x| t8 2^(K - floor K) stays below 2^-0.5.
constexpr double kLog2eD = 1.44269504088896340736;
constexpr double kLn2D = 0.69314718055994530942;
#define ET_ERFC_C(c, i) static_cast<float>((c) * (i) * kLog2eD)
#define ET_ERFC_C0(c) static_cast<float>(((c) + 2.0 * kLn2D) * kLog2eD)

__device__ inline float erfc_exp2_poly9(float t8) {
  float p = ET_ERFC_C(0.17087277, 134217728.0);
  p = __builtin_fmaf(p, t8, ET_ERFC_C(-0.82215223, 16777216.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(1.48851587, 2097152.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(-1.13520398, 262144.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0.27886807, 32768.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(-0.18628806, 4096.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0.09678418, 512.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0.37409196, 64.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(1.00002368, 8.0));
  return __builtin_fmaf(p, t8, ET_ERFC_C0(-1.26551223));
}

__device__ inline float erfc_exp2_poly5(float t8) {
  float p = ET_ERFC_C(0x1.d141fp-3, 32768.0);
  p = __builtin_fmaf(p, t8, ET_ERFC_C(-0x1.68beacp-1, 4096.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0x1.e0c8f6p-2, 512.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0x1.071e78p-2, 64.0));
  p = __builtin_fmaf(p, t8, ET_ERFC_C(0x1.04764ap+0, 8.0));
  return __builtin_fmaf(p, t8, ET_ERFC_C0(-0x1.4438d8p+0));
}
#undef ET_ERFC_C
#undef ET_ERFC_C0

// GELU-gated product, exact form: x Phi(x) u, with Phi(x) = erfc(-x/sqrt 2) / 2
// (the identity 1 + erf(z) = erfc(-z) keeps the tail of negative x, where
// 1 + erf cancels), Phi(-|x|) = t8 2^K as above and Phi(|x|) = 1 - Phi(-|x|).
// While K >= -100 (|x| below about 12: every gate a model produces), 2^K is
// a normal number, q = t8 2^K = Phi(-|x|) is at least 2^-105 and
// |x q| <= max x Phi(-x) < 0.17, so x q u is finite for every finite u,
// nonzero times an infinite one, and rounds once: one exp2 does.  Past that
// (and for x = +-inf), the exact tail below; a wave runs it only when one of
// its lanes needs it.
constexpr float kGeluA = 0x1.b2da4ep-1f;   // sqrt(log2(e) / 2): a' = |x| kGeluA
constexpr float kGeluT = 0x1.aa449ap+1f;   // 4 / sqrt(log2 e): 8 + 4a = 8 + kGeluT a'

template <typename S>
__device__ inline float gelu_erf_tail(float x, float u);

template <typename S>
__device__ inline float gelu_erf_mul(float x, float u) {
  const float ap = __builtin_fabsf(x) * kGeluA;
  const float t8 = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluT, ap, 8.0f));
  const float p = sizeof(S) == 4 ? erfc_exp2_poly9(t8) : erfc_exp2_poly5(t8);
  const float k = __builtin_fmaf(-ap, ap, p);
  if (k < -100.0f) return gelu_erf_tail<S>(x, u);
  const float q = t8 * __builtin_amdgcn_exp2f(k);              // Phi(-|x|)
  return x <= 0.0f ? x * q * u : x * (1.0f - q) * u;
}

// The tail, K < -100.  The hardware exp2 returns no subnormals, so 2^K alone
// would flush every Phi below 2^-126 -- results x Phi(x) u down to 2^-149
// from x near -13 on in f32 and bf16 storage, and every product with a large
// or infinite up beyond that.  So K (held above -320) is split into its floor
// n and a fraction: q = t8 2^(K - n), Phi(-|x|) = q 2^n, |x q| < 2^-0.5, so
// x q u is finite for every finite u (below 2^127.5) and ldexp(x q u, n)
// rounds a subnormal result once and correctly; at K = -320 every such
// product times 2^K is below half the smallest subnormal.  |x| is held at
// 2^100 (a' below 2^100, whose reciprocal in t8 would flush from 2^127 on),
// in the product on the negative side as well: past it the held K is -320,
// and a larger |x| against the held t8 would break the bound on |x q| (x =
// -3e38 gives |x q| near 2^26, and x q u overflows for |u| above 2^102
// before ldexp could scale it to zero).  So q is never 0 for a finite x: x
// Phi(x) is nonzero for every finite x, and its product with an infinite u
// is an infinity.  Phi(-inf) is 0 and -inf * 0 has no value: NaN.
template <typename S>
__device__ inline float gelu_erf_tail(float x, float u) {
  const float xa = __builtin_fminf(__builtin_fabsf(x), 0x1p100f);
  const float ap = xa * kGeluA;
  const float t8 = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluT, ap, 8.0f));
  const float p = sizeof(S) == 4 ? erfc_exp2_poly9(t8) : erfc_exp2_poly5(t8);
  const float kc = __builtin_fmaxf(__builtin_fmaf(-ap, ap, p), -320.0f);
  const float n = __builtin_floorf(kc);
  const int ni = static_cast<int>(n);
  const float q = t8 * __builtin_amdgcn_exp2f(kc - n);         // Phi(-|x|) = q 2^n
  const float r = x <= 0.0f ? __builtin_ldexpf(-xa * q * u, ni)
                            : x * (1.0f - __builtin_ldexpf(q, ni)) * u;
  return x == -__builtin_inff() ? __builtin_nanf("") : r;
}

// The exact form over one vector of W elements: the one-exp2 evaluation of
// every element first, then the tail, for the elements that need it, in one
// branch per vector instead of one per element (the same results element by
// element: the tail replaces exactly the elements gelu_erf_mul sends to it).
template <typename S, int W>
__device__ inline void gelu_erf_mul_vec(const float (&x)[W], const float (&u)[W], float (&o)[W]) {
  float k[W];
  bool tail = false;
#pragma unroll
  for (int e = 0; e < W; ++e) {
    const float ap = __builtin_fabsf(x[e]) * kGeluA;
    const float t8 = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluT, ap, 8.0f));
    const float p = sizeof(S) == 4 ? erfc_exp2_poly9(t8) : erfc_exp2_poly5(t8);
    k[e] = __builtin_fmaf(-ap, ap, p);
    tail = tail || k[e] < -100.0f;
    const float q = t8 * __builtin_amdgcn_exp2f(k[e]);           // Phi(-|x|)
    o[e] = x[e] <= 0.0f ? x[e] * q * u[e] : x[e] * (1.0f - q) * u[e];
  }
  if (tail) {
#pragma unroll
    for (int e = 0; e < W; ++e)
      if (k[e] < -100.0f) o[e] = gelu_erf_tail<S>(x[e], u[e]);
  }
}

// GELU, tanh form: (1 + tanh u) / 2 = 1 / (1 + e^(-2u)) with
// u = sqrt(2/pi) (x + 0.044715 x^3), so it is x / (1 + e^(-2u)) -- the SiLU
// shape, computed the same way (library expf and IEEE division in f32; the
// hardware exp2 and reciprocal with the 2^-64 rescale for 2-byte storage).
template <typename S>
__device__ inline float gelu_tanh(float x) {
  const float u2 = -1.59576912160573071176f * __builtin_fmaf(0.044715f * x, x * x, x);  // -2u
  if constexpr (sizeof(S) == 4) {
    return x / (1.0f + expf(u2));
  } else {
    const float e = __builtin_amdgcn_exp2f(u2 * 1.44269504088896340736f);
    const float t = 1.0f + e;
    const float sc = t > 0x1p+64f ? 0x1p-64f : 1.0f;
    return (x * sc) * __builtin_amdgcn_rcpf(t * sc);
  }
}

template <typename S, int OP>
__device__ inline float apply(float a, float b) {
  if constexpr (OP == kAdd) {
    return a + b;
  } else if constexpr (OP == kSiluMul) {
    return silu<S>(a) * b;
  } else if constexpr (OP == kGeluErfMul) {
    return gelu_erf_mul<S>(a, b);
  } else {
    return gelu_tanh<S>(a) * b;
  }
}

template <typename S, int OP>
__global__ __launch_bounds__(kBlock) void eltwise_vec(const S* a, const S* b, S* y, int64_t nvec,
                                                      int64_t n) {
  using E = Elem<S>;
  constexpr int V = E::V;
  const int64_t blk = blockIdx.x;
  if (nvec > 0) {
    u32x4 av[kU], bv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = slot_index(blk, threadIdx.x, u);
      const int64_t jc = j < nvec ? j : nvec - 1;
      av[u] = ld16(a, jc * V);
      bv[u] = ld16(b, jc * V);
    }
    // Stores go through a resource based at the block's first vector.
    const int64_t vbase = blk * (kBlock * kU);
    const __amdgpu_buffer_rsrc_t ry = out_rsrc(y + vbase * V, (nvec - vbase) * 16);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = slot_index(blk, threadIdx.x, u);
      float o[V];
      if constexpr (OP == kGeluErfMul) {
        float xa[V], xb[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xa[e] = E::get(av[u], e);
          xb[e] = E::get(bv[u], e);
        }
        gelu_erf_mul_vec<S, V>(xa, xb, o);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = apply<S, OP>(E::get(av[u], e), E::get(bv[u], e));
      }
      if (j < nvec) st16_buf(ry, static_cast<int>((j - vbase) * 16), E::pack(o));
    }
  }
  // Tail: fewer than V elements after the last whole vector.
  if (blockIdx.x == gridDim.x - 1) {
    const int64_t i = nvec * V + threadIdx.x;
    if (i < n) E::st(y, i, apply<S, OP>(E::ld(a, i), E::ld(b, i)));
  }
}

template <typename S, int OP>
__global__ __launch_bounds__(kBlock) void eltwise_scalar(const S* a, const S* b, S* y, int64_t n) {
  using E = Elem<S>;
  constexpr int kPer = kU * 4;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * (kBlock * kPer) + threadIdx.x;
  float av[kPer], bv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t i = first + u * kBlock;
    const int64_t ic = i < n ? i : n - 1;
    av[u] = E::ld(a, ic);
    bv[u] = E::ld(b, ic);
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t i = first + u * kBlock;
    if (i < n) E::st(y, i, apply<S, OP>(av[u], bv[u]));
  }
}

template <typename S, int OP>
et_status eltwise_entry(const S* a, const S* b, S* y, int64_t n, void* stream) {
  if (n < 0) return ET_ERR_BAD_SIZE;
  if (n == 0) return ET_OK;
  int64_t bytes = 0;
  if (!mul_ok(n, static_cast<int64_t>(sizeof(S)), &bytes)) return ET_ERR_BAD_SIZE;
  if (!a || !b || !y) return ET_ERR_NULL_POINTER;
  if (!ranges_ok(y, bytes, a, bytes, true) || !ranges_ok(y, bytes, b, bytes, true))
    return ET_ERR_OVERLAP;
  constexpr int V = Elem<S>::V;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (aligned16(a) && aligned16(b) && aligned16(y)) {
    // Split into launches of at most kMaxGrid blocks; each launch starts on
    // a vector boundary, only the last one has a tail.
    const int64_t per_launch = kMaxGrid * kBlock * kU;  // vectors
    const int64_t nvec_all = n / V;
    for (int64_t v0 = 0;; v0 += per_launch) {
      const int64_t nvec = nvec_all - v0 < per_launch ? nvec_all - v0 : per_launch;
      const bool last = v0 + nvec >= nvec_all;
      const int64_t elems = last ? n - v0 * V : nvec * V;
      const int64_t blocks = nvec > 0 ? (nvec + kBlock * kU - 1) / (kBlock * kU) : 1;
      const int64_t off = v0 * V;
      eltwise_vec<S, OP><<<static_cast<unsigned>(blocks), kBlock, 0, s>>>(a + off, b + off,
                                                                        y + off, nvec, elems);
      if (last) break;
    }
  } else {
    const int64_t per_launch = kMaxGrid * kBlock * kU * 4;
    for (int64_t i0 = 0; i0 < n; i0 += per_launch) {
      const int64_t m = n - i0 < per_launch ? n - i0 : per_launch;
      const int64_t blocks = (m + kBlock * kU * 4 - 1) / (kBlock * kU * 4);
      eltwise_scalar<S, OP><<<static_cast<unsigned>(blocks), kBlock, 0, s>>>(a + i0, b + i0,
                                                                             y + i0, m);
    }
  }
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

et_status et_add_f32(const float* a, const float* b, float* y, int64_t n, void* stream) {
  return et::eltwise_entry<float, et::kAdd>(a, b, y, n, stream);
}

et_status et_add_bf16(const et_bf16* a, const et_bf16* b, et_bf16* y, int64_t n, void* stream) {
  return et::eltwise_entry<Bf16, et::kAdd>(reinterpret_cast<const Bf16*>(a),
                                           reinterpret_cast<const Bf16*>(b),
                                           reinterpret_cast<Bf16*>(y), n, stream);
}

et_status et_add_f16(const et_f16* a, const et_f16* b, et_f16* y, int64_t n, void* stream) {
  return et::eltwise_entry<F16, et::kAdd>(reinterpret_cast<const F16*>(a),
                                           reinterpret_cast<const F16*>(b),
                                           reinterpret_cast<F16*>(y), n, stream);
}

et_status et_silu_mul_f32(const float* gate, const float* up, float* y, int64_t n, void* stream) {
  return et::eltwise_entry<float, et::kSiluMul>(gate, up, y, n, stream);
}

et_status et_silu_mul_bf16(const et_bf16* gate, const et_bf16* up, et_bf16* y, int64_t n,
                           void* stream) {
  return et::eltwise_entry<Bf16, et::kSiluMul>(reinterpret_cast<const Bf16*>(gate),
                                               reinterpret_cast<const Bf16*>(up),
                                               reinterpret_cast<Bf16*>(y), n, stream);
}

et_status et_silu_mul_f16(const et_f16* gate, const et_f16* up, et_f16* y, int64_t n,
                           void* stream) {
  return et::eltwise_entry<F16, et::kSiluMul>(reinterpret_cast<const F16*>(gate),
                                               reinterpret_cast<const F16*>(up),
                                               reinterpret_cast<F16*>(y), n, stream);
}

}  // extern "C"

extern "C" {

et_status et_geglu_f32(const float* gate, const float* up, float* y, int64_t n, int approximate,
                       void* stream) {
  if (approximate == ET_GELU_ERF) return et::eltwise_entry<float, et::kGeluErfMul>(gate, up, y, n, stream);
  if (approximate == ET_GELU_TANH) return et::eltwise_entry<float, et::kGeluTanhMul>(gate, up, y, n, stream);
  return n < 0 ? ET_ERR_BAD_SIZE : ET_ERR_BAD_ARG;
}

et_status et_geglu_bf16(const et_bf16* gate, const et_bf16* up, et_bf16* y, int64_t n,
                        int approximate, void* stream) {
  const auto* g = reinterpret_cast<const Bf16*>(gate);
  const auto* u = reinterpret_cast<const Bf16*>(up);
  auto* o = reinterpret_cast<Bf16*>(y);
  if (approximate == ET_GELU_ERF) return et::eltwise_entry<Bf16, et::kGeluErfMul>(g, u, o, n, stream);
  if (approximate == ET_GELU_TANH) return et::eltwise_entry<Bf16, et::kGeluTanhMul>(g, u, o, n, stream);
  return n < 0 ? ET_ERR_BAD_SIZE : ET_ERR_BAD_ARG;
}

et_status et_geglu_f16(const et_f16* gate, const et_f16* up, et_f16* y, int64_t n,
                        int approximate, void* stream) {
  const auto* g = reinterpret_cast<const F16*>(gate);
  const auto* u = reinterpret_cast<const F16*>(up);
  auto* o = reinterpret_cast<F16*>(y);
  if (approximate == ET_GELU_ERF) return et::eltwise_entry<F16, et::kGeluErfMul>(g, u, o, n, stream);
  if (approximate == ET_GELU_TANH) return et::eltwise_entry<F16, et::kGeluTanhMul>(g, u, o, n, stream);
  return n < 0 ? ET_ERR_BAD_SIZE : ET_ERR_BAD_ARG;
}

}  // extern "C"
