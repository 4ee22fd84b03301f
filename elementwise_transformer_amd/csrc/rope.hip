// rope.hip -- rotary position embedding (Q and K in one launch) and the
// fused per-head RMSNorm + RoPE (QK-norm) for gfx950.
//
// Definitions: "Operations" 3 Position encoding / Rope and 5 Attention /
// QK-norm; "Elementwise kernels in C ..." 2.2 RoPE and 4 The interface.
//   angle of pair i at token t: p_t * w_i formed in f64, rounded to f32
//   (a, b) -> mu (a cos - b sin, a sin + b cos)
//   layout 0 (half) pairs (i, i + r/2); layout 1 (interleaved) (2i, 2i+1)
//   entries r..D-1 pass through (RoPE) or are only normalised (QK-norm).
//
// Design (HBM-bound: each rotated element read and written once):
//   * Work is cut into "slots" of PS pairs of one head row: with 16-byte
//     vectors PS = V (two vectors: V pairs), else PS = 1 (two scalars).
//     Both layouts make a slot's pairs i0..i0+PS-1 contiguous in i.
//   * A workgroup owns kBlock*U consecutive slots (possibly spanning token
//     boundaries).  It first issues all its loads, then builds a table of
//     (mu cos, mu sin) for its tokens' pairs in LDS -- one sincosf per
//     (token, pair), shared by all Hq + Hk heads -- then rotates and stores.
//   * sin/cos come from sincos_angle below: f64 Cody-Waite reduction plus
//     f32 Taylor polynomials, accurate for the ~1e6 rad angles of positions
//     near 2^20 at a fraction of the library's large-argument cost.
//   * In place: each slot is read and written by one thread, reads first.
//   * QK-norm: a group of G = D/(2V) lanes owns one head row (two vectors per
//     lane); the sum of squares is per-lane then an xor butterfly over the G
//     lanes -- fixed by D, so rows are batch-invariant.  Shapes without that
//     vector layout use a one-wave-per-row kernel.
#include <algorithm>
#include <vector>

#include "et_common.hpp"

namespace et {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxTableBytes = 48 * 1024;
// Slots per lane of the RoPE kernel (plain and cached angles): one.  With
// non-temporal stores one slot per lane ran faster than two at every size
// measured (in-place q and k writing 42, 67 and 151 MB: 17.59 against 18.45
// us, 25.62 against 26.02, 50.35 against 51.27; four interleaved rounds over
// buffers rotated past the Infinity Cache), and the prefill step 0.1612
// against 0.1619 ms.  Head rows per lane group of the fused RMSNorm + RoPE:
// one, likewise (42, 134 and 151 MB in place: 18.35 against 19.16 us, 44.82
// against 45.31, 50.79 against 51.99).
constexpr int kRopeU = 1;
constexpr int kQkU = 1;

struct RopeArgs {
  int64_t T;
  int hq, hk, D, r, half, layout;
  float mu;
  uint32_t sph;       // slots per head row
  uint32_t spt;       // slots per token
  uint32_t total;     // slots in the call (T * spt)
  FastDiv fd_spt;     // divide by slots per token
  FastDiv fd_sph;     // divide by slots per head row
  FastDiv fd_half;    // divide by r/2
  int ntok_max;       // tokens one workgroup can touch (table rows)
  // Cos/sin cache ("Operations" 3 Rope): when cached is set, the table
  // reads (cos, sin) of pair i at position p from cos_c / sin_c[p * half + i]
  // instead of computing them; positions outside [0, max_pos) give NaN.
  int cached;
  int max_pos;
  const float* cos_c;
  const float* sin_c;
};

// Angle of pair i of position p: the f64 product rounded once to f32.
__device__ inline float rope_angle(int32_t p, float w) {
  return static_cast<float>(static_cast<double>(p) * static_cast<double>(w));
}

// sin and cos of an f32 angle x.  For |x| < 2^31 (every int32 position
// times a frequency <= 1): Cody-Waite reduction by pi/2 in f64 -- k =
// rint(x * 2/pi), r = x - k*(pi/2) with pi/2 held as two doubles and fused
// multiply-adds, so r is exact to ~1e-16 -- then the Taylor series of sin
// (to r^9) and cos (to r^10) on |r| <= pi/4 in f32, and the quadrant k mod 4.
// Absolute error < 1e-7 (about 1.5 ulp of the result away from its zeros).
// The library's sincosf takes a far slower reduction path for the ~1e6 rad
// angles of positions near 2^20; larger |x| still goes to it.
__device__ inline void sincos_angle(float x, float* s, float* c) {
  if (!(fabsf(x) < 0x1p31f)) {
    sincosf(x, s, c);
    return;
  }
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr double kPio2Hi = 0x1.921fb54442d18p+0;   // pi/2 = hi + lo + O(2^-108)
  constexpr double kPio2Lo = 0x1.1a62633145c07p-54;
  const double xd = static_cast<double>(x);
  const double k = rint(xd * kTwoOverPi);
  const double r = fma(-k, kPio2Lo, fma(-k, kPio2Hi, xd));
  const float rf = static_cast<float>(r);
  const float r2 = rf * rf;
  // (-1)^n / (2n+1)! and (-1)^n / (2n)!, rounded to f32
  float ps = __builtin_fmaf(r2, 0x1.71de3ap-19f, -0x1.a01a02p-13f);
  ps = __builtin_fmaf(r2, ps, 0x1.111112p-7f);
  ps = __builtin_fmaf(r2, ps, -0x1.555556p-3f);
  const float sn = __builtin_fmaf(rf * r2, ps, rf);
  float pc = __builtin_fmaf(r2, -0x1.27e4fcp-22f, 0x1.a01a02p-16f);
  pc = __builtin_fmaf(r2, pc, -0x1.6c16c2p-10f);
  pc = __builtin_fmaf(r2, pc, 0x1.555556p-5f);
  pc = __builtin_fmaf(r2, pc, -0.5f);
  const float cn = __builtin_fmaf(r2, pc, 1.0f);
  const int q = static_cast<int>(k - 4.0 * floor(k * 0.25));  // k mod 4, in 0..3
  const float s_ = (q & 1) ? cn : sn;
  const float c_ = (q & 1) ? sn : cn;
  *s = (q & 2) ? -s_ : s_;
  *c = ((q + 1) & 2) ? -c_ : c_;
}

// The block's angle table cs[tl * half + i] = (mu cos, mu sin) for tokens
// t0 .. t0 + ntok - 1, built in two steps.  table_inputs fetches the position
// and frequency of this thread's first kTabPre entries; it runs before the
// row loads, because the row loads are waited for in issue order and a table
// input fetched after them would wait for every one of them.  table_fill
// then computes those entries (and, rarely, further ones).
constexpr int kTabPre = 2;
struct TabIn {
  int32_t p[kTabPre];
  float w[kTabPre];
};

// Needs half >= 1 (the caller launches no table otherwise).  Both loads are
// unconditional, so no branch separates them from the row loads: an index
// clamped instead of guarded, and with a cached table (where inv_freq may
// be NULL and the frequency is not used) a valid stand-in address, pos[t0].
// A branch there let the compiler convert the frequency to f64 inside it,
// which made every workgroup wait for that load before issuing its row
// loads (1.2 us of a 52 us RoPE launch at [8192, 64 + 8, 128] bf16).
__device__ inline TabIn table_inputs(int64_t t0, int ntok, const RopeArgs& a,
                                     const int32_t* __restrict__ pos,
                                     const float* __restrict__ inv_freq) {
  TabIn in;
  const uint32_t n = static_cast<uint32_t>(ntok) * a.half;
  const float* wsrc = a.cached ? reinterpret_cast<const float*>(pos + t0) : inv_freq;
#pragma unroll
  for (int k = 0; k < kTabPre; ++k) {
    uint32_t idx = threadIdx.x + k * kBlock;
    if (idx >= n) idx = n - 1;  // clamped, never guarded (see above)
    const uint32_t tl = fdiv(idx, a.fd_half);
    in.p[k] = pos[t0 + tl];
    in.w[k] = wsrc[a.cached ? 0u : idx - tl * a.half];
  }
  return in;
}

// Cached (mu cos, mu sin) of pair i at position p; NaN outside the cache.
__device__ inline float2 cached_cs(int32_t p, uint32_t i, const RopeArgs& a) {
  // Out-of-range positions load nothing (the cache may even be empty).
  float cn = __builtin_nanf(""), sn = cn;
  if (p >= 0 && p < a.max_pos) {
    const int64_t ci = static_cast<int64_t>(p) * a.half + i;
    cn = a.cos_c[ci];
    sn = a.sin_c[ci];
  }
  return make_float2(a.mu * cn, a.mu * sn);
}

__device__ inline void table_fill(float2* cs, const TabIn& in, int64_t t0, int ntok,
                                  const RopeArgs& a, const int32_t* __restrict__ pos,
                                  const float* __restrict__ inv_freq) {
  const uint32_t n = static_cast<uint32_t>(ntok) * a.half;
  if (a.cached) {
    // The cache loads depend on the positions, so they are issued here,
    // after the row loads; the table is a copy, no trigonometry.
#pragma unroll
    for (int k = 0; k < kTabPre; ++k) {
      const uint32_t idx = threadIdx.x + k * kBlock;
      if (idx < n) cs[idx] = cached_cs(in.p[k], idx - fdiv(idx, a.fd_half) * a.half, a);
    }
    for (uint32_t idx = threadIdx.x + kTabPre * kBlock; idx < n; idx += kBlock) {
      const uint32_t tl = fdiv(idx, a.fd_half);
      cs[idx] = cached_cs(pos[t0 + tl], idx - tl * a.half, a);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < kTabPre; ++k) {
    const uint32_t idx = threadIdx.x + k * kBlock;
    if (idx < n) {
      float sn, cn;
      sincos_angle(rope_angle(in.p[k], in.w[k]), &sn, &cn);
      cs[idx] = make_float2(a.mu * cn, a.mu * sn);
    }
  }
  for (uint32_t idx = threadIdx.x + kTabPre * kBlock; idx < n; idx += kBlock) {
    const uint32_t tl = fdiv(idx, a.fd_half);
    float sn, cn;
    sincos_angle(rope_angle(pos[t0 + tl], inv_freq[idx - tl * a.half]), &sn, &cn);
    cs[idx] = make_float2(a.mu * cn, a.mu * sn);
  }
}

// Element offsets (within a head row) of the two halves of slot kk.
// Scalar slots (PS == 1) are one pair.  Vector slots are the 16-byte vectors
// at kk*V and kk*V + r/2 in both layouts, so each load instruction of a wave
// covers whole contiguous lines: half-layout pairs are (A[e], B[e]);
// interleaved pairs sit inside each vector.
template <int PS>
__device__ inline void slot_offsets(int kk, const RopeArgs& a, int* ea, int* eb) {
  if constexpr (PS == 1) {
    if (a.layout == ET_ROPE_HALF) {
      *ea = kk;
      *eb = kk + a.half;
    } else {
      *ea = 2 * kk;
      *eb = 2 * kk + 1;
    }
  } else {
    *ea = kk * PS;
    *eb = kk * PS + a.half;
  }
}

// Rotate one pair with the pre-scaled (mu cos, mu sin).  Each member is
// formed the same way, fma(own, mu cos, partner * (-+ mu sin)), so a kernel
// that holds only one member of a pair per lane (multi-axis RoPE) gives the
// same bits as one that holds both.
__device__ inline void rotate(float& x0, float& x1, float2 c) {
  const float a = x0, b = x1;
  x0 = __builtin_fmaf(a, c.x, b * -c.y);
  x1 = __builtin_fmaf(b, c.x, a * c.y);
}

// ------------------------------------------------------------------ RoPE

// Slot u of thread tid in a block whose slots start at base: each wave owns
// a contiguous run of 64 * U slots (slot u of lane l at u * 64 + l in it).
template <int U>
__device__ inline uint32_t rope_slot(uint32_t base, int tid, int u) {
  return base + static_cast<uint32_t>((tid / 64) * (64 * U) + u * 64 + (tid % 64));
}

// Vector stores of one workgroup go through two buffer resources, one based
// at the first q row and one at the first k row the workgroup touches.  Its
// head rows (token-major: t * (Hq + Hk) + h) are consecutive, and so are the
// q rows (t * Hq + h) and the k rows (t * Hk + h - Hq) among them, so every
// offset is below (head rows per workgroup) * D elements; the host keeps that
// below 2^31 bytes.
template <typename S>
struct QkOut {
  __amdgpu_buffer_rsrc_t rq, rk;
  int64_t qrow0, krow0;
  // t0, hh0: token and head of the workgroup's first head row; T: tokens in
  // the launch.
  __device__ QkOut(S* q, S* k, int64_t t0, int hh0, const RopeArgs& a) {
    const bool in_q = hh0 < a.hq;
    qrow0 = t0 * a.hq + (in_q ? hh0 : a.hq);
    krow0 = t0 * a.hk + (in_q ? 0 : hh0 - a.hq);
    constexpr int64_t es = sizeof(S);
    rq = out_rsrc(q + qrow0 * a.D, (a.T * a.hq - qrow0) * a.D * es);
    rk = out_rsrc(a.hk > 0 ? k + krow0 * a.D : q, a.hk > 0 ? (a.T * a.hk - krow0) * a.D * es : 0);
  }
  // Address of head row (t, hh) of the launch (a query row for hh < hq, else
  // a key row), and in *rel its element offset from this workgroup's
  // resource base.  A launch holds fewer than 2^31 head rows, so the row
  // index is a 32-bit value and the address one 32 x 32 + 64-bit
  // multiply-add; the offset is below 2^31 bytes, a 32-bit product.
  __device__ S* row(S* q, S* k, uint32_t t, int hh, const RopeArgs& a, int* rel_out) const {
    const bool isq = hh < a.hq;
    const uint32_t ri = isq ? t * static_cast<uint32_t>(a.hq) + static_cast<uint32_t>(hh)
                            : t * static_cast<uint32_t>(a.hk) + static_cast<uint32_t>(hh - a.hq);
    *rel_out = static_cast<int>((ri - static_cast<uint32_t>(isq ? qrow0 : krow0)) *
                                static_cast<uint32_t>(a.D));
    return reinterpret_cast<S*>(reinterpret_cast<char*>(isq ? q : k) +
                                static_cast<uint64_t>(ri) * static_cast<uint32_t>(a.D * sizeof(S)));
  }
  // Store v at element `elem` of the q or k rows (relative to this
  // workgroup's resource base); p is the same element's address.  A buffer
  // store needs its resource in scalar registers: a resource chosen per lane
  // makes the compiler wrap every store in a loop over the distinct values.
  // The rows of one store instruction are nearly always all query or all
  // key heads, so when the wave's active lanes agree the resource is chosen
  // for the whole wave (a uniform select); a wave that straddles the two
  // stores through p with a plain non-temporal store instead, which the
  // compiler cannot merge back into the buffer store.
  __device__ void store(bool isq, int elem, S* p, const u32x4& v) const {
    const int off = elem * static_cast<int>(sizeof(S));
    const unsigned long long lanes = __ballot(1), qlanes = __ballot(isq);
    if (qlanes == lanes) {
      st16_buf(rq, off, v);
    } else if (qlanes == 0) {
      st16_buf(rk, off, v);
    } else {
      st16(p, 0, v);
    }
  }
};

template <typename S, int PS, int U>
__global__ __launch_bounds__(kBlock) void rope_qk_kernel(S* q, S* k, const int32_t* __restrict__ pos,
                                                        const float* __restrict__ inv_freq,
                                                        RopeArgs a) {
  using E = Elem<S>;
  extern __shared__ float2 cs[];
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(kBlock * U);
  const uint32_t t0 = fdiv(base, a.fd_spt);
  uint32_t last = base + kBlock * U - 1;
  if (last >= a.total) last = a.total - 1;
  const int ntok = static_cast<int>(fdiv(last, a.fd_spt) - t0 + 1);
  const TabIn tin = table_inputs(t0, ntok, a, pos, inv_freq);
  const QkOut<S> out(q, k, t0, static_cast<int>(fdiv(base - t0 * a.spt, a.fd_sph)), a);

  // Phase 1: issue every load of this thread.
  S* rowp[U];
  int ea[U], eb[U], tl[U], kk[U], rel[U];
  bool isq[U];
  u32x4 va[U], vb[U];
  float sa[U], sb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t s = rope_slot<U>(base, threadIdx.x, u);
    if (s >= a.total) s = a.total - 1;  // clamped: loaded, never stored
    const uint32_t t = fdiv(s, a.fd_spt);
    const uint32_t rem = s - t * a.spt;
    const uint32_t hh = fdiv(rem, a.fd_sph);
    kk[u] = static_cast<int>(rem - hh * a.sph);
    tl[u] = static_cast<int>(t - t0);
    isq[u] = static_cast<int>(hh) < a.hq;
    rowp[u] = out.row(q, k, t, static_cast<int>(hh), a, &rel[u]);
    slot_offsets<PS>(kk[u], a, &ea[u], &eb[u]);
    if constexpr (PS == 1) {
      sa[u] = E::ld(rowp[u], ea[u]);
      sb[u] = E::ld(rowp[u], eb[u]);
    } else {
      va[u] = ld16(rowp[u], ea[u]);
      vb[u] = ld16(rowp[u], eb[u]);
    }
  }

  // Nothing below may be scheduled above this point: the table inputs must
  // not be consumed before every row load has been issued.
  __builtin_amdgcn_sched_barrier(0);

  // Phase 2: the angle table of this block's tokens.
  table_fill(cs, tin, t0, ntok, a, pos, inv_freq);
  __syncthreads();

  // Phase 3: rotate and store.
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t s = rope_slot<U>(base, threadIdx.x, u);
    if (s >= a.total) continue;
    const float2* tab = cs + tl[u] * a.half;  // this token's (mu cos, mu sin)
    if constexpr (PS == 1) {
      float x0 = sa[u], x1 = sb[u];
      rotate(x0, x1, tab[kk[u]]);
      E::st(rowp[u], ea[u], x0);
      E::st(rowp[u], eb[u], x1);
    } else {
      constexpr int V = E::V;
      float xa[V], xb[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xa[e] = E::get(va[u], e);
        xb[e] = E::get(vb[u], e);
      }
      if (a.layout == ET_ROPE_HALF) {
#pragma unroll
        for (int e = 0; e < V; ++e) rotate(xa[e], xb[e], tab[ea[u] + e]);
      } else {
        // element j of the head pairs as pair j / 2
#pragma unroll
        for (int e = 0; e < V; e += 2) {
          rotate(xa[e], xa[e + 1], tab[ea[u] / 2 + e / 2]);
          rotate(xb[e], xb[e + 1], tab[eb[u] / 2 + e / 2]);
        }
      }
      out.store(isq[u], rel[u] + ea[u], rowp[u] + ea[u], E::pack(xa));
      out.store(isq[u], rel[u] + eb[u], rowp[u] + eb[u], E::pack(xb));
    }
  }
}

// --------------------------------------------------------- RMSNorm + RoPE

struct QkNormArgs {
  RopeArgs rope;      // fd_spt unused here
  float eps;
  float inv_d;        // 1/D when D is a power of two (exact), else 0
  uint32_t rows;      // head rows in the call (T * (Hq + Hk))
  FastDiv fd_heads;   // divide by Hq + Hk
  int rsl;            // rotated slots per head row (r / (2V))
};

// 1/sqrt(ss/D + eps) of a head row's sum of squares.  The mean square is a
// multiplication by 1/D when D is a power of two (the same correctly rounded
// value as the division).  In the normal range the inverse root is the
// hardware estimate (within 1 ulp) refined by one Newton step,
// y (1.5 - 0.5 m y^2) with fused multiply-adds, which leaves it within about
// 1 ulp like the correctly rounded root and division it replaces, at a
// fraction of their instructions.  Zero, subnormal, huge, infinite and NaN
// arguments take the IEEE root and division, so those keep their exact
// results (1/0 = inf, 1/inf = 0, NaN).
__device__ inline float inv_rms(float ss, const QkNormArgs& a) {
  const float m = (a.inv_d > 0.0f ? ss * a.inv_d : ss / static_cast<float>(a.rope.D)) + a.eps;
  if (__builtin_expect(m >= 0x1p-126f && m <= 0x1p+126f, 1)) {
    const float y = __builtin_amdgcn_rsqf(m);
    return __builtin_fmaf(y, __builtin_fmaf(-0.5f * m * y, y, 0.5f), y);
  }
  return 1.0f / sqrtf(m);
}

// Vector path: G lanes per head row, each owns two 16-byte vectors A and B.
// Interleaved layout: A = vector kk, B = vector kk + G (element D/2 + kk*V),
// so each load instruction covers a contiguous half of the head rows; a
// vector rotates (pairs inside it) if it lies below r.  Half layout: lanes
// kk < rsl own the partners A = kk*V, B = kk*V + r/2; the other lanes own
// tail vectors r + m*V and r + (nt + m)*V (m = kk - rsl, nt = G - rsl).
template <typename S, int G, int U, bool ROT>
__global__ __launch_bounds__(kBlock) void rmsnorm_rope_kernel(S* q, const S* __restrict__ gq, S* k,
                                                             const S* __restrict__ gk,
                                                             const int32_t* __restrict__ pos,
                                                             const float* __restrict__ inv_freq,
                                                             QkNormArgs a) {
  using E = Elem<S>;
  constexpr int V = E::V;
  constexpr int kRowsPerPass = kBlock / G;
  extern __shared__ float2 cs[];
  const RopeArgs& ra = a.rope;
  const int heads = ra.hq + ra.hk;
  const int kk = threadIdx.x % G;
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(kRowsPerPass * U);
  // Head row of slot u of this lane group: each wave owns a contiguous run
  // of (64 / G) * U head rows (one row per lane group for G == 64).
  auto head_row = [&](int u) -> uint32_t {
    if constexpr (G < 64) {
      constexpr int kRowsPerWave = 64 / G;
      const int wave = threadIdx.x / 64;
      return base + static_cast<uint32_t>(wave * kRowsPerWave * U + u * kRowsPerWave +
                                          (threadIdx.x % 64) / G);
    } else {
      return base + static_cast<uint32_t>(u * kRowsPerPass + threadIdx.x / G);
    }
  };
  const uint32_t t0 = fdiv(base, a.fd_heads);
  uint32_t last = base + kRowsPerPass * U - 1;
  if (last >= a.rows) last = a.rows - 1;
  const int ntok = static_cast<int>(fdiv(last, a.fd_heads) - t0 + 1);
  TabIn tin{};
  if constexpr (ROT) tin = table_inputs(t0, ntok, ra, pos, inv_freq);

  int ea, eb;
  bool a_rot, b_rot;
  if (ra.layout == ET_ROPE_INTERLEAVED) {
    ea = kk * V;
    eb = ra.D / 2 + kk * V;
    a_rot = ea < ra.r;
    b_rot = eb < ra.r;
  } else if (kk < a.rsl) {
    ea = kk * V;
    eb = kk * V + ra.half;
    a_rot = b_rot = true;
  } else {
    const int m = kk - a.rsl;
    ea = ra.r + m * V;
    eb = ra.r + (G - a.rsl + m) * V;
    a_rot = b_rot = false;
  }

  const QkOut<S> out(q, k, t0, static_cast<int>(base - t0 * heads), ra);
  // The two gains (2G vectors each) go through LDS, widened to f32 once per
  // workgroup: thread t < 4G fetches vector t % 2G of gq (t < 2G) or gk,
  // before the row loads so that its LDS write waits for nothing else.  (gk
  // is gq when there are no key heads: the host passes it so.)
  __shared__ float gsh[4 * G * V];
  const int gi = threadIdx.x < 4 * G ? static_cast<int>(threadIdx.x) : 4 * G - 1;
  const u32x4 gv = ld16_keep(gi < 2 * G ? gq : gk, (gi % (2 * G)) * V);
  S* rowp[U];
  int tl[U], rel[U];
  bool isq[U];
  u32x4 va[U], vb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t hr = head_row(u);
    if (hr >= a.rows) hr = a.rows - 1;  // clamped: loaded, never stored
    const uint32_t t = fdiv(hr, a.fd_heads);
    const int hh = static_cast<int>(hr - t * heads);
    tl[u] = static_cast<int>(t - t0);
    isq[u] = hh < ra.hq;
    rowp[u] = out.row(q, k, t, hh, ra, &rel[u]);
    va[u] = ld16(rowp[u], ea);
    vb[u] = ld16(rowp[u], eb);
  }
  __builtin_amdgcn_sched_barrier(0);  // table inputs are used only below

  if (threadIdx.x < 4 * G) {
#pragma unroll
    for (int e = 0; e < V; ++e) gsh[threadIdx.x * V + e] = E::get(gv, e);
  }
  if constexpr (ROT) table_fill(cs, tin, t0, ntok, ra, pos, inv_freq);

  // Sums of squares of all U rows first, so their butterflies interleave.
  float inv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float x = E::get(va[u], e);
      ss = __builtin_fmaf(x, x, ss);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float x = E::get(vb[u], e);
      ss = __builtin_fmaf(x, x, ss);
    }
    inv[u] = ss;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) inv[u] = group_sum<G>(inv[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) inv[u] = inv_rms(inv[u], a);
  // The barrier after the norm statistics: a wave whose rows arrived early
  // finishes them while the workgroup's table and gains are completed.
  __syncthreads();

#pragma unroll
  for (int u = 0; u < U; ++u) {
    float xa[V], xb[V];
    const float* ga = gsh + ((isq[u] ? 0 : 2 * G) + ea / V) * V;
    const float* gb = gsh + ((isq[u] ? 0 : 2 * G) + eb / V) * V;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      xa[e] = E::get(va[u], e) * inv[u] * ga[e];
      xb[e] = E::get(vb[u], e) * inv[u] * gb[e];
    }
    const float2* tab = cs + tl[u] * ra.half;  // this token's (mu cos, mu sin)
    if (!ROT) {
    } else if (ra.layout == ET_ROPE_HALF) {
      if (a_rot) {
#pragma unroll
        for (int e = 0; e < V; ++e) rotate(xa[e], xb[e], tab[ea + e]);
      }
    } else {
      if (a_rot) {
#pragma unroll
        for (int e = 0; e < V; e += 2) rotate(xa[e], xa[e + 1], tab[ea / 2 + e / 2]);
      }
      if (b_rot) {
#pragma unroll
        for (int e = 0; e < V; e += 2) rotate(xb[e], xb[e + 1], tab[eb / 2 + e / 2]);
      }
    }
    if (head_row(u) < a.rows) {
      out.store(isq[u], rel[u] + ea, rowp[u] + ea, E::pack(xa));
      out.store(isq[u], rel[u] + eb, rowp[u] + eb, E::pack(xb));
    }
  }
}

// General path: one wave per head row.  Lane l owns pairs i = l, l+64, ...
// (i < r/2) and tail entries r + l, r + l + 64, ...; pass 1 sums their
// squares (pairs first, then tail, each in increasing order), pass 2 re-reads,
// normalises, rotates and writes.  A lane only touches what it owns.
template <typename S>
__global__ __launch_bounds__(kBlock) void rmsnorm_rope_wave_kernel(
    S* q, const S* __restrict__ gq, S* k, const S* __restrict__ gk,
    const int32_t* __restrict__ pos, const float* __restrict__ inv_freq, QkNormArgs a) {
  using E = Elem<S>;
  const RopeArgs& ra = a.rope;
  const int heads = ra.hq + ra.hk;
  const int lane = threadIdx.x % 64;
  const uint32_t hr = blockIdx.x * (kBlock / 64) + threadIdx.x / 64;
  if (hr >= a.rows) return;  // whole wave exits together; no block barrier below
  const uint32_t t = fdiv(hr, a.fd_heads);
  const int hh = static_cast<int>(hr - t * heads);
  const bool isq = hh < ra.hq;
  S* row = isq ? q + (static_cast<int64_t>(t) * ra.hq + hh) * ra.D
               : k + (static_cast<int64_t>(t) * ra.hk + (hh - ra.hq)) * ra.D;
  const S* g = isq ? gq : gk;

  float ss = 0.0f;
  for (int i = lane; i < ra.half; i += 64) {
    int ia, ib;
    slot_offsets<1>(i, ra, &ia, &ib);
    const float x0 = E::ld(row, ia), x1 = E::ld(row, ib);
    ss = __builtin_fmaf(x0, x0, ss);
    ss = __builtin_fmaf(x1, x1, ss);
  }
  for (int j = ra.r + lane; j < ra.D; j += 64) {
    const float x = E::ld(row, j);
    ss = __builtin_fmaf(x, x, ss);
  }
  ss = group_sum<64>(ss);
  const float inv = inv_rms(ss, a);
  const int32_t p = ra.half > 0 ? pos[t] : 0;  // pos may be NULL when nothing rotates
  for (int i = lane; i < ra.half; i += 64) {
    int ia, ib;
    slot_offsets<1>(i, ra, &ia, &ib);
    float x0 = E::ld(row, ia) * inv * E::ld(g, ia);
    float x1 = E::ld(row, ib) * inv * E::ld(g, ib);
    float sn, cn;
    sincos_angle(rope_angle(p, inv_freq[i]), &sn, &cn);
    rotate(x0, x1, make_float2(ra.mu * cn, ra.mu * sn));
    E::st(row, ia, x0);
    E::st(row, ib, x1);
  }
  for (int j = ra.r + lane; j < ra.D; j += 64) E::st(row, j, E::ld(row, j) * inv * E::ld(g, j));
}

// ---------------------------------------------------------------- host

template <typename S>
et_status check_rope(const S* q, int64_t hq, const S* k, int64_t hk, const int32_t* pos,
                     int64_t T, int64_t D, int64_t r, const float* inv_freq, float mu, int layout,
                     int64_t* qbytes, int64_t* kbytes, bool need_freq = true) {
  if (T < 0 || hq < 0 || hk < 0 || D < 0) return ET_ERR_BAD_SIZE;
  if (r < 0 || r > D || (r & 1)) return ET_ERR_BAD_ARG;
  if (layout != ET_ROPE_HALF && layout != ET_ROPE_INTERLEAVED) return ET_ERR_BAD_ARG;
  if (!__builtin_isfinite(mu)) return ET_ERR_BAD_ARG;
  int64_t qn = 0, kn = 0;
  if (!mul_ok(T, hq, &qn) || !mul_ok(qn, D, &qn) || !mul_ok(qn, int64_t(sizeof(S)), qbytes) ||
      !mul_ok(T, hk, &kn) || !mul_ok(kn, D, &kn) || !mul_ok(kn, int64_t(sizeof(S)), kbytes))
    return ET_ERR_BAD_SIZE;
  if (D > INT32_MAX / 2 || hq + hk > INT32_MAX / 2) return ET_ERR_BAD_SIZE;
  if ((*qbytes > 0 && !q) || (*kbytes > 0 && !k)) return ET_ERR_NULL_POINTER;
  if (T > 0 && (hq + hk) > 0 && r > 0 && (!pos || (need_freq && !inv_freq)))
    return ET_ERR_NULL_POINTER;
  if (!ranges_ok(q, *qbytes, k, *kbytes, false)) return ET_ERR_OVERLAP;
  const int64_t pbytes = T * int64_t(sizeof(int32_t)), fbytes = (r / 2) * int64_t(sizeof(float));
  if (!ranges_ok(q, *qbytes, pos, pbytes, false) || !ranges_ok(k, *kbytes, pos, pbytes, false) ||
      !ranges_ok(q, *qbytes, inv_freq, fbytes, false) ||
      !ranges_ok(k, *kbytes, inv_freq, fbytes, false))
    return ET_ERR_OVERLAP;
  return ET_OK;
}

RopeArgs make_args(int64_t T, int64_t hq, int64_t hk, int64_t D, int64_t r, float mu, int layout,
                   int ps) {
  RopeArgs a{};
  a.T = T;
  a.hq = static_cast<int>(hq);
  a.hk = static_cast<int>(hk);
  a.D = static_cast<int>(D);
  a.r = static_cast<int>(r);
  a.half = static_cast<int>(r / 2);
  a.layout = layout;
  a.mu = mu;
  a.sph = static_cast<uint32_t>(a.half / ps);
  a.spt = a.sph * static_cast<uint32_t>(hq + hk);
  a.fd_spt = make_fastdiv(a.spt > 0 ? a.spt : 1);
  a.fd_sph = make_fastdiv(a.sph > 0 ? a.sph : 1);
  a.fd_half = make_fastdiv(a.half > 0 ? a.half : 1);
  return a;
}

template <typename S, int PS, int U>
void launch_rope(S* q, S* k, const int32_t* pos, const float* inv_freq, RopeArgs a, int64_t T,
                 hipStream_t s) {
  // Tokens per launch keep slot indices below 2^31.
  const int64_t tok_per_launch = (int64_t{1} << 31) / a.spt;
  a.ntok_max = static_cast<int>((kBlock * U + a.spt - 1) / a.spt + 1);
  const size_t shmem = static_cast<size_t>(a.ntok_max) * a.half * sizeof(float2);
  for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
    const int64_t m = T - t0 < tok_per_launch ? T - t0 : tok_per_launch;
    a.T = m;
    a.total = static_cast<uint32_t>(m * a.spt);
    const unsigned grid = (a.total + kBlock * U - 1) / (kBlock * U);
    rope_qk_kernel<S, PS, U><<<grid, kBlock, shmem, s>>>(
        q + t0 * a.hq * a.D, a.hk ? k + t0 * a.hk * a.D : k, pos + t0, inv_freq, a);
  }
}

// Largest unroll (umax, umax / 2, ..., 1) whose angle table fits the LDS budget.
inline int pick_u(int64_t spt, int64_t half, int64_t per_u, int umax) {
  for (int u = umax; u >= 1; u >>= 1) {
    const int64_t ntok = (per_u * u + spt - 1) / spt + 1;
    if (ntok * half * int64_t(sizeof(float2)) <= kMaxTableBytes) return u;
  }
  return 0;
}

// A cos/sin cache of max_pos rows of r/2 f32 each, read instead of the
// frequencies.
struct RopeCache {
  const float* cos_c;
  const float* sin_c;
  int64_t max_pos;
};

template <typename S>
et_status rope_entry(S* q, int64_t hq, S* k, int64_t hk, const int32_t* pos, int64_t T, int64_t D,
                     int64_t r, const float* inv_freq, float mu, int layout, void* stream,
                     const RopeCache* cache = nullptr) {
  int64_t qb = 0, kb = 0;
  // With a cache the frequencies are not read; the cache is checked below.
  const et_status st = check_rope(q, hq, k, hk, pos, T, D, r, cache ? nullptr : inv_freq, mu,
                                  layout, &qb, &kb, !cache);
  if (st != ET_OK) return st;
  if (cache) {
    if (cache->max_pos < 0 || cache->max_pos > INT32_MAX) return ET_ERR_BAD_SIZE;
    int64_t cb = 0;
    if (!mul_ok(cache->max_pos, (r / 2) * int64_t(sizeof(float)), &cb)) return ET_ERR_BAD_SIZE;
    if (T > 0 && hq + hk > 0 && cb > 0 && (!cache->cos_c || !cache->sin_c))
      return ET_ERR_NULL_POINTER;
    if (!ranges_ok(q, qb, cache->cos_c, cb, false) || !ranges_ok(q, qb, cache->sin_c, cb, false) ||
        !ranges_ok(k, kb, cache->cos_c, cb, false) || !ranges_ok(k, kb, cache->sin_c, cb, false))
      return ET_ERR_OVERLAP;
  }
  if (T == 0 || hq + hk == 0 || r == 0) return ET_OK;
  constexpr int V = Elem<S>::V;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool vec = (r % (2 * V)) == 0 && (D % V) == 0 && aligned16(q) && (hk == 0 || aligned16(k));
  RopeArgs a = make_args(T, hq, hk, D, r, mu, layout, vec ? V : 1);
  if (a.spt > (1u << 30)) return ET_ERR_BAD_SIZE;
  const int u = pick_u(a.spt, a.half, kBlock, kRopeU);
  if (u == 0) return ET_ERR_BAD_SIZE;
  auto set_cache = [&](RopeArgs& ra) {
    if (!cache) return;
    ra.cached = 1;
    ra.cos_c = cache->cos_c;
    ra.sin_c = cache->sin_c;
    ra.max_pos = static_cast<int>(cache->max_pos);
  };
  set_cache(a);
  if (vec) {
    // The vector path stores at byte offsets below (head rows a workgroup
    // touches) * D * sizeof(S); past 2^31 take the scalar path.
    const int64_t rows_blk = (int64_t{kBlock} * u + a.sph - 1) / a.sph + 2;
    if (rows_blk * D * int64_t(sizeof(S)) >= (int64_t{1} << 31)) {
      vec = false;
      a = make_args(T, hq, hk, D, r, mu, layout, 1);
      set_cache(a);
      if (a.spt > (1u << 30)) return ET_ERR_BAD_SIZE;
      if (pick_u(a.spt, a.half, kBlock, kRopeU) == 0) return ET_ERR_BAD_SIZE;
    }
  }
  (void)hipGetLastError();
  if (vec)
    launch_rope<S, V, kRopeU>(q, k, pos, inv_freq, a, T, s);
  else
    launch_rope<S, 1, kRopeU>(q, k, pos, inv_freq, a, T, s);
  return launch_status();
}

template <typename S, int G, int U, bool ROT>
void launch_qknorm_vec(S* q, const S* gq, S* k, const S* gk, const int32_t* pos,
                       const float* inv_freq, QkNormArgs a, int64_t T, hipStream_t s) {
  constexpr int kRowsPerPass = kBlock / G;
  const int64_t heads = a.rope.hq + a.rope.hk;
  const int64_t tok_per_launch = (int64_t{1} << 31) / heads;
  const int64_t rows_per_block = int64_t{kRowsPerPass} * U;
  const int ntok_max = static_cast<int>((rows_per_block + heads - 1) / heads + 1);
  const size_t shmem = static_cast<size_t>(ntok_max) * a.rope.half * sizeof(float2);
  for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
    const int64_t m = T - t0 < tok_per_launch ? T - t0 : tok_per_launch;
    a.rows = static_cast<uint32_t>(m * heads);
    a.rope.T = m;
    const unsigned grid = static_cast<unsigned>((a.rows + rows_per_block - 1) / rows_per_block);
    rmsnorm_rope_kernel<S, G, U, ROT><<<grid, kBlock, shmem, s>>>(
        q + t0 * a.rope.hq * a.rope.D, gq, a.rope.hk ? k + t0 * a.rope.hk * a.rope.D : k, gk,
        pos + t0, inv_freq, a);
  }
}

template <typename S, int G>
void launch_qknorm_vec_rot(S* q, const S* gq, S* k, const S* gk, const int32_t* pos,
                           const float* inv_freq, QkNormArgs a, int64_t T, hipStream_t s) {
  if (a.rope.half > 0)
    launch_qknorm_vec<S, G, kQkU, true>(q, gq, k, gk, pos, inv_freq, a, T, s);
  else
    launch_qknorm_vec<S, G, kQkU, false>(q, gq, k, gk, pos, inv_freq, a, T, s);
}

template <typename S>
et_status qknorm_entry(S* q, const S* gq, int64_t hq, S* k, const S* gk, int64_t hk, float eps,
                       const int32_t* pos, int64_t T, int64_t D, int64_t r, const float* inv_freq,
                       float mu, int layout, void* stream) {
  int64_t qb = 0, kb = 0;
  et_status st = check_rope(q, hq, k, hk, pos, T, D, r, inv_freq, mu, layout, &qb, &kb);
  if (st != ET_OK) return st;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return ET_ERR_BAD_ARG;
  if (T == 0 || hq + hk == 0) return ET_OK;
  if (D == 0) return ET_ERR_BAD_SIZE;
  if ((hq > 0 && !gq) || (hk > 0 && !gk)) return ET_ERR_NULL_POINTER;
  const int64_t gbytes = D * int64_t(sizeof(S));
  if (!ranges_ok(q, qb, gq, gbytes, false) || !ranges_ok(q, qb, gk, gbytes, false) ||
      !ranges_ok(k, kb, gq, gbytes, false) || !ranges_ok(k, kb, gk, gbytes, false))
    return ET_ERR_OVERLAP;
  int64_t rows = 0;
  if (!mul_ok(T, hq + hk, &rows)) return ET_ERR_BAD_SIZE;
  constexpr int V = Elem<S>::V;
  hipStream_t s = static_cast<hipStream_t>(stream);
  QkNormArgs a{};
  a.eps = eps;
  a.inv_d = (D & (D - 1)) == 0 ? 1.0f / static_cast<float>(D) : 0.0f;
  const int64_t heads = hq + hk;
  a.fd_heads = make_fastdiv(static_cast<uint32_t>(heads));
  const int64_t g = D / (2 * V);
  const bool pow2 = g >= 1 && g <= 64 && (g & (g - 1)) == 0;
  const bool vec = pow2 && (D % (2 * V)) == 0 && (r % (2 * V)) == 0 && aligned16(q) &&
                   aligned16(gq) && (hk == 0 || (aligned16(k) && aligned16(gk)));
  (void)hipGetLastError();
  if (vec) {
    a.rope = make_args(T, hq, hk, D, r, mu, layout, V);
    a.rsl = static_cast<int>(r / (2 * V));
    if (pick_u(heads, a.rope.half, kBlock / g, kQkU) == 0) return ET_ERR_BAD_SIZE;
    const S* gkk = hk > 0 ? gk : gq;
    switch (g) {
      case 1: launch_qknorm_vec_rot<S, 1>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      case 2: launch_qknorm_vec_rot<S, 2>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      case 4: launch_qknorm_vec_rot<S, 4>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      case 8: launch_qknorm_vec_rot<S, 8>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      case 16: launch_qknorm_vec_rot<S, 16>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      case 32: launch_qknorm_vec_rot<S, 32>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
      default: launch_qknorm_vec_rot<S, 64>(q, gq, k, gkk, pos, inv_freq, a, T, s); break;
    }
  } else {
    a.rope = make_args(T, hq, hk, D, r, mu, layout, 1);
    const int64_t tok_per_launch = (int64_t{1} << 31) / heads;
    for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
      const int64_t m = T - t0 < tok_per_launch ? T - t0 : tok_per_launch;
      a.rows = static_cast<uint32_t>(m * heads);
      const unsigned grid = (a.rows + kBlock / 64 - 1) / (kBlock / 64);
      rmsnorm_rope_wave_kernel<S><<<grid, kBlock, 0, s>>>(
          q + t0 * hq * D, gq, hk ? k + t0 * hk * D : k, gk, pos + t0, inv_freq, a);
    }
  }
  return launch_status();
}

// cos_c / sin_c[p * half + i] of the angle rope_angle(p, inv_freq[i]), with
// the same sin/cos the computed tables use, so a cached rotation equals the
// computed one bit for bit.
__global__ __launch_bounds__(kBlock) void rope_cache_kernel(const float* __restrict__ inv_freq,
                                                            int64_t total, FastDiv fd_half,
                                                            int half, float* cos_c, float* sin_c) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const uint32_t p = fdiv(static_cast<uint32_t>(idx), fd_half);
  const uint32_t i = static_cast<uint32_t>(idx) - p * static_cast<uint32_t>(half);
  float sn, cn;
  sincos_angle(rope_angle(static_cast<int32_t>(p), inv_freq[i]), &sn, &cn);
  cos_c[idx] = cn;
  sin_c[idx] = sn;
}

et_status rope_cache_entry(const float* inv_freq, int64_t max_pos, int64_t r, float* cos_c,
                           float* sin_c, void* stream) {
  if (max_pos < 0 || r < 0) return ET_ERR_BAD_SIZE;
  if (r & 1) return ET_ERR_BAD_ARG;
  const int64_t half = r / 2;
  int64_t total = 0, bytes = 0;
  if (!mul_ok(max_pos, half, &total) || !mul_ok(total, int64_t(sizeof(float)), &bytes))
    return ET_ERR_BAD_SIZE;
  if (total == 0) return ET_OK;
  if (total > UINT32_MAX || max_pos > INT32_MAX) return ET_ERR_BAD_SIZE;
  if (!inv_freq || !cos_c || !sin_c) return ET_ERR_NULL_POINTER;
  const int64_t fb = half * int64_t(sizeof(float));
  if (!ranges_ok(cos_c, bytes, sin_c, bytes, false) || !ranges_ok(cos_c, bytes, inv_freq, fb, false) ||
      !ranges_ok(sin_c, bytes, inv_freq, fb, false))
    return ET_ERR_OVERLAP;
  (void)hipGetLastError();
  const int64_t grid = (total + kBlock - 1) / kBlock;
  rope_cache_kernel<<<static_cast<unsigned>(grid), kBlock, 0, static_cast<hipStream_t>(stream)>>>(
      inv_freq, total, make_fastdiv(static_cast<uint32_t>(half)), static_cast<int>(half), cos_c,
      sin_c);
  return launch_status();
}


// --------------------------------------------------------- multi-axis RoPE
//
// "Operations" 3 Rope, multi-axis RoPE: the first `span` entries of a head
// are cut into consecutive sub-ranges, one per axis of the token's position
// vector, and each is rotated as a whole head of its own width, with its own
// position and frequencies.  A sub-range's pairs may sit anywhere relative
// to the 16-byte vectors (half widths need not be multiples of V), so a
// workgroup stages its head rows in LDS and every element of the half
// pairing reads its partner from there (interleaved partners sit in the same
// vector):
//   * a workgroup owns rpb consecutive head rows (token-major: a token's q
//     heads, then its k heads), loads their first span entries once, 16
//     bytes at a time (scalars on the scalar path), and copies them to LDS;
//   * a descriptor per vector of a row: its elements form at most two runs
//     (split where an axis or, for the half pairing, a half begins), and in a
//     run the partner column and the pair index advance with the element,
//     so a run is its first element's partner and pair, and its member flag;
//   * an angle table holds (mu cos, mu sin) per (token, pair), built as the
//     RoPE kernel builds its own.
// Each element is then rotated exactly as the RoPE kernel rotates it, so a
// single axis of width r gives that kernel's bits.  In place: a workgroup
// reads all of its rows before the barrier and writes after it, each
// element by the thread that loaded it.  The host takes the scalar path when
// some vector would hold more than two runs (axes narrower than a vector).
// When the row's vectors fill whole lane groups and every 32-bit word's
// partners are one word of another lane (perm_fits), a separate instance
// takes the partners across lanes instead of from an LDS copy of the rows.

constexpr int kMaxAxes = 8;
constexpr int kMultiU = 4;
constexpr int kMultiMaxSpan = 1024;

struct MultiArgs {
  RopeArgs ra;              // T, hq, hk, D, layout and mu, as for the RoPE kernel
  int A;                    // axes
  int span;                 // rotated entries per head row (sum of the widths)
  int np;                   // pairs per head row (span / 2)
  int off[kMaxAxes + 1];    // first entry of axis a; off[A] = span
  int foff[kMaxAxes + 1];   // first pair (frequency) of axis a
  uint32_t rows;            // head rows in this launch
  int rpb;                  // head rows per workgroup
  int nv;                   // vectors (or scalars) per head row: span / PS
  int ntok_max;             // tokens one workgroup can touch
  int heads;                // hq + hk
  int perm;                 // half pairing with partners read across lanes (perm_fits)
  FastDiv fd_heads, fd_nv, fd_np;
  uint32_t d4_off, d1_off, xs_off;  // LDS byte offsets of the descriptors and the rows
};

// The axis a pair index i belongs to (zero-width axes are skipped: a later
// axis with the same start wins).
__device__ inline int axis_of_pair(int i, const MultiArgs& a) {
  int ax = 0;
#pragma unroll
  for (int b = 1; b < kMaxAxes; ++b)
    if (b < a.A && i >= a.foff[b]) ax = b;
  return ax;
}

// Partner column, pair index and first-member flag of column c; *next is the
// first column after c where the axis or (half pairing) the half changes.
__device__ inline void column_of(int c, const MultiArgs& a, int* partner, int* pair, bool* first,
                                 int* next) {
  int o = 0, w = a.off[1], h = 0;
#pragma unroll
  for (int b = 1; b < kMaxAxes; ++b) {
    if (b < a.A && c >= a.off[b]) {
      o = a.off[b];
      w = a.off[b + 1] - a.off[b];
      h = a.foff[b];
    }
  }
  const int l = c - o;
  if (a.ra.layout == ET_ROPE_HALF) {
    const int hd = w / 2;
    *first = l < hd;
    *pair = h + (*first ? l : l - hd);
    *partner = *first ? c + hd : c - hd;
    *next = *first ? o + hd : o + w;
  } else {
    *first = (l & 1) == 0;  // sub-ranges start at even entries
    *pair = h + (l >> 1);
    *partner = c ^ 1;
    *next = o + w;
  }
}

// Descriptor of vector cv (elements cv*PS .. cv*PS + PS-1): runs A = [0, k)
// and B = [k, PS); element e of run X has partner column pX + e and pair
// iX + e (half pairing) or iX + e/2 (interleaved).  d1 = k | fA << 8 | fB << 9.
template <int PS>
__device__ inline void vector_desc(int cv, const MultiArgs& a, int4* d4, int* d1) {
  const int c0 = cv * PS;
  int pa, ia, nx, pb, ib, nx2;
  bool fa, fb;
  column_of(c0, a, &pa, &ia, &fa, &nx);
  int k = nx - c0;
  if (k >= PS) k = PS;
  if (k < PS) {
    column_of(c0 + k, a, &pb, &ib, &fb, &nx2);
  } else {
    pb = pa + k;
    ib = ia + (a.ra.layout == ET_ROPE_HALF ? k : k / 2);
    fb = fa;
  }
  const bool half = a.ra.layout == ET_ROPE_HALF;
  *d4 = make_int4(pa, pb - k, ia, half ? ib - k : ib - k / 2);
  *d1 = k | (fa ? 0x100 : 0) | (fb ? 0x200 : 0);
}

template <typename S>
__device__ inline float lds_elem(const S* xs, int i) {
  if constexpr (sizeof(S) == 2) {
    return Elem<S>::lo(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(xs)[i]));
  } else {
    return xs[i];
  }
}

// W consecutive entries of a staged row from column p (p a multiple of W).
template <typename S, int W>
__device__ inline void lds_run(const S* xr, int p, float (&o)[W]) {
  if constexpr (W == 1) {
    o[0] = lds_elem(xr, p);
  } else if constexpr (sizeof(S) == 2) {
    if constexpr (W == 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(xr) + p);
      using E = Elem<S>;
      o[0] = E::lo(w.x); o[1] = E::hi(w.x); o[2] = E::lo(w.y); o[3] = E::hi(w.y);
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(xr) + p);
      o[0] = Elem<S>::lo(w); o[1] = Elem<S>::hi(w);
    }
  } else {
    if constexpr (W == 4) {
      const float4 w = *reinterpret_cast<const float4*>(xr + p);
      o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
    } else {
      const float2 w = *reinterpret_cast<const float2*>(xr + p);
      o[0] = w.x; o[1] = w.y;
    }
  }
}

// The angles of the PS entries of a vector with descriptor (d, d1), from the
// token's row tab of the angle table: entry e's (mu cos, +-mu sin), the sine
// negated for the first member of its pair, so that every entry rotates as
// y = x mu cos + x_partner (+-mu sin), the form of the RoPE kernel's rotate()
// (negation is exact: the bits are those of applying the sign afterwards).
template <int PS>
__device__ inline void entry_angles(const float2* tab, int4 d, int d1, bool half,
                                    float2 (&ang)[PS]) {
  const int kr = d1 & 0xFF;
#pragma unroll
  for (int e = 0; e < PS; ++e) {
    const bool in_a = e < kr;
    const float2 c = tab[(in_a ? d.z : d.w) + (half ? e : e / 2)];
    // a vector of PS > 1 starts at an even column, so for the interleaved
    // pairing the parity of e is the column's; a single entry (the scalar
    // path) takes its run's flag, as the half pairing does
    const bool first = (half || PS == 1) ? (d1 & (in_a ? 0x100 : 0x200)) != 0 : (e & 1) == 0;
    ang[e] = make_float2(c.x, first ? -c.y : c.y);
  }
}

// Half pairing (or the scalar path): element e of the vector belongs to run
// A (e < kr) or B; its partner is read from the staged row W entries at a
// time (the W entries share a run: kr is a multiple of W).
template <typename S, int PS, int W>
__device__ inline void rotate_runs(const S* xr, const float (&x)[PS], float (&y)[PS], int4 d, int kr,
                                   const float2 (&ang)[PS]) {
#pragma unroll
  for (int e0 = 0; e0 < PS; e0 += W) {
    float xp[W];
    lds_run<S, W>(xr, (e0 < kr ? d.x : d.y) + e0, xp);
#pragma unroll
    for (int j = 0; j < W; ++j)
      y[e0 + j] = __builtin_fmaf(x[e0 + j], ang[e0 + j].x, xp[j] * ang[e0 + j].y);
  }
}

// The PS partners of a vector whose two runs start their partner columns,
// and split, at multiples of 4, read 4 entries (8 or 16 bytes) at a time
// and kept packed: 2-byte storage two entries per word, f32 one.
template <typename S, int PS>
struct Partners {
  uint32_t w[PS * sizeof(S) / 4];
};

template <typename S, int PS>
__device__ inline void read_partners4(const S* xr, int4 d, int kr, Partners<S, PS>& r) {
#pragma unroll
  for (int e0 = 0; e0 < PS; e0 += 4) {
    const int p = (e0 < kr ? d.x : d.y) + e0;
    if constexpr (sizeof(S) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(xr) + p);
      r.w[e0 / 2] = w.x;
      r.w[e0 / 2 + 1] = w.y;
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(xr + p);
      r.w[e0] = w.x; r.w[e0 + 1] = w.y; r.w[e0 + 2] = w.z; r.w[e0 + 3] = w.w;
    }
  }
}

template <typename S, int PS>
__device__ inline float partner_of(const Partners<S, PS>& r, int e) {
  if constexpr (sizeof(S) == 2) {
    return (e & 1) ? Elem<S>::hi(r.w[e / 2]) : Elem<S>::lo(r.w[e / 2]);
  } else {
    return __uint_as_float(r.w[e]);
  }
}

template <typename S, int PS, int U, bool PERM>
__global__ __launch_bounds__(kBlock) void rope_multi_kernel(S* q, S* k,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ inv_freq,
                                                           MultiArgs a) {
  using E = Elem<S>;
  extern __shared__ __align__(16) unsigned char smem[];
  float2* cs = reinterpret_cast<float2*>(smem);
  int4* d4s = reinterpret_cast<int4*>(smem + a.d4_off);
  int* d1s = reinterpret_cast<int*>(smem + a.d1_off);
  S* xs = reinterpret_cast<S*>(smem + a.xs_off);

  const uint32_t row0 = blockIdx.x * static_cast<uint32_t>(a.rpb);
  uint32_t row_end = row0 + a.rpb;
  if (row_end > a.rows) row_end = a.rows;
  const uint32_t t0 = fdiv(row0, a.fd_heads);
  const int ntok = static_cast<int>(fdiv(row_end - 1, a.fd_heads) - t0 + 1);
  const int nslot = static_cast<int>(row_end - row0) * a.nv;
  const int ntab = ntok * a.np;

  // Phase 0: positions and frequencies of this thread's first angle-table
  // entries, fetched before the row loads (loads complete in issue order).
  int32_t tp[kTabPre];
  float tw[kTabPre];
#pragma unroll
  for (int kk = 0; kk < kTabPre; ++kk) {
    int idx = threadIdx.x + kk * kBlock;
    if (idx >= ntab) idx = ntab - 1;  // clamped: loaded, never used
    const int tl = static_cast<int>(fdiv(static_cast<uint32_t>(idx), a.fd_np));
    const int i = idx - tl * a.np;
    tp[kk] = pos[static_cast<int64_t>(t0 + tl) * a.A + axis_of_pair(i, a)];
    tw[kk] = inv_freq[i];
  }

  // Phase 1: every row load of this thread.
  const QkOut<S> out(q, k, t0, static_cast<int>(row0 - t0 * a.heads), a.ra);
  int sl[U], cv[U], tl[U], rel[U];
  bool isq[U];
  S* rowp[U];
  u32x4 v[U];
  float sv[U];
  // Cross-lane instance: nv divides 64, so it is a power of two, a lane keeps
  // one column for all its slots, and slot u lies u * 64 / nv rows below
  // slot 0.  Rows past the workgroup's are clamped to its last row (loaded,
  // never stored; their lanes only feed each other's partner reads).
  const int lg_nv = PERM ? __builtin_ctz(static_cast<unsigned>(a.nv)) : 0;
  const int s0 = static_cast<int>(rope_slot<U>(0, threadIdx.x, 0));
  const int last_row = static_cast<int>(row_end - row0) - 1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int r;
    if constexpr (PERM) {
      r = (s0 >> lg_nv) + u * (64 >> lg_nv);
      if (r > last_row) r = last_row;
      cv[u] = s0 & (a.nv - 1);
    } else {
      int s = static_cast<int>(rope_slot<U>(0, threadIdx.x, u));
      if (s >= nslot) s = nslot - 1;  // clamped: loaded, never stored
      r = static_cast<int>(fdiv(static_cast<uint32_t>(s), a.fd_nv));
      cv[u] = s - r * a.nv;
    }
    sl[u] = r;
    const uint32_t g = row0 + r;
    const uint32_t t = fdiv(g, a.fd_heads);
    const int hh = static_cast<int>(g - t * a.heads);
    tl[u] = static_cast<int>(t - t0);
    isq[u] = hh < a.ra.hq;
    rowp[u] = out.row(q, k, t, hh, a.ra, &rel[u]);
    if constexpr (PS == 1) sv[u] = E::ld(rowp[u], cv[u]);
    else v[u] = ld16(rowp[u], static_cast<int64_t>(cv[u]) * PS);
  }
  __builtin_amdgcn_sched_barrier(0);

  // Phase 2: angle table, vector descriptors, rows to LDS.
#pragma unroll
  for (int kk = 0; kk < kTabPre; ++kk) {
    const int idx = threadIdx.x + kk * kBlock;
    if (idx < ntab) {
      float sn, cn;
      sincos_angle(rope_angle(tp[kk], tw[kk]), &sn, &cn);
      cs[idx] = make_float2(a.ra.mu * cn, a.ra.mu * sn);
    }
  }
  for (int idx = threadIdx.x + kTabPre * kBlock; idx < ntab; idx += kBlock) {
    const int t = static_cast<int>(fdiv(static_cast<uint32_t>(idx), a.fd_np));
    const int i = idx - t * a.np;
    float sn, cn;
    sincos_angle(rope_angle(pos[static_cast<int64_t>(t0 + t) * a.A + axis_of_pair(i, a)],
                            inv_freq[i]), &sn, &cn);
    cs[idx] = make_float2(a.ra.mu * cn, a.ra.mu * sn);
  }
  for (int c = threadIdx.x; c < a.nv; c += kBlock) vector_desc<PS>(c, a, &d4s[c], &d1s[c]);
  // Partners come from LDS for the half pairing, and on the scalar path for
  // both; interleaved partners of a vector sit in the vector itself.
  const bool via_lds = PS == 1 || a.ra.layout == ET_ROPE_HALF;
  if (via_lds && !PERM) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = static_cast<int>(rope_slot<U>(0, threadIdx.x, u));
      if (s >= nslot) continue;
      S* dst = xs + sl[u] * a.span + cv[u] * PS;
      if constexpr (PS == 1) E::st(dst, 0, sv[u]);
      else *reinterpret_cast<u32x4*>(dst) = v[u];
    }
  }
  __syncthreads();

  // Phase 3: rotate and store.  A thread's slots usually share one column
  // (the row length divides the slot stride) and one token (a wave's rows
  // lie in one token when the head count is a multiple of the rows a wave
  // covers).  When that holds for every slot of every lane of the wave, and
  // the partner runs sit at multiples of 4 entries, the wave takes one
  // descriptor and one set of angles per lane and issues the partner reads
  // of all its slots before the first rotation: one LDS round trip instead
  // of one per slot, each of which held back that slot's store.  Otherwise
  // the descriptor is read again only when the column changes and the
  // angles are kept until the token or column changes.  Both paths give the
  // same bits.
  const bool half = a.ra.layout == ET_ROPE_HALF;
  if constexpr (PERM) {
    // Partners across lanes, no LDS copy of the rows.  A head row's nv
    // vectors sit in nv consecutive lanes (nv divides 64), and in every
    // vector each 32-bit word holds entries of one run whose partner
    // offset is a whole number of words (the host checks this layout).  The
    // partners of word j of a vector are then one word of another lane of
    // the row: word (j + off / EPD) mod 4 of the vector off / EPD words
    // away.  Each lane first rotates its own words by the amount its
    // readers need, (-off_own / EPD) mod 4 (the same for both of its runs,
    // also checked), so a reader fetches word j of the rotated set from
    // the source lane: four cross-lane reads per vector.  Every lane takes
    // part in the reads; clamped slots only feed rows that are not stored.
    constexpr int EPD = 4 / static_cast<int>(sizeof(S));   // entries per word
    const int4 dd = d4s[cv[0]];
    const int dd1 = d1s[cv[0]];
    const int krp = dd1 & 0xFF;
    const int c0 = cv[0] * PS;
    const int offA = dd.x - c0, offB = dd.y - c0;
    // offA is a whole number of words (the host checks it), and a partner
    // column is never negative: both quotients are plain shifts.
    constexpr int kLgEpd = EPD == 2 ? 1 : 0;
    const int rot = ((-offA) >> kLgEpd) & 3;
    const int rowlane = static_cast<int>(threadIdx.x % 64) - cv[0];
    int addr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = EPD * j < krp ? offA : offB;
      addr[j] = (rowlane + static_cast<int>(static_cast<unsigned>(c0 + EPD * j + off) / PS)) * 4;
    }
    float2 an[PS];
    int cur = -1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 r = (rot & 1) ? v[u].yzwx : v[u];
      r = (rot & 2) ? r.zwxy : r;
      u32x4 pw;
      pw.x = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr[0], static_cast<int>(r.x)));
      pw.y = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr[1], static_cast<int>(r.y)));
      pw.z = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr[2], static_cast<int>(r.z)));
      pw.w = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr[3], static_cast<int>(r.w)));
      const int s = static_cast<int>(rope_slot<U>(0, threadIdx.x, u));
      if (s < nslot) {
        if (tl[u] != cur) {
          entry_angles<PS>(cs + tl[u] * a.np, dd, dd1, half, an);
          cur = tl[u];
        }
        float y[PS];
#pragma unroll
        for (int e = 0; e < PS; ++e) {
          const uint32_t w = pw[e / EPD];
          float xp;
          if constexpr (EPD == 2) xp = (e & 1) ? E::hi(w) : E::lo(w);
          else xp = __uint_as_float(w);
          y[e] = __builtin_fmaf(E::get(v[u], e), an[e].x, xp * an[e].y);
        }
        out.store(isq[u], rel[u] + cv[u] * PS, rowp[u] + cv[u] * PS, E::pack(y));
      }
    }
    return;
  }
  if constexpr (PS > 1 && !PERM) {
    bool uni = static_cast<int>(rope_slot<U>(0, threadIdx.x, U - 1)) < nslot;
#pragma unroll
    for (int u = 1; u < U; ++u) uni = uni && cv[u] == cv[0] && tl[u] == tl[0];
    const int4 d0 = d4s[cv[0]];
    const int d10 = d1s[cv[0]];
    const int kr0 = d10 & 0xFF;
    if (via_lds) uni = uni && ((kr0 | d0.x | d0.y) & 3) == 0;
    if (__ballot(uni) == __ballot(1)) {
      float2 an[PS];
      entry_angles<PS>(cs + tl[0] * a.np, d0, d10, half, an);
      Partners<S, PS> pr[U];
      if (via_lds) {
#pragma unroll
        for (int u = 0; u < U; ++u) read_partners4<S, PS>(xs + sl[u] * a.span, d0, kr0, pr[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[PS], y[PS];
#pragma unroll
        for (int e = 0; e < PS; ++e) x[e] = E::get(v[u], e);
#pragma unroll
        for (int e = 0; e < PS; ++e) {
          const float xp = via_lds ? partner_of<S, PS>(pr[u], e) : x[e ^ 1];
          y[e] = __builtin_fmaf(x[e], an[e].x, xp * an[e].y);
        }
        out.store(isq[u], rel[u] + cv[u] * PS, rowp[u] + cv[u] * PS, E::pack(y));
      }
      return;
    }
  }
  int4 d = make_int4(0, 0, 0, 0);
  int d1 = 0, kr = 0, cur_cv = -1, cur_tl = -1;
  float2 ang[PS];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int s = static_cast<int>(rope_slot<U>(0, threadIdx.x, u));
    if (s >= nslot) continue;
    if (cv[u] != cur_cv) {
      d = d4s[cv[u]];
      d1 = d1s[cv[u]];
      kr = d1 & 0xFF;
      cur_cv = cv[u];
      cur_tl = -1;
    }
    if (tl[u] != cur_tl) {
      entry_angles<PS>(cs + tl[u] * a.np, d, d1, half, ang);
      cur_tl = tl[u];
    }
    float x[PS], y[PS];
#pragma unroll
    for (int e = 0; e < PS; ++e) x[e] = PS == 1 ? sv[u] : E::get(v[u], e);
    if (via_lds) {
      const S* xr = xs + sl[u] * a.span;
      // Partners are read W entries at a time when both runs' partner
      // columns and the split are multiples of W (the usual case: half
      // widths even), else one entry at a time.
      const int al = kr | d.x | d.y;
      if (PS >= 4 && (al & 3) == 0) {
        rotate_runs<S, PS, (PS >= 4 ? 4 : 1)>(xr, x, y, d, kr, ang);
      } else if (PS >= 2 && (al & 1) == 0) {
        rotate_runs<S, PS, (PS >= 2 ? 2 : 1)>(xr, x, y, d, kr, ang);
      } else {
        rotate_runs<S, PS, 1>(xr, x, y, d, kr, ang);
      }
    } else if constexpr (PS > 1) {
      // Interleaved pairs (e, e ^ 1) lie inside the vector.
#pragma unroll
      for (int e = 0; e < PS; ++e) y[e] = __builtin_fmaf(x[e], ang[e].x, x[e ^ 1] * ang[e].y);
    }
    if constexpr (PS == 1) {
      E::st(rowp[u], cv[u], y[0]);
    } else {
      out.store(isq[u], rel[u] + cv[u] * PS, rowp[u] + cv[u] * PS, E::pack(y));
    }
  }
}

// LDS bytes of a workgroup of rpb rows: angle table, descriptors, rows.
inline void multi_lds(MultiArgs& a, int es, size_t* bytes) {
  a.ntok_max = (a.rpb + a.heads - 1) / a.heads + 1;
  if (a.ntok_max > a.rpb) a.ntok_max = a.rpb;
  const uint32_t tab = static_cast<uint32_t>(a.ntok_max) * a.np * sizeof(float2);
  a.d4_off = (tab + 15u) & ~15u;
  a.d1_off = a.d4_off + static_cast<uint32_t>(a.nv) * 16u;
  a.xs_off = (a.d1_off + static_cast<uint32_t>(a.nv) * 4u + 15u) & ~15u;
  *bytes = a.xs_off + static_cast<size_t>(a.rpb) * a.span * es;
}

// Whether every vector of ps entries holds at most two runs: at most one
// place inside it where an axis or (half pairing) a half begins.
inline bool runs_fit(const int64_t* dims, int64_t A, int layout, int ps) {
  std::vector<int64_t> b;
  int64_t o = 0;
  for (int64_t ax = 0; ax < A; ++ax) {
    b.push_back(o);
    if (layout == ET_ROPE_HALF) b.push_back(o + dims[ax] / 2);
    o += dims[ax];
  }
  std::sort(b.begin(), b.end());
  b.erase(std::unique(b.begin(), b.end()), b.end());
  for (int64_t c0 = 0; c0 < o; c0 += ps) {
    int inside = 0;
    for (int64_t x : b) inside += (x > c0 && x < c0 + ps) ? 1 : 0;
    if (inside > 1) return false;
  }
  return true;
}

// Whether the half pairing can take its partners across lanes: a head row's
// vectors fill whole groups of lanes (nv divides 64), every 32-bit word of a
// vector holds entries of one run whose partner offset is a whole number of
// words, and the rotation (-offset / words) mod 4 is the same for every run
// of a vector (it is what the lanes reading that vector need).
inline bool perm_fits(const int64_t* dims, int64_t A, int layout, int ps, int es) {
  if (layout != ET_ROPE_HALF || ps <= 1) return false;
  int64_t span = 0;
  for (int64_t ax = 0; ax < A; ++ax) span += dims[ax];
  const int64_t nv = span / ps;
  if (nv <= 0 || 64 % nv != 0) return false;
  const int epd = 4 / es;
  std::vector<int64_t> off(static_cast<size_t>(span));
  int64_t o = 0;
  for (int64_t ax = 0; ax < A; ++ax) {
    const int64_t hd = dims[ax] / 2;
    for (int64_t l = 0; l < dims[ax]; ++l) off[static_cast<size_t>(o + l)] = l < hd ? hd : -hd;
    o += dims[ax];
  }
  for (int64_t c0 = 0; c0 < span; c0 += ps) {
    int rot = -1;
    for (int64_t c = c0; c < c0 + ps; c += epd) {
      const int64_t d = off[static_cast<size_t>(c)];
      for (int e = 1; e < epd; ++e)
        if (off[static_cast<size_t>(c + e)] != d) return false;
      if (d % epd != 0) return false;
      const int r = static_cast<int>((-d / epd) & 3);
      if (rot >= 0 && r != rot) return false;
      rot = r;
    }
  }
  return true;
}

template <typename S, int PS, bool PERM>
void launch_multi(S* q, S* k, const int32_t* pos, const float* inv_freq, MultiArgs a, int64_t T,
                  size_t shmem, hipStream_t s) {
  const int64_t tok_per_launch = (int64_t{1} << 30) / a.heads;
  for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
    const int64_t m = T - t0 < tok_per_launch ? T - t0 : tok_per_launch;
    a.ra.T = m;
    a.rows = static_cast<uint32_t>(m * a.heads);
    const unsigned grid = (a.rows + a.rpb - 1) / a.rpb;
    rope_multi_kernel<S, PS, kMultiU, PERM><<<grid, kBlock, shmem, s>>>(
        q + t0 * a.ra.hq * a.ra.D, a.ra.hk ? k + t0 * a.ra.hk * a.ra.D : k, pos + t0 * a.A,
        inv_freq, a);
  }
}

template <typename S>
et_status rope_multi_entry(S* q, int64_t hq, S* k, int64_t hk, const int32_t* pos, int64_t T,
                           int64_t D, int64_t A, const int64_t* dims, const float* inv_freq,
                           float mu, int layout, void* stream) {
  if (A < 1 || A > kMaxAxes) return ET_ERR_BAD_ARG;
  if (!dims) return ET_ERR_NULL_POINTER;
  int64_t span = 0;
  for (int64_t ax = 0; ax < A; ++ax) {
    if (dims[ax] < 0 || (dims[ax] & 1) || dims[ax] > D) return ET_ERR_BAD_ARG;
    span += dims[ax];
  }
  int64_t qb = 0, kb = 0;
  const et_status st = check_rope(q, hq, k, hk, pos, T, D, span, inv_freq, mu, layout, &qb, &kb);
  if (st != ET_OK) return st;
  if (span > kMultiMaxSpan) return ET_ERR_BAD_SIZE;
  int64_t pb = 0;
  if (!mul_ok(T, A * int64_t(sizeof(int32_t)), &pb)) return ET_ERR_BAD_SIZE;
  if (!ranges_ok(q, qb, pos, pb, false) || !ranges_ok(k, kb, pos, pb, false)) return ET_ERR_OVERLAP;
  if (T == 0 || hq + hk == 0 || span == 0) return ET_OK;

  constexpr int V = Elem<S>::V;
  const bool vec = span % V == 0 && D % V == 0 && aligned16(q) && (hk == 0 || aligned16(k)) &&
                   runs_fit(dims, A, layout, V);
  const int ps = vec ? V : 1;
  MultiArgs a{};
  a.ra.hq = static_cast<int>(hq);
  a.ra.hk = static_cast<int>(hk);
  a.ra.D = static_cast<int>(D);
  a.ra.layout = layout;
  a.ra.mu = mu;
  a.A = static_cast<int>(A);
  a.span = static_cast<int>(span);
  a.np = a.span / 2;
  int o = 0;
  for (int ax = 0; ax <= kMaxAxes; ++ax) {
    a.off[ax] = o;
    a.foff[ax] = o / 2;
    if (ax < A) o += static_cast<int>(dims[ax]);
  }
  a.heads = static_cast<int>(hq + hk);
  a.perm = vec && perm_fits(dims, A, layout, ps, static_cast<int>(sizeof(S))) ? 1 : 0;
  a.nv = a.span / ps;
  a.rpb = (kBlock * kMultiU) / a.nv;
  size_t shmem = 0;
  for (;;) {
    multi_lds(a, static_cast<int>(sizeof(S)), &shmem);
    if (shmem <= static_cast<size_t>(kMaxTableBytes) || a.rpb == 1) break;
    a.rpb /= 2;
  }
  if (a.rpb < 1 || shmem > static_cast<size_t>(kMaxTableBytes)) return ET_ERR_BAD_SIZE;
  a.fd_heads = make_fastdiv(static_cast<uint32_t>(a.heads));
  a.fd_nv = make_fastdiv(static_cast<uint32_t>(a.nv));
  a.fd_np = make_fastdiv(static_cast<uint32_t>(a.np));

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (vec && a.perm)
    launch_multi<S, V, true>(q, k, pos, inv_freq, a, T, shmem, s);
  else if (vec)
    launch_multi<S, V, false>(q, k, pos, inv_freq, a, T, shmem, s);
  else
    launch_multi<S, 1, false>(q, k, pos, inv_freq, a, T, shmem, s);
  return launch_status();
}

}  // namespace
}  // namespace et

using et::Bf16;
using et::F16;

extern "C" {

et_status et_rope_f32(float* x, const int32_t* pos, int64_t T, int64_t H, int64_t D, int64_t d_rot,
                      const float* inv_freq, float attn_scaling, int layout, void* stream) {
  return et::rope_entry<float>(x, H, nullptr, 0, pos, T, D, d_rot, inv_freq, attn_scaling, layout,
                               stream);
}

et_status et_rope_bf16(et_bf16* x, const int32_t* pos, int64_t T, int64_t H, int64_t D,
                       int64_t d_rot, const float* inv_freq, float attn_scaling, int layout,
                       void* stream) {
  return et::rope_entry<Bf16>(reinterpret_cast<Bf16*>(x), H, nullptr, 0, pos, T, D, d_rot,
                              inv_freq, attn_scaling, layout, stream);
}

et_status et_rope_f16(et_f16* x, const int32_t* pos, int64_t T, int64_t H, int64_t D,
                       int64_t d_rot, const float* inv_freq, float attn_scaling, int layout,
                       void* stream) {
  return et::rope_entry<F16>(reinterpret_cast<F16*>(x), H, nullptr, 0, pos, T, D, d_rot,
                              inv_freq, attn_scaling, layout, stream);
}

et_status et_rope_qk_f32(float* q, int64_t Hq, float* k, int64_t Hk, const int32_t* pos, int64_t T,
                         int64_t D, int64_t d_rot, const float* inv_freq, float attn_scaling,
                         int layout, void* stream) {
  return et::rope_entry<float>(q, Hq, k, Hk, pos, T, D, d_rot, inv_freq, attn_scaling, layout,
                               stream);
}

et_status et_rope_qk_bf16(et_bf16* q, int64_t Hq, et_bf16* k, int64_t Hk, const int32_t* pos,
                          int64_t T, int64_t D, int64_t d_rot, const float* inv_freq,
                          float attn_scaling, int layout, void* stream) {
  return et::rope_entry<Bf16>(reinterpret_cast<Bf16*>(q), Hq, reinterpret_cast<Bf16*>(k), Hk, pos,
                              T, D, d_rot, inv_freq, attn_scaling, layout, stream);
}

et_status et_rope_qk_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk, const int32_t* pos,
                          int64_t T, int64_t D, int64_t d_rot, const float* inv_freq,
                          float attn_scaling, int layout, void* stream) {
  return et::rope_entry<F16>(reinterpret_cast<F16*>(q), Hq, reinterpret_cast<F16*>(k), Hk, pos,
                              T, D, d_rot, inv_freq, attn_scaling, layout, stream);
}

et_status et_rmsnorm_rope_qk_f32(float* q, const float* gq, int64_t Hq, float* k, const float* gk,
                                 int64_t Hk, float eps, const int32_t* pos, int64_t T, int64_t D,
                                 int64_t d_rot, const float* inv_freq, float attn_scaling,
                                 int layout, void* stream) {
  return et::qknorm_entry<float>(q, gq, Hq, k, gk, Hk, eps, pos, T, D, d_rot, inv_freq,
                                 attn_scaling, layout, stream);
}

et_status et_rmsnorm_rope_qk_bf16(et_bf16* q, const et_bf16* gq, int64_t Hq, et_bf16* k,
                                  const et_bf16* gk, int64_t Hk, float eps, const int32_t* pos,
                                  int64_t T, int64_t D, int64_t d_rot, const float* inv_freq,
                                  float attn_scaling, int layout, void* stream) {
  return et::qknorm_entry<Bf16>(reinterpret_cast<Bf16*>(q), reinterpret_cast<const Bf16*>(gq), Hq,
                                reinterpret_cast<Bf16*>(k), reinterpret_cast<const Bf16*>(gk), Hk,
                                eps, pos, T, D, d_rot, inv_freq, attn_scaling, layout, stream);
}

et_status et_rmsnorm_rope_qk_f16(et_f16* q, const et_f16* gq, int64_t Hq, et_f16* k,
                                  const et_f16* gk, int64_t Hk, float eps, const int32_t* pos,
                                  int64_t T, int64_t D, int64_t d_rot, const float* inv_freq,
                                  float attn_scaling, int layout, void* stream) {
  return et::qknorm_entry<F16>(reinterpret_cast<F16*>(q), reinterpret_cast<const F16*>(gq), Hq,
                                reinterpret_cast<F16*>(k), reinterpret_cast<const F16*>(gk), Hk,
                                eps, pos, T, D, d_rot, inv_freq, attn_scaling, layout, stream);
}

et_status et_rope_cache_f32(const float* inv_freq, int64_t max_pos, int64_t d_rot,
                            float* cos_cache, float* sin_cache, void* stream) {
  return et::rope_cache_entry(inv_freq, max_pos, d_rot, cos_cache, sin_cache, stream);
}

et_status et_rope_qk_cached_f32(float* q, int64_t Hq, float* k, int64_t Hk, const int32_t* pos,
                                int64_t T, int64_t D, int64_t d_rot, const float* cos_cache,
                                const float* sin_cache, int64_t max_pos, float attn_scaling,
                                int layout, void* stream) {
  const et::RopeCache c{cos_cache, sin_cache, max_pos};
  return et::rope_entry<float>(q, Hq, k, Hk, pos, T, D, d_rot, nullptr, attn_scaling, layout,
                               stream, &c);
}

et_status et_rope_qk_cached_bf16(et_bf16* q, int64_t Hq, et_bf16* k, int64_t Hk,
                                 const int32_t* pos, int64_t T, int64_t D, int64_t d_rot,
                                 const float* cos_cache, const float* sin_cache, int64_t max_pos,
                                 float attn_scaling, int layout, void* stream) {
  const et::RopeCache c{cos_cache, sin_cache, max_pos};
  return et::rope_entry<Bf16>(reinterpret_cast<Bf16*>(q), Hq, reinterpret_cast<Bf16*>(k), Hk, pos,
                              T, D, d_rot, nullptr, attn_scaling, layout, stream, &c);
}

et_status et_rope_qk_cached_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk,
                                 const int32_t* pos, int64_t T, int64_t D, int64_t d_rot,
                                 const float* cos_cache, const float* sin_cache, int64_t max_pos,
                                 float attn_scaling, int layout, void* stream) {
  const et::RopeCache c{cos_cache, sin_cache, max_pos};
  return et::rope_entry<F16>(reinterpret_cast<F16*>(q), Hq, reinterpret_cast<F16*>(k), Hk, pos,
                              T, D, d_rot, nullptr, attn_scaling, layout, stream, &c);
}

et_status et_rope_multi_f32(float* q, int64_t Hq, float* k, int64_t Hk, const int32_t* pos,
                            int64_t T, int64_t D, int64_t n_axes, const int64_t* dims,
                            const float* inv_freq, float attn_scaling, int layout, void* stream) {
  return et::rope_multi_entry<float>(q, Hq, k, Hk, pos, T, D, n_axes, dims, inv_freq, attn_scaling,
                                     layout, stream);
}

et_status et_rope_multi_bf16(et_bf16* q, int64_t Hq, et_bf16* k, int64_t Hk, const int32_t* pos,
                             int64_t T, int64_t D, int64_t n_axes, const int64_t* dims,
                             const float* inv_freq, float attn_scaling, int layout, void* stream) {
  return et::rope_multi_entry<Bf16>(reinterpret_cast<Bf16*>(q), Hq, reinterpret_cast<Bf16*>(k), Hk,
                                    pos, T, D, n_axes, dims, inv_freq, attn_scaling, layout, stream);
}

et_status et_rope_multi_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk, const int32_t* pos,
                             int64_t T, int64_t D, int64_t n_axes, const int64_t* dims,
                             const float* inv_freq, float attn_scaling, int layout, void* stream) {
  return et::rope_multi_entry<F16>(reinterpret_cast<F16*>(q), Hq, reinterpret_cast<F16*>(k), Hk,
                                    pos, T, D, n_axes, dims, inv_freq, attn_scaling, layout, stream);
}

}  // extern "C"
