/*
 * et.h -- C ABI of libet.so: memory-bound transformer ops for AMD Instinct
 * MI355X (gfx950), as hand-written HIP kernels.
 *
 * Ops and the passages that define them (web pages, by section):
 *   [OPS] "Operations" (op spec of the glia runtime): 2 Normalization /
 *         RmsNorm, LayerNorm; 3 Position encoding / Rope; 4 Activation /
 *         Silu, SwiGlu, Gelu, GeGlu, Softmax;
 *         5 Attention / QK-norm; 8 Sampling / Greedy; 10 Fused ops
 *         (FusedSkipNorm, and fused = unfused within tolerance).
 *   [ELT] "Elementwise kernels in C: RMSNorm, RoPE, SiLU-mul, embedding,
 *         add, argmax": 2.1 RMSNorm; 2.2 RoPE; 2.3 SiLU-mul (SwiGLU);
 *         2.4 Embedding, add, argmax; 4 The interface (names and argument
 *         order of the six routines kept here).
 *   [DNN] "ruDNN User Guide": 7 LayerNorm, RMSNorm, and Softmax (softmax over
 *         the final axis, f32 statistics, output in the input type).
 *
 * Common rules for every entry point
 *   - Types: the _f32 variant stores float; the _bf16 variant stores
 *     bfloat16 bits (et_bf16) and the _f16 variant IEEE binary16 bits
 *     (et_f16, [OPS] gives F16 tolerances); both compute in f32, rounding
 *     each stored result once to nearest-even (f16 overflows to infinity
 *     past 65504 and keeps subnormals).  inv_freq, caches and scalars are
 *     f32 in every variant.
 *   - Pointers are DEVICE pointers of the current HIP device, except scalars
 *     passed by value.  The caller owns every buffer; the library allocates
 *     nothing, keeps no state and is reentrant.
 *   - stream is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; it never synchronises.  Device faults
 *     surface at the caller's next synchronisation.
 *   - Layout: every tensor is dense row-major with no padding.
 *   - Sizes are int64_t element counts.  A size of 0 makes the call a no-op
 *     returning ET_OK (argmax with n == 0 writes -1 per row, see below).
 *   - Aliasing: only the exact aliases stated per op are allowed (same start,
 *     same extent); any other overlap of an output with another buffer
 *     returns ET_ERR_OVERLAP before anything is enqueued.
 *   - Results are deterministic.  For the row ops (RMSNorm, fused
 *     add+RMSNorm, RoPE, fused RMSNorm+RoPE, softmax) the bits of a row depend only on
 *     that row's inputs, the row length and the 16-byte alignment of the
 *     buffers -- never on the number of rows in the call.
 *   - Errors: argument problems are reported before any launch and nothing is
 *     written; ET_ERR_HIP reports a failed launch.
 */
#ifndef ET_H
#define ET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ET_ABI_VERSION 1

/* Raw bfloat16 bits (sign, 8-bit exponent, 7-bit fraction). */
typedef uint16_t et_bf16;
/* Raw IEEE binary16 bits (sign, 5-bit exponent, 10-bit fraction). */
typedef uint16_t et_f16;

typedef enum {
    ET_OK = 0,
    ET_ERR_NULL_POINTER = 1, /* a required pointer is NULL while its size is nonzero */
    ET_ERR_BAD_SIZE = 2,     /* negative size, size product overflow, or a size past a limit */
    ET_ERR_BAD_ARG = 3,      /* d_rot odd / > D, bad layout, eps < 0 or not finite, ... */
    ET_ERR_OVERLAP = 4,      /* buffers overlap other than by an allowed exact alias */
    ET_ERR_WORKSPACE = 5,    /* argmax workspace smaller than et_argmax_workspace_bytes() */
    ET_ERR_HIP = 6           /* the HIP runtime rejected a launch */
} et_status;

enum { ET_ROPE_HALF = 0, ET_ROPE_INTERLEAVED = 1 };

/* Storage type codes, for the entry points that take the type as an argument. */
enum { ET_STORAGE_F32 = 0, ET_STORAGE_BF16 = 1, ET_STORAGE_F16 = 2 };

/* ------------------------------------------------------------------------
 * RMSNorm  ([OPS] RmsNorm; [ELT] 2.1)
 *   y[r, i] = x[r, i] / sqrt(mean_i(x[r, :]^2) + eps) * w[i]
 *   eps is added inside the root; a zero row maps to 0 (eps > 0).
 *   x, y: [rows, d]; w: [d].  eps: finite, >= 0.  d >= 1 when rows > 0.
 *   Alias allowed: y == x (in place).
 *   The sum of squares is f32 in a fixed order that depends on d only.
 */
et_status et_rmsnorm_f32(const float* x, const float* w, float* y,
                         int64_t rows, int64_t d, float eps, void* stream);
et_status et_rmsnorm_bf16(const et_bf16* x, const et_bf16* w, et_bf16* y,
                          int64_t rows, int64_t d, float eps, void* stream);
et_status et_rmsnorm_f16(const et_f16* x, const et_f16* w, et_f16* y,
                         int64_t rows, int64_t d, float eps, void* stream);

/* ------------------------------------------------------------------------
 * Fused residual add + RMSNorm  ([OPS] 10 Fused ops, FusedSkipNorm)
 *   h = x + residual, rounded to the storage type (the value returned);
 *   y = RMSNorm(h as stored, w, eps).  One pass; both outputs written.
 *   x, residual, y, h: [rows, d]; w: [d].
 *   Aliases allowed: y == x and/or h == residual (in place), h == x when
 *   y != x.
 */
et_status et_add_rmsnorm_f32(const float* x, const float* residual,
                             const float* w, float* y, float* h,
                             int64_t rows, int64_t d, float eps, void* stream);
et_status et_add_rmsnorm_bf16(const et_bf16* x, const et_bf16* residual,
                              const et_bf16* w, et_bf16* y, et_bf16* h,
                              int64_t rows, int64_t d, float eps, void* stream);
et_status et_add_rmsnorm_f16(const et_f16* x, const et_f16* residual,
                             const et_f16* w, et_f16* y, et_f16* h,
                             int64_t rows, int64_t d, float eps, void* stream);

/* ------------------------------------------------------------------------
 * RoPE, in place  ([OPS] Rope; [ELT] 2.2 and 4, tl_rope_f32)
 *   x: [T, H, D]; pos: int32 [T]; inv_freq: f32 [d_rot / 2].
 *   For token t and pair i < d_rot/2 the angle is p_t * w_i formed in f64
 *   and rounded to f32 (= f32(p) * f32(w) for |p| < 2^24); then
 *     a' = mu (a cos - b sin),  b' = mu (a sin + b cos),  mu = attn_scaling.
 *   layout ET_ROPE_HALF pairs (i, i + d_rot/2); ET_ROPE_INTERLEAVED pairs
 *   (2i, 2i + 1).  Entries d_rot..D-1 of each head are not touched.
 *   d_rot: even, 0 <= d_rot <= D.  attn_scaling: finite.
 */
et_status et_rope_f32(float* x, const int32_t* pos, int64_t T, int64_t H,
                      int64_t D, int64_t d_rot, const float* inv_freq,
                      float attn_scaling, int layout, void* stream);
et_status et_rope_bf16(et_bf16* x, const int32_t* pos, int64_t T, int64_t H,
                       int64_t D, int64_t d_rot, const float* inv_freq,
                       float attn_scaling, int layout, void* stream);
et_status et_rope_f16(et_f16* x, const int32_t* pos, int64_t T, int64_t H,
                      int64_t D, int64_t d_rot, const float* inv_freq,
                      float attn_scaling, int layout, void* stream);

/* RoPE on a query and a key tensor in one launch (one angle per (token,
 * pair) serves all Hq + Hk heads).  q: [T, Hq, D]; k: [T, Hk, D] (k may be
 * NULL when Hk == 0).  Same rules as et_rope_*; q and k must not overlap. */
et_status et_rope_qk_f32(float* q, int64_t Hq, float* k, int64_t Hk,
                         const int32_t* pos, int64_t T, int64_t D,
                         int64_t d_rot, const float* inv_freq,
                         float attn_scaling, int layout, void* stream);
et_status et_rope_qk_bf16(et_bf16* q, int64_t Hq, et_bf16* k, int64_t Hk,
                          const int32_t* pos, int64_t T, int64_t D,
                          int64_t d_rot, const float* inv_freq,
                          float attn_scaling, int layout, void* stream);
et_status et_rope_qk_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk,
                         const int32_t* pos, int64_t T, int64_t D,
                         int64_t d_rot, const float* inv_freq,
                         float attn_scaling, int layout, void* stream);

/* ------------------------------------------------------------------------
 * RoPE cos/sin cache  ([OPS] 3 Rope, cos/sin cache)
 *   Fills cos_cache[p * d_rot/2 + i] and sin_cache[p * d_rot/2 + i] (f32,
 *   device, [max_pos, d_rot/2], caller-owned) with the cosine and sine of
 *   the angle et_rope_* uses for position p and pair i, for 0 <= p < max_pos.
 *   Bit for bit the values et_rope_* computes, so a rotation from this cache
 *   equals the computed one.  d_rot even; max_pos <= 2^31 - 1 and
 *   max_pos * d_rot/2 < 2^32; the three buffers must not overlap.
 */
et_status et_rope_cache_f32(const float* inv_freq, int64_t max_pos,
                            int64_t d_rot, float* cos_cache, float* sin_cache,
                            void* stream);

/* RoPE on q and k with the rotation read from a cos/sin cache instead of
 * computed ([OPS] 3 Rope, cos/sin cache): for token t the pair i uses
 * c = cos_cache[pos[t] * d_rot/2 + i], s = sin_cache[same] (any values;
 * et_rope_cache_f32 makes the standard ones), then
 *   a' = mu (a c - b s),  b' = mu (a s + b c)
 * as et_rope_qk_*.  A position outside [0, max_pos) reads nothing from the
 * cache; that token's rotated entries become NaN (its other entries are
 * left alone).  0 <= max_pos <= 2^31 - 1; with max_pos == 0 the caches may
 * be NULL.  The caches must not overlap q or k.  inv_freq is not used.
 * Other rules as et_rope_qk_*.
 */
et_status et_rope_qk_cached_f32(float* q, int64_t Hq, float* k, int64_t Hk,
                                const int32_t* pos, int64_t T, int64_t D,
                                int64_t d_rot, const float* cos_cache,
                                const float* sin_cache, int64_t max_pos,
                                float attn_scaling, int layout, void* stream);
et_status et_rope_qk_cached_bf16(et_bf16* q, int64_t Hq, et_bf16* k,
                                 int64_t Hk, const int32_t* pos, int64_t T,
                                 int64_t D, int64_t d_rot,
                                 const float* cos_cache,
                                 const float* sin_cache, int64_t max_pos,
                                 float attn_scaling, int layout, void* stream);
et_status et_rope_qk_cached_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk,
                                const int32_t* pos, int64_t T, int64_t D,
                                int64_t d_rot, const float* cos_cache,
                                const float* sin_cache, int64_t max_pos,
                                float attn_scaling, int layout, void* stream);

/* ------------------------------------------------------------------------
 * Multi-axis RoPE on Q and K, in place  ([OPS] 3 Rope, multi-axis RoPE)
 *   Token t has a position vector pos[t * n_axes + a] (int32, device,
 *   [T, n_axes]).  The first span = dims[0] + ... + dims[n_axes-1] entries
 *   of every head are cut into consecutive sub-ranges, axis a owning the
 *   dims[a] entries from o_a = dims[0] + ... + dims[a-1].  Axis a rotates its
 *   sub-range as et_rope_qk_* rotates a whole head of dims[a] entries
 *   (same angle rule, same pairing per layout, relative to o_a), with
 *   position pos[t * n_axes + a] and frequencies inv_freq[h_a + j],
 *   j < dims[a]/2, h_a = o_a / 2 (inv_freq: f32, device, [span / 2]; each
 *   axis may have its own base).  Entries span..D-1 are not touched.
 *   dims: a HOST array of n_axes int64, each even and >= 0;
 *   1 <= n_axes <= 8; span <= D and span <= 1024 (else ET_ERR_BAD_SIZE).
 *   q: [T, Hq, D]; k: [T, Hk, D] (NULL with Hk == 0).  One axis of width r
 *   gives the bits of et_rope_qk_* with d_rot = r.
 */
et_status et_rope_multi_f32(float* q, int64_t Hq, float* k, int64_t Hk,
                            const int32_t* pos, int64_t T, int64_t D,
                            int64_t n_axes, const int64_t* dims,
                            const float* inv_freq, float attn_scaling,
                            int layout, void* stream);
et_status et_rope_multi_bf16(et_bf16* q, int64_t Hq, et_bf16* k, int64_t Hk,
                             const int32_t* pos, int64_t T, int64_t D,
                             int64_t n_axes, const int64_t* dims,
                             const float* inv_freq, float attn_scaling,
                             int layout, void* stream);
et_status et_rope_multi_f16(et_f16* q, int64_t Hq, et_f16* k, int64_t Hk,
                            const int32_t* pos, int64_t T, int64_t D,
                            int64_t n_axes, const int64_t* dims,
                            const float* inv_freq, float attn_scaling,
                            int layout, void* stream);

/* ------------------------------------------------------------------------
 * Fused RMSNorm + RoPE on Q and K, in place  ([OPS] 5 QK-norm)
 *   Each (token, head) row of length D is normalised over all D entries
 *   with the gain gq [D] (query heads) or gk [D] (key heads) and eps, then
 *   rotated as et_rope_qk_* on its first d_rot entries; the f32
 *   intermediate is not rounded; entries d_rot..D-1 are normalised only.
 *   The inverse root 1/sqrt(ss/D + eps) is the hardware estimate refined by
 *   one Newton step (within about 1 ulp) for mean squares in
 *   [2^-126, 2^126], the correctly rounded root and division outside it.
 *   q: [T, Hq, D]; k: [T, Hk, D] (NULL with Hk == 0; gk may then be NULL).
 */
et_status et_rmsnorm_rope_qk_f32(float* q, const float* gq, int64_t Hq,
                                 float* k, const float* gk, int64_t Hk,
                                 float eps, const int32_t* pos, int64_t T,
                                 int64_t D, int64_t d_rot,
                                 const float* inv_freq, float attn_scaling,
                                 int layout, void* stream);
et_status et_rmsnorm_rope_qk_bf16(et_bf16* q, const et_bf16* gq, int64_t Hq,
                                  et_bf16* k, const et_bf16* gk, int64_t Hk,
                                  float eps, const int32_t* pos, int64_t T,
                                  int64_t D, int64_t d_rot,
                                  const float* inv_freq, float attn_scaling,
                                  int layout, void* stream);
et_status et_rmsnorm_rope_qk_f16(et_f16* q, const et_f16* gq, int64_t Hq,
                                 et_f16* k, const et_f16* gk, int64_t Hk,
                                 float eps, const int32_t* pos, int64_t T,
                                 int64_t D, int64_t d_rot,
                                 const float* inv_freq, float attn_scaling,
                                 int layout, void* stream);

/* ------------------------------------------------------------------------
 * SiLU-gated multiply  ([OPS] Silu, SwiGlu; [ELT] 2.3, tl_silu_mul_f32)
 *   y[i] = gate[i] / (1 + exp(-gate[i])) * up[i]; for very negative gates
 *   exp overflows to +inf and the factor is -0 (never NaN).
 *   gate, up, y: [n].  Aliases allowed: y == gate, y == up.
 */
et_status et_silu_mul_f32(const float* gate, const float* up, float* y,
                          int64_t n, void* stream);
et_status et_silu_mul_bf16(const et_bf16* gate, const et_bf16* up, et_bf16* y,
                           int64_t n, void* stream);
et_status et_silu_mul_f16(const et_f16* gate, const et_f16* up, et_f16* y,
                          int64_t n, void* stream);

/* ------------------------------------------------------------------------
 * Residual add  ([OPS] Add; [ELT] 2.4, tl_add_f32)
 *   y[i] = a[i] + b[i], IEEE addition in the storage type (bf16: the f32
 *   sum rounded once, which is the correctly rounded bf16 sum).
 *   a, b, y: [n].  Aliases allowed: y == a, y == b.
 */
et_status et_add_f32(const float* a, const float* b, float* y, int64_t n,
                     void* stream);
et_status et_add_bf16(const et_bf16* a, const et_bf16* b, et_bf16* y,
                      int64_t n, void* stream);
et_status et_add_f16(const et_f16* a, const et_f16* b, et_f16* y,
                     int64_t n, void* stream);

/* ------------------------------------------------------------------------
 * Embedding gather  ([OPS] TokenEmbed; [ELT] 2.4, tl_embedding_f32)
 *   out[t, :] = table[ids[t], :], a bit copy of the row that starts at
 *   element ids[t] * d.  table: [V, d]; ids: int32 [n]; out: [n, d].
 *   The pages make valid ids the caller's duty; here an id outside [0, V)
 *   is never dereferenced and yields a row of quiet NaN instead.
 *   out must not overlap table or ids.
 */
et_status et_embedding_f32(const float* table, int64_t V, const int32_t* ids,
                           float* out, int64_t n, int64_t d, void* stream);
et_status et_embedding_bf16(const et_bf16* table, int64_t V,
                            const int32_t* ids, et_bf16* out, int64_t n,
                            int64_t d, void* stream);
et_status et_embedding_f16(const et_f16* table, int64_t V,
                           const int32_t* ids, et_f16* out, int64_t n,
                           int64_t d, void* stream);

/* ------------------------------------------------------------------------
 * Greedy argmax per row  ([OPS] Argmax, 8 Sampling / Greedy; [ELT] 2.4)
 *   out[r] = the lowest index of the largest non-NaN value of x[r, :]
 *   (-0 and +0 are equal; +inf is a number), or -1 when the row holds no
 *   number (all NaN, or n == 0).  x: [rows, n]; out: int32 [rows].
 *   n <= INT32_MAX.
 *   workspace: device scratch that lets the rows of a call of fewer than
 *   1024 rows be split over several workgroups (still one launch);
 *   et_argmax_workspace_bytes is 0 (none needed) for calls of 1024 rows or
 *   more, which get one workgroup per row.  Either workspace == NULL with
 *   workspace_bytes == 0 (one workgroup per row, no scratch), or
 *   workspace != NULL with workspace_bytes >= et_argmax_workspace_bytes(rows,
 *   n) and 16-byte aligned, else ET_ERR_WORKSPACE (ET_ERR_NULL_POINTER for
 *   NULL with a nonzero size).  The caller owns the workspace.  It must be
 *   zero-filled before its first use; every call leaves it zero-filled
 *   again, so it can be reused as is.  Calls that share a workspace must not
 *   run concurrently.  The result is the same with or without a workspace.
 */
size_t et_argmax_workspace_bytes(int64_t rows, int64_t n);
et_status et_argmax_f32(const float* x, int64_t rows, int64_t n, int32_t* out,
                        void* workspace, size_t workspace_bytes, void* stream);
et_status et_argmax_bf16(const et_bf16* x, int64_t rows, int64_t n,
                         int32_t* out, void* workspace, size_t workspace_bytes,
                         void* stream);
et_status et_argmax_f16(const et_f16* x, int64_t rows, int64_t n,
                        int32_t* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Greedy argmax for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same results as et_argmax_* with a workspace, with no workspace
 * argument and no allocation.  The split path's per-row key and counter
 * live in a 16 KiB array inside the library, one per GPU, held until the
 * process ends; it covers every call (the split path only runs for calls
 * of fewer than 1024 rows, 16 bytes per row), and a need beyond it would
 * be ET_ERR_WORKSPACE.  Each call that splits first clears the array with a
 * kernel on `stream`, then runs et_argmax_*'s kernel on it.
 *   storage: ET_STORAGE_F32, _BF16 or _F16 (x of that type), else
 *   ET_ERR_BAD_ARG; every other argument and status as et_argmax_*.
 *   Calls that overlap on one GPU (other streams, other host threads) share
 *   the array and race: serialise them. */
et_status et_argmax_noalloc(int storage, const void* x, int64_t rows,
                            int64_t n, int32_t* out, void* stream);

/* ------------------------------------------------------------------------
 * LayerNorm  ([OPS] 2 Normalization / LayerNorm; [DNN] 7)
 *   per row of d: mu = mean(x), var = mean((x - mu)^2) (the two-pass
 *   variance), y = (x - mu) / sqrt(var + eps) * gamma + beta.
 *   x, y: [rows, d]; gamma, beta: [d] in the storage type; beta may be NULL
 *   (no bias).  y may be x (in place).  eps finite and >= 0 (else
 *   ET_ERR_BAD_ARG); d == 0 with rows > 0 is ET_ERR_BAD_SIZE.
 */
et_status et_layernorm_f32(const float* x, const float* gamma, const float* beta,
                           float* y, int64_t rows, int64_t d, float eps,
                           void* stream);
et_status et_layernorm_bf16(const et_bf16* x, const et_bf16* gamma,
                            const et_bf16* beta, et_bf16* y, int64_t rows,
                            int64_t d, float eps, void* stream);
et_status et_layernorm_f16(const et_f16* x, const et_f16* gamma,
                           const et_f16* beta, et_f16* y, int64_t rows,
                           int64_t d, float eps, void* stream);

/* ------------------------------------------------------------------------
 * GELU-gated multiply, GeGLU  ([OPS] 4 Activation / Gelu, GeGlu)
 *   y = Gelu(gate) * up elementwise, with approximate = ET_GELU_ERF:
 *   Gelu(x) = x/2 (1 + erf(x/sqrt 2)), or ET_GELU_TANH:
 *   Gelu(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); any other value
 *   is ET_ERR_BAD_ARG.  gate, up, y: [n]; y may be gate or up.
 */
enum { ET_GELU_ERF = 0, ET_GELU_TANH = 1 };
et_status et_geglu_f32(const float* gate, const float* up, float* y, int64_t n,
                       int approximate, void* stream);
et_status et_geglu_bf16(const et_bf16* gate, const et_bf16* up, et_bf16* y,
                        int64_t n, int approximate, void* stream);
et_status et_geglu_f16(const et_f16* gate, const et_f16* up, et_f16* y,
                       int64_t n, int approximate, void* stream);

/* ------------------------------------------------------------------------
 * Softmax over the last axis with a temperature  ([OPS] 4 Activation /
 * Softmax, 8 Sampling / Temperature; [DNN] 7)
 *   y[r, i] = exp(z_i - m) / sum_j exp(z_j - m) with z = x[r, :] / temperature
 *   and m = max_j z_j, in f32.  x, y: [rows, n]; y may be x (in place).
 *   temperature must be finite and > 0, else ET_ERR_BAD_ARG.  n <= INT32_MAX.
 *   Special values follow the formula: a NaN anywhere in a row, or a row
 *   whose largest z is +-inf, gives a row of NaN.
 *   workspace: device scratch for rows longer than 32768 elements, which are
 *   then split over several workgroups in one launch (each element read
 *   once; rows of more than 1024 chunks of 8192 elements, over 8388608
 *   elements, in two launches, read twice).  Either workspace == NULL with
 *   workspace_bytes == 0 (one workgroup
 *   per long row, reading the row three times), or workspace != NULL,
 *   16-byte aligned, with workspace_bytes >= et_softmax_workspace_bytes(rows,
 *   n) (0 for rows of at most 32768 elements), else ET_ERR_WORKSPACE.  The
 *   caller owns the workspace.  It must be zero-filled before its first use;
 *   every call leaves its counters zero again, so it can be reused as is.
 *   Calls that share a workspace must not run concurrently.  The result is
 *   the same with or without a workspace.
 */
size_t et_softmax_workspace_bytes(int64_t rows, int64_t n);
/*   Precision: statistics in f32 (z = x * (1/t), the exponentials by the
 *   hardware exp2 of (z - m) log2 e).  That exp2 returns no subnormals, so a
 *   probability below 2^-126 (about 1.2e-38) may be returned as 0 where the
 *   exact value is a subnormal f32; no other result is affected.  Entries
 *   of -inf get exactly 0 whenever the row max is finite, however many of
 *   them there are and wherever they lie.
 *   In place (y == x) with a workspace, rows longer than 32768 elements take
 *   two launches (each element read twice), so that no workgroup reads a
 *   part of the row another one is already writing. */
et_status et_softmax_f32(const float* x, float* y, int64_t rows, int64_t n,
                         float temperature, void* workspace,
                         size_t workspace_bytes, void* stream);
et_status et_softmax_bf16(const et_bf16* x, et_bf16* y, int64_t rows,
                          int64_t n, float temperature, void* workspace,
                          size_t workspace_bytes, void* stream);
et_status et_softmax_f16(const et_f16* x, et_f16* y, int64_t rows,
                         int64_t n, float temperature, void* workspace,
                         size_t workspace_bytes, void* stream);

/* The softmax entry points with the chunk exchange's bounded wait given
 * explicitly: storage is ET_STORAGE_F32, _BF16 or _F16 (x and y of that
 * type), spin_limit the polls per thread, 0..65536 (the entry points above
 * use 8192), else ET_ERR_BAD_ARG; every other argument as above.  A
 * workgroup that runs out of polls computes its row's statistics itself,
 * with the same bits, so any limit gives the same result; 0 forces that
 * path in every workgroup.  For tests of the fallback, driven from the
 * host: no kernel waits without bound either way. */
et_status et_softmax_wait_limit(int storage, const void* x, void* y,
                                int64_t rows, int64_t n, float temperature,
                                void* workspace, size_t workspace_bytes,
                                int spin_limit, void* stream);

/* ------------------------------------------------------------------------
 * Library information. */
const char* et_status_string(et_status s); /* static string, never NULL */
int et_abi_version(void);                  /* ET_ABI_VERSION of the build */

#ifdef __cplusplus
}
#endif
#endif /* ET_H */
