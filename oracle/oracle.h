/*
 * oracle.h -- plain, slow CPU reference for the memory-bound transformer ops.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no source with the HIP kernels.
 *
 * Conventions
 *   dt      storage type of every tensor argument: ORC_F32 (float),
 *           ORC_BF16 (uint16_t holding bfloat16 bits) or ORC_F16 (uint16_t
 *           holding IEEE binary16 bits).
 *   y64     optional (may be NULL) f64 buffer receiving the unrounded result
 *           of each output element; tolerance checks use it.
 *   All arithmetic is IEEE f64 (libm sqrt/exp/sin/cos); inputs are widened
 *   exactly; each stored output is rounded once, round-to-nearest-even.
 */
#ifndef ET_ORACLE_H
#define ET_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };

/* Threads used by the row/element loops (OpenMP); <= 0 leaves the default. */
void     orc_set_threads(int n);
int      orc_get_threads(void);

/* f64 -> bfloat16 bits, one round-to-nearest-even (no pass through f32). */
uint16_t orc_bf16_from_f64(double v);
/* f64 -> IEEE binary16 bits, one round-to-nearest-even. */
uint16_t orc_f16_from_f64(double v);
/* The storage rounding (as every op stores) of n f64 values into out. */
void     orc_round_to(int dt, const double* v, int64_t n, void* out);
/* The RoPE angle of position p and frequency w: the f64 product rounded once
 * to f32. */
float    orc_rope_angle(int32_t p, float w);

void orc_rmsnorm(int dt, const void* x, const void* w, int64_t rows, int64_t d,
                 float eps, double* y64, void* y);
void orc_add_rmsnorm(int dt, const void* x, const void* res, const void* w,
                     int64_t rows, int64_t d, float eps, double* y64, void* y,
                     void* h);
void orc_rope(int dt, void* x, const int32_t* pos, int64_t T, int64_t H,
              int64_t D, int64_t r, const float* inv_freq, float mu,
              int layout, double* y64);
void orc_rmsnorm_rope(int dt, void* x, const void* g, float eps,
                      const int32_t* pos, int64_t T, int64_t H, int64_t D,
                      int64_t r, const float* inv_freq, float mu, int layout,
                      double* y64);
void orc_silu_mul(int dt, const void* gate, const void* up, int64_t n,
                  double* y64, void* y);
void orc_add(int dt, const void* a, const void* b, int64_t n, void* y);
void orc_embedding(int dt, const void* table, int64_t V, const int32_t* ids,
                   int64_t n, int64_t d, void* out);
void orc_argmax(int dt, const void* x, int64_t rows, int64_t n, int32_t* out);
void orc_softmax(int dt, const void* x, int64_t rows, int64_t n, float t,
                 double* y64, void* y);
void orc_layernorm(int dt, const void* x, const void* g, const void* b,
                   int64_t rows, int64_t d, float eps, double* y64, void* y);
void orc_geglu(int dt, const void* gate, const void* up, int64_t n, int form,
               double* y64, void* y);
void orc_rope_cache(const float* inv_freq, int64_t max_pos, int64_t r,
                    float* cos_c, float* sin_c);
void orc_rope_cached(int dt, void* x, const int32_t* pos, int64_t T,
                     int64_t H, int64_t D, int64_t r, const float* cos_c,
                     const float* sin_c, int64_t max_pos, float mu_f,
                     int layout, double* y64);

void orc_rope_multi(int dt, void* x, const int32_t* pos, int64_t T,
                    int64_t H, int64_t D, int64_t A, const int64_t* dims,
                    const float* inv_freq, float mu_f, int layout,
                    double* y64);

#ifdef __cplusplus
}
#endif
#endif
