/*
 * oracle.h -- plain, slow, scalar C reference for the quantized integer
 * matmul path.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may call it; the product library never
 * does, and this code shares nothing with the GPU library (no headers, no
 * helpers, no tables).
 *
 * Pages the definitions come from (cited by title and section):
 *   [NPU]    "Quantized GEMM: numeric contract, SRAM, DMA and result
 *            verification" (teaching-NPU case study), sections 1-6.
 *   [MNN]    MNN source page "ConvInt8TiledExecutor.cpp" (functions named
 *            where cited).
 *   [TRACT]  tract-linalg 0.23.9 source page "frame/pack.rs" (items named).
 *   [KLEIDI] pytorch/ao PR #997 "Kleidi 4b blockwise gemv prototype".
 *
 * Conventions: every integer sum is formed in int64; every function returns 0
 * on success and a negative value on a violated precondition.  Floating point
 * follows the pages' precision where they fix it (the dynamic quantizer is an
 * f32 op sequence) and is fp64 elsewhere.  Build with -O2 -ffp-contract=off
 * and without fast-math.
 */
#ifndef QPACK_ORACLE_H
#define QPACK_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- O1: integer affine GEMM ------------------------------------------- */
int64_t orc_int32_bound(int64_t K, int64_t max_abs_bias);
int orc_gemm_affine(int64_t M, int64_t N, int64_t K,
                    const int8_t* A, int64_t a_sm, int64_t a_sk, int32_t zA,
                    const int8_t* B, int64_t b_sk, int64_t b_sn, const int32_t* zB,
                    const int32_t* bias, int64_t* acc);
int orc_gemm_affine_points(int64_t npts, const int64_t* ms, const int64_t* ns, int64_t K,
                           const int8_t* A, int64_t a_sm, int64_t a_sk, int32_t zA,
                           const int8_t* B, int64_t b_sk, int64_t b_sn, const int32_t* zB,
                           const int32_t* bias, int64_t* acc);

/* ---- O5b / O6d: per-block activation quantization ------------------------ */
void orc_quantize_rows_s8_blocked(int64_t M, int64_t K, int64_t block, const float* X,
                                  int64_t ldx, int8_t* Q, int64_t ldq, float* scale,
                                  int32_t* zp, int64_t ldsz);
int orc_a8w4_blockwise_blockq(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                              int64_t lda, const float* sa, const int32_t* za, int64_t ldsz,
                              const int8_t* qw, int64_t ldw, const float* sw, int64_t ldsw,
                              const float* bias, float clamp_lo, float clamp_hi, float* Y,
                              int64_t ldy);

/* ---- O6c: asymmetric int4 (scale and offset per group) ------------------- */
int orc_a8w4_blockwise_asym(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                            int64_t lda, const float* sa, const int32_t* za, const int8_t* qw,
                            int64_t ldw, const float* sw, const float* bw, int64_t ldsw,
                            const float* bias, float clamp_lo, float clamp_hi, float* Y,
                            int64_t ldy);

/* ---- O6b: bf16 rounding of group scales ----------------------------------- */
float orc_round_bf16(float x);
void orc_round_bf16_array(int64_t n, const float* x, float* y);

/* ---- O8: f32 output of the INT8 GEMM ------------------------------------- */
int orc_dequant_matrix_f32(int64_t M, int64_t N, const int64_t* acc, float s_a,
                           const float* s_b, const float* bias, float lo, float hi, float* Y);

/* ---- O2: tiled model --------------------------------------------------- */
typedef struct {
  int64_t tiles_m, tiles_n, tiles_k, tiles;
  int64_t effective_mac, physical_slots;
  double shape_efficiency;
} orc_tile_stats;
typedef struct {
  int64_t s_input, s_acc, s_reserve, s_total;
} orc_tile_budget;
void orc_tile_budget_of(int64_t Tm, int64_t Tn, int64_t Tk, int64_t in_elem_bytes,
                        int64_t acc_elem_bytes, int64_t reserve, orc_tile_budget* out);
int orc_gemm_tiled(int64_t M, int64_t N, int64_t K,
                   const int8_t* A, int64_t a_sm, int64_t a_sk, int32_t zA,
                   const int8_t* B, int64_t b_sk, int64_t b_sn, const int32_t* zB,
                   const int32_t* bias, int64_t Tm, int64_t Tn, int64_t Tk,
                   int64_t* acc, orc_tile_stats* st);

/* ---- O3: integer multiplier/shift requantization ------------------------ */
double orc_real_multiplier(float s_a, float s_b, float s_out);
int orc_requant_params(double real_multiplier, int32_t* m0, int32_t* shift);
int64_t orc_rshift_rhe(int64_t t, int32_t shift);
int32_t orc_requant_value(int64_t acc, int32_t m0, int32_t shift, int32_t zp_out,
                          int32_t lo, int32_t hi);
int64_t orc_ideal_rhe(int64_t acc, double real_multiplier);
int orc_requant_matrix(int64_t M, int64_t N, const int64_t* acc, float s_a,
                       const float* s_b, float s_out, int32_t zp_out, int32_t relu,
                       int8_t* out, int64_t* n_differs_from_ideal);

/* ---- O4: convolution --------------------------------------------------- */
int orc_conv2d_direct(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X,
                      int32_t zp_in, int64_t OC, int64_t KH, int64_t KW, const int8_t* Wt,
                      int64_t stride_h, int64_t stride_w, int64_t pad_t, int64_t pad_l,
                      int64_t pad_b, int64_t pad_r, int64_t dil_h, int64_t dil_w,
                      const int32_t* bias, int64_t* acc);
int orc_im2col(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X, int32_t pad_value,
               int64_t KH, int64_t KW, int64_t stride_h, int64_t stride_w, int64_t pad_t,
               int64_t pad_l, int64_t pad_b, int64_t pad_r, int64_t dil_h, int64_t dil_w,
               int8_t* col);

int orc_conv2d_blockwise_f32(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X,
                             int32_t zx, float sx, int64_t OC, int64_t KH, int64_t KW,
                             const int8_t* Wt, int64_t stride_h, int64_t stride_w, int64_t pad_t,
                             int64_t pad_l, int64_t pad_b, int64_t pad_r, int64_t dil_h,
                             int64_t dil_w, int64_t icb, const float* sw, const float* bias,
                             float lo, float hi, float* Y);

/* ---- O5: dynamic per-row asymmetric int8 quantization (f32) ------------- */
void orc_quantize_row_s8(const float* x, int64_t K, int8_t* q, float* scale, int32_t* zp);
void orc_quantize_row_s8_sym(const float* x, int64_t K, int8_t* q, float* scale);
void orc_quantize_rows_s8_sym(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q,
                              int64_t ldq, float* scale);
void orc_quantize_rows_s8(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q,
                          int64_t ldq, float* scale, int32_t* zp);

/* ---- O6: A8W4 blockwise matmul with f32 dequantize + clamp --------------- */
int orc_a8w4_blockwise(int64_t M, int64_t N, int64_t K, int64_t group,
                       const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                       const int8_t* qw, int64_t ldw, const float* sw, int64_t ldsw,
                       const float* bias, float clamp_lo, float clamp_hi,
                       float* Y, int64_t ldy);

/* ---- O7: reference writer of the library's packed-weight blob ------------ */
int64_t orc_packed_s8_bytes(int64_t N, int64_t K);
int orc_pack_s8_ref(int64_t N, int64_t K, const int8_t* Wt, int64_t w_sn, int64_t w_sk,
                    int32_t per_channel, const float* scales, const int32_t* zps,
                    uint8_t* blob);
int64_t orc_packed_s4_bytes(int64_t N, int64_t K, int64_t group);
int orc_pack_s4_ref(int64_t N, int64_t K, int64_t group, const int8_t* Wt, int64_t w_sn,
                    int64_t w_sk, const float* sw, int64_t ldsw, uint8_t* blob);

#ifdef __cplusplus
}
#endif
#endif
