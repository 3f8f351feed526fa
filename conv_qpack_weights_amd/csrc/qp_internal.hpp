// qp_internal.hpp -- helpers shared by the library's translation units:
// error recording, the packed-blob header layout, integer helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/qpack.h"

namespace qp {

// ---- error recording (thread-local message behind qp_last_error) ----------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define QP_FAIL(code, ...)     \
  do {                         \
    ::qp::set_error(__VA_ARGS__); \
    return (code);             \
  } while (0)

#define QP_REQUIRE(cond, code, ...) \
  do {                              \
    if (!(cond)) QP_FAIL(code, __VA_ARGS__); \
  } while (0)

// Returns QP_EHIP with the runtime's message if the last launch failed.
qp_status check_launch(const char* what);

// ---- packed blob header (little endian, 256 bytes) ------------------------
constexpr uint32_t kMagic = 0x4B505149u;  // "IQPK"
constexpr uint32_t kVersion = 1u;
constexpr int64_t kHeaderBytes = 256;
constexpr int64_t kRegionAlign = 256;
constexpr int64_t kPadN = 64;       // Npad multiple
constexpr int64_t kPadK8 = 64;      // int8 Kpad multiple (one MFMA K-step)
constexpr int64_t kRunK4 = 32;      // int4: a 32-K group run
constexpr int64_t kBlockK4 = 128;   // int4: 128 K (64 bytes) interleaved per block
constexpr int kInvalidFlagOffset = 108;

struct alignas(16) BlobHeader {
  uint32_t magic, version, format, scheme;
  int64_t N, K, Npad, Kpad, group;
  int64_t data_off, data_bytes, scale_off, sum_off, zp_off, total_bytes;
  int32_t has_zp;
  int32_t invalid_values;
  // int8 (format 1): extremes of the per-channel weight scales, so that a
  // blob restored from its bytes validates requantization multipliers and
  // picks the epilogue exactly as the freshly packed one does.  0 elsewhere.
  float scale_min, scale_max;
  uint8_t zero[256 - 120];
};
static_assert(sizeof(BlobHeader) == 256, "header is 256 bytes");

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// The blob geometry for a given format; shared by the size query, the packer
// and qp_packed_info_from_header.
qp_status blob_geometry(int32_t format, int32_t scheme, int64_t N, int64_t K, int64_t group,
                        qp_packed_info* info);

// ---- entry points shared between translation units ------------------------
// perm: write each row permuted inside 128-K blocks (the A8W4 GEMM operand
// order; needs kfill % 128 == 0 and 16-byte aligned rows).
qp_status launch_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               int64_t ldq, int64_t kfill, float* row_scale, int32_t* row_zp,
                               bool perm, hipStream_t stream);
// Per-block (32 K) dynamic quantization: q [M][ldq] up to kpad (zeros past
// K), scale / zp [M][ldsz] for kpad/32 blocks (blocks past K: 1 and 0).
qp_status launch_quantize_blocks32(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                   int64_t ldq, int64_t kpad, float* scale, int32_t* zp,
                                   int64_t ldsz, hipStream_t stream);
qp_status conv_out_dims(int64_t H, int64_t W, int32_t KH, int32_t KW, int32_t sh, int32_t sw,
                        int32_t pt, int32_t pl, int32_t pb, int32_t pr, int32_t dh, int32_t dw,
                        int64_t* OH, int64_t* OW);
qp_status launch_im2col(const int8_t* X, int64_t NB, int64_t H, int64_t W, int64_t C,
                        int32_t pad_value, int32_t KH, int32_t KW, int32_t sh, int32_t sw,
                        int32_t pt, int32_t pl, int32_t dh, int32_t dw, int64_t OH, int64_t OW,
                        int8_t* col, int64_t ldcol, hipStream_t stream);
// Implicit-GEMM convolution (the im2col gather inside the operand loads).
// Needs C % 16 == 0, a 16-byte aligned X of fewer than 2^31 bytes and
// K*65025 + max|bias| within int32 (checked by the caller).
struct ConvShape {
  int64_t NB, H, W, C, OH, OW;
  int32_t KH, KW, sh, sw, pt, pl, dh, dw;
};
qp_status launch_conv_implicit(const int8_t* X, const ConvShape& cs, float sA, int32_t zA,
                               const qp_packed_info* w, const void* packedW,
                               const int32_t* bias, float sOut, int32_t zp_out, bool out32,
                               int32_t relu, void* Y, hipStream_t stream);
// The same gather with channel-blocked weights (a block-quantized int8 blob
// packed from OIHW weights) and f32 output.
qp_status launch_conv_implicit_blk(const int8_t* X, const ConvShape& cs, float sx, int32_t zx,
                                   const qp_packed_info* w, const void* packedW,
                                   const float* bias, float lo, float hi, float* Y,
                                   hipStream_t stream);
qp_status validate_gemm(const qp_packed_info* b, int64_t K, float sA, int32_t zA,
                        const int32_t* bias, int64_t max_abs_bias, const qp_qtensor* out,
                        bool* out32);
// f32 output of the INT8 GEMM: y = clamp(sA*sB[n]*acc + bias[n], lo, hi).
struct GemmF32Out {
  const float* bias;  // device f32 [N] or null
  float lo, hi;
};
qp_status run_gemm_s8(const int8_t* A, int64_t M, int64_t lda, float sA, int32_t zA,
                      const qp_packed_info* b, const void* packedB, const int32_t* bias,
                      float sOut, int32_t zp_out, bool out32, int32_t relu, void* C, int64_t ldc,
                      void* ws, size_t ws_bytes, bool a_is_padded, hipStream_t stream,
                      const GemmF32Out* f32 = nullptr);

}  // namespace qp
