/*
 * qpack.h -- C ABI of the MI355X (gfx950) quantized integer matmul library.
 *
 * The operations and their numeric contract come from these pages (cited by
 * title and section):
 *   [NPU]    "Quantized GEMM: numeric contract, SRAM, DMA and result
 *            verification" (teaching-NPU case study), sections 1-5.
 *   [MNN]    MNN "ConvInt8TiledExecutor.cpp" (functions named where cited).
 *   [TRACT]  tract-linalg 0.23.9 "frame/pack.rs" (items named where cited).
 *   [KLEIDI] pytorch/ao PR #997 "Kleidi 4b blockwise gemv prototype".
 *
 * General rules for every entry point:
 *   - Pointers named *_dev, and every tensor data pointer, are DEVICE
 *     pointers; descriptor structs and qp_packed_info are HOST memory.
 *   - The caller owns and allocates every buffer (inputs, packed blob,
 *     workspace, outputs); the library never allocates device memory.
 *   - All work is enqueued asynchronously on `stream` (0 = the null stream)
 *     except where a function says it synchronizes.
 *   - Arguments are validated on the host before any launch; a failure
 *     returns a negative qp_status, launches nothing and records a message
 *     readable with qp_last_error().  Nothing aborts or throws across the ABI.
 *   - Strides are in ELEMENTS, never bytes ([NPU] section 5 warns against
 *     mixing the two).  Logical shape and physical stride are separate
 *     ([NPU] section 2: logical N=70 may sit in a 128-byte physical row).
 */
#ifndef QPACK_H
#define QPACK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QP_OK = 0,
  QP_EINVAL = -1,        /* malformed descriptor or argument              */
  QP_EUNSUPPORTED = -2,  /* well-formed but outside what is implemented   */
  QP_EOVERFLOW = -3,     /* K*65025 + max|bias| does not fit INT32        */
  QP_ESIZE = -4,         /* a caller buffer is too small                  */
  QP_EALIGN = -5,        /* a pointer or stride breaks a stated alignment */
  QP_EHIP = -6           /* the HIP runtime reported an error             */
} qp_status;

typedef enum { QP_S8 = 1, QP_S4 = 2, QP_S32 = 3, QP_F32 = 4 } qp_dtype;

typedef enum {
  QP_PER_TENSOR = 0,
  QP_PER_CHANNEL = 1,
  QP_BLOCKWISE = 2,
  QP_DYNAMIC_PER_ROW = 3,
  /* blockwise int4 whose f32 group scales are stored rounded to bf16
   * (nearest, ties to even), as the KleidiAI kernel keeps them ([KLEIDI]
   * review of the wrapper's scale conversion); blob format 3 */
  QP_BLOCKWISE_BF16 = 4,
  /* asymmetric blockwise int4: `scales` holds f32 (offset, scale) pairs
   * [N][ceil(K/group)][2], real weight = scale*q + offset, the pair order of
   * [MNN] _computeReorderQuantInfo's quantization info; blob format 4 */
  QP_BLOCKWISE_ASYM = 5
} qp_qscheme;

typedef enum { QP_ROUND_HALF_EVEN = 0 } qp_rounding;

/*
 * Quantized tensor descriptor -- the fields [NPU] section 1 asks every tensor
 * to record: dtype, scale, zero point, quantization axis, rounding and
 * saturation range; plus the logical shape and physical strides of
 * [NPU] section 2.
 *   real = scale * (q - zero_point)
 *   dtype        qp_dtype of the stored values.  QP_S4 weights are given one
 *                value per int8 byte, each in [-8, 7].
 *   rank/shape   logical shape (rank 1..4).
 *   stride       physical strides in elements, one per dimension.
 *   scheme       qp_qscheme.
 *   axis         the channel axis of a per-channel scheme (the N axis).
 *   group_size   blockwise: consecutive K values sharing one scale.
 *   scale        per-tensor scale (host value).
 *   scales       per-channel f32 [N] or blockwise f32 [N][ceil(K/group)]
 *                scales, DEVICE pointer (NULL for per-tensor).
 *   zero_point   per-tensor zero point (host value).
 *   zero_points  per-channel int32 [N] zero points, DEVICE pointer, or NULL.
 *   qmin, qmax   saturation range; int8 outputs support [-128, 127] only
 *                (the symmetric [-127,127] is a different convention that
 *                must not be mixed in silently, [NPU] section 1).
 *   rounding     qp_rounding; only QP_ROUND_HALF_EVEN is implemented.
 */
typedef struct {
  int32_t dtype;
  int32_t rank;
  int64_t shape[4];
  int64_t stride[4];
  int32_t scheme;
  int32_t axis;
  int32_t group_size;
  float scale;
  const float* scales;
  int32_t zero_point;
  const int32_t* zero_points;
  int32_t qmin;
  int32_t qmax;
  int32_t rounding;
} qp_qtensor;

/*
 * Host-side description of a packed weight blob, filled by qpack_weights and
 * passed back to the compute entry points (so that no launch needs to read
 * the device header first).  The same fields open the blob itself as a
 * 256-byte little-endian header, so a saved blob describes itself; see
 * qp_packed_info_from_header.
 *   format       1 = int8 panels, 2 = int4 nibbles with group scales.
 *   scheme       qp_qscheme of the weight scales.
 *   N, K         logical output channels and reduction length.
 *   Npad, Kpad   padded extents: Npad = roundup(N, 64);
 *                Kpad = roundup(K, 64) for int8, roundup(K, max(group, 128))
 *                for int4.
 *   group        int4 group size (32, 64, 128 or a multiple of 128); 0 for
 *                int8.
 *   *_off        byte offsets of the regions inside the blob.
 *   total_bytes  blob size.
 *   has_zero_points  int8: some weight zero point is non-zero.
 *   scale_min/max    int8: extremes of the weight scales (validation).
 */
typedef struct {
  int32_t format;
  int32_t scheme;
  int64_t N, K, Npad, Kpad, group;
  int64_t data_off, data_bytes, scale_off, sum_off, zp_off, total_bytes;
  int32_t has_zero_points;
  float scale_min, scale_max;
} qp_packed_info;

/* Library version string and the message of the last failed call on this
 * host thread ("" if none). */
const char* qp_version(void);
const char* qp_last_error(void);

/*
 * qpack_weights_size -- bytes and alignment of the blob qpack_weights writes
 * for weights `w`.  Follows [TRACT] PackedFormat::len / PackedI8K4::len: the
 * size is a function of (N, K) and the format only.
 *   w       rank 2 with (k_axis, n_axis) a permutation of (0,1), or rank 4
 *           OIHW convolution weights with n_axis = 0, k_axis = 1 (then
 *           K = KH*KW*IC in (kh, kw, ic) order, the order of [MNN]
 *           reorderWeight).  dtype QP_S8 (per-tensor or per-channel) or
 *           QP_S4 (QP_BLOCKWISE, group_size a multiple of 32, K <= 65536
 *           after padding, else QP_EUNSUPPORTED; a restored int4 header is
 *           held to the same limit).
 *   bytes   out: blob size.      align  out: required alignment (256).
 */
qp_status qpack_weights_size(const qp_qtensor* w, int32_t k_axis, int32_t n_axis,
                             size_t* bytes, size_t* align);

/*
 * qpack_weights -- one-time weight pre-pack into the blob the GEMM kernels
 * read ([MNN] reorderWeight / packWeightAndQuantInfo, [TRACT] pack_tensor_view
 * and PackedI8K4::pack_view).
 * int8 blob: 256-byte header; data int8 in 32x32 sub-tiles (32 channels by
 *   32 K, 1 KiB each, row n%32 at byte 32*(n%32), K contiguous): sub-tile
 *   (n/32, k/32) starts at ((n/32)*(Kpad/32) + k/32)*1024, so one 64-lane
 *   16-byte load fills one MFMA weight fragment.  Zero-filled beyond N and
 *   K: the kernels compute on the padding, so it must hold defined values
 *   ([TRACT] pack_tensor_view).  Then f32 scale[Npad]; int32 colsum[Npad] =
 *   sum_{k<K} w[n,k] over the real K (the zero-point correction term,
 *   [MNN] kernel sums); int32 zp[Npad].
 * int4 blob: header; data Npad*Kpad/2 bytes -- each channel's K is cut in
 *   blocks of 128 (64 bytes) and the 16 channels of a tile store each block
 *   side by side: channel n, block b at ((n/16)*(Kpad/128) + b)*1024 +
 *   (n%16)*64.  Byte 16c+4t+j of a block holds k = 32t+8c+j in its low
 *   nibble and k = 32t+8c+4+j in its high nibble (t = group of 32 inside the
 *   block, c = 16-byte chunk), 4-bit two's complement, so one 16-byte chunk
 *   carries the same 8 K of four consecutive groups.  Scales f32 in quads
 *   of four groups with the tile's 16 channels side by side: sw[n][g] at
 *   float ((n/16)*ceil(G/4) + g/4)*64 + (n%16)*4 + g%4, G = Kpad/group
 *   (zero for groups past K).  Format 3 (scheme QP_BLOCKWISE_BF16) stores
 *   the same scale array as bf16, each the given f32 rounded to nearest,
 *   ties to even, at the same element index (2 bytes each).  Format 4
 *   (scheme QP_BLOCKWISE_ASYM) adds, after wsum, the f32 group offsets in
 *   the layout of the scales (zp_off points there);
 *   f32 wsum[Npad] = sum_g sw[n,g] * sum_{k in g} w[n,k] (with the stored
 *   scales; format 4 adds offset[n,g] * (real K in g): the sum of the real
 *   weights), accumulated in fp64
 *   (the weight kernel sum that folds the activation zero point,
 *   [MNN] _computeReorderQuantInfo / BatchAsyDynamicQuant).
 * block-quantized int8 blob (format 5, QP_S8 with QP_BLOCKWISE, group 64 or
 *   128): the int8 sub-tiles of format 1 with Kpad = roundup(K, 128), then
 *   f32 scale[Kpad/group][Npad] (block-major; zero past K and N) and f32 wsum[Npad] =
 *   sum_b scale[n,b] * sum_{k in b} w[n,k] (fp64); no zero points.  Rank-2
 *   weights give scales [N][ceil(K/group)], one per K block; OIHW weights
 *   give [OC][IC/group], one per block of input channels, stored repeated
 *   for every kernel tap (group must divide IC).
 * All padding bytes are zero.  int4 values outside [-8,7] set the header word
 * at byte 108 to non-zero (it is 0 for valid input).
 *   w_dev        device weights laid out as w->shape / w->stride.
 *   packed_dev   device blob, >= qpack_weights_size bytes, 256-byte aligned.
 *   info         out (host): the blob description.
 * Synchronizes `stream` once (copies the per-channel scales and zero points
 * to the host to validate them); it is a load-time call, not a hot-path one.
 */
qp_status qpack_weights(const qp_qtensor* w, const void* w_dev, int32_t k_axis, int32_t n_axis,
                        void* packed_dev, size_t packed_bytes, qp_packed_info* info,
                        hipStream_t stream);

/*
 * qrepack_weights -- refill an existing packed blob in place with new weights
 * of the same shape and format ([TRACT] PackedFormat::new_packed_buffer /
 * repack_tensor_view: an operand that changes between calls but keeps its
 * shape reuses its packed buffer instead of reallocating one).
 *   w, w_dev, k_axis, n_axis  as for qpack_weights.
 *   packed_dev   the blob `info` describes (at least info->total_bytes,
 *                256-byte aligned); its old contents are overwritten.
 *   info         in: the description of that blob (from qpack_weights or
 *                qp_packed_info_from_header); out: the refilled blob's
 *                description (zero points and scale extremes may change).
 * Fails with QP_EINVAL, leaving buffer and `info` untouched, unless the new
 * weights give the same format, scheme, N, K, group and region layout as
 * `info`.  Same synchronization as qpack_weights.  The caller must not use
 * the blob on another stream while it is being refilled.
 */
qp_status qrepack_weights(const qp_qtensor* w, const void* w_dev, int32_t k_axis, int32_t n_axis,
                          void* packed_dev, qp_packed_info* info, hipStream_t stream);

/* Parse a blob header copied to host memory (256 bytes) into `info`. */
qp_status qp_packed_info_from_header(const void* header_host, qp_packed_info* info);

/*
 * qunpack_weights -- logical weights of channels [n_begin, n_begin+n_count)
 * read back out of a blob ([TRACT] PackedFormat::extract_at_mn_f32: one
 * M/N row's K values taken out of the packed panels, optionally as floats).
 * For inspection and for checking a blob restored from bytes.
 *   w_out      int8 [n_count][ldw] (ldw >= K): the logical values (int4
 *              blobs: [-8, 7]); NULL to skip.
 *   scales_out int8 blob: f32 [n_count]; int4 blob: f32 [n_count][lds]
 *              (lds >= ceil(K/group)); asymmetric int4 (format 4): the
 *              (offset, scale) pairs, lds >= 2*ceil(K/group); NULL to skip.
 *   zp_out     int8 blob: int32 [n_count] (zeros when symmetric); must be
 *              NULL for int4 blobs.
 *   deq_out    f32 [n_count][ldd] (ldd >= K): sB[n]*(q - zB[n]) for int8,
 *              sw[n, k/group]*q for int4, one f32 rounding (format 4: then
 *              plus the group offset, a second rounding); NULL to skip.
 * Padding (K..Kpad, N..Npad) is never written.  Asynchronous on `stream`.
 */
qp_status qunpack_weights(const qp_packed_info* info, const void* packed_dev, int64_t n_begin,
                          int64_t n_count, int8_t* w_out, int64_t ldw, float* scales_out,
                          int64_t lds, int32_t* zp_out, float* deq_out, int64_t ldd,
                          hipStream_t stream);

/*
 * qquantize_rows_s8 -- dynamic per-row asymmetric int8 quantization of f32
 * activations ([MNN] BatchAsyDynamicQuant; the [KLEIDI] "qai8dx" format).
 * Per row, as one f32 sequence (round half to even, no contraction):
 *   rmin = min(0, min x); rmax = max(0, max x); scale = (rmax - rmin)/255
 *   (an all-zero row gives scale 1, zero point 0);
 *   zp = clamp(rint(-128 - rmin/scale), -128, 127);
 *   q  = clamp(rint(x/scale) + zp, -128, 127).
 *   x          device f32 [M][ldx];   q  device int8 [M][ldq] (ldq >= K).
 *   row_scale  device f32 [M];        row_zp  device int32 [M].
 * Inputs must be finite.
 */
qp_status qquantize_rows_s8(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                            int64_t ldq, float* row_scale, int32_t* row_zp, hipStream_t stream);

/*
 * qquantize_rows_s8_sym -- dynamic per-row symmetric int8 quantization
 * ([MNN] BatchSymDynamicQuant: largest magnitude per row, a scale from it,
 * zero point 0; the page does not print the helpers' arithmetic).  Per row,
 * f32, round half to even, no contraction:
 *   amax = max |x|; scale = amax / 127 (an all-zero row gives scale 1);
 *   q = clamp(rint(x/scale), -127, 127).
 *   x  device f32 [M][ldx];  q  device int8 [M][ldq] (ldq >= K);
 *   row_scale  device f32 [M].  The zero point is 0 for every row.
 * Inputs must be finite.
 */
qp_status qquantize_rows_s8_sym(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                int64_t ldq, float* row_scale, hipStream_t stream);

/*
 * qquantize_rows_s8_blocked -- the dynamic quantization of qquantize_rows_s8
 * applied to every block of `block` consecutive K of every row on its own
 * ([MNN] DenseConvInt8TiledExecutor::onResize: with dynamicQuantOption 2 the
 * input is cut into the weights' K blocks, mInputBlockNum = mBlockNum, and
 * BatchAsyDynamicQuant gives each block a scale and zero point).
 *   block    32 only (the int4 group size).
 *   kpad     >= K, a multiple of 32: q is written for k < kpad (zeros past
 *            K); parameters for kpad/32 blocks (blocks wholly past K get
 *            scale 1, zero point 0).
 *   q        device int8 [M][ldq], ldq >= kpad.
 *   scale, zp  device f32 / int32 [M][ldsz], ldsz >= kpad/32.
 */
qp_status qquantize_rows_s8_blocked(const float* x, int64_t M, int64_t K, int64_t ldx,
                                    int64_t block, int64_t kpad, int8_t* q, int64_t ldq,
                                    float* scale, int32_t* zp, int64_t ldsz, hipStream_t stream);

/*
 * qgemm_s8s8_requant -- C = requant(A x B + bias), INT8 affine operands
 * ([NPU] sections 1-5; [MNN] tileSplitFunction's post-treat parameters).
 *   acc[m,n] = sum_{k<K} (A[m,k]-zA)(B[k,n]-zB[n]) + bias[n]   (exact INT32,
 *              one accumulator over all of K)
 *   out int8:  C = clamp(RHE(acc*m0[n] / 2^shift[n]) + zp_out, lo, 127),
 *              lo = zp_out with relu, else -128; (m0, shift) from
 *              M_n = sA*sB[n]/s_out: M_n = f*2^e, f in [0.5,1),
 *              m0 = nearest-even(f*2^31) (2^31 -> 2^30 with e+1),
 *              shift = 31-e.
 *   out int32: C = acc (the raw accumulator after zero-point correction
 *              and bias; no requantization).
 *   a        QP_S8 [M,K], stride (lda, 1), per-tensor scale and zero point.
 *   b, packedB_dev  an int8 blob from qpack_weights (K must match).
 *   bias_dev int32 [N] at accumulator scale sA*sB[n], or NULL.
 *   out      QP_S8 or QP_S32 [M,N], stride (ldc, 1); scale/zero_point used
 *            for int8; qmin/qmax must be -128/127 for int8.
 *   ws, ws_bytes  device workspace of qgemm_s8s8_requant_ws_size bytes
 *            (may be 0: then ws may be NULL).  The size is 0 for GEMMs on
 *            64x64 tiles (fewer than 256 tiles of 128x128) with Kpad <= 960:
 *            their activations are read byte-exact at any stride and
 *            alignment.  Other GEMMs need it when K != Kpad, when the rows
 *            are not 16-byte aligned, or when the weights carry zero points
 *            (a padded copy of A and/or its row sums).
 *   max_abs_bias  host upper bound of |bias[n]| (>= 0; ignored when
 *            bias_dev is NULL).  The bias lives on the device, so the INT32
 *            check of [NPU] section 4 uses this bound: K*65025 + max_abs_bias
 *            must be <= 2^31-1, else QP_EOVERFLOW.  A false bound voids the
 *            exactness guarantee.
 * Errors: QP_EOVERFLOW as above; QP_EUNSUPPORTED when some m0/shift cannot
 *   be formed (multiplier >= 2^31, or not positive and finite).
 */
qp_status qgemm_s8s8_requant_ws_size(const qp_qtensor* a, const qp_packed_info* b,
                                     size_t* bytes);
qp_status qgemm_s8s8_requant(const qp_qtensor* a, const int8_t* A, const qp_packed_info* b,
                             const void* packedB_dev, const int32_t* bias_dev,
                             int64_t max_abs_bias, const qp_qtensor* out, int32_t relu,
                             void* C, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * qgemm_s8s8_dequant_f32 -- Y = clamp(sA*sB[n]*acc + bias[n], lo, hi) in f32
 * ([NPU] sections 1-4 for the exact accumulator; [MNN] tileSplitFunction's
 * post parameters for a float destination: float bias added after the
 * dequantization, then the f32 min/max thresholds, e.g. 0/6 for Relu6).
 *   acc[m,n] = sum_{k<K} (A[m,k]-zA)(B[k,n]-zB[n])   (exact INT32)
 *   y        = fmaf(f32(sA*sB[n]), f32(acc), bias[n]), then clamped.
 *   a        QP_S8 [M,K], stride (lda, 1), per-tensor scale and zero point.
 *   b, packedB_dev  an int8 blob from qpack_weights (K must match).
 *   bias_dev f32 [N] in output units, or NULL (no bias).
 *   clamp_lo, clamp_hi  f32 bounds, lo <= hi (use -FLT_MAX/FLT_MAX or
 *            +-inf for no clamp).
 *   Y        device f32 [M][ldy], ldy >= N.
 *   ws, ws_bytes  workspace sized by qgemm_s8s8_requant_ws_size (same plan).
 * The result is within a few f32 ulps of the exactly rounded value.
 * Errors: QP_EOVERFLOW when K*65025 > 2^31-1; QP_EINVAL on bad shapes,
 *   NaN or reversed bounds.
 */
qp_status qgemm_s8s8_dequant_f32(const qp_qtensor* a, const int8_t* A, const qp_packed_info* b,
                                 const void* packedB_dev, const float* bias_dev, float clamp_lo,
                                 float clamp_hi, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * qgemm_a8w4_blockwise_f32 -- Y = clamp(deq(qa) x deq(W)^T + bias, lo, hi)
 * with dynamically quantized int8 activations and int4 group weights
 * ([KLEIDI] matmul_clamp_f32_qai8dxp_qsi4c32p: f32 out, clamp, per-row int8
 * activations, signed int4 weights in groups of 32, no weight zero points;
 * [MNN] onExecute's KleidiAI path: quantize the rows, then the matmul).
 *   X        device f32 [M][ldx], quantized per row as qquantize_rows_s8.
 *   w, packedW_dev  an int4 blob from qpack_weights (K must match).
 *   bias     device f32 [N] or NULL; added after dequantization, before
 *            the clamp.
 *   Y        device f32 [M][ldy].
 *   ws       device workspace of qgemm_a8w4_blockwise_f32_ws_size bytes.
 * The sum inside a group of 32 is exact int32; the sum over groups is f32.
 */
qp_status qgemm_a8w4_blockwise_f32_ws_size(int64_t M, const qp_packed_info* w, size_t* bytes);
qp_status qgemm_a8w4_blockwise_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                   const qp_packed_info* w, const void* packedW_dev,
                                   const float* bias, float clamp_lo, float clamp_hi, float* Y,
                                   int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * qgemm_a8w4_blockwise_f32_noalloc -- qgemm_a8w4_blockwise_f32 with no
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as
 * qgemm_a8w4_blockwise_f32, whose kernels it runs; it calls no allocator.
 * The quantized activations go to a 4 MiB array in device memory that the
 * library owns, one per GPU, held until the process ends:
 * round_up(M*Kpad, 256) + round_up(8*M, 256) must not exceed 4 MiB (else
 * QP_ESIZE, nothing launched), e.g. M <= 1022 for K = 4096.  Every call on a
 * GPU shares that GPU's array and leaves its contents behind; calls that
 * overlap on one GPU (concurrent streams, several host threads) race on it,
 * so serialize them.  Nothing in it needs clearing: each call rewrites what
 * it reads.
 */
qp_status qgemm_a8w4_blockwise_f32_noalloc(const float* X, int64_t M, int64_t K, int64_t ldx,
                                           const qp_packed_info* w, const void* packedW_dev,
                                           const float* bias, float clamp_lo, float clamp_hi,
                                           float* Y, int64_t ldy, hipStream_t stream);

/*
 * qgemm_a8w4_prequant_f32 -- the same product on activations already
 * quantized by qquantize_rows_s8 (the matmul step alone).
 *   qa       device int8 [M][lda]; lda >= Kpad, 16-byte aligned rows, and
 *            qa[m][k] = 0 for K <= k < Kpad.
 *   sa, za   device f32 [M] / int32 [M] row scales and zero points.
 */
qp_status qgemm_a8w4_prequant_f32(const int8_t* qa, int64_t M, int64_t lda, const float* sa,
                                  const int32_t* za, const qp_packed_info* w,
                                  const void* packedW_dev, const float* bias, float clamp_lo,
                                  float clamp_hi, float* Y, int64_t ldy, hipStream_t stream);

/*
 * qgemm_a8w4_blockq_f32 -- the A8W4 product with the activations quantized
 * per block of 32 K (qquantize_rows_s8_blocked), each block being one int4
 * group, so every group carries its own activation scale and zero point:
 *   Y[m,n] = clamp(sum_g sa[m,g]*sw[n,g] * sum_{k in g} (qa[m,k]-za[m,g])*q[n,k]
 *                  + bias[n], lo, hi)
 *   the sum inside a group exact in int32, across groups f32.
 * Weights: int4 blobs with f32 or bf16 scales (not the asymmetric format).
 *   ws       device workspace of qgemm_a8w4_blockq_f32_ws_size bytes: 0
 *            for one row with Kpad <= 32768 (quantized inside the GEMV's
 *            own launch; ws may then be null).
 * qgemm_a8w4_blockq_prequant_f32 is the matmul step alone:
 *   qa       device int8 [M][lda], lda >= Kpad, a multiple of 16, 16-byte
 *            aligned, zero for K <= k < Kpad.
 *   sa, za   device f32 / int32 [M][ldsz], ldsz >= Kpad/32 and a multiple
 *            of 4, 16-byte aligned; entries past ceil(K/32) must be finite.
 */
qp_status qgemm_a8w4_blockq_f32_ws_size(int64_t M, const qp_packed_info* w, size_t* bytes);
qp_status qgemm_a8w4_blockq_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                const qp_packed_info* w, const void* packedW_dev,
                                const float* bias, float clamp_lo, float clamp_hi, float* Y,
                                int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);
qp_status qgemm_a8w4_blockq_prequant_f32(const int8_t* qa, int64_t M, int64_t lda,
                                         const float* sa, const int32_t* za, int64_t ldsz,
                                         const qp_packed_info* w, const void* packedW_dev,
                                         const float* bias, float clamp_lo, float clamp_hi,
                                         float* Y, int64_t ldy, hipStream_t stream);

/*
 * qgemm_a8w8_blockwise_f32 -- dynamically quantized int8 activations times
 * block-quantized int8 weights (scheme QP_BLOCKWISE on QP_S8 weights, blob
 * format 5: one f32 scale per output channel and block of 64 or 128 K;
 * [MNN] _computeReorderQuantInfo's blockNum > 1), f32 out with bias and clamp:
 *   Y[m,n] = clamp(sa[m] * sum_b sw[n,b] * sum_{k in b} (qa[m,k]-za[m])*q[n,k]
 *                  + bias[n], lo, hi)
 *   exact int32 inside a block, f32 across blocks; the rows quantized as by
 *   qquantize_rows_s8.  For a GEMM (a linear layer, or a 1x1 convolution
 *   whose OIHW weights were packed as K = C).
 *   ws       device workspace of qgemm_a8w8_blockwise_f32_ws_size bytes:
 *            0 for one row with Kpad <= 32768 (quantized inside the
 *            product's own launch; ws may then be null), else the quantized
 *            rows and their parameters.
 * qgemm_a8w8_blockwise_prequant_f32 is the matmul step alone (qa [M][lda],
 * lda >= Kpad and a multiple of 16, zero for K <= k < Kpad; sa, za [M]).
 */
qp_status qgemm_a8w8_blockwise_f32_ws_size(int64_t M, const qp_packed_info* w, size_t* bytes);
qp_status qgemm_a8w8_blockwise_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                   const qp_packed_info* w, const void* packedW_dev,
                                   const float* bias, float clamp_lo, float clamp_hi, float* Y,
                                   int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);
qp_status qgemm_a8w8_blockwise_prequant_f32(const int8_t* qa, int64_t M, int64_t lda,
                                            const float* sa, const int32_t* za,
                                            const qp_packed_info* w, const void* packedW_dev,
                                            const float* bias, float clamp_lo, float clamp_hi,
                                            float* Y, int64_t ldy, hipStream_t stream);

/*
 * qim2col_s8 -- explicit int8 im2col of an NHWC input ([MNN] tileSplitFunction:
 * out-of-image taps take the INPUT zero point so that they stand for real
 * zero; [TRACT] PackedI8K4::write_with_k_outer feeds im2col patches K-outer).
 *   col[m][k], m = (b*OH + oy)*OW + ox, k = (ky*KW + kx)*C + ic, for k < K;
 *   col[m][k] = 0 for K <= k < ldcol.  ldcol % 16 == 0.
 */
qp_status qim2col_s8(const int8_t* X, int64_t NB, int64_t H, int64_t W, int64_t C,
                     int32_t pad_value, int32_t KH, int32_t KW, int32_t stride_h,
                     int32_t stride_w, int32_t pad_t, int32_t pad_l, int32_t pad_b,
                     int32_t pad_r, int8_t* col, int64_t ldcol, hipStream_t stream);

/*
 * qconv2d_s8_im2col -- INT8 NHWC convolution as im2col + the INT8 GEMM with
 * the requantizing (or raw int32) epilogue.  Dilation 1.
 *   x        QP_S8 rank 4 NHWC, contiguous; per-tensor scale, zero point
 *            (the pad value).
 *   w, packedW_dev  int8 blob packed from OIHW weights (K = KH*KW*C).
 *   bias_dev int32 [OC] or NULL; y: QP_S8 or QP_S32 rank 4 NHWC contiguous.
 *   ws       device workspace of qconv2d_s8_im2col_ws_size bytes.
 */
qp_status qconv2d_s8_im2col_ws_size(const qp_qtensor* x, const qp_packed_info* w, int32_t KH,
                                    int32_t KW, int32_t stride_h, int32_t stride_w,
                                    int32_t pad_t, int32_t pad_l, int32_t pad_b, int32_t pad_r,
                                    size_t* bytes);
qp_status qconv2d_s8_im2col(const qp_qtensor* x, const int8_t* X, const qp_packed_info* w,
                            const void* packedW_dev, int32_t KH, int32_t KW, int32_t stride_h,
                            int32_t stride_w, int32_t pad_t, int32_t pad_l, int32_t pad_b,
                            int32_t pad_r, const int32_t* bias_dev, int64_t max_abs_bias,
                            const qp_qtensor* y, int32_t relu, void* Y, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * qconv2d_s8 -- the general INT8 NHWC convolution, with dilation.
 *   acc[b,oy,ox,oc] = sum_{ky,kx,ic} (xp(oy*sh + ky*dh - pt, ox*sw + kx*dw - pl, ic) - zx)
 *                                    * (w[oc,ic,ky,kx] - zw[oc]) + bias[oc],
 *   xp = x inside the image and zx outside ([MNN] tileSplitFunction: padded
 *   taps hold the input zero point); then the requantizing (or raw int32)
 *   epilogue of qgemm_s8s8_requant.  OH = (H + pt + pb - (dh*(KH-1)+1))/sh + 1,
 *   likewise OW.  Routes:
 *   - 1x1 kernel, stride 1, no padding: the GEMM on x viewed as [NB*H*W, C]
 *     ([MNN] DenseConvInt8TiledExecutor::onResize "fastway");
 *   - C % 16 == 0 (and x under 2^31 bytes): implicit GEMM, the im2col gather
 *     inside the operand loads, one launch, no workspace; x must then be
 *     16-byte aligned (QP_EALIGN otherwise);
 *   - otherwise the explicit im2col into the workspace, then the GEMM.
 *   Arguments as qconv2d_s8_im2col, plus dil_h, dil_w >= 1.
 *   ws       device workspace of qconv2d_s8_ws_size bytes (0 for the
 *            implicit route; then ws may be NULL).
 */
qp_status qconv2d_s8_ws_size(const qp_qtensor* x, const qp_packed_info* w, int32_t KH,
                             int32_t KW, int32_t stride_h, int32_t stride_w, int32_t pad_t,
                             int32_t pad_l, int32_t pad_b, int32_t pad_r, int32_t dil_h,
                             int32_t dil_w, size_t* bytes);
qp_status qconv2d_s8(const qp_qtensor* x, const int8_t* X, const qp_packed_info* w,
                     const void* packedW_dev, int32_t KH, int32_t KW, int32_t stride_h,
                     int32_t stride_w, int32_t pad_t, int32_t pad_l, int32_t pad_b,
                     int32_t pad_r, int32_t dil_h, int32_t dil_w, const int32_t* bias_dev,
                     int64_t max_abs_bias, const qp_qtensor* y, int32_t relu, void* Y, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * qconv2d_s8_blockwise_f32 -- INT8 NHWC convolution with channel-blocked int8
 * weights and f32 output ([MNN] _computeReorderQuantInfo and the dynamic-quant
 * path of DenseConvInt8TiledExecutor with blockNum > 1: one weight scale per
 * output channel and block of input channels, exact block sums combined in
 * float):
 *   Y[b,oy,ox,oc] = clamp(sx * sum_{ky,kx,ic} sw[oc][ic/icb] * (xp - zx) * w
 *                         + bias[oc], lo, hi)      (xp = zx outside the image)
 *   x        QP_S8 NHWC, contiguous, 16-byte aligned, per-tensor (sx, zx);
 *            C a multiple of 16 and of icb.
 *   w, packedW_dev  a block-quantized int8 blob packed from OIHW weights with
 *            scheme QP_BLOCKWISE, group_size = icb (64 or 128) and scales
 *            f32 [OC][IC/icb].
 *   bias_dev f32 [OC] or NULL; Y device f32 NHWC [N, OH, OW, OC].
 *   Geometry arguments as qconv2d_s8.  No workspace.  Implicit GEMM.
 */
qp_status qconv2d_s8_blockwise_f32(const qp_qtensor* x, const int8_t* X, const qp_packed_info* w,
                                   const void* packedW_dev, int32_t KH, int32_t KW,
                                   int32_t stride_h, int32_t stride_w, int32_t pad_t,
                                   int32_t pad_l, int32_t pad_b, int32_t pad_r, int32_t dil_h,
                                   int32_t dil_w, const float* bias_dev, float clamp_lo,
                                   float clamp_hi, float* Y, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QPACK_H */
