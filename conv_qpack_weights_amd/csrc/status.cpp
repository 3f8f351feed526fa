// status.cpp -- error strings, version, blob geometry.
#include <cmath>
#include <cstdarg>
#include <cstring>

#include "qp_internal.hpp"

namespace qp {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

qp_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) QP_FAIL(QP_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return QP_OK;
}

qp_status blob_geometry(int32_t format, int32_t scheme, int64_t N, int64_t K, int64_t group,
                        qp_packed_info* info) {
  QP_REQUIRE(N > 0 && K > 0, QP_EINVAL, "packed weights need N > 0 and K > 0 (got %lld, %lld)",
             (long long)N, (long long)K);
  qp_packed_info g;
  std::memset(&g, 0, sizeof(g));
  g.format = format;
  g.scheme = scheme;
  g.N = N;
  g.K = K;
  g.Npad = round_up(N, kPadN);
  g.data_off = kHeaderBytes;
  if (format == 1) {
    g.group = 0;
    g.Kpad = round_up(K, kPadK8);
    g.data_bytes = g.Npad * g.Kpad;
    g.scale_off = g.data_off + round_up(g.data_bytes, kRegionAlign);
    g.sum_off = g.scale_off + round_up(4 * g.Npad, kRegionAlign);
    g.zp_off = g.sum_off + round_up(4 * g.Npad, kRegionAlign);
    g.total_bytes = g.zp_off + round_up(4 * g.Npad, kRegionAlign);
  } else if (format >= 2 && format <= 4) {
    QP_REQUIRE(group > 0 && group % kRunK4 == 0 && (kBlockK4 % group == 0 || group % kBlockK4 == 0),
               QP_EUNSUPPORTED, "int4 group size must be 32, 64, 128 or a multiple of 128 (got %lld)",
               (long long)group);
    g.group = group;
    g.Kpad = round_up(K, group > kBlockK4 ? group : kBlockK4);
    // the int4 packer keeps a row's group sums in LDS, and the int4 product
    // kernels count 128-K blocks in 32 bits: a blob restored from bytes is
    // held to the same limit as one packed here
    QP_REQUIRE(g.Kpad <= 65536, QP_EUNSUPPORTED, "int4 weights support K <= 65536 (Kpad %lld)",
               (long long)g.Kpad);
    g.data_bytes = g.Npad * g.Kpad / 2;
    g.scale_off = g.data_off + round_up(g.data_bytes, kRegionAlign);
    // scales in quads of 4 groups: [Npad/16][ceil(G/4)][16][4] of f32
    // (format 2) or bf16 (format 3)
    const int64_t es = format == 3 ? 2 : 4;
    const int64_t scale_bytes = round_up(4 * es * g.Npad * ceil_div(g.Kpad / group, 4), kRegionAlign);
    g.sum_off = g.scale_off + scale_bytes;
    g.zp_off = 0;
    g.total_bytes = g.sum_off + round_up(4 * g.Npad, kRegionAlign);
    if (format == 4) {  // asymmetric: f32 group offsets, laid out as the scales
      g.zp_off = g.total_bytes;
      g.total_bytes += scale_bytes;
    }
  } else if (format == 5) {  // block-quantized int8: the int8 sub-tiles, a scale per block
    QP_REQUIRE(group == 64 || group == 128, QP_EUNSUPPORTED,
               "block-quantized int8 weights take blocks of 64 or 128 K (got %lld)",
               (long long)group);
    g.group = group;
    g.Kpad = round_up(K, 128);
    g.data_bytes = g.Npad * g.Kpad;
    g.scale_off = g.data_off + round_up(g.data_bytes, kRegionAlign);
    g.sum_off = g.scale_off + round_up(4 * g.Npad * (g.Kpad / group), kRegionAlign);
    g.zp_off = 0;
    g.total_bytes = g.sum_off + round_up(4 * g.Npad, kRegionAlign);
  } else {
    QP_FAIL(QP_EINVAL, "unknown packed format %d", format);
  }
  *info = g;
  return QP_OK;
}

}  // namespace qp

extern "C" {

const char* qp_version(void) { return "qpack 0.1 gfx950"; }

const char* qp_last_error(void) { return qp::g_last_error; }

qp_status qp_packed_info_from_header(const void* header_host, qp_packed_info* info) {
  QP_REQUIRE(header_host && info, QP_EINVAL, "qp_packed_info_from_header: null argument");
  qp::BlobHeader h;
  std::memcpy(&h, header_host, sizeof(h));
  QP_REQUIRE(h.magic == qp::kMagic && h.version == qp::kVersion, QP_EINVAL,
             "not a packed-weight blob (magic %08x, version %u)", h.magic, h.version);
  qp_packed_info g;
  qp_status st = qp::blob_geometry((int32_t)h.format, (int32_t)h.scheme, h.N, h.K, h.group, &g);
  if (st != QP_OK) return st;
  QP_REQUIRE(g.Npad == h.Npad && g.Kpad == h.Kpad && g.scale_off == h.scale_off &&
                 g.sum_off == h.sum_off && g.total_bytes == h.total_bytes,
             QP_EINVAL, "blob header is inconsistent with its own geometry");
  QP_REQUIRE(h.invalid_values == 0, QP_EINVAL, "blob was packed from out-of-range int4 values");
  g.has_zero_points = h.has_zp;
  if (g.format == 1) {
    // The scale range drives the multiplier validation of the GEMM entry
    // points; a blob without a valid one is refused rather than run unchecked.
    QP_REQUIRE(std::isfinite(h.scale_min) && std::isfinite(h.scale_max) && h.scale_min > 0.0f &&
                   h.scale_min <= h.scale_max,
               QP_EINVAL, "blob header holds no valid weight-scale range (%g, %g)",
               (double)h.scale_min, (double)h.scale_max);
    g.scale_min = h.scale_min;
    g.scale_max = h.scale_max;
  } else {
    g.scale_min = 0.0f;
    g.scale_max = 0.0f;
  }
  *info = g;
  return QP_OK;
}

}  // extern "C"
