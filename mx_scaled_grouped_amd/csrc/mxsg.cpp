// C ABI of the quantized MoE expert grouped GEMM: host-side validation and
// dispatch to the gfx950 kernels. Declarations and contracts: include/mxsg.h.
//
// Every argument check happens here, before any HIP call, so a malformed
// call returns an error code and enqueues nothing. The library keeps no
// mutable global state besides the per-thread error message.
#include "mxsg.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

mxsg_status fail(mxsg_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mxsg_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return MXSG_OK;
  }
  return fail(MXSG_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool recipe_ok(int32_t r) { return r >= MXSG_RECIPE_TENSORWISE && r <= MXSG_RECIPE_NVFP4; }
// e2m1 elements exist for the MX and NVFP4 recipes; NVFP4 has e2m1 elements only
bool fmt_recipe_ok(int32_t fmt, int32_t recipe) {
  if (recipe == MXSG_RECIPE_NVFP4) return fmt == MXSG_FMT_E2M1;
  return fmt != MXSG_FMT_E2M1 || recipe == MXSG_RECIPE_MX;
}
bool fmt_ok(int32_t f) { return f == MXSG_FMT_E4M3 || f == MXSG_FMT_E5M2 || f == MXSG_FMT_E2M1; }
bool fp8_fmt(int32_t f) { return f == MXSG_FMT_E4M3 || f == MXSG_FMT_E5M2; }
// contraction / feature elements per code byte
int64_t elems_per_byte(int32_t f) { return f == MXSG_FMT_E2M1 ? 2 : 1; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

// Shape rules shared by the size queries and the launching entry points;
// fn names the caller in the error message.
mxsg_status act_shape(const char *fn, int64_t M, int64_t C, int32_t recipe, int32_t fmt) {
  REQUIRE(recipe_ok(recipe), MXSG_INVALID_ARGUMENT, "%s: unknown recipe %d", fn, recipe);
  REQUIRE(fmt_ok(fmt), MXSG_INVALID_ARGUMENT, "%s: unknown format %d", fn, fmt);
  REQUIRE(fmt_recipe_ok(fmt, recipe), MXSG_UNSUPPORTED,
          "%s: e2m1 codes go with the MX or NVFP4 recipe, and NVFP4 with e2m1 only", fn);
  REQUIRE(M >= 0 && C > 0, MXSG_INVALID_ARGUMENT, "%s: M=%lld C=%lld", fn, (long long)M,
          (long long)C);
  REQUIRE(C % 128 == 0, MXSG_BAD_SHAPE, "%s: C=%lld is not a multiple of 128", fn, (long long)C);
  REQUIRE(M <= ((int64_t)1 << 31) - 1 && C <= ((int64_t)1 << 31) - 1, MXSG_BAD_SHAPE,
          "%s: M or C too large", fn);
  return MXSG_OK;
}

mxsg_status weight_shape(const char *fn, int32_t E, int64_t K, int64_t N, int32_t recipe,
                         int32_t fmt) {
  REQUIRE(recipe_ok(recipe), MXSG_INVALID_ARGUMENT, "%s: unknown recipe %d", fn, recipe);
  REQUIRE(fmt_ok(fmt), MXSG_INVALID_ARGUMENT, "%s: unknown format %d", fn, fmt);
  REQUIRE(fmt_recipe_ok(fmt, recipe), MXSG_UNSUPPORTED,
          "%s: e2m1 codes go with the MX or NVFP4 recipe, and NVFP4 with e2m1 only", fn);
  REQUIRE(E >= 1 && K > 0 && N > 0, MXSG_INVALID_ARGUMENT, "%s: E=%d K=%lld N=%lld", fn, E,
          (long long)K, (long long)N);
  REQUIRE(K % 128 == 0 && N % 128 == 0, MXSG_BAD_SHAPE,
          "%s: K=%lld and N=%lld must be multiples of 128", fn, (long long)K, (long long)N);
  // one workgroup per 128 x 128 tile of one expert, experts on grid.z
  REQUIRE(E <= 65535 && (K / 128) * (N / 128) <= INT32_MAX, MXSG_BAD_SHAPE, "%s: too large", fn);
  return MXSG_OK;
}

}  // namespace

static mxsg_status quantize_act_impl(const char *fn, const void *x, int64_t T,
                                     const int32_t *row_index, int64_t M, int64_t C,
                                     int32_t recipe, int32_t fmt, int32_t E,
                                     const int32_t *group_ends, void *row_codes, void *row_scales,
                                     void *col_codes, void *col_scales, int64_t ld,
                                     int32_t *padded_starts, float *amax, const float *dl_scale,
                                     const float *dl_inv, int32_t *status_word,
                                     mxsg_stream_t stream, bool swiglu = false) {
  mxsg_status st = act_shape(fn, M, C, recipe, fmt);
  if (st != MXSG_OK) return st;
  REQUIRE(row_codes || col_codes, MXSG_INVALID_ARGUMENT, "%s: no output requested", fn);
  REQUIRE(M == 0 || x, MXSG_INVALID_ARGUMENT, "%s: x is NULL", fn);
  if (row_index || T != M) {  // gathered rows: an index per routed row into x [T, C]
    REQUIRE(M == 0 || row_index, MXSG_INVALID_ARGUMENT, "%s: row_index is NULL", fn);
    REQUIRE(T >= 0 && T <= ((int64_t)1 << 31) - 1 && (M == 0 || T > 0), MXSG_BAD_SHAPE,
            "%s: x has %lld rows for %lld routed rows", fn, (long long)T, (long long)M);
  }
  const bool scaled_unit =
      recipe == MXSG_RECIPE_BLOCKWISE || recipe == MXSG_RECIPE_MX || recipe == MXSG_RECIPE_NVFP4;
  if (row_codes && scaled_unit)
    REQUIRE(row_scales, MXSG_INVALID_ARGUMENT, "%s: row_scales is NULL", fn);
  if (col_codes) {
    REQUIRE(E >= 1 && E <= (1 << 20), MXSG_INVALID_ARGUMENT,
            "%s: column-wise output needs 1 <= E <= 2^20, got %d", fn, E);
    REQUIRE(group_ends && padded_starts, MXSG_INVALID_ARGUMENT,
            "%s: column-wise output needs group_ends and padded_starts", fn);
    REQUIRE(ld % 128 == 0 && ld >= mxsg_padded_capacity(M, E), MXSG_BAD_SHAPE,
            "%s: ld=%lld must be a multiple of 128 and >= %lld", fn, (long long)ld,
            (long long)mxsg_padded_capacity(M, E));
    if (scaled_unit)
      REQUIRE(col_scales, MXSG_INVALID_ARGUMENT, "%s: col_scales is NULL", fn);
  }
  if (recipe == MXSG_RECIPE_TENSORWISE || recipe == MXSG_RECIPE_DELAYED || recipe == MXSG_RECIPE_NVFP4)
    REQUIRE(amax, MXSG_INVALID_ARGUMENT, "%s: amax is NULL", fn);
  if (recipe == MXSG_RECIPE_DELAYED)
    REQUIRE(dl_scale && dl_inv, MXSG_INVALID_ARGUMENT, "%s: dl_scale/dl_inv NULL", fn);
  {
    // one workgroup per 128 x 128 tile (row tiles, or padded-column tiles)
    const int64_t rt = col_codes ? ld / 128 : (M + 127) / 128;
    REQUIRE((rt > 0 ? rt : 1) * (C / 128) <= INT32_MAX, MXSG_BAD_SHAPE,
            "%s: %lld x %lld tiles exceed the launch limit", fn, (long long)rt,
            (long long)(C / 128));
  }

  mxsg::QuantActParams p{};
  p.x = static_cast<const uint16_t *>(x);
  p.M = M;
  p.C = C;
  p.recipe = recipe;
  p.fmt = fmt;
  p.E = col_codes ? E : 0;
  p.group_ends = group_ends;
  p.row_codes = static_cast<uint8_t *>(row_codes);
  p.row_scales = row_scales;
  p.col_codes = static_cast<uint8_t *>(col_codes);
  p.col_scales = col_scales;
  p.ld = ld;
  p.padded_starts = padded_starts;
  p.amax = amax;
  p.dl_scale = dl_scale;
  p.dl_inv = dl_inv;
  p.row_index = row_index;
  p.src_rows = T;
  p.status = status_word;
  p.swiglu = swiglu ? 1 : 0;
  if (status_word && group_ends && E >= 1) {
    const hipError_t e = mxsg::launch_check_ends(group_ends, E, M, status_word, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return from_hip(e, fn);
  }
  return from_hip(mxsg::launch_quantize_act(p, static_cast<hipStream_t>(stream)), fn);
}

extern "C" {

const char *mxsg_status_str(mxsg_status s) {
  switch (s) {
    case MXSG_OK: return "ok";
    case MXSG_INVALID_ARGUMENT: return "invalid argument";
    case MXSG_BAD_SHAPE: return "bad shape";
    case MXSG_UNSUPPORTED: return "unsupported";
    case MXSG_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

const char *mxsg_last_error(void) { return g_err; }

int32_t mxsg_version(void) { return 100; }  // 0.1.0

int64_t mxsg_padded_capacity(int64_t M, int32_t E) {
  if (M < 0 || E < 0) return -1;
  return ((M + 127 * (int64_t)E + 127) / 128) * 128;
}

mxsg_status mxsg_quantize_act_sizes(int64_t M, int64_t C, int32_t recipe, int32_t fmt, int32_t E,
                                    int64_t bytes[5]) {
  REQUIRE(bytes, MXSG_INVALID_ARGUMENT, "quantize_act_sizes: bytes is NULL");
  mxsg_status st = act_shape("quantize_act_sizes", M, C, recipe, fmt);
  if (st != MXSG_OK) return st;
  REQUIRE(E >= 0 && E <= (1 << 20), MXSG_INVALID_ARGUMENT, "quantize_act_sizes: E=%d", E);
  // scale bytes of n elements along a row: fp32 per 128, E8M0 per 32, or one fp32
  auto scale_bytes = [recipe](int64_t rows, int64_t n) -> int64_t {
    if (recipe == MXSG_RECIPE_BLOCKWISE) return rows * (n / 128) * 4;
    if (recipe == MXSG_RECIPE_MX) return rows * (n / 32);
    if (recipe == MXSG_RECIPE_NVFP4) return rows * (n / 16) + 4;   // block codes, then the tensor scale
    return 4;
  };
  const int64_t epb = elems_per_byte(fmt);
  bytes[0] = (M + (M & 1)) * (C / epb);
  bytes[1] = scale_bytes(M, C);
  if (E >= 1) {
    const int64_t ld = mxsg_padded_capacity(M, E);
    bytes[2] = C * (ld / epb);
    bytes[3] = scale_bytes(C, ld);
    bytes[4] = ((int64_t)E + 1) * 4;
  } else {
    bytes[2] = bytes[3] = bytes[4] = 0;
  }
  g_err[0] = 0;
  return MXSG_OK;
}

mxsg_status mxsg_quantize_weight_sizes(int32_t E, int64_t K, int64_t N, int32_t recipe,
                                       int32_t fmt, int64_t bytes[4]) {
  REQUIRE(bytes, MXSG_INVALID_ARGUMENT, "quantize_weight_sizes: bytes is NULL");
  mxsg_status st = weight_shape("quantize_weight_sizes", E, K, N, recipe, fmt);
  if (st != MXSG_OK) return st;
  const int64_t elems = (int64_t)E * K * N;
  bytes[0] = bytes[2] = elems / elems_per_byte(fmt);
  switch (recipe) {
    case MXSG_RECIPE_BLOCKWISE: bytes[1] = bytes[3] = (int64_t)E * (K / 128) * (N / 128) * 4; break;
    case MXSG_RECIPE_MX: bytes[1] = bytes[3] = elems / 32; break;
    case MXSG_RECIPE_NVFP4: bytes[1] = bytes[3] = elems / 16 + 4 * (int64_t)E; break;
    default: bytes[1] = bytes[3] = (int64_t)E * 4; break;
  }
  g_err[0] = 0;
  return MXSG_OK;
}

mxsg_status mxsg_quantize_act(const void *x, int64_t M, int64_t C, int32_t recipe, int32_t fmt,
                              int32_t E, const int32_t *group_ends, void *row_codes,
                              void *row_scales, void *col_codes, void *col_scales, int64_t ld,
                              int32_t *padded_starts, float *amax, const float *dl_scale,
                              const float *dl_inv, int32_t *status_word, mxsg_stream_t stream) {
  return quantize_act_impl("quantize_act", x, M, nullptr, M, C, recipe, fmt, E, group_ends,
                           row_codes, row_scales, col_codes, col_scales, ld, padded_starts, amax,
                           dl_scale, dl_inv, status_word, stream);
}

mxsg_status mxsg_quantize_act_swiglu(const void *x, int64_t M, int64_t C, int32_t recipe,
                                     int32_t fmt, int32_t E, const int32_t *group_ends,
                                     void *row_codes, void *row_scales, void *col_codes,
                                     void *col_scales, int64_t ld, int32_t *padded_starts,
                                     float *amax, const float *dl_scale, const float *dl_inv,
                                     int32_t *status_word, mxsg_stream_t stream) {
  return quantize_act_impl("quantize_act_swiglu", x, M, nullptr, M, C, recipe, fmt, E, group_ends,
                           row_codes, row_scales, col_codes, col_scales, ld, padded_starts, amax,
                           dl_scale, dl_inv, status_word, stream, true);
}

mxsg_status mxsg_quantize_act_gather(const void *x, int64_t T, const int32_t *row_index, int64_t M,
                                     int64_t C, int32_t recipe, int32_t fmt, int32_t E,
                                     const int32_t *group_ends, void *row_codes, void *row_scales,
                                     void *col_codes, void *col_scales, int64_t ld,
                                     int32_t *padded_starts, float *amax, const float *dl_scale,
                                     const float *dl_inv, int32_t *status_word, mxsg_stream_t stream) {
  REQUIRE(M == 0 || row_index, MXSG_INVALID_ARGUMENT, "quantize_act_gather: row_index is NULL");
  return quantize_act_impl("quantize_act_gather", x, T, row_index, M, C, recipe, fmt, E,
                           group_ends, row_codes, row_scales, col_codes, col_scales, ld,
                           padded_starts, amax, dl_scale, dl_inv, status_word, stream);
}

mxsg_status mxsg_quantize_weight(const void *w, int32_t E, int64_t K, int64_t N, int32_t recipe,
                                 int32_t fmt, void *kmajor_codes, void *kmajor_scales,
                                 void *nmajor_codes, void *nmajor_scales, float *amax,
                                 const float *dl_scale, const float *dl_inv, int32_t *status_word,
                                 mxsg_stream_t stream) {
  mxsg_status st = weight_shape("quantize_weight", E, K, N, recipe, fmt);
  if (st != MXSG_OK) return st;
  REQUIRE(w, MXSG_INVALID_ARGUMENT, "quantize_weight: w is NULL");
  REQUIRE(kmajor_codes || nmajor_codes, MXSG_INVALID_ARGUMENT, "quantize_weight: no output");
  if (kmajor_codes) REQUIRE(kmajor_scales, MXSG_INVALID_ARGUMENT, "quantize_weight: kmajor_scales NULL");
  if (nmajor_codes) REQUIRE(nmajor_scales, MXSG_INVALID_ARGUMENT, "quantize_weight: nmajor_scales NULL");
  if (recipe == MXSG_RECIPE_TENSORWISE || recipe == MXSG_RECIPE_DELAYED || recipe == MXSG_RECIPE_NVFP4)
    REQUIRE(amax, MXSG_INVALID_ARGUMENT, "quantize_weight: amax is NULL");
  if (recipe == MXSG_RECIPE_DELAYED)
    REQUIRE(dl_scale && dl_inv, MXSG_INVALID_ARGUMENT, "quantize_weight: dl_scale/dl_inv NULL");

  mxsg::QuantWeightParams p{};
  p.w = static_cast<const uint16_t *>(w);
  p.E = E;
  p.K = K;
  p.N = N;
  p.recipe = recipe;
  p.fmt = fmt;
  p.kmajor_codes = static_cast<uint8_t *>(kmajor_codes);
  p.kmajor_scales = kmajor_scales;
  p.nmajor_codes = static_cast<uint8_t *>(nmajor_codes);
  p.nmajor_scales = nmajor_scales;
  p.amax = amax;
  p.dl_scale = dl_scale;
  p.dl_inv = dl_inv;
  p.status = status_word;
  return from_hip(mxsg::launch_quantize_weight(p, static_cast<hipStream_t>(stream)),
                  "quantize_weight");
}

mxsg_status mxsg_delayed_update(float *history, int32_t *pos, float *amax, float *scale,
                                float *inv, int32_t units, int32_t L, int32_t fmt,
                                mxsg_stream_t stream) {
  REQUIRE(fp8_fmt(fmt), MXSG_INVALID_ARGUMENT, "delayed_update: unknown FP8 format %d", fmt);
  REQUIRE(units >= 0 && L >= 1, MXSG_INVALID_ARGUMENT, "delayed_update: units=%d L=%d", units, L);
  if (units > 0)
    REQUIRE(history && pos && amax && scale && inv, MXSG_INVALID_ARGUMENT,
            "delayed_update: NULL state array");
  return from_hip(mxsg::launch_delayed_update(history, pos, amax, scale, inv, units, L, fmt,
                                              static_cast<hipStream_t>(stream)),
                  "delayed_update");
}

mxsg_status mxsg_grouped_mm_check(int32_t mode, int32_t recipe, int32_t fmt_a, int32_t fmt_b,
                                  int32_t E, int64_t M, int64_t K, int64_t N, int64_t lda,
                                  int64_t ldb, int32_t accumulate) {
  REQUIRE(mode >= MXSG_MODE_FWD && mode <= MXSG_MODE_WGRAD, MXSG_INVALID_ARGUMENT,
          "grouped_mm: unknown mode %d", mode);
  REQUIRE(recipe_ok(recipe), MXSG_INVALID_ARGUMENT, "grouped_mm: unknown recipe %d", recipe);
  REQUIRE(fmt_ok(fmt_a) && fmt_ok(fmt_b), MXSG_INVALID_ARGUMENT, "grouped_mm: unknown format");
  REQUIRE(!(fmt_a == MXSG_FMT_E5M2 && fmt_b == MXSG_FMT_E5M2), MXSG_UNSUPPORTED,
          "grouped_mm: e5m2 x e5m2 is not built");
  REQUIRE((fmt_a == MXSG_FMT_E2M1) == (fmt_b == MXSG_FMT_E2M1), MXSG_UNSUPPORTED,
          "grouped_mm: 4-bit operands are built only against 4-bit operands");
  REQUIRE(fmt_recipe_ok(fmt_a, recipe) && fmt_recipe_ok(fmt_b, recipe), MXSG_UNSUPPORTED,
          "grouped_mm: e2m1 operands go with the MX or NVFP4 recipe, and NVFP4 with e2m1 only");
  const int64_t epb = elems_per_byte(fmt_a);
  REQUIRE(E >= 1 && M >= 0 && K > 0 && N > 0, MXSG_INVALID_ARGUMENT,
          "grouped_mm: E=%d M=%lld K=%lld N=%lld", E, (long long)M, (long long)K, (long long)N);
  REQUIRE(K % 128 == 0 && N % 128 == 0, MXSG_BAD_SHAPE,
          "grouped_mm: K=%lld and N=%lld must be multiples of 128", (long long)K, (long long)N);
  REQUIRE(M <= ((int64_t)1 << 31) - 1 && E <= (1 << 20), MXSG_BAD_SHAPE, "grouped_mm: too large");
  // the kernel addresses a tile's 256 rows with 32-bit offsets
  REQUIRE(lda < ((int64_t)1 << 23) && ldb < ((int64_t)1 << 23), MXSG_BAD_SHAPE,
          "grouped_mm: row strides must be below 2^23");
  REQUIRE(accumulate == 0 || mode == MXSG_MODE_WGRAD, MXSG_INVALID_ARGUMENT,
          "grouped_mm: accumulate is only defined for WGRAD");
  if (mode == MXSG_MODE_WGRAD) {
    const int64_t cap = mxsg_padded_capacity(M, E) / epb;   // code bytes
    const int64_t q = 128 / epb;
    REQUIRE(lda % q == 0 && ldb % q == 0 && lda >= cap && ldb >= cap, MXSG_BAD_SHAPE,
            "grouped_mm: WGRAD lda=%lld ldb=%lld (code bytes) must be multiples of %lld and >= %lld",
            (long long)lda, (long long)ldb, (long long)q, (long long)cap);
  } else {
    const int64_t L = (mode == MXSG_MODE_FWD ? K : N) / epb;   // code bytes
    REQUIRE(lda >= L && lda % 64 == 0, MXSG_BAD_SHAPE,
            "grouped_mm: lda=%lld must be >= %lld and a multiple of 64", (long long)lda,
            (long long)L);
    REQUIRE(ldb == L, MXSG_BAD_SHAPE, "grouped_mm: ldb=%lld must equal %lld", (long long)ldb,
            (long long)L);
    REQUIRE(recipe != MXSG_RECIPE_BLOCKWISE || L <= 65536, MXSG_UNSUPPORTED,
            "grouped_mm: blockwise contraction %lld > 65536 is not built", (long long)L);
  }
  // the blockwise kernel keeps row and column indices in 32 bits
  REQUIRE(recipe != MXSG_RECIPE_BLOCKWISE || (K < ((int64_t)1 << 31) && N < ((int64_t)1 << 31)),
          MXSG_UNSUPPORTED, "grouped_mm: blockwise K=%lld N=%lld must be below 2^31", (long long)K,
          (long long)N);
  g_err[0] = 0;
  return MXSG_OK;
}

mxsg_status mxsg_grouped_mm(int32_t mode, int32_t recipe, int32_t fmt_a, int32_t fmt_b, int32_t E,
                            int64_t M, int64_t K, int64_t N, const int32_t *group_ends,
                            const int32_t *padded_starts, const void *a_codes,
                            const void *a_scales, int64_t lda, const void *b_codes,
                            const void *b_scales, int64_t ldb, void *out, int32_t accumulate,
                            int32_t *status_word, mxsg_stream_t stream) {
  mxsg_status st = mxsg_grouped_mm_check(mode, recipe, fmt_a, fmt_b, E, M, K, N, lda, ldb, accumulate);
  if (st != MXSG_OK) return st;
  REQUIRE(a_codes && b_codes && out && a_scales && b_scales && group_ends, MXSG_INVALID_ARGUMENT,
          "grouped_mm: NULL operand");
  REQUIRE(mode != MXSG_MODE_WGRAD || padded_starts, MXSG_INVALID_ARGUMENT,
          "grouped_mm: WGRAD needs padded_starts");
  mxsg::GemmParams p{};
  p.mode = mode;
  p.recipe = recipe;
  p.fmt_a = fmt_a;
  p.fmt_b = fmt_b;
  p.E = E;
  p.M = M;
  p.K = K;
  p.N = N;
  p.group_ends = group_ends;
  p.padded_starts = padded_starts;
  p.a = static_cast<const uint8_t *>(a_codes);
  p.a_scales = a_scales;
  p.lda = lda;
  p.b = static_cast<const uint8_t *>(b_codes);
  p.b_scales = b_scales;
  p.ldb = ldb;
  p.out = out;
  p.accumulate = accumulate;
  if (status_word) {
    const hipError_t e = mxsg::launch_check_ends(group_ends, E, M, status_word, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return from_hip(e, "grouped_mm");
  }
  return from_hip(mxsg::launch_grouped_mm(p, static_cast<hipStream_t>(stream)), "grouped_mm");
}

mxsg_status mxsg_cast_sweep(uint32_t start_bits, int64_t n, int32_t fmt, void *out,
                            mxsg_stream_t stream) {
  REQUIRE(fmt_ok(fmt), MXSG_INVALID_ARGUMENT, "cast_sweep: unknown format %d", fmt);  // e2m1: one code per byte
  REQUIRE(n >= 0 && n <= ((int64_t)1 << 32), MXSG_INVALID_ARGUMENT, "cast_sweep: n=%lld",
          (long long)n);
  REQUIRE(n == 0 || out, MXSG_INVALID_ARGUMENT, "cast_sweep: out is NULL");
  return from_hip(mxsg::launch_cast_sweep(start_bits, n, fmt, static_cast<uint8_t *>(out),
                                          static_cast<hipStream_t>(stream)),
                  "cast_sweep");
}

mxsg_status mxsg_route(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E, int32_t *group_ends,
                       int32_t *row_index, int32_t *slot_row, int32_t *status_word, mxsg_stream_t stream) {
  REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= (1 << 20), MXSG_INVALID_ARGUMENT,
          "route: T=%lld k=%d E=%d", (long long)T, k, E);
  REQUIRE(T <= (((int64_t)1 << 31) - 1) / k, MXSG_BAD_SHAPE, "route: T * k must be below 2^31");
  REQUIRE(group_ends, MXSG_INVALID_ARGUMENT, "route: group_ends is NULL");
  REQUIRE(T == 0 || (expert_ids && row_index), MXSG_INVALID_ARGUMENT, "route: NULL pointer");
  return from_hip(mxsg::launch_route(expert_ids, T, k, E, group_ends, row_index, slot_row, status_word,
                                     static_cast<hipStream_t>(stream)),
                  "route");
}

mxsg_status mxsg_swiglu(const void *x, int64_t M, int64_t C, void *y, mxsg_stream_t stream) {
  REQUIRE(M >= 0 && C > 0 && C % 8 == 0, MXSG_BAD_SHAPE,
          "swiglu: M=%lld C=%lld (C must be a positive multiple of 8)", (long long)M, (long long)C);
  REQUIRE(M <= ((int64_t)1 << 31) - 1 && C <= ((int64_t)1 << 31) - 1, MXSG_BAD_SHAPE, "swiglu: too large");
  REQUIRE(M == 0 || (x && y), MXSG_INVALID_ARGUMENT, "swiglu: NULL pointer");
  REQUIRE(((uintptr_t)x | (uintptr_t)y) % 16 == 0, MXSG_INVALID_ARGUMENT,
          "swiglu: pointers must be 16-byte aligned");
  return from_hip(mxsg::launch_swiglu(static_cast<const uint16_t *>(x), M, C, static_cast<uint16_t *>(y),
                                      static_cast<hipStream_t>(stream)),
                  "swiglu");
}

mxsg_status mxsg_sigmoid_sweep(float *out, mxsg_stream_t stream) {
  REQUIRE(out, MXSG_INVALID_ARGUMENT, "sigmoid_sweep: out is NULL");
  return from_hip(mxsg::launch_sigmoid_sweep(out, static_cast<hipStream_t>(stream)), "sigmoid_sweep");
}

mxsg_status mxsg_stream_copy(const void *src, void *dst, int64_t bytes, mxsg_stream_t stream) {
  REQUIRE(bytes >= 0 && bytes % 16 == 0 && bytes / 16 / 256 < INT32_MAX, MXSG_INVALID_ARGUMENT,
          "stream_copy: bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
  REQUIRE(bytes == 0 || (src && dst), MXSG_INVALID_ARGUMENT, "stream_copy: NULL pointer");
  REQUIRE(((uintptr_t)src | (uintptr_t)dst) % 16 == 0, MXSG_INVALID_ARGUMENT,
          "stream_copy: pointers must be 16-byte aligned");
  return from_hip(mxsg::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)),
                  "stream_copy");
}

mxsg_status mxsg_clock_probe(int32_t blocks, int32_t iters, uint64_t *out, mxsg_stream_t stream) {
  REQUIRE(blocks >= 0 && blocks <= (1 << 20) && iters >= 0, MXSG_INVALID_ARGUMENT,
          "clock_probe: blocks=%d must be in [0, 2^20], iters=%d non-negative", blocks, iters);
  REQUIRE(blocks == 0 || out, MXSG_INVALID_ARGUMENT, "clock_probe: out is NULL");
  return from_hip(mxsg::launch_clock_probe(blocks, iters, out, static_cast<hipStream_t>(stream)),
                  "clock_probe");
}

mxsg_status mxsg_wall_clock_rate_khz(int32_t *khz) {
  REQUIRE(khz, MXSG_INVALID_ARGUMENT, "wall_clock_rate_khz: khz is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return from_hip(e, "wall_clock_rate_khz");
}

}  // extern "C"
