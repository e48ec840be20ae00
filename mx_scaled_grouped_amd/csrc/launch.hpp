// Internal launcher interface between the C ABI (mxsg.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxsg {

struct QuantActParams {
  const uint16_t *x;
  int64_t M, C;
  int recipe, fmt;
  int E;
  const int32_t *group_ends;
  uint8_t *row_codes;
  void *row_scales;
  uint8_t *col_codes;
  void *col_scales;
  int64_t ld;
  int32_t *padded_starts;
  float *amax;
  const float *dl_scale, *dl_inv;
  const int32_t *row_index;  // optional: routed row i is x row row_index[i]
  int64_t src_rows;          // rows of x when row_index is given
  int32_t *status;           // optional device status word (MXSG_STATUS_* bits)
  int32_t swiglu;            // x is a gate/up output [M, 2C]: quantize silu(gate) * up
};

struct QuantWeightParams {
  const uint16_t *w;
  int E;
  int64_t K, N;
  int recipe, fmt;
  uint8_t *kmajor_codes;
  void *kmajor_scales;
  uint8_t *nmajor_codes;
  void *nmajor_scales;
  float *amax;
  const float *dl_scale, *dl_inv;
  int32_t *status;           // optional device status word
};

struct GemmParams {
  int mode, recipe, fmt_a, fmt_b;
  int E;
  int64_t M, K, N;
  const int32_t *group_ends;
  const int32_t *padded_starts;
  const uint8_t *a;
  const void *a_scales;
  int64_t lda;
  const uint8_t *b;
  const void *b_scales;
  int64_t ldb;
  void *out;
  int accumulate;
};

hipError_t launch_zero(float *p, int n, hipStream_t st);
hipError_t launch_quantize_act(const QuantActParams &p, hipStream_t st);
hipError_t launch_quantize_weight(const QuantWeightParams &p, hipStream_t st);
hipError_t launch_delayed_update(float *hist, int32_t *pos, float *amax, float *scale, float *inv,
                                 int units, int L, int fmt, hipStream_t st);
hipError_t launch_cast_sweep(uint32_t start, int64_t n, int fmt, uint8_t *out, hipStream_t st);
hipError_t launch_route(const int32_t *ids, int64_t T, int k, int E, int32_t *ends, int32_t *row_index,
                        int32_t *slot_row, int32_t *status, hipStream_t st);
hipError_t launch_swiglu(const uint16_t *x, int64_t M, int64_t C, uint16_t *y, hipStream_t st);
hipError_t launch_sigmoid_sweep(float *out, hipStream_t st);
hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, hipStream_t st);
hipError_t launch_clock_probe(int blocks, int iters, uint64_t *out, hipStream_t st);
hipError_t launch_grouped_mm(const GemmParams &p, hipStream_t st);
// ORs MXSG_STATUS_ENDS_* bits into *status for malformed group ends
hipError_t launch_check_ends(const int32_t *ends, int E, int64_t M, int32_t *status, hipStream_t st);

}  // namespace mxsg
