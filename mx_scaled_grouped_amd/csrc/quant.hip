// Quantization kernels: amax reduction, scale computation, saturating RNE
// cast to OCP e4m3 / e5m2, and the LDS-staged transposed (column-wise)
// variant for wgrad, for the tensorwise, delayed, blockwise (1x128, 128x1,
// 128x128) and MX (32-element, E8M0) recipes.
//
// Design (gfx950): HBM-bound, so each element is read once per pass with
// 16-byte vector loads and each code written once with coalesced streaming
// (nontemporal) stores; inputs larger than the last-level cache are read
// with streaming loads too.
// A 256-thread workgroup owns a 128 x 128 tile of the input (128 rows of
// 128 features). Row-wise units (1x128, 1x32) are reduced across the 16 (or
// 4) lanes that hold one row; the tile is staged in LDS and re-read by
// columns for the column-wise units (128x1, 32x1), whose codes are written
// through an LDS code tile as 128-byte rows of the transposed output. The
// Transformer Engine blockwise issue's design note does the same: column
// (128x1) scaling with the transpose staged on chip rather than through a
// high-precision copy in memory, and a zero fill of partial blocks: a tile that runs past a group's last token reads
// zeros there, so padding never raises an amax and its codes are 0x00.
//
// Column-wise tiles are laid out in padded token space: group g owns padded
// columns [P_g, P_{g+1}), P_{g+1} = P_g + ceil(m_g/128)*128, so every
// 128-column tile lies inside one group and a 128x1 unit is one tile column.
//
// Every code matrix is written pair-interleaved (pi_off): the grouped GEMM
// reads 64 contraction bytes of two adjacent rows as one 128-byte line. A
// wave's stores still cover whole lines (four rows of 128 codes row-wise,
// eight feature rows of 128 positions column-wise).
#include "device_common.hpp"
#include "launch.hpp"
#include "mxsg.h"

namespace mxsg {

constexpr int QT = 128;       // tile rows (tokens or K) and columns (features)
constexpr int QTHREADS = 256;
constexpr int CODE_LD = 144;  // LDS row stride (bytes) of the transposed code tile
constexpr int CODE_LD4 = 80;  // the same for 4-bit codes (64 bytes of codes per feature row)

// ---------------------------------------------------------------------------
// small kernels

// status word: an amax reduction's maximum bf16 magnitude bits with an
// all-ones exponent mean an Inf or NaN input (only then an atomic)
__device__ __forceinline__ void flag_nonfinite(int32_t *status, uint32_t absbits) {
  if (status && absbits >= 0x7F80u) atomicOr(status, MXSG_STATUS_NONFINITE);
}

// status word: malformed group ends (one workgroup)
__global__ __launch_bounds__(256) void check_ends_kernel(const int32_t *__restrict__ ends, int E, int64_t M,
                                                         int32_t *__restrict__ status) {
  int bits = 0;
  for (int g = threadIdx.x; g < E; g += blockDim.x) {
    const int64_t e = ends[g], prev = g ? ends[g - 1] : 0;
    if (e < prev) bits |= MXSG_STATUS_ENDS_DECREASING;
    if (e < 0 || e > M) bits |= MXSG_STATUS_ENDS_RANGE;
    if (g == E - 1 && e != M) bits |= MXSG_STATUS_ENDS_TOTAL;
  }
  if (bits) atomicOr(status, bits);
}

__global__ void zero_f32_kernel(float *__restrict__ p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// amax of `units` contiguous units of `unit_elems` bf16 each (unit_elems % 8
// == 0); the result is max-reduced into amax_bits[u] (fp32 bit pattern; the
// slot must start at 0).
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t *__restrict__ x,
                                                   int64_t unit_elems,
                                                   uint32_t *__restrict__ amax_bits,
                                                   int32_t *__restrict__ status) {
  const int u = blockIdx.y;
  const uint4 *p = reinterpret_cast<const uint4 *>(x + (int64_t)u * unit_elems);
  const int64_t nvec = unit_elems / 8;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    m = absmax_bits8(p[i], m);
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    if (m) atomic_max_bits(amax_bits + u, m << 16);
    flag_nonfinite(status, m);
  }
}

// Source row of routed row i: row_index[i] clamped into [0, src_rows), or i
// itself without an index. A malformed index gives wrong rows, never an
// out-of-bounds read.
__device__ __forceinline__ int64_t source_row(const int32_t *row_index, int64_t src_rows, int64_t i) {
  if (!row_index) return i;
  const int64_t t = row_index[i];
  return t < 0 ? 0 : (t >= src_rows ? src_rows - 1 : t);
}

// amax over the routed rows x[row_index[i]], i < M, of a [src_rows, C]
// tensor (tensorwise dynamic scaling of a gathered operand): a workgroup
// takes whole rows, its threads the row's 16-byte chunks.
__global__ __launch_bounds__(256) void amax_rows_kernel(const uint16_t *__restrict__ x, int64_t C,
                                                        const int32_t *__restrict__ row_index,
                                                        int64_t M, int64_t src_rows,
                                                        uint32_t *__restrict__ amax_bits,
                                                        int32_t *__restrict__ status) {
  uint32_t m = 0;
  const int64_t nvec = C / 8;
  for (int64_t i = blockIdx.x; i < M; i += gridDim.x) {
    const uint4 *p = reinterpret_cast<const uint4 *>(x + source_row(row_index, src_rows, i) * C);
    for (int64_t c = threadIdx.x; c < nvec; c += blockDim.x) m = absmax_bits8(p[c], m);
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    if (m) atomic_max_bits(amax_bits, m << 16);
    flag_nonfinite(status, m);
  }
}

// ---------------------------------------------------------------------------
// the 128x128 tile quantizer

struct TileArgs {
  const uint16_t *x;      // [batch][rows, C]
  int64_t rows;           // M (tokens) or K (weights)
  int64_t C;              // features
  int32_t E;              // groups (column-wise token layout); 0 = one group of all rows
  const int32_t *ends;    // [E]
  uint8_t *row_codes;     // [batch][rows, C], pair-interleaved
  void *row_scales;
  uint8_t *col_codes;     // [batch][C, ld], pair-interleaved
  void *col_scales;
  int64_t ld;             // column-wise row stride (bytes)
  int32_t *padded_out;    // [E+1] or null
  float *amax;            // [batch]: TW read (computed before), DL max-reduced into
  const float *dl_scale;  // [batch]
  const float *dl_inv;    // [batch]
  int64_t x_bstride, row_bstride, col_bstride;       // per batch element (elements / bytes)
  int64_t rs_bstride, cs_bstride;                    // scale strides per batch element
  int32_t stream_x;       // read x with streaming loads (x far larger than the caches)
  const int32_t *row_index;  // optional gather: routed row i is x row row_index[i]
  int64_t src_rows;          // rows of x when row_index is given
  int32_t *status;           // optional status word (non-finite inputs)
  int32_t rgroup;            // row tiles per launch-order group (>= 1)
  int32_t swiglu;            // x is a gate/up output [rows, 2C]: quantize silu(gate) * up
  int64_t rs_tail, cs_tail;  // NVFP4: byte offset of the fp32 tensor scales in row_scales / col_scales
};

// ---------------------------------------------------------------------------
// SwiGLU between the expert GEMMs: the bf16 value nearest to the exact
// silu(g) * u (ties to even), silu(g) = g * sigmoid(g), for bf16 g and u.
// For finite g != 0 and u != 0 that value is transcendental, hence never a
// bf16 midpoint, so the rounding is well defined.
//
// Fast path, fp32. With a = |g| <= 64, e = exp(-a) = 2^-(a log2 e) is taken
// as 2^-n * 2^-f: n = rint(a * kL2eHi) (an exact product: a has 8 significant
// bits, kL2eHi 15), f = (a * kL2eHi - n) + a * kL2eLo (|f| <= 0.51, the
// difference exact), 2^-f from v_exp_f32 and 2^-n from an exact ldexp. Then
// sigmoid(a) = 1 / (1 + e) and sigmoid(-a) = e / (1 + e) with v_rcp_f32, and
// p = fl(g * u) * sigmoid(g), where g * u is exact (8 x 8 significant bits).
// Error budget in units of 2^-23 relative: e 1.1 (exp2 1 ulp, argument
// rounding 0.1), 1 + e 1.05, reciprocal 1, e * r 0.5: sigmoid <= 3.7, so
// with the last product p is within 4.2 * 2^-23 of the exact value, under
// 9 units in the last place of p's own binade. mxsg_sigmoid_sweep exposes
// the fast sigmoid so that its error can be checked on all 65536 bf16
// gates (bound used below: 2^-21, i.e. p within 9 ulps). Rounding p to bf16
// then gives the correctly rounded result unless p's low 16 bits lie within
// kTieUlps of 0x8000 (a bf16 midpoint). Those elements, and all outside the
// fast path's range (|g| > 64, zero, subnormal-range or overflowing p, NaN,
// Inf), take the fp64 path below.
constexpr float kL2eHi = 1.44268798828125f;          // log2(e) to 15 significant bits
constexpr float kL2eLo = 7.052607543300837e-06f;     // log2(e) - kL2eHi
constexpr int kTieUlps = 16;

// fast sigmoid(g) for |g| <= 64 (fp32; see above)
__device__ __forceinline__ float sigmoid_fast(float g) {
  const float a = __builtin_fabsf(g);
  const float xh = a * kL2eHi;                                  // exact
  const float n = __builtin_rintf(xh);
  const float f = __builtin_fmaf(a, kL2eLo, xh - n);            // xh - n exact
  const float e = __builtin_ldexpf(__builtin_amdgcn_exp2f(-f), -(int)n);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return g >= 0.0f ? r : e * r;
}

// fp64 path: the same formula in double (relative error < 2^-50), rounded to
// bf16 directly from the double. When that double lies within 2^-45 of a
// bf16 midpoint M, the side of M is decided from exact relations instead.
// With P = |g * u| (exact) and |silu(g) * u| = P / (1 + exp(-g)):
//   P <= M                 -> below M (the sigmoid is < 1);
//   else below M iff P - 2M < M expm1(-g), used for |g| < 1 (sigmoid in
//     (0.27, 0.73), so M < P < 4M and P - 2M is exact; expm1 keeps the
//     small difference 1 - exp(-g) that exp itself would round away);
//   else for g >= 1 iff P - M < M exp(-g) (P <= 2M: P - M exact), and for
//     g <= -1 iff P - M < M exp(|g|).
// (Only a value within ~2^-50 of M itself, which needs more than double
// precision, could still be misjudged.)
__device__ __attribute__((noinline)) uint32_t swiglu_bf16_fp64(float gf, float uf) {
  const double g = gf, u = uf;
  const double a = __builtin_fabs(g);
  const double e = exp(-a);
  const double sig = g >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
  const double p = (g * u) * sig;
  const uint32_t sign = __builtin_signbit(p) ? 0x8000u : 0u;
  const double ap = __builtin_fabs(p);
  if (!(ap == ap)) return 0x7FC0u | sign;                      // NaN
  if (ap == __builtin_inf()) return 0x7F80u | sign;
  if (ap == 0.0) return sign;
  int ex;
  (void)__builtin_frexp(ap, &ex);                               // ap in [2^(ex-1), 2^ex)
  const int eb = ex - 1 < -126 ? -126 : ex - 1;
  const double q = __builtin_ldexp(1.0, eb - 7);                // bf16 spacing around ap
  const double t = ap / q;                                      // exact
  const double k = __builtin_floor(t);
  const double frac = t - k;
  bool up;
  if (__builtin_fabs(frac - 0.5) * q > 0x1p-45 * ap) {
    up = frac > 0.5;
  } else {
    const double P = __builtin_fabs(g * u), M = (k + 0.5) * q;
    bool below;
    if (P <= M) below = true;
    else if (a < 1.0) below = P - 2.0 * M < M * expm1(-g);
    else if (g > 0.0) below = P - M < M * e;
    else below = P - M < M * exp(a);
    up = !below;
  }
  const float r = (float)((up ? k + 1.0 : k) * q);             // exact, or +inf past the bf16 range
  return (__float_as_uint(r) >> 16) | sign;
}

// bf16 bits of the activation; *tie = true when the fp64 path must decide
__device__ __forceinline__ uint32_t swiglu_fast(float g, float u, bool &redo) {
  const float p = (g * u) * sigmoid_fast(g);
  const uint32_t b = __float_as_uint(p);
  const uint32_t ex = (b >> 23) & 0xFFu;
  const int lo = (int)(b & 0xFFFFu) - 0x8000;
  redo = !(__builtin_fabsf(g) <= 64.0f) || ex < 24u || ex > 253u || (lo <= kTieUlps && lo >= -kTieUlps);
  return (b + 0x8000u) >> 16;                                   // nearest (not a tie here)
}

// eight activations (one 16-byte chunk) from a gate chunk and an up chunk
__device__ __forceinline__ uint4 swiglu8(uint4 g, uint4 u) {
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
  uint32_t redo = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bool r0, r1;
    const uint32_t lo = swiglu_fast(bf16_lo(gw[i]), bf16_lo(uw[i]), r0);
    const uint32_t hi = swiglu_fast(bf16_hi(gw[i]), bf16_hi(uw[i]), r1);
    o[i] = lo | (hi << 16);
    redo |= (r0 ? 1u : 0u) << (2 * i);
    redo |= (r1 ? 1u : 0u) << (2 * i + 1);
  }
  if (redo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (redo & (1u << (2 * i)))
        o[i] = (o[i] & 0xFFFF0000u) | swiglu_bf16_fp64(bf16_lo(gw[i]), bf16_lo(uw[i]));
      if (redo & (2u << (2 * i)))
        o[i] = (o[i] & 0x0000FFFFu) | (swiglu_bf16_fp64(bf16_hi(gw[i]), bf16_hi(uw[i])) << 16);
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// amax of the SwiGLU activation of x [M, 2C] (tensorwise scaling of a fused
// SwiGLU operand): 16-byte chunks of the gate half, each with its up chunk;
// the result is max-reduced into *amax_bits (starts at 0).
__global__ __launch_bounds__(256) void amax_swiglu_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                          int64_t C, uint32_t *__restrict__ amax_bits,
                                                          int32_t *__restrict__ status) {
  const int64_t cpr = C / 8;  // chunks per row
  const int64_t n = M * cpr;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cpr, c = (i - r * cpr) * 8;
    const uint16_t *src = x + r * 2 * C + c;
    m = absmax_bits8(swiglu8(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + C)), m);
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    if (m) atomic_max_bits(amax_bits, m << 16);
    flag_nonfinite(status, m);
  }
}

// the SwiGLU activation itself: y [M, C] bf16 from x [M, 2C], one 16-byte
// output chunk per thread
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t C,
                                                     uint16_t *__restrict__ y) {
  const int64_t cpr = C / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * cpr) return;
  const int64_t r = i / cpr, c = (i - r * cpr) * 8;
  const uint16_t *src = x + r * 2 * C + c;
  *reinterpret_cast<uint4 *>(y + r * C + c) =
      swiglu8(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + C));
}

// the fast-path sigmoid of every bf16 bit pattern (65536 outputs)
__global__ __launch_bounds__(256) void sigmoid_sweep_kernel(float *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 65536) out[i] = sigmoid_fast(bf16_lo((uint32_t)i));
}

// Padded start of the tile and its source rows. Returns false if the tile is
// past the last group. Uses LDS `scan` (>= 65 ints).
__device__ bool locate_padded_tile(const TileArgs &a, int64_t p0, int64_t &src0, int &nvalid,
                                   int32_t *scan) {
  // P_g prefix over groups, 64 groups per pass on wave 0, broadcast via LDS
  const int lane = threadIdx.x & 63;
  __shared__ int64_t s_src0;
  __shared__ int s_nvalid, s_found;
  if (threadIdx.x == 0) s_found = 0;
  __syncthreads();
  if (threadIdx.x < 64) {
    int64_t base = 0;  // P of the first group of this pass
    for (int g0 = 0; g0 < a.E; g0 += 64) {
      const int g = g0 + lane;
      int64_t lo = 0, hi = 0;
      if (g < a.E) group_bounds(a.ends, g, a.rows, lo, hi);
      const int64_t m = hi - lo;
      const int64_t padm = ((m + QT - 1) / QT) * QT;
      // inclusive scan of padm over the wave
      int64_t incl = padm;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int64_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int64_t start = base + incl - padm;
      if (g < a.E && p0 >= start && p0 < start + padm) {
        s_src0 = lo + (p0 - start);
        int64_t nv = m - (p0 - start);
        s_nvalid = (int)(nv > QT ? QT : nv);
        s_found = 1;
      }
      if (a.padded_out && blockIdx.x == 0 && blockIdx.z == 0 && g < a.E) {
        a.padded_out[g + 1] = (int32_t)(start + padm);
        if (g == 0) a.padded_out[0] = 0;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  src0 = s_src0;
  nvalid = s_nvalid;
  return s_found != 0;
}

template <int RECIPE, int FMT, bool ROW, bool COL>
__global__ __launch_bounds__(QTHREADS) void tile_quant_kernel(TileArgs a) {
  // 4-bit codes (MXFP4) exist for the MX recipe only; two codes per byte
  static_assert(FMT != kE2M1 || RECIPE == kMx || RECIPE == kNvfp4, "e2m1 codes are MX- or NVFP4-scaled");
  static_assert(RECIPE != kNvfp4 || FMT == kE2M1, "NVFP4 elements are e2m1");
  constexpr bool FP4 = FMT == kE2M1;
  __shared__ __attribute__((aligned(16))) uint16_t tile[QT * QT];       // bf16, row stride 256 B
  // codes [feature][pos] of the column-wise output, in the same LDS as the
  // bf16 tile (written once every thread has read its columns)
  uint8_t *const ctile = reinterpret_cast<uint8_t *>(tile);
  static_assert(QT * CODE_LD <= QT * QT * 2, "code tile fits in the bf16 tile");
  __shared__ uint32_t colmax[4][QT];
  __shared__ uint32_t red[4];
  __shared__ int32_t scan[72];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t b = blockIdx.z;
  // grid.x = row tiles x feature tiles, in groups of `rgroup` row tiles: the
  // feature tile runs slowest within a group, the row tile fastest. With
  // rgroup = 1 consecutive workgroups read the 256-byte pieces of the same 128
  // rows; with rgroup > 1 they also write adjacent 128-position pieces of the
  // same column-wise feature rows.
  const int nft = (int)(a.C / QT);
  int ftile;
  int64_t rtile;
  {
    const int64_t nrt = gridDim.x / (unsigned)nft;
    const int64_t per = (int64_t)a.rgroup * nft;
    const int64_t grp = blockIdx.x / per;
    const int64_t within = blockIdx.x - grp * per;
    const int64_t g0 = grp * a.rgroup;
    const int gs = (int)(nrt - g0 < a.rgroup ? nrt - g0 : a.rgroup);
    ftile = (int)(within / gs);
    rtile = g0 + within % gs;
  }
  const int64_t c0 = (int64_t)ftile * QT;
  const uint16_t *x = a.x + b * a.x_bstride;

  // the tensor scale (tensorwise / delayed) is written first, so that it is
  // there even when no tile holds a row (an empty tensor or empty groups)
  if (RECIPE == kNvfp4 && blockIdx.x == 0 && t == 0) {
    const float st = nv_tensor_scale(a.amax[b]);
    if (a.row_scales) reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(a.row_scales) + a.rs_tail)[b] = st;
    if (a.col_scales) reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(a.col_scales) + a.cs_tail)[b] = st;
  }
  if ((RECIPE == kTensorwise || RECIPE == kDelayed) && blockIdx.x == 0 &&
      t == 0) {
    float s0 = 1.0f, i0 = 1.0f;
    if (RECIPE == kTensorwise)
      scale_pair<FMT>(a.amax[b], s0, i0);
    else
      s0 = a.dl_scale[b];
    if (a.row_scales) reinterpret_cast<float *>(a.row_scales)[b] = s0;
    if (a.col_scales) reinterpret_cast<float *>(a.col_scales)[b] = s0;
  }

  // which rows does this tile cover?
  int64_t src0 = 0, p0 = 0;
  int nvalid = 0;
  if (COL) {
    p0 = rtile * QT;
    if (a.E > 0) {
      if (!locate_padded_tile(a, p0, src0, nvalid, scan)) return;
    } else {  // weights: one group of all rows, rows % 128 == 0
      src0 = p0;
      nvalid = 128;
    }
  } else {
    src0 = rtile * QT;
    int64_t nv = a.rows - src0;
    nvalid = (int)(nv > QT ? QT : nv);
  }

  // ---- load: chunk id = u*256 + t, row = id / 16, 16-byte chunk = id % 16
  const int cq = t & 15;   // chunk within the row (8 features)
  const int rq = t >> 4;   // row offset within a 16-row slab
  uint4 v[8];
  if (a.swiglu) {
    // gate/up rows of 2C: gate at column c, up at column C + c
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = u * 16 + rq;
      if (r < nvalid) {
        const uint16_t *src = x + (src0 + r) * (2 * a.C) + c0 + cq * 8;
        const uint4 gv = a.stream_x ? load16_stream(src) : *reinterpret_cast<const uint4 *>(src);
        const uint4 uv = a.stream_x ? load16_stream(src + a.C) : *reinterpret_cast<const uint4 *>(src + a.C);
        v[u] = swiglu8(gv, uv);
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = u * 16 + rq;
      if (r < nvalid) {
        const uint16_t *src = x + source_row(a.row_index, a.src_rows, src0 + r) * a.C + c0 + cq * 8;
        v[u] = a.stream_x ? load16_stream(src) : *reinterpret_cast<const uint4 *>(src);
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // ---- tensor-level scale (tensorwise / delayed)
  float t_s = 1.0f, t_inv = 1.0f;
  if (RECIPE == kTensorwise) {
    scale_pair<FMT>(a.amax[b], t_s, t_inv);
  } else if (RECIPE == kNvfp4) {
    t_s = nv_tensor_scale(a.amax[b]);
  } else if (RECIPE == kDelayed) {
    t_s = a.dl_scale[b];
    t_inv = a.dl_inv[b];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = absmax_bits8(v[u], m);
    m = wave_max_u32(m);
    if (lane == 0) red[wave] = m;
  } else if (RECIPE == kTile128) {
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = absmax_bits8(v[u], m);
    m = wave_max_u32(m);
    if (lane == 0) red[wave] = m;
  }
  if (RECIPE == kDelayed || RECIPE == kTile128) {
    __syncthreads();
    const uint32_t m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    if (t == 0) flag_nonfinite(a.status, m);
    if (RECIPE == kDelayed) {
      if (t == 0 && m) atomic_max_bits(reinterpret_cast<uint32_t *>(a.amax + b), m << 16);
    } else {
      scale_pair<FMT>(bits_to_amax(m), t_s, t_inv);
      if (t == 0) {
        // 128x128 tile scale: [K/128, N/128] per expert, shared by both layouts
        const int64_t idx = b * a.rs_bstride + rtile * (a.C / QT) + ftile;
        if (a.row_scales) reinterpret_cast<float *>(a.row_scales)[idx] = t_s;
        if (a.col_scales) reinterpret_cast<float *>(a.col_scales)[idx] = t_s;
      }
    }
  }

  // ---- row-wise output
  if (ROW) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = u * 16 + rq;
      float inv = t_inv;
      if (RECIPE == kBlockwise) {  // 1x128: the 16 lanes holding this row
        uint32_t m = absmax_bits8(v[u], 0);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, o, 64));
        if (cq == 0) flag_nonfinite(a.status, m);
        float s;
        scale_pair<FMT>(bits_to_amax(m), s, inv);
        if (cq == 0 && r < nvalid)
          reinterpret_cast<float *>(a.row_scales)[b * a.rs_bstride + (src0 + r) * (a.C / QT) +
                                                  ftile] = s;
      } else if (RECIPE == kNvfp4) {  // 1x16: the 2 lanes holding 16 features
        uint32_t m = absmax_bits8(v[u], 0);
        m = umax(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        if ((cq & 1) == 0) flag_nonfinite(a.status, m);
        const uint32_t code = nv_block_scale(bits_to_amax(m), t_s, inv);
        // piece-major: 8 scale bytes per row per 128-element piece, rows consecutive
        if ((cq & 1) == 0 && r < nvalid)
          reinterpret_cast<uint8_t *>(a.row_scales)[b * a.rs_bstride + ((c0 / QT) * a.rows + src0 + r) * 8 +
                                                    (cq >> 1)] = (uint8_t)code;
      } else if (RECIPE == kMx) {  // 1x32: the 4 lanes holding 32 features
        uint32_t m = absmax_bits8(v[u], 0);
        m = umax(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        m = umax(m, (uint32_t)__shfl_xor((int)m, 2, 64));
        if ((cq & 3) == 0) flag_nonfinite(a.status, m);
        const int k = mx_exponent<FMT>(bits_to_amax(m));
        inv = exp2_neg(k);
        // word-major E8M0 layout: word c0/128 of every row, then the next word
        if ((cq & 3) == 0 && r < nvalid)
          reinterpret_cast<uint8_t *>(a.row_scales)[b * a.rs_bstride + ((c0 / QT) * a.rows + src0 + r) * 4 +
                                                    (cq >> 2)] = (uint8_t)(k + 127);
      }
      if (r < nvalid) {
        if constexpr (FP4) {
          const uint32_t q = cvt8_e2m1(v[u], inv);
          // MXFP4: elements in order; NVFP4: the dword of (step cq / 2, half cq % 2)
          const int64_t col = RECIPE == kNvfp4 ? c0 / 2 + nv_dword_off(cq >> 1, cq & 1) : (c0 + cq * 8) / 2;
          *reinterpret_cast<uint32_t *>(a.row_codes + b * a.row_bstride + pi_off(src0 + r, col, a.C / 2)) = q;
        } else {
          const uint2 q = cvt8<FMT>(v[u], inv);
          store8_stream(a.row_codes + b * a.row_bstride + pi_off(src0 + r, c0 + cq * 8, a.C), q);
        }
      }
    }
  }

  if (!COL) return;

  // ---- column-wise output: stage the bf16 tile in LDS
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = u * 16 + rq;
    *reinterpret_cast<uint4 *>(&tile[r * QT + cq * 8]) = v[u];
  }
  __syncthreads();

  // thread -> feature pair fp (features 2fp, 2fp+1), row quarter q (32 rows)
  const int fp = t & 63;
  const int q = t >> 6;
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = *reinterpret_cast<const uint32_t *>(&tile[(q * 32 + i) * QT + fp * 2]);

  float inv0 = t_inv, inv1 = t_inv;
  float nvi[2][2];  // NVFP4: multipliers of [feature 2fp, 2fp + 1][block 2q, 2q + 1]
  if (RECIPE == kNvfp4) {  // 16x1 units: two per quarter column
    uint32_t m[2][2] = {{0, 0}, {0, 0}};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      m[0][i >> 4] = umax(m[0][i >> 4], w[i] & 0x7fffu);
      m[1][i >> 4] = umax(m[1][i >> 4], (w[i] >> 16) & 0x7fffu);
    }
    flag_nonfinite(a.status, umax(umax(m[0][0], m[0][1]), umax(m[1][0], m[1][1])));
    uint8_t *cs = reinterpret_cast<uint8_t *>(a.col_scales) + b * a.cs_bstride;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t code = nv_block_scale(bits_to_amax(m[f][k]), t_s, nvi[f][k]);
        // piece-major [ld/128, C, 8]: piece p0/128, feature row c, block 2q + k
        cs[((p0 / QT) * a.C + c0 + 2 * fp + f) * 8 + 2 * q + k] = (uint8_t)code;
      }
  }
  if (RECIPE == kBlockwise || RECIPE == kMx) {
    uint32_t m0 = 0, m1 = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      m0 = umax(m0, w[i] & 0x7fffu);
      m1 = umax(m1, (w[i] >> 16) & 0x7fffu);
    }
    flag_nonfinite(a.status, umax(m0, m1));
    if (RECIPE == kMx) {  // 32x1 units: one quarter of the tile column
      const int k0 = mx_exponent<FMT>(bits_to_amax(m0));
      const int k1 = mx_exponent<FMT>(bits_to_amax(m1));
      inv0 = exp2_neg(k0);
      inv1 = exp2_neg(k1);
      uint8_t *cs = reinterpret_cast<uint8_t *>(a.col_scales) + b * a.cs_bstride;
      // word-major [C, ld/32]: word p0/128 of feature row c, byte q
      const int64_t wrow = (p0 / QT) * a.C + c0 + 2 * fp;
      cs[wrow * 4 + q] = (uint8_t)(k0 + 127);
      cs[(wrow + 1) * 4 + q] = (uint8_t)(k1 + 127);
    } else {  // 128x1 units: the whole tile column, reduce the 4 quarters
      colmax[q][2 * fp] = m0;
      colmax[q][2 * fp + 1] = m1;
      __syncthreads();
      m0 = umax(umax(colmax[0][2 * fp], colmax[1][2 * fp]), umax(colmax[2][2 * fp], colmax[3][2 * fp]));
      m1 = umax(umax(colmax[0][2 * fp + 1], colmax[1][2 * fp + 1]),
                umax(colmax[2][2 * fp + 1], colmax[3][2 * fp + 1]));
      float s0, s1;
      scale_pair<FMT>(bits_to_amax(m0), s0, inv0);
      scale_pair<FMT>(bits_to_amax(m1), s1, inv1);
      if (q == 0) {
        float *cs = reinterpret_cast<float *>(a.col_scales) + b * a.cs_bstride;
        const int64_t ldb = a.ld / QT;
        cs[(c0 + 2 * fp) * ldb + p0 / QT] = s0;
        cs[(c0 + 2 * fp + 1) * ldb + p0 / QT] = s1;
      }
    }
  }

  // the code tile overwrites the bf16 tile: every thread must have read its
  // columns first (blockwise already synchronized after its column maxima)
  if (RECIPE != kBlockwise) __syncthreads();

  // codes of the two columns, 32 rows each -> LDS code tile [feature][pos]
  uint8_t *cc = a.col_codes + b * a.col_bstride;
  if constexpr (FP4) {
    // 32 codes of a column = 16 bytes: nibble i of dword j is row 8j + i
    uint32_t d0[4], d1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t *wj = &w[8 * j];
      // NVFP4: rows 16k .. 16k + 15 of the quarter share block 2q + k
      const float i0 = RECIPE == kNvfp4 ? nvi[0][j >> 1] : inv0;
      const float i1 = RECIPE == kNvfp4 ? nvi[1][j >> 1] : inv1;
      uint32_t x = 0, y = 0;
      x = e2m1_pk<0>(x, bf16_lo(wj[0]) * i0, bf16_lo(wj[1]) * i0);
      x = e2m1_pk<1>(x, bf16_lo(wj[2]) * i0, bf16_lo(wj[3]) * i0);
      x = e2m1_pk<2>(x, bf16_lo(wj[4]) * i0, bf16_lo(wj[5]) * i0);
      x = e2m1_pk<3>(x, bf16_lo(wj[6]) * i0, bf16_lo(wj[7]) * i0);
      y = e2m1_pk<0>(y, bf16_hi(wj[0]) * i1, bf16_hi(wj[1]) * i1);
      y = e2m1_pk<1>(y, bf16_hi(wj[2]) * i1, bf16_hi(wj[3]) * i1);
      y = e2m1_pk<2>(y, bf16_hi(wj[4]) * i1, bf16_hi(wj[5]) * i1);
      y = e2m1_pk<3>(y, bf16_hi(wj[6]) * i1, bf16_hi(wj[7]) * i1);
      d0[j] = x;
      d1[j] = y;
    }
    if constexpr (RECIPE == kNvfp4) {
      // dword j of this quarter = rows 32q + 8j .. + 7 = step 2q + j / 2, half j % 2
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = nv_dword_off(2 * q + (j >> 1), j & 1);
        *reinterpret_cast<uint32_t *>(&ctile[(2 * fp) * CODE_LD4 + off]) = d0[j];
        *reinterpret_cast<uint32_t *>(&ctile[(2 * fp + 1) * CODE_LD4 + off]) = d1[j];
      }
    } else {
      *reinterpret_cast<uint4 *>(&ctile[(2 * fp) * CODE_LD4 + q * 16]) = make_uint4(d0[0], d0[1], d0[2], d0[3]);
      *reinterpret_cast<uint4 *>(&ctile[(2 * fp + 1) * CODE_LD4 + q * 16]) =
          make_uint4(d1[0], d1[1], d1[2], d1[3]);
    }
    __syncthreads();
    // 128 feature rows x 64 bytes; 4 lanes per row
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = u * QTHREADS + t;
      const int f = id >> 2, ch = id & 3;
      const uint4 val = *reinterpret_cast<const uint4 *>(&ctile[f * CODE_LD4 + ch * 16]);
      store16_stream(cc + pi_off(c0 + f, p0 / 2 + ch * 16, a.ld / 2), val);
    }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < 32; i += 16) {
      uint32_t d0[4], d1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = i + 4 * j;
        d0[j] = cvt4<FMT>(bf16_lo(w[r]) * inv0, bf16_lo(w[r + 1]) * inv0, bf16_lo(w[r + 2]) * inv0,
                          bf16_lo(w[r + 3]) * inv0);
        d1[j] = cvt4<FMT>(bf16_hi(w[r]) * inv1, bf16_hi(w[r + 1]) * inv1, bf16_hi(w[r + 2]) * inv1,
                          bf16_hi(w[r + 3]) * inv1);
      }
      *reinterpret_cast<uint4 *>(&ctile[(2 * fp) * CODE_LD + q * 32 + i]) =
          make_uint4(d0[0], d0[1], d0[2], d0[3]);
      *reinterpret_cast<uint4 *>(&ctile[(2 * fp + 1) * CODE_LD + q * 32 + i]) =
          make_uint4(d1[0], d1[1], d1[2], d1[3]);
    }
    __syncthreads();

    // coalesced write-out: 128 feature rows x 128 bytes; 8 lanes per row
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = u * QTHREADS + t;
      const int f = id >> 3, ch = id & 7;
      const uint4 val = *reinterpret_cast<const uint4 *>(&ctile[f * CODE_LD + ch * 16]);
      store16_stream(cc + pi_off(c0 + f, p0 + ch * 16, a.ld), val);
    }
  }
}

// ---------------------------------------------------------------------------
// delayed-scaling update: one workgroup per unit

template <int FMT>
__global__ __launch_bounds__(256) void delayed_update_kernel(float *__restrict__ hist,
                                                             int32_t *__restrict__ pos,
                                                             float *__restrict__ amax,
                                                             float *__restrict__ scale,
                                                             float *__restrict__ inv, int L) {
  const int u = blockIdx.x;
  float *h = hist + (int64_t)u * L;
  int p = pos[u];
  p = p < 0 ? 0 : (p >= L ? L - 1 : p);
  const float am = amax[u];
  __syncthreads();  // every thread has read pos / amax before they change
  if (threadIdx.x == 0) h[p] = am;
  __syncthreads();
  // max over the ring; NaN / Inf propagate as "non-finite"
  float m = 0.0f;
  bool bad = false;
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    const float hv = (i == p) ? am : h[i];
    bad |= !(hv == hv) || hv == __builtin_inff();
    m = hv > m ? hv : m;
  }
  __shared__ float red[256];
  __shared__ int sbad[256];
  red[threadIdx.x] = m;
  sbad[threadIdx.x] = bad;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
      sbad[threadIdx.x] |= sbad[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float a = red[0];
    if (!sbad[0] && a > 0.0f) {
      scale[u] = __fdiv_rn(a, Fp8<FMT>::fmax);
      inv[u] = __fdiv_rn(Fp8<FMT>::fmax, a);
    }
    pos[u] = (p + 1) % L;
    amax[u] = 0.0f;
  }
}

// ---------------------------------------------------------------------------
// exhaustive cast check: out[i] = code(float(start + i))

template <int FMT>
__global__ __launch_bounds__(256) void cast_sweep_kernel(uint32_t start, int64_t n,
                                                         uint8_t *__restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  const uint32_t s = start + (uint32_t)i4;
  uint32_t c;
  if constexpr (FMT == kE2M1) {  // one 4-bit code per output byte
    const uint32_t p = e2m1_pk<1>(e2m1_pk<0>(0u, __uint_as_float(s), __uint_as_float(s + 1)),
                                  __uint_as_float(s + 2), __uint_as_float(s + 3));
    c = (p & 0xfu) | ((p & 0xf0u) << 4) | ((p & 0xf00u) << 8) | ((p & 0xf000u) << 12);
  } else {
    c = cvt4<FMT>(__uint_as_float(s), __uint_as_float(s + 1), __uint_as_float(s + 2),
                  __uint_as_float(s + 3));
  }
  if (i4 + 4 <= n) {
    *reinterpret_cast<uint32_t *>(out + i4) = c;
  } else {
    for (int j = 0; (int64_t)(i4 + j) < n; ++j) out[i4 + j] = (uint8_t)(c >> (8 * j));
  }
}

// ---------------------------------------------------------------------------
// streaming device copy (the HBM reference rate): one 16-byte chunk per thread

__global__ __launch_bounds__(256) void stream_copy_kernel(const uint8_t *__restrict__ src,
                                                          uint8_t *__restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) store16_stream(dst + 16 * i, load16_stream(src + 16 * i));
}

// ---------------------------------------------------------------------------
// launchers

static int tiles_of(int64_t n) { return (int)((n + QT - 1) / QT); }

// inputs above this size cannot stay in the last-level cache (256 MiB) for a
// later pass anyway, so the tile pass streams them past it
constexpr int64_t kStreamBytes = (int64_t)256 << 20;

// Launch-order group (row tiles) of a weight pass with k-major output. A group
// of g row tiles makes the workgroups in flight together write g adjacent
// 128-position pieces of each k-major row instead of one, which lets the
// scattered column-wise writes use HBM better. Measured per pass (weights of
// the Mixtral, DeepSeek and Llama4 shapes): 16 is best when the bf16 row
// stride is not a multiple of 32 KiB, and slower than 8 when it is (then the
// half-width row slices in flight read fewer distinct channel offsets).
static int weight_col_group(int64_t C) { return (C * 2) % 32768 == 0 ? 8 : 16; }

hipError_t launch_zero(float *p, int n, hipStream_t st) {
  zero_f32_kernel<<<(n + 255) / 256, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_check_ends(const int32_t *ends, int E, int64_t M, int32_t *status, hipStream_t st) {
  if (E <= 0 || !status) return hipSuccess;
  check_ends_kernel<<<1, 256, 0, st>>>(ends, E, M, status);
  return hipGetLastError();
}

hipError_t launch_amax(const uint16_t *x, int units, int64_t unit_elems, float *amax,
                       int32_t *status, hipStream_t st) {
  hipError_t e = launch_zero(amax, units, st);
  if (e != hipSuccess) return e;
  if (unit_elems == 0) return hipSuccess;
  int64_t nvec = unit_elems / 8;
  int64_t blocks = (nvec + 256 * 8 - 1) / (256 * 8);  // ~8 vectors per thread
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks, (unsigned)units);
  amax_kernel<<<grid, 256, 0, st>>>(x, unit_elems, reinterpret_cast<uint32_t *>(amax), status);
  return hipGetLastError();
}

template <int RECIPE, int FMT>
static hipError_t tile_dispatch(const TileArgs &a, bool row, bool col, dim3 grid, hipStream_t st) {
  if (row && col)
    tile_quant_kernel<RECIPE, FMT, true, true><<<grid, QTHREADS, 0, st>>>(a);
  else if (row)
    tile_quant_kernel<RECIPE, FMT, true, false><<<grid, QTHREADS, 0, st>>>(a);
  else
    tile_quant_kernel<RECIPE, FMT, false, true><<<grid, QTHREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t tile_by_recipe(int recipe, const TileArgs &a, bool row, bool col, dim3 grid,
                                 hipStream_t st) {
  switch (recipe) {
    case kTensorwise: return tile_dispatch<kTensorwise, FMT>(a, row, col, grid, st);
    case kDelayed: return tile_dispatch<kDelayed, FMT>(a, row, col, grid, st);
    case kBlockwise: return tile_dispatch<kBlockwise, FMT>(a, row, col, grid, st);
    case kMx: return tile_dispatch<kMx, FMT>(a, row, col, grid, st);
    case kTile128: return tile_dispatch<kTile128, FMT>(a, row, col, grid, st);
    default: return hipErrorInvalidValue;  // NVFP4 has e2m1 elements only
  }
}

hipError_t launch_swiglu(const uint16_t *x, int64_t M, int64_t C, uint16_t *y, hipStream_t st) {
  const int64_t n = M * (C / 8);
  if (n == 0) return hipSuccess;
  swiglu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, M, C, y);
  return hipGetLastError();
}

hipError_t launch_sigmoid_sweep(float *out, hipStream_t st) {
  sigmoid_sweep_kernel<<<256, 256, 0, st>>>(out);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const QuantActParams &p, hipStream_t st) {
  hipError_t e;
  // tensorwise and NVFP4 (its tensor scale) need the tensor's amax first
  const bool tensor_amax = p.recipe == kTensorwise || p.recipe == kNvfp4;
  if (tensor_amax && p.swiglu) {
    // the amax is that of the activation, computed from gate and up
    e = launch_zero(p.amax, 1, st);
    if (e != hipSuccess) return e;
    const int64_t n = p.M * (p.C / 8);
    if (n > 0) {
      int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
      blocks = blocks > 4096 ? 4096 : (blocks < 1 ? 1 : blocks);
      amax_swiglu_kernel<<<(unsigned)blocks, 256, 0, st>>>(p.x, p.M, p.C, reinterpret_cast<uint32_t *>(p.amax),
                                                           p.status);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (tensor_amax) {
    if (p.row_index) {
      e = launch_zero(p.amax, 1, st);
      if (e != hipSuccess) return e;
      if (p.M > 0) {
        const unsigned blocks = (unsigned)(p.M < 8192 ? p.M : 8192);
        amax_rows_kernel<<<blocks, 256, 0, st>>>(p.x, p.C, p.row_index, p.M, p.src_rows,
                                                 reinterpret_cast<uint32_t *>(p.amax), p.status);
        e = hipGetLastError();
      }
    } else {
      e = launch_amax(p.x, 1, p.M * p.C, p.amax, p.status, st);
    }
    if (e != hipSuccess) return e;
  }
  TileArgs a{};
  a.x = p.x;
  a.rows = p.M;
  a.C = p.C;
  a.E = p.E;
  a.ends = p.group_ends;
  a.row_codes = p.row_codes;
  a.row_scales = p.row_scales;
  a.col_codes = p.col_codes;
  a.col_scales = p.col_scales;
  a.ld = p.ld;
  a.padded_out = p.padded_starts;
  a.amax = p.amax;
  a.dl_scale = p.dl_scale;
  a.dl_inv = p.dl_inv;
  // a gathered operand re-reads token rows (one read per routed copy): those
  // reads can hit the last-level cache whenever the token tensor fits in it
  a.stream_x = (p.row_index ? p.src_rows : p.M) * p.C * 2 > kStreamBytes;
  a.row_index = p.row_index;
  a.src_rows = p.src_rows;
  a.status = p.status;
  const bool row = p.row_codes != nullptr, col = p.col_codes != nullptr;
  a.rgroup = 1;  // token passes: feature tile fastest (measured best)
  a.swiglu = p.swiglu;
  if (p.swiglu) a.stream_x = p.M * p.C * 4 > kStreamBytes;
  a.rs_tail = p.M * (p.C / 16);      // NVFP4: the tensor scale follows the block scales
  a.cs_tail = p.C * (p.ld / 16);
  // at least one tile: an empty tensor still gets its tensor scale written
  int64_t ytiles = col ? p.ld / QT : tiles_of(p.M);
  if (ytiles == 0) ytiles = 1;
  const int64_t tiles = ytiles * (p.C / QT);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)tiles, 1, 1);
  if (p.fmt == kE2M1)
    return p.recipe == kNvfp4 ? tile_dispatch<kNvfp4, kE2M1>(a, row, col, grid, st)
                              : tile_dispatch<kMx, kE2M1>(a, row, col, grid, st);
  return p.fmt == kE4M3 ? tile_by_recipe<kE4M3>(p.recipe, a, row, col, grid, st)
                        : tile_by_recipe<kE5M2>(p.recipe, a, row, col, grid, st);
}

hipError_t launch_quantize_weight(const QuantWeightParams &p, hipStream_t st) {
  hipError_t e;
  if (p.recipe == kTensorwise || p.recipe == kNvfp4) {
    e = launch_amax(p.w, p.E, p.K * p.N, p.amax, p.status, st);
    if (e != hipSuccess) return e;
  }
  TileArgs a{};
  a.x = p.w;
  a.rows = p.K;
  a.C = p.N;
  a.E = 0;
  a.ends = nullptr;
  a.row_codes = p.nmajor_codes;
  a.col_codes = p.kmajor_codes;
  a.ld = p.K;
  a.amax = p.amax;
  a.dl_scale = p.dl_scale;
  a.dl_inv = p.dl_inv;
  a.x_bstride = p.K * p.N;
  a.stream_x = (int64_t)p.E * p.K * p.N * 2 > kStreamBytes;
  a.status = p.status;
  const int64_t code_bytes = p.fmt == kE2M1 ? p.K * p.N / 2 : p.K * p.N;  // per expert
  a.row_bstride = code_bytes;
  a.col_bstride = code_bytes;
  int recipe = p.recipe;
  if (recipe == kBlockwise) {
    recipe = kTile128;
    a.row_scales = p.nmajor_scales;
    a.col_scales = p.kmajor_scales;
    a.rs_bstride = (p.K / QT) * (p.N / QT);
    a.cs_bstride = a.rs_bstride;
  } else if (recipe == kMx) {
    a.row_scales = p.nmajor_scales;  // [E, K, N/32]
    a.col_scales = p.kmajor_scales;  // [E, N, K/32]
    a.rs_bstride = p.K * (p.N / 32);
    a.cs_bstride = p.N * (p.K / 32);
  } else if (recipe == kNvfp4) {
    a.row_scales = p.nmajor_scales;  // [E, N/128, K, 8] block codes, then fp32 [E]
    a.col_scales = p.kmajor_scales;  // [E, K/128, N, 8] block codes, then fp32 [E]
    a.rs_bstride = p.K * (p.N / 16);
    a.cs_bstride = p.N * (p.K / 16);
    a.rs_tail = (int64_t)p.E * a.rs_bstride;
    a.cs_tail = (int64_t)p.E * a.cs_bstride;
  } else {
    a.row_scales = p.nmajor_scales;  // [E]
    a.col_scales = p.kmajor_scales;
  }
  const bool row = p.nmajor_codes != nullptr, col = p.kmajor_codes != nullptr;
  a.rgroup = col ? weight_col_group(p.N) : 1;
  const int64_t tiles = (p.K / QT) * (p.N / QT);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)tiles, 1, (unsigned)p.E);
  if (p.fmt == kE2M1)
    return recipe == kNvfp4 ? tile_dispatch<kNvfp4, kE2M1>(a, row, col, grid, st)
                            : tile_dispatch<kMx, kE2M1>(a, row, col, grid, st);
  return p.fmt == kE4M3 ? tile_by_recipe<kE4M3>(recipe, a, row, col, grid, st)
                        : tile_by_recipe<kE5M2>(recipe, a, row, col, grid, st);
}

hipError_t launch_delayed_update(float *hist, int32_t *pos, float *amax, float *scale, float *inv,
                                 int units, int L, int fmt, hipStream_t st) {
  if (units == 0) return hipSuccess;
  if (fmt == kE4M3)
    delayed_update_kernel<kE4M3><<<units, 256, 0, st>>>(hist, pos, amax, scale, inv, L);
  else
    delayed_update_kernel<kE5M2><<<units, 256, 0, st>>>(hist, pos, amax, scale, inv, L);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  stream_copy_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(
      static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_cast_sweep(uint32_t start, int64_t n, int fmt, uint8_t *out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  if (fmt == kE4M3)
    cast_sweep_kernel<kE4M3><<<(unsigned)blocks, 256, 0, st>>>(start, n, out);
  else if (fmt == kE5M2)
    cast_sweep_kernel<kE5M2><<<(unsigned)blocks, 256, 0, st>>>(start, n, out);
  else
    cast_sweep_kernel<kE2M1><<<(unsigned)blocks, 256, 0, st>>>(start, n, out);
  return hipGetLastError();
}

}  // namespace mxsg
