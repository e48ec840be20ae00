// Grouped FP8 GEMM for the MoE expert layer: forward, dgrad and wgrad over
// per-expert token groups (the grouped_mm that the torchao float8 MoE
// training PR replaces, in its Summary, by run-time quantization followed
// by a scaled grouped matmul, and the backward products its Testing section
// checks).
//
// Every mode is written as C[i, j] = sum_l A[i, l] * B[j, l] with both FP8
// code operands contiguous along the contraction index l:
//   FWD   i = token, j = n, l = k; B = k-major weight codes of expert g
//   DGRAD i = token, j = k, l = n; B = n-major weight codes of expert g
//   WGRAD i = k, j = n, l = padded tokens of group g (column-wise codes)
//
// gfx950 design (tensorwise, delayed and MX recipes; blockwise scaling has
// its own kernel, blockwise_gemm_kernel): a 256-thread workgroup (4 waves,
// 2 x 2) computes a 256 x 256 output tile; each wave owns 128 x 128 as
// 32 x 32 MFMA sub-tiles (v_mfma_scale_f32_32x32x64_f8f6f4). The
// contraction runs in 64-wide stages through a ring of four LDS buffers:
// direct-to-LDS buffer loads (no staging registers) land XOR-swizzled
// 16-byte chunks (bank-conflict-free fragment reads) three stages ahead of
// use. The code operands are pair-interleaved, so a stage
// of 64 bytes over a run of row pairs is whole 128-byte lines. A stage is
// one barrier: its first two MFMAs are issued before it, and after it every
// MFMA slot also issues one copy of the stage R - 1 ahead and part of the
// next stage's fragment reads (into a second register set), so the matrix
// pipe is not left idle while copies go out. Every stage issues the same
// number of copies (stages past the contraction read zeros), so each wait
// count is a constant and the loop has no branch.
// The grid is persistent (one workgroup per CU looping over tiles).
// Tiles never straddle expert groups (row tiles start at a group's first
// row pair; rows of a neighbouring group in the tile are computed and not
// stored); a workgroup finds its group from the device-resident offsets
// (no host sync). Workgroup ids are remapped so
// each XCD (and its L2) works on a contiguous run of tiles.
// Scales: tensorwise / delayed in the epilogue (acc * sA * sB); MX inside
// the MFMA through its per-32-element E8M0 scale operands.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace mxsg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int GBM = 256;   // tile rows (i)
constexpr int GBK = 64;    // contraction per stage (bytes of codes: one 128-byte line of a row pair)
constexpr int SBLK = 128;  // blockwise scaling block along the contraction (two stages)
constexpr int SB_TAB = 512; // blockwise FWD / DGRAD: contraction blocks per tile (L <= 65536)
constexpr int kUnitScale = 127;  // E8M0 code of 1.0

struct GemmArgs {
  const uint8_t *a;
  const uint8_t *b;
  const void *a_scales;
  const void *b_scales;
  void *out;
  const int32_t *ends;
  const int32_t *pstarts;
  int64_t lda, ldb, ldo;
  int64_t M;             // token rows (group ends live in [0, M])
  int64_t I, J, L;       // extents of i and j; L = code bytes of a contraction row (FWD / DGRAD)
  int64_t b_gstride;     // bytes of B per expert (FWD / DGRAD)
  int64_t bs_gstride;    // B scale entries per expert (FWD / DGRAD)
  int64_t sb_l, sb_j;    // blockwise weight scale strides along l-block and j-block
  int E;
  int slots;             // FWD / DGRAD: i-tile slots launched; WGRAD: i-tiles
  int jtiles;
  int nblocks;           // tiles (slots x jtiles, or E x slots x jtiles)
  int accumulate;
  int stream_out;        // FWD / DGRAD: write the bf16 output with streaming stores
  int64_t sa_tail, sb_tail;  // NVFP4: byte offset of the fp32 tensor scales in the scale buffers
};

// Workgroup bid runs on XCD bid % 8. Logical tiles are handed to the XCDs in
// interleaved chunks of XCHUNK consecutive ids: each XCD gets every 8th chunk
// (balanced even when groups differ wildly in size), and the tiles an XCD runs
// together are neighbours in the rasterized order (shared L2 data). Ids past
// the last full round of 8 chunks map to themselves. XCHUNK is 32: one tile
// per CU of an XCD (64 measured neutral to slower for 256x256 tiles).
template <int XCHUNK>
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int round = 8 * XCHUNK;
  if (bid >= (nblocks / round) * round) return bid;
  const int xcd = bid & 7, local = bid >> 3;
  return (local / XCHUNK) * round + xcd * XCHUNK + (local % XCHUNK);
}

// Grouped rasterization: runs of GM consecutive i-tiles sweep all j-tiles,
// so the workgroups an XCD runs at the same time (32, one per CU) cover
// GM x 32/GM tiles and share their A and B stage data through that XCD's L2.
// GM = 4 (4 x 8 tiles) measured 1-3% faster per step than 8 (8 x 4) on every
// workload, and 16 slower.
constexpr int GM = 4;
__device__ __forceinline__ void raster(int lid, int itiles, int jtiles, int &it, int &jt) {
  const int per = GM * jtiles;
  const int grp = lid / per;
  const int first = grp * GM;
  const int gm = (itiles - first) < GM ? (itiles - first) : GM;
  const int r = lid - grp * per;
  it = first + r % gm;
  jt = r / gm;
}

// FWD / DGRAD: find the group and rows of i-tile `slot`. Row tiles lie on
// the grid of row pairs (the codes are pair-interleaved): group g with rows
// [lo, hi) covers pairs [lo/2, (hi+1)/2), cut into tiles of GBM/2 pairs. The
// tile starts at the even row e0; its valid output rows are [ilo, ihi).
// Returns false past the last tile.
__device__ bool locate_row_tile(const GemmArgs &a, int slot, int &g_out, int64_t &e0,
                                int64_t &ilo, int64_t &ihi) {
  __shared__ int s_g, s_found;
  __shared__ int64_t s_e0, s_lo, s_hi;
  if (threadIdx.x == 0) s_found = 0;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t base = 0;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
      const int g = g0 + lane;
      int64_t lo = 0, hi = 0;
      if (g < a.E) group_bounds(a.ends, g, a.M, lo, hi);
      const int64_t ps = lo >> 1, pe = (hi + 1) >> 1;
      const int64_t nt = hi > lo ? (pe - ps + GBM / 2 - 1) / (GBM / 2) : 0;
      int64_t incl = nt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int64_t first = base + incl - nt;
      if (g < a.E && slot >= first && slot < first + nt) {
        const int64_t t0 = 2 * (ps + (int64_t)(slot - first) * (GBM / 2));
        s_g = g;
        s_e0 = t0;
        s_lo = lo > t0 ? lo : t0;
        s_hi = hi < t0 + GBM ? hi : t0 + GBM;
        s_found = 1;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  g_out = s_g;
  e0 = s_e0;
  ilo = s_lo;
  ihi = s_hi;
  return s_found != 0;
}

// Read-only copy source for the stages past a tile's contraction (the ring
// runs in whole turns): zero blockwise scales and NVFP4 block codes (the
// buffer copies, codes and MX scale words, read zeros through an empty
// resource on it instead). Reading it keeps every stage's copy count the
// same, so no wait depends on the stage.
__device__ __attribute__((aligned(1024))) const uint32_t kZeroSrc[256] = {};

// LDS stage tiles hold rows of GBK = 64 code bytes as four 16-byte chunks;
// chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so the lanes of a
// fragment read that share a bank sweep (rows r, r+4, r+8, r+12) hit
// different banks.
__device__ __forceinline__ int swz(int row, int ch) { return row * GBK + ((ch ^ ((row >> 2) & 3)) << 4); }

// The 16x16x128 fragment read (lane l: row l % 16, chunk l / 16) needs
// another placement. A ds_read_b128 serves 16 lanes per cycle: those with
// equal lane bit 5 and equal parity of lane bits 2-4 (measured: among
// sixteen probe patterns, only LDS models of this form give the conflict
// counts seen, with 64 four-byte banks). With the row swizzle above, each
// such read costs twice its conflict-free time; with chunk c of row r at
// c ^ 2 (bit 3 of r), the 16 lanes of every cycle hit 16 distinct bank
// quads.
__device__ __forceinline__ int bswz_chunk(int row, int ch) { return ch ^ (((row >> 3) & 1) << 1); }
__device__ __forceinline__ int bswz(int row, int ch) { return row * GBK + (bswz_chunk(row, ch) << 4); }

// Direct-to-LDS copies (buffer_load_dwordx4 ... lds, global_load_lds_dword(x4)):
// lane L of the wave lands at lds + 16 L (or 4 L); M0 holds the LDS byte
// address.
// Issued through inline asm, so the compiler inserts no waits for them: the
// main loop counts them itself (vmcnt) before each stage's barrier. Nor does
// it pad the wait states the ISA requires before a vector-memory read of an
// SGPR (5 after a VALU write of it, such as the v_readlane that reloads a
// spilled SGPR; 1 after an SALU write of M0). So each copy pads its own: the
// buffer copies read their soffset through an SALU copy made inside the asm
// (an SALU read of a VALU-written SGPR is interlocked), which also puts one
// instruction between the M0 write and the copy, and the per-lane-address
// copies start with s_nop 0. A spilled buffer resource is not covered this
// way; the build checks the device assembly for it (asmcheck.py). Without
// the padding, a few unrelated extra global stores in the kernel were
// enough to move a v_readlane reload of the soffset right before a copy,
// which then loaded whole stages of MX operands from a stale offset.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// Code copies are buffer loads (buffer_load_dwordx4 ... lds): a buffer
// resource (base, size, in SGPRs) per operand and tile, a constant 32-bit
// lane offset and the stage's byte offset in an SGPR, so a copy costs no
// vector ALU work (a 64-bit address per lane and stage cost three VALU ops:
// measured 1-4% of GEMM time, most for MXFP4). A stage past the
// contraction reads through a resource of size 0: every lane is out of
// range, reads nothing and lands zeros.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t num_records) {
  const uint64_t p = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF));  // stride 0: a raw buffer
  r[2] = (int)num_records;
  r[3] = 0x00020000;  // 32-bit data format (raw loads ignore it; it must be valid)
  return r;
}
__device__ __forceinline__ void bdma16(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t *lds) {
  uint32_t t;
  asm volatile("s_mov_b32 %0, %3\n\tbuffer_load_dwordx4 %1, %2, %0 offen lds"
               : "=&s"(t)
               : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr(lds)));
}
__device__ __forceinline__ void bdma4(rsrc_t rs, uint32_t voff, uint32_t soff, void *lds) {
  uint32_t t;  // the soffset through an SALU copy, as in bdma16
  asm volatile("s_mov_b32 %0, %3\n\tbuffer_load_dword %1, %2, %0 offen lds"
               : "=&s"(t)
               : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr(lds)));
}
// The NVFP4 kernel, at its register limit, keeps per-lane 64-bit addresses
// (global_load_lds_dwordx4): four more SGPRs of buffer resources made the
// compiler spill them.
__device__ __forceinline__ void dma16(const uint8_t *src, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr(lds)));
}
__device__ __forceinline__ void dma4(const void *src, void *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_addr(lds)));
}

// MFMA 32x32x64 f8 operand for one lane: the lane's row, and (measured lane
// layout) bytes 0-15 = k in [16h, 16h+16) of the first 32-block, bytes
// 16-31 = k in [32+16h, 48+16h) of the second, h = the lane's half of the
// wave; i.e. 16-byte chunks h and 2 + h of the 64-wide stage row. The scale
// operand of lane i + 32b covers row i and 32-block b.
__device__ __forceinline__ v8i frag(const uint8_t *buf, int row, int h) {
  const uint4 x0 = *reinterpret_cast<const uint4 *>(&buf[swz(row, h)]);
  const uint4 x1 = *reinterpret_cast<const uint4 *>(&buf[swz(row, 2 + h)]);
  return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// the upper 16 bytes of a fragment in the operand's low registers (a 4-bit
// MFMA reads only the first four)
__device__ __forceinline__ v8i upper4(v8i x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7, 4, 5, 6, 7); }

// one stage's operands of one lane, in registers
template <int MI, int NI>
struct Frags {
  v8i a[MI], b[NI];
  int sa[MI], sb[NI];  // MX: the rows' E8M0 words, shifted to this lane's half
};

// MFMA operand format code (cbsz / blgp) of an element format
__host__ __device__ constexpr int mfma_fmt(int f) { return f == kE2M1 ? 4 : f; }

template <int MODE, int RECIPE, int FA, int FB, int BN, bool ACC>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NW = 4;              // waves
  constexpr int WI = NW / 2;         // waves along i (2 along j)
  constexpr int WM = GBM / WI;       // wave tile height along i
  constexpr int WN = BN / 2;         // wave tile width along j
  constexpr int NI = WN / 32;        // 32-wide sub-tiles along j per wave
  constexpr int MI = WM / 32;        // 32-high sub-tiles along i per wave
  constexpr int AQ = GBM / 16 / NW;  // 1 KB copy groups (8 row pairs) of A per wave per stage
  constexpr int BQ = BN / 16 / NW;   // of B
  constexpr bool MX = RECIPE == kMx;
  static_assert(RECIPE != kBlockwise, "blockwise scaling runs in blockwise_gemm_kernel");
  // MXFP4: two e2m1 codes per byte, so a 64-byte stage is 128 contraction
  // elements (four 32-blocks, one E8M0 word per row) and each tile takes two
  // MFMAs per stage, on the first and second 32 bytes of the stage
  constexpr bool FP4 = FA == kE2M1;
  constexpr int EPB = FP4 ? 2 : 1;  // contraction elements per code byte
  constexpr int MPT = FP4 ? 2 : 1;  // MFMAs per tile and stage
  static_assert(!FP4 || (MX && FB == kE2M1), "4-bit operands: MX, both sides");
  static_assert(AQ >= 1 && BQ >= 1 && NI >= 1, "tile shape");
  static_assert(!MX || (MI == 4 && NI == 4 && BN == 256), "MX word layout");

  // the ring's stage buffers of A and B codes (and of their per-stage
  // scale words), always indexed by compile-time constants
  constexpr int R = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t As[R][GBM * GBK];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[R][BN * GBK];
  __shared__ __attribute__((aligned(256))) uint32_t dmy[64];  // target of filler copies
  // MX: per stage buffer, each tile row's E8M0 word (the 32-blocks 4w..4w+3
  // holding the stage's two), stored so the four words one lane needs are
  // contiguous: slot d holds tile row 128 (d / 128) + 32 (d % 4) + (d / 4) % 32
  __shared__ __attribute__((aligned(16))) uint32_t mAr[R][MX ? GBM : 4];
  __shared__ __attribute__((aligned(16))) uint32_t mBr[R][MX ? BN : 4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform (SGPR)
  const int wi = wave >> 1, wj = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;

  // ---- tile coordinates: rows [i0, i0 + GBM) of the tile (i0 even), valid
  // output rows [ilo, ihi); columns [j0, j0 + BN); contraction from l0
  // persistent: the grid is one workgroup per CU (a multiple of 8, so tile
  // vb runs on XCD vb % 8 as it would in a one-tile-per-workgroup grid), each
  // walking the tiles vb = blockIdx.x, + gridDim.x, ...; the next tile's
  // copies then start as soon as this tile's stores are issued
  for (int vb = blockIdx.x; vb < a.nblocks; vb += gridDim.x) {
  const int lid = xcd_remap<32>(vb, a.nblocks);
  int g = 0;
  int64_t i0 = 0, ilo = 0, ihi = 0, j0 = 0, l0 = 0;
  int nsteps = 0;
  if (MODE == kWgrad) {
    const int per_g = a.slots * a.jtiles;
    g = lid / per_g;
    int it, jt;
    raster(lid - g * per_g, a.slots, a.jtiles, it, jt);
    i0 = (int64_t)it * GBM;
    j0 = (int64_t)jt * BN;
    ilo = i0;
    ihi = a.I < i0 + GBM ? a.I : i0 + GBM;
    int64_t p_lo = a.pstarts[g], p_hi = a.pstarts[g + 1];
    const int64_t cap = (a.lda < a.ldb ? a.lda : a.ldb) * EPB;   // token positions
    p_lo = p_lo < 0 ? 0 : (p_lo > cap ? cap : p_lo);
    p_hi = p_hi < p_lo ? p_lo : (p_hi > cap ? cap : p_hi);
    l0 = p_lo & ~(int64_t)127;                       // padded starts are 128-aligned
    nsteps = (int)(((p_hi - l0) / 128) * (128 / (GBK * EPB)));
  } else {
    int slot, jt;
    raster(lid, a.slots, a.jtiles, slot, jt);
    j0 = (int64_t)jt * BN;
    if (!locate_row_tile(a, slot, g, i0, ilo, ihi)) continue;
    l0 = 0;
    nsteps = (int)(a.L / GBK);
  }
  // stages run: rounded up to whole ring turns (a partial turn's code raised
  // register use past the budget)
  const int vsteps = (nsteps + 3) & ~3;

  // ---- per-lane byte offsets of the 16-byte chunks this lane copies. Copy
  // group q of a wave is 8 row pairs (16 rows of the stage tile): lane L
  // takes tile row 16q' + L / 4 and lands at its LDS chunk L % 4, so it
  // reads the global chunk that the swizzle puts there. Pairs past the last
  // valid one re-read the last valid pair.
  const int64_t lb = l0 / (GBK * EPB);   // first contraction line of the tile
  const uint8_t *abase = a.a + (i0 >> 1) * 2 * a.lda + lb * 128;
  const uint8_t *bbase = a.b + (MODE == kWgrad ? 0 : (int64_t)g * a.b_gstride) + (j0 >> 1) * 2 * a.ldb + lb * 128;
  const rsrc_t rsA = make_rsrc(abase, 0xFFFFFFFFu), rsB = make_rsrc(bbase, 0xFFFFFFFFu);
  const rsrc_t rsZ = make_rsrc(kZeroSrc, 0u);
  const int apmax = (int)(((ihi - 1) >> 1) - (i0 >> 1));   // last valid pair, tile-relative
  const int64_t jlim = (a.J - j0) < BN ? (a.J - j0) : BN;
  const int bpmax = (int)((jlim - 1) >> 1);
  uint32_t aoff[AQ], boff[BQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int row = (wave * AQ + q) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int pr = (row >> 1) < apmax ? (row >> 1) : apmax;
    aoff[q] = (uint32_t)(pr * 2 * (int32_t)a.lda + (row & 1) * 64 + c * 16);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int row = (wave * BQ + q) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int pr = (row >> 1) < bpmax ? (row >> 1) : bpmax;
    boff[q] = (uint32_t)(pr * 2 * (int32_t)a.ldb + (row & 1) * 64 + c * 16);
  }
  // valid-row clamps for the per-row scale copies
  auto arow = [&](int r) -> int64_t {
    const int64_t i = i0 + r;
    return i < ilo ? ilo : (i >= ihi ? ihi - 1 : i);
  };
  auto brow = [&](int r) -> int64_t { return j0 + (r < jlim ? r : jlim - 1); };

  const bool b_wave = wave < BN / 64;   // copies B-row scale words
  // MX scale words: lane L of wave w copies word slot d = 64w + L (see the
  // slot layout above). The scale matrices are word-major (word w of all
  // rows, then word w + 1), so the words of one stage for a run of rows are
  // contiguous: a wave's copy reads four 64-byte runs. The word of stage kt
  // holds the 32-blocks 4w .. 4w+3 with w = l0/128 + (kt * EPB) / 2.
  // They are buffer copies like the code chunks: a resource from the tile's
  // first word, the row's byte offset per lane, the stage's word offset in
  // an SGPR (no per-lane 64-bit address, and the stage past the contraction
  // is a scalar select of the empty resource, so the ring turn has no branch).
  rsrc_t rsMA = rsZ, rsMB = rsZ;
  uint32_t maoff = 0, mboff = 0, ma_word = 0, mb_word = 0;  // bytes from one word of a matrix to the next
  if (MX) {
    const int d = wave * 64 + lane;
    const int r = (d >> 7) * 128 + (d & 3) * 32 + ((d >> 2) & 31);
    ma_word = (uint32_t)((MODE == kWgrad ? a.I : a.M) * 4);
    mb_word = (uint32_t)(a.J * 4);
    rsMA = make_rsrc(reinterpret_cast<const uint8_t *>(a.a_scales) + (l0 / 128) * (int64_t)ma_word, 0xFFFFFFFFu);
    maoff = (uint32_t)(arow(r) * 4);
    if (b_wave) {
      rsMB = make_rsrc(reinterpret_cast<const uint8_t *>(a.b_scales) +
                           (MODE == kWgrad ? 0 : (int64_t)g * a.bs_gstride) + (l0 / 128) * (int64_t)mb_word,
                       0xFFFFFFFFu);
      mboff = (uint32_t)(brow(r) * 4);
    }
  }
  // vector-memory instructions every wave issues per stage (the waits count
  // them): MX scale words first (a filler copy into dmy where the wave has
  // no B-side scale row), then the A and B code chunks
  constexpr int NSC = MX ? 2 : 0;
  constexpr int OPS = NSC + AQ + BQ;

  v16f acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  // copy C (0 <= C < OPS) of stage kt into the stage buffers; a stage past
  // the contraction copies zero codes (and MX: zero E8M0 words, 2^-127, a
  // finite factor of those zeros), so the MFMAs of the padding stages of the
  // last ring turn add exactly nothing. No branches: the empty resource is a
  // scalar select.
  auto copy = [&](auto c, int kt, uint8_t *as, uint8_t *bs, uint32_t *ma, uint32_t *mb) {
    constexpr int C = decltype(c)::value;
    const bool real = kt < nsteps;
    if constexpr (C < NSC) {  // MX: the E8M0 word holding this stage's 32-blocks
      const uint32_t w = (uint32_t)(kt * EPB) >> 1;
      if constexpr (C == 0)
        bdma4(real ? rsMA : rsZ, maoff, w * ma_word, ma + wave * 64);
      else
        bdma4(real && b_wave ? rsMB : rsZ, mboff, w * mb_word, b_wave ? mb + wave * 64 : dmy);
    } else if constexpr (C < NSC + AQ) {
      constexpr int q = C - NSC;
      bdma16(real ? rsA : rsZ, aoff[q], (uint32_t)kt * 128u, as + (wave * AQ + q) * 1024);
    } else {
      constexpr int q = C - NSC - AQ;
      bdma16(real ? rsB : rsZ, boff[q], (uint32_t)kt * 128u, bs + (wave * BQ + q) * 1024);
    }
  };
  auto load_stage = [&](int kt, uint8_t *as, uint8_t *bs, uint32_t *ma, uint32_t *mb) {
    [&]<int... Cs>(std::integer_sequence<int, Cs...>) {
      (copy(std::integral_constant<int, Cs>{}, kt, as, bs, ma, mb), ...);
    }(std::make_integer_sequence<int, OPS>{});
    __builtin_amdgcn_sched_barrier(0);
  };

  // wait until at most PEND stages of this wave's copies are in flight
  // (copies complete in issue order), then synchronize the workgroup
  auto sync_stage = [&](auto pend) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<decltype(pend)::value * OPS>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // in a stage's barrier: the next stage's copies have landed (R - 3 later
  // stages may still be in flight); after the prologue: the first stage's
  using WR = std::integral_constant<int, R - 3>;
  using WP = std::integral_constant<int, R - 2>;

  // an empty asm use of every accumulator: keeps the stage's MFMAs issued
  // before the next wait, and each accumulator in its register file (AGPRs)
  auto pin_acc = [&]() {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) asm volatile("" ::"a"(acc[mi][ni]));
#endif
  };

  // fragment unit U of a stage: A sub-tiles 0..MI-1, B sub-tiles MI..MI+NI-1,
  // then (MX) the scale words
  auto read_unit = [&](auto u, Frags<MI, NI> &f, const uint8_t *as, const uint8_t *bs, const uint32_t *ma,
                       const uint32_t *mb) {
    constexpr int U = decltype(u)::value;
    if constexpr (U < MI) {
      f.a[U] = frag(as, wi * WM + U * 32 + l32, h);
    } else if constexpr (U < MI + NI) {
      f.b[U - MI] = frag(bs, wj * WN + (U - MI) * 32 + l32, h);
    } else if constexpr (MX) {
      const uint4 wa = *reinterpret_cast<const uint4 *>(&ma[(wi * 32 + l32) * 4]);
      const uint4 wb = *reinterpret_cast<const uint4 *>(&mb[(wj * 32 + l32) * 4]);
      const uint32_t wav[4] = {wa.x, wa.y, wa.z, wa.w}, wbv[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f.sa[m] = (int)(wav[m] >> (8 * h));
        f.sb[m] = (int)(wbv[m] >> (8 * h));
      }
    }
  };
  constexpr int NUNIT = MI + NI + (MX ? 1 : 0);
  auto read_frags = [&](Frags<MI, NI> &f, const uint8_t *as, const uint8_t *bs, const uint32_t *ma,
                        const uint32_t *mb) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) f.a[mi] = frag(as, wi * WM + mi * 32 + l32, h);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) f.b[ni] = frag(bs, wj * WN + ni * 32 + l32, h);
    if (MX) {
      const uint4 wa = *reinterpret_cast<const uint4 *>(&ma[(wi * 32 + l32) * 4]);
      const uint4 wb = *reinterpret_cast<const uint4 *>(&mb[(wj * 32 + l32) * 4]);
      const uint32_t wav[4] = {wa.x, wa.y, wa.z, wa.w}, wbv[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f.sa[m] = (int)(wav[m] >> (8 * h));
        f.sb[m] = (int)(wbv[m] >> (8 * h));
      }
    }
  };

  // MFMAs LO..HI-1 (index mi * NI + ni) of stage kt; PH = the stage's
  // position in its 128-block (MX: which two bytes of the scale word)
  auto mfma_range = [&](const Frags<MI, NI> &f, auto ph, auto lo, auto hi) {
    constexpr int PH = decltype(ph)::value;
    constexpr int LO = decltype(lo)::value, HI = decltype(hi)::value;
#pragma unroll
    for (int x = LO; x < HI; ++x) {
      const int mi = x / NI, ni = x % NI;
      if (MX && FP4) {
        // stage blocks 2m + h of MFMA m = byte 2m + h of the word (shifted
        // by 8h): opsel 2m; its operands are the 16 bytes at 32m + 16h
        // (measured lane layout: lane half h holds the MFMA's 32-block h)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.a[mi], f.b[ni], acc[mi][ni], mfma_fmt(FA), mfma_fmt(FB), 0, f.sa[mi], 0, f.sb[ni]);
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            upper4(f.a[mi]), upper4(f.b[ni]), acc[mi][ni], mfma_fmt(FA), mfma_fmt(FB), 2, f.sa[mi], 2,
            f.sb[ni]);
      } else if (MX) {
        // lane half h takes byte 2*PH + h of the row's word (shifted by 8h): opsel 2*PH
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.a[mi], f.b[ni], acc[mi][ni], FA, FB, 2 * PH, f.sa[mi], 2 * PH, f.sb[ni]);
      } else {
        // unit E8M0 scales (127 = 2^0); the scaled form keeps the
        // accumulators in AGPRs
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.a[mi], f.b[ni], acc[mi][ni], FA, FB, 0, kUnitScale, 0, kUnitScale);
      }
    }
  };

  // MFMAs of a stage issued before its barrier (their operands are already
  // in registers, so they keep the MFMA pipe busy while the waves sync).
  constexpr int NPRE = 2;
  using C0 = std::integral_constant<int, 0>;
  using CPRE = std::integral_constant<int, NPRE>;

  // ---- main loop: a ring of R stage buffers; stage kt lives in buffer
  // kt % R and its copies are issued R - 1 stages ahead. The loop body is
  // one turn of the ring (R stages, no conditional MFMAs).
  Frags<MI, NI> F0, F1;
  {
    // stage k: its first NPRE MFMAs (fragments read during stage k-1), wait
    // for stage k+1's copies, barrier, then slot by slot: one MFMA, one copy
    // of stage k+R-1, and the fragment reads of stage k+1 spread over the slots
    auto step = [&](int k, Frags<MI, NI> &fc, Frags<MI, NI> &fn, const uint8_t *an, const uint8_t *bn,
                    const uint32_t *man, const uint32_t *mbn, uint8_t *al, uint8_t *bl, uint32_t *mal,
                    uint32_t *mbl, auto ph) __attribute__((always_inline)) {
      mfma_range(fc, ph, C0{}, CPRE{});
      sync_stage(WR{});
      constexpr int NS = MI * NI - NPRE;   // slots
      [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ([&] {
          constexpr int S = Ss;
          mfma_range(fc, ph, std::integral_constant<int, NPRE + S>{}, std::integral_constant<int, NPRE + S + 1>{});
          if constexpr (S < OPS) copy(std::integral_constant<int, S>{}, k + R - 1, al, bl, mal, mbl);
          constexpr int u0 = (NUNIT * S) / NS, u1 = (NUNIT * (S + 1)) / NS;
          if constexpr (u1 > u0) read_unit(std::integral_constant<int, u0>{}, fn, an, bn, man, mbn);
          if constexpr (u1 > u0 + 1) read_unit(std::integral_constant<int, u0 + 1>{}, fn, an, bn, man, mbn);
          __builtin_amdgcn_sched_barrier(0);
        }(), ...);
      }(std::make_integer_sequence<int, NS>{});
      if constexpr (OPS > NS) {
        [&]<int... Cs>(std::integer_sequence<int, Cs...>) {
          (copy(std::integral_constant<int, NS + Cs>{}, k + R - 1, al, bl, mal, mbl), ...);
        }(std::make_integer_sequence<int, OPS - NS>{});
      }
      pin_acc();
    };
    // step J of a ring turn starting at stage kt (a multiple of R): stage
    // kt + J lives in buffer J, its fragments in F0 (J even) or F1, the
    // next stage's in buffer J + 1, and its copies go to buffer J - 1
    auto step_at = [&](auto j, int kt) __attribute__((always_inline)) {
      constexpr int J = decltype(j)::value;
      constexpr int nxt = (J + 1) % R, cpy = (J + R - 1) % R;
      // (the register sets are named, not selected: a selected reference
      // would put them in scratch memory)
      if constexpr (J % 2 == 0)
        step(kt + J, F0, F1, As[nxt], Bs[nxt], mAr[nxt], mBr[nxt], As[cpy], Bs[cpy], mAr[cpy], mBr[cpy],
             std::integral_constant<int, 0>{});
      else
        step(kt + J, F1, F0, As[nxt], Bs[nxt], mAr[nxt], mBr[nxt], As[cpy], Bs[cpy], mAr[cpy], mBr[cpy],
             std::integral_constant<int, 1>{});
    };
    if (vsteps > 0) {
      [&]<int... Js>(std::integer_sequence<int, Js...>) {
        (load_stage(Js, As[Js], Bs[Js], mAr[Js], mBr[Js]), ...);
      }(std::make_integer_sequence<int, R - 1>{});
      sync_stage(WP{});
      read_frags(F0, As[0], Bs[0], mAr[0], mBr[0]);
    }
    for (int kt = 0; kt < vsteps; kt += R) {
      [&]<int... Js>(std::integer_sequence<int, Js...>) {
        (step_at(std::integral_constant<int, Js>{}, kt), ...);
      }(std::make_integer_sequence<int, R>{});
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the epilogue's first LDS writes read the last MFMAs' results: keep >= 40
  // wait states between them
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" ::: "memory");
  wait_vm<0>();     // the copies of the stages past the contraction have landed
  __syncthreads();  // every wave is done with the stage buffers

  // ---- epilogue: each wave stages 16-row half slabs through its own LDS
  // region, then writes rows of 8 outputs with 16-byte stores. The scale
  // multiply happens on the LDS copy.
  float scale = 1.0f;
  if (RECIPE == kTensorwise || RECIPE == kDelayed) {
    const float sa = reinterpret_cast<const float *>(a.a_scales)[0];
    const float sb = reinterpret_cast<const float *>(a.b_scales)[MODE == kWgrad ? 0 : g];
    scale = sa * sb;
  }
  if (ACC && nsteps == 0) continue;  // empty group: dW_g unchanged
  constexpr int STR = WN + 8;          // LDS row stride in floats
  constexpr int CPR = WN / 8;          // 8-value chunks per row (bf16 outputs: 16 bytes)
  constexpr int CPL = 16 * CPR / 64;   // chunks per lane per half slab
  float *cb = reinterpret_cast<float *>(As[wave]);  // this wave's staging region
  const int64_t jw = j0 + wj * WN;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int v = 8 * hs; v < 8 * hs + 8; ++v)
          cb[(((v >> 2) & 1) * 8 + h * 4 + (v & 3)) * STR + ni * 32 + l32] = acc[mi][ni][v];
      __builtin_amdgcn_wave_barrier();
      if constexpr (MODE == kWgrad) {
        // fp32 dW: 16-byte chunks, WN / 4 per row, so that one store
        // instruction writes whole 512-byte pieces of two rows (measured 4-6%
        // faster for wgrad than two interleaved 16-byte halves of 32-byte
        // chunks). Accumulating (a separate kernel instance, so the plain
        // one keeps its registers): every old value is loaded before the
        // first store, so no load waits behind an earlier store.
        constexpr int CPR4 = WN / 4;
        constexpr int CPL4 = 16 * CPR4 / 64;
        float4 old[ACC ? CPL4 : 1];
        if constexpr (ACC) {
#pragma unroll
          for (int k = 0; k < CPL4; ++k) {
            const int id = k * 64 + lane;
            const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + id / CPR4;
            const int64_t j = jw + (id % CPR4) * 4;
            old[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (i >= ilo && i < ihi && j < a.J)
              old[k] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.out) +
                                                         ((int64_t)g * a.I + i) * a.ldo + j);
          }
        }
#pragma unroll
        for (int k = 0; k < CPL4; ++k) {
          const int id = k * 64 + lane;
          const int r = id / CPR4, c4 = id % CPR4;
          const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + r;
          const int64_t j = jw + c4 * 4;
          const float4 x = *reinterpret_cast<const float4 *>(&cb[r * STR + c4 * 4]);
          if (i >= ilo && i < ihi && j < a.J) {  // J % 128 == 0: a chunk is all in or all out
            float4 y = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
            if constexpr (ACC) y = make_float4(y.x + old[k].x, y.y + old[k].y, y.z + old[k].z, y.w + old[k].w);
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + ((int64_t)g * a.I + i) * a.ldo + j) = y;
          }
        }
      } else {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int id = k * 64 + lane;
        const int r = id / CPR, c8 = id % CPR;
        const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + r;
        const int64_t j = jw + c8 * 8;
        const float4 x0 = *reinterpret_cast<const float4 *>(&cb[r * STR + c8 * 8]);
        const float4 x1 = *reinterpret_cast<const float4 *>(&cb[r * STR + c8 * 8 + 4]);
        if (i >= ilo && i < ihi && j < a.J) {  // J % 128 == 0: a chunk is all in or all out
          uint4 o;
          o.x = f32_to_bf16_bits(x0.x * scale) | (f32_to_bf16_bits(x0.y * scale) << 16);
          o.y = f32_to_bf16_bits(x0.z * scale) | (f32_to_bf16_bits(x0.w * scale) << 16);
          o.z = f32_to_bf16_bits(x1.x * scale) | (f32_to_bf16_bits(x1.y * scale) << 16);
          o.w = f32_to_bf16_bits(x1.z * scale) | (f32_to_bf16_bits(x1.w * scale) << 16);
          uint16_t *dst = reinterpret_cast<uint16_t *>(a.out) + i * a.ldo + j;
          if (a.stream_out)
            store16_stream(dst, o);
          else
            *reinterpret_cast<uint4 *>(dst) = o;
        }
      }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();  // the staging buffers are free before the next tile's copies land
  }
}


// ---------------------------------------------------------------------------
// Blockwise grouped GEMM (1x128 / 128x1 token scales, 128x128 weight scales,
// all fp32; DeepSeek-V3's recipe as the TE issue design note describes it):
// C[i, j] = sum over 128-blocks b of sA(i, b) * sB(b, j) * P_b[i, j], where
// P_b is the exact FP8 product over block b.
//
// One MFMA per block: v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales)
// contracts a whole 128-long block into a 16 x 16 partial of four registers
// per lane, which the lane then promotes into its fp32 totals with one FMA
// per element (the factor sA(i) * sB is one number per lane and sub-tile
// row: the MFMA is called with the B fragment first, so a lane holds one
// output row i and four consecutive columns). Small partials let a
// 256 x 256 tile fit: eight waves (two per SIMD) of 64 x 128, each with
// 4 x 8 sub-tiles (128 registers of totals, 32 of A fragments for the whole
// block, 8 per B fragment), so the tile's copy demand per MFMA is that of the
// tensorwise 256 x 256 tile instead of the 1.5x of a 256 x 128 one.
//
// The LDS holds two blocks (four 64-byte stages of A and of B, 128 KB) and
// the block loop is block-major: at a block's barrier its data has landed and
// every wave is done with the block before, whose buffers then receive the
// next block's copies (direct-to-LDS buffer loads, one block ahead, in five
// pieces spread over the block's MFMAs). Each wave walks its sub-tiles column
// by column (8 columns of 4 MFMAs), reading the next column's B fragment
// while the current one runs; a sub-tile's promotion is issued two MFMAs
// after its own, when its partial has certainly been written. The last
// column of a block runs after the next block's barrier, on fragments
// already in registers, while the new block's A fragments arrive.
//
// Tiles follow one another without a pause: the last block of a tile copies
// the first block of the workgroup's next tile, and the finished tile's
// totals leave during the next tile's first block, in 16-row slabs that
// each wave stages through its own copy destinations in the idle buffer
// pair (so neither the copy latency of a tile's first block nor the drain
// of its stores waits for the whole workgroup). The accumulating wgrad
// instance, which must read the old dW before it writes, ends each tile
// with a staged read-add-write epilogue instead.
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
}
__device__ __forceinline__ uint32_t clamp_u32(int64_t v) {
  return v <= 0 ? 0u : (v >= (int64_t)0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)v);
}

// One tile of the blockwise GEMM (all wave-uniform)
struct BwTile {
  int i0, ilo, ihi, j0;  // rows [i0, i0 + 256) (valid [ilo, ihi)), columns from j0
  int l0;                // first contraction element (wgrad: the group's padded start)
  int g, nblk, valid;
};
// A tile's copy sources: buffer resources sized to its valid rows (rows past
// them read zeros), so the per-lane copy offsets are the same for every tile
struct BwRes {
  rsrc_t ra, rb;  // A and B codes from the tile's first row pair and contraction line
  rsrc_t rs;      // the scales this wave copies: A rows (waves 0-3); waves 4-7: wgrad B columns,
                  // FWD / DGRAD the weight scales of the tile's two 128-column blocks
};
// what the stores of a finished tile need
struct BwOut {
  int i0, ilo, ihi, j0, g, valid;
};

template <int MODE, int FA, int FB, bool ACC>
__global__ __launch_bounds__(512) void blockwise_gemm_kernel(GemmArgs a) {
  constexpr int NW = 8;
  constexpr int BN = 256;
  constexpr int WM = 64, WN = 128;  // wave tile: 4 waves along i, 2 along j
  constexpr int AQ = GBM / 16 / NW, BQ = BN / 16 / NW;  // 1 KB copy groups per wave and stage
  constexpr bool WG = MODE == kWgrad;
  constexpr bool SEAMLESS = !ACC;  // stores overlap the next tile (see above)
  typedef float v4f __attribute__((ext_vector_type(4)));

  // stage buffers: AB[0] = A, AB[1] = B, four 64-byte stages each (one
  // array, so that a wave's staging region is plain address arithmetic)
  __shared__ __attribute__((aligned(1024))) uint8_t AB[2][4][GBM * GBK];
  uint8_t (*const As)[GBM * GBK] = AB[0];
  uint8_t (*const Bs)[BN * GBK] = AB[1];
  __shared__ __attribute__((aligned(16))) float sAr[2][GBM];          // per-row A scales of a block
  __shared__ __attribute__((aligned(16))) float sBr[2][WG ? BN : 64];  // wgrad: per-column B scales

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wi = wave & 3, wj = wave >> 2;
  const int l16 = lane & 15, g4 = lane >> 4;

  // ---- per-lane copy offsets. Copy group q of a wave is 8 row pairs (16
  // rows of the stage tile): lane L takes tile row 16q' + L / 4 and lands at
  // its LDS chunk L % 4, so it reads the global chunk the swizzle puts there.
  uint32_t aoff[AQ], boff[BQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int row = (wave * AQ + q) * 16 + (lane >> 2);
    const int c = bswz_chunk(row, lane & 3);  // (an involution: the chunk that lands at L % 4)
    aoff[q] = (uint32_t)((row >> 1) * 2 * (int32_t)a.lda + (row & 1) * 64 + c * 16);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int row = (wave * BQ + q) * 16 + (lane >> 2);
    const int c = bswz_chunk(row, lane & 3);
    boff[q] = (uint32_t)((row >> 1) * 2 * (int32_t)a.ldb + (row & 1) * 64 + c * 16);
  }
  // scales copied with each block: waves 0-3 the A scales of tile rows
  // 64w..64w+63; waves 4-7 (wgrad) the B scales of tile columns 64(w-4)..,
  // (FWD / DGRAD) lanes 0 and 1 the weight scales of the tile's two
  // 128-column blocks, into sBr[q][0..1] (the other lanes read past the
  // resource: zeros)
  const int64_t sa_row = WG ? a.lda : a.L;  // contraction elements per row of the scale matrices
  const int64_t sb_row = WG ? a.ldb : a.L;
  const uint32_t srow = (uint32_t)((wave < 4 ? sa_row : sb_row) / SBLK) * 4u;  // bytes per scale row
  const bool wscale = !WG && wave >= 4;  // copies weight scales
  const uint32_t svoff = wscale ? (uint32_t)lane * (uint32_t)a.sb_j * 4u : (uint32_t)((wave & 3) * 64 + lane) * srow;
  const uint32_t vstep = wscale ? (uint32_t)a.sb_l * 4u : 0u, sstep = wscale ? 0u : 4u;  // per block
  float *const sc_dst0 = wave < 4 ? &sAr[0][(wave & 3) * 64] : &sBr[0][WG ? (wave & 3) * 64 : 0];
  float *const sc_dst1 = wave < 4 ? &sAr[1][(wave & 3) * 64] : &sBr[1][WG ? (wave & 3) * 64 : 0];
  const rsrc_t rsZ = make_rsrc(kZeroSrc, 0u);

  // ---- tile vb: coordinates and resources; false for an unused FWD / DGRAD
  // slot (rows of a neighbouring group inside a tile are computed and not
  // stored)
  auto setup = [&](int vb, BwTile &T) -> bool {
    const int lid = xcd_remap<32>(vb, a.nblocks);
    int g = 0;
    int64_t i0 = 0, ilo = 0, ihi = 0, j0 = 0, l0 = 0;
    int nsteps = 0;
    if (WG) {
      const int per_g = a.slots * a.jtiles;
      g = lid / per_g;
      int it, jt;
      raster(lid - g * per_g, a.slots, a.jtiles, it, jt);
      i0 = (int64_t)it * GBM;
      j0 = (int64_t)jt * BN;
      ilo = i0;
      ihi = a.I < i0 + GBM ? a.I : i0 + GBM;
      int64_t p_lo = a.pstarts[g], p_hi = a.pstarts[g + 1];
      const int64_t cap = a.lda < a.ldb ? a.lda : a.ldb;  // token positions
      p_lo = p_lo < 0 ? 0 : (p_lo > cap ? cap : p_lo);
      p_hi = p_hi < p_lo ? p_lo : (p_hi > cap ? cap : p_hi);
      l0 = p_lo & ~(int64_t)127;  // padded starts are 128-aligned
      nsteps = (int)(((p_hi - l0) / 128) * 2);
    } else {
      int slot, jt;
      raster(lid, a.slots, a.jtiles, slot, jt);
      j0 = (int64_t)jt * BN;
      if (!locate_row_tile(a, slot, g, i0, ilo, ihi)) return false;
      // (read from LDS: wave-uniform values the compiler would keep in VGPRs)
      g = __builtin_amdgcn_readfirstlane(g);
      i0 = uni64(i0);
      ilo = uni64(ilo);
      ihi = uni64(ihi);
      nsteps = (int)(a.L / GBK);
    }
    T.g = g;
    T.i0 = (int)i0;  // row and column indices fit in 32 bits (M < 2^31; K, N < 2^31)
    T.ilo = (int)ilo;
    T.ihi = (int)ihi;
    T.j0 = (int)j0;
    T.l0 = (int)l0;
    T.nblk = nsteps >> 1;
    T.valid = 1;
    return true;
  };
  // the copy sources of tile T (zeros when T is not valid)
  auto resources = [&](const BwTile &T) -> BwRes {
    BwRes R;
    R.ra = R.rb = R.rs = rsZ;
    if (!T.valid) return R;
    const int64_t i0 = T.i0, ihi = T.ihi, j0 = T.j0, l0 = T.l0;
    const int64_t lb = l0 / GBK;
    const int64_t jlim = (a.J - j0) < BN ? (a.J - j0) : BN;
    const int64_t apairs = ((ihi - 1) >> 1) - (i0 >> 1) + 1, bpairs = ((jlim - 1) >> 1) + 1;
    R.ra = make_rsrc(a.a + (i0 >> 1) * 2 * a.lda + lb * 128, clamp_u32(apairs * 2 * a.lda));
    R.rb = make_rsrc(a.b + (WG ? 0 : (int64_t)T.g * a.b_gstride) + (j0 >> 1) * 2 * a.ldb + lb * 128,
                     clamp_u32(bpairs * 2 * a.ldb));
    if (wave < 4)
      R.rs = make_rsrc(reinterpret_cast<const float *>(a.a_scales) + i0 * (sa_row / SBLK) + l0 / SBLK,
                       clamp_u32((ihi - i0) * (int64_t)srow));
    else if (WG)
      R.rs = make_rsrc(reinterpret_cast<const float *>(a.b_scales) + j0 * (sb_row / SBLK) + l0 / SBLK,
                       clamp_u32(jlim * (int64_t)srow));
    else  // weight scales [E, blocks along l, blocks along j] from the tile's first j-block, to the
          // end of expert g's array (block offsets ride in the lane offset)
      R.rs = make_rsrc(reinterpret_cast<const float *>(a.b_scales) + (int64_t)T.g * a.bs_gstride +
                           (j0 / SBLK) * a.sb_j,
                       clamp_u32((a.bs_gstride - (j0 / SBLK) * a.sb_j) * 4));
    return R;
  };
  // the workgroup's next tile from vb on with a contraction (vb advanced to
  // it); an empty wgrad group's tiles get dW = 0 on the way (accumulating:
  // left as they are)
  auto next_tile = [&](int &vb, BwTile &T) {
    T.valid = 0;
    for (; vb < a.nblocks; vb += gridDim.x) {
      if (!setup(vb, T)) continue;
      if (T.nblk > 0) return;
      if (WG && !ACC) {
        for (int e = t; e < GBM * BN / 4; e += 64 * NW) {
          const int64_t i = T.i0 + e / (BN / 4), j = T.j0 + (e % (BN / 4)) * 4;
          if (i < T.ihi && j < a.J)
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + ((int64_t)T.g * a.I + i) * a.ldo + j) =
                make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
      T.valid = 0;
    }
  };

  // copy piece K of block bb from sources R into buffer pair q (stages 2q,
  // 2q+1): the A (K = 0, 2) or B (K = 1, 3) chunks of stage K / 2, or (K = 4)
  // the scales
  auto copy_piece = [&](const BwRes &R, int bb, int q, auto k_) __attribute__((always_inline)) {
    constexpr int K = decltype(k_)::value;
    if constexpr (K < 4) {
      constexpr int s = K / 2;
      const uint32_t soff = (uint32_t)(2 * bb + s) * 128u;
      if constexpr (K % 2 == 0) {
#pragma unroll
        for (int c = 0; c < AQ; ++c) bdma16(R.ra, aoff[c], soff, &As[2 * q + s][(wave * AQ + c) * 1024]);
      } else {
#pragma unroll
        for (int c = 0; c < BQ; ++c) bdma16(R.rb, boff[c], soff, &Bs[2 * q + s][(wave * BQ + c) * 1024]);
      }
    } else {
      // (the weight scales' block offset in the lane offset, the others' in
      // the scalar offset: an in-range lane offset then always addresses
      // memory inside the array)
      bdma4(R.rs, svoff + (uint32_t)bb * vstep, (uint32_t)bb * sstep, q ? sc_dst1 : sc_dst0);
    }
  };

  // fragment of sub-tile row `row` for the whole block in pair q: chunk g4
  // of the row in each of the block's two stages (the MFMA's k order is
  // the same for both operands, so any fixed assignment of the 128 k to
  // lanes contracts correctly)
  auto frag_blk = [&](const uint8_t (*buf)[GBM * GBK], int q, int row) -> v8i {
    const int o = bswz(row, g4);
    const uint4 x0 = *reinterpret_cast<const uint4 *>(&buf[2 * q][o]);
    const uint4 x1 = *reinterpret_cast<const uint4 *>(&buf[2 * q + 1][o]);
    return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  };
  auto fragA = [&](int q, int mi) { return frag_blk(As, q, wi * WM + mi * 16 + l16); };
  auto fragB = [&](int q, int ni) { return frag_blk(Bs, q, wj * WN + ni * 16 + l16); };
  // the four column scales of this lane in column ni of the wave tile (wgrad)
  auto col_scales = [&](int q, int ni) -> v4f {
    const float4 v = *reinterpret_cast<const float4 *>(&sBr[q][wj * WN + ni * 16 + 4 * g4]);
    return v4f{v.x, v.y, v.z, v.w};
  };

  v4f acc[4][8];
  // registers of the block schedule; zero before a tile's first block, whose
  // leading "previous column" then adds exact zeros
  v8i af[4], bfX, bfY;     // A fragments; B fragments of even / odd columns
  v4f p[4];                // partials, by sub-tile row
  float fo[4], fn[4];      // promotion factors per sub-tile row: previous block, this block
  v4f sbX, sbY;            // wgrad: column scales of even / odd columns
  float sbw = 1.0f;        // FWD / DGRAD: this block's weight scale for the wave's j-block
  auto reset = [&]() {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      af[m] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      p[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      fo[m] = 0.0f;
      fn[m] = 0.0f;
    }
    bfX = af[0];
    bfY = af[0];
    sbX = p[0];
    sbY = p[0];
  };
  reset();

  auto mma = [&](const v8i &bfr, const v8i &afr) -> v4f {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr, afr, z, FB, FA, 0, kUnitScale, 0, kUnitScale);
  };
  auto promote = [&](v4f &c, const v4f &pp, float f, const v4f &sb) __attribute__((always_inline)) {
    if constexpr (WG) {
#pragma unroll
      for (int v = 0; v < 4; ++v) c[v] += (pp[v] * sb[v]) * f;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) c[v] += pp[v] * f;
    }
  };

  // A finished tile's totals leave in 16-row slabs (one sub-tile row at a
  // time) staged in this wave's own 8 KB of buffer pair q1: its copy
  // destinations there (2 KB in each of the pair's four stage buffers), so no
  // other wave touches them and the wave's own next copies into the pair come
  // after its last read. Slab row r lives in stage buffer r / 4 (A0, B0, A1,
  // B1) at 512 (r % 4), its 16-byte column chunk c at c ^ r (the 16 lanes of
  // a write, one row each, and of a row read land on distinct banks). Rows
  // then leave as 16-byte chunks (bf16: 8 columns, rounded to nearest even;
  // fp32 dW: 4), and the totals are zeroed for the next tile.
  auto store_tile = [&](const BwOut &P, int q1) __attribute__((always_inline)) {
    uint8_t *const region = &AB[0][2 * q1][wave * 2048];
    // the lane index opaque here, so that the addresses are computed now
    // rather than before the main loop
    int ll = lane;
    asm volatile("" : "+v"(ll));
    const int rl = ll & 15, cg = ll >> 4;
    const bool jok = (int64_t)P.j0 + wj * WN < a.J;  // J % 128 == 0: the wave's 128 columns are all in or all out
    auto row_base = [&](int r) -> uint8_t * {
      // stage buffer r / 4: A0, B0, A1, B1 of the pair
      return region + ((r >> 2) & 1) * (4 * GBM * GBK) + (r >> 3) * (GBM * GBK) + (r & 3) * 512;
    };
    uint8_t *const wrow = row_base(rl);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        *reinterpret_cast<float4 *>(wrow + (((n * 4 + cg) ^ rl) << 4)) =
            make_float4(acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]);
        acc[m][n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      const int64_t ib = (int64_t)P.i0 + wi * WM + m * 16;
      const int64_t jw = (int64_t)P.j0 + wj * WN;
      if constexpr (WG) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int id = k * 64 + ll, r = id >> 5, c = id & 31;
          const float4 y = *reinterpret_cast<const float4 *>(row_base(r) + ((c ^ r) << 4));
          const int64_t i = ib + r;
          if (jok && i >= P.ilo && i < P.ihi)
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + ((int64_t)P.g * a.I + i) * a.ldo + jw +
                                        c * 4) = y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int id = k * 64 + ll, r = id >> 4, c8 = id & 15;
          const float4 x0 = *reinterpret_cast<const float4 *>(row_base(r) + (((2 * c8) ^ r) << 4));
          const float4 x1 = *reinterpret_cast<const float4 *>(row_base(r) + (((2 * c8 + 1) ^ r) << 4));
          const int64_t i = ib + r;
          if (jok && i >= P.ilo && i < P.ihi) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            typedef float f2 __attribute__((ext_vector_type(2)));
            const bf2 b0 = __builtin_convertvector((f2{x0.x, x0.y}), bf2);  // round to nearest even
            const bf2 b1 = __builtin_convertvector((f2{x0.z, x0.w}), bf2);
            const bf2 b2 = __builtin_convertvector((f2{x1.x, x1.y}), bf2);
            const bf2 b3 = __builtin_convertvector((f2{x1.z, x1.w}), bf2);
            uint4 o;
            __builtin_memcpy(&o.x, &b0, 4);
            __builtin_memcpy(&o.y, &b1, 4);
            __builtin_memcpy(&o.z, &b2, 4);
            __builtin_memcpy(&o.w, &b3, 4);
            uint16_t *dst = reinterpret_cast<uint16_t *>(a.out) + i * a.ldo + jw + c8 * 8;
            if (a.stream_out)
              store16_stream(dst, o);
            else
              *reinterpret_cast<uint4 *>(dst) = o;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
  };

  // Event E (0..31) of a block iteration: events 0-3 are column 7 of the
  // previous block (sub-tile rows 0-3), events 4 + 4n + m column n < 7 of
  // this block, row m. After its MFMA, the event promotes the sub-tile of
  // event E - 2 and issues reads whose target registers are free by then.
  // In a tile's first block (FIRST) the previous block's column is not this
  // tile's: events 0-5 run no MFMA and no promotion of it.
  auto event = [&](auto e_, int q, auto read_, auto first_) __attribute__((always_inline)) {
    constexpr int E = decltype(e_)::value;
    constexpr bool READ = decltype(read_)::value;  // false: the column after a tile's last block
    constexpr bool FIRST = decltype(first_)::value;
    constexpr int N = E < 4 ? 7 : (E - 4) / 4;  // column
    constexpr int M = E < 4 ? E : (E - 4) % 4;  // sub-tile row
    if constexpr (FIRST && E < 4) {
    } else if constexpr (N % 2 == 0)
      p[M] = mma(bfX, af[M]);
    else
      p[M] = mma(bfY, af[M]);
    // (kept first: the promotion below reads the partial of two MFMAs ago,
    // which is written by the time this MFMA issues; issued before it, the
    // read could come one MFMA after the write and see a stale value)
    __builtin_amdgcn_sched_barrier(0);
    // next column's B fragment, into the register set of column N - 1
    // (last read by the previous event's MFMA)
    if constexpr (E >= 4 && M == 0) {
      if constexpr ((N + 1) % 2 == 0)
        bfX = fragB(q, N + 1);
      else
        bfY = fragB(q, N + 1);
    }
    // promotion of event E - 2
    if constexpr (FIRST && E < 6) {
    } else if constexpr (E < 2) {
      promote(acc[2 + E][6], p[2 + E], fo[2 + E], sbX);
    } else if constexpr (E < 6) {
      promote(acc[E - 2][7], p[E - 2], fo[E - 2], sbY);
    } else {
      constexpr int PN = (E - 6) / 4, PM = (E - 6) % 4;
      if constexpr (PN % 2 == 0)
        promote(acc[PM][PN], p[PM], fn[PM], sbX);
      else
        promote(acc[PM][PN], p[PM], fn[PM], sbY);
    }
    // this block's A fragment of row M, once the previous block's is used
    if constexpr (E < 4 && READ) af[E] = fragA(q, E);
    // wgrad: the next column's scales, into the set of column N - 1 (whose
    // last promotion was just issued)
    if constexpr (WG && E >= 4 && M == 1) {
      if constexpr ((N + 1) % 2 == 0)
        sbX = col_scales(q, N + 1);
      else
        sbY = col_scales(q, N + 1);
    }
    if constexpr (WG && E == 1 && READ) sbX = col_scales(q, 0);
    if constexpr (!WG && E == 5) {
#pragma unroll
      for (int m = 0; m < 4; ++m) fn[m] *= sbw;
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // a block in buffer pair q; the next block's copies (block nbb from
  // sources R) go to pair q ^ 1
  auto run_block = [&](int q, const BwRes &R, int nbb, auto first_) __attribute__((always_inline)) {
    bfX = fragB(q, 0);
    // this block's factors: read now, multiplied at event 5 (first used at
    // event 6), so that no early MFMA waits for these reads
    if constexpr (!WG) sbw = sBr[q][wj];
#pragma unroll
    for (int m = 0; m < 4; ++m) fn[m] = sAr[q][wi * WM + m * 16 + l16];
    __builtin_amdgcn_sched_barrier(0);
    // the next block's copies go out in five pieces, after events 1, 5, 9,
    // 13 and 17: spread over the MFMAs, they ran 7-10% faster than as one
    // burst after event 1
    [&]<int... Es>(std::integer_sequence<int, Es...>) {
      ([&] {
        event(std::integral_constant<int, Es>{}, q, std::true_type{}, first_);
        if constexpr (Es % 4 == 1 && Es / 4 < 5) {
          copy_piece(R, nbb, q ^ 1, std::integral_constant<int, Es / 4>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      }(), ...);
    }(std::make_integer_sequence<int, 32>{});
#pragma unroll
    for (int m = 0; m < 4; ++m) fo[m] = fn[m];
  };
  // block b has landed (every wave waits for its own copies, then the
  // barrier), and every wave is done reading the block before's buffers
  auto block_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // column 7 of a tile's last block (events 0-3 without the next block's
  // reads) and the last promotions: column 6 rows 2-3, column 7. Out of the
  // event order, where the compiler (most of all in the accumulating
  // instance, at its register limit) hoisted promotions above the next MFMA
  // and sank MFMAs into the epilogue, each read of a partial here is behind
  // 40 explicit wait states: the partials pass through the padding asm, so
  // that no promotion (register-only work, which a memory clobber does not
  // order) moves above it and no MFMA below it.
  auto finish_tile = [&]() __attribute__((always_inline)) {
    p[0] = mma(bfY, af[0]);
    p[1] = mma(bfY, af[1]);
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7"
                 : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3])::"memory");
    __builtin_amdgcn_sched_barrier(0);
    promote(acc[2][6], p[2], fo[2], sbX);
    promote(acc[3][6], p[3], fo[3], sbX);
    promote(acc[0][7], p[0], fo[0], sbY);
    promote(acc[1][7], p[1], fo[1], sbY);
    __builtin_amdgcn_sched_barrier(0);
    p[2] = mma(bfY, af[2]);
    p[3] = mma(bfY, af[3]);
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+v"(p[2]), "+v"(p[3])::"memory");
    __builtin_amdgcn_sched_barrier(0);
    promote(acc[2][7], p[2], fo[2], sbY);
    promote(acc[3][7], p[3], fo[3], sbY);
  };

  int vb = blockIdx.x;
  BwTile T, N;
  BwOut P;
  next_tile(vb, T);
  P.valid = 0;
  int gb = 0;  // blocks run by the workgroup: block gb lives in buffer pair gb & 1
  // the sources of the next copies: this tile's, from the start of its last
  // block the next tile's
  BwRes R = resources(T);
  if (T.valid) {
    copy_piece(R, 0, 0, std::integral_constant<int, 0>{});
    copy_piece(R, 0, 0, std::integral_constant<int, 1>{});
    copy_piece(R, 0, 0, std::integral_constant<int, 2>{});
    copy_piece(R, 0, 0, std::integral_constant<int, 3>{});
    copy_piece(R, 0, 0, std::integral_constant<int, 4>{});
  }
  while (T.valid) {
    // first block: also finds the next tile and (seamless) writes the
    // previous tile's totals, whose stores then drain under this block's
    // MFMAs (the next block's wait covers them)
    block_sync();
    N.valid = 0;
    if constexpr (SEAMLESS) {
      vb += gridDim.x;
      next_tile(vb, N);
      if (P.valid) store_tile(P, (gb & 1) ^ 1);  // in the previous block's buffer pair
    }
    if (T.nblk == 1) R = resources(N);
    run_block(gb & 1, R, T.nblk > 1 ? 1 : 0, std::true_type{});
    ++gb;
    for (int b = 1; b < T.nblk; ++b) {
      block_sync();
      if (b + 1 == T.nblk) R = resources(N);
      run_block(gb & 1, R, b + 1 < T.nblk ? b + 1 : 0, std::false_type{});
      ++gb;
    }
    finish_tile();  // on registers: overlaps the next barrier's wait
    if constexpr (SEAMLESS) {
      P = BwOut{T.i0, T.ilo, T.ihi, T.j0, T.g, 1};
      T = N;
      continue;
    }
    // ---- accumulating wgrad: dW += C through 16-row slabs staged in each
    // wave's own 16 KB of the stage buffers
    wait_vm<0>();
    __syncthreads();  // every wave is done with the stage buffers
    {
      constexpr int STR = WN + 4;  // LDS row stride in floats (16-byte rows land on distinct banks)
      float *cb = reinterpret_cast<float *>(wave < 4 ? As[wave] : Bs[wave - 4]);
      const int64_t jw = T.j0 + wj * WN;
      // the lane index, opaque to the compiler here: otherwise it computes
      // every address before the main loop and spills them, and each reload
      // from scratch then waits for all earlier stores (vmcnt(0))
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
          *reinterpret_cast<float4 *>(&cb[l16 * STR + ni * 16 + 4 * g4]) =
              make_float4(acc[mi][ni][0], acc[mi][ni][1], acc[mi][ni][2], acc[mi][ni][3]);
        __builtin_amdgcn_wave_barrier();
        const int64_t ib = T.i0 + wi * WM + mi * 16;
        constexpr int CPR4 = WN / 4;  // float4 chunks per row
        constexpr int CPL4 = 16 * CPR4 / 64;
        float4 old[CPL4];
#pragma unroll
        for (int k = 0; k < CPL4; ++k) {
          const int id = k * 64 + lane_e;
          const int64_t i = ib + id / CPR4, j = jw + (id % CPR4) * 4;
          old[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (i >= T.ilo && i < T.ihi && j < a.J)
            old[k] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.out) +
                                                       ((int64_t)T.g * a.I + i) * a.ldo + j);
        }
#pragma unroll
        for (int k = 0; k < CPL4; ++k) {
          const int id = k * 64 + lane_e;
          const int r = id / CPR4, c4 = id % CPR4;
          const int64_t i = ib + r, j = jw + c4 * 4;
          const float4 y = *reinterpret_cast<const float4 *>(&cb[r * STR + c4 * 4]);
          if (i >= T.ilo && i < T.ihi && j < a.J)  // J % 128 == 0: a chunk is all in or all out
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + ((int64_t)T.g * a.I + i) * a.ldo + j) =
                make_float4(y.x + old[k].x, y.y + old[k].y, y.z + old[k].z, y.w + old[k].w);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();  // the staging buffers are free before the next tile's copies land
    reset();
    vb += gridDim.x;
    next_tile(vb, N);
    T = N;
    R = resources(T);
    if (T.valid) {
      copy_piece(R, 0, gb & 1, std::integral_constant<int, 0>{});
      copy_piece(R, 0, gb & 1, std::integral_constant<int, 1>{});
      copy_piece(R, 0, gb & 1, std::integral_constant<int, 2>{});
      copy_piece(R, 0, gb & 1, std::integral_constant<int, 3>{});
      copy_piece(R, 0, gb & 1, std::integral_constant<int, 4>{});
    }
  }
  if constexpr (SEAMLESS) {
    if (P.valid) {  // the workgroup's last tile, once every wave is done with the last block's buffers
      block_sync();
      store_tile(P, (gb & 1) ^ 1);
    }
  }
  wait_vm<0>();  // no copy into LDS is still in flight when the workgroup ends
}

// ---------------------------------------------------------------------------
// NVFP4 grouped GEMM: e2m1 codes with an e4m3 scale per 16 contraction
// elements and an fp32 scale per tensor (the NVFP4 rows of the Megatron-LM
// single-grouped-weight PR's coverage table). gfx950's scaled MFMAs take
// only power-of-two (E8M0) scales per 32 elements, so the block scale cannot
// ride on them; instead each lane turns its codes into f16 operands: the
// code pairs decode exactly to f16 (v_cvt_scalef32_pk_f16_fp4, scale 1) and
// a packed f16 multiply by the block scale is exact too (an e2m1 value has
// 2 significant bits and an e4m3 scale 4, and every product lies in
// [2^-10, 2688], inside f16's normal range; all three facts measured on the
// device for all codes and scales). The f16 products then go through the
// 32x32x16 f16 MFMA with fp32 accumulation, and the two tensor scales
// multiply the accumulators in the epilogue. The tile, the XCD mapping, the
// persistent grid and the direct-to-LDS ring of 64-byte (128-element) stages
// are those of grouped_gemm_kernel; a stage is one 128-element piece of each
// row, whose 8 e4m3 block codes per row arrive beside it, and whose codes
// are stored so that the 16-byte chunks a lane reads hold, for its half of
// the MFMA's k range, the 8 elements of each of the stage's 8 k16 steps.
typedef _Float16 nv_v2h __attribute__((ext_vector_type(2)));
typedef _Float16 nv_v8h __attribute__((ext_vector_type(8)));

// 8 e2m1 codes (one dword, element 2i in the low nibble of byte i) times the
// block scale dd (both halves equal): the f16 MFMA operand of one lane
__device__ __forceinline__ nv_v8h nv_operand(uint32_t x, nv_v2h dd) {
  const nv_v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * dd;
  const nv_v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * dd;
  const nv_v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * dd;
  const nv_v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * dd;
  return nv_v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// a row's 8 block scales of one stage (two dwords of e4m3 codes) as f16 pairs
struct NvScale {
  nv_v2h p[4];
};
__device__ __forceinline__ NvScale nv_scales(uint2 w) {
  NvScale r;
  r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false);
  r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true);
  r.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false);
  r.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true);
  return r;
}
template <int S>
__device__ __forceinline__ nv_v2h nv_dd(const NvScale &r) {
  return __builtin_shufflevector(r.p[S >> 1], r.p[S >> 1], S & 1, S & 1);
}

template <int MODE, bool ACC>
__global__ __launch_bounds__(256) void nvfp4_gemm_kernel(GemmArgs a) {
  constexpr int NW = 4, BN = 256, WM = 128, WN = 128, MI = 4, NI = 4;
  constexpr int AQ = GBM / 16 / NW, BQ = BN / 16 / NW;   // 1 KB copy groups of codes per wave per stage
  constexpr int OPS = 4 + AQ + BQ;                        // + two scale dwords of A rows and two of B rows
  __shared__ __attribute__((aligned(1024))) uint8_t As[4][GBM * GBK];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[4][BN * GBK];
  // per stage buffer: the 8 block-scale bytes of every tile row, row r at dwords 2r, 2r + 1
  __shared__ __attribute__((aligned(16))) uint32_t nA[4][2 * GBM];
  __shared__ __attribute__((aligned(16))) uint32_t nB[4][2 * BN];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const uint32_t *zsrc4 = kZeroSrc + lane;

  for (int vb = blockIdx.x; vb < a.nblocks; vb += gridDim.x) {
    const int lid = xcd_remap<32>(vb, a.nblocks);
    int g = 0;
    int64_t i0 = 0, ilo = 0, ihi = 0, j0 = 0, l0 = 0;
    int nsteps = 0;
    if (MODE == kWgrad) {
      const int per_g = a.slots * a.jtiles;
      g = lid / per_g;
      int it, jt;
      raster(lid - g * per_g, a.slots, a.jtiles, it, jt);
      i0 = (int64_t)it * GBM;
      j0 = (int64_t)jt * BN;
      ilo = i0;
      ihi = a.I < i0 + GBM ? a.I : i0 + GBM;
      int64_t p_lo = a.pstarts[g], p_hi = a.pstarts[g + 1];
      const int64_t cap = (a.lda < a.ldb ? a.lda : a.ldb) * 2;   // token positions
      p_lo = p_lo < 0 ? 0 : (p_lo > cap ? cap : p_lo);
      p_hi = p_hi < p_lo ? p_lo : (p_hi > cap ? cap : p_hi);
      l0 = p_lo & ~(int64_t)127;
      nsteps = (int)((p_hi - l0) / 128);
    } else {
      int slot, jt;
      raster(lid, a.slots, a.jtiles, slot, jt);
      j0 = (int64_t)jt * BN;
      if (!locate_row_tile(a, slot, g, i0, ilo, ihi)) continue;
      l0 = 0;
      nsteps = (int)(a.L / GBK);
    }

    // code copies: as in grouped_gemm_kernel (64-byte stages of row pairs)
    const int64_t lb = l0 / 128;   // first stage: 128 contraction elements per stage
    const uint8_t *abase = a.a + (i0 >> 1) * 2 * a.lda + lb * 128;
    const uint8_t *bbase = a.b + (MODE == kWgrad ? 0 : (int64_t)g * a.b_gstride) + (j0 >> 1) * 2 * a.ldb + lb * 128;
    const uint8_t *zsrc = reinterpret_cast<const uint8_t *>(kZeroSrc) + lane * 16;
    const int apmax = (int)(((ihi - 1) >> 1) - (i0 >> 1));
    const int64_t jlim = (a.J - j0) < BN ? (a.J - j0) : BN;
    const int bpmax = (int)((jlim - 1) >> 1);
    uint32_t aoff[AQ], boff[BQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int row = (wave * AQ + q) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      const int pr = (row >> 1) < apmax ? (row >> 1) : apmax;
      aoff[q] = (uint32_t)(pr * 2 * (int32_t)a.lda + (row & 1) * 64 + c * 16);
    }
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
      const int row = (wave * BQ + q) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      const int pr = (row >> 1) < bpmax ? (row >> 1) : bpmax;
      boff[q] = (uint32_t)(pr * 2 * (int32_t)a.ldb + (row & 1) * 64 + c * 16);
    }
    // block-scale copies: LDS dword d = 256 c + 64 wave + lane of a stage
    // buffer is dword d % 2 of tile row d / 2; block scales are piece-major,
    // [pieces, rows, 8 bytes], so a stage's bytes of consecutive rows are
    // consecutive in memory
    const int64_t RA = MODE == kWgrad ? a.I : a.M, RB = a.J;
    const uint8_t *nsa[2], *nsb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int d = c * 256 + wave * 64 + lane;
      const int r = d >> 1;
      const int64_t ia = i0 + r, jb = j0 + (r < jlim ? r : jlim - 1);
      const int64_t ra = ia < ilo ? ilo : (ia >= ihi ? ihi - 1 : ia);
      nsa[c] = reinterpret_cast<const uint8_t *>(a.a_scales) + (lb * RA + ra) * 8 + (d & 1) * 4;
      nsb[c] = reinterpret_cast<const uint8_t *>(a.b_scales) + (MODE == kWgrad ? 0 : (int64_t)g * a.bs_gstride) +
               (lb * RB + jb) * 8 + (d & 1) * 4;
    }
    // stage kt into buffer kt % 4; past the contraction: zero codes and zero
    // block scales (the operands are then zero). OPS copies per wave always.
    auto copy = [&](int kt) {
      const int buf = kt & 3;
      const bool real = kt < nsteps;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dma4(real ? (const void *)(nsa[c] + (int64_t)kt * RA * 8) : (const void *)zsrc4, &nA[buf][c * 256 + wave * 64]);
        dma4(real ? (const void *)(nsb[c] + (int64_t)kt * RB * 8) : (const void *)zsrc4, &nB[buf][c * 256 + wave * 64]);
      }
#pragma unroll
      for (int q = 0; q < AQ; ++q)
        dma16(real ? abase + (int64_t)kt * 128 + aoff[q] : zsrc, &As[buf][(wave * AQ + q) * 1024]);
#pragma unroll
      for (int q = 0; q < BQ; ++q)
        dma16(real ? bbase + (int64_t)kt * 128 + boff[q] : zsrc, &Bs[buf][(wave * BQ + q) * 1024]);
      __builtin_amdgcn_sched_barrier(0);
    };

    v16f acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    // operands of one lane: the raw codes and block scales of a stage, and the
    // f16 operands of k16 step S in register set S % 2
    v8i fa[MI], fb[NI];
    uint2 ra[MI], rb[NI];       // the rows' 8 e4m3 block codes of the stage
    NvScale sa[MI], sb[NI];     // the same as f16 pairs
    nv_v8h ao[2][MI], bo[2][NI];
    // raw unit U of stage buffer `buf` (A sub-tiles 0..MI-1, then B): LDS
    // reads only, so a run of them is in flight at once
    auto read_unit = [&](auto u, int buf) __attribute__((always_inline)) {
      constexpr int U = decltype(u)::value;
      if constexpr (U < MI) {
        const int row = wi * WM + U * 32 + l32;
        fa[U] = frag(As[buf], row, h);
        ra[U] = *reinterpret_cast<const uint2 *>(&nA[buf][2 * row]);
      } else {
        const int row = wj * WN + (U - MI) * 32 + l32;
        fb[U - MI] = frag(Bs[buf], row, h);
        rb[U - MI] = *reinterpret_cast<const uint2 *>(&nB[buf][2 * row]);
      }
    };
    // unit U's block scales to f16 (once per stage, before its first decode)
    auto prep_unit = [&](auto u) __attribute__((always_inline)) {
      constexpr int U = decltype(u)::value;
      if constexpr (U < MI)
        sa[U] = nv_scales(ra[U]);
      else
        sb[U - MI] = nv_scales(rb[U - MI]);
    };
    // the f16 operand U of k16 step S (into set S % 2)
    auto decode = [&](auto s, auto u) __attribute__((always_inline)) {
      constexpr int S = decltype(s)::value, U = decltype(u)::value;
      if constexpr (U < MI)
        ao[S % 2][U] = nv_operand((uint32_t)fa[U][S], nv_dd<S>(sa[U]));
      else
        bo[S % 2][U - MI] = nv_operand((uint32_t)fb[U - MI][S], nv_dd<S>(sb[U - MI]));
    };
    using US = std::make_integer_sequence<int, MI + NI>;

    // prologue: stages 0..2 in flight; once stages 0 and 1 have landed, the
    // operands of stage 0's first step are read and decoded
    if (nsteps > 0) {
      copy(0);
      copy(1);
      copy(2);
      wait_vm<1 * OPS>();
      __syncthreads();
      [&]<int... Us>(std::integer_sequence<int, Us...>) {
        (read_unit(std::integral_constant<int, Us>{}, 0), ...);
        (prep_unit(std::integral_constant<int, Us>{}), ...);
        (decode(std::integral_constant<int, 0>{}, std::integral_constant<int, Us>{}), ...);
      }(US{});
    }
    for (int kt = 0; kt < nsteps; ++kt) {
      const int nbuf = (kt + 1) & 3;
      // stage kt + 1 has landed (kt + 2 may be in flight); after the barrier
      // every wave is done with stage kt - 1, whose buffer the copies of
      // stage kt + 3 reuse. The operands of this stage's first step were
      // decoded during the previous stage.
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<1 * OPS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      copy(kt + 3);
      // step S's 16 MFMAs, each second one followed by the decode of one
      // operand of step S + 1; in the last step, the first half reads the
      // next stage's raw operands (the current ones are dead) and the second
      // half decodes the next stage's first step
      [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ([&] {
          constexpr int S = Ss;
          [&]<int... Xs>(std::integer_sequence<int, Xs...>) {
            ([&] {
              constexpr int X = Xs;
              constexpr int mi = X / NI, ni = X % NI;
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao[S % 2][mi], bo[S % 2][ni], acc[mi][ni], 0, 0, 0);
              if constexpr (S + 1 < 8) {
                if constexpr (X % 2 == 1) decode(std::integral_constant<int, S + 1>{}, std::integral_constant<int, X / 2>{});
              } else {
                if constexpr (X < MI + NI) {
                  read_unit(std::integral_constant<int, X>{}, nbuf);
                } else {
                  prep_unit(std::integral_constant<int, X - (MI + NI)>{});
                  decode(std::integral_constant<int, 0>{}, std::integral_constant<int, X - (MI + NI)>{});
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }(), ...);
          }(std::make_integer_sequence<int, MI * NI>{});
        }(), ...);
      }(std::make_integer_sequence<int, 8>{});
    }
    __builtin_amdgcn_sched_barrier(0);
    // the epilogue's first LDS writes read the last MFMAs' accumulators
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" ::: "memory");
    wait_vm<0>();     // every copy (also past the contraction) has landed
    __syncthreads();  // every wave is done with the stage buffers

    // ---- epilogue: the tensor scales, then as in grouped_gemm_kernel
    const float s_a = *reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(a.a_scales) + a.sa_tail);
    const float s_b = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(a.b_scales) +
                                                      a.sb_tail)[MODE == kWgrad ? 0 : g];
    const float scale = s_a * s_b;
    if (ACC && nsteps == 0) continue;  // empty group: dW_g unchanged
    constexpr int STR = WN + 8;
    float *cb = reinterpret_cast<float *>(As[wave]);
    const int64_t jw = j0 + wj * WN;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int v = 8 * hs; v < 8 * hs + 8; ++v)
            cb[(((v >> 2) & 1) * 8 + h * 4 + (v & 3)) * STR + ni * 32 + l32] = acc[mi][ni][v];
        __builtin_amdgcn_wave_barrier();
        if constexpr (MODE == kWgrad) {
          constexpr int CPR4 = WN / 4, CPL4 = 16 * CPR4 / 64;
          float4 old[ACC ? CPL4 : 1];
          if constexpr (ACC) {
#pragma unroll
            for (int k = 0; k < CPL4; ++k) {
              const int id = k * 64 + lane;
              const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + id / CPR4;
              const int64_t j = jw + (id % CPR4) * 4;
              old[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
              if (i >= ilo && i < ihi && j < a.J)
                old[k] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.out) +
                                                           ((int64_t)g * a.I + i) * a.ldo + j);
            }
          }
#pragma unroll
          for (int k = 0; k < CPL4; ++k) {
            const int id = k * 64 + lane;
            const int r = id / CPR4, c4 = id % CPR4;
            const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + r;
            const int64_t j = jw + c4 * 4;
            const float4 x = *reinterpret_cast<const float4 *>(&cb[r * STR + c4 * 4]);
            if (i >= ilo && i < ihi && j < a.J) {
              float4 y = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
              if constexpr (ACC) y = make_float4(y.x + old[k].x, y.y + old[k].y, y.z + old[k].z, y.w + old[k].w);
              *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + ((int64_t)g * a.I + i) * a.ldo + j) = y;
            }
          }
        } else {
          constexpr int CPR = WN / 8, CPL = 16 * CPR / 64;
#pragma unroll
          for (int k = 0; k < CPL; ++k) {
            const int id = k * 64 + lane;
            const int r = id / CPR, c8 = id % CPR;
            const int64_t i = i0 + wi * WM + mi * 32 + hs * 16 + r;
            const int64_t j = jw + c8 * 8;
            const float4 x0 = *reinterpret_cast<const float4 *>(&cb[r * STR + c8 * 8]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&cb[r * STR + c8 * 8 + 4]);
            if (i >= ilo && i < ihi && j < a.J) {
              uint4 o;
              o.x = f32_to_bf16_bits(x0.x * scale) | (f32_to_bf16_bits(x0.y * scale) << 16);
              o.y = f32_to_bf16_bits(x0.z * scale) | (f32_to_bf16_bits(x0.w * scale) << 16);
              o.z = f32_to_bf16_bits(x1.x * scale) | (f32_to_bf16_bits(x1.y * scale) << 16);
              o.w = f32_to_bf16_bits(x1.z * scale) | (f32_to_bf16_bits(x1.w * scale) << 16);
              uint16_t *dst = reinterpret_cast<uint16_t *>(a.out) + i * a.ldo + j;
              if (a.stream_out)
                store16_stream(dst, o);
              else
                *reinterpret_cast<uint4 *>(dst) = o;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();  // the staging buffers are free before the next tile's copies land
  }
}

// ---------------------------------------------------------------------------

// Tile counts of a launch with BN-wide tiles: a.jtiles, a.slots, a.nblocks.
// False when there is nothing to launch (a.nblocks = 0) or too many tiles
// (a.nblocks = -1).
template <int BN>
static bool plan_grid(int mode, GemmArgs &a) {
  a.jtiles = (int)((a.J + BN - 1) / BN);
  int64_t nblocks;
  if (mode == kWgrad) {
    a.slots = (int)((a.I + GBM - 1) / GBM);
    nblocks = (int64_t)a.E * a.slots * a.jtiles;
  } else {
    // upper bound of the row tiles: group g has at most (m_g + 2) / 2 row
    // pairs, so ceil(((m_g + 2) / 2) / (GBM / 2)) <= (m_g + 2) / GBM + 1 tiles
    a.slots = (int)((a.M + 2 * (int64_t)a.E + GBM - 1) / GBM) + a.E;
    nblocks = (int64_t)a.slots * a.jtiles;
  }
  if (nblocks > 0x7fffffff) {
    a.nblocks = -1;
    return false;
  }
  a.nblocks = (int)nblocks;
  return nblocks > 0;
}

// one workgroup per CU (the LDS ring allows one), rounded down to whole
// rounds of the 8 XCDs; each loops over its share of the tiles
static unsigned persistent_grid(int nblocks) {
  int64_t grid = nblocks;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu >= 8) {
    const int64_t persistent = (int64_t)(ncu / 8) * 8;
    grid = nblocks < persistent ? nblocks : persistent;
  }
  return (unsigned)grid;
}

template <int MODE, int RECIPE, int FA, int FB>
static hipError_t launch_cfg(const GemmArgs &a0, hipStream_t st) {
  constexpr int BN = 256;
  GemmArgs a = a0;
  if (!plan_grid<BN>(MODE, a)) return a.nblocks < 0 ? hipErrorInvalidValue : hipSuccess;
  const unsigned grid = persistent_grid(a.nblocks);
  if constexpr (RECIPE == kBlockwise) {
    if constexpr (MODE == kWgrad) {
      if (a.accumulate) {
        blockwise_gemm_kernel<MODE, FA, FB, true><<<grid, 512, 0, st>>>(a);
        return hipGetLastError();
      }
    }
    blockwise_gemm_kernel<MODE, FA, FB, false><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
  } else {
    // the accumulating instance exists for wgrad only
    if constexpr (MODE == kWgrad) {
      if (a.accumulate) {
        grouped_gemm_kernel<MODE, RECIPE, FA, FB, BN, true><<<grid, 256, 0, st>>>(a);
        return hipGetLastError();
      }
    }
    grouped_gemm_kernel<MODE, RECIPE, FA, FB, BN, false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
}

template <int MODE, int RECIPE>
static hipError_t launch_fmt(const GemmArgs &a, int fa, int fb, hipStream_t st) {
  if constexpr (RECIPE == kMx)
    if (fa == kE2M1 && fb == kE2M1) return launch_cfg<MODE, RECIPE, kE2M1, kE2M1>(a, st);
  if (fa == kE4M3 && fb == kE4M3) return launch_cfg<MODE, RECIPE, kE4M3, kE4M3>(a, st);
  if (fa == kE5M2 && fb == kE4M3) return launch_cfg<MODE, RECIPE, kE5M2, kE4M3>(a, st);
  if (fa == kE4M3 && fb == kE5M2) return launch_cfg<MODE, RECIPE, kE4M3, kE5M2>(a, st);
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t launch_nvfp4(const GemmArgs &a0, hipStream_t st) {
  GemmArgs a = a0;
  if (!plan_grid<256>(MODE, a)) return a.nblocks < 0 ? hipErrorInvalidValue : hipSuccess;
  const unsigned grid = persistent_grid(a.nblocks);
  if constexpr (MODE == kWgrad) {
    if (a.accumulate) {
      nvfp4_gemm_kernel<MODE, true><<<grid, 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  nvfp4_gemm_kernel<MODE, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_recipe(const GemmArgs &a, int recipe, int fa, int fb, hipStream_t st) {
  switch (recipe) {
    case kTensorwise:
    case kDelayed: return launch_fmt<MODE, kTensorwise>(a, fa, fb, st);
    case kBlockwise: return launch_fmt<MODE, kBlockwise>(a, fa, fb, st);
    case kNvfp4: return launch_nvfp4<MODE>(a, st);
    default: return launch_fmt<MODE, kMx>(a, fa, fb, st);
  }
}

hipError_t launch_grouped_mm(const GemmParams &p, hipStream_t st) {
  const int64_t epb = p.fmt_a == kE2M1 ? 2 : 1;  // contraction elements per code byte
  GemmArgs a{};
  a.a = p.a;
  a.b = p.b;
  a.a_scales = p.a_scales;
  a.b_scales = p.b_scales;
  a.out = p.out;
  a.ends = p.group_ends;
  a.pstarts = p.padded_starts;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.M = p.M;
  a.E = p.E;
  a.accumulate = p.accumulate;
  // A bf16 output larger than the 256 MiB last-level cache leaves with
  // streaming stores, so that it does not evict the operand lines other tiles
  // re-read (measured: forward / dgrad up to 4.5% faster on such outputs;
  // streaming stores of wgrad's fp32 output were slower, up to 35%, and it
  // keeps plain stores).
  const int64_t out_cols = p.mode == kFwd ? p.N : p.K;
  a.stream_out = p.M * out_cols * 2 > ((int64_t)256 << 20);
  if (p.mode == kFwd) {
    a.I = p.M;
    a.J = p.N;
    a.L = p.K / epb;  // code bytes per row
    a.ldo = p.N;
    a.b_gstride = p.N * p.ldb;
    // blockwise weight scales [E, K/128, N/128]: l-block = k, j-block = n
    a.bs_gstride = p.recipe == kMx ? p.N * (p.K / 32) : (p.K / SBLK) * (p.N / SBLK);
    if (p.recipe == kNvfp4) a.bs_gstride = p.N * (p.K / 16);   // block-code bytes per expert
    a.sa_tail = p.M * (p.K / 16);
    a.sb_tail = (int64_t)p.E * p.N * (p.K / 16);
    a.sb_l = p.N / SBLK;
    a.sb_j = 1;
    return launch_recipe<kFwd>(a, p.recipe, p.fmt_a, p.fmt_b, st);
  }
  if (p.mode == kDgrad) {
    a.I = p.M;
    a.J = p.K;
    a.L = p.N / epb;
    a.ldo = p.K;
    a.b_gstride = p.K * p.ldb;
    // same [E, K/128, N/128] array: l-block = n, j-block = k
    a.bs_gstride = p.recipe == kMx ? p.K * (p.N / 32) : (p.K / SBLK) * (p.N / SBLK);
    if (p.recipe == kNvfp4) a.bs_gstride = p.K * (p.N / 16);
    a.sa_tail = p.M * (p.N / 16);
    a.sb_tail = (int64_t)p.E * p.K * (p.N / 16);
    a.sb_l = 1;
    a.sb_j = p.N / SBLK;
    return launch_recipe<kDgrad>(a, p.recipe, p.fmt_a, p.fmt_b, st);
  }
  a.I = p.K;
  a.J = p.N;
  a.L = 0;
  a.ldo = p.N;
  a.sa_tail = p.K * (p.lda * epb / 16);
  a.sb_tail = p.N * (p.ldb * epb / 16);
  return launch_recipe<kWgrad>(a, p.recipe, p.fmt_a, p.fmt_b, st);
}

}  // namespace mxsg
