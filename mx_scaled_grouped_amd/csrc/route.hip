// Routing permutation of the MoE dispatch: top-k expert choices [T, k] ->
// the routed-row order the grouped GEMM consumes (rows contiguous per
// expert, ascending expert id; within an expert, in token order and then
// choice order), the group ends, and optionally the inverse map from each
// (token, choice) to its routed row. The float8 MoE pages hand the grouped
// matmul rows grouped by expert with cumulative offsets (torchao float8 MoE
// training PR, Summary and Limitations: the override covers the routed
// experts; Megatron-LM bug report, additional context: TEGroupedMLP pads
// those per-expert inputs for FP8).
//
// gfx950 design: 1024-thread workgroups, S per expert plus S for the entries
// with an id outside [0, E). The id array (4 bytes per choice) is small next
// to the activations it orders and stays in the L2 caches. Workgroup (e, s)
// reads all of it once to count the entries that precede expert e's group
// (ids below e), expert e's own, and those of them that come before its
// split s (the splits are consecutive runs of whole 4096-entry chunks); then
// it writes the rows of its split's entries. In that second pass, chunks of
// 4096 entries (4 consecutive ones per thread) are compacted in order with a
// wave prefix sum of the threads' hit counts and one prefix over the 16 wave
// totals, so the order within a group is the entry order (stable) without any
// sort; the next chunk's ids load while the current one is compacted. No
// scratch memory, no atomics on data. (The second pass runs one barrier per
// chunk; splitting it over S workgroups shortens that chain S-fold, at the
// price of S first-pass reads of the ids: 98304 choices over 64 experts,
// S = 6, 75 -> 67 us on their own.)
#include "device_common.hpp"
#include "launch.hpp"
#include "mxsg.h"

namespace mxsg {

constexpr int RT = 1024;          // threads per workgroup
constexpr int RW = RT / 64;       // waves

constexpr int PER = 4;                        // second pass: consecutive entries per thread and chunk
constexpr int64_t CH = (int64_t)RT * PER;     // entries per chunk
constexpr int64_t RSPLIT_CHUNKS = 4;          // at least this many chunks per split
constexpr int RSPLIT_MAX = 8;

// block-wide sums of three counters (RT threads)
__device__ __forceinline__ void block_sum3(int64_t &a, int64_t &b, int64_t &c, int64_t (*red)[RW]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
    c += __shfl_xor(c, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = a;
    red[1][wave] = b;
    red[2][wave] = c;
  }
  __syncthreads();
  a = b = c = 0;
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    a += red[0][w];
    b += red[1][w];
    c += red[2][w];
  }
}

__global__ __launch_bounds__(RT) void route_kernel(const int32_t *__restrict__ ids, int64_t n, int k, int E,
                                                   int32_t *__restrict__ ends, int32_t *__restrict__ row_index,
                                                   int32_t *__restrict__ slot_row, int32_t *__restrict__ status) {
  __shared__ int64_t red[3][RW];
  __shared__ int32_t wtot[2][RW];
  const int e = blockIdx.x;  // expert; e == E: the entries with an invalid id
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // this workgroup's split: entries [lo, hi), whole chunks
  const int64_t nch = (n + CH - 1) / CH;
  const int64_t lo = nch * (int64_t)blockIdx.y / gridDim.y * CH;
  const int64_t hi_c = nch * ((int64_t)blockIdx.y + 1) / gridDim.y * CH;
  const int64_t hi = hi_c < n ? hi_c : n;

  // pass 1: entries of lower experts (the group's start), of this one, and of
  // this one before the split. With 16-byte aligned ids each thread takes
  // four consecutive entries per load and eight loads per iteration, all in
  // flight together (with one 4-byte load per entry the kernel took 67 us
  // instead of 56 on 98304 choices over 64 experts); the tail, or every entry
  // of unaligned ids, one at a time.
  int64_t below = 0, mine = 0, before = 0;
  auto count = [&](int32_t v, int64_t i) __attribute__((always_inline)) {
    const bool valid = v >= 0 && v < E;
    const bool hit = e < E ? v == e : !valid;
    below += e < E ? (valid && v < e) : valid;
    mine += hit;
    before += hit && i < lo;
  };
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(ids) & 15) == 0) {
    const int64_t n4 = n >> 2;
    const int4 *ids4 = reinterpret_cast<const int4 *>(ids);
    for (int64_t b0 = 0; b0 < n4; b0 += (int64_t)RT * 8) {
      int4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t q = b0 + (int64_t)j * RT + t;
        v[j] = q < n4 ? ids4[q] : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t q = b0 + (int64_t)j * RT + t;
        if (q < n4) {
          count(v[j].x, 4 * q);
          count(v[j].y, 4 * q + 1);
          count(v[j].z, 4 * q + 2);
          count(v[j].w, 4 * q + 3);
        }
      }
    }
    done = n4 << 2;
  }
  for (int64_t i = done + t; i < n; i += RT) count(ids[i], i);
  block_sum3(below, mine, before, red);
  if (blockIdx.y == 0) {
    if (e < E) {
      if (t == 0) ends[e] = (int32_t)(below + mine);
    } else if (mine > 0 && t == 0 && status) {
      atomicOr(status, MXSG_STATUS_BAD_EXPERT);
    }
  }
  if (mine == 0 || lo >= hi) return;

  // pass 2: the rows of this split's entries of the group, in entry order,
  // after the group's entries of the earlier splits. The invalid-id
  // workgroups mark their entries' inverse map -1 and fill the row slots past
  // the last group (valid entries .. n) with -1. Chunks of RT * PER entries, PER consecutive
  // entries per thread; the next chunk's ids are loaded before this chunk's
  // barrier, so their latency overlaps it. (Measured on 98304 choices over
  // 64 experts: PER = 4 102 us; 1 entry per thread per chunk 147 us; 16
  // per thread 113 us; four coalesced 1024-entry sub-chunks per barrier 139
  // us.)
  auto load = [&](int64_t base, int32_t (&v)[PER]) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t i = base + (int64_t)t * PER + j;
      v[j] = i < hi ? ids[i] : 0;
    }
  };
  int64_t run = before;
  int buf = 0;
  int32_t cur[PER], nxt[PER];
  load(lo, cur);
  for (int64_t base = lo; base < hi; base += CH) {
    if (base + CH < hi) load(base + CH, nxt);
    unsigned hits = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t i = base + (int64_t)t * PER + j;
      const int32_t v = cur[j];
      const bool hit = i < hi && (e < E ? v == e : !(v >= 0 && v < E));
      hits |= (unsigned)hit << j;
    }
    // exclusive prefix of the threads' hit counts, in entry order
    const int c = __popc(hits);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wtot[buf][wave] = incl;
    __syncthreads();
    int64_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      const int32_t cw = wtot[buf][w];
      off += w < wave ? cw : 0;
      tot += cw;
    }
    int64_t pos = below + run + off + (incl - c);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (hits & (1u << j)) {
        const int64_t i = base + (int64_t)t * PER + j;
        if (e < E) {
          row_index[pos] = (int32_t)(i / k);
          if (slot_row) slot_row[i] = (int32_t)pos;
        } else {
          row_index[pos] = -1;
          if (slot_row) slot_row[i] = -1;
        }
        ++pos;
      }
    }
    run += tot;
    buf ^= 1;  // the next chunk's totals go to the other buffer: one barrier per chunk
#pragma unroll
    for (int j = 0; j < PER; ++j) cur[j] = nxt[j];
  }
}

hipError_t launch_route(const int32_t *ids, int64_t T, int k, int E, int32_t *ends, int32_t *row_index,
                        int32_t *slot_row, int32_t *status, hipStream_t st) {
  const int64_t n = T * k;
  const int64_t nch = (n + CH - 1) / CH;
  int64_t split = nch / RSPLIT_CHUNKS;
  split = split < 1 ? 1 : (split > RSPLIT_MAX ? RSPLIT_MAX : split);
  route_kernel<<<dim3(E + 1, (unsigned)split), RT, 0, st>>>(ids, n, k, E, ends, row_index, slot_row, status);
  return hipGetLastError();
}

}  // namespace mxsg
