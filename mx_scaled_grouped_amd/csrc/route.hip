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
// gfx950 design: one 1024-thread workgroup per expert, plus one for the
// entries with an id outside [0, E). The id array (4 bytes per choice) is
// small next to the activations it orders and stays in the L2 caches, so
// every workgroup reads all of it twice: once to count the entries that
// precede its expert's group (ids below e) and its own, once to write its
// rows. Within a pass, chunks of 1024 entries are compacted in order with a
// wave ballot (lane prefix = popcount of the lower lanes' bits) and one
// prefix over the 16 wave totals, so the order within a group is the entry
// order (stable) without any sort. No scratch memory, no atomics on data.
#include "device_common.hpp"
#include "launch.hpp"
#include "mxsg.h"

namespace mxsg {

constexpr int RT = 1024;          // threads per workgroup
constexpr int RW = RT / 64;       // waves

// block-wide sum of two counters (RT threads)
__device__ __forceinline__ void block_sum2(int64_t &a, int64_t &b, int64_t (*red)[RW]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = a;
    red[1][wave] = b;
  }
  __syncthreads();
  a = b = 0;
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    a += red[0][w];
    b += red[1][w];
  }
}

__global__ __launch_bounds__(RT) void route_kernel(const int32_t *__restrict__ ids, int64_t n, int k, int E,
                                                   int32_t *__restrict__ ends, int32_t *__restrict__ row_index,
                                                   int32_t *__restrict__ slot_row, int32_t *__restrict__ status) {
  __shared__ int64_t red[2][RW];
  __shared__ int32_t wtot[2][RW];
  const int e = blockIdx.x;  // expert; e == E: the entries with an invalid id
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // pass 1: entries of lower experts (the group's start) and of this one
  int64_t below = 0, mine = 0;
  for (int64_t i = t; i < n; i += RT) {
    const int32_t v = ids[i];
    const bool valid = v >= 0 && v < E;
    if (e < E) {
      below += valid && v < e;
      mine += v == e;
    } else {
      below += valid;
      mine += !valid;
    }
  }
  block_sum2(below, mine, red);
  if (e < E) {
    if (t == 0) ends[e] = (int32_t)(below + mine);
  } else if (mine > 0 && t == 0 && status) {
    atomicOr(status, MXSG_STATUS_BAD_EXPERT);
  }
  if (mine == 0) return;

  // pass 2: this group's rows in entry order. The invalid-id workgroup marks
  // its entries' inverse map -1 and fills the row slots past the last group
  // (valid entries .. n) with -1.
  int64_t run = 0;
  int buf = 0;
  for (int64_t base = 0; base < n; base += RT) {
    const int64_t i = base + t;
    bool hit = false;
    if (i < n) {
      const int32_t v = ids[i];
      hit = e < E ? v == e : !(v >= 0 && v < E);
    }
    const uint64_t m = __ballot(hit);
    if (lane == 0) wtot[buf][wave] = (int32_t)__popcll(m);
    __syncthreads();
    int64_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      const int32_t c = wtot[buf][w];
      off += w < wave ? c : 0;
      tot += c;
    }
    if (hit) {
      const int64_t pos = below + run + off + __popcll(m & ((1ull << lane) - 1ull));
      if (e < E) {
        row_index[pos] = (int32_t)(i / k);
        if (slot_row) slot_row[i] = (int32_t)pos;
      } else {
        row_index[pos] = -1;
        if (slot_row) slot_row[i] = -1;
      }
    }
    run += tot;
    buf ^= 1;  // the next chunk's totals go to the other buffer: one barrier per chunk
  }
}

hipError_t launch_route(const int32_t *ids, int64_t T, int k, int E, int32_t *ends, int32_t *row_index,
                        int32_t *slot_row, int32_t *status, hipStream_t st) {
  route_kernel<<<E + 1, RT, 0, st>>>(ids, T * k, k, E, ends, row_index, slot_row, status);
  return hipGetLastError();
}

}  // namespace mxsg
