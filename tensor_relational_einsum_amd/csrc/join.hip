// join.hip -- join enumeration.
//
// "Every Kernel Is a Join" (Ding et al.), Sec. 3.3: a join-agg spec built
// from interval counts holds one function specification per combination of
// intervals; Def. 3.7 step (1) pairs the input sub-tensors whose keys agree
// on every shared index.  With every input blocked by the same interval
// counts, the matching tuples of a combination are found by arithmetic on
// block coordinates: each input's tuple id is a weighted sum of the block
// coordinates of its letters.  One wavefront lists the combinations of one
// output key (the reduced letters' block coordinates, row-major in order of
// first appearance), compacting with a ballot where a causal pair drops
// some of them, so the list is deterministic.  A segment pair (packed
// sequences, Example 3.10) keeps only the combinations whose s and t blocks
// coincide.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

__global__ __launch_bounds__(256) void join_kernel(const JoinArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t key = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (key >= a.n_keys) return;  // whole wavefront leaves together; no barrier below

  // block coordinates of the output letters, and the part of every input's
  // tuple id they fix
  int64_t base[kMaxIn] = {0, 0, 0};
  int64_t ks = 0, kt_out = 0;
  uint32_t rem = uint32_t(key);
  for (int i = a.n_out - 1; i >= 0; --i) {
    const uint32_t q = fd_div(rem, a.out_div[i]);
    const int64_t kap = int64_t(rem - q * uint32_t(a.out_k[i]));
    rem = q;
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) base[j] += kap * a.w_out[j][i];
    if ((a.causal || a.seg) && !a.s_red && a.s_idx == i) ks = kap;
    if ((a.causal || a.seg) && !a.t_red && a.t_idx == i) kt_out = kap;
  }
  const int stride = 1 + a.n_in;
  int32_t *out = a.list + key * int64_t(a.per_key) * stride;
  int32_t count = 0;
  for (int32_t r0 = 0; r0 < a.per_key; r0 += 64) {
    const int32_t r = r0 + lane;
    bool keep = r < a.per_key;
    int64_t tid[kMaxIn] = {base[0], base[1], base[2]};
    int64_t kt = kt_out;
    uint32_t rr = uint32_t(keep ? r : 0);
    for (int i = a.n_red - 1; i >= 0; --i) {
      const uint32_t q = fd_div(rr, a.red_div[i]);
      const int64_t kap = int64_t(rr - q * uint32_t(a.red_k[i]));
      rr = q;
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j) tid[j] += kap * a.w_red[j][i];
      if ((a.causal || a.seg) && a.t_red && a.t_idx == i) kt = kap;
    }
    if (a.seg && keep) keep = kt == ks;  // segment pair: the same block only
    if (a.causal && keep) {
      const int64_t lo_t = kt * a.e_t;
      int64_t hi_s = (ks + 1) * a.e_s;
      if (hi_s > a.n_s) hi_s = a.n_s;
      keep = lo_t <= hi_s - 1;
    }
    const uint64_t mask = __ballot(keep);
    const int32_t rank = count + __popcll(mask & ((uint64_t(1) << lane) - 1));
    if (keep) {
      int32_t *e = out + int64_t(rank) * stride;
      e[0] = int32_t(key);
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j)
        if (j < a.n_in) e[1 + j] = int32_t(tid[j]);
    }
    count += __popcll(mask);
  }
  // unused slots of this key
  for (int32_t s = count * stride + lane; s < a.per_key * stride; s += 64) out[s] = -1;
  if (lane == 0) a.counts[key] = count;
}

hipError_t launch_join(const JoinArgs &a, hipStream_t st) {
  const int64_t grid = (a.n_keys + 3) / 4;
  hipLaunchKernelGGL(join_kernel, dim3(unsigned(grid)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace jagg
