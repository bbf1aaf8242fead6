// relayout.hip -- repartition of a relation on one GPU.
//
// "Every Kernel Is a Join" (Ding et al.), Sec. 5.3: the exchange between a
// producer's blocking and a consumer's blocking works on atoms, the cells of
// the overlay of both families of block bounds; decompose kernels slice
// blocks into atoms and recompose kernels concatenate atoms into the
// consumer's blocks.  On one GPU the two steps fuse into this single copy:
// every destination element (padding included, written as +0) is read from
// its source position.  The host planner expresses each letter's index as
// digits whose source and destination offsets are both affine (an atom is a
// box of such digits), so a thread never divides except for letters whose
// blocks do not nest.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

template <typename V, int VE>
__global__ __launch_bounds__(256) void relayout_kernel(const RelayoutArgs a) {
  constexpr int ESZ = int(sizeof(V)) / VE;
  const int tid = threadIdx.x;
  if (tid >= a.lanes) return;  // no barrier below

  // lane part, decoded once per thread (lane dim 0 counts vectors)
  int64_t lsrc = 0, ldst = 0;
  int64_t lx[kMaxChk];
#pragma unroll
  for (int c = 0; c < kMaxChk; ++c) lx[c] = 0;
  uint32_t rem = uint32_t(tid);
  for (int d = 0; d < a.n_lane; ++d) {
    const uint32_t ext = uint32_t(a.lane[d].ext);
    const uint32_t q = rem / ext;
    int64_t dig = int64_t(rem - q * ext);
    rem = q;
    if (d == 0) dig *= VE;
    lsrc += dig * a.lane[d].src;
    ldst += dig * a.lane[d].dst;
    const int chk = a.lane[d].chk;
#pragma unroll
    for (int c = 0; c < kMaxChk; ++c)
      if (chk == c) lx[c] += dig * a.lane[d].xs;
  }

  // four tiles per workgroup pass: all four reads are issued before the
  // first write
  constexpr int U = 4;
  for (int64_t t0 = int64_t(blockIdx.x) * U; t0 < a.n_tiles; t0 += int64_t(gridDim.x) * U) {
    V v[U];
    int64_t dof[U];
    bool wr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u;
      wr[u] = false;
      if (t >= a.n_tiles) continue;
      // tile part: uniform across the workgroup
      int64_t tsrc = 0, tdst = 0;
      int64_t tx[kMaxChk];
#pragma unroll
      for (int c = 0; c < kMaxChk; ++c) tx[c] = 0;
      uint32_t r = uint32_t(t);
      for (int d = a.n_tile - 1; d >= 0; --d) {
        const uint32_t q = fd_div(r, a.tile[d].div);
        const int64_t dig = int64_t(r - q * a.tile[d].div.d);
        r = q;
        tsrc += dig * a.tile[d].src;
        tdst += dig * a.tile[d].dst;
        const int chk = a.tile[d].chk;
#pragma unroll
        for (int c = 0; c < kMaxChk; ++c)
          if (chk == c) tx[c] += dig * a.tile[d].xs;
      }
      bool rd = true, w = true;
      int64_t so = tsrc + lsrc;
#pragma unroll
      for (int c = 0; c < kMaxChk; ++c) {
        if (c < a.n_chk) {
          const int64_t x = tx[c] + lx[c];
          rd = rd && (x < a.read_lim[c]);
          w = w && (x < a.write_lim[c]);
          if (a.irr[c]) {
            const uint32_t xv = uint32_t(x);
            const uint32_t kb = fd_div(xv, a.irr_div[c]);
            so += int64_t(kb) * a.irr_K[c] + int64_t(xv - kb * a.irr_div[c].d) * a.irr_E[c];
          }
        }
      }
      wr[u] = w;
      dof[u] = tdst + ldst;
      if (w && rd) {
        v[u] = *reinterpret_cast<const V *>(reinterpret_cast<const char *>(a.src) + so * ESZ);
      } else {
        v[u] = V{};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (wr[u]) *reinterpret_cast<V *>(reinterpret_cast<char *>(a.dst) + dof[u] * ESZ) = v[u];
  }
}

template <typename V, int VE>
static hipError_t go(const RelayoutArgs &a, hipStream_t st) {
  const int block = ((a.lanes + 63) / 64) * 64;
  int64_t grid = (a.n_tiles + 3) / 4;
  if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
  hipLaunchKernelGGL((relayout_kernel<V, VE>), dim3(unsigned(grid)), dim3(block), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_relayout(const RelayoutArgs &a, int vec_bytes, int elem_bytes, hipStream_t st) {
  if (elem_bytes == 2) {
    switch (vec_bytes) {
      case 16: return go<uint4, 8>(a, st);
      case 8: return go<uint2, 4>(a, st);
      case 4: return go<uint32_t, 2>(a, st);
      case 2: return go<uint16_t, 1>(a, st);
    }
  } else if (elem_bytes == 4) {
    switch (vec_bytes) {
      case 16: return go<uint4, 4>(a, st);
      case 8: return go<uint2, 2>(a, st);
      case 4: return go<uint32_t, 1>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace jagg
