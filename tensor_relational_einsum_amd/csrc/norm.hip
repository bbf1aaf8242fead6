// norm.hip -- a sum-of-squares reduce and the RMS-scale map that reads it,
// in one pass over the rows.
//
// The two specs (e.g. "bsh->bs" with g = square, SUM, then
// "bsh,bs,h->bsh" with g = rms_scale) each stream x from HBM once when run
// apart; run together a row is loaded once ("Stax (5): Caching and
// Measurement", Section 7: a reduction and the pointwise map that reads its
// result at the same row index fuse vertically; Section 13.2, Proposition
// 13.3: the gain is the ratio of bytes moved, (2 x + y + 2 ss) / (x + y +
// ss), about 1.67 for f32 x and bf16 y).  The arithmetic is the two specs' own: the row
// statistic is alpha_r * sum of x^2 over the valid columns, stored as f32,
// and y = alpha_m * (x * rsqrt(ss * beta + eps) * gamma), +0 past the valid
// extent of r.  Only the order of the row sum differs from the separate
// reduce (a wavefront tree instead of a lane-group one).
//
// CDNA4 mapping: one wavefront per row, four rows per workgroup, no LDS and
// no barrier.  Lane l holds elements 4 (l + 64 i) .. +3 of each r-block
// piece of the row (16-byte loads for f32, 8-byte for bf16), at most 16
// such vectors (64 registers), so a row of up to 4096 elements is read
// once, reduced with a butterfly of lane exchanges in a fixed order, and
// scaled from registers.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fd_rem(uint32_t n, const FastDiv &f) { return n - fd_div(n, f) * f.d; }

// four elements at element offset `off` of a f32 (dt 0) or bf16 (dt 1) array
__device__ __forceinline__ f32x4 load4(const void *base, int64_t off, int dt) {
  if (dt == 0) return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + off);
  const u32x2 w = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(base) + off);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

__device__ __forceinline__ void store4(void *base, int64_t off, int dt, f32x4 v) {
  if (dt == 0) {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + off) = v;
  } else {
    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(base) + off) =
        u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  }
}

// NVB: vectors per lane per r-block (e_r / 256); the key's joined tuples
// (its r-blocks) are taken in join-list order, at most kNormMaxVec / NVB.
template <int NVB, int XDT>
__global__ __launch_bounds__(256) void norm_pair_kernel(const NormArgs a) {
  constexpr int MAXE = kNormMaxVec / NVB;
  const uint32_t key = fd_div(blockIdx.x, a.div_chunks);
  const uint32_t chunk = blockIdx.x - key * uint32_t(a.chunks);
  const int lane = threadIdx.x & 63;
  const int32_t row = int32_t(chunk) * 4 + int32_t(threadIdx.x >> 6);
  // no barrier and no LDS: a wavefront past the block's rows just leaves
  if (row >= a.rows) return;
  const int32_t cnt = a.counts[key];
  const int32_t *ents = a.list + int64_t(key) * a.per_key * 2;

  // entry e of the key: its x tuple, r-block and valid columns (uniform
  // across the wavefront, recomputed where needed instead of held)
  auto entry = [&](int e, int64_t &xoff, int32_t &kr, int32_t &lim) {
    const uint32_t xt = uint32_t(ents[2 * e + 1]);
    kr = int32_t(fd_rem(fd_div(xt, a.div_wr), a.div_kr));
    const int32_t l = a.n_r - kr * a.e_r;
    lim = l < a.e_r ? l : a.e_r;
    xoff = int64_t(xt) * a.be_x + int64_t(row) * a.e_r;
  };
  f32x4 v[MAXE][NVB];
  float acc = 0.0f;
  bool nonempty = false;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
#pragma unroll
    for (int k = 0; k < NVB; ++k) v[e][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (e < cnt) {
      int64_t xoff;
      int32_t kr, lim;
      entry(e, xoff, kr, lim);
#pragma unroll
      for (int k = 0; k < NVB; ++k) {
        const int32_t c = 4 * (lane + 64 * k);
        v[e][k] = load4(a.x, xoff + c, XDT);
        // padding columns hold +0 already; the mask keeps the sum to the
        // valid columns exactly as the reduce takes them
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (c + w >= lim) v[e][k][w] = 0.0f;
      }
      nonempty = nonempty || lim > 0;
    }
  }
  // sum of squares, then across the wavefront in a fixed order
#pragma unroll
  for (int e = 0; e < MAXE; ++e)
#pragma unroll
    for (int k = 0; k < NVB; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += v[e][k][w] * v[e][k][w];
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  const float ssv = nonempty ? a.alpha_r * acc : 0.0f;
  if (lane == 0) a.ss[int64_t(key) * a.rows + row] = ssv;
  const float rs = rsqrtf(ssv * a.beta + a.eps);
  // y = alpha_m * g(x, ss, gamma), written in x's numbering and layout
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    if (e < cnt) {
      int64_t xoff;
      int32_t kr, lim;
      entry(e, xoff, kr, lim);
#pragma unroll
      for (int k = 0; k < NVB; ++k) {
        const int32_t c = 4 * (lane + 64 * k);
        const f32x4 g = load4(a.gam, int64_t(kr) * a.be_g + c, a.g_dt);
        f32x4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w) y[w] = c + w < lim ? a.alpha_m * (v[e][k][w] * rs * g[w]) : 0.0f;
        store4(a.y, xoff + c, a.y_dt, y);
      }
    }
  }
}

template <int NVB>
hipError_t go(const NormArgs &a, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.n_keys) * a.chunks));
  if (a.x_dt == 0) hipLaunchKernelGGL((norm_pair_kernel<NVB, 0>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((norm_pair_kernel<NVB, 1>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm(const NormArgs &a, hipStream_t st) {
  switch (a.nvb) {
    case 1: return go<1>(a, st);
    case 2: return go<2>(a, st);
    case 4: return go<4>(a, st);
    case 8: return go<8>(a, st);
    case 16: return go<16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace jagg
