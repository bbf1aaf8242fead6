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

// tiles per workgroup pass and workgroup cap of the affine kernel
#ifndef JAGG_RELAYOUT_TILES
#define JAGG_RELAYOUT_TILES 4
#endif
#ifndef JAGG_RELAYOUT_MAX_GRID
#define JAGG_RELAYOUT_MAX_GRID (1 << 20)
#endif
constexpr int kRelayoutTiles = JAGG_RELAYOUT_TILES;
constexpr int64_t kRelayoutMaxGrid = JAGG_RELAYOUT_MAX_GRID;

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

// The common case: every letter's blocks nest (no checked letter), so each
// destination vector has a source and both offsets are affine in the
// digits, and at most six tile dims.  The tile digits are decoded with the
// tile dims held in scalar registers; tail tiles re-read the last tile
// instead of branching around the loads, so all U loads are in flight
// together and only the stores are skipped.
template <typename V, int VE, int NT, bool STEP>
__global__ __launch_bounds__(256) void relayout_affine_kernel(const RelayoutArgs a) {
  constexpr int ESZ = int(sizeof(V)) / VE;
  const int tid = threadIdx.x;
  if (tid >= a.lanes) return;  // no barrier below
  int64_t lsrc = 0, ldst = 0;
  uint32_t rem = uint32_t(tid);
  for (int d = 0; d < a.n_lane; ++d) {
    const uint32_t ext = uint32_t(a.lane[d].ext);
    const uint32_t q = rem / ext;
    int64_t dig = int64_t(rem - q * ext);
    rem = q;
    if (d == 0) dig *= VE;
    lsrc += dig * a.lane[d].src;
    ldst += dig * a.lane[d].dst;
  }
  int64_t ts[NT], td[NT];
  FastDiv dv[NT];
#pragma unroll
  for (int d = 0; d < NT; ++d) {
    ts[d] = a.tile[d].src;
    td[d] = a.tile[d].dst;
    dv[d] = a.tile[d].div;
  }
  const char *src = reinterpret_cast<const char *>(a.src) + lsrc * ESZ;
  char *dst = reinterpret_cast<char *>(a.dst) + ldst * ESZ;
  const uint32_t nt = uint32_t(a.n_tiles);
  constexpr int U = kRelayoutTiles;
  for (uint32_t t0 = blockIdx.x * U; t0 < nt; t0 += gridDim.x * U) {
    int64_t so[U], dof[U];
    if constexpr (STEP) {
      // U divides the innermost tile extent and t0: the pass's tiles differ
      // only in that digit, so one decode serves all of them
      uint32_t r = t0;
      int64_t s0 = 0, d0 = 0;
#pragma unroll
      for (int d = NT - 1; d >= 0; --d) {
        const uint32_t q = fd_div(r, dv[d]);
        const int64_t dig = int64_t(r - q * dv[d].d);
        r = q;
        s0 += dig * ts[d];
        d0 += dig * td[d];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        so[u] = s0 + u * ts[NT - 1];
        dof[u] = d0 + u * td[NT - 1];
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t r = t0 + u < nt ? t0 + u : nt - 1;
        so[u] = 0;
        dof[u] = 0;
#pragma unroll
        for (int d = NT - 1; d >= 0; --d) {
          const uint32_t q = fd_div(r, dv[d]);
          const int64_t dig = int64_t(r - q * dv[d].d);
          r = q;
          so[u] += dig * ts[d];
          dof[u] += dig * td[d];
        }
      }
    }
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const V *>(src + so[u] * ESZ);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u < nt) *reinterpret_cast<V *>(dst + dof[u] * ESZ) = v[u];
  }
}

template <typename V, int VE, int NT>
static hipError_t go_affine(const RelayoutArgs &a, hipStream_t st) {
  const int block = ((a.lanes + 63) / 64) * 64;
  int64_t grid = (a.n_tiles + kRelayoutTiles - 1) / kRelayoutTiles;
  if (grid > kRelayoutMaxGrid) grid = kRelayoutMaxGrid;
  if (a.tile[NT - 1].ext % kRelayoutTiles == 0)
    hipLaunchKernelGGL((relayout_affine_kernel<V, VE, NT, true>), dim3(unsigned(grid)), dim3(block), 0, st, a);
  else
    hipLaunchKernelGGL((relayout_affine_kernel<V, VE, NT, false>), dim3(unsigned(grid)), dim3(block), 0, st, a);
  return hipGetLastError();
}

// A digit permutation whose shared innermost run is short on one side (the
// destination's contiguous order walks letters the source strides over, as
// in a transposition of two letters): each workgroup reads one in-tile box
// in source order (runs of at least ~1 KB), parks it in LDS, and writes it
// in destination order (runs of at least ~1 KB).  LDS runs are padded so
// the destination-order reads of 16 consecutive lanes hit distinct banks.
// The in-tile offsets are the same for every box, so each thread decodes
// its NV load and store offsets once.
template <typename V, int VE, int NV>
__global__ __launch_bounds__(256) void relayout_lds_kernel(const RelayoutArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lbuf[];
  constexpr int ESZ = int(sizeof(V)) / VE;  // offsets below count elements
  const int tid = threadIdx.x;
  const int64_t vl = a.lds_v, inner = a.lds_inner, pitch = a.lds_pitch;
  // chain parameters, read once; unused chain slots are identity (divide by
  // one, stride zero), so the decodes below run without branches
  FastDiv cdv[kMaxChain], csv[kMaxChain];
  int64_t cds[kMaxChain], csd[kMaxChain];
#pragma unroll
  for (int d = 0; d < kMaxChain; ++d) {
    cdv[d] = a.cd_div[d];
    cds[d] = a.cd_src[d];
    csv[d] = a.cs_div[d];
    csd[d] = a.cs_dst[d];
  }
  const FastDiv fR = a.lds_R, fRd = a.lds_Rd, fiv = a.lds_iv;
  int32_t ld_src[NV], ld_lds[NV], st_lds[NV], st_dst[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint32_t q = uint32_t(k * 256 + tid);
    // load order: source run `run`, vector `pos` in it; the run's source
    // offset comes from the destination-chain digits
    const uint32_t run = fd_div(q, fR), pos = q - run * fR.d;
    int64_t o = 0;
    uint32_t r = run;
#pragma unroll
    for (int d = 0; d < kMaxChain; ++d) {
      const uint32_t qq = fd_div(r, cdv[d]);
      o += int64_t(r - qq * cdv[d].d) * cds[d];
      r = qq;
    }
    ld_src[k] = int32_t(pos * vl + o);
    ld_lds[k] = int32_t(pos * vl + run * pitch);
    // store order: destination run `r2`, vector `dpos` in it; the run's
    // destination offset comes from the source-chain digits
    const uint32_t r2 = fd_div(q, fRd), dpos = q - r2 * fRd.d;
    o = 0;
    r = r2;
#pragma unroll
    for (int d = 0; d < kMaxChain; ++d) {
      const uint32_t qq = fd_div(r, csv[d]);
      o += int64_t(r - qq * csv[d].d) * csd[d];
      r = qq;
    }
    st_dst[k] = int32_t(dpos * vl + o);
    const uint32_t dr = fd_div(dpos, fiv), iv = dpos - dr * fiv.d;
    st_lds[k] = int32_t(iv * vl + r2 * inner + dr * pitch);
  }
  // outer dims (tile dims, outermost first)
  int64_t os[kMaxLdsOuter], od[kMaxLdsOuter];
  FastDiv ov[kMaxLdsOuter];
#pragma unroll
  for (int d = 0; d < kMaxLdsOuter; ++d) {
    os[d] = a.tile[d].src;
    od[d] = a.tile[d].dst;
    ov[d] = a.tile[d].div;
  }
  // the planner lists the outer dims first and pads the rest with identity
  // dims (extent one, stride zero), so the decode runs without branches
  auto base = [&](uint32_t t, int64_t &bs, int64_t &bd) {
    uint32_t r = t;
    bs = 0;
    bd = 0;
#pragma unroll
    for (int d = kMaxLdsOuter - 1; d >= 0; --d) {
      const uint32_t q = fd_div(r, ov[d]);
      const int64_t dig = int64_t(r - q * ov[d].d);
      r = q;
      bs += dig * os[d];
      bd += dig * od[d];
    }
  };
  // LDS offsets in vectors (every box offset is a multiple of the vector),
  // so the LDS accesses are known 16-byte aligned and stay single b128 ops
  V *lvec = reinterpret_cast<V *>(lbuf);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    ld_lds[k] /= VE;
    st_lds[k] /= VE;
  }
  const char *src = reinterpret_cast<const char *>(a.src);
  char *dst = reinterpret_cast<char *>(a.dst);
  const uint32_t nt = uint32_t(a.n_tiles);
  // one box per pass: its loads go straight into LDS (each box is its own
  // workgroup where the grid allows, so the hardware overlaps one box's
  // loads with another's stores; a register prefetch of the next box made
  // the compiler wait on each load in turn and ran 2.4x slower)
  for (uint32_t t = blockIdx.x; t < nt; t += gridDim.x) {
    int64_t bs, bd;
    base(t, bs, bd);
    V v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = *reinterpret_cast<const V *>(src + (bs + ld_src[k]) * ESZ);
#pragma unroll
    for (int k = 0; k < NV; ++k) lvec[ld_lds[k]] = v[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = lvec[st_lds[k]];
#pragma unroll
    for (int k = 0; k < NV; ++k) *reinterpret_cast<V *>(dst + (bd + st_dst[k]) * ESZ) = v[k];
    __syncthreads();
  }
}

template <typename V, int VE>
static hipError_t go(const RelayoutArgs &a, hipStream_t st) {
  if (a.lds) {
    const int64_t grid = a.n_tiles < (int64_t(1) << 20) ? a.n_tiles : (int64_t(1) << 20);
    switch (a.lds_nv) {
      case 1: hipLaunchKernelGGL((relayout_lds_kernel<V, VE, 1>), dim3(unsigned(grid)), dim3(256), a.lds_bytes, st, a); break;
      case 2: hipLaunchKernelGGL((relayout_lds_kernel<V, VE, 2>), dim3(unsigned(grid)), dim3(256), a.lds_bytes, st, a); break;
      case 4: hipLaunchKernelGGL((relayout_lds_kernel<V, VE, 4>), dim3(unsigned(grid)), dim3(256), a.lds_bytes, st, a); break;
      case 8: hipLaunchKernelGGL((relayout_lds_kernel<V, VE, 8>), dim3(unsigned(grid)), dim3(256), a.lds_bytes, st, a); break;
      case 16: hipLaunchKernelGGL((relayout_lds_kernel<V, VE, 16>), dim3(unsigned(grid)), dim3(256), a.lds_bytes, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (a.n_chk == 0 && a.n_tiles < (int64_t(1) << 31)) {
    switch (a.n_tile) {
      case 1: return go_affine<V, VE, 1>(a, st);
      case 2: return go_affine<V, VE, 2>(a, st);
      case 3: return go_affine<V, VE, 3>(a, st);
      case 4: return go_affine<V, VE, 4>(a, st);
      case 5: return go_affine<V, VE, 5>(a, st);
      case 6: return go_affine<V, VE, 6>(a, st);
    }
  }
  const int block = ((a.lanes + 63) / 64) * 64;
  int64_t grid = (a.n_tiles + 3) / 4;
  if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
  hipLaunchKernelGGL((relayout_kernel<V, VE>), dim3(unsigned(grid)), dim3(block), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- interval letters
// "Every Kernel Is a Join", Def. 3.1 and Sec. 3.3: a key is an interval per
// index, and an index may be cut only at legal positions (the ends of packed
// sequences), so blocks of one letter can differ in length; storage pads
// each to the longest.  The affine digit walk above needs nesting uniform
// blocks, so these copies take this kernel: per destination vector, decode
// the coordinates, zero-fill padding, locate the source block of each
// index (a division, or a search of that letter's bounds held in LDS).
// A vector never straddles a block or padding edge: the host picks the width
// so that every bound of the innermost letter is a multiple of it.
// source offset (elements) of destination vector i, or -1 for padding
__device__ __forceinline__ int64_t iv_source(const IvRelayoutArgs &a, const int32_t *bnd, uint32_t i,
                                             uint32_t vshift) {
  const uint32_t t0 = fd_div(i, a.be_v);
  uint32_t w = (i - t0 * a.be_v.d) << vshift;  // element offset inside the destination block
  uint32_t t = t0;
  uint32_t soff = 0;
  bool valid = true;
#pragma unroll
  for (int p = kMaxLetters - 1; p >= 0; --p) {
    if (p >= a.r) continue;
    const IvRelayoutDim &d = a.d[p];
    const uint32_t wq = fd_div(w, d.de), tq = fd_div(t, d.dk);
    const uint32_t wp = w - wq * d.de.d, kp = t - tq * d.dk.d;
    w = wq;
    t = tq;
    uint32_t lo, hi;
    if (d.d_bnd >= 0) {
      lo = uint32_t(bnd[d.d_bnd + kp]);
      hi = uint32_t(bnd[d.d_bnd + kp + 1]);
    } else {
      lo = kp * d.de.d;
      hi = min(lo + d.de.d, uint32_t(d.n));
    }
    const uint32_t x = lo + wp;
    valid = valid && x < hi;
    uint32_t ks, slo;
    if (d.s_bnd >= 0) {
      // largest ks with bound[ks] <= x, over ks in [0, s_k); s_k <= kMaxIv
      ks = 0;
#pragma unroll
      for (int step = kMaxIv / 2; step >= 1; step >>= 1)
        if (ks + step < uint32_t(d.s_k) && uint32_t(bnd[d.s_bnd + ks + step]) <= x) ks += step;
      slo = uint32_t(bnd[d.s_bnd + ks]);
    } else {
      ks = fd_div(x, d.s_e);
      slo = ks * d.s_e.d;
    }
    soff += ks * d.s_tw + (x - slo) * d.s_ew;
  }
  return valid ? int64_t(soff) : int64_t(-1);
}

// Vector form (short rows): one destination vector per thread and pass.
template <typename V>
__global__ __launch_bounds__(256) void relayout_iv_kernel(const IvRelayoutArgs a) {
  __shared__ int32_t bnd[kIvPool];
  for (int i = threadIdx.x; i < a.n_pool; i += blockDim.x) bnd[i] = a.pool[i];
  __syncthreads();
  const V *src = static_cast<const V *>(a.src);
  V *dst = static_cast<V *>(a.dst);
  const uint32_t vshift = a.v == 1 ? 0 : (a.v == 2 ? 1 : (a.v == 4 ? 2 : 3));
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n_vec; i += gridDim.x * blockDim.x) {
    const int64_t so = iv_source(a, bnd, i, vshift);
    V val;
    memset(&val, 0, sizeof(V));
    if (so >= 0) val = src[uint32_t(so) >> vshift];
    dst[i] = val;
  }
}

// vectors in flight per lane in the row form
constexpr int kIvUnroll = 4;

// Row form: with long rows along the innermost destination letter, a wave
// decodes the outer letters of one row once (uniform values) and its lanes
// stream the row, mapping only the innermost index per vector.
template <typename V>
__global__ __launch_bounds__(256) void relayout_iv_rows_kernel(const IvRelayoutArgs a) {
  __shared__ int32_t bnd[kIvPool];
  for (int i = threadIdx.x; i < a.n_pool; i += blockDim.x) bnd[i] = a.pool[i];
  __syncthreads();
  const V *src = static_cast<const V *>(a.src);
  V *dst = static_cast<V *>(a.dst);
  const uint32_t vshift = a.v == 1 ? 0 : (a.v == 2 ? 1 : (a.v == 4 ? 2 : 3));
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (uint32_t row = blockIdx.x * 4 + wave; row < a.n_rows; row += gridDim.x * 4) {
    uint32_t t = fd_div(row, a.rows_pt);
    uint32_t w = row - t * a.rows_pt.d;
    uint32_t soff = 0;
    bool valid = true;
    uint32_t lo_in = 0, hi_in = 0, k_in = 0, tw_in = 0, ew_in = 0;
    int32_t sb_in = -1;
    FastDiv se_in = a.d[0].s_e;
#pragma unroll
    for (int p = kMaxLetters - 1; p >= 0; --p) {
      if (p >= a.r) continue;
      const IvRelayoutDim &d = a.d[p];
      const uint32_t tq = fd_div(t, d.dk);
      const uint32_t kp = t - tq * d.dk.d;
      t = tq;
      uint32_t lo, hi;
      if (d.d_bnd >= 0) {
        lo = uint32_t(bnd[d.d_bnd + kp]);
        hi = uint32_t(bnd[d.d_bnd + kp + 1]);
      } else {
        lo = kp * d.de.d;
        hi = min(lo + d.de.d, uint32_t(d.n));
      }
      if (p == a.r - 1) {  // innermost: mapped per vector below
        lo_in = lo;
        hi_in = hi;
        sb_in = d.s_bnd;
        k_in = uint32_t(d.s_k);
        se_in = d.s_e;
        tw_in = d.s_tw;
        ew_in = d.s_ew;
        continue;
      }
      const uint32_t wq = fd_div(w, d.de);
      const uint32_t x = lo + (w - wq * d.de.d);
      w = wq;
      valid = valid && x < hi;
      uint32_t ks, slo;
      if (d.s_bnd >= 0) {
        ks = 0;
#pragma unroll
        for (int step = kMaxIv / 2; step >= 1; step >>= 1)
          if (ks + step < uint32_t(d.s_k) && uint32_t(bnd[d.s_bnd + ks + step]) <= x) ks += step;
        slo = uint32_t(bnd[d.s_bnd + ks]);
      } else {
        ks = fd_div(x, d.s_e);
        slo = ks * d.s_e.d;
      }
      soff += ks * d.s_tw + (x - slo) * d.s_ew;
    }
    V *drow = dst + size_t(row) * a.row_vecs;
    for (uint32_t j0 = 0; j0 < a.row_vecs; j0 += 64 * kIvUnroll) {
      V val[kIvUnroll];
#pragma unroll
      for (int u = 0; u < kIvUnroll; ++u) {
        const uint32_t j = j0 + u * 64 + lane;
        const uint32_t x = lo_in + (j << vshift);
        memset(&val[u], 0, sizeof(V));
        if (valid && j < a.row_vecs && x < hi_in) {
          uint32_t ks, slo;
          if (sb_in >= 0) {
            ks = 0;
#pragma unroll
            for (int step = kMaxIv / 2; step >= 1; step >>= 1)
              if (ks + step < k_in && uint32_t(bnd[sb_in + ks + step]) <= x) ks += step;
            slo = uint32_t(bnd[sb_in + ks]);
          } else {
            ks = fd_div(x, se_in);
            slo = ks * se_in.d;
          }
          val[u] = src[(soff + ks * tw_in + (x - slo) * ew_in) >> vshift];
        }
      }
#pragma unroll
      for (int u = 0; u < kIvUnroll; ++u) {
        const uint32_t j = j0 + u * 64 + lane;
        if (j < a.row_vecs) drow[j] = val[u];
      }
    }
  }
}

template <typename V>
hipError_t go_iv(const IvRelayoutArgs &a, hipStream_t st) {
  if (a.rows) {
    const int64_t want = (int64_t(a.n_rows) + 3) / 4;
    const int grid = int(want < 8192 ? (want > 0 ? want : 1) : 8192);
    relayout_iv_rows_kernel<V><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const int64_t want = (int64_t(a.n_vec) + 255) / 256;
  const int grid = int(want < 8192 ? (want > 0 ? want : 1) : 8192);
  relayout_iv_kernel<V><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_relayout_iv(const IvRelayoutArgs &a, int vec_bytes, hipStream_t st) {
  switch (vec_bytes) {
    case 16: return go_iv<uint4>(a, st);
    case 8: return go_iv<uint2>(a, st);
    case 4: return go_iv<uint32_t>(a, st);
    case 2: return go_iv<uint16_t>(a, st);
  }
  return hipErrorInvalidValue;
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
