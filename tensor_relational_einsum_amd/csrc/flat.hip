// flat.hip -- streaming map and row-reduce kernels for row-compatible operands.
//
// "Every Kernel Is a Join" (Ding et al.), Def. 3.7: f runs on every joined
// tuple of an output key and the results of equal key are combined with the
// aggregation.  For a map each key joins one tuple and f is g element by
// element; for a row reduce f is g followed by the aggregation along the
// one reduced letter, and the aggregation across the key's joined tuples
// happens in the same pass.
//
// These kernels are HBM streams, so they are written for bytes in flight:
// every load of an iteration is issued (as raw bits, through buffer loads
// whose out-of-range lanes read zeros) before anything is converted or
// combined, and all offsets are 32-bit within a block.  The planner sends
// here only operands whose in-block offsets are affine in the row index
// (see FlatArgs); everything else takes the general kernels.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kFar = 0x80000000u;  // byte offset past any block: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *p, int64_t tuple, uint32_t block_bytes) {
  const char *b = reinterpret_cast<const char *>(p) + tuple * int64_t(block_bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(b), (short)0, int(block_bytes), 0x00020000);
}

// Raw bits of V consecutive elements (inner = 1) or of one element repeated
// (inner = 0).  f32 uses V words, bf16 V/2.
template <int V>
struct Raw {
  uint32_t w[V];
};

template <int V>
__device__ __forceinline__ void raw_load(Raw<V> &r, __amdgpu_buffer_rsrc_t rs, uint32_t elem, bool in, int dt,
                                         int inner) {
  // every word is defined on every path, so the paths merge without copies
#pragma unroll
  for (int u = 0; u < V; ++u) r.w[u] = 0;
  if (inner) {
    if (dt) {
      const uint32_t off = in ? elem * 2 : kFar;
      if constexpr (V == 8) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, int(off), 0, 0);
        r.w[0] = q.x, r.w[1] = q.y, r.w[2] = q.z, r.w[3] = q.w;
      } else if constexpr (V == 4) {
        const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(rs, int(off), 0, 0);
        r.w[0] = q.x, r.w[1] = q.y;
      } else {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, int(off), 0, 0);
      }
    } else {
      const uint32_t off = in ? elem * 4 : kFar;
      if constexpr (V >= 4) {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
          const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, int(off + 16 * h), 0, 0);
          r.w[4 * h] = q.x, r.w[4 * h + 1] = q.y, r.w[4 * h + 2] = q.z, r.w[4 * h + 3] = q.w;
        }
      } else {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, int(off), 0, 0);
      }
    }
  } else {
    r.w[0] = dt ? uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rs, int(in ? elem * 2 : kFar), 0, 0))
                : __builtin_amdgcn_raw_buffer_load_b32(rs, int(in ? elem * 4 : kFar), 0, 0);
  }
}

// Conversion by selects on the (uniform) dtype and kind rather than
// branches: a branch on the same condition as the load's would be merged
// with it, and the conversion would then wait for each load in turn.
template <int V>
__device__ __forceinline__ void raw_to_f32(const Raw<V> &r, int dt, int inner, float *x) {
  if constexpr (V == 1) {
    x[0] = __uint_as_float(dt ? (r.w[0] << 16) : r.w[0]);
  } else {
    const uint32_t b0 = dt ? (r.w[0] << 16) : r.w[0];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const uint32_t hb = (u & 1) ? (r.w[u / 2] & 0xffff0000u) : (r.w[u / 2] << 16);
      const uint32_t v = inner ? (dt ? hb : r.w[u]) : b0;
      x[u] = __uint_as_float(v);
    }
  }
}

template <int V>
__device__ __forceinline__ void store_vec(void *base, int64_t off, int dt, const float *y) {
  if (dt) {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + off;
    if constexpr (V == 8) {
      *reinterpret_cast<uint4 *>(p) =
          uint4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    } else if constexpr (V == 4) {
      *reinterpret_cast<uint2 *>(p) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      p[0] = f32_to_bf16(y[0]);
    }
  } else {
    float *p = reinterpret_cast<float *>(base) + off;
    if constexpr (V >= 4) {
#pragma unroll
      for (int u = 0; u < V; u += 4) *reinterpret_cast<float4 *>(p + u) = make_float4(y[u], y[u + 1], y[u + 2], y[u + 3]);
    } else {
      p[0] = y[0];
    }
  }
}

__device__ __forceinline__ uint32_t fd_mod(uint32_t n, const FastDiv &f) { return n - fd_div(n, f) * f.d; }

}  // namespace

// ------------------------------------------------------------------ map
// Every input costs exactly two 16-byte buffer loads per vector of 8
// elements, whatever its dtype and kind: f32 along the row takes both, bf16
// along the row the first (the second is sent out of range and reads
// nothing), and a row-constant input the aligned 16 bytes that hold its
// element.  With no branch on the dtype, all loads of a pass are in flight
// together; the conversion selects on the uniform dtype and kind.
struct MapLoad {
  u32x4 a, b;
};

__device__ __forceinline__ void map_issue(MapLoad &m, __amdgpu_buffer_rsrc_t rs, const FlatIn &in, uint32_t row,
                                          uint32_t el, bool live, uint32_t &pos) {
  const uint32_t sh = in.dt ? 1u : 2u;
  const uint32_t off = (row * uint32_t(in.row_mul) + (in.inner ? el : 0u)) << sh;
  pos = off;
  const uint32_t oa = live ? (in.inner ? off : (off & ~15u)) : kFar;
  const uint32_t ob = (live && in.inner && !in.dt) ? off + 16u : kFar;
  m.a = __builtin_amdgcn_raw_buffer_load_b128(rs, int(oa), 0, 0);
  m.b = __builtin_amdgcn_raw_buffer_load_b128(rs, int(ob), 0, 0);
}

__device__ __forceinline__ void map_convert(const MapLoad &m, const FlatIn &in, uint32_t pos, float *x) {
  const uint32_t w[8] = {m.a.x, m.a.y, m.a.z, m.a.w, m.b.x, m.b.y, m.b.z, m.b.w};
  // row-constant element: word (pos / 4) % 4 of the aligned chunk, half (pos / 2) % 2 for bf16
  const uint32_t q = (pos >> 2) & 3u;
  const uint32_t word = q == 0 ? m.a.x : (q == 1 ? m.a.y : (q == 2 ? m.a.z : m.a.w));
  const uint32_t bc = in.dt ? ((pos & 2u) ? (word & 0xffff0000u) : (word << 16)) : word;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t hb = (u & 1) ? (w[u / 2] & 0xffff0000u) : (w[u / 2] << 16);
    const uint32_t v = in.inner ? (in.dt ? hb : w[u]) : bc;
    x[u] = __uint_as_float(v);
  }
}

// A thread handles U vectors 256 apart per pass.
template <int G, int U>
__global__ __launch_bounds__(256) void flat_map_kernel(const FlatArgs a) {
  constexpr int V = 8;
  const uint32_t key = fd_div(blockIdx.x, a.div_chunks);
  const uint32_t chunk = blockIdx.x - key * uint32_t(a.chunks);
  if (a.counts[key] == 0) return;  // tuple absent from the output relation
  const int32_t *ent = a.list + int64_t(key) * a.per_key * (1 + a.n_in);
  __amdgpu_buffer_rsrc_t rs[kMaxIn];
#pragma unroll
  for (int j = 0; j < kMaxIn; ++j)
    rs[j] = block_rsrc(a.in[j].p, j < a.n_in ? ent[1 + j] : 0, j < a.n_in ? a.in[j].block_bytes : 0);
  // valid extent of the innermost letter in this key, and the causal s block
  const uint32_t kap_last = fd_mod(key, a.div_klast);
  const int32_t t0 = int32_t(kap_last) * a.e_last;
  const int32_t valid_last = a.n_last - t0;
  int32_t s0 = 0;
  if (a.causal) s0 = int32_t(fd_mod(fd_div(key, a.div_Ws), a.div_ks)) * a.e_s;
  const int64_t obase = int64_t(key) * a.be_out;
  const uint32_t stride = uint32_t(a.chunks) * 256u * U;
  for (uint32_t p0 = chunk * 256u * U + threadIdx.x; p0 < uint32_t(a.slots); p0 += stride) {
    uint32_t row[U], el[U], pos[U][kMaxIn];
    bool live[U];
    MapLoad ld[U][kMaxIn];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t slot = p0 + u * 256u;
      live[u] = slot < uint32_t(a.slots);
      row[u] = fd_div(slot, a.div_vpr);
      el[u] = (slot - row[u] * uint32_t(a.vpr)) * V;
      // absent inputs have an empty buffer resource: their loads read zeros
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j) map_issue(ld[u][j], rs[j], a.in[j], row[u], el[u], live[u], pos[u][j]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[kMaxIn][V];
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j) {
        map_convert(ld[u][j], a.in[j], pos[u][j], x[j]);
        if (j >= a.n_in) {
#pragma unroll
          for (int w = 0; w < V; ++w) x[j][w] = g_fill<G>();
        }
      }
      // elements [0, lim) are inside the output and on the allowed side of a
      // causal pair (t <= s); the rest are padding and get +0
      int32_t lim = valid_last - int32_t(el[u]);
      if (a.causal) {
        const int32_t s = s0 + int32_t(fd_mod(fd_div(row[u], a.div_Rs), a.div_es));
        const int32_t m = s - t0 - int32_t(el[u]) + 1;
        lim = m < lim ? m : lim;
      }
      float y[V];
#pragma unroll
      for (int w = 0; w < V; ++w) {
        const float v = a.alpha * g_fn<G>(x[0][w], x[1][w], x[2][w], a.beta, a.eps);
        y[w] = w < lim ? v : 0.0f;
      }
      if (live[u]) store_vec<V>(a.out, obase + int64_t(row[u]) * a.e_last + el[u], a.out_dt, y);
    }
  }
}

// ------------------------------------------------------------------ row reduce
// A group of 2^lpr_log2 lanes owns one output element.  The key's joined
// tuples are taken EU at a time: the EU vectors a lane needs from them are
// loaded together and then combined in join-list order, so the result is
// deterministic.
// VU: row steps loaded together (1, or 4 where a row holds at least four)
template <int V, int G, int AGG, int EU, int DT0, int VU>
__global__ __launch_bounds__(256) void flat_reduce_kernel(const FlatArgs a, int lpr_log2) {
  const uint32_t key = fd_div(blockIdx.x, a.div_chunks);
  const uint32_t chunk = blockIdx.x - key * uint32_t(a.chunks);
  const int32_t cnt = a.counts[key];
  const int32_t width = 1 + a.n_in;
  const int32_t *ents = a.list + int64_t(key) * a.per_key * width;
  const int lpr = 1 << lpr_log2;
  const int sub = threadIdx.x & (lpr - 1);
  const int group = threadIdx.x >> lpr_log2;
  const int groups = 256 >> lpr_log2;
  const int step = lpr * V;
  int32_t s0 = 0;
  if (a.causal) s0 = int32_t(fd_mod(fd_div(key, a.div_Ws), a.div_ks)) * a.e_s;
  // broadcast inputs (no reduced letter) read the key's first joined tuple
  __amdgpu_buffer_rsrc_t bs[kMaxIn];
#pragma unroll
  for (int j = 0; j < kMaxIn; ++j)
    bs[j] = block_rsrc(a.in[j].p, (j < a.n_in && cnt > 0) ? ents[1 + j] : 0, (j < a.n_in && cnt > 0) ? a.in[j].block_bytes : 0);
  for (uint32_t q0 = chunk * uint32_t(groups); q0 < uint32_t(a.be_out); q0 += uint32_t(a.chunks * groups)) {
    const uint32_t q = q0 + group;
    const bool live = q < uint32_t(a.be_out);
    const int32_t s = a.causal ? s0 + int32_t(fd_mod(fd_div(q, a.div_Rs), a.div_es)) : 0;
    float bc[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) {
      bc[j] = g_fill<G>();
      if (j > 0 && j < a.n_in && !a.in[j].inner) {
        Raw<1> r;
        raw_load<1>(r, bs[j], q * uint32_t(a.in[j].row_mul), live, a.in[j].dt, 0);
        raw_to_f32<1>(r, a.in[j].dt, 0, &bc[j]);
      }
    }
    float acc = AGG == 2 ? -INFINITY : 0.0f;
    bool nonempty = false;
    // the walk over joined tuples is uniform across the workgroup (buffer
    // resources must be); lanes past the block simply see empty extents
    for (int32_t e0 = 0; e0 < cnt; e0 += EU) {
      __amdgpu_buffer_rsrc_t rs[EU][kMaxIn];
      int32_t lim[EU];
      int32_t maxlim = 0;
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        const bool have = e0 + u < cnt;
        const int32_t *ent = ents + (have ? e0 + u : 0) * width;
        const uint32_t kr = fd_mod(fd_div(uint32_t(ent[1]), a.div_wred), a.div_kred);
        const int32_t t0 = int32_t(kr) * a.e_red;
        int32_t l = a.n_red - t0;
        l = l < a.e_red ? l : a.e_red;
        if (a.causal) {
          const int32_t m = s - t0 + 1;  // t <= s
          l = m < l ? m : l;
        }
        lim[u] = (have && live) ? (l > 0 ? l : 0) : 0;
        maxlim = lim[u] > maxlim ? lim[u] : maxlim;
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j)
          rs[u][j] = block_rsrc(a.in[j].p, (j < a.n_in) ? ent[1 + j] : 0, (j < a.n_in) ? a.in[j].block_bytes : 0);
      }
      nonempty = nonempty || maxlim > 0;
      // VU steps of the row are loaded together (all EU tuples each), then
      // combined step by step, tuple by tuple: the same order as one step
      // at a time
      for (int32_t v0 = sub * V; v0 < maxlim; v0 += step * VU) {
        Raw<V> raw[VU][EU][kMaxIn];
#pragma unroll
        for (int vv = 0; vv < VU; ++vv) {
          const int32_t v = v0 + vv * step;
#pragma unroll
          for (int u = 0; u < EU; ++u) {
#pragma unroll
            for (int j = 0; j < kMaxIn; ++j) {
              if (j == 0 || (j < a.n_in && a.in[j].inner)) {
                const uint32_t e = q * uint32_t(a.in[j].row_mul) + uint32_t(v);
                raw_load<V>(raw[vv][u][j], rs[u][j], e, v < lim[u], j == 0 ? DT0 : a.in[j].dt, 1);
              }
            }
          }
        }
#pragma unroll
        for (int vv = 0; vv < VU; ++vv) {
          const int32_t v = v0 + vv * step;
#pragma unroll
          for (int u = 0; u < EU; ++u) {
            float x[kMaxIn][V];
#pragma unroll
            for (int j = 0; j < kMaxIn; ++j) {
              if (j == 0 || (j < a.n_in && a.in[j].inner)) {
                raw_to_f32<V>(raw[vv][u][j], j == 0 ? DT0 : a.in[j].dt, 1, x[j]);
              } else {
#pragma unroll
                for (int w = 0; w < V; ++w) x[j][w] = bc[j];
              }
            }
            const int32_t keep = lim[u] - v;
#pragma unroll
            for (int w = 0; w < V; ++w) {
              const float gv = g_fn<G>(x[0][w], x[1][w], x[2][w], a.beta, a.eps);
              if (w < keep) acc = AGG == 2 ? fmaxf(acc, gv) : acc + gv;
            }
          }
        }
      }
    }
    // butterfly inside the row group (fixed order)
    for (int m = lpr >> 1; m >= 1; m >>= 1) {
      const float o = __shfl_xor(acc, m, 64);
      acc = AGG == 2 ? fmaxf(acc, o) : acc + o;
    }
    if (sub == 0 && live) store_dt(a.out, int64_t(key) * a.be_out + q, a.out_dt, nonempty ? a.alpha * acc : 0.0f);
  }
}

// ------------------------------------------------------------------ launchers
namespace {

#ifndef JAGG_FLAT_MAP_U
#define JAGG_FLAT_MAP_U 2
#endif
#ifndef JAGG_FLAT_REDUCE_EU
#define JAGG_FLAT_REDUCE_EU 1
#endif
constexpr int kMapU = JAGG_FLAT_MAP_U;          // vectors per thread per pass (map)
constexpr int kReduceEU = JAGG_FLAT_REDUCE_EU;  // joined tuples loaded together (row reduce)

template <int G>
hipError_t map_go(const FlatArgs &a, hipStream_t st) {
  // every input varying along the row: four vectors per thread in one pass
  // (SiLU-up and residual adds 1-2% faster); with a row-constant input two
  // per pass, twice (an RMS scale 10% faster that way)
  bool all_inner = true;
  for (int j = 0; j < a.n_in; ++j) all_inner = all_inner && a.in[j].inner;
  const dim3 grid(unsigned(a.n_keys) * unsigned(a.chunks));
  if (all_inner) hipLaunchKernelGGL((flat_map_kernel<G, 2 * kMapU>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((flat_map_kernel<G, kMapU>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int V, int G, int VU>
hipError_t reduce_go(const FlatArgs &a, int lg, int agg, hipStream_t st) {
  const dim3 grid(unsigned(a.n_keys) * unsigned(a.chunks));
  if (a.in[0].dt) {
    if (agg == 2) hipLaunchKernelGGL((flat_reduce_kernel<V, G, 2, kReduceEU, 1, VU>), grid, dim3(256), 0, st, a, lg);
    else hipLaunchKernelGGL((flat_reduce_kernel<V, G, 1, kReduceEU, 1, VU>), grid, dim3(256), 0, st, a, lg);
  } else {
    if (agg == 2) hipLaunchKernelGGL((flat_reduce_kernel<V, G, 2, kReduceEU, 0, VU>), grid, dim3(256), 0, st, a, lg);
    else hipLaunchKernelGGL((flat_reduce_kernel<V, G, 1, kReduceEU, 0, VU>), grid, dim3(256), 0, st, a, lg);
  }
  return hipGetLastError();
}

template <int V, int G>
hipError_t reduce_vu(const FlatArgs &a, int lg, int agg, hipStream_t st) {
  // rows of four or more steps load four steps at once; shorter rows would
  // only issue out-of-range loads
  if (a.e_red >= 4 * (V << lg)) return reduce_go<V, G, 4>(a, lg, agg, st);
  return reduce_go<V, G, 1>(a, lg, agg, st);
}

template <int V>
hipError_t reduce_g(const FlatArgs &a, int lg, int g, int agg, hipStream_t st) {
  switch (g) {
    case 0: return reduce_vu<V, 0>(a, lg, agg, st);
    case 1: return reduce_vu<V, 1>(a, lg, agg, st);
    case 2: return reduce_vu<V, 2>(a, lg, agg, st);
    case 3: return reduce_vu<V, 3>(a, lg, agg, st);
    case 4: return reduce_vu<V, 4>(a, lg, agg, st);
    case 5: return reduce_vu<V, 5>(a, lg, agg, st);
    case 6: return reduce_vu<V, 6>(a, lg, agg, st);
    case 7: return reduce_vu<V, 7>(a, lg, agg, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_flat_map(const FlatArgs &a, int g, hipStream_t st) {
  switch (g) {
    case 0: return map_go<0>(a, st);
    case 1: return map_go<1>(a, st);
    case 2: return map_go<2>(a, st);
    case 3: return map_go<3>(a, st);
    case 4: return map_go<4>(a, st);
    case 5: return map_go<5>(a, st);
    case 6: return map_go<6>(a, st);
    case 7: return map_go<7>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_flat_reduce(const FlatArgs &a, int vec, int lpr, int g, int agg, hipStream_t st) {
  int lg = 0;
  while ((1 << lg) < lpr) ++lg;
  if ((1 << lg) != lpr || lpr > 64) return hipErrorInvalidValue;
  if (vec == 4) return reduce_g<4>(a, lg, g, agg, st);
  if (vec == 1) return reduce_g<1>(a, lg, g, agg, st);
  return hipErrorInvalidValue;
}

}  // namespace jagg
