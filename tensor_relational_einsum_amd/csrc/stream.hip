// stream.hip -- vectorised map and row-reduce block kernels.
//
// "Every Kernel Is a Join" (Ding et al.), Def. 3.7: f runs on every joined
// tuple and results of equal output key are combined with the aggregation.
// These two kernels cover the common HBM-bound forms:
//   - map (no reduced letter): one joined tuple per output key; g is applied
//     element by element, 8 elements per thread, with 16-byte loads for
//     inputs contiguous along the innermost output letter and one broadcast
//     load for inputs that lack it;
//   - row reduce: a single reduced letter, innermost in input 0 (softmax
//     statistics, RMS sums, matrix-vector products).  The joined tuples of
//     the workgroup's output key are decoded once into LDS; a group of lanes
//     owns one output element, walks the tuples in join-list order with
//     16-byte loads, and finishes with a butterfly inside the group, so the
//     result is deterministic.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

// V consecutive elements starting at element `off` (aligned to V): a vector
// load when contiguous, one broadcast load when the stride is 0.
template <int V>
__device__ __forceinline__ void load_run(const void *base, int64_t off, int dt, int64_t stride, float *x) {
  if (stride == 1) {
    if (dt) {
      const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + off;
      if constexpr (V == 8) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[2 * u] = __uint_as_float(w[u] << 16);
          x[2 * u + 1] = __uint_as_float(w[u] & 0xffff0000u);
        }
      } else if constexpr (V == 4) {
        const uint2 q = *reinterpret_cast<const uint2 *>(p);
        x[0] = __uint_as_float(q.x << 16);
        x[1] = __uint_as_float(q.x & 0xffff0000u);
        x[2] = __uint_as_float(q.y << 16);
        x[3] = __uint_as_float(q.y & 0xffff0000u);
      } else {
#pragma unroll
        for (int u = 0; u < V; ++u) x[u] = bf16_to_f32(p[u]);
      }
    } else {
      const float *p = reinterpret_cast<const float *>(base) + off;
      if constexpr (V % 4 == 0) {
#pragma unroll
        for (int u = 0; u < V; u += 4) {
          const float4 q = *reinterpret_cast<const float4 *>(p + u);
          x[u] = q.x;
          x[u + 1] = q.y;
          x[u + 2] = q.z;
          x[u + 3] = q.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < V; ++u) x[u] = p[u];
      }
    }
  } else if (stride == 0) {
    const float v = load_dt(base, off, dt);
#pragma unroll
    for (int u = 0; u < V; ++u) x[u] = v;
  } else {
#pragma unroll
    for (int u = 0; u < V; ++u) x[u] = load_dt(base, off + u * stride, dt);
  }
}

template <int V>
__device__ __forceinline__ void store_run(void *base, int64_t off, int dt, const float *x) {
  if (dt) {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + off;
    if constexpr (V == 8) {
      uint4 q;
      q.x = pack_bf16x2(x[0], x[1]);
      q.y = pack_bf16x2(x[2], x[3]);
      q.z = pack_bf16x2(x[4], x[5]);
      q.w = pack_bf16x2(x[6], x[7]);
      *reinterpret_cast<uint4 *>(p) = q;
    } else if constexpr (V == 4) {
      uint2 q;
      q.x = pack_bf16x2(x[0], x[1]);
      q.y = pack_bf16x2(x[2], x[3]);
      *reinterpret_cast<uint2 *>(p) = q;
    } else {
#pragma unroll
      for (int u = 0; u < V; ++u) p[u] = f32_to_bf16(x[u]);
    }
  } else {
    float *p = reinterpret_cast<float *>(base) + off;
    if constexpr (V % 4 == 0) {
#pragma unroll
      for (int u = 0; u < V; u += 4) *reinterpret_cast<float4 *>(p + u) = make_float4(x[u], x[u + 1], x[u + 2], x[u + 3]);
    } else {
#pragma unroll
      for (int u = 0; u < V; ++u) p[u] = x[u];
    }
  }
}

// output tuple id -> block coordinates
__device__ __forceinline__ void key_coords(const EwArgs &a, int64_t key, int64_t *kap) {
  int64_t rem = key;
#pragma unroll
  for (int i = kMaxLetters - 1; i >= 0; --i) {
    if (i < a.r_out) {
      kap[i] = rem % a.k_out[i];
      rem /= a.k_out[i];
    } else {
      kap[i] = 0;
    }
  }
}

// ------------------------------------------------------------------ map
template <int V, int G>
__global__ __launch_bounds__(256) void map_vec_kernel(const EwArgs a, StreamArgs sa) {
  const int64_t key = blockIdx.x / sa.chunks;
  const int64_t chunk = blockIdx.x - key * sa.chunks;
  if (a.counts[key] == 0) return;  // tuple absent from the output relation
  const int32_t *ent = a.list + key * int64_t(a.per_key) * (1 + a.n_in);
  int64_t tbase[kMaxIn];
#pragma unroll
  for (int j = 0; j < kMaxIn; ++j) tbase[j] = j < a.n_in ? int64_t(ent[1 + j]) * a.be_in[j] : 0;
  int64_t kap[kMaxLetters];
  key_coords(a, key, kap);
  const int r = a.r_out;
  int64_t kap_last = 0, e_last = 1, n_last = 1;
  int64_t s_last[kMaxIn] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < kMaxLetters; ++i)
    if (i == r - 1) {
      kap_last = kap[i];
      e_last = a.e_out[i];
      n_last = a.n_out[i];
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j) s_last[j] = a.s_out[j][i];
    }
  const int64_t obase = key * a.be_out;
  const uint32_t vpr = uint32_t(e_last / V);
  for (int64_t slot = chunk * 256 + threadIdx.x; slot < sa.slots; slot += sa.chunks * 256) {
    const uint32_t s32 = uint32_t(slot);
    uint32_t row = fd_div(s32, sa.div_vpr);
    const int64_t inner = int64_t(s32 - row * vpr) * V;
    bool ok = true;
    int64_t ooff = obase + int64_t(row) * e_last + inner;
    int64_t ioff[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) ioff[j] = tbase[j] + inner * s_last[j];
    int64_t s_glob = 0;
#pragma unroll
    for (int i = kMaxLetters - 1; i >= 0; --i) {
      if (i < r - 1) {
        const uint32_t q = fd_div(row, sa.div_out[i]);
        const int64_t c = int64_t(row - q * sa.div_out[i].d);
        row = q;
        ok = ok && (kap[i] * a.e_out[i] + c < a.n_out[i]);
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) ioff[j] += c * a.s_out[j][i];
        if (a.causal && a.s_pos == i) s_glob = kap[i] * a.e_out[i] + c;
      }
    }
    float x[kMaxIn][V];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) {
      if (j < a.n_in) load_run<V>(a.in[j], ioff[j], a.in_dt[j], s_last[j], x[j]);
      else {
#pragma unroll
        for (int u = 0; u < V; ++u) x[j][u] = g_fill<G>();
      }
    }
    // elements [0, keep) of the vector are inside the output (and on the
    // allowed side of a causal pair); the rest are padding and get +0
    const int64_t xl = kap_last * e_last + inner;
    int64_t lim = n_last - xl;
    if (a.causal && s_glob + 1 - xl < lim) lim = s_glob + 1 - xl;
    const int keep = ok ? int(lim < 0 ? 0 : (lim > V ? V : lim)) : 0;
    float y[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const float v = a.alpha * g_fn<G>(x[0][u], x[1][u], x[2][u], a.beta, a.eps);
      y[u] = u < keep ? v : 0.0f;
    }
    store_run<V>(a.out, ooff, a.out_dt, y);
  }
}

// ------------------------------------------------------------------ row reduce
constexpr int kMaxRowEntries = 256;

template <int V, int G, int AGG>
__global__ __launch_bounds__(256) void reduce_row_kernel(const EwArgs a, StreamArgs sa, int lpr_log2) {
  __shared__ int64_t s_base[kMaxIn][kMaxRowEntries];
  __shared__ int32_t s_lim[kMaxRowEntries];
  __shared__ int64_t s_t0[kMaxRowEntries];
  const int64_t key = blockIdx.x / sa.chunks;
  const int64_t chunk = blockIdx.x - key * sa.chunks;
  const int32_t cnt = a.counts[key];
  const int32_t *ents = a.list + key * int64_t(a.per_key) * (1 + a.n_in);
  // the key's joined tuples: block bases and the valid extent of the reduced letter
  for (int e = threadIdx.x; e < cnt; e += 256) {
    const int32_t *ent = ents + int64_t(e) * (1 + a.n_in);
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) s_base[j][e] = j < a.n_in ? int64_t(ent[1 + j]) * a.be_in[j] : 0;
    const int64_t kr = (int64_t(ent[1]) / a.w_red0[0]) % a.k_red[0];
    const int64_t lim = a.n_red_ext[0] - kr * a.e_red[0];
    s_lim[e] = int32_t(lim < a.e_red[0] ? lim : a.e_red[0]);
    s_t0[e] = kr * a.e_red[0];
  }
  __syncthreads();
  int64_t kap[kMaxLetters];
  key_coords(a, key, kap);
  const int r = a.r_out;
  const int lpr = 1 << lpr_log2;
  const int sub = threadIdx.x & (lpr - 1);      // lane inside the row group
  const int group = threadIdx.x >> lpr_log2;    // row group inside the workgroup
  const int groups = 256 >> lpr_log2;
  const int step = lpr * V;
  bool has_red[kMaxIn];
#pragma unroll
  for (int j = 0; j < kMaxIn; ++j) has_red[j] = j == 0 || (j < a.n_in && a.s_red[j][0] != 0);
  for (int64_t q0 = chunk * groups; q0 < a.be_out; q0 += sa.chunks * groups) {
    const int64_t q = q0 + group;
    const bool live = q < a.be_out;
    // output element -> coordinates, input offsets, validity
    bool ok = live;
    int64_t off[kMaxIn] = {0, 0, 0};
    int64_t s_glob = 0;
    uint32_t rem = uint32_t(live ? q : 0);
#pragma unroll
    for (int i = kMaxLetters - 1; i >= 0; --i) {
      if (i < r) {
        const uint32_t qq = fd_div(rem, sa.div_out[i]);
        const int64_t c = int64_t(rem - qq * sa.div_out[i].d);
        rem = qq;
        ok = ok && (kap[i] * a.e_out[i] + c < a.n_out[i]);
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) off[j] += c * a.s_out[j][i];
        if (a.causal && a.s_pos == i) s_glob = kap[i] * a.e_out[i] + c;
      }
    }
    // inputs without the reduced letter: one value per output element
    float bc[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) {
      bc[j] = g_fill<G>();
      if (j < a.n_in && !has_red[j] && ok && cnt > 0) bc[j] = load_dt(a.in[j], s_base[j][0] + off[j], a.in_dt[j]);
    }
    float acc = AGG == 2 ? -INFINITY : 0.0f;
    bool nonempty = false;
    const int32_t n_e = ok ? cnt : 0;
    for (int32_t e = 0; e < n_e; ++e) {
      int32_t lim = s_lim[e];
      if (a.causal) {
        const int64_t m = s_glob - s_t0[e] + 1;  // t <= s
        if (m < lim) lim = int32_t(m < 0 ? 0 : m);
      }
      nonempty = nonempty || lim > 0;
      int64_t base[kMaxIn];
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j) base[j] = s_base[j][e] + off[j];
      for (int v = sub * V; v < lim; v += step) {
        float x[kMaxIn][V];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) {
          if (j < a.n_in && has_red[j]) {
            load_run<V>(a.in[j], base[j] + v, a.in_dt[j], 1, x[j]);
          } else {
#pragma unroll
            for (int u = 0; u < V; ++u) x[j][u] = bc[j];
          }
        }
        const int keep = lim - v;  // >= 1
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const float gv = g_fn<G>(x[0][u], x[1][u], x[2][u], a.beta, a.eps);
          if (u == 0 || u < keep) acc = AGG == 2 ? fmaxf(acc, gv) : acc + gv;
        }
      }
    }
    // butterfly inside the row group (fixed order)
    for (int m = lpr >> 1; m >= 1; m >>= 1) {
      const float o = __shfl_xor(acc, m, 64);
      acc = AGG == 2 ? fmaxf(acc, o) : acc + o;
    }
    if (sub == 0 && live) store_dt(a.out, key * a.be_out + q, a.out_dt, (ok && nonempty) ? a.alpha * acc : 0.0f);
  }
}

template <int V, int G>
static void map_go(const EwArgs &a, const StreamArgs &sa, hipStream_t st) {
  hipLaunchKernelGGL((map_vec_kernel<V, G>), dim3(unsigned(a.n_keys * sa.chunks)), dim3(256), 0, st, a, sa);
}

template <int V>
static hipError_t map_vec_g(const EwArgs &a, const StreamArgs &sa, hipStream_t st) {
  switch (a.g) {
    case 0: map_go<V, 0>(a, sa, st); break;
    case 1: map_go<V, 1>(a, sa, st); break;
    case 2: map_go<V, 2>(a, sa, st); break;
    case 3: map_go<V, 3>(a, sa, st); break;
    case 4: map_go<V, 4>(a, sa, st); break;
    case 5: map_go<V, 5>(a, sa, st); break;
    case 6: map_go<V, 6>(a, sa, st); break;
    case 7: map_go<V, 7>(a, sa, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_map_vec(const EwArgs &a, StreamArgs sa, int vec, hipStream_t st) {
  if (vec == 8) return map_vec_g<8>(a, sa, st);
  if (vec == 4) return map_vec_g<4>(a, sa, st);
  return map_vec_g<1>(a, sa, st);
}

template <int V, int G>
static hipError_t reduce_go(const EwArgs &a, const StreamArgs &sa, int lpr_log2, hipStream_t st) {
  const dim3 grid(unsigned(a.n_keys * sa.chunks));
  if (a.agg == 2) hipLaunchKernelGGL((reduce_row_kernel<V, G, 2>), grid, dim3(256), 0, st, a, sa, lpr_log2);
  else hipLaunchKernelGGL((reduce_row_kernel<V, G, 1>), grid, dim3(256), 0, st, a, sa, lpr_log2);
  return hipGetLastError();
}

template <int V>
static hipError_t reduce_row_g(const EwArgs &a, const StreamArgs &sa, int lpr_log2, hipStream_t st) {
  switch (a.g) {
    case 0: return reduce_go<V, 0>(a, sa, lpr_log2, st);
    case 1: return reduce_go<V, 1>(a, sa, lpr_log2, st);
    case 2: return reduce_go<V, 2>(a, sa, lpr_log2, st);
    case 3: return reduce_go<V, 3>(a, sa, lpr_log2, st);
    case 4: return reduce_go<V, 4>(a, sa, lpr_log2, st);
    case 5: return reduce_go<V, 5>(a, sa, lpr_log2, st);
    case 6: return reduce_go<V, 6>(a, sa, lpr_log2, st);
    case 7: return reduce_go<V, 7>(a, sa, lpr_log2, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce_row(const EwArgs &a, StreamArgs sa, int vec, int lpr, hipStream_t st) {
  int lg = 0;
  while ((1 << lg) < lpr) ++lg;
  if ((1 << lg) != lpr || lpr > 64) return hipErrorInvalidValue;
  return vec == 4 ? reduce_row_g<4>(a, sa, lg, st) : reduce_row_g<1>(a, sa, lg, st);
}

}  // namespace jagg
