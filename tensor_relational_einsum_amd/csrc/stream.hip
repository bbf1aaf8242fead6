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

__device__ __forceinline__ float g_apply(int g, int n_in, float x0, float x1, float x2, float beta, float eps) {
  switch (g) {
    case 0: return n_in == 1 ? x0 : (n_in == 2 ? x0 * x1 : x0 * x1 * x2);
    case 1: return x0;
    case 2: return x0 * x0;
    case 3: return __expf(x0 - x1);
    case 4: return __expf(x0 - x1) / x2;
    case 5: return x0 * rsqrtf(x1 * beta + eps) * x2;
    case 6: return x0 / (1.0f + __expf(-x0)) * x1;
    case 7: return n_in == 1 ? x0 : (n_in == 2 ? x0 + x1 : x0 + x1 + x2);
  }
  return 0.0f;
}

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
      q.x = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
      q.y = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
      q.z = uint32_t(f32_to_bf16(x[4])) | (uint32_t(f32_to_bf16(x[5])) << 16);
      q.w = uint32_t(f32_to_bf16(x[6])) | (uint32_t(f32_to_bf16(x[7])) << 16);
      *reinterpret_cast<uint4 *>(p) = q;
    } else if constexpr (V == 4) {
      uint2 q;
      q.x = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
      q.y = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
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
template <int V>
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
        for (int u = 0; u < V; ++u) x[j][u] = 0.0f;
      }
    }
    const int64_t xl = kap_last * e_last + inner;
    float y[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const float v = a.alpha * g_apply(a.g, a.n_in, x[0][u], x[1][u], x[2][u], a.beta, a.eps);
      const bool keep = ok && (xl + u < n_last) && !(a.causal && xl + u > s_glob);
      y[u] = keep ? v : 0.0f;
    }
    store_run<V>(a.out, ooff, a.out_dt, y);
  }
}

// ------------------------------------------------------------------ row reduce
constexpr int kMaxRowEntries = 256;

template <int V, int LPR>
__global__ __launch_bounds__(256) void reduce_row_kernel(const EwArgs a, StreamArgs sa) {
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
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;                   // lane inside the row group
  const int group = threadIdx.x / LPR;          // row group inside the workgroup
  constexpr int GROUPS = 256 / LPR;
  const bool is_max = a.agg == 2;
  for (int64_t q0 = chunk * GROUPS; q0 < a.be_out; q0 += sa.chunks * GROUPS) {
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
    float bc[kMaxIn] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 1; j < kMaxIn; ++j)
      if (j < a.n_in && a.s_red[j][0] == 0 && ok && cnt > 0) bc[j] = load_dt(a.in[j], s_base[j][0] + off[j], a.in_dt[j]);
    float acc = is_max ? -INFINITY : 0.0f;
    int terms = 0;
    if (ok) {
      for (int32_t e = 0; e < cnt; ++e) {
        int32_t lim = s_lim[e];
        if (a.causal) {
          const int64_t m = s_glob - s_t0[e] + 1;  // t <= s
          if (m < lim) lim = int32_t(m < 0 ? 0 : m);
        }
        for (int v = sub * V; v < lim; v += LPR * V) {
          float x[kMaxIn][V];
          load_run<V>(a.in[0], s_base[0][e] + off[0] + v, a.in_dt[0], 1, x[0]);
#pragma unroll
          for (int j = 1; j < kMaxIn; ++j) {
            if (j < a.n_in && a.s_red[j][0] != 0) {
              load_run<V>(a.in[j], s_base[j][e] + off[j] + v, a.in_dt[j], 1, x[j]);
            } else {
#pragma unroll
              for (int u = 0; u < V; ++u) x[j][u] = bc[j];
            }
          }
#pragma unroll
          for (int u = 0; u < V; ++u) {
            if (v + u < lim) {
              const float gv = g_apply(a.g, a.n_in, x[0][u], x[1][u], x[2][u], a.beta, a.eps);
              acc = is_max ? fmaxf(acc, gv) : acc + gv;
              ++terms;
            }
          }
        }
      }
    }
    // butterfly inside the row group (fixed order)
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) {
      const float o = __shfl_xor(acc, m, 64);
      acc = is_max ? fmaxf(acc, o) : acc + o;
      terms += __shfl_xor(terms, m, 64);
    }
    if (sub == 0 && live) store_dt(a.out, key * a.be_out + q, a.out_dt, (ok && terms > 0) ? a.alpha * acc : 0.0f);
  }
}

hipError_t launch_map_vec(const EwArgs &a, StreamArgs sa, int vec, hipStream_t st) {
  const int64_t grid = a.n_keys * sa.chunks;
  if (vec == 8) hipLaunchKernelGGL(map_vec_kernel<8>, dim3(unsigned(grid)), dim3(256), 0, st, a, sa);
  else if (vec == 4) hipLaunchKernelGGL(map_vec_kernel<4>, dim3(unsigned(grid)), dim3(256), 0, st, a, sa);
  else hipLaunchKernelGGL(map_vec_kernel<1>, dim3(unsigned(grid)), dim3(256), 0, st, a, sa);
  return hipGetLastError();
}

hipError_t launch_reduce_row(const EwArgs &a, StreamArgs sa, int vec, int lpr, hipStream_t st) {
  const int64_t grid = a.n_keys * sa.chunks;
#define JAGG_RR(VV, LL)                                                                                  \
  if (vec == VV && lpr == LL) {                                                                          \
    hipLaunchKernelGGL((reduce_row_kernel<VV, LL>), dim3(unsigned(grid)), dim3(256), 0, st, a, sa);      \
    return hipGetLastError();                                                                            \
  }
  JAGG_RR(4, 64) JAGG_RR(4, 32) JAGG_RR(4, 16) JAGG_RR(4, 8) JAGG_RR(4, 4)
  JAGG_RR(1, 64) JAGG_RR(1, 32) JAGG_RR(1, 16) JAGG_RR(1, 8) JAGG_RR(1, 4)
#undef JAGG_RR
  return hipErrorInvalidValue;
}

}  // namespace jagg
