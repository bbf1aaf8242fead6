// elementwise.hip -- map (no aggregation) and reduce (SUM / MAX) block kernels.
//
// "Every Kernel Is a Join" (Ding et al.), Def. 3.7: the concrete operator f
// runs on every joined tuple and the outputs of equal output type are
// combined with an associative, commutative aggregation.  Here f is g
// applied element by element followed, for a reduce, by the aggregation
// over the block's reduced letters; the aggregation across the joined
// tuples of one output key happens in the same pass, in join-list order,
// so results are deterministic.  Both kernels stream HBM: a map reads each
// input element once and writes each output element once; a reduce reads
// its inputs once and writes one value per output element.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

__device__ __forceinline__ float apply_g(int g, int n_in, float x0, float x1, float x2, float beta, float eps) {
  switch (g) {
    case 0: return n_in == 1 ? x0 : (n_in == 2 ? x0 * x1 : x0 * x1 * x2);
    case 1: return x0;
    case 2: return x0 * x0;
    case 3: return expf(x0 - x1);
    case 4: return expf(x0 - x1) / x2;
    case 5: return x0 / sqrtf(x1 * beta + eps) * x2;
    case 6: return x0 / (1.0f + expf(-x0)) * x1;
    case 7: return n_in == 1 ? x0 : (n_in == 2 ? x0 + x1 : x0 + x1 + x2);
  }
  return 0.0f;
}

// Output tuple id -> block coordinates of the output letters (unrolled so
// the small arrays stay in registers).
__device__ __forceinline__ void decode_key(const EwArgs &a, int64_t key, int64_t *kap) {
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
// Grid: one workgroup per (output key, chunk of row-vectors).  A slot is one
// vector of VEC elements along the innermost output letter.
template <int VEC>
__global__ __launch_bounds__(256) void map_kernel(const EwArgs a, int64_t chunks, int64_t slots_per_key,
                                                   FastDiv vpr_div, FastDiv row_div0, FastDiv row_div1,
                                                   FastDiv row_div2) {
  const int64_t key = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - key * chunks;
  if (a.counts[key] == 0) return;  // tuple absent from the output relation
  const int32_t *ent = a.list + key * int64_t(a.per_key) * (1 + a.n_in);
  int64_t tbase[kMaxIn];
#pragma unroll
  for (int j = 0; j < kMaxIn; ++j) tbase[j] = j < a.n_in ? int64_t(ent[1 + j]) * a.be_in[j] : 0;
  int64_t kap[kMaxLetters];
  decode_key(a, key, kap);
  const int r = a.r_out;
  const int64_t obase = key * a.be_out;
  const int64_t e_last = a.e_out[r - 1];
  int64_t kap_last = 0;
#pragma unroll
  for (int i = 0; i < kMaxLetters; ++i)
    if (i == r - 1) kap_last = kap[i];

  for (int64_t slot = chunk * 256 + threadIdx.x; slot < slots_per_key; slot += chunks * 256) {
    const uint32_t s32 = uint32_t(slot);
    const uint32_t row = fd_div(s32, vpr_div);
    const int64_t inner = int64_t(s32 - row * vpr_div.d) * VEC;
    // row -> coordinates of output letters 0 .. r-2 (row-major)
    int64_t c[kMaxLetters];
    {
      uint32_t rem = row;
#pragma unroll
      for (int i = kMaxLetters - 1; i >= 0; --i) {
        if (i < r - 1) {
          uint32_t q;
          if (i == r - 2) q = fd_div(rem, row_div0);
          else if (i == r - 3) q = fd_div(rem, row_div1);
          else if (i == r - 4) q = fd_div(rem, row_div2);
          else q = rem / uint32_t(a.e_out[i]);
          c[i] = int64_t(rem - q * uint32_t(a.e_out[i]));
          rem = q;
        } else {
          c[i] = 0;
        }
      }
    }
    bool row_ok = true;
    int64_t ooff = obase + inner;
    int64_t ioff[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) ioff[j] = tbase[j];
    int64_t rowstride = e_last;
    int64_t s_glob = 0, t_glob_base = 0;
#pragma unroll
    for (int i = kMaxLetters - 1; i >= 0; --i) {
      if (i < r - 1) {
        row_ok = row_ok && (kap[i] * a.e_out[i] + c[i] < a.n_out[i]);
        ooff += c[i] * rowstride;
        rowstride *= a.e_out[i];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) ioff[j] += c[i] * a.s_out[j][i];
        if (a.causal && a.s_pos == i) s_glob = kap[i] * a.e_out[i] + c[i];
      }
    }
    int64_t s_in[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) {
      // innermost output letter's stride in input j
      int64_t sl = 0;
#pragma unroll
      for (int i = 0; i < kMaxLetters; ++i)
        if (i == r - 1) sl = a.s_out[j][i];
      s_in[j] = sl;
      ioff[j] += inner * sl;
    }
    const int64_t x_last = kap_last * e_last + inner;
    if (a.causal) {
      // the causal t letter is the innermost output letter
      t_glob_base = x_last;
    }
    float res[VEC];
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      float x[kMaxIn] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxIn; ++j)
        if (j < a.n_in) x[j] = load_dt(a.in[j], ioff[j] + u * s_in[j], a.in_dt[j]);
      float v = a.alpha * apply_g(a.g, a.n_in, x[0], x[1], x[2], a.beta, a.eps);
      const bool ok = row_ok && (x_last + u < a.n_out[r - 1]) && !(a.causal && t_glob_base + u > s_glob);
      res[u] = ok ? v : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < VEC; ++u) store_dt(a.out, ooff + u, a.out_dt, res[u]);
  }
}

hipError_t launch_map(const EwArgs &a, hipStream_t st) {
  const int r = a.r_out;
  const int64_t e_last = a.e_out[r - 1];
  const int vec = a.vec;
  const int64_t vpr = e_last / vec;
  const int64_t slots = a.rows_per_block * vpr;
  int64_t chunks = (slots + 256 * 4 - 1) / (256 * 4);
  if (chunks < 1) chunks = 1;
  const FastDiv vd = make_fastdiv(uint32_t(vpr));
  const FastDiv d0 = make_fastdiv(uint32_t(r >= 2 ? a.e_out[r - 2] : 1));
  const FastDiv d1 = make_fastdiv(uint32_t(r >= 3 ? a.e_out[r - 3] : 1));
  const FastDiv d2 = make_fastdiv(uint32_t(r >= 4 ? a.e_out[r - 4] : 1));
  const int64_t grid = a.n_keys * chunks;
  if (vec == 4)
    hipLaunchKernelGGL(map_kernel<4>, dim3(unsigned(grid)), dim3(256), 0, st, a, chunks, slots, vd, d0, d1, d2);
  else
    hipLaunchKernelGGL(map_kernel<1>, dim3(unsigned(grid)), dim3(256), 0, st, a, chunks, slots, vd, d0, d1, d2);
  return hipGetLastError();
}

// ------------------------------------------------------------------ reduce
__device__ __forceinline__ float agg_identity(int agg) { return agg == 2 ? -INFINITY : 0.0f; }
__device__ __forceinline__ float agg_combine(int agg, float acc, float v) { return agg == 2 ? fmaxf(acc, v) : acc + v; }

// Reduce where the innermost letter of input 0 is reduced: one wavefront per
// output element; lanes stride along that letter, the other reduced letters
// and the joined tuples are walked in order, and a butterfly over the 64
// lanes finishes the aggregation.
__global__ __launch_bounds__(256) void reduce_rows_kernel(const EwArgs a, int64_t waves_per_key) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t key = gw / waves_per_key;
  if (key >= a.n_keys) return;
  const int64_t first_q = gw - key * waves_per_key;
  const int32_t cnt = a.counts[key];
  const int32_t *ents = a.list + key * int64_t(a.per_key) * (1 + a.n_in);
  int64_t kap[kMaxLetters];
  decode_key(a, key, kap);
  const int r = a.r_out;
  const int ir = a.inner_red;
  for (int64_t q = first_q; q < a.be_out; q += waves_per_key) {
    // output element q of the block -> coordinates
    int64_t c[kMaxLetters];
    bool ok = true;
    int64_t rem = q;
    int64_t s_glob = 0, t_out = 0;
#pragma unroll
    for (int i = kMaxLetters - 1; i >= 0; --i) {
      if (i < r) {
        c[i] = rem % a.e_out[i];
        rem /= a.e_out[i];
        ok = ok && (kap[i] * a.e_out[i] + c[i] < a.n_out[i]);
        if (a.causal && !a.s_red_flag && a.s_pos == i) s_glob = kap[i] * a.e_out[i] + c[i];
        if (a.causal && !a.t_red_flag && a.t_pos == i) t_out = kap[i] * a.e_out[i] + c[i];
      } else {
        c[i] = 0;
      }
    }
    (void)t_out;
    float acc = agg_identity(a.agg);
    bool any = false;
    if (ok && cnt > 0) {
      for (int32_t e = 0; e < cnt; ++e) {
        const int32_t *ent = ents + int64_t(e) * (1 + a.n_in);
        int64_t off[kMaxIn];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) {
          off[j] = 0;
          if (j < a.n_in) {
            off[j] = int64_t(ent[1 + j]) * a.be_in[j];
#pragma unroll
            for (int i = 0; i < kMaxLetters; ++i)
              if (i < r) off[j] += c[i] * a.s_out[j][i];
          }
        }
        // block coordinates and valid extents of the reduced letters
        const int64_t t0 = ent[1];
        int64_t lim[kMaxLetters], kr[kMaxLetters];
        int64_t outer_total = 1;
#pragma unroll
        for (int i = 0; i < kMaxLetters; ++i) {
          if (i < a.n_red) {
            kr[i] = (t0 / a.w_red0[i]) % a.k_red[i];
            int64_t l = a.n_red_ext[i] - kr[i] * a.e_red[i];
            lim[i] = l < a.e_red[i] ? l : a.e_red[i];
            if (i != ir) outer_total *= lim[i];
          } else {
            kr[i] = 0;
            lim[i] = 1;
          }
        }
        for (int64_t o = 0; o < outer_total; ++o) {
          // decode the non-inner reduced coordinates (row-major over reduced letters)
          int64_t orem = o;
          int64_t roff[kMaxIn] = {off[0], off[1], off[2]};
          int64_t s_red_glob = s_glob;
#pragma unroll
          for (int i = kMaxLetters - 1; i >= 0; --i) {
            if (i < a.n_red && i != ir) {
              const int64_t ci = orem % lim[i];
              orem /= lim[i];
#pragma unroll
              for (int j = 0; j < kMaxIn; ++j) roff[j] += ci * a.s_red[j][i];
              if (a.causal && a.s_red_flag && a.s_pos == i) s_red_glob = kr[i] * a.e_red[i] + ci;
            }
          }
          int64_t sinner[kMaxIn];
#pragma unroll
          for (int j = 0; j < kMaxIn; ++j) {
            int64_t sv = 0;
#pragma unroll
            for (int i = 0; i < kMaxLetters; ++i)
              if (i == ir) sv = a.s_red[j][i];
            sinner[j] = sv;
          }
          int64_t lim_in = 1, k_in = 0, e_in = 1;
#pragma unroll
          for (int i = 0; i < kMaxLetters; ++i)
            if (i == ir) { lim_in = lim[i]; k_in = kr[i]; e_in = a.e_red[i]; }
          for (int64_t ci = lane; ci < lim_in; ci += 64) {
            if (a.causal && a.t_red_flag && a.t_pos == ir && k_in * e_in + ci > s_red_glob) continue;
            float x[kMaxIn] = {0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMaxIn; ++j)
              if (j < a.n_in) x[j] = load_dt(a.in[j], roff[j] + ci * sinner[j], a.in_dt[j]);
            const float v = apply_g(a.g, a.n_in, x[0], x[1], x[2], a.beta, a.eps);
            acc = agg_combine(a.agg, acc, v);
            any = true;
          }
        }
      }
    }
    // butterfly across the wavefront (fixed order: deterministic)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float o = __shfl_xor(acc, m, 64);
      acc = agg_combine(a.agg, acc, o);
    }
    const bool any_w = __ballot(any) != 0;
    if (lane == 0) store_dt(a.out, key * a.be_out + q, a.out_dt, (ok && any_w) ? a.alpha * acc : 0.0f);
  }
}

// Reduce where input 0's innermost letter is an output letter: one thread
// per output element, walking the joined tuples and every reduced
// coordinate in order (consecutive threads read consecutive elements).
__global__ __launch_bounds__(256) void reduce_cols_kernel(const EwArgs a, int64_t chunks) {
  const int64_t key = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - key * chunks;
  const int32_t cnt = a.counts[key];
  const int32_t *ents = a.list + key * int64_t(a.per_key) * (1 + a.n_in);
  int64_t kap[kMaxLetters];
  decode_key(a, key, kap);
  const int r = a.r_out;
  for (int64_t q = chunk * 256 + threadIdx.x; q < a.be_out; q += chunks * 256) {
    int64_t c[kMaxLetters];
    bool ok = true;
    int64_t rem = q;
    int64_t s_glob = 0;
#pragma unroll
    for (int i = kMaxLetters - 1; i >= 0; --i) {
      if (i < r) {
        c[i] = rem % a.e_out[i];
        rem /= a.e_out[i];
        ok = ok && (kap[i] * a.e_out[i] + c[i] < a.n_out[i]);
        if (a.causal && !a.s_red_flag && a.s_pos == i) s_glob = kap[i] * a.e_out[i] + c[i];
      } else {
        c[i] = 0;
      }
    }
    float acc = agg_identity(a.agg);
    bool any = false;
    if (ok) {
      for (int32_t e = 0; e < cnt; ++e) {
        const int32_t *ent = ents + int64_t(e) * (1 + a.n_in);
        int64_t off[kMaxIn];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) {
          off[j] = 0;
          if (j < a.n_in) {
            off[j] = int64_t(ent[1 + j]) * a.be_in[j];
#pragma unroll
            for (int i = 0; i < kMaxLetters; ++i)
              if (i < r) off[j] += c[i] * a.s_out[j][i];
          }
        }
        const int64_t t0 = ent[1];
        int64_t lim[kMaxLetters], kr[kMaxLetters];
        int64_t total = 1;
#pragma unroll
        for (int i = 0; i < kMaxLetters; ++i) {
          if (i < a.n_red) {
            kr[i] = (t0 / a.w_red0[i]) % a.k_red[i];
            int64_t l = a.n_red_ext[i] - kr[i] * a.e_red[i];
            lim[i] = l < a.e_red[i] ? l : a.e_red[i];
            total *= lim[i];
          } else {
            kr[i] = 0;
            lim[i] = 1;
          }
        }
        for (int64_t o = 0; o < total; ++o) {
          int64_t orem = o;
          int64_t roff[kMaxIn] = {off[0], off[1], off[2]};
          bool masked = false;
#pragma unroll
          for (int i = kMaxLetters - 1; i >= 0; --i) {
            if (i < a.n_red) {
              const int64_t ci = orem % lim[i];
              orem /= lim[i];
#pragma unroll
              for (int j = 0; j < kMaxIn; ++j) roff[j] += ci * a.s_red[j][i];
              if (a.causal && a.t_red_flag && a.t_pos == i && kr[i] * a.e_red[i] + ci > s_glob) masked = true;
            }
          }
          if (masked) continue;
          float x[kMaxIn] = {0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < kMaxIn; ++j)
            if (j < a.n_in) x[j] = load_dt(a.in[j], roff[j], a.in_dt[j]);
          acc = agg_combine(a.agg, acc, apply_g(a.g, a.n_in, x[0], x[1], x[2], a.beta, a.eps));
          any = true;
        }
      }
    }
    store_dt(a.out, key * a.be_out + q, a.out_dt, (ok && any) ? a.alpha * acc : 0.0f);
  }
}

hipError_t launch_reduce(const EwArgs &a, hipStream_t st) {
  if (a.inner_red >= 0) {
    // enough wavefronts per key to fill the chip, at most one per output element
    int64_t wpk = a.be_out;
    const int64_t target = 8192;
    if (a.n_keys * wpk > target * 16) wpk = (target * 16 + a.n_keys - 1) / a.n_keys;
    if (wpk < 1) wpk = 1;
    if (wpk > a.be_out) wpk = a.be_out;
    const int64_t waves = a.n_keys * wpk;
    hipLaunchKernelGGL(reduce_rows_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, st, a, wpk);
  } else {
    int64_t chunks = (a.be_out + 255) / 256;
    if (chunks > 64) chunks = 64;
    hipLaunchKernelGGL(reduce_cols_kernel, dim3(unsigned(a.n_keys * chunks)), dim3(256), 0, st, a, chunks);
  }
  return hipGetLastError();
}

}  // namespace jagg
