// attention.hip -- attention as one join-agg: the online-softmax triple.
//
// "Stax (5): Caching and Measurement", chapter summary on Section 9.10 and
// exercise 15: the (m, l, a) triple of online softmax
// lets attention be tiled like a reduction whose combine merges triples;
// "Every Kernel Is a Join" Def. 3.7 then makes it one join-agg over blocked
// Q, K, V: the join pairs each output (X, s, E) block with the K/V tuples of
// every t block (only t-block <= s-block under a causal pair), f of a joined
// tuple is the triple of its t range, the aggregation merges the triples of
// one output key in join-list order, and the recompose writes a / l.  Here
// the merge runs in registers as the workgroup walks the key's joined
// tuples, so neither scores nor probabilities reach memory.
//
// CDNA4 mapping (v_mfma_f32_32x32x16_bf16; fragment lane l holds row/column
// l % 32 and K values 8 * (l / 32) .. + 7):
//  - Scores are computed transposed, S^T = K Q^T (M = t, N = s, K = D), so
//    that lane l owns one query row s = l % 32 of its wavefront and 32 of
//    the tile's 64 keys; lane l ^ 32 holds the other 32.  A row maximum is
//    32 in-lane maxima and one cross-half exchange.
//  - The output is accumulated transposed too, O^T = V^T P^T (M = E, N = s,
//    K = t): lane l again owns row s, so rescaling by exp(m_old - m_new) is
//    one scalar per lane, and P^T is the B operand straight from the score
//    registers.  The score layout puts keys {0-3, 8-11} (+4 on the upper
//    half) in a lane's first 8 values; the V^T fragment is read with the
//    same key permutation through two ds_read_b64_tr_b16 (the sum over the
//    16 keys of an MFMA step does not depend on their order).
//  - Q fragments stay in registers for the whole walk; K and V tiles of 64
//    keys are staged in LDS (rows padded by 16 / 64 bytes against bank
//    conflicts) with two stages: the global loads of tile i+1 are in flight
//    while tile i is computed, one barrier per tile.
//  - Softmax works in base 2: the maximum is taken on the raw scores and
//    exp2(score * alpha log2 e - m) is one FMA and one exp (alpha > 0).
//  - The 128 x E output tile goes through LDS so that rows leave as 16-byte
//    stores.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;  // query rows per workgroup (32 per wavefront)
constexpr int kKeys = 64;   // keys per tile
constexpr uint32_t kOut = 0x80000000u;  // byte offset past any block: the load reads zeros

__device__ __forceinline__ f32x16 mma(const uint4 &a, const uint4 &b, const f32x16 &c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint32_t fd_mod(uint32_t n, const FastDiv &f) { return n - fd_div(n, f) * f.d; }

__device__ __forceinline__ uint4 tr_pair(const char *p0, const char *p1) {
  typedef __attribute__((address_space(3))) i16x4 *lds_v4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(const_cast<char *>(p0)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(const_cast<char *>(p1)));
  uint4 r;
  __builtin_memcpy(&r.x, &lo, 8);
  __builtin_memcpy(&r.z, &hi, 8);
  return r;
}

}  // namespace

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attention_kernel(const AttnArgs a) {
  constexpr int KP = D * 2 + 16;  // K tile row pitch (bytes)
  constexpr int VP = D * 2 + 64;  // V tile row pitch
  constexpr int KBYTES = kKeys * KP;
  constexpr int STAGE = KBYTES + kKeys * VP;
  constexpr int OESZ = OUT_BF16 ? 2 : 4;
  constexpr int OP = D * OESZ + 16;  // output staging row pitch
  constexpr int LDS = 2 * STAGE > kRows * OP ? 2 * STAGE : kRows * OP;
  constexpr int CPR = D / 8;       // 16-byte chunks per K / V row
  constexpr int RPP = 256 / CPR;   // rows per pass of the workgroup
  constexpr int NP = kKeys / RPP;  // passes per tile
  constexpr int KS = D / 16;       // MFMA steps over D
  constexpr int ET = D / 32;       // 32-wide E tiles
  __shared__ __attribute__((aligned(16))) char smem[LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // workgroup -> (batch index inside the block, output key, s tile).  With
  // xcd_group, the workgroups of one batch index (which share its K and V)
  // are numbered so that they all land on one XCD: dispatch deals
  // workgroups to the 8 XCDs round-robin, each XCD with its own L2.
  uint32_t w = blockIdx.x;
  if (a.xcd_group) {
    const uint32_t xcd = w & 7u, local = w >> 3;
    const uint32_t grp = fd_div(local, a.div_group);
    w = (grp * 8u + xcd) * a.div_group.d + (local - grp * a.div_group.d);
  }
  uint32_t st = fd_mod(w, a.div_st);
  if (a.reverse) st = a.div_st.d - 1 - st;  // causal: later row tiles walk more keys, so they go first
  w = fd_div(w, a.div_st);
  const uint32_t kq = w % uint32_t(a.n_keys);
  const uint32_t bi = w / uint32_t(a.n_keys);
  uint32_t key = kq;
  if (a.reverse) {
    // causal: a key's work grows with its s-block, so launch the keys by
    // s-block, heaviest first (key = (hi * ks + kappa_s) * Ws + lo)
    const uint32_t sb = fd_div(kq, a.div_per_s), rest = kq - sb * a.div_per_s.d;
    const uint32_t hi = fd_div(rest, a.div_Ws), lo = rest - hi * a.div_Ws.d;
    key = (hi * a.div_ks.d + (a.div_ks.d - 1 - sb)) * a.div_Ws.d + lo;
  }
  const int32_t cnt = a.counts[key];
  // the join list is read-only for the kernel's lifetime: reading it through
  // the constant address space keeps the tuple-id reads on the scalar unit.
  // A vector load there would make the walk wait (vmcnt counts in issue
  // order) for the next tile's K / V loads issued just before it.
  typedef const __attribute__((address_space(4))) int32_t *const_i32p;
  const const_i32p ents = (const_i32p)(a.list + int64_t(key) * a.per_key * 4);

  // offsets of the batch index inside each block
  int64_t oQ = 0, oK = 0, oV = 0, oO = 0;
  {
    uint32_t r = bi;
    for (int i = a.nx - 1; i >= 0; --i) {
      const uint32_t q = fd_div(r, a.xdiv[i]);
      const int64_t dig = int64_t(r - q * a.xdiv[i].d);
      r = q;
      oQ += dig * a.xQ[i];
      oK += dig * a.xK[i];
      oV += dig * a.xV[i];
      oO += dig * a.xO[i];
    }
  }
  // the block's interval of s (and, for a key tuple, of t): uniform blocks
  // of e, or the bounds of packed sequences
  const uint32_t kap_s = fd_mod(fd_div(key, a.div_Ws), a.div_ks);
  const int32_t S0 = a.iv ? a.bnd[kap_s] : int32_t(kap_s) * a.e_s;  // first s of the block
  const int32_t S_end = a.iv ? a.bnd[kap_s + 1] : a.n_s;            // rows from here on do not exist
  const int32_t s_tile0 = int32_t(st) * kRows;
  const int32_t s_loc = s_tile0 + 32 * wave + l32;  // this lane's query row, inside the block
  const int32_t s_glob = S0 + s_loc;
  const bool row_ok = s_loc < a.e_s && s_glob < S_end;
  auto t_lo = [&](uint32_t kap) { return a.iv ? a.bnd[kap] : int32_t(kap) * a.e_t; };
  auto t_end = [&](uint32_t kap) { return a.iv ? a.bnd[kap + 1] : a.n_t; };
  const int32_t s_hi = (s_tile0 + kRows < a.e_s ? s_tile0 + kRows : a.e_s) - 1;
  // last existing row of the workgroup (rows past the block's interval are padding)
  const int32_t wg_s_last = S0 + s_hi < S_end - 1 ? S0 + s_hi : S_end - 1;
  const int32_t wave_s_first = S0 + s_tile0 + 32 * wave;                   // first row of the wavefront
  const int32_t wave_s_last = S0 + (s_tile0 + 32 * wave + 31 < s_hi ? s_tile0 + 32 * wave + 31 : s_hi);

  // Q fragments (B operand of S^T = K Q^T), kept for the whole walk
  uint4 qf[KS];
  {
    const int64_t qt = cnt > 0 ? ents[1] : 0;
    const __amdgpu_buffer_rsrc_t rq = rsrc(static_cast<const char *>(a.Q) + (qt * a.beQ + oQ) * 2, (a.beQ - oQ) * 2);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qf[k] = bload(rq, s_loc < a.e_s ? uint32_t((int64_t(s_loc) * a.sQ + 16 * k + 8 * hi) * 2) : kOut);
  }

  // tiles of the walk: joined tuples in t-block order, 64 keys at a time;
  // under a causal pair the walk ends at the first tile past the last row
  const int tpe = (a.e_t + kKeys - 1) / kKeys;
  // a tile of padding rows only (a short packed sequence) walks nothing and
  // writes zeros
  int n_it = S0 + s_tile0 < S_end ? cnt * tpe : 0;
  if (CAUSAL && n_it > 0) {
    n_it = 0;
    for (int e = 0; e < cnt; ++e) {
      const int32_t T0 = t_lo(fd_mod(fd_div(uint32_t(ents[e * 4 + 2]), a.div_Wt), a.div_kt));
      if (T0 > wg_s_last) break;
      int tt = 0;
      while (tt < tpe && T0 + tt * kKeys <= wg_s_last) ++tt;
      n_it += tt;
      if (tt < tpe) break;
    }
  }

  // K / V tile loads: each lane's byte offset inside a tile is fixed; the
  // tile's origin goes into the (scalar) buffer base, and the buffer ends at
  // the tuple's last valid row, so rows past it read zeros
  uint32_t koff[NP], voff[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * RPP + tid / CPR, ch = tid % CPR;
    koff[p] = uint32_t((int64_t(row) * a.tK + ch * 8) * 2);
    voff[p] = uint32_t((int64_t(row) * a.tV + ch * 8) * 2);
  }
  // tuple ids and key range of one tile of the walk; the loop reads them one
  // iteration ahead, so the scalar loads overlap the LDS stores and the
  // barrier instead of stalling the top of an iteration
  struct TileIds {
    int64_t kt, vt;           // K and V tuple ids
    int32_t tt, T0, t_valid;  // tile inside the tuple, its first key, keys [0, t_valid) that exist
  };
  auto tile_ids = [&](int it) {
    const int e = it / tpe;
    TileIds r;
    r.tt = it - e * tpe;
    r.kt = ents[e * 4 + 2];
    r.vt = ents[e * 4 + 3];
    const uint32_t kap = fd_mod(fd_div(uint32_t(r.kt), a.div_Wt), a.div_kt);
    r.T0 = t_lo(kap) + r.tt * kKeys;
    int32_t tv = a.e_t - r.tt * kKeys;
    if (t_end(kap) - r.T0 < tv) tv = t_end(kap) - r.T0;
    r.t_valid = tv > kKeys ? kKeys : tv;
    return r;
  };
  uint4 kr[NP], vr[NP];
  auto load_tile = [&](const TileIds &ti) {
    const int64_t kt = ti.kt, vt = ti.vt;
    const int64_t r0 = int64_t(ti.tt) * kKeys;  // first row of the tile
    const int64_t kbase = kt * a.beK + oK + r0 * a.tK, vbase = vt * a.beV + oV + r0 * a.tV;
    const int64_t kend = oK + int64_t(a.e_t - 1) * a.tK + D, vend = oV + int64_t(a.e_t - 1) * a.tV + D;
    const __amdgpu_buffer_rsrc_t rk =
        rsrc(static_cast<const char *>(a.K) + kbase * 2, (kt * a.beK + kend - kbase) * 2);
    const __amdgpu_buffer_rsrc_t rv =
        rsrc(static_cast<const char *>(a.V) + vbase * 2, (vt * a.beV + vend - vbase) * 2);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      kr[p] = bload(rk, koff[p]);
      vr[p] = bload(rv, voff[p]);
    }
  };
  auto store_tile = [&](int stage) {
    char *ks = smem + stage * STAGE;
    char *vs = ks + KBYTES;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = p * RPP + tid / CPR, ch = tid % CPR;
      *reinterpret_cast<uint4 *>(ks + row * KP + ch * 16) = kr[p];
      *reinterpret_cast<uint4 *>(vs + row * VP + ch * 16) = vr[p];
    }
  };

  f32x16 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[et][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  TileIds cur{}, nxt{};  // the tile being computed, the one being loaded
  if (n_it > 0) {
    cur = tile_ids(0);
    load_tile(cur);
    store_tile(0);
  }
  if (n_it > 1) nxt = tile_ids(1);
  // Every global load so far (Q fragments, first tile) has landed: said
  // explicitly (vmcnt(0)), the compiler's wait counting enters the loop with
  // nothing pending and does not make the S^T MFMAs of each tile wait for
  // the next tile's loads, which it would otherwise treat as possibly
  // carrying Q
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  const int g = lane >> 4, s16 = lane & 15;
  const float scale = a.scale_log2;  // > 0
  for (int it = 0; it < n_it; ++it) {
    const bool more = it + 1 < n_it;
    if (more) load_tile(nxt);
    const int32_t T0 = cur.T0, t_valid = cur.t_valid;
    if (!(CAUSAL && T0 > wave_s_last)) {
      const char *ks = smem + (it & 1) * STAGE;
      const char *vs = ks + KBYTES;
      // S^T = K Q^T for the 64 keys x 32 rows of this wavefront
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[mt][v] = 0.0f;
      // K fragments two MFMAs ahead of their use, as the V fragments below
      auto kread = [&](int q) {
        return *reinterpret_cast<const uint4 *>(ks + (32 * (q & 1) + l32) * KP + 32 * (q >> 1) + 16 * hi);
      };
      {
        uint4 kring[3];
        kring[0] = kread(0);
        kring[1] = kread(1);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) {
          if (q + 2 < 2 * KS) kring[(q + 2) % 3] = kread(q + 2);
          __builtin_amdgcn_sched_barrier(0);
          sacc[q & 1] = mma(kring[q % 3], qf[q >> 1], sacc[q & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // drop missing keys and, under the causal pair, t > s
      const bool full = t_valid == kKeys && !(CAUSAL && T0 + kKeys - 1 > wave_s_first);
      if (!full) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int tl = 32 * mt + 8 * (v >> 2) + 4 * hi + (v & 3);
            if (tl >= t_valid || (CAUSAL && T0 + tl > s_glob)) sacc[mt][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[mt][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale;  // base-2 maximum of the tile (scale > 0)
      // The reference m of the running triple moves only when the tile's
      // maximum exceeds it by more than 8 (then p <= 2^8 always): the merge
      // is exact for any common reference, and most tiles skip the rescale.
      const float m_new = mx > m_run + 8.0f ? mx : m_run;
      const float base = m_new == -INFINITY ? 0.0f : m_new;
      const float corr = __builtin_amdgcn_exp2f(m_run - base);
      float sum = 0.0f;
      uint4 pf[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][8 * h + j], scale, -base));
            sum += p[j];
          }
          pf[2 * mt + h] = uint4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                 pack_bf16x2(p[6], p[7])};
        }
      if (!__all(m_new == m_run)) {  // some row moved its reference
        l_run *= corr;
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[et][v] *= corr;
      }
      l_run += sum;
      m_run = m_new;
      // O^T += V^T P^T, with V^T read in the keys' score order; the V
      // fragments are read two MFMAs ahead of their use (a ring of three),
      // so the LDS latency hides behind the MFMAs in between
      auto vread = [&](int q) {
        const int n = 32 * (q >> 2) + 16 * (g & 1) + 4 * (s16 & 3);
        const int kb = 16 * (q & 3) + 4 * (g >> 1) + (s16 >> 2);
        return tr_pair(vs + kb * VP + n * 2, vs + (kb + 8) * VP + n * 2);
      };
      uint4 vring[3];
      vring[0] = vread(0);
      vring[1] = vread(1);
#pragma unroll
      for (int q = 0; q < 4 * ET; ++q) {
        if (q + 2 < 4 * ET) vring[(q + 2) % 3] = vread(q + 2);
        __builtin_amdgcn_sched_barrier(0);
        acc[q >> 2] = mma(vring[q % 3], pf[q & 3], acc[q >> 2]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
    if (it + 2 < n_it) nxt = tile_ids(it + 2);
    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // recompose: a / l for rows that exist and are inside the relation, 0 elsewhere
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (row_ok && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  {
    char *orow = smem + (32 * wave + l32) * OP;
#pragma unroll
    for (int et = 0; et < ET; ++et)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e0 = 32 * et + 8 * q + 4 * hi;
        const float y0 = acc[et][4 * q] * inv, y1 = acc[et][4 * q + 1] * inv;
        const float y2 = acc[et][4 * q + 2] * inv, y3 = acc[et][4 * q + 3] * inv;
        if constexpr (OUT_BF16) {
          *reinterpret_cast<uint2 *>(orow + e0 * 2) = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        } else {
          *reinterpret_cast<float4 *>(orow + e0 * 4) = make_float4(y0, y1, y2, y3);
        }
      }
  }
  __syncthreads();
  constexpr int OCH = D * OESZ / 16;  // 16-byte chunks per output row
  char *ob = static_cast<char *>(a.O) + (int64_t(key) * a.beO + oO) * OESZ;
  for (int i = tid; i < kRows * OCH; i += 256) {
    const int row = i / OCH, ch = i - row * OCH;
    const int sl = s_tile0 + row;
    if (sl < a.e_s)
      *reinterpret_cast<uint4 *>(ob + int64_t(sl) * a.sO * OESZ + ch * 16) =
          *reinterpret_cast<const uint4 *>(smem + row * OP + ch * 16);
  }
}

template <int D, bool CAUSAL, bool OUT_BF16>
static hipError_t go(const AttnArgs &a, hipStream_t st) {
  const int64_t grid = int64_t(a.nbatch) * a.n_keys * a.s_tiles;
  hipLaunchKernelGGL((attention_kernel<D, CAUSAL, OUT_BF16>), dim3(unsigned(grid)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int d, bool causal, bool out_bf16, hipStream_t st) {
#define JAGG_ATT(DD, CC, OO) \
  if (d == DD && causal == CC && out_bf16 == OO) return go<DD, CC, OO>(a, st);
  JAGG_ATT(128, false, false) JAGG_ATT(128, false, true) JAGG_ATT(128, true, false) JAGG_ATT(128, true, true)
  JAGG_ATT(64, false, false) JAGG_ATT(64, false, true) JAGG_ATT(64, true, false) JAGG_ATT(64, true, true)
#undef JAGG_ATT
  return hipErrorInvalidValue;
}

}  // namespace jagg
