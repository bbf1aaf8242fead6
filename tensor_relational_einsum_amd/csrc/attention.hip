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
//    32 in-lane maxima and one exchange of the wavefront's halves
//    (v_permlane32_swap, no LDS round trip).
//  - The output is accumulated transposed too, O^T = V^T P^T (M = E, N = s,
//    K = t): lane l again owns row s, so rescaling by exp(m_old - m_new) is
//    one scalar per lane, and P^T is the B operand straight from the score
//    registers.  The score layout puts keys {0-3, 8-11} (+4 on the upper
//    half) in a lane's first 8 values; the V^T fragment is read with the
//    same key permutation through two ds_read_b64_tr_b16 (the sum over the
//    16 keys of an MFMA step does not depend on their order).
//  - Row sums l come from v_dot2c_f32_bf16 on the packed probabilities (one
//    instruction per two keys), so l adds exactly the bf16 values that the
//    PV product multiplies.
//  - Q fragments stay in registers for the whole walk.  K and V tiles of 64
//    keys are written to LDS by buffer loads with the LDS destination (no
//    registers hold data in flight), unpadded, with an XOR swizzle of
//    16-byte slots that keeps the fragment reads conflict-free:
//      K: slot c of key row r at c ^ ((r / RP) % SPR)
//      V: slot c of key row r at c ^ ((4 (r / RP)) % SPR)
//    (SPR = D / 8 slots per row, RP = 16 / SPR rows per 256 bytes).  Two K
//    and two V buffers: the loads of K for tile i + 2 and of V for tile
//    i + 1 are issued during iteration i, after the barrier that ends every
//    read of the buffers they overwrite, one between every other S MFMA.
//  - Software pipeline, per wavefront: iteration i issues the S MFMAs of
//    tile i + 1 with the exponentials of the upper key half of tile i
//    between them (phase A), then the PV MFMAs of tile i with the maximum,
//    reference update and lower-half exponentials of tile i + 1 between
//    them (phase B).  The VALU work of one tile thus runs in the shadow of
//    the MFMAs of its neighbours instead of between them.
//  - Every wavefront walks every tile of its workgroup's walk; under a
//    causal pair the masked scores of keys past a wavefront's rows give
//    probabilities 0 (a uniform pipeline costs the few diagonal tiles a
//    wavefront would otherwise skip).
//  - Softmax works in base 2: the maximum is taken on the raw scores and
//    exp2(score * alpha log2 e - m) is one FMA and one exp (alpha > 0).
//  - The 128 x E output tile goes through LDS so that rows leave as 16-byte
//    stores.
#include <type_traits>

#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
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

// maximum of x over lanes l and l ^ 32 (the two halves of a query row)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keeps x in place: an empty volatile asm that reads and writes x.  Volatile
// asm keeps its order against the scheduling barriers, so pinning a VALU
// slice's inputs and outputs holds the slice between the two MFMAs it was
// written between (pure arithmetic would otherwise be moved next to its
// first use, away from the MFMA shadow it is meant to fill).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

// acc + the two bf16 halves of w
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

}  // namespace

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attention_kernel(const AttnArgs a) {
  constexpr int SPR = D / 8;             // 16-byte slots per K / V row
  constexpr int RB = D * 2;              // bytes per K / V row
  constexpr int RP = 16 / SPR;           // rows per 256 bytes
  constexpr int TB = kKeys * RB;         // bytes of one K or V tile
  constexpr int NL = kKeys * SPR / 256;  // LDS loads per thread per tile and operand
  constexpr int OESZ = OUT_BF16 ? 2 : 4;
  constexpr int OP = D * OESZ + 16;  // output staging row pitch
  constexpr int LDS = 4 * TB > kRows * OP ? 4 * TB : kRows * OP;
  constexpr int KS = D / 16;       // MFMA steps over D
  constexpr int ET = D / 32;       // 32-wide E tiles
  constexpr int NQA = 2 * KS;      // S MFMAs per tile and wavefront
  constexpr int NQB = 4 * ET;      // PV MFMAs per tile and wavefront
  static_assert(NL >= 1 && NL <= 4 && RP * SPR == 16, "tile geometry");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  // per joined tuple of the key: K tuple, V tuple, first key, end of its keys
  __shared__ int4 etab[kMaxAttnTuples];
  char *const kbuf = smem;           // K tiles at kbuf + b * TB, b = 0, 1
  char *const vbuf = smem + 2 * TB;  // V tiles

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // workgroup -> (batch index inside the block, output key, s tile).  With
  // xcd_group (non-causal launches), the workgroups of one batch index
  // (which share its K and V) are numbered so that they all land on one
  // XCD: dispatch deals workgroups to the 8 XCDs round-robin, each XCD with
  // its own L2.  Causal launches are ordered by work instead (below).
  uint32_t w = blockIdx.x;
  if (a.xcd_group && !a.reverse) {
    const uint32_t xcd = w & 7u, local = w >> 3;
    const uint32_t grp = fd_div(local, a.div_group);
    w = (grp * 8u + xcd) * a.div_group.d + (local - grp * a.div_group.d);
  }
  uint32_t st, bi, key;
  if (a.reverse) {
    // causal: a workgroup walks more keys the later its rows, so every
    // workgroup of one work class is dispatched before any lighter one,
    // across all batch indices and keys (the longest first, which keeps the
    // launch's tail short).  Class: s-block, then s-tile; packed sequences:
    // s-tile, then s-block, each sequence starting its causal walk at its
    // own first row
    const uint32_t minor_n = uint32_t(a.nbatch) * a.div_per_s.d;
    const uint32_t cls = w / minor_n, minor = w - cls * minor_n;
    const uint32_t ks = a.div_ks.d, nst = a.div_st.d;
    uint32_t sb;
    if (a.iv) {
      st = nst - 1 - cls / ks;
      sb = cls % ks;
    } else {
      sb = ks - 1 - cls / nst;
      st = nst - 1 - cls % nst;
    }
    bi = minor / a.div_per_s.d;
    const uint32_t rest = minor - bi * a.div_per_s.d;
    const uint32_t hi = fd_div(rest, a.div_Ws), lo = rest - hi * a.div_Ws.d;
    key = (hi * ks + sb) * a.div_Ws.d + lo;
  } else {
    st = fd_mod(w, a.div_st);
    w = fd_div(w, a.div_st);
    key = w % uint32_t(a.n_keys);
    bi = w / uint32_t(a.n_keys);
  }
  const int32_t cnt = a.counts[key];
  // the join list is read-only for the kernel's lifetime: reading it through
  // the constant address space keeps the tuple-id reads on the scalar unit
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

  // LDS loads: lane l of load n of this wavefront fills physical slot
  // P = (4 n + wave) * 64 + l of a tile; the offsets below pick the global
  // 16 bytes that belong there under each operand's swizzle.  A tile's
  // origin goes into the (scalar) buffer base, and the buffer ends at the
  // tuple's last row, so rows past it read zeros.
  uint32_t kdo[NL], vdo[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int P = (4 * n + wave) * 64 + lane, r = P / SPR, ph = P % SPR;
    const int ck = ph ^ ((r / RP) % SPR), cv = ph ^ ((4 * (r / RP)) % SPR);
    kdo[n] = uint32_t((int64_t(r) * a.tK + 8 * ck) * 2);
    vdo[n] = uint32_t((int64_t(r) * a.tV + 8 * cv) * 2);
  }
  // Fragment read addresses inside a tile.  K (ds_read_b128): row l32 (+32
  // for the second key half), logical slot 2 k + hi; the swizzle makes the
  // address (row base with slot hi ^ f) ^ 32 k.  V (two ds_read_b64_tr_b16):
  // key row 16 (q % 4) + rl (+8), logical slot 4 (q / 4) + cl, half s16 % 2;
  // the swizzle flips only the 4 (q / 4) part.
  const int g = lane >> 4, s16 = lane & 15;
  uint32_t kaddr[KS], vaddr[ET];
  {
    const int fk = (l32 / RP) % SPR;
    const uint32_t kb0 = uint32_t(l32 * RB + 16 * (hi ^ fk));
#pragma unroll
    for (int k = 0; k < KS; ++k) kaddr[k] = kb0 ^ uint32_t(32 * k);
    const int rl = 4 * (g >> 1) + (s16 >> 2), cl = 2 * (g & 1) + ((s16 & 3) >> 1);
    const int fv4 = (((4 * (rl / RP)) % SPR) >> 2);
    const uint32_t vb0 = uint32_t(rl * RB + 16 * cl + 8 * (s16 & 1));
#pragma unroll
    for (int e = 0; e < ET; ++e) vaddr[e] = vb0 + uint32_t(64 * (e ^ fv4));
  }

  // tuple ids and key range of one tile of the walk
  // The joined tuples' ids and key ranges, one lane per tuple, into LDS:
  // the walk then reads a tuple's record with one LDS read instead of a
  // chain of scalar loads and divisions per tile.  (Scalar loads would also
  // share their wait counter with the fragment reads, and return out of
  // order, so every pending one would turn the fragment waits into full
  // waits.)
  for (int e = tid; e < cnt; e += 256) {
    const int32_t kt = a.list[int64_t(key) * a.per_key * 4 + e * 4 + 2];
    const int32_t vt = a.list[int64_t(key) * a.per_key * 4 + e * 4 + 3];
    const uint32_t kap = fd_mod(fd_div(uint32_t(kt), a.div_Wt), a.div_kt);
    etab[e] = int4{kt, vt, t_lo(kap), t_end(kap)};
  }
  struct TileIds {
    int32_t kt, vt;           // K and V tuple ids
    int32_t tt, T0, t_valid;  // tile inside the tuple, its first key, keys [0, t_valid) that exist
  };
  // tile tt of joined tuple e (the table is written and a barrier passed)
  auto tile_ids = [&](int e, int tt) {
    const int4 rec = etab[e];
    TileIds r;
    r.kt = __builtin_amdgcn_readfirstlane(rec.x);
    r.vt = __builtin_amdgcn_readfirstlane(rec.y);
    r.tt = tt;
    r.T0 = __builtin_amdgcn_readfirstlane(rec.z) + tt * kKeys;
    int32_t tv = a.e_t - tt * kKeys;
    const int32_t te = __builtin_amdgcn_readfirstlane(rec.w) - r.T0;
    if (te < tv) tv = te;
    r.t_valid = tv > kKeys ? kKeys : tv;
    return r;
  };
  // LDS address of this wavefront's first 1 KB of the K buffer 0; buffer b
  // of K, V and load n add compile-time constants
  const uint32_t lds_w = uint32_t(reinterpret_cast<uintptr_t>((lds_dma_ptr)(smem))) + uint32_t(wave_s) * 1024u;
  // byte geometry of a tile load: origin of the batch index's rows in tuple
  // 0, bytes per tuple, bytes per tile of keys, bytes from a tuple's row 0 to
  // the end of its last row
  const char *const k0 = static_cast<const char *>(a.K) + oK * 2;
  const char *const v0 = static_cast<const char *>(a.V) + oV * 2;
  const int64_t kblk = a.beK * 2, vblk = a.beV * 2;
  const int32_t ktile = int32_t(kKeys * a.tK * 2), vtile = int32_t(kKeys * a.tV * 2);
  const int32_t kspan = int32_t((int64_t(a.e_t - 1) * a.tK + D) * 2), vspan = int32_t((int64_t(a.e_t - 1) * a.tV + D) * 2);
  // buffer resources of a tile's K and V rows; a tile past the walk gets an
  // empty buffer (its loads write zeros and read no memory)
  auto rsrc_k = [&](const TileIds &ti, bool live) {
    const int32_t skip = ti.tt * ktile;
    return dma_rsrc(k0 + int64_t(ti.kt) * kblk + skip, live ? kspan - skip : 0);
  };
  auto rsrc_v = [&](const TileIds &ti, bool live) {
    const int32_t skip = ti.tt * vtile;
    return dma_rsrc(v0 + int64_t(ti.vt) * vblk + skip, live ? vspan - skip : 0);
  };
  // load n of a tile into the LDS buffer at byte offset BASE (n is a
  // constant once the callers are unrolled)
  auto dma_n = [&](auto base, int n, const i32x4_rsrc &r, const uint32_t (&off)[NL]) {
    constexpr uint32_t BASE = decltype(base)::value;
    if (n == 0) dma16_at<BASE>(r, off[0], lds_w);
    else if (n == 1) dma16_at<BASE + 4096>(r, off[NL > 1 ? 1 : 0], lds_w);
    else if (n == 2) dma16_at<BASE + 8192>(r, off[NL > 2 ? 2 : 0], lds_w);
    else if (n == 3) dma16_at<BASE + 12288>(r, off[NL > 3 ? 3 : 0], lds_w);
  };
  auto load_k = [&](auto par, const TileIds &ti) {
    constexpr uint32_t B = decltype(par)::value;
    const i32x4_rsrc rk = rsrc_k(ti, true);
#pragma unroll
    for (int n = 0; n < NL; ++n) dma_n(std::integral_constant<uint32_t, B * TB>{}, n, rk, kdo);
  };
  auto load_v = [&](auto par, const TileIds &ti) {
    constexpr uint32_t B = decltype(par)::value;
    const i32x4_rsrc rv = rsrc_v(ti, true);
#pragma unroll
    for (int n = 0; n < NL; ++n) dma_n(std::integral_constant<uint32_t, (2 + B) * TB>{}, n, rv, vdo);
  };
  f32x16 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[et][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f, base = 0.0f, corr = 1.0f;
  bool moved = false;
  const float scale = a.scale_log2;  // > 0

  // S^T of the tile in K buffer b: MFMA q (key half q % 2, D step q / 2),
  // with K fragments read two MFMAs ahead; between MFMA q and q + 1 runs
  // slice q of the VALU work `valu` (a callable taking the slice index)
  auto scores = [&](f32x16 (&sc)[2], int b, auto &&valu) {
    const char *ks = kbuf + b * TB;
    auto kread = [&](int q) { return *reinterpret_cast<const uint4 *>(ks + kaddr[q >> 1] + (q & 1) * 32 * RB); };
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[mt][v] = 0.0f;
    uint4 kring[3];
    kring[0] = kread(0);
    kring[1] = kread(1);
#pragma unroll
    for (int q = 0; q < NQA; ++q) {
      if (q + 2 < NQA) kring[(q + 2) % 3] = kread(q + 2);
      __builtin_amdgcn_sched_barrier(0);
      sc[q & 1] = mma(kring[q % 3], qf[q >> 1], sc[q & 1]);
      __builtin_amdgcn_sched_barrier(0);
      valu(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T for the tile in V buffer b, with slice q of `valu`
  // after MFMA q
  auto pv = [&](const uint32_t (&pw)[16], int b, auto &&valu) {
    const char *vs = vbuf + b * TB;
    auto vread = [&](int q) {
      const char *p = vs + vaddr[q >> 2] + (q & 3) * 16 * RB;
      return tr_pair(p, p + 8 * RB);
    };
    // MFMA q: E tile q % ET, keys 16 (q / ET) .. + 15, so that consecutive
    // MFMAs accumulate into different registers
    auto vq = [&](int q) { return vread(4 * (q % ET) + q / ET); };
    uint4 vring[3];
    vring[0] = vq(0);
    vring[1] = vq(1);
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      if (q + 2 < NQB) vring[(q + 2) % 3] = vq(q + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int k = q / ET;
      acc[q % ET] = mma(vring[q % 3], uint4{pw[4 * k], pw[4 * k + 1], pw[4 * k + 2], pw[4 * k + 3]}, acc[q % ET]);
      __builtin_amdgcn_sched_barrier(0);
      valu(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // drop missing keys and, under the causal pair, t > s
  auto mask = [&](f32x16 (&sc)[2], const TileIds &ti) {
    const bool full = ti.t_valid == kKeys && !(CAUSAL && ti.T0 + kKeys - 1 > wave_s_first);
    if (!full) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tl = 32 * mt + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (tl >= ti.t_valid || (CAUSAL && ti.T0 + tl > s_glob)) sc[mt][v] = -INFINITY;
        }
    }
  };
  // Softmax work of one tile as numbered items, spread over MFMA slices by
  // their VALU cost.  Phase B (under the PV MFMAs of the previous tile)
  // runs items 0..15, which fold the 32 scores into the maximum, item 16,
  // which moves the reference, and the first kLoB probability items; phase
  // A (under the S MFMAs of the next tile) runs the other 32 - kLoB.
  // Probability item u (key value u of the lane: half u / 16, value u % 16)
  // is one FMA and one exponential; an odd u also packs the pair into a bf16
  // word of P and adds it to the row sum.  kLoB balances the two phases.
  constexpr int kLoB = D == 128 ? 12 : 14;
  constexpr int kLoItems = 17 + kLoB;
  float mx = -INFINITY, ph = 0.0f;
  auto prob = [&](const f32x16 (&sc)[2], uint32_t (&pw)[16], int u) {
    float sv = sc[u >> 4][u & 15];
    pin(sv);
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, scale, -base));
    if ((u & 1) == 0) {
      ph = p;
      pin(ph);
    } else {
      pw[u >> 1] = pack_bf16x2(ph, p);
      l_run = add_pair(pw[u >> 1], l_run);
      pin(pw[u >> 1]);
      pin(l_run);
    }
  };
  auto lo_item = [&](const f32x16 (&sc)[2], uint32_t (&pw)[16], int it) {
    if (it < 16) {
      const int mt = it >> 3, v = 2 * (it & 7);
      mx = fmaxf(fmaxf(mx, sc[mt][v]), sc[mt][v + 1]);
      pin(mx);
    } else if (it == 16) {
      // The reference m of the running triple moves only when the tile's
      // maximum exceeds it by more than 8 (then p <= 2^8 always): the merge
      // is exact for any common reference, and most tiles skip the rescale.
      const float t = halves_max(mx) * scale;  // base-2 maximum of the tile (scale > 0)
      mx = -INFINITY;
      const float m_new = t > m_run + 8.0f ? t : m_run;
      base = m_new == -INFINITY ? 0.0f : m_new;
      corr = __builtin_amdgcn_exp2f(m_run - base);
      moved = !__all(m_new == m_run);
      l_run *= corr;
      m_run = m_new;
      pin(base);
      pin(l_run);
    } else {
      prob(sc, pw, it - 17);
    }
  };
  // relative VALU cost of an item and the slice it runs in: slices take
  // equal shares of their phase's total cost, items in order
  auto cost_lo = [](int it) { return it < 16 ? 1 : it == 16 ? 3 : ((it - 17) & 1) ? 7 : 5; };
  auto cost_u = [](int u) { return (u & 1) ? 7 : 5; };
  auto lo_slice = [&](int it) {
    int before = 0, total = 0;
#pragma unroll
    for (int x = 0; x < kLoItems; ++x) {
      if (x < it) before += cost_lo(x);
      total += cost_lo(x);
    }
    return before * NQB / total;
  };
  auto hi_slice = [&](int u) {  // u = kLoB .. 31
    int before = 0, total = 0;
#pragma unroll
    for (int x = kLoB; x < 32; ++x) {
      if (x < u) before += cost_u(x);
      total += cost_u(x);
    }
    return before * NQA / total;
  };
  auto none = [](int) {};

  // two score sets and two probability sets, alternating between tiles
  f32x16 sA[2], sB[2];
  uint32_t pA[16], pB[16];
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  TileIds t1{}, t2{};  // tiles i + 1 and i + 2 of the walk
  int ne = 0, ntt = 0;  // joined tuple and tile of the next tile whose ids are read
  auto next_ids = [&]() {
    const TileIds r = tile_ids(ne, ntt);
    if (++ntt == tpe) {
      ntt = 0;
      ++ne;
    }
    return r;
  };
  __syncthreads();  // the tuple table is written
  if (n_it > 0) {
    const TileIds t0 = next_ids();
    load_k(P0{}, t0);
    load_v(P0{}, t0);
    if (n_it > 1) {
      t1 = next_ids();
      load_k(P1{}, t1);
    }
    if (n_it > 2) t2 = next_ids();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and the first loads
    __syncthreads();
    scores(sA, 0, none);
    mask(sA, t0);
#pragma unroll
    for (int it = 0; it < kLoItems; ++it) lo_item(sA, pA, it);
  }

  // one iteration of the walk (parity par = i % 2), for a tile i with a
  // successor: tile i's scores in sc, the lower half of its probabilities in
  // pc; the next tile's scores go to sn, its lower half to pn
  auto top = [&]() {
    // every wavefront is done with iteration i - 1: the S reads of K buffer
    // i % 2 and the PV reads of V buffer (i + 1) % 2; the loads issued in
    // iteration i - 1 (K of tile i + 1, V of tile i) have landed
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  auto step = [&](auto par, int i, f32x16 (&sc)[2], f32x16 (&sn)[2], uint32_t (&pc)[16], uint32_t (&pn)[16]) {
    constexpr uint32_t B = decltype(par)::value;
    top();
    // this iteration loads K of tile i + 2 into K buffer i % 2 and V of tile
    // i + 1 into V buffer (i + 1) % 2, one load after every other S MFMA of
    // phase A: a burst of loads right after the barrier would back up the
    // vector memory path and hold up the in-order wavefront
    const i32x4_rsrc rk = rsrc_k(t2, i + 2 < n_it), rv = rsrc_v(t1, true);
    // the ids of tile i + 3
    TileIds t3{};
    if (i + 3 < n_it) t3 = next_ids();
    // phase A: S of tile i + 1 || upper-half probabilities of tile i, loads
    scores(sn, 1 - B, [&](int q) {
#pragma unroll
      for (int u = kLoB; u < 32; ++u)
        if (hi_slice(u) == q) prob(sc, pc, u);
      if (q & 1) {
        const int d = q >> 1;
        if (d < NL) dma_n(std::integral_constant<uint32_t, B * TB>{}, d, rk, kdo);
        else if (d < 2 * NL) dma_n(std::integral_constant<uint32_t, (3 - B) * TB>{}, d - NL, rv, vdo);
      }
    });
    mask(sn, t1);
    // phase B: PV of tile i || maximum and lower-half probabilities of tile i + 1
    pv(pc, B, [&](int q) {
#pragma unroll
      for (int it = 0; it < kLoItems; ++it)
        if (lo_slice(it) == q) lo_item(sn, pn, it);
    });
    // tile i + 1 moved the reference of some row: rescale what tiles <= i
    // accumulated (after their PV, before tile i + 1's)
    if (moved) {
#pragma unroll
      for (int et = 0; et < ET; ++et)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[et][v] *= corr;
    }
    t1 = t2;
    t2 = t3;
  };
  // the walk's last tile
  auto last = [&](auto par, int i, const f32x16 (&sc)[2], uint32_t (&pc)[16]) {
    constexpr int B = decltype(par)::value;
    top();
#pragma unroll
    for (int u = kLoB; u < 32; ++u) prob(sc, pc, u);
    pv(pc, B, none);
  };
  int i = 0;
  for (; i + 2 < n_it; i += 2) {
    step(P0{}, i, sA, sB, pA, pB);
    step(P1{}, i + 1, sB, sA, pB, pA);
  }
  if (n_it - i == 2) {
    step(P0{}, i, sA, sB, pA, pB);
    last(P1{}, i + 1, sB, pB);
  } else if (n_it - i == 1) {
    last(P0{}, i, sA, pA);
  }

  // recompose: a / l for rows that exist and are inside the relation, 0 elsewhere
  __syncthreads();  // every wavefront is done reading the last tiles
  const float l_tot = halves_sum(l_run);
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
