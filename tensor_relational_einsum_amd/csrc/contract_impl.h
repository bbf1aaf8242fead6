// contract_impl.h -- MFMA block contraction with the SUM aggregation fused.
//
// "Every Kernel Is a Join" (Ding et al.), Sec. 1 and Examples 3.8/3.9: in a
// product of two blocked matrices, the pairs of blocks that agree on the
// contracted index are matched, each pair is multiplied, and the partial
// products landing on one output block are added (Def. 3.7 step 2).  One workgroup owns one
// BM x BN tile of one output block (and one batch index) and walks every
// joined tuple of that output key and the K-tiles of each, accumulating in
// fp32 registers; the tile is written once, so the aggregation never goes
// through memory (the page's aggregation pushdown, on one GPU).
//
// CDNA4 mapping
//  - MFMA 32x32: bf16 v_mfma_f32_32x32x16_bf16, fp32 v_mfma_f32_32x32x2_f32.
//    Lane l of a fragment owns row/column l%32 and the K values
//    8*(l/32)..+7 (bf16) or 4*(l/32)..+3 (fp32, one per MFMA).
//  - Each operand tile is staged in LDS in its own global orientation, one
//    BK-deep slab of 128 bytes per row: K-contiguous tiles as [rows][BK],
//    M/N-contiguous tiles as [BK][rows].  Global loads (buffer loads whose
//    out-of-range lanes read zeros) and LDS stores are 16-byte vectors.
//    Rows are padded (16 bytes for K-contiguous tiles, 64 bytes for the
//    others) so the fragment reads below spread over the 64 LDS banks while
//    every fragment address stays a register base plus an immediate.
//  - Fragment reads: ds_read_b128 for K-contiguous tiles; for bf16
//    M/N-contiguous tiles two ds_read_b64_tr_b16, whose 16-lane transpose
//    turns four 4-element row pieces into four 4-element K columns; for
//    fp32 M/N-contiguous tiles one ds_read_b32 per MFMA.
//  - Two LDS stages: the global loads of step s+1 are in flight while the
//    MFMAs of step s run; one barrier per step.  This kernel serves fp32,
//    one-element loads, causal masks on the reduced letter and small tiles;
//    bf16 256 x 256 tiles over 16-byte vectors go to the LDS-pipelined
//    kernel of contract_dma.h.
//  - Workgroups are renumbered so that consecutive tiles of one output row
//    panel land on the same XCD (dispatch round-robins workgroups over the
//    8 XCDs, each with its own L2).
#pragma once
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;

template <int NB>
struct VecT;
template <>
struct VecT<16> {
  using type = uint4;
};
template <>
struct VecT<4> {
  using type = uint32_t;
};
template <>
struct VecT<2> {
  using type = uint16_t;
};

constexpr int kSlab = 128;  // bytes of K per tile row (BK = 128 / sizeof(T))
constexpr int kPitchKC = kSlab + 16;

// LDS row pitch of an operand tile of R rows
template <bool KC, int R, int ESZ>
constexpr int tile_pitch() {
  return KC ? kPitchKC : R * ESZ + 64;
}
template <bool KC, int R, int ESZ>
constexpr int tile_bytes() {
  return KC ? R * kPitchKC : (kSlab / ESZ) * (R * ESZ + 64);
}

// Buffer-resource loads: the scalar resource holds the tile origin and the
// bytes left in the block; a lane whose element lies outside the tile passes
// an offset past the end, and the hardware returns zeros for it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *origin, int64_t bytes_left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(origin), (short)0, int(bytes_left), 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // past any block (blocks stay under 2 GiB)

template <int NB>
__device__ __forceinline__ typename VecT<NB>::type buf_load(__amdgpu_buffer_rsrc_t rs, uint32_t off);
template <>
__device__ __forceinline__ uint4 buf_load<16>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, int(off), 0, 0);
  return uint4{v.x, v.y, v.z, v.w};
}
template <>
__device__ __forceinline__ uint32_t buf_load<4>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, int(off), 0, 0);
}
template <>
__device__ __forceinline__ uint16_t buf_load<2>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(rs, int(off), 0, 0);
}

// One operand tile: R rows (M or N) by BK, KC = contiguous along K.  Thread
// t's load i covers LDS row lr0 + i*DR (DR rows per sweep of the threads),
// at element lc0 of that row.
template <typename T, bool KC, int R, int VEC, int NT>
struct Tile {
  static constexpr int ESZ = int(sizeof(T));
  static constexpr int BK = kSlab / ESZ;
  static constexpr int PITCH = tile_pitch<KC, R, ESZ>();     // LDS row pitch (bytes)
  static constexpr int RUN = KC ? BK : R;                   // elements per LDS row
  static constexpr int RUNV = RUN / VEC;                    // vectors per LDS row
  static constexpr int DR = NT / RUNV;                      // LDS rows per sweep
  static constexpr int NV = R * BK / VEC / NT;              // loads per thread
  static_assert(NV >= 1 && NT % RUNV == 0 && R * BK % (VEC * NT) == 0, "tile does not split over the threads");
  using V = typename VecT<VEC * ESZ>::type;
  union U {
    V v;
    T e[VEC];
  };
  U r[NV];
  int lr0, lc0;
  uint32_t voff0;  // byte offset of load 0 from the tile origin
  uint32_t vstep;  // bytes between consecutive loads (uniform)

  __device__ __forceinline__ void init(int64_t s_row, int64_t s_k) {
    lr0 = int(threadIdx.x) / RUNV;
    lc0 = (int(threadIdx.x) % RUNV) * VEC;
    const int64_t row = KC ? lr0 : lc0, k = KC ? lc0 : lr0;
    voff0 = uint32_t((row * s_row + k * s_k) * ESZ);
    vstep = uint32_t(int64_t(DR) * (KC ? s_row : s_k) * ESZ);
  }

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int rows_left, int k_left) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int lr = lr0 + i * DR;
      const int row = KC ? lr : lc0, k = KC ? lc0 : lr;
      const uint32_t off = (row < rows_left && k < k_left) ? voff0 + uint32_t(i) * vstep : kOob;
      r[i].v = buf_load<VEC * ESZ>(rs, off);
    }
  }

  // zero every element with t > s (s along the tile rows, t along K)
  __device__ __forceinline__ void mask_causal(int64_t s0, int64_t t0, const FastDiv &ds, const FastDiv &dt, int m0,
                                              int k0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int lr = lr0 + i * DR;
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const uint32_t row = KC ? lr : lc0 + u, k = KC ? lc0 + u : lr;
        const uint32_t mr = m0 + row, kr = k0 + k;
        const int64_t sg = s0 + (mr - fd_div(mr, ds) * ds.d);
        const int64_t tg = t0 + (kr - fd_div(kr, dt) * dt.d);
        if (tg > sg) r[i].e[u] = T(0);
      }
    }
  }

  __device__ __forceinline__ void store(char *lds) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) *reinterpret_cast<V *>(lds + (lr0 + i * DR) * PITCH + lc0 * ESZ) = r[i].v;
  }
};

// Fragment readers --------------------------------------------------------
// bf16, K-contiguous tile: 8 K values of row `row`, K chunk `kc` (16 wide).
__device__ __forceinline__ uint4 frag_bf16_kc(const char *lds, int row, int kc, int lhalf) {
  return *reinterpret_cast<const uint4 *>(lds + row * kPitchKC + kc * 32 + lhalf * 16);
}

// bf16, M/N-contiguous tile [BK][R]: the same fragment through two
// transposing reads.  Lane s of each 16-lane group names the 4-element row
// piece at K row k0 + (s>>2), columns n0 + 4*(s&3); the read hands lane j of
// the group K rows k0..k0+3 of column n0 + j.
template <int PITCH>
__device__ __forceinline__ uint4 frag_bf16_rc(const char *lds, int col0, int kc, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int n = col0 + 16 * (g & 1) + 4 * (s & 3);
  const int kb = kc * 16 + 8 * (g >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) i16x4 *lds_v4;
  char *p0 = const_cast<char *>(lds) + kb * PITCH + n * 2;
  // C-style casts lower to an address-space cast from the generic pointer
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p0 + 4 * PITCH));
  uint4 r;
  __builtin_memcpy(&r.x, &lo, 8);
  __builtin_memcpy(&r.z, &hi, 8);
  return r;
}

// fp32, K-contiguous tile: K values 8*kc + 4*lhalf + 0..3 of row `row`.
__device__ __forceinline__ uint4 frag_f32_kc(const char *lds, int row, int kc, int lhalf) {
  return *reinterpret_cast<const uint4 *>(lds + row * kPitchKC + kc * 32 + lhalf * 16);
}

// fp32, M/N-contiguous tile [BK][R]: the same four K values of column `col`.
template <int PITCH>
__device__ __forceinline__ uint4 frag_f32_rc(const char *lds, int col, int kc, int lhalf) {
  const char *p = lds + (8 * kc + 4 * lhalf) * PITCH + col * 4;
  uint4 r;
  r.x = *reinterpret_cast<const uint32_t *>(p);
  r.y = *reinterpret_cast<const uint32_t *>(p + PITCH);
  r.z = *reinterpret_cast<const uint32_t *>(p + 2 * PITCH);
  r.w = *reinterpret_cast<const uint32_t *>(p + 3 * PITCH);
  return r;
}

template <typename T>
struct Mma;
template <>
struct Mma<uint16_t> {
  // one 16-wide K chunk
  __device__ __forceinline__ static void run(f32x16 &acc, const uint4 &a, const uint4 &b) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
};
template <>
struct Mma<float> {
  // one 8-wide K chunk: lane half h holds K = 4h + i for MFMA i, in both
  // operands alike, so the four MFMAs together cover the chunk
  __device__ __forceinline__ static void run(f32x16 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// One K chunk over a wavefront's TM x TN accumulators.  For fp32 the four
// MFMAs of a chunk go round the accumulators (sub-step x of every
// accumulator before sub-step x + 1 of any), so consecutive MFMAs do not wait
// on each other's results; each accumulator still adds its products in the
// same order.
template <typename T, int TM, int TN>
__device__ __forceinline__ void mma_chunk(f32x16 (&acc)[TM][TN], const uint4 *a, const uint4 *b) {
  if constexpr (sizeof(T) == 4) {
    auto part = [](const uint4 &v, int x) { return __uint_as_float(x == 0 ? v.x : x == 1 ? v.y : x == 2 ? v.z : v.w); };
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(part(a[i], x), part(b[j], x), acc[i][j], 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mma<T>::run(acc[i][j], a[i], b[j]);
  }
}

// workgroup -> (tile row, tile column, batch index, output key).  Where
// neighbouring tiles share operand panels, the numbering gives each XCD a
// contiguous run of tiles.  Dispatch deals workgroups round-robin to the 8
// XCDs, so XCD x runs workgroups x, x + 8, ...: q + (x < r) of them for a
// grid of G = 8 q + r.  With `remap` the i-th of them takes logical tile
// x q + min(x, r) + i, which numbers each XCD's workgroups as one contiguous
// range and covers 0 .. G-1 once for any G.
__device__ __forceinline__ int64_t logical_tile(bool remap) {
  int64_t w = blockIdx.x;
  if (remap) {
    const int64_t G = gridDim.x, q = G >> 3, r = G & 7, x = w & 7;
    w = x * q + (x < r ? x : r) + (w >> 3);
  }
  return w;
}

__device__ __forceinline__ void decode_tile(const ContractArgs &p, int64_t w, int &tm, int &tn, int &bt,
                                            int64_t &key) {
  if (p.group_m) {
    // Tiles of all output keys form one grid of M panels x N panels, walked
    // column-major in groups of group_m M panels: the tiles that run
    // together (a contiguous range on each XCD) cover a compact block of
    // panels, so their operand slices are shared through L2.
    const int64_t Mp = int64_t(p.km) * p.tiles_m, Np = int64_t(p.kn) * p.tiles_n;
    const int64_t per_group = int64_t(p.group_m) * Np;
    const int64_t g = w / per_group, r = w - g * per_group;
    const int64_t rows = Mp - g * p.group_m < p.group_m ? Mp - g * p.group_m : p.group_m;
    const int64_t pm = g * p.group_m + r % rows, pn = r / rows;
    key = (pm / p.tiles_m) * p.kn + pn / p.tiles_n;
    tm = int(pm % p.tiles_m);
    tn = int(pn % p.tiles_n);
    bt = 0;
  } else {
    tn = int(w % p.tiles_n);
    w /= p.tiles_n;
    tm = int(w % p.tiles_m);
    w /= p.tiles_m;
    bt = int(w % p.batch);
    key = w / p.batch;
  }
}

// Epilogue: scale, causal mask, convert, store the TM x TN fragments of one
// wavefront (fragment element v of lane l: row 8*(v/4) + 4*(l/32) + v%4,
// column l%32).  m0 / n0: tile origin plus the wavefront's offset.
template <int OUT_BF16, int TM, int TN>
__device__ __forceinline__ void store_tile_plain(const ContractArgs &p, const f32x16 (&acc)[TM][TN], int64_t out_id,
                                             int bt, int64_t key, int64_t ks, int m0, int n0, int lane) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  char *Cb = reinterpret_cast<char *>(p.C);
  const int64_t cbase = out_id * p.beC + int64_t(bt) * p.sCb;
  int64_t kt_out = 0;
  if (p.causal_out) kt_out = (key / p.ct_w) % p.ct_k;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + i * 32 + (v >> 2) * 8 + lhalf * 4 + (v & 3);
        const int n = n0 + j * 32 + lrow;
        if (m < p.M && n < p.N) {
          float x = p.alpha * acc[i][j][v];
          if (p.causal_out) {
            const int64_t sg = ks * p.e_s + (uint32_t(m) - fd_div(uint32_t(m), p.div_s) * p.div_s.d);
            const int64_t tg = kt_out * p.e_t + (uint32_t(n) - fd_div(uint32_t(n), p.div_t) * p.div_t.d);
            if (tg > sg) x = 0.0f;
          }
          const int64_t off = cbase + int64_t(m) * p.sCm + n;
          if (OUT_BF16)
            reinterpret_cast<uint16_t *>(Cb)[off] = f32_to_bf16(x);
          else
            reinterpret_cast<float *>(Cb)[off] = x;
        }
      }
}

// MUL_PLUS epilogue (XDT 0: f32 addend, 1: bf16): out = alpha * acc + X,
// X laid out as C.  Loads and stores are buffer operations on the output
// block: element (m, n) of the wavefront's fragments sits at a per-lane
// base plus a row term that is a compile-time row times the row stride, and
// elements outside the block get an offset past its end, which the hardware
// reads as 0 and drops on store -- no branches, 32-bit offsets.  The
// addends of fragment f + 1 are loaded before fragment f is stored: a load
// waits for the stores issued before it (vector memory operations complete
// in issue order), so a load between every two stores would make each
// addend a full round trip.  Without PREFETCH (kernels with no registers to
// spare) each fragment's addends are loaded just before its stores.
template <int OUT_BF16, int TM, int TN, int XDT, bool PREFETCH>
__device__ __forceinline__ void store_tile_plus(const ContractArgs &p, const f32x16 (&acc)[TM][TN], int64_t out_id,
                                                int bt, int m0, int n0, int lane) {
  constexpr int XSZ = XDT ? 2 : 4, OSZ = OUT_BF16 ? 2 : 4;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t cbase = out_id * p.beC + int64_t(bt) * p.sCb;
  const int64_t left = p.beC - int64_t(bt) * p.sCb;  // elements from cbase to the block's end
  const __amdgpu_buffer_rsrc_t rx = tile_rsrc(static_cast<const char *>(p.X) + cbase * XSZ, left * XSZ);
  const __amdgpu_buffer_rsrc_t rc = tile_rsrc(static_cast<char *>(p.C) + cbase * OSZ, left * OSZ);
  const int rows_left = p.M - (m0 + lhalf * 4);                    // valid rows from this lane's first
  const uint32_t lane_base = uint32_t((m0 + lhalf * 4) * p.sCm + n0 + lrow);
  bool col_ok[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) col_ok[j] = n0 + j * 32 + lrow < p.N;
  auto elem = [&](int i, int j, int v) {  // element offset inside the block, or past its end
    const int r = i * 32 + (v >> 2) * 8 + (v & 3);
    return (r < rows_left && col_ok[j]) ? lane_base + uint32_t(r * p.sCm + j * 32) : (kOob / 4);
  };
  float xs[2][16];
  auto load_frag = [&](int f, float (&dst)[16]) {
    const int i = f / TN, j = f % TN;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const uint32_t e = elem(i, j, v);
      if constexpr (XDT) dst[v] = bf16_to_f32(buf_load<2>(rx, e * 2));
      else dst[v] = __uint_as_float(buf_load<4>(rx, e * 4));
    }
  };
  if constexpr (PREFETCH) load_frag(0, xs[0]);
#pragma unroll
  for (int f = 0; f < TM * TN; ++f) {
    if constexpr (PREFETCH) {
      if (f + 1 < TM * TN) load_frag(f + 1, xs[(f + 1) & 1]);
    } else {
      load_frag(f, xs[f & 1]);
    }
    const int i = f / TN, j = f % TN;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x = p.alpha * acc[i][j][v] + xs[f & 1][v];
      const uint32_t e = elem(i, j, v);
      if constexpr (OUT_BF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), rc, int(e * 2), 0, 0);
      else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rc, int(e * 4), 0, 0);
    }
  }
}

// Epilogue of the LDS-DMA kernels, whose MFMAs take the B fragment as the
// first operand: the accumulator of fragment (i, j) then holds the tile
// transposed, element v of lane l at row 32 i + l % 32 and column
// 32 j + 8 (v / 4) + 4 (l / 32) + v % 4, so each group of four values is
// four consecutive columns of one row.  With rows and N a multiple of 4
// elements a group leaves as one 8-byte (bf16) or 16-byte (f32) buffer
// store, and a MUL_PLUS addend group arrives as one load of the same width:
// a quarter of the memory instructions of element stores.  Rows past M and
// groups past N take an offset past the block's end (nothing written, zeros
// read).  Other layouts store element by element.
// EPI: 0 scale (and the causal output mask), 1 / 2 add an f32 / bf16 addend
// laid out as C (MUL_PLUS); the addends of fragment f + 1 are loaded before
// fragment f is stored (vector memory operations complete in issue order,
// so a load issued after a store waits for it).
template <int OUT_BF16, int TM, int TN, int EPI>
__device__ __forceinline__ void store_tile_t(const ContractArgs &p, const f32x16 (&acc)[TM][TN], int64_t out_id,
                                             int bt, int64_t key, int64_t ks, int m0, int n0, int lane) {
  constexpr int OSZ = OUT_BF16 ? 2 : 4, XSZ = EPI == 2 ? 2 : 4;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t cbase = out_id * p.beC + int64_t(bt) * p.sCb;
  const int64_t left = p.beC - int64_t(bt) * p.sCb;  // elements from cbase to the block's end
  int64_t kt_out = 0;
  if (EPI == 0 && p.causal_out) kt_out = (key / p.ct_w) % p.ct_k;
  auto masked = [&](float x, int m, int n) {
    if (EPI == 0 && p.causal_out) {
      const int64_t sg = ks * p.e_s + (uint32_t(m) - fd_div(uint32_t(m), p.div_s) * p.div_s.d);
      const int64_t tg = kt_out * p.e_t + (uint32_t(n) - fd_div(uint32_t(n), p.div_t) * p.div_t.d);
      if (tg > sg) return 0.0f;
    }
    return x;
  };
  if (((p.sCm | int64_t(p.N) | cbase) & 3) == 0) {
    const __amdgpu_buffer_rsrc_t rc = tile_rsrc(static_cast<char *>(p.C) + cbase * OSZ, left * OSZ);
    __amdgpu_buffer_rsrc_t rx = rc;
    if constexpr (EPI != 0) rx = tile_rsrc(static_cast<const char *>(p.X) + cbase * XSZ, left * XSZ);
    // element offset of group g of fragment (i, j) inside the block, and
    // whether it exists
    auto goff = [&](int i, int j, int g, bool &ok) {
      const int m = m0 + 32 * i + lrow, n = n0 + 32 * j + 8 * g + 4 * lhalf;
      ok = m < p.M && n < p.N;
      return uint32_t(int64_t(m) * p.sCm + n);
    };
    float xs[2][16];
    auto load_frag = [&](int f, float (&dst)[16]) {
      const int i = f / TN, j = f % TN;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bool ok;
        const uint32_t e = goff(i, j, g, ok);
        if constexpr (EPI == 1) {
          const uint4 v = buf_load<16>(rx, ok ? e * 4 : kOob);
          dst[4 * g] = __uint_as_float(v.x);
          dst[4 * g + 1] = __uint_as_float(v.y);
          dst[4 * g + 2] = __uint_as_float(v.z);
          dst[4 * g + 3] = __uint_as_float(v.w);
        } else {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rx, int(ok ? e * 2 : kOob), 0, 0);
          dst[4 * g] = __uint_as_float(v.x << 16);
          dst[4 * g + 1] = __uint_as_float(v.x & 0xffff0000u);
          dst[4 * g + 2] = __uint_as_float(v.y << 16);
          dst[4 * g + 3] = __uint_as_float(v.y & 0xffff0000u);
        }
      }
    };
    if constexpr (EPI != 0) load_frag(0, xs[0]);
#pragma unroll
    for (int f = 0; f < TM * TN; ++f) {
      const int i = f / TN, j = f % TN;
      if constexpr (EPI != 0) {
        if (f + 1 < TM * TN) load_frag(f + 1, xs[(f + 1) & 1]);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bool ok;
        const uint32_t e = goff(i, j, g, ok);
        float x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[c] = p.alpha * acc[i][j][4 * g + c];
          if constexpr (EPI != 0) x[c] += xs[f & 1][4 * g + c];
          else x[c] = masked(x[c], m0 + 32 * i + lrow, n0 + 32 * j + 8 * g + 4 * lhalf + c);
        }
        if constexpr (OUT_BF16) {
          const u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          __builtin_amdgcn_raw_buffer_store_b64(v, rc, int(ok ? e * 2 : kOob), 0, 0);
        } else {
          const u32x4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                           __float_as_uint(x[3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, rc, int(ok ? e * 4 : kOob), 0, 0);
        }
      }
    }
  } else {
    char *Cb = reinterpret_cast<char *>(p.C);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 32 * i + lrow, n = n0 + 32 * j + 8 * (v >> 2) + 4 * lhalf + (v & 3);
          if (m < p.M && n < p.N) {
            const int64_t off = cbase + int64_t(m) * p.sCm + n;
            float x = p.alpha * acc[i][j][v];
            if constexpr (EPI == 1) x += reinterpret_cast<const float *>(p.X)[off];
            else if constexpr (EPI == 2) x += bf16_to_f32(reinterpret_cast<const uint16_t *>(p.X)[off]);
            else x = masked(x, m, n);
            if (OUT_BF16)
              reinterpret_cast<uint16_t *>(Cb)[off] = f32_to_bf16(x);
            else
              reinterpret_cast<float *>(Cb)[off] = x;
          }
        }
  }
}

// The epilogue, with the MUL_PLUS addend's dtype fixed per instantiation so
// that each version unrolls completely (accumulators stay in registers).
template <int OUT_BF16, int TM, int TN>
__device__ __forceinline__ void store_tile(const ContractArgs &p, const f32x16 (&acc)[TM][TN], int64_t out_id,
                                           int bt, int64_t key, int64_t ks, int m0, int n0, int lane) {
  if (p.epi == 1) {
    if (p.x_bf16) store_tile_plus<OUT_BF16, TM, TN, 1, false>(p, acc, out_id, bt, m0, n0, lane);
    else store_tile_plus<OUT_BF16, TM, TN, 0, false>(p, acc, out_id, bt, m0, n0, lane);
  } else {
    store_tile_plain<OUT_BF16, TM, TN>(p, acc, out_id, bt, key, ks, m0, n0, lane);
  }
}

// Epilogue through LDS: the wavefronts write their scaled (and causally
// masked) fragments into a BM x BN tile in LDS, then the workgroup writes the
// tile out row by row in 16-byte vectors, so a store instruction covers whole
// row runs instead of one element per lane.  Rows are padded by 16 bytes so
// the fragment writes (32 lanes along a row, the other 32 four rows down)
// spread over the banks.  The caller guarantees that every row start is
// 16-byte aligned in the output block (elsewhere the fragments are stored
// directly: the LDS pass would buy nothing).
template <int OUT_BF16, int TM, int TN, int BM, int BN, int NT>
__device__ __forceinline__ void store_tile_lds(const ContractArgs &p, const f32x16 (&acc)[TM][TN], int64_t out_id,
                                               int bt, int64_t key, int64_t ks, int m0, int n0, int wm, int wn,
                                               int lane, char *smem) {
  constexpr int OSZ = OUT_BF16 ? 2 : 4;
  constexpr int PITCH = BN * OSZ + 16;
  constexpr int VE = 16 / OSZ;      // elements per 16-byte vector
  constexpr int VPR = BN / VE;      // vectors per tile row
  const int lrow = lane & 31, lhalf = lane >> 5;
  int64_t kt_out = 0;
  if (p.causal_out) kt_out = (key / p.ct_w) % p.ct_k;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ml = wm + i * 32 + (v >> 2) * 8 + lhalf * 4 + (v & 3);
        const int nl = wn + j * 32 + lrow;
        float x = p.alpha * acc[i][j][v];
        if (p.causal_out) {
          const int m = m0 + ml, n = n0 + nl;
          const int64_t sg = ks * p.e_s + (uint32_t(m) - fd_div(uint32_t(m), p.div_s) * p.div_s.d);
          const int64_t tg = kt_out * p.e_t + (uint32_t(n) - fd_div(uint32_t(n), p.div_t) * p.div_t.d);
          if (tg > sg) x = 0.0f;
        }
        if (OUT_BF16)
          *reinterpret_cast<uint16_t *>(smem + ml * PITCH + nl * 2) = f32_to_bf16(x);
        else
          *reinterpret_cast<float *>(smem + ml * PITCH + nl * 4) = x;
      }
  __syncthreads();
  char *Cb = reinterpret_cast<char *>(p.C);
  const int64_t cbase = out_id * p.beC + int64_t(bt) * p.sCb;
  for (int i = threadIdx.x; i < BM * VPR; i += NT) {
    const int r = i / VPR, cv = i - r * VPR;
    const int m = m0 + r, n = n0 + cv * VE;
    if (m >= p.M || n >= p.N) continue;
    const char *src = smem + r * PITCH + cv * 16;
    char *dst = Cb + (cbase + int64_t(m) * p.sCm + n) * OSZ;
    if (n + VE <= p.N) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
      for (int e = 0; e < p.N - n; ++e) {
        if (OUT_BF16) reinterpret_cast<uint16_t *>(dst)[e] = reinterpret_cast<const uint16_t *>(src)[e];
        else reinterpret_cast<float *>(dst)[e] = reinterpret_cast<const float *>(src)[e];
      }
    }
  }
}

#ifndef JAGG_LDS_EPILOGUE
#define JAGG_LDS_EPILOGUE 1
#endif
#ifndef JAGG_SHORT_WALK
#define JAGG_SHORT_WALK 1
#endif
constexpr bool kShortWalk = JAGG_SHORT_WALK;

// NSTG: LDS stages.  Two overlap the loads of step s+1 with step s; one
// (for walks of one or two steps, e.g. a score block with K = 128) halves the
// LDS so that twice as many workgroups share a CU and overlap each other.
// The one-stage kernel is bound by its output writes: it asks the compiler
// for a register allocation that lets four wavefronts share a SIMD (its LDS
// allows four workgroups per CU), which keeps more stores in flight than the
// three its default allocation allows.
template <typename T, int OUT_BF16, bool A_KC, bool B_KC, int VA, int VB, int BM, int BN, int WAVES_M, int WAVES_N,
          bool MASK, int NSTG>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64)
__attribute__((amdgpu_waves_per_eu(NSTG == 1 ? 4 : 1))) void contract_kernel(const ContractArgs p) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int ESZ = int(sizeof(T));
  constexpr int BK = kSlab / ESZ;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KCH = ESZ == 2 ? BK / 16 : BK / 8;  // fragment chunks per K-tile
  using TA = Tile<T, A_KC, BM, VA, NT>;
  using TB = Tile<T, B_KC, BN, VB, NT>;
  constexpr int A_BYTES = tile_bytes<A_KC, BM, ESZ>(), B_BYTES = tile_bytes<B_KC, BN, ESZ>();
  constexpr int STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[NSTG * STAGE];

  int tn, tm, bt;
  int64_t key;
  decode_tile(p, logical_tile(p.remap), tm, tn, bt, key);

  const int32_t cnt = p.counts[key];
  if (cnt == 0) return;  // output tuple absent (causal); uniform, before any barrier
  const int32_t *ents = p.list + key * int64_t(p.per_key) * p.ent_w;

  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = (p.K + BK - 1) / BK;
  const int steps = cnt * KT;
  const int64_t a_org = int64_t(bt) * p.sAb + int64_t(m0) * p.sAm;
  const int64_t b_org = int64_t(bt) * p.sBb + int64_t(n0) * p.sBn;
  int64_t ks = 0;
  if (p.causal_out || p.causal_red) ks = (key / p.cs_w) % p.cs_k;

  // one register set per operand: the global loads of step s+1 are issued
  // while step s computes
  TA ta[1];
  TB tb[1];
  ta[0].init(p.sAm, p.sAk);
  tb[0].init(p.sBn, p.sBk);
  // the walk over (joined tuple, K-tile): the next load's position and tuple
  // ids are kept ahead, so a tuple's ids are read one step before they are
  // used and no step waits on a scalar load
  int le = 0, lkt = 0;  // position of the next load
  int64_t la = ents[p.a_slot], lb = ents[p.b_slot];
  // ids of the tuple after the current one (the last one's, at the end)
  int64_t la_n = ents[(cnt > 1 ? 1 : 0) * p.ent_w + p.a_slot], lb_n = ents[(cnt > 1 ? 1 : 0) * p.ent_w + p.b_slot];
  int pe = 0, pk0 = 0;  // position of the load in flight (for the causal mask)
  // live = false: a step past the walk's end, loaded from an empty buffer
  // (every lane reads zeros, no memory is touched)
  auto load_next = [&](TA &xa, TB &xb, bool live = true) {
    const int k0 = lkt * BK;
    pe = le;
    pk0 = k0;
    const int64_t ao = a_org + int64_t(k0) * p.sAk, bo = b_org + int64_t(k0) * p.sBk;
    const T *pa = reinterpret_cast<const T *>(p.A) + la * p.beA + ao;
    const T *pb = reinterpret_cast<const T *>(p.B) + lb * p.beB + bo;
    xa.load(tile_rsrc(pa, live ? (p.beA - ao) * ESZ : 0), p.M - m0, p.K - k0);
    xb.load(tile_rsrc(pb, live ? (p.beB - bo) * ESZ : 0), p.N - n0, p.K - k0);
    // Branch-free step of the walk: the next tuple's ids are read one call
    // ahead and taken where the current tuple's K walk ends, by arithmetic on
    // the 0/1 wrap flag.  A branch here splits the loop body, and the
    // accumulators are then copied out of and back into AGPRs on every step.
    const int wrap = int(lkt + 1 == KT);
    lkt = (lkt + 1) * (1 - wrap);
    le += wrap;
    la += int64_t(wrap) * (la_n - la);
    lb += int64_t(wrap) * (lb_n - lb);
    const int e_n = min(le + 1, cnt - 1);
    la_n = ents[e_n * p.ent_w + p.a_slot];
    lb_n = ents[e_n * p.ent_w + p.b_slot];
  };
  // causal pair with t reduced: zero A where t > s, on the diagonal block only;
  // applied just before the LDS store so the loads stay in flight meanwhile
  auto mask_step = [&](TA &xa) {
    if (MASK && p.causal_red) {
      const int64_t aid = ents[pe * p.ent_w + p.a_slot];
      const int64_t kt_blk = (aid / p.ct_w) % p.ct_k;
      if (kt_blk == ks) xa.mask_causal(ks * p.e_s, kt_blk * p.e_t, p.div_s, p.div_t, m0, pk0);
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave / WAVES_N) * WTM, wn = (wave % WAVES_N) * WTN;
  const int lrow = lane & 31, lhalf = lane >> 5;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto compute = [&](const char *As) {
    const char *Bs = As + A_BYTES;
    __builtin_amdgcn_iglp_opt(0);  // let the scheduler interleave LDS reads with MFMAs
    // fragments of K chunk kc+1 are read while the MFMAs of chunk kc run
    uint4 af[2][TM], bfr[2][TN];
    auto read_frags = [&](int kc, uint4 *a, uint4 *b) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (ESZ == 2) {
          if constexpr (A_KC) a[i] = frag_bf16_kc(As, wm + i * 32 + lrow, kc, lhalf);
          else a[i] = frag_bf16_rc<TA::PITCH>(As, wm + i * 32, kc, lane);
        } else {
          if constexpr (A_KC) a[i] = frag_f32_kc(As, wm + i * 32 + lrow, kc, lhalf);
          else a[i] = frag_f32_rc<TA::PITCH>(As, wm + i * 32 + lrow, kc, lhalf);
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (ESZ == 2) {
          if constexpr (B_KC) b[j] = frag_bf16_kc(Bs, wn + j * 32 + lrow, kc, lhalf);
          else b[j] = frag_bf16_rc<TB::PITCH>(Bs, wn + j * 32, kc, lane);
        } else {
          if constexpr (B_KC) b[j] = frag_f32_kc(Bs, wn + j * 32 + lrow, kc, lhalf);
          else b[j] = frag_f32_rc<TB::PITCH>(Bs, wn + j * 32 + lrow, kc, lhalf);
        }
      }
    };
    if constexpr (TM * TN <= 8) {
      read_frags(0, af[0], bfr[0]);
#pragma unroll
      for (int kc = 0; kc < KCH; ++kc) {
        if (kc + 1 < KCH) read_frags(kc + 1, af[(kc + 1) & 1], bfr[(kc + 1) & 1]);
        mma_chunk<T, TM, TN>(acc, af[kc & 1], bfr[kc & 1]);
      }
    } else {
      // 16 MFMAs per chunk give the reads of the next chunk room without a
      // second fragment set
#pragma unroll
      for (int kc = 0; kc < KCH; ++kc) {
        read_frags(kc, af[0], bfr[0]);
        mma_chunk<T, TM, TN>(acc, af[0], bfr[0]);
      }
    }
  };
  auto store_step = [&](TA &xa, TB &xb, char *lds) {
    mask_step(xa);
    xa.store(lds);
    xb.store(lds + A_BYTES);
  };

  // fp32 operands with two stages and no causal mask on the reduced letter
  // keep two register sets: step s+2's loads are issued before step s
  // computes, so a load has two steps of MFMA work to land instead of one
  // (fp32 operands are twice the bytes per FLOP of bf16, and a large A
  // streams from HBM rather than from the Infinity Cache)
  constexpr bool PF2 = NSTG == 2 && !MASK && ESZ == 4;
  if constexpr (NSTG == 1) {
    for (int s = 0; s < steps; ++s) {
      load_next(ta[0], tb[0]);
      store_step(ta[0], tb[0], smem);
      __syncthreads();
      compute(smem);
      __syncthreads();
    }
  } else if constexpr (PF2) {
    // step j is loaded into set j % 2; every iteration issues the same loads
    // (past the walk's end from an empty buffer) and stores one set, so the
    // waits the compiler places before a store cover only the older set
    TA ta1;
    TB tb1;
    ta1.init(p.sAm, p.sAk);
    tb1.init(p.sBn, p.sBk);
    load_next(ta[0], tb[0]);
    load_next(ta1, tb1, steps > 1);
    store_step(ta[0], tb[0], smem);
    __syncthreads();
    // iteration s (parity P): the set of parity P is free (step s is in
    // stage P); it takes step s+2's loads while stage P computes, then the
    // other set (step s+1) goes to stage P ^ 1, last read in iteration s-1
    auto iter = [&](auto par, int s) {
      constexpr int P = decltype(par)::value;
      TA &fa = P ? ta1 : ta[0];
      TB &fb = P ? tb1 : tb[0];
      TA &na = P ? ta[0] : ta1;
      TB &nb = P ? tb[0] : tb1;
      load_next(fa, fb, s + 2 < steps);
      compute(smem + P * STAGE);
      store_step(na, nb, smem + (P ^ 1) * STAGE);
      __syncthreads();
    };
    for (int s = 0; s < steps; s += 2) {
      iter(std::integral_constant<int, 0>{}, s);
      if (s + 1 < steps) iter(std::integral_constant<int, 1>{}, s + 1);
    }
  } else {
    load_next(ta[0], tb[0]);
    store_step(ta[0], tb[0], smem);
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
      const int cur = s & 1;
      if (s + 1 < steps) load_next(ta[0], tb[0]);
      compute(smem + cur * STAGE);
      if (s + 1 < steps) store_step(ta[0], tb[0], smem + (cur ^ 1) * STAGE);
      __syncthreads();
    }
  }

  if constexpr (JAGG_LDS_EPILOGUE && BM * (BN * (OUT_BF16 ? 2 : 4) + 16) <= NSTG * STAGE) {
    // the loop's last barrier has passed: the stages are free.  The LDS pass
    // pays only where output rows start 16-byte aligned (row stores); else
    // the fragments go out directly (the test is uniform over the workgroup)
    constexpr int VE = OUT_BF16 ? 8 : 4;
    if ((ents[0] * p.beC + int64_t(bt) * p.sCb) % VE == 0 && p.sCm % VE == 0 && p.epi == 0) {
      store_tile_lds<OUT_BF16, TM, TN, BM, BN, NT>(p, acc, ents[0], bt, key, ks, m0, n0, wm, wn, lane, smem);
      return;
    }
  }
  store_tile<OUT_BF16, TM, TN>(p, acc, ents[0], bt, key, ks, m0 + wm, n0 + wn, lane);
}

template <typename T, int OB, bool AK, bool BKC, int VA, int VB, int BM, int BN, int WM, int WN, bool MASK = false,
          int NSTG = 2>
static hipError_t launch_tile(const ContractArgs &a, hipStream_t st) {
  ContractArgs b = a;
  b.tiles_m = (a.M + BM - 1) / BM;
  b.tiles_n = (a.N + BN - 1) / BN;
  const int64_t grid = b.n_keys * b.batch * int64_t(b.tiles_m) * b.tiles_n;
  hipLaunchKernelGGL((contract_kernel<T, OB, AK, BKC, VA, VB, BM, BN, WM, WN, MASK, NSTG>), dim3(unsigned(grid)),
                     dim3(WM * WN * 64), 0, st, b);
  return hipGetLastError();
}

// walks of at most two K-steps per output tile with an fp32 output take the
// one-stage kernel (score blocks with K = 128: 622 -> 535 us for 4x32x2048^2;
// a bf16 output does better with two stages and the LDS epilogue)
template <typename T>
inline bool short_walk(const ContractArgs &a) {
  constexpr int BK = kSlab / int(sizeof(T));
  return kShortWalk && int64_t(a.per_key) * ((a.K + BK - 1) / BK) <= 2;
}

// big: 256x256 tiles, 8 wavefronts of 128x64; small: 128x128, 4 of 64x64, or
// 128x64 (4 of 64x32) where 64-wide tiles pad N less than 128-wide ones (e.g.
// N = 167: three 64-wide tiles keep 87% of the MFMA work useful, two
// 128-wide ones 65%).
template <typename T, int OB, bool AK, bool BKC>
static hipError_t launch_layout(const ContractArgs &a, int va, int vb, bool big, hipStream_t st) {
  constexpr int F = 16 / int(sizeof(T));
  if (a.causal_red) {
    // the masked variant: 128x128 tiles, 16-byte loads only
    if (va == F && vb == F && !big) return launch_tile<T, OB, AK, BKC, F, F, 128, 128, 2, 2, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (va == F && vb == F) {
    if (big) return launch_tile<T, OB, AK, BKC, F, F, 256, 256, 2, 4>(a, st);
    if ((a.N + 63) / 64 * 64 < (a.N + 127) / 128 * 128) return launch_tile<T, OB, AK, BKC, F, F, 128, 64, 2, 2>(a, st);
    if (OB == 0 && short_walk<T>(a)) return launch_tile<T, OB, AK, BKC, F, F, 128, 128, 2, 2, false, 1>(a, st);
    return launch_tile<T, OB, AK, BKC, F, F, 128, 128, 2, 2>(a, st);
  }
  if (va == F && vb == 1) {
    if ((a.N + 63) / 64 * 64 < (a.N + 127) / 128 * 128) return launch_tile<T, OB, AK, BKC, F, 1, 128, 64, 2, 2>(a, st);
    return launch_tile<T, OB, AK, BKC, F, 1, 128, 128, 2, 2>(a, st);
  }
  if (va == 1 && vb == F) return launch_tile<T, OB, AK, BKC, 1, F, 128, 128, 2, 2>(a, st);
  if (va == 1 && vb == 1) return launch_tile<T, OB, AK, BKC, 1, 1, 128, 128, 2, 2>(a, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_typed(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                               hipStream_t st) {
#define JAGG_LAYOUTS(OB)                                                              \
  if (a_kc && b_kc) return launch_layout<T, OB, true, true>(a, va, vb, big, st);      \
  if (a_kc && !b_kc) return launch_layout<T, OB, true, false>(a, va, vb, big, st);    \
  if (!a_kc && b_kc) return launch_layout<T, OB, false, true>(a, va, vb, big, st);    \
  return launch_layout<T, OB, false, false>(a, va, vb, big, st);
  if (out_bf16) {
    JAGG_LAYOUTS(1)
  } else {
    JAGG_LAYOUTS(0)
  }
#undef JAGG_LAYOUTS
}

}  // namespace jagg
