// jagg_internal.h -- argument blocks shared by the host planner (abi.cpp)
// and the HIP kernels.  Every block is passed to its kernel by value.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace jagg {

constexpr int kMaxLetters = 8;   // per relation
constexpr int64_t kMaxRelationElems = int64_t(1) << 36;  // elements of one relation
constexpr int kMaxIn = 3;        // inputs per spec
constexpr int kMaxDims = 24;     // relayout dims after splitting (<= 3 per letter)
constexpr int kMaxChk = 8;       // relayout letters whose range must be checked
constexpr int kMaxChain = 3;     // dims per run chain of the LDS-transposing relayout
constexpr int kMaxLdsOuter = 8;  // outer (box) dims of the LDS-transposing relayout
constexpr int kMaxIv = 32;       // intervals of one interval-blocked letter
constexpr int kIvPool = 192;     // interval bounds one interval relayout carries

// Unsigned 32-bit division by a run-time invariant d >= 1 through a
// multiply-high, after Granlund and Montgomery, "Division by Invariant
// Integers using Multiplication" (PLDI 1994), Fig. 4.1:
//   l = ceil(log2 d); m = floor(2^32 (2^l - d) / d) + 1;
//   t = mulhi(m, n); q = (t + ((n - t) >> min(l,1))) >> max(l-1, 0).
// Exact for every 32-bit n.
struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

__host__ __device__ inline uint32_t fd_div(uint32_t n, const FastDiv &f) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t t = __umulhi(f.m, n);
#else
  uint32_t t = uint32_t((uint64_t(f.m) * n) >> 32);
#endif
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// ---------------------------------------------------------------- relayout
// The copy is a strided walk over "dims": every letter's index x is split
// into digits (block coordinate and in-block offset, each possibly split
// again where the source and destination block extents nest), so that both
// the source and the destination offset are affine in the digits.  Dims are
// grouped into lane dims (decoded once per thread) and tile dims (decoded
// once per workgroup).  A letter whose blocks do not nest ("irregular") has
// its source offset computed from x by division.
struct RelayoutDim {
  int64_t ext;       // number of digit values
  int64_t src;       // source stride per digit (elements)
  int64_t dst;       // destination stride per digit (elements)
  int32_t chk;       // checked letter slot this digit feeds, or -1
  int64_t xs;        // contribution of one digit step to that letter's index
  FastDiv div;       // division by ext (tile dims)
};

struct RelayoutArgs {
  const void *src;
  void *dst;
  int n_tile;                  // tile dims, outermost first
  RelayoutDim tile[kMaxDims];
  int n_lane;                  // lane dims, innermost (vectorised) first
  RelayoutDim lane[kMaxDims];
  int64_t n_tiles;
  int32_t lanes;               // threads that carry a vector
  int n_chk;
  int64_t read_lim[kMaxChk];   // x < read_lim: the element exists in the source
  int64_t write_lim[kMaxChk];  // x < write_lim: the destination slot exists
  int32_t irr[kMaxChk];        // 1 when the slot's letter is irregular
  FastDiv irr_div[kMaxChk];    // division by the source block extent
  int64_t irr_K[kMaxChk];      // source tuple stride of the letter (elements)
  int64_t irr_E[kMaxChk];      // source in-block stride of the letter
  // LDS transpose (lds != 0): the tile dims above are the outer loop; each
  // workgroup moves one box of lds_nv * 256 vectors of lds_v elements.  The
  // box is the shared innermost run (lds_inner elements) extended two ways:
  // by the source chain (dims continuing the source run, to lds_R vectors)
  // and by the destination chain (dims continuing the destination run, to
  // lds_Rd vectors).  LDS holds it as source runs of lds_pitch elements.
  int32_t lds;
  int32_t lds_nv;
  int32_t lds_v, lds_inner, lds_pitch;
  FastDiv lds_R, lds_Rd, lds_iv;  // vectors per source run / destination run / inner run
  int32_t n_cs, n_cd;             // dims of the source chain / destination chain
  FastDiv cs_div[kMaxChain], cd_div[kMaxChain];
  int64_t cs_dst[kMaxChain];      // destination stride of each source-chain dim
  int64_t cd_src[kMaxChain];      // source stride of each destination-chain dim
  int32_t lds_bytes;
};

// vec_bytes: 16, 8, 4 or 2; elem_bytes 2 or 4.
hipError_t launch_relayout(const RelayoutArgs &a, int vec_bytes, int elem_bytes, hipStream_t st);

// ---------------------------------------------------------------- interval relayout
// Copy between relations where some letter is blocked by a list of bounds
// (non-uniform intervals).  For each destination vector: decode the
// destination tuple and in-block coordinates, form each letter's global
// index x from the destination interval, write +0 where x falls in the
// block's padding, and otherwise find the source block of x (division for a
// uniform letter, a search of the bounds for an interval letter) and read
// the vector there.  Row form: a wave decodes the outer letters of a row
// (one block extent of the innermost destination letter) once and streams
// the row; vector form (short rows): a thread decodes each vector.
struct IvRelayoutDim {   // one letter, destination order
  FastDiv dk, de;        // destination block count, padded block extent
  int32_t d_bnd;         // pool offset of the destination bounds, -1 if uniform
  int32_t n;             // extent of the letter
  int32_t s_bnd;         // pool offset of the source bounds, -1 if uniform
  int32_t s_k;           // source block count
  FastDiv s_e;           // source padded block extent
  uint32_t s_tw;         // source offset of one block step (elements)
  uint32_t s_ew;         // source in-block stride (elements)
};

struct IvRelayoutArgs {
  const void *src;
  void *dst;
  int32_t r;
  IvRelayoutDim d[kMaxLetters];
  uint32_t n_vec;        // destination vectors
  FastDiv be_v;          // destination block size, in vectors
  int32_t v;             // elements per vector
  // row form (rows != 0): a row is one block extent of the innermost
  // destination letter; a wave decodes a row once and streams its vectors
  int32_t rows;
  uint32_t n_rows;
  FastDiv rows_pt;       // rows per destination tuple
  uint32_t row_vecs;     // vectors per row
  int32_t n_pool;
  int32_t pool[kIvPool];
};

// vec_bytes: 16, 8, 4 or 2 (a multiple of elem_bytes).
hipError_t launch_relayout_iv(const IvRelayoutArgs &a, int vec_bytes, hipStream_t st);

// ---------------------------------------------------------------- join
struct JoinArgs {
  int n_in;
  int n_out;                       // output letters
  int n_red;                       // reduced letters
  int32_t out_k[kMaxLetters];      // block counts, output letter order
  FastDiv out_div[kMaxLetters];
  int32_t red_k[26];               // block counts, reduced letters in first-appearance order
  FastDiv red_div[26];
  int64_t w_out[kMaxIn][kMaxLetters];  // tuple-id weight of each output letter's block coordinate
  int64_t w_red[kMaxIn][26];           // tuple-id weight of each reduced letter's block coordinate
  int32_t per_key;
  int64_t n_keys;
  // causal or segment pair: letter s / t located as (is_reduced, index);
  // causal keeps t-blocks starting before the s-block ends, seg keeps only
  // the t-block equal to the s-block
  int32_t causal, seg;
  int32_t s_red, s_idx, t_red, t_idx;
  int64_t e_s, e_t, n_s;
  int32_t *list;
  int32_t *counts;
};
hipError_t launch_join(const JoinArgs &a, hipStream_t st);

// ---------------------------------------------------------------- contraction
struct ContractArgs {
  const void *A;
  const void *B;
  void *C;
  const int32_t *list;
  const int32_t *counts;
  int32_t per_key;
  int32_t a_slot, b_slot;       // position of A / B tuple ids inside an entry (1 or 2)
  int64_t beA, beB, beC;        // block elements
  int32_t batch, M, N, K;       // flattened padded block extents
  int64_t sAb, sAm, sAk;
  int64_t sBb, sBn, sBk;
  int64_t sCb, sCm;             // C is contiguous along N
  float alpha;
  int32_t tiles_m, tiles_n;
  int64_t n_keys;
  // causal pair with both letters in the output (s innermost of M, t innermost of N)
  int32_t causal_out;
  // causal pair with s in the output (innermost of M) and t reduced (innermost of K of A)
  int32_t causal_red;
  int64_t cs_w, cs_k;           // kappa_s = (out_tuple / cs_w) % cs_k
  int64_t ct_w, ct_k;           // kappa_t = (tuple / ct_w) % ct_k  (out tuple, or A tuple when reduced)
  int32_t e_s, e_t;
  FastDiv div_s, div_t;         // division by e_s / e_t
  int32_t remap;                // renumber workgroups per XCD (tiles share operand panels)
  // grouped tile order over the global panel grid, when the output key is
  // (M-letter blocks) x (N-letter blocks) in that order and batch == 1:
  // km, kn = key blocks along M and N; group_m = M panels per group (0: off)
  int32_t km, kn, group_m;
  int32_t ent_w;                // join-list entry width (1 + inputs)
  // recompose map: 0 none; 1 add the addend X (laid out as C) to each
  // element; 2 SwiGLU: C = silu(A B) * (A B2), B2 laid out as B
  int32_t epi;
  const void *X;
  int32_t x_bf16;
  const void *B2;
  // split walk (split > 1, bf16 256 x 256 tiles, no recompose map): part q
  // of a tile walks steps [q steps / split, (q + 1) steps / split) of its
  // (joined tuple, K-step) walk and writes fp32 sums, laid out as C, at
  // part + q * part_stride; launch_split_sum then adds the parts in order,
  // scales by alpha and writes C.  n_tiles: tiles of one part.
  int32_t split;
  int64_t n_tiles;
  float *part;
  int64_t part_stride;
};
hipError_t launch_split_sum(const ContractArgs &a, int out_bf16, int64_t n_out, hipStream_t st);
// Independent contractions of one geometry run as one launch of the bf16
// 256 x 256 LDS-pipelined kernel: `common` holds the shared geometry, the
// arrays each problem's addresses.
constexpr int kMaxGroup = 4;
struct DmaGroupArgs {
  ContractArgs common;
  const void *A[kMaxGroup];
  const void *B[kMaxGroup];
  void *C[kMaxGroup];
  const int32_t *list[kMaxGroup];
  const int32_t *counts[kMaxGroup];
  const void *X[kMaxGroup];
  const void *B2[kMaxGroup];
  int32_t n;
  int64_t tiles;  // tiles of one problem (set by the launcher)
};
// Launches the group when the common form takes the 256 x 256 LDS-pipelined
// kernel (bf16, 16-byte vectors, no causal mask on the reduced letter);
// returns false, launching nothing, otherwise.
bool launch_contract_bf16_group(const DmaGroupArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st, hipError_t *err);
// out_bf16: 0 f32 / 1 bf16 output; a_kc / b_kc: operand contiguous along K;
// va / vb: vector width (elements) of global loads (16 bytes or one element);
// big: 256x256 tiles (8 wavefronts) instead of 128x128 (4 wavefronts);
// *which names the kernel that ran (for tracing).
hipError_t launch_contract_bf16(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st, const char **which);
hipError_t launch_contract_f32(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                               hipStream_t st, const char **which);

// ---------------------------------------------------------------- map / reduce
struct EwArgs {
  int n_in;
  const void *in[kMaxIn];
  int32_t in_dt[kMaxIn];        // 0 f32, 1 bf16
  void *out;
  int32_t out_dt;
  int32_t g;                    // jagg_g
  int32_t agg;                  // jagg_agg
  float alpha, beta, eps;
  const int32_t *list;
  const int32_t *counts;
  int32_t per_key;
  int64_t n_keys;
  // output block: letters in output order
  int r_out;
  int64_t e_out[kMaxLetters];
  int64_t n_out[kMaxLetters];   // extents (valid bound on kappa*e + c)
  int64_t k_out[kMaxLetters];   // block counts (decode kappa from the output tuple id)
  int64_t be_out;
  // reduced letters (reduce only)
  int n_red;
  int64_t e_red[kMaxLetters];
  int64_t n_red_ext[kMaxLetters];
  int64_t k_red[kMaxLetters];
  int64_t w_red0[kMaxLetters];  // tuple-id weight of the reduced letter in input 0
  // inputs: in-block stride of each output / reduced letter (0 = absent)
  int64_t be_in[kMaxIn];
  int64_t s_out[kMaxIn][kMaxLetters];
  int64_t s_red[kMaxIn][kMaxLetters];
  // causal pair (letters located in the output or among reduced letters)
  int32_t causal;
  int32_t s_red_flag, s_pos, t_red_flag, t_pos;
  // rows: every output letter but the last is a row coordinate
  int64_t rows_per_block;
  int32_t vec;                  // elements per vector along the innermost letter (map)
  int32_t inner_red;            // reduce: index of the reduced letter innermost in input 0, or -1
};
hipError_t launch_map(const EwArgs &a, hipStream_t st);
hipError_t launch_reduce(const EwArgs &a, hipStream_t st);

// launch shape of the vectorised map / row-reduce kernels
struct StreamArgs {
  int64_t chunks;                  // workgroups per output key
  int64_t slots;                   // map: vectors per output block
  FastDiv div_vpr;                 // map: division by vectors per row
  FastDiv div_out[kMaxLetters];    // division by each output block extent
};
hipError_t launch_map_vec(const EwArgs &a, StreamArgs sa, int vec, hipStream_t st);
hipError_t launch_reduce_row(const EwArgs &a, StreamArgs sa, int vec, int lpr, hipStream_t st);

// ---------------------------------------------------------------- flat streams
// Map and row reduce for "row-compatible" operands: the output block is a
// row-major walk of rows (map: every output letter but the innermost;
// reduce: every output letter) and each input's in-block offset of row r is
// r * row_mul, plus, along the innermost letter of the walk, the element
// index (inner = 1) or nothing (inner = 0, a broadcast).  No row letter has a
// padded tail, every block is under 2 GiB, and ids fit 31 bits, so all index
// arithmetic is 32-bit.
struct FlatIn {
  const void *p;
  uint32_t block_bytes;
  int32_t dt;          // 0 f32, 1 bf16
  int32_t inner;       // 1 contiguous along the walk's innermost letter, 0 constant along it
  int32_t row_mul;
};
struct FlatArgs {
  FlatIn in[kMaxIn];
  int32_t n_in;
  void *out;
  int32_t out_dt;
  float alpha, beta, eps;
  const int32_t *list;
  const int32_t *counts;
  int32_t per_key;
  int32_t n_keys;
  int32_t chunks;            // workgroups per output key
  FastDiv div_chunks;
  int32_t be_out;            // output block elements
  // map: rows of vpr vectors; innermost letter valid extent n_last - kappa_last * e_last
  int32_t slots, vpr, e_last, n_last, k_last;
  FastDiv div_vpr, div_klast;
  // causal pair: s is a row letter with c_s = (row / R_s) % e_s and
  // kappa_s = (key / W_s) % k_s; t is the innermost letter of the walk
  int32_t causal, e_s, k_s;
  FastDiv div_Rs, div_es, div_Ws, div_ks;
  // reduce: the reduced letter (innermost in input 0); block coordinate of a
  // joined tuple = (input-0 tuple id / w_red) % k_red
  int32_t e_red, n_red, k_red;
  FastDiv div_wred, div_kred;
};
hipError_t launch_flat_map(const FlatArgs &a, int g, hipStream_t st);  // 8 elements per vector
hipError_t launch_flat_reduce(const FlatArgs &a, int vec, int lpr, int g, int agg, hipStream_t st);

// ---------------------------------------------------------- RMS-norm pair
// A sum-of-squares reduce over the innermost letter r of x and the RMS-scale
// map that reads its result, run as one pass ("Stax (5): Caching and
// Measurement", Section 7: vertical fusion of a reduction and the pointwise
// map that reads it at the same row index): one wavefront per row loads the
// row's pieces (one per r-block, listed by the reduce's join) once, writes
// the row statistic and then the scaled row.  y is numbered and laid out
// like x; the scale relation has the one letter r.
constexpr int kNormMaxVec = 16;  // 4-element vectors per lane: rows of at most 4096 elements
struct NormArgs {
  const void *x;           // f32 or bf16 blocks of be_x elements
  int32_t x_dt;
  int64_t be_x;
  float *ss;               // f32 blocks of `rows` elements, tuple id = reduce key
  const void *gam;         // r-block kr at tuple id kr, blocks of be_g elements
  int32_t g_dt;
  int64_t be_g;
  void *y;                 // tuple id = x's
  int32_t y_dt;
  const int32_t *list;     // the reduce's join list: (ss tuple, x tuple) per entry
  const int32_t *counts;
  int32_t per_key;
  int32_t n_keys;
  int32_t rows;            // rows per block
  int32_t chunks;          // workgroups per key (4 rows each)
  FastDiv div_chunks;
  int32_t e_r, n_r;        // block extent and extent of r
  int32_t nvb;             // vectors per lane per r-block: e_r / 256
  FastDiv div_wr, div_kr;  // r-block of an x tuple id: (id / w_r) % k_r
  float alpha_r, alpha_m, beta, eps;
};
hipError_t launch_norm(const NormArgs &a, hipStream_t st);

// ---------------------------------------------------------------- attention
// One workgroup: 128 rows of s (32 per wavefront) of one output key and one
// batch index inside the block; it walks the key's joined (K, V) tuples in
// join-list order, 64 keys t at a time.
struct AttnArgs {
  const void *Q, *K, *V;
  void *O;
  const int32_t *list;
  const int32_t *counts;
  int32_t per_key;
  int32_t n_keys;
  int64_t beQ, beK, beV, beO;          // block elements
  int32_t nx;                          // batch letters inside a block, innermost last
  FastDiv xdiv[kMaxLetters];           // their block extents
  int64_t xQ[kMaxLetters], xK[kMaxLetters], xV[kMaxLetters], xO[kMaxLetters];  // in-block strides
  int32_t nbatch;                      // product of the batch block extents
  int64_t sQ, sO, tK, tV;              // in-block strides of s (Q, O) and t (K, V)
  int32_t e_s, e_t;                    // padded block extents of s and t
  int32_t n_s, n_t;                    // extents of s and t
  int32_t s_tiles;                     // ceil(e_s / 128)
  FastDiv div_st, div_nb;              // division by s_tiles and by nbatch
  FastDiv div_Ws, div_ks;              // kappa_s = (output tuple / Ws) % ks
  FastDiv div_Wt, div_kt;              // kappa_t = (K tuple / Wt) % kt
  float scale_log2;                    // alpha * log2(e)
  int32_t reverse;                     // causal: launch keys by s-block, heaviest first
  FastDiv div_per_s;                   // keys per s-block value (n_keys / ks)
  int32_t xcd_group;                   // keep one batch index's workgroups on one XCD
  FastDiv div_group;                   // workgroups per batch index (n_keys * s_tiles)
  // packed sequences: s and t blocked by the same bounds (segment pair);
  // block kappa holds positions [bnd[kappa], bnd[kappa + 1])
  int32_t iv;
  int32_t bnd[kMaxIv + 1];
};
// joined K/V tuples per output tuple of the fused attention kernel (its
// per-tuple table lives in LDS)
constexpr int kMaxAttnTuples = 512;
// d: 64 or 128 (the padded D = E extent)
hipError_t launch_attention(const AttnArgs &a, int d, bool causal, bool out_bf16, hipStream_t st);

}  // namespace jagg
