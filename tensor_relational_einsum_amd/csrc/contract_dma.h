// contract_dma.h -- bf16 block contraction with a deep LDS pipeline fed by
// buffer loads that write LDS directly.
//
// Same computation as contract_kernel ("Every Kernel Is a Join", Sec. 1 and
// Examples 3.8/3.9: blocks matched on the contracted index, their products
// added per output block; one workgroup owns one output tile of one output key and
// accumulates every joined tuple's product in registers), for the case that
// dominates projection-heavy chains: bf16 operands read as 16-byte vectors,
// 256 x 256 output tiles, no causal pair on the reduced letter.
//
// CDNA4 mapping
//  - 4 wavefronts, one per SIMD, each owning a 128 x 128 quarter of the tile
//    (16 accumulators of 32 x 32 in AGPRs).  Per K chunk of 16 a wavefront
//    reads 8 fragments for 16 MFMAs: half the LDS bytes per MFMA of a
//    128 x 64 wavefront tile.
//  - The K walk (joined tuple, K-tile of 32) is served by NS LDS stages of
//    A[256 x 32] and B[256 x 32] (32 KB each, NS = 4 by default); a step's
//    loads are issued NS - 2 steps before the step that consumes them.  No
//    VGPRs hold data in flight.
//  - buffer_load_dwordx4 ... lds: each wavefront instruction fills 1 KB of
//    LDS contiguously, lane l at byte 16*l; which global vector lands in each
//    16-byte slot is chosen through the lane's offset.  The tiles are stored
//    unpadded with an XOR swizzle of 16-byte slots so that the fragment reads
//    below hit all 64 banks:
//      K-contiguous [256 rows][4 slots]: slot q of row r at q ^ ((r >> 2) & 3)
//      M/N-contiguous [32 K rows][32 slots]: slot c of row k at c ^ (4 * (k & 3))
//  - For bf16 outputs the MFMAs take the B fragment first, which computes
//    each 32 x 32 accumulator transposed: a lane then holds four consecutive
//    output columns per group of four values, and the epilogue writes a
//    group with one 8-byte store instead of four element stores.
//  - Out-of-range lanes (rows past the block edge, the K tail) pass an offset
//    past the buffer's end and write zeros, as the plain buffer load does.
//  - Each step is two phases of 16 MFMAs around one barrier; the fragment
//    reads of the next chunk and the step's loads are issued between the
//    MFMAs, so the in-order wavefront issues them in the MFMA shadow.
//    Issuing the loads as a burst after the barrier instead cost ~10% (the
//    vector memory path backs up and stalls MFMA issue).
//  - Waits: before the barrier a wavefront waits for its own loads of the
//    stage the next phase reads (vmcnt counts vector loads in issue order)
//    and for its LDS reads; the barrier then makes every wavefront's loads of
//    that stage visible and every read of the stage about to be refilled
//    complete.
#pragma once

#ifndef JAGG_DMA_STAGES
#define JAGG_DMA_STAGES 4
#endif

#include "contract_impl.h"

namespace jagg {

constexpr int kDmaBK = 32;                 // K elements per step
constexpr int kDmaRowBytes = kDmaBK * 2;   // bytes of one K-contiguous row
constexpr int kDmaTileBytes = 256 * kDmaRowBytes;  // one operand tile (16 KB)

// One operand's DMA loads: 256 rows (M or N) by 32 K values; R*4 slots over
// NT threads, NI instructions each.  SPLIT: the 256 rows are two operands of
// 128 rows each (the gate and up weights of SwiGLU): instructions i < NI/2
// fill rows 0..127 from the first, the others rows 128..255 from the second,
// each row index taken modulo 128 in its own operand.  An M/N-contiguous
// split tile is stored as two [32 K rows][16 slots] halves (slot c of K row
// k at c ^ 4 (k & 3)) so that one instruction's 1 KB stays in one half.
template <bool KC, int NT, bool SPLIT = false>
struct DmaOperand {
  static constexpr int SLOTS = 256 * 4;
  static constexpr int NI = SLOTS / NT;
  static_assert(SLOTS % NT == 0 && NT % 64 == 0, "tile does not split over the wavefronts");
  static_assert(!SPLIT || (NI % 2 == 0 && NT == 256), "split halves must fall on instruction boundaries");
  uint32_t off[NI];   // byte offset from the step's origin, or kOob for rows past the edge
  int32_t kidx[NI];   // K index of the lane's vector inside the step

  // wave: wavefront index; lane: lane index; rows_left: valid rows (M or N)
  __device__ __forceinline__ void init(int wave, int lane, int rows_left, int64_t s_row, int64_t s_k) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int P = (i * (NT / 64) + wave) * 64 + lane;  // 16-byte LDS slot this lane fills
      int row, k;
      if (KC) {
        const int r = P >> 2, q = (P & 3) ^ ((r >> 2) & 3);
        row = SPLIT ? (r & 127) : r;
        k = q * 8;
      } else if (SPLIT) {
        const int Q = P & 511, kr = Q >> 4, c = (Q & 15) ^ ((kr & 3) << 2);
        row = c * 8;
        k = kr;
      } else {
        const int kr = P >> 5, c = (P & 31) ^ ((kr & 3) << 2);
        row = c * 8;
        k = kr;
      }
      kidx[i] = k;
      off[i] = row < rows_left ? uint32_t((int64_t(row) * s_row + int64_t(k) * s_k) * 2) : kOob;
    }
  }

  // issue load i of one step into `lds` (this operand's 16 KB of a stage)
  __device__ __forceinline__ void issue(int i, i32x4_rsrc rs, int k_left, char *lds, int wave_s) const {
    dma16(rs, kidx[i] < k_left ? off[i] : kOob, lds + (i * (NT / 64) + wave_s) * 1024);
  }
};

// One 256 x 256 output tile: logical tile w of the contraction p.  SW
// (SwiGLU): the tile is 256 rows x 128 output columns, its B tile the same
// 128 columns of B and of B2; each wavefront owns 128 rows x 64 columns of
// both products (fragments j = 0, 1 of B, j = 2, 3 of B2, the same columns)
// and recomposes silu(AB) * (AB2) in registers.
// EPI: the recompose map, fixed per instantiation so that the epilogue
// unrolls with the accumulators in registers: 0 none, 1 / 2 add an f32 /
// bf16 addend laid out as C (MUL_PLUS), 3 SwiGLU.
// SPLIT: one part of a split walk (EPI 0 only; see ContractArgs::split).
template <int OUT_BF16, bool A_KC, bool B_KC, int NS, int EPI = 0, bool SPLIT = false>
__device__ __forceinline__ void dma_tile(const ContractArgs &p, int64_t w) {
  static_assert(!SPLIT || EPI == 0, "a split walk has no recompose map");
  constexpr bool SW = EPI == 3;
  // bf16 outputs: accumulators transposed (B fragment first), stored in
  // 8-byte column groups; f32 outputs keep the plain layout, whose element
  // stores write whole 128-byte row runs per half wavefront
  constexpr bool TR = OUT_BF16;
  // 4 wavefronts, one per SIMD, each owning a 128 x 128 quarter of the tile
  constexpr int NT = 256, WAVES_N = 2;
  constexpr int WTM = 128, WTN = SW ? 64 : 128, TM = WTM / 32, TN = 4;
  constexpr int BM = 256, BN = SW ? 128 : 256, BK = kDmaBK;
  constexpr int L = DmaOperand<A_KC, NT>::NI + DmaOperand<B_KC, NT, SW>::NI;  // loads per step per thread
  static_assert(NS >= 3 && NS <= 5, "stage count");
  __shared__ __attribute__((aligned(1024))) char smem[NS * 2 * kDmaTileBytes];
  auto stage = [&](int s) { return smem + (s % NS) * (2 * kDmaTileBytes); };

  // split walk: part q of the tile (the parts' tiles numbered part-major)
  int part = 0;
  if constexpr (SPLIT) {
    part = __builtin_amdgcn_readfirstlane(int(w / p.n_tiles));
    w -= int64_t(part) * p.n_tiles;
  }
  int tn, tm, bt;
  int64_t key;
  decode_tile(p, w, tm, tn, bt, key);
  const int32_t cnt = p.counts[key];
  if (cnt == 0) return;  // output tuple absent (causal); uniform, before any barrier
  // the join list is read-only for the kernel's lifetime: reading it through
  // the constant address space keeps the tuple-id reads on the scalar unit
  typedef const __attribute__((address_space(4))) int32_t *const_i32p;
  const const_i32p ents = (const_i32p)(p.list + key * int64_t(p.per_key) * p.ent_w);

  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = (p.K + BK - 1) / BK;
  int steps = cnt * KT, s_begin = 0;
  if constexpr (SPLIT) {
    // uniform values the compiler cannot prove uniform through the
    // divisions: the buffer resources built from them must be scalar
    s_begin = __builtin_amdgcn_readfirstlane(int(int64_t(steps) * part / p.split));
    steps = __builtin_amdgcn_readfirstlane(int(int64_t(steps) * (part + 1) / p.split)) - s_begin;
  }
  const int64_t a_org = int64_t(bt) * p.sAb + int64_t(m0) * p.sAm;
  const int64_t b_org = int64_t(bt) * p.sBb + int64_t(n0) * p.sBn;
  int64_t ks = 0;
  if (p.causal_out) ks = (key / p.cs_w) % p.cs_k;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  DmaOperand<A_KC, NT> da;
  DmaOperand<B_KC, NT, SW> db;
  da.init(wave, lane, p.M - m0, p.sAm, p.sAk);
  db.init(wave, lane, p.N - n0, p.sBn, p.sBk);

  // the walk over (joined tuple, K-tile): position and tuple ids of the next
  // step to load; past the last step the loads use an empty resource (every
  // lane reads zeros) so that every step issues the same number of loads.
  // The byte address of the step's origin in each operand and the bytes from
  // there to the end of its block are formed once per joined tuple and then
  // stepped by a constant: the per-step work stays a few scalar adds, which
  // issue in the shadow of one MFMA instead of idling the matrix core.
  int ld = 0, le = 0, lkt = 0;
  if constexpr (SPLIT) {
    le = __builtin_amdgcn_readfirstlane(s_begin / KT);
    lkt = s_begin - le * KT;
  }
  int64_t la = ents[le * p.ent_w + p.a_slot], lb = ents[le * p.ent_w + p.b_slot];
  int k_next = p.K - lkt * BK;
  const int64_t a_step = int64_t(BK) * p.sAk * 2, b_step = int64_t(BK) * p.sBk * 2;
  uint64_t pa, pb;  // byte addresses of the next step's origins
  uint64_t ea, eb;  // byte addresses of the ends of their blocks
  auto tuple_origin = [&]() {
    pa = reinterpret_cast<uint64_t>(p.A) + uint64_t(la * p.beA + a_org) * 2;
    pb = reinterpret_cast<uint64_t>(p.B) + uint64_t(lb * p.beB + b_org) * 2;
    ea = reinterpret_cast<uint64_t>(p.A) + uint64_t((la + 1) * p.beA) * 2;
    eb = reinterpret_cast<uint64_t>(p.B) + uint64_t((lb + 1) * p.beB) * 2;
  };
  tuple_origin();
  if constexpr (SPLIT) {  // a part starting inside a joined tuple's K walk
    pa += uint64_t(int64_t(lkt) * a_step);
    pb += uint64_t(int64_t(lkt) * b_step);
  }
  // Each operand has its own load state (resource, valid K, LDS target), so
  // that the next step's state is built in an MFMA slot of its own while the
  // other operand's loads of the current step are still being issued.
  i32x4_rsrc rs_a, rs_b, rs_b2;  // rs_b2: SwiGLU's B2
  int kl_a = 0, kl_b = 0;
  char *buf_a = smem, *buf_b = smem;
  auto prep_a = [&](char *buf) {
    rs_a = dma_rsrc(reinterpret_cast<const void *>(pa), ld < steps ? int64_t(ea - pa) : 0);
    kl_a = k_next;
    buf_a = buf;
  };
  auto prep_b = [&](char *buf) {
    const int64_t nb = ld < steps ? int64_t(eb - pb) : 0;
    rs_b = dma_rsrc(reinterpret_cast<const void *>(pb), nb);
    // B2 has B's geometry: the same offsets from its own base
    if constexpr (SW)
      rs_b2 = dma_rsrc(reinterpret_cast<const void *>(pb - reinterpret_cast<uint64_t>(p.B) +
                                                      reinterpret_cast<uint64_t>(p.B2)),
                       nb);
    kl_b = k_next;
    buf_b = buf;
  };
  auto dma_a = [&](int i) { da.issue(i, rs_a, kl_a, buf_a, wave_s); };
  auto dma_b = [&](int i) {
    constexpr int NBH = DmaOperand<B_KC, NT, SW>::NI / 2;
    if constexpr (SW) db.issue(i, i < NBH ? rs_b : rs_b2, kl_b, buf_b + kDmaTileBytes, wave_s);
    else db.issue(i, rs_b, kl_b, buf_b + kDmaTileBytes, wave_s);
  };
  // straight-line steps; a branch only where a joined tuple's K walk ends
  auto advance = [&]() {
    ++ld;
    k_next -= BK;
    pa += a_step;
    pb += b_step;
    if (__builtin_expect(++lkt == KT, 0)) {
      lkt = 0;
      k_next = p.K;
      if (++le < cnt) {
        la = ents[le * p.ent_w + p.a_slot];
        lb = ents[le * p.ent_w + p.b_slot];
      }
      tuple_origin();
    }
  };
  constexpr int NA = DmaOperand<A_KC, NT>::NI, NB = DmaOperand<B_KC, NT, SW>::NI;

  const int wm = (wave / WAVES_N) * WTM, wn = (wave % WAVES_N) * WTN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // fragment addresses inside a stage (bytes), per K chunk kc of 16
  //  K-contiguous: row wm + 32 i + lrow, slot (2 kc + lhalf) ^ ((lrow >> 2) & 3)
  //  M/N-contiguous (transposing reads): lane s of 16-lane group g reads K row
  //  16 kc + 8 (g >> 1) + (s >> 2), columns col0 + 16 (g & 1) + 4 (s & 3)
  const int g16 = lane >> 4, s16 = lane & 15;
  auto kc_addr = [&](int row0, int kc) {
    return (row0 + lrow) * kDmaRowBytes + (((2 * kc + lhalf) ^ ((lrow >> 2) & 3)) << 4);
  };
  auto rc_addr = [&](int col0) {
    const int kr = 8 * (g16 >> 1) + (s16 >> 2);
    const int slot = (col0 >> 3) + 2 * (g16 & 1) + ((s16 & 3) >> 1);
    return kr * 512 + ((slot ^ ((kr & 3) << 2)) << 4) + 8 * (s16 & 1);
  };
  // SwiGLU split halves, M/N-contiguous: [32 K rows][16 slots] per half
  auto rc_addr_h = [&](int col0) {
    const int kr = 8 * (g16 >> 1) + (s16 >> 2);
    const int slot = ((col0 & 127) >> 3) + 2 * (g16 & 1) + ((s16 & 3) >> 1);
    return (col0 >> 7) * 8192 + kr * 256 + ((slot ^ ((kr & 3) << 2)) << 4) + 8 * (s16 & 1);
  };
  // B row (N) of fragment j of this wavefront: j < 2 from B, j >= 2 from B2
  auto b_row = [&](int j) { return SW ? (j >> 1) * 128 + wn + 32 * (j & 1) : wn + 32 * j; };
  int a_addr[A_KC ? 2 : TM], b_addr[B_KC ? (SW ? 2 * TN : 2) : TN];
  if constexpr (A_KC) {
    a_addr[0] = kc_addr(wm, 0);
    a_addr[1] = kc_addr(wm, 1);
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) a_addr[i] = rc_addr(wm + 32 * i);
  }
  if constexpr (B_KC && SW) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      b_addr[2 * j] = kc_addr(b_row(j), 0) + kDmaTileBytes;
      b_addr[2 * j + 1] = kc_addr(b_row(j), 1) + kDmaTileBytes;
    }
  } else if constexpr (B_KC) {
    b_addr[0] = kc_addr(wn, 0) + kDmaTileBytes;
    b_addr[1] = kc_addr(wn, 1) + kDmaTileBytes;
  } else if constexpr (SW) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b_addr[j] = rc_addr_h(b_row(j)) + kDmaTileBytes;
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) b_addr[j] = rc_addr(wn + 32 * j) + kDmaTileBytes;
  }

  typedef __attribute__((address_space(3))) i16x4 *lds_v4;
  auto frag_kc = [&](const char *base, int addr, int i) {
    return *reinterpret_cast<const uint4 *>(base + addr + i * 32 * kDmaRowBytes);
  };
  // pitch: bytes per K row (512, or 256 in a SwiGLU half)
  auto frag_rc = [&](const char *base, int addr, int kc, int pitch = 512) {
    char *p0 = const_cast<char *>(base) + addr + kc * 16 * pitch;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p0 + 4 * pitch));
    uint4 r;
    __builtin_memcpy(&r.x, &lo, 8);
    __builtin_memcpy(&r.z, &hi, 8);
    return r;
  };
  // fragments of one K chunk of 16: TM of A, TN of B
  struct Frags {
    uint4 a[TM], b[TN];
  };
  // fragment x of chunk kc: x < TM is A's fragment x, else B's fragment x - TM
  auto read_frag = [&](const char *S, int kc, Frags &f, int x) {
    if (x < TM) {
      if constexpr (A_KC) f.a[x] = frag_kc(S, a_addr[kc], x);
      else f.a[x] = frag_rc(S, a_addr[x], kc);
    } else {
      if constexpr (B_KC && SW) f.b[x - TM] = *reinterpret_cast<const uint4 *>(S + b_addr[2 * (x - TM) + kc]);
      else if constexpr (B_KC) f.b[x - TM] = frag_kc(S, b_addr[kc], x - TM);
      else if constexpr (SW) f.b[x - TM] = frag_rc(S, b_addr[x - TM], kc, 256);
      else f.b[x - TM] = frag_rc(S, b_addr[x - TM], kc);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Step s (stage s mod NS), with chunk 0 of its stage already in f0:
  //   phase A: MFMAs of chunk 0, with the reads of chunk 1 and B's loads of
  //     step s+NS-2 (into stage s-2) between them; the walk moves to step
  //     s+NS-1 and A's load state for it is built, each in a free slot;
  //   wait for this wavefront's loads of stage s+1 and for its LDS reads,
  //     barrier (stage s+1 now visible to all; every read of stage s-1,
  //     last read in step s-1, complete);
  //   phase B: MFMAs of chunk 1, with the reads of chunk 0 of stage s+1 and
  //     A's loads of step s+NS-1 (into stage s-1) between them; B's load
  //     state for that step is built in a free slot after them.
  // One wavefront per SIMD issues in order, about one instruction per four
  // cycles, so everything placed between two MFMAs issues in the shadow of
  // the first as long as it fits in its 32 cycles: the reads, the loads and
  // the walk's scalar bookkeeping each get slots of their own instead of
  // meeting in one run between the phases.  Spreading the loads over the
  // step also keeps the vector memory path from being flooded right after
  // the barrier.  Scheduling barriers pin the order.
  // Stage s-2 is free since step s-1's barrier and stage s-1 since step s's.
  // Past the last step the reads see zero fill or stale data that no MFMA
  // consumes.
  static_assert(TM * TN == 16 && TM + TN <= 8 && NA <= 4 && NB <= 4, "interleave pattern");
  auto phase = [&](const Frags &fm, const char *rd_stage, int rd_kc, Frags &fr, auto &&dma, auto &&book) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (TR) Mma<uint16_t>::run(acc[k / TN][k % TN], fm.b[k % TN], fm.a[k / TN]);
      else Mma<uint16_t>::run(acc[k / TN][k % TN], fm.a[k / TN], fm.b[k % TN]);
      if (k < TM + TN) read_frag(rd_stage, rd_kc, fr, k);
      if (k >= 8 && (k & 1) == 0 && (k - 8) / 2 < 4) dma((k - 8) / 2);
      book(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  constexpr int PRO = NS - 2;  // steps loaded whole before the loop (plus A's half of one)
  constexpr int PRO_WAIT = (NS - 3) * (NA + NB) + NA;

  Frags f0, f1;
  // prologue: the first PRO steps whole, then step NS-2's A loads (its B
  // loads go out in the first phase of the loop)
  for (int s = 0; s < PRO; ++s) {
    prep_a(stage(s));
    prep_b(stage(s));
#pragma unroll
    for (int i = 0; i < NA; ++i) dma_a(i);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma_b(i);
    advance();
  }
  prep_a(stage(NS - 2));
  prep_b(stage(NS - 2));
#pragma unroll
  for (int i = 0; i < NA; ++i) dma_a(i);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(PRO_WAIT) : "memory");
#pragma unroll
  for (int x = 0; x < TM + TN; ++x) read_frag(stage(0), 0, f0, x);
  for (int s = 0; s < steps; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    phase(
        f0, stage(s), 1, f1,
        [&](int i) {
          if (i < NB) dma_b(i);
        },
        [&](int k) {
          if (k == 9) advance();
          if (k == 11) prep_a(stage(s + NS - 1));
        });
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NS - 3) * (NA + NB)) : "memory");
    phase(
        f1, stage(s + 1), 0, f0,
        [&](int i) {
          if (i < NA) dma_a(i);
        },
        [&](int k) {
          if (k == 13) prep_b(stage(s + NS - 1));
        });
  }

  // the zero-fill loads past the last step may still be in flight: let them
  // land before the workgroup's LDS can be handed to another workgroup
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (SPLIT) {
    // one part of a split walk: its fp32 sums, laid out as C, into the
    // part's slice of the workspace (the sum kernel applies alpha)
    ContractArgs q = p;
    q.C = p.part + int64_t(part) * p.part_stride;
    q.alpha = 1.0f;
    if constexpr (TR) store_tile_t<0, TM, TN, 0>(q, acc, ents[0], bt, key, ks, m0 + wm, n0 + wn, lane);
    else store_tile_plain<0, TM, TN>(q, acc, ents[0], bt, key, ks, m0 + wm, n0 + wn, lane);
  } else if constexpr (SW && TR) {
    // recompose: silu(A B) * (A B2), fragments j and j + 2 hold one column
    // range; transposed accumulators (B fragment first in the MFMA): group g
    // of lane l is row 32 i + l % 32, columns 32 j + 8 g + 4 (l / 32) + 0..3
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int OSZ = OUT_BF16 ? 2 : 4;
    const int lrow2 = lane & 31, lhalf2 = lane >> 5;
    const int64_t cbase = int64_t(ents[0]) * p.beC + int64_t(bt) * p.sCb;
    const bool wide = ((p.sCm | int64_t(p.N) | cbase) & 3) == 0;
    const __amdgpu_buffer_rsrc_t rc =
        tile_rsrc(static_cast<char *>(p.C) + cbase * OSZ, (p.beC - int64_t(bt) * p.sCb) * OSZ);
    auto gate = [&](float gv, float uv) { return p.alpha * gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv; };
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = m0 + wm + i * 32 + lrow2, n = n0 + wn + j * 32 + 8 * g + 4 * lhalf2;
          float x[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) x[c] = gate(acc[i][j][4 * g + c], acc[i][j + 2][4 * g + c]);
          if (wide) {
            const bool ok = m < p.M && n < p.N;
            const uint32_t e = uint32_t(int64_t(m) * p.sCm + n);
            if constexpr (OUT_BF16) {
              const u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
              __builtin_amdgcn_raw_buffer_store_b64(v, rc, int(ok ? e * 2 : kOob), 0, 0);
            } else {
              const u32x4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                               __float_as_uint(x[3])};
              __builtin_amdgcn_raw_buffer_store_b128(v, rc, int(ok ? e * 4 : kOob), 0, 0);
            }
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (m < p.M && n + c < p.N) {
                const int64_t off = cbase + int64_t(m) * p.sCm + n + c;
                if (OUT_BF16)
                  reinterpret_cast<uint16_t *>(p.C)[off] = f32_to_bf16(x[c]);
                else
                  reinterpret_cast<float *>(p.C)[off] = x[c];
              }
          }
        }
  } else if constexpr (SW) {
    // recompose: silu(A B) * (A B2), fragments j and j + 2 hold one column
    const int lrow2 = lane & 31, lhalf2 = lane >> 5;
    char *Cb = reinterpret_cast<char *>(p.C);
    const int64_t cbase = int64_t(ents[0]) * p.beC + int64_t(bt) * p.sCb;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm + i * 32 + (v >> 2) * 8 + lhalf2 * 4 + (v & 3);
          const int n = n0 + wn + j * 32 + lrow2;
          if (m < p.M && n < p.N) {
            const float gv = acc[i][j][v], uv = acc[i][j + 2][v];
            const float x = p.alpha * gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            const int64_t off = cbase + int64_t(m) * p.sCm + n;
            if (OUT_BF16)
              reinterpret_cast<uint16_t *>(Cb)[off] = f32_to_bf16(x);
            else
              reinterpret_cast<float *>(Cb)[off] = x;
          }
        }
  } else if constexpr (TR) {
    store_tile_t<OUT_BF16, TM, TN, EPI>(p, acc, ents[0], bt, key, ks, m0 + wm, n0 + wn, lane);
  } else {
    if constexpr (EPI == 0) store_tile_plain<OUT_BF16, TM, TN>(p, acc, ents[0], bt, key, ks, m0 + wm, n0 + wn, lane);
    else store_tile_plus<OUT_BF16, TM, TN, EPI - 1, true>(p, acc, ents[0], bt, m0 + wm, n0 + wn, lane);
  }
}

template <int OUT_BF16, bool A_KC, bool B_KC, int NS, int EPI = 0, bool SPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void contract_dma_kernel(
    const ContractArgs p) {
  dma_tile<OUT_BF16, A_KC, B_KC, NS, EPI, SPLIT>(p, logical_tile(p.remap));
}

// Several independent contractions of one geometry (every field of `common`
// but the operand, output and join-list addresses) in one launch of n T
// logical tiles, T per problem.  One launch instead of several shares the
// last partial wave of tiles and the launch edges.
template <int OUT_BF16, bool A_KC, bool B_KC, int NS, int EPI = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void contract_dma_group_kernel(
    const DmaGroupArgs ga) {
  const int64_t w = logical_tile(ga.common.remap);
  int g;
  int64_t local;
  const ContractArgs &c = ga.common;
  if (c.group_m) {
    // the grouped tile order of one problem walks M-panel groups, each over
    // every N panel; the problems take turns per M-panel group, so all XCDs
    // sweep one problem's B operand at a time (as one problem alone does)
    // and share the A panels of a group between the problems
    const int64_t Mp = int64_t(c.km) * c.tiles_m, Np = int64_t(c.kn) * c.tiles_n;
    const int64_t n_groups = (Mp + c.group_m - 1) / c.group_m;
    const int64_t per_group = int64_t(c.group_m) * Np;
    const int64_t full = (n_groups - 1) * ga.n * per_group;
    int64_t gi, r;
    if (w < full) {
      const int64_t vg = w / per_group;
      r = w - vg * per_group;
      gi = vg / ga.n;
      g = int(vg - gi * ga.n);
    } else {
      const int64_t last = (Mp - (n_groups - 1) * c.group_m) * Np;
      const int64_t rem = w - full;
      g = int(rem / last);
      r = rem - int64_t(g) * last;
      gi = n_groups - 1;
    }
    local = gi * per_group + r;
  } else {
    g = int(w / ga.tiles);
    local = w - int64_t(g) * ga.tiles;
  }
  ContractArgs p = ga.common;
  p.A = ga.A[g];
  p.B = ga.B[g];
  p.C = ga.C[g];
  p.list = ga.list[g];
  p.counts = ga.counts[g];
  p.X = ga.X[g];
  p.B2 = ga.B2[g];
  dma_tile<OUT_BF16, A_KC, B_KC, NS, EPI>(p, local);
}

template <int OB, bool AK, bool BKC, int EPI = 0>
static hipError_t launch_dma(const ContractArgs &a, hipStream_t st) {
  ContractArgs b = a;
  b.tiles_m = (a.M + 255) / 256;
  b.tiles_n = EPI == 3 ? (a.N + 127) / 128 : (a.N + 255) / 256;
  b.n_tiles = b.n_keys * b.batch * int64_t(b.tiles_m) * b.tiles_n;
  if constexpr (EPI == 0) {
    if (a.split > 1) {
      hipLaunchKernelGGL((contract_dma_kernel<OB, AK, BKC, JAGG_DMA_STAGES, 0, true>),
                         dim3(unsigned(b.n_tiles * a.split)), dim3(256), 0, st, b);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((contract_dma_kernel<OB, AK, BKC, JAGG_DMA_STAGES, EPI>), dim3(unsigned(b.n_tiles)), dim3(256), 0,
                     st, b);
  return hipGetLastError();
}

template <int OB, bool AK, bool BKC, int EPI = 0>
static hipError_t launch_dma_group(const DmaGroupArgs &a, hipStream_t st) {
  DmaGroupArgs b = a;
  b.common.tiles_m = (a.common.M + 255) / 256;
  b.common.tiles_n = EPI == 3 ? (a.common.N + 127) / 128 : (a.common.N + 255) / 256;
  b.tiles = b.common.n_keys * b.common.batch * int64_t(b.common.tiles_m) * b.common.tiles_n;
  const int64_t grid = b.tiles * b.n;
  hipLaunchKernelGGL((contract_dma_group_kernel<OB, AK, BKC, JAGG_DMA_STAGES, EPI>), dim3(unsigned(grid)), dim3(256),
                     0, st, b);
  return hipGetLastError();
}

}  // namespace jagg
