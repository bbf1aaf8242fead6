// contract.hip -- MFMA block contraction with the SUM aggregation fused.
//
// "Every Kernel Is a Join" (Ding et al.), Sec. 1 and Example 3.8/3.9: a
// matrix multiply is a join on the shared inner index followed by a SUM;
// every joined tuple multiplies one block of each input, and the products
// of equal output key are added (Def. 3.7 step 2).  One workgroup owns one
// 128x128 tile of one output block (and one batch index) and walks all the
// joined tuples of that output key and the K-tiles of each, accumulating in
// fp32 registers; the tile is written once, so the aggregation never goes
// through memory (the page's aggregation pushdown, taken to one GPU).
//
// CDNA4 mapping: 256 threads = 4 wavefronts in a 2x2 grid, each computing a
// 64x64 sub-tile with 2x2 MFMA 32x32 tiles (bf16: v_mfma_f32_32x32x16_bf16;
// fp32: v_mfma_f32_32x32x2_f32).  Operand tiles are staged through LDS in
// K-contiguous rows of 128 bytes (64 bf16 or 32 fp32) plus 16 bytes of
// padding, double-buffered: the global loads of step s+1 are in flight while
// the MFMAs of step s run.  An operand contiguous along M or N is transposed
// on its way into LDS.
#include "device_common.h"
#include "jagg_internal.h"

namespace jagg {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

template <int NB>
struct VecT;
template <>
struct VecT<16> {
  using type = uint4;
};
template <>
struct VecT<8> {
  using type = uint2;
};
template <>
struct VecT<4> {
  using type = uint32_t;
};
template <>
struct VecT<2> {
  using type = uint16_t;
};

constexpr int kBM = 128, kBN = 128;
constexpr int kRowBytes = 128;             // K bytes per LDS row
constexpr int kPitch = kRowBytes + 16;     // padded LDS row pitch
constexpr int kOpBytes = 128 * kPitch;     // one operand tile
constexpr int kStageBytes = 2 * kOpBytes;  // A and B

// Loads one 128-row x (128/ESZ)-K operand tile from global memory into
// registers and stores it K-contiguous into LDS.
template <typename T, bool KC, int VEC>
struct Loader {
  static constexpr int ESZ = int(sizeof(T));
  static constexpr int BK = kRowBytes / ESZ;
  static constexpr int NV = 128 * BK / VEC / 256;
  using V = typename VecT<VEC * ESZ>::type;
  union U {
    V v;
    T e[VEC];
  };
  U r[NV];

  // base: element (row 0, k 0) of the tile; s_row / s_k: strides; rows_left /
  // k_left: valid rows and K positions from the tile origin.
  __device__ __forceinline__ void load(const T *base, int64_t s_row, int64_t s_k, int rows_left, int k_left) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = t + 256 * i;
      int row, k;
      if (KC) {
        row = idx / (BK / VEC);
        k = (idx % (BK / VEC)) * VEC;
      } else {
        k = idx / (128 / VEC);
        row = (idx % (128 / VEC)) * VEC;
      }
      const bool ok = row < rows_left && k < k_left;
      if (ok) {
        const T *p = base + int64_t(row) * s_row + int64_t(k) * s_k;
        r[i].v = *reinterpret_cast<const V *>(p);
      } else {
        r[i].v = V{};
      }
    }
  }

  // zero every element with t > s (causal pair; s along rows, t along K)
  __device__ __forceinline__ void mask_causal(int64_t s0, int64_t t0, int e_s, int e_t, int m0, int k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = t + 256 * i;
      int row, k;
      if (KC) {
        row = idx / (BK / VEC);
        k = (idx % (BK / VEC)) * VEC;
      } else {
        k = idx / (128 / VEC);
        row = (idx % (128 / VEC)) * VEC;
      }
#pragma unroll
      for (int u = 0; u < VEC; ++u) {
        const int rr = KC ? row : row + u;
        const int kk = KC ? k + u : k;
        const int64_t sg = s0 + (m0 + rr) % e_s;
        const int64_t tg = t0 + (k0 + kk) % e_t;
        if (tg > sg) r[i].e[u] = T(0);
      }
    }
  }

  __device__ __forceinline__ void store(char *lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = t + 256 * i;
      if (KC) {
        const int row = idx / (BK / VEC);
        const int k = (idx % (BK / VEC)) * VEC;
        *reinterpret_cast<V *>(lds + row * kPitch + k * ESZ) = r[i].v;
      } else {
        const int k = idx / (128 / VEC);
        const int row = (idx % (128 / VEC)) * VEC;
#pragma unroll
        for (int u = 0; u < VEC; ++u) *reinterpret_cast<T *>(lds + (row + u) * kPitch + k * ESZ) = r[i].e[u];
      }
    }
  }
};

template <typename T>
struct Mma;

// bf16: one 32-byte K chunk (16 values) = one 32x32x16 MFMA.
template <>
struct Mma<uint16_t> {
  __device__ __forceinline__ static void run(f32x16 &acc, const uint4 &a, const uint4 &b) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
};

// fp32: one 32-byte K chunk (8 values, 4 per lane half) = four 32x32x2 MFMAs.
// Lane half h holds K positions 4h..4h+3 of the chunk; MFMA i pairs K
// position i (h = 0) with 4 + i (h = 1) in both operands alike, so the sum
// over K is complete.
template <>
struct Mma<float> {
  __device__ __forceinline__ static void run(f32x16 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

template <typename T, int OUT_BF16, bool A_KC, bool B_KC, int VA, int VB>
__global__ __launch_bounds__(256) void contract_kernel(const ContractArgs p) {
  constexpr int ESZ = int(sizeof(T));
  constexpr int BK = kRowBytes / ESZ;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];

  // workgroup -> (output key, batch, m-tile, n-tile)
  int64_t w = blockIdx.x;
  const int tn = int(w % p.tiles_n);
  w /= p.tiles_n;
  const int tm = int(w % p.tiles_m);
  w /= p.tiles_m;
  const int bt = int(w % p.batch);
  const int64_t key = w / p.batch;

  const int32_t cnt = p.counts[key];
  if (cnt == 0) return;  // output tuple absent (causal); uniform, before any barrier
  const int32_t *ents = p.list + key * int64_t(p.per_key) * 3;

  const int m0 = tm * kBM, n0 = tn * kBN;
  const int KT = (p.K + BK - 1) / BK;
  const int steps = cnt * KT;

  const T *Ab = reinterpret_cast<const T *>(p.A) + int64_t(bt) * p.sAb + int64_t(m0) * p.sAm;
  const T *Bb = reinterpret_cast<const T *>(p.B) + int64_t(bt) * p.sBb + int64_t(n0) * p.sBn;

  int64_t ks = 0;
  if (p.causal_out || p.causal_red) ks = (key / p.cs_w) % p.cs_k;

  Loader<T, A_KC, VA> la;
  Loader<T, B_KC, VB> lb;
  auto load_step = [&](int s) {
    const int e = s / KT;
    const int kt = s - e * KT;
    const int32_t *ent = ents + e * 3;
    const int64_t aid = ent[p.a_slot], bid = ent[p.b_slot];
    const int k0 = kt * BK;
    la.load(Ab + aid * p.beA + int64_t(k0) * p.sAk, p.sAm, p.sAk, p.M - m0, p.K - k0);
    lb.load(Bb + bid * p.beB + int64_t(k0) * p.sBk, p.sBn, p.sBk, p.N - n0, p.K - k0);
    if (p.causal_red) {
      const int64_t kt_blk = (aid / p.ct_w) % p.ct_k;
      if (kt_blk == ks) la.mask_causal(ks * p.e_s, kt_blk * p.e_t, p.e_s, p.e_t, m0, k0);
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int lrow = lane & 31, lhalf = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_step(0);
  la.store(smem);
  lb.store(smem + kOpBytes);
  __syncthreads();

  for (int s = 0; s < steps; ++s) {
    const int cur = s & 1;
    if (s + 1 < steps) load_step(s + 1);
    const char *As = smem + cur * kStageBytes;
    const char *Bs = As + kOpBytes;
#pragma unroll
    for (int ch = 0; ch < kRowBytes / 32; ++ch) {
      uint4 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const uint4 *>(As + (wm + i * 32 + lrow) * kPitch + ch * 32 + lhalf * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const uint4 *>(Bs + (wn + j * 32 + lrow) * kPitch + ch * 32 + lhalf * 16);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
    }
    if (s + 1 < steps) {
      char *nx = smem + (cur ^ 1) * kStageBytes;
      la.store(nx);
      lb.store(nx + kOpBytes);
    }
    __syncthreads();
  }

  // epilogue: scale, mask, convert, store (row = 8*(v/4) + 4*half + v%4, col = lane%32)
  const int32_t out_id = ents[0];
  char *Cb = reinterpret_cast<char *>(p.C);
  const int64_t cbase = int64_t(out_id) * p.beC + int64_t(bt) * p.sCb;
  int64_t kt_out = 0;
  if (p.causal_out) kt_out = (key / p.ct_w) % p.ct_k;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + i * 32 + (v >> 2) * 8 + lhalf * 4 + (v & 3);
        const int n = n0 + wn + j * 32 + lrow;
        if (m < p.M && n < p.N) {
          float x = p.alpha * acc[i][j][v];
          if (p.causal_out) {
            const int64_t sg = ks * p.e_s + m % p.e_s;
            const int64_t tg = kt_out * p.e_t + n % p.e_t;
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

template <typename T, int OB, bool AK, bool BK_, int VA, int VB>
static hipError_t go(const ContractArgs &a, hipStream_t st) {
  const int64_t grid = a.n_keys * a.batch * int64_t(a.tiles_m) * a.tiles_n;
  hipLaunchKernelGGL((contract_kernel<T, OB, AK, BK_, VA, VB>), dim3(unsigned(grid)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// vector widths: full 16 bytes or one element
template <typename T, int OB, bool AK, bool BK_>
static hipError_t pick_vec(const ContractArgs &a, int va, int vb, hipStream_t st) {
  constexpr int F = 16 / int(sizeof(T));
  if (va == F && vb == F) return go<T, OB, AK, BK_, F, F>(a, st);
  if (va == F && vb == 1) return go<T, OB, AK, BK_, F, 1>(a, st);
  if (va == 1 && vb == F) return go<T, OB, AK, BK_, 1, F>(a, st);
  if (va == 1 && vb == 1) return go<T, OB, AK, BK_, 1, 1>(a, st);
  return hipErrorInvalidValue;
}

template <typename T, int OB>
static hipError_t pick_layout(const ContractArgs &a, bool a_kc, bool b_kc, int va, int vb, hipStream_t st) {
  if (a_kc && b_kc) return pick_vec<T, OB, true, true>(a, va, vb, st);
  if (a_kc && !b_kc) return pick_vec<T, OB, true, false>(a, va, vb, st);
  if (!a_kc && b_kc) return pick_vec<T, OB, false, true>(a, va, vb, st);
  return pick_vec<T, OB, false, false>(a, va, vb, st);
}

hipError_t launch_contract(const ContractArgs &a, int dtype, int out_dtype, bool a_kc, bool b_kc, int va, int vb,
                           hipStream_t st) {
  if (dtype == 1) {
    return out_dtype ? pick_layout<uint16_t, 1>(a, a_kc, b_kc, va, vb, st)
                     : pick_layout<uint16_t, 0>(a, a_kc, b_kc, va, vb, st);
  }
  return out_dtype ? pick_layout<float, 1>(a, a_kc, b_kc, va, vb, st) : pick_layout<float, 0>(a, a_kc, b_kc, va, vb, st);
}

}  // namespace jagg
