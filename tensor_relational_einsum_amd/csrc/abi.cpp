// abi.cpp -- the C ABI of include/jagg.h: argument checking, relation
// geometry, and the planner that turns one join-agg spec into kernel
// launches on the context's stream.
//
// "Every Kernel Is a Join" (Ding et al.):
//   Def. 3.1 / Sec. 3.2  a block key is a tensor type, one interval per index;
//   Sec. 3.3             interval counts per index give the spec's blocking;
//   Def. 3.6 / 3.7       join, aggregate, recompose;
//   Sec. 5.3             repartition over the overlay (atoms) of two blockings.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/jagg.h"
#include "jagg_internal.h"

using namespace jagg;

struct jagg_ctx {
  int device;
  hipStream_t stream;
  std::string err;
  bool trace;
  bool debug_sync;
  bool capturing;  // between jagg_capture_begin and jagg_capture_end
  void *scratch;   // this device's copy of `scratch` (jagg_einsum_noalloc)
};

struct jagg_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

struct jagg_plan;  // holds a PlannedCall (defined with the planner below)

struct jagg_relation {
  jagg_ctx *ctx;
  int r;
  char letters[kMaxLetters + 1];
  int64_t n[kMaxLetters];
  int32_t k[kMaxLetters];
  int64_t e[kMaxLetters];
  jagg_dtype dt;
  void *buf;
  size_t bytes;
  int64_t n_tuples;
  int64_t be;  // elements per block
  // interval-blocked letters: iv[i] = 1 and bnd[i][0..k[i]] the bounds
  int32_t iv[kMaxLetters];
  int64_t bnd[kMaxLetters][kMaxIv + 1];
};

// Workspace of jagg_einsum_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never names it directly (the
// name is a host-side stand-in there); it uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device below.
static __device__ __align__(256) char scratch[JAGG_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch (device must be current); once per device.
hipError_t scratch_of_device(int device, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

jagg_status fail(jagg_ctx *ctx, jagg_status s, const char *fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return s;
}

int esz_of(jagg_dtype d) { return d == JAGG_BF16 ? 2 : 4; }

// ------------------------------------------------------------ geometry
// Fills block extents, tuple count and block size; checks the blocking.
// bnd (optional): bnd[i] NULL for a uniform letter, else its k[i]+1 bounds
// 0 = b_0 < ... < b_k = n; such a letter's blocks pad to the longest interval.
jagg_status geometry(jagg_ctx *ctx, int r, const int64_t *n, const int32_t *k, const int64_t *const *bnd,
                     int64_t *e, int64_t *n_tuples, int64_t *be) {
  int64_t nt = 1, b = 1;
  for (int i = 0; i < r; ++i) {
    if (n[i] < 1) return fail(ctx, JAGG_E_SHAPE, "extent %d of dimension %d must be >= 1", int(n[i]), i);
    if (k[i] < 1 || k[i] > n[i])
      return fail(ctx, JAGG_E_BLOCKING, "block count %d of dimension %d is outside [1, %lld]", k[i], i,
                  (long long)n[i]);
    if (bnd && bnd[i]) {
      const int64_t *q = bnd[i];
      if (k[i] > kMaxIv) return fail(ctx, JAGG_E_UNSUPPORTED, "dimension %d: more than %d intervals", i, kMaxIv);
      if (q[0] != 0 || q[k[i]] != n[i])
        return fail(ctx, JAGG_E_BLOCKING, "dimension %d: bounds must run from 0 to %lld", i, (long long)n[i]);
      e[i] = 0;
      for (int j = 0; j < k[i]; ++j) {
        if (q[j + 1] <= q[j])
          return fail(ctx, JAGG_E_BLOCKING, "dimension %d: bounds must increase strictly (%lld, %lld)", i,
                      (long long)q[j], (long long)q[j + 1]);
        e[i] = std::max(e[i], q[j + 1] - q[j]);
      }
      nt *= k[i];
      b *= e[i];
      continue;
    }
    e[i] = (n[i] + k[i] - 1) / k[i];
    if ((k[i] - 1) * e[i] >= n[i])
      return fail(ctx, JAGG_E_BLOCKING, "dimension %d: %lld cut into %d blocks of %lld leaves the last empty", i,
                  (long long)n[i], k[i], (long long)e[i]);
    nt *= k[i];
    b *= e[i];
  }
  *n_tuples = nt;
  *be = b;
  return JAGG_OK;
}

// tuple-id weight of dimension p (row-major over block coordinates)
int64_t tuple_w(const jagg_relation &R, int p) {
  int64_t w = 1;
  for (int q = p + 1; q < R.r; ++q) w *= R.k[q];
  return w;
}
// in-block stride of dimension p
int64_t inblock_s(const jagg_relation &R, int p) {
  int64_t s = 1;
  for (int q = p + 1; q < R.r; ++q) s *= R.e[q];
  return s;
}

// ------------------------------------------------------------ spec parsing
struct Spec {
  int n_in = 0;
  std::string in[kMaxIn];
  std::string out;
  std::string order;    // letters in order of first appearance
  std::string reduced;  // letters absent from the output, same order
};

jagg_status parse(jagg_ctx *ctx, const char *s, Spec &p) {
  if (!s) return fail(ctx, JAGG_E_INVALID, "NULL einsum string");
  const char *arrow = strstr(s, "->");
  if (!arrow) return fail(ctx, JAGG_E_INVALID, "einsum '%s' has no '->'", s);
  std::string cur;
  for (const char *c = s; c <= arrow; ++c) {
    if (c == arrow || *c == ',') {
      if (cur.empty()) return fail(ctx, JAGG_E_INVALID, "einsum '%s' has an empty operand", s);
      if (p.n_in >= kMaxIn) return fail(ctx, JAGG_E_UNSUPPORTED, "einsum '%s': more than %d inputs", s, kMaxIn);
      p.in[p.n_in++] = cur;
      cur.clear();
    } else if (*c >= 'a' && *c <= 'z') {
      cur.push_back(*c);
    } else {
      return fail(ctx, JAGG_E_INVALID, "einsum '%s': unexpected character '%c'", s, *c);
    }
  }
  for (const char *c = arrow + 2; *c; ++c) {
    if (*c < 'a' || *c > 'z') return fail(ctx, JAGG_E_INVALID, "einsum '%s': unexpected character '%c'", s, *c);
    p.out.push_back(*c);
  }
  for (int j = 0; j <= p.n_in; ++j) {
    const std::string &o = j < p.n_in ? p.in[j] : p.out;
    if (int(o.size()) > kMaxLetters)
      return fail(ctx, JAGG_E_UNSUPPORTED, "einsum '%s': operand with more than %d letters", s, kMaxLetters);
    for (size_t a = 0; a < o.size(); ++a)
      for (size_t b = a + 1; b < o.size(); ++b)
        if (o[a] == o[b]) return fail(ctx, JAGG_E_INVALID, "einsum '%s': letter '%c' repeats in an operand", s, o[a]);
  }
  for (int j = 0; j < p.n_in; ++j)
    for (char c : p.in[j])
      if (p.order.find(c) == std::string::npos) p.order.push_back(c);
  for (char c : p.out)
    if (p.order.find(c) == std::string::npos)
      return fail(ctx, JAGG_E_INVALID, "einsum '%s': output letter '%c' is in no input", s, c);
  for (char c : p.order)
    if (p.out.find(c) == std::string::npos) p.reduced.push_back(c);
  return JAGG_OK;
}

bool g_arity_ok(int g, int n) {
  switch (g) {
    case JAGG_G_MUL:
    case JAGG_G_ADD: return n >= 1;
    case JAGG_G_IDENT:
    case JAGG_G_SQUARE: return n == 1;
    case JAGG_G_EXP_SUB:
    case JAGG_G_SILU_MUL: return n == 2;
    case JAGG_G_EXP_SUB_DIV:
    case JAGG_G_RMS_SCALE:
    case JAGG_G_ATTENTION:
    case JAGG_G_MUL_PLUS:
    case JAGG_G_SWIGLU: return n == 3;
  }
  return false;
}

jagg_status check_spec(jagg_ctx *ctx, const jagg_spec *sp, const Spec &p) {
  if (sp->g < JAGG_G_MUL || sp->g > JAGG_G_SWIGLU) return fail(ctx, JAGG_E_INVALID, "unknown g %d", int(sp->g));
  if ((sp->g == JAGG_G_MUL_PLUS || sp->g == JAGG_G_SWIGLU) && (sp->agg != JAGG_AGG_SUM || sp->causal_s))
    return fail(ctx, JAGG_E_UNSUPPORTED, "g %d is a contraction with a recompose map: SUM, no causal pair",
                int(sp->g));
  if (sp->agg < JAGG_AGG_NONE || sp->agg > JAGG_AGG_SOFTMAX) return fail(ctx, JAGG_E_INVALID, "unknown aggregation");
  if ((sp->agg == JAGG_AGG_SOFTMAX) != (sp->g == JAGG_G_ATTENTION))
    return fail(ctx, JAGG_E_UNSUPPORTED, "the softmax-triple aggregation pairs only with g = ATTENTION");
  if (sp->out_dtype != JAGG_F32 && sp->out_dtype != JAGG_BF16) return fail(ctx, JAGG_E_INVALID, "unknown out dtype");
  if (!g_arity_ok(sp->g, p.n_in))
    return fail(ctx, JAGG_E_UNSUPPORTED, "g %d does not take %d inputs", int(sp->g), p.n_in);
  if (sp->agg == JAGG_AGG_NONE && !p.reduced.empty())
    return fail(ctx, JAGG_E_UNSUPPORTED, "letters '%s' are reduced but the aggregation is NONE", p.reduced.c_str());
  if ((sp->causal_s != 0) != (sp->causal_t != 0))
    return fail(ctx, JAGG_E_INVALID, "a causal pair needs both letters");
  if (sp->causal_s) {
    if (sp->causal_s == sp->causal_t) return fail(ctx, JAGG_E_INVALID, "causal letters must differ");
    if (p.order.find(sp->causal_s) == std::string::npos || p.order.find(sp->causal_t) == std::string::npos)
      return fail(ctx, JAGG_E_INVALID, "causal letters are not in the spec");
    if (p.out.find(sp->causal_s) == std::string::npos)
      return fail(ctx, JAGG_E_UNSUPPORTED, "causal letter s must be an output letter");
  }
  if ((sp->seg_s != 0) != (sp->seg_t != 0)) return fail(ctx, JAGG_E_INVALID, "a segment pair needs both letters");
  if (sp->seg_s) {
    if (sp->seg_s == sp->seg_t) return fail(ctx, JAGG_E_INVALID, "segment letters must differ");
    if (p.order.find(sp->seg_s) == std::string::npos || p.order.find(sp->seg_t) == std::string::npos)
      return fail(ctx, JAGG_E_INVALID, "segment letters are not in the spec");
    if (sp->g != JAGG_G_ATTENTION)
      return fail(ctx, JAGG_E_UNSUPPORTED, "a segment pair is taken by attention only");
    if (sp->causal_s && (sp->causal_s != sp->seg_s || sp->causal_t != sp->seg_t))
      return fail(ctx, JAGG_E_UNSUPPORTED, "the causal pair must be the segment pair");
  }
  return JAGG_OK;
}

// per-letter extents and block counts of a spec (index: letter - 'a')
struct LetterInfo {
  int64_t n[26];
  int32_t k[26];
};

// ------------------------------------------------------------ join
// Fills the join kernel's arguments from letters, extents and block counts.
jagg_status plan_join(jagg_ctx *ctx, const jagg_spec *sp, const Spec &p, const LetterInfo &L, JoinArgs &a) {
  memset(&a, 0, sizeof(a));
  a.n_in = p.n_in;
  a.n_out = int(p.out.size());
  a.n_red = int(p.reduced.size());
  int64_t n_keys = 1, per_key = 1;
  for (int i = 0; i < a.n_out; ++i) {
    const int c = p.out[i] - 'a';
    a.out_k[i] = L.k[c];
    a.out_div[i] = make_fastdiv(uint32_t(L.k[c]));
    n_keys *= L.k[c];
  }
  for (int i = 0; i < a.n_red; ++i) {
    const int c = p.reduced[i] - 'a';
    a.red_k[i] = L.k[c];
    a.red_div[i] = make_fastdiv(uint32_t(L.k[c]));
    per_key *= L.k[c];
  }
  if (n_keys * per_key > (int64_t(1) << 30))
    return fail(ctx, JAGG_E_UNSUPPORTED, "join of %lld tuples is too large", (long long)(n_keys * per_key));
  for (int j = 0; j < p.n_in; ++j) {
    const std::string &lt = p.in[j];
    for (size_t q = 0; q < lt.size(); ++q) {
      int64_t w = 1;
      for (size_t q2 = q + 1; q2 < lt.size(); ++q2) w *= L.k[lt[q2] - 'a'];
      const size_t io = p.out.find(lt[q]);
      if (io != std::string::npos) a.w_out[j][io] = w;
      const size_t ir = p.reduced.find(lt[q]);
      if (ir != std::string::npos) a.w_red[j][ir] = w;
    }
  }
  a.per_key = int32_t(per_key);
  a.n_keys = n_keys;
  // a causal or segment pair (s, t): locate both letters' block coordinates
  const char ps = sp->causal_s ? sp->causal_s : sp->seg_s, pt = sp->causal_s ? sp->causal_t : sp->seg_t;
  if (ps) {
    const int cs = ps - 'a', ct = pt - 'a';
    if (L.n[cs] != L.n[ct] || L.k[cs] != L.k[ct])
      return fail(ctx, JAGG_E_UNSUPPORTED, "causal or segment letters need equal extents and block counts");
    if (p.out.find(ps) == std::string::npos)
      return fail(ctx, JAGG_E_UNSUPPORTED, "the first letter of a causal or segment pair must be an output letter");
    a.causal = sp->causal_s ? 1 : 0;
    a.seg = sp->seg_s ? 1 : 0;
    a.s_red = 0;
    a.s_idx = int32_t(p.out.find(ps));
    const size_t to = p.out.find(pt);
    a.t_red = to == std::string::npos;
    a.t_idx = int32_t(a.t_red ? p.reduced.find(pt) : to);
    a.e_s = (L.n[cs] + L.k[cs] - 1) / L.k[cs];
    a.e_t = (L.n[ct] + L.k[ct] - 1) / L.k[ct];
    a.n_s = L.n[cs];
  }
  return JAGG_OK;
}

// ------------------------------------------------------------ relayout planner
struct Dim {
  int64_t ext, src, dst;
  int chk;
  int64_t xs;
};

int64_t largest_divisor_le(int64_t n, int64_t cap) {
  for (int64_t f = std::min(n, cap); f >= 1; --f)
    if (n % f == 0) return f;
  return 1;
}

// LDS-transposing plan for a digit permutation: the innermost dim is shared
// (stride 1 on both sides) but short, so one side would move it in short
// runs.  Dims whose source stride continues the source run are added to the
// box until the run reaches ~1 KB (the source chain), then dims continuing
// the destination run likewise (the destination chain); the box is read in
// source runs and written in destination runs.  Returns false when no such
// box of 1, 2, 4, 8 or 16 vectors per thread exists.
#ifndef JAGG_RELAYOUT_LDS
#define JAGG_RELAYOUT_LDS 1
#endif
constexpr bool kRelayoutLds = JAGG_RELAYOUT_LDS;
#ifndef JAGG_RELAYOUT_RUN_CAP
#define JAGG_RELAYOUT_RUN_CAP 2048
#endif
constexpr int64_t kRelayoutRunCap = JAGG_RELAYOUT_RUN_CAP;  // longest run a chain builds (bytes)
static bool plan_relayout_lds(const std::vector<Dim> &dims, int esz, int v, RelayoutArgs &a) {
  if (dims.size() < 2) return false;
  const Dim inner = dims.back();
  if (inner.src != 1 || inner.dst != 1 || inner.ext % v != 0 || inner.ext * esz >= 512) return false;
  std::vector<Dim> work(dims.begin(), dims.end() - 1);
  auto chain = [&](bool by_src, std::vector<Dim> &out) {
    int64_t run = inner.ext;
    while (run * esz < std::min<int64_t>(1024, kRelayoutRunCap) && int(out.size()) < kMaxChain) {
      int pick = -1;
      for (size_t i = 0; i < work.size(); ++i)
        if ((by_src ? work[i].src : work[i].dst) == run) pick = int(i);
      if (pick < 0) break;
      Dim d = work[pick];
      const int64_t f = largest_divisor_le(d.ext, std::max<int64_t>(1, kRelayoutRunCap / esz / run));
      if (f <= 1) break;
      Dim t = d;
      t.ext = f;
      out.push_back(t);
      if (f < d.ext) {
        work[pick].ext = d.ext / f;
        work[pick].src *= f;
        work[pick].dst *= f;
      } else {
        work.erase(work.begin() + pick);
      }
      run *= f;
    }
    return run;
  };
  std::vector<Dim> cs, cd;
  const int64_t s_run = chain(true, cs);
  const int64_t d_run = chain(false, cd);
  if (s_run * esz < 512 || d_run * esz < 512) return false;
  int64_t ncs = 1, ncd = 1;
  for (auto &d : cs) ncs *= d.ext;
  for (auto &d : cd) ncd *= d.ext;
  const int64_t vecs = inner.ext * ncs * ncd / v;
  if (vecs % 256 != 0) return false;
  const int64_t nv = vecs / 256;
  if (nv != 1 && nv != 2 && nv != 4 && nv != 8 && nv != 16) return false;
  // LDS: ncd source runs of s_run elements, each padded so that runs lie
  // inner-bytes apart modulo 256 (destination-order reads of 16 lanes then
  // cover distinct banks)
  const int64_t run_b = s_run * esz, in_b = inner.ext * esz;
  int64_t pad_b = 0;
  if (in_b < 256)
    while ((run_b + pad_b) % 256 != in_b % 256) pad_b += 16;
  const int64_t pitch = (run_b + pad_b) / esz;
  if (pitch * ncd * esz > 65536) return false;
  // in-box offsets must fit 32 bits
  int64_t smax = s_run, dmax = d_run;
  for (auto &d : cd) smax += (d.ext - 1) * d.src;
  for (auto &d : cs) dmax += (d.ext - 1) * d.dst;
  if (smax >= (int64_t(1) << 31) || dmax >= (int64_t(1) << 31)) return false;
  std::vector<Dim> outer;
  for (auto &d : work)
    if (d.ext > 1) outer.push_back(d);
  std::sort(outer.begin(), outer.end(), [](const Dim &x, const Dim &y) { return x.dst > y.dst; });
  if (int(outer.size()) > kMaxLdsOuter) return false;
  int64_t n_tiles = 1;
  for (auto &d : outer) n_tiles *= d.ext;
  if (n_tiles >= (int64_t(1) << 32)) return false;
  a.lds = 1;
  a.lds_nv = int32_t(nv);
  a.lds_v = v;
  a.lds_inner = int32_t(inner.ext);
  a.lds_pitch = int32_t(pitch);
  a.lds_R = make_fastdiv(uint32_t(s_run / v));
  a.lds_Rd = make_fastdiv(uint32_t(d_run / v));
  a.lds_iv = make_fastdiv(uint32_t(inner.ext / v));
  a.n_cs = int32_t(cs.size());
  a.n_cd = int32_t(cd.size());
  for (int i = 0; i < kMaxChain; ++i) {
    const bool s_on = i < int(cs.size()), d_on = i < int(cd.size());
    a.cs_div[i] = make_fastdiv(s_on ? uint32_t(cs[i].ext) : 1u);
    a.cs_dst[i] = s_on ? cs[i].dst : 0;
    a.cd_div[i] = make_fastdiv(d_on ? uint32_t(cd[i].ext) : 1u);
    a.cd_src[i] = d_on ? cd[i].src : 0;
  }
  a.lds_bytes = int32_t(pitch * ncd * esz);
  a.n_tile = int(outer.size());
  for (size_t i = 0; i < outer.size(); ++i)
    a.tile[i] = {outer[i].ext, outer[i].src, outer[i].dst, -1, 0, make_fastdiv(uint32_t(outer[i].ext))};
  for (int i = int(outer.size()); i < kMaxLdsOuter; ++i) a.tile[i] = {1, 0, 0, -1, 0, make_fastdiv(1)};
  a.n_lane = 0;
  if (n_tiles >= (int64_t(1) << 31)) return false;
  a.n_tiles = n_tiles;
  a.lanes = 256;
  return true;
}

jagg_status plan_relayout(jagg_ctx *ctx, const jagg_relation &S, const jagg_relation &D, RelayoutArgs &a,
                          int &vec_bytes) {
  memset(&a, 0, sizeof(a));
  const int r = D.r;
  const int64_t beS = S.be, beD = D.be;
  std::vector<Dim> kd, rd;
  int n_chk = 0;
  for (int p = 0; p < r; ++p) {
    const char c = D.letters[p];
    int q = 0;
    while (q < S.r && S.letters[q] != c) ++q;
    const int64_t n = D.n[p];
    const int64_t kD = D.k[p], eD = D.e[p], eS = S.e[q];
    const int64_t TKd = tuple_w(D, p) * beD, Ed = inblock_s(D, p);
    const int64_t TKs = tuple_w(S, q) * beS, Es = inblock_s(S, q);
    int slot = -1;
    auto need_slot = [&](int64_t rl, int64_t wl, bool irr) -> jagg_status {
      if (n_chk >= kMaxChk) return fail(ctx, JAGG_E_UNSUPPORTED, "too many padded letters");
      slot = n_chk++;
      a.read_lim[slot] = rl;
      a.write_lim[slot] = wl;
      a.irr[slot] = irr;
      if (irr) {
        a.irr_div[slot] = make_fastdiv(uint32_t(eS));
        a.irr_K[slot] = TKs;
        a.irr_E[slot] = Es;
      }
      return JAGG_OK;
    };
    jagg_status st = JAGG_OK;
    if (eD == eS) {
      if (kD * eD > n) st = need_slot(n, kD * eD, false);
      kd.push_back({kD, TKs, TKd, slot, eD});
      rd.push_back({eD, Es, Ed, slot, 1});
    } else if (eD % eS == 0) {
      const int64_t m = eD / eS;
      if (kD * eD > n) st = need_slot(n, kD * eD, false);
      kd.push_back({kD, m * TKs, TKd, slot, eD});
      rd.push_back({m, TKs, eS * Ed, slot, eS});
      rd.push_back({eS, Es, Ed, slot, 1});
    } else if (eS % eD == 0) {
      const int64_t m = eS / eD;
      const int64_t kh = (kD + m - 1) / m;
      if (kh * m * eD > n) st = need_slot(n, kD * eD, false);
      kd.push_back({kh, TKs, m * TKd, slot, eS});
      kd.push_back({m, eD * Es, TKd, slot, eD});
      rd.push_back({eD, Es, Ed, slot, 1});
    } else {
      st = need_slot(n, kD * eD, true);
      kd.push_back({kD, 0, TKd, slot, eD});
      rd.push_back({eD, 0, Ed, slot, 1});
    }
    if (st != JAGG_OK) return st;
  }
  a.n_chk = n_chk;
  std::vector<Dim> dims;
  for (auto &d : kd)
    if (d.ext > 1) dims.push_back(d);
  for (auto &d : rd)
    if (d.ext > 1) dims.push_back(d);
  if (dims.empty()) dims.push_back({1, 0, 0, -1, 0});
  // merge neighbours that walk both sides contiguously
  for (size_t i = dims.size() - 1; i >= 1 && i < dims.size(); --i) {
    Dim &o = dims[i - 1], &in = dims[i];
    const bool x_ok = (o.chk == -1 && in.chk == -1) || (o.chk == in.chk && o.xs == in.ext * in.xs);
    if (o.src == in.ext * in.src && o.dst == in.ext * in.dst && x_ok) {
      Dim m = in;
      m.ext = o.ext * in.ext;
      dims[i - 1] = m;
      dims.erase(dims.begin() + i);
    }
  }
  // vector width along the innermost destination dim
  const int esz = esz_of(D.dt);
  const Dim &inner = dims.back();
  int v = 16 / esz;
  for (; v > 1; v >>= 1) {
    bool ok = inner.dst == 1 && inner.ext % v == 0;
    if (inner.chk >= 0 && a.irr[inner.chk]) {
      ok = ok && a.irr_E[inner.chk] == 1 && a.irr_div[inner.chk].d % v == 0 && a.irr_K[inner.chk] % v == 0;
    } else {
      ok = ok && inner.src == 1;
    }
    if (inner.chk >= 0) ok = ok && a.read_lim[inner.chk] % v == 0 && a.write_lim[inner.chk] % v == 0;
    for (size_t i = 0; i + 1 < dims.size(); ++i) ok = ok && dims[i].src % v == 0 && dims[i].dst % v == 0;
    for (int c = 0; c < n_chk; ++c)
      if (a.irr[c]) ok = ok && a.irr_K[c] % v == 0 && (a.irr_E[c] % v == 0 || (inner.chk == c));
    if (ok) break;
  }
  vec_bytes = v * esz;
  a.src = S.buf;
  a.dst = D.buf;
  if (kRelayoutLds && n_chk == 0 && v * esz == 16 && plan_relayout_lds(dims, esz, v, a)) {
    if (ctx->trace) {
      fprintf(stderr, "[jagg] relayout %s -> %s: lds transpose, %d vectors/thread, %d B LDS, %lld boxes | run %d x %d, runs %u / %u vectors |",
              S.letters, D.letters, a.lds_nv, a.lds_bytes, (long long)a.n_tiles, a.lds_inner, a.lds_v, a.lds_R.d,
              a.lds_Rd.d);
      for (int i = 0; i < a.n_cs; ++i) fprintf(stderr, " S(%u d%lld)", a.cs_div[i].d, (long long)a.cs_dst[i]);
      for (int i = 0; i < a.n_cd; ++i) fprintf(stderr, " D(%u s%lld)", a.cd_div[i].d, (long long)a.cd_src[i]);
      for (int i = 0; i < a.n_tile; ++i)
        fprintf(stderr, " T(%lld s%lld d%lld)", (long long)a.tile[i].ext, (long long)a.tile[i].src,
                (long long)a.tile[i].dst);
      fprintf(stderr, "\n");
    }
    return JAGG_OK;
  }
  // lane dims: the vectorised inner dim, then dims that extend contiguity
  std::vector<Dim> lane, rest(dims.begin(), dims.end() - 1);
  int64_t lanes = 1;
  {
    Dim in = inner;
    const int64_t ev = in.ext / v;
    const int64_t f = largest_divisor_le(ev, 256);
    Dim l = in;
    l.ext = f;
    lane.push_back(l);
    lanes = f;
    if (f < ev) {
      Dim o = in;
      o.ext = ev / f;
      o.src *= f * v;
      o.dst *= f * v;
      o.xs *= f * v;
      rest.push_back(o);
    }
  }
  int64_t src_run = lane[0].src == 1 ? lane[0].ext * v : 0;
  while (lanes < 256 && !rest.empty()) {
    int pick = -1;
    for (size_t i = 0; i < rest.size(); ++i)
      if (src_run > 0 && rest[i].src == src_run) pick = int(i);
    if (pick < 0) {
      int64_t best = -1;
      for (size_t i = 0; i < rest.size(); ++i)
        if (best < 0 || rest[i].dst < best) {
          best = rest[i].dst;
          pick = int(i);
        }
    }
    Dim d = rest[pick];
    const int64_t f = largest_divisor_le(d.ext, 256 / lanes);
    if (f <= 1) break;
    Dim l = d;
    l.ext = f;
    lane.push_back(l);
    lanes *= f;
    if (src_run > 0 && d.src == src_run) src_run *= f;
    if (f < d.ext) {
      rest[pick].ext = d.ext / f;
      rest[pick].src *= f;
      rest[pick].dst *= f;
      rest[pick].xs *= f;
    } else {
      rest.erase(rest.begin() + pick);
    }
  }
  std::sort(rest.begin(), rest.end(), [](const Dim &x, const Dim &y) { return x.dst > y.dst; });
  if (int(rest.size()) > kMaxDims || int(lane.size()) > kMaxDims)
    return fail(ctx, JAGG_E_UNSUPPORTED, "repartition needs too many dims");
  int64_t n_tiles = 1;
  for (auto &d : rest) n_tiles *= d.ext;
  if (n_tiles >= (int64_t(1) << 32)) return fail(ctx, JAGG_E_UNSUPPORTED, "repartition too large");
  a.n_tile = int(rest.size());
  for (size_t i = 0; i < rest.size(); ++i) {
    a.tile[i] = {rest[i].ext, rest[i].src, rest[i].dst, rest[i].chk, rest[i].xs, make_fastdiv(uint32_t(rest[i].ext))};
  }
  a.n_lane = int(lane.size());
  for (size_t i = 0; i < lane.size(); ++i)
    a.lane[i] = {lane[i].ext, lane[i].src, lane[i].dst, lane[i].chk, lane[i].xs, make_fastdiv(uint32_t(lane[i].ext))};
  // the kernels count tiles in 32 bits
  if (n_tiles >= (int64_t(1) << 31))
    return fail(ctx, JAGG_E_UNSUPPORTED, "relayout of %lld tiles of %lld vectors exceeds 2^31 tiles",
                (long long)n_tiles, (long long)lanes);
  a.n_tiles = n_tiles;
  a.lanes = int32_t(lanes);
  a.src = S.buf;
  a.dst = D.buf;
  if (ctx->trace) {
    fprintf(stderr, "[jagg] relayout %s -> %s: vec %dB lanes %lld tiles %lld chk %d |", S.letters, D.letters, vec_bytes,
            (long long)lanes, (long long)n_tiles, n_chk);
    for (auto &d : lane) fprintf(stderr, " L(%lld s%lld d%lld)", (long long)d.ext, (long long)d.src, (long long)d.dst);
    for (auto &d : rest) fprintf(stderr, " T(%lld s%lld d%lld)", (long long)d.ext, (long long)d.src, (long long)d.dst);
    fprintf(stderr, "\n");
  }
  return JAGG_OK;
}

// Launch of a map or reduce: the vectorised stream kernels where the spec's
// layout allows them, the general ones otherwise.
// Flat-stream plan: every row letter unpadded, every operand's row offset a
// multiple of the row index, blocks under 2 GiB and 16-byte aligned.
// Returns false when the general kernels must run instead.
bool plan_flat(const EwArgs &a, FlatArgs &f, int &vec, int &lpr) {
  memset(&f, 0, sizeof(f));
  const bool map = a.agg == JAGG_AGG_NONE;
  const int r = a.r_out;
  const int nrow = map ? r - 1 : r;  // row letters
  const int64_t lim31 = (int64_t(1) << 31) - 1;
  auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // row strides of the output walk
  int64_t R[kMaxLetters];
  int64_t rows = 1;
  for (int i = nrow - 1; i >= 0; --i) {
    R[i] = rows;
    rows *= a.e_out[i];
    if (a.n_out[i] % a.e_out[i] != 0) return false;  // padded rows
  }
  const int64_t e_in = map ? a.e_out[r - 1] : a.e_red[0];  // walk's innermost extent
  if (map) {
    if (e_in % 8 != 0) return false;
    vec = 8;
  } else {
    if (a.n_red != 1 || a.inner_red != 0 || a.s_red[0][0] != 1) return false;
    vec = e_in % 4 == 0 ? 4 : 1;
  }
  f.n_in = a.n_in;
  for (int j = 0; j < a.n_in; ++j) {
    const int esz = a.in_dt[j] ? 2 : 4;
    const int64_t inner = map ? a.s_out[j][r - 1] : a.s_red[j][0];
    if (inner != 0 && inner != 1) return false;
    if (!map && j == 0 && inner != 1) return false;
    int64_t m = 0;
    for (int i = 0; i < nrow; ++i)
      if (a.s_out[j][i] != 0) m = a.s_out[j][i] / R[i];
    for (int i = 0; i < nrow; ++i)
      if (a.s_out[j][i] != m * R[i]) return false;
    const int64_t bytes = a.be_in[j] * esz;
    if (bytes > lim31 || (bytes % 16) != 0 || !aligned(a.in[j])) return false;
    if (inner && map && (m * esz) % 16 != 0) return false;
    if (inner && !map && vec == 4 && m % 4 != 0) vec = 1;
    f.in[j].p = a.in[j];
    f.in[j].block_bytes = uint32_t(bytes);
    f.in[j].dt = a.in_dt[j];
    f.in[j].inner = int32_t(inner);
    f.in[j].row_mul = int32_t(m);
  }
  for (int j = a.n_in; j < kMaxIn; ++j) f.in[j].p = a.in[0];  // block_bytes 0: every load reads zeros
  const int oesz = a.out_dt ? 2 : 4;
  if (a.be_out > lim31 || (a.be_out * oesz) % 16 != 0 || !aligned(a.out)) return false;
  if (a.n_keys > lim31) return false;
  f.out = a.out;
  f.out_dt = a.out_dt;
  f.alpha = a.alpha;
  f.beta = a.beta;
  f.eps = a.eps;
  f.list = a.list;
  f.counts = a.counts;
  f.per_key = a.per_key;
  f.n_keys = int32_t(a.n_keys);
  f.be_out = int32_t(a.be_out);
  // causal pair: s a row letter, t the walk's innermost letter
  if (a.causal) {
    if (map ? (a.t_red_flag || a.t_pos != r - 1 || a.s_pos >= r - 1) : (!a.t_red_flag || a.t_pos != 0)) return false;
    const int sp = a.s_pos;
    int64_t W = 1;
    for (int i = sp + 1; i < r; ++i) W *= a.k_out[i];
    f.causal = 1;
    f.e_s = int32_t(a.e_out[sp]);
    f.k_s = int32_t(a.k_out[sp]);
    f.div_Rs = make_fastdiv(uint32_t(R[sp]));
    f.div_es = make_fastdiv(uint32_t(a.e_out[sp]));
    f.div_Ws = make_fastdiv(uint32_t(W));
    f.div_ks = make_fastdiv(uint32_t(a.k_out[sp]));
  }
  int64_t chunks;
  if (map) {
    const int64_t slots = rows * (e_in / 8);
    if (slots > lim31) return false;
    f.slots = int32_t(slots);
    f.vpr = int32_t(e_in / 8);
    f.div_vpr = make_fastdiv(uint32_t(f.vpr));
    f.e_last = int32_t(e_in);
    f.n_last = int32_t(a.n_out[r - 1]);
    f.k_last = int32_t(a.k_out[r - 1]);
    f.div_klast = make_fastdiv(uint32_t(f.k_last));
    chunks = (slots + 1023) / 1024;  // two passes of two vectors per thread
  } else {
    lpr = 4;
    while (lpr < 64 && lpr * 2 <= e_in / vec) lpr *= 2;
    const int64_t groups = 256 / lpr;
    const int64_t per_key = (a.be_out + groups - 1) / groups;
    int64_t cap = 8192 / (a.n_keys > 0 ? a.n_keys : 1);
    chunks = per_key < cap ? per_key : (cap < 1 ? 1 : cap);
    f.e_red = int32_t(a.e_red[0]);
    f.n_red = int32_t(a.n_red_ext[0]);
    f.k_red = int32_t(a.k_red[0]);
    f.div_wred = make_fastdiv(uint32_t(a.w_red0[0]));
    f.div_kred = make_fastdiv(uint32_t(a.k_red[0]));
  }
  if (chunks < 1) chunks = 1;
  if (chunks * a.n_keys > lim31) return false;
  f.chunks = int32_t(chunks);
  f.div_chunks = make_fastdiv(uint32_t(chunks));
  return true;
}

hipError_t launch_ew(jagg_ctx *ctx, const EwArgs &a, int agg, const char **which) {
  {
    FlatArgs f;
    int vec = 1, lpr = 4;
    if (plan_flat(a, f, vec, lpr)) {
      if (agg == JAGG_AGG_NONE) {
        *which = "flat map";
        return launch_flat_map(f, a.g, ctx->stream);
      }
      *which = "flat reduce";
      return launch_flat_reduce(f, vec, lpr, a.g, agg, ctx->stream);
    }
  }
  StreamArgs sa;
  memset(&sa, 0, sizeof(sa));
  const int r = a.r_out;
  for (int i = 0; i < r; ++i) sa.div_out[i] = make_fastdiv(uint32_t(a.e_out[i]));
  if (agg == JAGG_AGG_NONE) {
    const int64_t e_last = a.e_out[r - 1];
    int vec = 1;
    for (int v : {8, 4}) {
      bool ok = e_last % v == 0 && a.be_out % v == 0;
      for (int j = 0; j < a.n_in; ++j) {
        const int64_t sl = a.s_out[j][r - 1];
        if (sl == 1) {
          ok = ok && a.be_in[j] % v == 0;
          for (int i = 0; i < r - 1; ++i) ok = ok && a.s_out[j][i] % v == 0;
        }
      }
      if (ok) {
        vec = v;
        break;
      }
    }
    sa.slots = a.rows_per_block * (e_last / vec);
    sa.div_vpr = make_fastdiv(uint32_t(e_last / vec));
    int64_t chunks = (sa.slots + 1023) / 1024;  // about one pass of four slots per thread
    sa.chunks = chunks < 1 ? 1 : chunks;
    *which = vec == 8 ? "map x8" : (vec == 4 ? "map x4" : "map x1");
    return launch_map_vec(a, sa, vec, ctx->stream);
  }
  // row reduce: one reduced letter, innermost in input 0; other inputs hold
  // it innermost or not at all; at most 256 joined tuples per key
  bool row = a.n_red == 1 && a.inner_red == 0 && a.per_key <= 256 && (!a.causal || a.t_red_flag);
  int vec = a.e_red[0] % 4 == 0 ? 4 : 1;
  for (int j = 0; j < a.n_in && row; ++j) {
    const int64_t sr = a.s_red[j][0];
    row = row && (sr == 0 || sr == 1);
    if (sr == 1 && (a.be_in[j] % 4 != 0)) vec = 1;
  }
  if (row) {
    int lpr = 4;
    while (lpr < 64 && lpr * 2 <= a.e_red[0] / vec) lpr *= 2;
    const int groups = 256 / lpr;
    int64_t per_key_groups = (a.be_out + groups - 1) / groups;
    int64_t cap = 4096 / (a.n_keys > 0 ? a.n_keys : 1);
    if (cap < 1) cap = 1;
    sa.chunks = per_key_groups < cap ? per_key_groups : cap;
    *which = "reduce rows";
    return launch_reduce_row(a, sa, vec, lpr, ctx->stream);
  }
  *which = "reduce general";
  return launch_reduce(a, ctx->stream);
}

jagg_status after_launch(jagg_ctx *ctx, hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(ctx, JAGG_E_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (ctx->debug_sync && !ctx->capturing) {
    e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return fail(ctx, JAGG_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  }
  return JAGG_OK;
}

#ifndef JAGG_IV_ROWS
#define JAGG_IV_ROWS 1
#endif
constexpr bool kIvRows = JAGG_IV_ROWS;

bool has_intervals(const jagg_relation &R) {
  for (int q = 0; q < R.r; ++q)
    if (R.iv[q]) return true;
  return false;
}

// Interval relayout plan: per destination letter its destination geometry
// and where its index lands in the source; the bounds of interval letters go
// to a shared pool.  Vectors run along the innermost destination letter when
// it is innermost in the source too and every bound of it, on both sides, is
// a multiple of the width (so no vector straddles a block or padding edge).
jagg_status plan_relayout_iv(jagg_ctx *ctx, const jagg_relation &S, const jagg_relation &D, IvRelayoutArgs &a,
                             int &vec_bytes) {
  memset(&a, 0, sizeof(a));
  a.src = S.buf;
  a.dst = D.buf;
  a.r = D.r;
  int pool = 0;
  auto put = [&](const jagg_relation &R, int q) -> int {
    if (!R.iv[q]) return -1;
    if (pool + R.k[q] + 1 > kIvPool) return -2;
    const int off = pool;
    for (int i = 0; i <= R.k[q]; ++i) a.pool[pool++] = int32_t(R.bnd[q][i]);
    return off;
  };
  for (int p = 0; p < D.r; ++p) {
    const int q = int(strchr(S.letters, D.letters[p]) - S.letters);
    IvRelayoutDim &d = a.d[p];
    d.dk = make_fastdiv(uint32_t(D.k[p]));
    d.de = make_fastdiv(uint32_t(D.e[p]));
    d.n = int32_t(D.n[p]);
    d.d_bnd = put(D, p);
    d.s_bnd = put(S, q);
    if (d.d_bnd == -2 || d.s_bnd == -2)
      return fail(ctx, JAGG_E_UNSUPPORTED, "more than %d interval bounds in one repartition", kIvPool);
    d.s_k = S.k[q];
    d.s_e = make_fastdiv(uint32_t(S.e[q]));
    d.s_tw = uint32_t(tuple_w(S, q) * S.be);
    d.s_ew = uint32_t(inblock_s(S, q));
  }
  a.n_pool = pool;
  const int esz = esz_of(D.dt);
  const int pi = D.r - 1;
  const int qi = int(strchr(S.letters, D.letters[pi]) - S.letters);
  int v = 16 / esz;
  for (; v > 1; v >>= 1) {
    bool ok = qi == S.r - 1 && D.n[pi] % v == 0 && D.e[pi] % v == 0 && S.e[qi] % v == 0;
    for (int i = 0; ok && D.iv[pi] && i <= D.k[pi]; ++i) ok = D.bnd[pi][i] % v == 0;
    for (int i = 0; ok && S.iv[qi] && i <= S.k[qi]; ++i) ok = S.bnd[qi][i] % v == 0;
    if (ok) break;
  }
  a.v = v;
  // the interval kernels index both relations with 32-bit element offsets
  if (S.n_tuples * S.be >= (int64_t(1) << 31) || D.n_tuples * D.be >= (int64_t(1) << 31))
    return fail(ctx, JAGG_E_UNSUPPORTED, "an interval relayout takes relations under 2^31 elements");
  a.n_vec = uint32_t(D.n_tuples * D.be / v);
  a.be_v = make_fastdiv(uint32_t(D.be / v));
  vec_bytes = v * esz;
  // rows of at least a wave's worth of vectors take the row form
  a.row_vecs = uint32_t(D.e[pi] / v);
  a.rows = kIvRows && a.row_vecs >= 64;
  a.n_rows = uint32_t(D.n_tuples * (D.be / D.e[pi]));
  a.rows_pt = make_fastdiv(uint32_t(D.be / D.e[pi]));
  if (ctx->trace)
    fprintf(stderr, "[jagg] relayout %s -> %s: intervals, %d-element vectors, %u vectors, %d bounds%s\n", S.letters,
            D.letters, v, a.n_vec, pool, a.rows ? ", rows" : "");
  return JAGG_OK;
}

jagg_status do_repartition(jagg_ctx *ctx, const jagg_relation &S, const jagg_relation &D) {
  if (has_intervals(S) || has_intervals(D)) {
    IvRelayoutArgs ia;
    int vb = 0;
    jagg_status st = plan_relayout_iv(ctx, S, D, ia, vb);
    if (st != JAGG_OK) return st;
    return after_launch(ctx, launch_relayout_iv(ia, vb, ctx->stream), "interval relayout");
  }
  RelayoutArgs a;
  int vb = 0;
  jagg_status st = plan_relayout(ctx, S, D, a, vb);
  if (st != JAGG_OK) return st;
  return after_launch(ctx, launch_relayout(a, vb, esz_of(D.dt), ctx->stream), "relayout");
}

// ------------------------------------------------------------ einsum binding
struct Bound {
  Spec p;
  LetterInfo L;
  const jagg_relation *in[kMaxIn];  // the inputs as the kernels see them (see shadow)
  // Interval-blocked letters (iv_letter[c]) run as uniform letters of
  // extent k * e (e the longest interval): every block is a full uniform
  // block whose padding holds +0, and the shadows below carry that view.
  bool iv_letter[26];
  const int64_t *iv_bnd[26];
  jagg_relation shadow[kMaxIn];
  bool needs_reblock[kMaxIn];
  size_t list_bytes, counts_bytes, reblock_bytes[kMaxIn], total;
  int split = 1;            // parts of a split contraction walk (1: none)
  size_t split_bytes = 0;   // workspace for their fp32 partial sums
  JoinArgs join;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Interval letters of a spec: every relation holding such a letter must
// carry the same bounds, and the requested block count must be theirs (a
// relation blocked otherwise is repartitioned by the caller first).  The
// kernels then compute the padding too, so only specs whose value is +0
// wherever an interval letter sits in its padding are taken: g = MUL, IDENT,
// SQUARE or SILU_MUL (a zero factor), ADD when every input holds every
// interval letter, RMS_SCALE when its first input does and eps > 0; MAX only over
// uniform letters; no causal pair on interval letters.  Attention takes
// intervals on its segment pair only (packed sequences): its kernel masks
// each block by the length of its own interval.
jagg_status bind_intervals(jagg_ctx *ctx, const jagg_spec *sp, const jagg_relation *const *in, int n_in, Bound &b) {
  bool any = false;
  for (int c = 0; c < 26; ++c) {
    b.iv_letter[c] = false;
    b.iv_bnd[c] = nullptr;
  }
  for (int j = 0; j < n_in; ++j)
    for (int q = 0; q < in[j]->r; ++q)
      if (in[j]->iv[q]) {
        b.iv_letter[b.p.in[j][q] - 'a'] = true;
        any = true;
      }
  for (int j = 0; j < n_in; ++j) b.in[j] = in[j];
  if (!any) return JAGG_OK;
  for (int j = 0; j < n_in; ++j) {
    const jagg_relation *R = in[j];
    for (int q = 0; q < R->r; ++q) {
      const int c = b.p.in[j][q] - 'a';
      if (!b.iv_letter[c]) continue;
      if (!R->iv[q])
        return fail(ctx, JAGG_E_BLOCKING, "letter '%c' is interval-blocked in one input and uniform in input %d",
                    'a' + c, j);
      if (R->k[q] != b.L.k[c])
        return fail(ctx, JAGG_E_BLOCKING, "letter '%c' holds %d intervals, the spec asks %d blocks", 'a' + c, R->k[q],
                    b.L.k[c]);
      if (!b.iv_bnd[c]) {
        b.iv_bnd[c] = R->bnd[q];
      } else if (memcmp(b.iv_bnd[c], R->bnd[q], sizeof(int64_t) * size_t(R->k[q] + 1)) != 0) {
        return fail(ctx, JAGG_E_BLOCKING, "letter '%c' has different bounds in two inputs", 'a' + c);
      }
    }
  }
  auto is_iv = [&](char c) { return b.iv_letter[c - 'a']; };
  if (sp->g == JAGG_G_ATTENTION) {
    // packed sequences: intervals only on the segment pair (s, t), which the
    // attention kernel masks by each block's own length
    if (!sp->seg_s)
      return fail(ctx, JAGG_E_UNSUPPORTED, "attention over interval-blocked letters needs a segment pair (s, t)");
    for (int c = 0; c < 26; ++c)
      if (b.iv_letter[c] && c != sp->seg_s - 'a' && c != sp->seg_t - 'a')
        return fail(ctx, JAGG_E_UNSUPPORTED, "attention: '%c' is interval-blocked but not a segment letter", 'a' + c);
    const int cs = sp->seg_s - 'a', ct = sp->seg_t - 'a';
    if (!is_iv(sp->seg_s) || !is_iv(sp->seg_t) || b.L.k[cs] != b.L.k[ct] ||
        memcmp(b.iv_bnd[cs], b.iv_bnd[ct], sizeof(int64_t) * size_t(b.L.k[cs] + 1)) != 0)
      return fail(ctx, JAGG_E_BLOCKING, "segment letters must be blocked by the same bounds");
  } else {
    if (sp->causal_s && (is_iv(sp->causal_s) || is_iv(sp->causal_t)))
      return fail(ctx, JAGG_E_UNSUPPORTED, "causal letters must be uniformly blocked");
    if (sp->g == JAGG_G_EXP_SUB || sp->g == JAGG_G_EXP_SUB_DIV)
      return fail(ctx, JAGG_E_UNSUPPORTED, "g %d is not zero on padding; interval letters need it", int(sp->g));
    if (sp->agg == JAGG_AGG_MAX)
      for (char c : b.p.reduced)
        if (is_iv(c)) return fail(ctx, JAGG_E_UNSUPPORTED, "MAX over the interval-blocked letter '%c'", c);
    // padded rows of an RMS scale see x0 = 0 and a sum of squares of 0:
    // 0 * rsqrt(eps) is +0 only for eps > 0
    if (sp->g == JAGG_G_RMS_SCALE && !(sp->eps > 0.0f))
      return fail(ctx, JAGG_E_UNSUPPORTED, "RMS_SCALE over interval-blocked letters needs eps > 0");
    for (int c = 0; c < 26; ++c) {
      if (!b.iv_letter[c]) continue;
      const int first = sp->g == JAGG_G_RMS_SCALE ? 1 : (sp->g == JAGG_G_ADD ? n_in : 0);
      for (int j = 0; j < first; ++j)
        if (b.p.in[j].find(char('a' + c)) == std::string::npos)
          return fail(ctx, JAGG_E_UNSUPPORTED, "g %d needs the interval-blocked letter '%c' in input %d", int(sp->g),
                      'a' + c, j);
    }
  }
  for (int j = 0; j < n_in; ++j) {
    jagg_relation &T = b.shadow[j];
    T = *in[j];
    for (int q = 0; q < T.r; ++q)
      if (T.iv[q]) {
        T.n[q] = int64_t(T.k[q]) * T.e[q];
        T.iv[q] = 0;
      }
    b.in[j] = &T;
  }
  for (int c = 0; c < 26; ++c)
    if (b.iv_letter[c]) {
      for (int j = 0; j < n_in; ++j) {
        const size_t q = b.p.in[j].find(char('a' + c));
        if (q != std::string::npos) {
          b.L.n[c] = b.shadow[j].n[q];
          break;
        }
      }
    }
  return JAGG_OK;
}

// Parts of a contraction's walk over (joined tuple, K-step of 32) run by
// separate workgroups when its 256 x 256 tiles fill the chip's 256 CUs in
// few or ragged waves (a chain product with a thin output and a deep
// reduction): each part writes fp32 partial sums and a sum kernel adds them
// in order.  The count minimises a cost in units of one K-step of a tile:
// waves(tiles x S) x (steps / S + 8 for a workgroup's start and end), plus,
// for S > 1, the partials written and read again (8 S bytes per output
// element, about 3 MB per unit at the copy rate).  At least 16 steps a
// part, and a split only where the estimate gains at least 5%: below that
// the estimate's error decides, and a split plan no longer shares a grouped
// launch (three 2.25-wave products of one chain, estimated 2.5% faster
// split, measured 4% slower as three split launches than as one group).
int split_parts(int64_t tiles, int64_t steps, int64_t out_elems) {
  constexpr int64_t kCUs = 256;
  if (tiles <= 0 || steps <= 0) return 1;
  double t1 = 0.0, best = 0.0;
  int best_s = 1;
  for (int S = 1; S <= 16; S *= 2) {
    if (S > 1 && steps / S < 16) break;
    double t = double((tiles * S + kCUs - 1) / kCUs) * (double(steps) / S + 8.0);
    if (S > 1) t += 8.0 * S * double(out_elems) / 3.0e6;
    if (S == 1) t1 = t;
    if (S == 1 || t < best) {
      best = t;
      best_s = S;
    }
  }
  return best < 0.95 * t1 ? best_s : 1;
}

// The split of a bf16 MUL / SUM contraction without a causal or segment pair
// or interval letters, counted as the 256 x 256 kernel tiles it (the kernel
// may still decline, e.g. for operands without 16-byte vectors; the space
// then goes unused).
void plan_split(const jagg_spec *sp, const jagg_relation *const *in, int n_in, Bound &b) {
  b.split = 1;
  b.split_bytes = 0;
  if (n_in != 2 || sp->g != JAGG_G_MUL || sp->agg != JAGG_AGG_SUM || sp->causal_s || sp->seg_s) return;
  if (in[0]->dt != JAGG_BF16 || in[1]->dt != JAGG_BF16) return;
  for (int c = 0; c < 26; ++c)
    if (b.iv_letter[c]) return;
  const Spec &p = b.p;
  if (p.reduced.empty()) return;
  auto e = [&](char c) { return (b.L.n[c - 'a'] + b.L.k[c - 'a'] - 1) / b.L.k[c - 'a']; };
  int64_t M = 1, N = 1, Bt = 1, K = 1, be_out = 1;
  bool m_any = false, n_any = false;
  for (char c : p.reduced) {
    if (p.in[0].find(c) == std::string::npos || p.in[1].find(c) == std::string::npos) return;
    K *= e(c);
  }
  for (char c : p.out) {
    const bool i0 = p.in[0].find(c) != std::string::npos, i1 = p.in[1].find(c) != std::string::npos;
    if (i0 && i1) Bt *= e(c);
    else if (i0) M *= e(c), m_any = true;
    else N *= e(c), n_any = true;
    be_out *= e(c);
  }
  if (!m_any || !n_any || M < 256 || N < 256) return;
  const int64_t tiles = b.join.n_keys * Bt * ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t steps = int64_t(b.join.per_key) * ((K + 31) / 32);
  const int64_t out_elems = b.join.n_keys * be_out;
  if (out_elems >= (int64_t(1) << 29)) return;  // each part addressed with 32-bit byte offsets
  const int S = split_parts(tiles, steps, out_elems);
  if (S <= 1) return;
  b.split = S;
  b.split_bytes = align256(size_t(S) * size_t((out_elems + 63) / 64 * 64) * 4);
}

jagg_status bind(jagg_ctx *ctx, const jagg_spec *sp, const jagg_relation *const *in, int n_in,
                 const int32_t *blockings, Bound &b) {
  if (!sp || !in || !blockings) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  jagg_status st = parse(ctx, sp->einsum, b.p);
  if (st != JAGG_OK) return st;
  if (n_in != b.p.n_in)
    return fail(ctx, JAGG_E_INVALID, "einsum has %d inputs, %d relations given", b.p.n_in, n_in);
  if ((st = check_spec(ctx, sp, b.p)) != JAGG_OK) return st;
  for (int i = 0; i < 26; ++i) {
    b.L.n[i] = 0;
    b.L.k[i] = 0;
  }
  for (size_t i = 0; i < b.p.order.size(); ++i) {
    if (blockings[i] < 1) return fail(ctx, JAGG_E_BLOCKING, "blocking of '%c' must be >= 1", b.p.order[i]);
    b.L.k[b.p.order[i] - 'a'] = blockings[i];
  }
  for (int j = 0; j < n_in; ++j) {
    const jagg_relation *R = in[j];
    if (!R) return fail(ctx, JAGG_E_INVALID, "input %d is NULL", j);
    b.in[j] = R;
    if (R->r != int(b.p.in[j].size()))
      return fail(ctx, JAGG_E_SHAPE, "input %d has %d dimensions, operand '%s' names %d", j, R->r,
                  b.p.in[j].c_str(), int(b.p.in[j].size()));
    b.needs_reblock[j] = false;
    for (int q = 0; q < R->r; ++q) {
      const int c = b.p.in[j][q] - 'a';
      if (b.L.n[c] == 0) b.L.n[c] = R->n[q];
      if (b.L.n[c] != R->n[q])
        return fail(ctx, JAGG_E_SHAPE, "letter '%c' has extent %lld and %lld", 'a' + c, (long long)b.L.n[c],
                    (long long)R->n[q]);
      if (R->k[q] != b.L.k[c]) b.needs_reblock[j] = true;
    }
  }
  if ((st = bind_intervals(ctx, sp, in, n_in, b)) != JAGG_OK) return st;
  // the requested blocking must be valid for every letter
  for (char c : b.p.order) {
    const int i = c - 'a';
    const int64_t e = (b.L.n[i] + b.L.k[i] - 1) / b.L.k[i];
    if (b.L.k[i] > b.L.n[i] || (b.L.k[i] - 1) * e >= b.L.n[i])
      return fail(ctx, JAGG_E_BLOCKING, "letter '%c': %lld cut into %d blocks leaves an empty block", c,
                  (long long)b.L.n[i], b.L.k[i]);
  }
  if ((st = plan_join(ctx, sp, b.p, b.L, b.join)) != JAGG_OK) return st;
  b.list_bytes = align256(size_t(b.join.n_keys) * b.join.per_key * (1 + n_in) * 4);
  b.counts_bytes = align256(size_t(b.join.n_keys) * 4);
  b.total = b.list_bytes + b.counts_bytes;
  for (int j = 0; j < n_in; ++j) {
    b.reblock_bytes[j] = 0;
    if (b.needs_reblock[j]) {
      int64_t nt = 1, be = 1;
      for (int q = 0; q < in[j]->r; ++q) {
        const int c = b.p.in[j][q] - 'a';
        const int64_t e = (b.L.n[c] + b.L.k[c] - 1) / b.L.k[c];
        nt *= b.L.k[c];
        be *= e;
      }
      b.reblock_bytes[j] = align256(size_t(nt * be) * esz_of(in[j]->dt));
      b.total += b.reblock_bytes[j];
    }
  }
  plan_split(sp, in, n_in, b);
  b.total += b.split_bytes;
  return JAGG_OK;
}

// ------------------------------------------------------------ map / reduce planning
jagg_status plan_ew(jagg_ctx *ctx, const jagg_spec *sp, const Bound &b, const jagg_relation *const *ins,
                    const jagg_relation *out, const int32_t *list, const int32_t *counts, EwArgs &a) {
  memset(&a, 0, sizeof(a));
  const Spec &p = b.p;
  a.n_in = p.n_in;
  for (int j = 0; j < p.n_in; ++j) {
    a.in[j] = ins[j]->buf;
    a.in_dt[j] = ins[j]->dt == JAGG_BF16;
    a.be_in[j] = ins[j]->be;
  }
  a.out = out->buf;
  a.out_dt = sp->out_dtype == JAGG_BF16;
  a.g = sp->g;
  a.agg = sp->agg;
  a.alpha = sp->alpha;
  a.beta = sp->beta;
  a.eps = sp->eps;
  a.list = list;
  a.counts = counts;
  a.per_key = b.join.per_key;
  a.n_keys = b.join.n_keys;
  a.r_out = int(p.out.size());
  a.be_out = out->be;
  a.rows_per_block = 1;
  for (int i = 0; i < a.r_out; ++i) {
    a.e_out[i] = out->e[i];
    a.n_out[i] = out->n[i];
    a.k_out[i] = out->k[i];
    if (i < a.r_out - 1) a.rows_per_block *= out->e[i];
  }
  a.n_red = int(p.reduced.size());
  for (int i = 0; i < a.n_red; ++i) {
    const int c = p.reduced[i] - 'a';
    a.n_red_ext[i] = b.L.n[c];
    a.k_red[i] = b.L.k[c];
    a.e_red[i] = (b.L.n[c] + b.L.k[c] - 1) / b.L.k[c];
  }
  for (int j = 0; j < p.n_in; ++j) {
    const jagg_relation &R = *ins[j];
    for (int q = 0; q < R.r; ++q) {
      const char c = p.in[j][q];
      const size_t io = p.out.find(c), ir = p.reduced.find(c);
      if (io != std::string::npos) a.s_out[j][io] = inblock_s(R, q);
      if (ir != std::string::npos) {
        a.s_red[j][ir] = inblock_s(R, q);
        if (j == 0) a.w_red0[ir] = tuple_w(R, q);
      }
    }
  }
  if (sp->causal_s) {
    a.causal = 1;
    a.s_red_flag = 0;
    a.s_pos = int32_t(p.out.find(sp->causal_s));
    const size_t to = p.out.find(sp->causal_t);
    a.t_red_flag = to == std::string::npos;
    a.t_pos = int32_t(a.t_red_flag ? p.reduced.find(sp->causal_t) : to);
  }
  a.inner_red = -1;
  a.vec = 1;
  if (sp->agg == JAGG_AGG_NONE) {
    if (a.causal && (a.t_red_flag || a.t_pos != a.r_out - 1))
      return fail(ctx, JAGG_E_UNSUPPORTED, "a causal map needs t as the innermost output letter");
    a.vec = (a.e_out[a.r_out - 1] % 4 == 0) ? 4 : 1;
  } else {
    // reduce: input 0 holds every letter, the others a subset
    if (p.in[0].size() != p.order.size())
      return fail(ctx, JAGG_E_UNSUPPORTED, "a reduce needs input 0 to hold every letter of the spec");
    if (a.n_red == 0) return fail(ctx, JAGG_E_UNSUPPORTED, "SUM/MAX with no reduced letter; use NONE");
    const char last = p.in[0].back();
    const size_t ir = p.reduced.find(last);
    a.inner_red = ir == std::string::npos ? -1 : int32_t(ir);
    if (a.causal && !a.t_red_flag)
      return fail(ctx, JAGG_E_UNSUPPORTED, "a causal reduce needs t among the reduced letters");
    if (a.causal && a.inner_red >= 0 && a.t_pos != a.inner_red)
      return fail(ctx, JAGG_E_UNSUPPORTED, "a causal row reduce needs t innermost in input 0");
  }
  return JAGG_OK;
}

// ------------------------------------------------------------ attention planning
// Roles of "X s D, X t D, X t E -> X s E" (see jagg.h) and the kernel's
// layout requirements; every violation is JAGG_E_UNSUPPORTED before launch.
jagg_status plan_attention(jagg_ctx *ctx, const jagg_spec *sp, const Bound &b, const jagg_relation *const *ins,
                           const jagg_relation *out, const int32_t *list, const int32_t *counts, AttnArgs &a,
                           int &d) {
  memset(&a, 0, sizeof(a));
  const Spec &p = b.p;
  // X: letters of every operand; G: letters of Q and the output only, i.e.
  // s and any query-group letters of grouped-query attention ("Every Kernel
  // Is a Join", Example 3.10: query heads 4m..4m+3 share key-value head m),
  // which run as batch letters whose K and V strides are 0
  std::string X, G;
  char s = 0, t = 0, dl = 0, el = 0;
  for (char c : p.order) {
    const bool q = p.in[0].find(c) != std::string::npos, k = p.in[1].find(c) != std::string::npos;
    const bool v = p.in[2].find(c) != std::string::npos, o = p.out.find(c) != std::string::npos;
    if (q && k && v && o) X += c;
    else if (q && !k && !v && o) G += c;
    else if (!q && k && v && !o && !t) t = c;
    else if (q && k && !v && !o && !dl) dl = c;
    else if (!q && !k && v && o && !el) el = c;
    else return fail(ctx, JAGG_E_UNSUPPORTED, "attention letter '%c' has no role of X G s D, X t D, X t E -> X G s E", c);
  }
  if (G.empty() || !t || !dl || !el) return fail(ctx, JAGG_E_UNSUPPORTED, "attention needs one s, t, D and E letter");
  for (int j = 0; j < 3; ++j)
    if (ins[j]->dt != JAGG_BF16) return fail(ctx, JAGG_E_UNSUPPORTED, "attention inputs must be bfloat16");
  const jagg_relation &Q = *ins[0], &K = *ins[1], &V = *ins[2], &O = *out;
  auto pos = [&](int j, char c) { return int(j < 3 ? p.in[j].find(c) : p.out.find(c)); };
  const char pair_s = sp->causal_s ? sp->causal_s : sp->seg_s, pair_t = sp->causal_s ? sp->causal_t : sp->seg_t;
  if (pair_s) {
    if (G.find(pair_s) == std::string::npos || pair_t != t)
      return fail(ctx, JAGG_E_UNSUPPORTED, "the causal / segment pair of attention must be (a query letter, %c)", t);
    s = pair_s;
  } else {  // the row letter: the innermost of G in Q
    for (char c : G)
      if (!s || inblock_s(Q, pos(0, c)) < inblock_s(Q, pos(0, s))) s = c;
  }
  const std::string grp = [&] {
    std::string r;
    for (char c : G)
      if (c != s) r += c;
    return r;
  }();
  X += grp;
  if (pos(0, dl) != Q.r - 1 || pos(1, dl) != K.r - 1 || pos(2, el) != V.r - 1 || pos(3, el) != O.r - 1)
    return fail(ctx, JAGG_E_UNSUPPORTED, "D must be innermost in Q and K, E innermost in V and the output");
  if (b.L.k[dl - 'a'] != 1 || b.L.k[el - 'a'] != 1)
    return fail(ctx, JAGG_E_UNSUPPORTED, "D and E must be one block each");
  const int64_t nd = b.L.n[dl - 'a'], ne = b.L.n[el - 'a'];
  if (nd != ne || (nd != 64 && nd != 128)) return fail(ctx, JAGG_E_UNSUPPORTED, "D = E must be 64 or 128");
  d = int(nd);
  a.sQ = inblock_s(Q, pos(0, s));
  a.tK = inblock_s(K, pos(1, t));
  a.tV = inblock_s(V, pos(2, t));
  a.sO = inblock_s(O, pos(3, s));
  const int64_t lim31 = (int64_t(1) << 31) - 1;
  for (const jagg_relation *R : {&Q, &K, &V, &O})
    if (R->be % 8 != 0 || R->be * esz_of(R->dt) > lim31)
      return fail(ctx, JAGG_E_UNSUPPORTED, "attention blocks must hold a multiple of 8 elements, under 2 GiB");
  if (a.sQ % 8 || a.tK % 8 || a.tV % 8 || a.sO % 8)
    return fail(ctx, JAGG_E_UNSUPPORTED, "attention row strides must be multiples of 8 elements");
  a.nx = int(X.size());
  if (a.nx > kMaxLetters) return fail(ctx, JAGG_E_UNSUPPORTED, "too many batch letters");
  int64_t nb = 1;
  {  // batch letters in output order
    int i = 0;
    for (char c : p.out) {
      if (X.find(c) == std::string::npos) continue;
      const int64_t e = O.e[pos(3, c)];
      a.xdiv[i] = make_fastdiv(uint32_t(e));
      const bool shared_kv = grp.find(c) != std::string::npos;  // a query-group letter
      a.xQ[i] = inblock_s(Q, pos(0, c));
      a.xK[i] = shared_kv ? 0 : inblock_s(K, pos(1, c));
      a.xV[i] = shared_kv ? 0 : inblock_s(V, pos(2, c));
      a.xO[i] = inblock_s(O, pos(3, c));
      if (a.xQ[i] % 8 || a.xK[i] % 8 || a.xV[i] % 8 || a.xO[i] % 8)
        return fail(ctx, JAGG_E_UNSUPPORTED, "attention batch strides must be multiples of 8 elements");
      nb *= e;
      ++i;
    }
  }
  a.nbatch = int32_t(nb);
  a.Q = Q.buf;
  a.K = K.buf;
  a.V = V.buf;
  a.O = O.buf;
  a.list = list;
  a.counts = counts;
  a.per_key = int32_t(b.join.per_key);
  if (a.per_key > kMaxAttnTuples)
    return fail(ctx, JAGG_E_UNSUPPORTED, "attention joins at most %d K/V tuples per output tuple (t blocked %d ways)",
                kMaxAttnTuples, a.per_key);
  a.n_keys = int32_t(b.join.n_keys);
  a.beQ = Q.be;
  a.beK = K.be;
  a.beV = V.be;
  a.beO = O.be;
  a.e_s = int32_t(O.e[pos(3, s)]);
  a.e_t = int32_t(K.e[pos(1, t)]);
  a.n_s = int32_t(b.L.n[s - 'a']);
  a.n_t = int32_t(b.L.n[t - 'a']);
  a.s_tiles = int32_t((a.e_s + 127) / 128);
  a.div_st = make_fastdiv(uint32_t(a.s_tiles));
  a.div_nb = make_fastdiv(uint32_t(a.nbatch));
  a.div_Ws = make_fastdiv(uint32_t(tuple_w(O, pos(3, s))));
  a.div_ks = make_fastdiv(uint32_t(O.k[pos(3, s)]));
  a.div_Wt = make_fastdiv(uint32_t(tuple_w(K, pos(1, t))));
  a.div_kt = make_fastdiv(uint32_t(K.k[pos(1, t)]));
  a.scale_log2 = float(double(sp->alpha) * 1.4426950408889634);
  a.reverse = sp->causal_s ? 1 : 0;
  a.div_per_s = make_fastdiv(uint32_t(a.n_keys / O.k[pos(3, s)]));
  a.iv = 0;
  if (b.iv_letter[s - 'a']) {  // packed sequences (bind_intervals checked the segment pair)
    a.iv = 1;
    for (int i = 0; i <= b.L.k[s - 'a']; ++i) a.bnd[i] = int32_t(b.iv_bnd[s - 'a'][i]);
  }
  a.xcd_group = a.nbatch % 8 == 0 ? 1 : 0;
  a.div_group = make_fastdiv(uint32_t(a.n_keys * a.s_tiles));
  if (!(sp->alpha > 0.0f)) return fail(ctx, JAGG_E_UNSUPPORTED, "attention needs a positive score scale alpha");
  if (int64_t(a.nbatch) * a.n_keys * a.s_tiles > lim31)
    return fail(ctx, JAGG_E_UNSUPPORTED, "attention grid too large");
  return JAGG_OK;
}

// ------------------------------------------------------------ contraction planning
struct Group {
  std::string letters;  // in canonical order
  int64_t ext = 1;
};

// Checks that `g`'s letters sit next to each other in operand `lt` in the
// same order with nesting strides, and returns the flattened stride.
bool group_stride(const Group &g, const std::string &lt, const jagg_relation &R, int64_t &stride) {
  if (g.letters.empty()) {
    stride = 0;
    return true;
  }
  const size_t p0 = lt.find(g.letters[0]);
  if (p0 == std::string::npos) return false;
  for (size_t i = 0; i < g.letters.size(); ++i)
    if (p0 + i >= lt.size() || lt[p0 + i] != g.letters[i]) return false;
  stride = inblock_s(R, int(p0 + g.letters.size() - 1));
  return true;
}

// M panels per group of the grouped tile order (measured best of 2/4/8/16)
#ifndef JAGG_GROUP_M
#define JAGG_GROUP_M 4
#endif
constexpr int kGroupM = JAGG_GROUP_M;

jagg_status plan_contract(jagg_ctx *ctx, const jagg_spec *sp, const Bound &b, const jagg_relation *const *ins,
                          const jagg_relation *out, const int32_t *list, const int32_t *counts, ContractArgs &a,
                          int &dtype, bool &a_kc, bool &b_kc, int &va, int &vb) {
  memset(&a, 0, sizeof(a));
  const Spec &p = b.p;
  if (ins[0]->dt != ins[1]->dt) return fail(ctx, JAGG_E_UNSUPPORTED, "contraction inputs differ in dtype");
  dtype = ins[0]->dt == JAGG_BF16;
  int ia = 0, ib = 1;
  Group Gb, Gm, Gn, Gk;
  auto build = [&]() {
    Gb = Group();
    Gm = Group();
    Gn = Group();
    Gk = Group();
    for (char c : p.out) {
      const bool inA = p.in[ia].find(c) != std::string::npos, inB = p.in[ib].find(c) != std::string::npos;
      Group &g = inA && inB ? Gb : (inA ? Gm : Gn);
      g.letters.push_back(c);
    }
    for (char c : p.in[ia])
      if (p.out.find(c) == std::string::npos) Gk.letters.push_back(c);
    for (Group *g : {&Gb, &Gm, &Gn, &Gk}) {
      g->ext = 1;
      for (char c : g->letters) g->ext *= (b.L.n[c - 'a'] + b.L.k[c - 'a'] - 1) / b.L.k[c - 'a'];
    }
  };
  build();
  for (char c : p.reduced)
    if (p.in[0].find(c) == std::string::npos || p.in[1].find(c) == std::string::npos)
      return fail(ctx, JAGG_E_UNSUPPORTED, "contraction letter '%c' is reduced but not in both inputs", c);
  int64_t sCn = 0, sCm = 0, sCb = 0;
  if (!group_stride(Gn, p.out, *out, sCn) || !group_stride(Gm, p.out, *out, sCm) || !group_stride(Gb, p.out, *out, sCb))
    return fail(ctx, JAGG_E_UNSUPPORTED, "output letters of one class are not adjacent in '%s'", p.out.c_str());
  if (!(sCn == 1 || Gn.letters.empty())) {
    // the output is contiguous along the other input's letters: swap roles
    std::swap(ia, ib);
    build();
    if (!group_stride(Gn, p.out, *out, sCn) || !group_stride(Gm, p.out, *out, sCm) ||
        !group_stride(Gb, p.out, *out, sCb))
      return fail(ctx, JAGG_E_UNSUPPORTED, "output letters of one class are not adjacent");
    if (!(sCn == 1 || Gn.letters.empty()))
      return fail(ctx, JAGG_E_UNSUPPORTED, "output '%s' is not contiguous along a non-batch letter", p.out.c_str());
  }
  const jagg_relation &RA = *ins[ia], &RB = *ins[ib];
  int64_t sAb, sAm, sAk, sBb, sBn, sBk;
  if (!group_stride(Gb, p.in[ia], RA, sAb) || !group_stride(Gm, p.in[ia], RA, sAm) ||
      !group_stride(Gk, p.in[ia], RA, sAk) || !group_stride(Gb, p.in[ib], RB, sBb) ||
      !group_stride(Gn, p.in[ib], RB, sBn) || !group_stride(Gk, p.in[ib], RB, sBk))
    return fail(ctx, JAGG_E_UNSUPPORTED, "contraction letters of one class are not adjacent in an input");
  if (Gm.letters.empty()) sAm = 0;
  if (Gn.letters.empty()) sBn = 0;
  a_kc = sAk == 1;
  b_kc = sBk == 1;
  if (!a_kc && !(sAm == 1)) return fail(ctx, JAGG_E_UNSUPPORTED, "input A is contiguous along a batch letter");
  if (!b_kc && !(sBn == 1)) return fail(ctx, JAGG_E_UNSUPPORTED, "input B is contiguous along a batch letter");
  const int F = dtype ? 8 : 4;
  auto vec_ok = [&](bool kc, int64_t rows, int64_t sRow, int64_t sK, int64_t sBat, int64_t be) {
    const int64_t contig = kc ? Gk.ext : rows;
    const int64_t other = kc ? sRow : sK;
    // fp32 operand contiguous along M or N: vectors may straddle the row end
    // (the extra lanes only feed output rows/columns that are never stored)
    // and start at any element (4-byte aligned)
    if (!kc && !dtype) return true;
    return contig % F == 0 && other % F == 0 && sBat % F == 0 && be % F == 0;
  };
  va = vec_ok(a_kc, Gm.ext, sAm, sAk, sAb, RA.be) ? F : 1;
  vb = vec_ok(b_kc, Gn.ext, sBn, sBk, sBb, RB.be) ? F : 1;
  a.A = RA.buf;
  a.B = RB.buf;
  a.C = out->buf;
  a.list = list;
  a.counts = counts;
  a.per_key = b.join.per_key;
  a.a_slot = 1 + ia;
  a.b_slot = 1 + ib;
  a.beA = RA.be;
  a.beB = RB.be;
  a.beC = out->be;
  if (Gb.ext > (1 << 30) || Gm.ext > (1 << 30) || Gn.ext > (1 << 30) || Gk.ext > (1 << 30))
    return fail(ctx, JAGG_E_UNSUPPORTED, "block too large");
  a.batch = int32_t(Gb.ext);
  a.M = int32_t(Gm.ext);
  a.N = int32_t(Gn.ext);
  a.K = int32_t(Gk.ext);
  a.sAb = sAb;
  a.sAm = sAm;
  a.sAk = sAk;
  a.sBb = sBb;
  a.sBn = sBn;
  a.sBk = sBk;
  a.sCb = sCb;
  a.sCm = sCm;
  a.alpha = sp->alpha;
  a.tiles_m = (a.M + 127) / 128;
  a.tiles_n = (a.N + 127) / 128;
  a.n_keys = b.join.n_keys;
  // key grid for the grouped tile order: every blocked output letter is an M
  // or N letter, the M ones before the N ones in the key's row-major order
  {
    int64_t km = 1, kn = 1;
    bool ok = Gb.ext == 1, seen_n = false;
    for (char c : p.out) {
      const int32_t k = b.L.k[c - 'a'];
      if (k == 1) continue;
      const bool m = Gm.letters.find(c) != std::string::npos, n = Gn.letters.find(c) != std::string::npos;
      if (m && !seen_n) km *= k;
      else if (n) {
        kn *= k;
        seen_n = true;
      } else {
        ok = false;
      }
    }
    if (ok && km * kn == a.n_keys && km < (1 << 20) && kn < (1 << 20)) {
      a.km = int32_t(km);
      a.kn = int32_t(kn);
    }
  }
  a.div_s = a.div_t = make_fastdiv(1);
  // blocks addressed through 32-bit buffer offsets
  if (RA.be * esz_of(RA.dt) >= (int64_t(1) << 31) || RB.be * esz_of(RB.dt) >= (int64_t(1) << 31))
    return fail(ctx, JAGG_E_UNSUPPORTED, "contraction block of 2 GiB or more");
  if (sp->causal_s) {
    const char s = sp->causal_s, t = sp->causal_t;
    const int cs = s - 'a', ct = t - 'a';
    auto out_w = [&](char c) {
      int64_t w = 1;
      for (size_t q = p.out.find(c) + 1; q < p.out.size(); ++q) w *= b.L.k[p.out[q] - 'a'];
      return w;
    };
    a.e_s = int32_t((b.L.n[cs] + b.L.k[cs] - 1) / b.L.k[cs]);
    a.e_t = int32_t((b.L.n[ct] + b.L.k[ct] - 1) / b.L.k[ct]);
    a.div_s = make_fastdiv(uint32_t(a.e_s));
    a.div_t = make_fastdiv(uint32_t(a.e_t));
    a.cs_w = out_w(s);
    a.cs_k = b.L.k[cs];
    a.ct_k = b.L.k[ct];
    if (Gm.letters.empty() || Gm.letters.back() != s)
      return fail(ctx, JAGG_E_UNSUPPORTED, "causal contraction needs s innermost among the M letters");
    if (p.out.find(t) != std::string::npos) {
      if (Gn.letters.empty() || Gn.letters.back() != t)
        return fail(ctx, JAGG_E_UNSUPPORTED, "causal contraction needs t innermost among the N letters");
      a.causal_out = 1;
      a.ct_w = out_w(t);
    } else {
      if (Gk.letters.empty() || Gk.letters.back() != t)
        return fail(ctx, JAGG_E_UNSUPPORTED, "causal contraction needs t innermost among the K letters");
      a.causal_red = 1;
      const size_t q = p.in[ia].find(t);
      a.ct_w = tuple_w(RA, int(q));
      const int F = dtype ? 8 : 4;
      if (va != F || vb != F)
        return fail(ctx, JAGG_E_UNSUPPORTED, "causal contraction over a reduced letter needs 16-byte aligned operands");
    }
  }
  a.ent_w = 1 + p.n_in;
  if (sp->g == JAGG_G_MUL_PLUS) {
    // the addend is laid out as the output: same letters in the same order,
    // same blocking, so its element offset is the output's
    const jagg_relation &X = *ins[2];
    if (p.in[2] != p.out || X.n_tuples != out->n_tuples || X.be != out->be)
      return fail(ctx, JAGG_E_UNSUPPORTED, "MUL_PLUS: input 2 must hold the output letters in the output's order");
    a.epi = 1;
    a.X = X.buf;
    a.x_bf16 = X.dt == JAGG_BF16;
  } else if (sp->g == JAGG_G_SWIGLU) {
    const jagg_relation &R2 = *ins[2];
    if (ib != 1 || p.in[2] != p.in[1] || R2.dt != RB.dt || R2.n_tuples != RB.n_tuples || R2.be != RB.be)
      return fail(ctx, JAGG_E_UNSUPPORTED, "SWIGLU: input 2 must be laid out as input 1, on the N side");
    if (R2.be * esz_of(R2.dt) >= (int64_t(1) << 31))
      return fail(ctx, JAGG_E_UNSUPPORTED, "contraction block of 2 GiB or more");
    a.epi = 2;
    a.B2 = R2.buf;
  }
  if (ctx->trace)
    fprintf(stderr, "[jagg] contract %s: %s batch %d M %d N %d K %d A%s/v%d B%s/v%d keys %lld per_key %d\n",
            sp->einsum, dtype ? "bf16" : "f32", a.batch, a.M, a.N, a.K, a_kc ? "k" : "m", va, b_kc ? "k" : "n", vb,
            (long long)a.n_keys, a.per_key);
  return JAGG_OK;
}

// Everything jagg_einsum decides on the host for one call: the kernel
// arguments (which embed the relation, join-list and workspace addresses)
// and the launch choices.  Built once per call, or once per jagg_plan.
struct PlannedCall {
  enum Kind { MAP, REDUCE, CONTRACT, ATTENTION, NORM } kind = MAP;
  std::string einsum;
  int agg = 0;
  bool out_bf16 = false, causal = false;
  bool has_iv = false;  // some letter is interval-blocked
  NormArgs norm;        // NORM: a fused reduce / RMS-scale pair (jagg_plan_fuse)
  std::vector<RelayoutArgs> reblocks;
  std::vector<int> reblock_vec;  // vector bytes * 16 + element bytes
  JoinArgs join;
  EwArgs ew;
  ContractArgs ca;
  int dtype = 0, va = 1, vb = 1;
  bool akc = true, bkc = true, big = false;
  AttnArgs at;
  int att_d = 0;
  size_t ws_total = 0;
  // device byte ranges the call reads (inputs) and writes (output, workspace)
  std::vector<std::pair<const char *, size_t>> reads, writes;
};

// Binds and checks the call and plans every launch, host only.  `noalloc`
// marks the static scratch as the workspace (a size error then names it).
jagg_status build_call(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                       const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes, bool noalloc,
                       PlannedCall &P) {
  if (!ctx || !out) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  Bound b;
  jagg_status st = bind(ctx, spec, in, n_in, blockings, b);
  if (st != JAGG_OK) return st;
  // output relation must be the spec's output under `blockings`
  if (out->r != int(b.p.out.size()))
    return fail(ctx, JAGG_E_SHAPE, "out relation has %d dimensions, output '%s' names %d", out->r, b.p.out.c_str(),
                int(b.p.out.size()));
  jagg_relation out_view = *out;  // interval letters as uniform ones, like the inputs
  for (int q = 0; q < out->r; ++q) {
    const int c = b.p.out[q] - 'a';
    if (out->iv[q] != int32_t(b.iv_letter[c]))
      return fail(ctx, JAGG_E_BLOCKING, "out letter '%c' must be %s-blocked like the inputs", 'a' + c,
                  b.iv_letter[c] ? "interval" : "uniformly");
    if (out->iv[q]) {
      if (out->k[q] != b.L.k[c] ||
          memcmp(out->bnd[q], b.iv_bnd[c], sizeof(int64_t) * size_t(out->k[q] + 1)) != 0)
        return fail(ctx, JAGG_E_BLOCKING, "out letter '%c' has other bounds than the inputs", 'a' + c);
      out_view.n[q] = int64_t(out->k[q]) * out->e[q];
      out_view.iv[q] = 0;
    }
    if (out_view.n[q] != b.L.n[c])
      return fail(ctx, JAGG_E_SHAPE, "out letter '%c' has extent %lld, expected %lld", 'a' + c, (long long)out->n[q],
                  (long long)b.L.n[c]);
    if (out->k[q] != b.L.k[c])
      return fail(ctx, JAGG_E_BLOCKING, "out letter '%c' has %d blocks, the spec asks %d", 'a' + c, out->k[q], b.L.k[c]);
  }
  out = &out_view;
  if (out->dt != spec->out_dtype) return fail(ctx, JAGG_E_SHAPE, "out relation dtype differs from spec->out_dtype");
  {
    const char *ob = static_cast<const char *>(out->buf);
    const size_t on = size_t(out->n_tuples * out->be) * esz_of(out->dt);
    for (int j = 0; j < n_in; ++j) {
      const char *ib = static_cast<const char *>(in[j]->buf);
      const size_t inn = size_t(in[j]->n_tuples * in[j]->be) * esz_of(in[j]->dt);
      if (ib < ob + on && ob < ib + inn) return fail(ctx, JAGG_E_INVALID, "out relation overlaps input %d", j);
    }
  }
  if (noalloc) {
    // the static scratch is sized for join lists and re-blocked inputs:
    // split walks take no part of it
    b.total -= b.split_bytes;
    b.split = 1;
    b.split_bytes = 0;
  }
  if (noalloc && b.total > ws_bytes)
    return fail(ctx, JAGG_E_WORKSPACE, "the call needs %zu bytes of workspace; the static scratch holds %zu",
                b.total, ws_bytes);
  if (!workspace || ws_bytes < b.total)
    return fail(ctx, JAGG_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, b.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(ctx, JAGG_E_WORKSPACE, "workspace not 256-byte aligned");
  P.ws_total = b.total;
  for (int j = 0; j < n_in; ++j)
    P.reads.push_back({static_cast<const char *>(in[j]->buf), size_t(in[j]->n_tuples * in[j]->be) * esz_of(in[j]->dt)});
  P.writes.push_back({static_cast<const char *>(out->buf), size_t(out->n_tuples * out->be) * esz_of(out->dt)});
  P.writes.push_back({static_cast<const char *>(workspace), b.total});
  P.einsum = spec->einsum;
  P.agg = spec->agg;
  P.out_bf16 = spec->out_dtype == JAGG_BF16;
  P.causal = spec->causal_s != 0;
  for (int c = 0; c < 26; ++c) P.has_iv = P.has_iv || b.iv_letter[c];

  // classify before launching anything: a contraction is a MUL/SUM over two
  // inputs where every reduced letter is in both inputs and each input
  // contributes output letters of its own; any other aggregating spec is a
  // streaming reduce, and a spec without aggregation is a map.
  P.kind = PlannedCall::MAP;
  if (spec->agg == JAGG_AGG_SOFTMAX) {
    P.kind = PlannedCall::ATTENTION;
  } else if (spec->agg != JAGG_AGG_NONE) {
    P.kind = PlannedCall::REDUCE;
    const bool recompose = spec->g == JAGG_G_MUL_PLUS || spec->g == JAGG_G_SWIGLU;
    if (spec->agg == JAGG_AGG_SUM && ((spec->g == JAGG_G_MUL && n_in == 2) || recompose) && !b.p.reduced.empty()) {
      bool both = true, m_any = false, n_any = false;
      for (char c : b.p.reduced)
        both = both && b.p.in[0].find(c) != std::string::npos && b.p.in[1].find(c) != std::string::npos;
      for (char c : b.p.out) {
        const bool i0 = b.p.in[0].find(c) != std::string::npos, i1 = b.p.in[1].find(c) != std::string::npos;
        m_any = m_any || (i0 && !i1);
        n_any = n_any || (i1 && !i0);
      }
      if (both && m_any && n_any) P.kind = PlannedCall::CONTRACT;
    }
    if (recompose && P.kind != PlannedCall::CONTRACT)
      return fail(ctx, JAGG_E_UNSUPPORTED, "g %d needs a contraction of inputs 0 and 1", int(spec->g));
  }

  char *ws = static_cast<char *>(workspace);
  int32_t *list = reinterpret_cast<int32_t *>(ws);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + b.list_bytes);
  size_t off = b.list_bytes + b.counts_bytes;
  // (0) inputs blocked differently: re-block into the workspace
  jagg_relation tmp[kMaxIn];
  const jagg_relation *use[kMaxIn];
  for (int j = 0; j < n_in; ++j) {
    use[j] = b.in[j];
    if (!b.needs_reblock[j]) continue;
    jagg_relation &T = tmp[j];
    T = *b.in[j];
    for (int q = 0; q < T.r; ++q) T.k[q] = b.L.k[b.p.in[j][q] - 'a'];
    if ((st = geometry(ctx, T.r, T.n, T.k, nullptr, T.e, &T.n_tuples, &T.be)) != JAGG_OK) return st;
    T.buf = ws + off;
    T.bytes = b.reblock_bytes[j];
    off += b.reblock_bytes[j];
    use[j] = &T;
  }
  // plan the block kernel (host only) before any launch
  if (P.kind == PlannedCall::CONTRACT &&
      (st = plan_contract(ctx, spec, b, use, out, list, counts, P.ca, P.dtype, P.akc, P.bkc, P.va, P.vb)) != JAGG_OK)
    return st;
  if (P.kind == PlannedCall::ATTENTION &&
      (st = plan_attention(ctx, spec, b, use, out, list, counts, P.at, P.att_d)) != JAGG_OK)
    return st;
  if ((P.kind == PlannedCall::MAP || P.kind == PlannedCall::REDUCE) &&
      (st = plan_ew(ctx, spec, b, use, out, list, counts, P.ew)) != JAGG_OK)
    return st;
  for (int j = 0; j < n_in; ++j) {
    if (!b.needs_reblock[j]) continue;
    RelayoutArgs ra;
    int vbytes = 0;
    if ((st = plan_relayout(ctx, *b.in[j], *use[j], ra, vbytes)) != JAGG_OK) return st;
    P.reblocks.push_back(ra);
    P.reblock_vec.push_back(vbytes * 16 + esz_of(in[j]->dt));
    if (ctx->trace) fprintf(stderr, "[jagg] %s: reblock input %d into the workspace\n", spec->einsum, j);
  }
  if (P.kind == PlannedCall::CONTRACT) {
    ContractArgs &ca = P.ca;
    // 256x256 tiles where the block is large enough and the grid still fills the chip
    const int F = P.dtype ? 8 : 4;
    const int BNt = ca.epi == 2 ? 128 : 256;
    const int64_t big_tiles = ca.n_keys * ca.batch * int64_t((ca.M + 255) / 256) * ((ca.N + BNt - 1) / BNt);
    // a split walk: the partial sums go after the join list and any
    // re-blocked inputs in the workspace (bind sized it)
    if (b.split > 1 && P.dtype && P.va == 8 && P.vb == 8 && ca.epi == 0 && !ca.causal_red && !ca.causal_out &&
        ca.M >= 256 && ca.N >= 256 && (reinterpret_cast<uintptr_t>(out->buf) & 15) == 0) {
      ca.split = b.split;
      ca.part = reinterpret_cast<float *>(ws + off);
      ca.part_stride = (int64_t(out->n_tuples) * out->be + 63) / 64 * 64;
    }
    // (a split walk fills the chip with its parts)
    P.big = P.va == F && P.vb == F && ca.M >= 256 && ca.N >= BNt && (big_tiles >= 256 || ca.split > 1) &&
            !ca.causal_red;
    // SWIGLU has only the 256 x 128 pipeline, which bounds-checks ragged M
    // and N, so it takes it at any size (the size rule above only picks the
    // faster kernel)
    if (ca.epi == 2) P.big = P.va == F && P.vb == F && !ca.causal_red;
    if (ca.epi == 2 && !(P.big && P.dtype && P.akc))
      return fail(ctx, JAGG_E_UNSUPPORTED, "SWIGLU runs on the 256 x 128 bf16 pipeline: bf16 operands in 16-byte "
                  "vectors, input 0 contiguous along the reduced letters");
    // per-XCD renumbering pays where several tiles of one output block share panels
    const int bm = P.big ? 256 : 128;
    ca.remap = !ca.causal_out && !ca.causal_red && int64_t((ca.M + bm - 1) / bm) * ((ca.N + bm - 1) / bm) >= 4;
    ca.group_m = (ca.remap && ca.km > 0 && ca.batch == 1) ? kGroupM : 0;
  }
  P.join = b.join;
  P.join.list = list;
  P.join.counts = counts;
  return JAGG_OK;
}

}  // namespace

struct jagg_plan {
  int device;
  PlannedCall call;
  // a group (jagg_plan_group): its members, and the members each launch runs
  std::vector<PlannedCall> members;
  std::vector<std::vector<int>> launches;
};

namespace {

jagg_status launch_join_of(jagg_ctx *ctx, const PlannedCall &P) {
  return after_launch(ctx, launch_join(P.join, ctx->stream), "join");
}

jagg_status launch_reblocks(jagg_ctx *ctx, const PlannedCall &P) {
  jagg_status st;
  for (size_t i = 0; i < P.reblocks.size(); ++i)
    if ((st = after_launch(ctx, launch_relayout(P.reblocks[i], P.reblock_vec[i] / 16, P.reblock_vec[i] % 16,
                                                ctx->stream),
                           "reblock input")) != JAGG_OK)
      return st;
  return JAGG_OK;
}

jagg_status launch_kernel(jagg_ctx *ctx, const PlannedCall &P);

// Launches a planned call: re-blocking copies, the join (unless a plan has
// already listed it), then the block kernel.
jagg_status launch_call(jagg_ctx *ctx, const PlannedCall &P, bool with_join) {
  jagg_status st;
  if ((st = launch_reblocks(ctx, P)) != JAGG_OK) return st;
  if (with_join && (st = launch_join_of(ctx, P)) != JAGG_OK) return st;
  return launch_kernel(ctx, P);
}

// True when two planned contractions differ only in their addresses (same
// kernel, same geometry): one grouped launch can run both.
bool same_contraction_form(const PlannedCall &x, const PlannedCall &y) {
  if (x.kind != PlannedCall::CONTRACT || y.kind != PlannedCall::CONTRACT) return false;
  if (x.dtype != y.dtype || x.va != y.va || x.vb != y.vb || x.akc != y.akc || x.bkc != y.bkc || x.big != y.big ||
      x.out_bf16 != y.out_bf16)
    return false;
  ContractArgs u, v;  // byte copies (plan_contract zeroes the padding)
  memcpy(&u, &x.ca, sizeof(u));
  memcpy(&v, &y.ca, sizeof(v));
  u.A = v.A = nullptr;
  u.B = v.B = nullptr;
  u.C = v.C = nullptr;
  u.list = v.list = nullptr;
  u.counts = v.counts = nullptr;
  u.X = v.X = nullptr;
  u.B2 = v.B2 = nullptr;
  u.part = v.part = nullptr;
  return memcmp(&u, &v, sizeof(u)) == 0;
}

// Block kernel of a planned call.
jagg_status launch_kernel(jagg_ctx *ctx, const PlannedCall &P) {
  const char *e_name = P.einsum.c_str();
  if (P.kind == PlannedCall::NORM) {
    const hipError_t e = launch_norm(P.norm, ctx->stream);
    if (ctx->trace)
      fprintf(stderr, "[jagg] %s: rms norm pair in one pass, %d keys x %d rows\n", e_name, P.norm.n_keys,
              P.norm.rows);
    return after_launch(ctx, e, "rms norm pair");
  }
  if (P.kind == PlannedCall::ATTENTION) {
    const hipError_t e = launch_attention(P.at, P.att_d, P.causal, P.out_bf16, ctx->stream);
    if (ctx->trace)
      fprintf(stderr, "[jagg] %s: attention d%d, %d keys x %d batch x %d s-tiles\n", e_name, P.att_d, P.at.n_keys,
              P.at.nbatch, P.at.s_tiles);
    return after_launch(ctx, e, "attention");
  }
  if (P.kind == PlannedCall::CONTRACT) {
    const int ob = P.out_bf16;
    const char *which = "";
    const hipError_t e = P.dtype ? launch_contract_bf16(P.ca, ob, P.akc, P.bkc, P.va, P.vb, P.big, ctx->stream, &which)
                                 : launch_contract_f32(P.ca, ob, P.akc, P.bkc, P.va, P.vb, P.big, ctx->stream, &which);
    if (ctx->trace)
      fprintf(stderr, "[jagg] %s: contract %s%s, %lld keys x %d batch\n", e_name, which,
              P.ca.split > 1 ? ", split walk" : "", (long long)P.ca.n_keys, P.ca.batch);
    if (P.ca.split > 1 && ctx->trace) fprintf(stderr, "[jagg] %s: walk in %d parts, then their sum\n", e_name, P.ca.split);
    jagg_status st = after_launch(ctx, e, "contract");
    if (st != JAGG_OK || P.ca.split <= 1) return st;
    return after_launch(ctx, launch_split_sum(P.ca, ob, P.ca.n_keys * P.ca.beC, ctx->stream), "split sum");
  }
  const char *which = "";
  const hipError_t e = launch_ew(ctx, P.ew, P.agg, &which);
  if (ctx->trace) fprintf(stderr, "[jagg] %s: %s, %lld keys\n", e_name, which, (long long)P.ew.n_keys);
  return after_launch(ctx, e, which);
}

jagg_status einsum_impl(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                        const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes,
                        bool noalloc) {
  PlannedCall P;
  jagg_status st = build_call(ctx, spec, in, n_in, blockings, out, workspace, ws_bytes, noalloc, P);
  if (st != JAGG_OK) return st;
  return launch_call(ctx, P, true);
}

// The checks of jagg_plan_fuse: `R` a sum-of-squares reduce of x over its
// innermost letter r, `M` the RMS-scale map of (x, R's output, a scale over
// r) into a relation laid out like x; every mismatch is JAGG_E_UNSUPPORTED
// (the caller runs the two plans apart).
jagg_status plan_norm_pair(jagg_ctx *ctx, const PlannedCall &R, const PlannedCall &M, NormArgs &n) {
  memset(&n, 0, sizeof(n));
  auto no = [&](const char *why) { return fail(ctx, JAGG_E_UNSUPPORTED, "no fused RMS-norm pair: %s", why); };
  if (R.kind != PlannedCall::REDUCE || M.kind != PlannedCall::MAP) return no("the first plan must be a reduce, the second a map");
  if (!R.reblocks.empty() || !M.reblocks.empty()) return no("a plan re-blocks an input");
  if (R.has_iv || M.has_iv) return no("interval-blocked letters");
  const EwArgs &r = R.ew, &m = M.ew;
  if (r.g != JAGG_G_SQUARE || r.agg != JAGG_AGG_SUM || r.n_in != 1 || r.n_red != 1 || r.causal || r.inner_red != 0 ||
      r.out_dt != 0)
    return no("the reduce must be an f32 SUM of squares over the innermost letter of its one input");
  if (m.g != JAGG_G_RMS_SCALE || m.agg != JAGG_AGG_NONE || m.n_in != 3 || m.causal)
    return no("the map must be RMS_SCALE of three inputs");
  if (m.in[0] != r.in[0] || m.in_dt[0] != r.in_dt[0] || m.be_in[0] != r.be_in[0])
    return no("the map's input 0 must be the reduce's input");
  if (m.in[1] != r.out) return no("the map's input 1 must be the reduce's output");
  Spec pr, pm;
  jagg_status st;
  if ((st = parse(ctx, R.einsum.c_str(), pr)) != JAGG_OK || (st = parse(ctx, M.einsum.c_str(), pm)) != JAGG_OK)
    return st;
  const std::string &X = pr.in[0], &Xm = pm.in[0];
  if (X.size() != Xm.size() || pr.out != X.substr(0, X.size() - 1) ||
      pm.in[1] != Xm.substr(0, Xm.size() - 1) || pm.in[2] != Xm.substr(Xm.size() - 1) || pm.out != Xm)
    return no("the letters must read 'X r -> X' and 'X r, X, r -> X r'");
  const int64_t e_r = r.e_red[0], rows = r.be_out;
  const int last = m.r_out - 1;
  if (r.be_in[0] != rows * e_r || m.be_out != r.be_in[0] || m.rows_per_block != rows || m.be_in[1] != rows ||
      m.be_in[2] != e_r || m.e_out[last] != e_r || m.n_out[last] != r.n_red_ext[0] || m.k_out[last] != r.k_red[0])
    return no("the relations' blocks do not line up");
  if (e_r % 256 != 0 || int64_t(r.per_key) * (e_r / 256) > kNormMaxVec)
    return no("rows must be a multiple of 256 elements per block and at most 4096 elements long");
  const int64_t chunks = (rows + 3) / 4;
  if (r.n_keys * chunks >= (int64_t(1) << 31)) return no("too many rows");
  auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (!al(r.in[0]) || !al(m.in[2]) || !al(m.out)) return no("x, the scale and the output must be 16-byte aligned");
  for (const auto &w : M.writes)
    for (const auto &q : R.reads)
      if (w.first < q.first + q.second && q.first < w.first + w.second)
        return fail(ctx, JAGG_E_INVALID, "the map's output overlaps the reduce's input");
  n.x = r.in[0];
  n.x_dt = r.in_dt[0];
  n.be_x = r.be_in[0];
  n.ss = static_cast<float *>(r.out);
  n.gam = m.in[2];
  n.g_dt = m.in_dt[2];
  n.be_g = m.be_in[2];
  n.y = m.out;
  n.y_dt = m.out_dt;
  n.list = r.list;
  n.counts = r.counts;
  n.per_key = r.per_key;
  n.n_keys = int32_t(r.n_keys);
  n.rows = int32_t(rows);
  n.chunks = int32_t(chunks);
  n.div_chunks = make_fastdiv(uint32_t(chunks));
  n.e_r = int32_t(e_r);
  n.n_r = int32_t(r.n_red_ext[0]);
  n.nvb = int32_t(e_r / 256);
  n.div_wr = make_fastdiv(uint32_t(r.w_red0[0]));
  n.div_kr = make_fastdiv(uint32_t(r.k_red[0]));
  n.alpha_r = r.alpha;
  n.alpha_m = m.alpha;
  n.beta = m.beta;
  n.eps = m.eps;
  return JAGG_OK;
}

const char *env_or(const char *k) {
  const char *v = getenv(k);
  return v ? v : "";
}

}  // namespace

// ================================================================= C ABI
extern "C" {

jagg_status jagg_ctx_create(int device, void *hip_stream, jagg_ctx **out) {
  if (!out) return JAGG_E_INVALID;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n || device >= kMaxDevices) return JAGG_E_DEVICE;
  if (hipSetDevice(device) != hipSuccess) return JAGG_E_DEVICE;
  void *scr = nullptr;
  if (scratch_of_device(device, &scr) != hipSuccess || !scr) return JAGG_E_DEVICE;
  jagg_ctx *c = new jagg_ctx;
  c->device = device;
  c->scratch = scr;
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  c->trace = env_or("JAGG_TRACE")[0] == '1';
  c->debug_sync = env_or("JAGG_DEBUG_SYNC")[0] == '1';
  c->capturing = false;
  *out = c;
  return JAGG_OK;
}

jagg_status jagg_ctx_destroy(jagg_ctx *ctx) {
  if (!ctx) return JAGG_E_INVALID;
  delete ctx;
  return JAGG_OK;
}

jagg_status jagg_capture_begin(jagg_ctx *ctx) {
  if (!ctx) return JAGG_E_INVALID;
  if (ctx->capturing) return fail(ctx, JAGG_E_INVALID, "capture already begun on this context");
  const hipError_t e = hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) return fail(ctx, JAGG_E_DEVICE, "capture begin: %s", hipGetErrorString(e));
  ctx->capturing = true;
  return JAGG_OK;
}

jagg_status jagg_capture_end(jagg_ctx *ctx, jagg_graph **out) {
  if (!ctx || !out) return JAGG_E_INVALID;
  if (!ctx->capturing) return fail(ctx, JAGG_E_INVALID, "capture end without a begin");
  ctx->capturing = false;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(ctx->stream, &g);
  if (e != hipSuccess) return fail(ctx, JAGG_E_DEVICE, "capture end: %s", hipGetErrorString(e));
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(g);
    return fail(ctx, JAGG_E_DEVICE, "graph instantiate: %s", hipGetErrorString(e));
  }
  *out = new jagg_graph{g, x};
  return JAGG_OK;
}

jagg_status jagg_graph_launch(jagg_ctx *ctx, const jagg_graph *g) {
  if (!ctx || !g) return JAGG_E_INVALID;
  const hipError_t e = hipGraphLaunch(g->exec, ctx->stream);
  if (e != hipSuccess) return fail(ctx, JAGG_E_DEVICE, "graph launch: %s", hipGetErrorString(e));
  return JAGG_OK;
}

jagg_status jagg_graph_destroy(jagg_graph *g) {
  if (!g) return JAGG_E_INVALID;
  hipGraphExecDestroy(g->exec);
  hipGraphDestroy(g->graph);
  delete g;
  return JAGG_OK;
}

jagg_status jagg_relation_bytes_iv(const char *letters, const int64_t *extents, const int32_t *nblocks,
                                   const int64_t *const *bounds, jagg_dtype dtype, size_t *bytes) {
  if (!letters || !extents || !nblocks || !bytes) return JAGG_E_INVALID;
  if (dtype != JAGG_F32 && dtype != JAGG_BF16) return JAGG_E_INVALID;
  const int r = int(strlen(letters));
  if (r < 1 || r > kMaxLetters) return JAGG_E_UNSUPPORTED;
  int64_t e[kMaxLetters], nt, be;
  jagg_status st = geometry(nullptr, r, extents, nblocks, bounds, e, &nt, &be);
  if (st != JAGG_OK) return st;
  *bytes = size_t(nt * be) * size_t(esz_of(dtype));
  return JAGG_OK;
}

jagg_status jagg_relation_bytes(const char *letters, const int64_t *extents, const int32_t *nblocks, jagg_dtype dtype,
                                size_t *bytes) {
  return jagg_relation_bytes_iv(letters, extents, nblocks, nullptr, dtype, bytes);
}

jagg_status jagg_relation_create(jagg_ctx *ctx, const char *letters, const int64_t *extents, const int32_t *nblocks,
                                 jagg_dtype dtype, void *dev_buf, size_t buf_bytes, jagg_relation **out) {
  return jagg_relation_create_iv(ctx, letters, extents, nblocks, nullptr, dtype, dev_buf, buf_bytes, out);
}

jagg_status jagg_relation_create_iv(jagg_ctx *ctx, const char *letters, const int64_t *extents,
                                    const int32_t *nblocks, const int64_t *const *bounds, jagg_dtype dtype,
                                    void *dev_buf, size_t buf_bytes, jagg_relation **out) {
  if (!ctx || !letters || !extents || !nblocks || !out) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  *out = nullptr;
  if (dtype != JAGG_F32 && dtype != JAGG_BF16) return fail(ctx, JAGG_E_INVALID, "unknown dtype %d", int(dtype));
  const int r = int(strlen(letters));
  if (r < 1 || r > kMaxLetters) return fail(ctx, JAGG_E_UNSUPPORTED, "relation rank %d outside [1, %d]", r, kMaxLetters);
  for (int i = 0; i < r; ++i) {
    if (letters[i] < 'a' || letters[i] > 'z') return fail(ctx, JAGG_E_INVALID, "bad letter '%c'", letters[i]);
    for (int j = i + 1; j < r; ++j)
      if (letters[i] == letters[j]) return fail(ctx, JAGG_E_INVALID, "letter '%c' repeats", letters[i]);
  }
  jagg_relation R;
  R.ctx = ctx;
  R.r = r;
  memset(R.letters, 0, sizeof(R.letters));
  memcpy(R.letters, letters, size_t(r));
  for (int i = 0; i < r; ++i) {
    R.n[i] = extents[i];
    R.k[i] = nblocks[i];
  }
  jagg_status st = geometry(ctx, r, R.n, R.k, bounds, R.e, &R.n_tuples, &R.be);
  if (st != JAGG_OK) return st;
  memset(R.iv, 0, sizeof(R.iv));
  memset(R.bnd, 0, sizeof(R.bnd));
  for (int i = 0; i < r; ++i)
    if (bounds && bounds[i]) {
      R.iv[i] = 1;
      for (int j = 0; j <= R.k[i]; ++j) R.bnd[i][j] = bounds[i][j];
    }
  // offsets across a relation are 64-bit in every kernel and tuple ids
  // 32-bit; each block kernel's planner checks the block sizes it takes
  const int64_t elems = R.n_tuples * R.be;
  if (elems >= kMaxRelationElems)
    return fail(ctx, JAGG_E_UNSUPPORTED, "relation of %lld elements reaches 2^36", (long long)elems);
  if (R.n_tuples >= (int64_t(1) << 31))
    return fail(ctx, JAGG_E_UNSUPPORTED, "relation of %lld tuples reaches 2^31", (long long)R.n_tuples);
  const size_t need = size_t(elems) * size_t(esz_of(dtype));
  if (!dev_buf) return fail(ctx, JAGG_E_INVALID, "NULL device buffer");
  if (reinterpret_cast<uintptr_t>(dev_buf) % 16) return fail(ctx, JAGG_E_INVALID, "device buffer not 16-byte aligned");
  if (buf_bytes < need)
    return fail(ctx, JAGG_E_SHAPE, "buffer of %zu bytes, relation needs %zu", buf_bytes, need);
  R.dt = dtype;
  R.buf = dev_buf;
  R.bytes = buf_bytes;
  *out = new jagg_relation(R);
  return JAGG_OK;
}

jagg_status jagg_relation_destroy(jagg_relation *rel) {
  if (!rel) return JAGG_E_INVALID;
  delete rel;
  return JAGG_OK;
}

jagg_status jagg_repartition(jagg_ctx *ctx, const jagg_relation *src, jagg_relation *dst) {
  if (!ctx || !src || !dst) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  if (src->dt != dst->dt) return fail(ctx, JAGG_E_SHAPE, "source and destination dtypes differ");
  if (src->r != dst->r) return fail(ctx, JAGG_E_SHAPE, "source and destination ranks differ");
  for (int p = 0; p < dst->r; ++p) {
    const char *q = strchr(src->letters, dst->letters[p]);
    if (!q) return fail(ctx, JAGG_E_SHAPE, "letter '%c' is not in the source", dst->letters[p]);
    if (src->n[q - src->letters] != dst->n[p])
      return fail(ctx, JAGG_E_SHAPE, "letter '%c' has extent %lld in the source, %lld in the destination",
                  dst->letters[p], (long long)src->n[q - src->letters], (long long)dst->n[p]);
  }
  const char *sb = static_cast<const char *>(src->buf), *db = static_cast<const char *>(dst->buf);
  const size_t sn = size_t(src->n_tuples * src->be) * esz_of(src->dt), dn = size_t(dst->n_tuples * dst->be) * esz_of(dst->dt);
  if (sb < db + dn && db < sb + sn) return fail(ctx, JAGG_E_INVALID, "source and destination overlap");
  return do_repartition(ctx, *src, *dst);
}

jagg_status jagg_einsum_workspace(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                                  const int32_t *blockings, size_t *bytes) {
  if (!ctx || !bytes) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  Bound b;
  jagg_status st = bind(ctx, spec, in, n_in, blockings, b);
  if (st != JAGG_OK) return st;
  *bytes = b.total;
  return JAGG_OK;
}

jagg_status jagg_einsum(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                        const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes) {
  return einsum_impl(ctx, spec, in, n_in, blockings, out, workspace, ws_bytes, false);
}

jagg_status jagg_einsum_noalloc(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                                const int32_t *blockings, jagg_relation *out) {
  if (!ctx) return JAGG_E_INVALID;
  return einsum_impl(ctx, spec, in, n_in, blockings, out, ctx->scratch, JAGG_NOALLOC_SCRATCH_BYTES, true);
}

jagg_status jagg_plan_create(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                             const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes,
                             jagg_plan **plan) {
  if (!ctx || !plan) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  *plan = nullptr;
  jagg_plan *P = new jagg_plan;
  P->device = ctx->device;
  jagg_status st = build_call(ctx, spec, in, n_in, blockings, out, workspace, ws_bytes, false, P->call);
  if (st == JAGG_OK) st = launch_join_of(ctx, P->call);
  if (st != JAGG_OK) {
    delete P;
    return st;
  }
  *plan = P;
  return JAGG_OK;
}

jagg_status jagg_plan_run(jagg_ctx *ctx, const jagg_plan *plan) {
  if (!ctx || !plan) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  if (plan->device != ctx->device)
    return fail(ctx, JAGG_E_INVALID, "plan made for device %d, context on device %d", plan->device, ctx->device);
  if (plan->members.empty()) return launch_call(ctx, plan->call, false);
  jagg_status st;
  for (const PlannedCall &m : plan->members)
    if ((st = launch_reblocks(ctx, m)) != JAGG_OK) return st;
  for (const std::vector<int> &L : plan->launches) {
    if (L.size() == 1) {
      if ((st = launch_kernel(ctx, plan->members[L[0]])) != JAGG_OK) return st;
      continue;
    }
    const PlannedCall &m0 = plan->members[L[0]];
    DmaGroupArgs ga;
    memset(&ga, 0, sizeof(ga));
    ga.common = m0.ca;
    ga.n = int32_t(L.size());
    for (size_t i = 0; i < L.size(); ++i) {
      const ContractArgs &c = plan->members[L[i]].ca;
      ga.A[i] = c.A;
      ga.B[i] = c.B;
      ga.C[i] = c.C;
      ga.list[i] = c.list;
      ga.counts[i] = c.counts;
      ga.X[i] = c.X;
      ga.B2[i] = c.B2;
    }
    hipError_t e = hipSuccess;
    if (!launch_contract_bf16_group(ga, m0.out_bf16, m0.akc, m0.bkc, m0.va, m0.vb, m0.big, ctx->stream, &e))
      return fail(ctx, JAGG_E_UNSUPPORTED, "grouped launch refused its form");  // jagg_plan_group checked it
    if (ctx->trace)
      fprintf(stderr, "[jagg] group of %d: contract bf16 256x256 lds pipeline, one launch (%s, ...)\n", ga.n,
              m0.einsum.c_str());
    if ((st = after_launch(ctx, e, "grouped contract")) != JAGG_OK) return st;
  }
  return JAGG_OK;
}

jagg_status jagg_plan_group(jagg_ctx *ctx, int n, const jagg_plan *const *plans, jagg_plan **group) {
  if (!ctx || !plans || !group || n < 1) return fail(ctx, JAGG_E_INVALID, "NULL argument or empty group");
  *group = nullptr;
  std::vector<const PlannedCall *> calls;
  for (int i = 0; i < n; ++i) {
    const jagg_plan *q = plans[i];
    if (!q) return fail(ctx, JAGG_E_INVALID, "plan %d is NULL", i);
    if (q->device != ctx->device) return fail(ctx, JAGG_E_INVALID, "plan %d is for another device", i);
    if (q->members.empty()) {
      calls.push_back(&q->call);
    } else {
      for (const PlannedCall &m : q->members) calls.push_back(&m);
    }
  }
  // independence: nothing one member writes may be read or written by another
  auto overlap = [](const std::pair<const char *, size_t> &x, const std::pair<const char *, size_t> &y) {
    return x.first < y.first + y.second && y.first < x.first + x.second;
  };
  for (size_t i = 0; i < calls.size(); ++i)
    for (size_t j = 0; j < calls.size(); ++j) {
      if (i == j) continue;
      for (const auto &w : calls[i]->writes) {
        for (const auto &r : calls[j]->reads)
          if (overlap(w, r)) return fail(ctx, JAGG_E_INVALID, "group member %zu writes what member %zu reads", i, j);
        for (const auto &w2 : calls[j]->writes)
          if (overlap(w, w2)) return fail(ctx, JAGG_E_INVALID, "group members %zu and %zu write the same memory", i, j);
      }
    }
  jagg_plan *G = new jagg_plan;
  G->device = ctx->device;
  for (const PlannedCall *c : calls) G->members.push_back(*c);
  // launches: members of one contraction form share a launch (up to kMaxGroup)
  std::vector<bool> done(calls.size(), false);
  for (size_t i = 0; i < calls.size(); ++i) {
    if (done[i]) continue;
    std::vector<int> L{int(i)};
    done[i] = true;
    const bool groupable = calls[i]->kind == PlannedCall::CONTRACT && calls[i]->dtype == 1 && calls[i]->big &&
                           calls[i]->va == 8 && calls[i]->vb == 8 && !calls[i]->ca.causal_red &&
                           (calls[i]->ca.epi == 0 || calls[i]->akc) && calls[i]->ca.split <= 1;
    for (size_t j = i + 1; groupable && j < calls.size() && int(L.size()) < kMaxGroup; ++j)
      if (!done[j] && same_contraction_form(*calls[i], *calls[j])) {
        L.push_back(int(j));
        done[j] = true;
      }
    G->launches.push_back(L);
  }
  *group = G;
  return JAGG_OK;
}

jagg_status jagg_plan_fuse(jagg_ctx *ctx, const jagg_plan *first, const jagg_plan *second, jagg_plan **fused) {
  if (!ctx || !first || !second || !fused) return fail(ctx, JAGG_E_INVALID, "NULL argument");
  *fused = nullptr;
  if (first->device != ctx->device || second->device != ctx->device)
    return fail(ctx, JAGG_E_INVALID, "a plan is for another device");
  if (!first->members.empty() || !second->members.empty())
    return fail(ctx, JAGG_E_UNSUPPORTED, "no fused RMS-norm pair: groups do not fuse");
  const PlannedCall &R = first->call, &M = second->call;
  NormArgs n;
  const jagg_status st = plan_norm_pair(ctx, R, M, n);
  if (st != JAGG_OK) return st;
  jagg_plan *F = new jagg_plan;
  F->device = ctx->device;
  PlannedCall &P = F->call;
  P.kind = PlannedCall::NORM;
  P.einsum = R.einsum + " + " + M.einsum;
  P.norm = n;
  P.reads = R.reads;
  for (const auto &q : M.reads)
    if (q.first != static_cast<const char *>(R.ew.out)) P.reads.push_back(q);
  P.writes = R.writes;
  P.writes.insert(P.writes.end(), M.writes.begin(), M.writes.end());
  *fused = F;
  return JAGG_OK;
}

jagg_status jagg_plan_destroy(jagg_plan *plan) {
  if (!plan) return JAGG_E_INVALID;
  delete plan;
  return JAGG_OK;
}

jagg_status jagg_join_shape(const jagg_spec *spec, const int64_t *extents_by_letter, const int32_t *blockings,
                            int64_t *n_keys, int64_t *per_key) {
  if (!spec || !extents_by_letter || !blockings || !n_keys || !per_key) return JAGG_E_INVALID;
  Spec p;
  jagg_status st = parse(nullptr, spec->einsum, p);
  if (st != JAGG_OK) return st;
  int64_t nk = 1, pk = 1;
  for (size_t i = 0; i < p.order.size(); ++i) {
    if (blockings[i] < 1 || blockings[i] > extents_by_letter[i]) return JAGG_E_BLOCKING;
    if (p.out.find(p.order[i]) != std::string::npos) nk *= blockings[i];
    else pk *= blockings[i];
  }
  *n_keys = nk;
  *per_key = pk;
  return JAGG_OK;
}

jagg_status jagg_join_list(jagg_ctx *ctx, const jagg_spec *spec, const int64_t *extents_by_letter,
                           const int32_t *blockings, int32_t *dev_list, int32_t *dev_counts) {
  if (!ctx || !spec || !extents_by_letter || !blockings || !dev_list || !dev_counts)
    return fail(ctx, JAGG_E_INVALID, "NULL argument");
  Spec p;
  jagg_status st = parse(ctx, spec->einsum, p);
  if (st != JAGG_OK) return st;
  if ((st = check_spec(ctx, spec, p)) != JAGG_OK) return st;
  LetterInfo L;
  for (int i = 0; i < 26; ++i) {
    L.n[i] = 0;
    L.k[i] = 0;
  }
  for (size_t i = 0; i < p.order.size(); ++i) {
    const int c = p.order[i] - 'a';
    L.n[c] = extents_by_letter[i];
    L.k[c] = blockings[i];
    if (L.n[c] < 1) return fail(ctx, JAGG_E_SHAPE, "extent of '%c' must be >= 1", p.order[i]);
    const int64_t e = (L.n[c] + L.k[c] - 1) / std::max(L.k[c], 1);
    if (L.k[c] < 1 || L.k[c] > L.n[c] || (L.k[c] - 1) * e >= L.n[c])
      return fail(ctx, JAGG_E_BLOCKING, "bad blocking %d of '%c'", L.k[c], p.order[i]);
  }
  JoinArgs a;
  if ((st = plan_join(ctx, spec, p, L, a)) != JAGG_OK) return st;
  a.list = dev_list;
  a.counts = dev_counts;
  return after_launch(ctx, launch_join(a, ctx->stream), "join");
}

const char *jagg_status_str(jagg_status s) {
  switch (s) {
    case JAGG_OK: return "ok";
    case JAGG_E_INVALID: return "invalid argument";
    case JAGG_E_SHAPE: return "shape mismatch";
    case JAGG_E_BLOCKING: return "bad blocking";
    case JAGG_E_UNSUPPORTED: return "unsupported spec";
    case JAGG_E_WORKSPACE: return "workspace too small";
    case JAGG_E_DEVICE: return "device error";
  }
  return "unknown status";
}

const char *jagg_last_error(const jagg_ctx *ctx) { return ctx ? ctx->err.c_str() : "NULL context"; }

}  // extern "C"
