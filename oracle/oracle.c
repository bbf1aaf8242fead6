/*
 * oracle.c -- plain, slow, obviously-correct CPU evaluation of join-agg einsum
 * specs over tensor relations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library; it parses specs, lays out blocks and rounds to bfloat16 by itself.
 *
 * Source: "Every Kernel Is a Join: Automatic Multi-GPU Parallelism for AI
 * Computations in Einsummable" (Ding et al.).
 *   - Def. 3.1  tensor type: per index a half-open interval [lower, upper).
 *   - Def. 3.2  tiling: index sets cover the tensor and are pairwise disjoint.
 *   - Sec. 1 / Sec. 3.2  tensor relation: the blocks of a tensor, each held
 *               with its key, the block's tensor type.
 *   - Def. 3.6  join-agg spec; Def. 3.7 implementation = join, aggregate with
 *               an associative and commutative op, recompose.
 *   - Sec. 3.3  one function specification per combination of intervals.
 * Everything is computed in IEEE double.  SUM accumulates in double, MAX is
 * exact, and rounding to the stored type happens once, at the end, in
 * oracle_round().
 *
 * Readings of points the page leaves open (each one is listed with the rest
 * of the design notes):
 *   - blocking of an index of extent n into k blocks: block extent
 *     e = ceil(n/k); block kappa covers [kappa*e, min((kappa+1)*e, n)); a
 *     blocking whose last block would be empty is rejected.
 *   - interval blocking (the `_iv` entry points): the caller lists the
 *     bounds 0 = b_0 < b_1 < ... < b_k = n of one index (Sec. 3.3 lets an
 *     index be split only at legal positions, e.g. the ends of packed
 *     sequences); block kappa covers [b_kappa, b_kappa+1), and every block is
 *     padded to the longest interval.  bnd26 holds 26 rows of ORIV+1 bounds,
 *     one per letter; a row whose first entry is negative means uniform.
 *   - storage of a relation: tuples in row-major order of the block
 *     coordinates, in the relation's own letter order; each block dense and
 *     row-major over the padded extents e; padding holds +0.
 *   - join-list order: by output tuple id, then by the block coordinates of
 *     the reduced letters, row-major in order of first appearance in the spec.
 *   - causal letters (s, t): the join keeps a combination only when some
 *     element with t <= s lies in it, and inside f every term with t > s is
 *     dropped; an output element whose own s, t have t > s is defined as 0.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <stdio.h>

#define OR_MAX_IN 3
#define OR_OK 0
#define OR_BAD_SPEC -1
#define OR_BAD_SHAPE -2
#define OR_BAD_BLOCKING -3
#define OR_UNSUPPORTED -4

/* elementwise functions g applied to the joined values before aggregation */
enum { G_MUL = 0, G_IDENT = 1, G_SQUARE = 2, G_EXP_SUB = 3, G_EXP_SUB_DIV = 4,
       G_RMS_SCALE = 5, G_SILU_MUL = 6, G_ADD = 7 };
/* aggregation (the page's associative, commutative combine) */
enum { AGG_NONE = 0, AGG_SUM = 1, AGG_MAX = 2 };

typedef struct {
  int n_in;
  char in[OR_MAX_IN][27];
  int in_len[OR_MAX_IN];
  char out[27];
  int out_len;
  char order[27];   /* every letter once, in order of first appearance */
  int n_letters;
  char reduced[27]; /* letters absent from the output, first-appearance order */
  int n_reduced;
} ospec;

static int letter_ok(char c) { return c >= 'a' && c <= 'z'; }

/* "ab,bc->ac": up to three inputs, lower-case letters, no letter twice in
 * one operand, every output letter present in some input. */
static int parse_spec(const char *s, ospec *p) {
  memset(p, 0, sizeof(*p));
  const char *arrow = strstr(s, "->");
  if (!arrow) return OR_BAD_SPEC;
  int cur = 0, len = 0;
  for (const char *c = s; c < arrow; ++c) {
    if (*c == ',') {
      if (len == 0) return OR_BAD_SPEC;
      p->in[cur][len] = 0; p->in_len[cur] = len;
      if (++cur >= OR_MAX_IN) return OR_BAD_SPEC;
      len = 0;
    } else if (letter_ok(*c)) {
      if (len >= 26) return OR_BAD_SPEC;
      p->in[cur][len++] = *c;
    } else {
      return OR_BAD_SPEC;
    }
  }
  if (len == 0) return OR_BAD_SPEC;
  p->in[cur][len] = 0; p->in_len[cur] = len;
  p->n_in = cur + 1;
  for (const char *c = arrow + 2; *c; ++c) {
    if (!letter_ok(*c) || p->out_len >= 26) return OR_BAD_SPEC;
    p->out[p->out_len++] = *c;
  }
  p->out[p->out_len] = 0;
  /* no repeated letter inside one operand */
  for (int j = 0; j <= p->n_in; ++j) {
    const char *o = j < p->n_in ? p->in[j] : p->out;
    int n = (int)strlen(o);
    for (int a = 0; a < n; ++a)
      for (int b = a + 1; b < n; ++b)
        if (o[a] == o[b]) return OR_BAD_SPEC;
  }
  for (int j = 0; j < p->n_in; ++j)
    for (int a = 0; a < p->in_len[j]; ++a)
      if (!strchr(p->order, p->in[j][a])) p->order[p->n_letters++] = p->in[j][a];
  for (int a = 0; a < p->out_len; ++a)
    if (!strchr(p->order, p->out[a])) return OR_BAD_SPEC; /* output letter from nowhere */
  for (int a = 0; a < p->n_letters; ++a)
    if (!strchr(p->out, p->order[a])) p->reduced[p->n_reduced++] = p->order[a];
  return OR_OK;
}

static double apply_g(int g, int n_in, const double *x, double beta, double eps) {
  switch (g) {
    case G_MUL: { double r = 1.0; for (int j = 0; j < n_in; ++j) r *= x[j]; return r; }
    case G_IDENT: return x[0];
    case G_SQUARE: return x[0] * x[0];
    case G_EXP_SUB: return exp(x[0] - x[1]);
    case G_EXP_SUB_DIV: return exp(x[0] - x[1]) / x[2];
    case G_RMS_SCALE: return x[0] / sqrt(x[1] * beta + eps) * x[2];
    case G_SILU_MUL: return x[0] / (1.0 + exp(-x[0])) * x[1];
    case G_ADD: { double r = 0.0; for (int j = 0; j < n_in; ++j) r += x[j]; return r; }
  }
  return NAN;
}

static int g_arity_ok(int g, int n_in) {
  switch (g) {
    case G_MUL: case G_ADD: return n_in >= 1;
    case G_IDENT: case G_SQUARE: return n_in == 1;
    case G_EXP_SUB: case G_SILU_MUL: return n_in == 2;
    case G_EXP_SUB_DIV: case G_RMS_SCALE: return n_in == 3;
  }
  return 0;
}

static int check_common(const ospec *p, int g, int agg, int causal_s, int causal_t) {
  if (agg < AGG_NONE || agg > AGG_MAX) return OR_UNSUPPORTED;
  if (!g_arity_ok(g, p->n_in)) return OR_UNSUPPORTED;
  if (agg == AGG_NONE && p->n_reduced) return OR_UNSUPPORTED; /* nothing to combine with */
  if ((causal_s >= 0) != (causal_t >= 0)) return OR_BAD_SPEC;
  if (causal_s >= 0) {
    if (!strchr(p->order, 'a' + causal_s) || !strchr(p->order, 'a' + causal_t)) return OR_BAD_SPEC;
    if (causal_s == causal_t) return OR_BAD_SPEC;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Dense form: out[o] = alpha * AGG_{r} g(in_1[..], ..., in_n[..]).           */
/* ------------------------------------------------------------------------ */

/* Evaluates the outputs whose row-major flat indices are listed in `idx`
 * (or all of them when idx == NULL, n_out then being the output size).
 * Inputs are dense, row-major in each operand's own letter order.  The
 * result is left unrounded in double. */
int oracle_dense(const char *spec, int g, int agg, double alpha, double beta, double eps,
                 int causal_s, int causal_t, const int64_t *ext26,
                 const double *const *ins, const int64_t *idx, int64_t n_out, double *out) {
  ospec p;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if ((rc = check_common(&p, g, agg, causal_s, causal_t))) return rc;
  for (int a = 0; a < p.n_letters; ++a)
    if (ext26[p.order[a] - 'a'] < 1) return OR_BAD_SHAPE;

  /* strides of each letter in each input (0 when the input lacks it) */
  int64_t in_stride[OR_MAX_IN][26];
  memset(in_stride, 0, sizeof(in_stride));
  for (int j = 0; j < p.n_in; ++j) {
    int64_t s = 1;
    for (int a = p.in_len[j] - 1; a >= 0; --a) {
      in_stride[j][p.in[j][a] - 'a'] = s;
      s *= ext26[p.in[j][a] - 'a'];
    }
  }
  int64_t out_total = 1;
  for (int a = 0; a < p.out_len; ++a) out_total *= ext26[p.out[a] - 'a'];
  int64_t red_total = 1;
  for (int a = 0; a < p.n_reduced; ++a) red_total *= ext26[p.reduced[a] - 'a'];
  if (!idx) n_out = out_total;

#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t q = 0; q < n_out; ++q) {
    int64_t flat = idx ? idx[q] : q;
    int64_t coord[26];
    memset(coord, 0, sizeof(coord));
    int64_t rem = flat;
    for (int a = p.out_len - 1; a >= 0; --a) {
      int64_t e = ext26[p.out[a] - 'a'];
      coord[p.out[a] - 'a'] = rem % e;
      rem /= e;
    }
    double acc = agg == AGG_MAX ? -INFINITY : 0.0;
    int any = 0;
    for (int64_t r = 0; r < red_total; ++r) {
      int64_t rr = r;
      for (int a = p.n_reduced - 1; a >= 0; --a) {
        int64_t e = ext26[p.reduced[a] - 'a'];
        coord[p.reduced[a] - 'a'] = rr % e;
        rr /= e;
      }
      if (causal_s >= 0 && coord[causal_t] > coord[causal_s]) continue;
      double x[OR_MAX_IN];
      for (int j = 0; j < p.n_in; ++j) {
        int64_t off = 0;
        for (int a = 0; a < p.in_len[j]; ++a) off += coord[p.in[j][a] - 'a'] * in_stride[j][p.in[j][a] - 'a'];
        x[j] = ins[j][off];
      }
      double v = apply_g(g, p.n_in, x, beta, eps);
      if (agg == AGG_MAX) { if (!any || v > acc) acc = v; }
      else acc += v;
      any = 1;
    }
    /* an element with no surviving term: 0 (the empty sum; under the causal
     * mask also for maps and maxima) */
    out[q] = any ? alpha * acc : 0.0;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Contractions whose recompose step applies a map to the aggregated value   */
/* (as attention's recompose writes a / l).  Def. 3.7: join, SUM the block   */
/* products of equal output key, then recompose; here the recompose also     */
/* takes an addend or a second sum of the same join:                         */
/*   RC_MUL_PLUS  out[o] = alpha * sum_r in0 in1 + in2[o]   (in2 holds only  */
/*                output letters: one addend per output element)             */
/*   RC_SWIGLU    a = sum_r in0 in1, b = sum_r in0 in2 (in1, in2 over the    */
/*                same letters), out[o] = alpha * a / (1 + e^-a) * b         */
/* Dense form, unrounded double; `idx` as for oracle_dense.                  */
/* ------------------------------------------------------------------------ */
enum { RC_MUL_PLUS = 0, RC_SWIGLU = 1 };

int oracle_dense_recompose(const char *spec, int kind, double alpha, const int64_t *ext26,
                           const double *const *ins, const int64_t *idx, int64_t n_out, double *out) {
  ospec p;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if (p.n_in != 3 || p.n_reduced == 0) return OR_UNSUPPORTED;
  if (kind == RC_MUL_PLUS) {
    for (int a = 0; a < p.in_len[2]; ++a)
      if (!strchr(p.out, p.in[2][a])) return OR_UNSUPPORTED; /* the addend holds output letters only */
  } else if (kind == RC_SWIGLU) {
    if (strcmp(p.in[1], p.in[2]) != 0) return OR_UNSUPPORTED; /* both sums over the same join */
  } else {
    return OR_UNSUPPORTED;
  }
  for (int a = 0; a < p.n_letters; ++a)
    if (ext26[p.order[a] - 'a'] < 1) return OR_BAD_SHAPE;
  int64_t in_stride[OR_MAX_IN][26];
  memset(in_stride, 0, sizeof(in_stride));
  for (int j = 0; j < p.n_in; ++j) {
    int64_t s = 1;
    for (int a = p.in_len[j] - 1; a >= 0; --a) {
      in_stride[j][p.in[j][a] - 'a'] = s;
      s *= ext26[p.in[j][a] - 'a'];
    }
  }
  int64_t out_total = 1;
  for (int a = 0; a < p.out_len; ++a) out_total *= ext26[p.out[a] - 'a'];
  int64_t red_total = 1;
  for (int a = 0; a < p.n_reduced; ++a) red_total *= ext26[p.reduced[a] - 'a'];
  if (!idx) n_out = out_total;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t q = 0; q < n_out; ++q) {
    int64_t coord[26];
    memset(coord, 0, sizeof(coord));
    int64_t rem = idx ? idx[q] : q;
    for (int a = p.out_len - 1; a >= 0; --a) {
      int64_t e = ext26[p.out[a] - 'a'];
      coord[p.out[a] - 'a'] = rem % e;
      rem /= e;
    }
    double s1 = 0.0, s2 = 0.0;
    for (int64_t r = 0; r < red_total; ++r) {
      int64_t rr = r;
      for (int a = p.n_reduced - 1; a >= 0; --a) {
        int64_t e = ext26[p.reduced[a] - 'a'];
        coord[p.reduced[a] - 'a'] = rr % e;
        rr /= e;
      }
      double x[OR_MAX_IN];
      for (int j = 0; j < p.n_in; ++j) {
        int64_t off = 0;
        for (int a = 0; a < p.in_len[j]; ++a) off += coord[p.in[j][a] - 'a'] * in_stride[j][p.in[j][a] - 'a'];
        x[j] = ins[j][off];
      }
      s1 += x[0] * x[1];
      if (kind == RC_SWIGLU) s2 += x[0] * x[2];
    }
    if (kind == RC_MUL_PLUS) {
      int64_t off = 0;
      for (int a = 0; a < p.in_len[2]; ++a) off += coord[p.in[2][a] - 'a'] * in_stride[2][p.in[2][a] - 'a'];
      out[q] = alpha * s1 + ins[2][off];
    } else {
      out[q] = alpha * (s1 / (1.0 + exp(-s1))) * s2;
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Relation geometry (Def. 3.1 intervals, padded blocks).                    */
/* ------------------------------------------------------------------------ */

/* Interval blockings (Sec. 3.2: a shardable index is decomposed into
 * intervals; Ex. 3.10: the intervals may sit at data-dependent positions,
 * such as the ends of packed sequences).  A letter blocked by explicit
 * bounds 0 = b_0 < b_1 < ... < b_k = n has block kappa = [b_kappa,
 * b_kappa+1); every block is stored padded to the longest one.  Bounds are
 * passed as 26 rows of ORIV + 1 entries, row L for letter 'a' + L; a row
 * whose first entry is negative leaves that letter uniformly blocked. */
#define ORIV 64

typedef struct {
  int r;
  char letters[27];
  int64_t n[26];      /* extents, by position in `letters` */
  int64_t k[26];      /* block counts */
  int64_t e[26];      /* padded block extents */
  int iv[26];         /* 1: blocked by the explicit bounds below */
  int64_t bnd[26][ORIV + 1];
  int64_t n_tuples;
  int64_t block_elems;
} orel;

static int make_rel_iv(const char *letters, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                       orel *R) {
  memset(R, 0, sizeof(*R));
  R->r = (int)strlen(letters);
  if (R->r > 26) return OR_BAD_SPEC;
  strcpy(R->letters, letters);
  R->n_tuples = 1; R->block_elems = 1;
  for (int a = 0; a < R->r; ++a) {
    int L = letters[a] - 'a';
    if (L < 0 || L >= 26) return OR_BAD_SPEC;
    R->n[a] = ext26[L];
    R->k[a] = nblk26[L];
    if (R->n[a] < 1 || R->k[a] < 1 || R->k[a] > R->n[a]) return OR_BAD_BLOCKING;
    const int64_t *b = bnd26 ? bnd26 + (size_t)L * (ORIV + 1) : NULL;
    if (b && b[0] >= 0) {
      if (R->k[a] > ORIV || b[0] != 0 || b[R->k[a]] != R->n[a]) return OR_BAD_BLOCKING;
      R->iv[a] = 1;
      R->e[a] = 0;
      for (int64_t q = 0; q < R->k[a]; ++q) {
        if (b[q + 1] <= b[q]) return OR_BAD_BLOCKING; /* empty or reversed interval */
        R->bnd[a][q] = b[q];
        if (b[q + 1] - b[q] > R->e[a]) R->e[a] = b[q + 1] - b[q];
      }
      R->bnd[a][R->k[a]] = R->n[a];
    } else {
      R->e[a] = (R->n[a] + R->k[a] - 1) / R->k[a];
      if ((R->k[a] - 1) * R->e[a] >= R->n[a]) return OR_BAD_BLOCKING; /* empty last block */
    }
    R->n_tuples *= R->k[a];
    R->block_elems *= R->e[a];
  }
  return OR_OK;
}

/* block coordinates of tuple t (row-major over the relation's letters) */
static void tuple_coords(const orel *R, int64_t t, int64_t *kappa) {
  for (int a = R->r - 1; a >= 0; --a) { kappa[a] = t % R->k[a]; t /= R->k[a]; }
}

/* the interval [lo, hi) of block kappa of the letter at position a */
static int64_t lo_of(const orel *R, int a, int64_t kappa) { return R->iv[a] ? R->bnd[a][kappa] : kappa * R->e[a]; }
static int64_t hi_of(const orel *R, int a, int64_t kappa) {
  if (R->iv[a]) return R->bnd[a][kappa + 1];
  int64_t h = (kappa + 1) * R->e[a];
  return h < R->n[a] ? h : R->n[a];
}

/* the block of the letter at position a that holds global coordinate x */
static int64_t block_of(const orel *R, int a, int64_t x) {
  if (!R->iv[a]) return x / R->e[a];
  int64_t q = 0;
  while (R->bnd[a][q + 1] <= x) ++q;
  return q;
}

/* value at global coordinates x (by letter) inside tuple `tid` (block coords kap) */
static double rel_at(const orel *R, const double *buf, int64_t tid, const int64_t *kap, const int64_t *x) {
  int64_t off = 0;
  for (int a = 0; a < R->r; ++a) off = off * R->e[a] + (x[R->letters[a] - 'a'] - lo_of(R, a, kap[a]));
  return buf[tid * R->block_elems + off];
}

int oracle_relation_elems_iv(const char *letters, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                             int64_t *elems) {
  orel R;
  int rc = make_rel_iv(letters, ext26, nblk26, bnd26, &R);
  if (rc) return rc;
  *elems = R.n_tuples * R.block_elems;
  return OR_OK;
}
int oracle_relation_elems(const char *letters, const int64_t *ext26, const int32_t *nblk26, int64_t *elems) {
  return oracle_relation_elems_iv(letters, ext26, nblk26, NULL, elems);
}

/* dense (row-major) -> relation storage, padding = +0; elements of `esz` bytes */
int oracle_to_relation_iv(const void *dense, int esz, const char *letters, const int64_t *ext26,
                          const int32_t *nblk26, const int64_t *bnd26, void *rel) {
  orel R;
  int rc = make_rel_iv(letters, ext26, nblk26, bnd26, &R);
  if (rc) return rc;
  memset(rel, 0, (size_t)(R.n_tuples * R.block_elems) * (size_t)esz);
  int64_t dstride[26], s = 1;
  for (int a = R.r - 1; a >= 0; --a) { dstride[a] = s; s *= R.n[a]; }
  for (int64_t t = 0; t < R.n_tuples; ++t) {
    int64_t kappa[26];
    tuple_coords(&R, t, kappa);
    for (int64_t w = 0; w < R.block_elems; ++w) {
      int64_t rem = w, doff = 0, valid = 1;
      for (int a = R.r - 1; a >= 0; --a) {
        int64_t x = lo_of(&R, a, kappa[a]) + rem % R.e[a];
        rem /= R.e[a];
        if (x >= hi_of(&R, a, kappa[a])) { valid = 0; break; }
        doff += x * dstride[a];
      }
      if (valid)
        memcpy((char *)rel + (size_t)(t * R.block_elems + w) * esz, (const char *)dense + (size_t)doff * esz, esz);
    }
  }
  return OR_OK;
}

/* relation storage -> dense (row-major); padding is dropped */
int oracle_to_relation(const void *dense, int esz, const char *letters, const int64_t *ext26,
                       const int32_t *nblk26, void *rel) {
  return oracle_to_relation_iv(dense, esz, letters, ext26, nblk26, NULL, rel);
}
/* relation storage -> dense (row-major); padding is skipped */
int oracle_from_relation_iv(const void *rel, int esz, const char *letters, const int64_t *ext26,
                            const int32_t *nblk26, const int64_t *bnd26, void *dense) {
  orel R;
  int rc = make_rel_iv(letters, ext26, nblk26, bnd26, &R);
  if (rc) return rc;
  int64_t dstride[26], s = 1;
  for (int a = R.r - 1; a >= 0; --a) { dstride[a] = s; s *= R.n[a]; }
  for (int64_t t = 0; t < R.n_tuples; ++t) {
    int64_t kappa[26];
    tuple_coords(&R, t, kappa);
    for (int64_t w = 0; w < R.block_elems; ++w) {
      int64_t rem = w, doff = 0, valid = 1;
      for (int a = R.r - 1; a >= 0; --a) {
        int64_t x = lo_of(&R, a, kappa[a]) + rem % R.e[a];
        rem /= R.e[a];
        if (x >= hi_of(&R, a, kappa[a])) { valid = 0; break; }
        doff += x * dstride[a];
      }
      if (valid)
        memcpy((char *)dense + (size_t)doff * esz, (const char *)rel + (size_t)(t * R.block_elems + w) * esz, esz);
    }
  }
  return OR_OK;
}
int oracle_from_relation(const void *rel, int esz, const char *letters, const int64_t *ext26,
                         const int32_t *nblk26, void *dense) {
  return oracle_from_relation_iv(rel, esz, letters, ext26, nblk26, NULL, dense);
}

/* Repartition: densify the source, then re-block into the destination's
 * letter order and blocking.  Works on raw element bytes, so it is exact. */
int oracle_repartition_iv(const void *src, int esz, const char *src_letters, const int32_t *src_nblk26,
                          const int64_t *src_bnd26, void *dst, const char *dst_letters, const int32_t *dst_nblk26,
                          const int64_t *dst_bnd26, const int64_t *ext26) {
  if (strlen(src_letters) != strlen(dst_letters)) return OR_BAD_SHAPE;
  for (const char *c = src_letters; *c; ++c)
    if (!strchr(dst_letters, *c)) return OR_BAD_SHAPE;
  int64_t n = 1;
  for (const char *c = src_letters; *c; ++c) n *= ext26[*c - 'a'];
  char *dense_src = malloc((size_t)n * esz), *dense_dst = malloc((size_t)n * esz);
  if (!dense_src || !dense_dst) { free(dense_src); free(dense_dst); return OR_BAD_SHAPE; }
  int rc = oracle_from_relation_iv(src, esz, src_letters, ext26, src_nblk26, src_bnd26, dense_src);
  if (!rc) {
    /* permute the dense tensor from the source letter order to the destination's */
    int r = (int)strlen(src_letters);
    int64_t sstride[26], s = 1;
    for (int a = r - 1; a >= 0; --a) { sstride[src_letters[a] - 'a'] = s; s *= ext26[src_letters[a] - 'a']; }
    for (int64_t i = 0; i < n; ++i) {
      int64_t rem = i, soff = 0;
      for (int a = r - 1; a >= 0; --a) {
        int64_t e = ext26[dst_letters[a] - 'a'];
        soff += (rem % e) * sstride[dst_letters[a] - 'a'];
        rem /= e;
      }
      memcpy(dense_dst + (size_t)i * esz, dense_src + (size_t)soff * esz, esz);
    }
    rc = oracle_to_relation_iv(dense_dst, esz, dst_letters, ext26, dst_nblk26, dst_bnd26, dst);
  }
  free(dense_src); free(dense_dst);
  return rc;
}
int oracle_repartition(const void *src, int esz, const char *src_letters, const int32_t *src_nblk26,
                       void *dst, const char *dst_letters, const int32_t *dst_nblk26,
                       const int64_t *ext26) {
  return oracle_repartition_iv(src, esz, src_letters, src_nblk26, NULL, dst, dst_letters, dst_nblk26, NULL, ext26);
}

/* ------------------------------------------------------------------------ */
/* Relational form, Def. 3.7 taken literally.                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t out_id;
  int64_t red_key;          /* row-major rank of the reduced letters' block coords */
  int64_t in_id[OR_MAX_IN];
} combo;

static int cmp_combo(const void *a, const void *b) {
  const combo *x = a, *y = b;
  if (x->out_id != y->out_id) return x->out_id < y->out_id ? -1 : 1;
  if (x->red_key != y->red_key) return x->red_key < y->red_key ? -1 : 1;
  return 0;
}

/* Join step: nested loops over the cross product of the input tuple sets,
 * keeping each combination whose key intervals agree on every letter the
 * inputs share (and, with causal letters, that holds some t <= s).
 * Returns a malloc'd array of combos sorted in canonical order. */
static int join(const ospec *p, const orel *in, const orel *out, int causal_s, int causal_t, int seg_s, int seg_t,
                combo **res, int64_t *n_res) {
  int64_t total = 1;
  for (int j = 0; j < p->n_in; ++j) total *= in[j].n_tuples;
  combo *list = malloc(sizeof(combo) * (size_t)(total ? total : 1));
  if (!list) return OR_BAD_SHAPE;
  int64_t n = 0;
  for (int64_t c = 0; c < total; ++c) {
    int64_t tid[OR_MAX_IN], rem = c;
    for (int j = p->n_in - 1; j >= 0; --j) { tid[j] = rem % in[j].n_tuples; rem /= in[j].n_tuples; }
    /* interval of every letter as fixed by the first input that holds it */
    int64_t lo[26], hi[26];
    int have[26];
    memset(have, 0, sizeof(have));
    int keep = 1;
    for (int j = 0; j < p->n_in && keep; ++j) {
      int64_t kappa[26];
      tuple_coords(&in[j], tid[j], kappa);
      for (int a = 0; a < in[j].r; ++a) {
        int L = in[j].letters[a] - 'a';
        int64_t l = lo_of(&in[j], a, kappa[a]), h = hi_of(&in[j], a, kappa[a]);
        if (!have[L]) { lo[L] = l; hi[L] = h; have[L] = 1; }
        else if (lo[L] != l || hi[L] != h) { keep = 0; break; }
      }
    }
    if (!keep) continue;
    if (causal_s >= 0 && lo[causal_t] > hi[causal_s] - 1) continue;
    /* segment pair: s and t must lie in the same interval */
    if (seg_s >= 0 && (lo[seg_s] != lo[seg_t] || hi[seg_s] != hi[seg_t])) continue;
    /* output key: the intervals of the output letters, as a tuple id */
    int64_t out_id = 0;
    for (int a = 0; a < out->r; ++a) {
      int L = out->letters[a] - 'a';
      out_id = out_id * out->k[a] + block_of(out, a, lo[L]);
    }
    /* reduced letters: block coordinates as the first input holding each one sees them */
    int64_t red_key = 0;
    for (int a = 0; a < p->n_reduced; ++a) {
      int L = p->reduced[a] - 'a';
      for (int j = 0; j < p->n_in; ++j) {
        const char *q = strchr(in[j].letters, 'a' + L);
        if (!q) continue;
        int ia = (int)(q - in[j].letters);
        red_key = red_key * in[j].k[ia] + block_of(&in[j], ia, lo[L]);
        break;
      }
    }
    list[n].out_id = out_id;
    list[n].red_key = red_key;
    for (int j = 0; j < OR_MAX_IN; ++j) list[n].in_id[j] = j < p->n_in ? tid[j] : -1;
    ++n;
  }
  qsort(list, (size_t)n, sizeof(combo), cmp_combo);
  *res = list;
  *n_res = n;
  return OR_OK;
}

static int build_rels(const ospec *p, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26, orel *in,
                      orel *out) {
  int rc;
  for (int j = 0; j < p->n_in; ++j)
    if ((rc = make_rel_iv(p->in[j], ext26, nblk26, bnd26, &in[j]))) return rc;
  return make_rel_iv(p->out, ext26, nblk26, bnd26, out);
}

/* Join list only: entries [out_id, in_id_0, ..., in_id_{n-1}] (int64), in
 * canonical order.  Pass list == NULL to get the count. */
int oracle_join_list_iv(const char *spec, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                        int causal_s, int causal_t, int64_t *list, int64_t cap, int64_t *n_entries) {
  ospec p;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if ((causal_s >= 0) != (causal_t >= 0)) return OR_BAD_SPEC;
  orel in[OR_MAX_IN], out;
  if ((rc = build_rels(&p, ext26, nblk26, bnd26, in, &out))) return rc;
  combo *c;
  int64_t n;
  if ((rc = join(&p, in, &out, causal_s, causal_t, -1, -1, &c, &n))) return rc;
  *n_entries = n;
  if (list) {
    if (cap < n) { free(c); return OR_BAD_SHAPE; }
    for (int64_t i = 0; i < n; ++i) {
      list[i * (p.n_in + 1)] = c[i].out_id;
      for (int j = 0; j < p.n_in; ++j) list[i * (p.n_in + 1) + 1 + j] = c[i].in_id[j];
    }
  }
  free(c);
  return OR_OK;
}
int oracle_join_list(const char *spec, const int64_t *ext26, const int32_t *nblk26, int causal_s,
                     int causal_t, int64_t *list, int64_t cap, int64_t *n_entries) {
  return oracle_join_list_iv(spec, ext26, nblk26, NULL, causal_s, causal_t, list, cap, n_entries);
}

/* Relational evaluation.  Inputs are relation buffers (double values) in the
 * operands' letter orders under `nblk26`; the output relation buffer gets the
 * aggregated blocks, +0 in its padding, unrounded.  `present` (optional, one
 * byte per output tuple) marks the output keys that the join produced. */
int oracle_relational_iv(const char *spec, int g, int agg, double alpha, double beta, double eps,
                         int causal_s, int causal_t, const int64_t *ext26, const int32_t *nblk26,
                         const int64_t *bnd26, const double *const *in_rel, double *out_rel, uint8_t *present) {
  ospec p;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if ((rc = check_common(&p, g, agg, causal_s, causal_t))) return rc;
  orel in[OR_MAX_IN], out;
  if ((rc = build_rels(&p, ext26, nblk26, bnd26, in, &out))) return rc;
  combo *c;
  int64_t n;
  if ((rc = join(&p, in, &out, causal_s, causal_t, -1, -1, &c, &n))) return rc;

  memset(out_rel, 0, sizeof(double) * (size_t)(out.n_tuples * out.block_elems));
  if (present) memset(present, 0, (size_t)out.n_tuples);
  double *agg_blk = malloc(sizeof(double) * (size_t)out.block_elems);
  uint8_t *touched = malloc((size_t)out.block_elems);

  for (int64_t first = 0; first < n;) {
    int64_t last = first;
    while (last < n && c[last].out_id == c[first].out_id) ++last;
    /* (2) Aggregate: combine the outputs of all combinations of this key */
    for (int64_t ci = first; ci < last; ++ci) {
      /* the combination's intervals per letter */
      int64_t lo[26], hi[26];
      for (int j = 0; j < p.n_in; ++j) {
        int64_t kappa[26];
        tuple_coords(&in[j], c[ci].in_id[j], kappa);
        for (int a = 0; a < in[j].r; ++a) {
          lo[in[j].letters[a] - 'a'] = lo_of(&in[j], a, kappa[a]);
          hi[in[j].letters[a] - 'a'] = hi_of(&in[j], a, kappa[a]);
        }
      }
      /* (1) Join: f on the projected blocks, i.e. the dense form restricted to
       * the valid index ranges of this combination's intervals */
      int64_t out_box = 1, red_box = 1;
      for (int a = 0; a < out.r; ++a) out_box *= hi[out.letters[a] - 'a'] - lo[out.letters[a] - 'a'];
      for (int a = 0; a < p.n_reduced; ++a) red_box *= hi[p.reduced[a] - 'a'] - lo[p.reduced[a] - 'a'];
      int64_t kout[26];
      tuple_coords(&out, c[ci].out_id, kout);
      for (int64_t o = 0; o < out_box; ++o) {
        int64_t x[26], rem = o;
        for (int a = out.r - 1; a >= 0; --a) {
          int L = out.letters[a] - 'a';
          x[L] = lo[L] + rem % (hi[L] - lo[L]);
          rem /= hi[L] - lo[L];
        }
        /* position inside the padded output block */
        int64_t w = 0;
        for (int a = 0; a < out.r; ++a) w = w * out.e[a] + (x[out.letters[a] - 'a'] - lo_of(&out, a, kout[a]));
        double acc = agg == AGG_MAX ? -INFINITY : 0.0;
        int any = 0;
        for (int64_t r = 0; r < red_box; ++r) {
          int64_t rr = r;
          for (int a = p.n_reduced - 1; a >= 0; --a) {
            int L = p.reduced[a] - 'a';
            x[L] = lo[L] + rr % (hi[L] - lo[L]);
            rr /= hi[L] - lo[L];
          }
          if (causal_s >= 0 && x[causal_t] > x[causal_s]) continue;
          double v[OR_MAX_IN];
          for (int j = 0; j < p.n_in; ++j) {
            int64_t kappa[26], off = 0;
            tuple_coords(&in[j], c[ci].in_id[j], kappa);
            for (int a = 0; a < in[j].r; ++a) {
              int L = in[j].letters[a] - 'a';
              off = off * in[j].e[a] + (x[L] - lo_of(&in[j], a, kappa[a]));
            }
            v[j] = in_rel[j][c[ci].in_id[j] * in[j].block_elems + off];
          }
          double gv = apply_g(g, p.n_in, v, beta, eps);
          if (agg == AGG_MAX) { if (!any || gv > acc) acc = gv; }
          else acc += gv;
          any = 1;
        }
        if (ci == first) { agg_blk[w] = any ? acc : (agg == AGG_MAX ? -INFINITY : 0.0); touched[w] = (uint8_t)any; }
        else if (any) {
          if (agg == AGG_MAX) { if (!touched[w] || acc > agg_blk[w]) agg_blk[w] = acc; }
          else agg_blk[w] += acc;
          touched[w] = 1;
        }
      }
    }
    /* (3) Recompose: the aggregated block takes its place in the output */
    int64_t kout[26], out_box = 1;
    tuple_coords(&out, c[first].out_id, kout);
    for (int a = 0; a < out.r; ++a) out_box *= hi_of(&out, a, kout[a]) - lo_of(&out, a, kout[a]);
    for (int64_t o = 0; o < out_box; ++o) {
      int64_t rem = o, w = 0, sub[26];
      for (int a = out.r - 1; a >= 0; --a) {
        int64_t ext = hi_of(&out, a, kout[a]) - lo_of(&out, a, kout[a]);
        sub[a] = rem % ext;
        rem /= ext;
      }
      for (int a = 0; a < out.r; ++a) w = w * out.e[a] + sub[a];
      double v = touched[w] ? alpha * agg_blk[w] : 0.0;
      out_rel[c[first].out_id * out.block_elems + w] = v;
    }
    if (present) present[c[first].out_id] = 1;
    first = last;
  }
  free(agg_blk); free(touched); free(c);
  return OR_OK;
}
int oracle_relational(const char *spec, int g, int agg, double alpha, double beta, double eps,
                      int causal_s, int causal_t, const int64_t *ext26, const int32_t *nblk26,
                      const double *const *in_rel, double *out_rel, uint8_t *present) {
  return oracle_relational_iv(spec, g, agg, alpha, beta, eps, causal_s, causal_t, ext26, nblk26, NULL, in_rel,
                              out_rel, present);
}

/* ------------------------------------------------------------------------ */
/* Attention as one join-agg: the online-softmax triple.                     */
/* ------------------------------------------------------------------------ */
/*
 * "Stax (5): Caching and Measurement", chapter summary (on its Section 9.10)
 * and exercise 15 on the triple (m, l, a): online softmax lets attention be
 * tiled like a reduction, the merge of triples being associative and
 * commutative; the summary's Proposition 9.1 gives the same semigroup on
 * (m, d) pairs for a single-pass softmax.  With "Every Kernel Is a Join"
 * Def. 3.7, attention over blocked Q, K, V is then one join-agg: f of a
 * joined (Q, K, V) tuple is the triple of its key range, the aggregation
 * merges triples, and the recompose step divides a by l.  The pages print
 * no formula for the merge; the reading taken here is the standard one:
 *   (m1, l1, a1) + (m2, l2, a2) = (M, l1 e^(m1-M) + l2 e^(m2-M),
 *                                    a1 e^(m1-M) + a2 e^(m2-M)),  M = max(m1, m2),
 * identity (-inf, 0, 0).
 *
 * Spec roles, "X s D, X t D, X t E -> X s E": X letters in every operand, s
 * in Q and the output only, t in K and V only (the reduced key letter), D
 * letters in Q and K only (contracted into the scores), E letters in V and
 * the output only.  score(s, t) = alpha * sum_D Q K; t > s is dropped under
 * a causal pair (s, t).
 *
 * Grouped-query attention (Sec. 3.3, Example 3.10: query heads 4m..4m+3 use
 * key-value head m): further letters in Q and the output only are query-
 * group letters G, "X G s D, X t D, X t E -> X G s E"; the rows of one group
 * share K and V.  With a causal pair s is its first letter; without one, the
 * last such letter of the spec (the choice changes nothing then).
 */
typedef struct {
  char x[27], d[27], e[27], g[27];
  int nx, nd, ne, ng;
  int s, t; /* letter indices 0..25 */
} oroles;

static int attention_roles(const ospec *p, int causal_s, oroles *r) {
  memset(r, 0, sizeof(*r));
  r->s = r->t = -1;
  if (p->n_in != 3) return OR_UNSUPPORTED;
  for (int a = 0; a < p->n_letters; ++a) {
    char c = p->order[a];
    int q = strchr(p->in[0], c) != NULL, k = strchr(p->in[1], c) != NULL;
    int v = strchr(p->in[2], c) != NULL, o = strchr(p->out, c) != NULL;
    if (q && k && v && o) r->x[r->nx++] = c;
    else if (q && !k && !v && o) r->g[r->ng++] = c; /* s or a query-group letter */
    else if (!q && k && v && !o) { if (r->t >= 0) return OR_UNSUPPORTED; r->t = c - 'a'; }
    else if (q && k && !v && !o) r->d[r->nd++] = c;
    else if (!q && !k && v && o) r->e[r->ne++] = c;
    else return OR_UNSUPPORTED;
  }
  if (r->ng == 0) return OR_UNSUPPORTED;
  if (causal_s >= 0) {
    if (!memchr(r->g, 'a' + causal_s, (size_t)r->ng)) return OR_BAD_SPEC;
    r->s = causal_s;
  } else {
    r->s = r->g[r->ng - 1] - 'a';
  }
  if (r->t < 0 || r->nd == 0 || r->ne == 0) return OR_UNSUPPORTED;
  return OR_OK;
}

/* offset of coordinate vector x (indexed by letter) in a dense operand */
static int64_t dense_off(const char *lt, const int64_t *ext26, const int64_t *x) {
  int64_t off = 0;
  for (const char *c = lt; *c; ++c) off = off * ext26[*c - 'a'] + x[*c - 'a'];
  return off;
}

/* score of (s, t) for the batch coordinates already in x: alpha * sum_D Q K */
static double att_score(const ospec *p, const oroles *r, const int64_t *ext26, const double *Q, const double *K,
                        int64_t *x, double alpha) {
  int64_t nd = 1;
  for (int a = 0; a < r->nd; ++a) nd *= ext26[r->d[a] - 'a'];
  double acc = 0.0;
  for (int64_t i = 0; i < nd; ++i) {
    int64_t rem = i;
    for (int a = r->nd - 1; a >= 0; --a) {
      int L = r->d[a] - 'a';
      x[L] = rem % ext26[L];
      rem /= ext26[L];
    }
    acc += Q[dense_off(p->in[0], ext26, x)] * K[dense_off(p->in[1], ext26, x)];
  }
  return alpha * acc;
}

/* Dense definition: out[X, s, E] = sum_t softmax_t(score(s, t)) V[X, t, E]
 * over the t that are kept (all, or t <= s under a causal pair, which must
 * name the s and t roles); 0 when none is.  Outputs at the row-major flat
 * indices in `idx` (all when idx == NULL). */
/* the segment (interval of seg_bnd) holding position x */
static int64_t segment_of(const int64_t *seg_bnd, int seg_k, int64_t x) {
  int64_t q = 0;
  while (q + 1 < seg_k && seg_bnd[q + 1] <= x) ++q;
  return q;
}

/* Packed sequences (Sec. 3.3, Example 3.10): with a segment pair (s, t) and
 * bounds seg_bnd[0..seg_k] (0 = b_0 < ... < b_k = extent of s and t), a
 * query position attends only to key positions of its own segment. */
int oracle_attention_dense_seg(const char *spec, double alpha, int causal_s, int causal_t, int seg_s, int seg_t,
                               const int64_t *seg_bnd, int seg_k, const int64_t *ext26, const double *Q,
                               const double *K, const double *V, const int64_t *idx, int64_t n_out, double *out) {
  ospec p;
  oroles r;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if ((rc = attention_roles(&p, causal_s, &r))) return rc;
  const int causal = causal_s >= 0;
  if (causal && (causal_s != r.s || causal_t != r.t)) return OR_BAD_SPEC;
  const int seg = seg_s >= 0;
  if ((seg_s >= 0) != (seg_t >= 0)) return OR_BAD_SPEC;
  if (seg) {
    if (seg_s != r.s || seg_t != r.t || ext26[r.s] != ext26[r.t] || seg_k < 1 || !seg_bnd) return OR_BAD_SPEC;
    if (seg_bnd[0] != 0 || seg_bnd[seg_k] != ext26[r.s]) return OR_BAD_BLOCKING;
    for (int q = 0; q < seg_k; ++q)
      if (seg_bnd[q + 1] <= seg_bnd[q]) return OR_BAD_BLOCKING;
  }
  int64_t out_total = 1;
  for (int a = 0; a < p.out_len; ++a) out_total *= ext26[p.out[a] - 'a'];
  if (!idx) n_out = out_total;
  const int64_t T = ext26[r.t];
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t q = 0; q < n_out; ++q) {
    int64_t x[26];
    memset(x, 0, sizeof(x));
    int64_t rem = idx ? idx[q] : q;
    for (int a = p.out_len - 1; a >= 0; --a) {
      int L = p.out[a] - 'a';
      x[L] = rem % ext26[L];
      rem /= ext26[L];
    }
    const int64_t s = x[r.s];
    const int64_t sg = seg ? segment_of(seg_bnd, seg_k, s) : 0;
    double m = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
      if (causal && t > s) continue;
      if (seg && segment_of(seg_bnd, seg_k, t) != sg) continue;
      x[r.t] = t;
      double sc = att_score(&p, &r, ext26, Q, K, x, alpha);
      if (sc > m) m = sc;
    }
    double l = 0.0, acc = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      if (causal && t > s) continue;
      if (seg && segment_of(seg_bnd, seg_k, t) != sg) continue;
      x[r.t] = t;
      double w = exp(att_score(&p, &r, ext26, Q, K, x, alpha) - m);
      l += w;
      acc += w * V[dense_off(p.in[2], ext26, x)];
    }
    out[q] = l > 0.0 ? acc / l : 0.0;
  }
  return OR_OK;
}

int oracle_attention_dense(const char *spec, double alpha, int causal_s, int causal_t, const int64_t *ext26,
                           const double *Q, const double *K, const double *V, const int64_t *idx, int64_t n_out,
                           double *out) {
  return oracle_attention_dense_seg(spec, alpha, causal_s, causal_t, -1, -1, NULL, 0, ext26, Q, K, V, idx, n_out,
                                    out);
}

/* the merge of two triples (the aggregation of the attention join-agg) */
void oracle_softmax_merge(double m1, double l1, double a1, double m2, double l2, double a2, double *res) {
  double M = m1 > m2 ? m1 : m2;
  if (M == -INFINITY) { res[0] = -INFINITY; res[1] = 0.0; res[2] = 0.0; return; }
  double w1 = m1 == -INFINITY ? 0.0 : exp(m1 - M), w2 = m2 == -INFINITY ? 0.0 : exp(m2 - M);
  res[0] = M;
  res[1] = l1 * w1 + l2 * w2;
  res[2] = a1 * w1 + a2 * w2;
}

/* Relational form: join the Q, K, V tuples (Def. 3.7 step 1, the same join
 * as every other spec), compute for each joined tuple and each output
 * element of its key the triple over the tuple's key range, merge the triples
 * of equal output key in canonical order (step 2), then write a / l into the
 * output relation (step 3).  Inputs are relation buffers of doubles; the D
 * letters must be one block each (a triple needs whole scores). */
int oracle_attention_relational_seg(const char *spec, double alpha, int causal_s, int causal_t, int seg_s,
                                    int seg_t, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                                    const double *const *in_rel, double *out_rel, uint8_t *present) {
  ospec p;
  oroles r;
  int rc = parse_spec(spec, &p);
  if (rc) return rc;
  if ((rc = attention_roles(&p, causal_s, &r))) return rc;
  const int causal = causal_s >= 0;
  if (causal && (causal_s != r.s || causal_t != r.t)) return OR_BAD_SPEC;
  for (int a = 0; a < r.nd; ++a)
    if (nblk26[r.d[a] - 'a'] != 1) return OR_UNSUPPORTED;
  orel in[OR_MAX_IN], out;
  if ((rc = build_rels(&p, ext26, nblk26, bnd26, in, &out))) return rc;
  combo *c;
  int64_t n;
  if ((seg_s >= 0) != (seg_t >= 0)) return OR_BAD_SPEC;
  if (seg_s >= 0 && (seg_s != r.s || seg_t != r.t)) return OR_BAD_SPEC;
  if ((rc = join(&p, in, &out, causal ? r.s : -1, causal ? r.t : -1, seg_s, seg_t, &c, &n))) return rc;
  memset(out_rel, 0, sizeof(double) * (size_t)(out.n_tuples * out.block_elems));
  if (present) memset(present, 0, (size_t)out.n_tuples);
  double *tm = malloc(sizeof(double) * (size_t)out.block_elems * 3);
  double *tl = tm + out.block_elems, *ta = tl + out.block_elems;
  for (int64_t first = 0; first < n;) {
    int64_t last = first;
    while (last < n && c[last].out_id == c[first].out_id) ++last;
    for (int64_t w = 0; w < out.block_elems; ++w) { tm[w] = -INFINITY; tl[w] = 0.0; ta[w] = 0.0; }
    int64_t kout[26];
    tuple_coords(&out, c[first].out_id, kout);
    for (int64_t ci = first; ci < last; ++ci) {
      int64_t lo[26], hi[26], kap[OR_MAX_IN][26];
      for (int j = 0; j < 3; ++j) {
        tuple_coords(&in[j], c[ci].in_id[j], kap[j]);
        for (int a = 0; a < in[j].r; ++a) {
          lo[in[j].letters[a] - 'a'] = lo_of(&in[j], a, kap[j][a]);
          hi[in[j].letters[a] - 'a'] = hi_of(&in[j], a, kap[j][a]);
        }
      }
      int64_t out_box = 1;
      for (int a = 0; a < out.r; ++a) out_box *= hi[out.letters[a] - 'a'] - lo[out.letters[a] - 'a'];
      int64_t nd = 1;
      for (int a = 0; a < r.nd; ++a) nd *= hi[r.d[a] - 'a'] - lo[r.d[a] - 'a'];
      for (int64_t o = 0; o < out_box; ++o) {
        int64_t x[26], rem = o;
        for (int a = out.r - 1; a >= 0; --a) {
          int L = out.letters[a] - 'a';
          x[L] = lo[L] + rem % (hi[L] - lo[L]);
          rem /= hi[L] - lo[L];
        }
        int64_t w = 0;
        for (int a = 0; a < out.r; ++a) w = w * out.e[a] + (x[out.letters[a] - 'a'] - lo_of(&out, a, kout[a]));
        /* f: the triple of this tuple's key range (two passes: max, then sums) */
        double m = -INFINITY, l = 0.0, acc = 0.0;
        for (int pass = 0; pass < 2; ++pass) {
          for (int64_t t = lo[r.t]; t < hi[r.t]; ++t) {
            if (causal && t > x[r.s]) continue;
            x[r.t] = t;
            double sc = 0.0;
            for (int64_t i = 0; i < nd; ++i) {
              int64_t rr = i;
              for (int a = r.nd - 1; a >= 0; --a) {
                int L = r.d[a] - 'a';
                x[L] = lo[L] + rr % (hi[L] - lo[L]);
                rr /= hi[L] - lo[L];
              }
              sc += rel_at(&in[0], in_rel[0], c[ci].in_id[0], kap[0], x) * rel_at(&in[1], in_rel[1], c[ci].in_id[1], kap[1], x);
            }
            sc *= alpha;
            if (pass == 0) {
              if (sc > m) m = sc;
            } else {
              double e = exp(sc - m);
              l += e;
              acc += e * rel_at(&in[2], in_rel[2], c[ci].in_id[2], kap[2], x);
            }
          }
        }
        double res[3];
        oracle_softmax_merge(tm[w], tl[w], ta[w], m, l, acc, res);
        tm[w] = res[0]; tl[w] = res[1]; ta[w] = res[2];
      }
    }
    /* recompose: a / l into the key's valid box; padding stays +0 */
    int64_t out_box = 1;
    for (int a = 0; a < out.r; ++a) out_box *= hi_of(&out, a, kout[a]) - lo_of(&out, a, kout[a]);
    for (int64_t o = 0; o < out_box; ++o) {
      int64_t rem = o, w = 0, sub[26];
      for (int a = out.r - 1; a >= 0; --a) {
        int64_t ext = hi_of(&out, a, kout[a]) - lo_of(&out, a, kout[a]);
        sub[a] = rem % ext;
        rem /= ext;
      }
      for (int a = 0; a < out.r; ++a) w = w * out.e[a] + sub[a];
      out_rel[c[first].out_id * out.block_elems + w] = tl[w] > 0.0 ? ta[w] / tl[w] : 0.0;
    }
    if (present) present[c[first].out_id] = 1;
    first = last;
  }
  free(tm);
  free(c);
  return OR_OK;
}
int oracle_attention_relational_iv(const char *spec, double alpha, int causal_s, int causal_t,
                                   const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                                   const double *const *in_rel, double *out_rel, uint8_t *present) {
  return oracle_attention_relational_seg(spec, alpha, causal_s, causal_t, -1, -1, ext26, nblk26, bnd26, in_rel,
                                         out_rel, present);
}
int oracle_attention_relational(const char *spec, double alpha, int causal_s, int causal_t, const int64_t *ext26,
                                const int32_t *nblk26, const double *const *in_rel, double *out_rel,
                                uint8_t *present) {
  return oracle_attention_relational_iv(spec, alpha, causal_s, causal_t, ext26, nblk26, NULL, in_rel, out_rel,
                                        present);
}

/* ------------------------------------------------------------------------ */
/* Rounding to the stored type, once, round-to-nearest-even.                 */
/* ------------------------------------------------------------------------ */

/* bfloat16: 8 significant bits, the exponent range of binary32.  Rounds the
 * exact double to the nearest representable value, ties to even, written
 * from the definition (scale so the quantum is 1, round, scale back). */
static double round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int ex;
  frexp(x, &ex);                 /* |x| = m * 2^ex, 0.5 <= m < 1 */
  int q = ex - 8;                /* quantum of an 8-bit significand */
  if (q < -133) q = -133;        /* subnormal quantum: 2^-126 * 2^-7 */
  double r = ldexp(nearbyint(ldexp(x, -q)), q);
  if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, x); /* beyond the largest finite */
  return r;
}

/* dtype 0 = float32, 1 = bfloat16; rounds n doubles in place */
void oracle_round(double *x, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) x[i] = dtype == 1 ? round_bf16(x[i]) : (double)(float)x[i];
}

/* padded block extents of a relation, in its letter order */
int oracle_block_shape_iv(const char *letters, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                          int64_t *e) {
  orel R;
  int rc = make_rel_iv(letters, ext26, nblk26, bnd26, &R);
  if (rc) return rc;
  for (int a = 0; a < R.r; ++a) e[a] = R.e[a];
  return OR_OK;
}
int oracle_block_shape(const char *letters, const int64_t *ext26, const int32_t *nblk26, int64_t *e) {
  return oracle_block_shape_iv(letters, ext26, nblk26, NULL, e);
}
