/* oracle_sanitize_driver.c -- test infrastructure: runs every entry point of
 * oracle/oracle.c on small, ragged cases so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only)
 * reports any out-of-bounds access, use of freed memory, leak or undefined
 * behaviour in the checker.  tests/test_oracle_sanitized.py compiles and
 * runs it.  The few value checks compare the oracle with itself (relational
 * against dense, a repartition round trip); the oracle's pins live in the
 * Python tests.  Exit status 0 and "0 failures" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_dense(const char *spec, int g, int agg, double alpha, double beta, double eps, int causal_s, int causal_t,
                 const int64_t *ext26, const double *const *ins, const int64_t *idx, int64_t n_out, double *out);
int oracle_dense_recompose(const char *spec, int kind, double alpha, const int64_t *ext26, const double *const *ins,
                           const int64_t *idx, int64_t n_out, double *out);
int oracle_relation_elems(const char *letters, const int64_t *ext26, const int32_t *nblk26, int64_t *elems);
int oracle_relation_elems_iv(const char *letters, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                             int64_t *elems);
int oracle_to_relation(const void *dense, int esz, const char *letters, const int64_t *ext26, const int32_t *nblk26,
                       void *rel);
int oracle_to_relation_iv(const void *dense, int esz, const char *letters, const int64_t *ext26,
                          const int32_t *nblk26, const int64_t *bnd26, void *rel);
int oracle_from_relation(const void *rel, int esz, const char *letters, const int64_t *ext26, const int32_t *nblk26,
                         void *dense);
int oracle_from_relation_iv(const void *rel, int esz, const char *letters, const int64_t *ext26,
                            const int32_t *nblk26, const int64_t *bnd26, void *dense);
int oracle_repartition(const void *src, int esz, const char *src_letters, const int32_t *src_nblk26, void *dst,
                       const char *dst_letters, const int32_t *dst_nblk26, const int64_t *ext26);
int oracle_repartition_iv(const void *src, int esz, const char *src_letters, const int32_t *src_nblk26,
                          const int64_t *src_bnd26, void *dst, const char *dst_letters, const int32_t *dst_nblk26,
                          const int64_t *dst_bnd26, const int64_t *ext26);
int oracle_join_list(const char *spec, const int64_t *ext26, const int32_t *nblk26, int causal_s, int causal_t,
                     int64_t *list, int64_t cap, int64_t *n_entries);
int oracle_join_list_iv(const char *spec, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                        int causal_s, int causal_t, int64_t *list, int64_t cap, int64_t *n_entries);
int oracle_relational(const char *spec, int g, int agg, double alpha, double beta, double eps, int causal_s,
                      int causal_t, const int64_t *ext26, const int32_t *nblk26, const double *const *in_rel,
                      double *out_rel, uint8_t *present);
int oracle_relational_iv(const char *spec, int g, int agg, double alpha, double beta, double eps, int causal_s,
                         int causal_t, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                         const double *const *in_rel, double *out_rel, uint8_t *present);
int oracle_attention_dense(const char *spec, double alpha, int causal_s, int causal_t, const int64_t *ext26,
                           const double *Q, const double *K, const double *V, const int64_t *idx, int64_t n_out,
                           double *out);
int oracle_attention_dense_seg(const char *spec, double alpha, int causal_s, int causal_t, int seg_s, int seg_t,
                               const int64_t *seg_bnd, int seg_k, const int64_t *ext26, const double *Q,
                               const double *K, const double *V, const int64_t *idx, int64_t n_out, double *out);
int oracle_attention_relational(const char *spec, double alpha, int causal_s, int causal_t, const int64_t *ext26,
                                const int32_t *nblk26, const double *const *in_rel, double *out_rel,
                                uint8_t *present);
int oracle_attention_relational_seg(const char *spec, double alpha, int causal_s, int causal_t, int seg_s, int seg_t,
                                    const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                                    const double *const *in_rel, double *out_rel, uint8_t *present);
void oracle_softmax_merge(double m1, double l1, double a1, double m2, double l2, double a2, double *res);
void oracle_round(double *x, int64_t n, int dtype);
int oracle_block_shape(const char *letters, const int64_t *ext26, const int32_t *nblk26, int64_t *e);
int oracle_block_shape_iv(const char *letters, const int64_t *ext26, const int32_t *nblk26, const int64_t *bnd26,
                          int64_t *e);

#define NB 65 /* bounds per letter row (64 intervals at most) */
#define LI(c) ((c) - 'a')

static int fails = 0;

static void check(int cond, const char *what) {
  if (!cond) {
    printf("FAIL: %s\n", what);
    ++fails;
  }
}

static void fill(double *x, int64_t n, uint32_t seed) {
  uint32_t s = seed * 2654435761u + 1u;
  for (int64_t i = 0; i < n; ++i) {
    s = s * 1664525u + 1013904223u;
    x[i] = ((double)(s >> 8) / 8388608.0) - 1.0;
  }
}

static double max_diff(const double *a, const double *b, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double d = fabs(a[i] - b[i]);
    if (d > m) m = d;
  }
  return m;
}

struct geo {
  int64_t ext[26];
  int32_t nb[26];
  int64_t bnd[26 * NB];
};

static void geo_init(struct geo *g) {
  memset(g->ext, 0, sizeof(g->ext));
  for (int i = 0; i < 26; ++i) g->nb[i] = 1;
  for (int i = 0; i < 26 * NB; ++i) g->bnd[i] = -1;
}

static double *relation_of(const double *dense, const char *letters, const struct geo *g, int64_t *n) {
  check(oracle_relation_elems_iv(letters, g->ext, g->nb, g->bnd, n) == 0, "relation_elems_iv");
  double *r = calloc((size_t)*n, sizeof(double));
  check(oracle_to_relation_iv(dense, 8, letters, g->ext, g->nb, g->bnd, r) == 0, "to_relation_iv");
  return r;
}

/* a contraction and a reduce: dense against relational over ragged blocks */
static void contraction_and_reduce(void) {
  struct geo g;
  geo_init(&g);
  g.ext[LI('i')] = 7, g.ext[LI('j')] = 5, g.ext[LI('k')] = 10;
  g.nb[LI('i')] = 3, g.nb[LI('j')] = 2, g.nb[LI('k')] = 4;
  double A[35], B[50], D[70], R[70];
  fill(A, 35, 1);
  fill(B, 50, 2);
  const double *ins[2] = {A, B};
  check(oracle_dense("ij,jk->ik", 0, 1, 1.0, 0.0, 0.0, -1, -1, g.ext, ins, NULL, 0, D) == 0, "dense ij,jk->ik");
  int64_t na, nbb, nc;
  double *Ar = relation_of(A, "ij", &g, &na), *Br = relation_of(B, "jk", &g, &nbb);
  check(oracle_relation_elems("ik", g.ext, g.nb, &nc) == 0, "relation_elems");
  double *Cr = calloc((size_t)nc, sizeof(double));
  uint8_t present[12];
  const double *rins[2] = {Ar, Br};
  check(oracle_relational("ij,jk->ik", 0, 1, 1.0, 0.0, 0.0, -1, -1, g.ext, g.nb, rins, Cr, present) == 0,
        "relational ij,jk->ik");
  check(oracle_from_relation(Cr, 8, "ik", g.ext, g.nb, R) == 0, "from_relation");
  check(max_diff(D, R, 70) < 1e-12, "relational equals dense");
  /* sampled outputs */
  int64_t idx[3] = {0, 31, 69};
  double S[3];
  check(oracle_dense("ij,jk->ik", 0, 1, 1.0, 0.0, 0.0, -1, -1, g.ext, ins, idx, 3, S) == 0, "dense sampled");
  check(S[1] == D[31], "sampled equals full");
  /* join list: count, then fill */
  int64_t ne = 0;
  check(oracle_join_list("ij,jk->ik", g.ext, g.nb, -1, -1, NULL, 0, &ne) == 0 && ne == 24, "join count");
  int64_t *lst = malloc((size_t)ne * 3 * sizeof(int64_t));
  check(oracle_join_list("ij,jk->ik", g.ext, g.nb, -1, -1, lst, ne, &ne) == 0, "join list");
  /* causal MAX reduce and a map with three inputs */
  struct geo h;
  geo_init(&h);
  h.ext[LI('b')] = 2, h.ext[LI('s')] = 6, h.ext[LI('t')] = 6, h.ext[LI('h')] = 5;
  h.nb[LI('s')] = 2, h.nb[LI('t')] = 2, h.nb[LI('h')] = 2;
  double X[72], M[12], Mr[12];
  fill(X, 72, 3);
  const double *xin[1] = {X};
  check(oracle_dense("bst->bs", 1, 2, 1.0, 0.0, 0.0, LI('s'), LI('t'), h.ext, xin, NULL, 0, M) == 0, "causal max");
  int64_t nx, nm;
  double *Xr = relation_of(X, "bst", &h, &nx);
  check(oracle_relation_elems("bs", h.ext, h.nb, &nm) == 0, "relation_elems bs");
  double *Mrel = calloc((size_t)nm, sizeof(double));
  uint8_t pm[2];
  const double *xr[1] = {Xr};
  check(oracle_relational("bst->bs", 1, 2, 1.0, 0.0, 0.0, LI('s'), LI('t'), h.ext, h.nb, xr, Mrel, pm) == 0,
        "relational causal max");
  check(oracle_from_relation(Mrel, 8, "bs", h.ext, h.nb, Mr) == 0 && max_diff(M, Mr, 12) == 0.0,
        "causal max relational equals dense");
  double Y[60], ssq[12], gam[5], Z[60];
  fill(Y, 60, 4);
  fill(gam, 5, 5);
  const double *yin[1] = {Y};
  check(oracle_dense("bsh->bs", 2, 1, 1.0, 0.0, 0.0, -1, -1, h.ext, yin, NULL, 0, ssq) == 0, "sum of squares");
  const double *zin[3] = {Y, ssq, gam};
  check(oracle_dense("bsh,bs,h->bsh", 5, 0, 1.0, 0.2, 1e-6, -1, -1, h.ext, zin, NULL, 0, Z) == 0, "rms scale");
  /* recompose maps */
  double P[70], B2[50], Q[70];
  const double *pin[3] = {A, B, D};
  check(oracle_dense_recompose("ij,jk,ik->ik", 0, 0.5, g.ext, pin, NULL, 0, P) == 0, "recompose mul_plus");
  fill(B2, 50, 11);
  const double *qin[3] = {A, B, B2};
  check(oracle_dense_recompose("ij,jk,jk->ik", 1, 1.0, g.ext, qin, NULL, 0, Q) == 0, "recompose swiglu");
  free(Ar), free(Br), free(Cr), free(lst), free(Xr), free(Mrel);
}

/* repartitions: uniform round trip, and through interval bounds */
static void repartitions(void) {
  struct geo s, d;
  geo_init(&s);
  s.ext[LI('a')] = 6, s.ext[LI('b')] = 11;
  d = s;
  s.nb[LI('a')] = 2, s.nb[LI('b')] = 3;
  d.nb[LI('a')] = 3, d.nb[LI('b')] = 4;
  double X[66], back[66];
  fill(X, 66, 6);
  int64_t ns, nd;
  double *Xs = relation_of(X, "ab", &s, &ns);
  check(oracle_relation_elems("ba", d.ext, d.nb, &nd) == 0, "relation_elems ba");
  double *Xd = calloc((size_t)nd, sizeof(double));
  check(oracle_repartition(Xs, 8, "ab", s.nb, Xd, "ba", d.nb, s.ext) == 0, "repartition");
  double T[66];
  check(oracle_from_relation(Xd, 8, "ba", d.ext, d.nb, T) == 0, "from_relation ba");
  for (int a = 0; a < 6; ++a)
    for (int b = 0; b < 11; ++b) back[a * 11 + b] = T[b * 6 + a];
  check(max_diff(X, back, 66) == 0.0, "repartition round trip");
  /* b as intervals [0, 2, 7, 11] */
  struct geo v = s;
  v.nb[LI('b')] = 3;
  const int64_t bb[4] = {0, 2, 7, 11};
  for (int i = 0; i < 4; ++i) v.bnd[LI('b') * NB + i] = bb[i];
  int64_t nv;
  check(oracle_relation_elems_iv("ab", v.ext, v.nb, v.bnd, &nv) == 0, "relation_elems_iv");
  double *Xv = calloc((size_t)nv, sizeof(double));
  check(oracle_repartition_iv(Xs, 8, "ab", s.nb, s.bnd, Xv, "ab", v.nb, v.bnd, s.ext) == 0, "repartition_iv");
  double U[66];
  check(oracle_from_relation_iv(Xv, 8, "ab", v.ext, v.nb, v.bnd, U) == 0 && max_diff(U, X, 66) == 0.0,
        "interval repartition round trip");
  int64_t e[2];
  check(oracle_block_shape("ab", s.ext, s.nb, e) == 0 && e[0] == 3 && e[1] == 4, "block shape");
  check(oracle_block_shape_iv("ab", v.ext, v.nb, v.bnd, e) == 0 && e[1] == 5, "block shape iv");
  /* an einsum and a join over the interval letter */
  double W[11], O[6], Or[6];
  fill(W, 11, 7);
  const double *win[2] = {X, W};
  check(oracle_dense("ab,b->a", 0, 1, 1.0, 0.0, 0.0, -1, -1, v.ext, win, NULL, 0, O) == 0, "dense ab,b->a");
  int64_t nw, no;
  double *Wv = relation_of(W, "b", &v, &nw);
  check(oracle_relation_elems_iv("a", v.ext, v.nb, v.bnd, &no) == 0, "relation_elems a");
  double *Ov = calloc((size_t)no, sizeof(double));
  uint8_t pr[2];
  const double *vin[2] = {Xv, Wv};
  check(oracle_relational_iv("ab,b->a", 0, 1, 1.0, 0.0, 0.0, -1, -1, v.ext, v.nb, v.bnd, vin, Ov, pr) == 0,
        "relational_iv");
  check(oracle_from_relation_iv(Ov, 8, "a", v.ext, v.nb, v.bnd, Or) == 0 && max_diff(O, Or, 6) < 1e-12,
        "interval relational equals dense");
  int64_t ne = 0;
  check(oracle_join_list_iv("ab,b->a", v.ext, v.nb, v.bnd, -1, -1, NULL, 0, &ne) == 0 && ne == 6, "join_iv count");
  free(Xs), free(Xd), free(Xv), free(Wv), free(Ov);
}

/* attention: dense against relational, causal, and over packed segments */
static void attention(void) {
  struct geo g;
  geo_init(&g);
  g.ext[LI('b')] = 2, g.ext[LI('s')] = 7, g.ext[LI('t')] = 7, g.ext[LI('d')] = 3, g.ext[LI('e')] = 4;
  g.nb[LI('s')] = 2, g.nb[LI('t')] = 2;
  double Q[42], K[42], V[56], Od[56], Or[56];
  fill(Q, 42, 8);
  fill(K, 42, 9);
  fill(V, 56, 10);
  const char *spec = "bsd,btd,bte->bse";
  check(oracle_attention_dense(spec, 0.5, LI('s'), LI('t'), g.ext, Q, K, V, NULL, 0, Od) == 0, "attention dense");
  int64_t nq, nk, nv, no;
  double *Qr = relation_of(Q, "bsd", &g, &nq), *Kr = relation_of(K, "btd", &g, &nk), *Vr = relation_of(V, "bte", &g, &nv);
  check(oracle_relation_elems("bse", g.ext, g.nb, &no) == 0, "relation_elems bse");
  double *Orel = calloc((size_t)no, sizeof(double));
  uint8_t pr[2];
  const double *ins[3] = {Qr, Kr, Vr};
  check(oracle_attention_relational(spec, 0.5, LI('s'), LI('t'), g.ext, g.nb, ins, Orel, pr) == 0,
        "attention relational");
  check(oracle_from_relation(Orel, 8, "bse", g.ext, g.nb, Or) == 0 && max_diff(Od, Or, 56) < 1e-12,
        "attention relational equals dense");
  /* two packed sequences [0, 3) and [3, 7) on s and t */
  const int64_t sb[3] = {0, 3, 7};
  double Os[56];
  check(oracle_attention_dense_seg(spec, 0.5, LI('s'), LI('t'), LI('s'), LI('t'), sb, 2, g.ext, Q, K, V, NULL, 0,
                                   Os) == 0,
        "attention dense segments");
  struct geo v = g;
  for (int i = 0; i < 3; ++i) v.bnd[LI('s') * NB + i] = sb[i], v.bnd[LI('t') * NB + i] = sb[i];
  int64_t mq, mk, mv, mo;
  double *Qv = relation_of(Q, "bsd", &v, &mq), *Kv = relation_of(K, "btd", &v, &mk), *Vv = relation_of(V, "bte", &v, &mv);
  check(oracle_relation_elems_iv("bse", v.ext, v.nb, v.bnd, &mo) == 0, "relation_elems_iv bse");
  double *Ov = calloc((size_t)mo, sizeof(double)), Ovd[56];
  uint8_t pv[4];
  const double *vins[3] = {Qv, Kv, Vv};
  check(oracle_attention_relational_seg(spec, 0.5, LI('s'), LI('t'), LI('s'), LI('t'), v.ext, v.nb, v.bnd, vins, Ov,
                                        pv) == 0,
        "attention relational segments");
  check(oracle_from_relation_iv(Ov, 8, "bse", v.ext, v.nb, v.bnd, Ovd) == 0 && max_diff(Os, Ovd, 56) < 1e-12,
        "segment attention relational equals dense");
  double res[3];
  oracle_softmax_merge(0.5, 2.0, 1.0, 1.5, 1.0, 3.0, res);
  double r[4] = {1.0, 1.00390625, 3.0e-39, -0.0};
  oracle_round(r, 4, 1);
  free(Qr), free(Kr), free(Vr), free(Orel), free(Qv), free(Kv), free(Vv), free(Ov);
}

int main(void) {
  contraction_and_reduce();
  repartitions();
  attention();
  printf("oracle sanitizer driver: %d failures\n", fails);
  return fails ? 1 : 0;
}
