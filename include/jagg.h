/*
 * jagg.h -- C ABI of the join-agg einsum executor for AMD MI355X (gfx950).
 *
 * A tensor is held as a *tensor relation*: one tuple per block of a
 * blocking of every index, each tuple pairing the block's key (its interval
 * along every index) with the dense block itself ("Every Kernel Is a Join",
 * Ding et al., Sec. 1 and Sec. 3.2; keys are tensor types, Def. 3.1).  An einsum spec is executed as a join-agg spec (Def. 3.6) by the
 * three steps of Def. 3.7: join the input tuples whose keys agree on every
 * shared index, apply a block function to each joined tuple, combine the
 * results of equal output key with an associative and commutative
 * aggregation, and recompose.  Re-tiling a relation (the exchange step of
 * Sec. 5.3, on one GPU: decompose into atoms and recompose) is
 * jagg_repartition.
 *
 * Conventions shared by every entry point
 *  - Letters: an index is named by one lower-case letter 'a'..'z'.
 *  - Blocking (Sec. 3.3, one interval count per index): an index of extent n
 *    cut into k blocks has block extent e = ceil(n/k); block kappa covers
 *    [kappa*e, min((kappa+1)*e, n)).  A blocking whose last block would be
 *    empty ((k-1)*e >= n) is rejected with JAGG_E_BLOCKING.
 *  - Storage of a relation (caller-owned device memory): tuples in row-major
 *    order of their block coordinates, in the relation's letter order; each
 *    tuple is a dense row-major block over the padded extents e, so a
 *    relation occupies prod(k) * prod(e) elements.  Positions beyond an
 *    index's extent (padding) hold +0: every producer in this library writes
 *    them, and the kernels rely on it.
 *  - Ownership: the caller allocates and frees all device memory (relation
 *    storage, workspaces, join lists).  The library never allocates device
 *    memory; it owns only the host-side metadata behind jagg_ctx and
 *    jagg_relation handles.
 *  - Streams: every launch goes, asynchronously, onto the stream given to
 *    jagg_ctx_create.  A context is used by one host thread at a time.
 *  - Errors: argument, shape, blocking and workspace errors, and spec forms
 *    the kernels do not implement, are found before anything is launched
 *    and reported by a negative status; jagg_last_error() gives the detail.
 *    There is no fallback path: an unsupported spec is an error.
 */
#ifndef JAGG_H
#define JAGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JAGG_OK = 0,
  JAGG_E_INVALID = -1,     /* malformed argument: NULL handle, bad spec string, bad enum */
  JAGG_E_SHAPE = -2,       /* extents or letters disagree, buffer too small */
  JAGG_E_BLOCKING = -3,    /* bad block count, or the out relation's blocking differs */
  JAGG_E_UNSUPPORTED = -4, /* a spec form the kernels do not implement */
  JAGG_E_WORKSPACE = -5,   /* workspace missing or smaller than jagg_einsum_workspace() */
  JAGG_E_DEVICE = -6       /* a HIP call or kernel launch failed */
} jagg_status;

typedef enum { JAGG_F32 = 0, JAGG_BF16 = 1 } jagg_dtype;

/* The aggregation of Def. 3.7 step (2); each is associative and commutative.
 * JAGG_AGG_SOFTMAX ("Stax (5): Caching and Measurement", chapter summary on
 * Section 9.10: the online-softmax triple lets attention be tiled like a
 * reduction) merges triples
 * (m, l, a) as (M, l1 e^(m1-M) + l2 e^(m2-M), a1 e^(m1-M) + a2 e^(m2-M)),
 * M = max(m1, m2), identity (-inf, 0, 0), and its recompose step writes
 * a / l (0 where l = 0).  It pairs only with JAGG_G_ATTENTION. */
typedef enum { JAGG_AGG_NONE = 0, JAGG_AGG_SUM = 1, JAGG_AGG_MAX = 2, JAGG_AGG_SOFTMAX = 3 } jagg_agg;

/* Block function g applied, element by element, to the joined input values
 * x0, x1, x2 before aggregation.  With g = MUL and agg = SUM the spec is a
 * contraction (the matmul of Example 3.4 is 'ij,jk->ik'). */
typedef enum {
  JAGG_G_MUL = 0,         /* x0 * x1 (* x2)                          */
  JAGG_G_IDENT = 1,       /* x0                                      */
  JAGG_G_SQUARE = 2,      /* x0 * x0                                 */
  JAGG_G_EXP_SUB = 3,     /* exp(x0 - x1)                            */
  JAGG_G_EXP_SUB_DIV = 4, /* exp(x0 - x1) / x2                       */
  JAGG_G_RMS_SCALE = 5,   /* x0 / sqrt(x1 * beta + eps) * x2         */
  JAGG_G_SILU_MUL = 6,    /* x0 / (1 + exp(-x0)) * x1                */
  JAGG_G_ADD = 7,         /* x0 + x1 (+ x2)                          */
  JAGG_G_ATTENTION = 8,   /* with JAGG_AGG_SOFTMAX; see below        */
  JAGG_G_MUL_PLUS = 9,    /* contraction + addend; see below         */
  JAGG_G_SWIGLU = 10      /* gated pair of contractions; see below   */
} jagg_g;

/* Contractions whose recompose step maps the aggregated value (Def. 3.7:
 * join, SUM the block products of equal output key, recompose; as the
 * attention aggregation's recompose writes a / l).  Both take three inputs
 * and agg = JAGG_AGG_SUM, no causal or segment pair:
 *  - JAGG_G_MUL_PLUS: out = alpha * sum_r x0 x1 + x2, where x2 holds exactly
 *    the output letters in the output's order and blocking (one addend per
 *    output element: a residual add fused into the product that feeds it).
 *  - JAGG_G_SWIGLU: a = sum_r x0 x1 and b = sum_r x0 x2 over one join (x2
 *    laid out as x1: the same letters, dtype and blocking), out = alpha *
 *    silu(a) * b with silu(a) = a / (1 + e^-a): the gate and up projections of
 *    a SwiGLU feed-forward layer and their product, without writing either
 *    projection.  Runs on the bf16 256 x 128-tile pipeline only: bf16
 *    operands in 16-byte vectors, x0 contiguous along the reduced letters,
 *    x1 / x2 contributing the output's innermost letters
 *    (JAGG_E_UNSUPPORTED otherwise); any extents.
 * The inputs are read as stored (bf16 or f32 addend); sums accumulate in
 * fp32 and the map is applied before the single rounding to out_dtype. */

/* Attention as one join-agg (g = JAGG_G_ATTENTION, agg = JAGG_AGG_SOFTMAX).
 * The spec is "Q,K,V->O" with the letter roles "X s D, X t D, X t E -> X s E":
 * X (any number of letters) in all four operands, s in Q and O only, t in
 * K and V only, one letter D in Q and K only, one letter E in V and O only.
 * out[X,s,E] = sum_t softmax_t(alpha * sum_D Q[X,s,D] K[X,t,D]) V[X,t,E],
 * over every t, or over t <= s when the causal pair is (s, t).  The join
 * pairs each (X, s, E) block with the K/V blocks of every t block; f of a
 * joined tuple is the triple of its t range, the aggregation merges the
 * triples in join-list order.  Requirements (else JAGG_E_UNSUPPORTED):
 * alpha > 0; Q, K and V in bfloat16; D and E one block each, of equal padded extent 64 or
 * 128, innermost in their operands; row strides and block sizes multiples of
 * 8 elements; blocks under 2 GiB; at most 512 joined K/V tuples per output
 * tuple (t blocked at most 512 ways). */

/* One join-agg spec.  out[o] = alpha * AGG over the reduced letters of
 * g(x0, ...).  `einsum` is "in0,in1,...->out" (1 to 3 inputs); operand
 * letters bind to the relations' dimensions by position, so a relation
 * created with letters "bsh" may appear in a spec as "bth" provided the
 * extents and block counts agree.  A letter may not repeat inside one
 * operand, and every output letter must occur in some input.
 * causal_s / causal_t: 0 for none, else two letters (s, t) of the spec; then
 * only elements with t <= s take part: the join drops every tuple
 * combination whose t-block starts after its s-block ends and terms with
 * t > s are left out of the aggregation.  When both s and t are output
 * letters, an output tuple whose t-block lies after its s-block has no
 * joined tuple and is absent from the output relation: its storage slot is
 * neither written nor read by any kernel (it keeps whatever the buffer held,
 * so a buffer cleared once when allocated keeps +0 there), while inside a
 * present tuple every element with t > s is written as 0.  A spec under the
 * same causal pair never reads an absent tuple; any other consumer (a
 * repartition, a spec without the pair) reads the slot's bytes as they are.
 * A causal pair needs s and t of equal extent and block count.
 * seg_s / seg_t: 0 for none, else a segment pair (s, t): only elements whose
 * s and t lie in the same block take part, and the join keeps only the
 * combinations whose s and t blocks coincide.  "Every Kernel Is a Join",
 * Sec. 3.3, Example 3.10: three sequences packed into one index, attention
 * never crossing a sequence end, the index cut only at those ends -- with s
 * and t blocked by the sequences' bounds (jagg_relation_create_iv) each
 * query attends to its own sequence only; on uniform blocks it is
 * block-local attention.  Taken by g = JAGG_G_ATTENTION only, with (s, t)
 * its query and key letters, blocked alike (same bounds, or the same count
 * of uniform blocks); a causal pair, if any, must be the same (s, t). */
typedef struct {
  const char *einsum;
  jagg_g g;
  jagg_agg agg;
  jagg_dtype out_dtype;
  float alpha; /* scales the aggregated result; 1 for none */
  float beta;  /* parameter of JAGG_G_RMS_SCALE */
  float eps;   /* parameter of JAGG_G_RMS_SCALE */
  char causal_s;
  char causal_t;
  char seg_s;
  char seg_t;
} jagg_spec;

typedef struct jagg_ctx jagg_ctx;
typedef struct jagg_relation jagg_relation;

/* Context bound to one device and one stream (a hipStream_t, borrowed: the
 * library never creates, synchronises or destroys it; NULL = the default
 * stream).  Makes `device` current on the calling thread. */
jagg_status jagg_ctx_create(int device, void *hip_stream, jagg_ctx **out);
jagg_status jagg_ctx_destroy(jagg_ctx *ctx);

/* Padded storage size in bytes of a relation with `rank` letters (see the
 * storage convention above); host only. */
jagg_status jagg_relation_bytes(const char *letters, const int64_t *extents, const int32_t *nblocks,
                                jagg_dtype dtype, size_t *bytes);

/* Describes a relation over caller-owned device memory `dev_buf` of
 * `buf_bytes` bytes (at least jagg_relation_bytes(), 16-byte aligned).
 * letters[i] names dimension i, extents[i] >= 1 its extent, nblocks[i] its
 * block count.  Host metadata only; nothing is launched, the buffer is not
 * touched.  Limits: at most 8 letters, fewer than 2^36 elements and 2^31
 * tuples (a block kernel may ask less of its blocks: JAGG_E_UNSUPPORTED from
 * the call that would run it). */
jagg_status jagg_relation_create(jagg_ctx *ctx, const char *letters, const int64_t *extents,
                                 const int32_t *nblocks, jagg_dtype dtype, void *dev_buf, size_t buf_bytes,
                                 jagg_relation **out);
/* Interval-blocked relations.  "Every Kernel Is a Join" (Ding et al.):
 * a key is an interval per index (Def. 3.1), and Sec. 3.3 lets an index be
 * cut only at legal positions -- Example 3.10 splits a packed sequence
 * index only at the ends of its sequences, and the query heads of grouped-
 * query attention along with their key-value heads.  So the blocks of one
 * letter may differ in length.
 *
 * bounds[i] is NULL for a uniformly blocked letter (as above), or points
 * to nblocks[i] + 1 strictly increasing positions 0 = b_0 < ... < b_k =
 * extents[i]; block kappa then covers [b_kappa, b_kappa+1).  Every block of
 * such a letter is padded to the longest interval, max(b_kappa+1 - b_kappa),
 * and the storage convention is otherwise the one above.  At most 32
 * intervals per letter, and at most 192 bounds over both relations of one
 * repartition (JAGG_E_UNSUPPORTED beyond); bounds that do not run
 * from 0 to the extent or do not increase give JAGG_E_BLOCKING.  The bounds
 * are copied; the caller keeps ownership of the arrays.  bounds == NULL is
 * the uniform case for every letter.
 *
 * jagg_repartition converts between any two blockings, interval or uniform.
 * jagg_einsum takes interval-blocked inputs when every relation holding such
 * a letter (the output included) carries the same bounds and `blockings`
 * names their count; a letter blocked differently in two relations is
 * repartitioned by the caller first.  The block kernels compute the padding
 * positions as well, so the spec's value must be +0 wherever an interval
 * letter sits in padding: g = MUL, IDENT, SQUARE or SILU_MUL; ADD only when
 * every input holds every interval letter; RMS_SCALE only when its first
 * input does and eps > 0 (padded rows compute 0 * rsqrt(eps)); MAX only
 * over uniformly blocked letters; a causal pair on interval letters only
 * with attention under the same segment pair.
 * ATTENTION takes interval blocking on its (s, t) letters under a segment
 * pair (packed sequences; see jagg_spec), masking each block by its own
 * interval's length (JAGG_E_UNSUPPORTED otherwise). */
jagg_status jagg_relation_bytes_iv(const char *letters, const int64_t *extents, const int32_t *nblocks,
                                   const int64_t *const *bounds, jagg_dtype dtype, size_t *bytes);
jagg_status jagg_relation_create_iv(jagg_ctx *ctx, const char *letters, const int64_t *extents,
                                    const int32_t *nblocks, const int64_t *const *bounds, jagg_dtype dtype,
                                    void *dev_buf, size_t buf_bytes, jagg_relation **out);

/* Frees the metadata only, never dev_buf. */
jagg_status jagg_relation_destroy(jagg_relation *rel);

/* Repartition (Sec. 5.3): writes into `dst` the tensor held by `src`,
 * re-tiled to dst's blocking and letter order.  src and dst must carry the
 * same set of letters with equal extents and the same dtype; their order
 * and blocking may differ.  Every element of dst, padding (+0) included, is
 * written; the copy is bit-exact.  src and dst must not overlap. */
jagg_status jagg_repartition(jagg_ctx *ctx, const jagg_relation *src, jagg_relation *dst);

/* Bytes of device workspace jagg_einsum needs for this call (join list,
 * key counts, room for re-blocking any input whose blocking differs from
 * `blockings`, and, for a bf16 MUL / SUM contraction whose output tiles
 * fill the GPU in few or ragged waves, the fp32 partial sums of its split
 * walk: see step (2) of jagg_einsum). `blockings` gives the block count of
 * every letter of the spec, in order of first appearance in the einsum
 * string. */
jagg_status jagg_einsum_workspace(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in,
                                  int n_in, const int32_t *blockings, size_t *bytes);

/* Executes one join-agg spec (Def. 3.7) on the ctx stream:
 *   (0) an input whose blocking differs from `blockings` is repartitioned
 *       into the workspace first;
 *   (1) join: the join-enumeration kernel lists, for every output key, the
 *       input tuples that agree on every shared letter;
 *   (2) each joined tuple goes through g and is aggregated into its output
 *       key, accumulation in fp32 (MFMA for contractions).  A bf16 MUL /
 *       SUM contraction (no causal or segment pair, no recompose map) whose
 *       256 x 256 output tiles would fill the GPU in few or ragged waves
 *       splits each tile's walk over its joined tuples and K into parts
 *       run side by side; their fp32 partial sums go to the workspace and
 *       a second kernel adds them in part order (Def. 3.7: the SUM is
 *       associative and commutative, so only the rounding order changes);
 *   (3) recompose: the output relation `out` (letters of the spec's output,
 *       blocked by `blockings`, dtype spec->out_dtype) is written in place,
 *       padding +0.
 * Inputs are bf16 or f32 (a contraction needs both inputs of one dtype).
 * `workspace` (device, 256-byte aligned) holds at least
 * jagg_einsum_workspace() bytes and is clobbered.  `out` must not overlap an
 * input. */
jagg_status jagg_einsum(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                        const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes);

/* Prepared specs.  A chain that runs the same spec over the same relations
 * again and again (every step of a model block) repeats the host planning
 * and the join enumeration of jagg_einsum each time, although both depend
 * only on the spec, the relations' geometry and `blockings` ("Every Kernel
 * Is a Join", Def. 3.7: the join is a function of the tuples' keys, not of
 * their blocks' values).  jagg_plan_create does what jagg_einsum does up to
 * the join: it checks and plans the call (same arguments and errors as
 * jagg_einsum) and launches the join-enumeration kernel, on the ctx stream,
 * into `workspace` (at least jagg_einsum_workspace() bytes, 256-byte
 * aligned).  jagg_plan_run then launches the rest of jagg_einsum -- any
 * re-blocking of inputs into the workspace and the block kernel -- without
 * joining again, and computes exactly what jagg_einsum computes on the
 * relations' current contents.
 * The plan keeps the device addresses it was given: the caller keeps the
 * input and output buffers and the workspace alive and unmoved while the
 * plan lives, and must not use the workspace for anything else (it holds
 * the plan's join list); the relation handles themselves may be destroyed.
 * A plan is run on a context of the device it was made on (JAGG_E_INVALID
 * otherwise); runs may be recorded by jagg_capture_begin / _end.
 * jagg_plan_destroy frees the host metadata only. */
typedef struct jagg_plan jagg_plan;
jagg_status jagg_plan_create(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                             const int32_t *blockings, jagg_relation *out, void *workspace, size_t ws_bytes,
                             jagg_plan **plan);
jagg_status jagg_plan_run(jagg_ctx *ctx, const jagg_plan *plan);
jagg_status jagg_plan_destroy(jagg_plan *plan);

/* A group of independent plans run as one unit: jagg_plan_run on the group
 * computes exactly what running its members in order computes.  Members
 * that are contractions of one form -- the bf16 kernel with 256 x 256 tiles,
 * and the same geometry (extents, blockings, layouts, dtypes, alpha), only
 * their relations differ -- share one launch, up to 4 per launch (e.g. the
 * Q, K and V projections of a block, or the gate and up projections): the
 * grid of each is one range of a common grid, so the last partial wave of
 * tiles and the launch edges are shared.  Other members launch one after
 * the other.  Members must be independent: no member may write memory
 * (output or workspace) that another reads or writes (JAGG_E_INVALID).  The
 * group copies what it needs from `plans` (which may be destroyed after);
 * the addresses they were made with must stay valid as for each plan.
 * Groups may be members of groups (their members are taken). */
jagg_status jagg_plan_group(jagg_ctx *ctx, int n, const jagg_plan *const *plans, jagg_plan **group);

/* A dependent pair run as one pass ("Stax (5): Caching and Measurement",
 * Section 7: a reduction and the pointwise map that reads its result at the
 * same row index fuse vertically; Section 13.2, Proposition 13.3: the gain
 * is the ratio of bytes moved).  `first` must be the plan of a SUM of
 * JAGG_G_SQUARE over the innermost letter r of its one input x, to an f32
 * output ss ("X r -> X"); `second` the plan of a JAGG_G_RMS_SCALE map
 * ("X r, X, r -> X r") whose inputs are that x, that ss and a scale over r,
 * into an output laid out like x.  jagg_plan_run on the fused plan writes
 * both ss and the map's output, each as running `first` then `second`
 * writes it, except that the row sums of squares are added in another
 * order (last-bit differences in ss, and in the output through it).
 * Limits: uniform blockings, no re-blocked input, a block extent of r that
 * is a multiple of 256, rows of at most 4096 elements (r-blocks x block
 * extent), x, the scale and the output 16-byte aligned; anything else
 * returns JAGG_E_UNSUPPORTED and the caller runs the two plans one after the
 * other.  The map's output must not overlap x (JAGG_E_INVALID).  The fused
 * plan reads the first plan's join list: both plans' buffers and
 * workspaces must stay valid and unmoved while it lives, as for a group;
 * `first` and `second` may be destroyed. */
jagg_status jagg_plan_fuse(jagg_ctx *ctx, const jagg_plan *first, const jagg_plan *second, jagg_plan **fused);

/* jagg_einsum without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It runs the same kernels as jagg_einsum
 * on the same arguments, with the workspace taken from a static device array
 * of JAGG_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends (its address is fetched once per device,
 * in jagg_ctx_create).  It allocates nothing.
 * It never splits a contraction's walk (step (2) of jagg_einsum), so its
 * workspace is jagg_einsum_workspace less the room for split partial sums; a
 * call whose workspace exceeds the scratch is refused with JAGG_E_WORKSPACE
 * before any launch.  Nothing in the scratch
 * needs clearing between calls: the join kernel writes every list slot and
 * key count, and a re-blocking copy writes every byte it later reads.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (several streams or contexts in flight at once) race and must be
 * serialised by the caller; calls queued on one stream are ordered. */
#define JAGG_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
jagg_status jagg_einsum_noalloc(jagg_ctx *ctx, const jagg_spec *spec, const jagg_relation *const *in, int n_in,
                                const int32_t *blockings, jagg_relation *out);

/* Number of output keys and reduced-letter combinations per key of the join
 * of this spec under `blockings`; host only. */
jagg_status jagg_join_shape(const jagg_spec *spec, const int64_t *extents_by_letter,
                            const int32_t *blockings, int64_t *n_keys, int64_t *per_key);

/* Runs only the join-enumeration kernel (step 1) into caller device memory:
 * `dev_list` receives int32 [n_keys][per_key][1 + n_in] and `dev_counts`
 * int32 [n_keys].  For output key o the first dev_counts[o] slots hold its
 * joined tuples as [out_tuple, in_tuple_0, ...], ordered by the block
 * coordinates of the reduced letters (row-major, in order of first
 * appearance); the remaining slots of the key are filled with -1.  Without a
 * causal pair every count is per_key.  `extents_by_letter` gives every
 * letter's extent, in the order of `blockings`. */
jagg_status jagg_join_list(jagg_ctx *ctx, const jagg_spec *spec, const int64_t *extents_by_letter,
                           const int32_t *blockings, int32_t *dev_list, int32_t *dev_counts);

/* Graph capture of a call chain.  "Every Kernel Is a Join" (Ding et al.),
 * Sec. 5.1, makes the executable artifact a graph of GPU kernels run
 * directly; "Stax (5): Caching and Measurement", Section 11.3, notes that
 * the host cost of a call grows with the number of kernels launched and
 * that replaying a recorded graph removes the per-launch term.
 *
 * jagg_capture_begin starts recording the context's stream (relaxed mode:
 * other host threads may allocate meanwhile); every later jagg_einsum /
 * jagg_repartition on this context is recorded, not run, until
 * jagg_capture_end, which instantiates the recording into *out.  The
 * recorded launches keep the device pointers they were given (relations,
 * workspaces): the caller keeps those buffers alive and unmoved for the
 * graph's lifetime and may change their contents between launches.
 * jagg_graph_launch replays the graph on the context's stream
 * (asynchronously, like every call); jagg_graph_destroy frees it.  The
 * library records no memset or allocation, so replays are exact repeats of
 * the recorded launches.  Errors: JAGG_E_INVALID for a NULL handle or an
 * end without a begin, JAGG_E_DEVICE when HIP refuses the capture (e.g. the
 * stream is already being captured); a failed capture leaves *out unset. */
typedef struct jagg_graph jagg_graph;
jagg_status jagg_capture_begin(jagg_ctx *ctx);
jagg_status jagg_capture_end(jagg_ctx *ctx, jagg_graph **out);
jagg_status jagg_graph_launch(jagg_ctx *ctx, const jagg_graph *g);
jagg_status jagg_graph_destroy(jagg_graph *g);

const char *jagg_status_str(jagg_status s);
/* Detail of the last error on this context (empty string if none). */
const char *jagg_last_error(const jagg_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* JAGG_H */
