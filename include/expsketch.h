/*
 * expsketch.h -- C ABI of the polynomial-method streaming sketch of the exp kernel
 * and of the exact streaming attention path, for AMD Instinct MI355X (gfx950).
 *
 * The method: "Rumo a Limites Estritos para Atenção em Streaming" (gist.science,
 * pt) and its French twin "Vers des Bornes Serrées pour l'Attention en Flux".
 *   - "Definição do Problema": a stream of key/value pairs (k_i, v_i) arrives in
 *     order; a query q asks for the kernel-density normaliser and the attention
 *     vector over everything seen so far.  Kernel: exp<q, k> (temperature is set
 *     by the radius of keys and queries, so no 1/sqrt(d) factor).
 *   - "Metodologia", pillar "O Método Polinomial": the head of the kernel is a
 *     truncated Taylor expansion; the stream is summarised by its low-degree
 *     moments.  Reading used here, for degree p:
 *         M_j = sum_i k_i^(x)j,   N_j = sum_i k_i^(x)j v_i^T        (j = 0..p)
 *         Zhat(q) = sum_j <q^(x)j, M_j> / j!
 *         ohat(q) = (sum_j <q^(x)j, N_j> / j!) / Zhat(q)
 *     which equals sum_i T_p(<q,k_i>) [1, v_i] / ... with T_p(x) = sum_{j<=p} x^j/j!.
 *   - "Metodologia", closing paragraph (Merge-and-Reduce): sketches of
 *     sub-streams are merged; moments are sums, so a merge is an addition.
 *
 * Conventions for every call below
 *   - All float arrays are fp32, row-major, contiguous, 16-byte aligned DEVICE
 *     pointers (hipMalloc / torch CUDA tensors), owned by the caller.
 *   - h independent heads are laid out head-major: K [h][n][d], V [h][n][dv],
 *     Q [h][m][d], out [h][m][dv], Z [h][m].
 *   - Supported shapes: d and dv are powers of two in [4, 128]; 0 <= p <= 16
 *     (p <= 7 in the multiset layout);
 *     h >= 1; the state (about h * D * (1+dv) floats, D = sum_{j<=p} d^j) must fit
 *     in device memory.  Anything else returns SK_EINVAL (shape) or SK_ENOMEM.
 *   - Calls are asynchronous on the HIP stream they are given (the handle's
 *     stream for sketch_* calls); nothing synchronises except sketch_destroy and
 *     sketch_state.  A kernel fault surfaces as SK_EHIP from a later call.
 *   - A handle is not thread-safe; use one thread (or external locking) per handle.
 *   - Results are deterministic: every reduction runs in a fixed order.
 */
#ifndef EXPSKETCH_H
#define EXPSKETCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued call. */
#define SK_OK         0
#define SK_EINVAL    -1  /* bad argument: shape, null or misaligned pointer, n < 0 */
#define SK_ENOMEM    -2  /* device memory for the state or a workspace not available */
#define SK_EMISMATCH -3  /* merge of sketches with different (d, dv, p, h) */
#define SK_EHIP      -4  /* a HIP runtime call or kernel launch failed */
#define SK_ESCRATCH  -5  /* request larger than an allocation-free call's fixed scratch */

typedef struct sk_sketch* sk_handle;  /* opaque; owned by the library */

/* Storage layouts of the moments (sketch_create_ex). */
#define SK_LAYOUT_FULL 0  /* every tensor index tuple: D = sum_{j<=p} d^j rows */
#define SK_LAYOUT_SYM  1  /* one row per multiset of indices: C(d + p, p) rows */

/*
 * sketch_create -- an empty sketch of degree p for h heads of key dimension d and
 * value dimension dv ("O Método Polinomial": the moment summary).
 *   hip_stream: hipStream_t the handle's calls are issued on (NULL = default).
 *   out: receives the handle.  The library allocates the state (zeroed) with
 *        hipMalloc; sketch_destroy frees it.
 * Errors: SK_EINVAL for unsupported shapes or out == NULL; SK_ENOMEM if the state
 * does not fit; SK_EHIP if a HIP call fails.  On error *out is set to NULL.
 */
int sketch_create(int d, int dv, int p, int h, void* hip_stream, sk_handle* out);

/*
 * sketch_create_ex -- sketch_create with a choice of storage layout.
 *   layout == SK_LAYOUT_FULL: as sketch_create.
 *   layout == SK_LAYOUT_SYM: the moment tensors are symmetric in their j indices
 *     (M_j[a_1..a_j] depends only on the multiset {a_1..a_j}), so one entry per
 *     multiset alpha is kept: M^s[alpha] = sum_i k_i^alpha, N^s[alpha] =
 *     sum_i k_i^alpha v_i, k^alpha = prod_l k[a_l].  Each entry stands for
 *     j!/alpha! index tuples (alpha! = product of the factorials of the
 *     multiplicities), so the answers are the same values as the full layout's:
 *         Zhat(q) = sum_alpha q^alpha M^s[alpha] / alpha!,  Ntilde likewise.
 *     C(d + p, p) rows instead of sum_j d^j ("O Método Polinomial": the pages
 *     keep the low-degree moments and leave their storage open).  Requires
 *     p <= 7.
 * Errors: as sketch_create; SK_EINVAL also for an unknown layout or p > 7 with
 * SK_LAYOUT_SYM.
 */
int sketch_create_ex(int d, int dv, int p, int h, int layout, void* hip_stream,
                     sk_handle* out);

/*
 * sketch_layout -- the handle's layout (SK_LAYOUT_FULL or SK_LAYOUT_SYM) and the
 * number of rows of its canonical view (sketch_state, sketch_export): D for the
 * full layout, C(d + p, p) for the multiset layout.  Either pointer may be NULL.
 * Errors: SK_EINVAL (NULL handle).
 */
int sketch_layout(sk_handle s, int* layout, int64_t* rows);

/* Update kernels (sketch_update_path). */
#define SK_UPDATE_TILES 0     /* full layout: feature tiles in LDS, any d */
#define SK_UPDATE_DIGITS 1    /* full layout, d = 16 or 32: operands scaled in registers */
#define SK_UPDATE_MULTISET 2  /* multiset layout */

/*
 * sketch_update_path -- which kernel the handle's update calls launch (one of
 * SK_UPDATE_*), fixed at creation.  All compute the same moments; this lets a
 * caller (a profiler, a benchmark) name the kernel it measures.
 * Errors: SK_EINVAL (NULL handle or NULL kind).
 */
int sketch_update_path(sk_handle s, int* kind);

/*
 * sketch_set_center -- recentre the expansion at a fixed centre c per head
 * ("Metodologia", pillar "Particionamento de Espaço e Recentramento": a dense
 * cluster is shifted to the origin, which shrinks the radius the expansion
 * covers).  Since exp<q,k> = e^{<q,c>} exp<q, k - c>, the sketch keeps the
 * moments of the shifted keys k - c and answers
 *     Z = e^{<q,c>} sum_j <q^(x)j, M_j(k - c)> / j!,    out unchanged by the factor.
 * Only on an empty sketch (count 0, e.g. right after create or reset; reset
 * keeps the centre).  c: device [h][d] (copied; the caller keeps ownership), or
 * NULL to remove the centre.  Synchronises the handle's stream.  Merging needs
 * equal centres (SK_EMISMATCH otherwise); sketch_state/sketch_export show the
 * moments of the shifted keys.
 * Errors: SK_EINVAL (NULL handle, misaligned c, sketch not empty), SK_ENOMEM,
 * SK_EHIP.
 */
int sketch_set_center(sk_handle s, const float* c);

/* sketch_destroy -- synchronises the handle's stream, frees everything the
 * handle owns.  NULL is accepted (no-op).  Returns SK_EHIP if a pending kernel
 * had failed (the memory is still freed). */
int sketch_destroy(sk_handle s);

/* sketch_set_stream -- issue later calls of this handle on another stream.  When
 * the stream changes, the library records an event on the old stream and makes
 * the new one wait for it, so work issued later on the handle runs after
 * everything issued before the change (the handle's own buffers are ordered by
 * its stream alone).  Setting the current stream again costs nothing.
 * Errors: SK_EINVAL (NULL handle), SK_EHIP. */
int sketch_set_stream(sk_handle s, void* hip_stream);

/* sketch_reset -- back to the empty sketch (all moments zero, count 0). */
int sketch_reset(sk_handle s);

/*
 * sketch_update -- ingest n more key/value pairs per head ("Definição do
 * Problema": the stream; "O Método Polinomial": M_j += sum k^(x)j,
 * N_j += sum k^(x)j v^T for j = 0..p).
 *   K: device [h][n][d]; V: device [h][n][dv]; n >= 0 keys per head (n == 0: no-op).
 * The inputs may be reused or freed once the stream has passed the call.
 * Small calls are staged: a call of at most half the staging size (by default
 * 32768 keys per head, at most 32 MB per handle; see sketch_set_staging) copies
 * its keys and values into a buffer the handle owns, and the buffer is
 * contracted in one launch when it fills or when anything reads or merges the
 * state.  The moments
 * are the same sums; only the grouping of keys into launches changes, and for a
 * given sequence of calls the results are deterministic.
 * A launch may split its keys over several workgroups per state entry; the
 * split partials go to two buffers the handle keeps (up to 1 GiB each: split
 * count x state bytes; the digit kernel of d = 16, 32, 64 keeps its count within
 * that while two splits fit) and are added into the state by the next launch or
 * the next reader; partials beyond that size take per-call buffers, reduced and
 * released within the call.
 * Errors: SK_EINVAL (NULL/misaligned pointer with n > 0, n < 0), SK_ENOMEM
 * (split workspace), SK_EHIP.
 */
int sketch_update(sk_handle s, const float* K, const float* V, int64_t n);

/*
 * sketch_set_staging -- staging size of sketch_update, in keys per head (rounded
 * down to a multiple of 32); 0 turns staging off.  Staged keys are contracted
 * first; synchronises the handle's stream.
 * Errors: SK_EINVAL (NULL handle, keys < 0), SK_EHIP.
 */
int sketch_set_staging(sk_handle s, int64_t keys);

/*
 * sketch_merge -- dst += src (Merge-and-Reduce, merge step: moments add, counts
 * add).  src is unchanged.  Both handles must have equal (d, dv, p, h), the
 * same layout and the same centre; the work runs on dst's stream, which first
 * waits for everything issued so far on src's stream when the two differ.
 * Errors: SK_EINVAL (NULL, dst == src), SK_EMISMATCH, SK_EHIP.
 */
int sketch_merge(sk_handle dst, sk_handle src);

/*
 * sketch_query -- answer m queries per head from the moments:
 *   Z[h][q]     = Zhat(q) = sum_j <q^(x)j, M_j> / j!      (KDE normaliser estimate)
 *   out[h][q][:] = ohat(q) = (sum_j <q^(x)j, N_j> / j!) / Zhat(q)
 * ("O Método Polinomial", query of the truncated expansion).  No clamping: an
 * empty sketch gives Z = 0 and out = NaN (0/0), as IEEE division does.
 *   Q: device [h][m][d]; out: device [h][m][dv]; Z: device [h][m]; m >= 0.
 * The per-tile partials live in a buffer the handle keeps (freed by
 * sketch_destroy), grown on demand up to 256 MB; larger ones are taken from the
 * stream-ordered allocator for the call.
 * Errors: SK_EINVAL, SK_ENOMEM (partials workspace), SK_EHIP.
 */
int sketch_query(sk_handle s, const float* Q, int64_t m, float* out, float* Z);

/*
 * sketch_step -- one streaming decode step per head: append the pair (k, v) to
 * the stream, then answer the query q over the stream including it
 * ("Definição do Problema": the stream answered query by query; "O Método
 * Polinomial": the same moments and answers as sketch_update with n = 1
 * followed by sketch_query with m = 1).  One pass over the state adds the
 * rank-one term of the new key to every stored entry and forms the query's
 * weighted sums of the updated entries; a second, small kernel adds them in a
 * fixed order and divides.  Nothing is allocated: the per-tile partials live in
 * a buffer the handle owns (sized at create), so calls on one handle must not
 * overlap.
 *   k: device [h][d]; v: device [h][dv]; q: device [h][d];
 *   out: device [h][dv] (ohat); Z: device [h] (Zhat).  count grows by 1.
 * Errors: SK_EINVAL (NULL handle or pointer), SK_EHIP.
 */
int sketch_step(sk_handle s, const float* k, const float* v, const float* q, float* out,
                float* Z);

/*
 * exact_attend -- the exact streaming path ("Definição do Problema": keep every
 * pair):  Z[h][q] = sum_i exp(<q, k_i>),  out[h][q] = sum_i exp(<q,k_i>) v_i / Z.
 * Computed with a running maximum (online softmax) over key slices and a
 * fixed-order combine of the slices.  n == 0 gives Z = 0, out = NaN.
 * Range: out is formed relative to the running maximum and stays finite for any
 * finite scores; Z is returned as a plain fp32 sum e^mu * l (mu the largest
 * score), so it overflows to +inf once ln Z exceeds about 88.7 (ln of the
 * largest fp32), e.g. a largest score of 80 with more than e^8.7 ~ 6000 keys at
 * that score.  The kernels take exponentials in base 2 (each query scaled by
 * log2 e in fp32), so a score's rounding error grows with its size: a few units
 * of 2^-24 times the largest |score|, relative, in Z.
 *   K [h][n][d], V [h][n][dv], Q [h][m][d], out [h][m][dv], Z [h][m]: device.
 *   hip_stream: hipStream_t to run on (NULL = default stream).
 * The per-slice partials (h * m * slices * (2 + dv) floats) live in a buffer
 * the library keeps per (device, stream), grown on demand up to 256 MB (growing
 * waits on the host for the stream's earlier work); larger ones are taken from
 * the stream-ordered allocator (hipMallocAsync) for the call.  At most 8 such
 * buffers are kept: a call on a ninth (device, stream) frees the one used least
 * recently, after waiting on the host for all work of the device.  Calls from
 * several host threads are serialised while they enqueue their kernels.
 * Errors: SK_EINVAL (shapes, NULL/misaligned pointers, n or m < 0), SK_ENOMEM,
 * SK_EHIP.
 */
int exact_attend(const float* K, const float* V, int64_t n, int d, int dv, int h,
                 const float* Q, int64_t m, float* out, float* Z, void* hip_stream);

/*
 * exact_attend_noalloc -- exact_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and kernels, with the per-slice
 * partials in a fixed scratch array of the library (16 MiB = 4,194,304 floats per
 * device, held until the process ends) instead of a kept or stream-ordered
 * allocation.  Nothing is allocated or freed.  The slice count is lowered until
 * h * m * slices * (2 + dv) floats fit; answers then differ from exact_attend's
 * only by summation order.  Every call on a device shares that device's array:
 * calls that overlap in time on one GPU (other streams, other threads) race and
 * must be ordered by the caller.  Every partial is written before it is read, so
 * nothing is cleared between calls.
 *   Arguments, layouts and results as exact_attend.
 * Errors: SK_EINVAL (as exact_attend), SK_ESCRATCH when even one slice per
 * query needs more than the scratch (h * m * (2 + dv) > 4,194,304), SK_EHIP.
 */
int exact_attend_noalloc(const float* K, const float* V, int64_t n, int d, int dv, int h,
                         const float* Q, int64_t m, float* out, float* Z, void* hip_stream);

/*
 * exact_timing -- kernel timing of the exact path with HIP events (for
 * measurement).  While enabled, each exact_attend call has its slice kernel (the
 * decode or batched kernel, not the combine) record a pair of library-owned
 * events at its own start and end (the launch takes them: hipExtLaunchKernel), up
 * to 256 pairs; enable != 0 starts (and clears) recording, 0 stops it.
 * exact_kernel_times -- waits for the last recorded pair, writes the elapsed
 * milliseconds of up to `cap` pairs into ms (host array), sets *count to the
 * number recorded, and clears them.
 * Errors: SK_EINVAL (cap < 0, ms NULL with cap > 0), SK_EHIP.
 */
int exact_timing(int enable);
int exact_kernel_times(float* ms, int cap, int* count);

/*
 * exact_release_workspaces -- frees every partials buffer exact_attend keeps
 * (waiting on the host for all work of each device first).  Later calls allocate
 * again.  For a caller that wants the memory back, e.g. before its streams are
 * destroyed.
 * Errors: SK_EHIP.
 */
int exact_release_workspaces(void);

/*
 * sketch_state -- a read-only view of the moments in the canonical layout
 * [M | N]: per head an array [D][1 + dv], rows stacked by level j = 0..p, level j
 * holding d^j rows in row-major Kronecker order (row a*d + b of level j is row a
 * of level j-1 times k[b]); column 0 is M_j, columns 1..dv are N_j; row 0 column
 * 0 is the count.  For a handle of layout SK_LAYOUT_SYM the view is the
 * multiset entries instead: rows_D = C(d + p, p) rows, the multisets of size
 * j = 0..p stacked by size, each size in lexicographic order of the sorted index
 * tuples (a_1 <= ... <= a_j); column 0 is M^s, columns 1..dv are N^s (raw
 * moments, without the 1/alpha! query weights).  The view is materialised on the
 * handle's stream into a library-owned device buffer [h][rows_D][1+dv], then the
 * stream is synchronised; it stays valid until the next call on the handle.  Any
 * output pointer may be NULL.
 * Errors: SK_EINVAL (NULL handle), SK_ENOMEM, SK_EHIP.
 */
int sketch_state(sk_handle s, const float** dev_state, int64_t* rows_D, int* cols,
                 int64_t* count);

/*
 * sketch_export -- the same canonical [M | N] view as sketch_state, written into
 * caller-owned device memory dst [h][rows][1 + dv] (rows from sketch_layout;
 * fp32, 16-byte aligned),
 * asynchronously on the handle's stream.
 * Errors: SK_EINVAL (NULL handle or dst, misaligned dst), SK_EHIP.
 */
int sketch_export(sk_handle s, float* dst);

/* sketch_info -- shape and count of a handle (host values; any pointer may be NULL). */
int sketch_info(sk_handle s, int* d, int* dv, int* p, int* h, int64_t* D,
                int64_t* count);

/*
 * sketch_timing -- kernel timing with HIP events on the handle's stream (for
 * measurement).  While enabled, each sketch_update records a pair of
 * library-owned events over its moment-update kernel(s) (kind 0), each
 * sketch_query over its contraction kernel(s) (kind 1) and each sketch_step over
 * its fused update-and-answer kernel (kind 2), up to 256 pairs per kind; the
 * launches take them (hipExtLaunchKernel: the first kernel's start, the last
 * kernel's end), so a pair spans the kernels and not the queue before them.
 * Later calls are not recorded until the pairs are collected.  enable != 0
 * starts (and clears) recording, 0 stops it.
 * sketch_kernel_times -- waits for the last recorded event of `kind`, writes the
 * elapsed milliseconds of up to `cap` recorded pairs into ms (host array), sets
 * *count to the number recorded, and clears them.
 * Errors: SK_EINVAL (NULL handle, kind not 0/1/2, cap < 0, ms NULL with cap > 0),
 * SK_EHIP.
 */
int sketch_timing(sk_handle s, int enable);
int sketch_kernel_times(sk_handle s, int kind, float* ms, int cap, int* count);

/*
 * Tail coreset -- the tail of the exp kernel's expansion answered from a weighted
 * subset of the stream ("Metodologia" > "1. Limites Superiores Algorítmicos",
 * pillar "Construções de Coreset Baseadas em Discrepância": small subsets built
 * with discrepancy theory approximate the kernel density for every query and
 * serve the tail of the expansion, while the moments serve its head; the closing
 * paragraph assembles the stream with Merge-and-Reduce).  The pages name results,
 * not a procedure; the readings implemented:
 *   - e^x = T_p(x) + R_p(x): the sketch answers sum_i T_p(<q,k_i>) [1, v_i]
 *     exactly; the coreset answers sum_i R_p(<q,k_i>) [1, v_i] by
 *     sum_s w_s R_p(<q,k_s>) [1, v_s] over its points.
 *   - Merge-and-Reduce as a binary counter of blocks of `block` points per head:
 *     points fill a buffer (weight 1); a full buffer enters level 0; two blocks of
 *     level l (older first, 2 * block points read as consecutive pairs) are halved
 *     into one block of level l + 1 (weight 2^(l+1)).
 *   - Halving: the self-balancing walk of Alweiss, Liu and Sawhney (STOC 2021)
 *     over the pairs in the feature space of <u(x), u(y)> = R_p(<k_x,k_y>)
 *     (1 + <v_x,v_y>): pair t has alpha_t = <psi, f_t> (psi the signed sum of the
 *     pairs before it, f_t the difference of its two points), P_t = (1 -
 *     alpha_t / c) / 2 clamped to [0, 1], c = c0 * max_t |f_t|^2; it keeps its
 *     second point when U_t < P_t, else its first.  U_t = (SplitMix64 output >>
 *     11) * 2^-53 (Steele, Lea and Flood, OOPSLA 2014) of counter
 *     (r * h + head) * block + t, r = the handle's reduce number, state `seed`.
 * The Gram matrix and the walk run in float64, so the kept points (copies of
 * input rows, bit for bit) match a float64 reference unless a uniform falls
 * within rounding of its threshold.
 */
typedef struct sk_coreset* sk_coreset_handle;  /* opaque; owned by the library */

/*
 * coreset_create -- an empty coreset of h heads (d, dv, p as sketch_create;
 * 64 <= block <= 2048, a multiple of 64; c0 > 0 the walk's threshold factor;
 * seed the generator's state).  The library allocates its block buffers on
 * demand (hipMalloc) and frees them in coreset_destroy.
 * Errors: SK_EINVAL (shapes, block, c0, out == NULL), SK_ENOMEM, SK_EHIP.
 */
int coreset_create(int d, int dv, int p, int h, int block, double c0, uint64_t seed,
                   void* hip_stream, sk_coreset_handle* out);

/* coreset_destroy -- synchronises the handle's stream and frees it (NULL: no-op). */
int coreset_destroy(sk_coreset_handle c);

/* coreset_set_stream -- later calls on another stream, which first waits for
 * everything issued on the old one.  Errors: SK_EINVAL, SK_EHIP. */
int coreset_set_stream(sk_coreset_handle c, void* hip_stream);

/* coreset_reset -- back to the empty coreset (count 0, reduce number 0). */
int coreset_reset(sk_coreset_handle c);

/*
 * coreset_update -- n more pairs per head: K [h][n][d], V [h][n][dv] (device,
 * caller-owned; they may be reused once the stream has passed the call).  Runs
 * the reduces the new points cause (Merge-and-Reduce): rounds of 64 whole
 * blocks of the input at once; blocks of smaller calls are copied and wait until
 * 64 blocks (or 64 MB) have gathered or a reader (coreset_query, coreset_export,
 * coreset_info, coreset_merge on either side) needs the coreset, so that several
 * calls' reduces share launches.  The blocks enter the binary counter in stream
 * order either way: the kept points do not depend on when they are reduced.
 * Errors: SK_EINVAL (NULL/misaligned pointer with n > 0, n < 0), SK_ENOMEM, SK_EHIP.
 */
int coreset_update(sk_coreset_handle c, const float* K, const float* V, int64_t n);

/*
 * coreset_merge -- dst takes src's points (Merge-and-Reduce across sub-streams):
 * src's buffered points enter dst's buffer in order (a full buffer enters level
 * 0), then src's blocks enter dst at their own levels, lowest first, with the
 * reduces this causes (numbered by dst).  src is unchanged.  Equal (d, dv, p, h,
 * block) required.  Runs on dst's stream, ordered after src's and before src's
 * later work.
 * Errors: SK_EINVAL, SK_EMISMATCH, SK_ENOMEM, SK_EHIP.
 */
int coreset_merge(sk_coreset_handle dst, sk_coreset_handle src);

/*
 * coreset_query -- adds the tail to a head answer, in place: on entry out [h][m][dv]
 * and Z [h][m] hold (ohat, Zhat) of the moments (sketch_query) or zeros; on
 * return Z = Zhat + tZ and out = (ohat * Zhat + tN) / Z, with tZ = sum_s w_s
 * R_p(<q,k_s>) and tN = sum_s w_s R_p(<q,k_s>) v_s over the coreset's points (fp32;
 * R_p by its series for |<q,k>| <= 16, else e^x - T_p(x)).  Q [h][m][d] device.
 * With no points the head answer is left as it is.  Partials live in a buffer the
 * handle keeps.
 * Errors: SK_EINVAL, SK_ENOMEM, SK_EHIP.
 */
int coreset_query(sk_coreset_handle c, const float* Q, int64_t m, float* out, float* Z);

/* coreset_info -- points per head, points ingested per head, reduces done (any
 * pointer may be NULL); first runs the reduces of waiting blocks.
 * Errors: SK_EINVAL, SK_ENOMEM, SK_EHIP. */
int coreset_info(sk_coreset_handle c, int64_t* points, int64_t* count, int64_t* reduces);

/*
 * coreset_export -- the points into caller-owned device memory: K [h][points][d],
 * V [h][points][dv], w [h][points] (points from coreset_info): the buffer first
 * (weight 1), then the blocks by increasing level (weight 2^l), each in its row
 * order.  Asynchronous on the handle's stream.
 * Errors: SK_EINVAL, SK_EHIP.
 */
int coreset_export(sk_coreset_handle c, float* K, float* V, float* w);

/* sk_strerror -- a static string for a status code. */
const char* sk_strerror(int code);

/* sk_version -- ABI version of this library (major * 100 + minor). */
int sk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXPSKETCH_H */
