/*
 * taylor_states.h -- C ABI of libtaylor_states.so
 *
 * Causal attention under the truncated Taylor kernel
 *     K_n(x) = sum_{m=0}^{n-1} x^m / m!,   x = q.k,
 * on L2-normalised q and k, computed through n additive recurrent states
 * ("Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
 * with a Fixed Number of Recurrent States", abstract): each Taylor term is a
 * tensor-power inner product, so the history of a head collapses into the
 * state
 *     S[t, c] = sum_j mu_t(k_j) * v_j[c]   (c < dv),   S[t, dv] = sum_j mu_t(k_j),
 * over W = C(dk+n-1, n-1) feature rows t.  mu_t is a packed symmetric
 * monomial (product of the coordinates named by the non-decreasing index
 * tuple t); the readout uses phi_t(q) = mu_t(q) / alpha(t)!, so that
 * phi(q).mu(k) = K_n(q.k), and
 *     o = phi(q).S[:, :dv] / phi(q).S[:, dv]
 * (the extra column carries the normaliser; comment thread on the paper,
 * item 46888355, reply on the "+1").
 *
 * Feature rows: blocks m = 0 .. n-1 in ascending order; inside block m the
 * non-decreasing index tuples of length m in lexicographic order.
 *
 * State buffer of B*H heads (floats, contiguous): first the value plane
 * [B][H][W][dv], then the normaliser plane [B][H][W].  Rows in feature
 * order.  tt_state_floats() gives W*(dv+1) per head.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     allocated and owned by the caller.  The library allocates nothing and
 *     keeps no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  Kernel faults surface at the caller's next
 *     synchronisation, not in the return code.
 *   - Arguments are validated before anything is launched.  On error the
 *     return value is negative, nothing is launched, and tt_last_error()
 *     describes the problem (thread-local, valid until the next call on the
 *     same thread).
 *   - Inputs are used as given: q and k are NOT re-normalised (unit norm is
 *     the caller's precondition), except by the *_normed entry points.
 *   - Non-finite inputs propagate.  A NaN or Inf in token j reaches the
 *     outputs of tokens i >= j and the states, as the definition says; in
 *     addition, a non-finite value v_j can reach the outputs of the earlier
 *     queries of its own prefill chunk (the intra-chunk product multiplies
 *     their masked zero weights by v_j), in the value columns where v_j is
 *     not finite.  Outputs of earlier chunks are not affected.  A normaliser
 *     that is exactly zero (possible for n = 2, where K_2(-1) = 0) gives
 *     0/0 = NaN; with bf16 inputs, after the first chunk of a span, the
 *     rounding of the state readout can leave a tiny nonzero normaliser
 *     instead.
 *   - Outputs must not alias inputs unless stated.
 *   - Supported shapes: dv = 64; (dk, n) with dk in {8, 16, 32, 64}:
 *     dk=8: n in 1..6 (W up to 1287), dk=16: n in 1..5 (W up to 4845),
 *     dk=32 and dk=64: n in 1..5 (W up to 58905 and 814385; one head's
 *     state at dk=64, n=5 is 212 MB).  The dk = 8 prefill takes fp32
 *     inputs (bf16 returns TT_ERR_UNSUPPORTED); its decode takes both.
 *     Other shapes return TT_ERR_UNSUPPORTED.
 *   - dk = 32 and 64 with n = 4 or 5: the row codes of these shapes live in
 *     a table that the library builds on a device the first time such a
 *     shape runs there (a synchronous host-to-device copy of up to 3.3 MB,
 *     kept until the process ends); a first call inside HIP graph capture
 *     therefore fails, later ones do not copy.
 */
#ifndef TAYLOR_STATES_H
#define TAYLOR_STATES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input dtype codes.  C++ sees the same enumeration with int as its fixed
 * underlying type, so that any int a caller passes is a value of the type and
 * a code other than these two is rejected (TT_ERR_INVALID_ARG) rather than
 * undefined; the size and values are those of the C declaration. */
#ifdef __cplusplus
typedef enum tt_dtype_code : int { TT_F32 = 0, TT_BF16 = 1 } tt_dtype;
#else
typedef enum { TT_F32 = 0, TT_BF16 = 1 } tt_dtype;
#endif

enum {
  TT_OK = 0,
  TT_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad enum      */
  TT_ERR_UNSUPPORTED = -2, /* valid but outside the compiled shapes          */
  TT_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  TT_ERR_HIP = -4          /* a HIP call or kernel launch reported an error  */
};

/* Number of feature rows W = sum_{m<n} C(dk+m-1, m) = C(dk+n-1, n-1): the
 * widths of the n states ("Expanding Attention", abstract).  Pure host
 * function; 0 if dk < 1, n < 1 or on overflow. */
size_t tt_state_rows(int dk, int n);

/* Floats of one head's state, W * (dv + 1) (9945 for dk=16, dv=64, n=3,
 * "Expanding Attention", abstract).  0 on invalid input or overflow. */
size_t tt_state_floats(int dk, int dv, int n);

/* Bytes of device workspace tt_prefill needs for this shape with either
 * input dtype (written to *bytes).  Returns TT_OK or an error code as
 * tt_prefill would. */
int tt_prefill_workspace_bytes(int B, int H, int N, int dk, int dv, int n,
                               int chunk, size_t *bytes);

/* The same for one input dtype: the exact workspace tt_prefill,
 * tt_prefill_from and tt_prefill_from_unnormalized need with in_dtype (at
 * most what tt_prefill_workspace_bytes reports; the two dtypes can run
 * different kernels with different workspaces).  Returns TT_OK or an error
 * code as tt_prefill would. */
int tt_prefill_workspace_bytes_dtype(int B, int H, int N, int dk, int dv, int n,
                                     int chunk, tt_dtype in_dtype, size_t *bytes);

/* Chunked causal prefill ("Expanding Attention", abstract: the states add
 * across chunks, so prefill is a parallel scan; comment thread item
 * 46888355, reply on (Q'K)V = Q'(KV)).
 *   Q, K : [B][H][N][dk]   in_dtype (TT_F32 or TT_BF16), read-only
 *   V    : [B][H][N][dv]   in_dtype, read-only
 *   O    : [B][H][N][dv]   fp32, written: o_i = sum_{j<=i} K_n(q_i.k_j) v_j
 *                          / sum_{j<=i} K_n(q_i.k_j)  (causal, inclusive)
 *   states : B*H*W*(dv+1) fp32 in the plane layout above, written with the
 *            states of all N tokens (prefill starts from zero states)
 *   workspace : device scratch of at least tt_prefill_workspace_bytes();
 *            contents undefined on return.  Plans with spans of a fixed
 *            length (at chunk 64: fp32 with more than 256 state rows W,
 *            bf16 with n=3 at dk=32 and 64, bf16 with n>=4 at dk>=16)
 *            also take a smaller workspace of at least one head's share:
 *            tt_prefill_workspace_bytes_dtype() for B = H = 1, which is the
 *            size for B*H heads divided by B*H.  The heads (b, h in
 *            flattened order) then run in as few groups as the workspace
 *            allows, spread evenly over them, one group after another on
 *            `stream`, with bit-identical results.  No group reads another group's
 *            share, so the only cost is fewer workgroups per launch.  Less
 *            than one head's share, or less than the whole workspace for
 *            the other plans, is TT_ERR_WORKSPACE.
 *   chunk : tokens per chunk of the intra-chunk quadratic block: 16, 32,
 *           64 or 128.  Results do not depend on it beyond fp32 rounding
 *           (it moves work between the quadratic block and the state).
 *           bf16 inputs take 32, 64 or 128.  128 runs the shapes whose
 *           tiles fit the 160 KB of LDS of a CU: fp32 dk=8 n<=4, dk=16
 *           n<=3, dk=32 n=1; bf16 dk=16 n<=3, dk=32 n<=2, dk=64 n=1.
 *           dk=32 and dk=64 with n=4 or 5 take 64 only.  Other values
 *           and combinations return TT_ERR_UNSUPPORTED.  64 is the tuned
 *           default (bf16 with W <= 256 then runs the warp-specialised
 *           kernel).
 * Q, K, V, O and workspace must be 16-byte aligned (TT_ERR_INVALID_ARG).
 * Any N >= 1 is accepted (the tail chunk is masked).  Results do not
 * depend on how the work is split beyond fp32 rounding. */
int tt_prefill(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
               int B, int H, int N, int dk, int dv, int n, int chunk,
               float *O, float *states, void *workspace, size_t workspace_bytes,
               void *stream);

/* Bytes of the fixed device scratch array that tt_prefill_noalloc uses in
 * place of a workspace (64 MiB per GPU). */
#define TT_NOALLOC_SCRATCH_BYTES (64u << 20)

/* tt_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results as tt_prefill, with the
 * workspace taken from a fixed array of TT_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on each GPU it runs on until the process
 * ends.  The call allocates nothing: the caller passes Q, K, V, O and
 * states as for tt_prefill (same layouts, alignment and errors).  Plans
 * that run heads in groups (see tt_prefill's workspace) use groups that
 * fit the array; a shape whose workspace for one head (those plans) or for
 * the whole call (the others) exceeds TT_NOALLOC_SCRATCH_BYTES returns
 * TT_ERR_WORKSPACE before anything is launched.  The first call on
 * a device looks the array up on the current device, which `stream` must
 * belong to.  Every call on one GPU shares that GPU's array, and each call
 * overwrites what it needs of it (nothing has to start at zero): calls
 * that may overlap on one GPU (other streams, other threads) race and give
 * undefined results, so serialise them. */
int tt_prefill_noalloc(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
                       int B, int H, int N, int dk, int dv, int n, int chunk,
                       float *O, float *states, void *stream);

/* Prefill that continues from carried-in states: the same computation as
 * tt_prefill for tokens that follow earlier ones whose summed states are
 * states_in ("Expanding Attention", abstract: the states are sums over
 * tokens and add across segments, so earlier tokens enter only through
 * their state; comment thread item 46888355, reply on the "+1" column):
 *   o_i = (phi(q_i).S_in[:, :dv] + sum_{j<=i} K_n(q_i.k_j) v_j)
 *       / (phi(q_i).S_in[:, dv]  + sum_{j<=i} K_n(q_i.k_j))
 *   states = S_in + the states of the N new tokens.
 * Arguments as for tt_prefill, plus
 *   states_in : B*H*W*(dv+1) fp32, plane layout, read-only.  It may be the
 *               same buffer as `states` (the call then continues in place)
 *               but must not otherwise overlap `states`, O or the
 *               workspace (TT_ERR_INVALID_ARG); NULL is TT_ERR_INVALID_ARG.
 * Uses the same workspace as tt_prefill (head groups included). */
int tt_prefill_from(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
                    int B, int H, int N, int dk, int dv, int n, int chunk,
                    const float *states_in, float *O, float *states,
                    void *workspace, size_t workspace_bytes, void *stream);

/* tt_prefill_from without the final division: for each query the numerator
 * and the normaliser of the expression above are returned separately,
 *   num_i = phi(q_i).S_in[:, :dv] + sum_{j<=i} K_n(q_i.k_j) v_j
 *   den_i = phi(q_i).S_in[:, dv]  + sum_{j<=i} K_n(q_i.k_j)
 * so that results computed over separate segments can still be combined
 * (num and den add across key segments; o_i = num_i / den_i), the step
 * that context-parallel prefill needs ("Expanding Attention", abstract: the
 * states add across segments).  Arguments as for tt_prefill_from, with
 *   states_in : may be NULL (zero states, as tt_prefill);
 *   num       : [B][H][N][dv] fp32, device, 16-byte aligned (in place of O);
 *   den       : [B][H][N] fp32, device, 4-byte aligned; NULL is
 *               TT_ERR_INVALID_ARG; it must not overlap num, the states,
 *               states_in or the workspace (TT_ERR_INVALID_ARG).
 * The numerators and normalisers are those the normalised call divides
 * (its O is num * (1/den) with the hardware reciprocal); the states are the
 * same.  Uses the same workspace as tt_prefill (head groups included). */
int tt_prefill_from_unnormalized(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
                                 int B, int H, int N, int dk, int dv, int n, int chunk,
                                 const float *states_in, float *num, float *den, float *states,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* L2 normalisation of q and k with an optional temperature, the input-side
 * prerequisite of the method ("Expanding Attention", abstract: unit q and k
 * keep q.k inside the series' convergence radius, and without it more terms
 * stop helping).  Every row x of d values becomes
 *     r(scale * x / ||x||_2),
 * where r rounds once to the nearest value of the input dtype (ties to
 * even; bf16 from the fp64 value directly, not through a rounded fp32
 * value).  The quotient is evaluated in fp64
 * in a fixed order (s = sum of x_i*x_i, exact squares, summed in groups of 8
 * consecutive coordinates and a balanced pairwise tree over the groups;
 * f = scale / sqrt(s); x_i * f), within about 10 fp64 ulps of the exact
 * unit coordinate, so the result is the correctly rounded unit row except
 * for coordinates whose exact value lies that close to a rounding boundary.
 * The result is a fixed function of the input bits.  A zero row gives NaN.
 *   x, out : [rows][d] in_dtype, 16-byte aligned; out may be x (in place)
 *            but must not otherwise overlap it
 *   d      : 8, 16, 32 or 64 (TT_ERR_UNSUPPORTED otherwise)
 *   scale  : finite and > 0 (TT_ERR_INVALID_ARG otherwise)
 * rows == 0 is a no-op.  The *_normed entry points below apply exactly this
 * function (with scale = temperature for q and 1 for k) inside the library. */
int tt_normalize_rows(const void *x, tt_dtype in_dtype, size_t rows, int d, float scale, void *out,
                      void *stream);

/* Bytes of workspace tt_prefill_normed needs: the tt_prefill workspace
 * (rounded up to 256 bytes) plus room for normalised copies of Q and K. */
int tt_prefill_normed_workspace_bytes(int B, int H, int N, int dk, int dv, int n, int chunk,
                                      size_t *bytes);

/* Prefill on raw (not normalised) Q and K: the kernel is
 *     K_n(temperature * q.k / (||q|| ||k||)),
 * i.e. tt_prefill (states_in == NULL) or tt_prefill_from (states_in given)
 * on q_hat = r(temperature * q/||q||), k_hat = r(k/||k||) as produced by
 * tt_normalize_rows.  The normalised copies live in the workspace, which
 * must hold tt_prefill_normed_workspace_bytes(); the plans that run heads in
 * groups (see tt_prefill) also take as little as one head's share, the size
 * that query reports for B = H = 1, and then normalise each group's rows
 * into the workspace before its prefill (same results).  temperature must be
 * finite and > 0; the other arguments, layouts and errors are those of
 * tt_prefill_from.  Q and K are read-only. */
int tt_prefill_normed(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
                      int B, int H, int N, int dk, int dv, int n, int chunk, float temperature,
                      const float *states_in, float *O, float *states,
                      void *workspace, size_t workspace_bytes, void *stream);

/* One generated token per head ("Expanding Attention", abstract: one
 * rank-one update per state per token, independent of context length):
 *   S += mu(k) (x) [v, 1];  o = phi(q).S[:, :dv] / phi(q).S[:, dv]
 * (update first, then read out: the token attends to itself).
 *   q, k   : [B][H][dk] in_dtype;  v : [B][H][dv] in_dtype
 *   states : B*H*W*(dv+1) fp32, plane layout, updated in place
 *   o      : [B][H][dv] fp32, written */
int tt_decode_step(const void *q, const void *k, const void *v, tt_dtype in_dtype,
                   int B, int H, int dk, int dv, int n,
                   float *states, float *o, void *stream);

/* tt_decode_step on raw q and k: each workgroup normalises its q (scaled
 * by temperature) and k with the function of tt_normalize_rows before the
 * update and readout, so a decode continues a tt_prefill_normed exactly.
 * temperature must be finite and > 0. */
int tt_decode_step_normed(const void *q, const void *k, const void *v, tt_dtype in_dtype,
                          int B, int H, int dk, int dv, int n, float temperature,
                          float *states, float *o, void *stream);

/* dst[i] = a[i] + b[i] for i < nfloats: the states of two disjoint token
 * sets add ("Expanding Attention", abstract: additivity across chunks).
 * dst may alias a or b.  nfloats == 0 is a no-op. */
int tt_state_merge(float *dst, const float *a, const float *b, size_t nfloats,
                   void *stream);

/* Feature map of `rows` vectors x[rows][dk] (in_dtype) into out[rows][W]
 * fp32: mu_t(x) (weighted = 0) or phi_t(x) = mu_t(x)/alpha(t)! (weighted =
 * 1), rows in feature order ("Expanding Attention", abstract: tensor-power
 * factorisation of each Taylor term).  A test hook for the device function
 * the prefill and decode kernels use. */
int tt_feature_map(const void *x, tt_dtype in_dtype, size_t rows, int dk, int n,
                   int weighted, float *out, void *stream);

/* ---- Softmax baseline ------------------------------------------------
 * Exact causal softmax attention, the kernel exp(q.k) that the truncated
 * series approximates, for timing the method against it on the same GPU
 * ("Expanding Attention", abstract: prefill time and decode time per token
 * are compared with softmax attention).  No scale inside exp:
 *     o_i = sum_{j<=i} exp(q_i.k_j) v_j / sum_{j<=i} exp(q_i.k_j).
 * Supported: dk in {16, 32, 64}, dv = 64 (TT_ERR_UNSUPPORTED otherwise). */

/* Causal prefill.  Q, K [B][H][N][dk], V [B][H][N][dv]: bf16 only
 * (TT_ERR_UNSUPPORTED for TT_F32); O [B][H][N][dv] fp32, written.  All
 * pointers 16-byte aligned.  Scores and the running maximum in fp32;
 * probabilities enter the value product as bf16 (hi + lo bf16 on the
 * diagonal block of 64 keys). */
int tt_softmax_prefill(const void *Q, const void *K, const void *V, tt_dtype in_dtype,
                       int B, int H, int N, int dk, int dv, float *O, void *stream);

/* Bytes of workspace tt_softmax_decode_step needs at position pos:
 * B*H*(pos/2048 + 1) records of dv + 2 floats. */
int tt_softmax_decode_workspace_bytes(int B, int H, int pos, size_t *bytes);

/* One generated token per head against a KV cache.  The token at position
 * pos is appended (k into Kcache row pos, v into Vcache row pos) and
 *     o = sum_{j<=pos} exp(q.k_j) v_j / sum_{j<=pos} exp(q.k_j)
 * is read out over cache rows 0 .. pos-1 and the new token.
 *   q, k   : [B][H][dk] in_dtype;  v : [B][H][dv] in_dtype
 *   Kcache : [B][H][capacity][dk] in_dtype, rows 0 .. pos-1 read, row pos written
 *   Vcache : [B][H][capacity][dv] in_dtype, likewise; both 16-byte aligned
 *   pos    : 0 <= pos < capacity (TT_ERR_INVALID_ARG otherwise)
 *   o      : [B][H][dv] fp32, written
 *   workspace : tt_softmax_decode_workspace_bytes(B, H, pos) bytes or more
 * B*H must not exceed 65535.  Work grows linearly with pos. */
int tt_softmax_decode_step(const void *q, const void *k, const void *v, tt_dtype in_dtype,
                           int B, int H, int dk, int dv, void *Kcache, void *Vcache,
                           int pos, int capacity, float *o, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Message for the last failed call on this thread ("" if none). */
const char *tt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TAYLOR_STATES_H */
