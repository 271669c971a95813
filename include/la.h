/*
 * la.h - C ABI of liblinattn: chunkwise-parallel causal linear attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For each of BH independent (batch, head) slices, with
 * feature map phi applied to queries and keys (never to values):
 *
 *   causal:      o_i = phi(q_i)^T S_i [/ phi(q_i)^T z_i],
 *                S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j)
 *   non-causal:  the same with every sum over all j
 *
 * The causal mask includes the diagonal (token i sees itself).  The causal
 * result is produced chunkwise with chunk size C: inside a chunk the output is
 * the lower-triangular (diagonal kept) product tril(Q_c K_c^T) V_c, across
 * chunks it is Q_c P_c with P_c the state carried from the chunks before, and
 * the state then grows by K_c^T V_c.  Every C gives the same value in exact
 * arithmetic; C <= 0 is treated as 1, C >= L is a single chunk, and the last
 * chunk may be shorter than C.
 *
 * Sources.  Page "attention と線形の間" (sharin-2a1.pages.dev/parts/
 * chunked.html): section ① (the association orders and the d x d state),
 * section ② (the chunked algorithm, its causal mask and its two ends).  Page
 * "Linear Attention / Performerの理論と実装" (disassemble-channel.com/
 * linear-attention/): the kernel re-formulation with the normaliser, the RNN
 * view (S_t, z_t recurrences), the elu+1 and FAVOR+ feature maps.
 *
 * Layout.  Every tensor is dense and row-major.  q, k: [BH, L, d_in];
 * v: [BH, L, d_v]; o: [BH, L, d_v]; states: [BH, (N,) d_k, d_v] with d_k the
 * feature width (d_k = d_in, or m for FAVOR+); normalisers z: [BH, (N,) d_k].
 * A [B, H, L, d] tensor is passed as BH = B * H slices.
 *
 * Precision.  LA_BF16 inputs: phi computed in fp32 and rounded to bf16,
 * products on bf16 matrix cores with fp32 accumulation, states fp32, output
 * bf16 (round to nearest even) or fp32.  LA_I8 inputs (identity map, no
 * normaliser): int8 x int8 products accumulated exactly in int32; states and
 * output int32; results are exact whenever they fit in int32 (two's-complement
 * wrap otherwise).
 *
 * Ownership and synchronisation.  The caller owns every buffer; all pointers
 * except those documented as host pointers are device pointers.  No entry
 * point allocates device memory: scratch comes from the caller's workspace.
 * Every call only enqueues work on the given stream (0 = the null stream) and
 * returns without waiting for it; there is no host synchronisation inside.
 *
 * Errors.  Invalid arguments are detected before anything is enqueued and
 * reported as LA_ERR_INVALID_ARG or LA_ERR_UNSUPPORTED; a launch failure
 * reported by the HIP runtime gives LA_ERR_HIP.  la_last_error() returns a
 * thread-local description of the most recent failure on the calling thread.
 * Nothing is thrown across the ABI.
 *
 * Supported sizes.  d_k in {16, 32, 64, 128, 256}, d_v in {16, 32, 64, 128,
 * 256}; FAVOR+: d_in in {16, 32, 64, 128} and m = d_k.  L >= 1, BH >= 1.
 */
#ifndef LIBLINATTN_LA_H
#define LIBLINATTN_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* la_stream_t; /* a hipStream_t */

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* a null required pointer, a non-positive size, mismatched sizes */
    LA_ERR_UNSUPPORTED = 2, /* a valid request this library does not implement */
    LA_ERR_HIP = 3,         /* the HIP runtime reported an error */
    LA_ERR_WORKSPACE = 4    /* the workspace is missing or smaller than required */
} la_status;

typedef enum { LA_BF16 = 0, LA_F32 = 1, LA_I8 = 2, LA_I32 = 3 } la_dtype;

typedef enum {
    LA_FMAP_IDENTITY = 0, /* phi(x) = x                                      */
    LA_FMAP_ELU1 = 1,     /* phi(x) = x + 1 for x >= 0, exp(x) for x < 0      */
    LA_FMAP_FAVOR = 2     /* phi(x)_l = exp(w_l . x - |x|^2 / 2) / sqrt(m)    */
} la_fmap;

/*
 * la_feature_map - y = phi(in_scale * x), row by row.
 *
 * Defined by the linear-attention page: its ELU feature map (elu with
 * alpha = 1, plus one) and its FAVOR+ positive random features (projection by
 * the m rows of W, minus half the squared norm, exponentiated, over sqrt(m)).
 *
 *   x    [rows, d_in] LA_BF16.
 *   W    [m, d_in] LA_BF16, FAVOR+ only (NULL otherwise); m is ignored unless
 *        f == LA_FMAP_FAVOR.
 *   y    [rows, d_k] of type ydt (LA_BF16 or LA_F32), d_k = m for FAVOR+,
 *        d_in otherwise.  y must not overlap x.
 */
la_status la_feature_map(la_fmap f, const void* x, la_dtype xdt, int64_t rows, int64_t d_in,
                         const void* W, int64_t m, float in_scale, void* y, la_dtype ydt,
                         la_stream_t stream);

/*
 * la_chunk_states - phase 1: local state of every chunk,
 *   S_n = K_c^T V_c (d_k x d_v) and, when z != NULL, z_n = sum of the rows of K_c,
 * for chunks [n*C, min((n+1)*C, L)), n = 0 .. N-1, N = ceil(L / C).
 *
 * Defined by the chunking page, section ②: the state each chunk adds before
 * the next one reads it.  k is taken as already feature-mapped.
 *
 *   k    [BH, L, d_k], v [BH, L, d_v], both of type in_dt (LA_BF16 or LA_I8).
 *   S    [BH, N, d_k, d_v]: LA_F32 for bf16 inputs, LA_I32 for int8 inputs.
 *   z    [BH, N, d_k], same type as S, or NULL.
 */
la_status la_chunk_states(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                          int64_t d_k, int64_t d_v, int64_t C, void* S, void* z,
                          la_stream_t stream);

/*
 * la_state_scan - phase 2: exclusive prefix over chunks, in place:
 *   P_0 = 0, P_n = P_{n-1} + S_{n-1}   (same for z when z != NULL)
 * and, when S_final / z_final are not NULL, the total sum_n S_n (the state
 * after the whole sequence) / sum_n z_n.
 *
 * Defined by the chunking page, section ②: chunk n reads the state carried
 * from every chunk before it; the state starts at zero.
 *
 *   S    [BH, N, d_k, d_v] of type st_dt (LA_F32 or LA_I32), overwritten by P.
 *   z    [BH, N, d_k] of the same type, or NULL.
 *   S_final [BH, d_k, d_v], z_final [BH, d_k]: optional outputs.
 * Sums run in chunk order, so the result is deterministic; int32 sums wrap.
 */
la_status la_state_scan(void* S, void* z, la_dtype st_dt, int64_t BH, int64_t N, int64_t d_k,
                        int64_t d_v, void* S_final, void* z_final, la_stream_t stream);

/*
 * la_chunk_output - phase 3 alone: the causal output of every chunk from the
 * prefix states of its group.  For each group of `group` consecutive chunks of
 * C rows, starting from P = P_prefix of that group (zero for the first group)
 * and, with normalize, z = z_prefix:
 *   O_c = Q_c P + tril(Q_c K_c^T) V_c   [ / (Q_c z + row sums of tril(Q_c K_c^T)) ]
 *   P  += K_c^T V_c ;  z += column sums of K_c        (then the next chunk)
 * The carried state of the chunked algorithm on the chunking page, section ②
 * (intra-chunk scores masked with the diagonal kept, inter-chunk read from the
 * carried state), with the linear-attention page's normaliser.
 *
 *   q, k [BH, L, d_k] (already feature-mapped), v [BH, L, d_v]: LA_BF16, or
 *        LA_I8 without normalize.
 *   group   chunks per group (>= 1); n_groups = ceil(ceil(L / C) / group).
 *   P_prefix [BH, n_groups, d_k, d_v] (LA_F32; LA_I32 for int8) and z_prefix
 *        [BH, n_groups, d_k] (LA_F32): the exclusive prefix at group
 *        granularity, i.e. la_chunk_states with chunk size C * group followed
 *        by la_state_scan.  May be NULL when n_groups == 1 (zero start).
 *   o, S_final, z_final: as for la_chunked_forward.
 */
la_status la_chunk_output(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                          int64_t L, int64_t d_k, int64_t d_v, int64_t C, int64_t group,
                          const void* P_prefix, const void* z_prefix, int normalize, void* o,
                          la_dtype out_dt, void* S_final, void* z_final, la_stream_t stream);

/*
 * la_chunked_forward - the whole forward: phi, then (causal) the chunked
 * computation with chunk size C, or (non-causal) phi(Q) (phi(K)^T V).
 * normalize != 0 divides each output row by phi(q_i)^T z_i (the numerator and
 * the denominator each sum their intra- and inter-chunk parts first; no
 * epsilon).
 *
 * Defined by the chunking page, section ② (Chunked and its two causal ends)
 * and the linear-attention page (normalised output, RNN view).
 *
 *   q, k [BH, L, d_in], v [BH, L, d_v] of type in_dt (LA_BF16, or LA_I8 with
 *        f == LA_FMAP_IDENTITY and normalize == 0).
 *   W    [m, d_in] LA_BF16 for FAVOR+ (d_k = m), else NULL.
 *   in_scale  multiplies q and k before phi (1.0f: none).
 *   o    [BH, L, d_v] of type out_dt (LA_BF16 or LA_F32 for bf16 inputs,
 *        LA_I32 for int8 inputs).
 *   S_final [BH, d_k, d_v] (LA_F32, or LA_I32 for int8) and z_final [BH, d_k]
 *        (LA_F32; only with normalize): optional final state.
 *   group  consecutive chunks one workgroup carries the state through (0 =
 *        chosen by the library).  The call runs la_chunk_states at group
 *        granularity (few long groups: in up to eight pieces per group),
 *        la_state_scan over those states and la_chunk_output; group = 1 is
 *        the literal three-phase form (one state per chunk), group >= N a
 *        single sequential walk per head.  Every value gives the same result
 *        in exact arithmetic.  With a feature map, a requested final state
 *        and normaliser are the scan's total over phase-1 states that keep
 *        phi(k) to about 2^-17 (bf16 value plus bf16 residual).
 *   workspace / ws_bytes  device scratch of at least
 *        la_chunked_forward_workspace(...) bytes (may be NULL when that is 0).
 */
la_status la_chunked_forward(const void* q, const void* k, const void* v, la_dtype in_dt,
                             int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                             int causal, int normalize, la_fmap f, const void* W, int64_t m,
                             float in_scale, void* o, la_dtype out_dt, void* S_final,
                             void* z_final, int64_t group, void* workspace, size_t ws_bytes,
                             la_stream_t stream);

/*
 * la_chunked_forward_noalloc - la_chunked_forward for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as la_chunked_forward, without workspace / ws_bytes: the
 * scratch it needs (at most la_chunked_forward_workspace bytes for the same
 * arguments; FAVOR+ with a bf16 output, mapped inside the kernels, needs only
 * the phase-1 states) comes from a static device array of
 * LA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per device, held until the process ends; its address is looked
 * up on the first call on each device (with that device current).  It calls no
 * allocator.  A call needing more scratch returns LA_ERR_UNSUPPORTED and
 * launches nothing.  Every call on a device shares that device's array, which
 * keeps the last call's contents (nothing in it needs to start at zero): calls
 * that overlap on one device (concurrent streams or threads) race on it.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
la_status la_chunked_forward_noalloc(const void* q, const void* k, const void* v, la_dtype in_dt,
                                     int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                                     int causal, int normalize, la_fmap f, const void* W, int64_t m,
                                     float in_scale, void* o, la_dtype out_dt, void* S_final,
                                     void* z_final, int64_t group, la_stream_t stream);

/* Bytes of workspace la_chunked_forward needs for these arguments (0 when it
 * needs none, and also on an invalid combination, which la_chunked_forward
 * then reports).  FAVOR+ stores phi(q), phi(k) and phi(k)'s bf16 residual
 * there; the phase-1 states (and normalisers) go there when there is more than
 * one group, or when a mapped forward may return its final state. */
size_t la_chunked_forward_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_in,
                                    int64_t d_v, int64_t C, int causal, int normalize,
                                    la_fmap f, int64_t m, float in_scale, int64_t group);

/* Chunks per group that la_chunked_forward uses for these arguments (its
 * group argument when positive, else the library's choice, capped at the
 * number of chunks); 0 on an invalid combination. */
int64_t la_chunked_forward_group(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_in, int64_t d_v,
                                 int64_t C, int causal, int normalize, la_fmap f, int64_t m,
                                 int64_t group);

/*
 * la_recurrent_step - one decode step for n_states independent states:
 *   S += phi(k) v^T;  z += phi(k);  o = phi(q)^T S [/ phi(q)^T z]
 * (update first, then read, as in the RNN view of the linear-attention page
 * and the token-by-token causal form of the chunking page).
 *
 *   q, k [n_states, d_in], v [n_states, d_v]: LA_BF16.
 *   W    [m, d_in] LA_BF16 for FAVOR+ (d_k = m), else NULL.
 *   S    [n_states, d_k, d_v] fp32, z [n_states, d_k] fp32: read and updated
 *        in place (z may be NULL when normalize == 0).
 *   o    [n_states, d_v] of type out_dt (LA_F32 or LA_BF16).
 */
la_status la_recurrent_step(const void* q, const void* k, const void* v, la_dtype in_dt,
                            int64_t n_states, int64_t d_in, int64_t d_v, la_fmap f,
                            const void* W, int64_t m, float in_scale, int normalize, float* S,
                            float* z, void* o, la_dtype out_dt, la_stream_t stream);

/*
 * The decode step on the exact int8 path (the int8 forward's arithmetic, one
 * token; the RNN view of the linear-attention page and the token-by-token form
 * of the chunking page, section ②): S += k^T v, then o = q S.  Identity map,
 * no normaliser.  Every product and sum is taken in wrapping 32-bit
 * arithmetic: exact modulo 2^32, hence exact whenever the true values fit
 * int32; steps after an int8 forward's final state continue it exactly.
 *
 *   q, k [n_states, d_k], v [n_states, d_v]: int8; d_k, d_v powers of two in 16..256.
 *   S    [n_states, d_k, d_v] int32, 16-byte aligned, read and updated in place.
 *   o    [n_states, d_v] int32.
 * Errors: LA_ERR_INVALID_ARG (NULL pointer, non-positive size, S not 16-byte aligned),
 * LA_ERR_UNSUPPORTED (other widths); nothing is launched on an error.
 */
la_status la_recurrent_step_i8(const void* q, const void* k, const void* v, int64_t n_states, int64_t d_k,
                               int64_t d_v, int32_t* S, int32_t* o, la_stream_t stream);

/*
 * The decayed recurrence (Retention): S_t = gamma S_{t-1} + phi(k_t) v_t^T and,
 * as read here, z_t = gamma z_{t-1} + phi(k_t), with 0 < gamma <= 1 shared by
 * every head; the output still reads y_t = phi(q_t)^T S_t [/ phi(q_t)^T z_t]
 * after the update.  Defined by the linear-attention page, RNN view, where
 * forgetting is introduced; gamma = 1 is plain linear attention.
 *
 * Each function below is its namesake with a gamma argument; a gamma outside
 * (0, 1] (or NaN) is LA_ERR_INVALID_ARG.  Chunk n's state is the state its rows
 * leave at the chunk's end: S_n = sum over its rows r (ending at row e) of
 * gamma^(e-1-r) phi(k_r)^T v_r.  The forward and the chunk output run on the
 * streaming kernel only: causal, LA_BF16 in and out, C in {32, 64, 128} with
 * d_k in {64, 128} and d_v a multiple of 64, or C in {32, 64} with d_k = 256;
 * any other combination is LA_ERR_UNSUPPORTED.  At C = 32 the streaming kernel
 * walks chunks in pairs: the forward rounds an odd group up to the next even
 * one, and la_chunk_output_decay needs an even group (or one that covers every
 * chunk).  The forward needs the workspace la_chunked_forward_workspace gives
 * for the same arguments.
 */
la_status la_chunked_forward_decay(const void* q, const void* k, const void* v, la_dtype in_dt,
                                   int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                                   int normalize, la_fmap f, const void* W, int64_t m,
                                   float in_scale, float gamma, void* o, la_dtype out_dt,
                                   void* S_final, void* z_final, int64_t group, void* workspace,
                                   size_t ws_bytes, la_stream_t stream);

/* Per-chunk states at each chunk's end (LA_BF16 inputs, LA_F32 states). */
la_status la_chunk_states_decay(const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                int64_t L, int64_t d_k, int64_t d_v, int64_t C, float gamma,
                                void* S, void* z, la_stream_t stream);

/* The decayed exclusive prefix, in place: P_0 = 0, P_n = gamma^len(n-1) P_{n-1}
 * + S_{n-1}, with len(n) the row count of chunk n of L rows in chunks of C
 * (N must be ceil(L / C)); the total is the final state.  LA_F32 states. */
la_status la_state_scan_decay(void* S, void* z, la_dtype st_dt, int64_t BH, int64_t N,
                              int64_t d_k, int64_t d_v, int64_t L, int64_t C, float gamma,
                              void* S_final, void* z_final, la_stream_t stream);

/* Phase 3 from decayed group prefixes (la_chunk_states_decay with chunk size
 * C * group, then la_state_scan_decay with the same L and chunk size). */
la_status la_chunk_output_decay(const void* q, const void* k, const void* v, la_dtype in_dt,
                                int64_t BH, int64_t L, int64_t d_k, int64_t d_v, int64_t C,
                                int64_t group, const void* P_prefix, const void* z_prefix,
                                int normalize, float gamma, void* o, la_dtype out_dt,
                                void* S_final, void* z_final, la_stream_t stream);

/* One decode step: S = gamma S + phi(k) v^T, z = gamma z + phi(k), then the read. */
la_status la_recurrent_step_decay(const void* q, const void* k, const void* v, la_dtype in_dt,
                                  int64_t n_states, int64_t d_in, int64_t d_v, la_fmap f,
                                  const void* W, int64_t m, float in_scale, int normalize,
                                  float gamma, float* S, float* z, void* o, la_dtype out_dt,
                                  la_stream_t stream);

/*
 * Log-linear attention (slide deck "Log-Linear Attention": the Fenwick-tree
 * partition of the past, the hierarchical mask and its chunkwise
 * computation).  Query t sees key s <= t at level 0 when s == t, else
 * floor(log2(t XOR s)) + 1 (level l >= 1 holds the 2^(l-1) keys just below t
 * with its bits under l-1 cleared); with per-token level weights lam:
 *     o_t = sum_{s <= t} lam[t, level(t, s)] (q_t . k_s) v_s
 * (lam = 1 everywhere is causal linear attention; no normaliser, no map).
 *
 *   q, k [BH, L, d_k], v [BH, L, d_v]: LA_BF16; d_k in {64, 128}, d_v in
 *        {64, 128, 256}; C must be 64 (chunks of 64 rows).
 *   lam  [BH, L, n_levels] float32 (device), n_levels = la_loglinear_levels(L).
 *   o    [BH, L, d_v] LA_BF16.
 *   S_levels  NULL, or [BH, n_state_levels, d_k, d_v] float32 (device): written
 *        with the level states after the last token, those that
 *        la_loglinear_prefix_levels gives for the same k, v (summed from this
 *        call's own chunk states and bucket sums), for decode steps that go on
 *        from position L.  n_state_levels (read only with S_levels) lies in
 *        [n_levels, 40]; levels above n_levels are written as zero.
 *   workspace  la_loglinear_forward_workspace(...) bytes (per-chunk states and
 *        their bucket sums; 0 for a single chunk).
 * Errors: LA_ERR_INVALID_ARG (NULL pointer, non-positive size, wrong
 * n_levels or n_state_levels), LA_ERR_UNSUPPORTED (other types, widths or
 * chunk sizes), LA_ERR_WORKSPACE; nothing is launched on an error.
 */
la_status la_loglinear_forward(const void* q, const void* k, const void* v, la_dtype in_dt,
                               int64_t BH, int64_t L, int64_t d_k, int64_t d_v, int64_t C,
                               const float* lam, int64_t n_levels, void* o, la_dtype out_dt,
                               float* S_levels, int64_t n_state_levels, void* workspace,
                               size_t ws_bytes, la_stream_t stream);
size_t la_loglinear_forward_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k,
                                      int64_t d_v, int64_t C);
/* Levels a sequence of L tokens uses: 1 + the bit length of L - 1 (0 for L < 1). */
int64_t la_loglinear_levels(int64_t L);

/*
 * One decode step of log-linear attention (slide deck "Log-Linear Attention",
 * the Fenwick tree recurrence and its per-level update): each stream keeps
 * level states S[l], the sum of k_s^T v_s over level l's bucket of the past.
 * The token at position t (t >= 0, the same for every stream) advances them:
 * with b the position of t's lowest set bit (t > 0), the buckets of levels
 * 0..b merge into level b + 1 and levels 1..b empty; level 0 takes k_t^T v_t;
 * the other levels stay.  Then o = sum_l lam[l] q_t S[l] (update, then read).
 * Steps t = 0, 1, 2, ... from zero states give, token by token,
 * la_loglinear_forward's outputs for the same inputs and weights.
 *
 *   q, k [n_states, d_k], v [n_states, d_v]: LA_BF16; d_k and d_v powers of
 *        two in 16..256.
 *   lam  [n_states, n_levels] float32 (device): this token's level weights
 *        (row t of the forward's lam).
 *   n_levels  levels each stream keeps: at least la_loglinear_levels(t + 1)
 *        (1 + the bit length of t), at most 40; la_loglinear_levels(T) covers
 *        every position below T.
 *   S    [n_states, n_levels, d_k, d_v] float32 (device), read and updated in
 *        place; all zero before position 0.  After the step, level l >= 1
 *        holds keys (and is otherwise zero) exactly when bit l - 1 of t is set.
 *   o    [n_states, d_v] of type out_dt (LA_F32 or LA_BF16).
 * Errors: LA_ERR_INVALID_ARG (NULL pointer, non-positive n_states, t < 0,
 * n_levels outside [la_loglinear_levels(t + 1), 40]), LA_ERR_UNSUPPORTED
 * (other types or widths); nothing is launched on an error.
 */
la_status la_recurrent_step_loglinear(const void* q, const void* k, const void* v, la_dtype in_dt,
                                      int64_t n_states, int64_t d_k, int64_t d_v, const float* lam,
                                      int64_t n_levels, int64_t t, float* S, void* o, la_dtype out_dt,
                                      la_stream_t stream);

/*
 * The level states of log-linear attention after a prefix (for a decode that
 * follows la_loglinear_forward): for each head, the states S[l] that decode
 * steps at positions 0 .. L - 1 from zero states would leave, computed
 * directly from k and v: level 0 = k_T^T v_T (T = L - 1); level l >= 1 = the
 * sum of k_s^T v_s over its Fenwick bucket [h - 2^(l-1), h), h = T with its
 * bits below l - 1 cleared, when bit l - 1 of T is set, else zero (slide deck
 * "Log-Linear Attention": the partition of the past and the per-level state).
 *
 *   k [BH, L, d_k], v [BH, L, d_v]: LA_BF16; d_k and d_v powers of two in 16..256.
 *   n_levels  levels per head in S: at least la_loglinear_levels(L), at most 40
 *        (la_loglinear_levels(T1) lets decode steps continue up to position T1 - 1).
 *   S    [BH, n_levels, d_k, d_v] float32 (device): written (every level).
 *   workspace  la_loglinear_prefix_levels_workspace(...) bytes: the states of the
 *        whole 64-row chunks before the last row's chunk (0 when L <= 64).
 * Errors: LA_ERR_INVALID_ARG (NULL pointer, non-positive size, n_levels out of
 * range), LA_ERR_UNSUPPORTED (other types or widths), LA_ERR_WORKSPACE; nothing
 * is launched on an error.
 */
la_status la_loglinear_prefix_levels(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                                     int64_t d_k, int64_t d_v, int64_t n_levels, float* S, void* workspace,
                                     size_t ws_bytes, la_stream_t stream);
size_t la_loglinear_prefix_levels_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v);

/*
 * The delta rule and its gated form (page "Kimi K3 と Qwen 3.8 の Attention 機構
 * 比較分析" (news.ainew.jp): section 3.1, equation (14): before writing, look up
 * what the current key maps to in the state, erase that old prediction along
 * the key, write the new value; section 2.4: the gated form adds a global
 * decay of the whole state).  With the state S (d_k x d_v, read as o = q S),
 * a write strength beta_t and a gate alpha_t per token:
 *     u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)
 *     S_t = alpha_t S_{t-1} + k_t u_t^T  = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = q_t^T S_t                     (read after the update)
 * alpha = 1 (alpha == NULL) is the delta rule without the gate; beta = 1 the
 * page's full-strength erase.  No feature map and no normaliser; keys are used
 * as given (the recurrence is stable for beta |k|^2 <= 2, e.g. unit keys).
 * Gates must lie in (0, 1]; a gate at or below 2^-100 acts as 2^-100.
 *
 * la_chunked_forward_delta - the causal forward, chunk by chunk.  Inside a
 * chunk of n rows starting from the state P, with g_i the product of the
 * chunk's gates up to row i, the recurrence unrolls to the unit
 * lower-triangular system (I + A) U = diag(beta) (V - diag(g) K P),
 * A[i][j] = beta_i (k_i . k_j) g_i / g_j (j < i), and
 *     O = diag(g) Q P + (tril(Q K^T) * G) U,   G[i][j] = g_i / g_j,
 *     P <- g_n P + K^T diag(g_n / g) U.
 *   q, k [BH, L, d_k], v [BH, L, d_v]: LA_BF16, d_k in {64, 128}, d_v in
 *        {64, 128, 256}; C must be 64.
 *   beta [BH, L] float32 (device); alpha [BH, L] float32 (device) or NULL.
 *   o    [BH, L, d_v] LA_BF16.  S_final [BH, d_k, d_v] float32 or NULL: the
 *        state after the last token.  The initial state is zero.
 *   workspace  la_chunked_forward_delta_workspace(...) bytes: the per-chunk
 *        transforms T = (I + A)^-1 diag(beta) and the gates' log products.
 * Errors: LA_ERR_INVALID_ARG (NULL pointer, non-positive size),
 * LA_ERR_UNSUPPORTED (other types, widths or chunk sizes), LA_ERR_WORKSPACE;
 * nothing is launched on an error.
 */
la_status la_chunked_forward_delta(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                   int64_t L, int64_t d_k, int64_t d_v, int64_t C, const float* beta,
                                   const float* alpha, void* o, la_dtype out_dt, float* S_final, void* workspace,
                                   size_t ws_bytes, la_stream_t stream);
size_t la_chunked_forward_delta_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v,
                                          int64_t C);

/*
 * la_delta_chunk_transform - the forward's first kernel alone: for every chunk
 * n of 64 rows (N = ceil(L / 64), the last one padded with zero keys and zero
 * strengths),
 *   T[bh, n] = (I + A)^-1 diag(beta)   (64 x 64, lower triangular, bf16) and
 *   lg[bh, n, i] = log2 of the product of the chunk's gates over rows 0..i
 *   (float32; rows past the end repeat the last).
 * T's row i holds column j at position p(j): inside each 32-column half, j with
 * j mod 32 = 4a + b < 16 at 8a + b, and j mod 32 = 16 + 4a + b at 8a + 4 + b
 * (the key order of the forward's matrix-core operands).
 *   k [BH, L, d_k] LA_BF16 (d_k in {64, 128}); beta, alpha as above; C = 64.
 *   T  [BH, N, 64, 64] LA_BF16 (device); lg [BH, N, 64] float32 (device).
 */
la_status la_delta_chunk_transform(const void* k, const float* beta, const float* alpha, la_dtype in_dt,
                                   int64_t BH, int64_t L, int64_t d_k, int64_t C, void* T, float* lg,
                                   la_stream_t stream);

/*
 * la_recurrent_step_delta - one decode step of the (gated) delta rule for
 * n_states independent states, in place:
 *   u = beta (v - alpha S^T k);  S = alpha S + k u^T;  o = q^T S.
 *   q, k [n_states, d_k], v [n_states, d_v]: LA_BF16, d_k, d_v in {16..256}
 *        powers of two.  beta [n_states] float32 (device); alpha [n_states]
 *        float32 (device) or NULL.
 *   S    [n_states, d_k, d_v] float32, read and updated.
 *   o    [n_states, d_v] LA_F32 or LA_BF16.
 */
la_status la_recurrent_step_delta(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                                  int64_t d_k, int64_t d_v, const float* beta, const float* alpha, float* S,
                                  void* o, la_dtype out_dt, la_stream_t stream);

/* Static description of a status code. */
const char* la_status_string(la_status s);
/* Thread-local description of the last failure on this thread ("" if none). */
const char* la_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBLINATTN_LA_H */
