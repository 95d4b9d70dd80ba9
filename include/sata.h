/*
 * sata.h -- C ABI of the SATA causal self-attention hot path on MI355X (gfx950).
 *
 * Method: Heinsen & Kozachkov, "Self-Attention at Constant Cost per Token via
 * Symmetry-Aware Taylor Approximation" (arXiv:2602.00294), as described on the
 * blog.hotdry.top post "self-attention-constant-cost-taylor-approximation"
 * ([TA], cited by section) and its companion "constant-cost-attention-hardware-
 * optimization" ([HW]).
 *
 * What is computed.  For one head with queries q_t, keys k_t (d_K) and values
 * v_t (d_V), the exponential kernel exp(q.k / c), c = sqrt(d_K), is truncated to
 * its first P Taylor terms ([TA] "Feature maps and linear attention"):
 *     w(q, k) = sum_{p=0}^{P-1} alpha_p (q.k)^p,   alpha_p = 1 / (p! c^p),
 * and causal attention with it is
 *     y_T = sum_{t<=T} w(q_T, k_t) v_t  /  sum_{t<=T} w(q_T, k_t).
 * Each (q.k)^p is written over the unique monomials of the symmetric tensor
 * q^{(x)p}: index tuples i1 <= ... <= ip (table M_p, m_p = binom(d_K+p-1, p)
 * rows, [TA] "The mathematical breakthrough of the Taylor approximation"), with
 * C_p the number of times each monomial occurs in the full expansion ([TA]
 * "Feature maps and linear attention").  With phi_p(x)[r] = prod_{i in M_p[r]} x_i,
 *     (q.k)^p = sum_r C_p[r] phi_p(q)[r] phi_p(k)[r],
 * so attention becomes a scan over the fixed-size state ([TA] "Feature maps ...",
 * "Hidden-state size and compute analysis")
 *     S = sum_t phi(k_t) [v_t | 1]^T        ((d_V + 1) x M entries, M = sum_p m_p),
 * read out by y_T = (q~_T^T S)[0:d_V] / (q~_T^T S)[d_V], q~[f] = alpha_p C_p[f] phi_p(q_T)[f].
 *
 * Conventions used by every entry point.
 *   Feature order.  f runs over the concatenation p = 0, 1, ..., P-1 of the rows
 *     of M_p, each M_p in lexicographic order of its (non-decreasing) tuples.
 *     M = binom(d_K + P - 1, P - 1).  M_pad = M rounded up to a multiple of 64.
 *   Tensors (row-major, contiguous, device memory, 16-byte aligned):
 *     prefill  q, k : [B][H][n][d_K]     v : [B][H][n][d_V]     y : [B][H][n][d_V]
 *     decode   q, k : [B][H][d_K]        v : [B][H][d_V]        y : [B][H][d_V]
 *     state    fp32 [B][H][d_V + 1][M_pad]: entry [b][h][j][f] is S[f][j] of
 *              head (b, h); column j = d_V is the normaliser Z = sum_t phi(k_t).
 *              The state is unweighted (no alpha_p, no C_p).  Entries f >= M are
 *              zero and stay zero.  An all-zero state is the empty prefix.
 *   Input dtype.  q, k, v are fp32 (SATA_F32) or bfloat16 (SATA_BF16); y and the
 *     state are always fp32.
 *   Causality.  Row T attends to t <= T (inclusive); the decode step adds the new
 *     token to the state before reading it out.
 *   Streams.  Work is enqueued on `stream` (a hipStream_t, NULL = default stream)
 *     and returns without waiting; apart from workspace growth (below) no call
 *     synchronises the host.
 *   Ownership.  The caller owns q, k, v, y and the state.  The library owns the
 *     tables handle (host and device copies) and scratch workspaces held by the
 *     handle, one per stream the handle is used on, grown on demand and released by
 *     sata_tables_free.  A handle is safe across threads (its host state is locked
 *     during each call) and streams (calls on different streams never share workspace
 *     memory, so they may overlap on the device).
 *   Workspace growth.  A call that needs more workspace than its stream's buffer holds
 *     waits for that stream (hipStreamSynchronize), frees the old buffer and allocates
 *     a larger one; that is the only host synchronisation of the compute calls.  Size
 *     it beforehand with sata_prefill_workspace / sata_decode_workspace and
 *     sata_reserve_workspace to keep every later call free of it.
 *   Errors.  Every int-returning call returns SATA_OK (0) or a negative code and
 *     never aborts; sata_last_error() gives the calling thread's last message.
 *     Arguments are checked before anything is enqueued, so on an argument error
 *     no output and no state is touched.  A failed HIP launch returns SATA_ERR_HIP.
 *   Supported sizes: 1 <= d_K <= 128, 1 <= d_V <= 128, 1 <= P <= 5,
 *     chunk in {16, 32, 64, 128}, n >= 1, B, H >= 1.  n need not be a multiple of
 *     chunk (the last chunk is masked).
 */
#ifndef SATA_H
#define SATA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sata_tables sata_tables;

typedef enum { SATA_F32 = 0, SATA_BF16 = 1 } sata_dtype;

enum {
    SATA_OK = 0,
    SATA_ERR_ARG = -1,          /* null pointer, bad size, handle mismatch        */
    SATA_ERR_UNSUPPORTED = -2,  /* size outside the supported set                  */
    SATA_ERR_ALIGN = -3,        /* a tensor pointer is not 16-byte aligned          */
    SATA_ERR_HIP = -4,          /* a HIP call or kernel launch failed              */
    SATA_ERR_OOM = -5           /* device or host allocation failed                */
};

/* Prefill flag: `state` holds the prefix on entry and is advanced in place. */
#define SATA_PREFILL_CONTINUE 1
/* Prefill flag: `state` is a half-precision state (layout below), not an fp32 one. */
#define SATA_STATE_F16 2

/*
 * Build the tables M_p, C_p (p = 0..P-1) for key dimension d_K on the host, plus
 * the device tables the kernels read, on the current HIP device.  The rows of
 * M_p are the non-decreasing index tuples in lexicographic order; C_p[r] =
 * p! / prod_i (count of i in row r)!  ([TA] "The mathematical breakthrough of the
 * Taylor approximation", "Feature maps and linear attention").
 * *out receives a new handle (free with sata_tables_free).  The handle is used on
 * the device that was current when it was built.
 */
int sata_tables_build(int d_K, int P, sata_tables **out);

/*
 * Host-only handle: builds the same host tables as sata_tables_build but no
 * device copies, so it needs no GPU.  It serves sata_tables_get (inspection,
 * tests); sata_prefill and sata_decode_step reject it with SATA_ERR_ARG after
 * checking their other arguments.
 */
int sata_tables_build_host(int d_K, int P, sata_tables **out);

/*
 * Host views of M_p ([m_p][p] int32, 0-based indices) and C_p ([m_p] int32) for
 * 0 <= p < P.  The pointers stay valid until sata_tables_free.  For p = 0, M_0 is
 * an empty row (*M_p may be NULL) and C_0 = {1}.
 */
int sata_tables_get(const sata_tables *t, int p, const int32_t **M_p,
                    const int32_t **C_p, int64_t *m_p);

/* Release a handle, its device tables and its workspaces.  NULL-safe. */
void sata_tables_free(sata_tables *t);

/* M = binom(d_K + P - 1, P - 1) ([TA] "Hidden-state size and compute analysis"),
 * or -1 outside the supported sizes. */
int64_t sata_feature_dim(int d_K, int P);

/* M_pad: M rounded up to a multiple of 64 (the feature stride of the state). */
int64_t sata_state_stride(int d_K, int P);

/* Bytes of the fp32 state of B x H heads: 4 B H (d_V + 1) M_pad. */
int64_t sata_state_bytes(int B, int H, int d_K, int d_V, int P);

/*
 * Half-precision state.  [TA] "Hidden-state size and compute analysis" sizes a head's state
 * in Float16 (about 6.2 MB at d_K = d_V = 64, P = 4).  In this form the d_V value columns are
 * stored as IEEE fp16 and the normaliser column stays fp32 (its degree-0 entry counts the
 * tokens, which fp16 cannot past 2048); the decode step moves about half the bytes of the
 * fp32 state.  Layout of one head, sata_state16_bytes(1, 1, ...) bytes, each part starting
 * on a multiple of 256 bytes:
 *   header  int32 expo[P][d_V], then float bound[P][d_V]
 *   Z       fp32 [Mh]              the normaliser column
 *   V       fp16 [d_V][Mh]         the value columns
 * Rows follow the feature order of the fp32 state, but the block of degree p starts at row
 * hoff[p] = sum_{p' < p} roundup(m_p', 64), and Mh = sata_state16_stride = sum_p
 * roundup(m_p, 64); rows past m_p in a block are zero.  Entry (row r of M_p, column j < d_V)
 * = V[j][hoff[p] + r] x 2^expo[p][j]; Z[hoff[p] + r] is the normaliser entry.  Each degree
 * block of each column has its own power-of-two exponent, chosen from the largest entry of the
 * block so that every finite state fits fp16's range; bound[p][j] holds that largest |entry|.
 * An all-zero block of bytes is the empty prefix.
 * Arithmetic is fp32; each write rounds a value entry to fp16 (to nearest even, relative
 * error at most 2^-11 of the entry).  Caller-owned, 16-byte aligned, like the fp32 state.
 */
int64_t sata_state16_stride(int d_K, int P);
int64_t sata_state16_bytes(int B, int H, int d_K, int d_V, int P);

/*
 * Conversions between the two state forms for `count` heads (1..65535): fp32 states
 * [count][d_V + 1][M_pad] and half-precision states [count][sata_state16_bytes(1, 1, ...)]
 * (pack rounds each value entry to fp16 and sets the exponents; unpack is exact).  Enqueued on
 * `stream`.  Errors: SATA_ERR_ARG (NULL, count), SATA_ERR_UNSUPPORTED (d_V), SATA_ERR_ALIGN.
 */
int sata_state_pack_f16(const sata_tables *t, const float *state, void *state16, int count,
                        int d_V, void *stream);
int sata_state_unpack_f16(const sata_tables *t, const void *state16, float *state, int count,
                          int d_V, void *stream);

/*
 * Causal prefill of n tokens per head: y for every row, by a chunked scan
 * ([TA] "Feature maps and linear attention": the state recurrence, evaluated by
 * chunks).  Within a chunk of `chunk` tokens the weights w(q_T, k_t) are formed
 * directly from q.k; earlier chunks enter through the state.
 *
 * t      handle built for (d_K, P) on the current device
 * q,k,v  inputs, in_dtype, layouts above
 * y      fp32 output [B][H][n][d_V]
 * state  nullable.  If non-NULL the state after the n tokens is written to it: an fp32
 *        state, or with flags & SATA_STATE_F16 a half-precision state (the scan then runs
 *        on an fp32 copy in the workspace, converted from and to the caller's state; y is
 *        the same either way).
 *        With flags & SATA_PREFILL_CONTINUE it must be non-NULL and on entry holds
 *        the state of a prefix that precedes these n tokens; y then attends to
 *        that prefix too.  Without the flag the prefix is empty.
 * stream hipStream_t (NULL = default stream)
 *
 * Precision: bf16 inputs with d_K, d_V in {64, 128}, P >= 2 and chunk 64 take the
 * matrix-core path: contractions with fp16 operands and fp32 accumulation, the state in
 * fp32.  q, k and v enter as q 2^-s_q, k 2^-s_k, v 2^-s_v, with per-head powers of two that
 * put each one's maximum in [1, 2); the readout's fp16 copy of the state and the per-slice
 * partial readouts (fp16) carry power-of-two exponents chosen from their own largest
 * entries, so no finite input overflows, whatever the magnitude of q, k or v or the length
 * of the context (a continued prefill included).  Per-row error against the exact attention
 * about 1e-3 (the fp16 operand rounding).  All other cases take the fp32 path (errors of
 * fp32 rounding).
 *
 * Two-level form (bf16 matrix-core path only): when the slices of all B x H heads
 * leave compute units idle (few heads), the sequence is cut into sub-segments of
 * whole readout windows; the local states of the first sub-segments (in pieces of
 * whole windows) are summed in parallel, added in order into each sub-segment's
 * starting state, and the sub-segments are then scanned in parallel from those
 * states ([TA] "Hardware optimisation path": the recurrence as a parallel prefix).
 * The results equal the one-segment scan up to rounding.
 * sata_set_prefill_split chooses when it is used.
 */
int sata_prefill(const sata_tables *t, const void *q, const void *k, const void *v,
                 float *y, void *state, int B, int H, int n, int d_K, int d_V,
                 int P, int chunk, sata_dtype in_dtype, int flags, void *stream);

/*
 * One decode step for B x H heads ([TA] "Feature maps and linear attention":
 * S_T = S_{T-1} + phi(k_T) [v_T | 1]^T, then the readout of q_T).  The state is
 * read, updated with the new token and written back in place; y receives the
 * readout of q against the updated state.
 */
int sata_decode_step(const sata_tables *t, float *state, const void *q,
                     const void *k, const void *v, float *y, int B, int H,
                     int d_K, int d_V, int P, sata_dtype in_dtype, void *stream);

/*
 * The decode step for a batch whose states live in a pool ([HW] "The fixed-size
 * hidden state of SATA attention": the state's memory is allocated up front and
 * requests take turns on the device).  A sequence's whole history is its state, so
 * sequences at different positions share a step, and sequences join and leave the
 * batch by the slot list alone.  Batch entry i uses pool slot slots[i]; otherwise as
 * sata_decode_step.
 *
 * state_pool  fp32 [pool_size][H][d_V + 1][M_pad], updated in place.  A slot is one
 *             contiguous block of sata_state_bytes(1, H, ...) bytes: a sequence is
 *             started by sata_prefill with B = 1 and `state` pointing at its slot, and
 *             saved or restored by copying that block.
 * slots       int32 [count], device memory, 4-byte aligned.  Slots of one call must be
 *             distinct (entries that share a slot race).  An entry whose slot is
 *             outside [0, pool_size) leaves the pool untouched and gets NaN in its y row.
 * q, k        [count][H][d_K]; v: [count][H][d_V]; y: fp32 [count][H][d_V]
 * Errors: SATA_ERR_ARG for NULL pointers, count, H or pool_size < 1; the checks of
 * sata_decode_step otherwise.
 */
int sata_decode_step_pool(const sata_tables *t, float *state_pool, int64_t pool_size,
                          const int32_t *slots, int count, const void *q, const void *k,
                          const void *v, float *y, int H, int d_K, int d_V, int P,
                          sata_dtype in_dtype, void *stream);

/*
 * The decode step for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same computation and
 * kernels as sata_decode_step, but the partial readouts go to a fixed device array of
 * 16 MiB that the library holds on each GPU it runs on until the process ends, instead of
 * the handle's workspace.  The call allocates nothing (no workspace, no timing events).
 * Limit: B x H x (d_V + 1) x ceil(M_pad / 1024) x 8 bytes <= 16 MiB (e.g. 512 heads at
 * d_K = d_V = 64, P = 4; 32 heads at d_K = d_V = 128, P = 4); larger batches return
 * SATA_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU shares that
 * array, so calls that overlap in time on one GPU (several streams, threads or handles)
 * race; issue them in order.  Errors otherwise as sata_decode_step.
 */
int sata_decode_step_noalloc(const sata_tables *t, float *state, const void *q,
                             const void *k, const void *v, float *y, int B, int H,
                             int d_K, int d_V, int P, sata_dtype in_dtype, void *stream);

/*
 * The decode step on half-precision states (layout above), dense and pool forms; otherwise as
 * sata_decode_step and sata_decode_step_pool.  The readout uses the fp32 entries before they
 * are rounded to fp16 for storage.  Each step sets the exponent of every degree block of every
 * column from the bound bound (1 + 2^-10) + kinf^p |u_j| on its new entries (kinf = max_i
 * |k_i|, u = [v | 1]; fp16 rounding of an entry is below 2^-11 of it) and records the blocks'
 * new largest entries as the next bounds.
 */
int sata_decode_step_f16(const sata_tables *t, void *state16, const void *q, const void *k,
                         const void *v, float *y, int B, int H, int d_K, int d_V, int P,
                         sata_dtype in_dtype, void *stream);
int sata_decode_step_pool_f16(const sata_tables *t, void *state16_pool, int64_t pool_size,
                              const int32_t *slots, int count, const void *q, const void *k,
                              const void *v, float *y, int H, int d_K, int d_V, int P,
                              sata_dtype in_dtype, void *stream);

/*
 * Gradients of the causal prefill: for a loss with dL/dy = dy, the gradients dq, dk, dv
 * of the y that sata_prefill computes from q, k, v (empty prefix; no state in or out).
 * With y_T = N_T / D_T ([TA] "Feature maps and linear attention": N_T = sum_{t<=T}
 * w(q_T.k_t) v_t, D_T = sum_{t<=T} w(q_T.k_t)), g_T = dy_T / D_T, h_T = -(dy_T . y_T) / D_T,
 * c_Tt = g_T . v_t + h_T and w'(x) = sum_{p>=1} p alpha_p x^{p-1}:
 *     dv_t = sum_{T>=t} w(q_T.k_t) g_T,
 *     dq_T = sum_{t<=T} c_Tt w'(q_T.k_t) k_t,     dk_t = sum_{T>=t} c_Tt w'(q_T.k_t) q_T.
 * The pages give the forward only; these are its derivatives.  The call recomputes the
 * forward in fp32 and then runs two chunked scans over fixed-size states: the forward
 * state for dq, and its mirror sum_{T>=t} alpha C phi(q_T) u_T^T (u = [g | h]) in reverse
 * chunk order for dk and dv; pairs inside a chunk are taken directly.  Arithmetic is fp32
 * for either input type (state contractions on the matrix cores with fp32 operands).
 *
 * q, k, v  [B][H][n][d_K or d_V], in_dtype (as for sata_prefill)
 * dy       fp32 [B][H][n][d_V]
 * dq, dk   fp32 [B][H][n][d_K] (written);  dv: fp32 [B][H][n][d_V] (written)
 * Errors: as sata_prefill; SATA_ERR_UNSUPPORTED when the chunk's tables do not fit LDS
 * (chunk 128 with d_K or d_V above 64, chunk 64 at d_K = d_V = 128).  The handle's
 * workspace holds y, D, u and the slice partials (segments of whole chunks under the cap).
 */
int sata_prefill_backward(const sata_tables *t, const void *q, const void *k, const void *v,
                          const float *dy, float *dq, float *dk, float *dv, int B, int H,
                          int n, int d_K, int d_V, int P, int chunk, sata_dtype in_dtype,
                          void *stream);

/* The calling thread's last error message ("" if none). */
const char *sata_last_error(void);

/*
 * Optional: cap (bytes) on the workspace a handle may hold per stream; prefill splits the
 * sequence into segments of whole readout windows to stay under it (a segment holds
 * at least one window: 4 chunks at d_K = 64, 2 at d_K = 128 on the bf16 matrix-core
 * path, 1 otherwise, even when one window alone exceeds the cap).  0 restores the
 * default (32 GiB: the bf16 Long prefill, 4 x 16 heads of 65536 tokens, takes about
 * 31 GB of it in 2 segments; query the need with sata_prefill_workspace).
 */
int sata_set_workspace_limit(sata_tables *t, int64_t bytes);

/*
 * Workspace that sata_prefill with these arguments would use under the handle's
 * current cap, and how it would cut the sequence; no device work, so a host-only
 * handle serves too.  with_state: nonzero if the call passes a state buffer.
 * *bytes receives the workspace bytes; the nullable outputs: *segments the number of
 * segments of the one-level scan, *segment_chunks their length in chunks (the last may
 * be shorter), *subsegments the sub-segments of the two-level form (1 when it is not
 * used).  Errors: those of sata_prefill's size checks.
 */
int sata_prefill_workspace(const sata_tables *t, int B, int H, int n, int d_K, int d_V,
                           int P, int chunk, sata_dtype in_dtype, int flags, int with_state,
                           int64_t *bytes, int *segments, int *segment_chunks,
                           int *subsegments);

/* Workspace bytes of the decode step (either state form, dense or pool with count = B) for
 * B x H heads. */
int sata_decode_workspace(const sata_tables *t, int B, int H, int d_V, int64_t *bytes);

/*
 * Grow the handle's workspace of `stream` to at least `bytes` now (growth waits for
 * `stream`, see "Workspace growth"), so that later calls on that stream needing at most
 * that much neither allocate nor synchronise.  SATA_ERR_OOM if the allocation fails.
 */
int sata_reserve_workspace(sata_tables *t, int64_t bytes, void *stream);

/*
 * Optional: sub-segments of the two-level prefill.  0 (the default): automatic,
 * used when B H times the number of feature slices is at most half the device's
 * compute units, with at least 4 readout windows per sub-segment; 1: never;
 * k >= 2: k sub-segments (fewer when the sequence has fewer readout windows)
 * whenever the matrix-core path runs.  The two-level form needs workspace for
 * the partials of the whole sequence plus one state per sub-segment and one per
 * piece of the update pass (sata_prefill_workspace reports it); beyond the
 * workspace cap the one-level form runs.  Errors: SATA_ERR_ARG for a NULL handle
 * or k outside [0, 4096].
 */
int sata_set_prefill_split(sata_tables *t, int nsub);

/*
 * Kernel timing.  With timing enabled, every kernel launch of the handle is
 * bracketed by two HIP events recorded on the launch stream.  sata_read_timing
 * waits for the recorded events, writes per kernel kind k (SATA_KERNEL_*) the
 * summed elapsed milliseconds ms[k] and the number of launches count[k] since
 * the previous read (either pointer may be NULL), and resets the record.
 * Enabling or disabling also resets it.  Timing adds two event records per
 * launch and no host synchronisation outside sata_read_timing.
 */
enum {
    SATA_KERNEL_SCAN = 0,          /* inter-chunk scan (partials + state update) */
    SATA_KERNEL_FINALIZE = 1,      /* intra-chunk part, reduction, y             */
    SATA_KERNEL_DECODE = 2,        /* decode state read-modify-write             */
    SATA_KERNEL_DECODE_REDUCE = 3, /* decode per-head reduction, y               */
    SATA_KERNEL_BACKWARD = 4,      /* one sata_prefill_backward call, all kernels */
    SATA_KERNEL_PREP = 5,          /* operand images of the matrix-core scan      */
    SATA_KERNEL_CONVERT = 6,       /* state conversions of a half-precision prefill */
    SATA_NUM_KERNELS = 7
};
int sata_set_timing(sata_tables *t, int enable);
int sata_read_timing(sata_tables *t, double *ms, int64_t *count);

#ifdef __cplusplus
}
#endif

#endif /* SATA_H */
