/*
 * libaaren -- exact single-query softmax attention on MI355X (gfx950).
 *
 * The library computes attention of ONE query per head over a sequence of
 * key/value pairs, and its many-to-many form, through the associative
 * online-softmax combine of a running maximum m, a normaliser u and a
 * weighted value sum w: the prefix scan (dense, strided and packed), its
 * gradients, the per-token and multi-token constant-memory updates and the
 * many-to-one reduction; and, built on the same combine, self-attention with
 * one query per token, one Aaren layer (projections + scan) and attention of
 * a mean query.
 *
 * Sources (the pages these calls implement):
 *  - "Self-attention Does Not Need O(n^2) Memory" (review), section 1
 *    Introduction: the attention of a single query is the sum of the values
 *    weighted by the softmax of the query-key dot products; section 2
 *    Algorithm: the constant-memory recurrence that accumulates v_i e^{s_i}
 *    and e^{s_i} in order and divides at the end; section 3 Numerical
 *    Stability (body lost; read as the running-maximum shift).
 *  - "Attention as an RNN" (review), abstract items (3) and (4) and the
 *    proposed method: the many-to-many RNN output computed by a parallel
 *    prefix scan, one learned query per head (the initial hidden state q),
 *    constant-memory updates with new tokens.
 *
 * Definitions used by every call:
 *   s_i = scale * <q_h, k_i>                  (scale: caller's, 1/sqrt(d) usual)
 *   many-to-many:  o_k = sum_{i<=k} e^{s_i} v_i / sum_{i<=k} e^{s_i}
 *   many-to-one:   o   = o_N
 *   state (m, u, w): m = max_i s_i, u = sum_i e^{s_i - m}, w = sum_i e^{s_i - m} v_i,
 *   so that o = w / u and the log-normaliser is L = m + ln u. The empty state
 *   is (m = -inf, u = 0, w = 0).
 *
 * Conventions:
 *  - All tensor pointers are DEVICE pointers owned by the caller; no call
 *    allocates except aaren_init (the layer's rocBLAS handle), and the library
 *    keeps no pointer after a call's work completes.
 *  - Tensors are dense, row-major, in the shapes given (aaren_scan_strided
 *    takes explicit strides); q, k and v share `in_dtype` unless a call says
 *    otherwise; every tensor base pointer must be 16-byte aligned.
 *  - d (head dimension) is 64 or 128.
 *  - Work runs on the calling thread's current HIP device: tensors,
 *    workspace and stream must belong to it.
 *  - `hip_stream` is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on that stream and returns; device-side faults surface at
 *    the caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued: on a non-OK status
 *    nothing is enqueued and no output is touched; aaren_last_error() then
 *    holds a description (thread-local).
 *  - Outputs must not alias inputs.
 *  - Thread safety: any number of host threads may call at once, on the
 *    same or different devices and streams, provided calls that can run at
 *    the same time (on different streams) use different workspaces and
 *    outputs. Library state shared between calls (the epoch counter, the
 *    record of cleared workspace bytes and of captured workspaces, the
 *    layer's rocBLAS handles) is guarded.
 *  - Environment: AAREN_LOG=1 prints each call's launch geometry to stderr;
 *    AAREN_STRESS=1 (tests only, read at every call) makes the scans and
 *    their gradients pause tiles at random to perturb the order in which
 *    tiles exchange states; results are unchanged, only slower.
 *    AAREN_HALF_TILES (tests only, read at every dense scan call) overrides
 *    the library's choice of ending each fp32 stream in half tiles: "1"
 *    always, "0" never; results move by rounding only.
 *  - HIP graphs: every call but aaren_init may be captured for replay
 *    (aaren_layer_forward once aaren_init has run on the device).
 *    The scans (aaren_scan, aaren_scan_strided, aaren_scan_segmented) and
 *    their gradients tag the states their workgroups exchange with an epoch:
 *    an eager call takes it from a counter on the host; a call made while its
 *    stream is being captured (hipStreamIsCapturing) enqueues one more
 *    one-thread kernel that advances an epoch word in the workspace header,
 *    which the call's kernels then read, so every replay runs with an epoch
 *    of its own. Eager and captured calls may share a workspace (the two
 *    kinds of epoch are drawn from disjoint ranges), but replays and calls
 *    on one workspace must not overlap in time, like any two calls on it.
 *    A captured scan also records the clearing of its ticket counters, and
 *    every later call on a workspace once used under capture clears its own
 *    (a replay can follow any call of another shape on that workspace).
 *    No call enqueues a memset.
 */
#ifndef AAREN_H
#define AAREN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum aaren_status {
    AAREN_OK = 0,
    AAREN_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad offsets header values */
    AAREN_ERR_UNSUPPORTED = 2,  /* d not in {64,128}, unknown dtype, size beyond limits */
    AAREN_ERR_ALIGNMENT = 3,    /* a base pointer not 16-byte aligned */
    AAREN_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the size query */
    AAREN_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} aaren_status;

typedef enum aaren_dtype {
    AAREN_F32 = 0,
    AAREN_BF16 = 1
} aaren_dtype;

/* Library version as major*10000 + minor*100 + patch. */
int aaren_version(void);

/* Static description of a status code. */
const char *aaren_status_string(aaren_status s);

/* Thread-local description of the last non-OK status returned on this thread. */
const char *aaren_last_error(void);

/* ---- set-up ------------------------------------------------------------------
 * Prepares the calling thread's current HIP device for the calls that keep
 * state in the library: creates the rocBLAS handle aaren_layer_forward runs
 * its projection with (rocBLAS allocates its workspace then), sets up the
 * static scan workspace of aaren_scan_noalloc, and asks the runtime once how
 * many workgroups of the dense scan the device holds at once (the scans pick
 * their tiling from it; without aaren_init the first scan call on the device
 * asks, and a call that gets no answer takes the default tiling, with the same
 * results up to rounding). Call it once per
 * device, before the first aaren_layer_forward there, and never while a stream
 * of the process is being captured into a graph (it allocates); further calls
 * on an initialised device do nothing. It is the only call that allocates.
 * HIP if the handle cannot be created. */
aaren_status aaren_init(void);

/* ---- workspaces ------------------------------------------------------------
 * The scans carry the running state across tiles of a sequence through a
 * caller-owned workspace (per-stream ticket counters and per-tile published
 * states, tagged with a per-call epoch; its header also keeps the epoch of
 * the calls captured into HIP graphs).
 * Contract:
 *  - size it with the matching *_workspace_size query;
 *  - zero it ONCE before its first use (aaren_workspace_clear does that on a
 *    stream, with a fill kernel); afterwards the library leaves it ready for
 *    the next call itself (it remembers, per workspace address, which part is
 *    known clean, and clears its counters again only when a call of another
 *    shape needs it) -- do not write it between calls, and zero it again if
 *    its memory is handed out anew;
 *  - calls of any shape, dense or packed, may share one workspace, but only
 *    one call at a time: calls that may overlap (different streams) need
 *    distinct workspaces.
 * aaren_reduce's workspace holds per-chunk partial states only and needs no
 * clearing.
 */
aaren_status aaren_workspace_clear(void *workspace, size_t workspace_bytes, void *hip_stream);

/* Whether the scans that used a workspace ran as they should. The scans
 * (dense, strided, packed) and their gradients note in the workspace header
 * when one of their workgroups could not take part normally, and then
 * their outputs are wrong: bit 0 (value 1), a workgroup drew a position
 * along its sequence outside the sequence (its ticket counter was not zero
 * when the call began); bit 1 (2), a workgroup walked past the first or
 * last tile of its sequence; bit 2 (4), a workgroup gave up after waiting
 * about a second for an earlier tile's state. None of them happens with a
 * workspace used by the contract above; each points to one that was not
 * zero-filled before first use, was written between calls, or was used by
 * calls that overlapped in time. The word accumulates over calls.
 * This call enqueues on `hip_stream` a copy of the word into `*flags` (a
 * DEVICE uint32, 4-byte aligned; read it after the stream's work is done)
 * and, when `reset` is nonzero, clears the word after copying it. It does
 * not synchronise. INVALID_ARG for NULL pointers, ALIGNMENT for a misaligned
 * workspace or flags, WORKSPACE for a workspace smaller than its 256-byte
 * header. */
aaren_status aaren_workspace_status(const void *workspace, size_t workspace_bytes,
                                    uint32_t *flags, int reset, void *hip_stream);

/* ---- many-to-many scan, dense batch ----------------------------------------
 * Many-to-many output of "Attention as an RNN" (abstract item (3): attention's
 * many-to-many RNN output by a parallel prefix scan; the form that lets the
 * module of item (4) be (i) trained in parallel), one query per head.
 *   q [H,d], k [B,H,N,d], v [B,H,N,d]  (in_dtype)
 *   o [B,H,N,d]                         (out_dtype), o[b,h,i] = attention of
 *                                       q[h] over pairs 0..i of (b,h)
 * B*H*N == 0 is a no-op. Returns WORKSPACE if workspace_bytes is below
 * aaren_scan_workspace_size(B,H,N,d). */
size_t aaren_scan_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_scan(const void *q, const void *k, const void *v, void *o,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/* aaren_scan that also writes, in the same pass,
 *   lse [B,H,N] float32 (not NULL: INVALID_ARG): the log-normaliser
 *   L_i = ln sum_{j<=i} e^{s_j} of every row, what aaren_scan_backward takes.
 * Same workspace, statuses and outputs as aaren_scan otherwise; lse must be
 * 4-byte aligned (ALIGNMENT). */
aaren_status aaren_scan_lse(const void *q, const void *k, const void *v, void *o, float *lse,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                            aaren_dtype in_dtype, aaren_dtype out_dtype,
                            void *workspace, size_t workspace_bytes, void *hip_stream);

/* aaren_scan for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same scan and
 * output, with the workspace taken from a static array the library keeps on
 * each GPU (64 MiB, held until the process ends) instead of a caller's
 * buffer. The call allocates nothing. Shapes whose
 * aaren_scan_workspace_size(B,H,N,d) exceeds 64 MiB are rejected with
 * UNSUPPORTED (e.g. B*H*N up to about 14.9 million rows at d = 64 fit).
 * The array is set up (its address resolved and zero-filled, with a device
 * synchronisation) by aaren_init, or by the first aaren_scan_noalloc call on
 * the device; if that first call is made under graph capture it returns
 * UNSUPPORTED and enqueues nothing. Every call on a GPU shares that GPU's
 * array: calls that can overlap in time on one GPU (different streams,
 * threads) race and give unspecified results. Other statuses as for
 * aaren_scan. */
aaren_status aaren_scan_noalloc(const void *q, const void *k, const void *v, void *o,
                                int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                aaren_dtype in_dtype, aaren_dtype out_dtype, void *hip_stream);

/* ---- gradients of the dense many-to-many scan -------------------------------
 * "Attention as an RNN" (review, proposed method) presents the many-to-many
 * form as differentiable and trained in parallel; the pages print no formula.
 * Derived from the definition, with p_ki = e^{s_i - L_k} and g_k = dloss/do_k:
 *   dv_i = sum_{k>=i} p_ki g_k
 *   ds_i = <dv_i, v_i> - sum_{k>=i} p_ki <g_k, o_k>
 *   dk_i = scale ds_i q_h,  dq_h = scale sum_{b,i} ds_i k_i  (summed over the batch)
 *   q [H,d], k, v, dout [B,H,N,d]  in_dtype (float32 or bfloat16)
 *   o [B,H,N,d] float32: the forward's output (aaren_scan_lse, out_dtype F32)
 *   lse [B,H,N] float32: the forward's log-normaliser
 *   dq [H,d], dk, dv [B,H,N,d] float32 outputs
 * One pass over K, V, O and dout; dq is reproducible bit for bit. bfloat16
 * inputs are widened exactly and everything after is float32 arithmetic. The
 * workspace follows the scan workspace contract (zero-filled once; may be
 * shared with the scans). With B*H*N == 0, dq is set to zero. */
size_t aaren_scan_backward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_scan_backward(const void *q, const void *k, const void *v, const void *o,
                                 const void *dout, const float *lse,
                                 float *dq, float *dk, float *dv,
                                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                 aaren_dtype in_dtype,
                                 void *workspace, size_t workspace_bytes, void *hip_stream);

/* The same scan over tensors laid out with arbitrary element strides, e.g.
 * token-major [B,N,H,d] as a projection produces them: row n of (b,h) of k
 * and v starts at b*kv_strides[0] + h*kv_strides[1] + n*kv_strides[2]
 * elements, and of o at the same with o_strides; the d elements of a row are
 * contiguous. Every stride (in bytes) must be a multiple of 16 (ALIGNMENT
 * otherwise, INVALID_ARG for a negative stride or NULL stride arrays). lse,
 * if given, is [B,H,N] contiguous. Rows of o must not overlap rows of k or v.
 * Workspace as for aaren_scan (same size query). */
aaren_status aaren_scan_strided(const void *q, const void *k, const void *v, void *o,
                                float *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                                const int64_t *kv_strides /* host, [3] */,
                                const int64_t *o_strides /* host, [3] */, float scale,
                                aaren_dtype in_dtype, aaren_dtype out_dtype, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/* ---- many-to-many scan, packed variable-length batch -----------------------
 * The same output for a packed batch of independent sequences (each one is
 * scanned on its own; the pages do not treat packed batches, this is the
 * dense call applied per sequence):
 *   q [H,d]; k, v, o [T,H,d] token-major (T = total_tokens);
 *   offsets [num_seqs+1] int64 DEVICE array, offsets[0] = 0, non-decreasing,
 *   offsets[num_seqs] = T; sequence s holds tokens offsets[s] .. offsets[s+1]-1
 *   (empty sequences allowed).
 * The host cannot read device offsets, so only their count is validated; a
 * decreasing array or one that does not end at T gives unspecified results.
 * num_seqs = 0 with T = 0 is a no-op; tokens without sequences INVALID_ARG;
 * offsets must be 8-byte aligned. */
size_t aaren_scan_segmented_workspace_size(int64_t num_seqs, int64_t total_tokens,
                                           int64_t H, int64_t d);
aaren_status aaren_scan_segmented(const void *q, const void *k, const void *v, void *o,
                                  const int64_t *offsets, int64_t num_seqs,
                                  int64_t total_tokens, int64_t H, int64_t d, float scale,
                                  aaren_dtype in_dtype, aaren_dtype out_dtype,
                                  void *workspace, size_t workspace_bytes, void *hip_stream);

/* aaren_scan_segmented that also writes lse [T,H] float32 (not NULL), the
 * log-normaliser of every row within its own sequence, as aaren_scan_lse
 * does for a dense batch (what aaren_scan_segmented_backward takes). */
aaren_status aaren_scan_segmented_lse(const void *q, const void *k, const void *v, void *o,
                                      float *lse, const int64_t *offsets, int64_t num_seqs,
                                      int64_t total_tokens, int64_t H, int64_t d, float scale,
                                      aaren_dtype in_dtype, aaren_dtype out_dtype,
                                      void *workspace, size_t workspace_bytes,
                                      void *hip_stream);

/* ---- constant-memory RNN step ----------------------------------------------
 * "Attention as an RNN" (abstract item (4)(ii) and method: update with new
 * tokens in constant memory); the update is the recurrence of section 2 of
 * the memory-efficient-attention review, stabilised by the running maximum.
 * Per (stream, head): absorb one pair (k_t, v_t) into the state, in place:
 *   q [H,d], k_t [S,H,d], v_t [S,H,d]  (in_dtype)
 *   m [S,H], u [S,H], w [S,H,d]  float32, in/out (m in natural score units)
 *   o_t [S,H,d] (out_dtype) or NULL: the output after this token, w/u.
 * aaren_state_init writes the empty state (m = -inf, u = 0, w = 0). */
aaren_status aaren_state_init(float *m, float *u, float *w, int64_t S, int64_t H, int64_t d,
                              void *hip_stream);
aaren_status aaren_step(const void *q, const void *k_t, const void *v_t,
                        float *m, float *u, float *w, void *o_t,
                        int64_t S, int64_t H, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype, void *hip_stream);

/* ---- multi-token append -----------------------------------------------------
 * The same update for T new pairs per (stream, head) in one call: a scan of
 * the new tokens whose carry-in is the stored state ("Attention as an RNN",
 * abstract item (4)(ii): new tokens are taken in with constant memory; the
 * update is the combine of the prefix scan in its method section). The
 * state is read and written once per call instead of once per token.
 *   q [H,d];  k, v [T,S,H,d] time-major (k[t] is what aaren_step takes as
 *   k_t for the t-th new token)  (in_dtype)
 *   m [S,H], u [S,H], w [S,H,d]  float32, in/out, as for aaren_step
 *   o [T,S,H,d] (out_dtype) or NULL: o[t] is the output after token t.
 * Each pair is absorbed with aaren_step's own fp32 arithmetic, so the outputs
 * and the state equal, bit for bit, those of T aaren_step calls.
 * T = 0 or S*H = 0: OK, nothing is read or written. No workspace. Errors as
 * for aaren_step (INVALID_ARG for a negative size or a NULL pointer other
 * than o, ALIGNMENT for tensors not 16-byte aligned or m, u not 4-byte
 * aligned, UNSUPPORTED for d or a dtype outside the supported set). */
aaren_status aaren_append(const void *q, const void *k, const void *v,
                          float *m, float *u, float *w, void *o,
                          int64_t S, int64_t T, int64_t H, int64_t d, float scale,
                          aaren_dtype in_dtype, aaren_dtype out_dtype, void *hip_stream);

/* ---- backward of the packed scan -------------------------------------------
 * Gradients of aaren_scan_segmented: each sequence's gradients are those of
 * a dense scan of that sequence alone; dq adds every sequence's.
 *   q [H,d]; k, v, dout [T,H,d] token-major, in_dtype (float32 or bfloat16);
 *   o [T,H,d] float32 and lse [T,H] (aaren_scan_segmented_lse's outputs);
 *   offsets [num_seqs+1] int64 device array as for the forward;
 *   dq [H,d], dk, dv [T,H,d] float32 outputs.
 * Workspace as for aaren_scan_backward (zero-filled once before first use;
 * size from the query). T = 0: dq is zeroed, OK. Tokens with num_seqs = 0:
 * INVALID_ARG. offsets must be 8-byte aligned. */
size_t aaren_scan_segmented_backward_workspace_size(int64_t num_seqs, int64_t total_tokens,
                                                    int64_t H, int64_t d);
aaren_status aaren_scan_segmented_backward(const void *q, const void *k, const void *v,
                                           const void *o, const void *dout, const float *lse,
                                           const int64_t *offsets, float *dq, float *dk,
                                           float *dv, int64_t num_seqs, int64_t total_tokens,
                                           int64_t H, int64_t d, float scale,
                                           aaren_dtype in_dtype, void *workspace,
                                           size_t workspace_bytes, void *hip_stream);

/* ---- many-to-one reduction -------------------------------------------------
 * Single-query attention over all N pairs ("Self-attention Does Not Need
 * O(n^2) Memory", sections 1-2; "Attention as an RNN", abstract item (1):
 * the many-to-one RNN output). The pairs are split into chunks whose partial
 * states are combined at the end; the result does not depend on the order of
 * the pairs beyond rounding.
 *   q [H,d], k [B,H,N,d], v [B,H,N,d] (in_dtype);  o [B,H,d] (out_dtype);
 *   m_out, u_out [B,H] float32 or NULL: the final state's m (natural units)
 *   and u, so that L = m + ln u.
 * N == 0 is INVALID_ARG (0/0 has no value); B*H == 0 is a no-op. */
size_t aaren_reduce_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_reduce(const void *q, const void *k, const void *v, void *o,
                          float *m_out, float *u_out,
                          int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                          aaren_dtype in_dtype, aaren_dtype out_dtype,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/* ---- one Aaren layer ------------------------------------------------------
 * "Attention as an RNN" (review, proposed method): an attention module
 * whose query is a learned initial hidden state q (one per head) and whose
 * many-to-many output is the prefix scan; layers are stacked like
 * Transformer attention. Here (the pages print no layer formula; this is
 * the plainest reading):
 *   K = x W_K, V = x W_V   (bf16 x, bf16 weights, fp32 products)
 *   o[b,n,h,:] = attention of q_h over K[b,0..n,h,:], V[b,0..n,h,:]
 * The attention needs K only through the scores <q_h, k_n> = x_n (W_K^h q_h):
 * the call folds q into W_K (u_h = W_K^h q_h, kept to fp32 precision as three
 * bf16 parts), so one rocBLAS GEMM gives V and the scores and K is never
 * formed; the result equals the definition's up to fp32 rounding.
 * x [B,N,Dm] bf16; w_kv [Dm, 2*H*d] bf16 row-major (columns 0..H*d-1 = W_K,
 * the rest W_V, head h in columns h*d..h*d+d-1 of each); q [H,d] float32;
 * o [B,N,H,d] (out_dtype; a stacked layer takes o, bf16, as its x with
 * Dm = H*d). The workspace (aaren_layer_workspace_size, which needs Dm for
 * the folded weights) holds those weights (bf16), V and the scores (fp32)
 * and the scan's state; zero-fill it once before first use, as for
 * aaren_scan; 0 means the sizes overflow. The projection runs through the
 * rocBLAS handle aaren_init created for the device; without it the call
 * returns UNSUPPORTED and enqueues nothing. It allocates nothing.
 * B*N*H = 0: OK, nothing done. Dm = 0 with rows: INVALID_ARG. Sizes beyond
 * the 32-bit GEMM interface: UNSUPPORTED. A GEMM failure: HIP. */
size_t aaren_layer_workspace_size(int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t d);
aaren_status aaren_layer_forward(const void *x, const void *w_kv, const float *q, void *o,
                                 int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t d,
                                 float scale, aaren_dtype out_dtype, void *workspace,
                                 size_t workspace_bytes, void *hip_stream);

/* ---- self-attention, one query per token ------------------------------------
 * "Self-attention Does Not Need O(n^2) Memory", section 2: the single-query
 * algorithm extended to self-attention by evaluating every query with the
 * same recurrence (and the review's chunked GPU/TPU implementation, section
 * 4, whose body is lost). Row i of each (b,h) is the attention of query q_i
 * over pairs 0..i (causal != 0) or over all N pairs:
 *   q, k, v [B,H,N,d] bfloat16 (in_dtype must be AAREN_BF16);
 *   o [B,H,N,d] (out_dtype F32 or BF16);
 *   lse [B,H,N] float32 or NULL: L_i = ln sum_j e^{s_ij} (natural units).
 * Scores (bf16 products) and the value sums are accumulated in fp32 on the
 * matrix cores. The value product takes the softmax weights and V in fp16
 * (11 significant bits): V is first multiplied per (b,h) by the power of two
 * that brings its largest finite magnitude just under 2^15, which is exact
 * for every value at or above 2^-17 of that scale, and the output is
 * multiplied back. An output then lies within about 2^-12 max|v| of exact
 * (max over the row's keys). Infinities and NaNs in V give non-finite
 * outputs in their dimension.
 * The workspace (size from the query; no zero-fill needed, every call
 * overwrites what it reads) holds the scaled V transposed and the per-(b,h)
 * magnitude maxima. B*H*N = 0: OK, nothing is read or written. Statuses as
 * for aaren_scan; UNSUPPORTED also for float32 inputs, for N > 2^22
 * (4,194,304) and for B*H > 65535. */
size_t aaren_self_attention_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_self_attention(const void *q, const void *k, const void *v, void *o,
                                  float *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                                  float scale, int causal, aaren_dtype in_dtype,
                                  aaren_dtype out_dtype, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/* ---- mean-query attention ---------------------------------------------------
 * The global aggregation of the pooling network reviewed on the
 * efficient-transformer page (PoNet, "Global aggregation" and its two
 * equations): the query of each sequence is the average of its query
 * projections, g = (1/N) sum_n hq_n, and attends over all N keys and values
 * (the page's value argument is printed as H_Q; read as H_V). It is the
 * many-to-one reduction above with one query per (b,h):
 *   hq, k, v [B,H,N,d] (in_dtype);  o [B,H,d] (out_dtype);
 *   g_out [B,H,d] float32 or NULL: the mean queries used.
 * g is summed in float64 in a fixed order and rounded to float32 once.
 * N = 0 with B*H > 0: INVALID_ARG; B*H = 0: OK, nothing done. Workspace from
 * the size query; no zero-fill needed. Other statuses as for aaren_reduce. */
size_t aaren_mean_query_attention_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_mean_query_attention(const void *hq, const void *k, const void *v, void *o,
                                        float *g_out, int64_t B, int64_t H, int64_t N,
                                        int64_t d, float scale, aaren_dtype in_dtype,
                                        aaren_dtype out_dtype, void *workspace,
                                        size_t workspace_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* AAREN_H */
