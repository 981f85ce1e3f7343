/*
 * jamba_mamba.h -- C ABI of the MI355X (gfx950) Mamba mixer layer library.
 *
 * The layer is the Mamba (selective state-space) block that fills seven of every
 * eight layers of Jamba (Jamba: A Hybrid Transformer-Mamba Language Model, §2
 * "Model architecture" and §3.1: blocks of l=8 layers with attention:Mamba =
 * 1:7). It carries no positional input (same paper, §6.5) and keeps a fixed-size
 * state per sequence in place of a KV cache (§2, the KV-cache paragraph and
 * Table 1), which is what the decode entry point carries between tokens.
 *
 * Per token t of a sequence (the pages give no formulas; this is the standard
 * selective-SSM block of the paper's citation [17]):
 *   [x ; z]        = W_in u_t                      in_proj   (x rows first)
 *   x^_t           = SiLU(b_conv + sum_k w_conv[:,k] * x_{t-3+k})   causal depthwise conv, k=4
 *   [delta; B; C]  = W_x x^_t                      x_proj    (rows delta | B | C)
 *   Delta_t        = softplus(W_dt delta + b_dt)   dt_proj
 *   h_t            = exp(Delta_t A) h_{t-1} + Delta_t B_t x^_t,  A = -exp(A_log)
 *   y_t            = C_t . h_t + D x^_t
 *   out_t          = W_out (y_t * SiLU(z_t))       gate + out_proj
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the name ends in _host. All tensors are
 *    dense row-major, owned by the caller, and must stay valid until the work
 *    enqueued on `stream` has finished. Weights are only read.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work and
 *    return without synchronising the host.
 *  - Every argument is validated on the host before anything is enqueued; on an
 *    error nothing is enqueued and a jm_status other than JM_OK is returned, with
 *    a detail message from jm_last_error() (thread-local). Launch failures return
 *    JM_ERR_HIP; faults inside kernels surface at the caller's next synchronisation.
 *  - The library never allocates device memory in these calls: temporaries live in
 *    the caller's workspace, sized by the *_workspace_size queries.
 *  - Calls on different streams with different workspaces may run concurrently.
 *  - Supported shapes: d_state == 16, d_conv == 4, d_model, d_inner % 64 == 0,
 *    dt_rank % 8 == 0; act/weight dtypes either both JM_F32 or both JM_BF16.
 *    A_log, D and dt_proj_b are fp32 and the SSM state is fp32 in both cases.
 */
#ifndef JAMBA_MAMBA_H
#define JAMBA_MAMBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JM_OK = 0,
    JM_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad enum value          */
    JM_ERR_SHAPE = 2,         /* cu_seqlens / token count / batch inconsistent         */
    JM_ERR_UNSUPPORTED = 3,   /* a dimension or dtype combination the kernels lack     */
    JM_ERR_ALIGNMENT = 4,     /* a pointer not 16-byte aligned                         */
    JM_ERR_WORKSPACE = 5,     /* workspace null or smaller than the query returned     */
    JM_ERR_HIP = 6            /* a HIP runtime call failed (message in jm_last_error)  */
} jm_status;

typedef enum { JM_F32 = 0, JM_BF16 = 1 } jm_dtype;

/* Layer sizes and dtypes (the sizes the Jamba-7B-class Mamba layer uses are
 * d_model 4096, d_inner 8192, d_state 16, d_conv 4, dt_rank 256). */
typedef struct {
    int32_t d_model;
    int32_t d_inner;
    int32_t d_state;
    int32_t d_conv;
    int32_t dt_rank;
    int32_t act_dtype;     /* jm_dtype of u, out, conv state and activations      */
    int32_t weight_dtype;  /* jm_dtype of in/x/dt/out projections and conv weights */
} jm_layer_dims;

/* Layer parameters; element type `weight_dtype` unless marked fp32. Zero-initialise the
 * struct (e.g. `jm_layer_weights w = {0};`) so that the optional fields read NULL / 0. */
typedef struct {
    const void  *in_proj_w;   /* (2*d_inner, d_model): rows [0, d_inner) give x, the rest z */
    const void  *conv_w;      /* (d_inner, d_conv): tap d_conv-1 multiplies the current token */
    const void  *conv_b;      /* (d_inner) or NULL for no bias                                */
    const void  *x_proj_w;    /* (dt_rank + 2*d_state, d_inner): rows delta | B | C            */
    const void  *dt_proj_w;   /* (d_inner, dt_rank)                                            */
    const float *dt_proj_b;   /* (d_inner) fp32                                                */
    const float *A_log;       /* (d_inner, d_state) fp32; A = -exp(A_log)                      */
    const float *D;           /* (d_inner) fp32 skip weight                                    */
    const void  *out_proj_w;  /* (d_model, d_inner)                                            */
    /* Optional inner RMSNorm (Jamba paper §2, the paragraph on the Mamba layer's
     * implementation, and §6.4 / Fig. 9: RMSNorm on the layer's internal activations,
     * placement not given). Here: right after x_proj, delta, B and C are each replaced
     * by v / sqrt(mean(v^2) + norm_eps) * gain over their own feature axis (fp32 math),
     * before dt_proj and the scan. All three gains NULL: no norm (the plain layer).
     * All three set: norm on, and norm_eps must be finite and > 0. Mixed: rejected. */
    const float *dt_norm_w;   /* (dt_rank) fp32 or NULL                                        */
    const float *B_norm_w;    /* (d_state) fp32 or NULL                                        */
    const float *C_norm_w;    /* (d_state) fp32 or NULL                                        */
    float        norm_eps;
    /* Optional decode copies of in_proj_w and out_proj_w in 64 x 64 tiles, filled by
     * jm_tile_decode_weights (same size and dtype as the matrices they copy); both set or
     * both NULL. Only the single-token decode reads them (jamba_mamba_decode_step and its
     * _slots and _noalloc forms), with results bit for bit equal to those from the row-major
     * matrices; the prefill reads the row-major ones. Set, they are accepted only where the
     * bf16 decode kernels apply (d_model % 256 == 0, d_inner % 1024 == 0, dt_rank 128 or
     * 256), else JM_ERR_UNSUPPORTED. */
    const void  *in_proj_w_tiles;
    const void  *out_proj_w_tiles;
} jm_layer_weights;

/* Human-readable name of a status. Never NULL. */
const char *jm_status_string(jm_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *jm_last_error(void);

/* Bytes of device workspace jamba_mamba_prefill needs for this many packed tokens
 * and sequences. */
jm_status jm_prefill_workspace_size(const jm_layer_dims *dims, int32_t n_seqs,
                                    int64_t total_tokens, size_t *bytes);

/* Bytes of device workspace jamba_mamba_decode_step needs for `batch` sequences. */
jm_status jm_decode_workspace_size(const jm_layer_dims *dims, int32_t batch, size_t *bytes);

/*
 * Prefill over packed variable-length sequences (the long-context path: one
 * sequence of 128K tokens runs in parallel along its length through a chunked
 * scan). Sequence i is rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of u/out; every
 * sequence starts from its own initial state (or zeros) and never sees another.
 *
 *  u                (total_tokens, d_model)  act_dtype, read
 *  cu_seqlens       (n_seqs + 1) int32 on the device, read by the kernels
 *  cu_seqlens_host  the same values in host memory (validation and planning);
 *                   must equal the device copy. cu[0] == 0, strictly increasing
 *                   (empty sequences are rejected), cu[n_seqs] == total_tokens.
 *  init_conv_state  (n_seqs, d_inner, d_conv-1) act_dtype or NULL (zeros): the
 *                   d_conv-1 pre-conv x values before each sequence, oldest first
 *  init_ssm_state   (n_seqs, d_inner, d_state) fp32 or NULL (zeros)
 *  out              (total_tokens, d_model) act_dtype, written
 *  final_conv_state (n_seqs, d_inner, d_conv-1) act_dtype or NULL: the last
 *                   d_conv-1 pre-conv x values of each sequence, oldest first
 *                   (may be the same buffer as init_conv_state)
 *  final_ssm_state  (n_seqs, d_inner, d_state) fp32 or NULL: h after each
 *                   sequence's last token (must NOT overlap init_ssm_state)
 *  workspace        >= jm_prefill_workspace_size bytes, 256-byte aligned
 * total_tokens must be below 2^31.
 */
jm_status jamba_mamba_prefill(const jm_layer_dims *dims, const jm_layer_weights *weights,
                              const void *u, const int32_t *cu_seqlens,
                              const int32_t *cu_seqlens_host, int32_t n_seqs,
                              int64_t total_tokens,
                              const void *init_conv_state, const float *init_ssm_state,
                              void *out, void *final_conv_state, float *final_ssm_state,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step: one new token for each of `batch` sequences, updating the
 * carried state in place (the constant-size replacement of a KV cache).
 *
 *  u           (batch, d_model) act_dtype, read
 *  conv_state  (batch, d_inner, d_conv-1) act_dtype, read and overwritten with the
 *              shifted window (oldest first)
 *  ssm_state   (batch, d_inner, d_state) fp32, read and overwritten
 *  out         (batch, d_model) act_dtype, written
 *  workspace   >= jm_decode_workspace_size bytes, 256-byte aligned
 */
jm_status jamba_mamba_decode_step(const jm_layer_dims *dims, const jm_layer_weights *weights,
                                  const void *u, int32_t batch, void *conv_state,
                                  float *ssm_state, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Fill the decode copies of the two large projections: in_proj_w_tiles from in_proj_w
 * (2*d_inner x d_model) and out_proj_w_tiles from out_proj_w (d_model x d_inner). Tile
 * (b, s) of an N x K matrix holds rows 64b .. 64b+63 and columns 64s .. 64s+63 as 64 rows of
 * 64 consecutive values; tiles are stored in order of b, then s. At one token per sequence
 * the decode step's cost is streaming these matrices (201 MB at the Jamba-7B-class sizes),
 * and a tile is one contiguous 8 KB run instead of 64 row pieces of 128 bytes, which reads
 * HBM faster when the weights are not cached (serving runs many layers between two steps
 * of one). The copies cost as much memory again as the two matrices. Bf16 layers with
 * d_model % 256 == 0, d_inner % 1024 == 0 and dt_rank 128 or 256 only (else
 * JM_ERR_UNSUPPORTED); all four pointers device memory, 16-byte aligned, the outputs
 * distinct from the inputs. Enqueued on `stream`; the copies must not change while a decode
 * that reads them runs.
 */
jm_status jm_tile_decode_weights(const jm_layer_dims *dims, const void *in_proj_w,
                                 const void *out_proj_w, void *in_proj_w_tiles,
                                 void *out_proj_w_tiles, void *stream);

/* Bytes of the fixed device-side scratch that jamba_mamba_decode_step_noalloc uses on each
 * GPU (32 MiB: a decode step at the Jamba-7B-class sizes needs about 4.2 MB plus 64 KB per
 * sequence, so batches up to about 440 fit). */
#define JM_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * jamba_mamba_decode_step without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The step's temporaries live in a fixed device-side scratch array of
 * JM_DECODE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the process
 * ends; the call allocates nothing (the first call on a device only looks up that device's
 * copy, a runtime query). Arguments and results as jamba_mamba_decode_step; the device of
 * `stream` must be the current device. A batch whose jm_decode_workspace_size exceeds the
 * scratch returns JM_ERR_WORKSPACE with nothing enqueued. All calls on one GPU share its one
 * scratch array: calls that overlap on one GPU (other streams or threads) race and must be
 * ordered by the caller.
 */
jm_status jamba_mamba_decode_step_noalloc(const jm_layer_dims *dims,
                                          const jm_layer_weights *weights, const void *u,
                                          int32_t batch, void *conv_state, float *ssm_state,
                                          void *out, void *stream);

/* ---- State cache (serving) ------------------------------------------------------------
 * The per-sequence state is what replaces the KV cache (Jamba paper §2, the KV-cache
 * paragraph and Table 1; §3.1: long contexts on one 80 GB GPU). A server keeps the states
 * of many sequences in one cache of n_slots rows, conv_cache (n_slots, d_inner, d_conv-1)
 * act dtype and ssm_cache (n_slots, d_inner, d_state) fp32, and runs each call on whichever
 * sequences are active: continuous batching, prefill in chunks that continue from the
 * carried state, and mixed batches (a decode token is a one-token sequence that continues
 * from its slot). States are read from and written to their slots in place.
 */

/* Workspace for jamba_mamba_prefill_slots (the prefill's, plus n_seqs final states). */
jm_status jm_prefill_slots_workspace_size(const jm_layer_dims *dims, int32_t n_seqs,
                                          int64_t total_tokens, size_t *bytes);

/*
 * Prefill over packed sequences against the state cache. Sequence i starts from slot
 * init_slots[i] (-1: from zeros) and leaves its final states in slot final_slots[i] (-1:
 * not kept). init_slots / final_slots are device arrays of n_seqs int32 with host copies
 * (*_host, equal values) used for validation; either pair may be NULL (all -1). A final
 * slot may be its own sequence's init slot (continue in place) but no other sequence's init
 * slot, and final slots are distinct. Other arguments as in jamba_mamba_prefill; workspace
 * >= jm_prefill_slots_workspace_size bytes.
 */
jm_status jamba_mamba_prefill_slots(const jm_layer_dims *dims, const jm_layer_weights *weights,
                                    const void *u, const int32_t *cu_seqlens,
                                    const int32_t *cu_seqlens_host, int32_t n_seqs,
                                    int64_t total_tokens, const int32_t *init_slots,
                                    const int32_t *init_slots_host, const int32_t *final_slots,
                                    const int32_t *final_slots_host, void *conv_cache,
                                    float *ssm_cache, int32_t n_slots, void *out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * One decode step for `batch` sequences whose states sit in slots slots[0..batch) of the
 * cache (device int32 array, distinct values in [0, n_slots), with an equal host copy
 * slots_host for validation); the slots are updated in place. u, out, workspace as in
 * jamba_mamba_decode_step (workspace >= jm_decode_workspace_size(batch)).
 */
jm_status jamba_mamba_decode_step_slots(const jm_layer_dims *dims,
                                        const jm_layer_weights *weights, const void *u,
                                        int32_t batch, const int32_t *slots,
                                        const int32_t *slots_host, void *conv_cache,
                                        float *ssm_cache, int32_t n_slots, void *out,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* ---- Plan inspection (host only; for tests of the packed-sequence indexing) ---- */

/* One run of consecutive tokens inside one scan chunk that belong to one sequence. */
typedef struct {
    int32_t chunk;        /* chunk index                                   */
    int32_t seq;          /* sequence index                                */
    int32_t begin;        /* first packed token row of the run             */
    int32_t end;          /* one past the last row                         */
    int32_t starts_seq;   /* 1 if `begin` is the sequence's first token    */
    int32_t ends_seq;     /* 1 if `end - 1` is the sequence's last token   */
} jm_chunk_segment;

/*
 * The chunking jamba_mamba_prefill uses for these sequences: chunk c covers rows
 * [c*chunk_len, min((c+1)*chunk_len, total_tokens)). Writes *chunk_len and
 * *n_chunks, and up to max_segments segments in chunk order (then row order);
 * *n_segments receives the full count. `segments` may be NULL when max_segments is 0.
 */
jm_status jm_prefill_plan(const jm_layer_dims *dims, const int32_t *cu_seqlens_host,
                          int32_t n_seqs, int64_t total_tokens, int32_t *chunk_len,
                          int32_t *n_chunks, jm_chunk_segment *segments,
                          int64_t max_segments, int64_t *n_segments);

/* Chunk length override for the scan (0 = automatic). Process-wide, for tuning and
 * for chunk-count invariance tests: it changes the chunk plan of every later prefill,
 * plan query and workspace-size query on every thread, so it must not change between a
 * *_workspace_size query and the call that uses that workspace. Returns
 * JM_ERR_INVALID_ARG if negative. */
jm_status jm_set_scan_chunk_len(int32_t chunk_len);

/* ---- Stage entry points (diagnostics) -------------------------------------------
 * Each runs one step of jamba_mamba_prefill on its own, with the same kernels and
 * launch configuration, so that a step can be checked against a reference fed the
 * same inputs. The steps are the lines of the per-token recurrence at the top of
 * this file. T = total_tokens (1 <= T < 2^31); all tensors row-major, T rows;
 * "act" = act_dtype. Validation and errors as for jamba_mamba_prefill; all weight
 * pointers must be valid even where a step does not read them.
 */

/* in_proj: [x ; z] = W_in u.  u (T, d_model) act -> x, z (T, d_inner) act. */
jm_status jm_stage_in_proj(const jm_layer_dims *dims, const jm_layer_weights *weights,
                           const void *u, int64_t total_tokens, void *x, void *z, void *stream);

/* Causal depthwise conv (k = d_conv) + SiLU per sequence of cu_seqlens:
 * x (T, d_inner) act -> x_hat (T, d_inner) act; init_conv_state / final_conv_state
 * as in jamba_mamba_prefill (both may be NULL). */
jm_status jm_stage_conv(const jm_layer_dims *dims, const jm_layer_weights *weights,
                        const void *x, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                        int32_t n_seqs, int64_t total_tokens, const void *init_conv_state,
                        void *x_hat, void *final_conv_state, void *stream);

/* x_proj: [delta ; B ; C] = W_x x_hat.  x_hat (T, d_inner) act -> delta (T, dt_rank) act,
 * B and C (T, d_state) fp32. */
jm_status jm_stage_x_proj(const jm_layer_dims *dims, const jm_layer_weights *weights,
                          const void *x_hat, int64_t total_tokens, void *delta, float *B,
                          float *C, void *stream);

/* dt_proj: Delta = softplus(W_dt delta + b_dt).  delta (T, dt_rank) act -> dt (T, d_inner) fp32. */
jm_status jm_stage_dt_proj(const jm_layer_dims *dims, const jm_layer_weights *weights,
                           const void *delta, int64_t total_tokens, float *dt, void *stream);

/* Bytes of workspace jm_stage_scan needs (the chunk aggregates of the chunked scan;
 * 0 when T fits one chunk). */
jm_status jm_stage_scan_workspace_size(const jm_layer_dims *dims, int64_t total_tokens,
                                       size_t *bytes);

/* Selective scan with D skip and gate, per sequence of cu_seqlens:
 *   h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_hat_t,  g_t = (C_t . h_t + D x_hat_t) * SiLU(z_t)
 * x_hat, z (T, d_inner) act; dt (T, d_inner) fp32; B, C (T, d_state) fp32 -> g (T, d_inner)
 * act. init_ssm_state / final_ssm_state as in jamba_mamba_prefill (may be NULL, must not
 * overlap). workspace >= jm_stage_scan_workspace_size bytes (may be NULL if that is 0). */
jm_status jm_stage_scan(const jm_layer_dims *dims, const jm_layer_weights *weights,
                        const void *x_hat, const float *dt, const float *B, const float *C,
                        const void *z, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                        int32_t n_seqs, int64_t total_tokens, const float *init_ssm_state,
                        void *g, float *final_ssm_state, void *workspace, size_t workspace_bytes,
                        void *stream);

/* out_proj: out = W_out g.  g (T, d_inner) act -> out (T, d_model) act. */
jm_status jm_stage_out_proj(const jm_layer_dims *dims, const jm_layer_weights *weights,
                            const void *g, int64_t total_tokens, void *out, void *stream);

/* Decode update: the fused step of jamba_mamba_decode_step that follows x_proj (and the
 * inner norm, which is not applied here), for each of `batch` sequences b:
 *   Delta_b = softplus(W_dt delta_b + b_dt),  h = exp(Delta_b A) h + Delta_b B_b x_hat_b,
 *   g_b = (C_b . h + D x_hat_b) * SiLU(z_b),
 * with the SSM state h updated in place. It runs the kernels the decode step runs.
 *  x_hat, z    (batch, d_inner) act, read
 *  delta       (batch, dt_rank) act, read
 *  B, C        (batch, d_state) fp32, read
 *  slots       NULL: ssm_state is (batch, d_inner, d_state) fp32 and row b is sequence b's;
 *              else a device int32 array of `batch` distinct slot ids in [0, n_slots) with an
 *              equal host copy slots_host (validated), and ssm_state is a cache of n_slots
 *              rows of which only rows slots[0..batch) are read and written
 *  g           (batch, d_inner) act, written
 * batch == 0 is a no-op. Errors as for the other stage entry points. */
jm_status jm_stage_decode_update(const jm_layer_dims *dims, const jm_layer_weights *weights,
                                 const void *x_hat, const void *z, const void *delta,
                                 const float *B, const float *C, int32_t batch,
                                 const int32_t *slots, const int32_t *slots_host, int32_t n_slots,
                                 float *ssm_state, void *g, void *stream);

/* ---- Backward of the scan step (training) ----------------------------------------------
 * Gradients of jm_stage_scan's output (g = (scan(x_hat, Delta, A, B, C; h0) + D x_hat) *
 * SiLU(z), per sequence of cu_seqlens) for the training step (Jamba paper §3.1: trained up to
 * 1M-token contexts; §6.4 on training stability), by reverse mode through the recurrence.
 * Inputs as jm_stage_scan's (x_hat, z act dtype; dt, B, C fp32; init_ssm_state fp32 or NULL),
 * plus dg (T, d_inner) act dtype = dL/dg and d_final_ssm_state (n_seqs, d_inner, d_state)
 * fp32 or NULL = dL/d(final state). Outputs, all fp32 and fully overwritten: dx_hat, ddt, dz
 * (T, d_inner); dB, dC (T, d_state); dA_log (d_inner, d_state); dD (d_inner); and
 * d_init_ssm_state (n_seqs, d_inner, d_state) or NULL. A_log and D are read from weights.
 * Deterministic (fixed-order reductions). workspace >= jm_scan_backward_workspace_size.
 */
jm_status jm_scan_backward_workspace_size(const jm_layer_dims *dims, int64_t total_tokens,
                                          size_t *bytes);
jm_status jamba_mamba_scan_backward(const jm_layer_dims *dims, const jm_layer_weights *weights,
                                    const void *x_hat, const float *dt, const float *B,
                                    const float *C, const void *z, const void *dg,
                                    const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                    int32_t n_seqs, int64_t total_tokens,
                                    const float *init_ssm_state, const float *d_final_ssm_state,
                                    float *dx_hat, float *ddt, float *dB, float *dC, float *dz,
                                    float *dA_log, float *dD, float *d_init_ssm_state,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* ---- Kernel timing (diagnostics; the benchmark reads per-kernel durations) ----
 * While enabled, every kernel the library enqueues is bracketed by a pair of HIP
 * events on the caller's stream. jm_profile_read synchronises those events and
 * reports, per kernel name, the number of launches and the summed milliseconds
 * since the last reset. Not for concurrent use from several threads. */
jm_status jm_profile_enable(int32_t enable);
jm_status jm_profile_reset(void);
typedef struct {
    char    name[32];
    int64_t launches;
    double  total_ms;
} jm_kernel_time;
jm_status jm_profile_read(jm_kernel_time *out, int32_t max_entries, int32_t *n_entries);

#ifdef __cplusplus
}
#endif

#endif /* JAMBA_MAMBA_H */
