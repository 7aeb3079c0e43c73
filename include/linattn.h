/*
 * linattn.h -- C ABI of liblinattn.so: causal (segment-carried), decode and
 * non-causal linear attention with the feature map phi(x) = elu(x) + 1, on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (web pages, cited by title and section):
 *  - "Attention Kernel Mask" (allenlu2009.github.io, 2024-11-17), section
 *    "Cumsum": running key sum S_t = S_{t-1} + phi(k_t), running context
 *    Z_t = Z_{t-1} + phi(k_t) v_t^T, normaliser D_t = phi(q_t) . S_t + eps and
 *    output out_t = phi(q_t)^T Z_t / D_t; token t sees positions <= t.
 *  - Same page, "How to accelerate causal linear attention": chunk-sequential
 *    mode (inter-chunk term from the carried state plus an intra-chunk masked
 *    quadratic term), the materialised mode (chunk states first, then the
 *    chunks in parallel), and mode 2 (recurrent generation).
 *  - Same page, "Non-causal Bi-Directional Attention Kernel".
 *  - "Segment-Wise Attention" (GitHub issue on Infini-attention): the sequence
 *    is cut into segments that are processed one after another with the
 *    compressive memory -- here the (Z, S) state -- carried between them; the
 *    memory update and retrieval follow the linear-attention rule of
 *    "Transformers are RNNs", whose feature map is elu + 1.
 *
 * Common conventions
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no device memory and keeps no global state; it is reentrant.
 *    Calls on different streams must not share output or workspace buffers.
 *  - q, k, v are [B, H, N, d] with element strides (b, h, n) given in
 *    la_strides and a unit stride along d.  dtype LA_BF16 or LA_F32.
 *  - out is float32 [B, H, N, d] with its own strides (unit stride along d).
 *  - State per head: Z float32 [d][d] row-major, Z[j][c] = sum phi(k)_j v_c
 *    (key dimension first), and S float32 [d].  State tensors are contiguous
 *    [B, H, d, d] and [B, H, d].
 *  - d must be 32, 64 or 128.  eps must be finite and >= 0.
 *  - Alignment: every tensor pointer 16-byte aligned; every stride times the
 *    element size a multiple of 16 bytes.
 *  - Errors: argument errors are detected synchronously before any device work
 *    and nothing is written.  A failed kernel launch returns LA_ERR_LAUNCH.
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Every call is asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *    null stream).
 *  - Results are deterministic: the same inputs, sizes and chunk give bitwise
 *    identical outputs (no floating-point atomics).
 *  - Non-finite inputs: a NaN or infinite q, k or v reaches the outputs of its
 *    own token and of every later token of its head and the carried state,
 *    as in the recurrent form.  The causal calls evaluate each 64-token chunk
 *    as the chunk formulas of "Attention Kernel Mask" print it, a masked
 *    score matrix times V; in IEEE arithmetic a masked (zero) score times an
 *    infinite value is NaN, so an infinite v_s may also turn column c of the
 *    outputs of earlier tokens of its chunk into NaN (c: the column that holds
 *    the infinity).  Outputs of tokens in earlier chunks, and other columns,
 *    are unaffected.  (Non-causal and memory calls: every output of the head
 *    reads the non-finite state.)
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL = -1,        /* a required pointer is NULL */
    LA_ERR_SHAPE = -2,       /* a negative size, or sizes too large for 32-bit indexing */
    LA_ERR_DTYPE = -3,       /* dtype is not LA_F32 or LA_BF16 */
    LA_ERR_ALIGN = -4,       /* a pointer or a stride is not 16-byte aligned */
    LA_ERR_UNSUPPORTED = -5, /* d not in {32,64,128}, chunk not in {0,16,32,64,128}, or a
                                causal call issued while its stream is being captured */
    LA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the query returned */
    LA_ERR_LAUNCH = -7,      /* a HIP launch failed */
    LA_ERR_VALUE = -8,       /* eps negative or not finite */
    LA_ERR_ALIAS = -9        /* an output state overlaps an input state other than exactly */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Element strides of a [B, H, N, d] tensor; the stride along d is 1. */
typedef struct {
    int64_t b, h, n;
} la_strides;

/* Human-readable name of a status code (static string, never NULL). */
const char *la_status_str(la_status s);

/* Library version as 10000*major + 100*minor + patch. */
int la_version(void);

/*
 * Causal linear attention forward ("Attention Kernel Mask", section "Cumsum",
 * computed chunk by chunk as in the chunk-sequential mode, with the sequence
 * split into groups whose starting states come from a scan of group states,
 * as in the materialised mode).  For every head (b, h) and token t:
 *   Z = Z_in + sum_{i<=t} phi(k_i) v_i^T,  S = S_in + sum_{i<=t} phi(k_i),
 *   out_t = phi(q_t)^T Z / (phi(q_t) . S + eps).
 * z_in / s_in: state carried in from earlier segments ("Segment-Wise
 * Attention"); NULL means zeros (each independently).
 * z_out / s_out: state after the last token; NULL means not written.  They may
 * equal z_in / s_in exactly (in place); any other overlap is LA_ERR_ALIAS.
 * out: NULL computes only the state from k and v (the prefill remark of
 * "Attention Kernel Mask": only the final sums are needed, formed in
 * parallel and summed); then q may be NULL and is not read, and z_out and
 * s_out must not both be NULL.
 * chunk: 0 = default; otherwise 16, 32, 64 or 128 tokens.  It is a tuning
 * choice only: results agree for every chunk up to rounding.  The kernels'
 * MFMA tiles span 64 tokens, so 16 and 32 run as 64; 128 runs as 128 for
 * bf16 inputs at d = 32 and 64 with out != NULL, and as 64 otherwise.
 * N = 0 copies the input state (or zeros) to the output state.
 * Workspace: at least la_causal_fwd_workspace(...) bytes of device memory,
 * any contents; 256-byte alignment recommended.  NULL is allowed when the
 * query returns 0.  The size covers both dtypes and both uses (with and
 * without out).
 * Look-back: workgroups of one call exchange partial states through the
 * workspace, each tagged by the call, and a workgroup waits for the tags of
 * the earlier token groups of its head.  The tag is chosen when the call is
 * issued, so a call issued while `hip_stream` is being captured into a HIP
 * graph (whose replays would reuse it) is refused with LA_ERR_UNSUPPORTED.
 * Every wait is bounded (about 2^20 polls); a wait that gives up writes NaN
 * into the state it was summing, so the outputs of its columns in that
 * token group and the final state turn NaN instead of silently wrong, and
 * it adds 1 to the 32-bit counter at byte offset 0 of the workspace.  The
 * library never resets that counter: a caller that wants to check it sets it
 * to zero once after allocating the workspace and reads it after
 * synchronising.
 */
size_t la_causal_fwd_workspace(int B, int H, int N, int d, int chunk);
la_status la_causal_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        float *out, la_strides so,
                        int B, int H, int N, int d, int chunk, float eps,
                        const float *z_in, const float *s_in,
                        float *z_out, float *s_out,
                        void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * la_causal_fwd without a workspace argument, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing: its scratch memory is a fixed array of
 * la_noalloc_scratch_bytes() bytes per GPU inside the library, held until
 * the process ends.  Arguments, results and errors are those of
 * la_causal_fwd, except:
 *  - a call whose workspace would exceed la_noalloc_scratch_bytes() (that
 *    is, la_causal_fwd_workspace(...) > la_noalloc_scratch_bytes()) returns
 *    LA_ERR_WORKSPACE before any device work;
 *  - every call on one GPU shares that GPU's array, so calls that can
 *    overlap on one GPU (different streams, different host threads without
 *    ordering) race and must not be issued;
 *  - the give-up counter of the look-back lives in the array and cannot be
 *    read; a wait that gives up still shows as NaN outputs and state;
 *  - like la_causal_fwd with outputs, it cannot be captured into a HIP graph
 *    (LA_ERR_UNSUPPORTED).
 */
la_status la_causal_fwd_noalloc(const void *q, la_strides sq, const void *k, la_strides sk,
                                const void *v, la_strides sv, la_dtype dt,
                                float *out, la_strides so,
                                int B, int H, int N, int d, int chunk, float eps,
                                const float *z_in, const float *s_in,
                                float *z_out, float *s_out, void *hip_stream);

/* Bytes of the per-GPU scratch array of la_causal_fwd_noalloc (32 MiB). */
size_t la_noalloc_scratch_bytes(void);

/*
 * The unnormalised causal form: the chunk formulas of "Attention Kernel Mask"
 * (section "How to accelerate causal linear attention", chunk-sequential and
 * materialised modes) as printed, with no denominator:
 *   out_t = phi(q_t)^T Z_t,  Z_t = Z_in + sum_{i<=t} phi(k_i) v_i^T.
 * Arguments, workspace, state handling (S is carried and written exactly as
 * by la_causal_fwd), aliasing and errors are those of la_causal_fwd; eps is
 * validated but does not enter the outputs.
 */
la_status la_causal_fwd_unnormalized(const void *q, la_strides sq, const void *k, la_strides sk,
                                     const void *v, la_strides sv, la_dtype dt,
                                     float *out, la_strides so,
                                     int B, int H, int N, int d, int chunk, float eps,
                                     const float *z_in, const float *s_in,
                                     float *z_out, float *s_out,
                                     void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * Backward pass of the causal form: the gradients of la_causal_fwd's outputs
 * and final state with respect to q, k, v and the carried-in state.
 * "Attention Kernel Mask" names this pass (the "Training-Backward" row of its
 * table under "Causal Attention Training and Inferencing"; training needs all
 * outputs, the cumsum problem of its "Causal linear attention" notes) but
 * does not write it out; it is computed as the exact derivative of the
 * forward definition.  With g_t = phi(q_t), f_t = phi(k_t), the running state
 * Z_t, S_t (carried-in state included), D_t = g_t . S_t + eps and
 * out_t = Z_t^T g_t / D_t:
 *   dn_t = dout_t / D_t,   dD_t = -(dout_t . out_t) / D_t,
 *   dq_t = phi'(q_t) * (Z_t dn_t + S_t dD_t),
 *   R_t = dz_out + sum_{u>=t} g_u dn_u^T,   r_t = ds_out + sum_{u>=t} g_u dD_u,
 *   dk_t = phi'(k_t) * (R_t v_t + r_t),   dv_t = R_t^T f_t,
 *   dz_in = R_0,   ds_in = r_0,
 * where phi'(x) = 1 for x > 0 and e^x otherwise.
 * q, k, v, dt, z_in, s_in, eps, B, H, N, d: the arguments of the forward call
 * whose gradients are taken (z_in / s_in NULL = zeros).  out: that call's
 * float32 output (it supplies dD_t).  dout: float32 [B, H, N, d], the
 * gradient reaching out.  dz_out / ds_out: the gradient reaching the final
 * state ([B, H, d, d] / [B, H, d]); NULL = zeros, which is the detached
 * memory of "Segment-Wise Attention" (its thread discusses carrying the
 * memory across segments without gradients).
 * dq, dk, dv: float32 [B, H, N, d] with their own strides (unit stride along
 * d).  dz_in / ds_in: the gradient reaching z_in / s_in; NULL = not written.
 * No gradient may overlap an input or another gradient (LA_ERR_ALIAS).
 * Strides, alignment, dtypes and sizes follow the common conventions.
 * Workspace: at least la_causal_bwd_workspace(...) bytes, any contents.
 */
size_t la_causal_bwd_workspace(int B, int H, int N, int d);
la_status la_causal_bwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        const float *out, la_strides so, const float *dout, la_strides sdo,
                        int B, int H, int N, int d, float eps,
                        const float *z_in, const float *s_in, const float *dz_out, const float *ds_out,
                        float *dq, la_strides sdq, float *dk, la_strides sdk, float *dv, la_strides sdv,
                        float *dz_in, float *ds_in,
                        void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * One generation step per head ("Attention Kernel Mask", mode 2: recurrent
 * generation with a fixed-size state and no KV cache):
 *   Z += phi(k) v^T;  S += phi(k);  out = phi(q)^T Z / (phi(q) . S + eps).
 * The update precedes the readout, so the new token attends to itself.
 * q, k, v: contiguous [B, H, d] of dtype dt.  z [B, H, d, d] and s [B, H, d]
 * are float32, read and updated in place.  out: float32 [B, H, d].
 */
la_status la_decode_step(const void *q, const void *k, const void *v, la_dtype dt,
                         float *z, float *s, float *out,
                         int B, int H, int d, float eps, void *hip_stream);

/*
 * Non-causal (bidirectional) linear attention ("Attention Kernel Mask",
 * section "Non-causal Bi-Directional Attention Kernel"): per head
 *   Z = sum_t phi(k_t) v_t^T,  S = sum_t phi(k_t),
 *   out_t = phi(q_t)^T Z / (phi(q_t) . S + eps)   for every t.
 * The sums over t are split across workgroups and reduced in a fixed order.
 * Workspace: at least la_noncausal_workspace(...) bytes, any contents (the
 * size covers both dtypes).
 */
size_t la_noncausal_workspace(int B, int H, int N, int d);
la_status la_noncausal_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                           const void *v, la_strides sv, la_dtype dt,
                           float *out, la_strides so,
                           int B, int H, int N, int d, float eps,
                           void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * Compressive memory of one segment, Infini-attention style ("Segment-Wise
 * Attention": the memory is an associative matrix, read and updated with the
 * linear-attention rule of "Transformers are RNNs", and a read is the
 * retrieved memory divided by the retrieved norm term).  Every query of the
 * segment reads only the memory that earlier segments left, then the
 * segment's keys and values are added to it:
 *   out_t = phi(q_t)^T Z_in / (phi(q_t) . S_in + eps)   for every t,
 *   Z_out = Z_in + sum_t phi(k_t) v_t^T,  S_out = S_in + sum_t phi(k_t).
 * q, k, v, out, strides, B, H, N, d, eps, dt: as for la_noncausal_fwd.
 * z_in / s_in: [B, H, d, d] / [B, H, d] float32, the memory before the
 * segment; NULL means zeros (the first segment: every read is 0 / eps).
 * z_out / s_out: the memory after the segment; NULL means not written.  They
 * may equal z_in / s_in exactly (in place); any other overlap is
 * LA_ERR_ALIAS.  out: NULL computes only the update; then z_out and s_out
 * must not both be NULL (LA_ERR_NULL).
 * N = 0 copies the input memory (or zeros) to the output.
 * The sum over the segment is split across workgroups and reduced in a fixed
 * order (deterministic).
 * Workspace: at least la_memory_workspace(...) bytes, any contents (the size
 * covers both dtypes).
 */
size_t la_memory_workspace(int B, int H, int N, int d);
la_status la_memory_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        float *out, la_strides so,
                        int B, int H, int N, int d, float eps,
                        const float *z_in, const float *s_in,
                        float *z_out, float *s_out,
                        void *workspace, size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
