/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * Operation (per head, state S in R^{dk x dv}):
 *   g_t     = g_min * sigmoid(exp(A_h) * z_t),  g_min = -5,  alpha_t = exp(g_t)
 *   S_t     = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t     = S_t^T q_t
 * -- devpress K3 technical-report walk-through §3.1 (Eq 1) and §3.2 (Eq 5);
 *    "Kimi K3：架构、训练与推理系统研究" §3.1-3.2; "Hybrid KDA–MLA：Kimi K3
 *    注意力机制解析" (core update and decay design).  No query scale is
 *    applied; q and k are expected to be L2-normalised by the caller (the
 *    feature path of "Kimi K3：架构、训练与推理系统研究" §3.2 ends in an
 *    L2Norm), which is not checked.
 *
 * Two entry points, matching the two execution paths the pages describe
 * ("Kimi K3：架构…" §14: chunked kernel for prompts, fused recurrent kernel
 * for cached single-token decode; §11.1-11.2: prefill saves the final
 * states, decode updates them in place):
 *   kda_prefill  packed variable-length sequences, chunkwise-parallel inside
 *                64-token chunks, state carried serially between chunks;
 *   kda_decode   one new token per sequence, state updated in place.
 *
 * Layouts (all row-major, all device memory unless noted):
 *   q, k, z      [T][H][dk]          v, o  [T][H][dv]
 *   beta         [T][H]  fp32, used as given (already passed through sigmoid)
 *   A            [H]     fp32 per-head log-scale
 *   z            fp32 decay logits (raw, before the gate)
 *   states       [N][H][dv][dk] fp32: element (n, h, j, i) is S_{i,j}
 *                (row j = value channel, contiguous over key channels; the
 *                [B,H,V,K] state shape of "Kimi K3：架构…" §13.1)
 *   cu_seqlens   [N+1] int32, cu[0] = 0, non-decreasing, cu[N] = T
 * The io dtype applies to q, k, v and o; z, A, beta and all states are fp32.
 *
 * Supported: dk == dv in {32, 64, 128}; io dtype KDA_BF16 or KDA_F32.
 * All pointers must be 16-byte aligned.  Every call is asynchronous on
 * `stream` (a hipStream_t; NULL is the default stream), never synchronises
 * the host and never throws.  The library keeps no pointer after a call
 * returns and allocates no device memory in these calls.
 *
 * Return value: KDA_OK (0) or a negative kda_status.  On an error the call
 * launches nothing and leaves every output untouched, except KDA_ERR_HIP,
 * which reports a failed launch (outputs then undefined).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_dtype {
    KDA_BF16 = 0, /* bfloat16 q, k, v, o; bf16 MFMA with split-precision operands */
    KDA_F32 = 1   /* fp32 q, k, v, o; fp32 MFMA throughout */
} kda_dtype;

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = -1,     /* negative size, bad cu_seqlens size, ... */
    KDA_ERR_NULL_POINTER = -2,         /* a required pointer is NULL */
    KDA_ERR_UNSUPPORTED_DIM = -3,      /* dk != dv or d not in {32, 64, 128} */
    KDA_ERR_UNSUPPORTED_DTYPE = -4,    /* io dtype not KDA_BF16 / KDA_F32 */
    KDA_ERR_MISALIGNED = -5,           /* a pointer is not 16-byte aligned */
    KDA_ERR_WORKSPACE_TOO_SMALL = -6,  /* workspace_bytes < kda_prefill_workspace_size */
    KDA_ERR_HIP = -7,                  /* a kernel launch failed */
    KDA_ERR_ALIAS = -8,                /* an output overlaps an input it may not alias */
    KDA_ERR_SCRATCH_TOO_SMALL = -9     /* kda_prefill_noalloc: the sizes need more workspace
                                          than KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

/*
 * Per-call options of kda_prefill_ex and kda_prefill_backward.  A NULL
 * options pointer, or a zero-initialised struct, means the defaults.
 *
 * segments: intra-device context parallelism ("Kimi K3：架构、训练与推理系统
 *   研究" §11.1, and the devpress K3 technical-report walk-through §8.1: a
 *   planner splits one sequence over a device's compute units; the pieces'
 *   state transitions are computed without the incoming state and merged
 *   exactly).  The prefill may cut each sequence into up to P segments of
 *   consecutive 64-token chunks.  For every segment but a sequence's last it
 *   computes the affine map S_in -> M S_in + S~ of its chunks (M in
 *   R^{dk x dk}, S~ in R^{dk x dv}), composes the maps in order from h0 (the
 *   merge S = S~ + M S_in of the KCP scheme, devpress walk-through §8.1,
 *   Eq 17), and then runs every segment's outputs from its own incoming state
 *   in parallel.  The result equals the unsplit recurrence up to rounding.
 *     0  automatic (default): split only when the workgroups of one pass
 *        would fill less than half of the device (few sequences times heads,
 *        long sequences); kda_prefill_segments reports the choice
 *     1  never split
 *     2..KDA_MAX_PREFILL_SEGMENTS  split every sequence of at least that many
 *        chunks into that many segments (shorter ones into one per chunk)
 *
 * checkpoint_interval, checkpoints, checkpoint_offsets: state checkpoints
 *   for prefix reuse ("Kimi K3：架构…" §12.2: KDA checkpoints are large, so
 *   they are kept at a coarser grain than the token hash blocks, e.g. at
 *   512-token endpoints; the s1mplewind "kimi-k3" notes, "KDA存checkpoint").
 *   Prefill only; all three must be zero / NULL for the backward.
 *     checkpoint_interval  tokens between checkpoints, a positive multiple of
 *                          64 (ignored when both pointers are NULL)
 *     checkpoints          [T / interval][H][dv][dk] fp32 device buffer or
 *                          NULL (T / interval rounded down: an upper bound on
 *                          the count for any cu_seqlens); checkpoint j of
 *                          sequence n is the state after the first
 *                          (j + 1) * interval tokens of the sequence (h0
 *                          included), for j < floor(len_n / interval), stored
 *                          at index checkpoint_offsets[n] + j; sequence-major
 *     checkpoint_offsets   [N + 1] int32 device buffer or NULL: first
 *                          checkpoint index of every sequence, then the total
 *   Entries past the total are left untouched; checkpoints and offsets may
 *   overlap no other argument.
 *
 * blocks: the chunk-block pipeline of the bf16 prefill (the pages' kernel
 *   overlaps intra-chunk work with the serial state propagation: devpress
 *   walk-through §8.1; "Kimi K3：架构…" §13.1).  The chunk table is cut into
 *   `blocks` runs of consecutive chunks; the intra-chunk kernel of run j + 1
 *   runs on the caller's stream beside the inter-chunk kernel of run j on a
 *   helper stream of the calling thread (created on its first pipelined call,
 *   default priority, kept until the process ends), and a sequence's state
 *   crosses run boundaries through the workspace.  Events order the two
 *   streams, and the call is still asynchronous on `stream` and may be
 *   captured in a graph.  The outputs are bit-identical to blocks = 1.
 *     0  automatic (default): on the bf16 path without segments or
 *        checkpoints, when the chain's workgroups leave CUs free for the
 *        intra kernel and the sequences are long (three runs; six in the
 *        fused prefill), or when at least 16 sequences average at least 128
 *        chunks (four runs: the next run fills the CUs that the chain's
 *        longest sequences leave idle); the fused prefill pipelines at the
 *        same sizes
 *     1  off
 *     2..KDA_MAX_PREFILL_BLOCKS  that many runs (with segments = 0 the
 *        segment count is then 1; with segments >= 2 the call is rejected);
 *        ignored, segments included, on the fp32 path and with checkpoints;
 *        ignored by the backward
 */
#define KDA_MAX_PREFILL_SEGMENTS 16
#define KDA_MAX_PREFILL_BLOCKS 16
typedef struct kda_prefill_options {
    int segments;
    int checkpoint_interval;
    float *checkpoints;
    int32_t *checkpoint_offsets;
    int blocks;
} kda_prefill_options;

/*
 * Workspace bytes kda_prefill needs for these sizes (automatic segments).
 * Depends only on the arguments (an upper bound over every cu_seqlens with
 * N sequences and T tokens) and the current device's compute-unit count.
 * Returns 0 for sizes kda_prefill would reject.
 */
size_t kda_prefill_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype);

/*
 * The same for kda_prefill_ex with these options (NULL: the defaults).
 * Returns 0 for sizes or options kda_prefill_ex would reject.
 */
size_t kda_prefill_ex_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                     const kda_prefill_options *options);

/*
 * The segment count a prefill with options.segments = 0 uses for these
 * sizes on the current device (>= 1), or 0 for sizes it would reject.
 */
int kda_prefill_segments(int N, int T, int H, int dk, int dv, kda_dtype io_dtype);

/*
 * Chunkwise prefill over N packed sequences (T tokens in total).
 *
 *   q, k, v      inputs, io dtype (layouts above)
 *   z, A, beta   fp32 gate inputs
 *   h0           [N][H][dv][dk] initial states, or NULL for zeros
 *   cu_seqlens   [N+1] int32 device array; sequence n is tokens
 *                [cu[n], cu[n+1]); its chunks of 64 start at cu[n], the last
 *                one may be partial; a zero-length sequence gives hT = h0
 *   o            [T][H][dv] output, io dtype
 *   hT           [N][H][dv][dk] final states, or NULL to skip; may be the
 *                same pointer as h0 (each block reads its slice of h0 before
 *                writing that slice of hT), but must not overlap it otherwise
 *   workspace    device scratch of at least kda_prefill_workspace_size(...)
 *                bytes, 256-byte aligned, owned by the caller; contents on
 *                entry are ignored, on return undefined.  The call uses it
 *                until its work on `stream` completes: calls in flight at the
 *                same time need workspaces of their own.  A pipelined call's
 *                chain runs on a helper stream of the calling thread, so two
 *                pipelined calls from one thread run their chains one after
 *                the other, whatever streams they were given
 *
 * cu_seqlens content is not read on the host.  With KDA_DEBUG_CHECK_CU=1 in
 * the environment the call copies it to the host, synchronises `stream`
 * and returns KDA_ERR_INVALID_ARGUMENT if it is not a valid prefix sum.
 */
int kda_prefill(kda_dtype io_dtype, const void *q, const void *k, const void *v,
                const float *z, const float *A, const float *beta, const float *h0,
                const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, void *o,
                float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill with per-call options (segments, checkpoints; see
 * kda_prefill_options).  The workspace must hold
 * kda_prefill_ex_workspace_size(..., options) bytes.  Invalid options return
 * KDA_ERR_INVALID_ARGUMENT.  With options NULL this is kda_prefill.
 */
int kda_prefill_ex(kda_dtype io_dtype, const void *q, const void *k, const void *v,
                   const float *z, const float *A, const float *beta, const float *h0,
                   const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, void *o,
                   float *hT, const kda_prefill_options *options, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * The fused prefill: the feature path, the chunkwise prefill and the output
 * gate in one call, with o never written to memory ("Kimi K3：架构、训练与推理
 * 系统研究" §13.2: the production kernel fuses ShortConv, the input norms, the
 * gate, the KDA recurrence and the output norm, so that the large state and
 * its inputs make fewer HBM round trips; §3.2 and §3.3 define the pieces, as
 * do kda_qkv_shortconv and kda_output_gate below).  The gate is applied where
 * the inter-chunk kernel stores o.  The feature path runs inside the
 * intra-chunk kernel, except where the call is pipelined (see
 * kda_prefill_options.blocks): there it runs as a pass of its own that
 * stages q, k, v in the workspace, which is faster on this device.  It computes
 *   q, k, v = kda_qkv_shortconv(xq, xk, xv, wq, wk, wv, conv_state_in)
 *   o, hT   = kda_prefill(q, k, v, z, A, beta, h0, cu_seqlens)
 *   y       = kda_output_gate(o, gate, norm_weight, eps)
 * with q, k, v rounded to bf16 as kda_qkv_shortconv delivers them, and o kept
 * in fp32 up to the gate (only y is rounded).  conv_state_out, when given,
 * receives the window after the call and may be conv_state_in.
 *
 *   io_dtype         KDA_BF16 only (KDA_ERR_UNSUPPORTED_DTYPE otherwise)
 *   xq, xk, xv ... conv_state_out   as for kda_qkv_shortconv
 *   z .. dv          as for kda_prefill (dk == dv)
 *   gate             [T][H][dv] bf16 gate projection g;  norm_weight [dv] fp32
 *   y                [T][H][dv] bf16 output;  hT as for kda_prefill
 *   workspace        kda_prefill_fused_workspace_size(N, T, H, dk, dv, KDA_BF16, NULL) bytes
 * Outputs may overlap no input (except the window in place) and no other
 * output.  Errors and asynchrony as for kda_prefill.
 */
int kda_prefill_fused(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                      const float *wk, const float *wv, const void *conv_state_in, void *conv_state_out,
                      const float *z, const float *A, const float *beta, const float *h0,
                      const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, const void *gate,
                      const float *norm_weight, float eps, void *y, float *hT, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * kda_prefill_fused with per-call options (NULL: the defaults, which is
 * kda_prefill_fused): the segment count and the chunk-block pipeline as for
 * kda_prefill_ex.  Checkpoints are not available here (the gated output pass
 * stores no states): a non-NULL checkpoint pointer or a non-zero
 * checkpoint_interval gives KDA_ERR_INVALID_ARGUMENT.  The workspace is
 * kda_prefill_fused_workspace_size(N, T, H, dk, dv, KDA_BF16, options) bytes.
 * For any blocks >= 2 the outputs are bit for bit the same; with blocks = 1
 * (the feature path inside the intra kernel) q and k may differ from the
 * feature kernel's in the last bit, from the order of the L2 norm's sum.
 */
int kda_prefill_fused_ex(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                         const float *wk, const float *wv, const void *conv_state_in, void *conv_state_out,
                         const float *z, const float *A, const float *beta, const float *h0,
                         const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, const void *gate,
                         const float *norm_weight, float eps, void *y, float *hT,
                         const kda_prefill_options *options, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Workspace bytes of kda_prefill_fused_ex with these options (NULL: the
 * defaults, kda_prefill_fused): kda_prefill_ex_workspace_size's, plus
 * 3 T H dk bf16 values where the call is pipelined (the staged q, k, v).
 * Returns 0 for sizes or options the call would reject.
 */
size_t kda_prefill_fused_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                        const kda_prefill_options *options);

/*
 * kda_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are kda_prefill's (automatic segments),
 * without the workspace: the call uses a device array of
 * KDA_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds on every GPU it
 * runs on until the process ends, and calls no allocating routine.  Sizes
 * whose workspace (kda_prefill_workspace_size) exceeds the array return
 * KDA_ERR_SCRATCH_TOO_SMALL and launch nothing; 256 MiB holds, for example,
 * a 1024-token chunk of a 96-head prefill at d = 128, or 8 heads x 16384
 * tokens.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (two streams, or two threads without ordering) race and
 * give undefined results.  Nothing in the array needs clearing between calls.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int kda_prefill_noalloc(kda_dtype io_dtype, const void *q, const void *k, const void *v,
                        const float *z, const float *A, const float *beta, const float *h0,
                        const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, void *o,
                        float *hT, void *stream);

/*
 * One decode step for N sequences, one token each.
 *
 *   q, k         [N][H][dk] io dtype;  v [N][H][dv] io dtype
 *   z            [N][H][dk] fp32;  A [H] fp32;  beta [N][H] fp32
 *   S_inout      [N][H][dv][dk] fp32 state, read once and overwritten once
 *   o            [N][H][dv] output, io dtype
 *
 * Each (sequence, head) state is read from HBM exactly once and written
 * back exactly once ("Kimi K3：架构…" §11.4 and §13.2: a decode step costs
 * one full read and write of the state).
 */
int kda_decode(kda_dtype io_dtype, const void *q, const void *k, const void *v,
               const float *z, const float *A, const float *beta, float *S_inout, int N,
               int H, int dk, int dv, void *o, void *stream);

/*
 * The fused decode step: the feature path of the new token, one decode step
 * and the output gate in one pass over the state ("Kimi K3：架构、训练与推理
 * 系统研究" §13.2: the production decode kernel runs ShortConv, the input
 * norms, the gate, the KDA recurrence and the output norm in one recurrent
 * loop; §3.2–3.4 define the pieces).  For N sequences with one token each it
 * computes
 *   q, k, v = kda_qkv_shortconv(xq, xk, xv, wq, wk, wv, conv_state_in)   (T = N)
 *   o       = kda_decode(q, k, v, z, A, beta, S_inout)
 *   y       = kda_output_gate(o, gate, norm_weight, eps)
 * with q, k, v and o kept in fp32 (kda_qkv_shortconv and kda_decode hand them
 * over in bf16; here only y is rounded).
 *
 *   io_dtype         KDA_BF16 only (KDA_ERR_UNSUPPORTED_DTYPE otherwise)
 *   xq, xk, xv       [N][H][d] bf16 pre-convolution projections of the token
 *   wq, wk, wv       [H][d][4] fp32 ShortConv taps (tap 3 on the new token)
 *   conv_state_in    [N][3][H][3 d] bf16 carried window (q | k | v channels,
 *                    oldest token first), or NULL for zeros
 *   conv_state_out   the window after this token, or NULL; may be
 *                    conv_state_in (updated in place), else must not overlap it
 *   z, A, beta       as for kda_decode;  S_inout [N][H][d][d] fp32, in place
 *   gate             [N][H][d] bf16 gate projection g;  norm_weight [d] fp32
 *   eps              RMSNorm epsilon, >= 0
 *   dk == dv == d    32, 64 or 128
 *   y                [N][H][d] bf16 output
 * Outputs (y, S_inout, conv_state_out) may overlap no input and no other
 * output, except the window in place (KDA_ERR_ALIAS).  Pointers 16-byte
 * aligned.  Asynchronous on `stream`; N = 0 launches nothing.
 */
int kda_decode_fused(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv,
                     const float *wq, const float *wk, const float *wv, const void *conv_state_in,
                     void *conv_state_out, const float *z, const float *A, const float *beta,
                     float *S_inout, const void *gate, const float *norm_weight, float eps, int N,
                     int H, int dk, int dv, void *y, void *stream);

/*
 * Multi-token decode with replay (speculative decoding).  A state updated in
 * place cannot be rolled back when draft tokens are rejected; instead the
 * caller keeps the committed state and the small per-token inputs of the
 * draft window, and once the verifier has decided, the accepted tokens are
 * replayed on chip in the same pass that runs the next window ("Kimi K3：
 * 架构…" §11.3 and §13.2: projected inputs cached, accepted tokens replayed,
 * replay + bonus token + next draft window merged into one decode loop).
 *
 * Per sequence n and head, in one pass over the state:
 *   1. the first a = clamp(n_accept[n], 0, Lr) tokens of the replay window
 *      advance S_inout (no outputs);
 *   2. that state is written back to S_inout (the committed state);
 *   3. the L tokens of the new window advance a copy of it and produce
 *      o_t = S_t^T q_t for every window token; the copy is dropped, or, when
 *      commit_window is 1, written back instead of the state of step 2.
 * The state is read once and written at most once per call (not at all when
 * a = 0 and commit_window is 0).
 *
 *   rk, rv, rz, rbeta   replay window [N][Lr][H][dk or dv] (io dtype for rk,
 *                       rv; fp32 rz; rbeta [N][Lr][H] fp32): the k, v, z,
 *                       beta passed as the window of the previous call
 *   n_accept            [N] int32 device array, accepted replay tokens
 *   q, k, v, z, beta    new window [N][L][H][...], same dtypes as kda_decode
 *   A                   [H] fp32;  S_inout [N][H][dv][dk] fp32
 *   o                   [N][L][H][dv] io dtype
 *   0 <= Lr, L <= KDA_MAX_DECODE_WINDOW; pointers of an empty window may be
 *   NULL.  Lr = 0, L = 1, commit_window = 1 is one kda_decode step.
 */
#define KDA_MAX_DECODE_WINDOW 16
int kda_decode_window(kda_dtype io_dtype, const void *rk, const void *rv, const float *rz,
                      const float *rbeta, const int32_t *n_accept, int Lr, const void *q,
                      const void *k, const void *v, const float *z, const float *beta, int L,
                      const float *A, float *S_inout, int N, int H, int dk, int dv, void *o,
                      int commit_window, void *stream);

/*
 * The q/k/v feature path ("Kimi K3：架构…" §3.2; devpress K3 walk-through
 * §3.1):  q = L2Norm(Swish(ShortConv(xq))), k = L2Norm(Swish(ShortConv(xk))),
 * v = Swish(ShortConv(xv)), with Swish(u) = u * sigmoid(u) and the L2 norm over
 * each (token, head) row.  ShortConv is a causal depthwise convolution over the
 * tokens of each sequence with 4 taps per channel:
 *   c_t = w[0] x_{t-3} + w[1] x_{t-2} + w[2] x_{t-1} + w[3] x_t,
 * where positions before the sequence's first token read the carried window.
 *
 *   xq, xk, xv         [T][H][d] io dtype: the projected inputs W_q x, W_k x, W_v x
 *   wq, wk, wv         [H][d][4] fp32 taps
 *   cu_seqlens         [N+1] int32 device array, as for kda_prefill
 *   conv_state_in      [N][3][H][3d] io dtype or NULL (zeros): per sequence the
 *                      last three pre-convolution tokens before it, oldest
 *                      first, channels [xq | xk | xv]
 *   conv_state_out     same shape or NULL: the window after the sequence (the
 *                      last three tokens of [window, sequence]); may be
 *                      conv_state_in itself
 *   q, k, v            [T][H][d] io dtype outputs, ready for kda_prefill; for a
 *                      decode step use T = N and cu_seqlens = 0, 1, ..., N
 * dk == dv in {32, 64, 128}.  Outputs may overlap no input (except the state
 * in place) and no other output.
 */
int kda_qkv_shortconv(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv,
                      const float *wq, const float *wk, const float *wv,
                      const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv,
                      const void *conv_state_in, void *conv_state_out, void *q, void *k,
                      void *v, void *stream);

/*
 * The output gate ("Kimi K3：架构…" §3.3; devpress §3.3, Eq 6):
 *   y = Sigmoid(g) * RMSNorm(o),  RMSNorm(o) = o / sqrt(mean(o^2) + eps) * w
 * per (token, head) row of dv channels.  g is the gate projection W_g x.
 *
 *   o, g, y     [T][H][dv] io dtype; y may be o or g (in place)
 *   w           [dv] fp32 weight, shared by the heads;  eps >= 0
 * The final projection W_o is not part of the op.
 */
int kda_output_gate(kda_dtype io_dtype, const void *o, const void *g, const float *w, float eps,
                    int T, int H, int dv, void *y, void *stream);

/*
 * Gradients of the chunkwise prefill, for training.  The pages give the
 * forward recurrence and its chunk form (the s1mplewind "kimi-k3" notes,
 * "Chunkwise 形式"; "Kimi K3：架构…" §3.1) and note that training keeps
 * per-head intermediate states (the "分析" part of the same notes); they give
 * no backward formula.  This call returns the exact reverse-mode gradients of
 *   L = sum(grad_o * o) + sum(grad_hT * hT)
 * with o, hT = kda_prefill(q, k, v, z, A, beta, h0, cu_seqlens), obtained by
 * differentiating the chunk form as matrices: it runs the forward prefill
 * again, keeping the state at every 64-token chunk boundary, then walks each
 * sequence's chunks backwards carrying dL/dS, then computes every input
 * gradient per (chunk, head).  Arithmetic after the forward recompute is fp32.
 *
 *   q .. cu_seqlens, N .. dv   as for kda_prefill (the same inputs)
 *   options     NULL or options with only `segments` set (the forward
 *               recompute's segment split); sized by the same pointer
 *   grad_o      [T][H][dv] io dtype
 *   grad_hT     [N][H][dv][dk] fp32, or NULL for zeros
 *   grad_q, grad_k, grad_z   [T][H][dk] fp32;  grad_v [T][H][dv] fp32
 *   grad_beta   [T][H] fp32;  grad_A [H] fp32 (summed over every token,
 *               in a fixed order: the result does not vary between runs)
 *   grad_h0     [N][H][dv][dk] fp32 (state layout), or NULL to skip
 *   workspace   at least kda_prefill_backward_workspace_size(...) bytes,
 *               256-byte aligned; contents on entry ignored, on return undefined
 * Outputs may overlap no input, no other output and the workspace
 * (KDA_ERR_ALIAS).  Errors and asynchrony as for kda_prefill.
 */
size_t kda_prefill_backward_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                           const kda_prefill_options *options);
int kda_prefill_backward(kda_dtype io_dtype, const void *q, const void *k, const void *v,
                         const float *z, const float *A, const float *beta, const float *h0,
                         const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv,
                         const void *grad_o, const float *grad_hT, float *grad_q, float *grad_k,
                         float *grad_v, float *grad_z, float *grad_beta, float *grad_A,
                         float *grad_h0, const kda_prefill_options *options, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Static, human-readable text for a kda_status value. */
const char *kda_status_string(int status);

/* Static build description (target, chunk size, library version). */
const char *kda_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
