/*
 * gdn.h -- C ABI of libgdn: the Gated DeltaNet layer core on AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (the oxydllm 0.0.0-alpha.12.2 release notes, "New Features",
 * Gated DeltaNet runtime) keeps, per sequence and v-head, a d_k x d_v fp32
 * memory S and for every token t does
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,          alpha_t = exp(g_t),
 *
 * (S stored [d_k][d_v]; this is the usual d_v x d_k formulation transposed).
 * Prefill runs it as a chunked parallel scan, decode as an O(1) recurrent
 * step; a short causal depthwise convolution (+SiLU) produces q, k, v from
 * the projected activations (Vallmo.jl README, "What's here": causal conv1d
 * and the fused/recurrent DeltaNet paths are the hybrid layer's kernels).
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers, allocated and owned by the
 *    caller.  The library never allocates device memory; scratch space is
 *    the caller's `workspace` (size from gdn_prefill_workspace_size).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  It returns once the work is queued.  Host-side
 *    validation happens first: a call that returns an error other than
 *    GDN_ERR_HIP has queued nothing and touched no memory.
 *  - Layouts are token-major and row-major:
 *      q, k   [N_tok][H_k][d_k]   (token stride stride_q / stride_k elements)
 *      v      [N_tok][H_v][d_v]   (token stride stride_v)
 *      o      [N_tok][H_v][d_v]   (packed)
 *      g,beta [N_tok][H_v]        fp32 (log-decay and write strength)
 *      state  [N_seq][H_v][d_k][d_v] fp32
 *    q/k/v/o/conv tensors are fp32 or bf16 (gdn_dims.dtype); gates and
 *    states are always fp32 (the same notes: DeltaNet scalar parameters
 *    stay F32 end to end).
 *  - Pointers to bf16/fp32 tensors must be 16-byte aligned and token strides
 *    multiples of 8 elements (bf16) or 4 (fp32), so rows load as 128-bit words.
 *  - Errors: a gdn_status; gdn_last_error() gives a message for the calling
 *    thread.  If the environment has GDN_DEBUG=1 the library also
 *    synchronises after each call and scans outputs for NaN/Inf
 *    (GDN_ERR_NONFINITE), in the spirit of the per-stage NaN/Inf probe the
 *    oxydllm notes list under "GDN debug aids".
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* bad shape, null pointer, misalignment, bad flag */
    GDN_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim 96) */
    GDN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = 4,         /* a HIP runtime call failed */
    GDN_ERR_NONFINITE = 5    /* GDN_DEBUG=1 only: NaN/Inf found in an output */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

enum {
    /* q and k are L2-normalised per head before use: x / sqrt(|x|^2 + 1e-6). */
    GDN_QK_L2NORM = 1u,
    /* v-head h reads q/k head (h % H_k) -- the tiled V-head order that GGUF
     * files use (oxydllm notes, "GGUF qwen35 architecture").  Default: head
     * h / (H_v / H_k), the repeat-interleave order. */
    GDN_HEADS_TILED = 2u
};

/* Problem description shared by the scan entry points. */
typedef struct gdn_dims {
    int32_t num_seqs;     /* N >= 1 */
    int32_t total_tokens; /* N_tok = sum of sequence lengths (>= 0) */
    int32_t seqlen;       /* > 0: every sequence has this length (dense, N_tok = N*seqlen);
                             0: lengths come from cu_seqlens (varlen) */
    int32_t num_qk_heads; /* H_k >= 1 */
    int32_t num_v_heads;  /* H_v, a multiple of H_k */
    int32_t head_dim_k;   /* d_k in {64, 128} */
    int32_t head_dim_v;   /* d_v in {64, 128} (d_k != d_v allowed) */
    int32_t chunk_size;   /* prefill chunk C in {16, 32, 64}; ignored by decode */
    int32_t dtype;        /* gdn_dtype of q, k, v, o */
    uint32_t flags;       /* GDN_QK_L2NORM | GDN_HEADS_TILED */
    float scale;          /* multiplies q (after the L2 norm, if any) */
    int32_t reserved;     /* must be 0 */
    int64_t stride_q;     /* elements between consecutive tokens of q; 0 = H_k*d_k */
    int64_t stride_k;     /* same for k; 0 = H_k*d_k */
    int64_t stride_v;     /* same for v; 0 = H_v*d_v */
} gdn_dims;

/*
 * The gates' raw inputs, for the calls that compute g and beta themselves
 * (see gdn_gating for the map): the decay and beta projections a, b
 * [N_tok][H_v] in the problem's dtype with token strides stride_a, stride_b
 * (elements, >= H_v; they may be column blocks of one projection output),
 * aligned to their element size, and the fp32 per-head A_log, dt_bias [H_v].
 */
typedef struct gdn_gate_inputs {
    const void *a;
    int64_t stride_a;
    const void *b;
    int64_t stride_b;
    const float *A_log;
    const float *dt_bias;
} gdn_gate_inputs;

/* Human-readable name of a status code (static storage). */
const char *gdn_status_string(gdn_status s);

/* Message describing the most recent error on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* Library version, e.g. "0.1.0". */
const char *gdn_version(void);

/*
 * Host-only check of a problem description, no GPU needed: the shape rules
 * the entry points apply before queuing anything.  The shapes are those of
 * the layer as the oxydllm notes describe it ("New Features": a per-head
 * d_k x d_v fp32 memory, grouped q/k heads shared by several v-heads, in
 * repeat-interleave or tiled order); head dims 64 and 128 and chunks of 16,
 * 32 or 64 are the ones this library implements.  op: 0 = prefill,
 * 1 = decode.  Returns GDN_OK or the status the entry points would return.
 */
gdn_status gdn_validate_dims(const gdn_dims *d, int32_t op);

/*
 * Host-only check of a whole call, no GPU needed: exactly the checks that
 * gdn_prefill_chunked (op 0) or gdn_decode_step (op 1) run before queuing
 * anything -- shapes, NULL pointers, 16-byte alignment, state overlap and
 * workspace size -- with the pointers only compared, never dereferenced.
 * ptrs holds the call's pointer arguments in the order of its signature:
 *   op 0: q, k, v, g, beta, state_in, cu_seqlens, o, state_out, workspace
 *         (n_ptrs = 10); extent = the workspace size in bytes;
 *   op 1: q, k, v, g, beta, state, state_slots, o (n_ptrs = 8);
 *         extent = num_slots.
 * Returns what the entry point would return for these arguments had the
 * GPU accepted the launch (GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED
 * or GDN_ERR_WORKSPACE); gdn_last_error() says why.
 */
gdn_status gdn_validate(const gdn_dims *d, int32_t op, const void *const *ptrs, int32_t n_ptrs,
                        int64_t extent);

/*
 * Causal depthwise conv1d (+ optional SiLU) over packed sequences: the short
 * convolution that produces the layer's q, k and v (Vallmo.jl README,
 * "What's here": causal conv1d is one of the hybrid layer's kernels; PicoLM
 * fork changelog, "GPU: Device-Native Pipeline Rewrite": conv1d runs as its
 * own device kernel), with the per-sequence causal-conv window the oxydllm
 * notes ("New Features") keep beside the recurrent memory.
 *
 * For sequence i and channel c, with x_i its tokens and w[c][0..W-1]:
 *     y[t][c] = act( bias[c] + sum_{j=0}^{W-1} w[c][j] * xx[t - (W-1) + j][c] )
 * where positions before the sequence start read the conv window
 * conv_state[i][W-1 + pos][c] (slot W-2 is the newest), or zero when
 * conv_state is NULL.  Tap W-1 multiplies the current token.  act is SiLU,
 * a / (1 + e^{-a}), when activation == 1, identity when 0.  The sum is
 * evaluated in fp32 as acc = bias (or 0), acc = fma(w_j, x_j, acc) for j = 0..W-1,
 * with one fixed exponential, so results are bit-reproducible; bf16 outputs
 * are rounded to nearest even.
 *
 * num_seqs, total_tokens, seqlen, cu_seqlens: as in gdn_dims (cu_seqlens is
 * a device int32[N+1] array, required iff seqlen == 0).
 * channels: C; width: W in [2, 8]; dtype: of x, y and conv_state.
 * x: [N_tok] rows with token stride stride_x (>= C); y: [N_tok][C] rows
 * with stride stride_y (>= C).  weight: fp32 [C][W]; bias: fp32 [C] or NULL.
 * conv_state: [N][W-1][C] in dtype, in/out, or NULL: on return it holds the
 * last W-1 raw inputs of (old window ++ sequence), ready for the next call.
 * x, y and conv_state must not overlap one another (GDN_ERR_INVALID_ARG).
 * A sequence with zero tokens leaves its window unchanged.  With
 * seqlen == 1 this is the decode-time conv step.
 */
gdn_status gdn_conv1d(int32_t num_seqs, int32_t total_tokens, int32_t seqlen,
                      const int32_t *cu_seqlens, int32_t channels, int32_t width,
                      int32_t dtype, const void *x, int64_t stride_x,
                      const float *weight, const float *bias, void *conv_state,
                      int32_t activation, void *y, int64_t stride_y, void *stream);

/*
 * Device workspace (bytes) that gdn_prefill_chunked / gdn_prefill_prepare /
 * gdn_prefill_scan need for this problem: per chunk and v-head the inverse
 * Tt and room for the score matrix P (both C x C in the q/k/v dtype) and
 * eight C-vectors of fp32 per-token factors, plus the chunk table for varlen
 * input; for bf16 with chunk 32 or 64 also, per carry segment and v-head,
 * an fp32 start state and a bf16 d_k x d_k transition (and, for varlen
 * input, a segment table with the order in which the carry takes the
 * segments).  0 on invalid dims (gdn_last_error says why).
 */
size_t gdn_prefill_workspace_size(const gdn_dims *d);

/*
 * Chunked prefill of the gated delta rule (the chunked parallel scan of the
 * oxydllm notes, "New Features"), for N sequences packed along tokens.
 *
 * q, k, v, g, beta: see the layout table above.  state_in: fp32
 * [N][H_v][d_k][d_v] or NULL (zero state).  cu_seqlens: device int32 [N+1]
 * (required iff d->seqlen == 0; each sequence is chunked from its own
 * start).  o: [N_tok][H_v][d_v] in dtype.  state_out: fp32
 * [N][H_v][d_k][d_v] or NULL (discarded); it may alias state_in exactly.
 * workspace: >= gdn_prefill_workspace_size(d) bytes, 256-byte aligned.
 *
 * The result equals the token recurrence above up to rounding: per chunk,
 * the unit-lower-triangular system (I + A) is inverted blockwise (a
 * doubling product on 16x16 diagonal blocks, then pairwise merging of
 * blocks -- the oxydllm notes' remedy for fp32 overflow of plain doubling
 * on repeated tokens), the state-independent products are formed per chunk,
 * and the state is carried across chunks sequentially in fp32.
 * Equivalent to gdn_prefill_prepare followed by gdn_prefill_scan.
 */
gdn_status gdn_prefill_chunked(const gdn_dims *d, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const float *state_in, const int32_t *cu_seqlens,
                               void *o, float *state_out, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is instead a 64 MiB
 * device array inside the library (one per GPU, held until the process
 * ends; it fits the 4096-token layer with 16 q/k and 32 v-heads of 128 in
 * bf16, which needs 62.9 MB).  Problems whose gdn_prefill_workspace_size
 * exceeds 64 MiB return GDN_ERR_UNSUPPORTED before any HIP call.  Allocates
 * nothing and frees nothing.  Every call on one GPU shares that GPU's array
 * (each call writes every workspace byte it reads, so no clearing is
 * needed): calls that overlap in time on one GPU -- on different streams,
 * or from different host threads -- race and must not be issued.  The
 * first call on a device looks the array's address up (a HIP runtime
 * query, no allocation).  Arguments and results as gdn_prefill_chunked.
 */
gdn_status gdn_prefill_chunked_noalloc(const gdn_dims *d, const void *q, const void *k,
                                       const void *v, const float *g, const float *beta,
                                       const float *state_in, const int32_t *cu_seqlens,
                                       void *o, float *state_out, void *stream);

/*
 * Phase 1 of the prefill: everything that does not depend on the carried
 * state (the oxydllm notes, "Performance": the cross-chunk loop precomputes
 * all state-independent work in batch).  For every chunk and v-head it
 * writes into the workspace Tt = (I + A)^{-1} diag(beta), the causal score
 * matrix P[r][s] = e^{gamma_r - gamma_s} q_hat_r . k_hat_s (s <= r) and the
 * per-token scale factors; fully parallel over chunks.  Tt and P are kept
 * as their nonzero (lower) 16x16 blocks only.  For bf16 with chunk 32 or 64
 * the carry forms P itself from q and k, so P is not written.  The
 * workspace layout is private to the library.  Arguments as
 * gdn_prefill_chunked.
 */
gdn_status gdn_prefill_prepare(const gdn_dims *d, const void *q, const void *k,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * Phase 2 of the prefill: the sequential carry over chunks, reading the
 * workspace written by gdn_prefill_prepare for the same inputs, and writing
 * o and state_out.  Arguments as gdn_prefill_chunked.
 */
gdn_status gdn_prefill_scan(const gdn_dims *d, const void *q, const void *k,
                            const void *v, const float *g, const float *beta,
                            const float *state_in, const int32_t *cu_seqlens,
                            void *o, float *state_out, const void *workspace,
                            size_t ws_bytes, void *stream);

/*
 * The prefill's carry (gdn_prefill_scan) with the gated RMS norm on the
 * layer's output fused into it (the oxydllm notes, "Performance": the Gated
 * DeltaNet's gated norm runs as a fused kernel): instead of o it writes
 *     y[t][h][j] = norm_weight[j] * o[t][h][j] / sqrt(mean_i o[t][h][i]^2 + eps)
 *                  * silu(z[t][h][j]),   silu(a) = a / (1 + e^-a),
 * the map of gdn_gated_rmsnorm, with o rounded to the problem's dtype first
 * (what gdn_gated_rmsnorm would read).  For bf16 with chunk 32 or 64 the
 * norm runs inside the carry kernel, so o never goes through memory; other
 * problems run the carry into y and then the norm in place.  The result
 * equals gdn_prefill_scan followed by gdn_gated_rmsnorm within rounding
 * (the row sums are added in another order).
 *
 * z: [N_tok][H_v][d_v] in the problem's dtype, token stride stride_z
 * (elements, >= H_v d_v, a multiple of 16 bytes), 16-byte aligned; the heads
 * of a token are packed.  norm_weight: fp32 [d_v], shared by all heads.
 * eps: finite, >= 0.  y: [N_tok][H_v][d_v] like o; it must not overlap z.
 * Every other argument as gdn_prefill_scan; state_out is the carry's.
 */
gdn_status gdn_prefill_scan_gated_norm(const gdn_dims *d, const void *q, const void *k,
                                      const void *v, const float *g, const float *beta,
                                      const float *state_in, const int32_t *cu_seqlens,
                                      const void *z, int64_t stride_z, const float *norm_weight,
                                      float eps, void *y, float *state_out,
                                      const void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_prefill_chunked with the gated norm fused as in
 * gdn_prefill_scan_gated_norm: gdn_prefill_prepare followed by
 * gdn_prefill_scan_gated_norm, both validated before anything is queued.
 */
gdn_status gdn_prefill_chunked_gated_norm(const gdn_dims *d, const void *q, const void *k,
                                         const void *v, const float *g, const float *beta,
                                         const float *state_in, const int32_t *cu_seqlens,
                                         const void *z, int64_t stride_z,
                                         const float *norm_weight, float eps, void *y,
                                         float *state_out, void *workspace, size_t ws_bytes,
                                         void *stream);

/*
 * Convolution and prefill phase 1 in one call: the layer's short causal
 * conv1d + SiLU (Vallmo.jl README, "What's here") over the raw projected rows
 * x, whose channels are ordered [q | k | v] (C_conv = 2 H_k d_k + H_v d_v),
 * followed by gdn_prefill_prepare on the q and k it produced.  The result is
 * exactly that of
 *     gdn_conv1d(N, N_tok, seqlen, cu_seqlens, C_conv, conv_width, dtype, x,
 *                stride_x, conv_weight, conv_bias, conv_state, 1, y, stride_y)
 *     gdn_prefill_prepare(d, y, y + H_k d_k, g, beta, cu_seqlens, workspace)
 * bit for bit (y, conv_state and the workspace); it is those two calls
 * with one validation.  Afterwards gdn_prefill_scan(d, y, y + H_k d_k,
 * y + 2 H_k d_k, ...) with the same workspace completes the prefill
 * (gdn_prefill_conv_chunked does both).
 *
 * d: the problem; its stride_q, stride_k and stride_v must all equal
 * stride_y (q, k, v are column blocks of y).  conv_width, x, stride_x,
 * conv_weight, conv_bias, conv_state: as gdn_conv1d (conv_state is read and
 * then advanced to the last conv_width-1 raw inputs of each sequence).
 * y: [N_tok] rows of C_conv channels in dtype, token stride stride_y; it
 * must not overlap x.  g, beta, cu_seqlens, workspace: as gdn_prefill_chunked.
 * Errors as gdn_prefill_prepare and gdn_conv1d; nothing is queued on error.
 */
gdn_status gdn_prefill_conv_prepare(const gdn_dims *d, int32_t conv_width,
                                    const void *x, int64_t stride_x,
                                    const float *conv_weight,
                                    const float *conv_bias, void *conv_state,
                                    const float *g, const float *beta,
                                    const int32_t *cu_seqlens, void *y,
                                    int64_t stride_y, void *workspace,
                                    size_t ws_bytes, void *stream);

/*
 * The whole prefill from raw rows: gdn_prefill_conv_prepare followed by
 * gdn_prefill_scan on the q, k, v column blocks of y, on one stream.
 * state_in, o, state_out: as gdn_prefill_chunked.  Both halves are
 * validated before anything is queued.
 */
gdn_status gdn_prefill_conv_chunked(const gdn_dims *d, int32_t conv_width,
                                    const void *x, int64_t stride_x,
                                    const float *conv_weight,
                                    const float *conv_bias, void *conv_state,
                                    const float *g, const float *beta,
                                    const float *state_in,
                                    const int32_t *cu_seqlens, void *y,
                                    int64_t stride_y, void *o, float *state_out,
                                    void *workspace, size_t ws_bytes,
                                    void *stream);

/*
 * One decode step (the O(1) recurrent step of the oxydllm notes): one new
 * token for each of d->num_seqs sequences (d->seqlen must be 1 and
 * d->total_tokens == d->num_seqs; chunk_size is ignored).
 *
 * q, k [B][H_k][d_k], v [B][H_v][d_v] (token strides from d), g, beta
 * [B][H_v] fp32, o [B][H_v][d_v].  state: fp32 [num_slots][H_v][d_k][d_v],
 * updated in place; sequence b uses slot state_slots[b] (device int32 [B])
 * or slot b when state_slots is NULL (then num_slots >= B).  Two sequences
 * must not share a slot.  A slot index outside [0, num_slots) is caught on
 * the device: that sequence's output is set to NaN and no state is touched.
 */
gdn_status gdn_decode_step(const gdn_dims *d, const void *q, const void *k,
                           const void *v, const float *g, const float *beta,
                           float *state, int32_t num_slots,
                           const int32_t *state_slots, void *o, void *stream);

/*
 * One decode step from the raw projected row: the layer's short causal
 * conv1d + SiLU (Vallmo.jl README, "What's here") for the new token, its
 * window kept per sequence as the oxydllm notes ("New Features") keep it,
 * fused with the recurrent step of gdn_decode_step on the q, k, v it
 * produces, which never go through memory.  The result (o, state and the
 * windows) equals, bit for bit,
 *     gdn_conv1d(B, B, 1, NULL, C_conv, conv_width, dtype, x, stride_x,
 *                conv_weight, conv_bias, W_b, 1, y, C_conv)
 *     gdn_decode_step(d, y, y + H_k d_k, y + 2 H_k d_k, g, beta, state, ...)
 * where W_b holds, in sequence order, the windows of the sequences' slots
 * (d's token strides set to C_conv).
 *
 * d: as gdn_decode_step, with at most 4 v-heads per q/k head
 * (GDN_ERR_UNSUPPORTED otherwise: one workgroup convolves a q/k head once
 * for all its v-heads); its stride_q, stride_k and stride_v are not used
 * (0 or any value gdn_validate_dims accepts).  x: [B] rows of C_conv =
 * 2 H_k d_k + H_v d_v channels ordered [q | k | v], token stride stride_x
 * (>= C_conv, a multiple of 16 bytes), 16-byte aligned.  conv_width: W in
 * [2, 8]; conv_weight fp32 [C_conv][W]; conv_bias fp32 [C_conv] or NULL.
 * conv_state: [num_slots][W-1][C_conv] in dtype, required, 16-byte aligned,
 * not overlapping x: sequence b reads and advances the window of slot
 * state_slots[b] (or b), the same slot as its recurrent state.  g, beta,
 * state, num_slots, state_slots, o: as gdn_decode_step (two sequences must
 * not share a slot; a slot outside [0, num_slots) gives NaN outputs for that
 * sequence and leaves its state and window alone).
 */
gdn_status gdn_decode_conv_step(const gdn_dims *d, int32_t conv_width,
                                const void *x, int64_t stride_x,
                                const float *conv_weight,
                                const float *conv_bias, void *conv_state,
                                const float *g, const float *beta,
                                float *state, int32_t num_slots,
                                const int32_t *state_slots, void *o,
                                void *stream);

/*
 * The gated RMS norm on the layer's output, the step before the output
 * projection (oxydllm notes, "Performance": the Gated DeltaNet's gated norm
 * runs as one fused kernel over the token batch; "New Features", GGUF
 * qwen35: its weight is used as stored, with no plus-one).  Per token t and
 * v-head h, over the head_dim values of that row:
 *     y[t][h][j] = weight[j] * o[t][h][j] / sqrt(mean_i o[t][h][i]^2 + eps)
 *                  * silu(z[t][h][j]),   silu(a) = a / (1 + e^-a).
 *
 * total_tokens: rows of o, z and y (0 queues nothing).  num_heads: H_v in
 * [1, 4096]; head_dim: d_v, 64 or 128; dtype: of o, z and y.  o, z, y:
 * [total_tokens][num_heads][head_dim] with token strides stride_o,
 * stride_z, stride_y (elements, >= num_heads * head_dim, multiples of 16
 * bytes), 16-byte aligned; the heads of a token are packed.  weight: fp32
 * [head_dim], shared by all heads.  eps: finite, >= 0.  y may be o itself
 * (same pointer and stride: the norm in place) but must not otherwise
 * overlap o or z.  Arithmetic in fp32; a bf16 y is rounded to nearest even.
 */
gdn_status gdn_gated_rmsnorm(int32_t total_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t dtype, const void *o,
                             int64_t stride_o, const void *z, int64_t stride_z,
                             const float *weight, float eps, void *y,
                             int64_t stride_y, void *stream);

/*
 * The per-token gates from the layer's small raw projections (oxydllm
 * notes, "Performance": the beta and decay projections; "New Features",
 * GGUF qwen35: the per-head decay rate is the negated exponential of A_log,
 * and the scalar parameters stay fp32).  Per token t and v-head h:
 *     g[t][h]    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *     beta[t][h] = 1 / (1 + exp(-b[t][h]))
 * softplus(x) = log(1 + e^x).  g (a log-decay, <= 0) and beta are what the
 * prefill and decode calls take.
 *
 * total_tokens: rows (0 queues nothing).  num_heads: H_v in [1, 4096].
 * dtype: of a and b.  a, b: [total_tokens][num_heads] with token strides
 * stride_a, stride_b (elements, >= num_heads; they may be column blocks of
 * one projection output), aligned to their element size.  A_log, dt_bias:
 * fp32 [num_heads].  g, beta: fp32 [total_tokens][num_heads], packed,
 * 4-byte aligned, overlapping neither each other nor a or b.  Arithmetic in
 * fp32 with the accurate exponential and log1p.
 */
gdn_status gdn_gating(int32_t total_tokens, int32_t num_heads, int32_t dtype,
                      const void *a, int64_t stride_a, const void *b,
                      int64_t stride_b, const float *A_log,
                      const float *dt_bias, float *g, float *beta,
                      void *stream);

/*
 * The whole prefill from the layer's raw projections: gdn_prefill_conv_chunked
 * with g and beta computed inside the prepare from gates (the gdn_gating map,
 * the same fp32 arithmetic), so they never go through memory.  The result
 * equals gdn_gating into g, beta followed by gdn_prefill_conv_chunked with
 * them, bit for bit.  gates: see gdn_gate_inputs, required.  Every other
 * argument as gdn_prefill_conv_chunked.
 */
gdn_status gdn_prefill_conv_gated(const gdn_dims *d,
                                  const gdn_gate_inputs *gates,
                                  int32_t conv_width, const void *x,
                                  int64_t stride_x, const float *conv_weight,
                                  const float *conv_bias, void *conv_state,
                                  const float *state_in,
                                  const int32_t *cu_seqlens, void *y,
                                  int64_t stride_y, void *o, float *state_out,
                                  void *workspace, size_t ws_bytes,
                                  void *stream);

/*
 * One decode step from the layer's raw projections: gdn_decode_conv_step
 * with g and beta computed in the step's kernel from gates (one token per
 * sequence: a and b are [B][H_v] rows).  Equals gdn_gating followed by
 * gdn_decode_conv_step, bit for bit.  gates: required; every other argument
 * as gdn_decode_conv_step.
 */
gdn_status gdn_decode_conv_gated_step(const gdn_dims *d,
                                      const gdn_gate_inputs *gates,
                                      int32_t conv_width, const void *x,
                                      int64_t stride_x,
                                      const float *conv_weight,
                                      const float *conv_bias,
                                      void *conv_state, float *state,
                                      int32_t num_slots,
                                      const int32_t *state_slots, void *o,
                                      void *stream);

/*
 * Recurrent-state snapshots for prefix caching.  The per-sequence state --
 * the fp32 memories of all v-heads and the causal-conv window -- lives in a
 * caller-owned slot per (sequence, layer); a prompt prefix is reused by
 * restoring the state saved at its end rather than recomputing it
 * (Vallmo.jl README, "What's here": recurrent state snapshot/restore gives
 * prefix caching; PicoLM fork changelog, "SSM State Checkpointing": the state
 * is saved periodically during prefill and generation, and the nearest
 * saved state is restored on partial reuse).  One layer per call.
 *
 * gdn_snapshot_push copies, for each of num_seqs sequences b, live slot
 * slots[b] (or b when slots is NULL) of
 *     state      fp32 [num_slots][state_elems]   (state_elems = H_v d_k d_v)
 *     conv_state      [num_slots][window_bytes]  ((W-1) C_conv elements)
 * into entry e = (*ring_head mod ring_len) of the caller's ring
 *     ring_state  fp32 [ring_len][num_seqs][state_elems]
 *     ring_window      [ring_len][num_seqs][window_bytes]
 * and then adds one to *ring_head (a device int32 counting the pushes; the
 * caller sets it, normally to 0).  The entry is read on the device, so a
 * captured decode graph can push every N tokens with no host work; entry
 * n mod ring_len then holds push number n (the caller keeps the count on
 * the host, or reads the counter back).  Pushes sharing a counter must be
 * ordered (one stream).
 *
 * gdn_snapshot_restore copies ring entry `entry` (host int in [0, ring_len))
 * back into the live slots slots[b] (or b), state and window.  Continuing
 * from a restored entry gives, bit for bit, what continuing from the pushed
 * moment gave: the copies are exact.
 *
 * state_elems: a multiple of 4 (>= 0); window_bytes: a multiple of 16
 * (>= 0; 0 with conv_state and ring_window NULL copies states only).  All
 * pointers 16-byte aligned (slots and ring_head 4), device memory; the live
 * slots and the ring must not overlap.  A slot index outside [0, num_slots)
 * skips that sequence (its ring entry and slot are left as they were).
 * Errors as the other calls; nothing is queued on an invalid argument.
 */
gdn_status gdn_snapshot_push(int32_t num_seqs, const int32_t *slots, int32_t num_slots,
                             int64_t state_elems, const float *state, int64_t window_bytes,
                             const void *conv_state, int32_t ring_len, float *ring_state,
                             void *ring_window, int32_t *ring_head, void *stream);

gdn_status gdn_snapshot_restore(int32_t num_seqs, const int32_t *slots, int32_t num_slots,
                                int64_t state_elems, float *state, int64_t window_bytes,
                                void *conv_state, int32_t ring_len, const float *ring_state,
                                const void *ring_window, int32_t entry, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
