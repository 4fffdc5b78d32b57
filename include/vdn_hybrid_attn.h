/*
 * vdn_hybrid_attn.h -- C ABI of the Video DeltaNet (VDN) hybrid video-to-video
 * attention layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (arXiv abstract page "Video DeltaNet: A Video-Native Hybrid Attention
 * for Livestream Video Generation", Abstract; sd114.wiki article "VDN-Minimax-H3 ...",
 * sections 双向滑动窗口Softmax分支 and 双向线性注意力分支) combines
 *   (a) softmax attention over a block-sliding window: five latent frames form a
 *       chunk, a chunk attends to itself and to its previous and next chunk, every
 *       frame also attends to all tokens of the first and last frame, and the first
 *       and last frame attend to every frame;
 *   (b) a bidirectional linear branch, Video Delta Attention (VDA), whose memory is
 *       updated once per frame by all of the frame's tokens jointly; for query frame
 *       i the forward state summarises the frames before its window and the backward
 *       state the frames after it (never the window or the anchor frames), and the
 *       query reads both and adds the results;
 *   (c) a gated merge of the two branches (besthub article "VDN-H3 Generates
 *       14-Second 768p Video ...", section Hybrid Attention Architecture).
 * The pages give no algebra for the VDA update; this library implements the
 * proximal least-squares step
 *       S_t = (S_{t-1} + beta_t V_t K_t^T) (I + beta_t K_t K_t^T)^-1,
 * with K_t, V_t the d x N keys and values of frame t as columns, S_0 = 0, and the
 * readout o = S_fwd q + S_bwd q.  The merge is O = O_soft + g (.) O_lin with a
 * per-(head, channel) gate g.
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, O are [F, N, H, d] row-major: F latent frames, N tokens per
 *     frame, H heads, head dim d; one token's H*d values are contiguous.
 *     Element type by `precision`: fp32 for VDN_PREC_FP32, bf16 (raw 16-bit
 *     bfloat16 bit patterns) for VDN_PREC_BF16 and VDN_PREC_BF16_FP8QK.
 *   - beta is fp32 [F, H], gate is fp32 [H, d], states are fp32 [C, H, d, d] with
 *     C = ceil(F / 5) chunks; state row = value channel, column = key channel.
 *   - Every pointer except the host-side `table` of vdn_schedule is a DEVICE
 *     pointer (HIP global memory on the current device), owned by the caller; the
 *     library neither allocates nor frees memory and keeps no state across calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work: the return status covers argument checks and kernel launches; results
 *     are valid once the stream has been synchronised, and inputs must stay
 *     unchanged until then.  Outputs must not alias inputs.
 *   - `workspace` is caller-owned device scratch of at least
 *     vdn_workspace_bytes(F, N, H, d, precision) bytes, 256-byte aligned; it holds
 *     no meaning between calls.  Calls that share a workspace must not overlap.
 *   - Supported: F >= 1, N >= 1, H >= 1, d in {32, 64, 128}; VDN_PREC_BF16_FP8QK
 *     needs d in {64, 128}.  Anything else returns an error and launches nothing.
 *   - Results are deterministic: no atomics take part in value reductions.
 */
#ifndef VDN_HYBRID_ATTN_H
#define VDN_HYBRID_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define VDN_OK                0
#define VDN_ERR_INVALID_ARG  (-1)  /* null pointer, non-positive size, misaligned buffer */
#define VDN_ERR_UNSUPPORTED  (-2)  /* valid but unsupported (d, precision) combination   */
#define VDN_ERR_WORKSPACE    (-3)  /* workspace smaller than vdn_workspace_bytes()      */
#define VDN_ERR_HIP          (-4)  /* a HIP call failed; see vdn_last_hip_error()       */
#define VDN_ERR_TOO_LARGE    (-5)  /* the shape needs more scratch than the built-in
                                      array of vdn_hybrid_attn_noalloc holds            */

/* Precisions. */
#define VDN_PREC_FP32        0     /* q, k, v, O fp32; fp32 arithmetic                      */
#define VDN_PREC_BF16        1     /* q, k, v, O bf16; fp32 accumulation                    */
#define VDN_PREC_BF16_FP8QK  2     /* bf16 I/O; the softmax branch's q.k products use OCP
                                      E4M3 codes with per-head power-of-two scales computed
                                      internally (q first multiplied by log2(e)/sqrt(d));
                                      P.V, the VDA branch and the merge as bf16 */
#define VDN_PREC_FP8         3     /* bf16 I/O; the softmax branch runs on E4M3 codes: q.k as
                                      in VDN_PREC_BF16_FP8QK, and P.V with v coded per head
                                      the same way (power-of-two scale, prescale 1) and the
                                      probabilities rounded to E4M3 after the running-max
                                      shift (the row sums add the same rounded values); the VDA
                                      branch and the merge as bf16.  d = 64 or 128;
                                      vdn_hybrid_attn, vdn_hybrid_attn_noalloc,
                                      vdn_softmax_branch, vdn_vda_states and vdn_vda_linear
                                      only (the extra-token and projection entry points
                                      return VDN_ERR_UNSUPPORTED) */

/* Bytes of workspace the calls below need for this shape; 0 if the shape or
 * precision is invalid or unsupported. */
size_t vdn_workspace_bytes(int F, int N, int H, int d, int precision);

/* The whole hybrid layer: O = O_soft + g (.) O_lin.
 * Cited definition: see the header comment (all three parts).
 * q, k, v, O: [F, N, H, d]; beta: [F, H] (beta_t > 0 for a meaningful update);
 * gate: [H, d].  O must not alias q, k or v.  With bf16 I/O the readout and
 * merge run in the softmax kernel's epilogue: O is written once, as the bf16
 * rounding of O_soft + g (.) O_lin (fp32: O_soft is written, then the readout adds
 * g (.) O_lin to it). */
int vdn_hybrid_attn(const void* q, const void* k, const void* v,
                    const float* beta, const float* gate,
                    int F, int N, int H, int d, int precision,
                    void* O, void* workspace, size_t workspace_bytes, void* stream);

/* vdn_hybrid_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same result, bit for bit, with the workspace taken from a
 * static device array of VDN_NOALLOC_SCRATCH_BYTES bytes that the library holds
 * on every GPU it runs on until the process ends.  The call itself allocates and
 * frees nothing.  Shapes whose vdn_workspace_bytes exceeds the array return
 * VDN_ERR_TOO_LARGE before any device work (the 256-token, 30-frame, 8-head,
 * d = 64 workload fits, in bf16 and fp8 q.k).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents: calls that overlap on one
 * GPU (several streams or threads) race and must be serialised by the caller.
 * Arguments and the other errors as in vdn_hybrid_attn. */
#define VDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int vdn_hybrid_attn_noalloc(const void* q, const void* k, const void* v,
                            const float* beta, const float* gate,
                            int F, int N, int H, int d, int precision,
                            void* O, void* stream);

/* The layer with T extra (text or audio) tokens in the same sequence (arXiv
 * abstract page, Abstract; ananclaw note "Video DeltaNet ... critical read",
 * section 一、方法拆解: the hybrid covers video-to-video interactions only, every
 * interaction that involves a text or audio token stays plain softmax).
 * q, k, v, O: [F*N + T, H, d], the F*N video tokens (frame-major, as in
 * vdn_hybrid_attn) followed by the T extra tokens; beta: [F, H]; gate: [H, d].
 *   - a video query's softmax covers its key frames and all T extra tokens, in one
 *     normalisation; its linear output and merge are as in vdn_hybrid_attn;
 *   - an extra token's output is softmax attention over all F*N + T tokens;
 *   - the states see the video tokens only.
 * T = 0 is vdn_hybrid_attn.  T > 0 needs VDN_PREC_BF16 or VDN_PREC_BF16_FP8QK
 * (else VDN_ERR_UNSUPPORTED; the fp8 per-head scales then cover all F*N + T
 * tokens) and a workspace of vdn_workspace_bytes_mixed bytes. */
size_t vdn_workspace_bytes_mixed(int F, int N, int T, int H, int d, int precision);
int vdn_hybrid_attn_mixed(const void* q, const void* k, const void* v,
                          const float* beta, const float* gate,
                          int F, int N, int T, int H, int d, int precision,
                          void* O, void* workspace, size_t workspace_bytes, void* stream);

/* The layer followed by the two branches' separate output projections (arXiv
 * abstract page, Abstract; ananclaw note, section 一、方法拆解: separate output
 * projections and learnable gates calibrate the two branches):
 *     Y = O_soft W_s^T + (g (.) O_lin) W_l^T,
 * with O_soft, O_lin per token flattened head-major to H*d values and g the
 * per-(head, channel) gate of vdn_hybrid_attn (W_s = W_l = W gives vdn_hybrid_attn's
 * O times W^T; a gate on the projected output folds into W_l's rows).
 * q, k, v: [F, N, H, d] bf16; beta: [F, H]; gate: [H, d] fp32;
 * Wp: [D, 2*H*d] bf16 row-major, [W_s | W_l] (row n: W_s[n, :] then W_l[n, :]);
 * Y: [F*N, D] bf16 (fp32 accumulation).  precision VDN_PREC_BF16 or
 * VDN_PREC_BF16_FP8QK (fp32: VDN_ERR_UNSUPPORTED); D a multiple of 8.  The
 * workspace (vdn_workspace_bytes_proj bytes) also holds [O_soft | g (.) O_lin] as
 * bf16 [F*N][2][H][d]. */
size_t vdn_workspace_bytes_proj(int F, int N, int H, int d, int D, int precision);
int vdn_hybrid_attn_proj(const void* q, const void* k, const void* v,
                         const float* beta, const float* gate, const void* Wp,
                         int F, int N, int H, int d, int D, int precision,
                         void* Y, void* workspace, size_t workspace_bytes, void* stream);

/* The projection GEMM alone: Y[M, N] = A[M, K] B[N, K]^T, bf16 row-major
 * operands and output, fp32 accumulation (the product vdn_hybrid_attn_proj takes
 * with A = [O_soft | g (.) O_lin], B = Wp).  K a multiple of 64, N a multiple of 8
 * (else VDN_ERR_UNSUPPORTED).  No workspace. */
int vdn_out_proj(const void* A, const void* B, int M, int K, int N, void* Y, void* stream);

/* Softmax branch alone (part (a)): O_soft[i, n, h] = sum over tokens (j, m) of
 * the key frames of query frame i of softmax_{(j,m)}(q_{i,n,h} . k_{j,m,h} / sqrt(d))
 * v_{j,m,h}, with the window + anchor frame sets of the sd114.wiki article,
 * section 双向滑动窗口Softmax分支.  Same layouts as vdn_hybrid_attn. */
int vdn_softmax_branch(const void* q, const void* k, const void* v,
                       int F, int N, int H, int d, int precision,
                       void* O_soft, void* workspace, size_t workspace_bytes, void* stream);

/* VDA states alone (part (b), memory side): S_fwd[c, h] is the state after the
 * frames before chunk c's window (ascending, anchors excluded), S_bwd[c, h] the
 * state after the frames after the window (absorbed latest first); zero where
 * the set is empty, and zero for a chunk that holds no non-anchor frame (the
 * last chunk when F = 5m + 1), whose state no query reads (sd114.wiki article,
 * section 双向线性注意力分支; besthub article, section Video Delta Attention (VDA)).
 * k, v: [F, N, H, d]; beta: [F, H]; S_fwd, S_bwd: fp32 [C, H, d, d] outputs. */
int vdn_vda_states(const void* k, const void* v, const float* beta,
                   int F, int N, int H, int d, int precision,
                   float* S_fwd, float* S_bwd,
                   void* workspace, size_t workspace_bytes, void* stream);

/* VDA readout alone (part (b), query side): O_lin[i, n, h] = (S_fwd[c(i), h] +
 * S_bwd[c(i), h]) q[i, n, h] for non-anchor frames i (c(i) = i / 5), and 0 on the
 * first and last frame (sd114.wiki article, section 双向线性注意力分支: a query
 * reads the forward and the backward state and adds the two results; the anchor
 * frames, covered by softmax over every frame, are not computed again).  Ungated.  q, O_lin: [F, N, H, d] in the precision's I/O
 * type; S_fwd, S_bwd: fp32 [C, H, d, d].  Needs no workspace beyond
 * vdn_workspace_bytes (the same workspace convention applies). */
int vdn_vda_linear(const void* q, const float* S_fwd, const float* S_bwd,
                   int F, int N, int H, int d, int precision,
                   void* O_lin, void* workspace, size_t workspace_bytes, void* stream);

/* The fp8 quantiser of VDN_PREC_BF16_FP8QK, exposed for byte-exact checks.  The
 * pages run the softmax branch in FP8 (besthub article, section Performance
 * Results: branch-specific Ulysses sequence parallelism and FP8; model card
 * "Video DeltaNet: Hybrid Attention to Speed Up Video Models with Near-Lossless
 * Quality", section Your first render: the 8nfe_tuned_fp8 configuration) without
 * naming the format or the scaling; this library takes OCP E4M3 with one
 * power-of-two scale per head, so that the matrix core applies the scales exactly
 * (E8M0 operand scales) and the scores need no rescaling on the vector units:
 *   y = fp32(x * prescale);  amax[h] = max |y| over head h;
 *   scale_exp[h] = the smallest integer e with amax[h] <= 448 * 2^e, clamped to
 *                  [-127, 127] (0 where amax[h] is 0);
 *   code = E4M3(RNE, saturating) of fp32(y * 2^-scale_exp[h]).
 * The layer quantises q with prescale = fp32(log2(e) / sqrt(d)) (so that a score
 * in base-2 units is 2^(e_q + e_k) times the code products) and k with 1.
 * x: bf16 [F, N, H, d]; prescale: finite and > 0, else VDN_ERR_INVALID_ARG;
 * codes: uint8 [F, N, H, d] (OCP E4M3 "FN" bit patterns); scale_exp: int32 [H],
 * also used as scratch during the call.  d: 64 or 128. */
int vdn_fp8_quantize(const void* x, int F, int N, int H, int d, float prescale,
                     unsigned char* codes, int* scale_exp, void* stream);

/* Frame partition of the layer for F frames (host only, no device work): the
 * softmax key frames of every query frame (sd114.wiki article, section
 * 双向滑动窗口Softmax分支: its own chunk of five frames, the previous and the next
 * chunk, the first and the last frame; the first and last frame see every frame)
 * and the frames of its forward and backward states (section 双向线性注意力分支:
 * the non-anchor frames before and after the window, so that the three sets are
 * disjoint and together cover every frame).
 * One row of VDN_SCHED_COLS ints per group of query frames that share their
 * sets: { q_first, q_last, n_soft,  s0_first, s0_last, s1_first, s1_last,
 *         s2_first, s2_last,  fwd_first, fwd_last, bwd_first, bwd_last }
 * (frame indices, inclusive; unused softmax ranges and empty linear sets are
 * -1, -1).  Rows: the first frame, each chunk's non-anchor frames, the last
 * frame, in ascending q_first.  Writes at most `cap` rows to `table` (may be
 * NULL when cap is 0) and returns the number of rows, or a negative status. */
#define VDN_SCHED_COLS 13
int vdn_schedule(int F, int* table, int cap);

/* Stages of the launch sequence, for vdn_set_stage_events. */
#define VDN_STAGE_PREP     0   /* one pass over k, v: v re-laid out for P.V, frame Grams */
#define VDN_STAGE_FACTOR   1   /* per-frame Cholesky: M_t = A_t^-1, C_t = beta B_t M_t     */
#define VDN_STAGE_SCAN     2   /* serial state scan, both directions                     */
#define VDN_STAGE_WPREP    3   /* readout weights g (.) (S_fwd + S_bwd)                   */
#define VDN_STAGE_ATTN     4   /* windowed + anchored softmax attention (bf16 I/O layer:
                                  with the readout + gated merge in its epilogue)       */
#define VDN_STAGE_COMBINE  5   /* merge of the anchor rows' key slices                   */
#define VDN_STAGE_READOUT  6   /* linear readout (+ gated merge in the fp32 layer; the
                                  readout of vdn_vda_linear)                            */
#define VDN_STAGE_QUANT    7   /* fp8 quantiser of q and k                               */
#define VDN_STAGE_PROJ     8   /* output projections (vdn_hybrid_attn_proj, vdn_out_proj) */
#define VDN_NUM_STAGES     9

/* Measurement aid for the calling thread: while set, every entry point records
 * the hipEvent_t `before` on its stream immediately before it enqueues the
 * kernels of `stage`, and `after` immediately after.  The events are created
 * and owned by the caller; pass NULL, NULL to stop recording.  Returns VDN_OK or
 * VDN_ERR_INVALID_ARG for an unknown stage. */
int vdn_set_stage_events(int stage, void* before, void* after);

/* Human-readable text of a status code (static storage). */
const char* vdn_status_string(int status);

/* The hipError_t of the last failed HIP call on the calling thread (0 if none). */
int vdn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* VDN_HYBRID_ATTN_H */
