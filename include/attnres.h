/*
 * attnres.h -- C ABI of libattnres, the gfx950 (MI355X) library for the
 * Attention Residuals (AttnRes) depth-aggregation hot path.
 *
 * Pages cited (title, then section / equation):
 *   [K3] K3 course notes, section "Attention Residual 深度残差":
 *        9.1 eqs. (A1)-(A4); 9.2 DepthResidual; 9.3 Full vs Block and
 *        forward_naive; 9.4 the two-phase algorithm, eqs. (OS1), (OS2);
 *        9.6 atomic_block_size and config validation.
 *   [WC] "Attention Residuals" survey page (wineandchord.com): "Block
 *        AttnRes", "Online softmax keeps the two phases exact", "Depth
 *        attention & online merge reference", "Inference: block
 *        representations as a depth KV cache".
 *   [RH] Reading notes on "Attention Residuals" (ranhao.site), 4.2
 *        Inference: Phase 1 and Phase 2.
 *   [ZZ] "Attention Residuals" notes (zhangzhe.space): the block_attn_res
 *        listing, where every sublayer applies its own RMSNorm to the
 *        aggregate it receives (attn(attn_norm(h)), mlp(mlp_norm(h))).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers unless marked (host). A token tensor
 *     [B, T, D] is passed as R = B*T rows of D contiguous elements ("[R,D]",
 *     row-major, row r = b*T + t). Rows are independent: attention weights are
 *     per token and never mix positions [K3 9.1].
 *   - dtype selects the I/O element type of every [R,D] tensor of a call:
 *     ATTNRES_F32 or ATTNRES_BF16. Queries, gains and statistics are always
 *     fp32. Arithmetic is fp32; bf16 results are rounded nearest-even.
 *   - D*sizeof(dtype) must be a multiple of 16 bytes and at most
 *     ATTNRES_MAX_ROW_BYTES; every pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call validates ALL of its arguments before it enqueues anything,
 *     then enqueues its kernels asynchronously on `stream` and returns.
 *     Nothing here allocates, frees or synchronises device memory; the caller
 *     owns every buffer and the library keeps no pointer after a call returns.
 *   - Return value: ATTNRES_OK, or a negative status with nothing enqueued
 *     (for ATTNRES_EINVAL / EUNSUPPORTED / EWORKSPACE) and a detail message in
 *     attnres_last_error() (thread-local). R == 0 is a successful no-op once
 *     the shape, count and eps arguments are valid; tensor pointers are then
 *     not inspected (they may be NULL) and no callback is invoked.
 *     Asynchronous device faults surface at the caller's next synchronisation.
 *     NaN / Inf inputs are not checked; their results are unspecified.
 *   - eps must be finite and >= 0. The score of a source v under the folded
 *     query q~ = w * gamma is  q~ . v / sqrt(mean_d(v^2) + eps)  [K3 (A1),
 *     9.2 (1)-(2); WC reference code: eps inside the root, mean over D].
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTNRES_F32 0
#define ATTNRES_BF16 1

#define ATTNRES_OK 0
#define ATTNRES_EINVAL (-1)       /* an argument is out of its documented domain */
#define ATTNRES_EUNSUPPORTED (-2) /* valid but beyond this build's limits         */
#define ATTNRES_EWORKSPACE (-3)   /* workspace smaller than required              */
#define ATTNRES_EHIP (-4)         /* a HIP launch / runtime call failed            */
#define ATTNRES_ECALLBACK (-5)    /* the sublayer callback returned nonzero        */

#define ATTNRES_MAX_SOURCES 64     /* sources of one aggregate / Phase-1 call   */
#define ATTNRES_MAX_ROW_BYTES 32768 /* D * sizeof(dtype) upper bound            */

/* ---------------------------------------------------------------------------
 * attnres_aggregate -- one depth aggregation per token row [K3 9.1 (A1)-(A3),
 * 9.2 DepthResidual.forward; WC depth_summary + finish]:
 *     s_i = q~ . v_i / sqrt(mean_d(v_i^2) + eps),  q~ = w * gamma (fp32)
 *     a   = softmax_i(s)                            (over the source axis)
 *     out = sum_i a_i v_i                           (the RAW sources)
 *   sources (host) : n device pointers, each [R,D] dtype (1 <= n <= 64)
 *   w, gamma       : [D] fp32 query and RMSNorm gain; gamma NULL means ones
 *   out            : [R,D] dtype, may not alias a source
 *   m_out, lse_out : [R] fp32 or NULL: max_i s_i and m + log(sum_i e^(s_i-m))
 *                    [K3 9.4 (OS1); RH 4.2]
 * ------------------------------------------------------------------------- */
int attnres_aggregate(const void* const* sources, int n, int64_t R, int64_t D, int dtype,
                      const float* w, const float* gamma, float eps, void* out, float* m_out,
                      float* lse_out, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_phase1_batched -- Phase 1 of two-phase Block AttnRes: the S
 * pseudo-queries of one block, stacked into [S,D], each aggregate the same
 * fixed list of completed sources [b_0 .. b_k] in one pass over them; returns
 * each query's normalised output and its max / log-sum-exp statistics
 * [K3 9.4 step 1 and _run_block_two_phase; RH 4.2 Phase 1; WC "Inference"].
 *   blocks (host)  : n device pointers [R,D] dtype (b_0 = the embedding)
 *   W, Gamma       : [S,D] fp32 queries and gains (Gamma NULL means ones)
 *   out            : [S,R,D] dtype; out[s] = sum_i a_{s,i} b_i
 *   m_out, lse_out : [S,R] fp32; m_out may be NULL, lse_out is required
 *   1 <= S <= 1024.
 * ------------------------------------------------------------------------- */
int attnres_phase1_batched(const void* const* blocks, int n, int64_t R, int64_t D, int dtype,
                           const float* W, const float* Gamma, int S, float eps, void* out,
                           float* m_out, float* lse_out, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_phase2_merge -- Phase 2 of two-phase Block AttnRes for one
 * sublayer [K3 9.4 step 2, eq. (OS2), single_source_stats; RH 4.2 Phase 2]:
 *     p   = p_prev ? round(p_prev + v_prev) : v_prev      (partial, I/O dtype)
 *     s_p = q~ . p / sqrt(mean_d(p^2) + eps)             (score of the ROUNDED p)
 *     h   = OS2 merge of the Phase-1 group (lse, o, 1) with (s_p, p, 1), normalised:
 *           M = max(lse, s_p), h = (e^(lse-M) o + e^(s_p-M) p) / (e^(lse-M) + e^(s_p-M))
 *   o, lse         : this sublayer's Phase-1 output [R,D] dtype and lse [R] fp32
 *   w, gamma       : [D] fp32 (gamma NULL means ones)
 *   p_prev         : [R,D] partial before this sublayer's update, or NULL for the
 *                    first merge of a block (then p := v_prev, p_out must be NULL)
 *   v_prev         : [R,D] the previous sublayer's output
 *   p_out          : [R,D] receives p (may equal p_prev: in-place is safe); it may
 *                    be NULL only when p_prev is NULL
 *   h_out          : [R,D] dtype; must not alias o, p_prev, v_prev or p_out
 * ------------------------------------------------------------------------- */
int attnres_phase2_merge(const void* o, const float* lse, const float* w, const float* gamma,
                         float eps, const void* p_prev, const void* v_prev, void* p_out,
                         void* h_out, int64_t R, int64_t D, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * The input norm of the sublayer that consumes an aggregate. In the block
 * listing of [ZZ] every sublayer applies its own RMSNorm to h first
 * (attn(attn_norm(h)), mlp(mlp_norm(h))); [WC "Depth attention & online merge
 * reference"] notes the reference operator's optional fused output RMSNorm.
 * The norm is the same RMS form as the keys' [WC reference code], with the
 * sublayer's own gain and eps:
 *   hn[r][d] = round(gamma_f[d] * h_r[r][d] / sqrt(mean_d h_r[r][:]^2 + eps_f))
 * where h_r is h rounded to dtype (exactly what the sublayer would receive).
 *
 * attnres_phase2_merge_norm: attnres_phase2_merge with the norm fused in.
 *   gamma_f : [D] fp32, or NULL for ones
 *   eps_f   : finite, >= 0
 *   hn_out  : [R,D] dtype, required
 *   h_out   : [R,D] dtype, or NULL (then h itself is not written)
 *   Errors as attnres_phase2_merge, plus ATTNRES_EINVAL for a bad eps_f, or
 *   h_out / hn_out aliasing an input, p_out or each other.
 * attnres_rmsnorm: hn = RMSNorm(x) * gamma for one [R,D] tensor (x and out
 *   may be the same buffer); gamma [D] fp32 or NULL for ones.
 * ------------------------------------------------------------------------- */
int attnres_phase2_merge_norm(const void* o, const float* lse, const float* w, const float* gamma,
                              float eps, const void* p_prev, const void* v_prev, void* p_out,
                              void* h_out, const float* gamma_f, float eps_f, void* hn_out,
                              int64_t R, int64_t D, int dtype, void* stream);
int attnres_rmsnorm(const void* x, int64_t R, int64_t D, int dtype, const float* gamma, float eps,
                    void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Sublayer callback of the stack forward: eq. (A4) v_l = f_l(h_l) [K3 9.1].
 * Called on the calling thread with l = 1..L in order. h_l is a device [R,D]
 * dtype buffer inside the workspace, valid until the callback returns; the
 * callback must consume it with work enqueued on `stream` (or synchronise).
 * It stores in *v_out a 16-byte aligned device pointer to v_l [R,D] dtype and
 * returns 0; a nonzero return aborts the forward with ATTNRES_ECALLBACK.
 * The library enqueues its last read of v_l before it invokes the callback for
 * sublayer l+2, so a 3-slot ring written on the same stream is safe -- except
 * for S == 1 with block_sums == NULL, where every v_l stays a source (below).
 * ------------------------------------------------------------------------- */
typedef int (*attnres_sublayer_fn)(void* ctx, int l, const void* h_l, const void** v_out,
                                   void* stream);

/* Built-in callback for pre-computed sublayer outputs: ctx is a (host) array
 * of L device pointers, v_l = ((const void* const*)ctx)[l-1]; h_l is ignored. */
int attnres_table_sublayer(void* ctx, int l, const void* h_l, const void** v_out, void* stream);

/* Bytes of workspace attnres_block_stack_forward needs for (L, S, R, D, dtype);
 * 0 for invalid arguments. It holds the folded queries, one block's Phase-1
 * outputs and statistics, the partial sum and h; for bf16 stacks of at least
 * 4096 rows (D a multiple of 256 up to 8192, at most 32 queries) whose
 * widest block has more than 8 queries or a width outside {1024, 2048, 3072,
 * 4096}, or that have more than 8 blocks, also the query parts
 * [32 ceil(S/8), D] bf16 and the softmax weights [S, R, 8] fp32 ([S, R, 16]
 * with more than 8 blocks) of the matrix-core scores pass, which then runs
 * Phase 1 for blocks of at most 16 sources. */
size_t attnres_stack_workspace_bytes(int L, int S, int64_t R, int64_t D, int dtype);

/* ---------------------------------------------------------------------------
 * attnres_block_stack_forward -- the Block AttnRes stack forward, two-phase
 * [K3 9.3 forward_naive semantics, 9.4 _run_block_two_phase; WC "Block
 * AttnRes", "Online softmax"], Full AttnRes when S == 1 [WC: N = L limit].
 *   Sublayers l = 1..L are cut into nb = ceil(L/S) blocks of S (the last may
 *   be short). Block k (0-based) runs Phase 1 with its queries over
 *   [b_0 .. b_k], hands h = o_0 to its first sublayer, then for each further
 *   sublayer merges the running partial by Phase 2; after its last sublayer
 *   b_{k+1} = round(p + v_last) is stored. Finally
 *   y = aggregate([b_0 .. b_nb]; q~_{L+1}) [K3 9.1 is_final_aggregate].
 *   x          : [R,D] dtype, the embedding b_0
 *   W, Gamma   : [L+1, D] fp32; row l-1 belongs to sublayer l, row L to the
 *                final aggregate (Gamma NULL means ones)
 *   f, f_ctx   : sublayer callback (see above)
 *   block_sums : (host) nb device pointers [R,D] receiving b_1..b_nb, or NULL
 *                only when S == 1 (then b_l is v_l itself and every v_l must
 *                stay valid for the whole call)
 *   y          : [R,D] dtype
 *   workspace  : device scratch of at least attnres_stack_workspace_bytes()
 *                bytes, 256-byte aligned; contents on return are unspecified
 *   Limits: 1 <= S, 1 <= L, nb + 1 <= ATTNRES_MAX_SOURCES.
 *   A failure after work was enqueued (ATTNRES_ECALLBACK, ATTNRES_EHIP) leaves
 *   that work enqueued and the outputs undefined.
 * ------------------------------------------------------------------------- */
int attnres_block_stack_forward(const void* x, int L, int S, int64_t R, int64_t D, int dtype,
                                const float* W, const float* Gamma, float eps,
                                attnres_sublayer_fn f, void* f_ctx, void* const* block_sums,
                                void* y, void* workspace, size_t workspace_bytes, void* stream);

/* attnres_block_stack_forward whose sublayers receive their normalised input
 * (see attnres_phase2_merge_norm): the callback for sublayer l gets
 * hn_l = RMSNorm(h_l) * Gamma_f[l-1] in place of h_l, and h_l itself is not
 * materialised (in Block AttnRes h_l feeds only its sublayer). Gamma_f
 * [L, D] fp32 or NULL for ones; eps_f finite and >= 0. Workspace, ownership,
 * limits and errors as attnres_block_stack_forward. The norm is fused into
 * Phase 2 and into the aggregate of a one-sublayer block. A block's first
 * sublayer (h = Phase-1 output 0) gets it from the Phase-1 pass itself where
 * that pass is the one-source statistics pass or the register-resident
 * matrix-core pass (bf16, at most 8 queries, D in {1024, 2048, 3072, 4096},
 * up to 7 sources at D = 4096); other Phase-1 passes are followed by a
 * separate RMSNorm pass. */
int attnres_block_stack_forward_norm(const void* x, int L, int S, int64_t R, int64_t D, int dtype,
                                     const float* W, const float* Gamma, float eps,
                                     const float* Gamma_f, float eps_f, attnres_sublayer_fn f,
                                     void* f_ctx, void* const* block_sums, void* y, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_block_stack_forward_overlap -- the stack forward with the decode
 * schedule [WC "Kimi Linear and K3 integration", decode: the batched
 * inter-block pass runs on a side stream, overlapped with the main stream's
 * work; K3 9.4 (OS2): merging source groups is exact]. Block k+1's Phase 1
 * needs every completed source, but the merge of groups lets it start early:
 * while block k's sublayers run on `stream`, `side_stream` scores block
 * k+1's queries over [b_0 .. b_k]; the block sum b_{k+1} that block k closes
 * with then joins as one more single-source term (one launch that performs
 * the close and gives block k+1's first sublayer its input, and a
 * three-term merge in each later Phase-2 step). Results equal the naive
 * forward's (the same reading as attnres_block_stack_forward; only the
 * grouping of the softmax terms differs). Meant for decode (few rows), where
 * a Phase-1 launch on the main stream is latency on the critical path; with
 * many rows the three-term merges read one more [R,D] tensor per sublayer.
 *   Arguments as attnres_block_stack_forward, plus:
 *   out_norm       : nonzero: sublayer l receives RMSNorm(h_l) * Gamma_f[l-1]
 *                    with eps_f, as attnres_block_stack_forward_norm; zero:
 *                    h_l (Gamma_f and eps_f are then ignored)
 *   block_sums     : (host) nb device pointers, required (also for S == 1)
 *   workspace      : attnres_stack_overlap_workspace_bytes(L, S, R, D, dtype)
 *                    bytes, 256-byte aligned (two Phase-1 slots)
 *   stream         : the main stream; the callback is handed this stream
 *   side_stream    : a second stream of the same device and the same
 *                    (default) priority, not `stream` (ATTNRES_EINVAL
 *                    otherwise). The library orders the two streams with
 *                    two HIP events of its own (per thread and device,
 *                    created at the first call, timing disabled; no device
 *                    memory). Every side-stream launch is joined back into
 *                    `stream` before the call returns, so work the caller
 *                    enqueues on `stream` afterwards sees all results, and a
 *                    capture of `stream` into a HIP graph takes the side
 *                    stream's work along.
 * ------------------------------------------------------------------------- */
size_t attnres_stack_overlap_workspace_bytes(int L, int S, int64_t R, int64_t D, int dtype);
int attnres_block_stack_forward_overlap(const void* x, int L, int S, int64_t R, int64_t D,
                                        int dtype, const float* W, const float* Gamma, float eps,
                                        int out_norm, const float* Gamma_f, float eps_f,
                                        attnres_sublayer_fn f, void* f_ctx,
                                        void* const* block_sums, void* y, void* workspace,
                                        size_t workspace_bytes, void* stream, void* side_stream);

/* ---------------------------------------------------------------------------
 * attnres_block_layout -- the integer plan of forward_naive [K3 9.3 listing;
 * WC "Block AttnRes"]. block_start[k] (host, nb+1 entries or NULL) is the
 * first sublayer (1-based) of block k, with block_start[nb] = L + 1.
 * n_sources[l-1] (host, L+1 entries or NULL) is the number of sources sublayer
 * l attends over (k+1 completed, plus the partial once it exists);
 * n_sources[L] is the final aggregate's, nb + 1. Returns nb, or a negative
 * status for L < 1 or S < 1.
 * ------------------------------------------------------------------------- */
int attnres_block_layout(int L, int S, int* block_start, int* n_sources);

/* DecoderBlock count -> atomic sublayers per block [K3 9.6 atomic_block_size]:
 * each DecoderBlock is an attention and an MLP sublayer; layers_per_block <= 0
 * stands for "None", which targets about eight blocks: max(1, ceil(L/8)).
 * Returns ATTNRES_EINVAL for num_decoder_layers < 1. */
int attnres_atomic_block_size(int num_decoder_layers, int layers_per_block);

/* Static description of a status code. */
const char* attnres_status_string(int code);

/* Detail message of the last failing call on this thread ("" if none). */
const char* attnres_last_error(void);

/* ---------------------------------------------------------------------------
 * Full AttnRes (every sublayer output is a source of its own [K3 9.3 Full;
 * WC "Full AttnRes"]) with the two-phase schedule [K3 9.4: given a schedule
 * block size the Full mixer runs the two-phase algorithm and matches the
 * naive one; WC "Inference": the (S+N)d residual I/O of two-phase Full].
 *
 * attnres_merge_sources -- the intra-chunk step: merge the summary of an
 *   earlier group (its normalised output o [R,D] dtype and log-sum-exp lse
 *   [R] fp32, as Phase 1 returns them) with n more sources [K3 9.4 (OS2),
 *   each new source its own term]:
 *     out = (e^(lse-M) o + sum_i e^(s_i-M) v_i) / (e^(lse-M) + sum_i e^(s_i-M)),
 *   s_i the usual score of source i under q~ = w * gamma, M the max of lse and
 *   the s_i. m_out / lse_out [R] (optional) receive the merged statistics.
 *   1 <= n <= ATTNRES_MAX_SOURCES; out must not alias o or a source.
 *
 * attnres_full_stack_forward -- the Full stack forward over L sublayers with
 *   schedule block size C: chunk [s, s+C-1] runs Phase 1 with its queries over
 *   [x, v_1 .. v_{s-1}] in one pass, hands h_s = o_0 to its first sublayer,
 *   and gives sublayer s+j the merge of (lse_j, o_j) with v_s .. v_{s+j-1};
 *   y = aggregate([x, v_1 .. v_L]; q~_{L+1}). C = 1 is the naive schedule.
 *   W, Gamma [L+1, D] fp32 as in attnres_block_stack_forward. Every v_l
 *   returned by the callback is a source to the end of the call and must
 *   stay valid until then. Workspace: attnres_full_workspace_bytes(L, C, R,
 *   D, dtype) bytes, 256-byte aligned; for bf16 stacks of at least 4096 rows
 *   it also holds the matrix-core scores pass's query parts and weights when
 *   a chunk of up to 16 sources takes that pass. Limits: L + 1 <=
 *   ATTNRES_MAX_SOURCES. Errors as attnres_block_stack_forward.
 * ------------------------------------------------------------------------- */
int attnres_merge_sources(const void* o, const float* lse, const void* const* sources, int n,
                          int64_t R, int64_t D, int dtype, const float* w, const float* gamma,
                          float eps, void* out, float* m_out, float* lse_out, void* stream);
size_t attnres_full_workspace_bytes(int L, int C, int64_t R, int64_t D, int dtype);
int attnres_full_stack_forward(const void* x, int L, int C, int64_t R, int64_t D, int dtype,
                               const float* W, const float* Gamma, float eps,
                               attnres_sublayer_fn f, void* f_ctx, void* y, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_aggregate_backward -- gradients of one aggregate (attnres_aggregate)
 * for an upstream gradient dh, with recomputation: no forward state is kept;
 * the scores and weights are recomputed from the sources [K3 9.1 (A1)-(A3)
 * differentiated; WC "Depth attention & online merge reference" and "Public
 * implementation boundary": the fused operator computes forward and backward
 * with online softmax and recomputation]. Per row, with r_i = sqrt(mean_d
 * v_i^2 + eps), s_i = q~ . v_i / r_i, a = softmax(s), g_i = dh . v_i and
 * ds_i = a_i (g_i - sum_j a_j g_j):
 *     dV_i  = a_i dh + ds_i (q~ / r_i - s_i v_i / (D r_i^2))
 *     dq~   = sum over rows of sum_i ds_i v_i / r_i
 *     dw    = dq~ * gamma (dq~ without a gain),  dgamma = dq~ * w
 * (the fold q~ = w * gamma is differentiated as an exact product).
 *   sources (host) : n device pointers [R,D] dtype (1 <= n <= 64)
 *   w, gamma       : [D] fp32 (gamma NULL means ones)
 *   dh             : [R,D] dtype, the gradient of the loss w.r.t. the output
 *   dV (host)      : n device pointers [R,D] fp32; dV[i] receives the gradient
 *                    of sources[i]. They must be distinct and alias no input.
 *   dw             : [D] fp32, required; dgamma : [D] fp32 or NULL (not wanted)
 *   accumulate     : 0 writes the gradients, nonzero adds them to dV, dw and
 *                    dgamma (for a source, query or gain used by several
 *                    aggregates)
 *   workspace      : device scratch of attnres_aggregate_backward_workspace_bytes
 *                    (R, D, dtype) bytes, 256-byte aligned, owned by the caller
 *                    and not read before it is written (EWORKSPACE if smaller).
 *   Arithmetic is fp32; gradients stay fp32 so that sums over many aggregates
 *   do not round. The sum over rows runs in a fixed order that depends only
 *   on (R, D, dtype): results are deterministic. With R == 0, dw and dgamma
 *   are still written (zeros) or left unchanged (accumulate).
 * ------------------------------------------------------------------------- */
size_t attnres_aggregate_backward_workspace_bytes(int64_t R, int64_t D, int dtype);
int attnres_aggregate_backward(const void* const* sources, int n, int64_t R, int64_t D, int dtype,
                               const float* w, const float* gamma, float eps, const void* dh,
                               float* const* dV, int accumulate, float* dw, float* dgamma,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_block_stack_backward -- the gradients of the Block stack forward
 * through its two-phase schedule, with recomputation [K3 9.1 (A1)-(A4) and
 * 9.4 (OS1)-(OS2) differentiated; WC "Depth attention & online merge
 * reference", "Public implementation boundary": a fused forward and backward
 * with online softmax and recomputation]. The loss reaches the stack through
 * every aggregate: L = sum_l <dh_l, h_l> + <dy, y>, where the sublayers
 * supply dh_l. Blocks are walked in reverse; per block the library
 *   - recomputes its Phase 1 (o_j, lse_j over [b_0 .. b_k]) and partials;
 *   - for each sublayer from the last to the second, runs the backward of
 *     its Phase-2 merge h = OS2((lse_j, o_j), (s_p, p_j)): the gradient of
 *     p_j (through the weighted sum and through s_p) joins that of the
 *     partial's later uses, which is exactly dv of the sublayer before;
 *   - then the Phase-1 backward of each query: its output received a_j dh_j
 *     (a_j the group's merge weight; dh itself for the first sublayer, whose
 *     h is o_0) and its log-sum-exp the merge's d lse_j;
 *   - block sum b_k's gradient is that of block k-1's last output.
 * Rounding to the I/O dtype (outputs, partials, block sums) is taken as the
 * identity in the backward.
 *   x, v (host)   : the forward's embedding [R,D] and its L sublayer outputs
 *   W, Gamma      : [L+1, D] fp32 as in the forward (Gamma NULL means ones)
 *   block_sums    : (host) the forward's nb block sums, or NULL when S == 1
 *                   (then b_l = v_l)
 *   dy            : [R,D] dtype, the upstream gradient of y
 *   fb, fb_ctx    : the sublayer backward, called with l = L down to 1 once
 *                   dv_l (fp32 [R,D], the gradient of v_l) is complete; it
 *                   returns in *dh_out the upstream gradient of h_l, [R,D]
 *                   dtype, which must stay valid until the callback for the
 *                   previous block's last sublayer returns (or the call
 *                   ends); attnres_table_sublayer_bwd serves a table of L
 *                   given gradients
 *   dx            : [R,D] fp32, the gradient of x (written)
 *   dv (host)     : L device pointers [R,D] fp32, distinct, receiving dv_l
 *                   (written; the callback reads dv_l from dv[l-1])
 *   dW, dGamma    : [L+1, D] fp32, written; dGamma NULL when not wanted
 *                   (and required NULL when Gamma is NULL)
 *   workspace     : attnres_stack_backward_workspace_bytes(L, S, R, D, dtype)
 *                   bytes, 256-byte aligned
 * Errors as attnres_block_stack_forward (ATTNRES_ECALLBACK for a failing
 * sublayer backward). With R == 0, dW and dGamma are written as zeros.
 * ------------------------------------------------------------------------- */
typedef int (*attnres_sublayer_bwd_fn)(void* ctx, int l, const float* dv_l, const void** dh_out,
                                       void* stream);
int attnres_table_sublayer_bwd(void* ctx, int l, const float* dv_l, const void** dh_out,
                               void* stream);
size_t attnres_stack_backward_workspace_bytes(int L, int S, int64_t R, int64_t D, int dtype);
int attnres_block_stack_backward(const void* x, const void* const* v, int L, int S, int64_t R,
                                 int64_t D, int dtype, const float* W, const float* Gamma, float eps,
                                 const void* const* block_sums, const void* dy,
                                 attnres_sublayer_bwd_fn fb, void* fb_ctx, float* dx,
                                 float* const* dv, float* dW, float* dGamma, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attnres_aggregate_backward_noalloc -- attnres_aggregate_backward without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving or training loops, and harnesses
 * that forbid hipMalloc. It allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine) and runs the same kernels with the same
 * results: every argument, output and error is as for
 * attnres_aggregate_backward.
 *   Its scratch (the per-workgroup dq~ partials) is a fixed device array of
 *   ATTNRES_NOALLOC_SCRATCH_BYTES (33 MiB) that each GPU holds from the
 *   library's first use there until the process ends. It covers every row
 *   of at most 8192 elements, whatever R is. A bf16 row with D > 8192 needs
 *   more once R fills the backward's grid (a few thousand rows); such a call
 *   is rejected with ATTNRES_EUNSUPPORTED before anything is enqueued (the
 *   rule: attnres_aggregate_backward_workspace_bytes(R, D, dtype) >
 *   ATTNRES_NOALLOC_SCRATCH_BYTES).
 *   `stream` must belong to the calling thread's current device
 *   (ATTNRES_EINVAL otherwise).
 *   All calls on one GPU share that GPU's array and nothing guards it: two
 *   calls whose work overlaps on one GPU (on different streams, or from
 *   different threads without ordering) race and give undefined results.
 *   Calls ordered on one stream are safe; the array keeps the last call's
 *   contents, and every call writes its partials before reading them.
 * attnres_noalloc_scratch_bytes returns ATTNRES_NOALLOC_SCRATCH_BYTES.
 * ------------------------------------------------------------------------- */
#define ATTNRES_NOALLOC_SCRATCH_BYTES (33u << 20)
size_t attnres_noalloc_scratch_bytes(void);
int attnres_aggregate_backward_noalloc(const void* const* sources, int n, int64_t R, int64_t D,
                                       int dtype, const float* w, const float* gamma, float eps,
                                       const void* dh, float* const* dV, int accumulate, float* dw,
                                       float* dgamma, void* stream);

/* ---------------------------------------------------------------------------
 * Optional launch timing (instrumentation for benchmarks; off by default).
 * attnres_timing_enable(capacity) makes this thread's subsequent launches
 * record a HIP event pair around each kernel on its stream, for up to
 * `capacity` launches (0 disables and releases the events). The library keeps
 * per-kind totals: kind 0 Phase 1, 1 Phase 2, 2 aggregate, 3 block close,
 * 4 query fold, 5 standalone output norm, 6 aggregate backward (main
 * kernel), 7 its reduction over rows, 8 Phase-1 statistics of a block whose
 * only source is the embedding (a stack forward's first block: its outputs
 * are the embedding itself and are not formed). attnres_timing_read synchronises
 * the recorded events and returns, for `kind`, the number of timed launches,
 * their summed duration in milliseconds and their summed algorithmic bytes
 * (inputs read once plus outputs written once, queries excluded).
 * attnres_timing_reset clears the
 * totals and the recorded events. attnres_timing_pause(1) stops recording
 * (launches run untimed, with no event overhead) until attnres_timing_pause(0);
 * enabling does not change the paused state.
 * ------------------------------------------------------------------------- */
int attnres_timing_enable(int capacity);
int attnres_timing_pause(int paused);
int attnres_timing_reset(void);
int attnres_timing_read(int kind, int64_t* launches, double* total_ms, double* total_bytes);
/* The kernels that the timed launches of `kind` ran since the last reset:
 * distinct names, comma-separated ("" if none, or for an invalid kind); a
 * launch of several kernels is named "first+second". Valid until the next
 * timing call on this thread. */
const char* attnres_timing_kernels(int kind);
/* The launches timed since the previous collection (attnres_timing_read,
 * _kernels or _trace collect), in the order they were enqueued: for up to
 * `max` of them their kind, their stream and the start and end of the kernel
 * in milliseconds after the first one's start (any output may be NULL).
 * Returns the number written, or a negative status. */
int attnres_timing_trace(int max, int* kinds, uint64_t* streams, double* start_ms, double* end_ms);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
