/*
 * dflash2.h -- C ABI of the DFlash 2 draft-select-verify step on MI355X (gfx950).
 *
 * The step (per block of L drafted positions):
 *   1. two-tap local conv            dflash2_twotap_conv
 *   2. LM-head logits + top-16       dflash2_logits_topk  (= dflash2_lmhead_logits_tilemax
 *                                                            then dflash2_topk16_tilemax;
 *                                    without a logits buffer, bf16: dflash2_lmhead_candidates
 *                                                            then dflash2_topk16_candidates)
 *   3. adjacent-pair scores          dflash2_pair_score
 *   4. max-plus path walk            dflash2_path_select
 *   5. greedy verification           dflash2_verify_greedy
 *
 * Variants that follow the pages more literally:
 *   per-16-channel conv corrections  dflash2_twotap_conv_mm
 *   context-gated pair scores        dflash2_context_gate, dflash2_pair_score_gated
 *   best-successor (greedy) walk     dflash2_path_select_mode(..., DFLASH2_PATH_GREEDY, ...)
 *   steps 3-5 in one launch          dflash2_pair_select_verify
 *   scores + sampling walk, one launch  dflash2_pair_sample (_mode: whole-path draws)
 *   sampling at T > 0, lossless      dflash2_path_sample (_mode), dflash2_target_lse,
 *   rejection verification           dflash2_verify_rejection
 *                                    (dflash2_verify_rejection_lazy: no lse pass;
 *                                    dflash2_verify_rejection_staged: the first
 *                                    rows of every block summed up front)
 *
 * Sources are cited by page title and section:
 *   [POST]   "DFlash 2: Keep Drafting Parallel" (Inco AI).
 *   [GLONCE] "Inco AI's DFlash 2 lifts LLM decoding output 16-25%".
 *
 * Conventions shared by every call
 *   - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a pointer past the call.
 *   - Tensors are dense row-major, last index fastest.
 *   - Each call validates its arguments on the host BEFORE launching anything.
 *     On failure it returns a negative dflash2_status and no output is
 *     touched.  On success it has only enqueued kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and returns
 *     without synchronising; a fault inside a kernel surfaces at the caller's
 *     next synchronisation.  Launch errors return DFLASH2_EHIP.
 *   - Calls are re-entrant and keep no state; concurrent calls on different
 *     streams may share read-only inputs.
 *   - Token ids are int32 in [0, V).  Kernels never read outside their
 *     buffers: an id outside [0, V) yields NaN scores instead of a read.
 *   - dtype selects the storage type of activations and weights:
 *     DFLASH2_F32 (fp32) or DFLASH2_BF16 (bf16).  Accumulation is fp32,
 *     except where a call states otherwise (the convs evaluate in fp64).
 *     The LM-head calls also take DFLASH2_BF16_PACKED: bf16 h with W
 *     re-laid out once by dflash2_lmhead_pack.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH2_OK = 0,
  DFLASH2_EINVAL = -1,        /* bad pointer, size, shape or aliasing */
  DFLASH2_EUNSUPPORTED = -2,  /* valid request the library does not implement */
  DFLASH2_EHIP = -3,          /* a HIP launch or runtime call failed */
  DFLASH2_EWORKSPACE = -4,    /* workspace missing or smaller than queried */
  DFLASH2_ESCRATCH = -5       /* larger than the fixed scratch of an allocation-free call */
} dflash2_status;

typedef enum {
  DFLASH2_F32 = 0,
  DFLASH2_BF16 = 1,
  DFLASH2_BF16_PACKED = 2 /* LM-head calls only: bf16 h, W from dflash2_lmhead_pack */
} dflash2_dtype;

/* Path walks of dflash2_path_select_mode. */
typedef enum { DFLASH2_PATH_VITERBI = 0, DFLASH2_PATH_GREEDY = 1 } dflash2_path_mode;
/* What a sampling walk draws: each position from its chosen predecessor's
 * row (CHAIN), or the whole path from exp(score / T) (PATH). */
typedef enum { DFLASH2_SAMPLE_CHAIN = 0, DFLASH2_SAMPLE_PATH = 1 } dflash2_sample_mode;

#define DFLASH2_TOPK 16      /* candidates per position ([POST] "A lightweight path selector") */
#define DFLASH2_MAX_L 64     /* longest block the path walk accepts */
#define DFLASH2_MAX_RANK 256 /* largest pair-factor rank */

/* Library version as 10000*major + 100*minor + patch. */
int dflash2_version(void);

/* Static text for a status code. */
const char* dflash2_strerror(int status);

/*
 * Two-tap dynamic depthwise conv over each block.
 * [POST] "A lightweight local convolution", eq. Conv_k and Fig. 4:
 *   y[b,t,c] = (k0[c] + D[b,t,g(c),0]) * x[b,t,c] + (k1[c] + D[b,t,g(c),1]) * p[b,t,c]
 *   p[b,t,:] = x[b,t-1,:] for t > 0, anchor_h[b,:] for t = 0 (the last verified
 *              token's representation; zeros when anchor_h is NULL)
 *   D[b,t,g,j] = sum_c x[b,t,c] * proj[c, 2g+j]   (0 when proj is NULL)
 *   g(c) = c / (H / groups)
 * x, y     [B, L, H] of dtype; y must not overlap x, anchor_h, k0, k1 or proj.
 * anchor_h [B, H] of dtype, or NULL.
 * k0, k1   [H] fp32 base taps.
 * proj     [H, 2*groups] fp32 correction map, or NULL for static taps.
 * groups   >= 1, divides H (ignored when proj is NULL).
 * B >= 0 (0 is a no-op), L >= 1, H >= 8 with H % 8 == 0.  All pointers 16-byte aligned.
 * Arithmetic in fp64 (taps, corrections, products and the sum); each output is rounded
 * once to dtype (round to nearest even).
 * EUNSUPPORTED with proj when B*L > 2^31 - 1, or when groups > 1 and (H + 2*groups)
 * doubles exceed 64 KiB of LDS.
 */
int dflash2_twotap_conv(const void* x, const void* anchor_h, void* y,
                        const float* k0, const float* k1,
                        const float* proj, int groups,
                        int B, int L, int H, int dtype, void* stream);

/*
 * Two-tap conv with the corrections on the matrix cores, for many groups.
 * [POST] "A lightweight local convolution": each coefficient is a base tap
 * plus a small correction from the current hidden state, one correction
 * shared by every 16 channels (groups = H / 16).  At that width the
 * corrections of a batch are a matrix product, so the map is given
 * transposed, in bf16, like a weight matrix:
 *   D[b,t,g,j] = sum_c x[b,t,c] * projT[2g+j, c]
 * and y is dflash2_twotap_conv's formula with these D.
 * projT [2*groups, H] bf16; groups >= 1 divides H; dtype must be
 * DFLASH2_BF16 (DFLASH2_F32 returns DFLASH2_EUNSUPPORTED).  Other arguments
 * as for dflash2_twotap_conv; y must not overlap x, anchor_h, k0, k1 or projT.
 * D is accumulated in fp32 from the exact bf16 products; the mix is
 * evaluated in fp64 from it and rounded once to bf16.  With groups of at
 * least 16 channels the call may compute D in four K quarters whose fp32
 * partial sums it keeps in y's rows until it writes them (y is then scratch
 * as well as output; it must not overlap the inputs in any case).
 */
int dflash2_twotap_conv_mm(const void* x, const void* anchor_h, void* y,
                           const float* k0, const float* k1, const void* projT, int groups,
                           int B, int L, int H, int dtype, void* stream);

/*
 * LM-head logits: logits[m, n] = sum_c h[m, c] * W[n, c]  (fp32 accumulate).
 * [POST] "A lightweight path selector": the unary term of every pair score is
 * the drafter's own logit, computed once and reused.
 * h [M, H] of dtype, W [V, H] of dtype (K-contiguous: "NT" product),
 * logits [M, V] fp32.  M >= 0, H >= 8 with H % 8 == 0, V >= 16; h, W, logits
 * 16-byte aligned.
 * bf16 operands run on the gfx950 bf16 matrix cores.  With
 * DFLASH2_BF16_PACKED, W is the output of dflash2_lmhead_pack for the same
 * V and H (dflash2_lmhead_pack_bytes bytes); the logits are bit for bit those
 * of DFLASH2_BF16 with the unpacked W.
 */
int dflash2_lmhead_logits(const void* h, const void* W, float* logits,
                          int M, int H, int V, int dtype, void* stream);

/*
 * The LM-head weight in the bf16 GEMM's tile layout, for the repeated calls
 * of a decoding loop: W [V, H] bf16 row-major is copied to
 *   Wp[ceil(V / 256)][ceil(H / 64)][256][64]   (rows past V, columns past H: 0)
 * so every 256 x 64 slice the GEMM reads is one contiguous 32 KiB run (fewer
 * DRAM page switches than 256 rows of 128 bytes at a stride of H).
 * dflash2_lmhead_pack_bytes returns the size of Wp (0 for invalid V, H).
 * dflash2_lmhead_pack: V >= 1, H >= 8 with H % 8 == 0, H <= 2^21; W and Wp
 * 16-byte aligned, not overlapping.  Wp is fully written (padding included).
 */
size_t dflash2_lmhead_pack_bytes(int V, int H);
int dflash2_lmhead_pack(const void* W, void* Wp, int V, int H, void* stream);

/* Columns covered by one tile maximum (see dflash2_lmhead_logits_tilemax). */
#define DFLASH2_TILEMAX_COLS 256

/*
 * dflash2_lmhead_logits that also writes the row maxima of every
 * DFLASH2_TILEMAX_COLS-column tile of the logits:
 *   tilemax[m, t] = max over n in [256 t, min(256 t + 256, V)) of logits[m, n]
 * (NaN entries ignored; a tile with nothing else gives -inf).
 * tilemax [M, ceil(V / 256)] fp32,
 * 4-byte aligned, overlapping nothing else.  The bf16 GEMM computes them in
 * its epilogue from the values it stores; fp32 runs one extra pass.
 */
int dflash2_lmhead_logits_tilemax(const void* h, const void* W, float* logits, float* tilemax,
                                  int M, int H, int V, int dtype, void* stream);

/*
 * dflash2_topk16 given the tile maxima of the same logits (exactly as
 * dflash2_lmhead_logits_tilemax writes them).  The 16 largest tile maxima
 * are 16 distinct elements, so every top-16 element lies in a tile whose
 * maximum reaches the 16th largest maximum; only those tiles are read
 * (usually 16 of them).  Same order, ties and special values as
 * dflash2_topk16, bit for bit.  Needs no workspace.
 */
int dflash2_topk16_tilemax(const float* logits, const float* tilemax, float* top_val,
                           int32_t* top_idx, int M, int V, int K, void* stream);

/* Bytes of workspace dflash2_topk16 needs for an [M, V] problem with K = 16. */
size_t dflash2_topk16_workspace(int M, int V, int K);

/*
 * Per-row top-16 of fp32 logits [M, V]:
 * [POST] "A lightweight path selector": the drafter keeps its 16 best tokens
 * at every position.  Order: value descending, equal values by lower token id
 * first.  -0 compares equal to +0 and is reported as +0; NaN ranks as -inf
 * and is reported as -inf.
 * top_val [M, 16] fp32, top_idx [M, 16] int32 (slot 0 = top-1).
 * K must be 16; V >= 16.  workspace: at least dflash2_topk16_workspace bytes
 * (may be NULL when that is 0), 256-byte aligned.
 */
int dflash2_topk16(const float* logits, float* top_val, int32_t* top_idx,
                   int M, int V, int K, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Workspace for dflash2_logits_topk: the tile maxima, and the logits too
 * when logits_given == 0 (the caller passes no logits buffer); for bf16
 * operands without a logits buffer also the candidate form's parts (below):
 * 64 bytes per row and 36 bytes per row and 256-column tile.
 */
size_t dflash2_logits_topk_workspace(int M, int H, int V, int K, int dtype, int logits_given);

/*
 * LM-head logits and the per-position top-16 candidates in one call.
 * [POST] "A lightweight path selector": the unary term of every pair score
 * is the drafter's own logit, computed once per position, and the walk
 * chooses among the 16 best tokens of each position.
 *   logits[m, n] = sum_c h[m, c] * W[n, c]   (fp32 accumulation, fp32 out)
 *   top_val / top_idx [M, 16]: the 16 largest logits of row m, value
 *   descending, equal values by lower token id (as dflash2_topk16).
 * h [M, H] and W [V, H] of dtype (W may be packed, DFLASH2_BF16_PACKED),
 * 16-byte aligned.  With a logits buffer it runs
 * dflash2_lmhead_logits_tilemax then dflash2_topk16_tilemax, the tile maxima
 * in the workspace.  logits may be NULL: with fp32 operands the workspace
 * then holds the logits (same two calls); with bf16 operands the call runs
 * the candidate form below and no [M, V] logits are written.  Either way
 * top_val / top_idx are the same bit for bit.  The workspace is required
 * (256-byte aligned) whenever M > 0.  K must be 16.  Errors as for the calls
 * it runs; nothing is launched unless every check passes.
 */
int dflash2_logits_topk(const void* h, const void* W, float* logits,
                        float* top_val, int32_t* top_idx,
                        int M, int H, int V, int K, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * dflash2_logits_topk with logits == NULL and bf16 operands (DFLASH2_BF16 or
 * DFLASH2_BF16_PACKED) runs the GEMM in a candidate form that leaves out
 * most of the [M, V] logits, and is these two calls on its workspace
 * (dflash2_logits_topk_workspace(M, H, V, 16, dtype, 0) bytes, 256-byte
 * aligned), which a caller may also make itself (to time or schedule the
 * two launches apart; nothing may touch the workspace in between).
 * [POST] "A lightweight path selector": only the 16 best tokens of each
 * position are used, so the logits outside them need not leave the chip.
 *   dflash2_lmhead_candidates: the GEMM.  Every row keeps 16 running group
 *     maxima (group = 256-column tile index mod 16, reset at the start of
 *     the call); once all 16 are set, their minimum is a lower bound on the
 *     row's 16th largest logit.  A row of a tile that finishes with that
 *     bound in hand writes only its values at or above it (at most 4, as
 *     value and column); a row without the bound, or with more than 4 such
 *     values, writes its 256 logits.  Tile maxima as for
 *     dflash2_lmhead_logits_tilemax.  EUNSUPPORTED for fp32 operands; other
 *     errors as for dflash2_lmhead_logits; the workspace may not overlap h
 *     or W.
 *   dflash2_topk16_candidates: the top-16 from that workspace (M and V as
 *     given to the GEMM): the tiles whose maximum reaches the 16th largest
 *     tile maximum, each read whole or as its slots.  Results bit for bit
 *     those of dflash2_logits_topk with a logits buffer (the same GEMM
 *     values, the same order and ties).  top_val / top_idx may not overlap
 *     the workspace.
 * Both return DFLASH2_EWORKSPACE for a missing, short or misaligned
 * workspace and DFLASH2_EINVAL for K != 16 or bad sizes.
 */
int dflash2_lmhead_candidates(const void* h, const void* W, int M, int H, int V, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);
int dflash2_topk16_candidates(const void* workspace, size_t workspace_bytes, float* top_val,
                              int32_t* top_idx, int M, int H, int V, int K, void* stream);

/*
 * Measurement aid, not a step of the path: the attainable matrix-core rate
 * behind the LM-head GEMM's roofline.  `workgroups` workgroups of the
 * GEMM's eight waves each issue `iters` x 8 v_mfma_f32_32x32x16_bf16 on
 * register operands loaded once from `operands` (bf16 bit patterns,
 * dflash2_probe_mfma_operand_bytes(workgroups) bytes, 16-byte aligned: the
 * bits set the power the matrix cores draw); no other memory traffic.
 * Work: workgroups * 8 * iters * 8 * 32768 flop.  out [workgroups * 512]
 * fp32 receives per-thread sums of the accumulators (so nothing is
 * optimised away).  EINVAL for iters < 1, workgroups outside [1, 2^20],
 * null, misaligned or overlapping buffers.
 */
size_t dflash2_probe_mfma_operand_bytes(int workgroups);
int dflash2_probe_mfma(const void* operands, int workgroups, int iters, float* out, void* stream);

/* Bytes of the fixed device scratch of dflash2_logits_topk_noalloc (16 MiB). */
#define DFLASH2_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * dflash2_logits_topk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * allocation.  It takes no workspace and calls no allocating routine: the
 * tile maxima between the GEMM and the top-16 (M * ceil(V / 256) * 4 bytes)
 * live in a fixed device array of DFLASH2_NOALLOC_SCRATCH_BYTES that each
 * GPU the library runs on holds until the process ends (its address is
 * looked up on the first call made on that device; the stream must belong
 * to the current device).
 *   logits [M, V] fp32 is required here (a caller-given output, 16-byte
 *   aligned); every other argument, result and error is as for
 *   dflash2_logits_topk, and the results equal its results bit for bit.
 * Returns DFLASH2_ESCRATCH, before any launch, when the tile maxima do not
 * fit (M * ceil(V / 256) * 4 > DFLASH2_NOALLOC_SCRATCH_BYTES; at V = 151936
 * that is M > 7061).  Every call on one GPU shares that GPU's array and
 * leaves its tile maxima there; each call writes all the entries it reads,
 * so nothing needs clearing, but calls that overlap in time on one GPU
 * (other streams, other threads) race on the array and must be serialised
 * by the caller.
 */
int dflash2_logits_topk_noalloc(const void* h, const void* W, float* logits,
                                float* top_val, int32_t* top_idx,
                                int M, int H, int V, int K, int dtype, void* stream);

/*
 * Adjacent-pair scores.  [POST] "A lightweight path selector", eq. S_t(a,b):
 * the candidate's own logit plus a low-rank match with the previous token, in
 * the ungated form (context gate = 1) with per-token factors U, V:
 *   S0[b, j]        = top_val[b,0,j] + U[anchor_tok[b]] . Vf[top_idx[b,0,j]]
 *   S[b, t-1, i, j] = top_val[b,t,j] + U[top_idx[b,t-1,i]] . Vf[top_idx[b,t,j]],  t = 1..L-1
 * top_val [B, L, 16] fp32, top_idx [B, L, 16] int32 in [0, V).
 * anchor_tok [B] int32 (last verified token), or NULL for no match term at t = 0.
 * U, Vf [V, r] of dtype; 1 <= r <= 256.
 * S0 [B, 16] fp32; S [B, L-1, 16, 16] fp32 (may be NULL when L == 1).
 * fp32 accumulation; ids outside [0, V) give NaN entries.
 */
int dflash2_pair_score(const float* top_val, const int32_t* top_idx,
                       const int32_t* anchor_tok, const void* U, const void* Vf,
                       int B, int L, int V, int r, int dtype,
                       float* S0, float* S, void* stream);

/*
 * Context gate of the gated pair score.  [POST] "A lightweight path selector",
 * eq. S_t(a,b): the match of A(a) with B(b) is weighted per channel by H(h_t),
 * computed from the drafter's hidden state at position t.  The pages give no
 * form for H; this call takes a sigmoid of a linear map:
 *   gate[m, k] = 1 / (1 + exp(-sum_c h[m, c] * Wg[k, c]))
 * h [M, H] of dtype (the hidden states fed to the LM head, m = b*L + t),
 * Wg [r, H] of dtype (K-contiguous), gate [M, r] fp32.  M >= 0, H >= 8 with
 * H % 8 == 0, 1 <= r <= 256.  h and Wg 16-byte aligned, gate 4-byte aligned,
 * gate must not overlap h or Wg.  bf16 operands run on the matrix cores;
 * fp32 accumulation, fp32 sigmoid.
 */
int dflash2_context_gate(const void* h, const void* Wg, float* gate,
                         int M, int H, int r, int dtype, void* stream);

/*
 * Gated pair scores: dflash2_pair_score with the previous-token factor
 * scaled channel by channel by the gate of the CURRENT position,
 *   S0[b, j]        = top_val[b,0,j] + (U[anchor_tok[b]] * gate[b,0]) . Vf[top_idx[b,0,j]]
 *   S[b, t-1, i, j] = top_val[b,t,j] + (U[top_idx[b,t-1,i]] * gate[b,t]) . Vf[top_idx[b,t,j]]
 * gate [B, L, r] fp32 (required, 4-byte aligned, not overlapping the outputs);
 * a gate of all ones gives dflash2_pair_score's result.  Every other
 * argument, limit and error is as for dflash2_pair_score.
 */
int dflash2_pair_score_gated(const float* top_val, const int32_t* top_idx,
                             const int32_t* anchor_tok, const void* U, const void* Vf,
                             const float* gate, int B, int L, int V, int r, int dtype,
                             float* S0, float* S, void* stream);

/*
 * Max-plus (Viterbi) path over the pair scores, one wavefront per block.
 * [POST] "A lightweight path selector" walks the precomputed scores serially
 * from the last verified token; this call takes the exact best path:
 *   d_0 = S0,  d_t[j] = max_i fl32(d_{t-1}[i] + S[t-1,i,j]),
 * the lowest slot wins every tie (each max and the final argmax).
 * S0 [B,16], S [B,L-1,16,16] (NULL allowed when L == 1), 1 <= L <= 64.
 * path_slot [B, L] int32 slots; path_score [B] fp32 = d_{L-1}[final slot].
 * top_idx [B, L, 16] and path_tok [B, L]: both given (path_tok[b,t] =
 * top_idx[b,t,path_slot[b,t]]) or both NULL.
 * Scores are expected finite (or -inf); a NaN score leaves the slot it
 * decides unspecified (but in [0, 16)).
 */
int dflash2_path_select(const float* S0, const float* S, const int32_t* top_idx,
                        int B, int L, int32_t* path_slot, int32_t* path_tok,
                        float* path_score, void* stream);

/*
 * dflash2_path_select with a choice of walk.  DFLASH2_PATH_VITERBI is
 * dflash2_path_select.  DFLASH2_PATH_GREEDY is the pages' own walk ([POST]
 * "A lightweight path selector": from the last verified token, follow the
 * best successor at each step):
 *   p_0 = argmax_j S0[j],  p_t = argmax_j S[t-1, p_{t-1}, j]  (lowest slot on ties),
 *   path_score = fl32 running sum S0[p_0] + S[0,p_0,p_1] + ... in position order.
 * Greedy mode needs S 16-byte aligned (when L > 1).  Other mode values: EINVAL.
 */
int dflash2_path_select_mode(const float* S0, const float* S, const int32_t* top_idx,
                             int B, int L, int mode, int32_t* path_slot, int32_t* path_tok,
                             float* path_score, void* stream);

/*
 * Sampling walk at temperature T > 0.  [POST] "A lightweight path selector":
 * besides the greedy walk, sampling draws from the same precomputed scores.
 * The sampling twin of the greedy walk, with the caller's uniforms:
 *   q[b,0,:] = softmax(S0[b] / T),  q[b,t,:] = softmax(S[b,t-1,p_{t-1},:] / T),
 *   p_t = first slot j with u[b,t] < q[b,t,0] + ... + q[b,t,j]
 *         (if rounding leaves u above the last sum: the last slot with q > 0).
 * u [B, L] fp32 in [0, 1).  q [B, L, 16] fp32 receives each position's
 * proposal distribution (what dflash2_verify_rejection needs).  Scores must
 * be finite or -inf with at least one finite per row.  S 16-byte aligned.
 * Other arguments as for dflash2_path_select.  fp32 softmax and sums.
 */
int dflash2_path_sample(const float* S0, const float* S, const int32_t* top_idx,
                        const float* u, float temperature, int B, int L,
                        int32_t* path_slot, int32_t* path_tok, float* q, void* stream);

/*
 * dflash2_path_sample with a choice of what is drawn.  DFLASH2_SAMPLE_CHAIN
 * is dflash2_path_sample.  DFLASH2_SAMPLE_PATH draws the whole slot path
 * from the distribution the same scores define over all 16^L paths, the
 * sampling twin of the max-plus walk ([POST] "A lightweight path selector":
 * sampling draws from the precomputed scores):
 *   P(p) proportional to exp(score(p) / T),
 *   score(p) = S0[p_0] + sum_t S[t-1, p_{t-1}, p_t].
 * Drawn by backward messages, then forward draws:
 *   beta[L-1][.] = 0,  beta[t][i] = log sum_j exp(S[b,t,i,j] / T + beta[t+1][j]),
 *   q[b,0,:] = softmax(S0[b] / T + beta[0]),
 *   q[b,t,:] = softmax(S[b,t-1,p_{t-1},:] / T + beta[t]),
 * each p_t by inverse CDF with u[b,t] as above, so q[b,t] is position t's
 * proposal given the slots before it (what dflash2_verify_rejection needs).
 * fp32 messages (each row shifted by its maximum), softmax and sums.  Other
 * mode values: EINVAL.  Everything else as for dflash2_path_sample.
 */
int dflash2_path_sample_mode(const float* S0, const float* S, const int32_t* top_idx,
                             const float* u, float temperature, int B, int L, int mode,
                             int32_t* path_slot, int32_t* path_tok, float* q, void* stream);

/*
 * Log-sum-exp of target logits at temperature T:
 *   lse[r] = log sum_v exp(z[r, v] / T),  z [R, V] fp32 (16-byte aligned),
 * lse [R] fp32.  -inf entries carry no mass.  One pass over z.
 */
int dflash2_target_lse(const float* z, int R, int V, float temperature, float* lse,
                       void* stream);

/*
 * Lossless verification of a sampled path.  [POST] "A lightweight path
 * selector": rejection sampling restores the target's exact distribution.
 * The speculative-sampling rule: with p_t = softmax(z[b,t,:] / T) (lse from
 * dflash2_target_lse on the same z) and q_t the proposal of position t,
 *   accept x_t = path_tok[b,t] while u_acc[b,t] * q[b,t,path_slot[b,t]] < p_t(x_t);
 *   n = number accepted, accept_len[b] = n + 1;
 *   next_tok[b] = a draw from max(0, p_n - q_n) (n < L; q_n lives on the
 *   candidates top_idx[b,n,:]) or from p_L (n = L), by inverse CDF in token
 *   order with u_res[b] scaled by the residual mass.
 * z [B, L+1, V] fp32 (position L: the token after a fully accepted block),
 * lse [B, L+1], u_acc [B, L], u_res [B], q [B, L, 16], path_slot/path_tok
 * [B, L], top_idx [B, L, 16].  V >= 16, V <= 4194304.  fp32 arithmetic.
 */
int dflash2_verify_rejection(const int32_t* path_slot, const int32_t* path_tok,
                             const float* q, const int32_t* top_idx, const float* z,
                             const float* lse, float temperature, const float* u_acc,
                             const float* u_res, int B, int L, int V,
                             int32_t* accept_len, int32_t* next_tok, void* stream);

/*
 * dflash2_verify_rejection without the lse pass: the same rule, with each
 * row's log-sum-exp computed inside the call and only for the rows the test
 * reaches.  Row t is read once, in 256-token tiles whose maxima and sums stay
 * on chip; they give lse for the test at t and, at the row where the test
 * stops, the tile masses of the draw.  A block that stops at position n
 * reads n + 1 rows of z, where dflash2_target_lse and
 * dflash2_verify_rejection together read L + 2.  The result follows the same
 * rule as dflash2_target_lse then dflash2_verify_rejection; rounding of the
 * sums differs, so a decision or a draw within a few fp32 ulps of the mass
 * of a boundary can differ.  Arguments as for dflash2_verify_rejection
 * without lse; V <= 2097152 (larger: DFLASH2_EUNSUPPORTED).  fp32 arithmetic.
 */
int dflash2_verify_rejection_lazy(const int32_t* path_slot, const int32_t* path_tok,
                                  const float* q, const int32_t* top_idx, const float* z,
                                  float temperature, const float* u_acc, const float* u_res,
                                  int B, int L, int V, int32_t* accept_len, int32_t* next_tok,
                                  void* stream);

/*
 * dflash2_verify_rejection_lazy with the first `rows` target rows of every
 * block summed up front, all blocks at once.  [POST] "A lightweight path
 * selector": rejection sampling restores the target's exact distribution.
 * A first launch sums rows 0 .. rows-1 of every block (one wave per batch of
 * 2048 tokens) into the workspace; the second runs the accept tests and the
 * draw, one workgroup per block, and reads a row of z itself only when the
 * test reaches a position past those rows.  Every row is summed with the
 * same arithmetic, in the same order, as in dflash2_verify_rejection_lazy,
 * so accept_len and next_tok are bit for bit those of that call.  A block
 * that stops at position n reads max(n + 1, rows) rows of z.
 * Arguments as for dflash2_verify_rejection_lazy, plus:
 *   rows       1 .. L + 1 (else DFLASH2_EINVAL);
 *   workspace  device memory of at least
 *              dflash2_verify_rejection_staged_workspace(B, L, V, rows)
 *              bytes, 4-byte aligned, overlapping no input or output; the
 *              call overwrites it (DFLASH2_EINVAL if NULL or too small).
 * V <= 2097152 (larger: DFLASH2_EUNSUPPORTED).  fp32 arithmetic.
 * dflash2_verify_rejection_staged_workspace returns the workspace bytes, or
 * 0 when B, L, V or rows is out of range.
 */
size_t dflash2_verify_rejection_staged_workspace(int B, int L, int V, int rows);
int dflash2_verify_rejection_staged(const int32_t* path_slot, const int32_t* path_tok,
                                    const float* q, const int32_t* top_idx, const float* z,
                                    float temperature, const float* u_acc, const float* u_res,
                                    int B, int L, int V, int rows, void* workspace,
                                    size_t workspace_bytes, int32_t* accept_len,
                                    int32_t* next_tok, void* stream);

/*
 * Greedy verification.  [POST] "The right token is already in the candidates",
 * Table 1: the acceptance length counts the verifier's next token.
 *   n = number of leading t with path_tok[b,t] == target[b,t]  (0 <= n <= L)
 *   accept_len[b] = n + 1,  next_tok[b] = target[b, n]
 * path_tok [B, L], target [B, L+1] (target[b, L] is the token after a fully
 * accepted block), accept_len [B], next_tok [B] (may be NULL).
 */
int dflash2_verify_greedy(const int32_t* path_tok, const int32_t* target,
                          int B, int L, int32_t* accept_len, int32_t* next_tok,
                          void* stream);

/*
 * Steps 3-5 in one launch: dflash2_pair_score_gated (gate != NULL) or
 * dflash2_pair_score (gate == NULL), then dflash2_path_select_mode with
 * `mode`, then dflash2_verify_greedy on the walked tokens, for each block in
 * one workgroup with the scores kept on chip.  [POST] "A lightweight path
 * selector" (scores, walk) and "The right token is already in the
 * candidates", Table 1 (acceptance length).  The outputs are bit for bit
 * those of the three calls.  Arguments, layouts, limits and errors are
 * theirs, with these differences: S0 and S are optional outputs (NULL: the
 * scores stay on chip); path_tok may be NULL; target [B, L+1], accept_len [B]
 * are required, next_tok [B] may be NULL.  Every pointer is 4-byte aligned
 * (U and Vf: 2-byte for bf16), and no output may overlap an input or another
 * output.
 */
int dflash2_pair_select_verify(const float* top_val, const int32_t* top_idx,
                               const int32_t* anchor_tok, const void* U, const void* Vf,
                               const float* gate, const int32_t* target, int B, int L, int V,
                               int r, int dtype, int mode, float* S0, float* S,
                               int32_t* path_slot, int32_t* path_tok, float* path_score,
                               int32_t* accept_len, int32_t* next_tok, void* stream);

/*
 * The sampling twin of dflash2_pair_select_verify: dflash2_pair_score_gated
 * (gate != NULL) or dflash2_pair_score (gate == NULL), then
 * dflash2_path_sample, for each block in one workgroup with the scores kept
 * on chip.  [POST] "A lightweight path selector" (scores; sampling from the
 * same scores).  The outputs are bit for bit those of the two calls.
 * Arguments, layouts, limits and errors are theirs, with these differences:
 * S0 and S are optional outputs (NULL: the scores stay on chip); path_tok
 * may be NULL; u [B, L], path_slot [B, L] and q [B, L, 16] are required.
 * Every pointer is 4-byte aligned (U and Vf: 2-byte for bf16), and no output
 * may overlap an input or another output.
 */
int dflash2_pair_sample(const float* top_val, const int32_t* top_idx,
                        const int32_t* anchor_tok, const void* U, const void* Vf,
                        const float* gate, const float* u, float temperature, int B, int L,
                        int V, int r, int dtype, float* S0, float* S, int32_t* path_slot,
                        int32_t* path_tok, float* q, void* stream);

/*
 * dflash2_pair_sample with the sampling walk's mode (dflash2_sample_mode,
 * as in dflash2_path_sample_mode); bit for bit dflash2_pair_score(_gated)
 * followed by dflash2_path_sample_mode.  Other mode values: EINVAL.
 */
int dflash2_pair_sample_mode(const float* top_val, const int32_t* top_idx,
                             const int32_t* anchor_tok, const void* U, const void* Vf,
                             const float* gate, const float* u, float temperature, int B, int L,
                             int V, int r, int dtype, int mode, float* S0, float* S,
                             int32_t* path_slot, int32_t* path_tok, float* q, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH2_H */
