/*
 * wf_attn.h -- C ABI of libwfattn.so: multi-head self-attention over a video
 * diffusion transformer's 3D latent token grid on AMD Instinct MI355X (gfx950).
 *
 * Two forms of the same operation, as described in "Anatomy of Wan2.2's 53.6x
 * speedup" (zharfai.com, review of Baseten's Wan2.2 work):
 *
 *   - dense attention, section "Why video attention becomes the bottleneck":
 *     every query token of the T x H x W grid against every key token,
 *     O = softmax(scale * Q K^T) V per (batch, head), no mask;
 *   - Video Sparse Attention (VSA), section "VSA selects cubes": the grid is
 *     padded to multiples of 4 and cut into 4x4x4 cubes of 64 tokens; a coarse
 *     stage scores cube-mean queries against cube-mean keys and keeps the
 *     top-k key cubes of every query cube; a fine stage runs token-level
 *     attention of each query cube over its kept cubes only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Tensors are [B][Hh][N][D] row-major and contiguous, tokens in row-major
 *   (t, h, w) order: n = (t*H + h)*W + w.  q, k, v are bfloat16 (passed as raw
 *   pointers to 2-byte elements), outputs are float32.  Every pointer is a
 *   device pointer (hipMalloc'd or equivalent) aligned to 16 bytes.
 *   D (head dimension) is 64 or 128 for dense attention and 128 for VSA.
 *
 *   Ownership: the caller allocates and frees every buffer, workspaces
 *   included.  The library never allocates or frees device memory and never
 *   synchronises the stream (the opt-in WF_VALIDATE=1 index check in
 *   wf_vsa_fine is the only exception, and it says so).  Work is enqueued on
 *   `stream` (a hipStream_t; NULL means the null stream) in call order.
 *   Calls are reentrant; concurrent calls must use distinct workspaces.
 *   A call enqueues kernel launches only (no memset, no copy), so calls may
 *   be captured into a HIP graph and replayed; a replay reads the buffers'
 *   contents at replay time (WF_VALIDATE=1 and wf_profile_enable(1) are not
 *   for use under capture: they synchronise or record events).
 *
 *   Errors: every entry point returns a wf_status.  Argument checks run on
 *   the host before anything is enqueued; on failure nothing is enqueued and
 *   wf_last_error_detail() (thread-local) says which argument was rejected.
 *   WF_ERR_HIP reports a launch error from the HIP runtime.  There is no
 *   fallback path: unsupported input is rejected, never rerouted.
 */
#ifndef WF_ATTN_H
#define WF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wf_status {
  WF_OK = 0,
  WF_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad size, non-finite scale */
  WF_ERR_UNSUPPORTED = 2,  /* a head dimension or size the library does not handle */
  WF_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes query */
  WF_ERR_BAD_INDEX = 4,    /* a top-k plan that is out of range or not strictly ascending */
  WF_ERR_HIP = 5           /* the HIP runtime reported an error */
} wf_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* wf_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* wf_last_error_detail(void);

/* ABI version of this library; bumped on any signature change. */
int32_t wf_abi_version(void);

/* ------------------------------------------------------------------ dense */

/* Workspace bytes wf_attn_dense needs for these sizes (0 on invalid sizes). */
size_t wf_attn_dense_workspace_bytes(int32_t B, int32_t Hh, int32_t N, int32_t D);

/*
 * Dense bidirectional attention ("Why video attention becomes the
 * bottleneck"; the Wan2.1 blog, bafh001.com, section 4.2, calls it
 * non-causally with QK^T, softmax and PV fused on chip).  Per (b, h):
 *     o[i]   = sum_j softmax_j(scale * q[i] . k[j]) v[j]
 *     lse[i] = log sum_j exp(scale * q[i] . k[j])          (natural log)
 *
 *   q, k, v    bf16 [B][Hh][N][D], read only.
 *   o          fp32 [B][Hh][N][D], written.
 *   lse        fp32 [B][Hh][N], written; may be NULL.
 *   N          tokens (T*H*W), 1 <= N, and one head's K (N rounded up to 64,
 *              times D bf16) below 2 GiB: 64*ceil(N/64)*D*2 < 2^31, else
 *              WF_ERR_UNSUPPORTED (N <= 8,388,544 at D = 128).
 *   D          64 or 128.
 *   scale      finite and > 0 (1/sqrt(D) for the standard operation).
 *   workspace  device scratch of at least wf_attn_dense_workspace_bytes(),
 *              16-byte aligned; contents on entry are ignored and the call
 *              leaves it holding V transposed, one D x 64 tile per 64 keys
 *              of each head.
 * The softmax keeps a running row maximum (section "Fixed-max softmax is a
 * numerical contract" of the Wan2.2 review), so any finite input yields
 * finite output.
 */
int32_t wf_attn_dense(const void* q, const void* k, const void* v, float* o, float* lse,
                      int32_t B, int32_t Hh, int32_t N, int32_t D, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and result bits as wf_attn_dense, with the transposed
 * V kept in the library's own static scratch instead of a caller workspace.
 * The scratch is one file-scope device array of WF_DENSE_NOALLOC_SCRATCH_BYTES
 * per GPU, taken on that GPU's first call and held until the process ends; the
 * call allocates and frees nothing.  Every call on a GPU uses the same array,
 * so calls that overlap on one GPU (another stream, another thread) race and
 * must be serialised by the caller; calls in one stream are ordered as usual.
 *
 *   Arguments as wf_attn_dense, without the workspace.  Sizes whose
 *   wf_attn_dense_workspace_bytes() exceeds WF_DENSE_NOALLOC_SCRATCH_BYTES
 *   (128 MiB: e.g. up to 16 heads of 32,760 tokens at D = 128) return
 *   WF_ERR_WORKSPACE with nothing enqueued.
 */
#define WF_DENSE_NOALLOC_SCRATCH_BYTES (128u << 20)
int32_t wf_attn_dense_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                              int32_t B, int32_t Hh, int32_t N, int32_t D, float scale, void* stream);

/* -------------------------------------------------------------------- VSA */

/* Number of 4x4x4 cubes of a T x H x W grid after padding each side up to a
 * multiple of 4 ("VSA selects cubes": 21x30x52 gives 6x8x13 = 624); 0 if invalid. */
int32_t wf_vsa_num_cubes(int32_t T, int32_t H, int32_t W);

/* Workspace bytes that wf_vsa_coarse_topk fills and the fine-stage calls read
 * (cube-ordered Q, K and V, cube means of Q, K and V, coarse scores and their
 * row statistics, the coarse-branch output). 0 if invalid. */
size_t wf_vsa_workspace_bytes(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D);

/*
 * VSA coarse stage ("VSA selects cubes", part 1).  With C = wf_vsa_num_cubes():
 *   1. gathers q, k, v into cube order inside `workspace` (padded slots zero);
 *   2. pools cube means Qbar, Kbar, Vbar over each cube's real tokens, in fp32
 *      (Vbar is kept for the coarse-branch output);
 *   3. scores S[c][c'] = scale * Qbar[c] . Kbar[c'] to fp32 accuracy (bf16
 *      matrix cores on an exact three-part bf16 split of each fp32 mean) and
 *      records each row's softmax maximum and sum;
 *   4. writes idx[b][h][c][0..topk) = the topk key cubes c' with the largest
 *      S[c][c'], equal scores resolved toward the smaller c', listed in
 *      strictly ascending order.
 * Cube c of the padded grid is (ct*nh + ch)*nw + cw with cube coordinates
 * (ct, ch, cw) = (t/4, h/4, w/4).
 *
 *   q, k, v        bf16 [B][Hh][T*H*W][D], read only.
 *   T, H, W        real grid, each >= 1; D must be 128.
 *   topk           1 <= topk <= C.
 *   idx            int32 [B][Hh][C][topk], written.
 *   coarse_scores  fp32 [B][Hh][C][C], written; may be NULL.
 *   workspace      at least wf_vsa_workspace_bytes(); keep it untouched
 *                  between this call and wf_vsa_fine.
 */
int32_t wf_vsa_coarse_topk(const void* q, const void* k, const void* v,
                           int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                           float scale, int32_t topk, int32_t* idx, float* coarse_scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * VSA fine stage ("VSA selects cubes", part 2): each real query token of cube
 * c attends over the real key tokens of cubes idx[b][h][c][0..topk):
 *     o[i]   = sum_{j in J(c)} softmax_j(scale * q[i] . k[j]) v[j]
 *     lse[i] = log sum_{j in J(c)} exp(scale * q[i] . k[j])
 * Padded key slots are masked out; padded query slots are not written.
 *
 *   workspace      as filled by wf_vsa_coarse_topk with the same B, Hh, T, H, W, D.
 *   idx            int32 [B][Hh][C][topk]: any plan (the coarse stage's or the
 *                  caller's) with entries in [0, C) strictly ascending per row.
 *                  Without a check the kernels take it as given, but they
 *                  never read outside the workspace whatever it holds: every
 *                  key-cube copy is range-checked against the head's C cubes,
 *                  and an entry outside [0, C) reads zero keys and values (the
 *                  rows of that query cube are then meaningless, not a
 *                  fault).  With the environment variable WF_VALIDATE=1 a
 *                  check kernel runs first and the call synchronises `stream`
 *                  to return WF_ERR_BAD_INDEX on a bad plan (nothing else
 *                  enqueued).
 *   o              fp32 [B][Hh][T*H*W][D] in grid order, written.
 *   lse            fp32 [B][Hh][T*H*W], written; may be NULL.
 */
int32_t wf_vsa_fine(const void* workspace, size_t workspace_bytes, const int32_t* idx,
                    int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                    float scale, int32_t topk, float* o, float* lse, void* stream);

/*
 * VSA in one call: the coarse stage and the fine stage of wf_vsa_coarse_topk
 * followed by wf_vsa_fine (or, with a gate, wf_vsa_fine_gated) on the plan it
 * selects, with the same result (o, lse, idx and o_coarse bit for bit).  The
 * one call needs no cube-ordered copies of Q, K and V: the fine stage reads
 * q, k and v in grid order (v with LDS transpose reads), so the gather only
 * pools the cube means and moves under a third of the bytes.
 *
 *   q, k, v        bf16 [B][Hh][T*H*W][D], read only; D must be 128.
 *   topk           1 <= topk <= C.
 *   idx            int32 [B][Hh][C][topk], written (the plan, as wf_vsa_coarse_topk).
 *   gate           bf16 [B][Hh][T*H*W][D] or NULL: with a gate the call adds the
 *                  gated coarse branch, o = o_fine + gate * Oc, as wf_vsa_fine_gated.
 *   o, lse         as for wf_vsa_fine (lse may be NULL).
 *   o_coarse       fp32 [B][Hh][C][D]: Oc, written; may be NULL, and must be
 *                  NULL without a gate.
 *   workspace      at least wf_vsa_workspace_bytes(); its contents afterwards
 *                  are not a workspace that wf_vsa_fine or wf_vsa_fine_gated
 *                  can take (the cube-ordered Q, K and V are not written).
 */
int32_t wf_vsa(const void* q, const void* k, const void* v, int32_t B, int32_t Hh, int32_t T, int32_t H,
               int32_t W, int32_t D, float scale, int32_t topk, int32_t* idx, const void* gate, float* o,
               float* lse, float* o_coarse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * VSA fine stage with the gated merge ("VSA selects cubes", part 3: the fine
 * result is kept whole and a learned share of the coarse branch is added).
 * The coarse branch's output for query cube c is the cube-level attention of
 * the coarse stage over all C key cubes,
 *     Oc[c] = sum_{c'} softmax_{c'}(S[c][c']) Vbar[c'],
 * from the scores S of the preceding wf_vsa_coarse_topk (its scale), with the
 * product P Vbar taken to about fp32 accuracy (bf16 matrix products of split
 * hi/lo operands, fp32 sums).  Every real token i
 * of query cube c then receives, elementwise over the head dimension,
 *     o[i] = o_fine[i] + gate[i] * Oc[c]
 * where o_fine is exactly what wf_vsa_fine writes (gate = 0 reproduces it bit
 * for bit).  lse is the fine stage's.  The gate comes from learned weights
 * in the model, so the caller supplies it.
 *
 *   workspace      as filled by wf_vsa_coarse_topk with the same B, Hh, T, H,
 *                  W, D; this call also writes its coarse-output region.
 *   gate           bf16 [B][Hh][T*H*W][D], read only.
 *   o_coarse       fp32 [B][Hh][C][D]: Oc, written; may be NULL (it is then
 *                  kept in the workspace only).
 *   idx, scale, topk, o, lse, stream: as for wf_vsa_fine, including the
 *                  WF_VALIDATE=1 plan check.
 */
int32_t wf_vsa_fine_gated(void* workspace, size_t workspace_bytes, const int32_t* idx,
                          const void* gate, int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W,
                          int32_t D, float scale, int32_t topk, float* o, float* lse,
                          float* o_coarse, void* stream);

/* ------------------------------------------------------ sliding-tile attention */

/*
 * Sliding-tile attention (STA).  "推理优化" (Inference optimization,
 * WorldFoundry docs), approximate-attention section, entry "sta": weight-free
 * sliding-tile attention for the Wan DiT, accepted only on its tuned token
 * grids (36, 48, 48) and (18, 48, 80) and refused, before any GPU work, on any
 * other (the page's example is the default (31, 22, 40)).  It gives no tile or
 * window size; the library's definition:
 *   - tiles are 6 x 8 x 8 tokens (t, h, w), which both accepted grids divide
 *     exactly (6x6x6 and 3x6x10 tiles; no padding), tile id (tt*nh + th)*nw + tw;
 *   - a query tile attends to the tiles of a wt x wh x ww-tile window that on
 *     each axis starts at clamp(c - (w-1)/2, 0, n - w): centred where it fits,
 *     pushed inward at the grid's edge, so every tile sees wt*wh*ww tiles;
 *   - each query token attends to every key token of those tiles:
 *     o[i] = sum_j softmax_j(scale * q[i] . k[j]) v[j], lse as in wf_vsa_fine.
 * The kernels run it as VSA's fine stage over 1x8x8-token slabs with a fixed
 * plan (six slabs per tile).
 *
 *   T, H, W     36 x 48 x 48 or 18 x 48 x 80, else WF_ERR_UNSUPPORTED.
 *   q, k, v     bf16 [B][Hh][T*H*W][D]; D must be 128.
 *   wt, wh, ww  window in tiles, 1 <= wt <= T/6, 1 <= wh <= H/8, 1 <= ww <= W/8.
 *   o           fp32 [B][Hh][T*H*W][D], written; lse fp32 [B][Hh][T*H*W] or NULL.
 *   plan        int32 [T/6 * H/8 * W/8][wt*wh*ww], the key tiles of every
 *               query tile, written (ascending rows); may be NULL.
 *   workspace   at least wf_sta_workspace_bytes() bytes (0 for a grid or
 *               window the call would refuse).
 */
size_t wf_sta_workspace_bytes(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                              int32_t wt, int32_t wh, int32_t ww);
int32_t wf_sta(const void* q, const void* k, const void* v, int32_t B, int32_t Hh, int32_t T, int32_t H,
               int32_t W, int32_t D, float scale, int32_t wt, int32_t wh, int32_t ww, float* o, float* lse,
               int32_t* plan, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ softmax reference policies */

/*
 * "Anatomy of Wan2.2's 53.6x speedup", section "Fixed-max softmax is a
 * numerical contract", weighs the online softmax's running row maximum (exact
 * and stable, but every new maximum rescales the accumulated output) against
 * a reduction constant taken once from the first selected tile (one pass, and
 * the probabilities are unchanged by the shift, but a later, much larger score
 * overflows the exponential).  The _ex entry points below take the policy:
 *
 *   WF_SOFTMAX_GUARDED          the library default (what wf_attn_dense and
 *                               wf_vsa_fine use): the reference is an integer,
 *                               set on the first tile and raised only when a
 *                               tile's probabilities would exceed 2^16, which
 *                               one vote per tile detects; exact and
 *                               overflow-safe, one pass on the common path.
 *   WF_SOFTMAX_RUNNING_MAX      the textbook online softmax: row maximum of
 *                               every tile, output and row sum rescaled every
 *                               tile.  Exact and safe; the comparison point.
 *   WF_SOFTMAX_FIXED_FIRST_TILE the page's contract without a guard: the
 *                               reference comes from the first tile and never
 *                               moves.  Exact while every later score stays
 *                               within about 88 (natural-log units) of the
 *                               first tile's maximum; beyond that the row's
 *                               output and lse become inf or NaN.  For
 *                               measurement and for reproducing that failure,
 *                               not for use.
 */
enum {
  WF_SOFTMAX_GUARDED = 0,
  WF_SOFTMAX_RUNNING_MAX = 1,
  WF_SOFTMAX_FIXED_FIRST_TILE = 2
};

/* wf_attn_dense with a softmax policy (above); otherwise identical. */
int32_t wf_attn_dense_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                         int32_t B, int32_t Hh, int32_t N, int32_t D, float scale,
                         int32_t softmax_mode, void* workspace, size_t workspace_bytes,
                         void* stream);

/* wf_vsa_fine with a softmax policy (above); otherwise identical. */
int32_t wf_vsa_fine_ex(const void* workspace, size_t workspace_bytes, const int32_t* idx,
                       int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                       float scale, int32_t topk, int32_t softmax_mode, float* o, float* lse,
                       void* stream);

/* ------------------------------------------------------ 3D RoPE */

/*
 * 3D rotary position embedding of Q and K.  "推理优化" (Inference
 * optimization, WorldFoundry docs), section "Exact or numerically equivalent
 * Wan kernels", entry fused_rope, names a fused 3D RoPE whose rotation runs in
 * fp32 or fp64 but gives no frequencies; the library takes the common
 * Wan-style definition and offers both precisions:
 *   - the head dimension is cut into consecutive parts of D - 4*floor(D/6),
 *     2*floor(D/6) and 2*floor(D/6) dims for the t, h and w axes
 *     (D = 128: 44, 42, 42; D = 64: 24, 20, 20);
 *   - inside a part of d_a dims, elements (2i, 2i+1) form pair i and rotate by
 *     phi = pos * theta^(-2i/d_a), pos being the token's 0-based coordinate
 *     on that axis: (x0, x1) -> (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi);
 *   - precision 64: the rotation is computed in fp64 and rounded once to
 *     bf16 (nearest, ties to even); a result below the normal bf16 range
 *     (|y| < 2^-126, which rotated inputs of normal size never reach)
 *     becomes a signed zero;
 *   - precision 32: cos and sin (taken in fp64) are rounded to fp32, each
 *     product and sum is rounded to fp32 (no fused multiply-add), and that
 *     fp32 value is rounded to bf16 (nearest, ties to even).  About 3x less
 *     arithmetic; it differs from precision 64 by one bf16 step on a small
 *     fraction of near-tie elements.
 *
 *   q, k           bf16 [B][Hh][T*H*W][D], read.
 *   q_out, k_out   bf16, same shape, written.  Each may be the same pointer
 *                  as its input (in place); otherwise no two of the four
 *                  buffers may overlap.
 *   D              64 or 128.   theta: finite, > 0 (Wan uses 10000).
 *   precision      32 or 64.
 */
int32_t wf_rope_qk(const void* q, const void* k, void* q_out, void* k_out, int32_t B, int32_t Hh,
                   int32_t T, int32_t H, int32_t W, int32_t D, double theta, int32_t precision,
                   void* stream);

/*
 * wf_vsa_coarse_topk with the 3D RoPE of wf_rope_qk (frequency base
 * rope_theta, finite and > 0; rope_precision 32 or 64) applied to Q and K
 * inside the gather, so the
 * rotation costs no separate pass over Q and K.  Cube means, scores, the plan
 * and the fine stage (wf_vsa_fine, wf_vsa_fine_gated, which read the gathered
 * Q and K from the workspace) all see the rotated vectors; the result equals
 * wf_rope_qk followed by wf_vsa_coarse_topk bit for bit.  Arguments otherwise
 * as for wf_vsa_coarse_topk.
 */
int32_t wf_vsa_coarse_topk_rope(const void* q, const void* k, const void* v,
                                int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                                float scale, int32_t topk, double rope_theta,
                                int32_t rope_precision, int32_t* idx, float* coarse_scores,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ per-kernel timing */

/*
 * Optional timing of every kernel this library launches, with HIP events
 * recorded on the launch stream just before and after each kernel.
 * wf_profile_enable(1) clears earlier records and starts recording;
 * wf_profile_enable(0) stops.  Recording adds no synchronisation.
 * At most 65536 launches are recorded per enable; later ones are counted
 * as dropped and not timed.
 */
int32_t wf_profile_enable(int32_t on);

/*
 * Waits for the recorded events, then reports the kernel named `name`
 * (e.g. "wf_dense_fwd"): number of timed launches and their summed time.
 * Returns WF_ERR_INVALID_ARG if no launch of that kernel was recorded.
 */
int32_t wf_profile_query(const char* name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* WF_ATTN_H */
