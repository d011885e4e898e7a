/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) hot path of DeepSeek Sparse
 * Attention (DSA): lightning-indexer scores, per-query top-k token selection,
 * and sparse MLA attention in MQA mode.
 *
 * Source of the method: "Paper Breakdown: DeepSeek-V3.2", section 2
 * "Architecture: DSA (§2.1)" (index-score formula, top-k selector, attention
 * over the selected latent entries, "DSA under MLA (MQA Mode)"), and
 * "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models", Key
 * points (k = 2048 selected tokens, ReLU, few indexer heads, FP8, MLA in MQA
 * mode).
 *
 * Conventions shared by every entry point
 *  - Every tensor argument is a DEVICE pointer to contiguous row-major memory
 *    (last dimension innermost) that the CALLER owns.  Pointers must be
 *    16-byte aligned.  The library never allocates, frees or synchronises
 *    device memory; kernels are enqueued on `stream` (a hipStream_t, NULL =
 *    the default stream) and the call returns without waiting.
 *  - Query token t of batch entry b sits at absolute position q_offset + t
 *    and its causal candidate set is s in [0, min(N, q_offset + t + 1)).
 *    Prefill: T = N, q_offset = 0.  Decode: T = 1, q_offset = N - 1.
 *    Chunked prefill: q_offset = N - T.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns DSA_ERR_INVALID_ARG, a shape outside the supported set
 *    returns DSA_ERR_UNSUPPORTED, a too-small workspace DSA_ERR_WORKSPACE and
 *    a failed launch DSA_ERR_HIP.  No exception crosses the ABI.  Device data
 *    is never validated (NaN inputs do not fault; see each call).
 *  - Stateless and re-entrant: concurrent calls on different streams with
 *    disjoint outputs and workspaces are safe.
 *  - Debug validation: when the environment variable DSA_VALIDATE is "1" at
 *    the time of the call, the entry points that take token indices or cache
 *    positions from the caller (dsa_sparse_mla_attn, dsa_sparse_mla_attn_bwd,
 *    dsa_indexer_kl with idx, dsa_cache_append) first check them on the
 *    stream: an index that is neither -1 nor inside [0, N), or a cache row
 *    pos[b] + t outside [0, N), makes the call return DSA_ERR_BAD_INDEX
 *    without launching anything else.  Such calls wait for the stream (the
 *    only calls that do), and validated calls that overlap on one device
 *    share the library's single device counter.  Without it, such entries
 *    are skipped as each call describes.
 *
 * Supported shapes
 *  - indexer: (H_I, d_I, idx_dtype) = (8, 128, DSA_FP8_E4M3FN) with
 *    N < 2^24 keys per sequence (32-bit byte offsets into the keys and the
 *    score rows), or (1..16, 1..256, DSA_F32);
 *  - attention: (H, d_qk, d_v, attn_dtype) = (128, 576, 512, DSA_BF16) with
 *    N < 2^31 / 1152 latent rows per sequence (the gather addresses one
 *    sequence's rows with 32-bit byte offsets), or (1..32, 1..256, 1..d_qk,
 *    DSA_F32);
 *  - 1 <= k <= 2048; q_offset >= 0; q_offset + T <= N; B*T*N < 2^40.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,
    DSA_ERR_UNSUPPORTED = 2,
    DSA_ERR_WORKSPACE = 3,
    DSA_ERR_BAD_INDEX = 4,
    DSA_ERR_HIP = 5
} dsa_status;

typedef enum dsa_dtype {
    DSA_F32 = 0,        /* IEEE binary32 */
    DSA_BF16 = 1,       /* bfloat16 */
    DSA_FP8_E4M3FN = 2  /* OCP 8-bit float E4M3 (bias 7, max 448, 0x7F/0xFF NaN) */
} dsa_dtype;

typedef enum dsa_op {
    DSA_OP_TOPK = 0,
    DSA_OP_ATTN = 1,
    DSA_OP_FORWARD = 2,
    DSA_OP_SELECT = 3,
    DSA_OP_ATTN_BWD = 4,
    DSA_OP_ATTN_MHA = 5
} dsa_op;

/*
 * Lightning-indexer scores ("Paper Breakdown: DeepSeek-V3.2", section 2,
 * index-score formula):
 *     scores[b,t,s] = sum_j w[b,t,j] * ReLU(q_idx[b,t,j,:] . k_idx[b,s,:])
 * for s <= q_offset + t, and -inf for every other s < N.  One indexer key per
 * token is shared by all H_I heads.
 *
 *  q_idx       [B,T,H_I,d_I]  FP8 codes (uint8) or f32, per idx_dtype
 *  q_idx_scale [B,T,H_I] f32  dequantisation scale of each query head
 *                             (FP8 only; must be NULL for f32)
 *  k_idx       [B,N,d_I]      FP8 codes or f32
 *  k_idx_scale [B,N]     f32  dequantisation scale of each key (FP8 only)
 *  w           [B,T,H_I] f32  head weights w[t,j] (any sign)
 *  scores      [B,T,N]   f32  output, fully overwritten
 * With FP8 the value of an operand is scale * decode(code); the kernel
 * computes k_scale * sum_j (w * q_scale) * ReLU(q8 . k8) with an exact FP8
 * product and fp32 accumulation, which equals the formula for positive
 * scales (the only kind the amax/448 rule produces).  Accumulation is fp32.
 */
DSA_API dsa_status dsa_indexer_scores(const void* q_idx, const float* q_idx_scale,
                              const void* k_idx, const float* k_idx_scale,
                              const float* w, float* scores,
                              int B, int T, int N, int H_I, int d_I, int q_offset,
                              dsa_dtype idx_dtype, void* stream);

/*
 * Top-k token selection ("Paper Breakdown: DeepSeek-V3.2", section 2: query t
 * keeps the tokens whose score is in Top-k(I[t,:]); the selector keeps only
 * earlier tokens, "DeepSeek V3.2: Sparse Attention and Reinforcement Learning
 * Updates", Summary).
 *
 *  scores [B,T,N] f32   only s < min(N, q_offset+t+1) is read per row
 *  idx    [B,T,k] int32 output: the n = min(k, #candidates) selected token
 *                       indices in ascending order, then -1 padding
 * Ranking: larger score first; equal scores go to the lower index; -0 equals
 * +0; NaN ranks below every number.  The result is unique and deterministic.
 * Batches of at most 255 rows (B*T <= 255, e.g. decode) are selected by
 * several workgroups per row and need dsa_workspace_size(DSA_OP_TOPK, ...)
 * bytes of workspace (per row: a 4096-bin histogram, counters and candidate
 * lists), which the call overwrites; larger batches need none and workspace
 * may then be NULL.
 */
DSA_API dsa_status dsa_topk_select(const float* scores, int32_t* idx,
                           int B, int T, int N, int k, int q_offset,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse MLA attention in MQA mode ("Paper Breakdown: DeepSeek-V3.2",
 * section 2, attention formula u_t = Attn(h_t, {c_s : selected}) and "DSA
 * under MLA (MQA Mode)": every query head attends to the same latent vector
 * c_s of each selected token):
 *     z[h,i]   = sm_scale * q[b,t,h,:] . kv[b,idx[b,t,i],:]        (d_qk wide)
 *     out[b,t,h,:] = sum_i softmax_i(z[h,:]) * kv[b,idx[b,t,i],0:d_v]
 *     lse[b,t,h]   = log sum_i exp(z[h,i])
 *
 *  q   [B,T,H,d_qk] bf16 or f32 (attn_dtype)
 *  kv  [B,N,d_qk]   bf16 or f32: latent (first d_v columns, also the value)
 *                   followed by the rope part
 *  idx [B,T,k] int32: slots equal to -1 or otherwise outside [0, N) are
 *                   skipped; duplicates count once per occurrence
 *  out [B,T,H,d_v]  bf16 or f32 (attn_dtype), fully overwritten
 *  lse [B,T,H] f32 or NULL
 * A row with no valid slot gets out = 0 and lse = -inf.  bf16 runs the
 * products on bf16 MFMA with fp32 logits/softmax/accumulation and rounds the
 * softmax weights to bf16 before the value product.  bf16 batches with fewer
 * rows than the GPU has compute units split each row's slots over several
 * workgroups; the workspace (dsa_workspace_size(DSA_OP_ATTN, ...) bytes,
 * 16-byte aligned, overwritten) then holds their normalised bf16 partial
 * outputs and fp32 (max, exp-sum) pairs.
 */
DSA_API dsa_status dsa_sparse_mla_attn(const void* q, const void* kv, const int32_t* idx,
                               void* out, float* lse,
                               int B, int T, int N, int H, int d_qk, int d_v, int k,
                               float sm_scale, dsa_dtype attn_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of dsa_sparse_mla_attn (bf16 MQA mode) for the sparse training
 * stage ("Paper Breakdown: DeepSeek-V3.2", section 2, "Continued
 * Pre-Training (§2.1.1)": the main model is trained through the sparse
 * attention over the selected entries).  With z, P = softmax(z) and out as
 * in dsa_sparse_mla_attn and dout the gradient of the loss w.r.t. out:
 *     dP[h,i] = dout[b,t,h,:] . kv[b,idx[b,t,i],0:d_v]
 *     dS[h,i] = sm_scale * P[h,i] * (dP[h,i] - dout[b,t,h,:] . out[b,t,h,:])
 *     dq[b,t,h,:]         = sum_i dS[h,i] * kv[b,idx[b,t,i],:]
 *     dkv[b,s,:]          = sum over (t,i) with idx[b,t,i] = s of
 *                           sum_h dS[h,i] q[b,t,h,:]  (+ sum_h P[h,i] dout[b,t,h,:]
 *                           on the first d_v columns)
 * P is recomputed as exp(z - lse) from the forward's lse.
 *
 *  q, kv, idx  as passed to the forward (bf16; H = 128, d_qk = 576, d_v = 512)
 *  out  [B,T,H,d_v] bf16  the forward's output
 *  lse  [B,T,H]     f32   the forward's log-sum-exp (required)
 *  dout [B,T,H,d_v] bf16
 *  dq   [B,T,H,d_qk] f32  output, fully overwritten
 *  dkv  [B,N,d_qk]   f32  output, fully overwritten (0 for rows no slot selects)
 * Slots outside [0, N) contribute nothing; a token in several slots receives
 * the sum.  Products run on bf16 MFMA with fp32 accumulation; P and dS are
 * rounded to bf16 before the products that produce dq and dkv.  Each slot's
 * latent-gradient vector (summed over the heads in fp32) is rounded to bf16,
 * and the vectors of a token are summed in fp32 in an order that depends on
 * scheduling, so the last bits of dkv vary from run to run.  Rows are
 * processed 2048 at a time; the workspace (dsa_workspace_size(
 * DSA_OP_ATTN_BWD, ...) bytes, 16-byte aligned, overwritten) holds one such
 * block's P and dS tiles, slot vectors and per-token lists, a count and an
 * offset per token of the batch (B*N of each) and the list of the tokens a
 * block selects.  attn_dtype must be DSA_BF16.
 */
DSA_API dsa_status dsa_sparse_mla_attn_bwd(const void* q, const void* kv, const int32_t* idx,
                                   const void* out, const float* lse, const void* dout,
                                   float* dq, float* dkv,
                                   int B, int T, int N, int H, int d_qk, int d_v, int k,
                                   float sm_scale, dsa_dtype attn_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse MLA attention in MHA mode (the DeepSeek-V3.2 paper's section list,
 * page aipaper.jasonlin.tech, "Sections": "Appendix A MHA and MQA Modes of
 * MLA"; DSA itself runs in MQA mode, dsa_sparse_mla_attn).  Every head h
 * attends over its own keys and values, up-projected from the same latent
 * entries c_s = kv[b,s,:] (d_c latent columns, then d_r rope columns):
 *     key(s, h)   = [W_UK[h] c_s[0:d_c] ; c_s[d_c:d_c+d_r]]     (d_n + d_r)
 *     value(s, h) = W_UV[h] c_s[0:d_c]                          (d_vh)
 *     z[h,i]      = sm_scale * q[b,t,h,:] . key(idx[b,t,i], h)
 *     out[b,t,h,:] = sum_i softmax_i(z[h,:]) * value(idx[b,t,i], h)
 *     lse[b,t,h]   = log sum_i exp(z[h,i])
 * After absorbing W_UK into the query and W_UV into the output this is what
 * MQA mode computes; in MHA mode every selected token costs one key and one
 * value row per head instead of one shared latent row.
 *
 *  q    [B,T,H,d_n+d_r] bf16  per-head queries [q_nope ; q_rope]
 *  kv   [B,N,d_c+d_r]   bf16  latent entries
 *  w_uk [H,d_n,d_c]     bf16  key up-projection of each head
 *  w_uv [H,d_vh,d_c]    bf16  value up-projection of each head
 *  idx  [B,T,k] int32         as for dsa_sparse_mla_attn (-1 and indices
 *                             outside [0, N) skipped, duplicates counted)
 *  out  [B,T,H,d_vh]    bf16  fully overwritten
 *  lse  [B,T,H] f32 or NULL
 * Supported: H = 128, d_c = 512, d_r = 64, d_n = 128, d_vh = 128, bf16.
 * The head-dependent parts of every latent row's keys and values
 * (W_UK[h] c_s[:d_c], W_UV[h] c_s[:d_c]) are computed first (bf16 MFMA, fp32
 * accumulation, rounded to bf16) into the workspace
 * (dsa_workspace_size(DSA_OP_ATTN_MHA, B, T, N, 1, H, d_vh, k) bytes =
 * B*N*H*(128 + 128)*2 rounded up, 16-byte aligned, overwritten; after the
 * call it holds the key parts as [B*N][H][d_n] bf16 from byte 0 and the
 * value parts as [B*N][H][d_vh] bf16 from byte B*N*H*d_n*2 rounded up to a
 * multiple of 256); the rope part of the key, shared by all heads, is read
 * from kv;
 * logits, softmax and accumulation are fp32, the output is rounded to bf16.
 * The call suits prefill-sized caches: a decode batch would up-project every
 * cached row of every sequence.
 */
DSA_API dsa_status dsa_sparse_mla_attn_mha(const void* q, const void* kv, const void* w_uk,
                                   const void* w_uv, const int32_t* idx,
                                   void* out, float* lse,
                                   int B, int T, int N, int H, int d_c, int d_r, int d_n, int d_vh,
                                   int k, float sm_scale, dsa_dtype attn_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Index scores and top-k selection in one call: idx as dsa_topk_select would
 * return it for the scores dsa_indexer_scores computes (same arguments,
 * same ranking and tie rule), without handing the score matrix to the
 * caller ("Paper Breakdown: DeepSeek-V3.2", section 2: the indexer's scores
 * serve only to pick Top-k(I[t,:])).
 *
 *  idx [B,T,k] int32 output, ascending indices then -1 padding
 * For FP8 batches with T < 16 and at most 255 rows (decode) the scores are
 * never materialised: a per-row threshold taken from a sample of 1024 keys
 * filters the keys into a candidate list and the exact selection is made
 * among the candidates; a row whose list holds fewer than k keys or
 * overflows is rescored in full and selected from that, so the result is
 * always the exact one.  Other shapes compute the scores and select.  The
 * workspace (dsa_workspace_size(DSA_OP_SELECT, ...) bytes, 16-byte aligned)
 * holds the score matrix and the selection lists.
 */
DSA_API dsa_status dsa_indexer_select(const void* q_idx, const float* q_idx_scale,
                              const void* k_idx, const float* k_idx_scale,
                              const float* w, int32_t* idx,
                              int B, int T, int N, int H_I, int d_I, int k, int q_offset,
                              dsa_dtype idx_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole DSA path ("Paper Breakdown: DeepSeek-V3.2", section 2
 * "Architecture: DSA (§2.1)": the lightning indexer scores every earlier
 * token, the fine-grained selector keeps the tokens in Top-k(I[t,:]), and
 * attention runs over their latent entries, under "DSA under MLA (MQA
 * Mode)"): indexer scores -> top-k selection -> sparse attention, for
 * prefill, decode and chunked prefill alike (see q_offset above).
 * Arguments are those of the calls above; idx_out [B,T,k] receives the
 * selected indices when non-NULL.  The selection is dsa_indexer_select's.
 * The workspace holds the score matrix and the other intermediates: size it
 * with dsa_workspace_size(DSA_OP_FORWARD, B, T, N, H_I, H, d_v, k).
 * Errors as for the calls above; nothing is launched when an argument check
 * fails.
 */
DSA_API dsa_status dsa_forward(const void* q_idx, const float* q_idx_scale,
                       const void* k_idx, const float* k_idx_scale,
                       const float* w, const void* q, const void* kv,
                       void* out, float* lse, int32_t* idx_out,
                       int B, int T, int N, int H_I, int d_I, int H, int d_qk, int d_v,
                       int k, int q_offset, float sm_scale,
                       dsa_dtype idx_dtype, dsa_dtype attn_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what dsa_forward
 * computes, with the same kernels and checks, and calls no allocating
 * routine.  Its intermediates live in one fixed array of 128 MiB per device
 * (DSA_NOALLOC_SCRATCH_BYTES) inside the library, held from the library's
 * first use on that device until the process ends; a call whose
 * dsa_workspace_size(DSA_OP_FORWARD, B, T, N, H_I, H, d_v, k) exceeds it
 * returns DSA_ERR_UNSUPPORTED without launching anything (decode of 64
 * sequences at 131072 tokens needs 72.3 MiB; batches with a large [B,T,N]
 * score matrix, e.g. prefill, do not fit).  The array is the one of the
 * device current at the call, and `stream` must belong to that device
 * (otherwise DSA_ERR_INVALID_ARG).  Every call on a device shares its array
 * and leaves its own intermediates there: calls that overlap on one device
 * (on different streams, or concurrent host threads) race and must be
 * serialised by the caller.  The kernels clear what they count in, so no
 * call depends on what an earlier call left.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
DSA_API dsa_status dsa_forward_noalloc(const void* q_idx, const float* q_idx_scale,
                               const void* k_idx, const float* k_idx_scale,
                               const float* w, const void* q, const void* kv,
                               void* out, float* lse, int32_t* idx_out,
                               int B, int T, int N, int H_I, int d_I, int H, int d_qk, int d_v,
                               int k, int q_offset, float sm_scale,
                               dsa_dtype idx_dtype, dsa_dtype attn_dtype, void* stream);

/*
 * Cache append, the step before the path at decode.  Each token keeps its
 * indexer key, in FP8 ("Paper Breakdown: DeepSeek-V3.2", section 2
 * "Architecture: DSA (§2.1)": the indexer runs in FP8), and its latent entry
 * c_s (same section, the attention formula).  New token t of sequence b is
 * written to cache row pos[b] + t:
 *  k_new         [B,T,d_I]  f32        indexer keys of the new tokens
 *  kv_new        [B,T,d_qk] bf16/f32   latent rows of the new tokens (attn_dtype)
 *  k_cache       [B,N,d_I]  FP8 codes or f32 (idx_dtype), updated in place
 *  k_cache_scale [B,N]      f32        per-token scale (FP8 only; NULL for f32)
 *  kv_cache      [B,N,d_qk] attn_dtype, updated in place
 *  pos           [B]        int32      row of each sequence's first new token
 * FP8: scale = amax / 448 (IEEE float32 division; 1 for a row of zeros) and
 * code = round-to-nearest-even e4m3fn of clamp(x / scale, -448, 448), the
 * quotient again an IEEE float32 division; this is the per-token scaling the
 * FP8 indexer operands use.  f32 keys and all latent rows are copied
 * unchanged.  Rows whose position lies outside [0, N) are dropped (pos is
 * device data and is not otherwise checked); no other cache row is touched.
 * Key rows must be finite.  Supported: (idx_dtype, d_I) = (FP8_E4M3FN, 128)
 * or (F32, 1..256); (attn_dtype, d_qk) = (BF16, 576) or (F32, 1..256).
 * Positions of one call must not repeat within a sequence's cache rows
 * (distinct t give distinct rows).
 */
DSA_API dsa_status dsa_cache_append(const float* k_new, const void* kv_new, void* k_cache,
                                    float* k_cache_scale, void* kv_cache, const int32_t* pos,
                                    int B, int T, int N, int d_I, int d_qk,
                                    dsa_dtype idx_dtype, dsa_dtype attn_dtype, void* stream);

/*
 * Indexer alignment objective and its gradient with respect to the index
 * scores ("Paper Breakdown: DeepSeek-V3.2", section 2, "Continued
 * Pre-Training (§2.1.1)": the dense warm-up minimises
 * L^I = sum_t KL(p_t || Softmax(I_t)); sparse training keeps the KL on the
 * selected set S_t).  For each row b,t, over its entries E (below):
 *     lse  = log sum_{s in E} exp(I_s)
 *     loss[b,t] = sum_{s in E, p_s > 0} p_s (log p_s - (I_s - lse))
 *     grad_s    = P exp(I_s - lse) - p_s,   P = sum_{s in E} p_s
 * The target is taken as given (a distribution has P = 1; terms with
 * p_s = 0 vanish).
 *  Dense (idx == NULL): E = the causal candidates s <= q_offset + t.
 *    scores [B,T,N] f32, p [B,T,N] f32 (entries outside E are ignored),
 *    grad [B,T,N] f32 (0 outside E) or NULL; k is ignored.
 *  Selected set (idx != NULL): E = the slots of idx [B,T,k] int32 whose
 *    token lies in [0, N) (others are skipped, duplicates count per slot).
 *    scores [B,T,N] f32, p [B,T,k] f32 = the target of each slot,
 *    grad [B,T,k] f32 (0 for skipped slots) or NULL; q_offset is ignored.
 *  loss [B,T] f32.  Scores must be finite or -inf, p finite and >= 0.
 * fp32 throughout (library expf/logf); a row whose entries are all -inf
 * gives NaN, as the formula does.
 */
DSA_API dsa_status dsa_indexer_kl(const float* scores, const float* p, const int32_t* idx,
                                  float* loss, float* grad, int B, int T, int N, int k,
                                  int q_offset, void* stream);

/*
 * Workspace bytes needed by op (a dsa_op) for these sizes; 0 means none.
 * The sizes are those passed to the call the workspace is for: B, T, N as
 * above, H_I indexer heads (DSA_OP_SELECT, DSA_OP_FORWARD), H query heads
 * and d_v value width (DSA_OP_ATTN, DSA_OP_ATTN_BWD, DSA_OP_FORWARD), k
 * selected tokens per query; an op ignores the sizes it does not use, but
 * each must be >= 1.  Returns (size_t)-1 for arguments that no call would
 * accept (an unknown op, a size below 1, k above 2048).
 */
DSA_API size_t dsa_workspace_size(int op, int B, int T, int N, int H_I, int H, int d_v, int k);

/*
 * Per-kernel timing, a diagnostic (off by default).  dsa_profile_start opens
 * a window of at most max_launches kernel launches: every kernel the library
 * launches until dsa_profile_stop records a HIP event on its stream right
 * before and right after itself.  The events are host-side objects created by
 * dsa_profile_start (no device memory is allocated); DSA_ERR_INVALID_ARG if a
 * window is already open or max_launches is outside [1, 2^20].
 * dsa_profile_stop waits for the recorded events (the only waiting these
 * two calls do), closes the window and fills out[0..n) with one entry per
 * distinct kernel (its static name, the number of launches and the summed
 * event-to-event time in milliseconds); it returns n (<= max_out) or -1 when
 * no window was open or an event failed.  *dropped (if not NULL) receives
 * the number of launches beyond max_launches, which were not recorded.  No
 * library call may run concurrently with dsa_profile_stop, and profiled
 * calls must not be captured into a graph.
 */
typedef struct dsa_kernel_time {
    const char* name;
    int launches;
    double total_ms;
} dsa_kernel_time;
DSA_API dsa_status dsa_profile_start(int max_launches);
DSA_API int dsa_profile_stop(dsa_kernel_time* out, int max_out, int* dropped);

/*
 * Peak probes, a diagnostic: what this GPU sustains, for comparing kernels
 * against measured as well as published peaks.  Each runs its probe kernel
 * five times on `stream`, waits for it, and returns the best rate, or a
 * negative value on a bad argument or a HIP error.
 *  DSA_PROBE_STREAM_READ  GB/s of a plain streaming read (16-byte loads,
 *                         grid-stride) over the first bytes - 64 KiB of buf,
 *                         a device buffer of bytes >= 1 MiB (16-byte
 *                         aligned); its last 32 KiB are overwritten
 *  DSA_PROBE_MFMA_BF16    TFLOP/s of back-to-back v_mfma_f32_16x16x32_bf16
 *  DSA_PROBE_MFMA_FP8     TFLOP/s of back-to-back
 *                         v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3)
 *  DSA_PROBE_MFMA_BF16_32X32  TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16
 * The MFMA probes read no memory; buf must be a device pointer to at least
 * 8 KiB, which they practically never write.  The MFMA rates reflect the
 * engine clock the chip runs at under that load.
 */
enum { DSA_PROBE_STREAM_READ = 0, DSA_PROBE_MFMA_BF16 = 1, DSA_PROBE_MFMA_FP8 = 2,
       DSA_PROBE_MFMA_BF16_32X32 = 3 };
DSA_API double dsa_probe_peak(int what, const void* buf, size_t bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
DSA_API const char* dsa_status_string(dsa_status s);

/* ABI version: (major << 16) | minor. */
DSA_API int dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
