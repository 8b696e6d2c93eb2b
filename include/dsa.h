/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on one AMD Instinct MI355X (gfx950).
 *
 * The path has three steps, each an entry point, plus two entry points that run all three:
 *
 *   1. dsa_indexer_scores   lightning-indexer scores   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
 *   2. dsa_topk             per-query selection of the k keys with the largest I[t,:]
 *   3. dsa_sparse_mla_attn  attention of every query head over the selected latent rows only,
 *                           each latent row shared by all heads (MLA in MQA mode)
 *   dsa_forward_prefill / dsa_forward_decode   1 -> 2 -> 3 on one stream
 *
 * Definitions: velog summary "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models",
 * section 1.1 (the index score equation, ReLU, few FP8 indexer heads, scores against the preceding
 * tokens), section 1.2 (top-k retrieval of key/value entries and u_t = Attn(h_t, {c_s})), section
 * 1.3 (MQA mode, every latent KV entry shared by all query heads), Continued Pre-Training stage 2
 * (2048 selected tokens per query); notes.yuuk.io page of the same title, section on DSA.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Sequences.  A call covers B independent sequences.  Each has n_kv visible tokens and carries its
 *   last n_q tokens as queries: query t (0 <= t < n_q) sits at position pos_t = n_kv - n_q + t and
 *   sees keys s = 0..pos_t (the causal domain includes the query's own token).  Decode is n_q = 1.
 * Memory.  Every pointer is a device pointer unless stated otherwise; all tensors are dense,
 *   row-major, with the batch as the outermost dimension.  The caller owns all memory; the library
 *   never allocates, frees or synchronises.  Fast paths need 16-byte aligned base pointers.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *   enqueued asynchronously; a kernel fault surfaces at the caller's next synchronisation.
 * Errors.  Arguments are validated before anything is enqueued; on failure nothing is enqueued
 *   and a status other than DSA_OK is returned.  dsa_last_error() returns a text of the last
 *   failure on the calling thread.  No C++ exception crosses the ABI.
 * fp8 is OCP E4M3 ("e4m3fn": bias 7, max 448, no infinities).  Row scales must be finite and > 0.
 * Softmax scale.  Every attention, backward and warm-up entry point takes sm_scale, which must be
 *   finite and > 0 (the scores are multiplied by it inside the exponent); anything else returns
 *   DSA_ERR_INVALID_ARG with nothing enqueued.
 * Threading.  All entry points are reentrant.  Mutable global state: the thread-local error text,
 *   a per-device record that the top-k kernels' opt-in to the full 160 KiB of LDS was made (an
 *   idempotent runtime call; two threads racing on it only repeat it), and the per-device address of
 *   the fixed scratch array of dsa_forward_decode_noalloc (looked up once per device, under a lock).
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, n_q > n_kv, bad leading dimension ... */
  DSA_ERR_UNSUPPORTED = 2, /* valid arguments no kernel here implements (dtype / shape combination) */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned                          */
  DSA_ERR_HIP = 4          /* the HIP runtime refused a launch                                    */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,      /* IEEE binary32                                   */
  DSA_BF16 = 1,     /* bfloat16                                        */
  DSA_FP8_E4M3 = 2  /* OCP e4m3fn codes (uint8) with fp32 row scales   */
} dsa_dtype_t;

/* Library version, as 10000*major + 100*minor + patch. */
int dsa_version(void);

/* Constant text for a status code (never NULL). */
const char* dsa_status_string(dsa_status_t status);

/* Text describing the last failure on the calling thread ("" if none).  Valid until the next call
 * into the library from the same thread. */
const char* dsa_last_error(void);

/* ------------------------------------------------------------------------------------------------
 * dsa_indexer_scores -- lightning-indexer scores (section 1.1 of the velog summary).
 *
 *   scores[b][t][s] = sum_{j<H_I} w[b][t][j] * ReLU( qhat[b][t][j][:] . khat[b][s][:] ),  s <= pos_t
 *
 * dtype = DSA_FP8_E4M3: q is uint8 codes [B][n_q][H_I][d_I] with q_scale [B][n_q][H_I] (fp32), k is
 *   uint8 codes [B][n_kv][d_I] with k_scale [B][n_kv]; qhat = e4m3(q) * q_scale, khat = e4m3(k) *
 *   k_scale.  Because scales are positive, the kernel evaluates
 *   k_scale[s] * sum_j (w * q_scale)[t][j] * ReLU(e4m3(q) . e4m3(k)) with fp32 accumulation.
 * dtype = DSA_F32: q [B][n_q][H_I][d_I] and k [B][n_kv][d_I] are float; q_scale, k_scale must be NULL.
 * w is [B][n_q][H_I] fp32 (any sign).  scores is [B][n_q][ld_scores] fp32, ld_scores >= n_kv; only
 *   entries s <= pos_t are written, the rest of each row is left untouched.
 * Fast path: FP8 with H_I = 64, d_I = 128 (CDNA4 FP8 matrix cores).  Other shapes: a generic kernel
 *   (H_I <= 64, d_I <= 256, d_I % 4 == 0); anything else returns DSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_indexer_scores(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                const float* w, int B, int n_q, int n_kv, int H_I, int d_I,
                                dsa_dtype_t dtype, float* scores, int64_t ld_scores, void* stream);

/* ------------------------------------------------------------------------------------------------
 * dsa_topk -- fine-grained token selection (section 1.2 of the velog summary; k = 2048 in stage 2).
 *
 * For each query row: the min(k, pos_t + 1) positions s <= pos_t with the largest scores[b][t][s],
 * preferring the higher score and, among equal scores, the lower s; -0.0 equals +0.0.  Written to
 * idx[b][t][0..k) in ascending s, padded with -1.  scores is read only at s <= pos_t.
 * scores [B][n_q][ld_scores] fp32 (ld_scores >= n_kv), idx [B][n_q][k] int32.  1 <= k <= 65536.
 * Non-finite scores: NaN is not allowed (result unspecified); +-inf are ordered as usual.
 * workspace: device memory of at least dsa_topk_workspace_size(B, n_q, n_kv, k) bytes, 256-byte
 *   aligned (may be NULL when that size is 0).  Long rows, or too few rows to fill the GPU, are
 *   selected in two stages whose intermediate candidates live there; its contents are scratch.
 *   Too small, misaligned or missing when needed: DSA_ERR_WORKSPACE, nothing enqueued.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int B, int n_q, int n_kv, int k,
                      int32_t* idx, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes dsa_topk needs for this shape (0 for invalid sizes or when none is needed). */
size_t dsa_topk_workspace_size(int B, int n_q, int n_kv, int k);

/* ------------------------------------------------------------------------------------------------
 * dsa_sparse_mla_attn -- attention over the selected latent rows (sections 1.2 and 1.3 of the
 * velog summary).  For every query t and head h:
 *
 *   z_i   = sm_scale * q[b][t][h][:] . kv[b][s_i][:]     over s_i = idx[b][t][i] != -1
 *   out   = sum_i softmax(z)_i * kv[b][s_i][0:d_v]        (V = the first d_v columns of the row)
 *   lse   = log sum_i exp(z_i)                            (natural log)
 *
 * q [B][n_q][H][d_qk], kv [B][n_kv][d_qk] (one latent row per token, shared by all H heads),
 * idx [B][n_q][k] int32 with entries -1 (skipped) or in [0, n_kv) (entries outside are skipped too),
 * out [B][n_q][H][d_v] in `dtype`, lse [B][n_q][H] fp32 or NULL.  A row with no valid entry gets
 * out = 0 and lse = -inf.  sm_scale finite and > 0.
 * dtype = DSA_BF16: q, kv, out are bf16 (fp32 accumulation).  Fast path H = 128, d_qk = 576,
 *   d_v = 512 (CDNA4 bf16 matrix cores), n_kv <= 2^21 (DSA_ERR_UNSUPPORTED otherwise).
 * dtype = DSA_F32: q, kv, out fp32 (generic kernel: H <= 64, d_qk <= 256, d_v <= d_qk).
 * workspace: device memory of at least dsa_sparse_mla_attn_workspace_size(...) bytes, 256-byte
 *   aligned (may be NULL when that size is 0).
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_sparse_mla_attn(const void* q, const void* kv, const int32_t* idx, int B, int n_q,
                                 int n_kv, int H, int d_qk, int d_v, int k, float sm_scale,
                                 dsa_dtype_t dtype, void* out, float* lse, void* workspace,
                                 size_t ws_bytes, void* stream);

size_t dsa_sparse_mla_attn_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                          dsa_dtype_t dtype);

/* ------------------------------------------------------------------------------------------------
 * dsa_masked_mha_attn -- masked MHA mode for short prefills (velog summary, section 3.3 Inference
 * Cost; notes.yuuk.io, section on inference cost): attention in MHA form, each head with its own
 * key and value rows, computed densely over the causal keys with every key outside the query's
 * top-k selection masked out of the softmax.  For every query t (pos_t = n_kv - n_q + t) and head h:
 *
 *   z_s   = sm_scale * q[b][t][h][:] . k[b][s][h][:]     over S_t = { s = idx[b][t][i] : 0 <= s <= pos_t }
 *   out   = sum_{s in S_t} softmax(z)_s * v[b][s][h][:]
 *   lse   = log sum_{s in S_t} exp(z_s)                  (natural log)
 *
 * which is the attention over the selected entries (entries -1, duplicates-free as dsa_topk writes
 * them; entries outside [0, pos_t] are ignored).  A row with no such entry gets out = 0, lse = -inf.
 * q [B][n_q][H][d_qk], k [B][n_kv][H][d_qk], v [B][n_kv][H][d_v] (token-major, as an up-projection
 * of the latent rows writes them), idx [B][n_q][k_sel] int32, out [B][n_q][H][d_v],
 * lse [B][n_q][H] fp32 or NULL.
 * dtype = DSA_BF16 only, with d_qk = 192 and d_v = 128 (CDNA4 bf16 matrix cores, fp32 accumulation),
 *   any H; n_kv <= 524288.  q, k, v, out 16-byte aligned.  Other shapes: DSA_ERR_UNSUPPORTED.
 * workspace: device memory of at least dsa_masked_mha_workspace_size(B, n_q, n_kv) bytes, 256-byte
 *   aligned; it receives the selection as one bit per (query, key) (scratch).  Too small,
 *   misaligned or missing: DSA_ERR_WORKSPACE, nothing enqueued.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_masked_mha_attn(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                                 int n_q, int n_kv, int H, int d_qk, int d_v, int k_sel, float sm_scale,
                                 dsa_dtype_t dtype, void* out, float* lse, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Workspace bytes dsa_masked_mha_attn needs (0 for invalid sizes). */
size_t dsa_masked_mha_workspace_size(int B, int n_q, int n_kv);

/* ------------------------------------------------------------------------------------------------
 * dsa_warmup_loss -- the indexer's dense warm-up loss (velog summary, Continued Pre-Training, Stage 1):
 * the main model is frozen and the indexer learns to reproduce its attention.  For every query t
 * (pos_t = n_kv - n_q + t) and s <= pos_t:
 *
 *   target[t][s] = (1/H) sum_h exp(sm_scale * q[t][h] . kv[s] - lse[t][h])
 *                  (the main attention summed over heads and L1-normalised; lse[t][h] is that dense causal
 *                   attention's natural-log log-sum-exp, as its forward pass produces it)
 *   loss[t]      = KL(target[t] || softmax(I[t])) = sum_s target (log target - log softmax(I[t])_s)
 *   scores[t][s] <- softmax(I[t])_s - target[t][s]      (the gradient of sum_t loss[t] with respect to I)
 *
 * q [B][n_q][H][d_qk], kv [B][n_kv][d_qk] bf16 (the MQA-mode inputs of dsa_sparse_mla_attn, 16-byte
 * aligned), lse [B][n_q][H] fp32; scores [B][n_q][ld_scores] fp32 holds the index scores I on entry
 * (as dsa_indexer_scores writes them) and the gradient on return; target [B][n_q][ld_target] fp32
 * receives the target; loss [B][n_q] fp32.  Entries past pos_t are neither read nor written.
 * bf16 with H = 128 and d_qk = 576 only, n_kv <= 2^21 (DSA_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_warmup_loss(const void* q, const void* kv, const float* lse, int B, int n_q, int n_kv, int H,
                             int d_qk, float sm_scale, dsa_dtype_t dtype, float* scores, int64_t ld_scores,
                             float* target, int64_t ld_target, float* loss, void* stream);

/* dsa_warmup_indexer_backward -- gradients of sum_t loss[t] (dsa_warmup_loss) through the indexer
 * I[t][s] = sum_j w[t][j] ReLU(q^[t][j] . k^[s]), with q^ = q_i * q_i_scale and k^ = k_i * k_i_scale the
 * dequantised inputs, given grad = dL/dI (the scores buffer dsa_warmup_loss returns):
 *
 *   dw[t][j]      = sum_{s <= pos_t} grad[t][s] ReLU(q^[t][j] . k^[s])
 *   dq_i[t][j][:] = sum_{s <= pos_t} grad[t][s] w[t][j] [q^[t][j] . k^[s] > 0] k^[s][:]
 *   dk_i[s][:]    = sum_t sum_j grad[t][s] w[t][j] [q^[t][j] . k^[s] > 0] q^[t][j][:]
 *
 * Inputs as dsa_indexer_scores (fp8 e4m3 codes, fp32 scales, H_I = 64, d_I = 128); grad
 * [B][n_q][ld_grad] fp32 (entries past pos_t are not read).  Outputs fp32: dq_i [B][n_q][64][128]
 * (16-byte aligned), dw [B][n_q][64], dk_i [B][n_kv][128] (overwritten: zeroed, then parts of the queries
 * added with fp32 atomics, so the order of its sums varies between calls).  The ReLU decision is taken on
 * the codes' dot product in fp32 (the scales are positive).  n_kv <= 2^21.
 */
dsa_status_t dsa_warmup_indexer_backward(const void* q_i, const float* q_i_scale, const void* k_i,
                                         const float* k_i_scale, const float* w, const float* grad,
                                         int64_t ld_grad, int B, int n_q, int n_kv, int H_I, int d_I,
                                         dsa_dtype_t dtype, float* dq_i, float* dw, float* dk_i, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Sparse training stage (velog summary, Continued Pre-Training, Stage 2): the whole model trains
 * through the top-k selection; the indexer is detached from the main model and trained on its own loss.
 *
 * dsa_sparse_mla_backward -- gradients of dsa_sparse_mla_attn.  With P[t][h][j] the attention
 * probabilities over the valid entries of idx[t] (exp(sm_scale q . kv[s_j] - lse)), dP = dout . V and
 * D[t][h] = dout . out:
 *
 *   dS      = P (dP - D)
 *   dq[t][h]  = sm_scale sum_j dS_j kv[s_j]                              (576 columns)
 *   dkv[s]    = sum_{t,h,j: s_j = s} sm_scale dS_j q[t][h] + [P_j dout[t][h], 0]   (K and V share the row)
 *   pbar[t][j] = (1/H) sum_h P_j      (the indexer's target in this stage; 0 for invalid entries)
 *
 * Inputs as dsa_sparse_mla_attn (q [B][n_q][128][576], kv [B][n_kv][576] bf16, idx [B][n_q][k] int32 with
 * entries -1 or >= n_kv ignored, as there, and valid entries distinct), plus its outputs out
 * [B][n_q][128][512] bf16 and lse [B][n_q][128] fp32, and dout [B][n_q][128][512] bf16; q, kv, out, dout
 * 16-byte aligned.  Outputs fp32: dq [B][n_q][128][576], dkv [B][n_kv][576] (overwritten; the order in
 * which a key's terms are summed varies between calls), pbar [B][n_q][k] (may be NULL).  P, dS and each
 * entry's dkv terms pass through the workspace as bf16 (the second products round P and dS, as the
 * forward rounds P).  bf16, H = 128, d_qk = 576, d_v = 512, k <= 2048, n_kv <= 2^21, B n_kv <= 2^26 only
 * (DSA_ERR_UNSUPPORTED otherwise).  The workspace (256-byte aligned) holds P, dS and the dkv terms of up
 * to 512 query rows at a time and the per-key entry lists.
 */
size_t dsa_sparse_mla_backward_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                              dsa_dtype_t dtype);
dsa_status_t dsa_sparse_mla_backward(const void* q, const void* kv, const int32_t* idx, const void* out,
                                     const float* lse, const void* dout, int B, int n_q, int n_kv, int H,
                                     int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t dtype, float* dq,
                                     float* dkv, float* pbar, void* workspace, size_t ws_bytes, void* stream);

/* dsa_sparse_kl_loss -- the indexer loss of this stage, in the warm-up form with the sparse target:
 * p[t] = pbar[t] scattered to the entries idx[t] (0 elsewhere), loss[t] = KL(p[t] || softmax(I[t])) over
 * s <= pos_t, and scores[t][s] <- softmax(I[t])_s - p[t][s] (the gradient with respect to I, for
 * dsa_warmup_indexer_backward).  scores [B][n_q][ld_scores] fp32 (index scores in), pbar [B][n_q][k] fp32,
 * idx as above (entries outside [0, pos_t] are outside the loss and ignored), loss [B][n_q] fp32.
 */
dsa_status_t dsa_sparse_kl_loss(float* scores, int64_t ld_scores, const float* pbar, const int32_t* idx, int B,
                                int n_q, int n_kv, int k, float* loss, void* stream);

/* ------------------------------------------------------------------------------------------------
 * MQA-mode projections either side of dsa_sparse_mla_attn (velog summary, section 1.3: MLA in MQA
 * mode shares each latent entry across the query heads, so the key up-projection W_UK is absorbed
 * into the query and the value up-projection W_UV is applied after attention).  Per head h of each
 * of `rows` tokens (rows = B * n_q, any batch layout that is token-major):
 *
 *   dsa_mla_absorb_q:  q_mqa[r][h][0:d_c]        = sum_d q_mha[r][h][d] * W_UK,h[d][:]   (d < d_nope)
 *                      q_mqa[r][h][d_c:d_c+d_rope] = q_mha[r][h][d_nope:d_nope+d_rope]   (copied)
 *   dsa_mla_out_proj:  o[r][h][v]                = sum_c W_UV,h[v][c] * o_lat[r][h][c]
 *
 * Layouts: q_mha [rows][H][d_nope + d_rope], q_mqa [rows][H][d_c + d_rope] (the dsa_sparse_mla_attn
 * query), o_lat [rows][H][d_c] (its output), o [rows][H][d_v].  Weights are row-major with the
 * contraction dimension last: w_ukt [H][d_c][d_nope] (w_ukt[h][c][d] = W_UK,h[d][c]) and
 * w_uv [H][d_v][d_c].  bf16 in and out, fp32 accumulation; d_nope = 128, d_rope = 64, d_c = 512,
 * d_v = 128, any H, rows <= 2^30 and at most 2^31 - 1 workgroups (rows / 128 * H * 4 for the absorption).
 * All pointers 16-byte aligned.  Other shapes: DSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_mla_absorb_q(const void* q_mha, const void* w_ukt, void* q_mqa, int rows, int H,
                              int d_nope, int d_rope, int d_c, dsa_dtype_t dtype, void* stream);

dsa_status_t dsa_mla_out_proj(const void* o_lat, const void* w_uv, void* o, int rows, int H, int d_c,
                              int d_v, dsa_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------------------------------
 * dsa_forward_prefill -- the whole path for B sequences of n_kv tokens whose last n_q tokens are
 * queries: dsa_indexer_scores -> dsa_topk -> dsa_sparse_mla_attn on one stream.  Chunked prefill
 * is one call per chunk with n_kv growing by the chunk length (all state is in the caller's caches).
 *
 * Indexer inputs as in dsa_indexer_scores (idx_dtype, q_i, q_i_scale, k_i, k_i_scale, w, H_I, d_I);
 * attention inputs as in dsa_sparse_mla_attn (attn_dtype, q, kv, H, d_qk, d_v, sm_scale, out, lse).
 * idx_out: NULL, or [B][n_q][k] int32 that receives the selection (else it stays in the workspace).
 * workspace: at least dsa_forward_workspace_size(...) bytes, 256-byte aligned.  It holds the score
 *   rows ([B][n_q][ld] fp32, ld = n_kv rounded up to 64), the selection, the top-k candidates and
 *   the attention scratch.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_forward_prefill(const void* q_i, const float* q_i_scale, const void* k_i,
                                 const float* k_i_scale, const float* w, const void* q, const void* kv,
                                 int B, int n_q, int n_kv, int H_I, int d_I, int H, int d_qk, int d_v,
                                 int k, float sm_scale, dsa_dtype_t idx_dtype, dsa_dtype_t attn_dtype,
                                 void* out, float* lse, int32_t* idx_out, void* workspace,
                                 size_t ws_bytes, void* stream);

/* dsa_forward_decode -- the whole path for B sequences with one new query each (n_q = 1) at position
 * n_kv - 1, whose own key is already in the caches.  Same arguments as dsa_forward_prefill without
 * n_q; kernels tuned for few long rows (keys split over many workgroups, split-k attention). */
dsa_status_t dsa_forward_decode(const void* q_i, const float* q_i_scale, const void* k_i,
                                const float* k_i_scale, const float* w, const void* q, const void* kv,
                                int B, int n_kv, int H_I, int d_I, int H, int d_qk, int d_v, int k,
                                float sm_scale, dsa_dtype_t idx_dtype, dsa_dtype_t attn_dtype,
                                void* out, float* lse, int32_t* idx_out, void* workspace,
                                size_t ws_bytes, void* stream);

/* Workspace bytes for dsa_forward_prefill (n_q queries) or dsa_forward_decode (n_q = 1). */
size_t dsa_forward_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                  dsa_dtype_t attn_dtype);

/* ------------------------------------------------------------------------------------------------
 * Decode stage entry points: the three stages for B sequences with one new query each (n_q = 1) at
 * position n_kv - 1.  Each computes exactly what its general counterpart computes with n_q = 1 (same
 * sections of the pages, same layouts with the n_q dimension of size 1, same errors); they exist so a
 * decode step can be driven stage by stage through the kernels tuned for few long rows (keys split over
 * many workgroups, the selection in two stages, split-k attention with a merge).  The general calls pick
 * the same kernels when n_q = 1.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_indexer_scores_decode(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                       const float* w, int B, int n_kv, int H_I, int d_I, dsa_dtype_t dtype,
                                       float* scores, int64_t ld_scores, void* stream);
dsa_status_t dsa_topk_decode(const float* scores, int64_t ld_scores, int B, int n_kv, int k, int32_t* idx,
                             void* workspace, size_t ws_bytes, void* stream);
size_t dsa_topk_decode_workspace_size(int B, int n_kv, int k);
dsa_status_t dsa_sparse_mla_attn_decode(const void* q, const void* kv, const int32_t* idx, int B, int n_kv,
                                        int H, int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t dtype,
                                        void* out, float* lse, void* workspace, size_t ws_bytes,
                                        void* stream);
size_t dsa_sparse_mla_attn_decode_workspace_size(int B, int n_kv, int H, int d_qk, int d_v, int k,
                                                 dsa_dtype_t dtype);

/* ------------------------------------------------------------------------------------------------
 * dsa_forward_prefill_masked_mha -- the short-prefill form of the path (velog summary, section 3.3
 * Inference Cost: short prefills run MHA mode with a mask that reproduces the sparse selection;
 * notes.yuuk.io, section on inference cost): dsa_indexer_scores -> dsa_topk -> dsa_masked_mha_attn on
 * one stream.  The result equals the attention over the selected entries, in MHA form.
 *
 * Indexer inputs and idx_out as in dsa_forward_prefill; attention inputs as in dsa_masked_mha_attn
 * (q [B][n_q][H][192], k [B][n_kv][H][192], v [B][n_kv][H][128] bf16, out [B][n_q][H][128] bf16, lse
 * [B][n_q][H] fp32 or NULL), k_sel selected entries per query, n_kv <= 524288.  Which mode serves a
 * given prefill length is the caller's choice: masked MHA pays per causal (query, key) pair, the sparse
 * MQA path (dsa_forward_prefill) per selected entry, and the measured crossing is a prefill length of
 * about 9K tokens at k_sel = 2048.
 * workspace: at least dsa_forward_prefill_masked_mha_workspace_size(...) bytes, 256-byte aligned (score
 *   rows [B][n_q][ld] with ld = n_kv rounded up to 64, the selection, the top-k candidates and the
 *   selection bitmask).
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_forward_prefill_masked_mha(const void* q_i, const float* q_i_scale, const void* k_i,
                                            const float* k_i_scale, const float* w, const void* q, const void* k,
                                            const void* v, int B, int n_q, int n_kv, int H_I, int d_I, int H,
                                            int d_qk, int d_v, int k_sel, float sm_scale, dsa_dtype_t idx_dtype,
                                            dsa_dtype_t attn_dtype, void* out, float* lse, int32_t* idx_out,
                                            void* workspace, size_t ws_bytes, void* stream);
size_t dsa_forward_prefill_masked_mha_workspace_size(int B, int n_q, int n_kv, int k_sel);

/* ------------------------------------------------------------------------------------------------
 * dsa_forward_decode_noalloc -- dsa_forward_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments
 * and result as dsa_forward_decode without the workspace: the call's intermediates (score rows, the
 * selection unless idx_out is given, top-k candidates, split-k partials) live in a fixed device array of
 * dsa_forward_decode_noalloc_max_bytes() bytes (128 MiB) that the library holds on each device it runs
 * on until the process ends; nothing is allocated or freed by the call.  A shape whose intermediates
 * need more (dsa_forward_workspace_size(B, 1, n_kv, ...) above the limit; 64 sequences of 131072
 * tokens fit) returns DSA_ERR_UNSUPPORTED with nothing enqueued.  All calls on one device share that
 * device's array: calls that may overlap on one device (several streams or threads) race and must be
 * ordered by the caller.  No part of the array needs to start at zero.
 * ------------------------------------------------------------------------------------------------ */
dsa_status_t dsa_forward_decode_noalloc(const void* q_i, const float* q_i_scale, const void* k_i,
                                        const float* k_i_scale, const float* w, const void* q, const void* kv,
                                        int B, int n_kv, int H_I, int d_I, int H, int d_qk, int d_v, int k,
                                        float sm_scale, dsa_dtype_t idx_dtype, dsa_dtype_t attn_dtype,
                                        void* out, float* lse, int32_t* idx_out, void* stream);
size_t dsa_forward_decode_noalloc_max_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
