/*
 * sprint.h -- C ABI of libsprint.so: the SPRINT block-wise masked-diffusion
 * denoising step as HIP kernels for MI355X (gfx950).
 *
 * Method: "LLaDA2.0-Uni: Unifying Multimodal Understanding and Generation with
 * Diffusion Large Language Model" (arXiv 2604.20796), the SPRINT paragraphs
 * ("Sparse Prefix Retention", "Non-uniform Token Unmasking") and the block
 * notation of its "BDLM Loss" paragraph.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless a comment says "host".
 *  - The caller owns all memory; the library never allocates or frees.
 *    Scratch memory is a caller buffer `ws` of at least the bytes returned by
 *    the matching *_ws() query.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on it; no call synchronises the device.
 *  - Arguments are validated on the host before any HIP call; a failure
 *    returns its SPRINT_E* code and writes nothing.  A kernel launch failure
 *    returns SPRINT_EHIP.  Device faults surface at the caller's next sync.
 *  - Tensors are dense, row-major and position-major.  Large operands (K, V,
 *    Q, O, W, hidden, K_out, V_out, ws) must be 16-byte aligned; 4-byte
 *    arrays 4-byte aligned.
 *  - dtype: SPRINT_F32 (float) or SPRINT_BF16 (bfloat16 bit patterns);
 *    reductions and softmax statistics are computed in fp32.
 *  - Results are deterministic: no floating-point atomics are used, so the
 *    same inputs give bitwise-identical outputs.
 *  - Non-finite inputs violate the preconditions; results are then unspecified.
 *  - Calls that share a workspace must not overlap in time.
 *  - Size limits common to every call (SPRINT_EUNSUPPORTED beyond them):
 *    nseq <= 2^24 sequences; a key/value row (Hkv * D * element size) of at
 *    most 1 MiB, and a K or V array (all layers) under 2^48 bytes.  The
 *    *_ws() queries return 0 for sizes beyond their call's range.
 */
#ifndef SPRINT_H
#define SPRINT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPRINT_OK = 0,
  SPRINT_EINVAL = 1,       /* bad pointer, size or shape */
  SPRINT_EUNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim not 64/128) */
  SPRINT_EWORKSPACE = 3,   /* ws smaller than the *_ws() query */
  SPRINT_EHIP = 4          /* a HIP launch failed */
};

enum { SPRINT_F32 = 0, SPRINT_BF16 = 1 };

/* Human-readable name of a status code (static string). */
const char* sprint_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int sprint_version(void);

/* ------------------------------------------------------------------------
 * Keep counts (host only).  Sparse Prefix Retention keeps floor(r*n) positions
 * of a modality that has n prefix positions.  Evaluated as IEEE fp64
 * floor(r*n), clamped to [0, n]; no minimum of one.
 * ------------------------------------------------------------------------ */
int64_t sprint_keep_count(double r, int64_t n);

/* Per-sequence keep counts and output offsets, all HOST arrays:
 *   n_text, n_img [nseq]   prefix positions of each modality per sequence
 *   keep   [nseq*2]        out: (text, image) counts = sprint_keep_count(r_m, n_m)
 *   cu_kept[nseq+1]        out: exclusive prefix sum of keep per sequence
 *   total_kept             out: cu_kept[nseq]
 * Returns SPRINT_EINVAL on NULL pointers, nseq < 1 or negative counts. */
int sprint_plan_keep(const int64_t* n_text, const int64_t* n_img, int32_t nseq,
                     double r_text, double r_img, int32_t* keep, int32_t* cu_kept,
                     int64_t* total_kept);

/* ------------------------------------------------------------------------
 * LM-head confidence.  Sparse Prefix Retention scores position i with its
 * top-1 softmax probability c_i = max_v p(v | x_t); Non-uniform Token
 * Unmasking uses c_n = p(x0_hat | x_t) for the greedy prediction, the same
 * number.  For each row x of `hidden`:
 *     z = W x  (z_v = sum_h W[v,h] x[h], fp32 accumulation),
 *     argmax = lowest v with z_v = max z,
 *     conf = 1 / sum_v exp(z_v - max z),   lse = max z + log(sum_v exp(z_v - max z)).
 * The [M, V] logits never reach memory: each vocabulary tile keeps a running
 * (max, sum of exp, argmax) that a merge kernel combines.
 *   hidden [M, H] dtype;  W [V, H] dtype (nn.Linear layout)
 *   conf [M] float out;  argmax [M] int32 out;  lse [M] float out or NULL
 * Requires M >= 1, V >= 1, H a multiple of 64 (<= 65536); V < 2^30.
 * ------------------------------------------------------------------------ */
size_t lmhead_confidence_ws(int64_t M, int32_t H, int32_t V, int32_t dtype);
int lmhead_confidence(const void* hidden, int64_t M, int32_t H, const void* W, int32_t V,
                      int32_t dtype, float* conf, int32_t* argmax, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Composite prefix score (Sparse Prefix Retention).
 *   n_i   = ||K[i,:,:]||_2  over all KV heads and head dims (the position's key
 *           is the concatenation of its KV heads),
 *   I_i   = n_i / ((1/L) sum_{j in seq} n_j)   (1 when the sequence's keys are all 0),
 *   s_i   = alpha * I_i + (1 - alpha) * c_i.
 * The page's score equation is missing; the linear blend is the reading used.
 *   K     [total_L, Hkv, D] dtype, sequences packed by cu_len [nseq+1] (int32,
 *         cu_len[0] = 0, non-decreasing, cu_len[nseq] = total_L)
 *   conf  [total_L] float   prefix confidences (lmhead_confidence over the prefix)
 *   ibar  [total_L] float out;  score [total_L] float out
 * ------------------------------------------------------------------------ */
size_t sprint_score_ws(int64_t total_L, int32_t nseq);
int sprint_score(const void* K, const float* conf, const int32_t* cu_len, int32_t nseq,
                 int64_t total_L, int32_t Hkv, int32_t D, int32_t dtype, float alpha,
                 float* ibar, float* score, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Modality-aware pruning and compaction of the prefix KV cache (Sparse Prefix
 * Retention).  For each sequence s and modality m (0 text, 1 image) the
 * min(keep[2s+m], n_{s,m}) positions with the largest score are kept; equal
 * scores keep the lower position; all runs of one modality in a sequence are
 * pooled.  The kept rows, in ascending position order, are copied into a
 * contiguous pruned cache:
 *   kept_idx[j] = global row of K kept at output row j (ascending),
 *   K_out[j] = K[kept_idx[j]],  V_out[j] = V[kept_idx[j]]  (bit copies).
 *   score    [total_L] float;  modality [total_L] uint8 (0 text, 1 image)
 *   keep     [nseq*2] int32 device (from sprint_plan_keep)
 *   cu_kept  [nseq+1] int32 device (from sprint_plan_keep); total_kept = cu_kept[nseq]
 *   K, V     [total_L, Hkv, D] dtype;  K_out, V_out [total_kept, Hkv, D] dtype out
 *   kept_idx [total_kept] int32 out
 * Precondition: cu_kept must be the prefix sum of min(keep, n) per sequence;
 * the kernels never write outside [cu_kept[s], cu_kept[s+1]) or total_kept.
 * Scores are ranked as IEEE values (-0 equal to +0); NaN scores, and modality
 * bytes other than 0 and 1, have no defined ranking.
 * K_out and V_out (per layer) must be under 2 GiB each: total_kept * Hkv * D *
 * element size >= 2^31 returns SPRINT_EUNSUPPORTED.
 * ------------------------------------------------------------------------ */
size_t sprint_prune_kv_ws(int64_t total_L, int32_t nseq);
int sprint_prune_kv(const float* score, const uint8_t* modality, const int32_t* cu_len,
                    const int32_t* keep, const int32_t* cu_kept, int32_t nseq, int64_t total_L,
                    int64_t total_kept, const void* K, const void* V, int32_t Hkv, int32_t D,
                    int32_t dtype, void* K_out, void* V_out, int32_t* kept_idx, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Several layers sharing one kept set (Sparse Prefix Retention applied to a
 * model whose every layer holds a prefix KV cache; the page scores positions,
 * not layers, so one set serves every layer).  The key-norm importance is
 * the mean over layers of each layer's mean-normalised key norm:
 *   I_i = (1/n_layers) sum_l n_i^l / ((1/L) sum_{j in seq} n_j^l),
 *   s_i = alpha * I_i + (1 - alpha) * c_i,
 * and the kept set selected from s is compacted in every layer's cache.
 *   K, V    [n_layers, total_L, Hkv, D] dtype (layer-major)
 *   K_out, V_out [n_layers, total_kept, Hkv, D] dtype out
 *   kept_idx [total_kept] int32 out (one set for all layers)
 * Other arguments as for sprint_score / sprint_prune_kv; n_layers = 1 gives
 * exactly their results.  1 <= n_layers <= 65535.  The prune's workspace is
 * sprint_prune_kv_ws(total_L, nseq) for any number of layers.
 * ------------------------------------------------------------------------ */
size_t sprint_score_layers_ws(int64_t total_L, int32_t nseq, int32_t n_layers);
int sprint_score_layers(const void* K, int32_t n_layers, const float* conf, const int32_t* cu_len,
                        int32_t nseq, int64_t total_L, int32_t Hkv, int32_t D, int32_t dtype,
                        float alpha, float* ibar, float* score, void* ws, size_t ws_bytes,
                        void* stream);
int sprint_prune_kv_layers(const float* score, const uint8_t* modality, const int32_t* cu_len,
                           const int32_t* keep, const int32_t* cu_kept, int32_t nseq,
                           int64_t total_L, int64_t total_kept, const void* K, const void* V,
                           int32_t n_layers, int32_t Hkv, int32_t D, int32_t dtype, void* K_out,
                           void* V_out, int32_t* kept_idx, void* ws, size_t ws_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * Several layers, each with its own kept set (Sparse Prefix Retention
 * applied layer by layer: every layer scores its own keys with the shared
 * prefix confidences and keeps its own top positions).  One call does what
 * n_layers calls of sprint_score, then of sprint_prune_kv, do, with the
 * same results bit for bit:
 *   I_i^l = n_i^l / ((1/L) sum_{j in seq} n_j^l),  s_i^l = alpha*I_i^l + (1-alpha)*c_i.
 *   K, V     [n_layers, total_L, Hkv, D] dtype (layer-major)
 *   ibar, score [n_layers, total_L] float out (score: in, for the prune)
 *   K_out, V_out [n_layers, total_kept, Hkv, D] dtype out
 *   kept_idx [n_layers, total_kept] int32 out (layer l's set in row l)
 * keep / cu_kept / total_kept are per sequence and modality, so every layer
 * keeps the same number of rows.  1 <= n_layers <= 65535.  The score's
 * workspace is sprint_score_layers_ws(total_L, nseq, n_layers); the prune's
 * is sprint_prune_kv_per_layer_ws(total_L, nseq, n_layers).
 * ------------------------------------------------------------------------ */
int sprint_score_per_layer(const void* K, int32_t n_layers, const float* conf,
                           const int32_t* cu_len, int32_t nseq, int64_t total_L, int32_t Hkv,
                           int32_t D, int32_t dtype, float alpha, float* ibar, float* score,
                           void* ws, size_t ws_bytes, void* stream);
size_t sprint_prune_kv_per_layer_ws(int64_t total_L, int32_t nseq, int32_t n_layers);
int sprint_prune_kv_per_layer(const float* score, const uint8_t* modality, const int32_t* cu_len,
                              const int32_t* keep, const int32_t* cu_kept, int32_t nseq,
                              int64_t total_L, int64_t total_kept, const void* K, const void* V,
                              int32_t n_layers, int32_t Hkv, int32_t D, int32_t dtype,
                              void* K_out, void* V_out, int32_t* kept_idx, void* ws,
                              size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Block attention of a denoising step (LLaDA2.0-Uni: "Sparse Prefix
 * Retention" -- the block's first step attends to the full prefix cache and
 * every later step to the pruned one; "BDLM Loss" -- a block is predicted
 * from the clean earlier blocks and its own noisy tokens, so the block's own
 * keys join the context, without a mask inside the block).  With GQA, query
 * head h reads KV head floor(h*Hkv/Hq).  O = softmax(Q K^T * scale) V per
 * (sequence, head) over the keys [prefix cache ; block].
 *   Q      [nseq, Lq, Hq, D] dtype
 *   Kp, Vp [total_kv, Hkv, D] dtype, sequences packed by cu_kv [nseq+1]
 *          (full cache, or the pruned cache of sprint_prune_kv)
 *   max_kv host estimate of the longest sequence's cache length; it sizes the
 *          split of each cache into key ranges (and so the workspace).  A
 *          longer sequence is still attended in full (its last key range
 *          covers the rest; only slower).  With nseq = 1 the one cache is all
 *          total_kv rows, so total_kv > max_kv is SPRINT_EINVAL there
 *   Kb, Vb [nseq, Lq, Hkv, D] dtype, or both NULL for prefix-only attention
 *   scale  softmax scale, finite and > 0 (usually 1/sqrt(D))
 *   O      [nseq, Lq, Hq, D] dtype out (bf16 rounded to nearest even)
 * Supports D in {64, 128}, Hq % Hkv == 0, (Hq/Hkv)*Lq <= 256, Lq <= 64, and
 * Kp, Vp, Kb, Vb each under 2 GiB (SPRINT_EUNSUPPORTED otherwise).
 * Every (sequence) must have at least one key (cache length + block >= 1).
 * Partial results of key ranges are kept in ws in fp32 (fp32 inputs) or in
 * fp16 with a power-of-two scale per row (bf16 inputs), so every finite bf16
 * value is in range; products that overflow fp32 are out of range.
 * ------------------------------------------------------------------------ */
size_t block_attend_ws(int32_t nseq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_kv, int32_t has_block);
int block_attend(const void* Q, int32_t nseq, int32_t Lq, int32_t Hq, const void* Kp,
                 const void* Vp, const int32_t* cu_kv, int64_t total_kv, int32_t max_kv,
                 const void* Kb, const void* Vb, int32_t Hkv, int32_t D, float scale,
                 int32_t dtype, void* O, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * block_attend without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as block_attend, bit for
 * bit; the key-range partials live in a fixed device array of 16 MiB
 * (16 << 20 bytes) that each GPU the library runs on holds until the
 * process ends.  A call whose block_attend_ws(...) exceeds 16 MiB returns
 * SPRINT_EWORKSPACE before any HIP call.  The call allocates nothing:
 * the array's address is looked up (hipGetSymbolAddress) on the first call
 * on each device.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (on different streams, or from several
 * host threads) race; serialise them.  Nothing in the array needs to start
 * at any value: every partial is written before it is read.
 * ------------------------------------------------------------------------ */
int block_attend_noalloc(const void* Q, int32_t nseq, int32_t Lq, int32_t Hq, const void* Kp,
                         const void* Vp, const int32_t* cu_kv, int64_t total_kv, int32_t max_kv,
                         const void* Kb, const void* Vb, int32_t Hkv, int32_t D, float scale,
                         int32_t dtype, void* O, void* stream);

/* ------------------------------------------------------------------------
 * Confidence-adaptive unmasking, one step (Non-uniform Token Unmasking).
 * For each sequence: m = number of masked positions; q = min(m, ceil(m /
 * steps_left)) where steps_left = T - t (steps_left <= 0 accepts all m);
 * count = max(#{masked i : conf[i] > tau}, q).  The `count` masked positions
 * first in (conf descending, position ascending) order are accepted:
 * tokens[i] = argmax[i], masked[i] = 0.  With tau > 1 only the minimum acts.
 * A huge steps_left gives "at least one per step".
 *   conf [nseq, Lq] float;  argmax [nseq, Lq] int32
 *   masked [nseq, Lq] uint8 in/out (1 = masked);  tokens [nseq, Lq] int32 in/out
 *   n_accepted [nseq] int32 out
 * Requires 1 <= Lq <= 64.
 * ------------------------------------------------------------------------ */
int unmask_select(const float* conf, const int32_t* argmax, int32_t nseq, int32_t Lq, float tau,
                  int32_t steps_left, uint8_t* masked, int32_t* tokens, int32_t* n_accepted,
                  void* stream);

/* ------------------------------------------------------------------------
 * The end of one denoising step, fused: lmhead_confidence over the block's
 * rows, then unmask_select on the result (Non-uniform Token Unmasking: the
 * confidences c_n of the greedy predictions decide which masked positions
 * are accepted).  Same results, bit for bit, as
 *     lmhead_confidence(hidden, nseq*Lq, H, W, V, dtype, conf, argmax, NULL, ...)
 *     unmask_select(conf, argmax, nseq, Lq, tau, steps_left, masked, tokens,
 *                   n_accepted, ...)
 * in one call.  For bf16 with nseq*Lq <= 64 and H a multiple of 256 it takes
 * two launches instead of three: the block that merges the last row of a
 * sequence also runs that sequence's unmasking step.  Other shapes run the
 * two calls' launches in turn.
 *   hidden [nseq*Lq, H] dtype;  W [V, H] dtype;  conf [nseq*Lq] float out;
 *   argmax [nseq*Lq] int32 out;  masked [nseq, Lq] uint8 in/out;
 *   tokens [nseq, Lq] int32 in/out;  n_accepted [nseq] int32 out
 * Requires the limits of both calls (1 <= Lq <= 64, H a multiple of 64 up
 * to 65536, V < 2^30).  The workspace holds lmhead_confidence's plus one
 * counter per sequence; the call sets what it needs, so it may hold
 * anything on entry.  Calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------ */
size_t lmhead_confidence_unmask_ws(int32_t nseq, int32_t Lq, int32_t H, int32_t V,
                                   int32_t dtype);
int lmhead_confidence_unmask(const void* hidden, int32_t nseq, int32_t Lq, int32_t H,
                             const void* W, int32_t V, int32_t dtype, float* conf,
                             int32_t* argmax, float tau, int32_t steps_left, uint8_t* masked,
                             int32_t* tokens, int32_t* n_accepted, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Prefix growth between blocks (block-wise generation, SPRINT introduction;
 * Sparse Prefix Retention: each block's first step sees the complete cache,
 * so a finished block joins the prefix before the next block is scored and
 * pruned).  Appends n_blk rows to every sequence of a packed array:
 *   out rows [cu_old[s] + s*n_blk, cu_old[s+1] + s*n_blk) = old rows
 *   [cu_old[s], cu_old[s+1]), followed by blk rows [s*n_blk, (s+1)*n_blk).
 * Rows are opaque bytes (K, V, hidden-state or modality rows), bit-copied.
 *   old    [total_old rows of row_bytes], packed by cu_old [nseq+1] int32
 *          (cu_old[0] = 0, non-decreasing, cu_old[nseq] = total_old)
 *   blk    [nseq * n_blk rows] (sequence s's rows first-to-last)
 *   out    [total_old + nseq*n_blk rows] out; must not overlap old or blk
 *   cu_out [nseq+1] int32 out, cu_old[s] + s*n_blk; may be NULL; must not
 *          alias cu_old
 * Rows of 16-byte multiples with 16-byte aligned pointers move as 16-byte
 * vectors, other rows byte by byte.  Rows whose sequence range is
 * inconsistent with total_old are left unwritten (no out-of-range access).
 * ------------------------------------------------------------------------ */
int sprint_append_rows(const void* old, const int32_t* cu_old, int32_t nseq, int64_t total_old,
                       const void* blk, int32_t n_blk, int64_t row_bytes, void* out,
                       int32_t* cu_out, void* stream);

/* ------------------------------------------------------------------------
 * MoE FFN on synthetic weights (the backbone's expert layer; LLaDA2.0-Uni,
 * "Load Balancing Strategy": an auxiliary-loss-free bias steers expert
 * selection, and routing gates are scaled by 2.5).  Per token t:
 *   s_e  = sigmoid(x_t . w_router[e]),
 *   the top_k experts by s_e + bias[e] (lower expert index on ties), in
 *   selection order e_{t,0..top_k-1},
 *   g_j  = route_scale * s_{e_j} / sum_j s_{e_j},
 *   y_t  = residual_t + sum_j g_j * w_down[e_j] (silu(w_gate[e_j] x_t) * (w_up[e_j] x_t)).
 *   x        [M, H] dtype;  w_router [E, H] dtype;  bias [E] float
 *   w_gate, w_up [E, inter, H] dtype;  w_down [E, H, inter] dtype
 *   residual [M, H] dtype or NULL;  y [M, H] dtype out (may equal residual)
 *   expert_ids [M, top_k] int32 out;  gates [M, top_k] float out
 * Every chosen expert's weights are read once per call (a grouped
 * matrix-vector product for the few tokens of a denoising step).
 * Supported: H a multiple of 512 (bf16) or 256 (fp32) up to 2048 / 1024,
 * inter a multiple of 512 / 256 up to 1024 / 512, E <= 1024, top_k <= 16,
 * M <= 1024, M * top_k <= 8192; other shapes return SPRINT_EUNSUPPORTED.
 * top_k > n_experts or a non-finite route_scale is SPRINT_EINVAL.
 * ------------------------------------------------------------------------ */
size_t moe_ffn_ws(int32_t M, int32_t H, int32_t n_experts, int32_t top_k, int32_t inter);
int moe_ffn(const void* x, int32_t M, int32_t H, const void* w_router, const float* bias,
            int32_t n_experts, int32_t top_k, float route_scale, const void* w_gate,
            const void* w_up, const void* w_down, int32_t inter, int32_t dtype,
            const void* residual, void* y, int32_t* expert_ids, float* gates, void* ws,
            size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPRINT_H */
