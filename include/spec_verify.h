/*
 * spec_verify.h -- C ABI of the speculative-decoding verify step on MI355X
 * (gfx950).
 *
 * The verify step takes the target model's hidden states at the K+1 verify
 * positions of each sequence (the last accepted token and the K drafts), turns
 * them into logits with the LM head, and decides how many drafts to keep:
 *
 *   spec_verify_logits  -- logits = hidden . W_lmheadᵀ (the target's single
 *                          pass yields one distribution per draft position plus
 *                          one after the last draft: "Inference-4",
 *                          Draft-model speculative decoding, step 2; the
 *                          weights are read once for all positions:
 *                          "speculative-decoding" blog, Verification mechanism).
 *   spec_accept_greedy  -- accept drafts while they equal the target's most
 *                          likely token, then emit the target's token at the
 *                          first mismatch or the bonus token after the last
 *                          draft ("Inference-4", greedy bullet).
 *   spec_accept_sample  -- speculative sampling: accept draft x with
 *                          probability min(1, q(x)/p(x)) (q target, p draft),
 *                          stop at the first rejection and redraw it from
 *                          norm(max(0, q - p)); if all K are accepted draw a
 *                          bonus token from q after the last draft
 *                          ("Inference-4", sampling bullet; "speculative-
 *                          decoding" blog, Rejection sampling; "What is
 *                          speculative decoding" guide, How speculative
 *                          decoding works).
 *   spec_accept_greedy_ragged, spec_accept_sample_ragged
 *                       -- the same two rules on a batch whose sequences carry
 *                          different draft counts K_b (0 <= K_b <= K_max),
 *                          rows packed without padding.  A drafter may return
 *                          fewer drafts than asked, or none ("Inference-4",
 *                          Prompt lookup decoding, and the draft count capped
 *                          by the context window in its verification loop);
 *                          a scheduler may choose how many drafts to verify
 *                          per request ("speculative-decoding" blog, DSpark,
 *                          confidence-scheduled verification) or shorten them
 *                          under load ("Speculative decoding" course page, Why
 *                          engines disable speculation under load).
 *   spec_tree_accept_greedy
 *                       -- greedy verification of a draft tree: keep the
 *                          longest root-to-node path the target agrees with
 *                          ("Inference-4", Medusa; "speculative-decoding"
 *                          blog, Medusa and EAGLE-2; "Speculative decoding"
 *                          course page, One pass, many candidate
 *                          continuations).
 *   spec_verify_step    -- the whole step in one call: LM head, statistics
 *                          (computed by the LM-head kernel itself wherever a
 *                          bf16 kernel with that option runs, which saves a
 *                          pass over the logits) and both accept rules.
 *   spec_verify_step_ragged
 *                       -- the same for ragged batches (packed rows, a draft
 *                          count per sequence).
 *   spec_tree_verify_step
 *                       -- the same for draft trees: LM head and the greedy
 *                          tree rule in one call.
 *   spec_ngram_propose  -- the step before verification for prompt lookup:
 *                          drafts copied from the most recent earlier
 *                          occurrence of the sequence's last n tokens
 *                          ("Inference-4", Prompt lookup decoding).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory on the current HIP device, owned
 *     by the caller.  The library allocates nothing and keeps no state between
 *     calls other than a per-device cache of the compute-unit count and of
 *     the address of spec_verify_step_noalloc's scratch array.
 *   - Every call is asynchronous: it validates its arguments on the host,
 *     enqueues kernels on `stream` and returns.  It never synchronises.  The
 *     caller synchronises (event or stream) before reading outputs.
 *   - Sizes: B sequences, K drafts per sequence (0 <= K <= 63; the accept
 *     kernel scans the K+1 positions of a sequence in one 64-lane wavefront),
 *     vocabulary V >= 1, hidden size H (a positive multiple of 8, so rows are
 *     16-byte aligned for 128-bit loads).  M = B*(K+1) verify rows.
 *   - Layouts are row-major and contiguous:
 *       hidden        [B, K+1, H]   bf16 or fp32
 *       w_lmhead      [V, H]        bf16 or fp32 (same dtype as hidden)
 *       logits        [B, K+1, V]   fp32  (target logits, row b*(K+1)+i)
 *       draft_logits  [B, K, V]     fp32  (draft logits, row b*K+i)
 *       draft_tokens  [B, K]        int32
 *       seeds         [B]           uint64 (per-sequence Philox key)
 *       accepted_len  [B]           int32
 *       out_tokens    [B, K+1]      int32
 *   - Errors the host can see (null pointers, bad sizes, misalignment, a
 *     non-positive or non-finite temperature, a short workspace) return a
 *     status before anything is enqueued.  A failed HIP launch returns
 *     SPEC_ERR_HIP; spec_last_error_detail() then names the HIP error.
 *   - Data faults found on the device mark the sequence instead of failing
 *     the call: accepted_len[b] = -1 and out_tokens[b, :] = -1 when a draft
 *     token lies outside [0, V), or any of the sequence's target (or, in
 *     sampled mode, draft) rows holds a NaN or +inf, or has no finite entry.
 *
 * Random numbers (sampled mode): for sequence slot b and verify position i the
 * step draws one Philox4x32-10 block (Salmon et al., SC'11) with counter
 * (i, b, 0, 0) and key (low 32 bits of seeds[b], high 32 bits).  Word 0 gives
 * the accept uniform u_i = (w0 >> 8) * 2^-24 and word 1 the terminal uniform
 * u'_i = (w1 >> 8) * 2^-24.  A draft is accepted iff u_i < r_i; the terminal
 * token is t = min{v : C_v > u'_n * Z}, C the in-order cumulative sum of the
 * terminal weights and Z their total.  The result is a pure function of the
 * inputs and seeds: a round replays exactly.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
    SPEC_OK = 0,
    SPEC_ERR_ARG = 1,        /* null pointer, size out of range, bad temperature */
    SPEC_ERR_DTYPE = 2,      /* unsupported element type */
    SPEC_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned */
    SPEC_ERR_WORKSPACE = 4,  /* workspace NULL or smaller than spec_workspace_bytes() */
    SPEC_ERR_HIP = 5,        /* a HIP call or kernel launch failed */
    SPEC_STATUS_MAX_ENUM = 0x7fffffff   /* not a status: makes every non-negative int a value
                                           of the type, so an unknown code is well defined */
} spec_status_t;

typedef enum spec_dtype {
    SPEC_BF16 = 0,           /* bfloat16, storage as uint16 bit patterns */
    SPEC_F32 = 1,            /* IEEE binary32 */
    SPEC_DTYPE_MAX_ENUM = 0x7fffffff    /* not a type: as above (rejected with SPEC_ERR_DTYPE) */
} spec_dtype_t;

/* A hipStream_t.  NULL selects the null stream of the current device. */
typedef void* spec_stream_t;

/*
 * spec_verify_logits -- LM-head contraction of the K+1 verify positions.
 *
 *   logits[m, v] = sum_h hidden[m, h] * w_lmhead[v, h],  m < B*(K+1), v < V
 *
 * Products and sums are in fp32 (bf16 x bf16 products are exact in fp32; the
 * bf16 path runs on the matrix cores).  The order of the fp32 sum over h is
 * the kernel's and is fixed for a given (B, K, V, H, dtype).
 *
 *   hidden     device, [B, K+1, H] of `dtype`, 16-byte aligned
 *   w_lmhead   device, [V, H] of `dtype`, 16-byte aligned
 *   dtype      SPEC_BF16 or SPEC_F32 (hidden and weights share it)
 *   logits     device, [B, K+1, V] fp32, written, 16-byte aligned
 *   B, K, V, H sizes as above
 *   stream     HIP stream
 *
 * Returns SPEC_ERR_ARG for null pointers or sizes out of range,
 * SPEC_ERR_DTYPE for an unknown dtype, SPEC_ERR_ALIGN for misaligned pointers,
 * SPEC_ERR_HIP if a launch fails.
 */
spec_status_t spec_verify_logits(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                 float* logits, int B, int K, int V, int H,
                                 spec_stream_t stream);

/*
 * spec_accept_greedy -- greedy verification of the selected sequences.
 *
 * For each selected sequence b: a_i = argmax_v logits[b, i, v] for i = 0..K
 * (the lowest index wins a tie); n = the number of leading drafts with
 * draft_tokens[b, i] == a_i; then accepted_len[b] = n and out_tokens[b, :] =
 * (d_0, ..., d_{n-1}, a_n, -1, ..., -1).  a_K is the bonus token.
 *
 *   logits        device, [B, K+1, V] fp32, 16-byte aligned
 *   draft_tokens  device, [B, K] int32 (may be NULL when K == 0)
 *   rows          device, [n_rows] int32: the sequences to verify, distinct,
 *                 each in [0, B) (entries outside are skipped).  NULL means
 *                 all B sequences (n_rows is then ignored).
 *   n_rows        0 <= n_rows <= B
 *   accepted_len  device, [B] int32, written for the selected rows only
 *   out_tokens    device, [B, K+1] int32, written for the selected rows only
 *   workspace     device scratch of at least spec_workspace_bytes(B, K, V)
 *                 bytes, 16-byte aligned; its contents on entry do not matter.
 *                 Calls that share a workspace must be ordered on one stream.
 *   workspace_bytes  its size
 *   stream        HIP stream
 */
spec_status_t spec_accept_greedy(const float* logits, const int32_t* draft_tokens,
                                 const int32_t* rows, int n_rows, int B, int K, int V,
                                 int32_t* accepted_len, int32_t* out_tokens,
                                 void* workspace, size_t workspace_bytes,
                                 spec_stream_t stream);

/*
 * spec_accept_sample -- speculative sampling of the selected sequences.
 *
 * q_i = softmax(logits[b, i, :] / T) for i = 0..K and p_i =
 * softmax(draft_logits[b, i, :] / T) for i < K (the same temperature divides
 * both).  With d_i = draft_tokens[b, i] and (u_i, u'_i) the Philox uniforms
 * above:
 *   r_i = min(1, q_i(d_i) / p_i(d_i))   (r_i = 0 if q_i(d_i) = 0; 1 if p_i(d_i) = 0 < q_i(d_i))
 *   n   = the first i < K with u_i >= r_i, else K
 *   w   = max(0, q_n - p_n) if n < K (q_n itself if that has no mass), else q_K
 *   t   = min{v : C_v > u'_n * Z},  C_v = w_0 + ... + w_v,  Z = C_{V-1}
 * accepted_len[b] = n;  out_tokens[b, :] = (d_0, ..., d_{n-1}, t, -1, ...).
 *
 *   logits, draft_tokens, rows, n_rows, accepted_len, out_tokens, workspace,
 *   workspace_bytes, stream: as in spec_accept_greedy
 *   draft_logits    device, [B, K, V] fp32, 16-byte aligned (NULL when K == 0)
 *   temperature     T, finite and > 0
 *   seeds           device, [B] uint64
 *   probs_at_draft  device, [B, K, 2] fp32 or NULL: (q_i(d_i), p_i(d_i)) for
 *                   every i < K of the selected rows
 */
spec_status_t spec_accept_sample(const float* logits, const float* draft_logits,
                                 const int32_t* draft_tokens, float temperature,
                                 const uint64_t* seeds, const int32_t* rows, int n_rows,
                                 int B, int K, int V,
                                 int32_t* accepted_len, int32_t* out_tokens,
                                 float* probs_at_draft,
                                 void* workspace, size_t workspace_bytes,
                                 spec_stream_t stream);

/*
 * Ragged batches.  Sequence b has K_b drafts, 0 <= K_b <= K_max <= 63, and its
 * rows are packed in sequence order with no padding:
 *   row_start     device, [B+1] int32, 4-byte aligned: row_start[0] = 0 and
 *                 row_start[b+1] = row_start[b] + K_b + 1, so row_start[B] =
 *                 total_rows.  Sequence b owns target rows row_start[b] ..
 *                 row_start[b] + K_b and draft rows / tokens row_start[b] - b
 *                 .. row_start[b] - b + K_b - 1.
 *   total_rows    R = sum_b (K_b + 1), with B <= R <= B*(K_max+1)
 *   logits        device, [R, V] fp32 (spec_verify_logits with B = R, K = 0
 *                 computes it from hidden states packed the same way)
 *   draft_logits  device, [R-B, V] fp32 (sampled; may be NULL when R == B)
 *   draft_tokens  device, [R-B] int32 (may be NULL when R == B)
 *   accepted_len  device, [B] int32, n in 0..K_b
 *   out_tokens    device, [R] int32: entries row_start[b] .. row_start[b]+K_b
 *                 hold (d_0, ..., d_{n-1}, t, -1, ...) of sequence b
 *   probs_at_draft  device, [R-B, 2] fp32 or NULL (sampled)
 *   workspace     at least spec_workspace_bytes(B, K_max, V) bytes
 *   rows, n_rows, seeds, temperature, stream: as in the dense calls.
 * Each sequence is verified exactly as a dense sequence with K = K_b in batch
 * slot b (so the Philox counter is (i, b, 0, 0)); a batch where every K_b = K
 * gives the dense calls' results bit for bit.  Host checks: row_start non-NULL
 * and aligned, B <= total_rows <= B*(K_max+1).  The device checks each
 * selected sequence's own entries (0 <= K_b <= K_max, row_start[b] >= b, and
 * row_start[b+1] leaving room for the later sequences' rows); a sequence that
 * fails them gets accepted_len[b] = -1 and none of its rows is read or
 * written.  Other data faults are marked as in the dense calls.
 */
spec_status_t spec_accept_greedy_ragged(const float* logits, const int32_t* draft_tokens,
                                        const int32_t* row_start, int total_rows,
                                        const int32_t* rows, int n_rows, int B, int K_max, int V,
                                        int32_t* accepted_len, int32_t* out_tokens,
                                        void* workspace, size_t workspace_bytes,
                                        spec_stream_t stream);

spec_status_t spec_accept_sample_ragged(const float* logits, const float* draft_logits,
                                        const int32_t* draft_tokens,
                                        const int32_t* row_start, int total_rows,
                                        float temperature, const uint64_t* seeds,
                                        const int32_t* rows, int n_rows, int B, int K_max, int V,
                                        int32_t* accepted_len, int32_t* out_tokens,
                                        float* probs_at_draft,
                                        void* workspace, size_t workspace_bytes,
                                        spec_stream_t stream);

/*
 * spec_tree_accept_greedy -- greedy verification of draft trees.
 *
 * Each sequence carries a tree of N draft nodes (0 <= N <= 63) in
 * topological order: node 0 is the root (the last accepted token), node
 * v >= 1 holds token d_v and has parent p_v with 0 <= p_v < v.  Row v of the
 * sequence's logits is the target's prediction after the path root -> v (the
 * verify pass runs every node under a mask that lets it see only its
 * ancestors; spec_verify_logits with K = N computes the rows from the hidden
 * states of such a pass).  With a_u = argmax_v logits[b, u, v] (lowest index
 * on ties): node v is accepted iff its parent is and d_v == a_{p_v}; the root
 * is.  The kept node k is the deepest accepted node, the lowest index among
 * equally deep ones; n = its depth.  Then accepted_len[b] = n, out_tokens[b,
 * :] = (the tokens on the path root -> k, a_k, -1, ...) and out_nodes[b, :] =
 * (the node indices on that path, -1, ...): the caller keeps the cache
 * entries of exactly those nodes.  A chain (p_v = v - 1) is the linear
 * greedy rule of spec_accept_greedy.
 *
 *   logits        device, [B, N+1, V] fp32, 16-byte aligned
 *   parents       device, [B, N+1] int32 (entry 0 ignored; NULL when N == 0)
 *   tokens        device, [B, N+1] int32 (entry 0 ignored; NULL when N == 0)
 *   rows, n_rows  as in spec_accept_greedy
 *   accepted_len  device, [B] int32
 *   out_tokens    device, [B, N+1] int32
 *   out_nodes     device, [B, N+1] int32, or NULL
 *   workspace     at least spec_workspace_bytes(B, N, V) bytes
 * Data faults (a parent outside [0, v), a token outside [0, V), a NaN or
 * +inf logit or a row with no finite entry anywhere in the tree) give
 * accepted_len[b] = -1 and rows of -1.
 */
spec_status_t spec_tree_accept_greedy(const float* logits, const int32_t* parents,
                                      const int32_t* tokens, const int32_t* rows, int n_rows,
                                      int B, int N, int V,
                                      int32_t* accepted_len, int32_t* out_tokens,
                                      int32_t* out_nodes,
                                      void* workspace, size_t workspace_bytes,
                                      spec_stream_t stream);

/*
 * spec_tree_verify_step -- LM head and greedy tree verification in one call.
 *
 * Same results as spec_verify_logits (K = N) followed by
 * spec_tree_accept_greedy: identical logits, accepted lengths, tokens and
 * nodes (the rule needs each row's argmax only, which does not depend on the
 * order of any sum).  Where a bf16 LM-head kernel computes statistics on the
 * side (as in spec_verify_step: M = B*(N+1) <= 16 with H <= 8192, or M > 16
 * with H % 64 == 0) the rows' argmaxes come from its records and the logits
 * are not read back; otherwise the call enqueues the two calls' kernels.
 *
 *   hidden, w_lmhead, dtype, logits, B, V, H: as in spec_verify_logits, with
 *                 K = N (hidden [B, N+1, H], logits [B, N+1, V])
 *   parents, tokens, rows, n_rows, accepted_len, out_tokens, out_nodes:
 *                 as in spec_tree_accept_greedy (0 <= N <= 63)
 *   workspace     at least spec_verify_step_workspace_bytes(B, N, V) bytes,
 *                 16-byte aligned; contents on entry do not matter
 * Errors as in the two calls it replaces.
 */
spec_status_t spec_tree_verify_step(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                    const int32_t* parents, const int32_t* tokens,
                                    const int32_t* rows, int n_rows, int B, int N, int V, int H,
                                    float* logits, int32_t* accepted_len, int32_t* out_tokens,
                                    int32_t* out_nodes,
                                    void* workspace, size_t workspace_bytes,
                                    spec_stream_t stream);

/*
 * spec_verify_step -- the whole verify step in one call.
 *
 * Same results as spec_verify_logits followed by spec_accept_greedy over
 * greedy_rows and spec_accept_sample over sampled_rows, up to the rounding
 * order of the softmax sums (so a sampled decision with a margin below about
 * 1e-6 may differ; greedy decisions and the logits are identical).  The
 * logits are written once and not read back for statistics where a bf16
 * LM-head kernel computes them itself:
 *   - M = B*(K+1) <= 16, H <= 8192 (the cooperative kernel): each workgroup
 *     keeps the logits of its vocabulary range in LDS and writes one record
 *     per target row, plus one per draft row from the draft logits it loads
 *     while the weights stream; the accept kernels merge these records;
 *   - M > 16, H % 64 == 0 (the direct-to-LDS kernel): the target rows'
 *     statistics come from the kernel's epilogue while the logits are in
 *     registers, the draft rows' from a pass before the LM head, and the
 *     epilogue's records are folded into that pass's layout.
 * Otherwise (other hidden sizes, fp32) the call enqueues exactly the kernels
 * of the three separate calls.
 *
 *   hidden, w_lmhead, dtype, logits, B, K, V, H: as in spec_verify_logits
 *   draft_logits, draft_tokens, temperature, seeds, probs_at_draft,
 *   accepted_len, out_tokens: as in spec_accept_sample (draft_logits, seeds and
 *                 temperature are needed only when sampled rows exist)
 *   greedy_rows, n_greedy / sampled_rows, n_sampled
 *                 the sequences verified by each rule: a device list of
 *                 distinct entries (as `rows` in the accept calls), or NULL
 *                 with n = 0 (none) or n = B (all)
 *   workspace     at least spec_verify_step_workspace_bytes(B, K, V) bytes,
 *                 16-byte aligned; contents on entry do not matter
 * Errors as in the three calls it replaces.
 */
spec_status_t spec_verify_step(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                               const float* draft_logits, const int32_t* draft_tokens,
                               float temperature, const uint64_t* seeds,
                               const int32_t* greedy_rows, int n_greedy,
                               const int32_t* sampled_rows, int n_sampled,
                               int B, int K, int V, int H,
                               float* logits, int32_t* accepted_len, int32_t* out_tokens,
                               float* probs_at_draft,
                               void* workspace, size_t workspace_bytes,
                               spec_stream_t stream);

/* Bytes of workspace spec_verify_step needs (0 if the sizes are out of range). */
size_t spec_verify_step_workspace_bytes(int B, int K, int V);

/*
 * spec_verify_step_ragged -- the whole verify step for a ragged batch (each
 * sequence its own draft count K_b, rows packed; the ragged calls above
 * define the layout and cite where the pages vary the draft count).
 *
 * Same results as spec_verify_logits over the R = total_rows packed hidden
 * rows (B = R, K = 0) followed by spec_accept_greedy_ragged over greedy_rows
 * and spec_accept_sample_ragged over sampled_rows, with the same caveat on
 * sampled decisions within about 1e-6 of a boundary as spec_verify_step.
 * The LM-head kernel that runs for M = R rows computes the statistics as in
 * spec_verify_step (cooperative kernel for R <= 16, epilogue records for
 * R > 16 with H % 64 == 0); elsewhere the call enqueues the separate calls'
 * kernels.
 *
 *   hidden        device, [R, H] in dtype, 16-byte aligned (rows packed as
 *                 the logits)
 *   w_lmhead, dtype, V, H: as in spec_verify_logits
 *   logits        device, [R, V] fp32, 16-byte aligned (written)
 *   row_start, total_rows, K_max, draft_logits, draft_tokens, accepted_len,
 *   out_tokens, probs_at_draft, temperature, seeds: as in the ragged accept
 *                 calls
 *   greedy_rows, n_greedy / sampled_rows, n_sampled: as in spec_verify_step
 *   workspace     at least spec_verify_step_ragged_workspace_bytes(B, K_max,
 *                 V) bytes, 16-byte aligned; contents on entry do not matter
 * Errors as in the calls it replaces (host checks of row_start and
 * total_rows as in the ragged accept calls; a sequence whose row_start
 * entries fail the device checks gets accepted_len[b] = -1).
 */
spec_status_t spec_verify_step_ragged(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                      const float* draft_logits, const int32_t* draft_tokens,
                                      const int32_t* row_start, int total_rows,
                                      float temperature, const uint64_t* seeds,
                                      const int32_t* greedy_rows, int n_greedy,
                                      const int32_t* sampled_rows, int n_sampled,
                                      int B, int K_max, int V, int H,
                                      float* logits, int32_t* accepted_len, int32_t* out_tokens,
                                      float* probs_at_draft,
                                      void* workspace, size_t workspace_bytes,
                                      spec_stream_t stream);

/* Bytes of workspace spec_verify_step_ragged needs for any total_rows in
 * [B, B*(K_max+1)] (0 if the sizes are out of range). */
size_t spec_verify_step_ragged_workspace_bytes(int B, int K_max, int V);

/*
 * spec_verify_step_noalloc -- spec_verify_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, kernels and results as spec_verify_step, without the
 * workspace: the step's scratch is a 64 MiB array the library holds per GPU
 * (in its code object, for the life of the process), so every workload with
 * spec_verify_step_workspace_bytes(B, K, V) <= 67108864 fits (the largest
 * benchmark workload, B = 512, K = 3, V = 262144, needs 36 MiB).  Larger
 * sizes return SPEC_ERR_WORKSPACE before anything is enqueued, and
 * spec_last_error_detail() says why.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress, with the device
 * current); no call allocates or frees memory.
 *
 * Every call on one GPU uses that GPU's one array.  Calls ordered on one
 * stream are safe (each clears what its kernels count on, so what an earlier
 * call left there does not matter); calls that may overlap on one GPU (other
 * streams, other threads without ordering) race on it and must use
 * spec_verify_step with workspaces of their own.
 */
spec_status_t spec_verify_step_noalloc(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                       const float* draft_logits, const int32_t* draft_tokens,
                                       float temperature, const uint64_t* seeds,
                                       const int32_t* greedy_rows, int n_greedy,
                                       const int32_t* sampled_rows, int n_sampled,
                                       int B, int K, int V, int H,
                                       float* logits, int32_t* accepted_len, int32_t* out_tokens,
                                       float* probs_at_draft, spec_stream_t stream);

/*
 * spec_ngram_propose -- prompt-lookup drafts for B token histories.
 *
 * For history s of length L: for n = max_ngram, ..., 1, look for the window
 * s[j .. j+n-1] == s[L-n .. L-1] with the largest j <= L-1-n (a window ending
 * before the last token); the first n that has one fixes start = j + n and
 * the drafts s[start .. start + n_drafts - 1], cut at L.  No window for any n:
 * no drafts.  Only token equality is used, so the result is exact.
 *
 *   history       device, int32 tokens of all histories, packed
 *   history_len   number of int32 entries behind `history` (>= 0); no
 *                 kernel reads past it
 *   hist_start    device, [B+1] int64, 8-byte aligned: history b is
 *                 history[hist_start[b] .. hist_start[b+1]-1]
 *   B             number of histories, >= 1
 *   max_len       bound on every history's length (0 <= max_len < 2^31 - 1);
 *                 it sizes the launch
 *   max_ngram     longest n-gram tried, 1 ..16 (the page's listing uses 3)
 *   n_drafts      drafts wanted per history, 0 .. 63
 *   drafts        device, [B, n_drafts] int32: the drafts, then -1
 *   draft_count   device, [B] int32: drafts proposed (0 .. n_drafts)
 *   row_start     device, [B+1] int32, or NULL: row_start[0] = 0,
 *                 row_start[b+1] = row_start[b] + draft_count[b] + 1 -- the
 *                 packing the ragged verify calls take (a history with bad
 *                 offsets counts as 0 drafts there)
 *   workspace     device scratch of spec_ngram_workspace_bytes(B, max_len)
 *                 bytes, 8-byte aligned; contents on entry do not matter
 * A history whose offsets are malformed (negative start, negative length, a
 * length above max_len, or an end past history_len) gets draft_count[b] = -1
 * and drafts of -1, and is not read.
 */
spec_status_t spec_ngram_propose(const int32_t* history, int64_t history_len, const int64_t* hist_start, int B,
                                 int max_len, int max_ngram, int n_drafts,
                                 int32_t* drafts, int32_t* draft_count, int32_t* row_start,
                                 void* workspace, size_t workspace_bytes,
                                 spec_stream_t stream);

/* Bytes of workspace spec_ngram_propose needs for B histories of at most
 * max_len tokens (one 8-byte slot per 4096-position segment; 0 if B < 1 or
 * max_len is out of range). */
size_t spec_ngram_workspace_bytes(int B, int max_len);

/* Bytes of workspace any accept call needs for these sizes (K = K_max for the
 * ragged calls; 0 if the sizes are out of range). */
size_t spec_workspace_bytes(int B, int K, int V);

/* Bound on the one kind of cross-workgroup wait in this library.  In the
 * residual / bonus draw of sampled sequences, launches of at most 256
 * workgroups (all resident at once: the one-launch acceptance + residual draw
 * of small batches, and the draw of moderate batches that follows a separate
 * acceptance launch) publish each chunk's weight sum and then poll the other
 * sums of the sequence, up to `rounds` rounds (about a microsecond each),
 * before a workgroup gives up and sums every chunk itself.  The result does
 * not depend on the bound, only the time: giving up costs a read of the whole
 * terminal row per workgroup.  A negative value restores the default
 * (65536).  Process-wide; applies to launches enqueued after the call.
 * Returns the previous bound.  Meant for tests of the give-up path. */
int spec_set_poll_limit(int rounds);

/* Static, human-readable name of a status code. */
const char* spec_status_string(spec_status_t status);

/* Detail of the last SPEC_ERR_HIP returned on the calling thread (a static
 * string owned by the HIP runtime), or of spec_verify_step_noalloc's
 * SPEC_ERR_WORKSPACE (a static string of the library); "" if none. */
const char* spec_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
