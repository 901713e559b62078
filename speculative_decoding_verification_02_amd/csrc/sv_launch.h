// sv_launch.h -- host-side launchers of the verify-step kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_common.h"

namespace sv {

// LM-head contraction, the kernel picked by shape (cooperative for M <= 16
// and H <= 4096, small-M streaming for wider H, direct-to-LDS for M > 16
// with H % 64 == 0, LDS-tiled otherwise).  With stats non-null the
// direct-to-LDS kernel also writes its statistics epilogue's *n_rec records
// per row (one per 256 vocabulary entries), stats[m * *n_rec + k], in
// vocabulary order, with sums relative to c = log2(e) / T; *n_rec = 0 means
// the chosen kernel has no epilogue and the caller runs the statistics pass.
hipError_t launch_lmhead_bf16(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                              int num_cus, hipStream_t stream, StatRec* stats = nullptr, float c = 0.f,
                              int* n_rec = nullptr);
hipError_t launch_lmhead_f32(const float* hidden, const float* W, float* logits, int M, int V, int H,
                             hipStream_t stream);
// Statistics the cooperative LM-head kernel (M <= 16) computes on the side:
// per workgroup w of n_rec, the record of hidden row m over the workgroup's
// contiguous vocabulary range at tgt[m * n_rec + w], and likewise of draft
// row d (n_draft rows of V fp32 logits at draft) at drf[d * n_rec + w], sums
// relative to c = log2(e) / T; workgroup 0 also zeroes n_zero ints at zero.
struct CoopStats {
    StatRec* tgt;
    const float* draft;
    int n_draft;
    StatRec* drf;
    float c;
    int* zero;
    int n_zero;
};
constexpr int kCoopMaxRecs = 1024;   // records per row at most (workgroups of the cooperative kernel)
// Records per row the cooperative kernel writes for this shape with n_draft
// draft rows (its workgroup count), else 0 (it does not run for this shape,
// or the rows' logits would not fit its LDS).
int lmhead_coop_records(int M, int V, int H, int n_draft, int num_cus);
hipError_t launch_lmhead_coop_stats(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                                    int num_cus, hipStream_t stream, const CoopStats& st);
// Fold rows x recs_per_row epilogue records (one per 256 vocabulary entries,
// row r at in + r * recs_per_row) into rows x n_chunks(V) chunk records, the
// layout the statistics pass writes; sums relative to inv_t_log2e.
hipError_t launch_fold_records(const StatRec* in, int recs_per_row, int rows, int V, float inv_t_log2e, StatRec* out,
                               hipStream_t stream);
// Records per row the direct-to-LDS kernel's statistics epilogue writes (one
// per 256 vocabulary entries) when launch_lmhead_bf16 picks it for this
// shape, else 0.
int lmhead_big_records(int M, int V, int H);

// Softmax statistics of the rows the accept step needs, per chunk.
//   jobs = (if logits) n_rows*(K+1) target slots, then (if draft_logits)
//   n_rows*K draft slots, K = seq.K; slots past a ragged sequence's own rows
//   are skipped.
//   zero, n_zero (optional): ints zeroed on the way (the completion counters
//   and poll slots of a fused accept + residual launch that follows).
hipError_t launch_softmax_stats(const float* logits, const float* draft_logits, const int32_t* rows, int n_rows,
                                SeqRows seq, int V, float inv_t_log2e, bool need_sum, StatRec* stats,
                                hipStream_t stream, int* zero = nullptr, int n_zero = 0);

// Where the accept kernel finds the statistics records of a sequence's rows.
// Target rows: tgt + (tgt_by_row ? t0 + i : j*(K+1) + i) * tgt_nc (by packed
// row for the LM-head epilogue's records, by selection slot for the
// statistics pass).  Draft rows: drf + (drf_by_row ? t0 - b + i : j*K + i) *
// drf_nc.
struct RecLayout {
    const StatRec* tgt;
    int tgt_nc;
    bool tgt_by_row;
    const StatRec* drf;
    int drf_nc;
    bool drf_by_row;
};

// Rows per sequence (target plus draft) up to which the accept kernels merge
// records straight from memory, one 16-lane group per row, however many
// records a row has; longer sequences want the statistics pass's layout
// (4096-entry chunk records).
constexpr int kAcceptRowsDirect = 16;

// Greedy or sampled acceptance: one workgroup per selected sequence.  The
// sampled variant also zeroes the sequence's residual counter and, with
// slots, its slots_per_seq poll slots at slots[j * slots_per_seq].
hipError_t launch_accept(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                         const uint64_t* seeds, const int32_t* rows, int n_rows, SeqRows seq, int V,
                         float inv_t_log2e, bool sampled, RecLayout rec, int32_t* accepted_len,
                         int32_t* out_tokens, float* probs_at_draft, AcceptInfo* info, int* counters,
                         hipStream_t stream, unsigned long long* slots = nullptr, int slots_per_seq = 0);

// Greedy and sampled acceptance in one launch: workgroups 0 .. n_greedy-1
// take greedy_rows, the rest sampled_rows (AcceptInfo and residual counter
// of sampled slot j at info[j], counters[j]); each with its own layout.
hipError_t launch_accept_both(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                              const uint64_t* seeds, const int32_t* greedy_rows, int n_greedy,
                              const int32_t* sampled_rows, int n_sampled, SeqRows seq, int V, float inv_t_log2e,
                              RecLayout rec_greedy, RecLayout rec_sampled, int32_t* accepted_len,
                              int32_t* out_tokens, float* probs_at_draft, AcceptInfo* info, int* counters,
                              hipStream_t stream, unsigned long long* slots = nullptr, int slots_per_seq = 0);

// Acceptance and residual draw of sampled sequences in one launch (small
// batches); needs its counters and slots zeroed by the kernel before it
// (launch_softmax_stats or the cooperative LM head, over accept_zero_ints
// ints from the counters).  Used while sequences x (2K+1) rows stay within
// this bound (measured: 17 vs 20 us at one sequence with K = 5; 45 vs 35 us at
// 16 sequences with K = 15).
constexpr int kFusedAcceptMaxRows = 48;
// The one-launch accept + residual splits the terminal rows into chunks of
// kFusedPer entries per thread (1024 entries), a quarter of a statistics chunk.
constexpr int kFusedPer = 4;
inline int n_fused_chunks(int V) { return (V + kFusedPer * kStatThreads - 1) / (kFusedPer * kStatThreads); }
// Launches of at most this many workgroups publish their chunk sums in
// tagged 64-bit slots that every workgroup polls (all of them fit on the GPU
// at once); larger ones count the sums in and select in the last workgroup.
constexpr int kPollMaxBlocks = 256;
constexpr unsigned long long kPollTag = 1ull << 32;   // a written slot: tag | float bits of the sum
// Poll rounds a workgroup waits for its sequence's sums before it sums every
// chunk itself (the default of the library; tests may lower it).
constexpr int kDefaultPollLimit = 1 << 16;
// Ints from the counters to zero before a launch of n_rows sequences: the
// counters of up to B sequences (their 256-byte-aligned block), then the
// slots that directly follow them.
inline int accept_zero_ints(int B, int n_rows, int V) {
    const long nc = n_fused_chunks(V);
    const int counter_ints = (int)((((long)B * 4 + 255) / 256) * 64);
    return (long)n_rows * nc <= kPollMaxBlocks ? counter_ints + (int)(2 * n_rows * nc) : counter_ints;
}
hipError_t launch_accept_residual(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                                  const uint64_t* seeds, const int32_t* rows, int n_rows, SeqRows seq, int V,
                                  float inv_t_log2e, RecLayout rec, int32_t* accepted_len, int32_t* out_tokens,
                                  float* probs_at_draft, float* chunk_sums, int* counters,
                                  unsigned long long* slots, int spin_limit, hipStream_t stream);

// Greedy verification of draft trees (N+1 rows per sequence): recs_per_row
// records per row (0: the statistics pass's n_chunks(V)), rows by selection
// slot (the pass over the dense layout with K = N) or, by_row, by sequence
// (the LM head's records, folded or per workgroup).
hipError_t launch_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* rows, int n_rows, int B,
                              int N, int V, const StatRec* stats, int32_t* accepted_len, int32_t* out_tokens,
                              int32_t* out_nodes, hipStream_t stream, int recs_per_row = 0, bool by_row = false);

// Residual / bonus draw of the sampled sequences: per-chunk weight sums, and
// the inverse-CDF selection of the terminal token.  Launches of at most
// kPollMaxBlocks workgroups (residual_poll_group chunks each) poll tagged
// slots, one per (sequence, chunk), which the accept kernel zeroes first
// (launch_accept / launch_accept_both with slots_per_seq = n_chunks(V));
// larger ones count the chunk blocks in and select in the last one.
constexpr int kPollMaxSlots = 2048;       // tagged slots in the workspace
constexpr int kResidualMaxGroup = 4;      // chunks per workgroup of the polled draw at most (1, 2 or 4)
int residual_poll_group(int n_rows, int V);
hipError_t launch_residual(const float* logits, const float* draft_logits, int n_rows, int V,
                           float inv_t_log2e, const AcceptInfo* info, float* chunk_sums, int* counters,
                           unsigned long long* slots, int spin_limit, int32_t* out_tokens, hipStream_t stream);

// Prompt-lookup drafter: per-sequence best (match length, end position) keys
// (B x 8 bytes of scratch), then drafts, counts and verify-row offsets.  A
// span reaching past hist_len entries of hist is malformed and never read.
constexpr int kNgMaxGram = 16;                     // longest n-gram tried
constexpr int kNgMaxDrafts = 63;                   // drafts per history at most
constexpr int kNgSeg = 4096;                       // end positions per scan workgroup
inline int ngram_segments(int max_len) { return max_len >= 2 ? (max_len - 2) / kNgSeg + 1 : 0; }
hipError_t launch_ngram(const int32_t* hist, int64_t hist_len, const int64_t* hist_start, int B, int max_len, int G,
                        int n_drafts,
                        int32_t* drafts, int32_t* count, int32_t* row_start, unsigned long long* keys,
                        hipStream_t stream);

}  // namespace sv
