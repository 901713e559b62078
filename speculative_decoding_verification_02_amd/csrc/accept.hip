// accept.hip -- greedy and sampled acceptance of the verify step.
//
// One workgroup per selected sequence.  The chunk statistics of the
// sequence's rows are staged in LDS with every load in flight at once and
// merged row by row, one wavefront per row; then wavefront 0, lane i = verify
// position i (i <= kb <= 63, kb = the sequence's draft count: K in a dense
// batch, its own K_b in a ragged one), decides whether draft i would be
// accepted on its own, and one ballot finds the first rejection:
//   greedy  ("Inference-4", greedy bullet): ok_i = [d_i == argmax_v z_t[i, v]]
//   sampled (same page, sampling bullet; "speculative-decoding" blog,
//            Rejection sampling): ok_i = [u_i < min(1, q_i(d_i) / p_i(d_i))]
// n = index of the first lane i < kb with !ok_i, else kb.  Drafts before n
// are committed; greedy rows commit argmax z_t[n] at n (the target's token at
// the mismatch, or the bonus token when n = kb), sampled rows leave position
// n to the residual kernels, which draw it from norm(max(0, q_n - p_n)) or
// q_kb.
//
// The ratio is evaluated in log2 space so tiny probabilities do not underflow:
//   r = min(1, exp2(lq - lp) * S_d / S_t),  lq = (z_t[d] - M_t) * c, lp = (z_d[d] - M_d) * c
// with r = 0 when z_t[d] = -inf (the target rules d out) and r = 1 when
// z_d[d] = -inf < z_t[d].
#include <limits.h>

#include "sv_accept.h"

namespace sv {

template <bool SAMPLED>
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, const int32_t* __restrict__ draft_tokens,
    const uint64_t* __restrict__ seeds, const int32_t* __restrict__ rows, int n_rows, SeqRows seq, int V,
    float c, RecLayout rec, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probs_at_draft, AcceptInfo* __restrict__ info, int* __restrict__ counters,
    unsigned long long* __restrict__ slots, int spq) {
    __shared__ StatRec recs[kRecBuf];
    __shared__ Merged merged[kMaxRows];
    __shared__ AcceptInfo sinfo;
    const int j = blockIdx.x;
    const int b = rows ? rows[j] : j;
    if (SAMPLED && threadIdx.x == 0) counters[j] = 0;   // the residual kernel counts its chunk blocks from zero
    if (SAMPLED && (int)threadIdx.x < spq) slots[(size_t)j * spq + threadIdx.x] = 0ull;   // or polls these
    const AcceptInfo a = accept_sequence<SAMPLED>(logits, draft_logits, draft_tokens, seeds, j, b, seq, V, c, rec,
                                                  true, accepted_len, out_tokens, probs_at_draft, recs, merged,
                                                  &sinfo);
    if (SAMPLED && threadIdx.x == 0) info[j] = a;
}

// Both rules in one launch: workgroup j < n_greedy decides greedy_rows[j],
// the others sampled_rows[j - n_greedy] (their AcceptInfo and residual
// counter in slot j - n_greedy), each exactly as accept_kernel does.
__global__ __launch_bounds__(kAcceptThreads) void accept_both_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, const int32_t* __restrict__ draft_tokens,
    const uint64_t* __restrict__ seeds, const int32_t* __restrict__ greedy_rows, int n_greedy,
    const int32_t* __restrict__ sampled_rows, SeqRows seq, int V, float c, RecLayout rec_greedy,
    RecLayout rec_sampled, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probs_at_draft, AcceptInfo* __restrict__ info, int* __restrict__ counters,
    unsigned long long* __restrict__ slots, int spq) {
    __shared__ StatRec recs[kRecBuf];
    __shared__ Merged merged[kMaxRows];
    __shared__ AcceptInfo sinfo;
    const int j = blockIdx.x;
    if (j < n_greedy) {
        const int b = greedy_rows ? greedy_rows[j] : j;
        accept_sequence<false>(logits, nullptr, draft_tokens, nullptr, j, b, seq, V, kLog2e, rec_greedy, true,
                               accepted_len, out_tokens, nullptr, recs, merged, &sinfo);
        return;
    }
    const int js = j - n_greedy;
    const int b = sampled_rows ? sampled_rows[js] : js;
    if (threadIdx.x == 0) counters[js] = 0;   // the residual kernel counts its chunk blocks from zero
    if ((int)threadIdx.x < spq) slots[(size_t)js * spq + threadIdx.x] = 0ull;   // or polls these
    const AcceptInfo a = accept_sequence<true>(logits, draft_logits, draft_tokens, seeds, js, b, seq, V, c,
                                               rec_sampled, true, accepted_len, out_tokens, probs_at_draft, recs,
                                               merged, &sinfo);
    if (threadIdx.x == 0) info[js] = a;
}

// ----------------------------------------------------------- draft trees --
// Greedy verification of a draft tree of N <= 63 nodes per sequence
// ("Inference-4", Medusa; "speculative-decoding" blog, EAGLE-2's dynamic
// draft trees; "Speculative decoding" course page, One pass, many candidate
// continuations).  Row v of the sequence's logits is the target's prediction
// after the path root -> v; node v >= 1 extends its parent p(v) < v by token
// d_v.  Node v is accepted iff its parent is and d_v == argmax of row p(v);
// the deepest accepted node (lowest index among equals) is kept: its path's
// tokens are committed and the argmax of its own row is the bonus token.
//
// One workgroup per sequence merges the chunk statistics of its N+1 rows as
// the linear kernel does; then wavefront 0 holds node v in lane v and finds,
// by pointer jumping over the parent links (six rounds of shuffles reach any
// depth below 64), each node's depth and whether its whole path is accepted.
__global__ __launch_bounds__(kAcceptThreads) void tree_accept_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens, const int32_t* __restrict__ rows,
    int n_rows, int B, int N, int V, int nc, const StatRec* __restrict__ stats, bool by_row,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nodes) {
    __shared__ StatRec recs[kRecBuf];
    __shared__ Merged merged[kWave];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = blockIdx.x;
    const int b = rows ? rows[j] : j;
    if (b < 0 || b >= B) return;

    const int v = lane;
    const bool node = wave == 0 && v <= N;
    const size_t base = (size_t)b * (N + 1);
    int par = 0, tok = 0;
    if (node && v > 0) {
        par = parents[base + v];
        tok = tokens[base + v];
    }

    const int rows_per_pass = max(1, min(N + 1, kRecBuf / nc));
    for (int r0 = 0; r0 <= N; r0 += rows_per_pass) {
        const int nr = min(rows_per_pass, N + 1 - r0);
        // rows r0 .. r0+nr-1 of the sequence, contiguous: nc records per row,
        // rows by selection slot j (the statistics pass) or by sequence b
        const StatRec* src = stats + ((size_t)(by_row ? b : j) * (N + 1) + r0) * nc;
        stage_records(recs, nr * nc, tid, [&](int e) { return src + e; });
        __syncthreads();
        // one row per 16-lane DPP row: four rows per wavefront at a time
        // (the argmax does not depend on the order records are combined in)
        const int gl = lane & 15;
        for (int base = wave * 4; base < nr; base += kAcceptWaves * 4) {
            const int rr = base + (lane >> 4);
            if (rr < nr) {
                const Merged x = row16_merge(recs + rr * nc, nc, 0.f, false, gl);
                if (gl == 0) merged[r0 + rr] = x;
            }
        }
        __syncthreads();
    }
    if (wave != 0) return;

    Merged t{-INFINITY, 0.f, INT_MAX, 0};
    int bad = 0;
    if (node) {
        t = merged[v];
        bad = t.bad | (t.m == -INFINITY);
        if (v > 0) bad |= par < 0 || par >= v || tok < 0 || tok >= V;
    }
    int32_t* orow = out_tokens + base;
    int32_t* nrow = out_nodes ? out_nodes + base : nullptr;
    if (__ballot(node && bad) != 0ull) {  // data fault anywhere in the tree
        if (node) {
            orow[v] = -1;
            if (nrow) nrow[v] = -1;
        }
        if (lane == 0) accepted_len[b] = -1;
        return;
    }

    // lanes past N stand for nothing: parked at the root, never accepted
    const int p0 = (node && v > 0) ? par : 0;
    const int arg_parent = __shfl(t.idx, p0, kWave);
    int ok = node && (v == 0 || tok == arg_parent);
    int anc = p0;
    int dist = (node && v > 0) ? 1 : 0;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const int ok_a = __shfl(ok, anc, kWave);
        const int dist_a = __shfl(dist, anc, kWave);
        const int anc_a = __shfl(anc, anc, kWave);
        ok &= ok_a;
        dist += dist_a;
        anc = anc_a;
    }
    // deepest accepted node, lowest index among equals (the root always qualifies)
    int key = ok ? (dist << 6) | (63 - v) : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, kWave));
    const int best = 63 - (key & 63);
    const int depth = key >> 6;

    // commit the path: walk from the kept node up to the root
    int cur = best;
    for (int s = depth - 1; s >= 0; --s) {
        const int tv = __shfl(tok, cur, kWave);
        if (lane == 0) {
            orow[s] = tv;
            if (nrow) nrow[s] = cur;
        }
        cur = __shfl(p0, cur, kWave);
    }
    const int bonus = __shfl(t.idx, best, kWave);
    if (node) {
        if (v == depth) orow[v] = bonus;
        else if (v > depth) orow[v] = -1;
        if (nrow && v >= depth) nrow[v] = -1;
    }
    if (lane == 0) accepted_len[b] = depth;
}

hipError_t launch_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* rows, int n_rows, int B,
                              int N, int V, const StatRec* stats, int32_t* accepted_len, int32_t* out_tokens,
                              int32_t* out_nodes, hipStream_t stream, int recs_per_row, bool by_row) {
    if (recs_per_row > kRecBuf) return hipErrorInvalidValue;
    if (n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(tree_accept_kernel, dim3(n_rows), dim3(kAcceptThreads), 0, stream, parents, tokens, rows,
                       n_rows, B, N, V, recs_per_row > 0 ? recs_per_row : n_chunks(V), stats, by_row, accepted_len,
                       out_tokens, out_nodes);
    return hipGetLastError();
}

hipError_t launch_accept(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                         const uint64_t* seeds, const int32_t* rows, int n_rows, SeqRows seq, int V,
                         float inv_t_log2e, bool sampled, RecLayout rec, int32_t* accepted_len,
                         int32_t* out_tokens, float* probs_at_draft, AcceptInfo* info, int* counters,
                         hipStream_t stream, unsigned long long* slots, int slots_per_seq) {
    if (n_rows == 0) return hipSuccess;
    if (!slots || slots_per_seq > kAcceptThreads) slots_per_seq = 0;
    if (sampled)
        hipLaunchKernelGGL(accept_kernel<true>, dim3(n_rows), dim3(kAcceptThreads), 0, stream, logits, draft_logits,
                           draft_tokens, seeds, rows, n_rows, seq, V, inv_t_log2e, rec, accepted_len,
                           out_tokens, probs_at_draft, info, counters, slots, slots_per_seq);
    else
        hipLaunchKernelGGL(accept_kernel<false>, dim3(n_rows), dim3(kAcceptThreads), 0, stream, logits, draft_logits,
                           draft_tokens, seeds, rows, n_rows, seq, V, inv_t_log2e, rec, accepted_len,
                           out_tokens, probs_at_draft, info, counters, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_accept_both(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                              const uint64_t* seeds, const int32_t* greedy_rows, int n_greedy,
                              const int32_t* sampled_rows, int n_sampled, SeqRows seq, int V, float inv_t_log2e,
                              RecLayout rec_greedy, RecLayout rec_sampled, int32_t* accepted_len,
                              int32_t* out_tokens, float* probs_at_draft, AcceptInfo* info, int* counters,
                              hipStream_t stream, unsigned long long* slots, int slots_per_seq) {
    if (n_greedy + n_sampled == 0) return hipSuccess;
    if (!slots || slots_per_seq > kAcceptThreads) slots_per_seq = 0;
    hipLaunchKernelGGL(accept_both_kernel, dim3(n_greedy + n_sampled), dim3(kAcceptThreads), 0, stream, logits,
                       draft_logits, draft_tokens, seeds, greedy_rows, n_greedy, sampled_rows, seq, V, inv_t_log2e,
                       rec_greedy, rec_sampled, accepted_len, out_tokens, probs_at_draft, info, counters, slots,
                       slots_per_seq);
    return hipGetLastError();
}

}  // namespace sv
