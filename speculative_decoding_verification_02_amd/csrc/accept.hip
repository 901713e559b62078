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

#include "sv_common.h"
#include "sv_launch.h"

namespace sv {

constexpr int kAcceptThreads = 256;          // one workgroup per sequence
constexpr int kAcceptWaves = kAcceptThreads / kWave;
constexpr int kRecBuf = 2048;                // chunk records staged in LDS per pass (32 KB)
constexpr int kMaxRows = 2 * 63 + 1;         // target rows 0..K plus draft rows 0..K-1

struct Merged {
    float m;
    float s;
    int idx;
    int bad;
};

// Merge the chunk records of one row across a wavefront (records in LDS):
//   M = max m_c (lowest index on ties), S = sum s_c * exp2((m_c - M) * c).
__device__ __forceinline__ Merged wave_merge(const StatRec* rec, int nc, float c, bool need_sum, int lane) {
    float m = -INFINITY;
    int idx = INT_MAX;
    int bad = 0;
    for (int k = lane; k < nc; k += kWave) {
        const StatRec x = rec[k];
        argmax_combine(m, idx, x.m, x.idx);
        bad |= x.bad;
    }
    wave_argmax(m, idx);
    bad = __ballot(bad) != 0ull;
    float s = 0.f;
    if (need_sum && m != -INFINITY) {
        for (int k = lane; k < nc; k += kWave) {
            const StatRec x = rec[k];
            if (x.m != -INFINITY) s += x.s * exp2f((x.m - m) * c);
        }
        s = wave_sum(s);
    }
    return Merged{m, s, idx, bad};
}

// Merge the records of n consecutive rows (nc records each, row r at
// base + r*nc) into merged[out0 + r], one wavefront per row.  Rows are staged
// through LDS with every load in flight at once when they fit; rows longer
// than the buffer are merged straight from global memory.  Called by the
// whole workgroup.
__device__ void merge_rows(const StatRec* __restrict__ base, int n, int nc, float c, bool need_sum, StatRec* recs,
                           Merged* merged, int out0) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (nc > kRecBuf) {
        for (int rr = wave; rr < n; rr += kAcceptWaves) {
            const Merged x = wave_merge(base + (size_t)rr * nc, nc, c, need_sum, lane);
            if (lane == 0) merged[out0 + rr] = x;
        }
        __syncthreads();
        return;
    }
    const int rows_per_pass = max(1, min(n, kRecBuf / nc));
    for (int r0 = 0; r0 < n; r0 += rows_per_pass) {
        const int nr = min(rows_per_pass, n - r0);
        const StatRec* src = base + (size_t)r0 * nc;
        for (int e = tid; e < nr * nc; e += kAcceptThreads) recs[e] = src[e];
        __syncthreads();
        for (int rr = wave; rr < nr; rr += kAcceptWaves) {
            const Merged x = wave_merge(recs + rr * nc, nc, c, need_sum, lane);
            if (lane == 0) merged[out0 + r0 + rr] = x;
        }
        __syncthreads();
    }
}

template <bool SAMPLED>
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, const int32_t* __restrict__ draft_tokens,
    const uint64_t* __restrict__ seeds, const int32_t* __restrict__ rows, int n_rows, SeqRows seq, int V,
    float c, RecLayout rec, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probs_at_draft, AcceptInfo* __restrict__ info, int* __restrict__ counters) {
    __shared__ StatRec recs[kRecBuf];
    __shared__ Merged merged[kMaxRows];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = seq.K;
    const int j = blockIdx.x;
    const int b = rows ? rows[j] : j;
    if (SAMPLED && tid == 0) counters[j] = 0;   // the residual kernel counts its chunk blocks from zero
    if (b < 0 || b >= seq.B) {
        if (SAMPLED && tid == 0) info[j] = AcceptInfo{-1, b, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f, {0, 0, 0}};
        return;
    }
    int t0 = 0, kb = 0;
    if (!seq.get(b, t0, kb)) {   // malformed row_start: no row of this sequence is touched
        if (tid == 0) {
            accepted_len[b] = -1;
            if (SAMPLED) info[j] = AcceptInfo{-1, b, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f, {0, 0, 0}};
        }
        return;
    }
    const size_t d0 = (size_t)(t0 - b);   // first draft row / token of the sequence

    // wavefront 0, lane i: the draft token and (sampled) its two logits, loaded
    // up front so the loads overlap the statistics merge
    const int i = lane;
    const bool active = wave == 0 && i <= kb;
    const bool has_draft = wave == 0 && i < kb;
    int tok = 0;
    float zt_tok = 0.f, zd_tok = 0.f;
    if (has_draft) {
        tok = draft_tokens[d0 + i];
        if (SAMPLED && tok >= 0 && tok < V) {
            zt_tok = logits[((size_t)t0 + i) * V + tok];
            zd_tok = draft_logits[(d0 + i) * V + tok];
        }
    }

    // merged statistics of the target rows 0..kb, then (sampled) the draft
    // rows 0..kb-1 (merged[kb+1+i])
    const StatRec* tgt0 = rec.tgt + (size_t)(rec.tgt_by_row ? t0 : j * (K + 1)) * rec.tgt_nc;
    merge_rows(tgt0, kb + 1, rec.tgt_nc, c, SAMPLED, recs, merged, 0);
    if (SAMPLED && kb > 0) merge_rows(rec.drf + (size_t)j * K * rec.drf_nc, kb, rec.drf_nc, c, true, recs, merged, kb + 1);
    if (wave != 0) return;

    Merged t{-INFINITY, 0.f, INT_MAX, 0}, d{-INFINITY, 0.f, INT_MAX, 0};
    int bad = 0;
    if (active) {
        t = merged[i];
        bad = t.bad | (t.m == -INFINITY);
    }
    if (has_draft) {
        bad |= (tok < 0 || tok >= V);
        if (SAMPLED) {
            d = merged[kb + 1 + i];
            bad |= d.bad | (d.m == -INFINITY);
        }
    }
    int32_t* orow = out_tokens + t0;
    if (__ballot(active && bad) != 0ull) {  // data fault anywhere in the sequence
        if (active) orow[i] = -1;
        if (lane == 0) {
            accepted_len[b] = -1;
            if (SAMPLED) info[j] = AcceptInfo{-1, b, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f, {0, 0, 0}};
        }
        return;
    }

    bool ok = false;
    float u_term = 0.f;
    if (SAMPLED) {
        if (active) {
            const uint64_t seed = seeds[b];
            const uint4 w = philox4x32_10(make_uint4((uint32_t)i, (uint32_t)b, 0u, 0u), (uint32_t)seed,
                                          (uint32_t)(seed >> 32));
            u_term = uniform24(w.y);
            if (has_draft) {
                const float zt = zt_tok, zd = zd_tok;
                const float lq = (zt - t.m) * c;
                const float lp = (zd - d.m) * c;
                float r;
                if (zt == -INFINITY)
                    r = 0.f;
                else if (zd == -INFINITY)
                    r = 1.f;
                else
                    r = fminf(1.f, exp2f(lq - lp) * (d.s / t.s));
                ok = uniform24(w.x) < r;
                if (probs_at_draft) {
                    float* pp = probs_at_draft + (d0 + i) * 2;
                    pp[0] = exp2f(lq) / t.s;
                    pp[1] = exp2f(lp) / d.s;
                }
            }
        }
    } else {
        ok = has_draft && tok == t.idx;
    }

    const unsigned long long rej = __ballot(has_draft && !ok);
    const int n = rej ? (__ffsll((long long)rej) - 1) : kb;
    if (active) {
        if (i < n)
            orow[i] = tok;
        else if (i > n)
            orow[i] = -1;
        else
            orow[i] = SAMPLED ? -1 : t.idx;  // sampled: filled in by the residual draw
    }
    if (lane == 0) accepted_len[b] = n;
    if (SAMPLED && i == n)
        info[j] = AcceptInfo{n, b, t0, kb, u_term, t.m, t.s, has_draft ? d.m : 0.f, has_draft ? d.s : 0.f, {0, 0, 0}};
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
    int n_rows, int B, int N, int V, int nc, const StatRec* __restrict__ stats, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nodes) {
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
        for (int e = tid; e < nr * nc; e += kAcceptThreads) {
            const int rr = r0 + e / nc, k = e - (e / nc) * nc;
            recs[e] = stats[((size_t)j * (N + 1) + rr) * nc + k];
        }
        __syncthreads();
        for (int rr = wave; rr < nr; rr += kAcceptWaves) {
            const Merged x = wave_merge(recs + rr * nc, nc, 0.f, false, lane);
            if (lane == 0) merged[r0 + rr] = x;
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
                              int32_t* out_nodes, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(tree_accept_kernel, dim3(n_rows), dim3(kAcceptThreads), 0, stream, parents, tokens, rows,
                       n_rows, B, N, V, n_chunks(V), stats, accepted_len, out_tokens, out_nodes);
    return hipGetLastError();
}

hipError_t launch_accept(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                         const uint64_t* seeds, const int32_t* rows, int n_rows, SeqRows seq, int V,
                         float inv_t_log2e, bool sampled, RecLayout rec, int32_t* accepted_len,
                         int32_t* out_tokens, float* probs_at_draft, AcceptInfo* info, int* counters,
                         hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    if (sampled)
        hipLaunchKernelGGL(accept_kernel<true>, dim3(n_rows), dim3(kAcceptThreads), 0, stream, logits, draft_logits,
                           draft_tokens, seeds, rows, n_rows, seq, V, inv_t_log2e, rec, accepted_len,
                           out_tokens, probs_at_draft, info, counters);
    else
        hipLaunchKernelGGL(accept_kernel<false>, dim3(n_rows), dim3(kAcceptThreads), 0, stream, logits, draft_logits,
                           draft_tokens, seeds, rows, n_rows, seq, V, inv_t_log2e, rec, accepted_len,
                           out_tokens, probs_at_draft, info, counters);
    return hipGetLastError();
}

}  // namespace sv
