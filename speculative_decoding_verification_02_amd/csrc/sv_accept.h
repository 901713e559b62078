// sv_accept.h -- the acceptance decision of one sequence, shared by the
// accept kernel and the fused accept + residual kernel (internal).
//
// Greedy ("Inference-4", greedy bullet): ok_i = [d_i == argmax_v z_t[i, v]].
// Sampled (same page, sampling bullet; "speculative-decoding" blog, Rejection
// sampling): ok_i = [u_i < min(1, q_i(d_i) / p_i(d_i))].  n = the first
// position i < kb with !ok_i, else kb.  The ratio is evaluated in log2 space
// so tiny probabilities do not underflow:
//   r = min(1, exp2(lq - lp) * S_d / S_t),  lq = (z_t[d] - M_t) * c, lp = (z_d[d] - M_d) * c
// with r = 0 when z_t[d] = -inf (the target rules d out) and r = 1 when
// z_d[d] = -inf < z_t[d].
#pragma once

#include <limits.h>

#include "sv_common.h"
#include "sv_launch.h"

namespace sv {

constexpr int kAcceptThreads = 256;          // one workgroup per sequence
constexpr int kAcceptWaves = kAcceptThreads / kWave;
constexpr int kRecBuf = 2048;                // chunk records staged in LDS per pass (32 KB)
constexpr int kMaxRows = 2 * 63 + 1;         // target rows 0..K plus draft rows 0..K-1
static_assert(kAcceptRowsDirect == kAcceptWaves * 4, "one 16-lane group per row merged from memory");

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

// The same merge by the 16 lanes of a DPP row (gl = lane % 16), so a
// wavefront merges four rows at once with DPP reductions.
__device__ __forceinline__ Merged row16_merge(const StatRec* rec, int nc, float c, bool need_sum, int gl) {
    float m = -INFINITY;
    int idx = INT_MAX;
    int bad = 0;
    for (int k = gl; k < nc; k += 16) {
        const StatRec x = rec[k];
        argmax_combine(m, idx, x.m, x.idx);
        bad |= x.bad;
    }
    row16_argmax(m, idx);
    bad = row16_or(bad) != 0;
    float s = 0.f;
    if (need_sum && m != -INFINITY) {
        for (int k = gl; k < nc; k += 16) {
            const StatRec x = rec[k];
            if (x.m != -INFINITY) s += x.s * exp2f((x.m - m) * c);
        }
        s = row16_sum(s);
    }
    return Merged{m, s, idx, bad};
}

// The same merge by the 16 lanes of a DPP row, reading the records straight
// from global memory (rows with many records, such as one per LM-head
// workgroup): each lane keeps a running record over its batches of loads,
// all loads of a batch in flight at once, then the 16 lanes combine.
__device__ __forceinline__ Merged row16_merge_global(const StatRec* __restrict__ rec, int nc, float c, bool need_sum,
                                                     int gl) {
    constexpr int kBatch = 16;
    float m = -INFINITY, s = 0.f;
    int idx = INT_MAX, bad = 0;
    for (int k0 = 0; k0 < nc; k0 += 16 * kBatch) {
        // every load goes out (an index past nc reads the last record and is
        // masked), so a batch is one round trip
        StatRec x[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int k = k0 + j * 16 + gl;
            const StatRec y = rec[min(k, nc - 1)];
            x[j] = k < nc ? y : StatRec{-INFINITY, 0.f, INT_MAX, 0};
        }
        float bm = m;
        int bi = idx;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            argmax_combine(bm, bi, x[j].m, x[j].idx);
            bad |= x[j].bad;
        }
        if (need_sum && bm != -INFINITY) {
            s = m == -INFINITY ? 0.f : s * exp2f((m - bm) * c);
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (x[j].m != -INFINITY) s += x[j].s * exp2f((x[j].m - bm) * c);
        }
        m = bm;
        idx = bi;
    }
    float M = m;
    int I = idx;
    row16_argmax(M, I);
    bad = row16_or(bad) != 0;
    float S = 0.f;
    if (need_sum && M != -INFINITY) S = row16_sum(m == -INFINITY ? 0.f : s * exp2f((m - M) * c));
    return Merged{M, S, I, bad};
}

// Copy records 0 .. n-1 (record e at src(e)) into LDS: each thread's loads
// in batches of kStageBatch, all of a batch in flight at once (an index past
// n reads the last record and is not stored).  Called by the whole workgroup.
constexpr int kStageBatch = 4;
template <typename Src>
__device__ __forceinline__ void stage_records(StatRec* recs, int n, int tid, Src src) {
    for (int e0 = tid; e0 < n; e0 += kStageBatch * kAcceptThreads) {
        StatRec t[kStageBatch];
#pragma unroll
        for (int u = 0; u < kStageBatch; ++u) t[u] = *src(min(e0 + u * kAcceptThreads, n - 1));
#pragma unroll
        for (int u = 0; u < kStageBatch; ++u)
            if (e0 + u * kAcceptThreads < n) recs[e0 + u * kAcceptThreads] = t[u];
    }
}

// Merge the records of n consecutive rows (nc records each, row r at
// base + r*nc) into merged[out0 + r], one wavefront per row.  Rows are staged
// through LDS with every load in flight at once when they fit; rows longer
// than the buffer are merged straight from global memory.  Called by the
// whole workgroup.
__device__ inline void merge_rows(const StatRec* __restrict__ base, int n, int nc, float c, bool need_sum, StatRec* recs,
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
        stage_records(recs, nr * nc, tid, [&](int e) { return src + e; });
        __syncthreads();
        for (int rr = wave; rr < nr; rr += kAcceptWaves) {
            const Merged x = wave_merge(recs + rr * nc, nc, c, need_sum, lane);
            if (lane == 0) merged[out0 + r0 + rr] = x;
        }
        __syncthreads();
    }
}

// Decide sequence b (slot j of the selection).  Called by a whole workgroup
// of kAcceptThreads threads; every thread gets the returned AcceptInfo (n = -1:
// skipped, malformed or faulted), which is a pure function of the inputs, so
// every workgroup that decides the same sequence gets the same one.  Only a
// caller with `write` stores the outputs: accepted_len, the committed drafts
// (and, greedy, the terminal token; sampled leaves it to the residual draw),
// probs_at_draft, and the -1 rows of a fault.
template <bool SAMPLED>
__device__ AcceptInfo accept_sequence(const float* __restrict__ logits, const float* __restrict__ draft_logits,
                                      const int32_t* __restrict__ draft_tokens, const uint64_t* __restrict__ seeds,
                                      int j, int b, SeqRows seq, int V, float c, RecLayout rec, bool write,
                                      int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
                                      float* __restrict__ probs_at_draft, StatRec* recs, Merged* merged,
                                      AcceptInfo* shared_info) {
    const AcceptInfo fail{-1, b, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f, {0, 0, 0}};
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = seq.K;
    if (b < 0 || b >= seq.B) return fail;
    int t0 = 0, kb = 0;
    if (!seq.get(b, t0, kb)) {   // malformed row_start: no row of this sequence is touched
        if (write && tid == 0) accepted_len[b] = -1;
        return fail;
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
    const StatRec* drf0 = rec.drf + (rec.drf_by_row ? d0 : (size_t)j * K) * rec.drf_nc;
    const int n_drf = SAMPLED ? kb : 0;
    if (rec.tgt_nc == rec.drf_nc && (kb + 1 + n_drf) * rec.tgt_nc <= kRecBuf) {
        // everything in one pass: all record loads of both groups in flight
        const int nc = rec.tgt_nc;
        const int n_tgt = (kb + 1) * nc, n_all = (kb + 1 + n_drf) * nc;
        stage_records(recs, n_all, tid, [&](int e) { return e < n_tgt ? tgt0 + e : drf0 + (e - n_tgt); });
        __syncthreads();
        // four rows per wavefront, one per 16-lane DPP row
        for (int rr = wave * 4 + (lane >> 4); rr < kb + 1 + n_drf; rr += kAcceptWaves * 4) {
            const Merged x = row16_merge(recs + rr * nc, nc, c, SAMPLED, lane & 15);
            if ((lane & 15) == 0) merged[rr] = x;
        }
        __syncthreads();
    } else if (kb + 1 + n_drf <= kAcceptRowsDirect) {
        // few rows with many records each: one row per 16-lane DPP row,
        // straight from global memory
        const int rr = wave * 4 + (lane >> 4);
        if (rr < kb + 1 + n_drf) {
            const bool tgt_row = rr <= kb;
            const StatRec* src = tgt_row ? tgt0 + (size_t)rr * rec.tgt_nc : drf0 + (size_t)(rr - kb - 1) * rec.drf_nc;
            const Merged x = row16_merge_global(src, tgt_row ? rec.tgt_nc : rec.drf_nc, c, !tgt_row || SAMPLED,
                                                lane & 15);
            if ((lane & 15) == 0) merged[rr] = x;
        }
        __syncthreads();
    } else {
        merge_rows(tgt0, kb + 1, rec.tgt_nc, c, SAMPLED, recs, merged, 0);
        if (n_drf > 0) merge_rows(drf0, n_drf, rec.drf_nc, c, true, recs, merged, kb + 1);
    }

    if (wave == 0) {
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
            if (write && active) orow[i] = -1;
            if (lane == 0) {
                if (write) accepted_len[b] = -1;
                *shared_info = fail;
            }
        } else {
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
                        if (write && probs_at_draft) {
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
            // position n: the greedy terminal token here; a sampled one only by
            // the residual draw (in the fused kernel another workgroup writes
            // it, so nothing here may touch that entry)
            if (write && active) {
                if (i < n)
                    orow[i] = tok;
                else if (i > n)
                    orow[i] = -1;
                else if (!SAMPLED)
                    orow[i] = t.idx;
            }
            if (write && lane == 0) accepted_len[b] = n;
            if (i == n)
                *shared_info = AcceptInfo{n, b, t0, kb, u_term, t.m, t.s, has_draft ? d.m : 0.f,
                                          has_draft ? d.s : 0.f, {0, 0, 0}};
        }
    }
    __syncthreads();
    return *shared_info;
}

}  // namespace sv
