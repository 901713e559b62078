// ngram.hip -- the prompt-lookup drafter.
//
// Prompt lookup proposes, as drafts, the tokens that followed the most recent
// earlier occurrence of the sequence's last n tokens, trying the longest n
// (up to max_ngram) first, and proposes nothing if no suffix n-gram occurred
// before ("Inference-4", Prompt lookup decoding; "What is speculative
// decoding" guide, the n-gram simple method).  The search is recast so that
// every position is examined once, independently: for each end position
// e <= L-2 of the history s (length L), let m(e) be the number of trailing
// tokens that agree, s[e-k] == s[L-1-k] for k = 0, 1, ..., capped at
// max_ngram.  A window of n tokens ending at e matches the suffix n-gram iff
// m(e) >= n, so the drafter's choice -- the largest n that matches anywhere,
// then its most recent window -- is the e that maximises (m(e), e) in
// lexicographic order; the drafts are s[e+1 .. e+n_drafts], cut at L.
//
// Two launches: one workgroup per (sequence, segment of kNgSeg end positions)
// stages its segment with coalesced loads, scores every position and stores
// the segment's best key (m << 32 | e); one workgroup, four threads per
// sequence, takes the best key of each sequence, copies the drafts and
// prefix-sums the verify-row offsets row_start[b+1] = row_start[b] +
// count_b + 1.  The history is read once, so the scan is bound by HBM
// bandwidth; the second launch is two dependent rounds of loads (span and
// keys, then the drafts).
#include "sv_common.h"
#include "sv_launch.h"

namespace sv {

constexpr int kNgThreads = 256;
constexpr int kNgPerThread = kNgSeg / kNgThreads;   // end positions per thread
constexpr int kNgFinThreads = 1024;
constexpr int kNgFinLanes = 4;                            // threads per sequence
constexpr int kNgFinSeqs = kNgFinThreads / kNgFinLanes;   // sequences per pass
static_assert(kNgSeg % kNgThreads == 0, "segment must split evenly");

// history span of sequence b, or false if its offsets are malformed (a
// negative start or length, a length above max_len, or an end past the
// hist_len entries behind the history pointer)
__device__ __forceinline__ bool ng_span(const int64_t* hist_start, int b, int max_len, int64_t hist_len, int64_t& s0,
                                        int& L) {
    s0 = hist_start[b];
    const int64_t len = hist_start[b + 1] - s0;
    if (s0 < 0 || len < 0 || len > max_len || s0 > hist_len - len) return false;
    L = (int)len;
    return true;
}

// One workgroup per (sequence, segment): the best key (m << 32 | e) of the
// segment's end positions goes to keys[b * segs + seg] (0: no match, or no
// position in the segment), so no slot needs clearing beforehand.  Thread tid
// loads s[e] for e = e0 + i * kNgThreads + tid, all loads in flight at once,
// and compares it with the sequence's last token in registers; only a hit
// (rare unless the vocabulary is tiny or the text repeats) reads the earlier
// tokens of its window, from the cache the segment was just streamed through.
__global__ __launch_bounds__(kNgThreads) void ngram_scan_kernel(const int32_t* __restrict__ hist,
                                                                int64_t hist_len,
                                                                const int64_t* __restrict__ hist_start, int max_len,
                                                                int G, int segs, unsigned long long* keys) {
    __shared__ unsigned long long red[kNgThreads / kWave];

    const int b = blockIdx.x / segs;
    const int seg = blockIdx.x - b * segs;
    const int tid = threadIdx.x;
    int64_t s0 = 0;
    int L = 0;
    const bool ok = ng_span(hist_start, b, max_len, hist_len, s0, L);
    const int e0 = seg * kNgSeg;                 // end positions e0 .. e1-1, e <= L-2
    const int e1 = ok ? min(e0 + kNgSeg, L - 1) : 0;
    if (e0 >= e1) {
        if (tid == 0) keys[blockIdx.x] = 0ull;
        return;
    }
    const int32_t* s = hist + s0;
    const int32_t last = s[L - 1];

    // every load goes out (a position past the segment re-reads its last
    // position, which is not scored), so all of a thread's loads are in
    // flight together
    int32_t v[kNgPerThread];
#pragma unroll
    for (int i = 0; i < kNgPerThread; ++i) {
        const int e = e0 + i * kNgThreads + tid;
        v[i] = s[min(e, e1 - 1)];
    }
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < kNgPerThread; ++i) {
        const int e = e0 + i * kNgThreads + tid;
        if (e < e1 && v[i] == last) {
            int m = 1;
            while (m < G && e - m >= 0 && s[e - m] == s[L - 1 - m]) ++m;
            const unsigned long long key = ((unsigned long long)m << 32) | (unsigned)e;
            best = key > best ? key : best;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long y = __shfl_xor(best, o, kWave);
        best = y > best ? y : best;
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kNgThreads / kWave; ++w) best = red[w] > best ? red[w] : best;
        keys[blockIdx.x] = best;
    }
}

// One workgroup: per sequence (four threads, a DPP quad), the best key over
// its segments, the drafts that follow the chosen window, and the prefix sum
// of the verify rows.  The span and the keys are loaded together (thread q
// takes segments q, q+4, ...), then the drafts (thread q takes positions q,
// q+4, ...).
__device__ __forceinline__ unsigned long long quad_max_u64(unsigned long long x) {
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const int lo = (int)(unsigned)x, hi = (int)(unsigned)(x >> 32);
        const int plo = step ? dpp_xor2(lo) : dpp_xor1(lo), phi = step ? dpp_xor2(hi) : dpp_xor1(hi);
        const unsigned long long y = ((unsigned long long)(unsigned)phi << 32) | (unsigned)plo;
        x = y > x ? y : x;
    }
    return x;
}

__global__ __launch_bounds__(kNgFinThreads) void ngram_finalize_kernel(
    const int32_t* __restrict__ hist, int64_t hist_len, const int64_t* __restrict__ hist_start, int B, int max_len,
    int n_drafts,
    int segs, const unsigned long long* __restrict__ keys, int32_t* __restrict__ drafts, int32_t* __restrict__ count,
    int32_t* __restrict__ row_start) {
    __shared__ int wsum[kNgFinThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = tid & (kNgFinLanes - 1);
    constexpr int kKeyBatch = 8;
    constexpr int kDraftPer = (kNgMaxDrafts + kNgFinLanes - 1) / kNgFinLanes;
    int carry = 0;
    if (row_start && tid == 0) row_start[0] = 0;
    for (int base = 0; base < B; base += kNgFinSeqs) {
        const int b = base + tid / kNgFinLanes;
        const bool live = b < B;   // whole quads
        int64_t s0 = 0;
        int L = 0;
        bool ok = false;
        unsigned long long key = 0ull;
        if (live) {
            ok = ng_span(hist_start, b, max_len, hist_len, s0, L);
            const unsigned long long* kb = keys + (size_t)b * segs;
            for (int g0 = q; g0 < segs; g0 += kNgFinLanes * kKeyBatch) {
                unsigned long long k[kKeyBatch];
#pragma unroll
                for (int g = 0; g < kKeyBatch; ++g) {
                    const int idx = g0 + g * kNgFinLanes;
                    k[g] = idx < segs ? kb[idx] : 0ull;
                }
#pragma unroll
                for (int g = 0; g < kKeyBatch; ++g) key = k[g] > key ? k[g] : key;
            }
        }
        key = quad_max_u64(key);
        int c = 0;
        if (live) {
            int32_t* drow = drafts + (size_t)b * n_drafts;
            if (!ok) {
                for (int i = q; i < n_drafts; i += kNgFinLanes) drow[i] = -1;
                if (q == 0) count[b] = -1;
            } else {
                const int start = (int)(key & 0xffffffffull) + 1;   // after the matched window
                if (key >> 32) c = min(n_drafts, L - start);          // a match: L - start >= 1
                int32_t t[kDraftPer];
#pragma unroll
                for (int j = 0; j < kDraftPer; ++j) {
                    const int i = q + j * kNgFinLanes;
                    t[j] = i < c ? hist[s0 + start + i] : -1;
                }
#pragma unroll
                for (int j = 0; j < kDraftPer; ++j) {
                    const int i = q + j * kNgFinLanes;
                    if (i < n_drafts) drow[i] = t[j];
                }
                if (q == 0) count[b] = c;
            }
        }
        if (row_start) {
            // inclusive scan of count + 1 (one value per quad, at its first
            // thread) over the pass, then the running carry
            const int x = wave_inclusive_scan_int(live && q == 0 ? c + 1 : 0);
            if (lane == kWave - 1) wsum[wave] = x;
            __syncthreads();
            int pre = carry;
            for (int w = 0; w < wave; ++w) pre += wsum[w];
            if (live && q == 0) row_start[b + 1] = pre + x;
            int tot = 0;
            for (int w = 0; w < kNgFinThreads / kWave; ++w) tot += wsum[w];
            carry += tot;
            __syncthreads();
        }
    }
}

hipError_t launch_ngram(const int32_t* hist, int64_t hist_len, const int64_t* hist_start, int B, int max_len, int G,
                        int n_drafts,
                        int32_t* drafts, int32_t* count, int32_t* row_start, unsigned long long* keys,
                        hipStream_t stream) {
    if (n_drafts < 0 || n_drafts > kNgMaxDrafts) return hipErrorInvalidValue;
    const int segs = ngram_segments(max_len);
    if (segs > 0) {
        hipLaunchKernelGGL(ngram_scan_kernel, dim3((unsigned)((long)B * segs)), dim3(kNgThreads), 0, stream, hist,
                           hist_len, hist_start, max_len, G, segs, keys);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(ngram_finalize_kernel, dim3(1), dim3(kNgFinThreads), 0, stream, hist, hist_len, hist_start, B,
                       max_len, n_drafts, segs, keys, drafts, count, row_start);
    return hipGetLastError();
}

}  // namespace sv
