// residual.hip -- terminal draw of sampled sequences.
//
// After the first rejection at position n < kb (the sequence's draft count)
// the replacement token is drawn from norm(max(0, q_n - p_n)); when all kb
// drafts are accepted the bonus token is drawn from q_kb ("Inference-4", sampling bullet; "speculative-decoding"
// blog, Rejection sampling; "What is speculative decoding" guide, How
// speculative decoding works).  The draw is an inverse CDF:
//     t = min{v : C_v > u' * Z},  C_v = w_0 + ... + w_v,  Z = C_{V-1}.
//
// Workgroups sum the weights of one chunk each, or of a small group of
// chunks (fixed-order reductions); then, for a sequence, a prefix over the
// chunk sums finds the chunk c* holding u'Z and a workgroup scan over c*'s
// weights finds t.  Where the selection runs depends on the launch:
//   - at most 256 workgroups (all resident at once): each publishes its sums
//     in tagged slots and polls its sequence's slots; the workgroup that holds
//     c* picks t (a bounded wait; a workgroup that gives up sums every chunk
//     itself);
//   - up to 4096 workgroups: the one that finishes last, counted in with an
//     atomic;
//   - beyond: a second launch, one workgroup per sequence.
// Both phases evaluate a weight with the same function from the same inputs,
// so a chunk's elements agree bitwise between them; only the order of the
// within-chunk sum differs, and the selection falls back to the last (or first)
// token of positive weight in c* if rounding leaves u'Z outside the scanned
// range.  A token of zero weight is never drawn.  If the residual has no mass
// (possible only through rounding when q_n ~ p_n) the draw uses q_n instead.
#include <limits.h>

#include <type_traits>

#include "sv_accept.h"

namespace sv {

constexpr int kMaxChunks = 1024;  // V <= kMaxChunks * kChunk (checked on the host)
// Above this many (sequence, chunk) blocks the draw runs in two launches
// (sums, then selection) instead of one with a last-block selection: at
// B = 256 64 + 8 us against 84, at B = 512 117 + 8 against 140.
constexpr long kResidualSplitBlocks = 4096;

// w_v for the terminal row: q_n(v) - p_n(v) clipped at 0, or q_n(v) itself,
// each probability as one exp2 with its normaliser folded into the exponent:
// q = 2^((z - M) c - log2 S).  The exp2 is the hardware instruction alone:
// a probability below 2^-126 becomes 0 (exp2f would rescale to keep it as a
// denormal, at five more instructions per exp2, and the draws are
// bandwidth-bound only without them).
struct TermNorm {
    float mt, lst, md, lsd;   // maxima and log2 of the sums of the terminal rows
};
__device__ __forceinline__ TermNorm term_norm(const AcceptInfo& a) {
    return TermNorm{a.mt, log2f(a.st), a.md, a.sd > 0.f ? log2f(a.sd) : 0.f};
}
__device__ __forceinline__ float term_weight(float zt, float zd, const TermNorm& t, float c, bool use_q) {
    const float q = __builtin_amdgcn_exp2f(fmaf(zt - t.mt, c, -t.lst));
    if (use_q) return q;
    const float p = __builtin_amdgcn_exp2f(fmaf(zd - t.md, c, -t.lsd));
    return fmaxf(q - p, 0.f);
}

// The thread's PER weights of one chunk of PER * kStatThreads entries, in the
// coalesced order of the statistics pass: element (q * kStatThreads + tid) * 4
// + e of the chunk.  VEC (V % 4 ==
// 0): 128-bit loads, else 32-bit ones; USE_Q: the target row only.  No load
// sits in a branch (entries past V read an in-range address and get weight
// 0), so all of a thread's loads are in flight together.  Two phases, so a
// caller can have the next chunk's loads in flight while it weighs this one.
template <bool NT>
__device__ __forceinline__ float4 load4(const float* p) {
    if constexpr (NT) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        const f4v f = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
        return float4{f.x, f.y, f.z, f.w};
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

// NT: stream the rows past the caches (the split draw of large batches,
// whose terminal rows were not read recently).
template <bool VEC, bool USE_Q, int PER, bool NT = false>
__device__ __forceinline__ void chunk_load(const float* __restrict__ zt_row, const float* __restrict__ zd_row,
                                           int v_begin, int V, int tid, float zt[PER], float zd[PER]) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
        const int v = v_begin + (q * kStatThreads + tid) * 4;
        if constexpr (VEC) {
            const int vc = min(v, V - 4);
            const float4 f = load4<NT>(zt_row + vc);
            zt[4 * q] = f.x; zt[4 * q + 1] = f.y; zt[4 * q + 2] = f.z; zt[4 * q + 3] = f.w;
            if constexpr (!USE_Q) {
                const float4 g = load4<NT>(zd_row + vc);
                zd[4 * q] = g.x; zd[4 * q + 1] = g.y; zd[4 * q + 2] = g.z; zd[4 * q + 3] = g.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vc = min(v + e, V - 1);
                zt[4 * q + e] = zt_row[vc];
                if constexpr (!USE_Q) zd[4 * q + e] = zd_row[vc];
            }
        }
    }
}
template <bool USE_Q, int PER>
__device__ __forceinline__ void chunk_weigh(const float zt[PER], const float zd[PER], int v_begin, int V, int tid,
                                            const TermNorm& tn, float c, float w[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) w[k] = term_weight(zt[k], USE_Q ? 0.f : zd[k], tn, c, USE_Q);
    // entries past V were weighed from a valid duplicate: zero them, in the
    // last chunk of a row only (the test is the same for the whole workgroup)
    if (v_begin + PER * kStatThreads > V) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int v = v_begin + ((k >> 2) * kStatThreads + tid) * 4 + (k & 3);
            w[k] = v < V ? w[k] : 0.f;
        }
    }
}
template <bool VEC, bool USE_Q, int PER, bool NT>
__device__ __forceinline__ void chunk_weights_impl(const float* __restrict__ zt_row, const float* __restrict__ zd_row,
                                                   int v_begin, int V, int tid, const TermNorm& tn, float c,
                                                   float w[PER]) {
    float zt[PER], zd[PER];
    chunk_load<VEC, USE_Q, PER, NT>(zt_row, zd_row, v_begin, V, tid, zt, zd);
    chunk_weigh<USE_Q, PER>(zt, zd, v_begin, V, tid, tn, c, w);
}

template <int PER = kStatPerThread, bool NT = false>
__device__ __forceinline__ void chunk_weights(const float* __restrict__ zt_row, const float* __restrict__ zd_row,
                                              int v_begin, int V, bool vec, int tid, const AcceptInfo& a, float c,
                                              bool use_q, float w[PER]) {
    const TermNorm tn = term_norm(a);
    if (vec) {
        if (use_q) chunk_weights_impl<true, true, PER, NT>(zt_row, zd_row, v_begin, V, tid, tn, c, w);
        else chunk_weights_impl<true, false, PER, NT>(zt_row, zd_row, v_begin, V, tid, tn, c, w);
    } else {
        if (use_q) chunk_weights_impl<false, true, PER, NT>(zt_row, zd_row, v_begin, V, tid, tn, c, w);
        else chunk_weights_impl<false, false, PER, NT>(zt_row, zd_row, v_begin, V, tid, tn, c, w);
    }
}

__device__ __forceinline__ float block_sum(float s, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    s = wave_sum(s);
    __syncthreads();
    if (lane == 0) red[wave] = s;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int k = 1; k < kStatThreads / kWave; ++k) t += red[k];
    return t;
}

struct TermRows {
    const float* zt;
    const float* zd;
    bool bonus;
};

__device__ __forceinline__ TermRows term_rows(const float* logits, const float* draft_logits, const AcceptInfo& a,
                                              int V) {
    TermRows r;
    r.bonus = a.n == a.kb;
    r.zt = logits + ((size_t)a.t0 + a.n) * V;
    r.zd = r.bonus ? r.zt : draft_logits + ((size_t)(a.t0 - a.b) + a.n) * V;
    return r;
}

// pre[0] = 0, pre[k+1] = chunk_sums[0] + ... + chunk_sums[k] for k < nc, by
// one wavefront: 64 chunks at a time, a shuffle scan plus the running carry.
// (src may alias pre + 1: each element is read before it is overwritten.)
__device__ __forceinline__ void chunk_prefix(const float* src, int nc, int lane, float* pre, bool from_global) {
    float carry = 0.f;
    for (int base = 0; base < nc; base += kWave) {
        const int k = base + lane;
        float v = 0.f;
        if (k < nc)
            v = from_global ? __hip_atomic_fetch_add(const_cast<float*>(src) + k, 0.f, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                            : src[k];
        v = wave_inclusive_scan(v) + carry;
        if (k < nc) pre[k + 1] = v;
        carry = __shfl(v, kWave - 1, kWave);
    }
    if (lane == 0) pre[0] = 0.f;
}

// c* = the first chunk whose inclusive prefix exceeds x; if rounding leaves
// none, the last chunk with positive mass.  One wavefront; every lane gets it.
__device__ __forceinline__ int choose_chunk(const float* pre, int nc, float x, int lane) {
    int cs = -1, last_pos = 0;
    for (int base = 0; base < nc && cs < 0; base += kWave) {
        const int k = base + lane;
        const bool in = k < nc;
        const unsigned long long over = __ballot(in && pre[k + 1] > x);
        const unsigned long long pos = __ballot(in && pre[k + 1] > pre[k]);
        if (over) cs = base + __ffsll((long long)over) - 1;
        if (pos) last_pos = base + 63 - __clzll((long long)pos);
    }
    return cs < 0 ? last_pos : cs;
}

// The token of one chunk at which the running sum of its weights first
// exceeds xr.  Thread tid owns tokens [tid*PER, tid*PER+PER) of the chunk,
// weights mine[]; a token of zero weight is never taken, and if rounding puts
// xr outside the chunk's scanned range the first (xr < 0) or last token of
// positive weight is.  Called by the whole workgroup; the returned index
// (relative to v_begin, plus v_begin) is the same in every thread.
template <int PER>
__device__ int pick_in_chunk(const float (&mine)[PER], float xr, int v_begin, int* sel, float* wtot, int* redi) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sel[1] = -1;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) s += mine[e];
    // inclusive scan of the thread sums: within the wave, then across waves
    float incl = wave_inclusive_scan(s);
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    float base = 0.f;
    for (int w2 = 0; w2 < wave; ++w2) base += wtot[w2];
    incl += base;
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = base;

    if (excl <= xr && xr < incl) {  // exactly one thread's interval can hold xr
        float run = excl;
        int tok = -1, lastp = -1;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (mine[e] > 0.f) lastp = e;
            run += mine[e];
            if (tok < 0 && run > xr && mine[e] > 0.f) tok = e;
        }
        if (tok < 0) tok = lastp;
        sel[1] = v_begin + tid * PER + tok;
    }
    __syncthreads();
    if (sel[1] < 0) {  // block-uniform: read after the barrier
        const bool low = xr < 0.f;
        int cand = low ? INT_MAX : -1;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid * PER + e;
            if (mine[e] > 0.f) cand = low ? min(cand, idx) : max(cand, idx);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const int y = __shfl_xor(cand, o, kWave);
            cand = low ? min(cand, y) : max(cand, y);
        }
        if (lane == 0) redi[wave] = cand;
        __syncthreads();
        if (tid == 0) {
            int best = redi[0];
            for (int w2 = 1; w2 < kStatThreads / kWave; ++w2) best = low ? min(best, redi[w2]) : max(best, redi[w2]);
            sel[1] = v_begin + best;
        }
        __syncthreads();
    }
    return sel[1];
}

// Where select_terminal finds the chunk sums: published by the chunk
// workgroups and read back with atomic read-modify-writes, written by an
// earlier launch (plain loads), or not at all (the workgroup sums every chunk
// itself, with the same function and reduction order as the chunk workgroups,
// so the sums are the same bits).
enum class SumSrc { Atomic, Plain, Local };

// Inverse-CDF selection of the terminal token of one sequence.  With
// w_lo >= 0 the token is written only if it falls in chunks [w_lo, w_hi) (so
// several workgroups may run the selection and exactly one writes).
template <int PER = kStatPerThread>
__device__ void select_terminal(const float* __restrict__ logits, const float* __restrict__ draft_logits,
                                int V, int nc, float c, const AcceptInfo& a, const float* chunk_sums,
                                int32_t* __restrict__ out_tokens, SumSrc src = SumSrc::Atomic, int w_lo = -1,
                                int w_hi = -1) {
    constexpr int CH = PER * kStatThreads;               // entries per chunk
    __shared__ float pre[kMaxChunks * kChunk / CH + 1];  // prefix over chunk sums
    __shared__ float wl[CH];                             // weights of the selected chunk, token order
    __shared__ float red[kStatThreads / kWave];
    __shared__ float wtot[kStatThreads / kWave];
    __shared__ int sel[2];                  // selected chunk, selected token
    __shared__ int redi[kStatThreads / kWave];

    const TermRows tr = term_rows(logits, draft_logits, a, V);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool vec = (V & 3) == 0;

    // pre[k+1] = the sum of chunk k, summed here, then the prefix in place
    auto local_prefix = [&](bool q_only) {
        for (int k = 0; k < nc; ++k) {
            float w[PER];
            chunk_weights<PER>(tr.zt, tr.zd, k * CH, V, vec, tid, a, c, q_only, w);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) s += w[e];
            s = block_sum(s, red);
            if (tid == 0) pre[k + 1] = s;
        }
        __syncthreads();
        if (wave == 0) chunk_prefix(pre + 1, nc, lane, pre, false);
        __syncthreads();
    };

    bool use_q = tr.bonus;
    if (src == SumSrc::Local) {
        local_prefix(use_q);
    } else {
        if (wave == 0) chunk_prefix(chunk_sums, nc, lane, pre, src == SumSrc::Atomic);
        __syncthreads();
    }
    if (!(pre[nc] > 0.f) && !use_q) {
        // residual without mass: draw from q_n, recomputing the chunk sums
        use_q = true;
        local_prefix(true);
    }
    const float Z = pre[nc];
    const float x = a.u_term * Z;
    if (wave == 0) {
        const int cs = choose_chunk(pre, nc, x, lane);
        if (lane == 0) sel[0] = cs;
    }
    __syncthreads();
    const int cs = sel[0];
    if (w_lo >= 0 && (cs < w_lo || cs >= w_hi)) return;   // block-uniform
    const int v_begin = cs * CH;

    // weights of chunk cs into LDS in token order
    {
        float w[PER];
        chunk_weights<PER>(tr.zt, tr.zd, v_begin, V, vec, tid, a, c, use_q, w);
#pragma unroll
        for (int q = 0; q < PER / 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) wl[(q * kStatThreads + tid) * 4 + e] = w[4 * q + e];
    }
    __syncthreads();
    float mine[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) mine[e] = wl[tid * PER + e];
    const int tok = pick_in_chunk<PER>(mine, x - pre[cs], v_begin, sel, wtot, redi);
    if (tid == 0) out_tokens[(size_t)a.t0 + a.n] = tok;
}

// Wave 0 reads the n (<= kPollMaxBlocks) tagged slots of a sequence until
// every one is written, at most spin_limit + 1 rounds of one memory round
// trip each, and leaves the sums in psum.  Returns, in every thread of the
// workgroup, whether it saw them all.  Each slot is its own publication (the
// sum and its tag in one atomic word), so no ordering between slots is needed.
__device__ bool poll_sums(const unsigned long long* slots, int n, int spin_limit, float* psum) {
    __shared__ int seen;
    constexpr int kPer = kPollMaxBlocks / kWave;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < kWave) {
        bool all = false;
        for (int round = 0;; ++round) {
            // every load goes out (a slot past n re-reads the last one), so a
            // round is one memory round trip
            unsigned long long v[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                v[i] = __hip_atomic_load(const_cast<unsigned long long*>(slots) + min(lane + i * kWave, n - 1),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool miss = false;
#pragma unroll
            for (int i = 0; i < kPer; ++i) miss |= (v[i] >> 32) != (kPollTag >> 32);
            if (__ballot(miss) == 0ull) {
#pragma unroll
                for (int i = 0; i < kPer; ++i)
                    if (lane + i * kWave < n) psum[lane + i * kWave] = __uint_as_float((uint32_t)v[i]);
                all = true;
                break;
            }
            if (round >= spin_limit) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) seen = all;
    }
    __syncthreads();
    return seen != 0;
}

// The selection of the one-launch accept + residual for small launches, by
// every chunk workgroup of the sequence once it has seen all the chunk sums
// (psum, in LDS): the prefix, the chunk, and, in the workgroup that owns the
// chosen chunk only, the token, from the weights it still holds in
// registers.  Same arithmetic and order as select_terminal, so the same
// token.  Without residual mass the workgroup of chunk 0 draws from q alone.
template <int PER>
__device__ void select_polled(const float* __restrict__ logits, const float* __restrict__ draft_logits, int V,
                              int nc, float c, const AcceptInfo& a, int chunk, const float (&w)[PER],
                              const float* psum, int32_t* __restrict__ out_tokens) {
    static_assert(PER == 4, "one float4 per thread: the registers hold the chunk in token order");
    constexpr int CH = PER * kStatThreads;
    __shared__ float pre[kPollMaxBlocks + 1];
    __shared__ float wtot[kStatThreads / kWave];
    __shared__ int sel[2];
    __shared__ int redi[kStatThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave == 0) chunk_prefix(psum, nc, lane, pre, false);
    __syncthreads();
    if (!(pre[nc] > 0.f) && a.n != a.kb) {
        if (chunk == 0) select_terminal<PER>(logits, draft_logits, V, nc, c, a, nullptr, out_tokens, SumSrc::Local);
        return;
    }
    const float x = a.u_term * pre[nc];
    if (wave == 0) {
        const int cs = choose_chunk(pre, nc, x, lane);
        if (lane == 0) sel[0] = cs;
    }
    __syncthreads();
    const int cs = sel[0];
    if (cs != chunk) return;   // block-uniform
    const int tok = pick_in_chunk<PER>(w, x - pre[cs], cs * CH, sel, wtot, redi);
    if (tid == 0) out_tokens[(size_t)a.t0 + a.n] = tok;
}

// One workgroup per (sampled sequence, chunk): the sum of the terminal weights
// over the chunk; the last workgroup of a sequence to finish (counted with an
// atomic; the accept kernel zeroed the counter) then selects the token.
__global__ __launch_bounds__(kStatThreads) void residual_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, int V, int nc, float c,
    const AcceptInfo* __restrict__ info, float* __restrict__ chunk_sums, int* __restrict__ counters,
    int32_t* __restrict__ out_tokens) {
    __shared__ float red[kStatThreads / kWave];
    __shared__ int last;
    const int j = blockIdx.x / nc;
    const int chunk = blockIdx.x - j * nc;
    const AcceptInfo a = info[j];
    if (a.n < 0) return;
    const TermRows tr = term_rows(logits, draft_logits, a, V);
    float w[kStatPerThread];
    chunk_weights(tr.zt, tr.zd, chunk * kChunk, V, (V & 3) == 0, threadIdx.x, a, c, tr.bonus, w);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kStatPerThread; ++k) s += w[k];
    s = block_sum(s, red);
    if (threadIdx.x == 0) {
        // Publish the chunk sum with a device-scope atomic exchange and wait for
        // its returned value, so the exchange has been performed, before
        // counting this block in; the selecting block reads the sums back with
        // atomic read-modify-writes, which are performed where the exchanges
        // were.  (A device-scope release fence would publish it too, but by
        // writing back and invalidating the XCD's whole L2.)
        const float prev = __hip_atomic_exchange(chunk_sums + blockIdx.x, s, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(prev));
        last = __hip_atomic_fetch_add(counters + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nc - 1;
    }
    __syncthreads();
    if (!last) return;
    select_terminal(logits, draft_logits, V, nc, c, a, chunk_sums + (size_t)j * nc, out_tokens);
}

// The same draw in two launches, for large batches: the chunk sums with
// plain stores (a workgroup retires as soon as its chunk is summed, with no
// device-scope atomics to wait for), then one workgroup per sequence selects
// (the sums are visible to the next launch).
__global__ __launch_bounds__(kStatThreads) void residual_sums_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, int V, int nc, float c,
    const AcceptInfo* __restrict__ info, float* __restrict__ chunk_sums) {
    __shared__ float red[kStatThreads / kWave];
    const int j = blockIdx.x / nc;
    const int chunk = blockIdx.x - j * nc;
    const AcceptInfo a = info[j];
    if (a.n < 0) return;
    const TermRows tr = term_rows(logits, draft_logits, a, V);
    float w[kStatPerThread];
    chunk_weights<kStatPerThread, true>(tr.zt, tr.zd, chunk * kChunk, V, (V & 3) == 0, threadIdx.x, a, c, tr.bonus,
                                        w);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kStatPerThread; ++k) s += w[k];
    s = block_sum(s, red);
    if (threadIdx.x == 0) chunk_sums[blockIdx.x] = s;
}

__global__ __launch_bounds__(kStatThreads) void residual_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, int V, int nc, float c,
    const AcceptInfo* __restrict__ info, const float* __restrict__ chunk_sums, int32_t* __restrict__ out_tokens) {
    const int j = blockIdx.x;
    const AcceptInfo a = info[j];
    if (a.n < 0) return;
    select_terminal(logits, draft_logits, V, nc, c, a, chunk_sums + (size_t)j * nc, out_tokens, SumSrc::Plain);
}

// The draw for moderate batches in one launch of at most kPollMaxBlocks
// workgroups: workgroup (sequence j, group g) sums chunks [g*G, g*G + G) of
// the terminal row (all of its loads in flight at once: with one workgroup
// per CU, a chunk at a time streamed too slowly; each sum with the code and
// order of residual_kernel), puts each sum in its own tagged slot (zeroed by
// the accept kernel before), then polls all nc slots of its sequence.  Every
// workgroup computes the prefix and the chunk the same way; the one whose
// chunks hold it re-reads that chunk (it streamed it moments ago) and picks
// the token, as select_terminal does.  The wait is bounded: a workgroup that
// runs out sums every chunk itself and writes the token if it falls in its
// chunks.
template <int G>
__global__ __launch_bounds__(kStatThreads) void residual_polled_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, int V, int nc, int ngroups,
    float c, const AcceptInfo* __restrict__ info, unsigned long long* __restrict__ slots, int spin_limit,
    int32_t* __restrict__ out_tokens) {
    __shared__ float red[kStatThreads / kWave];
    __shared__ float psum[kPollMaxBlocks];
    const int j = blockIdx.x / ngroups;
    const int grp = blockIdx.x - j * ngroups;
    const AcceptInfo a = info[j];
    if (a.n < 0) return;
    const TermRows tr = term_rows(logits, draft_logits, a, V);
    const TermNorm tn = term_norm(a);
    const int k0 = grp * G, k1 = min(nc, k0 + G);   // k0 < nc: ngroups = ceil(nc / G)
    unsigned long long* mine = slots + (size_t)j * nc;
    const int tid = threadIdx.x;
    auto run = [&](auto vec_tag, auto q_tag) {
        constexpr bool VEC = decltype(vec_tag)::value, USE_Q = decltype(q_tag)::value;
        float zt[G][kStatPerThread], zd[G][kStatPerThread];
        // every load first (past the group's last chunk: that chunk again,
        // loaded and not used)
#pragma unroll
        for (int g = 0; g < G; ++g)
            chunk_load<VEC, USE_Q, kStatPerThread>(tr.zt, tr.zd, min(k0 + g, k1 - 1) * kChunk, V, tid, zt[g], zd[g]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (k0 + g >= k1) break;   // the same in the whole workgroup
            float w[kStatPerThread];
            chunk_weigh<USE_Q, kStatPerThread>(zt[g], zd[g], (k0 + g) * kChunk, V, tid, tn, c, w);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < kStatPerThread; ++e) s += w[e];
            s = block_sum(s, red);
            if (tid == 0)
                __hip_atomic_store(mine + k0 + g, kPollTag | __float_as_uint(s), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    const bool vec = (V & 3) == 0;
    if (vec) {
        if (tr.bonus) run(std::true_type{}, std::true_type{});
        else run(std::true_type{}, std::false_type{});
    } else {
        if (tr.bonus) run(std::false_type{}, std::true_type{});
        else run(std::false_type{}, std::false_type{});
    }
    if (poll_sums(mine, nc, spin_limit, psum))
        select_terminal(logits, draft_logits, V, nc, c, a, psum, out_tokens, SumSrc::Plain, k0, k1);
    else
        select_terminal(logits, draft_logits, V, nc, c, a, nullptr, out_tokens, SumSrc::Local, k0, k1);
}

// Chunks per workgroup of the grouped polled draw for n_rows sequences over V
// entries (one slot per chunk), or 0 when the launch would not fit it.
int residual_poll_group(int n_rows, int V) {
    const long nc = n_chunks(V);
    if (n_rows <= 0 || nc > kPollMaxBlocks || (long)n_rows * nc > kPollMaxSlots) return 0;
    for (int G = 1; G <= kResidualMaxGroup; G *= 2)
        if ((long)n_rows * ((nc + G - 1) / G) <= kPollMaxBlocks) return G;
    return 0;
}

// Acceptance and residual draw in one launch, for small batches where the
// two kernels' latency dominates: one workgroup per (sampled sequence, chunk).
// Every workgroup of a sequence takes the acceptance decision itself (a few
// hundred statistics records and K token logits: cheap next to the chunk it
// streams), the one of chunk 0 writes it out, and each sums its chunk of the
// terminal weights.  Then, with POLL (at most kPollMaxBlocks workgroups, so
// all of them are resident together), each publishes its sum in a 64-bit
// slot tagged as written and reads all the slots of its sequence until every
// one is tagged; the workgroup owning the chosen chunk picks the token from
// its registers (select_polled).  The wait is bounded by spin_limit rounds;
// a workgroup that runs out sums every chunk itself and writes the token if
// it owns the chosen chunk, so the result does not depend on the bound.
// Without POLL the sums are counted in with an atomic and the last workgroup
// to finish selects, re-reading the chosen chunk.  The counters and slots are
// zeroed by the kernel that runs first (the statistics pass or the
// cooperative LM head).
template <int PER, bool POLL>
__global__ __launch_bounds__(kStatThreads) void accept_residual_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, const int32_t* __restrict__ draft_tokens,
    const uint64_t* __restrict__ seeds, const int32_t* __restrict__ rows, SeqRows seq, int V, int nc, float c,
    RecLayout rec, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probs_at_draft, float* __restrict__ chunk_sums, int* __restrict__ counters,
    unsigned long long* __restrict__ slots, int spin_limit) {
    static_assert(kStatThreads == kAcceptThreads, "one workgroup shape for both phases");
    __shared__ StatRec recs[kRecBuf];
    __shared__ Merged merged[kMaxRows];
    __shared__ AcceptInfo sinfo;
    __shared__ float red[kStatThreads / kWave];
    __shared__ int last;
    const int j = blockIdx.x / nc;
    const int chunk = blockIdx.x - j * nc;
    const int b = rows ? rows[j] : j;
    const AcceptInfo a = accept_sequence<true>(logits, draft_logits, draft_tokens, seeds, j, b, seq, V, c, rec,
                                               chunk == 0, accepted_len, out_tokens, probs_at_draft, recs, merged,
                                               &sinfo);
    if (a.n < 0) return;
    const TermRows tr = term_rows(logits, draft_logits, a, V);
    float w[PER];
    chunk_weights<PER>(tr.zt, tr.zd, chunk * (PER * kStatThreads), V, (V & 3) == 0, threadIdx.x, a, c, tr.bonus, w);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) s += w[k];
    s = block_sum(s, red);
    if constexpr (POLL) {
        __shared__ float psum[kPollMaxBlocks];
        unsigned long long* mine = slots + (size_t)j * nc;
        if (threadIdx.x == 0)
            __hip_atomic_store(mine + chunk, kPollTag | __float_as_uint(s), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (poll_sums(mine, nc, spin_limit, psum)) {
            select_polled<PER>(logits, draft_logits, V, nc, c, a, chunk, w, psum, out_tokens);
        } else {
            select_terminal<PER>(logits, draft_logits, V, nc, c, a, nullptr, out_tokens, SumSrc::Local, chunk,
                                 chunk + 1);
        }
        return;
    }
    if (threadIdx.x == 0) {
        // published as in residual_kernel: an exchange whose result is waited
        // for, then the count
        const float prev = __hip_atomic_exchange(chunk_sums + blockIdx.x, s, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(prev));
        last = __hip_atomic_fetch_add(counters + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nc - 1;
    }
    __syncthreads();
    if (!last) return;
    select_terminal<PER>(logits, draft_logits, V, nc, c, a, chunk_sums + (size_t)j * nc, out_tokens);
}

hipError_t launch_accept_residual(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                                  const uint64_t* seeds, const int32_t* rows, int n_rows, SeqRows seq, int V,
                                  float inv_t_log2e, RecLayout rec, int32_t* accepted_len, int32_t* out_tokens,
                                  float* probs_at_draft, float* chunk_sums, int* counters,
                                  unsigned long long* slots, int spin_limit, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    // small chunks: every workgroup sums (and the selecting one re-reads) a
    // quarter of a statistics chunk, one memory round trip each
    const int nc = n_fused_chunks(V);
    const long blocks = (long)n_rows * nc;
    auto kern = blocks <= kPollMaxBlocks ? accept_residual_kernel<kFusedPer, true>
                                         : accept_residual_kernel<kFusedPer, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kStatThreads), 0, stream, logits, draft_logits,
                       draft_tokens, seeds, rows, seq, V, nc, inv_t_log2e, rec, accepted_len, out_tokens,
                       probs_at_draft, chunk_sums, counters, slots, max(spin_limit, 0));
    return hipGetLastError();
}

hipError_t launch_residual(const float* logits, const float* draft_logits, int n_rows, int V,
                           float inv_t_log2e, const AcceptInfo* info, float* chunk_sums, int* counters,
                           unsigned long long* slots, int spin_limit, int32_t* out_tokens, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    const int nc = n_chunks(V);
    const int G = slots ? residual_poll_group(n_rows, V) : 0;
    if (G > 0) {
        const int ngroups = (nc + G - 1) / G;
        auto kern = G == 1 ? residual_polled_kernel<1> : G == 2 ? residual_polled_kernel<2> : residual_polled_kernel<4>;
        hipLaunchKernelGGL(kern, dim3((unsigned)(n_rows * ngroups)), dim3(kStatThreads), 0, stream, logits,
                           draft_logits, V, nc, ngroups, inv_t_log2e, info, slots, max(spin_limit, 0), out_tokens);
        return hipGetLastError();
    }
    const long blocks = (long)n_rows * nc;
    if (blocks > kResidualSplitBlocks) {
        hipLaunchKernelGGL(residual_sums_kernel, dim3((unsigned)blocks), dim3(kStatThreads), 0, stream, logits,
                           draft_logits, V, nc, inv_t_log2e, info, chunk_sums);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(residual_select_kernel, dim3((unsigned)n_rows), dim3(kStatThreads), 0, stream, logits,
                           draft_logits, V, nc, inv_t_log2e, info, chunk_sums, out_tokens);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)blocks), dim3(kStatThreads), 0, stream, logits,
                       draft_logits, V, nc, inv_t_log2e, info, chunk_sums, counters, out_tokens);
    return hipGetLastError();
}

}  // namespace sv
