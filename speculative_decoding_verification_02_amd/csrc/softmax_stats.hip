// softmax_stats.hip -- per-chunk softmax statistics of the verify rows.
//
// The accept rules need, per row z of logits: its maximum and the lowest
// index attaining it (the greedy rule compares drafts against the target's
// most likely token, "Inference-4", greedy bullet), and the normaliser
// s = sum_v exp((z_v - max) / T) of softmax(z / T) (the sampled rule compares
// target and draft probabilities of the draft token, same page, sampling
// bullet).  A row of V logits is split into chunks of kChunk entries; one
// workgroup reads one chunk once (128-bit coalesced loads into registers),
// reduces max/argmax across the wavefronts, then sums exp2((z - max) * c),
// c = log2(e) / T, from the same registers.  The accept kernel merges the
// chunk records of a row in chunk order:
//     M = max_c m_c,  S = sum_c s_c * exp2((m_c - M) * c),  idx = first chunk's idx with m_c = M.
// Every reduction has a fixed order, so results are bitwise reproducible.
#include <float.h>
#include <limits.h>

#include "sv_common.h"
#include "sv_launch.h"

namespace sv {

// Thread tid of a chunk workgroup owns elements v_begin + (q * kStatThreads + tid) * 4 + e,
// q < 4, e < 4: each load instruction of a wavefront covers 1 KB contiguous.
// STREAM: the logits are read once per step, so large passes stream past the
// caches; small ones keep them cached for the accept kernels' reads of the
// terminal rows that follow.  VEC (V % 4 == 0): four 128-bit loads, else
// sixteen 32-bit loads.  No load sits in a branch: entries past V read an
// in-range address (with a vector/scalar branch per load the compiler waited
// for the first loads before issuing the last one, which halved the bytes in
// flight); mask_tail then sets them to -inf, in the last chunk of a row only.
template <bool STREAM, bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int v_begin, int V, int tid,
                                           float x[kStatPerThread]) {
#pragma unroll
    for (int q = 0; q < kStatPerThread / 4; ++q) {
        const int v = v_begin + (q * kStatThreads + tid) * 4;
        if constexpr (VEC) {
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v* p = reinterpret_cast<const f4v*>(row + min(v, V - 4));
            f4v f;
            if constexpr (STREAM)
                f = __builtin_nontemporal_load(p);
            else
                f = *p;
            x[4 * q + 0] = f.x;
            x[4 * q + 1] = f.y;
            x[4 * q + 2] = f.z;
            x[4 * q + 3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * q + e] = row[min(v + e, V - 1)];
        }
    }
}

__device__ __forceinline__ void mask_tail(int v_begin, int V, int tid, float x[kStatPerThread]) {
#pragma unroll
    for (int q = 0; q < kStatPerThread / 4; ++q) {
        const int v = v_begin + (q * kStatThreads + tid) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = v + e < V ? x[4 * q + e] : -INFINITY;
    }
}

__device__ __forceinline__ int chunk_index(int v_begin, int tid, int k) {
    return v_begin + ((k >> 2) * kStatThreads + tid) * 4 + (k & 3);
}

template <bool NEED_SUM, bool STREAM, bool VEC>
__global__ __launch_bounds__(kStatThreads) void softmax_stats_kernel(
    const float* __restrict__ logits, const float* __restrict__ draft_logits, const int32_t* __restrict__ rows,
    int n_rows, SeqRows seq, int V, int nc, float c, StatRec* __restrict__ stats, int* __restrict__ zero, int n_zero) {
    __shared__ float sm[kStatThreads / kWave];
    __shared__ int si[kStatThreads / kWave];
    __shared__ int sb[kStatThreads / kWave];
    __shared__ float ss[kStatThreads / kWave];

    const int K = seq.K;
    // completion counters and poll slots of a fused accept + residual launch
    // that follows
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < n_zero; i += kStatThreads) zero[i] = 0;
    // chunk positions rotate with the row: workgroups go to the XCDs
    // round-robin, and with chunk = blockIdx % nc each XCD would read the
    // same chunk positions of every row (per-workgroup timestamps put those
    // XCDs' workgroups at 10 to 31 us for the same work; the pass as a whole
    // measured the same either way, and the records are the same bits)
    const int job = blockIdx.x / nc;
    const int chunk = (int)(((long)(blockIdx.x - job * nc) + job) % nc);
    const long slot = (long)job * nc + chunk;              // the record's place: (job, chunk)
    const int tgt_jobs = logits ? n_rows * (K + 1) : 0;   // no target rows: draft rows only
    const bool target = job < tgt_jobs;
    int j, i;
    if (target) {
        j = job / (K + 1);
        i = job - j * (K + 1);
    } else {
        const int jj = job - tgt_jobs;
        j = jj / K;
        i = jj - j * K;
    }
    const int b = rows ? rows[j] : j;
    const int tid = threadIdx.x;
    int t0 = 0, kb = -1;
    // skipped sequence, malformed row_start, or a position past this
    // sequence's drafts: the accept kernel never reads the record
    if (b < 0 || b >= seq.B || !seq.get(b, t0, kb) || (target ? i > kb : i >= kb)) {
        if (tid == 0) stats[slot] = StatRec{-INFINITY, 0.f, INT_MAX, 0};
        return;
    }
    const float* row = target ? logits + ((size_t)t0 + i) * V : draft_logits + ((size_t)(t0 - b) + i) * V;

    const int v_begin = chunk * kChunk;
    float x[kStatPerThread];
    load_chunk<STREAM, VEC>(row, v_begin, V, tid, x);
    if (v_begin + kChunk > V) mask_tail(v_begin, V, tid, x);   // the same for the whole workgroup

    // The pass was bound by its arithmetic per element, not by the loads, so
    // each element costs a compare for the data check, half a max3 for the
    // maximum and a subtract, multiply, exp and add for the sum; the index of
    // the maximum is searched for only by the threads that hold it.  The
    // exponent is (z - max) c, exact at the maximum: z c - max c would round
    // max c, an error in every term that grows as T shrinks (1e-5 in the
    // probabilities at T = 0.05).
    //   bad: some entry is NaN or +inf (the row is unusable);
    //   tm:  the thread's maximum (NaN never compares greater).
    bool bad = false;
    float tm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kStatPerThread; ++k) {
        bad = bad || !(x[k] < INFINITY);
        tm = fmaxf(tm, x[k]);
    }
    const int lane = tid & 63, wave = tid >> 6;
    const float wm = wave_max(tm);
    const unsigned long long anybad = __ballot(bad);
    if (lane == 0) {
        sm[wave] = wm;
        sb[wave] = anybad != 0ull;
    }
    __syncthreads();
    float bm = sm[0];
    int bbad = sb[0];
#pragma unroll
    for (int w = 1; w < kStatThreads / kWave; ++w) {
        bm = max_cs(bm, sm[w]);
        bbad |= sb[w];
    }
    if (bbad) {   // canonical record of an unusable chunk: only its flag is read
        if (tid == 0) stats[slot] = StatRec{-INFINITY, 0.f, INT_MAX, 1};
        return;
    }

    // lowest index attaining the maximum: a thread's indices ascend with k
    int mi = INT_MAX;
    if (tm == bm && bm != -INFINITY) {
#pragma unroll
        for (int k = kStatPerThread - 1; k >= 0; --k)
            if (x[k] == bm) mi = chunk_index(v_begin, tid, k);
    }
    float s = 0.f;
    if (NEED_SUM && bm != -INFINITY) {
#pragma unroll
        for (int k = 0; k < kStatPerThread; ++k) s += __builtin_amdgcn_exp2f((x[k] - bm) * c);
        s = wave_sum(s);
    }
    mi = wave_min(mi);
    if (lane == 0) {
        si[wave] = mi;
        ss[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
        int bi = si[0];
        float bs = ss[0];
#pragma unroll
        for (int w = 1; w < kStatThreads / kWave; ++w) {
            bi = min(bi, si[w]);
            bs += ss[w];
        }
        stats[slot] = StatRec{bm, bs, bi, 0};
    }
}

// Fold the LM-head epilogue's records (one per 256 vocabulary entries of a
// row, in vocabulary order) into the chunk records the statistics pass
// writes (one per kChunk entries): 16 lanes per chunk, one DPP row, lane t
// holding record 16k + t, combined by the DPP row all-reduce (xor 1, xor 2,
// half-row mirror, row mirror).  Both partners of a step compute the same
// combination (the sum is commutative), so every lane of the row ends with
// the same record; bad records contribute only their flag, as in the
// epilogue's own fold.
constexpr int kRecsPerChunk = kChunk / 256;
static_assert(kRecsPerChunk == 16, "one DPP row per chunk");

__device__ __forceinline__ StatRec rec_combine(StatRec a, StatRec b, float c) {
    StatRec r;
    r.bad = a.bad | b.bad;
    if (a.m == -INFINITY) {
        r.m = b.m; r.s = b.s; r.idx = b.idx;
    } else if (b.m == -INFINITY) {
        r.m = a.m; r.s = a.s; r.idx = a.idx;
    } else {
        r.m = fmaxf(a.m, b.m);
        r.s = a.s * __builtin_amdgcn_exp2f((a.m - r.m) * c) + b.s * __builtin_amdgcn_exp2f((b.m - r.m) * c);
        r.idx = (a.m > b.m || (a.m == b.m && a.idx < b.idx)) ? a.idx : b.idx;
    }
    return r;
}

template <int (*MOVE)(int)>
__device__ __forceinline__ StatRec rec_move(const StatRec& a) {
    return StatRec{as_f(MOVE(as_i(a.m))), as_f(MOVE(as_i(a.s))), MOVE(a.idx), MOVE(a.bad)};
}

__global__ __launch_bounds__(kStatThreads) void fold_records_kernel(const StatRec* __restrict__ in, int recs, long items,
                                                                    int nc, float c, StatRec* __restrict__ out) {
    const long g = (long)blockIdx.x * (kStatThreads / kRecsPerChunk) + threadIdx.x / kRecsPerChunk;   // (row, chunk)
    if (g >= items) return;   // whole 16-lane groups (DPP rows) leave together
    const int t = threadIdx.x % kRecsPerChunk;
    const long row = g / nc;
    const int chunk = (int)(g - row * nc);
    const int k = chunk * kRecsPerChunk + t;
    StatRec a{-INFINITY, 0.f, INT_MAX, 0};
    if (k < recs) {
        const StatRec x = in[row * recs + k];
        a = StatRec{x.bad ? -INFINITY : x.m, x.bad ? 0.f : x.s, x.idx, x.bad};
    }
    a = rec_combine(a, rec_move<dpp_xor1>(a), c);
    a = rec_combine(a, rec_move<dpp_xor2>(a), c);
    a = rec_combine(a, rec_move<dpp_half_mirror>(a), c);
    a = rec_combine(a, rec_move<dpp_mirror>(a), c);
    if (t == 0) out[g] = a;
}

hipError_t launch_fold_records(const StatRec* in, int recs_per_row, int rows, int V, float inv_t_log2e, StatRec* out,
                               hipStream_t stream) {
    const int nc = n_chunks(V);
    const long items = (long)rows * nc;
    if (items == 0) return hipSuccess;
    constexpr int kGroups = kStatThreads / kRecsPerChunk;
    const long blocks = (items + kGroups - 1) / kGroups;
    hipLaunchKernelGGL(fold_records_kernel, dim3((unsigned)blocks), dim3(kStatThreads), 0, stream, in, recs_per_row,
                       items, nc, inv_t_log2e, out);
    return hipGetLastError();
}

hipError_t launch_softmax_stats(const float* logits, const float* draft_logits, const int32_t* rows, int n_rows,
                                SeqRows seq, int V, float inv_t_log2e, bool need_sum, StatRec* stats,
                                hipStream_t stream, int* zero, int n_zero) {
    const int nc = n_chunks(V);
    const long jobs = (logits ? (long)n_rows * (seq.K + 1) : 0) + (draft_logits ? (long)n_rows * seq.K : 0);
    const long blocks = jobs * nc;
    if (blocks == 0) return hipSuccess;
    // stream past the caches above 64 MB of logits (4096 chunks of 16 KB)
    const bool stream_hint = blocks > 4096;
    const bool vec = (V & 3) == 0;
    auto kern = need_sum ? (stream_hint ? (vec ? softmax_stats_kernel<true, true, true>
                                               : softmax_stats_kernel<true, true, false>)
                                        : (vec ? softmax_stats_kernel<true, false, true>
                                               : softmax_stats_kernel<true, false, false>))
                         : (stream_hint ? (vec ? softmax_stats_kernel<false, true, true>
                                               : softmax_stats_kernel<false, true, false>)
                                        : (vec ? softmax_stats_kernel<false, false, true>
                                               : softmax_stats_kernel<false, false, false>));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kStatThreads), 0, stream, logits, draft_logits, rows, n_rows,
                       seq, V, nc, inv_t_log2e, stats, zero, zero ? n_zero : 0);
    return hipGetLastError();
}

}  // namespace sv
