// sv_common.h -- device-side helpers shared by the verify-step kernels
// (gfx950, wave64).  Internal to the library: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- sizes ----

constexpr int kWave = 64;
// Softmax statistics and residual sums split each vocabulary row into fixed
// chunks; one workgroup of kStatThreads threads owns a chunk, each thread
// kStatPerThread of its elements (see the kernels for the order).
constexpr int kStatThreads = 256;
constexpr int kStatPerThread = 16;
constexpr int kChunk = kStatThreads * kStatPerThread;  // 4096 logits per chunk

inline int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// ------------------------------------------------------------- records ----

// Partial softmax statistics of one chunk of one row: m = max of the raw
// logits z over the chunk, s = sum exp((z - m) / T) over the chunk, idx = the
// lowest index attaining m, bad = the chunk held a NaN or +inf.
struct __align__(16) StatRec {
    float m;
    float s;
    int idx;
    int bad;
};

// What the accept kernel hands to the residual kernels for one sampled
// sequence: terminal position n (-1 = sequence faulted or skipped), its batch
// slot b, first target row t0 and draft count kb, the terminal uniform, and
// the merged statistics of the terminal target row and (if n < kb) draft row.
struct __align__(16) AcceptInfo {
    int n;
    int b;
    int t0;
    int kb;
    float u_term;
    float mt;
    float st;
    float md;
    float sd;
    int pad[3];
};

// Where the verify rows of sequence b sit.  Rows of all sequences are packed
// in sequence order: target rows t0 .. t0+kb of sequence b, and its draft
// rows / tokens t0-b .. t0-b+kb-1 (sequence b' < b contributes kb'+1 target
// rows and kb' drafts).  Dense batches (row_start == nullptr) have
// t0 = b*(K+1) and kb = K; ragged ones read row_start[b], row_start[b+1] and
// K bounds every kb.  get() rejects a sequence whose entries would put any of
// its rows outside the total / total-B rows the caller declared, so a
// malformed row_start faults only the sequences it names.
struct SeqRows {
    const int32_t* row_start;
    int B;
    int K;
    int total;

    __device__ __forceinline__ bool get(int b, int& t0, int& kb) const {
        if (!row_start) {
            t0 = b * (K + 1);
            kb = K;
            return true;
        }
        const long long s0 = row_start[b], s1 = row_start[b + 1];
        const long long k = s1 - s0 - 1;
        if (k < 0 || k > K || s0 < b || s1 > (long long)total - (B - 1 - b)) return false;
        t0 = (int)s0;
        kb = (int)k;
        return true;
    }
};

// ---------------------------------------------------------- reductions ----

// max with lowest-index tie break; NaN never enters (callers mask it).
__device__ __forceinline__ void argmax_combine(float& m, int& i, float m2, int i2) {
    if (m2 > m || (m2 == m && i2 < i)) {
        m = m2;
        i = i2;
    }
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15) with DPP
// moves, a few cycles each instead of a shuffle's LDS round trip: xor 1 and
// xor 2 (quad permutes), then the half-row mirror and the row mirror.  Every
// step combines a lane with a partner holding an equally reduced value and
// the combinations are symmetric, so all 16 lanes end with the same result.
__device__ __forceinline__ int dpp_xor1(int x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_half_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); }

__device__ __forceinline__ float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_i(float x) { return __builtin_bit_cast(int, x); }

__device__ __forceinline__ void row16_argmax(float& m, int& i) {
    argmax_combine(m, i, as_f(dpp_xor1(as_i(m))), dpp_xor1(i));
    argmax_combine(m, i, as_f(dpp_xor2(as_i(m))), dpp_xor2(i));
    argmax_combine(m, i, as_f(dpp_half_mirror(as_i(m))), dpp_half_mirror(i));
    argmax_combine(m, i, as_f(dpp_mirror(as_i(m))), dpp_mirror(i));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += as_f(dpp_xor1(as_i(x)));
    x += as_f(dpp_xor2(as_i(x)));
    x += as_f(dpp_half_mirror(as_i(x)));
    x += as_f(dpp_mirror(as_i(x)));
    return x;
}
__device__ __forceinline__ int row16_or(int x) {
    x |= dpp_xor1(x);
    x |= dpp_xor2(x);
    x |= dpp_half_mirror(x);
    x |= dpp_mirror(x);
    return x;
}

// Whole-wavefront reductions: the 16-lane DPP reduction, then two shuffles
// across the rows (xor 16, xor 32); every lane ends with the result.
__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// Maximum of values that are never NaN (compare-select: no canonicalising
// of the operands) and minimum of ints, over the wavefront.
__device__ __forceinline__ float max_cs(float a, float b) { return b > a ? b : a; }
__device__ __forceinline__ float wave_max(float x) {
    x = max_cs(x, as_f(dpp_xor1(as_i(x))));
    x = max_cs(x, as_f(dpp_xor2(as_i(x))));
    x = max_cs(x, as_f(dpp_half_mirror(as_i(x))));
    x = max_cs(x, as_f(dpp_mirror(as_i(x))));
    x = max_cs(x, __shfl_xor(x, 16, kWave));
    x = max_cs(x, __shfl_xor(x, 32, kWave));
    return x;
}
__device__ __forceinline__ int wave_min(int x) {
    x = min(x, dpp_xor1(x));
    x = min(x, dpp_xor2(x));
    x = min(x, dpp_half_mirror(x));
    x = min(x, dpp_mirror(x));
    x = min(x, __shfl_xor(x, 16, kWave));
    x = min(x, __shfl_xor(x, 32, kWave));
    return x;
}

__device__ __forceinline__ void wave_argmax(float& m, int& i) {
    row16_argmax(m, i);
#pragma unroll
    for (int o = 16; o < kWave; o <<= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const int i2 = __shfl_xor(i, o, kWave);
        argmax_combine(m, i, m2, i2);
    }
}

// Inclusive prefix sum over the wavefront with DPP: row shifts by 1, 2, 4, 8
// (zero-filled at the row start) give each 16-lane row its prefix, then the
// row broadcasts of lane 15 and lane 31 carry the earlier rows' totals.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x111, 0xF, 0xF, true));   // row_shr:1
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x112, 0xF, 0xF, true));   // row_shr:2
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x114, 0xF, 0xF, true));   // row_shr:4
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x118, 0xF, 0xF, true));   // row_shr:8
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x142, 0xA, 0xF, false));  // row_bcast:15 into rows 1, 3
    x += as_f(__builtin_amdgcn_update_dpp(0, as_i(x), 0x143, 0xC, 0xF, false));  // row_bcast:31 into rows 2, 3
    return x;
}

// The same inclusive prefix sum over 32-bit integers.
__device__ __forceinline__ int wave_inclusive_scan_int(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// Fold the statistics (m, s, i, bad) of one span of a row into a running
// record a, both relative to c = log2(e) / T:
//   M = max(a.m, m),  S = a.s * 2^((a.m - M) c) + s * 2^((m - M) c),
//   idx = the lower index among spans attaining M.
// Spans with no finite entry (m = -inf) only contribute their bad flag.
__device__ __forceinline__ void stat_fold(StatRec& a, float m, float s, int i, int bad, float c) {
    a.bad |= bad;
    if (m == -INFINITY) return;
    if (a.m == -INFINITY) {
        a.m = m;
        a.s = s;
        a.idx = i;
        return;
    }
    const float M = fmaxf(a.m, m);
    a.s = a.s * exp2f((a.m - M) * c) + s * exp2f((m - M) * c);
    if (m > a.m || (m == a.m && i < a.idx)) a.idx = i;
    a.m = M;
}

// A logit that makes its row unusable (NaN or +inf): the row is marked bad
// and the value takes no part in the statistics.
__device__ __forceinline__ bool stat_bad_value(float z) { return z != z || z == INFINITY; }

// ----------------------------------------------------------------- Philox --
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of
//   (c0,c1,c2,c3) -> (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
// with the key bumped by the Weyl increments between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint32_t hi0 = __umulhi(kPhiloxM0, c.x);
        const uint32_t lo0 = kPhiloxM0 * c.x;
        const uint32_t hi1 = __umulhi(kPhiloxM1, c.z);
        const uint32_t lo1 = kPhiloxM1 * c.z;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// 32-bit word -> [0, 1) on the 24-bit grid (exact in fp32).
__device__ __forceinline__ float uniform24(uint32_t w) {
    return static_cast<float>(w >> 8) * (1.0f / 16777216.0f);
}

// log2(e): exp(x) = exp2(x * log2e).  Weights are computed as
// exp2((z - m) * c) with c = log2(e) / T.
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace sv
