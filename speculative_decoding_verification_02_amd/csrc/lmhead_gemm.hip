// lmhead_gemm.hip -- LM-head contraction of the verify step on gfx950.
//
//   logits[m, v] = sum_h hidden[m, h] * W[v, h]      (m < M = B*(K+1), v < V)
//
// The target's one verify pass reads the LM-head weights once for all K+1
// positions ("speculative-decoding" blog, Verification mechanism; "Speculative
// decoding" course page, Memory-bound, not compute-bound).  With M a handful of
// rows the product is a stream over W (2 bytes per weight, 2*M flops per
// weight), so the small-M kernels are built to keep HBM busy; from a few
// dozen rows up it becomes a dense contraction and the direct-to-LDS kernel
// keeps the matrix cores busy (the LDS-tiled kernel covers hidden sizes that
// are not a multiple of 64).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): the A operand is a
// 16 x 32 tile of W (16 vocabulary rows, 32 hidden columns), the B operand a
// 32 x 16 tile of hiddenᵀ.  Lane l holds A[l % 16][8*(l/16) .. +8) and
// B[8*(l/16) .. +8)[l % 16] -- eight consecutive bf16, one 128-bit load -- and
// receives D[4*(l/16) + i][l % 16], i < 4: four consecutive vocabulary entries
// of one hidden row, stored as one float4.  The contraction does not depend on
// the order of the hidden columns, only on A and B pairing the same column in
// the same (lane group, element) slot, which both loads below guarantee.
#include <limits.h>

#include <type_traits>

#include "sv_common.h"
#include "sv_launch.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8, u32x4{v.x, v.y, v.z, v.w});
}

// 128-bit load of W that bypasses reuse in the caches: every weight is read
// exactly once per verify step.
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0; the fourth
// word sets the 32-bit data format a raw load needs to be valid).  A load
// whose per-lane byte offset is at or past `bytes` returns zero and does not
// access memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, (int)bytes, 0x00020000);
}
constexpr unsigned kOutOfRange = 0xFFFFFFF0u;   // past any resource built here (16 rows of at most 8 KB)

// 16 bytes at byte offset `off` of the resource, non-temporal (the whole
// offset is the range-checked per-lane offset; the scalar offset is 0)
__device__ __forceinline__ u32x4 load_stream_buf(__amdgpu_buffer_rsrc_t rs, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
}

__device__ __forceinline__ void store_row4(float* __restrict__ out, int v, int V, f32x4 acc, bool vec_ok) {
    if (vec_ok && v + 3 < V) {
        *reinterpret_cast<float4*>(out + v) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (v + i < V) out[v + i] = acc[i];
    }
}

// ------------------------------------------------------------ small M ------
// Streaming kernel for M <= 16.  The MFMA operand layout puts 16 vocabulary
// rows in one instruction with only 64 bytes per row; loaded that way, HBM
// streams at ~5.5 TB/s on MI355X, while 256-byte (or longer) runs per row
// stream at ~6.9-7.0 TB/s.  So W is loaded with RPL rows per instruction
// (64/RPL lanes per row, 1024/RPL contiguous bytes per row), written to a
// per-wave LDS buffer, and read back in MFMA layout.  In the buffer the
// 16-byte chunk c of tile row R sits at R*CPR + (c ^ (R % CPR)) (CPR = chunks
// per row per stage): the writes (a run of chunks of one row) and the reads
// (one chunk of 16 rows) both touch distinct banks.
//
// One wave owns tiles of 16 vocabulary rows (grid stride) and runs one
// continuous load pipeline over all of its (tile, stage) steps, P stages deep,
// so loads stay in flight across tile boundaries.  The hidden states (M <= 16
// rows) are staged once per workgroup in LDS.  Each wave's buffer is private:
// LDS operations of one wave complete in order, so no workgroup barrier is
// needed between its writes and reads.
template <int RPL, int P, int THREADS>
struct Skinny {
    static constexpr int kLanesPerRow = 64 / RPL;          // lanes sharing a row in one load
    static constexpr int kCPR = kLanesPerRow;              // 16-byte chunks per row per stage
    static constexpr int kKS = kCPR * 8;                   // k (hidden) elements per stage
    static constexpr int kLoads = 16 / RPL;                // load instructions per stage
    static constexpr int kSteps = kKS / 32;                // MFMA steps per stage
    static constexpr int kWaves = THREADS / 64;
    static constexpr int kBufChunks = 16 * kCPR;           // per-wave LDS buffer, 16-byte chunks
    static size_t lds_bytes(int M, int H) { return (size_t)M * (H + 8) * 2 + (size_t)kWaves * kBufChunks * 16; }
};

template <int RPL, int P, int THREADS>
__global__ __launch_bounds__(THREADS) void lmhead_skinny_bf16(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H, int n_tiles) {
    using S = Skinny<RPL, P, THREADS>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
    const int ld = H + 8;                 // LDS row stride of the hidden states, elements
    const int cpr = H >> 3;
    for (int i = threadIdx.x; i < M * cpr; i += THREADS) {
        const int m = i / cpr, c = i - m * cpr;
        *reinterpret_cast<uint4*>(hs + m * ld + c * 8) =
            *reinterpret_cast<const uint4*>(hidden + (size_t)m * H + c * 8);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4* buf = reinterpret_cast<u32x4*>(smem + (size_t)M * ld * 2) + wave * S::kBufChunks;
    __syncthreads();

    // load-side coordinates: lane -> (row within the load, chunk)
    const int la = lane / S::kLanesPerRow, lc = lane % S::kLanesPerRow;
    // MFMA-side coordinates: lane -> (row r, k group g)
    const int r = lane & 15, g = lane >> 4;
    const bool hrow_ok = r < M;
    const uint16_t* hp = hs + (hrow_ok ? r : 0) * ld;
    const bool vec_ok = (V & 3) == 0;
    const int n_stages = (H + S::kKS - 1) / S::kKS;

    const int wstride = gridDim.x * S::kWaves;
    const int t0 = blockIdx.x * S::kWaves + wave;
    if (t0 >= n_tiles) return;
    const int my_tiles = (n_tiles - t0 + wstride - 1) / wstride;
    const int n_steps = my_tiles * n_stages;

    // issue the loads of step i (tile t0 + (i / n_stages) * wstride, stage i % n_stages)
    auto issue = [&](int i, u32x4 (&dst)[S::kLoads]) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        if (i >= n_steps) {
#pragma unroll
            for (int q = 0; q < S::kLoads; ++q) dst[q] = zero;
            return;
        }
        const int ti = i / n_stages, st = i - ti * n_stages;
        const int v0 = (t0 + ti * wstride) << 4;
        const int k = st * S::kKS + lc * 8;
#pragma unroll
        for (int q = 0; q < S::kLoads; ++q) {
            const int row = min(v0 + q * RPL + la, V - 1);
            dst[q] = (k < H) ? load_stream(W + (size_t)row * H + k) : zero;
        }
    };

    u32x4 pipe[P][S::kLoads];
#pragma unroll
    for (int p = 0; p < P - 1; ++p) issue(p, pipe[p]);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < n_steps; base += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = base + p;
            if (i >= n_steps) break;
            issue(i + P - 1, pipe[(p + P - 1) % P]);
            // transpose step i through the wave's LDS buffer
#pragma unroll
            for (int q = 0; q < S::kLoads; ++q) {
                const int R = q * RPL + la;
                buf[R * S::kCPR + (lc ^ (R % S::kCPR))] = pipe[p][q];
            }
            __builtin_amdgcn_wave_barrier();
            const int ti = i / n_stages, st = i - ti * n_stages;
            const int kb = st * S::kKS;
#pragma unroll
            for (int j = 0; j < S::kSteps; ++j) {
                const int c = j * 4 + g;
                const u32x4 wv = buf[r * S::kCPR + (c ^ (r % S::kCPR))];
                const int k = kb + c * 8;
                u32x4 hv = {0u, 0u, 0u, 0u};
                if (hrow_ok && k < H) hv = *reinterpret_cast<const u32x4*>(hp + k);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(hv), acc, 0, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
            if (st == n_stages - 1) {
                const int v0 = (t0 + ti * wstride) << 4;
                if (hrow_ok) store_row4(logits + (size_t)r * V, v0 + 4 * g, V, acc, vec_ok);
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

// Fallback for M <= 16 with hidden sizes beyond the cooperative kernel's
// register-resident slices (chosen by measurement on MI355X).
constexpr int kSkRPL = 2;
constexpr int kSkP = 3;
constexpr int kSkThreads = 512;
using SkinnyCfg = Skinny<kSkRPL, kSkP, kSkThreads>;

bool skinny_fits(int M, int H) { return M <= 16 && SkinnyCfg::lds_bytes(M, H) <= 160 * 1024; }

template <int RPL, int P, int THREADS>
hipError_t launch_skinny(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H, int num_cus,
                         hipStream_t stream) {
    using S = Skinny<RPL, P, THREADS>;
    auto kern = lmhead_skinny_bf16<RPL, P, THREADS>;
    const int n_tiles = (V + 15) / 16;
    const size_t lds = S::lds_bytes(M, H);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, THREADS, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    // fewest grid-stride iterations the resident waves allow, then just
    // enough waves to cover the tiles in that many iterations
    const long max_waves = (long)num_cus * occ * S::kWaves;
    const long iters = (n_tiles + max_waves - 1) / max_waves;
    const long waves = (n_tiles + iters - 1) / iters;
    const int grid = (int)((waves + S::kWaves - 1) / S::kWaves);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds, stream, hidden, W, logits, M, V, H, n_tiles);
    return hipGetLastError();
}

// ------------------------------------------------- small M, cooperative ----
// A workgroup of NW waves streams one 16-row vocabulary tile at a time (one
// contiguous 16 * H * 2-byte block of W), the hidden dimension split into NW
// slices of SLICE columns, one per wave.  Each wave keeps the B-operand
// fragments of its hidden slice (M <= 16 rows) in registers for the whole
// kernel, transposes its W fragments through a private LDS buffer as above,
// and the NW partial 16 x 16 accumulators of a tile are summed in LDS in wave
// order (fixed order: bitwise reproducible).  Loads run one tile ahead: while
// stage st of tile t is consumed, stage st of the next tile is issued.  Each
// workgroup takes a contiguous range of tiles (sized by the parity of its XCD,
// below), so it streams one contiguous region of W.
//
// The weight loads are buffer loads, exactly kLoads per stage with no branch
// around them: the vector-memory counter of gfx9 counts in issue order, and
// only when the compiler can count the loads issued after the ones a stage
// needs can it wait for those alone (with a load skipped on some path, or a
// store between them, it must wait for every load in flight, and the next
// tile's loads would never overlap this tile's work).  For the same reason
// the loop stores nothing to memory: with STASH the wave that sums a tile
// keeps its logits in LDS, and the workgroup writes its rows out after the
// last tile, one contiguous run per row.  Without STASH (a vocabulary range
// too long for LDS) it stores each tile's logits as it goes.
//
// With STATS (which needs STASH) the kernel also writes softmax statistics
// records (see CoopStats) over each workgroup's vocabulary range.  The draft
// rows' entries are loaded at the start, ahead of W, and written next to the
// logits' rows before the first tile (with the -inf padding of the target
// rows), so after the last tile one barrier leaves the stash complete.  Then
// one 32-lane group per row reduces its row from LDS: max, first index of
// the max, sum of 2^((z - max) c).  No per-entry checks: a NaN or +inf shows
// in the maximum or the sum and marks the record bad.
// Tile ranges of the cooperative kernel.  Each workgroup owns a contiguous
// range of 16-row tiles, sized in proportion to a weight that depends on the
// parity of its index, which is the parity of the XCD it runs on (workgroups
// go to the XCDs round-robin).  Per-workgroup timestamps of this kernel on
// MI355X with equal ranges put the workgroups of the even XCDs at the end of
// their ranges ~15% sooner than those of the odd XCDs (129-135 against
// 150-155 us at B=1, K=5, H=4096, V=128256), the same way on every box
// measured.  The odd ones get the smaller ranges: with weights 1000 : 800 the
// kernel took 149.4 us against 155.7 us with equal ones (920: 153.3, 830:
// 150.9, 770: 151.0, 700: 153.1; one box, medians of 5 x 200 launches).  The
// ranges are a fixed function of (n_tiles, grid), so results are
// reproducible.
#ifndef SV_COOP_WEIGHT_ODD
#define SV_COOP_WEIGHT_ODD 800
#endif
constexpr long kCoopWeightEven = 1000, kCoopWeightOdd = SV_COOP_WEIGHT_ODD;
__host__ __device__ inline long coop_weight_below(int b) {
    return (long)((b + 1) / 2) * kCoopWeightEven + (long)(b / 2) * kCoopWeightOdd;
}
// first tile of workgroup b (b = grid: n_tiles)
__host__ __device__ inline int coop_tile_begin(int b, int n_tiles, int grid) {
    return (int)(((long)n_tiles * coop_weight_below(b)) / coop_weight_below(grid));
}
// the most tiles any workgroup gets: floor(a + x) - floor(a) <= ceil(x)
__host__ __device__ inline int coop_max_tiles(int n_tiles, int grid) {
    const long wmax = kCoopWeightEven > kCoopWeightOdd ? kCoopWeightEven : kCoopWeightOdd;
    const long wt = coop_weight_below(grid);
    return (int)(((long)n_tiles * wmax + wt - 1) / wt);
}

template <int RPL, int MAXST, int NW>
struct Coop {
    static constexpr int kLanesPerRow = 64 / RPL;
    static constexpr int kCPR = kLanesPerRow;
    static constexpr int kKS = kCPR * 8;          // k elements per stage
    static constexpr int kLoads = 16 / RPL;
    static constexpr int kSteps = kKS / 32;
    static constexpr int kSlice = MAXST * kKS;    // k elements per wave
    static constexpr int kBufChunks = 16 * kCPR;
    static constexpr int kThreads = NW * 64;
    static constexpr size_t kLdsBase = (size_t)NW * kBufChunks * 16 + 2 * (size_t)NW * 64 * 16;
    static size_t lds_bytes() { return kLdsBase; }
    // LDS with the stash: M target and n_draft draft rows, each as long as
    // the most columns a workgroup owns (whole tiles of 16) plus 16 floats,
    // which puts the two rows a wavefront reads at once 16 banks apart
    __host__ __device__ static int stash_stride(int n_tiles, int grid) { return coop_max_tiles(n_tiles, grid) * 16 + 16; }
    static size_t lds_bytes_stats(int n_tiles, int grid, int rows) {
        return lds_bytes() + (size_t)rows * stash_stride(n_tiles, grid) * sizeof(float);
    }
    static bool fits(int M, int H) { return M <= 16 && H <= NW * kSlice; }
};

template <int RPL, int MAXST, int NW, bool STATS, bool STASH, int PIPE>
__global__ __launch_bounds__(NW * 64) void lmhead_coop_bf16(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H, int n_tiles, CoopStats cs) {
    using S = Coop<RPL, MAXST, NW>;
    static_assert(STASH || !STATS, "the statistics are taken from the stash");
    static_assert(PIPE >= 1 && MAXST % PIPE == 0, "stages in flight divide the stages of a tile");
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4* buf = reinterpret_cast<u32x4*>(smem) + wave * S::kBufChunks;
    f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)NW * S::kBufChunks * 16);   // [2][NW][64]

    const int la = lane / S::kLanesPerRow, lc = lane % S::kLanesPerRow;
    const int r = lane & 15, g = lane >> 4;
    const int k_lo = wave * S::kSlice;
    const int n_st = max(0, min(MAXST, (H - k_lo + S::kKS - 1) / S::kKS));
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // B operand (hidden rows) for this wave's slice, kept in registers
    u32x4 hreg[MAXST * S::kSteps];
#pragma unroll
    for (int st = 0; st < MAXST; ++st)
#pragma unroll
        for (int j = 0; j < S::kSteps; ++j) {
            const int k = k_lo + st * S::kKS + (j * 4 + g) * 8;
            hreg[st * S::kSteps + j] =
                (r < M && k < H) ? *reinterpret_cast<const u32x4*>(hidden + (size_t)r * H + k) : zero;
        }

    // this workgroup's tiles: a contiguous range [t_begin, t_end), sized by
    // the parity weights above
    const int t_begin = coop_tile_begin(blockIdx.x, n_tiles, gridDim.x);
    const int t_end = coop_tile_begin(blockIdx.x + 1, n_tiles, gridDim.x);

    // The loads of stage st of tile t: the buffer resource spans the tile's
    // rows below V (none for a tile at or past t_end), and the whole offset
    // is the range-checked per-lane offset, so a row past the resource reads
    // zero without touching memory; so does a column past H, whose offset is
    // set beyond any resource.  A stage past this wave's slice (H < NW *
    // SLICE) loads and is not used.
    auto issue = [&](int t, int st, u32x4 (&dst)[S::kLoads]) {
        const int k = k_lo + st * S::kKS + lc * 8;
        const int v0 = t << 4;
        const int rows = t < t_end ? min(16, V - v0) : 0;
        const unsigned vo = k < H ? (unsigned)(la * H + k) * 2u : kOutOfRange;
#pragma unroll
        for (int q = 0; q < S::kLoads; ++q) {
            // load q covers tile rows q * RPL .. q * RPL + RPL - 1: its own
            // resource (scalar registers), so one per-lane offset serves all
            const int rq = min(max(rows - q * RPL, 0), RPL);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(W + (rq ? (size_t)(v0 + q * RPL) * H : 0), (unsigned)(rq * H * 2));
            dst[q] = load_stream_buf(rs, vo);
        }
    };

    // draft row `wave` over this workgroup's vocabulary range: the first
    // kDraftPer * 64 entries are loaded now, ahead of W, and go into the
    // stash before the first tile, so the statistics never hold up the
    // weight stream
    constexpr int kDraftPer = 8;
    const int dcb = t_begin << 4, dce = min(t_end << 4, V);
    float dz[kDraftPer];
    if constexpr (STATS) {
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < cs.n_zero; i += NW * 64) cs.zero[i] = 0;
        if (wave < cs.n_draft) {
            const float* row = cs.draft + (size_t)wave * V;
#pragma unroll
            for (int j = 0; j < kDraftPer; ++j) {
                const int v = dcb + j * 64 + lane;
                dz[j] = v < dce ? row[v] : -INFINITY;
            }
        }
    }

    u32x4 pipe[PIPE][S::kLoads];
#pragma unroll
    for (int st = 0; st < PIPE; ++st) {
        issue(t_begin, st, pipe[st]);
        // issue order kept: the loop waits for stage 0 with the later ones in flight
        __builtin_amdgcn_sched_barrier(0);
    }

    // logits of this workgroup's tiles, [row][column - dcb] (STASH only;
    // sized by the launcher)
    float* stash = reinterpret_cast<float*>(smem + S::kLdsBase);   // [M + n_draft][stash_cols]
    const int stash_cols = S::stash_stride(n_tiles, gridDim.x);
    if constexpr (STATS) {
        // before the tiles: the target rows' columns past this workgroup's
        // tiles (-inf) and the draft rows (row `wave`'s first entries from the
        // registers loaded above, the oldest loads in flight)
        const int span = stash_cols - 16, n = dce - dcb;
        for (int row = wave; row < M; row += NW)
            for (int k = (t_end - t_begin) * 16 + lane; k < span; k += 64) stash[row * stash_cols + k] = -INFINITY;
        for (int d = wave; d < cs.n_draft; d += NW) {
            const float* drow = cs.draft + (size_t)d * V + dcb;
            float* dst = stash + (M + d) * stash_cols;
            for (int k0 = 0; k0 < span; k0 += kDraftPer * 64) {
#pragma unroll
                for (int j = 0; j < kDraftPer; ++j) {
                    const int k = k0 + j * 64 + lane;
                    if (k < span) dst[k] = k >= n ? -INFINITY : (d == wave && k0 == 0 ? dz[j] : drow[k]);
                }
            }
        }
    }

    const bool vec_ok = (V & 3) == 0;
    for (int t = t_begin, it = 0; t < t_end; ++t, ++it) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < MAXST; ++st) {
            const bool live = st < n_st;   // this wave's slice reaches stage st
            if (live) {
                // columns past H are zeroed (their hidden values are zero too,
                // but the bytes loaded there may be anything)
                const bool k_in = k_lo + st * S::kKS + lc * 8 < H;
#pragma unroll
                for (int q = 0; q < S::kLoads; ++q) {
                    const int R = q * RPL + la;
                    buf[R * S::kCPR + (lc ^ (R % S::kCPR))] = k_in ? pipe[st % PIPE][q] : zero;
                }
            }
            __builtin_amdgcn_wave_barrier();
            // the step PIPE stages on: later in this tile, or in the next one
            if (st + PIPE < MAXST) issue(t, st + PIPE, pipe[st % PIPE]);
            else issue(t + 1, st + PIPE - MAXST, pipe[st % PIPE]);
            if (live) {
#pragma unroll
                for (int j = 0; j < S::kSteps; ++j) {
                    const int c = j * 4 + g;
                    const u32x4 wv = buf[r * S::kCPR + (c ^ (r % S::kCPR))];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(hreg[st * S::kSteps + j]),
                                                                  acc, 0, 0, 0);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        // cross-wave sum of the tile's partial accumulators, in wave order
        f32x4* rb = red + (it & 1) * NW * 64;
        rb[wave * 64 + lane] = acc;
        __syncthreads();
        if (wave == (it % NW)) {
            f32x4 s = rb[lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) s += rb[w * 64 + lane];
            const int v0 = (t << 4) + 4 * g;
            if (r < M) {
                if constexpr (STASH) {
                    f32x4 z = s;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (v0 + i >= V) z[i] = -INFINITY;
                    *reinterpret_cast<f32x4*>(stash + r * stash_cols + (v0 - dcb)) = z;
                } else {
                    store_row4(logits + (size_t)r * V, v0, V, s, vec_ok);
                }
            }
        }
    }

    if constexpr (STASH) {
        // this workgroup's logits, one contiguous run per row
        __syncthreads();   // every tile's logits are in the stash
        const int n = dce - dcb;
        for (int row = wave; row < M; row += NW) {
            const float* src = stash + row * stash_cols;
            float* dst = logits + (size_t)row * V + dcb;
            if (vec_ok) {   // dcb and n are multiples of 4 when V is
                for (int k = lane * 4; k < n; k += 256)
                    *reinterpret_cast<f32x4*>(dst + k) = *reinterpret_cast<const f32x4*>(src + k);
            } else {
                for (int k = lane; k < n; k += 64) dst[k] = src[k];
            }
        }
    }

    if constexpr (STATS) {
        // rows reduced over span = stash_cols - 16 columns (the stash is
        // complete after the barrier above)
        const int span = stash_cols - 16;
        // one 32-lane group per row (target rows 0..M-1, then the draft
        // rows); lane l holds columns 4l + 128j + i, ascending in (j, i)
        const int l32 = lane & 31;
        for (int q = wave * 2 + (lane >> 5); q < M + cs.n_draft; q += NW * 2) {
            const float* src = stash + q * stash_cols;
            StatRec a{-INFINITY, 0.f, INT_MAX, 0};
            for (int c0 = 0; c0 < span; c0 += 512) {   // span is a multiple of 16: whole float4s
                float z[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = c0 + 128 * j + 4 * l32;
                    const f32x4 x = k < span ? *reinterpret_cast<const f32x4*>(src + k)
                                             : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[4 * j + i] = x[i];
                }
                float bm = -INFINITY;
                int bi = INT_MAX;
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (z[k] > bm) {
                        bm = z[k];
                        bi = dcb + c0 + 128 * (k / 4) + 4 * l32 + (k % 4);
                    }
                const float mz = bm == -INFINITY ? 0.f : bm;   // (z - max) c: exact at the maximum
                float bs = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) bs += __builtin_amdgcn_exp2f((z[k] - mz) * cs.c);
                stat_fold(a, bm, bs, bi, (bs != bs) | (bm == INFINITY), cs.c);
            }
            // the 32 lanes of the group: DPP within each 16-lane row, then
            // the two rows (lane ^ 16)
            float m = a.m;
            int idx = a.idx;
            row16_argmax(m, idx);
            argmax_combine(m, idx, __shfl_xor(m, 16, kWave), __shfl_xor(idx, 16, kWave));
            float sum = row16_sum(a.m == -INFINITY ? 0.f : a.s * exp2f((a.m - m) * cs.c));
            sum += __shfl_xor(sum, 16, kWave);
            int bad = row16_or(a.bad);
            bad |= __shfl_xor(bad, 16, kWave);
            bad |= (m == INFINITY) | (sum != sum);
            if (l32 == 0) {
                StatRec* out = q < M ? cs.tgt + (size_t)q * gridDim.x : cs.drf + (size_t)(q - M) * gridDim.x;
                out[blockIdx.x] = StatRec{m, sum, idx, bad};
            }
        }
    }
}

// Workgroups of the cooperative kernel: one per compute unit, as many as
// there are tiles at most (and at most kCoopMaxRecs with statistics, so the
// records fit the caller's workspace).
inline int coop_grid(int V, int num_cus, bool stats) {
    const int n_tiles = (V + 15) / 16;
    const int g = min(n_tiles, max(1, num_cus));
    return stats ? min(g, kCoopMaxRecs) : g;
}

// The logits go through the stash whenever it fits in LDS (always with the
// statistics; their launcher checks that first).
template <int RPL, int MAXST, int NW, int PIPE, bool STATS>
hipError_t launch_coop(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H, int num_cus,
                       hipStream_t stream, CoopStats st = CoopStats{}) {
    using S = Coop<RPL, MAXST, NW>;
    const int n_tiles = (V + 15) / 16;
    const int grid = coop_grid(V, num_cus, STATS);
    const size_t lds_stash = S::lds_bytes_stats(n_tiles, grid, M + (STATS ? st.n_draft : 0));
    const bool stash = STATS || lds_stash <= 160 * 1024;
    auto kern = !stash ? lmhead_coop_bf16<RPL, MAXST, NW, false, false, PIPE>
                       : lmhead_coop_bf16<RPL, MAXST, NW, STATS, true, PIPE>;
    const size_t lds = stash ? lds_stash : S::lds_bytes();
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (STATS && (st.n_zero > (1 << 20) || st.n_zero < 0 || st.n_draft < 0 || M > 16 || !st.tgt ||
                  (st.n_draft > 0 && (!st.draft || !st.drf)) || (st.n_zero > 0 && !st.zero)))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(S::kThreads), lds, stream, hidden, W, logits, M, V, H, n_tiles, st);
    return hipGetLastError();
}

// Small-M configurations of the cooperative kernel: up to H = 4096 (measured
// best on MI355X for B = 1, K = 5: 2 rows per load, 2 stages, 8 waves), and
// up to H = 8192 with 4 stages per tile, 2 of them in flight (each wave's
// hidden slice takes 128 registers).
using CoopCfg = Coop<2, 2, 8>;
using CoopWideCfg = Coop<2, 4, 8>;
constexpr int kCoopWidePipe = 2;
// 1: the H <= 4096 configuration, 2: the wide one, 0: neither fits
inline int coop_kind(int M, int H) { return CoopCfg::fits(M, H) ? 1 : CoopWideCfg::fits(M, H) ? 2 : 0; }

// ------------------------------------------------------------ large M ------
// Classic LDS-tiled contraction: a workgroup of 4 waves computes a 128 (vocab)
// x 128 (hidden rows) tile, 64 x 64 per wave as 4 x 4 MFMA blocks, over
// 64-column k-tiles double-buffered in LDS.  LDS rows are 128 bytes (8 chunks
// of 16 bytes); chunk c of row r is stored at c ^ (r & 7) so the 16 rows one
// MFMA operand read touches spread over the banks.
constexpr int kTileN = 128;   // vocabulary rows per workgroup
constexpr int kTileM = 128;   // hidden rows per workgroup
constexpr int kTileK = 64;    // columns per k-tile
constexpr int kTiledThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ __launch_bounds__(kTiledThreads) void lmhead_tiled_bf16(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H, int tiles_n, int tiles_m) {
    __shared__ uint4 lw[2][kTileN * 8];
    __shared__ uint4 lh[2][kTileM * 8];

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give
    // each XCD a contiguous run of tiles that share vocabulary rows of W so
    // the W tile is fetched into that XCD's L2 once.
    const int total = tiles_n * tiles_m;
    const int per_xcd = (total + 7) / 8;
    const int seq = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (seq >= total) return;
    const int tn = seq / tiles_m, tm = seq - tn * tiles_m;
    const int v0 = tn * kTileN, m0 = tm * kTileM;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;

    // global -> LDS assignment: 1024 chunks per operand tile, 4 per thread
    uint4 rw[4], rh[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * kTiledThreads;
            const int row = idx >> 3, ch = idx & 7;
            const int k = k0 + ch * 8;
            const int vr = v0 + row, mr = m0 + row;
            rw[j] = (vr < V && k < H) ? *reinterpret_cast<const uint4*>(W + (size_t)vr * H + k)
                                      : make_uint4(0, 0, 0, 0);
            rh[j] = (mr < M && k < H) ? *reinterpret_cast<const uint4*>(hidden + (size_t)mr * H + k)
                                      : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * kTiledThreads;
            const int row = idx >> 3, ch = idx & 7;
            lw[buf][swz(row, ch)] = rw[j];
            lh[buf][swz(row, ch)] = rh[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (H + kTileK - 1) / kTileK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kTileK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 4 + g;
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) fa[a] = as_bf16x8(lw[buf][swz(wn + a * 16 + r, ch)]);
#pragma unroll
            for (int b = 0; b < 4; ++b) fb[b] = as_bf16x8(lh[buf][swz(wm + b * 16 + r, ch)]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    const bool vec_ok = (V & 3) == 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = m0 + wm + b * 16 + r;
        if (m >= M) continue;
        float* out = logits + (size_t)m * V;
#pragma unroll
        for (int a = 0; a < 4; ++a) store_row4(out, v0 + wn + a * 16 + 4 * g, V, acc[a][b], vec_ok);
    }
}

// ------------------------------------------------------------- big M -----
// Dense contraction for M from a few dozen rows up (MFMA-bound at large M).
// A workgroup of NW = 4 or 8 waves (one or two per SIMD) owns a 256 (vocab) x
// BM (hidden rows) tile; each wave a 32*NA x 32*NB part as NA x NB blocks of
// v_mfma_f32_32x32x16_bf16 (16*NA*NB fp32 accumulators per lane), the waves
// laid out 8/NA along the vocabulary and NW*NA/8 along the rows, so
// BM = 32*NB*NW*NA/8.  With two waves per SIMD each holds half the
// accumulators and one wave's MFMAs cover the other's waits.  On MI355X the
// 32x32x16 form issues at about twice the rate of 16x16x32 (measured ~2.0 vs
// ~0.8 PFLOP/s at one wave per SIMD), so the dense path uses it.  Operand layout: lane l holds A[l % 32][8*(l/32) .. +8) (W
// rows) and B[8*(l/32) .. +8)[l % 32] (hidden rows) and receives
// D[8*(i/4) + 4*(l/32) + i%4][l % 32], i < 16: four runs of four consecutive
// vocabulary entries of one hidden row.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4, no
// register staging) into a ring of SLOTS k-slices of BK columns (256 W rows
// then BM hidden rows, BK*2 bytes per row).  A DMA instruction writes 1 KB of
// LDS in lane order; each lane picks the global chunk that belongs at its LDS
// position, so the slice lands swizzled (Big::pos), which spreads any 16
// consecutive rows read at one chunk over the 16 bank groups.  The loads that
// refill a slot are issued one per MFMA, and each k-step's fragments are read
// from LDS during the previous k-step's MFMAs (across slice boundaries too),
// so neither a full load queue nor an LDS read stalls the matrix pipe.
// Synchronisation is explicit: a wait on the wave's own outstanding loads
// (vmcnt), then one barrier per slice.  Where several row tiles share each
// vocabulary tile (M > 320), the hidden rows are the operand fetched again
// from the last-level cache in every round, so they get a ring of three
// slots of their own beside the weights' two (160 KB at 256 rows): the waves
// that load hidden rows run one slice further ahead.  Tiles are ordered XCD-aware, so the
// M-tiles of one vocabulary tile share an L2.
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBigBN = 256;

// Geometry of one k-slice of BK columns: 256 W rows then BM hidden rows, CPR
// 16-byte chunks per row; a DMA instruction fills RPI rows (1 KB).
template <int BK, int SLOTS, int NA, int NB, int NW = 4>
struct Big {
    static constexpr int kThreads = NW * 64;
    static constexpr int kWN = 8 / NA;                  // waves along the vocabulary
    static constexpr int kWM = NW / kWN;                // waves along the hidden rows
    static constexpr int kBM = kWM * NB * 32;
    static constexpr int kCPR = BK / 8;
    static constexpr int kRPI = 64 / kCPR;
    static constexpr int kSliceChunks = (kBigBN + kBM) * kCPR;
    static constexpr int kLoads = kSliceChunks / 64 / NW;                   // DMA per lane per slice
    static constexpr int kWLoads = kBigBN * kCPR / 64;                      // DMA blocks holding W rows
    static constexpr int kSteps = BK / 16;                                  // MFMA k-steps per slice
    static constexpr size_t kLds = (size_t)SLOTS * kSliceChunks * 16;
    static_assert(kSliceChunks % kThreads == 0, "slice must split evenly over the lanes");
    static_assert(kWN * NA == 8 && kWN * kWM == NW, "wave layout must tile 256 x BM");
    static_assert(kLoads <= kSteps * NA * NB, "every load must find an MFMA to ride on");
    static_assert(kLds <= 160 * 1024, "LDS ring exceeds the 160 KB of a CU");
    // chunk c of row r sits at r*CPR + (c ^ f(r)), f(r) = (r / (16/CPR)) % CPR:
    // 16 consecutive rows read at one chunk fall in 16 distinct bank groups
    static __device__ __forceinline__ int pos(int row, int chunk) {
        return row * kCPR + (chunk ^ ((row / (16 / kCPR)) % kCPR));
    }
};

// the wave's index as a scalar (a non-template wrapper: inside a kernel
// template the builtin would drop the host-side launch stub)
__device__ __forceinline__ int wave_index_uniform(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most `after` slices' loads (of L each) are outstanding
template <int L, int MAXAFTER>
__device__ __forceinline__ void wait_slices(int after) {
    if constexpr (MAXAFTER >= 3) {
        if (after >= 3) { wait_vmcnt<3 * L>(); return; }
    }
    if constexpr (MAXAFTER >= 2) {
        if (after >= 2) { wait_vmcnt<2 * L>(); return; }
    }
    if constexpr (MAXAFTER >= 1) {
        if (after >= 1) { wait_vmcnt<L>(); return; }
    }
    wait_vmcnt<0>();
}

// loop phase of the direct-to-LDS kernel: which of a slice's loads go out
template <bool MAIN, bool NEXT>
struct BigPhase {
    static constexpr bool kMain = MAIN, kNext = NEXT;
};

// Work items of the direct-to-LDS kernel per XCD: the first item of XCD x of
// n_items (x = 8: n_items).  A CU runs one workgroup at a time, so an XCD
// (32 CUs) with n items runs ceil(n / 32) rounds.  The count of the even
// XCDs is the larger share at weights 103 : 100 (their tiles ran 2-4%
// faster than the odd XCDs' in per-workgroup timestamps at B=256 and B=512),
// but no more than the rounds an equal split needs allow, so no XCD runs a
// round more than it would with equal counts.  (Whole vocabulary tiles per
// XCD left 675 items on two XCDs at B=256, K=8, V=152064: a 22nd round of 3
// tiles.  Contiguous items: 4850 -> 4717 us there.  Letting the even XCDs
// run one partial round more, so that the odd ones run fewer tiles, measured
// no better at B=512.)
__host__ __device__ inline long big_items_begin(int x, long n_items) {
    const long per = (n_items + 7) / 8;                    // most items of an equal split
    const long cap = ((per + 31) / 32) * 32;               // in the rounds that split needs
    long even = (n_items * 103 + 4 * 203 - 1) / (4 * 203); // share at 103 : 100, rounded up
    even = even < cap ? even : cap;
    even = even < n_items / 4 ? even : n_items / 4;         // the four even XCDs take at most all
    even = even > n_items / 8 ? even : n_items / 8;         // never below the equal share
    const long rest = n_items - 4 * even;                   // for the four odd XCDs
    const long evens_below = (x + 1) / 2, odds_below = x / 2;
    return evens_below * even + (odds_below * rest) / 4;
}

// With STATS, the workgroup also writes the softmax statistics of each of its
// hidden rows over its 256 vocabulary columns: stats[m * tiles_n + tn].
template <int BK, int SLOTS, int NA, int NB, bool STATS, int NW, int HS>
__global__ __launch_bounds__(NW * 64, 1) void lmhead_big_bf16(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H, int tiles_n, int tiles_m, StatRec* __restrict__ stats, float c) {
    using G = Big<BK, SLOTS, NA, NB, NW>;
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4* lds = reinterpret_cast<u32x4*>(smem);   // [slot][W rows 0..255 | hidden rows 0..BM-1][CPR chunks]

    // Workgroups go to the XCDs round-robin.  The work items (vocabulary
    // tile, hidden-row tile) are ordered vocabulary-major and XCD x owns the
    // contiguous range of them that big_items_begin gives it, so the
    // workgroups running together on an XCD share operand slices through its
    // L2 (all row tiles of a vocabulary tile run next to each other).
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const long i_lo = big_items_begin(xcd, (long)tiles_n * tiles_m), i_hi = big_items_begin(xcd + 1, (long)tiles_n * tiles_m);
    if (local >= i_hi - i_lo) return;
    const long item = i_lo + local;
    const int tn = (int)(item / tiles_m), tm = (int)(item - (long)tn * tiles_m);
    const int v0 = tn * kBigBN, m0 = tm * G::kBM;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int wn = (wave % G::kWN) * (32 * NA), wm = (wave / G::kWN) * (32 * NB);

    // DMA source of each of this lane's loads: instruction q of this wave fills
    // 1 KB block bi = wave * kLoads + q of the slice (RPI rows; the first
    // kWLoads blocks hold W rows, the rest hidden rows); the lane's position in
    // the block fixes its row and, through the swizzle, its chunk.  Sources are
    // kept as 32-bit element offsets (the launcher checks V*H and M*H fit) to
    // leave registers for the accumulators.
    const int wave_u = wave_index_uniform(tid);
    uint32_t off[G::kLoads];
#pragma unroll
    for (int q = 0; q < G::kLoads; ++q) {
        const int bi = wave_u * G::kLoads + q;
        const int row = bi * G::kRPI + lane / G::kCPR;   // row of the slice, W rows first
        const int chunk = (lane % G::kCPR) ^ ((row / (16 / G::kCPR)) % G::kCPR);
        if (bi < G::kWLoads) {
            const int vr = min(v0 + row, V - 1);          // rows past V: read a valid row, outputs dropped
            off[q] = (uint32_t)vr * (uint32_t)H + chunk * 8;
        } else {
            const int mr = min(m0 + row - kBigBN, M - 1);
            off[q] = (uint32_t)mr * (uint32_t)H + chunk * 8;
        }
    }
    auto src = [&](int q, int kt) {
        const uint16_t* base = wave_u * G::kLoads + q < G::kWLoads ? W : hidden;
        return base + off[q] + (size_t)kt * BK;
    };

    f32x16 acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    // Pipeline.  The slice barrier sits one k-step early: before the last
    // k-step of slice kt every wave holds that step's fragments in registers,
    // so after the barrier slice kt+1 is visible to all and slot kt is free.
    // Each wave then reads slice kt+1's first fragments while it multiplies
    // the last k-step of slice kt, and no wave leaves a barrier with nothing
    // to multiply.  The loads issued between two barriers (a window) refill
    // the slot freed by the first of them and ride on the window's MFMAs,
    // window-local index q = 0, 1, ...  Within a k-step the order is pinned:
    // one MFMA, the next step's fragment reads, then the remaining MFMAs each
    // followed by at most one load.  The slice body has no branches (which
    // loads go out is a compile-time property of the loop phase), so the
    // compiler's waits on fragment reads stay exact.
    const int nk = H / BK;
    constexpr int kLast = G::kSteps - 1;
    constexpr int kPerStep = NA * NB;
    // Rings: HS == 0, one ring of SLOTS slices [W rows | hidden rows]; HS > 0,
    // the W rows in a ring of SLOTS slots and the hidden rows in a ring of HS
    // slots of their own.  Waves 0 .. kWWaves-1 load only W blocks and the
    // others only hidden blocks, so each role runs its own prefetch depth.
    constexpr int kWChunks = kBigBN * G::kCPR, kHChunks = G::kBM * G::kCPR;
    constexpr size_t kPartBytes = (size_t)G::kWN * G::kBM * sizeof(StatRec);   // statistics exchange (STATS)
    constexpr int kWWaves = G::kWLoads / G::kLoads;
    static_assert(HS == 0 || (G::kWLoads % G::kLoads == 0 && kWWaves < NW), "roles split by wave");
    auto wslot = [&](int slice) -> u32x4* {
        return HS ? lds + (slice % SLOTS) * kWChunks : lds + (slice % SLOTS) * G::kSliceChunks;
    };
    auto hslot = [&](int slice) -> u32x4* {
        return HS ? lds + SLOTS * kWChunks + (slice % (HS ? HS : 1)) * kHChunks
                  : lds + (slice % SLOTS) * G::kSliceChunks + kWChunks;
    };
    auto dma = [&](int q, int slice) {
        const int bi = wave_u * G::kLoads + q;
        u32x4* dst = HS ? (bi < G::kWLoads ? wslot(slice) + bi * 64 : hslot(slice) + (bi - G::kWLoads) * 64)
                        : lds + (slice % SLOTS) * G::kSliceChunks + bi * 64;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src(q, slice)),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    };
    // fragments of k-step ks of a slice: the NA weight ones, and hidden one b
    auto frag_a = [&](int slice, int ks, bf16x8 (&xa)[NA]) {
        const u32x4* lw = wslot(slice);
        const int ch = ks * 2 + h;
#pragma unroll
        for (int a = 0; a < NA; ++a) xa[a] = as_bf16x8(lw[G::pos(wn + a * 32 + r, ch)]);
    };
    auto frag_b = [&](int slice, int ks, int b) {
        return as_bf16x8(hslot(slice)[G::pos(wm + b * 32 + r, ks * 2 + h)]);
    };

    // The weight fragments are double-buffered (every product of a k-step
    // uses them); the hidden ones are not: a k-step runs its products
    // b-major, hidden fragment b is dead after its NA products, and the next
    // k-step's fragment b is read into its registers right then.  (With both
    // double-buffered the 320-row tile spilled registers, and each reload was
    // a vector-memory load the loop had to wait for behind every DMA.)
    bf16x8 fa[2][NA], fb[NB];
    // prologue and loop of a wave whose loads run SL slices deep
    auto run = [&](auto sl_tag) {
        constexpr int SL = decltype(sl_tag)::value;
#pragma unroll
        for (int p = 0; p < SL - 1; ++p) {
            if (p >= nk) break;
#pragma unroll
            for (int q = 0; q < G::kLoads; ++q) dma(q, p);
        }
        // this lane's loads of slice 0 have landed once at most the slices
        // issued after it are outstanding; after the barrier everyone's have
        wait_slices<G::kLoads, SL - 2>(min(SL - 2, nk - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        frag_a(0, 0, fa[0]);
#pragma unroll
        for (int b = 0; b < NB; ++b) fb[b] = frag_b(0, 0, b);
        // the loads of slice SL-1 that would ride on the last k-step of the
        // (absent) slice before slice 0; that slot has not been used yet
        if (SL - 1 < nk) {
#pragma unroll
            for (int q = 0; q < G::kLoads && q < kPerStep; ++q) dma(q, SL - 1);
        }

        // MAIN: this window's loads (slice kt+SL-1) go out; NEXT: the next
        // window's first loads (slice kt+SL) go out after the early barrier
        auto slice = [&](int kt, auto phase) {
            constexpr bool MAIN = decltype(phase)::kMain, NEXT = decltype(phase)::kNext;
#pragma unroll
            for (int ks = 0; ks < G::kSteps; ++ks) {
                const int cur = ks & 1;
                if (ks == kLast) {
                    // this wave's reads of slot kt have completed and its loads
                    // of slice kt+1 have landed (at most the slices issued after
                    // it outstanding); after the barrier the same holds for
                    // everyone.  On the last slice this only costs one barrier
                    // and reads of a stale slot that nothing uses.  The
                    // scheduling fences keep every MFMA of the previous k-step
                    // ahead of the waits.
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
                    wait_slices<G::kLoads, SL - 2>(min(SL - 2, nk - 2 - kt));
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                }
                // the next k-step: the next one of this slice, or the first of
                // slice kt+1 (visible after the barrier above)
                const int nsl = ks < kLast ? kt : kt + 1, nks = ks < kLast ? ks + 1 : 0;
#pragma unroll
                for (int i = 0; i < kPerStep; ++i) {
                    const int b = i / NA, a = i % NA;
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[b], acc[a][b], 0, 0, 0);
                    if (i == 0) frag_a(nsl, nks, fa[cur ^ 1]);
                    if (a == NA - 1) fb[b] = frag_b(nsl, nks, b);
                    const int q = ks == kLast ? i : kPerStep * (ks + 1) + i;
                    if (q < G::kLoads) {
                        if (ks == kLast && NEXT) dma(q, kt + SL);
                        if (ks < kLast && MAIN) dma(q, kt + SL - 1);
                    }
                }
                // pin the order: each MFMA, then the fragment reads it frees
                // (after the first, the next step's weight fragments), then
                // the load that rides on it
#pragma unroll
                for (int i = 0; i < kPerStep; ++i) {
                    const int a = i % NA;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);   // LDS reads (weights)
                    if (a == NA - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read (hidden)
                    const int q = ks == kLast ? i : kPerStep * (ks + 1) + i;
                    if (q < G::kLoads && ((ks == kLast && NEXT) || (ks < kLast && MAIN)))
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // memory load
                }
            }
        };
        int kt = 0;
        for (; kt + SL < nk; ++kt) slice(kt, BigPhase<true, true>{});
        if (kt + SL - 1 < nk) slice(kt++, BigPhase<true, false>{});
        for (; kt < nk; ++kt) slice(kt, BigPhase<false, false>{});
    };
    if constexpr (HS > 0) {
        if (wave_u < kWWaves) run(std::integral_constant<int, SLOTS>{});
        else run(std::integral_constant<int, HS>{});
    } else {
        run(std::integral_constant<int, SLOTS>{});
    }

    // Logits out through LDS (the ring is free once every wave is past its
    // last slice), one row block at a time: the kWM * 32 rows that all waves'
    // block b covers land in LDS as whole 256-entry rows, then each store
    // instruction writes one row's 1 KB run.  Stored straight from the MFMA
    // layout, an instruction wrote 16-byte pieces of 32 rows.
    const bool vec_ok = (V & 3) == 0;
    auto store_logits = [&](auto off_tag) {
        constexpr size_t kOff = decltype(off_tag)::value;   // bytes of LDS in use below the staging rows
        constexpr int kRowF = kBigBN + 4;                  // floats per staged row (16-byte pad)
        constexpr int kRows = G::kWM * 32;                 // rows per row block
        float* stg = reinterpret_cast<float*>(smem + kOff);
        const int lr0 = (wave / G::kWN) * 32;              // this wave's first staged row
        const bool full_v = vec_ok && v0 + kBigBN <= V;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            __syncthreads();
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v4 = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                                      acc[a][b][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(stg + (lr0 + r) * kRowF + wn + a * 32 + 8 * q + 4 * h) = v4;
                }
            __syncthreads();
            for (int lr = wave; lr < kRows; lr += NW) {
                const int m = m0 + (lr / 32) * (32 * NB) + 32 * b + (lr % 32);
                if (m >= M) continue;
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(stg + lr * kRowF + 4 * lane);
                float* out = logits + (size_t)m * V + v0;
                if (full_v) {
                    *reinterpret_cast<f32x4*>(out + 4 * lane) = v4;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (v0 + 4 * lane + e < V) out[4 * lane + e] = v4[e];
                }
            }
        }
    };

    if constexpr (STATS) {
        // per hidden row: this lane's 16*NA entries (ascending vocabulary
        // index), then its partner lane^32 (the other half of the columns),
        // then the kWN waves side by side along the vocabulary, in order,
        // through the LDS ring (free once every wave is past its last slice);
        // the logits follow, staged above these records.
        // No per-entry checks: NaN never wins the maximum, and a NaN or +inf
        // shows in the maximum or the sum, which marks the row bad; entries
        // past V are masked only in the last vocabulary tile.
        __syncthreads();
        StatRec* part = reinterpret_cast<StatRec*>(smem);   // [kWN][BM]
        // This loop runs after the main loop with the matrix cores idle, so
        // its vector instructions count: per entry a compare and two selects
        // for the maximum and its index (NaN never compares greater), then
        // subtract, multiply, exp and add for the sum.  The mask past V is a separate copy of
        // the loop, taken by the last vocabulary tile only.
        const auto fold_rows = [&](auto masked) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float mx = -INFINITY;
                int mi = INT_MAX;
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int v = v0 + wn + a * 32 + 8 * (i / 4) + 4 * h + (i % 4);
                        const float z = (!masked || v < V) ? acc[a][b][i] : -INFINITY;
                        if (z > mx) {   // ascending index within a lane: strict > keeps the first
                            mx = z;
                            mi = v;
                        }
                    }
                argmax_combine(mx, mi, __shfl_xor(mx, 32, kWave), __shfl_xor(mi, 32, kWave));
                // (z - max) c, not z c - max c: the second rounds max c, an
                // absolute error in every exponent that grows as T shrinks
                const float mz = mx == -INFINITY ? 0.f : mx;
                float sum = 0.f;
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int v = v0 + wn + a * 32 + 8 * (i / 4) + 4 * h + (i % 4);
                        const float z = (!masked || v < V) ? acc[a][b][i] : -INFINITY;
                        sum += __builtin_amdgcn_exp2f((z - mz) * c);
                    }
                sum += __shfl_xor(sum, 32, kWave);
                const int bad = mx == INFINITY || sum != sum;
                if (h == 0) part[(wave % G::kWN) * G::kBM + wm + b * 32 + r] = StatRec{mx, sum, mi, bad};
            }
        };
        if (v0 + wn + 32 * NA <= V)
            fold_rows(std::false_type{});
        else
            fold_rows(std::true_type{});
        __syncthreads();
        for (int row = threadIdx.x; row < G::kBM; row += G::kThreads) {
            if (m0 + row >= M) continue;
            StatRec t{-INFINITY, 0.f, INT_MAX, 0};
#pragma unroll
            for (int w = 0; w < G::kWN; ++w) {
                const StatRec x = part[w * G::kBM + row];
                stat_fold(t, x.bad ? -INFINITY : x.m, x.s, x.idx, x.bad, c);
            }
            stats[(size_t)(m0 + row) * tiles_n + tn] = t;
        }
        store_logits(std::integral_constant<size_t, kPartBytes>{});   // staged above the records
    }

    if constexpr (!STATS) store_logits(std::integral_constant<size_t, 0>{});
}

template <int BK, int SLOTS, int NA, int NB, bool STATS, int NW = 4, int HS = 0>
hipError_t launch_big_cfg(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                          hipStream_t stream, StatRec* stats = nullptr, float c = 0.f) {
    using G = Big<BK, SLOTS, NA, NB, NW>;
    constexpr size_t kLds = HS ? (size_t)(SLOTS * kBigBN + HS * G::kBM) * G::kCPR * 16 : G::kLds;
    static_assert(kLds <= 160 * 1024, "rings exceed the 160 KB of a CU");
    static_assert(!STATS || (size_t)G::kWN * G::kBM * sizeof(StatRec) <= kLds, "statistics exchange fits the ring");
    static_assert((STATS ? (size_t)G::kWN * G::kBM * sizeof(StatRec) : 0) + (size_t)G::kWM * 32 * (kBigBN + 4) * 4 <=
                      kLds,
                  "a staged row block of logits fits the ring");
    auto kern = lmhead_big_bf16<BK, SLOTS, NA, NB, STATS, NW, HS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    const int tiles_n = (V + kBigBN - 1) / kBigBN;
    const int tiles_m = (M + G::kBM - 1) / G::kBM;
    long most = 0;                           // most items any XCD owns
    for (int x = 0; x < 8; ++x) {
        const long n = (long)tiles_n * tiles_m;
        most = std::max(most, big_items_begin(x + 1, n) - big_items_begin(x, n));
    }
    const long grid = 8 * most;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::kThreads), kLds, stream, hidden, W, logits, M, V, H,
                       tiles_n, tiles_m, stats, c);
    return hipGetLastError();
}

// Configurations the library launches, all with whole 128-byte rows per
// slice.  The tile height follows M so that little of the tile is padding,
// and from 65 rows up the tiles run with 8 waves (two per SIMD, each with
// half the accumulators), so one wave's MFMAs cover the other's waits.
// Measured on MI355X (us per GEMM, H = 4096, V = 128256 unless noted; taken
// before the loop's order was pinned, which made the large tiles 3-7% faster):
//   M = 40:  183 (64-row tile, 4 waves) vs 246 for the 128 x 128 tiled kernel
//   M = 128: 208 (128 rows, 8 waves) vs 214 (4 waves)
//   M = 150: 230 (160 rows, 4 waves, 3 slots) vs 255 (192 rows, 8 waves)
//   M = 192: 264 (192 rows, 8 waves) vs 269 (4 waves)
//   M = 256: 285 (256 rows, 8 waves) vs 301-313 (4 waves)
//   M = 320: 333-341 (one 320-row tile, 8 waves) vs 388 (2 x 160, 4 waves)
//   M = 640: 654 (2 x 320) vs 740-764 (3 x 256)
//   M = 2304, H = 8192, V = 152064: 5.25 ms (256 rows, 8 waves) vs 5.5-5.9
//   M = 2048, H = 5120, V = 262144: 5.23-5.32 ms vs 5.5
// Above 320 rows the tile is 256 or 320 rows, whichever gives the smaller
// sum of per-tile times (measured 285 and 339 us per 256-/320-row tile here);
// the 256-row tiles there use the split rings: M = 2048, H = 5120, V = 262144
// 5.01 vs 5.18 ms and M = 2304, H = 8192 5.11 vs 5.17 ms (interleaved, one
// box), M = 512 unchanged.
constexpr int kBigBK = 64;
constexpr int kBigMinM = 17;

// sources are 32-bit element offsets into W and hidden
bool big_fits(int M, int V, int H) {
    return M >= kBigMinM && H % kBigBK == 0 && (uint64_t)V * H < (1ull << 32) && (uint64_t)M * H < (1ull << 32);
}

template <bool STATS>
hipError_t launch_big(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                      hipStream_t stream, StatRec* stats, float c) {
    if (M <= 64) return launch_big_cfg<kBigBK, 3, 4, 1, STATS, 4>(hidden, W, logits, M, V, H, stream, stats, c);
    if (M <= 128) return launch_big_cfg<kBigBK, 3, 2, 2, STATS, 8>(hidden, W, logits, M, V, H, stream, stats, c);
    if (M <= 160) return launch_big_cfg<kBigBK, 3, 2, 5, STATS, 4>(hidden, W, logits, M, V, H, stream, stats, c);
    if (M <= 192) return launch_big_cfg<kBigBK, 2, 2, 3, STATS, 8>(hidden, W, logits, M, V, H, stream, stats, c);
    if (M <= 256) return launch_big_cfg<kBigBK, 2, 2, 4, STATS, 8>(hidden, W, logits, M, V, H, stream, stats, c);
    const long cost256 = (long)((M + 255) / 256) * 285, cost320 = (long)((M + 319) / 320) * 339;
    if (cost320 < cost256)
        return launch_big_cfg<kBigBK, 2, 2, 5, STATS, 8>(hidden, W, logits, M, V, H, stream, stats, c);
    return launch_big_cfg<kBigBK, 2, 2, 4, STATS, 8, 3>(hidden, W, logits, M, V, H, stream, stats, c);
}

// ------------------------------------------------------------------ fp32 ---
// Plain fp32 FMA contraction for fp32 weights (small workloads): one wave per
// vocabulary row, lanes split the hidden dimension in float4 steps, a wave
// reduction per hidden row.
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void lmhead_f32(
    const float* __restrict__ hidden, const float* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H) {
    const int lane = threadIdx.x & 63;
    const int v = blockIdx.x * (kF32Threads / 64) + (threadIdx.x >> 6);
    if (v >= V) return;
    const float* wr = W + (size_t)v * H;
    for (int m = 0; m < M; ++m) {
        const float* hr = hidden + (size_t)m * H;
        float s = 0.f;
        for (int k = lane * 4; k < H; k += 256) {
            const float4 a = *reinterpret_cast<const float4*>(wr + k);
            const float4 b = *reinterpret_cast<const float4*>(hr + k);
            s = fmaf(a.x, b.x, s);
            s = fmaf(a.y, b.y, s);
            s = fmaf(a.z, b.z, s);
            s = fmaf(a.w, b.w, s);
        }
        s = wave_sum(s);
        if (lane == 0) logits[(size_t)m * V + v] = s;
    }
}

// ------------------------------------------------------------ launchers ----

int lmhead_coop_records(int M, int V, int H, int n_draft, int num_cus) {
    if (!coop_kind(M, H) || n_draft < 0) return 0;
    const int grid = coop_grid(V, num_cus, true);
    // both configurations have the same LDS layout
    return CoopCfg::lds_bytes_stats((V + 15) / 16, grid, M + n_draft) <= 160 * 1024 ? grid : 0;
}

hipError_t launch_lmhead_coop_stats(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                                    int num_cus, hipStream_t stream, const CoopStats& st) {
    switch (coop_kind(M, H)) {
    case 1: return launch_coop<2, 2, 8, 2, true>(hidden, W, logits, M, V, H, num_cus, stream, st);
    case 2: return launch_coop<2, 4, 8, kCoopWidePipe, true>(hidden, W, logits, M, V, H, num_cus, stream, st);
    default: return hipErrorInvalidValue;
    }
}

int lmhead_big_records(int M, int V, int H) {
    return !coop_kind(M, H) && big_fits(M, V, H) ? (V + kBigBN - 1) / kBigBN : 0;
}

hipError_t launch_lmhead_bf16(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                              int num_cus, hipStream_t stream, StatRec* stats, float c, int* n_rec) {
    if (n_rec) *n_rec = 0;
    if (CoopCfg::fits(M, H)) return launch_coop<2, 2, 8, 2, false>(hidden, W, logits, M, V, H, num_cus, stream);
    if (CoopWideCfg::fits(M, H))
        return launch_coop<2, 4, 8, kCoopWidePipe, false>(hidden, W, logits, M, V, H, num_cus, stream);
    if (big_fits(M, V, H)) {
        if (stats) {
            if (n_rec) *n_rec = (V + kBigBN - 1) / kBigBN;
            return launch_big<true>(hidden, W, logits, M, V, H, stream, stats, c);
        }
        return launch_big<false>(hidden, W, logits, M, V, H, stream, nullptr, 0.f);
    }
    if (skinny_fits(M, H)) return launch_skinny<kSkRPL, kSkP, kSkThreads>(hidden, W, logits, M, V, H, num_cus, stream);
    const int tiles_n = (V + kTileN - 1) / kTileN;
    const int tiles_m = (M + kTileM - 1) / kTileM;
    const int total = tiles_n * tiles_m;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL(lmhead_tiled_bf16, dim3(grid), dim3(kTiledThreads), 0, stream, hidden, W, logits, M, V, H,
                       tiles_n, tiles_m);
    return hipGetLastError();
}

hipError_t launch_lmhead_f32(const float* hidden, const float* W, float* logits, int M, int V, int H,
                             hipStream_t stream) {
    const int grid = (V + (kF32Threads / 64) - 1) / (kF32Threads / 64);
    hipLaunchKernelGGL(lmhead_f32, dim3(grid), dim3(kF32Threads), 0, stream, hidden, W, logits, M, V, H);
    return hipGetLastError();
}

}  // namespace sv
