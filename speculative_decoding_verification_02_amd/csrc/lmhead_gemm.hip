// lmhead_gemm.hip -- LM-head contraction of the verify step on gfx950.
//
//   logits[m, v] = sum_h hidden[m, h] * W[v, h]      (m < M = B*(K+1), v < V)
//
// The target's one verify pass reads the LM-head weights once for all K+1
// positions ("speculative-decoding" blog, Verification mechanism; "Speculative
// decoding" course page, Memory-bound, not compute-bound).  With M a handful of
// rows the product is a stream over W (2 bytes per weight, 2*M flops per
// weight), so the small-M kernel is built to keep HBM busy; with M in the
// hundreds or thousands it becomes a dense contraction and the tiled kernel
// keeps the matrix cores busy.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): the A operand is a
// 16 x 32 tile of W (16 vocabulary rows, 32 hidden columns), the B operand a
// 32 x 16 tile of hiddenᵀ.  Lane l holds A[l % 16][8*(l/16) .. +8) and
// B[8*(l/16) .. +8)[l % 16] -- eight consecutive bf16, one 128-bit load -- and
// receives D[4*(l/16) + i][l % 16], i < 4: four consecutive vocabulary entries
// of one hidden row, stored as one float4.  The contraction does not depend on
// the order of the hidden columns, only on A and B pairing the same column in
// the same (lane group, element) slot, which both loads below guarantee.
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
// One wave owns a tile of 16 vocabulary rows over the whole hidden dimension
// and walks the tiles of the vocabulary with a grid stride.  The hidden states
// (M <= 16 rows) are staged once per workgroup in LDS; W streams from HBM with
// one 128-bit load per lane per 32 columns, kU loads in flight per stage and
// two stages in registers.
constexpr int kSkinnyThreads = 512;
constexpr int kSkinnyU = 8;   // 32-column steps per pipeline stage

__global__ __launch_bounds__(kSkinnyThreads) void lmhead_skinny_bf16(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, float* __restrict__ logits,
    int M, int V, int H, int n_tiles) {
    extern __shared__ __align__(16) uint16_t hs[];
    const int ld = H + 8;  // LDS row stride in elements (16-byte pad)
    const int cpr = H >> 3;  // 16-byte chunks per row
    for (int i = threadIdx.x; i < M * cpr; i += blockDim.x) {
        const int m = i / cpr, c = i - m * cpr;
        *reinterpret_cast<uint4*>(hs + m * ld + c * 8) =
            *reinterpret_cast<const uint4*>(hidden + (size_t)m * H + c * 8);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int wpb = blockDim.x >> 6;
    const bool hrow_ok = r < M;
    const uint16_t* hp = hs + (hrow_ok ? r : 0) * ld + g * 8;
    const bool vec_ok = (V & 3) == 0;
    const int n_steps = (H + 31) >> 5;        // 32-column steps
    const int n_stages = (n_steps + kSkinnyU - 1) / kSkinnyU;

    for (int t = blockIdx.x * wpb + (threadIdx.x >> 6); t < n_tiles; t += gridDim.x * wpb) {
        const int v0 = t << 4;
        const int vrow = min(v0 + r, V - 1);
        const uint16_t* wp = W + (size_t)vrow * H + g * 8;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 cur[kSkinnyU], nxt[kSkinnyU];

#pragma unroll
        for (int u = 0; u < kSkinnyU; ++u) {
            const int k = u * 32;
            cur[u] = (k + g * 8 < H) ? load_stream(wp + k) : zero;
        }
        for (int s = 0; s < n_stages; ++s) {
            const int kn = (s + 1) * kSkinnyU * 32;
            if (s + 1 < n_stages) {
#pragma unroll
                for (int u = 0; u < kSkinnyU; ++u) {
                    const int k = kn + u * 32;
                    nxt[u] = (k + g * 8 < H) ? load_stream(wp + k) : zero;
                }
            }
            const int kc = s * kSkinnyU * 32;
#pragma unroll
            for (int u = 0; u < kSkinnyU; ++u) {
                const int k = kc + u * 32;
                u32x4 hv = zero;
                if (hrow_ok && k + g * 8 < H) hv = *reinterpret_cast<const u32x4*>(hp + k);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur[u]), as_bf16x8(hv), acc, 0, 0, 0);
            }
            if (s + 1 < n_stages) {
#pragma unroll
                for (int u = 0; u < kSkinnyU; ++u) cur[u] = nxt[u];
            }
        }
        if (hrow_ok) store_row4(logits + (size_t)r * V, v0 + 4 * g, V, acc, vec_ok);
    }
}

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

size_t skinny_lds_bytes(int M, int H) { return (size_t)M * (H + 8) * 2; }

bool skinny_fits(int M, int H) { return M <= 16 && skinny_lds_bytes(M, H) <= 64 * 1024; }

hipError_t launch_lmhead_bf16(const uint16_t* hidden, const uint16_t* W, float* logits, int M, int V, int H,
                              int num_cus, hipStream_t stream, int force_kernel) {
    const bool skinny = force_kernel == 1 || (force_kernel == 0 && skinny_fits(M, H));
    if (skinny) {
        const int n_tiles = (V + 15) / 16;
        const size_t lds = skinny_lds_bytes(M, H);
        int occ = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, lmhead_skinny_bf16, kSkinnyThreads, lds);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
        const int wpb = kSkinnyThreads / 64;
        const long max_waves = (long)num_cus * occ * wpb;
        const long iters = (n_tiles + max_waves - 1) / max_waves;
        const long waves = (n_tiles + iters - 1) / iters;
        const int grid = (int)((waves + wpb - 1) / wpb);
        hipLaunchKernelGGL(lmhead_skinny_bf16, dim3(grid), dim3(kSkinnyThreads), lds, stream, hidden, W, logits, M,
                           V, H, n_tiles);
        return hipGetLastError();
    }
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
