// tb_project.hip -- key projection into the projected-key cache, and the
// append of new K/V rows (gfx950).
//
// TokenButler (gist.science technical summary, Methodology > Core
// Architecture): at each consumer layer the cached keys are mapped into the
// low-dimensional importance space by one learned matrix W [D][d].  Inference
// Strategy > Optimizations: this projection is done for a batch of new tokens
// at a time.
//
// Precision contract: kp = round_to_dtype( sum_{i ascending} k[i] * W[i][j] )
// with the sum in fp64.  Every product of two bf16 (or two fp32) values is
// exact in fp64, so a fused multiply-add in ascending i yields the same bits
// as the plain fp64 sum; the result is rounded once.  Small batches use the
// vector ALU; prefill-sized batches use the fp64 matrix cores, whose
// 16x16x4 instruction keeps the same order and rounding (see below).
#include "tb_internal.h"

#include <atomic>

namespace tb {
namespace {

// W [D][DI] into LDS as fp64, read in 16-byte pieces that are all requested
// before any is used (256 threads).
template <typename T, int D, int DI>
__device__ __forceinline__ void stage_w_f64(const T *__restrict__ w, double *sW)
{
    constexpr int EPC = 16 / sizeof(T);
    constexpr int WP = D * DI / EPC;
    constexpr int WPT = (WP + 255) / 256;
    uint4 wp[WPT];
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
        const int pi = threadIdx.x + q * 256;
        wp[q] = reinterpret_cast<const uint4 *>(w)[pi < WP ? pi : 0];
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
        const int pi = threadIdx.x + q * 256;
        if (pi < WP) {
            T v[EPC];
            __builtin_memcpy(v, &wp[q], 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                sW[pi * EPC + e] = to_f64(v[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// Few rows (the per-step append): one thread per (row, output column).  The
// W matrix and the work-group's K rows are staged in LDS as fp64.
// ---------------------------------------------------------------------------
template <typename T, int D, int DI, bool APPEND>
__global__ __launch_bounds__(256) void project_rows_kernel(
    const T *__restrict__ src, const T *__restrict__ vsrc, const T *__restrict__ w,
    const int32_t *__restrict__ pos_or_len, int n_tokens, int Hkv, int cap, int rows_total,
    T *__restrict__ k_cache, T *__restrict__ v_cache, T *__restrict__ kp)
{
    constexpr int ROWS = 256 / DI;
    __shared__ double sW[D * DI];
    __shared__ double sK[ROWS][D + 1];

    stage_w_f64<T, D, DI>(w, sW);

    const int rl = threadIdx.x / DI;
    const int j = threadIdx.x % DI;
    const int row = blockIdx.x * ROWS + rl;
    bool valid = row < rows_total;
    int bg = 0, t = 0, jj = 0;
    if (valid) {
        bg = row / n_tokens;
        jj = row - bg * n_tokens;
        const int b = bg / Hkv;
        if (APPEND)
            t = clamp_len(pos_or_len[b], cap) - n_tokens + jj;
        else
            t = pos_or_len[b] + jj;
        valid = t >= 0 && t < cap;
    }
    const size_t crow = ((size_t)bg * cap + t) * D;
    const size_t srow = APPEND ? ((size_t)bg * n_tokens + jj) * D : crow;
    if (valid) {
        for (int i = j; i < D; i += DI) {
            const T kv = src[srow + i];
            sK[rl][i] = to_f64(kv);
            if (APPEND) {
                k_cache[crow + i] = kv;
                v_cache[crow + i] = vsrc[srow + i];
            }
        }
    }
    __syncthreads();
    if (valid) {
        double acc = 0.0;
#pragma unroll 8
        for (int i = 0; i < D; ++i)
            acc = fma(sK[rl][i], sW[i * DI + j], acc);
        kp[((size_t)bg * cap + t) * DI + j] = from_f64<T>(acc);
    }
}

// ---------------------------------------------------------------------------
// Many rows (prefill-sized batches): the dense contraction on the fp64 matrix
// cores.  v_mfma_f64_16x16x4f64 adds its four products to the accumulator one
// after another in k order, rounding after each addition (crafted inputs
// whose fp64 sum depends on the order give the sequential result); the
// products here are exact in fp64, so a chain of these instructions over
// head_dim in ascending order is the fp64 chain of the precision contract.
//
// Operand layout of the instruction: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[l / 16 + 4 v][l % 16] in its v-th double.
// Here A is 16 key rows x 4 head_dim values, B the matching 4 rows of W.
// A work-group of 4 waves loops over blocks of rows; each wave owns 16 rows
// (32 when d = 16, so that two independent accumulators alternate) and all d
// outputs.  W stays in registers for the whole launch: lane l holds
// W[4 s + l / 16][16 n + l % 16] for every head_dim step s and output tile n.
// A block of keys is read with consecutive lanes on consecutive 16-byte
// pieces of whole rows (coalesced, every byte once), the next block in flight
// while the current one is multiplied, and stored in LDS as [row][i % 4][i / 4]
// so that a lane's A operands for 8 (bf16) or 4 (fp32) consecutive steps are
// one 16-byte read.  Results pass through a per-wave LDS tile to 16-byte
// stores of whole output rows.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 256;
constexpr int kWidePosLds = 256; // sequences whose pos0 is kept in LDS

template <typename T, int DI> struct WideTile {
    static constexpr int NT = DI / 16; // output tiles of 16
    static constexpr int RT = NT >= 2 ? 1 : 2; // row tiles of 16 per wave
    static constexpr int WROWS = 16 * RT;      // rows per wave
    static constexpr int BROWS = 4 * WROWS;    // rows per block
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T, int D, int DI>
__global__ __launch_bounds__(kWideThreads) void project_wide_kernel(
    const T *__restrict__ k_cache, const T *__restrict__ w, const int32_t *__restrict__ pos0,
    int batch, int n_tokens, int Hkv, int cap, int rows_total, int n_blocks, T *__restrict__ kp)
{
    using Tile = WideTile<T, DI>;
    constexpr int NT = Tile::NT, RT = Tile::RT, WROWS = Tile::WROWS, BROWS = Tile::BROWS;
    constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte piece
    constexpr int CPR = D / EPC;                    // pieces per key row
    constexpr int CPT = BROWS * CPR / kWideThreads; // pieces per thread and block
    static_assert(CPT * kWideThreads == BROWS * CPR, "whole pieces per thread");
    constexpr int S = D / 4;                        // head_dim steps of 4
    constexpr int GRPB = S * (int)sizeof(T);        // bytes of one i % 4 group
    constexpr int ROWB = 4 * GRPB + 16;             // bytes of one staged row (padded)
    constexpr int OB = DI * (int)sizeof(T);         // bytes of one output row
    constexpr int OPR = OB / 16;                    // 16-byte pieces per output row
    constexpr int OPL = WROWS * OPR / 64;           // output pieces per lane
    static_assert(OPL * 64 == WROWS * OPR, "whole output pieces per lane");
    __shared__ __align__(16) unsigned char sK[2][BROWS * ROWB];
    __shared__ __align__(16) unsigned char sO[4][WROWS * OB];
    __shared__ int32_t sPos[kWidePosLds];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lk = lane >> 4;

    for (int i = threadIdx.x; i < batch && i < kWidePosLds; i += kWideThreads)
        sPos[i] = pos0[i];
    __syncthreads();
    // row = (b Hkv + g) n_tokens + jj: one division pair per run of rows,
    // then steps along the run
    struct RowAt {
        int b, g, jj;
    };
    auto row_at = [&](int row) {
        const int bg = row / n_tokens, b = bg / Hkv;
        return RowAt{b, bg - b * Hkv, row - bg * n_tokens};
    };
    auto advance = [&](RowAt &r, int k) {
        r.jj += k;
        while (r.jj >= n_tokens) {
            r.jj -= n_tokens;
            if (++r.g == Hkv) {
                r.g = 0;
                ++r.b;
            }
        }
    };
    // cache row, or -1 (past the last row, or t outside [0, cap))
    auto cache_of = [&](int row, const RowAt &r) -> long long {
        if (row >= rows_total)
            return -1;
        const int t = (r.b < kWidePosLds ? sPos[r.b] : pos0[r.b]) + r.jj;
        if (t < 0 || t >= cap)
            return -1;
        return ((long long)r.b * Hkv + r.g) * cap + t;
    };
    // piece p = tid + q * threads of a block is piece p % CPR of block row
    // p / CPR; rows that are not stored read row 0
    constexpr int QS = kWideThreads / CPR; // block rows between a thread's pieces
    uint4 pc[CPT];
    auto load_block = [&](int blk) {
        const int row0 = blk * BROWS + (int)threadIdx.x / CPR;
        RowAt at = row_at(row0);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const long long cr = cache_of(row0 + q * QS, at);
            pc[q] = *reinterpret_cast<const uint4 *>(k_cache + (size_t)(cr < 0 ? 0 : cr) * D +
                                                     (size_t)(threadIdx.x % CPR) * EPC);
            if (q + 1 < CPT)
                advance(at, QS);
        }
    };
    if ((int)blockIdx.x < n_blocks)
        load_block(blockIdx.x);

    double wr[S][NT];
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
        for (int n = 0; n < NT; ++n)
            wr[st][n] = to_f64(w[(4 * st + lk) * DI + 16 * n + lr]);

    int it = 0;
    for (int blk = blockIdx.x; blk < n_blocks; blk += gridDim.x, ++it) {
        unsigned char *buf = sK[it & 1];
        // element i of a row goes to [i % 4][i / 4]
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int p = threadIdx.x + q * kWideThreads;
            unsigned char *row = buf + (p / CPR) * ROWB;
            const int c = p % CPR;
            if constexpr (EPC == 8) { // elements e and e + 4 are neighbours in group e
                const uint32_t x[4] = {pc[q].x, pc[q].y, pc[q].z, pc[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t hi = (x[2 + (e >> 1)] >> (16 * (e & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t *>(row + e * GRPB + c * 4) = lo | (hi << 16);
                }
            } else {
                const uint32_t x[4] = {pc[q].x, pc[q].y, pc[q].z, pc[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<uint32_t *>(row + e * GRPB + c * 4) = x[e];
            }
        }
        __syncthreads(); // this block staged; the other buffer is free again
        if (blk + (int)gridDim.x < n_blocks)
            load_block(blk + gridDim.x);

        f64x4 acc[RT][NT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int n = 0; n < NT; ++n)
                acc[rt][n] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int q = 0; q < S / EPC; ++q) {
            T av[RT][EPC];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                __builtin_memcpy(av[rt], buf + (wave * WROWS + rt * 16 + lr) * ROWB + lk * GRPB + q * 16,
                                 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const double a = to_f64(av[rt][e]);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc[rt][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, wr[q * EPC + e][n],
                                                                          acc[rt][n], 0, 0, 0);
                }
        }
        // outputs to the wave's LDS tile, then whole rows to the cache
        unsigned char *ot = sO[wave];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<T *>(ot + (rt * 16 + lk + 4 * v) * OB +
                                           (16 * n + lr) * (int)sizeof(T)) = from_f64<T>(acc[rt][n][v]);
        wave_lds_sync();
        {
            const int row0 = blk * BROWS + wave * WROWS + lane / OPR;
            RowAt at = row_at(row0);
#pragma unroll
            for (int u = 0; u < OPL; ++u) {
                const int pi = lane + 64 * u;
                const uint4 val = *reinterpret_cast<const uint4 *>(ot + pi * 16);
                const long long cr = cache_of(row0 + u * (64 / OPR), at);
                if (cr >= 0)
                    *reinterpret_cast<uint4 *>(kp + (size_t)cr * DI + (pi % OPR) * (16 / (int)sizeof(T))) = val;
                if (u + 1 < OPL)
                    advance(at, 64 / OPR);
            }
        }
        wave_lds_sync(); // the tile is read before the next block writes it
    }
}

template <typename T, int D, int DI>
hipError_t project_dispatch_t(const tb_shape &s, const void *k_cache, const void *w,
                              const int32_t *pos0, int n, void *kp, hipStream_t st)
{
    const long rows = (long)s.batch * s.n_kv_heads * n;
    if (rows >= 16384) {
        // persistent work-groups: as many as fit on the device at once
        static std::atomic<int> per_cu{0};
        int fit = per_cu.load(std::memory_order_relaxed);
        if (fit <= 0) {
            hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &fit, reinterpret_cast<const void *>(&project_wide_kernel<T, D, DI>), kWideThreads, 0);
            if (e != hipSuccess)
                return e;
            fit = fit < 1 ? 1 : fit;
            per_cu.store(fit, std::memory_order_relaxed);
        }
        int cus = 0;
        const hipError_t e = device_cus(cus);
        if (e != hipSuccess)
            return e;
        const int n_blocks = (int)((rows + WideTile<T, DI>::BROWS - 1) / WideTile<T, DI>::BROWS);
        const int grid = n_blocks < fit * cus ? n_blocks : fit * cus;
        hipLaunchKernelGGL((project_wide_kernel<T, D, DI>), dim3(grid), dim3(kWideThreads), 0, st,
                           (const T *)k_cache, (const T *)w, pos0, s.batch, n, s.n_kv_heads,
                           s.ctx_cap, (int)rows, n_blocks, (T *)kp);
    } else {
        constexpr int ROWS = 256 / DI;
        const int grid = (int)((rows + ROWS - 1) / ROWS);
        hipLaunchKernelGGL((project_rows_kernel<T, D, DI, false>), dim3(grid), dim3(256), 0, st,
                           (const T *)k_cache, (const T *)nullptr, (const T *)w, pos0, n,
                           s.n_kv_heads, s.ctx_cap, (int)rows, (T *)nullptr, (T *)nullptr,
                           (T *)kp);
    }
    return hipGetLastError();
}

template <typename T, int D, int DI>
hipError_t append_dispatch_t(const tb_shape &s, const void *k_new, const void *v_new, int n,
                             const void *w, void *k_cache, void *v_cache, void *kp,
                             const int32_t *ctx_len, hipStream_t st)
{
    const long rows = (long)s.batch * s.n_kv_heads * n;
    constexpr int ROWS = 256 / DI;
    const int grid = (int)((rows + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((project_rows_kernel<T, D, DI, true>), dim3(grid), dim3(256), 0, st,
                       (const T *)k_new, (const T *)v_new, (const T *)w, ctx_len, n,
                       s.n_kv_heads, s.ctx_cap, (int)rows, (T *)k_cache, (T *)v_cache, (T *)kp);
    return hipGetLastError();
}

#define TB_DISPATCH_D_DI(FN, T, ...)                                                         \
    do {                                                                                      \
        if (s.head_dim == 64 && s.d_imp == 16) return FN<T, 64, 16>(__VA_ARGS__);            \
        if (s.head_dim == 64 && s.d_imp == 32) return FN<T, 64, 32>(__VA_ARGS__);            \
        if (s.head_dim == 128 && s.d_imp == 16) return FN<T, 128, 16>(__VA_ARGS__);          \
        if (s.head_dim == 128 && s.d_imp == 32) return FN<T, 128, 32>(__VA_ARGS__);          \
    } while (0)

} // namespace

hipError_t launch_project(const tb_shape &s, const void *k_cache, const void *w,
                          const int32_t *pos0, int n_tokens, void *kp_cache, hipStream_t st)
{
    if (s.dtype == TB_BF16)
        TB_DISPATCH_D_DI(project_dispatch_t, bf16_t, s, k_cache, w, pos0, n_tokens, kp_cache, st);
    else
        TB_DISPATCH_D_DI(project_dispatch_t, float, s, k_cache, w, pos0, n_tokens, kp_cache, st);
    return hipErrorInvalidValue;
}

hipError_t launch_append_project(const tb_shape &s, const void *k_new, const void *v_new,
                                 int n_new, const void *w, void *k_cache, void *v_cache,
                                 void *kp_cache, const int32_t *ctx_len, hipStream_t st)
{
    if (s.dtype == TB_BF16)
        TB_DISPATCH_D_DI(append_dispatch_t, bf16_t, s, k_new, v_new, n_new, w, k_cache, v_cache,
                         kp_cache, ctx_len, st);
    else
        TB_DISPATCH_D_DI(append_dispatch_t, float, s, k_new, v_new, n_new, w, k_cache, v_cache,
                         kp_cache, ctx_len, st);
    return hipErrorInvalidValue;
}

} // namespace tb
