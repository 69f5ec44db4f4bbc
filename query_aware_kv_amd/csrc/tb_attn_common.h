// tb_attn_common.h -- pieces shared by the attention kernels (gfx950): the
// lane dot products, row reductions, and the publication and merge of
// per-chunk softmax partials across work-groups.  Not part of the public ABI.
#pragma once

#include "tb_internal.h"

namespace tb {

constexpr int kMaxChunks = kMaxCtxCap / kAttnChunk;

// Sum of x over aligned groups of N lanes (N in {1, 2, 4, 8, 16, 32}); every
// lane of the group receives the sum.  Within a 16-lane DPP row the partners
// come from quad permutations and the half/full row mirrors.
template <int N> __device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    if constexpr (N >= 4)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    if constexpr (N >= 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    if constexpr (N >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    if constexpr (N >= 32)
        x += __shfl_xor(x, 16);
    return x;
}

// Combines x over the lanes that differ from this one in the bits above
// the low log2(N) bits (the row slots of a wave when N lanes serve a row);
// every lane receives the result.  Lane pairs 8 apart meet through a DPP row
// rotation, 16 and 32 apart through the permlane swaps, so no LDS is used.
// op must be commutative (the two operands arrive in lane order).
template <int N, typename Op> __device__ __forceinline__ float across_slots(float x, Op op)
{
    if constexpr (N <= 8)
        x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF,
                                                             0xF, false))); // row_ror:8
    if constexpr (N <= 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    if constexpr (N <= 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    return x;
}

// Dot product of the 16-byte q and k pieces held by one lane.
__device__ __forceinline__ float lane_dot_bf16(const uint4 &q, const uint4 &k)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                        __builtin_bit_cast(bf16x2, k.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                        __builtin_bit_cast(bf16x2, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                        __builtin_bit_cast(bf16x2, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                        __builtin_bit_cast(bf16x2, k.w), d, false);
    return d;
}
__device__ __forceinline__ float lane_dot_f32(const uint4 &q, const uint4 &k)
{
    float d = __uint_as_float(q.x) * __uint_as_float(k.x);
    d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
    d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
    d = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
    return d;
}
template <typename T> __device__ __forceinline__ float lane_dot(const uint4 &q, const uint4 &k)
{
    if constexpr (sizeof(T) == 2)
        return lane_dot_bf16(q, k);
    else
        return lane_dot_f32(q, k);
}

// Stores one chunk partial: acc value O of dimension dim (lane pairs of
// consecutive dimensions store together) and, from dimension 0, the chunk's
// (max, sum).  pc = query head * chunks + chunk.  Every lane of the wave must
// take part (the pairing reads the neighbor lane).
template <int D>
__device__ __forceinline__ void publish_partial(float *part_o, float *part_ml, size_t pc, int dim,
                                                float O, float M, float Ls)
{
    const float On = __uint_as_float(dpp<0xB1>(__float_as_uint(O)));
    if ((dim & 1) == 0)
        store2_agent(&part_o[pc * D + dim], O, On);
    if (dim == 0)
        __hip_atomic_store(reinterpret_cast<double *>(part_ml) + pc,
                           __builtin_bit_cast(double, make_float2(M, Ls)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Shared memory of the cross-chunk merge (at most NCH chunks).
template <int GQ, int THREADS, int NCH = kMaxChunks> struct CombineLds {
    float f[GQ][NCH]; // chunk maxima, then chunk weights
    float l[GQ][NCH]; // chunk sums
    float Ls[GQ];            // total sum per query head
    float4 red[THREADS];
    uint32_t last;
};

// Arrival of one work-group of the (sequence b, KV head g) group of nchunk
// chunks; the last to arrive merges the nact chunk partials of the GQ query
// heads head0 .. head0+GQ-1 into out, and resets the arrival counter for the
// next call.  The caller's partial stores must precede the call.
template <typename T, int D, int GQ, int THREADS, int NCH>
__device__ __forceinline__ void arrive_and_combine(CombineLds<GQ, THREADS, NCH> &S,
                                                   uint32_t *counter,
                                                   const float *part_o, const float *part_ml,
                                                   int nchunk, int nact, size_t head0, T *out)
{
    constexpr int NWAVES = THREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // The partial stores complete (vmcnt 0) before the counter moves; the
    // signal fence keeps the compiler from sinking them below it.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        S.last = old == (uint32_t)(nchunk - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (S.last == 0u)
        return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // Every load of the merge is issued up front: the chunk (max, sum) pairs
    // into LDS, and each thread's weighted-sum inputs into registers.
    constexpr int NCOL = GQ * D / 4;
    constexpr int NPART = THREADS / NCOL;
    static_assert(NPART >= 1 && NPART * NCOL == THREADS, "column split");
    const int col = tid % NCOL, part = tid / NCOL;
    const int chl = col / (D / 4), d4 = col % (D / 4);
    for (int e = tid; e < GQ * nact; e += THREADS) {
        const int hl = e / nact, cc = e % nact;
        const size_t pc = (head0 + hl) * nchunk + cc;
        const double ml = __hip_atomic_load(reinterpret_cast<const double *>(part_ml) + pc,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float2 v = __builtin_bit_cast(float2, ml);
        S.f[hl][cc] = v.x;
        S.l[hl][cc] = v.y;
    }
    // this thread's column of the group's partials, [GQ][nchunk][D] floats
    const __amdgpu_buffer_rsrc_t po =
        coherent_rsrc(part_o + head0 * nchunk * D, (uint32_t)(GQ * nchunk * D * sizeof(float)));
    const uint32_t col0 = (uint32_t)((chl * nchunk * D + d4 * 4) * sizeof(float));
    auto part_at = [&](int cc) {
        return load4_coherent(po, col0 + (uint32_t)((cc < nact ? cc : 0) * D * sizeof(float)));
    };
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // chunk weights need the maxima; the first batch of partial sums is
    // loaded meanwhile
    constexpr int BATCH = 8;
    float4 v0[BATCH];
#pragma unroll
    for (int r = 0; r < BATCH; ++r) {
        const int cc = part + r * NPART;
        v0[r] = part_at(cc);
    }
    // the (max, sum) pairs are in LDS; the partial sums stay in flight
    lds_barrier();
    for (int hl = wave; hl < GQ; hl += NWAVES) {
        float M = -INFINITY;
        for (int cc = lane; cc < nact; cc += 64)
            M = fmaxf(M, S.f[hl][cc]);
        M = wave_max(M);
        float Ls = 0.f;
        for (int cc = lane; cc < nact; cc += 64) {
            const float mc = S.f[hl][cc];
            const float f = (mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
            S.f[hl][cc] = f;
            Ls = fmaf(S.l[hl][cc], f, Ls);
        }
        Ls = wave_sum(Ls);
        if (lane == 0)
            S.Ls[hl] = Ls;
    }
    __syncthreads();
    for (int c0b = part; c0b < nact; c0b += BATCH * NPART) {
        float4 v[BATCH];
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            const int cc = c0b + r * NPART;
            v[r] = c0b == part ? v0[r] : part_at(cc);
        }
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            const int cc = c0b + r * NPART;
            const float f = cc < nact ? S.f[chl][cc] : 0.f;
            s4.x = fmaf(v[r].x, f, s4.x);
            s4.y = fmaf(v[r].y, f, s4.y);
            s4.z = fmaf(v[r].z, f, s4.z);
            s4.w = fmaf(v[r].w, f, s4.w);
        }
    }
    S.red[part * NCOL + col] = s4;
    __syncthreads();
    for (int cl = tid; cl < NCOL; cl += THREADS) {
        const int hl = cl / (D / 4), dd = cl % (D / 4);
        float4 s = S.red[cl];
        for (int p = 1; p < NPART; ++p) {
            const float4 t = S.red[p * NCOL + cl];
            s.x += t.x;
            s.y += t.y;
            s.z += t.z;
            s.w += t.w;
        }
        const float Ls = S.Ls[hl];
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        T *o = out + (head0 + hl) * D + dd * 4;
        o[0] = from_f32<T>(s.x * inv);
        o[1] = from_f32<T>(s.y * inv);
        o[2] = from_f32<T>(s.z * inv);
        o[3] = from_f32<T>(s.w * inv);
    }
    if (tid == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

} // namespace tb
