// Device-side helpers for the gfx950 RMSNorm kernels: BF16 pack/unpack,
// 16-byte vector access, row addressing and lane-group reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsn_internal.h"

namespace rmsn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// BF16 -> FP32 is exact: the 16 bits are the top half of the FP32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two FP32 -> two BF16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with a cache policy: NT marks it non-temporal (streamed), for
// inputs that no later access in the step will find in the caches anyway.
template <bool NT>
__device__ __forceinline__ uint4 ld16p(const uint16_t* p) {
    if constexpr (NT) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(w.x, w.y, w.z, w.w);
    } else {
        return ld16(p);
    }
}

// Streaming store for the large outputs (y, dx, and the residual form's h):
// marked non-temporal so they do not displace inputs from the caches, and so
// that a step's forward leaves less dirty data to drain while the backward
// runs (h is read again by the backward, but at training sizes it does not
// stay cached anyway: 16384 x 6144 residual step 298 -> 290 us with h
// streamed).
__device__ __forceinline__ void st16_stream(uint16_t* p, const uint4& v) {
    u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// Weight vector of 8 elements as FP32 (BF16 widened exactly).
template <typename WT>
__device__ __forceinline__ void load_w8(const void* w, int v, float (&f)[8]);

template <>
__device__ __forceinline__ void load_w8<uint16_t>(const void* w, int v, float (&f)[8]) {
    uint4 q = ld16(static_cast<const uint16_t*>(w) + (int64_t)v * kVec);
    unpack8(q, f);
}

template <>
__device__ __forceinline__ void load_w8<float>(const void* w, int v, float (&f)[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + (int64_t)v * kVec);
    float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Element offset of row r = (t, head) under an addressing rule.
__device__ __forceinline__ int64_t row_offset(int64_t r, int32_t heads, const RowAddr& a) {
    if (heads == 1) return r * a.st_t;
    // rows fit in 32 bits for every supported shape (checked on the host)
    uint32_t ur = (uint32_t)r, uh = (uint32_t)heads;
    uint32_t t = ur / uh;
    uint32_t hd = ur - t * uh;
    return (int64_t)t * a.st_t + (int64_t)hd * a.st_h;
}

// Make the compiler wait here for the loads that produced v. The memory
// counter the compiler waits on is in-order and counts stores too, so a wait
// for an older load also waits for every newer load or store. Forcing the
// first tile of a software-pipelined loop to be complete before the loop
// keeps the loop body free of such a wait, which would otherwise also drain
// the next tile's prefetch at every iteration.
__device__ __forceinline__ void use_now(const uint4& v) {
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}
__device__ __forceinline__ void use_now(float v) { asm volatile("" ::"v"(v)); }

// A copy of v that the compiler cannot see through: values derived from it
// are recomputed rather than kept live from an earlier identical expression.
// Used where the unpacked row would otherwise stay in registers across a row
// reduction (twice the registers of the packed 16-byte vectors).
__device__ __forceinline__ uint4 opaque(uint4 v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    return v;
}

// Workgroup barrier that orders LDS traffic only. A plain __syncthreads()
// also waits for the wave's outstanding global loads and stores (the vector
// memory counter covers both on gfx9-family parts), which would drain the
// rows prefetched for the next iteration at every row.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Butterfly sum over aligned groups of G lanes (G a power of two <= 64);
// every lane of the group receives the group's sum. The pairing order is
// fixed, so the result is bit-reproducible. The exchanges run through the
// LDS crossbar (ds_bpermute), next to the vector ALU that the row
// arithmetic keeps busy.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int G>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Runtime-width variant (g a power of two <= 64).
__device__ __forceinline__ float group_sum_rt(float v, int g) {
    for (int m = g >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ double group_sum_rt(double v, int g) {
    for (int m = g >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Lane exchanges on the vector ALU (no LDS): DPP quad permutes (partner
// i^1, i^2), row rotations inside 16-lane rows, and the gfx950 permlane
// swaps across 16-lane rows and 32-lane halves, where both partners receive
// the lower and the upper lane's value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ double dpp_partner(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp32<CTRL>((uint32_t)u), hi = dpp32<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}

// v(lower) + v(upper) over the lane pairs i, i ^ 16 (X = 16) or i, i ^ 32.
template <int X>
__device__ __forceinline__ double swap_sum(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto rl = X == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = X == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const double a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
    return a + b;
}

// FP64 sums over the 64 lanes of a wave of U per-lane values (U rows), for
// rows that span whole waves, where only one lane per row needs the sum. The
// first log2(U) stages scatter the rows: each lane keeps half of its rows,
// adds its partner's values for them and hands over the other half (DPP
// xor 1, xor 2, then, for U = 8, a row rotation by 4, whose source lane
// always differs from the receiver in lane bit 2). Then each lane carries one
// row: rotations by 4 and 8 inside 16-lane rows (they keep lane bits 0-1, so
// the added values belong to the same row) and the two permlane swaps finish
// the sum. Lane q < U returns the sum of row wave_row<U>(q). log2(U) + 4
// exchanges instead of 6U; the order is fixed, so sums are reproducible.
template <int N, int CTRL, typename T>
__device__ __forceinline__ void scatter_stage(const T (&in)[2 * N], T (&out)[N], bool hi) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const T keep = hi ? in[N + j] : in[j];
        const T give = hi ? in[j] : in[N + j];
        out[j] = keep + dpp_partner<CTRL>(give);
    }
}

template <int U, typename T>
__device__ __forceinline__ T wave_sums(const T (&v)[U], int lane) {
    static_assert(U == 1 || U == 2 || U == 4 || U == 8, "rows per wave sum");
    T s;
    if constexpr (U == 1) {
        s = v[0] + dpp_partner<0xB1>(v[0]);
        s = s + dpp_partner<0x4E>(s);
    } else if constexpr (U == 2) {
        T a[1];
        scatter_stage<1, 0xB1>(v, a, lane & 1);
        s = a[0] + dpp_partner<0x4E>(a[0]);
    } else if constexpr (U == 4) {
        T a[2], b[1];
        scatter_stage<2, 0xB1>(v, a, lane & 1);
        scatter_stage<1, 0x4E>(a, b, (lane >> 1) & 1);
        s = b[0];
    } else {
        T a[4], b[2], c[1];
        scatter_stage<4, 0xB1>(v, a, lane & 1);
        scatter_stage<2, 0x4E>(a, b, (lane >> 1) & 1);
        scatter_stage<1, 0x124>(b, c, (lane >> 2) & 1);
        s = c[0];
    }
    if constexpr (U <= 4) s = s + dpp_partner<0x124>(s);  // row_ror:4
    s = s + dpp_partner<0x128>(s);                        // row_ror:8
    s = swap_sum<16>(s);
    s = swap_sum<32>(s);
    return s;
}

// The row whose sum wave_sums<U> leaves in lane q (q < U).
template <int U>
__device__ __forceinline__ int wave_row(int q) {
    if constexpr (U == 1) return 0;
    if constexpr (U == 2) return q & 1;
    if constexpr (U == 4) return 2 * (q & 1) + ((q >> 1) & 1);
    return 4 * (q & 1) + 2 * ((q >> 1) & 1) + ((q >> 2) & 1);
}

}  // namespace rmsn
