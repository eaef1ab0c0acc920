// gdr_device.hpp -- device-side building blocks shared by the gated delta rule
// kernels for gfx950 (CDNA4): element types, 16x16 MFMA tiles and their operand
// fragments, wave reductions.
//
// Matrix-core convention used everywhere ("NT" products):
//     C[m][n] += sum_k A[m][k] * B[n][k]
// with 16x16 output tiles.  For every 16x16 MFMA shape on CDNA the lane that
// carries operand element (row, k) is lane = row%16 + 16*g, where g selects a
// group of k values; the accumulator lane l holds C[4*(l/16)+i][l%16], i<4.
// Only the pairing of A's and B's k-slots matters for a contraction, so both
// operands are loaded with the same lane->k map (k = k0 + KPL*(l/16) + j).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MFMA shapes.  bf16: v_mfma_f32_16x16x32_bf16 (8 k-values per lane).
//                fp32: v_mfma_f32_16x16x4_f32  (1 k-value per lane).
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<__bf16> {
    static constexpr int KS = 32;   // k per instruction
    static constexpr int KPL = 8;   // k values per lane
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// LDS row padding (elements): 16 bytes, so consecutive rows start 4 banks apart.
template <typename E> struct Pad { static constexpr int v = 16 / sizeof(E); };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f32(float x) { return (E)x; }

// ---------------------------------------------------------------------------
// Operand fragments from LDS.
// frag_rk:  element (row, k) stored at p[row*rs + k]   (k contiguous)
// frag_kr:  element (row, k) stored at p[k*rs + row]   (row contiguous)
// frag_rk_f32: like frag_rk, source fp32, converted to E.
// row0 / k0 are tile origins; the lane's row is row0 + lane%16.
// ---------------------------------------------------------------------------
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag frag_rk(const E* p, int rs, int row0, int k0,
                                                         int lane) {
    if constexpr (Mma<E>::KPL == 8) {
        const E* q = p + (row0 + (lane & 15)) * rs + k0 + 8 * (lane >> 4);
        return *reinterpret_cast<const bf16x8*>(q);
    } else {
        return p[(row0 + (lane & 15)) * rs + k0 + (lane >> 4)];
    }
}

template <typename E>
__device__ __forceinline__ typename Mma<E>::frag frag_kr(const E* p, int rs, int row0, int k0,
                                                         int lane) {
    if constexpr (Mma<E>::KPL == 8) {
        const E* q = p + (k0 + 8 * (lane >> 4)) * rs + row0 + (lane & 15);
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = q[j * rs];
        return f;
    } else {
        return p[(k0 + (lane >> 4)) * rs + row0 + (lane & 15)];
    }
}

template <typename E>
__device__ __forceinline__ typename Mma<E>::frag frag_rk_f32(const float* p, int rs, int row0,
                                                             int k0, int lane) {
    if constexpr (Mma<E>::KPL == 8) {
        const float* q = p + (row0 + (lane & 15)) * rs + k0 + 8 * (lane >> 4);
        const float4 a = *reinterpret_cast<const float4*>(q);
        const float4 b = *reinterpret_cast<const float4*>(q + 4);
        bf16x8 f;
        f[0] = (__bf16)a.x; f[1] = (__bf16)a.y; f[2] = (__bf16)a.z; f[3] = (__bf16)a.w;
        f[4] = (__bf16)b.x; f[5] = (__bf16)b.y; f[6] = (__bf16)b.z; f[7] = (__bf16)b.w;
        return f;
    } else {
        return p[(row0 + (lane & 15)) * rs + k0 + (lane >> 4)];
    }
}

// 4 consecutive elements <-> float4 (8-byte bf16 or 16-byte fp32 access).
template <typename E>
__device__ __forceinline__ float4 load4(const E* p) {
    if constexpr (sizeof(E) == 4) {
        return *reinterpret_cast<const float4*>(p);
    } else {
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
        return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
    }
}

template <typename E>
__device__ __forceinline__ void store4(E* p, float4 v) {
    if constexpr (sizeof(E) == 4) {
        *reinterpret_cast<float4*>(p) = v;
    } else {
        bf16x4 x;
        x[0] = (__bf16)v.x; x[1] = (__bf16)v.y; x[2] = (__bf16)v.z; x[3] = (__bf16)v.w;
        *reinterpret_cast<bf16x4*>(p) = x;
    }
}

// Accumulator coordinates of lane l, element i: (row, col) inside the tile.
__device__ __forceinline__ int acc_row(int lane, int i) { return 4 * (lane >> 4) + i; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// 16-byte global vector access helpers.
// ---------------------------------------------------------------------------
struct alignas(16) V16 { uint32_t w[4]; };

__device__ __forceinline__ V16 ld16(const void* p) { return *reinterpret_cast<const V16*>(p); }
__device__ __forceinline__ void st16(void* p, V16 v) { *reinterpret_cast<V16*>(p) = v; }
__device__ __forceinline__ V16 zero16() { return V16{{0u, 0u, 0u, 0u}}; }

// XCD-aware block index: consecutive logical blocks share one XCD (workgroups
// are dispatched round-robin over the 8 XCDs), so blocks that re-read the same
// data hit the same L2.  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    if (nblocks % 8 != 0) return bid;
    const int per = nblocks / 8;
    return (bid % 8) * per + bid / 8;
}

}  // namespace gdr
