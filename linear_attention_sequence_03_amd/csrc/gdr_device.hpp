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

// Gate prologue maps of one raw value.
//   beta from its logit:        1 / (1 + e^-x)
//   log alpha from its logit:   -softplus(x) = -(max(x, 0) + ln(1 + e^-|x|)),
//                               so alpha = 1 / (1 + e^x) lies in (0, 1); the
//                               log1p keeps the relative accuracy of small
//                               decays (x << 0, where -softplus(x) ~ -e^x).
__device__ __forceinline__ float sigmoid_of(float x) { return 1.f / (1.f + __expf(-x)); }
__device__ __forceinline__ float neg_softplus(float x) {
    return -(fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));
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

// ---------------------------------------------------------------------------
// Permuted k-map, so that accumulator tiles can feed the next product.
// An accumulator tile hands lane (col, g) the rows 4g..4g+3.  A contraction
// whose B operand comes from accumulators therefore uses, in k-step s,
//   bf16 (16x16x32): slot j of lane group g  <->  k = 32s + 4g + (j&3) + 16(j>>2)
//                    (rows of the two tiles 2s and 2s+1)
//   fp32 (16x16x4):  lane group g            <->  k = 16(s>>2) + 4g + (s&3)
//                    (element s&3 of tile s>>2)
// and the A operand is read from LDS with the same map.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define GDR_LDS __attribute__((address_space(3)))

// A operand, natural storage p[m*rs + k].
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag afrag_nat(const E* p, int rs, int m0, int s,
                                                           int lane) {
    if constexpr (Mma<E>::KPL == 8) {
        const E* q = p + (m0 + (lane & 15)) * rs + 32 * s + 4 * (lane >> 4);
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(q);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(q + 16);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
        return p[(m0 + (lane & 15)) * rs + 16 * (s >> 2) + 4 * (lane >> 4) + (s & 3)];
    }
}

// A operand, transposed storage p[k*rs + m] (used for K^T in the state update).
// bf16: two ds_read_b64_tr_b16; in a 16-lane group, lane 4j+q reads row
// kbase+j, columns m0+4q..m0+4q+3, and lane i receives column m0+i of rows
// kbase..kbase+3.
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag afrag_tr(const E* p, int rs, int m0, int s,
                                                          int lane) {
    if constexpr (Mma<E>::KPL == 8) {
        const int g = lane >> 4, j = (lane & 15) >> 2, qd = lane & 3;
        const E* q = p + (32 * s + 4 * g + j) * rs + m0 + 4 * qd;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS s16x4*)(q));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS s16x4*)(q + 16 * rs));
        const bf16x4 l = __builtin_bit_cast(bf16x4, lo);
        const bf16x4 h = __builtin_bit_cast(bf16x4, hi);
        return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    } else {
        return p[(16 * (s >> 2) + 4 * (lane >> 4) + (s & 3)) * rs + m0 + (lane & 15)];
    }
}

// Token contractions with chunk C = 16 on the bf16 path cover only half of a
// 32-wide k-step: the upper 16 slots are zero on both sides (HALF = true).
template <typename E, bool HALF>
__device__ __forceinline__ typename Mma<E>::frag afrag_nat_tok(const E* p, int rs, int m0, int s,
                                                               int lane) {
    if constexpr (HALF) {
        const E* q = p + (m0 + (lane & 15)) * rs + 4 * (lane >> 4);
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(q);
        const __bf16 z = (__bf16)0.f;
        return bf16x8{lo[0], lo[1], lo[2], lo[3], z, z, z, z};
    } else {
        return afrag_nat<E>(p, rs, m0, s, lane);
    }
}

template <typename E, bool HALF>
__device__ __forceinline__ typename Mma<E>::frag afrag_tr_tok(const E* p, int rs, int m0, int s,
                                                              int lane) {
    if constexpr (HALF) {
        const int g = lane >> 4, j = (lane & 15) >> 2, qd = lane & 3;
        const E* q = p + (4 * g + j) * rs + m0 + 4 * qd;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS s16x4*)(q));
        const bf16x4 l = __builtin_bit_cast(bf16x4, lo);
        const __bf16 z = (__bf16)0.f;
        return bf16x8{l[0], l[1], l[2], l[3], z, z, z, z};
    } else {
        return afrag_tr<E>(p, rs, m0, s, lane);
    }
}

// B operand for k-step s from accumulator tiles t[] (16 rows each).
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag bfrag_acc(const f32x4* t, int s) {
    if constexpr (Mma<E>::KPL == 8) {
        const f32x4 a = t[2 * s], b = t[2 * s + 1];
        return bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                      (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
    } else {
        return t[s >> 2][s & 3];
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

// ---------------------------------------------------------------------------
// DPP shift within rows of 16 lanes, LDS-DMA tile copies, output stores.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_shr(float x) {
    // lanes without a source in their row of 16 get 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf,
                                                                  0xf, false));
}

// One tile of a chunk's inputs, copied global -> LDS by global_load_lds_dwordx4:
// lane l of an instruction lands at LDS base + 16 l, so an instruction fills
// 64 consecutive 16-byte slots and each lane fetches the global bytes of its
// slot.  Rows are stored with a 16-byte pad, and the tile's LDS region is
// rounded up to whole instructions; lanes whose slot is a pad or lies past the
// tile fetch the tile's first 16 bytes again (in bounds, never read back), so
// every lane of every instruction is active.  The per-lane source offsets are
// fixed for the kernel and computed once.
template <int ROWS, int ROWB, int NW>
struct DmaTile {
    static constexpr int RS = ROWB / 16 + 1;                 // slots per row, with the pad
    static constexpr int NSLOT = ROWS * RS;
    static constexpr int NINS = (NSLOT + 63) / 64;           // instructions per tile
    static constexpr int BYTES = NINS * 1024;                // LDS region
    static constexpr int PER_WAVE = (NINS + NW - 1) / NW;    // instructions per wave
    // Offsets for row stride gstride; rows >= valid read row valid-1 instead
    // (kept finite; their contributions are cancelled by zero rows of T).
    static __device__ __forceinline__ void offsets(int* off, int64_t gstride, int valid, int wave,
                                                   int lane) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int slot = (wave + j * NW) * 64 + lane;
            const int r = slot / RS, sg = slot - r * RS;
            const int rr = r < valid ? r : valid - 1;
            off[j] = (slot < NSLOT && sg < RS - 1) ? (int)(rr * gstride) + sg * 16 : 0;
        }
    }
    static __device__ __forceinline__ void issue(char* lds, const char* src, const int* off, int wave) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int ins = wave + j * NW;
            if (j + 1 < PER_WAVE || ins < NINS)   // wave-uniform
                __builtin_amdgcn_global_load_lds(src + off[j], (GDR_LDS void*)(lds + ins * 1024), 16,
                                                 0, 0);
        }
    }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One wave's staged [C][16] output tile -> o, 16 bytes per store (rows < len).
template <typename E, int C, int LO>
__device__ __forceinline__ void store_out(E* o, const E* ostg, int64_t row0, int H, int DV, int c0,
                                          int len, int lane) {
    constexpr int ES = sizeof(E);
    constexpr int PPR = 16 * ES / 16;   // 16-byte pieces per row
#pragma unroll
    for (int p = lane; p < C * PPR; p += 64) {
        const int r = p / PPR, pc = p % PPR;
        if (r < len)
            *reinterpret_cast<V16*>(o + (row0 + (int64_t)r * H) * DV + c0 + pc * (16 / ES)) =
                *reinterpret_cast<const V16*>(ostg + r * LO + pc * (16 / ES));
    }
}

}  // namespace gdr
