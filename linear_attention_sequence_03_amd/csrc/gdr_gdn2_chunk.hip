// gdr_gdn2_chunk.hip -- chunkwise forward pass of Gated DeltaNet-2's decoupled
// erase and write gates ("Daily Papers" pages: the Gated DeltaNet-2 abstract and
// citation notes, which state the update in words; the chunk organisation is
// the one of the "FG2-GDN" page, section 3.6).
//
// Token step (state S is dv x dk, e_t = b_t * k_t, vt_t = w_t * v_t):
//   S~ = S Diag(alpha_t);  r_t = S~ k_t;  S_t = S~ - r_t e_t^T + vt_t k_t^T;  o_t = S_t q_t.
// Inside a chunk starting from state S, with g the inclusive cumulative log
// decay (a dk-vector per row, Gamma_r = exp(g_r), gamma_C the last row's):
//   L_k[t][i] = (k_t Gamma_t).(k_i / Gamma_i),  L_e[t][i] = (k_t Gamma_t).(e_i / Gamma_i)   (i < t)
//   P_k[t][i] = (q_t Gamma_t).(k_i / Gamma_i),  P_e[t][i] = (q_t Gamma_t).(e_i / Gamma_i)   (i <= t)
//   reads    R = (I + L_e)^-1 (Kg S^T + L_k Vt)           Kg = K Gamma, Qg = Q Gamma
//   outputs  O = Qg S^T + P_k Vt - P_e R
//   state    S_C^T = Diag(gamma_C) S^T + Kh^T Vt - Eh^T R   Kh = K gamma_C / Gamma, Eh = E gamma_C / Gamma
// With Ti = (I + L_e)^-1, M = Ti L_k and Z = P_e Ti, everything that involves
// neither S nor V folds into per-chunk operands
//   W = Ti Kg,  QP = Qg - Z Kg,  PP = P_k - Z L_k,  KHP = Kh - M^T Eh,  EHN = -Eh,
// and the sequential part of a chunk becomes
//   X = W S^T;   O = QP S^T + PP Vt;   S^T <- Diag(gamma_C) S^T + KHP^T Vt + EHN^T X.
// This is the token recurrence reorganised, with no approximation.
//
// Two kernels per call (bf16 io, 64-token chunks):
//  1. gdn2_prep -- one workgroup of four waves per (b, h, chunk), fully
//     parallel.  Wave b owns rows 16b..16b+15.  The four Gram matrices are
//     built on bf16 MFMAs with the decay split at block boundaries (the same
//     scheme as the KDA prep).  The rest runs on fp16 16x16x16 MFMAs, one
//     16-token block per k-step: the unit-lower inverse Ti (forward
//     substitution on the 16x16 diagonal blocks, then a block row wavefront),
//     Z, M and the five operands above.  Entries of L, P, Ti, Z and M stay small
//     for unit-norm keys and gates in [0, 1], well inside fp16's range.
//  2. gdn2_state_pass -- each compute wave owns 16 value columns of one (b, h)
//     and keeps its fp32 state slice in MFMA accumulators across the chunks.
//     W, QP, PP, V and w are double-buffered in LDS; KHP, EHN and gamma_C are
//     needed only by the state update at the end of a chunk and are copied
//     while the chunk's other products run.  The loaders also warm L2 with the
//     chunk after next (the head's workspace block split over its workgroups).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int GC = 64;               // chunk
constexpr int GNB = GC / 16;         // 16-row blocks per chunk
constexpr float kG2Log2e = 1.4426950408889634f;
constexpr float kG2MinLogAlpha = -200.f;                // exp(-200): 0 in fp32
constexpr float kG2SafeSpan2 = 64.f * 1.4426950408889634f;   // in-block decay span (log2 units)

__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 h4(f32x4 x) {
    return f16x4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ bf16x4 b4(f32x4 x) {
    return bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
// LDS written by some lanes of a wave and read by others.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Byte layout of one (b, h, chunk) workspace block: bf16 row-major tiles W,
// QP, KHP, EHN [C][DK] and PP [C][C] (zero above the diagonal blocks), then
// gamma_C [DK] fp32.
template <int DK>
struct G2Ws {
    static constexpr size_t TILE = (size_t)GC * DK * 2;
    static constexpr size_t W = 0, QP = TILE, KHP = 2 * TILE, EHN = 3 * TILE, PP = 4 * TILE;
    static constexpr size_t VEC = PP + (size_t)GC * GC * 2;
    static constexpr size_t BYTES = (VEC + DK * 4 + 255) / 256 * 256;
};

// Operand layouts of a 16x16 tile X held by a wave as four values per lane
// (lane = col + 16 g):
//   R: lane (x, g) holds X[x][4g + e]        (a row per lane)
//   A: lane (c, g) holds X[4g + e][c]        (the accumulator layout)
// mma16(a, b) sums a(i, k) b(j, k) into element [i][j] of an accumulator, so
// for P = A B:  mma16(R(A), A-layout(B)) gives P in the accumulator layout and
// mma16(A-layout(B), R(A)) gives P in R.
template <int DK>
struct G2PrepSmem {
    static constexpr int NS = DK / 32;
    static constexpr int LT = GC + 4;   // f16 row stride of C x C tiles and transposed tiles
    struct Grams {                      // B sides of the Gram products, blocks 0..NB-2
        bf16x8 bk[GNB - 1][NS][64];
        bf16x8 be[GNB - 1][NS][64];
    };
    struct Solve {
        _Float16 ti[GC * LT];           // Ti, row-major (lower blocks)
        _Float16 lk[GC * LT];           // L_k, row-major (lower blocks)
        f16x4 tpub[6][64];              // Ti tiles of rows < NB-1 for the wavefront (A-layout)
        f16x4 m1[10][64];               // M blocks (j, n), n <= j (A-layout)
    };
    union Shared {
        Grams g;
        Solve s;
    };
    alignas(16) float tot[GNB][DK];     // per-block totals of g (log2 units)
    alignas(16) Shared u;
    alignas(16) _Float16 kgt[DK * LT];  // Kg transposed: [channel][token]
    alignas(16) _Float16 eht[DK * LT];  // Eh transposed
    alignas(16) float xa[GNB][16 * 16]; // diagonal L_e blocks, transposed, for the substitution
    alignas(16) float xx[GNB][16 * 17]; // their inverses
};

__host__ __device__ constexpr int tri_idx(int m, int j) { return m * (m + 1) / 2 + j; }

// One wave's share (rows 16BW..16BW+15) of the per-chunk preparation.
//  Channel map of a 32-channel step s for the bf16 Gram products: slot j of
//  lane group g is channel 32s + 16(j/4) + 4g + j%4, so the two halves of the
//  slots are the R-layout channels of 16-channel tiles 2s and 2s+1.
template <int DK, int BW, bool CH>
__device__ __forceinline__ void gdn2_prep_wave(G2PrepSmem<DK>& sm, const __bf16* __restrict__ q,
                                               const __bf16* __restrict__ k,
                                               const float* __restrict__ log_alpha,
                                               const float* __restrict__ erase, uint8_t* __restrict__ ws,
                                               int64_t T, int H, int NT) {
    using L = G2Ws<DK>;
    using M = Mma<__bf16>;
    constexpr int NB = GNB, NS = DK / 32, NCT = DK / 16;
    constexpr int LT = G2PrepSmem<DK>::LT;
    constexpr int b = BW;
    const int lane = threadIdx.x & 63;
    const int x = lane & 15, kg = lane >> 4;
    const int64_t bid = blockIdx.x;
    const int n = (int)(bid % NT);
    const int64_t bh = bid / NT;
    const int64_t bi = bh / H, h = bh % H;
    const int64_t t0 = (int64_t)n * GC;
    const int len = (int)((T - t0) < GC ? (T - t0) : GC);
    const int64_t row0 = (bi * T + t0) * H + h;
    uint8_t* blk = ws + (size_t)bid * L::BYTES;
    const int r = 16 * b + x;
    const bool valid = r < len;   // rows past len read row len-1 and are zeroed
    const int64_t grow = row0 + (int64_t)(valid ? r : len - 1) * H;

    auto chan = [&](int s, int j) { return 32 * s + 16 * (j >> 2) + 4 * kg + (j & 3); };
    auto ld_bf = [&](const __bf16* p, int s, float* out) {
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(p + grow * DK + 32 * s + 4 * kg);
        const bf16x4 c = *reinterpret_cast<const bf16x4*>(p + grow * DK + 32 * s + 16 + 4 * kg);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[j] = valid ? (float)a[j] : 0.f;
            out[4 + j] = valid ? (float)c[j] : 0.f;
        }
    };
    auto ld_f = [&](const float* p, int s, float* out) {
        const float4 a = *reinterpret_cast<const float4*>(p + grow * DK + 32 * s + 4 * kg);
        const float4 c = *reinterpret_cast<const float4*>(p + grow * DK + 32 * s + 16 + 4 * kg);
        const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = valid ? v[j] : 0.f;
    };
    auto ld_la = [&](int s, float* g) {   // log alpha in log2 units, 0 past len
        if constexpr (CH) {
            float t[8];
            ld_f(log_alpha, s, t);
#pragma unroll
            for (int j = 0; j < 8; ++j) g[j] = fmaxf(t[j], kG2MinLogAlpha) * kG2Log2e;
        } else {
            const float a = valid ? fmaxf(log_alpha[grow], kG2MinLogAlpha) * kG2Log2e : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) g[j] = a;
        }
    };
    auto scan = [&](float* v) {   // inclusive scan over the 16 rows of the block
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float u = v[j];
            u += dpp_shr<0x111>(u);
            u += dpp_shr<0x112>(u);
            u += dpp_shr<0x114>(u);
            u += dpp_shr<0x118>(u);
            v[j] = u;
        }
    };
    auto ld_tot = [&](int cb, int s, float* tv) {
        const float4 a = *reinterpret_cast<const float4*>(&sm.tot[cb][32 * s + 4 * kg]);
        const float4 c = *reinterpret_cast<const float4*>(&sm.tot[cb][32 * s + 16 + 4 * kg]);
        tv[0] = a.x; tv[1] = a.y; tv[2] = a.z; tv[3] = a.w;
        tv[4] = c.x; tv[5] = c.y; tv[6] = c.z; tv[7] = c.w;
    };
    auto to8 = [](const float* v) {
        bf16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (__bf16)v[j];
        return o;
    };

    // ---- phase 1: decay, kept operands, Gram tiles (R layout, column blocks <= b) ----
    f32x4 lk[NB], le[NB], pk[NB], pe[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) lk[cb] = le[cb] = pk[cb] = pe[cb] = zero4();
    f32x4 qgk[NCT], khk[NCT];   // Qg and Kh of row r, R layout per 16-channel tile
    bool unsafe = false;
    // Raw loads of a channel step, issued one step ahead of their use.
    struct RawStep {
        bf16x4 k0, k1, q0, q1;
        float4 l0, l1, e0, e1;
    };
    auto ld_raw = [&](int s) {
        RawStep y;
        const int64_t o0 = grow * DK + 32 * s + 4 * kg;
        y.k0 = *reinterpret_cast<const bf16x4*>(k + o0);
        y.k1 = *reinterpret_cast<const bf16x4*>(k + o0 + 16);
        y.q0 = *reinterpret_cast<const bf16x4*>(q + o0);
        y.q1 = *reinterpret_cast<const bf16x4*>(q + o0 + 16);
        if constexpr (CH) {
            y.l0 = *reinterpret_cast<const float4*>(log_alpha + o0);
            y.l1 = *reinterpret_cast<const float4*>(log_alpha + o0 + 16);
        } else {
            const float a = log_alpha[grow];
            y.l0 = make_float4(a, a, a, a);
            y.l1 = y.l0;
        }
        y.e0 = *reinterpret_cast<const float4*>(erase + o0);
        y.e1 = *reinterpret_cast<const float4*>(erase + o0 + 16);
        return y;
    };
    RawStep nxt = ld_raw(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const RawStep cur = nxt;
        if (s + 1 < NS) nxt = ld_raw(s + 1);
        float gs[8], kv[8], qv[8], ev[8];
        {
            const float lr[8] = {cur.l0.x, cur.l0.y, cur.l0.z, cur.l0.w, cur.l1.x, cur.l1.y, cur.l1.z, cur.l1.w};
            const float er[8] = {cur.e0.x, cur.e0.y, cur.e0.z, cur.e0.w, cur.e1.x, cur.e1.y, cur.e1.z, cur.e1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const __bf16 kr = j < 4 ? cur.k0[j & 3] : cur.k1[j & 3];
                const __bf16 qr = j < 4 ? cur.q0[j & 3] : cur.q1[j & 3];
                kv[j] = valid ? (float)kr : 0.f;
                qv[j] = valid ? (float)qr : 0.f;
                ev[j] = valid ? er[j] * kv[j] : 0.f;   // e = b * k
                gs[j] = valid ? fmaxf(lr[j], kG2MinLogAlpha) * kG2Log2e : 0.f;
            }
        }
        scan(gs);
        if (x == 15) {
            *reinterpret_cast<float4*>(&sm.tot[b][32 * s + 4 * kg]) = make_float4(gs[0], gs[1], gs[2], gs[3]);
            *reinterpret_cast<float4*>(&sm.tot[b][32 * s + 16 + 4 * kg]) = make_float4(gs[4], gs[5], gs[6], gs[7]);
        }
        __syncthreads();
        float off[8], end[8], last[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) off[j] = end[j] = last[j] = 0.f;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            float tv[8];
            ld_tot(cb, s, tv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (cb < b) off[j] += tv[j];
                if (cb <= b) end[j] += tv[j];
                last[j] += tv[j];
                if (cb == b && !(-tv[j] <= kG2SafeSpan2)) unsafe = true;
            }
        }
        float g[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = gs[j] + off[j];
        {
            float eh[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float eg = __builtin_amdgcn_exp2f(g[j]);
                const float fh = __builtin_amdgcn_exp2f(last[j] - g[j]);
                qgk[2 * s + (j >> 2)][j & 3] = qv[j] * eg;
                khk[2 * s + (j >> 2)][j & 3] = kv[j] * fh;
                eh[j] = ev[j] * fh;
                const int c = chan(s, j);
                sm.kgt[c * LT + r] = (_Float16)(kv[j] * eg);
                sm.eht[c * LT + r] = (_Float16)eh[j];
            }
            __bf16* ehn = reinterpret_cast<__bf16*>(blk + L::EHN) + (size_t)r * DK + 32 * s + 4 * kg;
            *reinterpret_cast<bf16x4*>(ehn) = bf16x4{(__bf16)-eh[0], (__bf16)-eh[1], (__bf16)-eh[2], (__bf16)-eh[3]};
            *reinterpret_cast<bf16x4*>(ehn + 16) =
                bf16x4{(__bf16)-eh[4], (__bf16)-eh[5], (__bf16)-eh[6], (__bf16)-eh[7]};
        }
        if (b == 0 && x == 0) {
            float* vec = reinterpret_cast<float*>(blk + L::VEC) + 32 * s + 4 * kg;
            *reinterpret_cast<float4*>(vec) =
                make_float4(__builtin_amdgcn_exp2f(last[0]), __builtin_amdgcn_exp2f(last[1]),
                            __builtin_amdgcn_exp2f(last[2]), __builtin_amdgcn_exp2f(last[3]));
            *reinterpret_cast<float4*>(vec + 16) =
                make_float4(__builtin_amdgcn_exp2f(last[4]), __builtin_amdgcn_exp2f(last[5]),
                            __builtin_amdgcn_exp2f(last[6]), __builtin_amdgcn_exp2f(last[7]));
        }
        if constexpr (b < NB - 1) {   // B sides of this block, decayed to its end (factors <= 1)
            float kb[8], eb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f = __builtin_amdgcn_exp2f(end[j] - g[j]);
                kb[j] = kv[j] * f;
                eb[j] = ev[j] * f;
            }
            sm.u.g.bk[b][s][lane] = to8(kb);
            sm.u.g.be[b][s][lane] = to8(eb);
        }
        __syncthreads();
        // Blocks cb < b: A sides decayed from the end of block cb (factors <= 1).
        float ref[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ref[j] = 0.f;
#pragma unroll
        for (int cb = 0; cb < b; ++cb) {
            float tv[8], ka[8], qa[8];
            ld_tot(cb, s, tv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ref[j] += tv[j];
                const float f = __builtin_amdgcn_exp2f(g[j] - ref[j]);
                ka[j] = kv[j] * f;
                qa[j] = qv[j] * f;
            }
            const bf16x8 kab = to8(ka), qab = to8(qa);
            const bf16x8 bkf = sm.u.g.bk[cb][s][lane], bef = sm.u.g.be[cb][s][lane];
            lk[cb] = M::mma(bkf, kab, lk[cb]);
            le[cb] = M::mma(bef, kab, le[cb]);
            pk[cb] = M::mma(bkf, qab, pk[cb]);
            pe[cb] = M::mma(bef, qab, pe[cb]);
        }
        // Diagonal block: decay split at the block start (B-side factors >= 1,
        // bounded by the span check).
        {
            float ka[8], qa[8], kd[8], ed[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f = __builtin_amdgcn_exp2f(gs[j]);
                const float fi = __builtin_amdgcn_exp2f(-gs[j]);
                ka[j] = kv[j] * f;
                qa[j] = qv[j] * f;
                kd[j] = kv[j] * fi;
                ed[j] = ev[j] * fi;
            }
            const bf16x8 kab = to8(ka), qab = to8(qa), kdb = to8(kd), edb = to8(ed);
            lk[b] = M::mma(kdb, kab, lk[b]);
            le[b] = M::mma(edb, kab, le[b]);
            pk[b] = M::mma(kdb, qab, pk[b]);
            pe[b] = M::mma(edb, qab, pe[b]);
        }
    }
    if (__ballot(unsafe) != 0) {   // wave-uniform, rare: exact diagonal block, pair by pair
        f32x4 xk = zero4(), xe = zero4(), xpk = zero4(), xpe = zero4();
#pragma unroll 1
        for (int y = 0; y < 16; ++y) {
            float ak = 0.f, ae = 0.f, apk = 0.f, ape = 0.f;
#pragma unroll 1
            for (int s = 0; s < NS; ++s) {
                float gs[8], kv[8], qv[8], ev[8];
                ld_la(s, gs);
                ld_bf(k, s, kv);
                ld_bf(q, s, qv);
                ld_f(erase, s, ev);
                scan(gs);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float ky = __shfl(kv[j], y + 16 * kg);
                    const float ey = __shfl(ev[j] * kv[j], y + 16 * kg);
                    const float gy = __shfl(gs[j], y + 16 * kg);
                    const float f = y <= x ? __builtin_amdgcn_exp2f(gs[j] - gy) : 0.f;
                    ak += kv[j] * ky * f;
                    ae += kv[j] * ey * f;
                    apk += qv[j] * ky * f;
                    ape += qv[j] * ey * f;
                }
            }
            ak += __shfl_xor(ak, 16);
            ak += __shfl_xor(ak, 32);
            ae += __shfl_xor(ae, 16);
            ae += __shfl_xor(ae, 32);
            apk += __shfl_xor(apk, 16);
            apk += __shfl_xor(apk, 32);
            ape += __shfl_xor(ape, 16);
            ape += __shfl_xor(ape, 32);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (y == 4 * kg + e) {
                    xk[e] = ak;
                    xe[e] = ae;
                    xpk[e] = apk;
                    xpe[e] = ape;
                }
        }
        lk[b] = xk;
        le[b] = xe;
        pk[b] = xpk;
        pe[b] = xpe;
    }
    // masks: L strictly lower, P lower with the diagonal
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int cl = 4 * kg + e;
        lk[b][e] = cl < x ? lk[b][e] : 0.f;
        le[b][e] = cl < x ? le[b][e] : 0.f;
        pk[b][e] = cl <= x ? pk[b][e] : 0.f;
        pe[b][e] = cl <= x ? pe[b][e] : 0.f;
    }
    __syncthreads();   // the Gram B sides are dead; their LDS is reused below

    // ---- phase 2: Ti = (I + L_e)^-1 ----
    float* xab = sm.xa[b];
    float* xxb = sm.xx[b];
#pragma unroll
    for (int e = 0; e < 4; ++e) xab[(4 * kg + e) * 16 + x] = le[b][e];   // xab[m][i] = L_e[i][m]
    wave_sync();
    {   // lane x (mod 16) builds column x of (I + L_e,bb)^-1 by forward substitution
        float xv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) xv[i] = i == x ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            float am[16];
#pragma unroll
            for (int qd = (m + 1) / 4; qd < 4; ++qd) {
                const float4 t = *reinterpret_cast<const float4*>(xab + m * 16 + 4 * qd);
                am[4 * qd] = t.x; am[4 * qd + 1] = t.y; am[4 * qd + 2] = t.z; am[4 * qd + 3] = t.w;
            }
#pragma unroll
            for (int i = m + 1; i < 16; ++i) xv[i] -= am[i] * xv[m];
        }
        if (kg == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) xxb[i * 17 + x] = xv[i];
        }
    }
    wave_sync();
    f32x4 xr, tt[NB];   // X_bb in R layout; Ti row block b (column blocks <= b), A layout
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        xr[e] = xxb[x * 17 + 4 * kg + e];
        tt[b][e] = xxb[(4 * kg + e) * 17 + x];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (j != b) tt[j] = zero4();
    if constexpr (b < NB - 1) sm.u.s.tpub[tri_idx(b, b)][lane] = h4(tt[b]);
    // row wavefront: Ti_tj = -X_tt sum_{m=j}^{t-1} L_e[t][m] Ti_mj, on wave t
#pragma unroll
    for (int t = 1; t < NB; ++t) {
        __syncthreads();
        if (b == t) {
#pragma unroll
            for (int j = 0; j < t; ++j) {
                f32x4 y = zero4();
#pragma unroll
                for (int m = j; m < t; ++m) y = mma16(h4(le[m]), sm.u.s.tpub[tri_idx(m, j)][lane], y);
                tt[j] = -mma16(h4(xr), h4(y), zero4());
                if (t < NB - 1) sm.u.s.tpub[tri_idx(t < NB - 1 ? t : 0, j)][lane] = h4(tt[j]);
            }
        }
    }
    // publish Ti and L_k (row-major f16, lower blocks)
#pragma unroll
    for (int j = 0; j <= b; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.u.s.ti[(16 * b + 4 * kg + e) * LT + 16 * j + x] = (_Float16)tt[j][e];
#pragma unroll
    for (int cb = 0; cb <= b; ++cb)
        *reinterpret_cast<f16x4*>(&sm.u.s.lk[(16 * b + x) * LT + 16 * cb + 4 * kg]) = h4(lk[cb]);
    __syncthreads();

    // ---- phase 3: Z, M, PP, W, QP, KHP ----
    f32x4 z[NB];   // Z[b][m], R layout
#pragma unroll
    for (int m = 0; m <= b; ++m) {
        z[m] = zero4();
#pragma unroll
        for (int j = m; j <= b; ++j) {
            f16x4 a;   // A layout of Ti[j][m]
            if (j == b) {
                a = h4(tt[m]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = sm.u.s.ti[(16 * j + 4 * kg + e) * LT + 16 * m + x];
            }
            z[m] = mma16(a, h4(pe[j]), z[m]);
        }
    }
    f16x4 tib[NB], nz[NB];   // R layout of Ti[b][m] and of -Z[b][m]
#pragma unroll
    for (int m = 0; m <= b; ++m) {
        tib[m] = *reinterpret_cast<const f16x4*>(&sm.u.s.ti[(16 * b + x) * LT + 16 * m + 4 * kg]);
        nz[m] = h4(-z[m]);
    }
    // M[b][nb] (A layout, published) and PP[b][nb] (R layout), nb <= b
    f32x4 pp[NB];
#pragma unroll
    for (int nb = 0; nb <= b; ++nb) {
        f32x4 mm = zero4();
        pp[nb] = pk[nb];
#pragma unroll
        for (int m = nb; m <= b; ++m) {
            f16x4 lkc;   // A layout of L_k[m][nb]
#pragma unroll
            for (int e = 0; e < 4; ++e) lkc[e] = sm.u.s.lk[(16 * m + 4 * kg + e) * LT + 16 * nb + x];
            mm = mma16(tib[m], lkc, mm);
            pp[nb] = mma16(lkc, nz[m], pp[nb]);
        }
        sm.u.s.m1[tri_idx(b, nb)][lane] = h4(mm);
    }
    // W = Ti Kg and QP = Qg - Z Kg (R layout), per 16-channel tile
#pragma unroll
    for (int cc = 0; cc < NCT; ++cc) {
        f32x4 wa = zero4(), qa = qgk[cc];
#pragma unroll
        for (int m = 0; m <= b; ++m) {
            const f16x4 a = *reinterpret_cast<const f16x4*>(&sm.kgt[(16 * cc + x) * LT + 16 * m + 4 * kg]);
            wa = mma16(a, tib[m], wa);
            qa = mma16(a, nz[m], qa);
        }
        const size_t o = ((size_t)r * DK + 16 * cc + 4 * kg) * 2;
        *reinterpret_cast<bf16x4*>(blk + L::W + o) = b4(wa);
        *reinterpret_cast<bf16x4*>(blk + L::QP + o) = b4(qa);
    }
    // PP rows, zero above the diagonal blocks
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<bf16x4*>(blk + L::PP + ((size_t)r * GC + 16 * nb + 4 * kg) * 2) =
            b4(nb <= b ? pp[nb] : zero4());
    __syncthreads();   // every M block published
    // KHP = Kh - M^T Eh (R layout): block jb >= b of M^T's row block b is M[jb][b]
#pragma unroll
    for (int cc = 0; cc < NCT; ++cc) {
        f32x4 ka = khk[cc];
#pragma unroll
        for (int jb = b; jb < NB; ++jb) {
            const f16x4 a = *reinterpret_cast<const f16x4*>(&sm.eht[(16 * cc + x) * LT + 16 * jb + 4 * kg]);
            ka = mma16(a, -sm.u.s.m1[tri_idx(jb, b)][lane], ka);
        }
        *reinterpret_cast<bf16x4*>(blk + L::KHP + ((size_t)r * DK + 16 * cc + 4 * kg) * 2) = b4(ka);
    }
}

}  // namespace

template <int DK, bool CH>
__global__ __launch_bounds__(256, 2) void gdn2_prep(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                    const float* __restrict__ log_alpha,
                                                    const float* __restrict__ erase, uint8_t* __restrict__ ws,
                                                    int64_t T, int H, int NT) {
    __shared__ G2PrepSmem<DK> sm;
    const int w = threadIdx.x >> 6;
    if (w == 0) gdn2_prep_wave<DK, 0, CH>(sm, q, k, log_alpha, erase, ws, T, H, NT);
    if (w == 1) gdn2_prep_wave<DK, 1, CH>(sm, q, k, log_alpha, erase, ws, T, H, NT);
    if (w == 2) gdn2_prep_wave<DK, 2, CH>(sm, q, k, log_alpha, erase, ws, T, H, NT);
    if (w == 3) gdn2_prep_wave<DK, 3, CH>(sm, q, k, log_alpha, erase, ws, T, H, NT);
}

// ---------------------------------------------------------------------------
// Sequential pass.
// ---------------------------------------------------------------------------
namespace {

template <int DK, int NW>
struct G2Stage {
    static constexpr int VT = 16 * NW, NL = 2;
    using DQ = DmaTile<GC, DK * 2, NL>;    // W, QP, KHP, EHN
    using DT = DmaTile<GC, GC * 2, NL>;    // PP
    using DVt = DmaTile<GC, VT * 2, NL>;   // V (bf16)
    using DWt = DmaTile<GC, VT * 4, NL>;   // w (fp32)
    static constexpr int LQ = DK + 8, LT = GC + 8, LV = VT + 8, LW = VT + 4;
    static constexpr int QB = DQ::BYTES, TB = DT::BYTES, VB = DVt::BYTES, WB = DWt::BYTES;
    // double-buffered part, used by the products of the chunk
    static constexpr int OW = 0, OQP = QB, OPP = 2 * QB, OV = OPP + TB, OWR = OV + VB;
    static constexpr int ABYTES = (OWR + WB + 15) / 16 * 16;
    // single part, used by the state update at the end of the chunk
    static constexpr int OKHP = 2 * ABYTES, OEHN = OKHP + QB, OVEC = OEHN + QB;
    static constexpr int LO = 16 + 8;      // output staging row (bf16)
    static constexpr int OSTG = (OVEC + DK * 4 + 15) / 16 * 16;
    static constexpr int OWARM = (OSTG + NW * GC * LO * 2 + 15) / 16 * 16;   // L2-warming loads land here
    static constexpr int TOTAL = OWARM + 256;
};

// S^T <- Diag(gamma_C) S^T + KHP^T Vt + EHN^T X for the chunk whose single part
// is in LDS.
template <int DK, int NW>
__device__ __forceinline__ void gdn2_state_update(f32x4* S, const bf16x8* vb, const bf16x8* xb,
                                                  const char* smem, int g4, int lane) {
    using SL = G2Stage<DK, NW>;
    using M = Mma<__bf16>;
    constexpr int NKT = GC / 32, CT = DK / 16;
    const __bf16* khs = reinterpret_cast<const __bf16*>(smem + SL::OKHP);
    const __bf16* ehs = reinterpret_cast<const __bf16*>(smem + SL::OEHN);
    const float* vec = reinterpret_cast<const float*>(smem + SL::OVEC);
#pragma unroll
    for (int mc = 0; mc < CT; ++mc) {
        const float4 gl = *reinterpret_cast<const float4*>(vec + 16 * mc + 4 * g4);
        S[mc][0] *= gl.x; S[mc][1] *= gl.y; S[mc][2] *= gl.z; S[mc][3] *= gl.w;
    }
#pragma unroll
    for (int s = 0; s < NKT; ++s) {
        bf16x8 kf[CT], ef[CT];
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) {
            kf[mc] = afrag_tr_tok<__bf16, false>(khs, SL::LQ, 16 * mc, s, lane);
            ef[mc] = afrag_tr_tok<__bf16, false>(ehs, SL::LQ, 16 * mc, s, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) {
            S[mc] = M::mma(kf[mc], vb[s], S[mc]);
            S[mc] = M::mma(ef[mc], xb[s], S[mc]);
        }
    }
}

__device__ __forceinline__ int64_t g2_row0(int64_t b, int64_t h, int n, int64_t T, int H) {
    return (b * T + (int64_t)n * GC) * H + h;
}
__device__ __forceinline__ int g2_len(int n, int64_t T) {
    return (int)((T - (int64_t)n * GC) < GC ? (T - (int64_t)n * GC) : GC);
}

// Loader wave lw: chunk n's double-buffered part goes to buffer n & 1 one
// chunk ahead; its single part is copied during the chunk's own products.
template <int DK, int NW>
__device__ __forceinline__ void gdn2_loader(char* smem, const __bf16* v, const float* wr, const uint8_t* ws,
                                            int64_t b, int64_t h, int64_t T, int H, int NT, int DV, int vt,
                                            int lw, int lane) {
    using SL = G2Stage<DK, NW>;
    using L = G2Ws<DK>;
    using DQ = typename SL::DQ;
    using DT = typename SL::DT;
    using DVt = typename SL::DVt;
    using DWt = typename SL::DWt;
    constexpr int VT = SL::VT;
    const int64_t bh = b * H + h;
    int oq[DQ::PER_WAVE], ot[DT::PER_WAVE], ov[DVt::PER_WAVE], ow[DWt::PER_WAVE];
    DQ::offsets(oq, DK * 2, GC, lw, lane);
    DT::offsets(ot, GC * 2, GC, lw, lane);
    DVt::offsets(ov, (int64_t)H * DV * 2, g2_len(0, T), lw, lane);
    DWt::offsets(ow, (int64_t)H * DV * 4, g2_len(0, T), lw, lane);
    for (int n = -1; n < NT; ++n) {
        if (n > 0) __syncthreads();                                        // B1
        if (n >= 0) {   // single part of chunk n
            const char* blk = reinterpret_cast<const char*>(ws + (size_t)(bh * NT + n) * L::BYTES);
            DQ::issue(smem + SL::OKHP, blk + L::KHP, oq, lw);
            DQ::issue(smem + SL::OEHN, blk + L::EHN, oq, lw);
            constexpr int NVEC = DK * 4 / 16;
            for (int s = lw * 64 + lane; s < NVEC; s += SL::NL * 64)
                __builtin_amdgcn_global_load_lds(blk + L::VEC + 16 * s,
                                                 (GDR_LDS void*)(smem + SL::OVEC + 16 * (s - lane)), 16, 0, 0);
        }
        const int na = n + 1;   // double-buffered part of chunk n + 1
        if (na < NT) {
            const int len = g2_len(na, T);
            if (len < GC) {   // ragged last chunk: rows past len repeat row len - 1
                DVt::offsets(ov, (int64_t)H * DV * 2, len, lw, lane);
                DWt::offsets(ow, (int64_t)H * DV * 4, len, lw, lane);
            }
            char* base = smem + (na & 1) * SL::ABYTES;
            const char* blk = reinterpret_cast<const char*>(ws + (size_t)(bh * NT + na) * L::BYTES);
            const int64_t row0 = g2_row0(b, h, na, T, H);
            DQ::issue(base + SL::OW, blk + L::W, oq, lw);
            DQ::issue(base + SL::OQP, blk + L::QP, oq, lw);
            DT::issue(base + SL::OPP, blk + L::PP, ot, lw);
            DVt::issue(base + SL::OV, reinterpret_cast<const char*>(v + row0 * DV + vt * VT), ov, lw);
            DWt::issue(base + SL::OWR, reinterpret_cast<const char*>(wr + row0 * DV + vt * VT), ow, lw);
        }
        // Warm L2 with chunk n + 2: this workgroup's share of the head's
        // workspace block (one 4-byte load per 128-byte line, a fixed number
        // of loads per wave, lanes past the share repeating its last line),
        // then its own V (loader 0) or w (loader 1) rows.  The copies above
        // are waited for; the warming loads stay in flight.
        constexpr int NLINES = (int)((L::BYTES + 127) / 128);
        constexpr int NVT = DK / VT;
        constexpr int PER = (NLINES + NVT - 1) / NVT;
        constexpr int ROUNDS = (PER + 2 * 64 - 1) / (2 * 64);
        const int nw = n + 2;
        if (nw >= 0 && nw < NT) {
            const char* blk = reinterpret_cast<const char*>(ws + (size_t)(bh * NT + nw) * L::BYTES);
            const int lo = vt * PER, hi = (lo + PER < NLINES ? lo + PER : NLINES);
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j) {
                const int i = lo + (2 * j + lw) * 64 + lane;
                __builtin_amdgcn_global_load_lds(blk + 128 * (i < hi ? i : hi - 1), (GDR_LDS void*)(smem + SL::OWARM), 4, 0, 0);
            }
            const int len = g2_len(nw, T);
            const int64_t r = g2_row0(b, h, nw, T, H) + (int64_t)(lane < len ? lane : len - 1) * H;
            if (lw == 0)
                __builtin_amdgcn_global_load_lds(v + r * DV + vt * VT, (GDR_LDS void*)(smem + SL::OWARM), 4, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(wr + r * DV + vt * VT, (GDR_LDS void*)(smem + SL::OWARM), 4, 0, 0);
            static_assert(ROUNDS + 1 <= 15, "vmcnt field");
            __builtin_amdgcn_s_waitcnt(0x0F70 | (ROUNDS + 1));
        } else {
            wait_dma();
        }
        __syncthreads();                                                   // B0 (n = -1) or B2
    }
}

}  // namespace

template <int DK, int NW>
__global__ __launch_bounds__(64 * (NW + 2)) __attribute__((amdgpu_waves_per_eu(1, 1))) void gdn2_state_pass(
    const __bf16* __restrict__ v, const float* __restrict__ wr, const float* __restrict__ S0,
    __bf16* __restrict__ o, float* __restrict__ ST, const uint8_t* __restrict__ ws, int64_t T, int H, int NT,
    int DV) {
    using SL = G2Stage<DK, NW>;
    using M = Mma<__bf16>;
    constexpr int VT = SL::VT;
    constexpr int NKC = DK / 32, NKT = GC / 32, MT = GC / 16, CT = DK / 16;
    static_assert(SL::TOTAL <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char smem[SL::TOTAL];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, col = lane & 15;
    const int NVT = DV / VT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = bid % NVT;
    const int64_t bh = bid / NVT;
    const int64_t b = bh / H, h = bh % H;

    // Waves NW and NW+1 copy global -> LDS; both roles pass the same barriers:
    //   B0;  chunk n: [n > 0: B1] B2.
    if (wave >= NW) {
        gdn2_loader<DK, NW>(smem, v, wr, ws, b, h, T, H, NT, DV, vt, wave - NW, lane);
        return;
    }

    const int vcol = vt * VT + 16 * wave + col;   // this lane's value column
    __bf16* ostg = reinterpret_cast<__bf16*>(smem + SL::OSTG + wave * GC * SL::LO * 2);
    f32x4 S[CT];   // S^T tile mc: lane (v, g) holds channel 16mc + 4g + i
#pragma unroll
    for (int mc = 0; mc < CT; ++mc) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S0) x = *reinterpret_cast<const float4*>(S0 + (bh * DV + vcol) * DK + 16 * mc + 4 * g4);
        S[mc] = f32x4{x.x, x.y, x.z, x.w};
    }
    bf16x8 vb[NKT], xb[NKT];   // Vt and X as B operands, carried to the state update
    __syncthreads();                                                       // B0

    for (int n = 0; n < NT; ++n) {
        if (n > 0) {
            gdn2_state_update<DK, NW>(S, vb, xb, smem, g4, lane);
            __syncthreads();                                               // B1
            store_out<__bf16, GC, SL::LO>(o, ostg, g2_row0(b, h, n - 1, T, H), H, DV, vt * VT + 16 * wave, GC, lane);
        }
        const char* st = smem + (n & 1) * SL::ABYTES;
        const __bf16* Ws = reinterpret_cast<const __bf16*>(st + SL::OW);
        const __bf16* QPs = reinterpret_cast<const __bf16*>(st + SL::OQP);
        const __bf16* PPs = reinterpret_cast<const __bf16*>(st + SL::OPP);
        const __bf16* Vs = reinterpret_cast<const __bf16*>(st + SL::OV);
        const float* wrs = reinterpret_cast<const float*>(st + SL::OWR);

        // X = W S^T, O = QP S^T (rows = tokens, cols = v)
        bf16x8 sb[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) sb[s] = bfrag_acc<__bf16>(S, s);
        f32x4 X[MT], Oa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) X[mt] = Oa[mt] = zero4();
#pragma unroll
        for (int s0 = 0; s0 < NKC; s0 += 2) {
            bf16x8 wf[2][MT], qf[2][MT];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    wf[s][mt] = afrag_nat<__bf16>(Ws, SL::LQ, 16 * mt, s0 + s, lane);
                    qf[s][mt] = afrag_nat<__bf16>(QPs, SL::LQ, 16 * mt, s0 + s, lane);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    X[mt] = M::mma(wf[s][mt], sb[s0 + s], X[mt]);
                    Oa[mt] = M::mma(qf[s][mt], sb[s0 + s], Oa[mt]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Vt = w * v (accumulator layout)
        f32x4 vt4[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * mt + 4 * g4 + i;
                vt4[mt][i] = (float)Vs[rr * SL::LV + 16 * wave + col] * wrs[rr * SL::LW + 16 * wave + col];
            }
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            vb[s] = bfrag_acc<__bf16>(vt4, s);
            xb[s] = bfrag_acc<__bf16>(X, s);
        }
        // O += PP Vt
        {
            bf16x8 pf[MT][NKT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < NKT; ++s) pf[mt][s] = afrag_nat_tok<__bf16, false>(PPs, SL::LT, 16 * mt, s, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NKT; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) Oa[mt] = M::mma(pf[mt][s], vb[s], Oa[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ostg[(16 * mt + 4 * g4 + i) * SL::LO + col] = (__bf16)Oa[mt][i];
        __syncthreads();                                                   // B2
    }
    gdn2_state_update<DK, NW>(S, vb, xb, smem, g4, lane);
    store_out<__bf16, GC, SL::LO>(o, ostg, g2_row0(b, h, NT - 1, T, H), H, DV, vt * VT + 16 * wave,
                                  g2_len(NT - 1, T), lane);
    if (ST) {
#pragma unroll
        for (int mc = 0; mc < CT; ++mc)
            *reinterpret_cast<float4*>(ST + (bh * DV + vcol) * DK + 16 * mc + 4 * g4) =
                make_float4(S[mc][0], S[mc][1], S[mc][2], S[mc][3]);
    }
}

namespace {

template <int DK, bool CH>
hipError_t launch_gdn2_chunk(const Gdn2Args& a, void* ws) {
    const int NT = (int)((a.T + GC - 1) / GC);
    const int H = (int)a.H, DV = (int)a.dv;
    const int64_t units = a.B * a.H;
    hipLaunchKernelGGL((gdn2_prep<DK, CH>), dim3((unsigned)(units * NT)), dim3(256), 0, a.stream,
                       reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const __bf16*>(a.k), a.log_alpha,
                       a.erase, reinterpret_cast<uint8_t*>(ws), a.T, H, NT);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool two = units * (a.dv / 32) >= 256;
    if (two) {
        hipLaunchKernelGGL((gdn2_state_pass<DK, 2>), dim3((unsigned)(units * (a.dv / 32))), dim3(64 * 4), 0,
                           a.stream, reinterpret_cast<const __bf16*>(a.v), a.write, a.S0,
                           reinterpret_cast<__bf16*>(a.o), a.S_T, reinterpret_cast<const uint8_t*>(ws), a.T, H,
                           NT, DV);
    } else {
        hipLaunchKernelGGL((gdn2_state_pass<DK, 1>), dim3((unsigned)(units * (a.dv / 16))), dim3(64 * 3), 0,
                           a.stream, reinterpret_cast<const __bf16*>(a.v), a.write, a.S0,
                           reinterpret_cast<__bf16*>(a.o), a.S_T, reinterpret_cast<const uint8_t*>(ws), a.T, H,
                           NT, DV);
    }
    return hipGetLastError();
}

}  // namespace

bool gdn2_chunk_supported(int64_t dk, int64_t dv, int64_t chunk, bool bf16) {
    return bf16 && chunk == GC && dk == dv && (dk == 64 || dk == 128);
}

size_t gdn2_chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk) {
    const int64_t nt = (T + GC - 1) / GC;
    const size_t blk = dk == 64 ? G2Ws<64>::BYTES : G2Ws<128>::BYTES;
    return (size_t)(B * H * nt) * blk;
}

hipError_t gdn2_chunk_fwd_launch(const Gdn2Args& a, void* ws) {
    if (a.dk == 128) return a.channel ? launch_gdn2_chunk<128, true>(a, ws) : launch_gdn2_chunk<128, false>(a, ws);
    return a.channel ? launch_gdn2_chunk<64, true>(a, ws) : launch_gdn2_chunk<64, false>(a, ws);
}

}  // namespace gdr
