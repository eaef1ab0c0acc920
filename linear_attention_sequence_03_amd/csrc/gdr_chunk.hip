// gdr_chunk.hip -- chunkwise-parallel WY forward pass of the gated delta rule
// ("FG2-GDN" page, section 3.6, Chunkwise Parallel Training: split the sequence
// into chunks of C tokens, accumulate the tied diagonal-plus-rank-1 transitions
// of a chunk with the WY representation and the UT transform, solve a
// triangular system for the UT factor, propagate the state between chunks and
// add the intra-chunk causal product).
//
// Derivation used here (state S is dv x dk, o_t = S_t q_t).  Inside a chunk
// that starts from state S, with g_r = sum_{j<=r} log alpha_j (a scalar for
// Gated DeltaNet, a dk-vector for KDA), gamma_r = exp(g_r), rows r,i < C:
//   A[r][i] = beta_r * sum_c k_rc k_ic exp(g_rc - g_ic)        (i < r, else 0)
//   T       = (I + A)^-1 Diag(beta)                              (UT factor)
//   D       = T (V - Kg S^T),       Kg[r] = k_r * gamma_r        (written values u_r)
//   P[r][i] = sum_c q_rc k_ic exp(g_rc - g_ic)                  (i <= r, else 0)
//   O       = Qg S^T + P D,         Qg[r] = q_r * gamma_r
//   S_next  = S Diag(gamma_last) + D^T Kh,  Kh[r] = k_r * gamma_last / gamma_r
// which is exactly the token recurrence reorganised (no approximation).
//
// Two kernels per call:
//  1. wy_prep  -- one workgroup per (b, h, chunk), fully parallel: the decay
//     cumsum, A and P on the matrix cores, the triangular solve in LDS (fp32),
//     and T, P (and the gate-scaled operands for the channel gate) into the
//     workspace.
//  2. state_pass -- one workgroup per (b, h, dv-slice of VT columns): walks the
//     chunks in order carrying its fp32 state slice in LDS; per chunk three
//     dependent MFMA phases (R = V - Kg S^T and Qg S^T; D = T R; O += P D and
//     S <- S Diag(gamma_last) + D^T Kh).  dv-slices are independent, which is
//     what gives the sequential part enough workgroups to fill the chip.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int X, int A> struct RoundUp { static constexpr int v = (X + A - 1) / A * A; };

// Byte layout of one (b, h, chunk) workspace block.
template <typename E, int DK, int C, bool CHANNEL>
struct WsLayout {
    static constexpr size_t T = 0;                                   // E [C][C]
    static constexpr size_t P = T + (size_t)C * C * sizeof(E);       // E [C][C]
    static constexpr size_t G = P + (size_t)C * C * sizeof(E);       // f32 [C]   (scalar)
    static constexpr size_t QG = G;                                  // E [C][DK] (channel)
    static constexpr size_t KG = QG + (size_t)C * DK * sizeof(E);    // E [C][DK]
    static constexpr size_t KH = KG + (size_t)C * DK * sizeof(E);    // E [C][DK]
    static constexpr size_t GL = KH + (size_t)C * DK * sizeof(E);    // f32 [DK]
    static constexpr size_t END = CHANNEL ? GL + DK * 4 : G + C * 4;
    static constexpr size_t BYTES = (END + 255) / 256 * 256;
};

// Copy a [ROWS][COLS] tile of E from global (row stride gstride elements) into
// LDS (row stride ls elements); rows >= valid are zero-filled.  16-byte moves.
template <typename E, int ROWS, int COLS>
__device__ __forceinline__ void g2s(E* dst, int ls, const E* src, int64_t gstride, int valid,
                                    int tid) {
    constexpr int EPS = 16 / sizeof(E);
    constexpr int SEGS = COLS / EPS;
#pragma unroll 4
    for (int idx = tid; idx < ROWS * SEGS; idx += kThreads) {
        const int r = idx / SEGS, s = idx % SEGS;
        const V16 x = r < valid ? ld16(src + r * gstride + s * EPS) : zero16();
        st16(dst + r * ls + s * EPS, x);
    }
}

// Triangular solve in LDS: Xs <- (I + As)^-1 for a strictly lower C x C matrix
// As (fp32, row stride LA).  Diagonal 16x16 blocks by forward substitution (one
// lane per column, all diagonal blocks at once in wave 0); off-diagonal blocks
// by increasing distance from the diagonal:
//   X_ij = -X_ii * sum_{m=j}^{i-1} A_im X_mj
// with fp32 16x16x4 MFMAs.  Ys: scratch of (C/16 - 1) 16x17 fp32 tiles.
template <int C, int LA>
__device__ __forceinline__ void solve_unit_lower(const float* As, float* Xs, float* Ys, int tid) {
    constexpr int NB = C / 16;
    const int lane = tid & 63, wave = tid >> 6;
    if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        if (blk < NB) {
            const float* Ab = As + (16 * blk) * LA + 16 * blk;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s -= Ab[i * LA + m] * x[m];
                x[i] = s;
            }
            float* Xb = Xs + (16 * blk) * LA + 16 * blk;
#pragma unroll
            for (int i = 0; i < 16; ++i) Xb[i * LA + j] = x[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        for (int p = wave; p < NB - d; p += kWaves) {
            const int i = p + d, j = p;
            f32x4 y = zero4();
            for (int m = j; m < i; ++m) {
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4) {
                    const float a = As[(16 * i + (lane & 15)) * LA + 16 * m + kk + (lane >> 4)];
                    const float b = Xs[(16 * m + kk + (lane >> 4)) * LA + 16 * j + (lane & 15)];
                    y = Mma<float>::mma(a, b, y);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ys[p * 16 * 17 + acc_row(lane, e) * 17 + acc_col(lane)] = y[e];
        }
        __syncthreads();
        for (int p = wave; p < NB - d; p += kWaves) {
            const int i = p + d, j = p;
            f32x4 x = zero4();
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4) {
                const float a = Xs[(16 * i + (lane & 15)) * LA + 16 * i + kk + (lane >> 4)];
                const float b = Ys[p * 16 * 17 + (kk + (lane >> 4)) * 17 + (lane & 15)];
                x = Mma<float>::mma(a, b, x);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Xs[(16 * i + acc_row(lane, e)) * LA + 16 * j + acc_col(lane)] = -x[e];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Kernel 1, scalar gate (Gated DeltaNet).
// ---------------------------------------------------------------------------
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void wy_prep_scalar(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, uint8_t* __restrict__ ws, int64_t T, int H, int NT) {
    using L = WsLayout<E, DK, C, false>;
    using M = Mma<E>;
    constexpr int LDK = DK + Pad<E>::v;
    constexpr int NB = C / 16;
    constexpr int LA = C + 1;
    __shared__ __attribute__((aligned(16))) E Ks[C * LDK];
    __shared__ __attribute__((aligned(16))) E Qs[C * LDK];
    __shared__ float As[C * LA];
    __shared__ float Xs[C * LA];
    __shared__ float Ys[(NB > 1 ? NB - 1 : 1) * 16 * 17];
    __shared__ float gs[C], bs[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bid = blockIdx.x;
    const int n = (int)(bid % NT);
    const int64_t bh = bid / NT;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = (int64_t)n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t row0 = ((b * T + t0) * H + h);   // token-row index of row 0

    g2s<E, C, DK>(Ks, LDK, k + row0 * DK, (int64_t)H * DK, len, tid);
    g2s<E, C, DK>(Qs, LDK, q + row0 * DK, (int64_t)H * DK, len, tid);
    for (int idx = tid; idx < C * LA; idx += kThreads) { As[idx] = 0.f; Xs[idx] = 0.f; }
    if (wave == 0) {
        float x = 0.f, bb = 0.f;
        if (lane < len) {
            x = log_alpha[row0 + (int64_t)lane * H];
            bb = beta[row0 + (int64_t)lane * H];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane < C) { gs[lane] = x; bs[lane] = bb; }
    }
    __syncthreads();

    uint8_t* blk = ws + (size_t)bid * L::BYTES;
    E* Tw = reinterpret_cast<E*>(blk + L::T);
    E* Pw = reinterpret_cast<E*>(blk + L::P);

    // Lower block tiles of A = K K^T (gated) and P = Q K^T (gated).
    constexpr int NTILE = NB * (NB + 1) / 2;
    for (int t = wave; t < 2 * NTILE; t += kWaves) {
        const bool isP = t >= NTILE;
        const int tt = isP ? t - NTILE : t;
        int rb = 0;
        while ((rb + 1) * (rb + 2) / 2 <= tt) ++rb;
        const int cb = tt - rb * (rb + 1) / 2;
        const E* Ap = isP ? Qs : Ks;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += M::KS)
            acc = M::mma(frag_rk(Ap, LDK, 16 * rb, k0, lane), frag_rk(Ks, LDK, 16 * cb, k0, lane),
                         acc);
        const int col = 16 * cb + acc_col(lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * rb + acc_row(lane, e);
            const bool keep = isP ? (col <= row) : (col < row);
            const float dec = keep ? expf(gs[row] - gs[col]) : 0.f;
            if (isP)
                Pw[row * C + col] = from_f32<E>(keep ? acc[e] * dec : 0.f);
            else
                As[row * LA + col] = keep ? acc[e] * bs[row] * dec : 0.f;
        }
    }
    // Upper blocks of P are zero.
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) Pw[idx] = from_f32<E>(0.f);
    }
    __syncthreads();

    solve_unit_lower<C, LA>(As, Xs, Ys, tid);

    // T = X Diag(beta), lower triangle; g for the state pass.
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        Tw[idx] = from_f32<E>(c <= r ? Xs[r * LA + c] * bs[c] : 0.f);
    }
    float* gw = reinterpret_cast<float*>(blk + L::G);
    if (tid < C) gw[tid] = gs[tid];
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential state pass over the chunks of one (b, h, dv-slice).
// ---------------------------------------------------------------------------
template <typename E, int DK, int C, int VT, bool CHANNEL>
__global__ __launch_bounds__(kThreads) void state_pass(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ S0, E* __restrict__ o, float* __restrict__ ST,
    const uint8_t* __restrict__ ws, int64_t T, int H, int NT, int DV) {
    using L = WsLayout<E, DK, C, CHANNEL>;
    using M = Mma<E>;
    constexpr int PAD = Pad<E>::v;
    constexpr int LDK = DK + PAD;          // Q / K rows
    constexpr int CK = C > M::KS ? C : M::KS; // contraction length over tokens (zero padded)
    constexpr int LC = CK + PAD;           // T / P / R^T / D^T rows
    constexpr int LV = VT + PAD;           // V rows
    constexpr int LS = DK + 4;             // fp32 state rows
    constexpr int MT = C / 16, NTL = VT / 16, TA = MT * NTL, TS = (DK / 16) * NTL;
    constexpr int SLOTS = (TA + kWaves - 1) / kWaves;

    // Q/K tiles hold CK rows: the S update contracts over tokens in steps of
    // the MFMA K, so rows C..CK-1 (only when C < K) must exist and be zero.
    __shared__ __attribute__((aligned(16))) E Qs[CK * LDK];
    __shared__ __attribute__((aligned(16))) E Ks[CK * LDK];
    __shared__ __attribute__((aligned(16))) E Khs[CHANNEL ? CK * LDK : 8];
    __shared__ __attribute__((aligned(16))) E Ts[C * LC];
    __shared__ __attribute__((aligned(16))) E Ps[C * LC];
    __shared__ __attribute__((aligned(16))) E Vs[C * LV];
    __shared__ __attribute__((aligned(16))) E Rt[VT * LC];
    __shared__ __attribute__((aligned(16))) E Dt[VT * LC];
    __shared__ __attribute__((aligned(16))) E Dst[CHANNEL ? 8 : VT * LC];
    __shared__ __attribute__((aligned(16))) float Ss[VT * LS];
    __shared__ float gs[CHANNEL ? DK : C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NVT = DV / VT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = bid % NVT;
    const int64_t bh = bid / NVT;
    const int64_t b = bh / H, h = bh % H;
    const int v0 = vt * VT;

    // Zero the token-padding rows / columns once (never written afterwards).
    for (int idx = C * LDK + tid; idx < CK * LDK; idx += kThreads) {
        Qs[idx] = from_f32<E>(0.f); Ks[idx] = from_f32<E>(0.f);
        if constexpr (CHANNEL) Khs[idx] = from_f32<E>(0.f);
    }
    for (int idx = tid; idx < C * LC; idx += kThreads) { Ts[idx] = from_f32<E>(0.f); Ps[idx] = from_f32<E>(0.f); }
    for (int idx = tid; idx < VT * LC; idx += kThreads) {
        Rt[idx] = from_f32<E>(0.f); Dt[idx] = from_f32<E>(0.f);
        if constexpr (!CHANNEL) Dst[idx] = from_f32<E>(0.f);
    }
    // Initial state slice.
    for (int idx = tid; idx < VT * (DK / 4); idx += kThreads) {
        const int r = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S0) x = *reinterpret_cast<const float4*>(S0 + (bh * DV + v0 + r) * DK + c);
        *reinterpret_cast<float4*>(Ss + r * LS + c) = x;
    }

    for (int n = 0; n < NT; ++n) {
        const int64_t t0 = (int64_t)n * C;
        const int len = (int)((T - t0) < C ? (T - t0) : C);
        const int64_t row0 = (b * T + t0) * H + h;
        const uint8_t* blk = ws + (size_t)(bh * NT + n) * L::BYTES;
        __syncthreads();  // previous chunk fully consumed
        if constexpr (CHANNEL) {
            g2s<E, C, DK>(Qs, LDK, reinterpret_cast<const E*>(blk + L::QG), DK, C, tid);
            g2s<E, C, DK>(Ks, LDK, reinterpret_cast<const E*>(blk + L::KG), DK, C, tid);
            g2s<E, C, DK>(Khs, LDK, reinterpret_cast<const E*>(blk + L::KH), DK, C, tid);
            for (int idx = tid; idx < DK; idx += kThreads)
                gs[idx] = reinterpret_cast<const float*>(blk + L::GL)[idx];
        } else {
            g2s<E, C, DK>(Qs, LDK, q + row0 * DK, (int64_t)H * DK, len, tid);
            g2s<E, C, DK>(Ks, LDK, k + row0 * DK, (int64_t)H * DK, len, tid);
            for (int idx = tid; idx < C; idx += kThreads)
                gs[idx] = reinterpret_cast<const float*>(blk + L::G)[idx];
        }
        g2s<E, C, C>(Ts, LC, reinterpret_cast<const E*>(blk + L::T), C, C, tid);
        g2s<E, C, C>(Ps, LC, reinterpret_cast<const E*>(blk + L::P), C, C, tid);
        g2s<E, C, VT>(Vs, LV, v + row0 * DV + v0, (int64_t)H * DV, len, tid);
        __syncthreads();

        // Phase A: R = V - Kg S^T  and  Oi = Qg S^T   (rows = tokens, cols = v)
        f32x4 oacc[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int t = wave + s * kWaves;
            oacc[s] = zero4();
            if (t >= TA) continue;
            const int mt = t / NTL, nt = t % NTL;
            f32x4 ar = zero4(), ao = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += M::KS) {
                const auto bf = frag_rk_f32<E>(Ss, LS, 16 * nt, k0, lane);
                ar = M::mma(frag_rk(Ks, LDK, 16 * mt, k0, lane), bf, ar);
                ao = M::mma(frag_rk(Qs, LDK, 16 * mt, k0, lane), bf, ao);
            }
            const int vc = 16 * nt + acc_col(lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + acc_row(lane, e);
                const float gam = CHANNEL ? 1.f : expf(gs[r]);
                const float rv = to_f32(Vs[r * LV + vc]) - gam * ar[e];
                Rt[vc * LC + r] = from_f32<E>(rv);
                oacc[s][e] = gam * ao[e];
            }
        }
        __syncthreads();

        // Phase B: D = T R
        for (int t = wave; t < TA; t += kWaves) {
            const int mt = t / NTL, nt = t % NTL;
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < CK; k0 += M::KS)
                acc = M::mma(frag_rk(Ts, LC, 16 * mt, k0, lane), frag_rk(Rt, LC, 16 * nt, k0, lane),
                             acc);
            const int vc = 16 * nt + acc_col(lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + acc_row(lane, e);
                Dt[vc * LC + r] = from_f32<E>(acc[e]);
                if constexpr (!CHANNEL)
                    Dst[vc * LC + r] = from_f32<E>(acc[e] * expf(gs[C - 1] - gs[r]));
            }
        }
        __syncthreads();

        // Phase C1: O = Oi + P D  -> global
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int t = wave + s * kWaves;
            if (t >= TA) continue;
            const int mt = t / NTL, nt = t % NTL;
            f32x4 acc = oacc[s];
#pragma unroll
            for (int k0 = 0; k0 < CK; k0 += M::KS)
                acc = M::mma(frag_rk(Ps, LC, 16 * mt, k0, lane), frag_rk(Dt, LC, 16 * nt, k0, lane),
                             acc);
            const int vc = 16 * nt + acc_col(lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + acc_row(lane, e);
                if (r < len) o[(row0 + (int64_t)r * H) * DV + v0 + vc] = from_f32<E>(acc[e]);
            }
        }
        // Phase C2: S^T[c][v] <- gamma_last[c] S^T[c][v] + sum_r Kh[r][c] D[r][v]
        const E* Kh = CHANNEL ? Khs : Ks;
        const E* Dsrc = CHANNEL ? Dt : Dst;
        const float glast_s = CHANNEL ? 0.f : expf(gs[C - 1]);
        for (int t = wave; t < TS; t += kWaves) {
            const int mc = t / NTL, nt = t % NTL;
            const int vr = 16 * nt + acc_col(lane);
            const int c = 16 * mc + acc_row(lane, 0);
            float4 sv = *reinterpret_cast<const float4*>(Ss + vr * LS + c);
            f32x4 acc;
            if constexpr (CHANNEL) {
                acc[0] = sv.x * expf(gs[c + 0]); acc[1] = sv.y * expf(gs[c + 1]);
                acc[2] = sv.z * expf(gs[c + 2]); acc[3] = sv.w * expf(gs[c + 3]);
            } else {
                acc[0] = sv.x * glast_s; acc[1] = sv.y * glast_s;
                acc[2] = sv.z * glast_s; acc[3] = sv.w * glast_s;
            }
#pragma unroll
            for (int k0 = 0; k0 < CK; k0 += M::KS)
                acc = M::mma(frag_kr(Kh, LDK, 16 * mc, k0, lane),
                             frag_rk(Dsrc, LC, 16 * nt, k0, lane), acc);
            *reinterpret_cast<float4*>(Ss + vr * LS + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
    __syncthreads();
    if (ST) {
        for (int idx = tid; idx < VT * (DK / 4); idx += kThreads) {
            const int r = idx / (DK / 4), c = 4 * (idx % (DK / 4));
            *reinterpret_cast<float4*>(ST + (bh * DV + v0 + r) * DK + c) =
                *reinterpret_cast<const float4*>(Ss + r * LS + c);
        }
    }
}

// T = 0: S_T = S0 (or zeros).
__global__ void copy_state(const float* __restrict__ S0, float* __restrict__ ST, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S0) x = reinterpret_cast<const float4*>(S0)[i];
        reinterpret_cast<float4*>(ST)[i] = x;
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
template <typename E, int DK, int C, bool CHANNEL>
static hipError_t launch_chunk(const ChunkArgs& a) {
    const int NT = (int)((a.T + C - 1) / C);
    const int64_t BH = a.B * a.H;
    if constexpr (CHANNEL) {
        return hipErrorNotSupported;  // channel-gate prep kernel: not built yet
    } else {
        hipLaunchKernelGGL((wy_prep_scalar<E, DK, C>), dim3((unsigned)(BH * NT)), dim3(kThreads), 0,
                           a.stream, (const E*)a.q, (const E*)a.k, a.log_alpha, a.beta,
                           (uint8_t*)a.ws, a.T, (int)a.H, NT);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // dv-slice width: 32 when that already gives a workgroup per CU, else 16.
    // (fp32 operands only ever use 16-wide slices: a 32-wide one does not fit in LDS.)
    if constexpr (sizeof(E) == 2) {
        if (BH * (a.dv / 32) >= 256) {
            hipLaunchKernelGGL((state_pass<E, DK, C, 32, CHANNEL>),
                               dim3((unsigned)(BH * (a.dv / 32))), dim3(kThreads), 0, a.stream,
                               (const E*)a.q, (const E*)a.k, (const E*)a.v, a.S0, (E*)a.o,
                               a.S_T, (const uint8_t*)a.ws, a.T, (int)a.H, NT, (int)a.dv);
            return hipGetLastError();
        }
    }
    {
        hipLaunchKernelGGL((state_pass<E, DK, C, 16, CHANNEL>), dim3((unsigned)(BH * (a.dv / 16))),
                           dim3(kThreads), 0, a.stream, (const E*)a.q, (const E*)a.k,
                           (const E*)a.v, a.S0, (E*)a.o, a.S_T, (const uint8_t*)a.ws, a.T,
                           (int)a.H, NT, (int)a.dv);
    }
    return hipGetLastError();
}

template <typename E, bool CHANNEL>
static hipError_t dispatch_shape(const ChunkArgs& a) {
    if (a.dk == 64) {
        if (a.chunk == 16) return launch_chunk<E, 64, 16, CHANNEL>(a);
        if (a.chunk == 32) return launch_chunk<E, 64, 32, CHANNEL>(a);
        return launch_chunk<E, 64, 64, CHANNEL>(a);
    }
    if (a.chunk == 16) return launch_chunk<E, 128, 16, CHANNEL>(a);
    if (a.chunk == 32) return launch_chunk<E, 128, 32, CHANNEL>(a);
    return launch_chunk<E, 128, 64, CHANNEL>(a);
}

template <typename E, bool CHANNEL>
static size_t block_bytes_t(int64_t dk, int64_t chunk) {
    if (dk == 64) {
        if (chunk == 16) return WsLayout<E, 64, 16, CHANNEL>::BYTES;
        if (chunk == 32) return WsLayout<E, 64, 32, CHANNEL>::BYTES;
        return WsLayout<E, 64, 64, CHANNEL>::BYTES;
    }
    if (chunk == 16) return WsLayout<E, 128, 16, CHANNEL>::BYTES;
    if (chunk == 32) return WsLayout<E, 128, 32, CHANNEL>::BYTES;
    return WsLayout<E, 128, 64, CHANNEL>::BYTES;
}

size_t chunk_block_bytes(int64_t dk, int64_t chunk, bool bf16, bool channel) {
    if (bf16)
        return channel ? block_bytes_t<__bf16, true>(dk, chunk) : block_bytes_t<__bf16, false>(dk, chunk);
    return channel ? block_bytes_t<float, true>(dk, chunk) : block_bytes_t<float, false>(dk, chunk);
}

size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t chunk, bool bf16,
                             bool channel) {
    const int64_t NT = (T + chunk - 1) / chunk;
    return (size_t)(B * H * NT) * chunk_block_bytes(dk, chunk, bf16, channel);
}

hipError_t chunk_fwd_launch(const ChunkArgs& a) {
    if (a.T == 0) {
        if (!a.S_T) return hipSuccess;
        const int64_t n4 = a.B * a.H * a.dv * a.dk / 4;
        hipLaunchKernelGGL(copy_state, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, a.stream,
                           a.S0, a.S_T, n4);
        return hipGetLastError();
    }
    if (a.bf16)
        return a.channel ? dispatch_shape<__bf16, true>(a) : dispatch_shape<__bf16, false>(a);
    return a.channel ? dispatch_shape<float, true>(a) : dispatch_shape<float, false>(a);
}

}  // namespace gdr
