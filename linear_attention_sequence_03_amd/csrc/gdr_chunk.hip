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
//  1. wy_prep_{scalar,channel} -- one workgroup per (b, h, chunk), fully
//     parallel: decay cumsum, A and P on the matrix cores, the triangular solve
//     in LDS (fp32), and T, P and the decay factors (plus, for the channel gate,
//     the decay-scaled Qg, Kg, Kh) into the workspace.
//  2. state_pass -- each wave owns 16 value columns of one (b, h) and walks the
//     chunks in order with its fp32 state slice S^T[dk][16] held in MFMA
//     accumulator registers.  Per chunk, all in registers and with no
//     synchronisation between waves:
//        R = V - Kg S^T ;  Oi = Qg S^T ;  D = T R ;  O = Oi + P D ;
//        S^T <- Diag(gamma_last) S^T + Kh^T D
//     Each product's accumulator tiles are the next product's B operand (the
//     permuted k-map in gdr_device.hpp), so nothing round-trips through LDS.
//     The shared per-chunk inputs are copied global->LDS with global_load_lds
//     (no registers), one chunk ahead, into a double buffer.  For the bf16
//     channel gate the loaders also warm L2 with the chunk after that (the
//     head's workspace block split over its workgroups, and the V rows).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kMinLogAlpha = -200.f;  // exp(-200) ~ 1e-87: 0 in fp32
constexpr float kSafeSpan = 64.f;       // see wy_prep_channel

// Byte layout of one (b, h, chunk) workspace block.
template <typename E, int DK, int C, bool CHANNEL>
struct WsLayout {
    static constexpr size_t T = 0;                                   // E [C][C]
    static constexpr size_t P = T + (size_t)C * C * sizeof(E);       // E [C][C]
    static constexpr size_t QG = P + (size_t)C * C * sizeof(E);      // E [C][DK] (channel)
    static constexpr size_t KG = QG + (size_t)C * DK * sizeof(E);    // E [C][DK] (channel)
    static constexpr size_t KH = KG + (size_t)C * DK * sizeof(E);    // E [C][DK] (channel)
    // Per-chunk decay vector read by the state pass:
    //   scalar gate : gam[C] = exp(g_r), gh[C] = exp(g_last - g_r)
    //   channel gate: gl[DK] = exp(g_last,c)
    static constexpr size_t VEC = CHANNEL ? KH + (size_t)C * DK * sizeof(E) : QG;
    static constexpr size_t VEC_DATA = CHANNEL ? DK * 4 : 2 * C * 4;
    // bf16: T may travel as a hi/lo pair.  FLAG (int, after the decay vector,
    // copied with it) says whether this chunk's TL = T - bf16(T) was written
    // and is to be applied; TL is read from global memory only then.
    static constexpr bool PAIR = sizeof(E) == 2;
    static constexpr size_t FLAG = VEC + VEC_DATA;
    static constexpr size_t VEC_BYTES = VEC_DATA + (PAIR ? 16 : 0);
    static constexpr size_t TL = VEC + VEC_BYTES;                     // E [C][C] (bf16)
    static constexpr size_t BYTES = ((PAIR ? TL + (size_t)C * C * sizeof(E) : VEC + VEC_BYTES) + 255) / 256 * 256;
    static constexpr size_t WARM_BYTES = PAIR ? TL : BYTES;           // read by every state pass
};

// A chunk applies T as a bf16 pair when some entry of its strictly lower A
// exceeds this in magnitude (keys nearly repeated or opposed with a write rate
// near 1 and weak decay): T then holds entries of size ~1 whose row sums are
// small, and a single bf16 rounding of T loses them.
constexpr float kPairThresh = 0.5f;

// Store x as E at hi[i]; with a residual buffer, also x - E(x) at lo[i].
template <typename E>
__device__ __forceinline__ void put_pair(E* hi, E* lo, int i, float x) {
    const E h = from_f32<E>(x);
    hi[i] = h;
    if (lo) lo[i] = from_f32<E>(x - to_f32(h));
}

// Copy a [ROWS][COLS] tile of E from global (row stride gstride elements) into
// LDS (row stride ls elements) through registers; rows >= valid are zero.
template <typename E, int ROWS, int COLS, int NTHR>
__device__ __forceinline__ void g2s(E* dst, int ls, const E* src, int64_t gstride, int valid,
                                    int tid) {
    constexpr int EPS = 16 / sizeof(E);
    constexpr int SEGS = COLS / EPS;
#pragma unroll 4
    for (int idx = tid; idx < ROWS * SEGS; idx += NTHR) {
        const int r = idx / SEGS, s = idx % SEGS;
        const V16 x = r < valid ? ld16(src + r * gstride + s * EPS) : zero16();
        st16(dst + r * ls + s * EPS, x);
    }
}

// Triangular solve in LDS: Xs <- (I + As)^-1 for a strictly lower C x C matrix
// As (fp32, row stride LA).  Diagonal 16x16 blocks by right-looking forward
// substitution in wave 0 (lane = column j of diagonal block lane>>4; critical
// path of 15 dependent FMAs); off-diagonal blocks by increasing distance from
// the diagonal, X_ij = -X_ii * sum_{m=j}^{i-1} A_im X_mj, on fp32 MFMAs.
// Ys: scratch of (C/16 - 1) 16x17 fp32 tiles.
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
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
#pragma unroll
                for (int i = m + 1; i < 16; ++i) x[i] -= Ab[i * LA + m] * x[m];
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

// Lower 16x16 block tiles of a C x C matrix, stored tile by tile (fp32, rows
// padded to 17): tile (i, j), j <= i, starts at tl(i, j) * kTS.
constexpr int kTS = 16 * 17;
__device__ __forceinline__ int tl(int i, int j) { return i * (i + 1) / 2 + j; }
__device__ __forceinline__ int ablk(int row, int col) {
    return tl(row >> 4, col >> 4) * kTS + (row & 15) * 17 + (col & 15);
}

// exp(x) through the hardware base-2 exponential (x <= 0 here; underflows to 0).
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Copy two [ROWS][COLS] tiles (same row strides) global -> LDS through
// registers, all loads issued before any LDS store (one memory round trip).
template <typename E, int ROWS, int COLS, int NTHR>
__device__ __forceinline__ void g2s_pair(E* d0, E* d1, int ls, const E* s0, const E* s1,
                                         int64_t gstride, int valid, int tid) {
    constexpr int EPS = 16 / sizeof(E);
    constexpr int SEGS = COLS / EPS;
    constexpr int PER = (ROWS * SEGS + NTHR - 1) / NTHR;
    V16 a[PER], b[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + i * NTHR;
        const int r = idx / SEGS, sg = idx % SEGS;
        const bool ok = idx < ROWS * SEGS && r < valid;
        a[i] = ok ? ld16(s0 + r * gstride + sg * EPS) : zero16();
        b[i] = ok ? ld16(s1 + r * gstride + sg * EPS) : zero16();
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + i * NTHR;
        const int r = idx / SEGS, sg = idx % SEGS;
        if (idx < ROWS * SEGS) {
            st16(d0 + r * ls + sg * EPS, a[i]);
            st16(d1 + r * ls + sg * EPS, b[i]);
        }
    }
}

// T = (I + A)^-1 Diag(beta) from the lower block tiles of A (Ablk; strictly
// lower inside the diagonal tiles), written to the workspace.  Wave 0 inverts
// the diagonal 16x16 blocks by right-looking forward substitution (one lane
// per column of every diagonal block; 15 dependent FMAs deep) into Xd; then
// wave j builds column block j of X = (I + A)^-1 alone, in registers:
//   X_ij = -X_ii * sum_{m=j}^{i-1} A_im X_mj      (i = j+1 .. NB-1)
// on fp32 16x16x4 MFMAs, each new tile feeding the next product as its B
// operand, and stores T_ij = X_ij Diag(beta_j) straight from the accumulators.
template <typename E, int C>
__device__ __forceinline__ void solve_store_T(const float* Ablk, float* Xd, const float* bs, E* Tw, E* Tl,
                                              int tid) {
    constexpr int NB = C / 16;
    using MF = Mma<float>;
    const int lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, col = lane & 15;
    if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        if (blk < NB) {
            const float* Ab = Ablk + tl(blk, blk) * kTS;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
#pragma unroll
                for (int i = m + 1; i < 16; ++i) x[i] -= Ab[i * 17 + m] * x[m];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Xd[blk * kTS + i * 17 + j] = x[i];
        }
    }
    __syncthreads();
    const int j = wave;
    if (j >= NB) return;
    const float bcol = bs[16 * j + col];
    // diagonal tile and the zero tiles above it
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        put_pair<E>(Tw, Tl, (16 * j + r) * C + 16 * j + col, Xd[j * kTS + r * 17 + col] * bcol);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i < j)
#pragma unroll
            for (int e = 0; e < 4; ++e) put_pair<E>(Tw, Tl, (16 * i + 4 * g4 + e) * C + 16 * j + col, 0.f);
    }
    f32x4 X[NB];
#pragma unroll
    for (int i = 1; i < NB; ++i) {
        X[i] = zero4();
        if (i <= j) continue;
        f32x4 Y = zero4();
#pragma unroll
        for (int m = 0; m < i; ++m) {
            if (m < j) continue;
            const float* Aim = Ablk + tl(i, m) * kTS;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float a = Aim[col * 17 + 4 * g4 + s];
                const float b = (m == j) ? Xd[j * kTS + (4 * g4 + s) * 17 + col] : X[m][s];
                Y = MF::mma(a, b, Y);
            }
        }
        f32x4 Z = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) Z = MF::mma(Xd[i * kTS + col * 17 + 4 * g4 + s], Y[s], Z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            X[i][e] = -Z[e];
            put_pair<E>(Tw, Tl, (16 * i + 4 * g4 + e) * C + 16 * j + col, -Z[e] * bcol);
        }
    }
}

// Write T = X Diag(beta) (lower triangle, E) to the workspace, 16 bytes per store.
template <typename E, int C, int LA>
__device__ __forceinline__ void store_T(E* Tw, const float* Xs, const float* bs, int tid) {
    constexpr int EPS = 16 / sizeof(E);
    for (int idx = tid; idx < C * C / EPS; idx += kThreads) {
        const int r = (idx * EPS) / C, c0 = (idx * EPS) % C;
        alignas(16) E vals[EPS];
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
            const int c = c0 + e;
            vals[e] = from_f32<E>(c <= r ? Xs[r * LA + c] * bs[c] : 0.f);
        }
        *reinterpret_cast<V16*>(Tw + r * C + c0) = *reinterpret_cast<const V16*>(vals);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1, scalar gate (Gated DeltaNet).  Tiles: wave w takes the A tiles
// (w even) or P tiles (w odd) of row blocks {p, NB-1-p}, p = w/2, which gives
// every wave 5 tiles at C = 64.
// ---------------------------------------------------------------------------
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void wy_prep_scalar(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, uint8_t* __restrict__ ws, int64_t T, int H, int NT) {
    using L = WsLayout<E, DK, C, false>;
    using M = Mma<E>;
    constexpr int LDK = DK + Pad<E>::v;
    constexpr int NB = C / 16;
    __shared__ __attribute__((aligned(16))) E Ks[C * LDK];
    __shared__ __attribute__((aligned(16))) E Qs[C * LDK];
    __shared__ float Ablk[NB * (NB + 1) / 2 * kTS];
    __shared__ float Xd[NB * kTS];
    __shared__ float gs[C], bs[C];
    __shared__ int pair_sh;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, col = lane & 15;
    if (tid == 0) pair_sh = 0;
    const int64_t bid = blockIdx.x;
    const int n = (int)(bid % NT);
    const int64_t bh = bid / NT;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = (int64_t)n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t row0 = ((b * T + t0) * H + h);   // token-row index of row 0

    g2s_pair<E, C, DK, kThreads>(Ks, Qs, LDK, k + row0 * DK, q + row0 * DK, (int64_t)H * DK, len, tid);
    if (wave == 0) {
        float x = 0.f, bb = 0.f;
        if (lane < len) {
            x = fmaxf(log_alpha[row0 + (int64_t)lane * H], kMinLogAlpha);
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

    // Tiles of A = K K^T (gated, beta-scaled, strictly lower) into Ablk and of
    // P = Q K^T (gated, lower incl. diagonal) straight to the workspace.
    const int pr = wave >> 1;
    const bool isP = wave & 1;
    float amax = 0.f;   // largest |A| entry this wave computed
    if (pr < (NB + 1) / 2) {
        const E* Ap = isP ? Qs : Ks;
#pragma unroll
        for (int sel = 0; sel < 2; ++sel) {
            const int rb = sel == 0 ? pr : NB - 1 - pr;
            if (sel == 1 && rb == pr) break;
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (cb > rb) {
                    if (isP)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            Pw[(16 * rb + 4 * g4 + e) * C + 16 * cb + col] = from_f32<E>(0.f);
                    continue;
                }
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += M::KS)
                    acc = M::mma(frag_rk(Ap, LDK, 16 * rb, k0, lane), frag_rk(Ks, LDK, 16 * cb, k0, lane),
                                 acc);
                const int c = 16 * cb + col;
                const float gc = gs[c];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e;
                    const bool keep = isP ? (c <= r) : (c < r);
                    const float dec = keep ? fast_exp(gs[r] - gc) : 0.f;
                    if (isP) {
                        Pw[r * C + c] = from_f32<E>(acc[e] * dec);
                    } else {
                        const float a = acc[e] * bs[r] * dec;
                        Ablk[ablk(r, c)] = a;
                        amax = fmaxf(amax, fabsf(a));
                    }
                }
            }
        }
    }
    if constexpr (L::PAIR)
        if (__ballot(amax > kPairThresh) != 0 && lane == 0) pair_sh = 1;
    __syncthreads();

    const bool pair = L::PAIR && pair_sh != 0;
    solve_store_T<E, C>(Ablk, Xd, bs, Tw, pair ? reinterpret_cast<E*>(blk + L::TL) : nullptr, tid);
    float* vec = reinterpret_cast<float*>(blk + L::VEC);
    if (tid < C) {
        vec[tid] = expf(gs[tid]);
        vec[C + tid] = expf(gs[C - 1] - gs[tid]);
    }
    if constexpr (L::PAIR)
        if (tid == 0) *reinterpret_cast<int*>(blk + L::FLAG) = pair ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Kernel 1, channel gate (KDA).
//
// The gated products A[r][i] = beta_r sum_c k_rc k_ic exp(g_rc - g_ic) and
// P[r][i] = sum_c q_rc k_ic exp(g_rc - g_ic) are taken per pair of 16-row
// blocks (rb, cb <= rb) as plain MFMA products of rescaled rows, around the
// reference g_ref(rb) = g at the row just before block rb (0 for rb = 0):
//   A side  x_r * exp(g_r - g_ref(rb))     <= 1          (r in block rb)
//   B side  k_i * exp(g_ref(rb) - g_i)     <= 1 if cb < rb,  >= 1 if cb == rb
// whose products are x_r k_i exp(g_r - g_i) exactly.  Off the diagonal no
// factor exceeds 1, so nothing overflows and a factor that underflows bounds a
// negligible true value.  On a diagonal block the B side grows like
// exp(span), span = g_ref(rb) - g(last row of rb); if any channel's span
// exceeds kSafeSpan that block is computed exactly, pair by pair, from the
// in-block cumulative sums instead.
// Thread (seg, rg) owns channels 4seg..4seg+3 of rows 8rg..8rg+7: a local
// cumsum plus a scan of the row-group totals gives g without a [C][DK] array.
// ---------------------------------------------------------------------------
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void wy_prep_channel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, uint8_t* __restrict__ ws, int64_t T, int H, int NT) {
    using L = WsLayout<E, DK, C, true>;
    using M = Mma<E>;
    constexpr int LDK = DK + Pad<E>::v;
    constexpr int NB = C / 16;
    constexpr int LA = C + 1;
    constexpr int NSEG = DK / 4;
    constexpr int NRG = C / 8;
    static_assert(NSEG * NRG <= kThreads, "one (segment, row group) per thread");
    __shared__ __attribute__((aligned(16))) E Ka[C * LDK];   // A-side keys
    __shared__ __attribute__((aligned(16))) E Qa[C * LDK];   // A-side queries
    __shared__ __attribute__((aligned(16))) E Bb[C * LDK];   // B-side keys of one stage
    __shared__ float As[C * LA];
    __shared__ float Xs[C * LA];
    __shared__ float Ys[(NB > 1 ? NB - 1 : 1) * 16 * 17];
    __shared__ __attribute__((aligned(16))) float tot[NRG * DK];
    __shared__ __attribute__((aligned(16))) float gb[NB * DK];  // g at the last row of each block
    __shared__ float bs[C];
    __shared__ int unsafe_blk[NB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bid = blockIdx.x;
    const int n = (int)(bid % NT);
    const int64_t bh = bid / NT;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = (int64_t)n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t row0 = ((b * T + t0) * H + h);

    uint8_t* blk = ws + (size_t)bid * L::BYTES;
    E* Tw = reinterpret_cast<E*>(blk + L::T);
    E* Pw = reinterpret_cast<E*>(blk + L::P);
    E* Qgw = reinterpret_cast<E*>(blk + L::QG);
    E* Kgw = reinterpret_cast<E*>(blk + L::KG);
    E* Khw = reinterpret_cast<E*>(blk + L::KH);
    float* glw = reinterpret_cast<float*>(blk + L::VEC);

    const bool active = tid < NSEG * NRG;
    const int seg = tid % NSEG, rg = tid / NSEG;
    const int c0 = 4 * seg;
    const int rblk = (8 * rg) >> 4;
    float g[8][4], kr[8][4], qr[8][4];
    if (active) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * rg + j;
            float4 la = make_float4(0.f, 0.f, 0.f, 0.f), kv = la, qv = la;
            if (r < len) {
                const int64_t off = (row0 + (int64_t)r * H) * DK + c0;
                la = *reinterpret_cast<const float4*>(log_alpha + off);
                kv = load4(k + off);
                qv = load4(q + off);
            }
            const float l4[4] = {fmaxf(la.x, kMinLogAlpha), fmaxf(la.y, kMinLogAlpha),
                                 fmaxf(la.z, kMinLogAlpha), fmaxf(la.w, kMinLogAlpha)};
            kr[j][0] = kv.x; kr[j][1] = kv.y; kr[j][2] = kv.z; kr[j][3] = kv.w;
            qr[j][0] = qv.x; qr[j][1] = qv.y; qr[j][2] = qv.z; qr[j][3] = qv.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) g[j][e] = (j ? g[j - 1][e] : 0.f) + l4[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tot[rg * DK + c0 + e] = g[7][e];
    }
    if (tid < C) bs[tid] = tid < len ? beta[row0 + (int64_t)tid * H] : 0.f;
    if (tid < NB) unsafe_blk[tid] = 0;
    for (int idx = tid; idx < C * LA; idx += kThreads) { As[idx] = 0.f; Xs[idx] = 0.f; }
    __syncthreads();
    if (active) {
        float off[4] = {0.f, 0.f, 0.f, 0.f};
        for (int r2 = 0; r2 < rg; ++r2)
#pragma unroll
            for (int e = 0; e < 4; ++e) off[e] += tot[r2 * DK + c0 + e];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) g[j][e] += off[e];
        if (rg & 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) gb[(rg >> 1) * DK + c0 + e] = g[7][e];
    }
    __syncthreads();
    for (int idx = tid; idx < NB * DK; idx += kThreads) {
        const int rb = idx / DK, c = idx % DK;
        const float ref = rb ? gb[(rb - 1) * DK + c] : 0.f;
        if (!(ref - gb[rb * DK + c] <= kSafeSpan)) unsafe_blk[rb] = 1;
    }
    if (active) {
        float gref[4], glast[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gref[e] = rblk ? gb[(rblk - 1) * DK + c0 + e] : 0.f;
            glast[e] = gb[(NB - 1) * DK + c0 + e];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * rg + j;
            float ea[4], eg[4], eh[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ea[e] = expf(g[j][e] - gref[e]);
                eg[e] = expf(g[j][e]);
                eh[e] = expf(glast[e] - g[j][e]);
            }
            store4(Ka + r * LDK + c0, make_float4(kr[j][0] * ea[0], kr[j][1] * ea[1],
                                                  kr[j][2] * ea[2], kr[j][3] * ea[3]));
            store4(Qa + r * LDK + c0, make_float4(qr[j][0] * ea[0], qr[j][1] * ea[1],
                                                  qr[j][2] * ea[2], qr[j][3] * ea[3]));
            store4(Qgw + r * DK + c0, make_float4(qr[j][0] * eg[0], qr[j][1] * eg[1],
                                                  qr[j][2] * eg[2], qr[j][3] * eg[3]));
            store4(Kgw + r * DK + c0, make_float4(kr[j][0] * eg[0], kr[j][1] * eg[1],
                                                  kr[j][2] * eg[2], kr[j][3] * eg[3]));
            store4(Khw + r * DK + c0, make_float4(kr[j][0] * eh[0], kr[j][1] * eh[1],
                                                  kr[j][2] * eh[2], kr[j][3] * eh[3]));
        }
    }
    if (tid < DK) glw[tid] = expf(gb[(NB - 1) * DK + tid]);

    // Stage rb: B side around g_ref(rb) for rows i < 16(rb+1); tiles (rb, cb<=rb).
    for (int rb = 0; rb < NB; ++rb) {
        if (active && rblk <= rb) {
            float gr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) gr[e] = rb ? gb[(rb - 1) * DK + c0 + e] : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 8 * rg + j;
                store4(Bb + r * LDK + c0,
                       make_float4(kr[j][0] * expf(gr[0] - g[j][0]), kr[j][1] * expf(gr[1] - g[j][1]),
                                   kr[j][2] * expf(gr[2] - g[j][2]), kr[j][3] * expf(gr[3] - g[j][3])));
            }
        }
        __syncthreads();
        for (int t = wave; t < 2 * (rb + 1); t += kWaves) {
            const bool isP = t > rb;
            const int cb = isP ? t - rb - 1 : t;
            if (cb == rb && unsafe_blk[rb]) continue;
            const E* Ap = isP ? Qa : Ka;
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += M::KS)
                acc = M::mma(frag_rk(Ap, LDK, 16 * rb, k0, lane), frag_rk(Bb, LDK, 16 * cb, k0, lane),
                             acc);
            const int col = 16 * cb + acc_col(lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * rb + acc_row(lane, e);
                if (isP)
                    Pw[row * C + col] = from_f32<E>((cb < rb || col <= row) ? acc[e] : 0.f);
                else
                    As[row * LA + col] = (cb < rb || col < row) ? acc[e] * bs[row] : 0.f;
            }
        }
        __syncthreads();
    }

    // Exact path for diagonal blocks whose decay span is too large to factor.
    for (int rb = wave; rb < NB; rb += kWaves) {
        if (!unsafe_blk[rb]) continue;
        constexpr int CPL = DK / 64;
        float gl[16][CPL], kk[16][CPL], qq[16][CPL];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 16 * rb + j;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int c = lane + 64 * m;
                float la = 0.f, kv = 0.f, qv = 0.f;
                if (r < len) {
                    const int64_t off = (row0 + (int64_t)r * H) * DK + c;
                    la = fmaxf(log_alpha[off], kMinLogAlpha);
                    kv = to_f32(k[off]);
                    qv = to_f32(q[off]);
                }
                gl[j][m] = (j ? gl[j - 1][m] : 0.f) + la;
                kk[j][m] = kv;
                qq[j][m] = qv;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float a = 0.f, p = 0.f;
                if (i <= r) {
#pragma unroll
                    for (int m = 0; m < CPL; ++m) {
                        const float f = expf(gl[r][m] - gl[i][m]);
                        a += kk[r][m] * kk[i][m] * f;
                        p += qq[r][m] * kk[i][m] * f;
                    }
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) {
                        a += __shfl_xor(a, off);
                        p += __shfl_xor(p, off);
                    }
                }
                if (lane == 0) {
                    const int row = 16 * rb + r, col = 16 * rb + i;
                    As[row * LA + col] = i < r ? a * bs[row] : 0.f;
                    Pw[row * C + col] = from_f32<E>(p);
                }
            }
        }
    }
    // Upper blocks of P are zero.
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) Pw[idx] = from_f32<E>(0.f);
    }
    __syncthreads();

    solve_unit_lower<C, LA>(As, Xs, Ys, tid);
    store_T<E, C, LA>(Tw, Xs, bs, tid);
}

// ---------------------------------------------------------------------------
// Kernel 1, channel gate (KDA), bf16 io.  One wave per 16-token block b of the
// chunk (C/16 waves); the block's q, k and log alpha stay in registers in MFMA
// operand layout: lane (x, kg) = (lane % 16, lane / 16) holds token row
// 16b + x, channels 32s + 8kg + (0..7) of channel step s.
//  - g (per channel, in-chunk cumulative, log2 units): a scan over the 16 lanes
//    of a DPP row (row_shr 1, 2, 4, 8) plus the totals of the earlier blocks,
//    exchanged through LDS.
//  - Gram tiles (b, cb <= b) of A = Diag(beta) (K.Gamma)(K/Gamma)^T and of
//    P = (Q.Gamma)(K/Gamma)^T on the matrix cores, around reference points that
//    keep the factors in range:
//      cb < b: ref = g at the last row of block cb; A side x_r 2^{g_r - ref} <= 1,
//              B side k_i 2^{ref - g_i} <= 1 (built once by wave cb, in LDS);
//      cb = b: ref = g at the last row of block b - 1 (0 for b = 0); the B side
//              k_i 2^{ref - g_i} >= 1 grows with the block's decay span, and if
//              some channel's span exceeds kSafeSpan nats the block is summed
//              exactly, pair by pair.
//    The tiles come out transposed ("row layout": lane (x, kg) holds row x,
//    columns 4kg..4kg+3), which is the A operand of the fp32 MFMA below.
//  - T = (I + A)^-1 Diag(beta): each wave inverts its diagonal block by forward
//    substitution in fp32, then row block by row block
//        T_bj = -X_bb sum_{m=j}^{b-1} A_bm T_mj
//    on fp32 16x16x4 MFMAs, the tiles of earlier rows coming through LDS.
//  - Outputs in the workspace layout the state pass reads: T and P (row-major,
//    zero above the diagonal blocks), Qg = Q.Gamma, Kg = K.Gamma,
//    Kh = K.(gamma_C / Gamma) and gl = gamma_C.
// ---------------------------------------------------------------------------
// LDS of one workgroup of wy_prep_channel_bf16.
template <int DK, int C>
struct ChanPrepSmem {
    static constexpr int NB = C / 16, NKS = DK / 32;
    static constexpr int NPUB = NB > 1 ? NB - 1 : 1;
    static constexpr int NTP = NB > 1 ? NB * (NB - 1) / 2 : 1;
    static constexpr int SR = C + 8;                     // staging row stride (bf16)
    alignas(16) float tot[NB][DK];                       // block totals of g
    alignas(16) bf16x8 bpub[NPUB][NKS][64];              // B sides of blocks < NB-1
    alignas(16) float xa[NB][16 * 16];                   // A_bb^T for the substitution
    alignas(16) float xx[NB][16 * 17];                   // X_bb = (I + A_bb)^-1
    alignas(16) f32x4 tpub[NTP][64];                     // T tiles of rows < NB-1
    alignas(16) __bf16 stg[NB][16 * SR];                 // row-block staging of P, T
    alignas(16) float bsh[C];
    int pair;                                            // T travels as a bf16 pair
};

// The work of wave BW (16-row block BW).  The block index is a compile-time
// constant, so no matrix instruction sits under a wave-dependent condition.
template <int DK, int C, int BW, bool NORM>
__device__ __forceinline__ void chan_prep_wave(ChanPrepSmem<DK, C>& sm, const __bf16* __restrict__ q,
                                               const __bf16* __restrict__ k,
                                               const float* __restrict__ log_alpha,
                                               const float* __restrict__ beta, uint8_t* __restrict__ ws,
                                               int64_t T, int H, int NT, int gflags) {
    using L = WsLayout<__bf16, DK, C, true>;
    using M = Mma<__bf16>;
    using MF = Mma<float>;
    constexpr int NB = C / 16;
    constexpr int NKS = DK / 32;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kSafeSpan2 = kSafeSpan * kLog2e;
    constexpr int NPUB = NB > 1 ? NB - 1 : 1;
    constexpr int NTP = NB > 1 ? NB * (NB - 1) / 2 : 1;
    constexpr int SR = C + 8;                 // staging row stride (bf16), 16-byte aligned rows
    constexpr int NPC = 2 * C;                // 16-byte pieces of a 16-row block of a C x C tile
    auto& tot = sm.tot;
    auto& bpub = sm.bpub;
    auto& xa = sm.xa;
    auto& xx = sm.xx;
    auto& tpub = sm.tpub;
    auto& stg = sm.stg;
    auto& bsh = sm.bsh;
    constexpr int b = BW;   // this wave's 16-row block
    const int lane = threadIdx.x & 63;
    const int x = lane & 15, kg = lane >> 4;
    const int64_t bid = blockIdx.x;
    const int n = (int)(bid % NT);
    const int64_t bh = bid / NT;
    const int64_t bi = bh / H, h = bh % H;
    const int64_t t0 = (int64_t)n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t row0 = (bi * T + t0) * H + h;
    uint8_t* blk = ws + (size_t)bid * L::BYTES;

    if (b == 0 && lane == 0) sm.pair = 0;   // set below by any wave whose A needs the pair
    const int r = 16 * b + x;
    const bool valid = r < len;   // rows past len read row len-1 and are zeroed
    const int64_t grow = row0 + (int64_t)(valid ? r : len - 1) * H;
    float be = beta[grow];
    if (gflags & kPrologueBetaSigmoid) be = sigmoid_of(be);   // prologue: beta from its logit
    be = valid ? be : 0.f;
    if (kg == 0) bsh[r] = be;

    // Prologue: inverse L2 norms of this lane's q and k rows (the row's
    // channels are spread over the lanes x, x+16, x+32, x+48 and the steps s).
    float nk = 1.f, nq = 1.f;
    if constexpr (NORM) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const bf16x8 tk = *reinterpret_cast<const bf16x8*>(k + grow * DK + 32 * s + 8 * kg);
            const bf16x8 tq = *reinterpret_cast<const bf16x8*>(q + grow * DK + 32 * s + 8 * kg);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sk += (float)tk[j] * (float)tk[j];
                sq += (float)tq[j] * (float)tq[j];
            }
        }
        sk += __shfl_xor(sk, 16);
        sk += __shfl_xor(sk, 32);
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        nk = 1.f / sqrtf(sk + 1e-6f);
        nq = 1.f / sqrtf(sq + 1e-6f);
    }

    // Loads of channel step s: k or q (bf16x8, normalised by the prologue),
    // log alpha (in log2 units); the raw loads and their mapping are split so
    // that the main loop can issue a step's loads one step ahead.
    struct Raw {
        bf16x8 k, q;
        float4 l0, l1;
    };
    auto ld_raw = [&](int s) {
        Raw w;
        w.k = *reinterpret_cast<const bf16x8*>(k + grow * DK + 32 * s + 8 * kg);
        w.q = *reinterpret_cast<const bf16x8*>(q + grow * DK + 32 * s + 8 * kg);
        const float* p = log_alpha + grow * DK + 32 * s + 8 * kg;
        w.l0 = *reinterpret_cast<const float4*>(p);
        w.l1 = *reinterpret_cast<const float4*>(p + 4);
        return w;
    };
    auto map_qk = [&](bf16x8 t, float sc) {
        if constexpr (NORM) {
            bf16x8 u;
#pragma unroll
            for (int j = 0; j < 8; ++j) u[j] = (__bf16)((float)t[j] * sc);
            return valid ? u : bf16x8{};
        } else {
            return valid ? t : bf16x8{};
        }
    };
    auto map_la = [&](float4 l0, float4 l1, float* la) {
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = (gflags & kPrologueDecaySoftplus) ? neg_softplus(lv[j]) : lv[j];
            la[j] = valid ? fmaxf(x, kMinLogAlpha) * kLog2e : 0.f;
        }
    };
    // In-block inclusive scan over the 16 rows (one DPP row per channel group).
    auto scan = [&](float* v) {
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
        const float* tp = &tot[cb][32 * s + 8 * kg];
        const float4 a0 = *reinterpret_cast<const float4*>(tp);
        const float4 a1 = *reinterpret_cast<const float4*>(tp + 4);
        tv[0] = a0.x; tv[1] = a0.y; tv[2] = a0.z; tv[3] = a0.w;
        tv[4] = a1.x; tv[5] = a1.y; tv[6] = a1.z; tv[7] = a1.w;
    };

    f32x4 ga[NB], gp[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) ga[cb] = gp[cb] = zero4();
    bool unsafe_lane = false;
    // ---- per channel step s: g, the scaled operands, this block's B side,
    //      then the Gram tiles (b, cb <= b) ----
    // (64-token chunks without the prologue: elsewhere the extra registers
    // spill or lower the occupancy)
    constexpr bool PREFETCH = !NORM && C == 64;
    Raw nxt{};
    if constexpr (PREFETCH) nxt = ld_raw(0);
#pragma unroll 1
    for (int s = 0; s < NKS; ++s) {
        Raw cur;
        if constexpr (!PREFETCH) {
            cur = ld_raw(s);
        } else {
            cur = nxt;
            if (s + 1 < NKS) nxt = ld_raw(s + 1);
        }
        float gs[8];
        map_la(cur.l0, cur.l1, gs);
        const bf16x8 kv = map_qk(cur.k, nk), qv = map_qk(cur.q, nq);
        scan(gs);
        if (x == 15) {
            float* tp = &tot[b][32 * s + 8 * kg];
            *reinterpret_cast<float4*>(tp) = make_float4(gs[0], gs[1], gs[2], gs[3]);
            *reinterpret_cast<float4*>(tp + 4) = make_float4(gs[4], gs[5], gs[6], gs[7]);
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
                if (cb == b && !(-tv[j] <= kSafeSpan2)) unsafe_lane = true;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) gs[j] += off[j];
        const size_t eo = ((size_t)r * DK + 32 * s + 8 * kg) * sizeof(__bf16);
        {
            bf16x8 qg, kgv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float eg = __builtin_amdgcn_exp2f(gs[j]);
                qg[j] = (__bf16)((float)qv[j] * eg);
                kgv[j] = (__bf16)((float)kv[j] * eg);
            }
            *reinterpret_cast<bf16x8*>(blk + L::QG + eo) = qg;
            *reinterpret_cast<bf16x8*>(blk + L::KG + eo) = kgv;
        }
        {
            bf16x8 kh;
#pragma unroll
            for (int j = 0; j < 8; ++j) kh[j] = (__bf16)((float)kv[j] * __builtin_amdgcn_exp2f(last[j] - gs[j]));
            *reinterpret_cast<bf16x8*>(blk + L::KH + eo) = kh;
        }
        if (b < NB - 1) {
            bf16x8 kb;
#pragma unroll
            for (int j = 0; j < 8; ++j) kb[j] = (__bf16)((float)kv[j] * __builtin_amdgcn_exp2f(end[j] - gs[j]));
            bpub[b < NPUB ? b : 0][s][lane] = kb;
        }
        if (b == 0 && x == 0) {
            float* glw = reinterpret_cast<float*>(blk + L::VEC) + 32 * s + 8 * kg;
            *reinterpret_cast<float4*>(glw) =
                make_float4(__builtin_amdgcn_exp2f(last[0]), __builtin_amdgcn_exp2f(last[1]),
                            __builtin_amdgcn_exp2f(last[2]), __builtin_amdgcn_exp2f(last[3]));
            *reinterpret_cast<float4*>(glw + 4) =
                make_float4(__builtin_amdgcn_exp2f(last[4]), __builtin_amdgcn_exp2f(last[5]),
                            __builtin_amdgcn_exp2f(last[6]), __builtin_amdgcn_exp2f(last[7]));
        }
        __syncthreads();

        // A sides around the end of block cb (cb < b) against wave cb's B sides;
        // the last one (cb = b - 1) is also the diagonal's A side.
        bf16x8 ka, qa;
        float ref[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ref[j] = 0.f;
#pragma unroll
        for (int cb = 0; cb < NB - 1; ++cb) {
            if (cb < b) {
                float tv[8];
                ld_tot(cb, s, tv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ref[j] += tv[j];
                    const float e = __builtin_amdgcn_exp2f(gs[j] - ref[j]);
                    ka[j] = (__bf16)((float)kv[j] * e);
                    qa[j] = (__bf16)((float)qv[j] * e);
                }
                const bf16x8 bs = bpub[cb][s][lane];
                ga[cb] = M::mma(bs, ka, ga[cb]);
                gp[cb] = M::mma(bs, qa, gp[cb]);
            }
        }
        if (b == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = __builtin_amdgcn_exp2f(gs[j]);
                ka[j] = (__bf16)((float)kv[j] * e);
                qa[j] = (__bf16)((float)qv[j] * e);
            }
        }
        bf16x8 kd;
#pragma unroll
        for (int j = 0; j < 8; ++j) kd[j] = (__bf16)((float)kv[j] * __builtin_amdgcn_exp2f(ref[j] - gs[j]));
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
            if (cb == b) {
                ga[cb] = M::mma(kd, ka, ga[cb]);
                gp[cb] = M::mma(kd, qa, gp[cb]);
            }
    }
    if (__ballot(unsafe_lane) != 0) {   // wave-uniform
        // Exact diagonal block: sum_c x_rc k_ic 2^{g_rc - g_ic} (i <= r), row i
        // of the block fetched from lane (i, kg); g (the in-block part suffices:
        // the offsets cancel), q and k rebuilt per step.  Rare, so kept small.
        f32x4 ea = zero4(), ep = zero4();
#pragma unroll 1
        for (int y = 0; y < 16; ++y) {
            float a = 0.f, p = 0.f;
#pragma unroll 1
            for (int s = 0; s < NKS; ++s) {
                float gs[8];
                const Raw raw = ld_raw(s);
                map_la(raw.l0, raw.l1, gs);
                const bf16x8 kv = map_qk(raw.k, nk), qv = map_qk(raw.q, nq);
                scan(gs);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float kf = (float)kv[j];
                    const float ky = __shfl(kf, y + 16 * kg);
                    const float gy = __shfl(gs[j], y + 16 * kg);
                    const float f = y <= x ? __builtin_amdgcn_exp2f(gs[j] - gy) : 0.f;
                    a += kf * ky * f;
                    p += (float)qv[j] * ky * f;
                }
            }
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            p += __shfl_xor(p, 16);
            p += __shfl_xor(p, 32);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (y == 4 * kg + e) {
                    ea[e] = a;
                    ep[e] = p;
                }
        }
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
            if (cb == b) {
                ga[cb] = ea;
                gp[cb] = ep;
            }
    }
    // beta and the masks: A strictly lower, P lower including the diagonal
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int y = 4 * kg + e;
            ga[cb][e] = (cb < b || (cb == b && y < x)) ? ga[cb][e] * be : 0.f;
            gp[cb][e] = (cb < b || (cb == b && y <= x)) ? gp[cb][e] : 0.f;
        }
    {
        float amax = 0.f;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(ga[cb][e]));
        if (__ballot(amax > kPairThresh) != 0 && lane == 0) sm.pair = 1;
    }

    // ---- P: row block b through the staging tile to the workspace ----
    __bf16* sb = stg[b];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const bf16x4 v = {(__bf16)gp[cb][0], (__bf16)gp[cb][1], (__bf16)gp[cb][2], (__bf16)gp[cb][3]};
        *reinterpret_cast<bf16x4*>(sb + x * SR + 16 * cb + 4 * kg) = v;
    }
    __builtin_amdgcn_wave_barrier();
    uint8_t* Pw = blk + L::P + (size_t)(16 * b) * C * sizeof(__bf16);
#pragma unroll
    for (int i = 0; i < (NPC + 63) / 64; ++i) {
        const int p = lane + 64 * i;
        if (p < NPC) {
            const int rr = p / (C / 8), pc = p % (C / 8);
            *reinterpret_cast<V16*>(Pw + (size_t)p * 16) = *reinterpret_cast<const V16*>(sb + rr * SR + 8 * pc);
        }
    }

    // ---- X_bb = (I + A_bb)^-1: lane j (mod 16) builds column j ----
    float* xab = xa[b];
    float* xxb = xx[b];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
        if (cb == b)
#pragma unroll
            for (int e = 0; e < 4; ++e) xab[(4 * kg + e) * 16 + x] = ga[cb][e];   // xab[m][i] = A[i][m]
    __builtin_amdgcn_wave_barrier();
    {
        const int jc = x;
        float xv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) xv[i] = i == jc ? 1.f : 0.f;
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
#pragma unroll
        for (int i = 0; i < 16; ++i) xxb[i * 17 + jc] = xv[i];
    }
    __builtin_amdgcn_wave_barrier();
    f32x4 xr, tt[NB];   // X_bb in row layout; T row block b (tiles j <= b), accumulator layout
    {
        f32x4 xn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xr[e] = xxb[x * 17 + 4 * kg + e];
            xn[e] = xxb[(4 * kg + e) * 17 + x];
        }
        const float bc = bsh[16 * b + x];
#pragma unroll
        for (int j = 0; j < NB; ++j) tt[j] = (j == b) ? xn * bc : zero4();
    }
    if (b < NB - 1) {
#pragma unroll
        for (int j = 0; j < NB - 1; ++j)
            if (j == b) tpub[(j * (j + 1) / 2 + j) < NTP ? j * (j + 1) / 2 + j : 0][lane] = tt[j];
    }
    // ---- row wavefront: step t builds T_tj, j < t, on wave t ----
#pragma unroll
    for (int t = 1; t < NB; ++t) {
        __syncthreads();
        if (b == t) {
#pragma unroll
            for (int j = 0; j < t; ++j) {
                f32x4 y = zero4();
#pragma unroll
                for (int m = j; m < t; ++m) {
                    const f32x4 tm = tpub[m * (m + 1) / 2 + j][lane];
#pragma unroll
                    for (int s = 0; s < 4; ++s) y = MF::mma(ga[m][s], tm[s], y);
                }
                f32x4 zt = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) zt = MF::mma(xr[s], y[s], zt);
                tt[j] = -zt;
                if (t < NB - 1) tpub[t * (t + 1) / 2 + j][lane] = tt[j];
            }
        }
    }

    // ---- T (and, when any wave flagged the chunk, its bf16 residual TL):
    //      row block b through the staging tile to the workspace ----
    __syncthreads();   // every wave's flag is in
    const bool pair = sm.pair != 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half == 1 && !pair) break;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const __bf16 hi = (__bf16)tt[j][e];
                sb[(4 * kg + e) * SR + 16 * j + x] = half == 0 ? hi : (__bf16)(tt[j][e] - (float)hi);
            }
        __builtin_amdgcn_wave_barrier();
        uint8_t* Tw = blk + (half == 0 ? L::T : L::TL) + (size_t)(16 * b) * C * sizeof(__bf16);
#pragma unroll
        for (int i = 0; i < (NPC + 63) / 64; ++i) {
            const int p = lane + 64 * i;
            if (p < NPC) {
                const int rr = p / (C / 8), pc = p % (C / 8);
                *reinterpret_cast<V16*>(Tw + (size_t)p * 16) = *reinterpret_cast<const V16*>(sb + rr * SR + 8 * pc);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (b == 0 && lane == 0) *reinterpret_cast<int*>(blk + L::FLAG) = pair ? 1 : 0;
}

template <int DK, int C, bool NORM>
__global__ __launch_bounds__(64 * (C / 16), 4) void wy_prep_channel_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, uint8_t* __restrict__ ws, int64_t T, int H, int NT, int gflags) {
    __shared__ ChanPrepSmem<DK, C> sm;
    const int w = threadIdx.x >> 6;
    constexpr int NB = C / 16;
    if (w == 0) chan_prep_wave<DK, C, 0, NORM>(sm, q, k, log_alpha, beta, ws, T, H, NT, gflags);
    if constexpr (NB > 1)
        if (w == 1) chan_prep_wave<DK, C, (NB > 1 ? 1 : 0), NORM>(sm, q, k, log_alpha, beta, ws, T, H, NT, gflags);
    if constexpr (NB > 2) {
        if (w == 2) chan_prep_wave<DK, C, (NB > 2 ? 2 : 0), NORM>(sm, q, k, log_alpha, beta, ws, T, H, NT, gflags);
        if (w == 3) chan_prep_wave<DK, C, (NB > 3 ? 3 : 0), NORM>(sm, q, k, log_alpha, beta, ws, T, H, NT, gflags);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential state pass.
// ---------------------------------------------------------------------------

template <typename E, int DK, int C, int NW, bool CHANNEL>
struct StageLayout {
    static constexpr int ES = sizeof(E);
    static constexpr int VT = 16 * NW;
    static constexpr int LQ = DK + 16 / ES;   // Q / K / Kh rows (elements)
    static constexpr int LT = C + 16 / ES;    // T / P rows
    static constexpr int LV = VT + 16 / ES;   // V rows
    static constexpr int NL = 2;              // loader waves per workgroup
    static constexpr int QB = DmaTile<C, DK * ES, NL>::BYTES;
    static constexpr int TB = DmaTile<C, C * ES, NL>::BYTES;
    static constexpr int VB = DmaTile<C, VT * ES, NL>::BYTES;
    static constexpr int VECB = (int)WsLayout<E, DK, C, CHANNEL>::VEC_BYTES;
    static constexpr int OQ = 0, OK = QB, OKH = 2 * QB;
    static constexpr int OT = (CHANNEL ? 3 : 2) * QB, OP = OT + TB, OV = OP + TB, OVEC = OV + VB;
    static constexpr int BYTES = (OVEC + VECB + 15) / 16 * 16;
    static constexpr int LO = 16 + 16 / ES;   // output staging rows (elements), per wave
    static constexpr int OSTG = C * LO * ES;
    // Double-buffered (copy of chunk n+1 overlaps chunk n) when it fits.
    static constexpr int NSTAGE = 2 * BYTES + NW * OSTG <= 160 * 1024 ? 2 : 1;
    // bf16 channel-gate calls warm L2 one chunk further ahead; those loads
    // land in a small scratch area.
    static constexpr bool WARM = CHANNEL && sizeof(E) == 2 && NSTAGE == 2;
    static constexpr int OWARM = NSTAGE * BYTES + NW * OSTG;
    static constexpr int TOTAL = OWARM + (WARM ? 256 : 0);
};

// Copies of chunk n's inputs into one LDS stage (see DmaTile).  PARTS selects
// the keys/queries (bit 0) and the T, P, V and decay-vector tiles (bit 1), so
// a chunk's copies can be spread over the previous chunk's computation.
template <typename E, int DK, int C, int NW, bool CHANNEL, int PARTS>
__device__ __forceinline__ void issue_chunk(char* base, int n, const E* q, const E* k, const E* v,
                                            const uint8_t* wsb, int64_t bh, int64_t b, int64_t h,
                                            int64_t T, int H, int DV, int NT, int vt,
                                            int64_t qk_stride, int* oq, const int* ot, int* ov,
                                            int wave, int lane) {
    using L = WsLayout<E, DK, C, CHANNEL>;
    using SL = StageLayout<E, DK, C, NW, CHANNEL>;
    using DQ = DmaTile<C, DK * sizeof(E), SL::NL>;
    using DT = DmaTile<C, C * sizeof(E), SL::NL>;
    using DV_ = DmaTile<C, 16 * NW * sizeof(E), SL::NL>;
    constexpr int ES = sizeof(E);
    constexpr int VT = SL::VT;
    const int64_t t0 = (int64_t)n * C;
    const int64_t row0 = (b * T + t0) * H + h;
    const char* blk = reinterpret_cast<const char*>(wsb + (size_t)(bh * NT + n) * L::BYTES);
    if (T - t0 < C) {   // ragged last chunk: clamp rows of the caller's tensors
        const int len = (int)(T - t0);
        if constexpr (!CHANNEL && (PARTS & 1)) DQ::offsets(oq, qk_stride, len, wave, lane);
        if constexpr ((PARTS & 2) != 0) DV_::offsets(ov, (int64_t)H * DV * ES, len, wave, lane);
    }
    if constexpr ((PARTS & 1) == 0) {
    } else if constexpr (CHANNEL) {
        DQ::issue(base + SL::OQ, blk + L::QG, oq, wave);
        DQ::issue(base + SL::OK, blk + L::KG, oq, wave);
        DQ::issue(base + SL::OKH, blk + L::KH, oq, wave);
    } else {
        DQ::issue(base + SL::OQ, reinterpret_cast<const char*>(q + row0 * DK), oq, wave);
        DQ::issue(base + SL::OK, reinterpret_cast<const char*>(k + row0 * DK), oq, wave);
    }
    if constexpr ((PARTS & 2) != 0) {
        DT::issue(base + SL::OT, blk + L::T, ot, wave);
        DT::issue(base + SL::OP, blk + L::P, ot, wave);
        DV_::issue(base + SL::OV, reinterpret_cast<const char*>(v + row0 * DV + vt * VT), ov, wave);
        constexpr int NVEC = SL::VECB / 16;
        for (int s = wave * 64 + lane; s < NVEC; s += SL::NL * 64)
            __builtin_amdgcn_global_load_lds(blk + L::VEC + 16 * s,
                                             (GDR_LDS void*)(base + SL::OVEC + 16 * (s - lane)), 16, 0, 0);
    }
}

// L2 warming for chunk n of a bf16 channel-gate call: this workgroup's share
// of the head's workspace block (the block split evenly over the head's value
// tiles; one 4-byte load per 128-byte line, a fixed number of loads per wave,
// lanes past the share repeating its last line), then loader 0's own V rows.
// Then waits for every copy issued before it; the warming loads stay in
// flight (loads complete in issue order).
template <typename E, int DK, int C, int NW, bool CHANNEL>
__device__ __forceinline__ void warm_chunk_l2(char* scratch, int n, const E* v, const uint8_t* wsb,
                                              int64_t bh, int64_t b, int64_t h, int64_t T, int H, int DV,
                                              int NT, int vt, int lw, int lane) {
    using L = WsLayout<E, DK, C, CHANNEL>;
    using SL = StageLayout<E, DK, C, NW, CHANNEL>;
    constexpr int NLINES = (int)((L::WARM_BYTES + 127) / 128);
    constexpr int NVT = DK / SL::VT;
    constexpr int PER = (NLINES + NVT - 1) / NVT;
    constexpr int ROUNDS = (PER + SL::NL * 64 - 1) / (SL::NL * 64);
    static_assert(ROUNDS + 1 <= 15, "vmcnt field");
    const char* blk = reinterpret_cast<const char*>(wsb + (size_t)(bh * NT + n) * L::BYTES);
    const int lo = vt * PER, hi = lo + PER < NLINES ? lo + PER : NLINES;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
        const int i = lo + (SL::NL * j + lw) * 64 + lane;
        __builtin_amdgcn_global_load_lds(blk + 128 * (i < hi ? i : hi - 1), (GDR_LDS void*)scratch, 4, 0, 0);
    }
    const int64_t t0 = (int64_t)n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t r = (b * T + t0 + (lane < len ? lane : len - 1)) * H + h;
    __builtin_amdgcn_global_load_lds(v + r * DV + vt * SL::VT, (GDR_LDS void*)scratch, 4, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (ROUNDS + 1));
}

// S^T <- Diag(gamma_last) S^T + Kh^T Ds for the chunk held in one LDS stage.
template <typename E, int DK, int C, int NW, bool CHANNEL>
__device__ __forceinline__ void state_update(f32x4* S, const typename Mma<E>::frag* dsb,
                                             const char* st, int g4, int lane) {
    using SL = StageLayout<E, DK, C, NW, CHANNEL>;
    using M = Mma<E>;
    constexpr bool HALF = (M::KPL == 8 && C < 32);
    constexpr int NKT = HALF ? 1 : C / M::KS;
    constexpr int CT = DK / 16;
    const E* Khs = reinterpret_cast<const E*>(st + (CHANNEL ? SL::OKH : SL::OK));
    const float* vec = reinterpret_cast<const float*>(st + SL::OVEC);
    if constexpr (CHANNEL) {
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) {
            const float4 gl = *reinterpret_cast<const float4*>(vec + 16 * mc + 4 * g4);
            S[mc][0] *= gl.x; S[mc][1] *= gl.y; S[mc][2] *= gl.z; S[mc][3] *= gl.w;
        }
    } else {
        const float gl = vec[C - 1];
#pragma unroll
        for (int mc = 0; mc < CT; ++mc)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[mc][i] *= gl;
    }
    // All transposed key fragments first, so their LDS latencies overlap.
    typename M::frag kf[CT][NKT];
#pragma unroll
    for (int mc = 0; mc < CT; ++mc)
#pragma unroll
        for (int s = 0; s < NKT; ++s) kf[mc][s] = afrag_tr_tok<E, HALF>(Khs, SL::LQ, 16 * mc, s, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NKT; ++s)
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) S[mc] = M::mma(kf[mc][s], dsb[s], S[mc]);
}

template <typename E, int DK, int C, int NW, bool CHANNEL>
__global__ __launch_bounds__(64 * (NW + 2)) __attribute__((amdgpu_waves_per_eu(1, 1))) void state_pass(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ S0, E* __restrict__ o, float* __restrict__ ST,
    const uint8_t* __restrict__ ws, int64_t T, int H, int NT, int DV) {
    using SL = StageLayout<E, DK, C, NW, CHANNEL>;
    using L = WsLayout<E, DK, C, CHANNEL>;
    using M = Mma<E>;
    using frag = typename M::frag;
    using DQ = DmaTile<C, DK * sizeof(E), SL::NL>;    // Q, K (and Kh) tiles
    using DT = DmaTile<C, C * sizeof(E), SL::NL>;     // T, P tiles
    using DV_ = DmaTile<C, 16 * NW * sizeof(E), SL::NL>;
    constexpr int ES = sizeof(E);
    constexpr int VT = SL::VT;
    constexpr int NKC = DK / M::KS;                        // k-steps over channels
    constexpr bool HALF = (M::KPL == 8 && C < 32);         // bf16 with C = 16
    constexpr int NKT = HALF ? 1 : C / M::KS;              // k-steps over tokens
    constexpr int MT = C / 16, CT = DK / 16;
    static_assert(SL::TOTAL <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char smem[SL::TOTAL];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, col = lane & 15;
    const int NVT = DV / VT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = bid % NVT;
    const int64_t bh = bid / NVT;
    const int64_t b = bh / H, h = bh % H;
    const uint8_t* wsb = ws;

    // Waves NW and NW+1 only copy the chunk inputs global -> LDS (their copy
    // instructions may stall issue for a long time; the compute waves never
    // issue any).  Both roles pass the same barriers in the same order:
    //   prologue: B0;  chunk n: [n>0: B1] [1 stage, n>0: Bready] [2 stages: B2]
    if (wave >= NW) {
        const int lw = wave - NW;
        const int64_t qk_stride = CHANNEL ? (int64_t)DK * ES : (int64_t)H * DK * ES;
        int oq[DQ::PER_WAVE], ot[DT::PER_WAVE], ov[DV_::PER_WAVE];
        DQ::offsets(oq, qk_stride, C, lw, lane);
        DT::offsets(ot, (int64_t)C * ES, C, lw, lane);
        DV_::offsets(ov, (int64_t)H * DV * ES, C, lw, lane);
        issue_chunk<E, DK, C, NW, CHANNEL, 3>(smem, 0, q, k, v, wsb, bh, b, h, T, H, DV, NT, vt,
                                              qk_stride, oq, ot, ov, lw, lane);
        wait_dma();
        __syncthreads();                                                   // B0
        for (int n = 0; n < NT; ++n) {
            if (n > 0) __syncthreads();                                    // B1
            if constexpr (SL::NSTAGE == 2) {
                if (n + 1 < NT) {
                    issue_chunk<E, DK, C, NW, CHANNEL, 3>(smem + ((n + 1) & 1) * SL::BYTES, n + 1, q, k, v,
                                                          wsb, bh, b, h, T, H, DV, NT, vt, qk_stride, oq,
                                                          ot, ov, lw, lane);
                    if constexpr (SL::WARM) {
                        if (n + 2 < NT) {
                            warm_chunk_l2<E, DK, C, NW, CHANNEL>(smem + SL::OWARM, n + 2, v, wsb, bh, b, h, T,
                                                                 H, DV, NT, vt, lw, lane);
                        } else {
                            wait_dma();
                        }
                    } else {
                        wait_dma();
                    }
                }
                __syncthreads();                                           // B2
            } else if (n > 0) {
                issue_chunk<E, DK, C, NW, CHANNEL, 3>(smem, n, q, k, v, wsb, bh, b, h, T, H, DV, NT, vt,
                                                      qk_stride, oq, ot, ov, lw, lane);
                wait_dma();
                __syncthreads();                                           // Bready
            }
        }
        return;
    }

    const int vcol = vt * VT + 16 * wave + col;            // this lane's value column
    E* ostg = reinterpret_cast<E*>(smem + SL::NSTAGE * SL::BYTES + wave * SL::OSTG);

    // State slice S^T[c][v]: tile mc, lane (v, g) holds c = 16mc + 4g + i.
    f32x4 S[CT];
#pragma unroll
    for (int mc = 0; mc < CT; ++mc) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S0) x = *reinterpret_cast<const float4*>(S0 + (bh * DV + vcol) * DK + 16 * mc + 4 * g4);
        S[mc] = f32x4{x.x, x.y, x.z, x.w};
    }
    frag dsb[NKT];   // the state update's D operand, carried to the next chunk
    __syncthreads();                                                       // B0

    for (int n = 0; n < NT; ++n) {
        const int cur = SL::NSTAGE == 2 ? (n & 1) : 0;
        const int64_t t0 = (int64_t)n * C;
        const int64_t row0 = (b * T + t0) * H + h;
        if (n > 0) {
            // The previous chunk's state update, from its stage; then every
            // wave is done with that stage and the loaders may refill it.
            state_update<E, DK, C, NW, CHANNEL>(S, dsb, smem + (SL::NSTAGE == 2 ? (cur ^ 1) : 0) * SL::BYTES,
                                                g4, lane);
            __syncthreads();                                               // B1
            store_out<E, C, SL::LO>(o, ostg, row0 - (int64_t)C * H, H, DV, vt * VT + 16 * wave, C, lane);
            if constexpr (SL::NSTAGE == 1) __syncthreads();                // Bready
        }
        const char* st = smem + cur * SL::BYTES;
        const E* Qs = reinterpret_cast<const E*>(st + SL::OQ);
        const E* Ks = reinterpret_cast<const E*>(st + SL::OK);
        const E* Ts = reinterpret_cast<const E*>(st + SL::OT);
        const E* Ps = reinterpret_cast<const E*>(st + SL::OP);
        const E* Vs = reinterpret_cast<const E*>(st + SL::OV);
        const float* vec = reinterpret_cast<const float*>(st + SL::OVEC);

        // Phase A: R = V - Kg S^T, Oi = Qg S^T  (rows = tokens, cols = v)
        frag sb[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) sb[s] = bfrag_acc<E>(S, s);
        f32x4 R[MT], Oa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) { R[mt] = zero4(); Oa[mt] = zero4(); }
        // Fragments are loaded a whole k-step pair ahead of their MFMAs (LDS
        // returns in order, so each MFMA waits only for its own operands).
        constexpr int KH2 = NKC >= 2 ? 2 : 1;
#pragma unroll
        for (int s0 = 0; s0 < NKC; s0 += KH2) {
            frag kf[KH2][MT], qf[KH2][MT];
#pragma unroll
            for (int s = 0; s < KH2; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    kf[s][mt] = afrag_nat(Ks, SL::LQ, 16 * mt, s0 + s, lane);
                    qf[s][mt] = afrag_nat(Qs, SL::LQ, 16 * mt, s0 + s, lane);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < KH2; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    R[mt] = M::mma(kf[s][mt], sb[s0 + s], R[mt]);
                    Oa[mt] = M::mma(qf[s][mt], sb[s0 + s], Oa[mt]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float4 gam = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (!CHANNEL) gam = *reinterpret_cast<const float4*>(vec + 16 * mt + 4 * g4);
            const float gv[4] = {gam.x, gam.y, gam.z, gam.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i;
                const float vv = to_f32(Vs[r * SL::LV + 16 * wave + col]);
                R[mt][i] = vv - gv[i] * R[mt][i];
                Oa[mt][i] *= gv[i];
            }
        }

        // Phase B: D = T R
        frag rb[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            if constexpr (HALF) {
                const __bf16 z = (__bf16)0.f;
                rb[s] = bf16x8{(__bf16)R[0][0], (__bf16)R[0][1], (__bf16)R[0][2], (__bf16)R[0][3],
                               z, z, z, z};
            } else {
                rb[s] = bfrag_acc<E>(R, s);
            }
        }
        f32x4 D[MT];
        {
            frag tf[MT][NKT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < NKT; ++s) tf[mt][s] = afrag_nat_tok<E, HALF>(Ts, SL::LT, 16 * mt, s, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) D[mt] = zero4();
#pragma unroll
            for (int s = 0; s < NKT; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) D[mt] = M::mma(tf[mt][s], rb[s], D[mt]);
        }
        // Chunks the prep flagged: D += TL R, TL = T - bf16(T) read from the
        // workspace (rare; the flag sits after the decay vector in the stage).
        int pair = 0;
        if constexpr (L::PAIR) {
            pair = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(st + SL::OVEC + L::VEC_DATA));
            if (pair) {
                const E* TLg = reinterpret_cast<const E*>(wsb + (size_t)(bh * NT + n) * L::BYTES + L::TL);
                frag tl[MT][NKT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int s = 0; s < NKT; ++s) tl[mt][s] = afrag_nat_tok<E, HALF>(TLg, C, 16 * mt, s, lane);
#pragma unroll
                for (int s = 0; s < NKT; ++s)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) D[mt] = M::mma(tl[mt][s], rb[s], D[mt]);
            }
        }

        // Phase C: O = Oi + P D; the state update's operand Ds is kept for the
        // next iteration (scalar gate: rows scaled by gamma_last / gamma_r).
        frag db[NKT];
        f32x4 Dsc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float4 gh = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (!CHANNEL) gh = *reinterpret_cast<const float4*>(vec + C + 16 * mt + 4 * g4);
            Dsc[mt] = f32x4{D[mt][0] * gh.x, D[mt][1] * gh.y, D[mt][2] * gh.z, D[mt][3] * gh.w};
        }
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            if constexpr (HALF) {
                const __bf16 z = (__bf16)0.f;
                db[s] = bf16x8{(__bf16)D[0][0], (__bf16)D[0][1], (__bf16)D[0][2], (__bf16)D[0][3],
                               z, z, z, z};
                dsb[s] = bf16x8{(__bf16)Dsc[0][0], (__bf16)Dsc[0][1], (__bf16)Dsc[0][2],
                                (__bf16)Dsc[0][3], z, z, z, z};
            } else {
                db[s] = bfrag_acc<E>(D, s);
                dsb[s] = bfrag_acc<E>(Dsc, s);
            }
        }
        {
            frag pf[MT][NKT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < NKT; ++s) pf[mt][s] = afrag_nat_tok<E, HALF>(Ps, SL::LT, 16 * mt, s, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NKT; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) Oa[mt] = M::mma(pf[mt][s], db[s], Oa[mt]);
            if constexpr (L::PAIR) {
                if (pair) {   // O += P (D - bf16(D)): the output keeps D's low bits too
                    f32x4 Dr[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Dr[mt][i] = D[mt][i] - (float)(__bf16)D[mt][i];
                    frag dl[NKT];
#pragma unroll
                    for (int s = 0; s < NKT; ++s) {
                        if constexpr (HALF) {
                            const __bf16 z = (__bf16)0.f;
                            dl[s] = bf16x8{(__bf16)Dr[0][0], (__bf16)Dr[0][1], (__bf16)Dr[0][2], (__bf16)Dr[0][3],
                                           z, z, z, z};
                        } else {
                            dl[s] = bfrag_acc<E>(Dr, s);
                        }
                    }
#pragma unroll
                    for (int s = 0; s < NKT; ++s)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) Oa[mt] = M::mma(pf[mt][s], dl[s], Oa[mt]);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ostg[(16 * mt + 4 * g4 + i) * SL::LO + col] = from_f32<E>(Oa[mt][i]);
        if constexpr (SL::NSTAGE == 2) __syncthreads();                    // B2
    }
    state_update<E, DK, C, NW, CHANNEL>(S, dsb, smem + (SL::NSTAGE == 2 ? ((NT - 1) & 1) : 0) * SL::BYTES,
                                        g4, lane);
    {
        const int64_t t0 = (int64_t)(NT - 1) * C;
        store_out<E, C, SL::LO>(o, ostg, (b * T + t0) * H + h, H, DV, vt * VT + 16 * wave,
                                (int)(T - t0), lane);
    }
    if (ST) {
#pragma unroll
        for (int mc = 0; mc < CT; ++mc)
            *reinterpret_cast<float4*>(ST + (bh * DV + vcol) * DK + 16 * mc + 4 * g4) =
                make_float4(S[mc][0], S[mc][1], S[mc][2], S[mc][3]);
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
template <typename E, int DK, int C, bool CHANNEL, int NW>
static hipError_t launch_state(const ChunkArgs& a, int NT) {
    const int64_t BH = a.B * a.H;
    const int64_t grid = BH * (a.dv / (16 * NW));
    hipLaunchKernelGGL((state_pass<E, DK, C, NW, CHANNEL>), dim3((unsigned)grid), dim3(64 * (NW + 2)), 0,
                       a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.S0, (E*)a.o, a.S_T,
                       (const uint8_t*)a.ws, a.T, (int)a.H, NT, (int)a.dv);
    return hipGetLastError();
}

template <typename E, int DK, int C, bool CHANNEL>
static hipError_t launch_chunk(const ChunkArgs& a) {
    const int NT = (int)((a.T + C - 1) / C);
    const int64_t BH = a.B * a.H;
    if constexpr (CHANNEL && sizeof(E) == 2) {
        const int gflags = (int)(a.prologue & kPrologueGates);
        if (a.prologue & kPrologueL2NormQK)
            hipLaunchKernelGGL((wy_prep_channel_bf16<DK, C, true>), dim3((unsigned)(BH * NT)), dim3(64 * (C / 16)),
                               0, a.stream, (const __bf16*)a.q, (const __bf16*)a.k, a.log_alpha, a.beta,
                               (uint8_t*)a.ws, a.T, (int)a.H, NT, gflags);
        else
            hipLaunchKernelGGL((wy_prep_channel_bf16<DK, C, false>), dim3((unsigned)(BH * NT)), dim3(64 * (C / 16)),
                               0, a.stream, (const __bf16*)a.q, (const __bf16*)a.k, a.log_alpha, a.beta,
                               (uint8_t*)a.ws, a.T, (int)a.H, NT, gflags);
    } else if constexpr (CHANNEL) {
        hipLaunchKernelGGL((wy_prep_channel<E, DK, C>), dim3((unsigned)(BH * NT)), dim3(kThreads), 0,
                           a.stream, (const E*)a.q, (const E*)a.k, a.log_alpha, a.beta,
                           (uint8_t*)a.ws, a.T, (int)a.H, NT);
    } else {
        hipLaunchKernelGGL((wy_prep_scalar<E, DK, C>), dim3((unsigned)(BH * NT)), dim3(kThreads), 0,
                           a.stream, (const E*)a.q, (const E*)a.k, a.log_alpha, a.beta,
                           (uint8_t*)a.ws, a.T, (int)a.H, NT);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // Two waves (32 value columns) per workgroup when that still gives at
    // least one workgroup per CU, otherwise one.
    if (BH * (a.dv / 32) >= 256) return launch_state<E, DK, C, CHANNEL, 2>(a, NT);
    return launch_state<E, DK, C, CHANNEL, 1>(a, NT);
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
    if (NT == 0 || fused_chunk_supported(dk, chunk, bf16, channel)) return 0;
    return (size_t)(B * H * NT) * chunk_block_bytes(dk, chunk, bf16, channel);
}

bool prologue_fused(int64_t chunk, bool bf16, bool channel) {
    // fused into the loads of the single-kernel path and of the bf16
    // channel-gate prep (the state pass reads only the prep's outputs then)
    return bf16 && (channel || chunk == 64);
}

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The gate prologue as an elementwise pass, for the calls whose kernels do not
// fuse it: fp32 io, and the scalar gate at chunks 16 and 32 (whose state pass
// reads q and k straight from the caller's tensors).  Writes what the flags
// select into the staging part of the workspace:
//   unit-norm q and k (io dtype, x / sqrt(sum x^2 + 1e-6) per row),
//   beta from its logit, and the log decay from its logit (fp32).
// A group of DK/4 lanes takes one (token, head) row, 4 channels per lane.
template <typename E, int DK, bool CHANNEL>
__global__ __launch_bounds__(256) void prologue_stage(const E* __restrict__ q, const E* __restrict__ k,
                                                      const float* __restrict__ log_alpha,
                                                      const float* __restrict__ beta, E* __restrict__ qs,
                                                      E* __restrict__ ks, float* __restrict__ las,
                                                      float* __restrict__ bes, int64_t rows, unsigned flags) {
    constexpr int LPR = DK / 4;
    constexpr int RPB = 256 / LPR;
    const int gl = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= rows) return;   // whole lane groups leave together
    const int64_t e0 = row * DK + 4 * gl;
    if (flags & kPrologueL2NormQK) {
        float4 qq = load4(q + e0), kk = load4(k + e0);
        float sq = qq.x * qq.x + qq.y * qq.y + qq.z * qq.z + qq.w * qq.w;
        float sk = kk.x * kk.x + kk.y * kk.y + kk.z * kk.z + kk.w * kk.w;
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
            sq += __shfl_xor(sq, m);
            sk += __shfl_xor(sk, m);
        }
        const float nq = 1.f / sqrtf(sq + 1e-6f), nk = 1.f / sqrtf(sk + 1e-6f);
        store4(qs + e0, make_float4(qq.x * nq, qq.y * nq, qq.z * nq, qq.w * nq));
        store4(ks + e0, make_float4(kk.x * nk, kk.y * nk, kk.z * nk, kk.w * nk));
    }
    if ((flags & kPrologueBetaSigmoid) && gl == 0) bes[row] = sigmoid_of(beta[row]);
    if (flags & kPrologueDecaySoftplus) {
        if constexpr (CHANNEL) {
            const float4 x = *reinterpret_cast<const float4*>(log_alpha + e0);
            *reinterpret_cast<float4*>(las + e0) =
                make_float4(neg_softplus(x.x), neg_softplus(x.y), neg_softplus(x.z), neg_softplus(x.w));
        } else if (gl == 0) {
            las[row] = neg_softplus(log_alpha[row]);
        }
    }
}

template <typename E, int DK, bool CHANNEL>
hipError_t launch_prologue_stage(const ChunkArgs& a, ChunkArgs& b) {
    const int64_t rows = a.B * a.T * a.H;
    const size_t es = sizeof(E);
    char* st = static_cast<char*>(a.ws) +
               align256(chunk_workspace_bytes(a.B, a.T, a.H, a.dk, a.chunk, a.bf16, a.channel));
    E* qs = nullptr;
    E* ks = nullptr;
    float *las = nullptr, *bes = nullptr;
    if (a.prologue & kPrologueL2NormQK) {
        qs = reinterpret_cast<E*>(st);
        st += align256(rows * DK * es);
        ks = reinterpret_cast<E*>(st);
        st += align256(rows * DK * es);
        b.q = qs;
        b.k = ks;
    }
    if (a.prologue & kPrologueBetaSigmoid) {
        bes = reinterpret_cast<float*>(st);
        st += align256(rows * 4);
        b.beta = bes;
    }
    if (a.prologue & kPrologueDecaySoftplus) {
        las = reinterpret_cast<float*>(st);
        b.log_alpha = las;
    }
    b.prologue = 0;
    constexpr int RPB = 256 / (DK / 4);
    hipLaunchKernelGGL((prologue_stage<E, DK, CHANNEL>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, a.stream, (const E*)a.q, (const E*)a.k, a.log_alpha, a.beta, qs, ks, las, bes, rows,
                       a.prologue);
    return hipGetLastError();
}

template <typename E>
hipError_t prologue_stage_e(const ChunkArgs& a, ChunkArgs& b) {
    if (a.dk == 64)
        return a.channel ? launch_prologue_stage<E, 64, true>(a, b) : launch_prologue_stage<E, 64, false>(a, b);
    return a.channel ? launch_prologue_stage<E, 128, true>(a, b) : launch_prologue_stage<E, 128, false>(a, b);
}

}  // namespace

size_t prologue_stage_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, bool bf16, bool channel,
                            unsigned flags) {
    const size_t rows = (size_t)(B * T * H);
    size_t n = 0;
    if (flags & kPrologueL2NormQK) n += 2 * align256(rows * dk * (bf16 ? 2 : 4));
    if (flags & kPrologueBetaSigmoid) n += align256(rows * 4);
    if (flags & kPrologueDecaySoftplus) n += align256(rows * (channel ? dk : 1) * 4);
    return n;
}

size_t chunk_prologue_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t chunk,
                                      bool bf16, bool channel, unsigned flags) {
    const size_t base = chunk_workspace_bytes(B, T, H, dk, chunk, bf16, channel);
    if (T == 0 || flags == 0 || prologue_fused(chunk, bf16, channel)) return base;
    return align256(base) + prologue_stage_bytes(B, T, H, dk, bf16, channel, flags);
}

hipError_t chunk_fwd_launch(const ChunkArgs& a) {
    if (a.T == 0) {
        if (!a.S_T) return hipSuccess;
        const int64_t n4 = a.B * a.H * a.dv * a.dk / 4;
        hipLaunchKernelGGL(copy_state, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, a.stream,
                           a.S0, a.S_T, n4);
        return hipGetLastError();
    }
    if (a.prologue && !prologue_fused(a.chunk, a.bf16, a.channel)) {
        ChunkArgs b = a;
        const hipError_t err = a.bf16 ? prologue_stage_e<__bf16>(a, b) : prologue_stage_e<float>(a, b);
        if (err != hipSuccess) return err;
        return chunk_fwd_launch(b);
    }
    if (fused_chunk_supported(a.dk, a.chunk, a.bf16, a.channel)) return fused_chunk_launch(a);
    if (a.bf16)
        return a.channel ? dispatch_shape<__bf16, true>(a) : dispatch_shape<__bf16, false>(a);
    return a.channel ? dispatch_shape<float, true>(a) : dispatch_shape<float, false>(a);
}

}  // namespace gdr
