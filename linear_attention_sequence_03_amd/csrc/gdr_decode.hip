// gdr_decode.hip -- one recurrent decode step of the gated delta rule.
//
// Per (b,h) and value row i of the fp32 state S [dv][dk]:
//   s~ = S[i,:] * alpha            decay                 ("FG2-GDN" page, section 1)
//   p  = s~ . k                    read the memory at k
//   u  = beta (v_i - p)            delta-rule correction ("FG2-GDN" page, section 5,
//                                                         "Delta Rule and Online Learning")
//   S'[i,:] = s~ + u k             rank-1 write
//   o_i = S'[i,:] . q              read-out after the update
//
// The step is a pure HBM stream over the state (read once, write once; no
// reuse), so the kernel is built for bytes in flight: each lane owns one
// 16-byte slice (4 key channels) of a row, a wave covers 64*16 bytes = 2 rows
// (dk=128) or 4 rows (dk=64) per pass, and every lane issues all NPASS row
// loads before any arithmetic.  Loads and stores are non-temporal (the state
// is far larger than the caches and is not re-read).  The two dot products are
// reduced across the lanes of a row with xor shuffles.  In-place (S_out ==
// S_in) is safe: each 16-byte slice is read and written by the same lane.
//
// The gate prologue ("FG2-GDN" page, section 3.5: unit-norm q and k, beta as
// the sigmoid of its logit, the decay from its logit as alpha = 1 / (1 + e^x))
// runs in the kernel when asked for: each row's lanes sum the squares of their
// key and query channels; beta and log alpha are mapped as they are loaded.
//
// With channel-wise write rates (FG2, "FG2-GDN" page, sections 3.2 and 3.4)
// the same step runs with unit rate on the scaled key sqrt(beta^k) * k and the
// scaled value sqrt(beta^v) * v (beta^v = beta^k unless given).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <typename E, bool CHANNEL, int DK, bool FG2>
__global__ __launch_bounds__(256) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ beta_k, const float* __restrict__ beta_v,
    const float* S_in, float* S_out, E* __restrict__ o, int64_t BH, int DV, int prologue) {
    constexpr int LPR = DK / 4;      // lanes per state row
    constexpr int RPP = kWave / LPR; // rows per pass of one wave
    constexpr int NPASS = 4;
    constexpr int RPW = RPP * NPASS; // rows per wave
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int wpb = DV / RPW;        // waves per (b,h)
    const int64_t bh = gw / wpb;
    if (bh >= BH) return;
    const int row0 = (int)(gw % wpb) * RPW + lane / LPR;
    const int c0 = 4 * (lane % LPR);

    float4 kk = load4(k + bh * DK + c0);
    if constexpr (FG2) {
        const float4 r = *reinterpret_cast<const float4*>(beta_k + bh * DK + c0);
        kk = make_float4(sqrtf(r.x) * kk.x, sqrtf(r.y) * kk.y, sqrtf(r.z) * kk.z, sqrtf(r.w) * kk.w);
    }
    float4 qq = load4(q + bh * DK + c0);
    if (prologue & kPrologueL2NormQK) {   // unit-norm q and k: sums over the row's lanes
        float sk = kk.x * kk.x + kk.y * kk.y + kk.z * kk.z + kk.w * kk.w;
        float sq = qq.x * qq.x + qq.y * qq.y + qq.z * qq.z + qq.w * qq.w;
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
            sk += __shfl_xor(sk, m);
            sq += __shfl_xor(sq, m);
        }
        const float nk = 1.f / sqrtf(sk + 1e-6f), nq = 1.f / sqrtf(sq + 1e-6f);
        kk = make_float4(kk.x * nk, kk.y * nk, kk.z * nk, kk.w * nk);
        qq = make_float4(qq.x * nq, qq.y * nq, qq.z * nq, qq.w * nq);
    }
    float4 aa;
    const bool lsp = !FG2 && (prologue & kPrologueDecaySoftplus);   // decay from its logit
    if constexpr (CHANNEL) {
        float4 la = *reinterpret_cast<const float4*>(log_alpha + bh * DK + c0);
        if (lsp) la = make_float4(neg_softplus(la.x), neg_softplus(la.y), neg_softplus(la.z), neg_softplus(la.w));
        aa = make_float4(expf(la.x), expf(la.y), expf(la.z), expf(la.w));
    } else {
        const float la = log_alpha[bh];
        const float a = expf(lsp ? neg_softplus(la) : la);
        aa = make_float4(a, a, a, a);
    }
    float b = FG2 ? 1.f : beta[bh];
    if (!FG2 && (prologue & kPrologueBetaSigmoid)) b = sigmoid_of(b);
    const float* vrate = FG2 ? (beta_v ? beta_v : beta_k) : nullptr;

    const int64_t base = bh * (int64_t)DV * DK;
    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
        s[p] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(S_in + base + (int64_t)(row0 + p * RPP) * DK + c0));

#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = row0 + p * RPP;
        f32x4 sd;
        sd[0] = s[p][0] * aa.x; sd[1] = s[p][1] * aa.y;
        sd[2] = s[p][2] * aa.z; sd[3] = s[p][3] * aa.w;
        float pd = sd[0] * kk.x + sd[1] * kk.y + sd[2] * kk.z + sd[3] * kk.w;
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) pd += __shfl_xor(pd, m);
        float vi = to_f32(v[bh * DV + row]);
        if constexpr (FG2) vi *= sqrtf(vrate[bh * DV + row]);
        const float u = b * (vi - pd);
        f32x4 sn;
        sn[0] = sd[0] + u * kk.x; sn[1] = sd[1] + u * kk.y;
        sn[2] = sd[2] + u * kk.z; sn[3] = sd[3] + u * kk.w;
        __builtin_nontemporal_store(
            sn, reinterpret_cast<f32x4*>(S_out + base + (int64_t)row * DK + c0));
        float od = sn[0] * qq.x + sn[1] * qq.y + sn[2] * qq.z + sn[3] * qq.w;
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) od += __shfl_xor(od, m);
        if (lane % LPR == 0) o[bh * DV + row] = from_f32<E>(od);
    }
}

// Sum over the LPR (4 or 8) consecutive lanes that share a state row, left in
// every one of them: DPP quad permutations (xor 1, xor 2), then the half-row
// mirror (lane i <-> 7 - i) for 8 lanes.  No LDS traffic.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
    if constexpr (LPR == 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
    return x;
}

// Several tokens per sequence in one pass over the state (speculative decoding:
// verify a run of draft tokens, then keep the state of the accepted prefix;
// "FG2-GDN" page, "Limitations / Inference Challenges").  The state rows stay
// in registers while the tokens t = 0..Td-1 are applied in order, so the work
// per token is arithmetic and two row reductions; the layout is chosen for
// cheap reductions: LPR = DK/16 lanes share a row, lane c holds the 16
// channels 4(c + LPR j) + e (j, e < 4: each of its four 16-byte accesses is
// part of one contiguous row segment across the row's lanes), and a row sum is
// three DPP steps.  o_t is written after token t (when o is given), and the
// state after the first n tokens is stored, n = accepted[b] clamped to
// [0, Td] (Td when accepted is NULL; nothing stored when S_out is NULL).
// S_out may equal S_in: a lane writes only the slices it read, after reading.
//
// Every wave of a workgroup works on the same (b, h), so the draft tokens'
// inputs (k, q, the decay, beta, and the values of the workgroup's rows) are
// staged in LDS once per workgroup, kMultiGroup tokens at a time, with the
// loads of the first group in flight together with the state loads; the token
// loop then reads them from LDS instead of waiting on global memory per token.
constexpr int kMultiGroup = 16;

// Rows per lane: the channel gate's per-token decay factors (an exp per key
// channel) are shared by four rows of a lane, the scalar gate's by two (more
// rows cost registers and occupancy that the scalar gate does not win back).
template <int DK, bool CHANNEL>
struct MultiShape {
    static constexpr int LPR = DK / 16;           // lanes per state row
    static constexpr int RPP = kWave / LPR;       // rows per pass of one wave
    static constexpr int NPASS = CHANNEL ? 4 : 2;
    static constexpr int RPW = RPP * NPASS;       // rows per wave
    static constexpr int WPH = DK / RPW;          // waves per (b, h) (d_v = d_k)
    static constexpr int WPB = WPH < 4 ? WPH : 4; // waves per workgroup
    static constexpr int ROWS = WPB * RPW;        // state rows per workgroup
};

template <typename E, bool CHANNEL, int DK>
__global__ __launch_bounds__(64 * MultiShape<DK, CHANNEL>::WPB) void decode_multi_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* S_in,
    float* S_out, const int32_t* __restrict__ accepted, E* __restrict__ o, int H, int Td, int DV) {
    using MS = MultiShape<DK, CHANNEL>;
    constexpr int LPR = MS::LPR, RPP = MS::RPP, NPASS = MS::NPASS, RPW = MS::RPW, ROWS = MS::ROWS;
    constexpr int NTH = 64 * MS::WPB;
    constexpr int G = kMultiGroup;
    constexpr int LA = CHANNEL ? DK : 1;          // decay values per token
    __shared__ __attribute__((aligned(16))) float sk[G][DK], sq[G][DK], sla[G][LA], sbt[G], sv[G][ROWS];

    const int tid = threadIdx.x, lane = tid & 63;
    // workgroups tile the (b, h) rows exactly: every wave of one is on the same (b, h)
    const int nblk = DV / ROWS;
    const int64_t bh = blockIdx.x / nblk;
    const int rbase = (int)(blockIdx.x % nblk) * ROWS;   // first row of the workgroup
    const int64_t b = bh / H, h = bh % H;
    const int row0 = rbase + (tid >> 6) * RPW + lane / LPR;
    const int cl = lane % LPR;
    int nacc = Td;
    if (accepted) nacc = min(max(accepted[b], 0), Td);

    const int64_t base = bh * (int64_t)DV * DK;
    auto sp = [&](int p, int j) { return base + (int64_t)(row0 + p * RPP) * DK + 4 * (cl + LPR * j); };
    f32x4 s[NPASS][4];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[p][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S_in + sp(p, j)));
    auto store_state = [&]() {
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_nontemporal_store(s[p][j], reinterpret_cast<f32x4*>(S_out + sp(p, j)));
    };
    if (S_out && nacc == 0) store_state();
    for (int t0 = 0; t0 < Td; t0 += G) {
        const int ng = Td - t0 < G ? Td - t0 : G;
        if (t0 > 0) __syncthreads();   // every wave is done with the previous group
        // ---- stage tokens t0 .. t0 + ng - 1 (as fp32) ----
        for (int e = tid; e < ng * (DK / 4); e += NTH) {
            const int i = e / (DK / 4), c = 4 * (e % (DK / 4));
            const int64_t bth = (b * Td + t0 + i) * H + h;
            *reinterpret_cast<float4*>(&sk[i][c]) = load4(k + bth * DK + c);
            *reinterpret_cast<float4*>(&sq[i][c]) = load4(q + bth * DK + c);
            if constexpr (CHANNEL)
                *reinterpret_cast<float4*>(&sla[i][c]) = *reinterpret_cast<const float4*>(log_alpha + bth * DK + c);
        }
        for (int e = tid; e < ng * ROWS; e += NTH) {
            const int i = e / ROWS, r = e % ROWS;
            const int64_t bth = (b * Td + t0 + i) * H + h;
            sv[i][r] = to_f32(v[bth * DV + rbase + r]);
        }
        if (tid < ng) {
            const int64_t bth = (b * Td + t0 + tid) * H + h;
            sbt[tid] = beta[bth];
            if constexpr (!CHANNEL) sla[tid][0] = log_alpha[bth];
        }
        __syncthreads();
        for (int i = 0; i < ng; ++i) {
            const int t = t0 + i;
            const int64_t bth = (b * Td + t) * H + h;   // token row of [B, Td, H, *]
            float4 kk[4], qq[4], aa[4];
            float a1 = 1.f;
            if constexpr (!CHANNEL) a1 = expf(sla[i][0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 4 * (cl + LPR * j);
                kk[j] = *reinterpret_cast<const float4*>(&sk[i][c]);
                qq[j] = *reinterpret_cast<const float4*>(&sq[i][c]);
                if constexpr (CHANNEL) {
                    const float4 la = *reinterpret_cast<const float4*>(&sla[i][c]);
                    aa[j] = make_float4(expf(la.x), expf(la.y), expf(la.z), expf(la.w));
                } else {
                    aa[j] = make_float4(a1, a1, a1, a1);
                }
            }
            const float bt = sbt[i];
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int row = row0 + p * RPP;
                float pd = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s[p][j][0] *= aa[j].x; s[p][j][1] *= aa[j].y;
                    s[p][j][2] *= aa[j].z; s[p][j][3] *= aa[j].w;
                    pd += s[p][j][0] * kk[j].x + s[p][j][1] * kk[j].y + s[p][j][2] * kk[j].z +
                          s[p][j][3] * kk[j].w;
                }
                pd = row_sum<LPR>(pd);
                const float u = bt * (sv[i][row - rbase] - pd);
                float od = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s[p][j][0] += u * kk[j].x; s[p][j][1] += u * kk[j].y;
                    s[p][j][2] += u * kk[j].z; s[p][j][3] += u * kk[j].w;
                    od += s[p][j][0] * qq[j].x + s[p][j][1] * qq[j].y + s[p][j][2] * qq[j].z +
                          s[p][j][3] * qq[j].w;
                }
                if (o) {
                    od = row_sum<LPR>(od);
                    if (cl == 0) o[bth * DV + row] = from_f32<E>(od);
                }
            }
            if (S_out && t + 1 == nacc) store_state();
        }
    }
}

template <typename E, bool CHANNEL, int DK>
static hipError_t launch_decode_multi(const DecodeMultiArgs& a) {
    using MS = MultiShape<DK, CHANNEL>;
    const int64_t blocks = a.B * a.H * (a.dv / MS::ROWS);
    hipLaunchKernelGGL((decode_multi_kernel<E, CHANNEL, DK>), dim3((unsigned)blocks), dim3(64 * MS::WPB), 0,
                       a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_alpha, a.beta,
                       a.S_in, a.S_out, a.accepted, (E*)a.o, (int)a.H, (int)a.Td, (int)a.dv);
    return hipGetLastError();
}

template <typename E, bool CHANNEL>
static hipError_t launch_decode_multi_dk(const DecodeMultiArgs& a) {
    return a.dk == 64 ? launch_decode_multi<E, CHANNEL, 64>(a) : launch_decode_multi<E, CHANNEL, 128>(a);
}

hipError_t decode_multi_launch(const DecodeMultiArgs& a) {
    if (a.bf16)
        return a.channel ? launch_decode_multi_dk<__bf16, true>(a) : launch_decode_multi_dk<__bf16, false>(a);
    return a.channel ? launch_decode_multi_dk<float, true>(a) : launch_decode_multi_dk<float, false>(a);
}

template <typename E, bool CHANNEL, int DK>
static hipError_t launch_decode(const DecodeArgs& a) {
    constexpr int RPW = (kWave / (DK / 4)) * 4;
    const int64_t waves = a.B * a.H * (a.dv / RPW);
    const int64_t blocks = (waves + 3) / 4;
    if (a.beta_k)
        hipLaunchKernelGGL((decode_kernel<E, CHANNEL, DK, true>), dim3((unsigned)blocks), dim3(256), 0,
                           a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_alpha,
                           a.beta, a.beta_k, a.beta_v, a.S_in, a.S_out, (E*)a.o, a.B * a.H,
                           (int)a.dv, 0);
    else
        hipLaunchKernelGGL((decode_kernel<E, CHANNEL, DK, false>), dim3((unsigned)blocks), dim3(256),
                           0, a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_alpha,
                           a.beta, a.beta_k, a.beta_v, a.S_in, a.S_out, (E*)a.o, a.B * a.H,
                           (int)a.dv, (int)a.prologue);
    return hipGetLastError();
}

template <typename E, bool CHANNEL>
static hipError_t launch_decode_dk(const DecodeArgs& a) {
    return a.dk == 64 ? launch_decode<E, CHANNEL, 64>(a) : launch_decode<E, CHANNEL, 128>(a);
}

hipError_t decode_step_launch(const DecodeArgs& a) {
    if (a.bf16)
        return a.channel ? launch_decode_dk<__bf16, true>(a) : launch_decode_dk<__bf16, false>(a);
    return a.channel ? launch_decode_dk<float, true>(a) : launch_decode_dk<float, false>(a);
}

}  // namespace gdr
