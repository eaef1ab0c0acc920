// gdr_gdn2.hip -- decoupled erase and write gates (Gated DeltaNet-2; "Daily
// Papers" pages, the Gated DeltaNet-2 abstract and citation notes):
//
//   S_t = S_{t-1} Diag(alpha_t) (I - k_t (b_t * k_t)^T) + (w_t * v_t) k_t^T,
//   o_t = S_t q_t,
//
// with a channel-wise erase gate b_t in R^{d_k} (key side) and write gate
// w_t in R^{d_v} (value side).  This is a token-sequential scan: the state of
// one (b, h) is spread over the waves of its workgroups (LPR = d_k/8 lanes
// per state row, 8 key channels per lane, two rows per lane group), stays in
// registers for the whole sequence, and every token is applied in order with
// its output written after it; the next token's inputs are loaded while the
// current one is applied (and only waited for at the top of the next step).
// The state is read and written once; the time goes into the per-token
// arithmetic, the row reductions (three or four DPP steps) and the latency of
// the token loads that the ring does not cover.  Two rows per lane share each
// token's decay factors and widened q, k, and the update is two FMAs per
// element.  No load or store sits under a branch inside the ring's whole
// rounds: with a load that may or may not have been issued the compiler
// cannot count the loads in flight and waits for all of them.
#include <type_traits>

#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

// Input buffers per wave (tokens in flight plus one).  One wave per SIMD runs
// the scan, so nothing else hides a token's load latency: five tokens in
// flight keep it covered, in 27 registers per buffer (deeper rings spill
// into the accumulation registers).
constexpr int kGdn2Ring = 6;
// Key channels per lane (NJ float4 groups): a state row spans DK / 8 lanes.
constexpr int kGdn2NJ = 2;

// Sum over the LPR lanes of a state row (4, 8 or 16 consecutive lanes): quad
// xor 1, quad xor 2, half-row mirror, row mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_src(float x) {   // folds into the add as its DPP source
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_src<0xB1>(x);
    x += dpp_src<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp_src<0x141>(x);
    if constexpr (LPR == 16) x += dpp_src<0x140>(x);
    return x;
}

// One token's inputs exactly as a lane loads them (q, k, v still in the io
// type), so that the next token's loads can be in flight while the current
// token is applied: nothing touches them until the next iteration.
template <typename E>
using Raw4 = typename std::conditional<sizeof(E) == 4, float4, bf16x4>::type;

// Value-side pair of one token's rows (the RL = 2 rows of a lane group).
template <typename E>
using Raw2 = typename std::conditional<sizeof(E) == 4, float2, __bf16 __attribute__((ext_vector_type(2)))>::type;

template <typename E, bool CHANNEL>
struct TokenIn {
    Raw4<E> k[kGdn2NJ], q[kGdn2NJ];
    float4 e[kGdn2NJ], la[kGdn2NJ];
    Raw2<E> v;   // rows row0, row0 + 1
    float2 w;
};

template <typename E>
__device__ __forceinline__ float4 widen(const Raw4<E>& x) {
    if constexpr (sizeof(E) == 4) return x;
    else return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

template <typename E, bool CHANNEL, int DK, int LPR>
__device__ __forceinline__ void load_token(TokenIn<E, CHANNEL>& in, const E* __restrict__ q,
                                           const E* __restrict__ k, const E* __restrict__ v,
                                           const float* __restrict__ log_alpha,
                                           const float* __restrict__ erase,
                                           const float* __restrict__ write, int64_t bth, int DV,
                                           int row0, int cl) {
    // wave-uniform token bases, 32-bit lane offsets (scalar-base addressing)
    const char* kb = reinterpret_cast<const char*>(k + bth * DK);
    const char* qb = reinterpret_cast<const char*>(q + bth * DK);
    const char* eb = reinterpret_cast<const char*>(erase + bth * DK);
    const char* lb = reinterpret_cast<const char*>(log_alpha + bth * DK);
#pragma unroll
    for (int j = 0; j < kGdn2NJ; ++j) {
        const uint32_t c = 4u * (uint32_t)(cl + LPR * j);
        in.k[j] = *reinterpret_cast<const Raw4<E>*>(kb + c * sizeof(E));
        in.q[j] = *reinterpret_cast<const Raw4<E>*>(qb + c * sizeof(E));
        in.e[j] = *reinterpret_cast<const float4*>(eb + c * 4u);
        if constexpr (CHANNEL) in.la[j] = *reinterpret_cast<const float4*>(lb + c * 4u);
    }
    if constexpr (!CHANNEL) in.la[0].x = log_alpha[bth];
    in.v = *reinterpret_cast<const Raw2<E>*>(reinterpret_cast<const char*>(v + bth * DV) + (uint32_t)row0 * sizeof(E));
    in.w = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(write + bth * DV) + (uint32_t)row0 * 4u);
}

// Reads every register of a token's inputs (an empty asm), which places the
// wait for their loads here.  At the top of an iteration this waits only for
// the loads issued one iteration earlier: the compiler cannot count loads in
// flight across the loop's back edge, and would otherwise wait for all of
// them, the new prefetch included, at the first use.
__device__ __forceinline__ void touch(const float4& x) { asm volatile("" ::"v"(__builtin_bit_cast(f32x4, x))); }
__device__ __forceinline__ void touch(const float2& x) { asm volatile("" ::"v"(x.x), "v"(x.y)); }
__device__ __forceinline__ void touch(const bf16x4& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void touch(__bf16 __attribute__((ext_vector_type(2))) x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void touch(float x) { asm volatile("" ::"v"(x)); }

template <typename E, bool CHANNEL>
__device__ __forceinline__ void landed(const TokenIn<E, CHANNEL>& in) {
#pragma unroll
    for (int j = 0; j < kGdn2NJ; ++j) {
        touch(in.k[j]);
        touch(in.q[j]);
        touch(in.e[j]);
        if constexpr (CHANNEL) touch(in.la[j]);
    }
    if constexpr (!CHANNEL) touch(in.la[0].x);
    touch(in.v);
    touch(in.w);
}

template <typename E>
__device__ __forceinline__ float2 widen2(const Raw2<E>& x) {
    if constexpr (sizeof(E) == 4) return x;
    else return make_float2((float)x[0], (float)x[1]);
}

template <typename E, bool CHANNEL, int DK, int RING>
__global__ __launch_bounds__(256) void gdn2_scan(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ erase,
    const float* __restrict__ write, const float* __restrict__ S0, E* __restrict__ o,
    float* __restrict__ ST, int64_t BH, int H, int64_t T, int DV) {
    constexpr int LPR = DK / (4 * kGdn2NJ);   // lanes per state row
    constexpr int RL = 2;                     // state rows per lane (one lane group)
    constexpr int RPW = kWave / LPR * RL;     // rows per wave
    const int lane = threadIdx.x & 63;
    // the wave index is uniform per wave (readfirstlane tells the compiler,
    // so the per-token bases stay in scalar registers)
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = DV / RPW;
    const int64_t bh = gw / wpb;
    if (bh >= BH) return;
    const int64_t b = bh / H, h = bh % H;
    const int row0 = (int)(gw % wpb) * RPW + (lane / LPR) * RL;
    const int cl = lane % LPR;
    const int64_t base = bh * (int64_t)DV * DK + (int64_t)row0 * DK;

    f32x4 s[RL][kGdn2NJ];
#pragma unroll
    for (int r = 0; r < RL; ++r)
#pragma unroll
        for (int j = 0; j < kGdn2NJ; ++j)
            s[r][j] = S0 ? *reinterpret_cast<const f32x4*>(S0 + base + (int64_t)r * DK + 4 * (cl + LPR * j))
                         : f32x4{0.f, 0.f, 0.f, 0.f};

    // A ring of RING input buffers, unrolled so that no buffer is ever copied:
    // the step for token t applies it from one buffer and loads token
    // t + RING - 1 into the buffer the previous step emptied, so each token's
    // loads have RING - 1 steps to land.  The decay factors and the widened
    // q, k serve both rows of the lane.
    auto step = [&](TokenIn<E, CHANNEL>& cur, TokenIn<E, CHANNEL>& nxt, int64_t t) {
        const int64_t bth = (b * T + t) * H + h;    // token row of [B, T, H, *]
        landed(cur);
        __builtin_amdgcn_sched_barrier(0);
        {   // past the end, the last token again: every step issues the same loads
            const int64_t tn = t + RING - 1 < T ? t + RING - 1 : T - 1;
            load_token<E, CHANNEL, DK, LPR>(nxt, q, k, v, log_alpha, erase, write, (b * T + tn) * H + h, DV,
                                            row0, cl);
        }
        float4 kk[kGdn2NJ], qq[kGdn2NJ], a[kGdn2NJ];
        const float a1 = CHANNEL ? 1.f : __expf(cur.la[0].x);
#pragma unroll
        for (int j = 0; j < kGdn2NJ; ++j) {
            kk[j] = widen<E>(cur.k[j]);
            qq[j] = widen<E>(cur.q[j]);
            if constexpr (CHANNEL)
                a[j] = make_float4(__expf(cur.la[j].x), __expf(cur.la[j].y), __expf(cur.la[j].z), __expf(cur.la[j].w));
            else a[j] = make_float4(a1, a1, a1, a1);
        }
        const float2 vv = widen2<E>(cur.v);
        const float u[RL] = {cur.w.x * vv.x, cur.w.y * vv.y};
        float rd[RL], od[RL];
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            rd[r] = 0.f;
#pragma unroll
            for (int j = 0; j < kGdn2NJ; ++j) {
                s[r][j][0] *= a[j].x; s[r][j][1] *= a[j].y; s[r][j][2] *= a[j].z; s[r][j][3] *= a[j].w;
                rd[r] += s[r][j][0] * kk[j].x + s[r][j][1] * kk[j].y + s[r][j][2] * kk[j].z + s[r][j][3] * kk[j].w;
            }
        }
#pragma unroll
        for (int r = 0; r < RL; ++r) rd[r] = row_sum<LPR>(rd[r]);
        // s += k * (u - rd e): the write along k and the erase along b * k
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            od[r] = 0.f;
#pragma unroll
            for (int j = 0; j < kGdn2NJ; ++j) {
                s[r][j][0] += kk[j].x * (u[r] - rd[r] * cur.e[j].x);
                s[r][j][1] += kk[j].y * (u[r] - rd[r] * cur.e[j].y);
                s[r][j][2] += kk[j].z * (u[r] - rd[r] * cur.e[j].z);
                s[r][j][3] += kk[j].w * (u[r] - rd[r] * cur.e[j].w);
                od[r] += s[r][j][0] * qq[j].x + s[r][j][1] * qq[j].y + s[r][j][2] * qq[j].z + s[r][j][3] * qq[j].w;
            }
        }
#pragma unroll
        for (int r = 0; r < RL; ++r) od[r] = row_sum<LPR>(od[r]);
        // every lane of a row holds its sum: all store it (no branch around the store)
        o[bth * DV + row0] = from_f32<E>(od[0]);
        o[bth * DV + row0 + 1] = from_f32<E>(od[1]);
    };
    TokenIn<E, CHANNEL> buf[RING];
    if (T > 0) {
#pragma unroll
        for (int i = 0; i + 1 < RING; ++i)
            load_token<E, CHANNEL, DK, LPR>(buf[i], q, k, v, log_alpha, erase, write,
                                            (b * T + (i < T ? i : T - 1)) * H + h, DV, row0, cl);
#pragma unroll
        for (int i = 0; i + 1 < RING; ++i) landed(buf[i]);   // nothing enters the loop in flight
#pragma unroll
        for (int r = 0; r < RL; ++r)
#pragma unroll
            for (int j = 0; j < kGdn2NJ; ++j) asm volatile("" ::"v"(s[r][j]));
    }
    // Whole rounds of RING tokens with no condition around any step (so the
    // compiler can count the loads in flight), then the tail.
    int64_t t = 0;
    for (; t + RING <= T; t += RING) {
#pragma unroll
        for (int i = 0; i < RING; ++i) step(buf[i], buf[(i + RING - 1) % RING], t + i);
    }
#pragma unroll
    for (int i = 0; i < RING; ++i)
        if (t + i < T) step(buf[i], buf[(i + RING - 1) % RING], t + i);
    if (ST) {
#pragma unroll
        for (int r = 0; r < RL; ++r)
#pragma unroll
            for (int j = 0; j < kGdn2NJ; ++j)
                *reinterpret_cast<f32x4*>(ST + base + (int64_t)r * DK + 4 * (cl + LPR * j)) = s[r][j];
    }
}

template <typename E, bool CHANNEL, int DK>
hipError_t launch_gdn2_t(const Gdn2Args& a) {
    constexpr int RPW = kWave / (DK / (4 * kGdn2NJ)) * 2;
    const int64_t waves = a.B * a.H * (a.dv / RPW);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((gdn2_scan<E, CHANNEL, DK, kGdn2Ring>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_alpha, a.erase, a.write,
                       a.S0, (E*)a.o, a.S_T, a.B * a.H, (int)a.H, a.T, (int)a.dv);
    return hipGetLastError();
}

template <typename E, bool CHANNEL>
hipError_t launch_gdn2_dk(const Gdn2Args& a) {
    return a.dk == 64 ? launch_gdn2_t<E, CHANNEL, 64>(a) : launch_gdn2_t<E, CHANNEL, 128>(a);
}

}  // namespace

hipError_t gdn2_fwd_launch(const Gdn2Args& a) {
    if (a.bf16) return a.channel ? launch_gdn2_dk<__bf16, true>(a) : launch_gdn2_dk<__bf16, false>(a);
    return a.channel ? launch_gdn2_dk<float, true>(a) : launch_gdn2_dk<float, false>(a);
}

}  // namespace gdr
