// gdr_gdn2.hip -- decoupled erase and write gates (Gated DeltaNet-2; "Daily
// Papers" pages, the Gated DeltaNet-2 abstract and citation notes):
//
//   S_t = S_{t-1} Diag(alpha_t) (I - k_t (b_t * k_t)^T) + (w_t * v_t) k_t^T,
//   o_t = S_t q_t,
//
// with a channel-wise erase gate b_t in R^{d_k} (key side) and write gate
// w_t in R^{d_v} (value side).  This is a token-sequential scan: the state of
// one (b, h) is spread over the waves of its workgroups (LPR = d_k/16 lanes
// per state row, 16 key channels per lane, one row per lane group), stays in
// registers for the whole sequence, and every token is applied in order with
// its output written after it; the next token's inputs are loaded while the
// current one is applied.  The state is read and written once; the time goes
// into the per-token arithmetic and row reductions (three DPP steps).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

template <int LPR>
__device__ __forceinline__ float row_sum16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
    if constexpr (LPR == 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
    return x;
}

// One token's inputs as a lane loads them (raw), so the next token's loads can
// be in flight while the current token is applied.
template <typename E, bool CHANNEL>
struct TokenIn {
    float4 k[4], q[4], e[4], la[4];
    float v, w;
};

template <typename E, bool CHANNEL, int DK, int LPR>
__device__ __forceinline__ void load_token(TokenIn<E, CHANNEL>& in, const E* __restrict__ q,
                                           const E* __restrict__ k, const E* __restrict__ v,
                                           const float* __restrict__ log_alpha,
                                           const float* __restrict__ erase,
                                           const float* __restrict__ write, int64_t bth, int DV,
                                           int row, int cl) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * (cl + LPR * j);
        in.k[j] = load4(k + bth * DK + c);
        in.q[j] = load4(q + bth * DK + c);
        in.e[j] = *reinterpret_cast<const float4*>(erase + bth * DK + c);
        if constexpr (CHANNEL) in.la[j] = *reinterpret_cast<const float4*>(log_alpha + bth * DK + c);
    }
    if constexpr (!CHANNEL) in.la[0].x = log_alpha[bth];
    in.v = to_f32(v[bth * DV + row]);
    in.w = write[bth * DV + row];
}

template <typename E, bool CHANNEL, int DK>
__global__ __launch_bounds__(256) void gdn2_scan(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ erase,
    const float* __restrict__ write, const float* __restrict__ S0, E* __restrict__ o,
    float* __restrict__ ST, int64_t BH, int H, int64_t T, int DV) {
    constexpr int LPR = DK / 16;
    constexpr int RPW = kWave / LPR;    // rows per wave (one per lane group)
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int wpb = DV / RPW;
    const int64_t bh = gw / wpb;
    if (bh >= BH) return;
    const int64_t b = bh / H, h = bh % H;
    const int row = (int)(gw % wpb) * RPW + lane / LPR;
    const int cl = lane % LPR;
    const int64_t base = bh * (int64_t)DV * DK + (int64_t)row * DK;

    f32x4 s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        s[j] = S0 ? *reinterpret_cast<const f32x4*>(S0 + base + 4 * (cl + LPR * j)) : f32x4{0.f, 0.f, 0.f, 0.f};

    TokenIn<E, CHANNEL> cur, nxt;
    if (T > 0) load_token<E, CHANNEL, DK, LPR>(cur, q, k, v, log_alpha, erase, write, (b * T) * H + h, DV, row, cl);
    for (int64_t t = 0; t < T; ++t) {
        const int64_t bth = (b * T + t) * H + h;    // token row of [B, T, H, *]
        if (t + 1 < T)
            load_token<E, CHANNEL, DK, LPR>(nxt, q, k, v, log_alpha, erase, write, bth + H, DV, row, cl);
        float rd = 0.f;
        const float a1 = CHANNEL ? 1.f : __expf(cur.la[0].x);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 a;
            if constexpr (CHANNEL) a = make_float4(__expf(cur.la[j].x), __expf(cur.la[j].y), __expf(cur.la[j].z), __expf(cur.la[j].w));
            else a = make_float4(a1, a1, a1, a1);
            s[j][0] *= a.x; s[j][1] *= a.y; s[j][2] *= a.z; s[j][3] *= a.w;
            rd += s[j][0] * cur.k[j].x + s[j][1] * cur.k[j].y + s[j][2] * cur.k[j].z + s[j][3] * cur.k[j].w;
        }
        rd = row_sum16<LPR>(rd);
        const float u = cur.w * cur.v;
        float od = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j][0] += u * cur.k[j].x - rd * cur.e[j].x * cur.k[j].x;
            s[j][1] += u * cur.k[j].y - rd * cur.e[j].y * cur.k[j].y;
            s[j][2] += u * cur.k[j].z - rd * cur.e[j].z * cur.k[j].z;
            s[j][3] += u * cur.k[j].w - rd * cur.e[j].w * cur.k[j].w;
            od += s[j][0] * cur.q[j].x + s[j][1] * cur.q[j].y + s[j][2] * cur.q[j].z + s[j][3] * cur.q[j].w;
        }
        od = row_sum16<LPR>(od);
        if (cl == 0) o[bth * DV + row] = from_f32<E>(od);
        cur = nxt;
    }
    if (ST) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(ST + base + 4 * (cl + LPR * j)) = s[j];
    }
}

template <typename E, bool CHANNEL, int DK>
hipError_t launch_gdn2_t(const Gdn2Args& a) {
    constexpr int RPW = kWave / (DK / 16);
    const int64_t waves = a.B * a.H * (a.dv / RPW);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((gdn2_scan<E, CHANNEL, DK>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
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
