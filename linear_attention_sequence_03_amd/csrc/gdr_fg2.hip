// gdr_fg2.hip -- channel-wise write rates (FG2-GDN and FG2-GDN+, "FG2-GDN" page,
// sections 3.2 and 3.4-3.6) on top of the chunkwise path.
//
// The write rate is a vector beta^k_t in R^{d_k} that enters through the scaled
// key k~_t = sqrt(beta^k_t) * k_t (elementwise); the value is scaled the same
// way, v~_t = sqrt(beta^v_t) * v_t, with beta^v = beta^k for FG2-GDN and a
// separate d_v-vector for FG2-GDN+.  The update is the tied delta rule with
// unit rate on the scaled vectors,
//     S_t = S_{t-1} Diag(alpha_t) (I - k~ k~^T) + v~ k~^T,   o_t = S_t q_t,
// so the page's point that the chunkwise WY algorithm carries over unchanged
// holds literally: this file scales k and v once (a prologue over the whole
// call, into the caller's workspace) and runs the ordinary chunk path on
// (q, k~, v~) with beta = 1.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// One thread per 8 elements of a row of k (the first dk/8 groups of a token)
// or of v (the rest): one 16-byte (bf16) or 32-byte (fp32) load of the vector,
// two 16-byte non-temporal loads of the rates (read once), one store of the
// scaled result.  The unit rates are written by the first ntok threads.
template <typename E>
__global__ __launch_bounds__(256) void fg2_scale(const E* __restrict__ k, const E* __restrict__ v,
                                                 const float* __restrict__ beta_k,
                                                 const float* __restrict__ beta_v,
                                                 E* __restrict__ ks, E* __restrict__ vs,
                                                 float* __restrict__ ones, int64_t ntok, int dk,
                                                 int dv) {
    const int gk = dk / 8, gt = (dk + dv) / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ntok * gt) return;
    if (i < ntok) ones[i] = 1.f;
    const int64_t tok = i / gt;
    const int g = (int)(i - tok * gt);
    const bool isk = g < gk;
    const int64_t off = isk ? tok * dk + 8 * g : tok * dv + 8 * (g - gk);
    const float* rate = (isk ? beta_k : (beta_v ? beta_v : beta_k)) + off;
    const f32x4 r0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rate));
    const f32x4 r1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rate + 4));
    const float sr[8] = {sqrtf(r0[0]), sqrtf(r0[1]), sqrtf(r0[2]), sqrtf(r0[3]),
                         sqrtf(r1[0]), sqrtf(r1[1]), sqrtf(r1[2]), sqrtf(r1[3])};
    const E* src = (isk ? k : v) + off;
    E* dst = (isk ? ks : vs) + off;
    if constexpr (sizeof(E) == 2) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(src);
        bf16x8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (__bf16)(sr[j] * (float)x[j]);
        *reinterpret_cast<bf16x8*>(dst) = y;
    } else {
        const float4 x0 = *reinterpret_cast<const float4*>(src);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
        *reinterpret_cast<float4*>(dst) = make_float4(sr[0] * x0.x, sr[1] * x0.y, sr[2] * x0.z, sr[3] * x0.w);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(sr[4] * x1.x, sr[5] * x1.y, sr[6] * x1.z, sr[7] * x1.w);
    }
}

}  // namespace

size_t fg2_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                           bool bf16, bool channel) {
    if (T == 0) return 0;
    const size_t es = bf16 ? 2 : 4;
    const size_t ntok = (size_t)(B * T * H);
    return align_up(chunk_workspace_bytes(B, T, H, dk, chunk, bf16, channel)) +
           align_up(ntok * dk * es) + align_up(ntok * dv * es) + align_up(ntok * 4);
}

hipError_t fg2_chunk_fwd_launch(const ChunkArgs& a, const float* beta_k, const float* beta_v) {
    if (a.T == 0) return chunk_fwd_launch(a);   // copies S0 to S_T
    const size_t es = a.bf16 ? 2 : 4;
    const int64_t ntok = a.B * a.T * a.H;
    char* ws = static_cast<char*>(a.ws);
    const size_t inner = align_up(chunk_workspace_bytes(a.B, a.T, a.H, a.dk, a.chunk, a.bf16, a.channel));
    char* ks = ws + inner;
    char* vs = ks + align_up((size_t)ntok * a.dk * es);
    float* ones = reinterpret_cast<float*>(vs + align_up((size_t)ntok * a.dv * es));
    const int64_t work = ntok * ((a.dk + a.dv) / 8);
    const int64_t blocks = (work + 255) / 256;
    if (a.bf16)
        hipLaunchKernelGGL((fg2_scale<__bf16>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           (const __bf16*)a.k, (const __bf16*)a.v, beta_k, beta_v, (__bf16*)ks,
                           (__bf16*)vs, ones, ntok, (int)a.dk, (int)a.dv);
    else
        hipLaunchKernelGGL((fg2_scale<float>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           (const float*)a.k, (const float*)a.v, beta_k, beta_v, (float*)ks,
                           (float*)vs, ones, ntok, (int)a.dk, (int)a.dv);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ChunkArgs b = a;
    b.k = ks;
    b.v = vs;
    b.beta = ones;
    b.ws = inner > 0 ? a.ws : nullptr;
    return chunk_fwd_launch(b);
}

}  // namespace gdr
