// gdr_tree.hip -- draft trees in speculative decoding: every node of a tree of
// draft tokens verified in one pass over the committed state, and the state of
// the accepted node rebuilt afterwards (the TreeWY note on the mindpattern
// "Gated DeltaNet-2" page: a tree-structured WY transform gives every node's
// output from one triangular solve, and only the accepted state is rebuilt,
// from a small matrix of pseudo-values instead of per-node state snapshots).
//
// Per (b, h), with nodes i = 0..Td-1 in topological order (parent p(i) < i, or
// -1 for a child of the committed state S) and anc(i) the strict ancestors of
// i, the chunkwise WY form of the "FG2-GDN" page (section 3.6) holds with the
// causal mask replaced by the ancestor relation:
//   g_i   = sum of log alpha over the root path of i (per key channel for KDA)
//   A[i][j] = beta_i sum_c k_ic k_jc e^{g_ic - g_jc}      (j in anc(i), else 0)
//   T     = (I + A)^-1 Diag(beta)            (same sparsity: anc(i) plus i)
//   R     = V - Kg S^T,   Kg[i] = k_i * e^{g_i}
//   D     = T R                              (the written value of every node)
//   P[i][j] = sum_c q_ic k_jc e^{g_ic - g_jc}                (j in anc(i) or i)
//   O     = Qg S^T + P D = Qg S^T + (P T) R, Qg[i] = q_i * e^{g_i}
// and the state after node a is
//   S_a = S Diag(e^{g_a}) + sum_{j on the path of a} D_j (k_j * e^{g_a - g_j})^T.
// Every exponent is <= 0 (decays are at most 1), so nothing overflows.
//
// gdr_decode_tree: one workgroup per (b, h).  The workgroup builds the path
// decays, A, T and M = P T of its tree in LDS (fp32), then each
// group of LPR = DK/16 lanes takes a state row (16 channels per lane, as in the
// multi-token decode), reduces R_i and (Qg S^T)_i for every node with DPP row
// sums, and the row's lanes split the nodes for D_i = T R and o_i = O0_i + M R.
// gdr_decode_tree_commit: one workgroup per (b, h, 64 rows); the path of the
// accepted node and its key weights in LDS, then S_a row by row.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

constexpr int kTreeMax = 64;      // nodes per tree
constexpr int kTreeRows = 64;     // state rows per workgroup

// Sum over the LPR (4 or 8) consecutive lanes of a state row, left in each.
template <int LPR>
__device__ __forceinline__ float tree_row_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
    if constexpr (LPR == 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
    return x;
}

// Parent of node i as the kernels read it: anything but -1 or an earlier node
// is read as -1 (keeps every index in range; the header documents it).
__device__ __forceinline__ int tree_parent(const int32_t* parent, int i) {
    const int p = parent[i];
    return (p >= 0 && p < i) ? p : -1;
}

// LDS carve-up of the verify kernel for Td nodes (in floats): the nodes' raw
// keys and queries (fp32), their path log-decays (then the decays e^g), A
// (then M = P T), T and P, the per-wave staging of R and Qg S^T (in P's place
// once P is spent, when it fits), beta and the ancestor masks.
struct TreeLds {
    int td, dk;
    __host__ __device__ size_t rpp() const { return 1024 / dk; }                 // rows per wave pass
    __host__ __device__ size_t stg_n() const { return 4 * rpp() * td * 2; }
    __host__ __device__ bool stg_in_p() const { return stg_n() <= (size_t)td * td; }
    __host__ __device__ size_t kr() const { return 0; }                          // [Td][dk]
    __host__ __device__ size_t qr() const { return kr() + (size_t)td * dk; }    // [Td][dk]
    __host__ __device__ size_t ge() const { return qr() + (size_t)td * dk; }    // [Td][dk] g, then e^g
    __host__ __device__ size_t am() const { return ge() + (size_t)td * dk; }    // [Td][Td] A, then M = P T
    __host__ __device__ size_t tm() const { return am() + (size_t)td * td; }    // [Td][Td] T
    __host__ __device__ size_t pm() const { return tm() + (size_t)td * td; }    // [Td][Td] P
    __host__ __device__ size_t stg() const { return stg_in_p() ? pm() : pm() + (size_t)td * td; }
    __host__ __device__ size_t bet() const { return pm() + (size_t)td * td + (stg_in_p() ? 0 : stg_n()); }
    __host__ __device__ size_t anc() const { return (bet() + td + 1) / 2 * 2; }  // [Td] uint64
    __host__ __device__ size_t off() const { return anc() + 2 * (size_t)td; }   // [Td + 1] int: pair offsets
    __host__ __device__ size_t floats() const { return off() + td + 1; }
};

// One workgroup per (b, h): the whole head's rows, in passes of 4 * RPP.
template <typename E, bool CHANNEL, int DK>
__global__ __launch_bounds__(256) void tree_verify_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* __restrict__ S_in,
    const int32_t* __restrict__ parent, E* __restrict__ o, float* __restrict__ D, int H, int Td, int DV) {
    constexpr int LPR = DK / 16;         // lanes per state row
    constexpr int RPP = kWave / LPR;     // rows per wave pass
    constexpr int CPL = DK / kWave;      // channels per lane in the pair sums
    extern __shared__ __attribute__((aligned(16))) float tl[];
    const TreeLds L{Td, DK};
    float* kr = tl + L.kr();
    float* qr = tl + L.qr();
    float* ge = tl + L.ge();
    float* am = tl + L.am();
    float* tm = tl + L.tm();
    float* pm = tl + L.pm();
    float* bet = tl + L.bet();
    uint64_t* anc = reinterpret_cast<uint64_t*>(tl + L.anc());
    int* off = reinterpret_cast<int*>(tl + L.off());

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H, h = bh % H;
    const int32_t* par = parent + b * Td;
    auto node_row = [&](int i) { return (b * Td + i) * H + h; };   // row of [B, Td, H, *]

    // ---- inputs of every node into LDS; ancestor masks, and the offsets of
    //      each node's (ancestor-or-self) pairs in one list ----
    if (tid == 0) {
        int n = 0;
        for (int i = 0; i < Td; ++i) {
            const int p = tree_parent(par, i);
            const uint64_t a = p < 0 ? 0ull : (anc[p] | (1ull << p));
            anc[i] = a;
            off[i] = n;
            n += __builtin_popcountll(a) + 1;
        }
        off[Td] = n;
    }
    if (tid < Td) bet[tid] = beta[node_row(tid)];
    for (int e = tid; e < Td * DK; e += 256) {
        const int i = e / DK, c = e % DK;
        kr[e] = to_f32(k[node_row(i) * DK + c]);
        qr[e] = to_f32(q[node_row(i) * DK + c]);
        if (CHANNEL || c == 0) ge[e] = CHANNEL ? log_alpha[node_row(i) * DK + c] : log_alpha[node_row(i)];
    }
    __syncthreads();
    // ---- path log-decays: thread c follows channel c down the tree ----
    if (tid < (CHANNEL ? DK : 1)) {
        for (int i = 0; i < Td; ++i) {
            const int p = tree_parent(par, i);
            if (p >= 0) ge[i * DK + tid] += ge[p * DK + tid];
        }
    }
    __syncthreads();
    // ---- A and P over the (ancestor-or-self) pairs: the pairs of the list
    //      one per thread, each a sum over the channels from LDS ----
    for (int e = tid; e < Td * Td; e += 256) {
        am[e] = 0.f;
        pm[e] = 0.f;
    }
    __syncthreads();
    const int npairs = off[Td];
    for (int t = tid; t < npairs; t += 256) {
        int lo = 0, hi = Td - 1;   // the node i with off[i] <= t < off[i + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int i = lo;
        uint64_t m = anc[i] | (1ull << i);
        for (int r = t - off[i]; r > 0; --r) m &= m - 1ull;
        const int j = __builtin_ctzll(m);
        const float* ki = kr + i * DK;
        const float* kj = kr + j * DK;
        const float* qi = qr + i * DK;
        float a = 0.f, pp = 0.f;
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
            const float4 x = *reinterpret_cast<const float4*>(ki + c);
            float4 y = *reinterpret_cast<const float4*>(kj + c);
            const float4 z = *reinterpret_cast<const float4*>(qi + c);
            if constexpr (CHANNEL) {
                const float4 gi = *reinterpret_cast<const float4*>(ge + i * DK + c);
                const float4 gj = *reinterpret_cast<const float4*>(ge + j * DK + c);
                y = make_float4(y.x * __expf(gi.x - gj.x), y.y * __expf(gi.y - gj.y), y.z * __expf(gi.z - gj.z),
                                y.w * __expf(gi.w - gj.w));
            }
            a += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            pp += z.x * y.x + z.y * y.y + z.z * y.z + z.w * y.w;
        }
        if constexpr (!CHANNEL) {
            const float w = __expf(ge[i * DK] - ge[j * DK]);
            a *= w;
            pp *= w;
        }
        if (j != i) am[i * Td + j] = a * bet[i];
        pm[i * Td + j] = pp;
    }
    __syncthreads();
    // ---- decays e^g (g is spent); T = (I + A)^-1 Diag(beta): thread j builds
    //      column j by forward substitution (only ancestors contribute) ----
    for (int e = tid; e < Td * (CHANNEL ? DK : 1); e += 256) {
        const int i = CHANNEL ? e / DK : e, c = CHANNEL ? e % DK : 0;
        ge[i * DK + c] = __expf(ge[i * DK + c]);
    }
    if (tid < Td) {
        const int j = tid;
        for (int i = 0; i < Td; ++i) {
            float x = 0.f;
            if (i == j) {
                x = 1.f;
            } else if (i > j && ((anc[i] >> j) & 1ull)) {
                uint64_t m = anc[i] & ~((1ull << j) - 1ull);   // ancestors m >= j
                while (m) {
                    const int mi = __builtin_ctzll(m);
                    m &= m - 1ull;
                    x -= am[i * Td + mi] * tm[mi * Td + j];
                }
            }
            tm[i * Td + j] = x;
        }
    }
    __syncthreads();
    if (tid < Td) {
        const float bj = bet[tid];
        for (int i = 0; i < Td; ++i) tm[i * Td + tid] *= bj;
    }
    __syncthreads();
    // ---- M = P T (in A's place) ----
    for (int e = tid; e < Td * Td; e += 256) {
        const int i = e / Td, j = e % Td;
        float x = 0.f;
        uint64_t m = (anc[i] | (1ull << i)) & ~((1ull << j) - 1ull);
        while (m) {
            const int mi = __builtin_ctzll(m);
            m &= m - 1ull;
            x += pm[i * Td + mi] * tm[mi * Td + j];
        }
        am[e] = x;   // A is no longer read
    }
    __syncthreads();   // P is spent: the staging may take its place

    // ---- the state rows ----
    const int cl = lane % LPR, rw = lane / LPR;
    float* stg = tl + L.stg() + (size_t)wave * RPP * Td * 2;
    for (int p0 = 0; p0 < DV; p0 += 4 * RPP) {
        const int row = p0 + wave * RPP + rw;
        const int64_t sbase = (bh * DV + row) * (int64_t)DK;
        f32x4 s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S_in + sbase + 4 * (cl + LPR * j)));
        // v of every node for this row, loaded together (the R slots take it)
        for (int i = cl; i < Td; i += LPR) stg[(rw * Td + i) * 2] = to_f32(v[node_row(i) * DV + row]);
        __syncthreads();
#pragma unroll 2
        for (int i = 0; i < Td; ++i) {
            float pd = 0.f, od = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 4 * (cl + LPR * j);
                float4 kv = *reinterpret_cast<const float4*>(kr + i * DK + c);
                float4 qv = *reinterpret_cast<const float4*>(qr + i * DK + c);
                if constexpr (CHANNEL) {
                    const float4 ev = *reinterpret_cast<const float4*>(ge + i * DK + c);
                    kv = make_float4(kv.x * ev.x, kv.y * ev.y, kv.z * ev.z, kv.w * ev.w);
                    qv = make_float4(qv.x * ev.x, qv.y * ev.y, qv.z * ev.z, qv.w * ev.w);
                }
                pd += s[j][0] * kv.x + s[j][1] * kv.y + s[j][2] * kv.z + s[j][3] * kv.w;
                od += s[j][0] * qv.x + s[j][1] * qv.y + s[j][2] * qv.z + s[j][3] * qv.w;
            }
            pd = tree_row_sum<LPR>(pd);
            od = tree_row_sum<LPR>(od);
            if constexpr (!CHANNEL) {
                const float ei = ge[i * DK];
                pd *= ei;
                od *= ei;
            }
            if (cl == 0) {
                stg[(rw * Td + i) * 2] -= pd;         // R_i = v_i - (Kg S^T)_i
                stg[(rw * Td + i) * 2 + 1] = od;      // (Qg S^T)_i
            }
        }
        __syncthreads();
        // the row's lanes split the nodes: D_i = T R, o_i = O0_i + M R
        for (int i = cl; i < Td; i += LPR) {
            float d = 0.f, y = stg[(rw * Td + i) * 2 + 1];
            uint64_t m = anc[i] | (1ull << i);
            while (m) {
                const int j = __builtin_ctzll(m);
                m &= m - 1ull;
                const float r = stg[(rw * Td + j) * 2];
                d += tm[i * Td + j] * r;
                y += am[i * Td + j] * r;
            }
            if (D) D[node_row(i) * DV + row] = d;
            if (o) o[node_row(i) * DV + row] = from_f32<E>(y);
        }
        __syncthreads();
    }
}

template <typename E, bool CHANNEL, int DK>
__global__ __launch_bounds__(256) void tree_commit_kernel(
    const E* __restrict__ k, const float* __restrict__ log_alpha, const int32_t* __restrict__ parent,
    const float* __restrict__ D, const int32_t* __restrict__ accepted, const float* S_in, float* S_out,
    int H, int Td, int DV) {
    constexpr int LPR = DK / 16;
    constexpr int RPP = kWave / LPR;
    __shared__ __attribute__((aligned(16))) float w[kTreeMax * DK];   // k_j * e^{g_a - g_j}, path order
    __shared__ __attribute__((aligned(16))) float ga[DK];             // e^{g_a}
    __shared__ int path[kTreeMax];
    __shared__ int npath;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nrb = DV / kTreeRows;
    const int64_t bh = blockIdx.x / nrb;
    const int rb = (int)(blockIdx.x % nrb);
    const int64_t b = bh / H, h = bh % H;
    const int32_t* par = parent + b * Td;
    auto node_row = [&](int i) { return (b * Td + i) * H + h; };
    int a = accepted[b];
    a = (a >= 0 && a < Td) ? a : -1;

    if (tid == 0) {
        int n = 0;
        for (int i = a; i >= 0; i = tree_parent(par, i)) path[n++] = i;   // leaf first
        npath = n;
    }
    __syncthreads();
    const int np = npath;
    // path log-decay from the root: thread c walks channel c (leaf-first list)
    if (tid < DK) {
        const int c = tid;
        float gc = 0.f;
        for (int n = np - 1; n >= 0; --n) {
            const int j = path[n];
            gc += CHANNEL ? log_alpha[node_row(j) * DK + c] : log_alpha[node_row(j)];
            w[n * DK + c] = gc;   // g_j for now
        }
        for (int n = 0; n < np; ++n)
            w[n * DK + c] = to_f32(k[node_row(path[n]) * DK + c]) * __expf(gc - w[n * DK + c]);
        ga[c] = __expf(gc);
    }
    __syncthreads();
    const int cl = lane % LPR;
    for (int p0 = 0; p0 < kTreeRows; p0 += 4 * RPP) {
        const int row = rb * kTreeRows + p0 + wave * RPP + lane / LPR;
        const int64_t sbase = (bh * DV + row) * (int64_t)DK;
        f32x4 s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * (cl + LPR * j);
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S_in + sbase + c));
            const float4 gv = *reinterpret_cast<const float4*>(ga + c);
            s[j][0] *= gv.x; s[j][1] *= gv.y; s[j][2] *= gv.z; s[j][3] *= gv.w;
        }
        for (int n = 0; n < np; ++n) {
            const float dj = D[node_row(path[n]) * DV + row];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 wv = *reinterpret_cast<const float4*>(w + n * DK + 4 * (cl + LPR * j));
                s[j][0] += dj * wv.x; s[j][1] += dj * wv.y; s[j][2] += dj * wv.z; s[j][3] += dj * wv.w;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f32x4*>(S_out + sbase + 4 * (cl + LPR * j)));
    }
}

template <typename E, bool CHANNEL, int DK>
hipError_t launch_tree(const TreeArgs& a) {
    const int64_t grid = a.B * a.H;
    if (a.o || a.D) {
        const size_t lds = TreeLds{(int)a.Td, DK}.floats() * sizeof(float);
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tree_verify_kernel<E, CHANNEL, DK>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((tree_verify_kernel<E, CHANNEL, DK>), dim3((unsigned)grid), dim3(256), lds, a.stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_alpha, a.beta, a.S_in, a.parent,
                           (E*)a.o, a.D, (int)a.H, (int)a.Td, (int)a.dv);
    }
    return hipGetLastError();
}

template <typename E, bool CHANNEL, int DK>
hipError_t launch_tree_commit(const TreeArgs& a) {
    const int64_t grid = a.B * a.H * (a.dv / kTreeRows);
    hipLaunchKernelGGL((tree_commit_kernel<E, CHANNEL, DK>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                       (const E*)a.k, a.log_alpha, a.parent, a.D, a.accepted, a.S_in, a.S_out, (int)a.H,
                       (int)a.Td, (int)a.dv);
    return hipGetLastError();
}

template <bool COMMIT, typename E, bool CHANNEL>
hipError_t tree_dk(const TreeArgs& a) {
    if (a.dk == 64) return COMMIT ? launch_tree_commit<E, CHANNEL, 64>(a) : launch_tree<E, CHANNEL, 64>(a);
    return COMMIT ? launch_tree_commit<E, CHANNEL, 128>(a) : launch_tree<E, CHANNEL, 128>(a);
}

template <bool COMMIT>
hipError_t tree_dispatch(const TreeArgs& a) {
    if (a.bf16) return a.channel ? tree_dk<COMMIT, __bf16, true>(a) : tree_dk<COMMIT, __bf16, false>(a);
    return a.channel ? tree_dk<COMMIT, float, true>(a) : tree_dk<COMMIT, float, false>(a);
}

}  // namespace

size_t tree_verify_lds_bytes(int64_t Td, int64_t dk) { return TreeLds{(int)Td, (int)dk}.floats() * sizeof(float); }

hipError_t decode_tree_launch(const TreeArgs& a) { return tree_dispatch<false>(a); }
hipError_t decode_tree_commit_launch(const TreeArgs& a) { return tree_dispatch<true>(a); }

}  // namespace gdr
