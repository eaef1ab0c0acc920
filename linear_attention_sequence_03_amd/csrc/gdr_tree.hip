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
// decays, A and P of its tree in LDS (fp32) and T as a blocked dense inverse
// (forward substitution on the 16 x 16 diagonal blocks, then the blocks below
// on fp32 MFMA; T keeps A's zeros exactly), scales the keys and queries by
// their path decays, then each wave takes 16-column tiles of the values and
// forms R, Qg S^T, D = T R and o = Qg S^T + P D with fp32 MFMA (every product
// is a small dense contraction; node slots past Td are zeros).
// gdr_decode_tree_commit: one workgroup per (b, h, 64 rows); the path of the
// accepted node and its key weights in LDS, then S_a row by row.
#include <type_traits>

#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

constexpr int kTreeMax = 64;      // nodes per tree
constexpr int kTreeRows = 64;     // state rows per workgroup

// Sum over the four lanes of a quad, left in each (DPP quad permutations).
__device__ __forceinline__ float quad_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
    return x;
}

// Parent of node i as the kernels read it: anything but -1 or an earlier node
// is read as -1 (keeps every index in range; the header documents it).
__device__ __forceinline__ int tree_parent(const int32_t* parent, int i) {
    const int p = parent[i];
    return (p >= 0 && p < i) ? p : -1;
}

// LDS carve-up of the verify kernel for Td nodes in NP = 16 ceil(Td / 16) node
// slots (in floats): the nodes' keys and queries (fp32; raw for A and P, then
// scaled by their path decays) and their path log-decays, rows padded to
// DK + 4 floats so that the pair sums (one node pair per thread, every thread
// at the same channel) spread over the banks; A, T and P as NP x NP tiles (rows
// of NP + 4 floats, zero outside the nodes), the inverted diagonal blocks of
// I + A, beta (zero past Td), the root paths (ancestor-or-self masks), the
// offsets of each node's pairs in the pair list and the parents as the kernel
// reads them (then the pointer-jumping targets).
struct TreeLds {
    int td, dk, np;
    __host__ __device__ int ks() const { return dk + 4; }                       // key row stride
    __host__ __device__ int ns() const { return np + 4; }                       // A / T / P row stride
    __host__ __device__ size_t kr() const { return 0; }                          // [Td][ks]
    __host__ __device__ size_t qr() const { return kr() + (size_t)td * ks(); }  // [Td][ks]
    __host__ __device__ size_t ge() const { return qr() + (size_t)td * ks(); }  // [Td][ks] path log-decay
    __host__ __device__ size_t am() const { return ge() + (size_t)td * ks(); }  // [NP][ns] A
    __host__ __device__ size_t tm() const { return am() + (size_t)np * ns(); }  // [NP][ns] T
    __host__ __device__ size_t pm() const { return tm() + (size_t)np * ns(); }  // [NP][ns] P
    __host__ __device__ size_t xd() const { return pm() + (size_t)np * ns(); }  // [NP/16][16][16] (I + A_bb)^-1
    __host__ __device__ size_t bet() const { return xd() + (size_t)np * 16; }   // [NP]
    __host__ __device__ size_t anc() const { return (bet() + np + 1) / 2 * 2; }  // [Td] uint64
    __host__ __device__ size_t off() const { return anc() + 2 * (size_t)td; }   // [Td + 1] int
    __host__ __device__ size_t pa() const { return off() + td + 1; }            // [Td] int parents
    __host__ __device__ size_t floats() const { return pa() + td; }
};

template <typename E>
using Raw4 = typename std::conditional<sizeof(E) == 4, float4, bf16x4>::type;

template <typename E>
__device__ __forceinline__ float4 widen4(const Raw4<E>& x) {
    if constexpr (sizeof(E) == 4) return x;
    else return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

// One workgroup per (b, h); NT = ceil(Td / 16) node tiles.  Wave w owns the
// value columns of tiles w, w + 4, ... (DK / 64 tiles of 16 columns); its
// slice of the state and of the values, and the nodes' inputs, are loaded
// first, so that the loads are in flight together.
template <typename E, bool CHANNEL, int DK, int NT>
__global__ __launch_bounds__(256) void tree_verify_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* __restrict__ S_in,
    const int32_t* __restrict__ parent, E* __restrict__ o, float* __restrict__ D, int H, int Td, int DV) {
    using MF = Mma<float>;
    constexpr int TPW = DK / 64;          // value tiles per wave
    constexpr int KT = DK / 16;           // channel groups of the contraction
    constexpr int NP = 16 * NT;           // node slots
    constexpr int NS = NP + 4;            // A / T / P row stride
    constexpr int V4 = DK / 4;            // 16-byte units of a key row
    constexpr int NU = (NP * V4 + 255) / 256;   // node-input units per thread
    extern __shared__ __attribute__((aligned(16))) float tl[];
    const TreeLds L{Td, DK, NP};
    const int KS = L.ks();
    float* kr = tl + L.kr();
    float* qr = tl + L.qr();
    float* ge = tl + L.ge();
    float* am = tl + L.am();
    float* tm = tl + L.tm();
    float* pm = tl + L.pm();
    float* xd = tl + L.xd();
    float* bet = tl + L.bet();
    uint64_t* anc = reinterpret_cast<uint64_t*>(tl + L.anc());
    int* off = reinterpret_cast<int*>(tl + L.off());
    int* pa = reinterpret_cast<int*>(tl + L.pa());

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g4 = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H, h = bh % H;
    const int32_t* par = parent + b * Td;
    auto node_row = [&](int i) { return (b * Td + i) * H + h; };   // row of [B, Td, H, *]

    // ---- this wave's state columns and values (lane (col, g4) holds value
    //      column 16 nt + col: the state row's channels 16 t + 4 g4 .. + 3 and
    //      the values of nodes 16 mt + 4 g4 + e), and the nodes' keys, queries
    //      and decays, all loads issued before any is used ----
    f32x4 sb[TPW][KT];
    float vv[TPW][NT][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int vcol = 16 * (wave + 4 * u) + col;
#pragma unroll
        for (int t = 0; t < KT; ++t)
            sb[u][t] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S_in + (bh * DV + vcol) * (int64_t)DK + 16 * t + 4 * g4));
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int nd = 16 * mt + 4 * g4 + e;
                vv[u][mt][e] = nd < Td ? to_f32(v[node_row(nd) * DV + vcol]) : 0.f;
            }
    }
    Raw4<E> kb[NU], qb[NU];
    float4 lb[CHANNEL ? NU : 1];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int e = tid + 256 * u;
        if (e < Td * V4) {
            const int64_t src = node_row(e / V4) * DK + 4 * (e % V4);
            kb[u] = *reinterpret_cast<const Raw4<E>*>(k + src);
            qb[u] = *reinterpret_cast<const Raw4<E>*>(q + src);
            if constexpr (CHANNEL) lb[u] = *reinterpret_cast<const float4*>(log_alpha + src);
        }
    }

    // ---- A, T and P start at zero; beta (zero past Td), parents, and the
    //      node inputs into LDS ----
    for (int e = tid; e < 3 * NP * NS; e += 256) am[e] = 0.f;   // am, tm, pm are contiguous
    if (tid < NP) bet[tid] = tid < Td ? beta[node_row(tid)] : 0.f;
    if (tid < Td) {
        pa[tid] = tree_parent(par, tid);
        anc[tid] = 1ull << tid;
        if constexpr (!CHANNEL) ge[tid * KS] = log_alpha[node_row(tid)];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int e = tid + 256 * u;
        if (e < Td * V4) {
            const int i = e / V4, c = 4 * (e % V4);
            *reinterpret_cast<float4*>(kr + i * KS + c) = widen4<E>(kb[u]);
            *reinterpret_cast<float4*>(qr + i * KS + c) = widen4<E>(qb[u]);
            if constexpr (CHANNEL) *reinterpret_cast<float4*>(ge + i * KS + c) = lb[u];
        }
    }
    __syncthreads();
    // ---- root paths by pointer jumping: anc[i] holds the nodes from i up to,
    //      not including, pa[i]; each round joins the segment of pa[i] and
    //      jumps twice as far, so ceil(log2 Td) rounds reach the root ----
    for (int r = Td > 1 ? 32 - __builtin_clz(Td - 1) : 0; r > 0; --r) {
        uint64_t nm = 0;
        int nj = -1;
        if (tid < Td) {
            const int j = pa[tid];
            nm = anc[tid] | (j >= 0 ? anc[j] : 0ull);
            nj = j >= 0 ? pa[j] : -1;
        }
        __syncthreads();
        if (tid < Td) {
            anc[tid] = nm;
            pa[tid] = nj;
        }
        __syncthreads();
    }
    // ---- path log-decays g_i = sum of log alpha over the root path of i,
    //      summed root first (per key channel for KDA); on the last wave, the
    //      offsets of each node's (ancestor-or-self) pairs in one list ----
    constexpr int GN = (NP * (CHANNEL ? DK : 1) + 255) / 256;
    float gsum[GN];
#pragma unroll
    for (int u = 0; u < GN; ++u) {
        const int e = tid + 256 * u;
        gsum[u] = 0.f;
        if (e < Td * (CHANNEL ? DK : 1)) {
            const int i = CHANNEL ? e / DK : e, c = CHANNEL ? e % DK : 0;
            for (uint64_t m = anc[i]; m; m &= m - 1ull) gsum[u] += ge[__builtin_ctzll(m) * KS + c];
        }
    }
    if (tid == 192) {
        int n = 0;
        for (int i = 0; i < Td; ++i) {
            off[i] = n;
            n += __builtin_popcountll(anc[i]);
        }
        off[Td] = n;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < GN; ++u) {
        const int e = tid + 256 * u;
        if (e < Td * (CHANNEL ? DK : 1)) {
            const int i = CHANNEL ? e / DK : e, c = CHANNEL ? e % DK : 0;
            ge[i * KS + c] = gsum[u];
        }
    }
    __syncthreads();
    // ---- A and P over the (ancestor-or-self) pairs: the pairs of the list
    //      four lanes each (a quad; lane s of it sums channels 16 cc + 4 s ..
    //      + 3), the partial sums joined by two DPP steps ----
    const int npairs = off[Td];
    const int sub = tid & 3;
    for (int t = tid >> 2; t < (npairs + 63) / 64 * 64; t += 64) {   // quad-uniform trip count
        float a = 0.f, pp = 0.f;
        int i = 0, j = 0;
        if (t < npairs) {
            int lo = 0, hi = Td - 1;   // the node i with off[i] <= t < off[i + 1]
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= t) lo = mid;
                else hi = mid - 1;
            }
            i = lo;
            uint64_t m = anc[i];   // ancestors and i itself
            for (int r = t - off[i]; r > 0; --r) m &= m - 1ull;
            j = __builtin_ctzll(m);
            const float* ki = kr + i * KS;
            const float* kj = kr + j * KS;
            const float* qi = qr + i * KS;
#pragma unroll 4
            for (int c = 4 * sub; c < DK; c += 16) {
                const float4 x = *reinterpret_cast<const float4*>(ki + c);
                float4 y = *reinterpret_cast<const float4*>(kj + c);
                const float4 z = *reinterpret_cast<const float4*>(qi + c);
                if constexpr (CHANNEL) {
                    const float4 gi = *reinterpret_cast<const float4*>(ge + i * KS + c);
                    const float4 gj = *reinterpret_cast<const float4*>(ge + j * KS + c);
                    y = make_float4(y.x * __expf(gi.x - gj.x), y.y * __expf(gi.y - gj.y),
                                    y.z * __expf(gi.z - gj.z), y.w * __expf(gi.w - gj.w));
                }
                a += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
                pp += z.x * y.x + z.y * y.y + z.z * y.z + z.w * y.w;
            }
        }
        a = quad_sum(a);
        pp = quad_sum(pp);
        if (t < npairs && sub == 0) {
            if constexpr (!CHANNEL) {
                const float w = __expf(ge[i * KS] - ge[j * KS]);
                a *= w;
                pp *= w;
            }
            if (j != i) am[i * NS + j] = a * bet[i];
            pm[i * NS + j] = pp;
        }
    }
    __syncthreads();
    // ---- keys and queries scaled by their path decays, Kg = k e^g and
    //      Qg = q e^g (the raw ones are spent); the diagonal blocks of
    //      T = (I + A)^-1 Diag(beta) on wave 0: lane (bb, jc) builds column jc
    //      of X_bb = (I + A_bb)^-1 by forward substitution in registers (dense:
    //      the tree's zeros of A stay exact zeros of T), keeps X_bb and writes
    //      T_bb = X_bb Diag(beta_bb) ----
    for (int e = tid; e < Td * DK; e += 256) {
        const int i = e / DK, c = e % DK;
        const float w = __expf(ge[i * KS + (CHANNEL ? c : 0)]);
        kr[i * KS + c] *= w;
        qr[i * KS + c] *= w;
    }
    if (wave == 0 && g4 < NT) {
        const int bb = g4, jc = col;
        const float* Ab = am + 16 * bb * NS + 16 * bb;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float arow[16];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
                if (4 * qd < i) {
                    const float4 t = *reinterpret_cast<const float4*>(Ab + i * NS + 4 * qd);
                    arow[4 * qd] = t.x; arow[4 * qd + 1] = t.y; arow[4 * qd + 2] = t.z; arow[4 * qd + 3] = t.w;
                }
            float acc = i == jc ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc -= arow[m] * x[m];
            x[i] = acc;
        }
        const float bj = bet[16 * bb + jc];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            xd[bb * 256 + i * 16 + jc] = x[i];
            tm[(16 * bb + i) * NS + 16 * bb + jc] = x[i] * bj;
        }
    }
    // ---- the tiles below the diagonal, one block row at a time (wave jt
    //      builds T_{it, jt}): T_ij = -X_ii sum_{m = j}^{i - 1} A_im T_mj ----
#pragma unroll
    for (int it = 1; it < NT; ++it) {
        __syncthreads();
        if (wave < it) {
            const int jt = wave;
            f32x4 y = zero4();
#pragma unroll
            for (int mt = 0; mt < it; ++mt) {
                if (mt < jt) continue;
                const float4 a = *reinterpret_cast<const float4*>(am + (16 * it + col) * NS + 16 * mt + 4 * g4);
                const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    y = MF::mma(av[s2], tm[(16 * mt + 4 * g4 + s2) * NS + 16 * jt + col], y);
            }
            const float4 xa = *reinterpret_cast<const float4*>(xd + it * 256 + col * 16 + 4 * g4);
            f32x4 z = zero4();
            z = MF::mma(xa.x, y[0], z);
            z = MF::mma(xa.y, y[1], z);
            z = MF::mma(xa.z, y[2], z);
            z = MF::mma(xa.w, y[3], z);
#pragma unroll
            for (int e = 0; e < 4; ++e) tm[(16 * it + 4 * g4 + e) * NS + 16 * jt + col] = -z[e];
        }
    }
    __syncthreads();

    // ---- the outputs on the matrix cores (fp32 16x16x4), per value tile:
    //      R = V - Kg S^T and Qg S^T for every node tile, D = T R, then
    //      o = Qg S^T + P D.  The contractions over channels and over nodes
    //      use the permuted k-map: k-step s of lane group g is channel (or
    //      node) 16(s/4) + 4g + s%4, so an accumulator tile is directly the B
    //      operand of the next product and each lane's state slice is one
    //      16-byte load per four steps. ----
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int vcol = 16 * (wave + 4 * u) + col;
        f32x4 R[NT], O[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            R[mt] = zero4();
            O[mt] = zero4();
            const int node = 16 * mt + col;
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                float4 ka = make_float4(0.f, 0.f, 0.f, 0.f), qa = ka;
                if (node < Td) {
                    ka = *reinterpret_cast<const float4*>(kr + node * KS + 16 * t + 4 * g4);
                    qa = *reinterpret_cast<const float4*>(qr + node * KS + 16 * t + 4 * g4);
                }
                R[mt] = MF::mma(ka.x, sb[u][t][0], R[mt]);
                O[mt] = MF::mma(qa.x, sb[u][t][0], O[mt]);
                R[mt] = MF::mma(ka.y, sb[u][t][1], R[mt]);
                O[mt] = MF::mma(qa.y, sb[u][t][1], O[mt]);
                R[mt] = MF::mma(ka.z, sb[u][t][2], R[mt]);
                O[mt] = MF::mma(qa.z, sb[u][t][2], O[mt]);
                R[mt] = MF::mma(ka.w, sb[u][t][3], R[mt]);
                O[mt] = MF::mma(qa.w, sb[u][t][3], O[mt]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) R[mt][e] = vv[u][mt][e] - R[mt][e];
        }
        // D = T R, then o = O + P D (T and P are lower triangular in node order)
        f32x4 Dt[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            Dt[mt] = zero4();
#pragma unroll
            for (int jt = 0; jt <= mt; ++jt) {
                const float4 ta = *reinterpret_cast<const float4*>(tm + (16 * mt + col) * NS + 16 * jt + 4 * g4);
                Dt[mt] = MF::mma(ta.x, R[jt][0], Dt[mt]);
                Dt[mt] = MF::mma(ta.y, R[jt][1], Dt[mt]);
                Dt[mt] = MF::mma(ta.z, R[jt][2], Dt[mt]);
                Dt[mt] = MF::mma(ta.w, R[jt][3], Dt[mt]);
            }
        }
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            f32x4 Ot = O[mt];
#pragma unroll
            for (int jt = 0; jt <= mt; ++jt) {
                const float4 pa4 = *reinterpret_cast<const float4*>(pm + (16 * mt + col) * NS + 16 * jt + 4 * g4);
                Ot = MF::mma(pa4.x, Dt[jt][0], Ot);
                Ot = MF::mma(pa4.y, Dt[jt][1], Ot);
                Ot = MF::mma(pa4.z, Dt[jt][2], Ot);
                Ot = MF::mma(pa4.w, Dt[jt][3], Ot);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int nd = 16 * mt + 4 * g4 + e;
                if (nd < Td) {
                    if (D) D[node_row(nd) * DV + vcol] = Dt[mt][e];
                    if (o) o[node_row(nd) * DV + vcol] = from_f32<E>(Ot[e]);
                }
            }
        }
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

template <typename E, bool CHANNEL, int DK, int NT>
hipError_t launch_tree_nt(const TreeArgs& a) {
    const int64_t grid = a.B * a.H;
    const size_t lds = tree_verify_lds_bytes(a.Td, DK);   // NT = ceil(Td / 16) node tiles
    const auto fn = &tree_verify_kernel<E, CHANNEL, DK, NT>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), lds, a.stream, (const E*)a.q, (const E*)a.k,
                       (const E*)a.v, a.log_alpha, a.beta, a.S_in, a.parent, (E*)a.o, a.D, (int)a.H, (int)a.Td,
                       (int)a.dv);
    return hipGetLastError();
}

template <typename E, bool CHANNEL, int DK>
hipError_t launch_tree(const TreeArgs& a) {
    if (!a.o && !a.D) return hipSuccess;
    switch ((a.Td + 15) / 16) {   // node tiles; Td is in [1, 64]
        case 1: return launch_tree_nt<E, CHANNEL, DK, 1>(a);
        case 2: return launch_tree_nt<E, CHANNEL, DK, 2>(a);
        case 3: return launch_tree_nt<E, CHANNEL, DK, 3>(a);
        default: return launch_tree_nt<E, CHANNEL, DK, 4>(a);
    }
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

size_t tree_verify_lds_bytes(int64_t Td, int64_t dk) {
    return TreeLds{(int)Td, (int)dk, (int)(16 * ((Td + 15) / 16))}.floats() * sizeof(float);
}

hipError_t decode_tree_launch(const TreeArgs& a) { return tree_dispatch<false>(a); }
hipError_t decode_tree_commit_launch(const TreeArgs& a) { return tree_dispatch<true>(a); }

}  // namespace gdr
