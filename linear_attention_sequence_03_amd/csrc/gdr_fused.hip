// gdr_fused.hip -- the chunkwise forward pass in a single kernel, for the
// scalar gate (Gated DeltaNet) with bf16 q/k/v and 64-token chunks.
//
// Same algebra as gdr_chunk.hip (the WY / UT form of the "FG2-GDN" page,
// section 3.6), per chunk with g_r the in-chunk cumulative log decay and
// gamma_r = e^{g_r}:
//   A[r][i] = beta_r (k_r . k_i) e^{g_r - g_i}  (i < r),   T = (I + A)^-1 Diag(beta)
//   P[r][i] = (q_r . k_i) e^{g_r - g_i}         (i <= r)
//   R = V - Diag(gamma) K S^T,   D = T R,   O = Diag(gamma) Q S^T + P D
//   S^T <- gamma_last S^T + K^T Diag(gamma_last / gamma) D
//
// One workgroup per (b, h, 16*NW value columns).  Its waves have fixed roles
// and advance together one chunk per window, with one barrier per window:
//   compute  (NW waves)  window w: chunk w    state chain and output
//   prep T   (1 wave)    window w: chunk w+1  diagonal blocks of A, the solve for T
//   prep P   (1 wave)    window w: chunk w+1  decay vectors, off-diagonal blocks
//                                             of A (handed to prep T through an
//                                             LDS flag), P
//   loaders  (2 waves)   window w: chunk w+2  global -> LDS copies; loader 0
//                                             then builds the chunk's gate table
// A chunk's inputs therefore live in a 3-deep ring of LDS stages and its T / P
// tiles in a 2-deep ring; T and P never leave the chip, and every global byte
// is read once per workgroup.
//
// Layout conventions (all LDS tiles are XOR-swizzled in 16-byte pieces so the
// row-wise and the transposing reads are both free of bank conflicts):
//  - Q, K stage tiles: [64 tokens][DK] bf16, piece p of row r at p ^ swz_qk(r).
//  - V stage tile:     [64 tokens][16*NW] bf16, piece p at p ^ swz_v(r).
//  - T tiles (and T's rounding residual where a chunk needs it) are stored
//    transposed, Tt[i][r] = T[r][i] (64 x 64 bf16), piece p of row i at
//    p ^ swz_t(i): the prep waves write accumulator tiles with one 8-byte store
//    per lane and the compute waves read operand fragments with
//    ds_read_b64_tr_b16.  P tiles are stored in the compute waves' operand
//    order, lane by lane (see frag_store).
//  - The d_k axis of the register-resident state is permuted: accumulator
//    position p = 32s + 16h + 4g + e holds channel 32s + 8g + 4h + e, so a
//    state tile pair is the B operand whose k-slots are 8 consecutive
//    channels, and every row-wise Q / K fragment is one 16-byte LDS read.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {
namespace {

constexpr int FC = 64;          // tokens per chunk
constexpr int FNB = FC / 16;    // 16-token blocks per chunk
constexpr float kFMinLogAlpha = -200.f;   // e^-200 is 0 in fp32

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x4 to_f16(f32x4 x) {
    return f16x4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}

// Swizzles (piece index XOR), functions of the row's low 4 bits only, so rows
// r and r + 16 share one.  LDS has 32 banks of 4 bytes (128 bytes per cycle);
// a 16-byte read serves 8 lanes per cycle, a 64-bit transposing read 16.
// Q / K tiles: the 8 lanes of a row-fragment read (rows r..r+7, one piece
// column) land on 8 distinct 16-byte bank groups; the K^T reads (4 rows x 4
// pieces per 16 lanes, one 8-byte half of each piece) use every group twice,
// the least possible for a fixed half.  The low three bits are r & 7 with bits
// 1 and 2 swapped, flipped in bit 0 for rows 8..15.
template <int DK>
__device__ __forceinline__ int swz_qk(int r) {
    const int lo = ((r & 1) | ((r & 2) << 1) | ((r & 4) >> 1)) ^ ((r >> 3) & 1);
    if constexpr (DK == 128) return lo | (r & 8);   // 16 pieces per row
    else return lo;                                 // 8 pieces per row
}
template <int VT>
__device__ __forceinline__ int swz_v(int r) {
    if constexpr (VT == 32) return ((r >> 2) & 1) << 1;                // 4 pieces per row
    else return 0;                                                     // 2 pieces per row
}

// The T solve's fp32 scratch (four 16x16 tiles): rows of 20 floats, tiles of
// 336, so that its float4 row accesses, its column reads and the substitution's
// stores all spread over the 32 banks.
constexpr int XROW = 20, XTILE = 16 * XROW + 16;

template <int DK, int NW>
struct FLayout {
    static constexpr int VT = 16 * NW;
    static constexpr int QB = FC * DK * 2;
    static constexpr int VB = FC * VT * 2;
    // K and V stages, a 3-deep ring (chunk n in slot n % 3).
    static constexpr int S_K = 0, S_V = QB;
    static constexpr int STAGE = S_V + VB;
    static constexpr int NSTAGE = 3;
    // Q tiles, a 2-deep ring (chunk n in slot n % 2): a chunk's Q is read in
    // the window before its state chain (prep P and the output's Q S^T part).
    static constexpr int QR0 = NSTAGE * STAGE;
    // T (with its bf16 residual T_lo where needed) and P tiles, a 2-deep ring (chunk n in slot n % 2).
    static constexpr int T_T = 0, T_L = FC * FC * 2, T_P = 2 * FC * FC * 2;
    static constexpr int T_FLAG = 3 * FC * FC * 2;   // int: this chunk applies T as a bf16 pair
    static constexpr int TPB = 3 * FC * FC * 2 + 16;
    static constexpr int TP0 = QR0 + 2 * QB;
    static constexpr int XA = TP0 + 2 * TPB;              // solve wave's scratch: diagonal blocks of A
                                                          // (transposed), then blockdiag of their 8x8
                                                          // inverses; fp32, rows of XROW, tiles of XTILE
    // Gate tables, a 3-deep ring (chunk n in slot n % 3), 64 floats per field:
    static constexpr int G_G2 = 0;        // g_r * log2(e), g the in-chunk cumulative log decay
    static constexpr int G_BE = 1;        // beta_r
    static constexpr int G_EB = 2;        // e^{g_r - g_end(blk(r) - 1)}  (decay since the previous block's end)
    static constexpr int G_FB = 3;        // e^{g_end(blk(r)) - g_r}       (decay until the own block's end)
    static constexpr int G_GM = 4;        // gamma_r = e^{g_r}
    static constexpr int G_GH = 5;        // e^{g_last - g_r}
    static constexpr int G_CX = 6;        // e^{g_end(rb-1) - g_end(cb)} for (cb, rb) = (0,2), (0,3), (1,3)
    // With the q/k normalisation of the prologue (written by the P wave for
    // the compute waves; n_k, n_q the inverse row norms):
    static constexpr int G_GMK = 7;       // gamma_r n_k(r)
    static constexpr int G_GQ = 8;        // gamma_r n_q(r)
    static constexpr int G_GHK = 9;       // e^{g_last - g_r} n_k(r)
    static constexpr int GSLOT = 10 * FC * 4;
    static constexpr int GT0 = XA + FNB * XTILE * 4;
    // The rest depends on how T is built (see the kernel):
    // - one T wave: the off-diagonal blocks of A (P wave -> T wave), fp16 per
    //   lane, and the index + 1 of the chunk whose blocks are there;
    static constexpr int AO = GT0 + 3 * GSLOT;
    static constexpr int FLAG = AO + 6 * 64 * 8;
    // - solve and recurrence waves: a 2-deep ring (chunk c in slot c % 2) of
    //   the inverted diagonal blocks X_bb (fp16, A-operand layout, 64 lanes x 4
    //   per block), the inverse key norms n_k (prologue) and the diagonal
    //   blocks' pair flag, then the solve wave's own g (log2 units) and beta rows.
    static constexpr int XH = GT0 + 3 * GSLOT;
    static constexpr int XHB = FNB * 64 * 8 + FC * 4 + 16;
    static constexpr int TG = XH + 2 * XHB;
    static constexpr int WARM = FLAG + 16;   // L2-warming target of the loaders (never read)
    template <bool SPLIT>
    static constexpr int total() { return SPLIT ? TG + 2 * FC * 4 : WARM + 256; }
    static_assert(total<true>() <= 160 * 1024 && total<false>() <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ bf16x8 lds_b128(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds_tr(const char* p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS s16x4*)(p)));
}
__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Row-wise operand fragment of a Q / K tile: rows 16*rb + lane%16, channels
// 32s + 8(lane/16) .. +7 (the k-slots of channel step s).
template <int DK>
__device__ __forceinline__ bf16x8 qk_frag(const char* tile, int rb, int s, int lane) {
    const int r = 16 * rb + (lane & 15);
    return lds_b128(tile + r * (DK * 2) + 16 * ((4 * s + (lane >> 4)) ^ swz_qk<DK>(r)));
}

// K^T operand of the state update: rows = state positions 16mc + lane%16,
// k-slots = tokens 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3).
template <int DK>
__device__ __forceinline__ bf16x8 kt_frag(const char* tile, int mc, int s, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, qd = lane & 3;
    const int r = 32 * s + 4 * g + j;
    const char* p = tile + r * (DK * 2) + 16 * ((4 * (mc >> 1) + qd) ^ swz_qk<DK>(r)) + 8 * (mc & 1);
    return join(lds_tr(p), lds_tr(p + 16 * DK * 2));
}

// V in accumulator layout of tile mt: lane (col, g) gets V[16mt + 4g + e][16w + col].
template <int VT>
__device__ __forceinline__ bf16x4 v_frag(const char* tile, int mt, int w, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, qd = lane & 3;
    const int r = 16 * mt + 4 * g + j;
    return lds_tr(tile + r * (VT * 2) + 16 * ((2 * w + (qd >> 1)) ^ swz_v<VT>(r)) + 8 * (qd & 1));
}

__device__ __forceinline__ int swz_t(int i) { return (((i >> 1) & 3) << 1) | ((i >> 3) & 1); }

// T tiles: accumulator tile (rows 16rb + 4g + e, cols 16cb + lane%16) into
// transposed storage, Tt[i][r] = T[r][i] (64 x 64 bf16), piece p of row i at
// p ^ swz_t(i); the compute waves read operand fragments with
// ds_read_b64_tr_b16.
__device__ __forceinline__ void tp_store(char* tile, int rb, int cb, int lane, f32x4 x) {
    const int i = 16 * cb + (lane & 15), g = lane >> 4;
    const bf16x4 y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<bf16x4*>(tile + i * 128 + 16 * ((2 * rb + (g >> 1)) ^ swz_t(i)) + 8 * (g & 1)) = y;
}

// T's rounding residual x - bf16(x), stored the same way into a second tile.
// Chunks whose keys repeat or nearly repeat (large entries of A) apply T as the
// bf16 pair (D = T R + T_lo R): T's rows then hold entries of size ~1 whose
// sums are small, and one bf16 rounding of T alone would lose those sums.
__device__ __forceinline__ void tp_store_lo(char* lo, int rb, int cb, int lane, f32x4 x) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = x[e] - (float)(__bf16)x[e];
    tp_store(lo, rb, cb, lane, r);
}
// A chunk takes the pair when some strictly lower entry of A exceeds this in
// size.  Unit keys in general position stay well below it
// (|k_r . k_i| is about 1/sqrt(d_k)); it catches keys that repeat or nearly
// repeat over a stretch of the chunk at beta near 1 and weak decay.
constexpr float kPairThresh = 0.5f;

// P tiles are kept in the compute waves' operand order, lane by lane: fragment
// (rb, s) of the 64 x 64 tile is 64 lanes x 16 bytes, and lane (r, g) holds
// row 16rb + r, columns 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3) (the
// token k-slots of the output product), so a compute wave reads an operand
// with one 16-byte load of its own.  The P wave computes transposed 16 x 16
// blocks: in a transposed accumulator block (block row rb, block column cb)
// lane (col, g4) holds P[16rb + col][16cb + 4g4 + e], e < 4, which is exactly
// half of what the same lane reads back.
__device__ __forceinline__ void frag_store(char* tile, int rb, int cb, int lane, f32x4 x) {
    const bf16x4 y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<bf16x4*>(tile + ((rb * (FC / 32) + (cb >> 1)) * 64 + lane) * 16 + 8 * (cb & 1)) = y;
}
__device__ __forceinline__ bf16x8 frag_load(const char* tile, int rb, int s, int lane) {
    return lds_b128(tile + ((rb * (FC / 32) + s) * 64 + lane) * 16);
}

// Per-lane LDS byte offsets of the compute waves' fragment reads, computed once:
// every read is then one of these plus a wave-uniform offset (row block,
// k-step, stage), which keeps the address registers few.
template <int DK, int VT>
struct FragOffsets {
    int qk[DK / 32];   // row-wise Q / K fragment, channel step s (row block 0)
    int kt[DK / 32];   // K^T fragment, state tile pair mc/2 (token step 0, tile mc even)
    int tp[FNB];       // T fragment, row block mt (token step 0)
    int v;             // V fragment, tile 0
    __device__ __forceinline__ FragOffsets(int lane, int wave) {
        const int g = lane >> 4, j = (lane >> 2) & 3, qd = lane & 3, c = lane & 15;
        const int r = 4 * g + j;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            qk[s] = c * (DK * 2) + 16 * ((4 * s + g) ^ swz_qk<DK>(c));
            kt[s] = r * (DK * 2) + 16 * ((4 * s + qd) ^ swz_qk<DK>(r));
        }
#pragma unroll
        for (int mt = 0; mt < FNB; ++mt) tp[mt] = r * 128 + 16 * ((2 * mt + (qd >> 1)) ^ swz_t(r)) + 8 * (qd & 1);
        v = r * (VT * 2) + 16 * ((2 * wave + (qd >> 1)) ^ swz_v<VT>(r)) + 8 * (qd & 1);
    }
    __device__ __forceinline__ bf16x8 qkf(const char* tile, int rb, int s) const {
        return lds_b128(tile + qk[s] + rb * 16 * DK * 2);
    }
    __device__ __forceinline__ bf16x8 ktf(const char* tile, int mc, int s) const {
        const char* p = tile + kt[mc >> 1] + 8 * (mc & 1) + s * 32 * DK * 2;
        return join(lds_tr(p), lds_tr(p + 16 * DK * 2));
    }
    // Operand of a transposed-stored T tile: lane%16 selects r = 16mt + lane%16,
    // k-slots = tokens i = 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3).
    __device__ __forceinline__ bf16x8 tpf(const char* tile, int mt, int s) const {
        const char* p = tile + tp[mt] + s * 32 * 128;
        return join(lds_tr(p), lds_tr(p + 16 * 128));
    }
    __device__ __forceinline__ bf16x4 vf(const char* tile, int mt) const {
        return lds_tr(tile + v + mt * 16 * VT * 2);
    }
};

// Loader wave lw (of NL): copies of chunk inputs into one stage, every NL-th
// 1 KB copy instruction.  The per-lane source offsets (bytes from the chunk's
// first row) are fixed for full chunks and computed once; rows at or past len
// repeat row len-1 (finite; the prep masks them out).
template <int DK, int NW, int NL>
struct LoadOffsets {
    static constexpr int NIQ = FLayout<DK, NW>::QB / 1024 / NL;   // Q (and K) instructions per loader
    static constexpr int NIV = FLayout<DK, NW>::VB / 1024 / NL;   // V instructions per loader
    static_assert(NIV * NL * 1024 == FLayout<DK, NW>::VB, "V tile split");
    int qk[NIQ];
    int v[NIV];
    __device__ __forceinline__ void set(int len, int H, int DV, int vt, int lw, int lane) {
        constexpr int VT = 16 * NW, RP = DK / 8, RPV = VT / 8;
#pragma unroll
        for (int j = 0; j < NIQ; ++j) {
            const int slot = 64 * (NL * j + lw) + lane;
            const int r = slot / RP, pp = slot % RP;
            qk[j] = (r < len ? r : len - 1) * (H * DK * 2) + 16 * (pp ^ swz_qk<DK>(r));
        }
#pragma unroll
        for (int j = 0; j < NIV; ++j) {
            const int slot = 64 * (NL * j + lw) + lane;
            const int r = slot / RPV, pp = slot % RPV;
            v[j] = (r < len ? r : len - 1) * (H * DV * 2) + vt * VT * 2 + 16 * (pp ^ swz_v<VT>(r));
        }
    }
};

template <int DK, int NW, int NL>
__device__ __forceinline__ void load_chunk(char* stg, char* qtile, const __bf16* q, const __bf16* k,
                                           const __bf16* v, int64_t row0, int DV, const LoadOffsets<DK, NW, NL>& lo,
                                           int lw) {
    using L = FLayout<DK, NW>;
    using LO = LoadOffsets<DK, NW, NL>;
    const char* qb = reinterpret_cast<const char*>(q + row0 * DK);
    const char* kb = reinterpret_cast<const char*>(k + row0 * DK);
    const char* vb = reinterpret_cast<const char*>(v + row0 * DV);
#pragma unroll
    for (int j = 0; j < LO::NIQ; ++j) {
        const int ins = NL * j + lw;
        __builtin_amdgcn_global_load_lds(qb + (uint32_t)lo.qk[j], (GDR_LDS void*)(qtile + 1024 * ins), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(kb + (uint32_t)lo.qk[j], (GDR_LDS void*)(stg + L::S_K + 1024 * ins), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LO::NIV; ++j) {
        const int ins = NL * j + lw;
        __builtin_amdgcn_global_load_lds(vb + (uint32_t)lo.v[j], (GDR_LDS void*)(stg + L::S_V + 1024 * ins), 16, 0, 0);
    }
}

// L2 warming of the chunk copied in the next window: one 4-byte LDS-DMA load
// per 128-byte line of its Q rows (loader 0) and of its K rows and the
// workgroup's V segment (loader 1), into a scratch word per lane that nothing
// reads.  These loads stay in flight across the window barrier, and the next
// window's copies then find the lines in L2.
template <int DK, int NW>
__device__ __forceinline__ void warm_chunk(char* scratch, const __bf16* q, const __bf16* k, const __bf16* v,
                                           int64_t row0, int len, int H, int DV, int vt, int lw, int lane) {
    const int64_t r = row0 + (int64_t)(lane < len ? lane : len - 1) * H;
    if (lw == 0) {
#pragma unroll
        for (int j = 0; j < DK / 64; ++j)
            __builtin_amdgcn_global_load_lds(q + r * DK + 64 * j, (GDR_LDS void*)scratch, 4, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < DK / 64; ++j)
            __builtin_amdgcn_global_load_lds(k + r * DK + 64 * j, (GDR_LDS void*)scratch, 4, 0, 0);
        __builtin_amdgcn_global_load_lds(v + r * DV + vt * 16 * NW, (GDR_LDS void*)scratch, 4, 0, 0);
    }
}

// DPP move of x (row_shr, row_bcast); lanes without a source get 0.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK,
                                                                  0xf, false));
}

// Inclusive prefix sum over the 64 lanes: shifts 1, 2, 4, 8 inside each row of
// 16 lanes, then the row totals carried into rows 1 and 3 (row_bcast:15) and
// into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_scan(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    x += dpp<0x142, 0xa>(x);
    x += dpp<0x143, 0xc>(x);
    return x;
}

__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// The gate table of one chunk (layout in FLayout), built by loader 0 from the
// chunk's gate values (lane r holds log alpha and beta of token r).  Lane = token row r; rows >= len get
// log alpha = 0 and beta = 0.  With the block-boundary factors, for r in block
// rb > cb >= blk(i):
//   e^{g_r - g_i} = EB[r] * CX(cb, rb) * FB[i],
// a product of factors <= 1 (no overflow; an underflow bounds a negligible value).
template <int DK, int NW>
__device__ __forceinline__ void gate_table(float la, float bb, int len, int lane, float* tab, int gflags) {
    using L = FLayout<DK, NW>;
    if (gflags & kPrologueDecaySoftplus) la = neg_softplus(la);   // prologue: decay from its logit
    if (gflags & kPrologueBetaSigmoid) bb = sigmoid_of(bb);       // prologue: beta from its logit
    la = lane < len ? fmaxf(la, kFMinLogAlpha) : 0.f;
    bb = lane < len ? bb : 0.f;
    const float g2 = wave_scan(la * 1.4426950408889634f);
    const float e0 = lane_value(g2, 15), e1 = lane_value(g2, 31), e2 = lane_value(g2, 47),
                e3 = lane_value(g2, 63);
    const int blk = lane >> 4;
    const float gprev = blk == 0 ? 0.f : (blk == 1 ? e0 : (blk == 2 ? e1 : e2));
    const float gend = blk == 0 ? e0 : (blk == 1 ? e1 : (blk == 2 ? e2 : e3));
    tab[L::G_G2 * FC + lane] = g2;
    tab[L::G_BE * FC + lane] = bb;
    tab[L::G_EB * FC + lane] = __builtin_amdgcn_exp2f(g2 - gprev);
    tab[L::G_FB * FC + lane] = __builtin_amdgcn_exp2f(gend - g2);
    tab[L::G_GM * FC + lane] = __builtin_amdgcn_exp2f(g2);
    tab[L::G_GH * FC + lane] = __builtin_amdgcn_exp2f(e3 - g2);
    if (lane < 3) {
        const float d = lane == 0 ? e1 - e0 : (lane == 1 ? e2 - e0 : e2 - e1);
        tab[L::G_CX * FC + lane] = __builtin_amdgcn_exp2f(d);
    }
}

// CX(cb, rb) (1 when the blocks are adjacent), from the table.
template <int DK, int NW>
__device__ __forceinline__ float cross_decay(const float* tab, int cb, int rb) {
    using L = FLayout<DK, NW>;
    if (rb == cb + 1) return 1.f;
    return tab[L::G_CX * FC + (cb == 0 ? rb - 2 : 2)];
}

// Inverse L2 norms of the 16 rows of one block from its diagonal Gram tile
// G = X X^T (accumulator layout: lane (col, g4) holds G[4g4 + e][col]).  The
// diagonal sits on the lanes with g4 = col / 4, element col % 4; every lane
// takes the candidate of its own element col % 4 and two register broadcasts
// (no memory round trip) hand each lane the values it needs:
//   c  = n(col)              (the column form),
//   r  = n(4g4 + e), e < 4   (the row form: a permute to quad lane col % 4,
//                             then a broadcast of each quad lane).
constexpr float kNormEps = 1e-6f;
struct InvNorms {
    float c;
    float r[4];
};
__device__ __forceinline__ float bcast_quad(float x, int e) {
    const int v = __builtin_bit_cast(int, x);
    const int y = e == 0 ? __builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false)
                : e == 1 ? __builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false)
                : e == 2 ? __builtin_amdgcn_mov_dpp(v, 0xAA, 0xf, 0xf, false)
                         : __builtin_amdgcn_mov_dpp(v, 0xFF, 0xf, 0xf, false);
    return __builtin_bit_cast(float, y);
}
__device__ __forceinline__ InvNorms inv_norms(const f32x4& G, int lane) {
    const int col = lane & 15, g4 = lane >> 4, e = col & 3;
    const float d = e == 0 ? G[0] : e == 1 ? G[1] : e == 2 ? G[2] : G[3];
    const int nd = __builtin_bit_cast(int, __builtin_amdgcn_rsqf(d + kNormEps));
    InvNorms n;
    n.c = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (col + 16 * (col >> 2)), nd));
    const float t = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (20 * g4 + e), nd));
#pragma unroll
    for (int i = 0; i < 4; ++i) n.r[i] = bcast_quad(t, i);
    return n;
}

// Whether a chunk applies T as a bf16 pair: some entry of the off-diagonal
// 16 x 16 blocks of A (scaled, fp32) exceeds kPairThresh in size (the diagonal
// blocks are tested where they are formed, below).  Wave-uniform.
template <int N>
__device__ __forceinline__ bool pair_needed(const f32x4 (&a)[N]) {
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < N; ++t) m = fmaxf(m, fmaxf(fmaxf(fabsf(a[t][0]), fabsf(a[t][1])), fmaxf(fabsf(a[t][2]), fabsf(a[t][3]))));
    return __builtin_amdgcn_ballot_w64(m > kPairThresh) != 0;
}

// The same test on the diagonal blocks: strictly lower entries of A_bb in B
// layout (lane (col, g4) holds A_bb[4g4 + e][col]).
__device__ __forceinline__ bool pair_needed_diag(const f32x4 (&Ab)[FNB], int lane) {
    const int col = lane & 15, g4 = lane >> 4;
    float m = 0.f;
#pragma unroll
    for (int b = 0; b < FNB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, col < 4 * g4 + e ? fabsf(Ab[b][e]) : 0.f);
    return __builtin_amdgcn_ballot_w64(m > kPairThresh) != 0;
}

// Prep T: T = (I + A)^-1 Diag(beta) for one chunk, in one wave.
//  - The diagonal Gram tiles K_b K_b^T on the matrix cores; the off-diagonal
//    blocks of A come from the P wave (A-operand layout) through LDS.
//  - Diagonal blocks: with A_bb = [[A11, 0], [A21, A22]] (8x8 blocks),
//    D = blockdiag((I + A11)^-1, (I + A22)^-1) and N = [[0, 0], [A21, 0]],
//        X_bb = (I + A_bb)^-1 = D - D N D.
//    The 8x8 inverses come from forward substitution in fp32 (lane = column j
//    of half h of block b; at most 7 dependent steps), the correction from fp16
//    16x16x16 MFMAs, in both operand layouts.
//  - Off-diagonal blocks of X = (I + A)^-1 by the block recurrence
//        X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj
//    (carried out for T = X Diag(beta) directly) on fp16 16x16x16 MFMAs with
//    fp32 accumulation, row block by row block.
//  Entries of A and X are bounded by small constants here (unit-norm keys,
//  beta <= 1, decays <= 1), well inside fp16's range; T is rounded to bf16 after.
template <int DK, int NW, bool NORM>
__device__ __forceinline__ void prep_t(char* smem, const char* st, const float* tab, char* tp, int n,
                                       int lane) {
    using L = FLayout<DK, NW>;
    constexpr int NKC = DK / 32;
    float* xa = reinterpret_cast<float*>(smem + L::XA);
    const int col = lane & 15, g4 = lane >> 4;

    bf16x8 kf[FNB][NKC];
#pragma unroll
    for (int rb = 0; rb < FNB; ++rb)
#pragma unroll
        for (int s = 0; s < NKC; ++s) kf[rb][s] = qk_frag<DK>(st + L::S_K, rb, s, lane);
    // Gram tiles of the diagonal blocks (symmetric): element (4g4 + e, col).
    f32x4 Gd[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) Gd[b] = zero4();
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int b = 0; b < FNB; ++b) Gd[b] = Mma<__bf16>::mma(kf[b][s], kf[b][s], Gd[b]);
    // A_bb in B layout (row 4g4 + e, column col), also stored transposed:
    // xa[b][m][i] = A_bb[i][m].  Entries on or above the diagonal are not
    // masked: nothing reads them (the substitution uses rows i > m only, and N
    // lies strictly below).
    f32x4 Ab[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) {
        const float4 gr = *reinterpret_cast<const float4*>(tab + L::G_G2 * FC + 16 * b + 4 * g4);
        const float4 br = *reinterpret_cast<const float4*>(tab + L::G_BE * FC + 16 * b + 4 * g4);
        const float gc = tab[L::G_G2 * FC + 16 * b + col];
        const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) Ab[b][e] = Gd[b][e] * brv[e] * __builtin_amdgcn_exp2f(grv[e] - gc);
        if constexpr (NORM) {   // prologue: A from the normalised keys
            const InvNorms nk = inv_norms(Gd[b], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ab[b][e] *= nk.r[e] * nk.c;
        }
        *reinterpret_cast<float4*>(xa + b * XTILE + col * XROW + 4 * g4) =
            make_float4(Ab[b][0], Ab[b][1], Ab[b][2], Ab[b][3]);
    }
    const bool pair_diag = pair_needed_diag(Ab, lane);
    // 8x8 forward substitution: lane (blk, h, j) builds column j of (I + A_hh)^-1.
    {
        const int blk = lane >> 4, h = (lane >> 3) & 1, j = lane & 7;
        float* Ab8 = xa + blk * XTILE + 8 * h * XROW + 8 * h;   // element (i, m) of A_hh at Ab8[m * XROW + i]
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 7; ++m) {
            float am[8];
#pragma unroll
            for (int qv = (m + 1) / 4; qv < 2; ++qv) {
                const float4 t = *reinterpret_cast<const float4*>(Ab8 + m * XROW + 4 * qv);
                am[4 * qv] = t.x; am[4 * qv + 1] = t.y; am[4 * qv + 2] = t.z; am[4 * qv + 3] = t.w;
            }
#pragma unroll
            for (int i = m + 1; i < 8; ++i) x[i] -= am[i] * x[m];
        }
        // D = blockdiag of the 8x8 inverses, staged row-major over the diagonal
        // quadrants of the A tile: D[blk][r][c] at blk*XTILE + r*XROW + c.  The
        // upper-right quadrant (rows < 8, columns >= 8) keeps A transposed, i.e.
        // the lower-left block N of A_bb: N[c][r] at blk*XTILE + r*XROW + c.
#pragma unroll
        for (int i = 0; i < 8; ++i) Ab8[i * XROW + j] = x[i];
    }
    // Operands of X_bb = D - D N D for all four blocks (loads first, selects after).
    const bool same = (g4 >> 1) == (col >> 3);   // rows 4g4.. and column col in one 8x8 half
    f32x4 DbB[FNB], DbA[FNB], NA[FNB], NB[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) {
        const float* Db = xa + b * XTILE;
        // element (4g4 + e, col) of the staged tile: D there on the diagonal
        // quadrants, N[col][4g4 + e] on the upper-right one
        f32x4 tb;
#pragma unroll
        for (int e = 0; e < 4; ++e) tb[e] = Db[(4 * g4 + e) * XROW + col];
        const float4 t = *reinterpret_cast<const float4*>(Db + col * XROW + 4 * g4);
        const bool nb = g4 >= 2 && col < 8, na = col >= 8 && g4 < 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            DbB[b][e] = same ? tb[e] : 0.f;
            NA[b][e] = na ? tb[e] : 0.f;
            NB[b][e] = nb ? Ab[b][e] : 0.f;
        }
        DbA[b] = same ? f32x4{t.x, t.y, t.z, t.w} : zero4();
    }
    f32x4 Xb[FNB];   // X_bb, B layout: (4g4 + e, col)
    f16x4 Xa[FNB];   // X_bb, A layout: (col, 4g4 + e)
    {
        f16x4 dB[FNB], dA[FNB];
        f32x4 nd[FNB], ntdt[FNB];
#pragma unroll
        for (int b = 0; b < FNB; ++b) {
            dB[b] = to_f16(DbB[b]);
            dA[b] = to_f16(DbA[b]);
            nd[b] = mma16(to_f16(NA[b]), dB[b], zero4());       // B layout of N D
            ntdt[b] = mma16(to_f16(NB[b]), dA[b], zero4());     // B layout of N^T D^T
        }
#pragma unroll
        for (int b = 0; b < FNB; ++b) {
            Xb[b] = DbB[b] - mma16(dA[b], to_f16(nd[b]), zero4());            // D - (D N D), B layout
            Xa[b] = to_f16(DbA[b] - mma16(dB[b], to_f16(ntdt[b]), zero4()));  // the same, A layout
        }
    }
    // Off-diagonal blocks of A, from the P wave (A-operand layout).
    while (__hip_atomic_load(reinterpret_cast<int*>(smem + L::FLAG), __ATOMIC_ACQUIRE,
                             __HIP_MEMORY_SCOPE_WORKGROUP) != n + 1)
        __builtin_amdgcn_s_sleep(1);
    f16x4 Ao[FNB][FNB];
    {
        const f16x4* ao = reinterpret_cast<const f16x4*>(smem + L::AO);
#pragma unroll
        for (int rb = 1; rb < FNB; ++rb)
#pragma unroll
            for (int cb = 0; cb < rb; ++cb) Ao[rb][cb] = ao[(rb * (rb - 1) / 2 + cb) * 64 + lane];
    }
    // T = X Diag(beta) satisfies the same recurrence, T_ij = -X_ii sum A_im T_mj,
    // from T_jj = X_jj Diag(beta_j).  Row wavefront: for row block i, every
    // column block j < i at once (the T_mj it needs, m < i, are done), so
    // independent chains interleave.
    char* Tt = tp + L::T_T;
    char* Tl = tp + L::T_L;
    const bool pair = pair_diag ||
                      __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(tp + L::T_FLAG)) != 0;
    if (pair_diag && lane == 0) *reinterpret_cast<int*>(tp + L::T_FLAG) = 1;
    f16x4 xm[FNB][FNB];   // B layout of T_mj, fp16
    f32x4 tb[FNB * (FNB + 1) / 2];   // the blocks of T, stored after the recurrence
#pragma unroll
    for (int j = 0; j < FNB; ++j) {
        tb[j * (j + 1) / 2 + j] = Xb[j] * tab[L::G_BE * FC + 16 * j + col];
        xm[j][j] = to_f16(tb[j * (j + 1) / 2 + j]);
    }
#pragma unroll
    for (int i = 1; i < FNB; ++i) {
        f32x4 y[FNB];
#pragma unroll
        for (int j = 0; j < i; ++j) y[j] = zero4();
#pragma unroll
        for (int m = 0; m < i; ++m)
#pragma unroll
            for (int j = 0; j <= m; ++j) y[j] = mma16(Ao[i][m], xm[m][j], y[j]);
#pragma unroll
        for (int j = 0; j < i; ++j) {
            tb[i * (i + 1) / 2 + j] = -mma16(Xa[i], to_f16(y[j]), zero4());
            xm[i][j] = to_f16(tb[i * (i + 1) / 2 + j]);
        }
    }
#pragma unroll
    for (int i = 0; i < FNB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) tp_store(Tt, i, j, lane, tb[i * (i + 1) / 2 + j]);
    if (pair) {
#pragma unroll
        for (int i = 0; i < FNB; ++i)
#pragma unroll
            for (int j = 0; j <= i; ++j) tp_store_lo(Tl, i, j, lane, tb[i * (i + 1) / 2 + j]);
    }
}

// Within one wave, LDS written by some lanes and read by others: the fences
// keep the compiler from moving the reads above the writes (the hardware keeps
// one wave's LDS accesses in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// With the gate prologue (whose P wave carries the norm work), T = (I + A)^-1
// Diag(beta) is built by two waves instead, so that neither waits on the other
// inside a window:
//  - the solve wave inverts the diagonal blocks of chunk c one window before
//    the recurrence wave needs them, from K fragments and gate values it reads
//    from global memory itself (prefetched one window earlier still; the LDS
//    stage of chunk c is being filled in the same window);
//  - the recurrence wave forms the off-diagonal blocks of A from the chunk's
//    LDS stage and runs the block recurrence.
//
// The solve wave's inputs of one chunk, from global memory: K fragments in the
// row-wise operand layout (rows 16rb + lane%16, channels 32s + 8(lane/16) ..
// +7) and the gate values of token row = lane; rows at or past len repeat row
// len - 1, as in the LDS stages.
template <int DK>
__device__ __forceinline__ void solve_loads(const __bf16* k, const float* log_alpha, const float* beta,
                                            int64_t row0, int len, int H, int lane,
                                            bf16x8 (&kf)[FNB][DK / 32], float& la, float& bb) {
#pragma unroll
    for (int rb = 0; rb < FNB; ++rb) {
        const int r = 16 * rb + (lane & 15);
        const __bf16* p = k + (row0 + (int64_t)(r < len ? r : len - 1) * H) * DK + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) kf[rb][s] = *reinterpret_cast<const bf16x8*>(p + 32 * s);
    }
    const int64_t go = row0 + (int64_t)(lane < len ? lane : len - 1) * H;
    la = log_alpha[go];
    bb = beta[go];
}

// Solve: X_bb = (I + A_bb)^-1 of the four diagonal 16x16 blocks.
//  - The diagonal Gram tiles K_b K_b^T on the matrix cores.
//  - With A_bb = [[A11, 0], [A21, A22]] (8x8 blocks),
//    D = blockdiag((I + A11)^-1, (I + A22)^-1) and N = [[0, 0], [A21, 0]],
//        X_bb = (I + A_bb)^-1 = D - D N D.
//    The 8x8 inverses come from forward substitution in fp32 (lane = column j
//    of half h of block b; at most 7 dependent steps), the correction from fp16
//    16x16x16 MFMAs.
//  Entries of A and X are bounded by small constants here (unit-norm keys,
//  beta <= 1, decays <= 1), well inside fp16's range; T is rounded to bf16 after.
//  Output: X_bb in A-operand layout (fp16) and, with the prologue, n_k, into
//  the chunk's hand-off slot xh.
template <int DK, int NW, bool NORM>
__device__ __forceinline__ void solve_diag(char* smem, const bf16x8 (&kf)[FNB][DK / 32], float la, float bb,
                                           int len, int gflags, char* xh, int lane) {
    using L = FLayout<DK, NW>;
    constexpr int NKC = DK / 32;
    float* xa = reinterpret_cast<float*>(smem + L::XA);
    float* tg = reinterpret_cast<float*>(smem + L::TG);
    const int col = lane & 15, g4 = lane >> 4;

    // The chunk's g (log2 units) and beta rows, as the gate table has them.
    {
        if (gflags & kPrologueDecaySoftplus) la = neg_softplus(la);
        if (gflags & kPrologueBetaSigmoid) bb = sigmoid_of(bb);
        la = lane < len ? fmaxf(la, kFMinLogAlpha) : 0.f;
        bb = lane < len ? bb : 0.f;
        tg[lane] = wave_scan(la * 1.4426950408889634f);
        tg[FC + lane] = bb;
    }
    // Gram tiles of the diagonal blocks (symmetric): element (4g4 + e, col).
    f32x4 Gd[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) Gd[b] = zero4();
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int b = 0; b < FNB; ++b) Gd[b] = Mma<__bf16>::mma(kf[b][s], kf[b][s], Gd[b]);
    wave_lds_sync();
    float nkl = 0.f;   // prologue: n_k of row = lane
    // A_bb in B layout (row 4g4 + e, column col), also stored transposed:
    // xa[b][m][i] = A_bb[i][m].  Entries on or above the diagonal are not
    // masked: nothing reads them (the substitution uses rows i > m only, and N
    // lies strictly below).
    f32x4 Ab[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) {
        const float4 gr = *reinterpret_cast<const float4*>(tg + 16 * b + 4 * g4);
        const float4 br = *reinterpret_cast<const float4*>(tg + FC + 16 * b + 4 * g4);
        const float gc = tg[16 * b + col];
        const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) Ab[b][e] = Gd[b][e] * brv[e] * __builtin_amdgcn_exp2f(grv[e] - gc);
        if constexpr (NORM) {   // prologue: A from the normalised keys
            const InvNorms nk = inv_norms(Gd[b], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ab[b][e] *= nk.r[e] * nk.c;
            nkl = g4 == b ? nk.c : nkl;
        }
        *reinterpret_cast<float4*>(xa + b * XTILE + col * XROW + 4 * g4) =
            make_float4(Ab[b][0], Ab[b][1], Ab[b][2], Ab[b][3]);
    }
    wave_lds_sync();
    const bool pair_diag = pair_needed_diag(Ab, lane);
    // 8x8 forward substitution: lane (blk, h, j) builds column j of (I + A_hh)^-1.
    {
        const int blk = lane >> 4, h = (lane >> 3) & 1, j = lane & 7;
        float* Ab8 = xa + blk * XTILE + 8 * h * XROW + 8 * h;   // element (i, m) of A_hh at Ab8[m * XROW + i]
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 7; ++m) {
            float am[8];
#pragma unroll
            for (int qv = (m + 1) / 4; qv < 2; ++qv) {
                const float4 t = *reinterpret_cast<const float4*>(Ab8 + m * XROW + 4 * qv);
                am[4 * qv] = t.x; am[4 * qv + 1] = t.y; am[4 * qv + 2] = t.z; am[4 * qv + 3] = t.w;
            }
#pragma unroll
            for (int i = m + 1; i < 8; ++i) x[i] -= am[i] * x[m];
        }
        // D = blockdiag of the 8x8 inverses, staged row-major over the diagonal
        // quadrants of the A tile: D[blk][r][c] at blk*XTILE + r*XROW + c.  The
        // upper-right quadrant (rows < 8, columns >= 8) keeps A transposed, i.e.
        // the lower-left block N of A_bb: N[c][r] at blk*XTILE + r*XROW + c.
#pragma unroll
        for (int i = 0; i < 8; ++i) Ab8[i * XROW + j] = x[i];
    }
    wave_lds_sync();
    // Operands of X_bb = D - D N D for all four blocks (loads first, selects after).
    const bool same = (g4 >> 1) == (col >> 3);   // rows 4g4.. and column col in one 8x8 half
    f32x4 DbB[FNB], DbA[FNB], NA[FNB], NB[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) {
        const float* Db = xa + b * XTILE;
        // element (4g4 + e, col) of the staged tile: D there on the diagonal
        // quadrants, N[col][4g4 + e] on the upper-right one
        f32x4 tb;
#pragma unroll
        for (int e = 0; e < 4; ++e) tb[e] = Db[(4 * g4 + e) * XROW + col];
        const float4 t = *reinterpret_cast<const float4*>(Db + col * XROW + 4 * g4);
        const bool nb = g4 >= 2 && col < 8, na = col >= 8 && g4 < 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            DbB[b][e] = same ? tb[e] : 0.f;
            NA[b][e] = na ? tb[e] : 0.f;
            NB[b][e] = nb ? Ab[b][e] : 0.f;
        }
        DbA[b] = same ? f32x4{t.x, t.y, t.z, t.w} : zero4();
    }
    f16x4 Xa[FNB];   // X_bb, A layout: (col, 4g4 + e)
    {
        f16x4 dB[FNB], dA[FNB];
        f32x4 nd[FNB], ntdt[FNB];
#pragma unroll
        for (int b = 0; b < FNB; ++b) {
            dB[b] = to_f16(DbB[b]);
            dA[b] = to_f16(DbA[b]);
            nd[b] = mma16(to_f16(NA[b]), dB[b], zero4());       // B layout of N D
            ntdt[b] = mma16(to_f16(NB[b]), dA[b], zero4());     // B layout of N^T D^T
        }
#pragma unroll
        for (int b = 0; b < FNB; ++b)
            Xa[b] = to_f16(DbA[b] - mma16(dB[b], to_f16(ntdt[b]), zero4()));  // D - (D N D), A layout
    }
    f16x4* xo = reinterpret_cast<f16x4*>(xh);
#pragma unroll
    for (int b = 0; b < FNB; ++b) xo[b * 64 + lane] = Xa[b];
    if constexpr (NORM) reinterpret_cast<float*>(xh + FNB * 64 * 8)[lane] = nkl;
    if (lane == 0) *reinterpret_cast<int*>(xh + FNB * 64 * 8 + FC * 4) = pair_diag ? 1 : 0;
}

// Recurrence: the off-diagonal blocks of A (K_cb K_rb^T, scaled) in A-operand
// layout, then the off-diagonal blocks of X = (I + A)^-1 by
//     X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj
// (carried out for T = X Diag(beta) directly) on fp16 16x16x16 MFMAs with fp32
// accumulation, row block by row block.  The decay of A[r][i] = beta_r
// e^{g_r - g_i} G[r][i] is split at the block boundaries (see gate_table).
template <int DK, int NW, bool NORM>
__device__ __forceinline__ void recur_off(const char* st, const float* tab, const char* xh, char* tp,
                                          int lane) {
    using L = FLayout<DK, NW>;
    constexpr int NKC = DK / 32;
    const int col = lane & 15, g4 = lane >> 4;

    bf16x8 kf[FNB][NKC];
#pragma unroll
    for (int rb = 0; rb < FNB; ++rb)
#pragma unroll
        for (int s = 0; s < NKC; ++s) kf[rb][s] = qk_frag<DK>(st + L::S_K, rb, s, lane);
    const f16x4* xi = reinterpret_cast<const f16x4*>(xh);
    f16x4 Xa[FNB];   // X_bb, A layout: (col, 4g4 + e)
#pragma unroll
    for (int b = 0; b < FNB; ++b) Xa[b] = xi[b * 64 + lane];
    const float* nkv = reinterpret_cast<const float*>(xh + FNB * 64 * 8);
    // lane (col, g4) of block (rb, cb) holds A[16rb + col][16cb + 4g4 + e]
    constexpr int NOFF = FNB * (FNB - 1) / 2;
    f32x4 go[NOFF];
#pragma unroll
    for (int t = 0; t < NOFF; ++t) go[t] = zero4();
#pragma unroll
    for (int s = 0; s < NKC; ++s) {
        int t = 0;
#pragma unroll
        for (int rb = 1; rb < FNB; ++rb)
#pragma unroll
            for (int cb = 0; cb < rb; ++cb, ++t) go[t] = Mma<__bf16>::mma(kf[cb][s], kf[rb][s], go[t]);
    }
    f16x4 Ao[FNB][FNB];
#pragma unroll
    for (int rb = 1; rb < FNB; ++rb) {
        const float f0 = tab[L::G_BE * FC + 16 * rb + col] * tab[L::G_EB * FC + 16 * rb + col];
#pragma unroll
        for (int cb = 0; cb < rb; ++cb) {
            const float4 fr = *reinterpret_cast<const float4*>(tab + L::G_FB * FC + 16 * cb + 4 * g4);
            const float f = f0 * cross_decay<DK, NW>(tab, cb, rb);
            f32x4 acc = go[rb * (rb - 1) / 2 + cb];
            acc[0] *= f * fr.x;
            acc[1] *= f * fr.y;
            acc[2] *= f * fr.z;
            acc[3] *= f * fr.w;
            if constexpr (NORM) {
                const float nr = nkv[16 * rb + col];
                const float4 nc = *reinterpret_cast<const float4*>(nkv + 16 * cb + 4 * g4);
                acc[0] *= nr * nc.x; acc[1] *= nr * nc.y; acc[2] *= nr * nc.z; acc[3] *= nr * nc.w;
            }
            go[rb * (rb - 1) / 2 + cb] = acc;
            Ao[rb][cb] = to_f16(acc);
        }
    }
    // X_bb in B layout (4g4 + e, col) from the A layout: X_bb = X_bb I.
    f16x4 eye;
#pragma unroll
    for (int j = 0; j < 4; ++j) eye[j] = col == 4 * g4 + j ? (_Float16)1.f : (_Float16)0.f;
    f32x4 Xb[FNB];
#pragma unroll
    for (int b = 0; b < FNB; ++b) Xb[b] = mma16(Xa[b], eye, zero4());
    // T = X Diag(beta) satisfies the same recurrence, T_ij = -X_ii sum A_im T_mj,
    // from T_jj = X_jj Diag(beta_j).  Row wavefront: for row block i, every
    // column block j < i at once (the T_mj it needs, m < i, are done), so
    // independent chains interleave.
    char* Tt = tp + L::T_T;
    char* Tl = tp + L::T_L;
    const bool pair = pair_needed(go) ||
                      __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(xh + FNB * 64 * 8 + FC * 4)) != 0;
    if (lane == 0) *reinterpret_cast<int*>(tp + L::T_FLAG) = pair ? 1 : 0;
    f16x4 xm[FNB][FNB];   // B layout of T_mj, fp16
    f32x4 tb[FNB * (FNB + 1) / 2];   // the blocks of T, stored after the recurrence
#pragma unroll
    for (int j = 0; j < FNB; ++j) {
        tb[j * (j + 1) / 2 + j] = Xb[j] * tab[L::G_BE * FC + 16 * j + col];
        xm[j][j] = to_f16(tb[j * (j + 1) / 2 + j]);
    }
#pragma unroll
    for (int i = 1; i < FNB; ++i) {
        f32x4 y[FNB];
#pragma unroll
        for (int j = 0; j < i; ++j) y[j] = zero4();
#pragma unroll
        for (int m = 0; m < i; ++m)
#pragma unroll
            for (int j = 0; j <= m; ++j) y[j] = mma16(Ao[i][m], xm[m][j], y[j]);
#pragma unroll
        for (int j = 0; j < i; ++j) {
            tb[i * (i + 1) / 2 + j] = -mma16(Xa[i], to_f16(y[j]), zero4());
            xm[i][j] = to_f16(tb[i * (i + 1) / 2 + j]);
        }
    }
#pragma unroll
    for (int i = 0; i < FNB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) tp_store(Tt, i, j, lane, tb[i * (i + 1) / 2 + j]);
    if (pair) {
#pragma unroll
        for (int i = 0; i < FNB; ++i)
#pragma unroll
            for (int j = 0; j <= i; ++j) tp_store_lo(Tl, i, j, lane, tb[i * (i + 1) / 2 + j]);
    }
}

// Prep P: with one T wave, first the off-diagonal blocks of A for it; then
// P = (Q K^T) masked and decayed, stored transposed (and, with the prologue,
// the compute waves' per-token norm factors).
template <int DK, int NW, bool NORM, bool SPLIT>
__device__ __forceinline__ void prep_p(char* smem, const char* st, const char* qt, float* tab, char* tp, int n,
                                       int lane) {
    using L = FLayout<DK, NW>;
    constexpr int NKC = DK / 32;
    const int col = lane & 15, g4 = lane >> 4;

    bf16x8 kf[FNB][NKC], qf[FNB][NKC];
#pragma unroll
    for (int rb = 0; rb < FNB; ++rb)
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            kf[rb][s] = qk_frag<DK>(st + L::S_K, rb, s, lane);
            qf[rb][s] = qk_frag<DK>(qt, rb, s, lane);
        }
    InvNorms nk[FNB], nq[FNB];   // prologue: inverse row norms of k and q
    if constexpr (NORM) {
        // |k_r|^2 and |q_r|^2 from the diagonal Gram blocks, on the matrix cores
        f32x4 gk[FNB], gq[FNB];
#pragma unroll
        for (int b = 0; b < FNB; ++b) gk[b] = gq[b] = zero4();
#pragma unroll
        for (int s = 0; s < NKC; ++s)
#pragma unroll
            for (int b = 0; b < FNB; ++b) {
                gk[b] = Mma<__bf16>::mma(kf[b][s], kf[b][s], gk[b]);
                gq[b] = Mma<__bf16>::mma(qf[b][s], qf[b][s], gq[b]);
            }
#pragma unroll
        for (int b = 0; b < FNB; ++b) {
            nk[b] = inv_norms(gk[b], lane);
            nq[b] = inv_norms(gq[b], lane);
        }
        // per-token factors of the compute waves, lane = token row (this
        // chunk's slot; the compute waves read it in the next window)
        const float nk1 = g4 == 0 ? nk[0].c : g4 == 1 ? nk[1].c : g4 == 2 ? nk[2].c : nk[3].c;
        const float nq1 = g4 == 0 ? nq[0].c : g4 == 1 ? nq[1].c : g4 == 2 ? nq[2].c : nq[3].c;
        const float gm = tab[L::G_GM * FC + lane];
        tab[L::G_GMK * FC + lane] = gm * nk1;
        tab[L::G_GQ * FC + lane] = gm * nq1;
        tab[L::G_GHK * FC + lane] = tab[L::G_GH * FC + lane] * nk1;
    }
    // Off-diagonal blocks of A for the T wave, first: lane (col, g4) of block
    // (rb, cb) holds A[16rb + col][16cb + 4g4 + e], computed as K_cb K_rb^T
    // (the transpose of the needed block of the symmetric Gram matrix), with
    // A[r][i] = beta_r e^{g_r - g_i} G[r][i] and the decay split at the block
    // boundaries (see gate_table).
    if constexpr (!SPLIT) {
        constexpr int NOFF = FNB * (FNB - 1) / 2;
        f32x4 go[NOFF];
#pragma unroll
        for (int t = 0; t < NOFF; ++t) go[t] = zero4();
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            int t = 0;
#pragma unroll
            for (int rb = 1; rb < FNB; ++rb)
#pragma unroll
                for (int cb = 0; cb < rb; ++cb, ++t) go[t] = Mma<__bf16>::mma(kf[cb][s], kf[rb][s], go[t]);
        }
        f16x4* ao = reinterpret_cast<f16x4*>(smem + L::AO);
#pragma unroll
        for (int rb = 1; rb < FNB; ++rb) {
            const float f0 = tab[L::G_BE * FC + 16 * rb + col] * tab[L::G_EB * FC + 16 * rb + col];
#pragma unroll
            for (int cb = 0; cb < rb; ++cb) {
                const float4 fr = *reinterpret_cast<const float4*>(tab + L::G_FB * FC + 16 * cb + 4 * g4);
                const float f = f0 * cross_decay<DK, NW>(tab, cb, rb);
                f32x4 acc = go[rb * (rb - 1) / 2 + cb];
                acc[0] *= f * fr.x;
                acc[1] *= f * fr.y;
                acc[2] *= f * fr.z;
                acc[3] *= f * fr.w;
                if constexpr (NORM) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] *= nk[rb].c * nk[cb].r[e];
                }
                go[rb * (rb - 1) / 2 + cb] = acc;
                ao[(rb * (rb - 1) / 2 + cb) * 64 + lane] = to_f16(acc);
            }
        }
        // whether this chunk applies T as a bf16 pair (read by the T wave and the
        // compute waves; published with the blocks below)
        if (lane == 0) *reinterpret_cast<int*>(tp + L::T_FLAG) = pair_needed(go) ? 1 : 0;
        __hip_atomic_store(reinterpret_cast<int*>(smem + L::FLAG), n + 1, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    constexpr int NP = FNB * (FNB + 1) / 2;
    f32x4 pa[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t) pa[t] = zero4();
#pragma unroll
    for (int s = 0; s < NKC; ++s) {
        int t = 0;
#pragma unroll
        for (int rb = 0; rb < FNB; ++rb)
#pragma unroll
            for (int cb = 0; cb <= rb; ++cb, ++t) pa[t] = Mma<__bf16>::mma(kf[cb][s], qf[rb][s], pa[t]);
    }
    // Transposed blocks: lane (col, g4) holds P[r][i], r = 16rb + col, i = 16cb + 4g4 + e.
    char* Pt = tp + L::T_P;
#pragma unroll
    for (int rb = 0; rb < FNB; ++rb) {
        const float gr = tab[L::G_G2 * FC + 16 * rb + col];
        const float er = tab[L::G_EB * FC + 16 * rb + col];
#pragma unroll
        for (int cb = 0; cb <= rb; ++cb) {
            f32x4 acc = pa[rb * (rb + 1) / 2 + cb];
            if (cb == rb) {
                const float4 gi = *reinterpret_cast<const float4*>(tab + L::G_G2 * FC + 16 * cb + 4 * g4);
                const float giv[4] = {gi.x, gi.y, gi.z, gi.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = 4 * g4 + e <= col ? acc[e] * __builtin_amdgcn_exp2f(gr - giv[e]) : 0.f;
            } else {
                const float f = cross_decay<DK, NW>(tab, cb, rb) * er;
                const float4 fb = *reinterpret_cast<const float4*>(tab + L::G_FB * FC + 16 * cb + 4 * g4);
                acc[0] *= f * fb.x;
                acc[1] *= f * fb.y;
                acc[2] *= f * fb.z;
                acc[3] *= f * fb.w;
            }
            if constexpr (NORM) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= nq[rb].c * nk[cb].r[e];
            }
            frag_store(Pt, rb, cb, lane, acc);
        }
    }
}

template <int DK, int NW, bool NORM, int NL>
__global__ __launch_bounds__(64 * (NW + 2 + NL + (NORM ? 1 : 0))) void fused_chunk(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    __bf16* __restrict__ o, float* __restrict__ ST, int64_t T, int H, int NT, int DV, int gflags) {
    using L = FLayout<DK, NW>;
    using M = Mma<__bf16>;
    constexpr int VT = L::VT;
    constexpr int NKC = DK / 32;     // channel k-steps
    constexpr int NKT = FC / 32;     // token k-steps
    constexpr int CT = DK / 16;      // state tiles
    // With the gate prologue T is built by a solve and a recurrence wave (seven
    // waves at NW = 2); without it by one T wave fed by the P wave (six).
    constexpr bool SPLIT = NORM;
    // L2 warming from the loaders where they set the window (one compute wave,
    // eight workgroups per head: -7 % on the 1x32x32768 shape); with two
    // compute waves the prep waves set it and the extra loads cost 1-2 %.
    constexpr bool WARMING = !SPLIT && NW == 1;
    __shared__ __attribute__((aligned(16))) char smem[L::template total<SPLIT>()];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, col = lane & 15;
    const int NVT = DV / VT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = bid % NVT;
    const int64_t bh = bid / NVT;
    const int64_t b = bh / H, h = bh % H;
#define GDR_STAGE(n) (smem + ((n) % 3) * L::STAGE)
#define GDR_TPBUF(n) (smem + L::TP0 + ((n) & 1) * L::TPB)
#define GDR_QTILE(n) (smem + L::QR0 + ((n) & 1) * L::QB)
#define GDR_GTAB(n) (reinterpret_cast<float*>(smem + L::GT0 + ((n) % 3) * L::GSLOT))
#define GDR_LEN(n) ((int)((T - (int64_t)(n) * FC) < FC ? (T - (int64_t)(n) * FC) : FC))
#define GDR_ROW0(n) ((b * T + (int64_t)(n) * FC) * H + h)

    if (wave < NW) {
        // ---------------- compute ----------------
        const int vcol0 = vt * VT + 16 * wave;
        const int vcol = vcol0 + col;
        const FragOffsets<DK, VT> fo(lane, wave);
        const int olane = (col * H * DV + vcol0 + 4 * g4) * 2;   // byte offset of the lane's output piece
        f32x4 S[CT];
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            const int c0 = 32 * (mc >> 1) + 8 * g4 + 4 * (mc & 1);
            if (S0) x = *reinterpret_cast<const float4*>(S0 + (bh * DV + vcol) * DK + c0);
            S[mc] = f32x4{x.x, x.y, x.z, x.w};
        }
        // The start state must have landed before the loop: the compiler cannot
        // count loads across the loop's back edge, and a load pending at its entry
        // makes it wait for every memory operation at the first use of S in each
        // window, the previous window's output stores included.
#pragma unroll
        for (int mc = 0; mc < CT; ++mc) asm volatile("" ::"v"(S[mc]));
        // The state as a bf16 B operand, converted once per window (at its end):
        // it serves the next chunk's K S^T and Q S^T.
        M::frag sb[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) sb[s] = bfrag_acc<__bf16>(S, s);
        // K fragments (first half of the channel steps) of the chunk computed
        // next, read one window ahead (its stage is complete then and stays
        // untouched until after it is used).
        constexpr int NKP = NKC / 2;
        M::frag kn[FNB][NKP];
        // S Q^T of the chunk computed next (O^T tiles, rows = value columns),
        // made in the window before, where its Q tile is read anyway.
        f32x4 Oa[FNB];
        for (int w = -2; w < NT; ++w) {
            if (w == -1) {
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                    for (int s = 0; s < NKP; ++s) kn[mt][s] = fo.qkf(GDR_STAGE(0) + L::S_K, mt, s);
                M::frag qf[FNB][NKC];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                    for (int s = 0; s < NKC; ++s) qf[mt][s] = fo.qkf(GDR_QTILE(0), mt, s);
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt) Oa[mt] = zero4();
#pragma unroll
                for (int s = 0; s < NKC; ++s)
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) Oa[mt] = M::mma(sb[s], qf[mt][s], Oa[mt]);
            }
            if (w >= 0) {
                const int n = w;
                const char* st = GDR_STAGE(n);
                const char* tp = GDR_TPBUF(n);
                const int len = GDR_LEN(n);
                const float* tab = GDR_GTAB(n);

                // The window's work in phases; each phase first issues the LDS
                // reads of a later phase, so their latency is covered by MFMAs
                // (sched_barrier keeps the compiler from sinking reads to uses).
                // Phase 0: the other K fragments, V, decay factors.
                M::frag kr[FNB][NKC - NKP];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                    for (int s = NKP; s < NKC; ++s) kr[mt][s - NKP] = fo.qkf(st + L::S_K, mt, s);
                bf16x4 vv[FNB];
                float4 gm[FNB];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt) {
                    vv[mt] = fo.vf(st + L::S_V, mt);
                    gm[mt] = *reinterpret_cast<const float4*>(tab + (NORM ? L::G_GMK : L::G_GM) * FC + 16 * mt + 4 * g4);
                }
                // Phase 1: R = K S^T (rows = tokens) from the prefetched K fragments.
                f32x4 R[FNB];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt) R[mt] = zero4();
#pragma unroll
                for (int s = 0; s < NKC; ++s)
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt)
                        R[mt] = M::mma(s < NKP ? kn[mt][s] : kr[mt][s - NKP], sb[s], R[mt]);
                __builtin_amdgcn_sched_barrier(0);
                // T, read while R is finished on the VALU.
                M::frag tf[FNB][NKT];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                    for (int s = 0; s < NKT; ++s) tf[mt][s] = fo.tpf(tp + L::T_T, mt, s);
                __builtin_amdgcn_sched_barrier(0);
                // Phase 2: R = V - Diag(gamma) R;  D = (T + T_lo) R.
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt) {
                    R[mt][0] = (float)vv[mt][0] - gm[mt].x * R[mt][0];
                    R[mt][1] = (float)vv[mt][1] - gm[mt].y * R[mt][1];
                    R[mt][2] = (float)vv[mt][2] - gm[mt].z * R[mt][2];
                    R[mt][3] = (float)vv[mt][3] - gm[mt].w * R[mt][3];
                }
                M::frag rb[NKT];
#pragma unroll
                for (int s = 0; s < NKT; ++s) rb[s] = bfrag_acc<__bf16>(R, s);
                f32x4 D[FNB];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt) D[mt] = zero4();
#pragma unroll
                for (int s = 0; s < NKT; ++s)
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) D[mt] = M::mma(tf[mt][s], rb[s], D[mt]);
                __builtin_amdgcn_sched_barrier(0);
                // T's rounding residual, for chunks that take the pair (read once T's
                // fragments are consumed).
                const int pair = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(tp + L::T_FLAG));
                if (pair) {
                    M::frag tl[FNB][NKT];
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                        for (int s = 0; s < NKT; ++s) tl[mt][s] = fo.tpf(tp + L::T_L, mt, s);
#pragma unroll
                    for (int s = 0; s < NKT; ++s)
#pragma unroll
                        for (int mt = 0; mt < FNB; ++mt) D[mt] = M::mma(tl[mt][s], rb[s], D[mt]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // K^T fragments for the state update, the remaining decay factors.
                M::frag kh[CT][NKT];
#pragma unroll
                for (int mc = 0; mc < CT; ++mc)
#pragma unroll
                    for (int s = 0; s < NKT; ++s) kh[mc][s] = fo.ktf(st + L::S_K, mc, s);
                float4 gh[FNB];
#pragma unroll
                for (int mt = 0; mt < FNB; ++mt)
                    gh[mt] = *reinterpret_cast<const float4*>(tab + (NORM ? L::G_GHK : L::G_GH) * FC + 16 * mt + 4 * g4);
                const float gl = tab[L::G_GM * FC + FC - 1];
                __builtin_amdgcn_sched_barrier(0);
                // Phase 3: S^T <- gamma_last S^T + K^T (Diag(gamma_last / gamma) D).
                M::frag dsb[NKT];
                {
                    f32x4 Dsc[FNB];
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt)
                        Dsc[mt] = f32x4{D[mt][0] * gh[mt].x, D[mt][1] * gh[mt].y, D[mt][2] * gh[mt].z,
                                        D[mt][3] * gh[mt].w};
#pragma unroll
                    for (int s = 0; s < NKT; ++s) dsb[s] = bfrag_acc<__bf16>(Dsc, s);
                }
#pragma unroll
                for (int mc = 0; mc < CT; ++mc) S[mc] *= gl;
#pragma unroll
                for (int s = 0; s < NKT; ++s)
#pragma unroll
                    for (int mc = 0; mc < CT; ++mc) S[mc] = M::mma(kh[mc][s], dsb[s], S[mc]);
                __builtin_amdgcn_sched_barrier(0);
                // Phase 4: O^T = Diag-scaled S Q^T (made one window ahead) + D^T P^T,
                // with D as a bf16 pair as well.
                {
                    M::frag pf[FNB][NKT];
                    float gc[FNB];
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) {
#pragma unroll
                        for (int s = 0; s < NKT; ++s) pf[mt][s] = frag_load(tp + L::T_P, mt, s, lane);
                        gc[mt] = tab[(NORM ? L::G_GQ : L::G_GM) * FC + 16 * mt + col];
                    }
                    f32x4 Dl[FNB];
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) Dl[mt][e] = D[mt][e] - (float)(__bf16)D[mt][e];
                    M::frag db[NKT], dl[NKT];
#pragma unroll
                    for (int s = 0; s < NKT; ++s) {
                        db[s] = bfrag_acc<__bf16>(D, s);
                        dl[s] = bfrag_acc<__bf16>(Dl, s);
                    }
                    f32x4 Op[FNB];
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) Op[mt] = zero4();
#pragma unroll
                    for (int s = 0; s < NKT; ++s)
#pragma unroll
                        for (int mt = 0; mt < FNB; ++mt) Op[mt] = M::mma(db[s], pf[mt][s], Op[mt]);
                    if (pair) {
#pragma unroll
                        for (int s = 0; s < NKT; ++s)
#pragma unroll
                            for (int mt = 0; mt < FNB; ++mt) Op[mt] = M::mma(dl[s], pf[mt][s], Op[mt]);
                    }
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) Oa[mt] = Oa[mt] * gc[mt] + Op[mt];
                }
                // Output rows: lane (col, g4) of tile mt holds o[16mt + col][vcol0 + 4g4 + e]
                // (wave-uniform row base, per-lane 32-bit offset).
                char* ob = reinterpret_cast<char*>(o) + GDR_ROW0(n) * DV * 2;
                const int64_t tstride = (int64_t)16 * H * DV * 2;
                if (len == FC) {
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) {
                        const bf16x4 y = {(__bf16)Oa[mt][0], (__bf16)Oa[mt][1], (__bf16)Oa[mt][2], (__bf16)Oa[mt][3]};
                        *reinterpret_cast<bf16x4*>(ob + mt * tstride + olane) = y;
                    }
                } else {
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt) {
                        const bf16x4 y = {(__bf16)Oa[mt][0], (__bf16)Oa[mt][1], (__bf16)Oa[mt][2], (__bf16)Oa[mt][3]};
                        if (16 * mt + col < len) *reinterpret_cast<bf16x4*>(ob + mt * tstride + olane) = y;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // Phase 5: the next chunk's B operand of the state, its S Q^T and K fragments.
#pragma unroll
                for (int s = 0; s < NKC; ++s) sb[s] = bfrag_acc<__bf16>(S, s);
                if (n + 1 < NT) {
                    // (two row tiles at a time, to bound the live Q fragments)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        M::frag qf[2][NKC];
#pragma unroll
                        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                            for (int s = 0; s < NKC; ++s) qf[m2][s] = fo.qkf(GDR_QTILE(n + 1), 2 * half + m2, s);
#pragma unroll
                        for (int m2 = 0; m2 < 2; ++m2) Oa[2 * half + m2] = zero4();
#pragma unroll
                        for (int s = 0; s < NKC; ++s)
#pragma unroll
                            for (int m2 = 0; m2 < 2; ++m2)
                                Oa[2 * half + m2] = M::mma(sb[s], qf[m2][s], Oa[2 * half + m2]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int mt = 0; mt < FNB; ++mt)
#pragma unroll
                        for (int s = 0; s < NKP; ++s)
                            kn[mt][s] = fo.qkf(GDR_STAGE(n + 1) + L::S_K, mt, s);
                }
            }
            __syncthreads();
        }
        if (ST) {
#pragma unroll
            for (int mc = 0; mc < CT; ++mc) {
                const int c0 = 32 * (mc >> 1) + 8 * g4 + 4 * (mc & 1);
                *reinterpret_cast<float4*>(ST + (bh * DV + vcol) * DK + c0) =
                    make_float4(S[mc][0], S[mc][1], S[mc][2], S[mc][3]);
            }
        }
    } else if (wave == NW) {
        if constexpr (SPLIT) {
            // ---------------- prep P ----------------
            for (int w = -2; w < NT; ++w) {
                const int n = w + 1;
                if (n >= 0 && n < NT) prep_p<DK, NW, NORM, SPLIT>(smem, GDR_STAGE(n), GDR_QTILE(n), GDR_GTAB(n), GDR_TPBUF(n), n, lane);
                __syncthreads();
            }
        } else {
            // ---------------- prep T ----------------
            // The strictly upper tiles of T and P are zero in both buffers for good.
            for (int bf = 0; bf < 2; ++bf)
#pragma unroll
                for (int rb = 0; rb < FNB; ++rb)
#pragma unroll
                    for (int cb = rb + 1; cb < FNB; ++cb) {
                        tp_store(GDR_TPBUF(bf) + L::T_T, rb, cb, lane, zero4());
                        tp_store(GDR_TPBUF(bf) + L::T_L, rb, cb, lane, zero4());
                        frag_store(GDR_TPBUF(bf) + L::T_P, rb, cb, lane, zero4());
                    }
            for (int w = -2; w < NT; ++w) {
                const int n = w + 1;
                if (n >= 0 && n < NT) prep_t<DK, NW, NORM>(smem, GDR_STAGE(n), GDR_GTAB(n), GDR_TPBUF(n), n, lane);
                __syncthreads();
            }
        }
    } else if (wave == NW + 1) {
        if constexpr (SPLIT) {
            // ---------------- solve: diagonal blocks of T, one chunk ahead ----------------
            // Window w inverts the diagonal blocks of chunk c = w + 2 from K
            // fragments and gate values loaded from global memory in the window
            // before, and loads chunk c + 1's.
            bf16x8 kc[FNB][NKC];
            float la, bb;
            solve_loads<DK>(k, log_alpha, beta, GDR_ROW0(0), GDR_LEN(0), H, lane, kc, la, bb);
            // Nothing may enter the loop in flight: the compiler cannot count loads
            // across the loop's back edge, and a load pending at its entry would
            // make it wait for every load at the first use in each window, the new
            // prefetch included.  The empty asm reads the values, which places the
            // wait for them here.
    #pragma unroll
            for (int rb = 0; rb < FNB; ++rb)
    #pragma unroll
                for (int s = 0; s < NKC; ++s) asm volatile("" ::"v"(kc[rb][s]));
            asm volatile("" ::"v"(la), "v"(bb));
            for (int w = -2; w < NT; ++w) {
                const int c = w + 2;
                if (c < NT) {
                    bf16x8 kn[FNB][NKC];
                    float la1 = 0.f, bb1 = 0.f;
                    if (c + 1 < NT)
                        solve_loads<DK>(k, log_alpha, beta, GDR_ROW0(c + 1), GDR_LEN(c + 1), H, lane, kn, la1, bb1);
                    solve_diag<DK, NW, NORM>(smem, kc, la, bb, GDR_LEN(c), gflags,
                                             smem + L::XH + (c & 1) * L::XHB, lane);
                    // The prefetch has landed by now (a window of work after it
                    // was issued); the copies wait for it here.
                    if (c + 1 < NT) {
    #pragma unroll
                        for (int rb = 0; rb < FNB; ++rb)
    #pragma unroll
                            for (int s = 0; s < NKC; ++s) kc[rb][s] = kn[rb][s];
                        la = la1;
                        bb = bb1;
                    }
                }
                __syncthreads();
            }
        } else {
            // ---------------- prep P ----------------
            if (lane == 0) *reinterpret_cast<int*>(smem + L::FLAG) = 0;
            for (int w = -2; w < NT; ++w) {
                const int n = w + 1;
                if (n >= 0 && n < NT) prep_p<DK, NW, NORM, SPLIT>(smem, GDR_STAGE(n), GDR_QTILE(n), GDR_GTAB(n), GDR_TPBUF(n), n, lane);
                __syncthreads();
            }
        }
    } else if (SPLIT && wave == NW + 2 + NL) {
        if constexpr (SPLIT) {
            // ---------------- recurrence: off-diagonal blocks of T ----------------
            // The strictly upper tiles of T and P are zero in both buffers for good.
            for (int bf = 0; bf < 2; ++bf)
    #pragma unroll
                for (int rb = 0; rb < FNB; ++rb)
    #pragma unroll
                    for (int cb = rb + 1; cb < FNB; ++cb) {
                        tp_store(GDR_TPBUF(bf) + L::T_T, rb, cb, lane, zero4());
                        tp_store(GDR_TPBUF(bf) + L::T_L, rb, cb, lane, zero4());
                        frag_store(GDR_TPBUF(bf) + L::T_P, rb, cb, lane, zero4());
                    }
            for (int w = -2; w < NT; ++w) {
                const int n = w + 1;
                if (n >= 0 && n < NT)
                    recur_off<DK, NW, NORM>(GDR_STAGE(n), GDR_GTAB(n), smem + L::XH + (n & 1) * L::XHB,
                                            GDR_TPBUF(n), lane);
                __syncthreads();
            }
        }
    } else {
        // ---------------- loaders ----------------
        // Window w copies chunk c = w + 2 into its stage; loader 0 then builds
        // chunk c's gate table from gate values gathered one window earlier
        // (so nothing waits inside the window), and both gather chunk c + 1's.
        const int lw = wave - NW - 2;
        LoadOffsets<DK, NW, NL> lo;
        lo.set(FC, H, DV, vt, lw, lane);
        float la, bb;
        {
            const int64_t go = GDR_ROW0(0) + (int64_t)(lane < GDR_LEN(0) ? lane : GDR_LEN(0) - 1) * H;
            la = log_alpha[go];
            bb = beta[go];
        }
        // No load may be in flight at the loop entry (the compiler cannot count
        // loads across the back edge and would then wait for all of them, the
        // warming loads included, at each window's first use of la / bb).
        asm volatile("" ::"v"(la), "v"(bb));
        for (int w = -2; w < NT; ++w) {
            const int n = w + 2;
            if (n < NT) {
                const int len = GDR_LEN(n);
                if (len < FC) lo.set(len, H, DV, vt, lw, lane);   // ragged last chunk
                load_chunk<DK, NW, NL>(GDR_STAGE(n), GDR_QTILE(n), q, k, v, GDR_ROW0(n), DV, lo, lw);
                if (lw == 0) gate_table<DK, NW>(la, bb, len, lane, GDR_GTAB(n), gflags);
                if (n + 1 < NT) {
                    const int len1 = GDR_LEN(n + 1);
                    const int64_t go = GDR_ROW0(n + 1) + (int64_t)(lane < len1 ? lane : len1 - 1) * H;
                    la = log_alpha[go];
                    bb = beta[go];
                }
                if (WARMING && n + 1 < NT) {
                    warm_chunk<DK, NW>(smem + L::WARM, q, k, v, GDR_ROW0(n + 1), GDR_LEN(n + 1), H, DV, vt, lw,
                                       lane);
                    // copies and gathers landed; the warming loads (issued last) stay in flight
                    if (lw == 0) {
                        if constexpr (DK == 128) __builtin_amdgcn_s_waitcnt(0x0F72);   // vmcnt(2)
                        else __builtin_amdgcn_s_waitcnt(0x0F71);                       // vmcnt(1)
                    } else {
                        if constexpr (DK == 128) __builtin_amdgcn_s_waitcnt(0x0F73);   // vmcnt(3)
                        else __builtin_amdgcn_s_waitcnt(0x0F72);                       // vmcnt(2)
                    }
                } else {
                    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): copies and gathers landed
                }
            }
            __syncthreads();
        }
    }
#undef GDR_STAGE
#undef GDR_TPBUF
#undef GDR_QTILE
#undef GDR_LEN
#undef GDR_ROW0
#undef GDR_GTAB
}

// Loader waves per workgroup.  One loader (every role alone on a SIMD at
// NW = 1) measured 9 % slower on the 1x32x32768 shape and no faster at NW = 2.
template <int NW, bool NORM>
constexpr int kLoaders = 2;

template <int DK, int NW, bool NORM>
hipError_t launch_fused(const ChunkArgs& a) {
    const int NT = (int)((a.T + FC - 1) / FC);
    const int64_t grid = a.B * a.H * (a.dv / (16 * NW));
    constexpr int NL = kLoaders<NW, NORM>;
    hipLaunchKernelGGL((fused_chunk<DK, NW, NORM, NL>), dim3((unsigned)grid), dim3(64 * (NW + 2 + NL + (NORM ? 1 : 0))), 0,
                       a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.log_alpha, a.beta,
                       a.S0, (__bf16*)a.o, a.S_T, a.T, (int)a.H, NT, (int)a.dv,
                       (int)(a.prologue & kPrologueGates));
    return hipGetLastError();
}

template <bool NORM>
hipError_t launch_fused_n(const ChunkArgs& a) {
    // Two compute waves (32 value columns) per workgroup when that still
    // gives at least one workgroup per CU, otherwise one.
    const bool two = a.B * a.H * (a.dv / 32) >= 256;
    if (a.dk == 64) return two ? launch_fused<64, 2, NORM>(a) : launch_fused<64, 1, NORM>(a);
    return two ? launch_fused<128, 2, NORM>(a) : launch_fused<128, 1, NORM>(a);
}

}  // namespace

bool fused_chunk_supported(int64_t dk, int64_t chunk, bool bf16, bool channel) {
    return bf16 && !channel && chunk == FC && (dk == 64 || dk == 128);
}

hipError_t fused_chunk_launch(const ChunkArgs& a) {
    return (a.prologue & kPrologueL2NormQK) ? launch_fused_n<true>(a) : launch_fused_n<false>(a);
}

}  // namespace gdr
