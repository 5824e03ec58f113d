// Chunkwise KDA forward for chunk sizes other than 64 (C = 32 or 128), gfx950.
//
// The pages give the chunk size as 64 or 128 and tabulate 32 to 256 ("Linear
// Attention KDA Gating in a 3:1 Hybrid Architecture", section 3.1 and its
// chunk-size table); the result does not depend on C in exact arithmetic.
// The C = 64 kernels (kda_chunk.hip) are laid out for that one size; this
// path computes the same chunked algorithm for C in {32, 128} with every
// product on the fp32 matrix cores (the backward's building blocks), in
// three launches after the shared chunk-table kernel:
//
//   gprep_kernel   one 512-thread WG per (chunk, head).  The key channels are
//                  taken 32 at a time: b = cumsum(log2 alpha), Gamma.Q,
//                  (gamma/Gamma).K and gamma go to the record, and the
//                  16 x 16 tiles of A = StrictTril(Diag(beta) Kh Kb^T) and
//                  P = Tril(Qh Kb^T) accumulate in registers over the slices.
//                  T = (I + A)^-1 by 16 x 16 blocks (diagonal blocks by
//                  substitution, then T_ij = -T_ii sum_k A_ik T_kj), A and T
//                  kept as packed lower-triangular tiles (C = 128 fits in
//                  LDS); W = T Diag(beta) Kh and U = T Diag(beta) V, again 32
//                  columns at a time.
//   gchain_kernel  one 512-thread WG per (sequence, head, 16 value columns),
//                  chunks in order: writes the state entering each chunk and
//                  U' = U - W S, then S <- Diag(gamma) S + Kt^T U'; the final
//                  state at the end.
//   gout_kernel    one 512-thread WG per (chunk, head, 32 value columns):
//                  O = Qh S + P U'.
#include "kda_chunk.h"
#include "kda_common.h"
#include "kda_mm32.h"

namespace kda {
namespace {

using namespace mm32;

constexpr int kThreads = 512, kWaves = kThreads / 64;
constexpr int kSL = 32, kLS = kSL + 4;     // channel / value slice and its LDS row stride

// packed lower-triangular 16 x 16 tiles: tile (i, j), j <= i
__host__ __device__ constexpr int lt(int i, int j) { return i * (i + 1) / 2 + j; }

__device__ __forceinline__ void lt_decode(int idx, int& i, int& j) {
    i = 0;
    while (idx > i) {
        idx -= i + 1;
        ++i;
    }
    j = idx;
}

// Per-(head, chunk) fp32 record (byte offsets); rows are chunk-local tokens.
template <int DK, int DV, int C> struct GRec {
    static constexpr size_t CK = size_t(C) * DK * 4, CV = size_t(C) * DV * 4, CC = size_t(C) * C * 4;
    static constexpr size_t QH = 0;              // Gamma . Q                 [C][DK]
    static constexpr size_t KT = QH + CK;        // (gamma / Gamma) . K       [C][DK]
    static constexpr size_t W = KT + CK;         // T Diag(beta) (Gamma . K)  [C][DK]
    static constexpr size_t B = W + CK;          // b = cumsum(log2 alpha)     [C][DK]
    static constexpr size_t U = B + CK;          // T Diag(beta) V            [C][DV]
    static constexpr size_t P = U + CV;          // Tril(Qh Kb^T)             [C][C]
    static constexpr size_t GAM = P + CC;        // gamma                     [DK]
    static constexpr size_t SIN = GAM + size_t(DK) * 4;   // state entering  [DK][DV]
    static constexpr size_t UC = SIN + size_t(DK) * DV * 4;   // U - W S    [C][DV]
    static constexpr size_t END = UC + CV;
};

struct GParams {
    const void* q;
    const void* k;
    const void* v;
    const void* gate;
    const float* beta;
    const float* initial_state;
    float* final_state;
    void* o;
    const int32_t* ctrl;
    const int32_t* first;
    const int32_t* order;
    const int4* table;
    unsigned char* rec;
    size_t rec_bytes;
    int64_t gmax;
    int N, H;
};

__device__ __forceinline__ float* grec(const GParams& P, int h, int g, size_t off) {
    return reinterpret_cast<float*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
}

// ---------------------------------------------------------------------------
// gprep_kernel
// ---------------------------------------------------------------------------
template <int C> struct GPrepB {
    static constexpr int NB = C / 16, NLT = NB * (NB + 1) / 2, NS = kThreads / kSL;
    static constexpr int bytes = (3 * C * kLS + 2 * NLT * 256 + kWaves * 256 + 2 * C + NS * kSL + kSL) * 4;
};

template <int DK, int DV, int C, bool ABF16, int GATE>
__global__ __launch_bounds__(kThreads) void gprep_kernel(const GParams P) {
    using R = GRec<DK, DV, C>;
    constexpr int NTH = kThreads, NW = kWaves, SL = kSL, LS = kLS;
    constexpr int NB = GPrepB<C>::NB, NLT = GPrepB<C>::NLT, NS = GPrepB<C>::NS, SEG = C / NS;
    constexpr int NTASK = 2 * NLT, TW = (NTASK + NW - 1) / NW;
    constexpr bool GBF16 = GATE == KDA_GATE_SOFTPLUS_BF16;
    extern __shared__ float lds[];
    float* sKh = lds;                    // K -> Gamma.K; pass 2: K -> beta.Gamma.K, V -> beta.V   [C][LS]
    float* sKb = sKh + C * LS;           // gate -> log2 alpha -> K / Gamma; pass 2: b             [C][LS]
    float* sQ = sKb + C * LS;            // Q -> Gamma.Q                                         [C][LS]
    float* sA = sQ + C * LS;             // A, packed lower tiles                                [NLT][256]
    float* sT = sA + NLT * 256;          // T, packed lower tiles                                [NLT][256]
    float* sX = sT + NLT * 256;          // T-solve scratch, one tile per wave                   [NW][256]
    float* sBeta = sX + NW * 256;        // [C]
    float* sGs = sBeta + C;              // scalar gate per row                                   [C]
    float* sPart = sGs + C;              // scan segment sums                                     [NS][SL]
    float* sGam = sPart + NS * SL;       // gamma of the current slice                            [SL]

    const int H = P.H;
    const int h = blockIdx.x % H, g = blockIdx.x / H;
    if (g >= P.ctrl[0]) return;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), lane = lane_id(), i = lane & 15, j = lane >> 4;

    if (tid < C) {
        sBeta[tid] = tid < len ? P.beta[(row0 + tid) * H + h] : 0.f;
        if constexpr (GATE == KDA_GATE_SCALAR)
            sGs[tid] = tid < len ? static_cast<const float*>(P.gate)[(row0 + tid) * H + h] : 1.f;
    }
    float* gB = grec(P, h, g, R::B);
    float* gQh = grec(P, h, g, R::QH);
    float* gKt = grec(P, h, g, R::KT);
    float* gGam = grec(P, h, g, R::GAM);

    // ---- pass 1: per 32-channel slice, decay, Gamma-scaled operands, A and P tiles
    f4 acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = zero4();
    for (int cs = 0; cs < DK; cs += SL) {
        {
            Tok<ABF16, DK, SL, NTH, C> tk, tq;
            tk.load(P.k, row0, len, h, H, cs);
            tq.load(P.q, row0, len, h, H, cs);
            if constexpr (GATE != KDA_GATE_SCALAR) {
                Tok<GBF16, DK, SL, NTH, C> tg;
                tg.load(P.gate, row0, len, h, H, cs);
                tg.put(sKb, LS);
            }
            tk.put(sKh, LS);
            tq.put(sQ, LS);
        }
        __syncthreads();
        {   // log2 alpha per element (padding rows: 0), segment sums
            const int c = tid % SL, sg = tid / SL;
            float part = 0.f;
            for (int r = sg * SEG; r < sg * SEG + SEG; ++r) {
                float l2 = 0.f;
                if (r < len) {
                    if constexpr (GATE == KDA_GATE_SCALAR) l2 = __builtin_amdgcn_logf(sGs[r]);
                    else if constexpr (GBF16) l2 = log2_alpha_from_softplus_arg(sKb[r * LS + c]);
                    else l2 = __builtin_amdgcn_logf(sKb[r * LS + c]);
                }
                sKb[r * LS + c] = l2;
                part += l2;
            }
            sPart[sg * SL + c] = part;
        }
        __syncthreads();
        {   // b = cumsum(log2 alpha); Kh = 2^b K, Kb = 2^-b K, Qh = 2^b Q
            const int c = tid % SL, sg = tid / SL;
            float b = 0.f;
            for (int s2 = 0; s2 < sg; ++s2) b += sPart[s2 * SL + c];
            for (int r = sg * SEG; r < sg * SEG + SEG; ++r) {
                b += sKb[r * LS + c];
                const float G = __builtin_amdgcn_exp2f(b), Gi = __builtin_amdgcn_exp2f(-b);
                const float kv = sKh[r * LS + c];
                sKh[r * LS + c] = G * kv;
                sKb[r * LS + c] = Gi * kv;
                sQ[r * LS + c] *= G;
                gB[r * DK + cs + c] = b;
            }
            if (sg == NS - 1) gGam[cs + c] = sGam[c] = __builtin_amdgcn_exp2f(b);
        }
        __syncthreads();
        for (int idx = tid; idx < C * SL; idx += NTH) {
            const int r = idx / SL, c = idx % SL;
            gKt[r * DK + cs + c] = sGam[c] * sKb[r * LS + c];
            gQh[r * DK + cs + c] = sQ[r * LS + c];
        }
        // this slice's share of the A (Kh Kb^T) and P (Qh Kb^T) tiles
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int task = wave + NW * t;
            if (task >= NTASK) continue;
            int ti, tj;
            lt_decode(task % NLT, ti, tj);
            acc[t] = mm<SL, true, true>((task < NLT ? sKh : sQ) + ti * 16 * LS, LS, 1, sKb + tj * 16 * LS, 1, LS,
                                        acc[t]);
        }
        __syncthreads();
    }

    // ---- A tiles (strictly lower, row-scaled by beta) to LDS; P tiles to the record
    float* gP = grec(P, h, g, R::P);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int task = wave + NW * t;
        if (task >= NTASK) continue;
        int ti, tj;
        lt_decode(task % NLT, ti, tj);
        f4 x = acc[t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = ti * 16 + 4 * j + e, s = tj * 16 + i;
            if (task < NLT) x[e] = s < r ? sBeta[r] * x[e] : 0.f;
            else x[e] = s <= r ? x[e] : 0.f;
        }
        if (task < NLT) store_tile(sA + lt(ti, tj) * 256, 16, x);
        else store_tile(gP + ti * 16 * C + tj * 16, C, x);
    }
    for (int idx = tid; idx < (NB * NB - NLT) * 256; idx += NTH) {     // P above the diagonal
        int u = idx >> 8;
        const int e = idx & 255;
        int ti = 0, tj = 1;
        while (u >= NB - 1 - ti) {
            u -= NB - 1 - ti;
            ++ti;
        }
        tj = ti + 1 + u;
        gP[(ti * 16 + (e >> 4)) * C + tj * 16 + (e & 15)] = 0.f;
    }
    __syncthreads();

    // ---- T = (I + A)^-1 by 16 x 16 blocks
    if (wave < NB && lane < 16) {
        const float* a = sA + lt(wave, wave) * 256;
        const int col = lane;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = r == col ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) x -= a[r * 16 + s2] * t[s2];
            t[r] = x;
        }
        float* tt = sT + lt(wave, wave) * 256;
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r * 16 + col] = t[r];
    }
    __syncthreads();
    for (int d = 1; d < NB; ++d) {
        if (wave < NB - d) {
            const int bi = wave + d, bj = wave;
            f4 x = zero4();
            for (int bk = bj; bk < bi; ++bk)
                x = mm<16, true, false>(sA + lt(bi, bk) * 256, 16, 1, sT + lt(bk, bj) * 256, 16, 1, x);
            store_tile(sX + wave * 256, 16, x);
        }
        __syncthreads();
        if (wave < NB - d) {
            const int bi = wave + d, bj = wave;
            const f4 y = mm<16, true, false>(sT + lt(bi, bi) * 256, 16, 1, sX + wave * 256, 16, 1, zero4());
            store_tile(sT + lt(bi, bj) * 256, 16, -y);
        }
        __syncthreads();
    }

    // ---- pass 2: W = T Diag(beta) Kh and U = T Diag(beta) V, 32 columns at a time
    float* gW = grec(P, h, g, R::W);
    float* gU = grec(P, h, g, R::U);
    for (int cs = 0; cs < DK + DV; cs += SL) {
        const bool isw = cs < DK;
        const int c0 = isw ? cs : cs - DK;
        if (isw) {
            Tok<ABF16, DK, SL, NTH, C> tk;
            Blk<C, SL, NTH> bb;
            tk.load(P.k, row0, len, h, H, c0);
            bb.load(gB + c0, DK);
            tk.put(sKh, LS);
            bb.put(sKb, LS);
        } else {
            Tok<ABF16, DV, SL, NTH, C> tv;
            tv.load(P.v, row0, len, h, H, c0);
            tv.put(sKh, LS);
        }
        __syncthreads();
        for (int idx = tid; idx < C * SL; idx += NTH) {
            const int r = idx / SL, c = idx % SL;
            const float sc = isw ? __builtin_amdgcn_exp2f(sKb[r * LS + c]) * sBeta[r] : sBeta[r];
            sKh[r * LS + c] *= sc;
        }
        __syncthreads();
        for (int t = wave; t < NB * (SL / 16); t += NW) {
            const int mb = t / (SL / 16), nb = t % (SL / 16);
            f4 x = zero4();
            for (int kb = 0; kb <= mb; ++kb)
                x = mm<16, true, false>(sT + lt(mb, kb) * 256, 16, 1, sKh + kb * 16 * LS + nb * 16, LS, 1, x);
            if (isw) store_tile(gW + mb * 16 * DK + c0 + nb * 16, DK, x);
            else store_tile(gU + mb * 16 * DV + c0 + nb * 16, DV, x);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// gchain_kernel: wave w holds state row block w (and w + 8); the C x 16
// product U' = U - W S is split over the waves: row block w % (C/16), part
// w / (C/16) of the d_k reduction, the parts handed to part 0 through LDS.
// ---------------------------------------------------------------------------
template <int DK, int C> struct GChainB {
    static constexpr int LK = Ld<DK>::value, NSPLIT = kWaves / (C / 16);
    static constexpr int bytes = (2 * C * LK + DK * L16 + C * L16 + (NSPLIT - 1) * C * L16 + DK) * 4;
};

template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void gchain_kernel(const GParams P) {
    using R = GRec<DK, DV, C>;
    constexpr int NTH = kThreads, NW = kWaves, LK = GChainB<DK, C>::LK, NT = DV / 16;
    constexpr int NB = C / 16, NSPLIT = GChainB<DK, C>::NSPLIT, KP = DK / NSPLIT;
    constexpr int NRB = DK / 16, RBW = (NRB + NW - 1) / NW;
    extern __shared__ float lds[];
    float* sW = lds;                 // [C][LK]
    float* sKt = sW + C * LK;        // [C][LK]
    float* sS = sKt + C * LK;        // [DK][16]
    float* sU = sS + DK * L16;       // [C][16]
    float* sPart = sU + C * L16;     // [NSPLIT - 1][C][16]
    float* sGam = sPart + (NSPLIT - 1) * C * L16;   // [DK]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int n = P.order[pair / P.H], h = pair % P.H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = wave_id(), j = lane_id() >> 4;
    const int c0 = tile * 16;
    const int mb = wave % NB, part = wave / NB;
    const size_t sbase = (static_cast<size_t>(n) * P.H + h) * DK * DV;

    f4 S[RBW];
    for (int u = 0; u < RBW; ++u) {
        const int rb = wave + NW * u;
        S[u] = (P.initial_state && rb < NRB) ? load_tile(P.initial_state + sbase + rb * 16 * DV + c0, DV) : zero4();
    }
    Blk<C, DK, NTH> nW, nKt;
    f4 nU = zero4();
    float nGam = 0.f;
    auto fetch = [&](int g) {
        nW.load(grec(P, h, g, R::W), DK);
        nKt.load(grec(P, h, g, R::KT), DK);
        if (part == 0) nU = load_tile(grec(P, h, g, R::U) + mb * 16 * DV + c0, DV);
        if (threadIdx.x < DK) nGam = grec(P, h, g, R::GAM)[threadIdx.x];
    };
    if (g0 < g1) fetch(g0);
    for (int g = g0; g < g1; ++g) {
        nW.put(sW, LK);
        nKt.put(sKt, LK);
        const f4 uu = nU;
        if (threadIdx.x < DK) sGam[threadIdx.x] = nGam;
        float* gS = grec(P, h, g, R::SIN);
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(sS + rb * 16 * L16, L16, S[u]);
            store_tile(gS + rb * 16 * DV + c0, DV, S[u]);
        }
        __syncthreads();
        if (g + 1 < g1) fetch(g + 1);
        // U' = U - W S
        const f4 x = mm<KP, true, false>(sW + mb * 16 * LK + part * KP, LK, 1, sS + part * KP * L16, L16, 1, zero4());
        if (part) store_tile(sPart + ((part - 1) * C + mb * 16) * L16, L16, x);
        __syncthreads();
        if (part == 0) {
            f4 uc = uu - x;
#pragma unroll
            for (int p2 = 1; p2 < NSPLIT; ++p2) uc -= load_tile(sPart + ((p2 - 1) * C + mb * 16) * L16, L16);
            store_tile(sU + mb * 16 * L16, L16, uc);
            store_tile(grec(P, h, g, R::UC) + mb * 16 * DV + c0, DV, uc);
        }
        __syncthreads();
        // S <- Diag(gamma) S + Kt^T U'
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            f4 sv = S[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] *= sGam[rb * 16 + 4 * j + e];
            S[u] = mm<C, false, false>(sKt + rb * 16, 1, LK, sU, L16, 1, sv);
        }
        __syncthreads();
    }
    if (P.final_state) {
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(P.final_state + sbase + rb * 16 * DV + c0, DV, S[u]);
        }
    }
}

// ---------------------------------------------------------------------------
// gout_kernel: O[:, 32 columns] = Qh S + P U' for one (chunk, head).
// ---------------------------------------------------------------------------
template <int DK, int C> struct GOutB {
    static constexpr int LK = Ld<DK>::value, NB = C / 16, NLT = NB * (NB + 1) / 2;
    static constexpr int bytes = (C * LK + DK * kLS + NLT * 256 + C * kLS) * 4;
};

template <int DK, int DV, int C, bool OBF16>
__global__ __launch_bounds__(kThreads) void gout_kernel(const GParams P) {
    using R = GRec<DK, DV, C>;
    constexpr int NTH = kThreads, NW = kWaves, LK = GOutB<DK, C>::LK, SL = kSL, LS = kLS;
    constexpr int NB = GOutB<DK, C>::NB, NLT = GOutB<DK, C>::NLT, NSV = DV / SL;
    constexpr int PIT = (NLT * 256 + NTH - 1) / NTH;
    extern __shared__ float lds[];
    float* sQh = lds;                // [C][LK]
    float* sS = sQh + C * LK;        // S[:, slice]   [DK][LS]
    float* sP = sS + DK * LS;        // P, packed lower tiles [NLT][256]
    float* sU = sP + NLT * 256;      // U'[:, slice]  [C][LS]

    const int H = P.H;
    const int sv = blockIdx.x % NSV, gh = blockIdx.x / NSV;
    const int h = gh % H, g = gh / H;
    if (g >= P.ctrl[0]) return;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), i = lane_id() & 15, j = lane_id() >> 4;
    const int s0 = sv * SL;

    {
        Blk<C, DK, NTH> bq;
        Blk<DK, SL, NTH> bs;
        Blk<C, SL, NTH> bu;
        float pv[PIT];
        bq.load(grec(P, h, g, R::QH), DK);
        bs.load(grec(P, h, g, R::SIN) + s0, DV);
        bu.load(grec(P, h, g, R::UC) + s0, DV);
        const float* gP = grec(P, h, g, R::P);
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
            const int idx = tid + it * NTH;
            if (idx < NLT * 256) {
                int ti, tj;
                lt_decode(idx >> 8, ti, tj);
                const int e = idx & 255;
                pv[it] = gP[(ti * 16 + (e >> 4)) * C + tj * 16 + (e & 15)];
            }
        }
        bq.put(sQh, LK);
        bs.put(sS, LS);
        bu.put(sU, LS);
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
            const int idx = tid + it * NTH;
            if (idx < NLT * 256) sP[idx] = pv[it];
        }
    }
    __syncthreads();
    for (int t = wave; t < NB * (SL / 16); t += NW) {
        const int mb = t / (SL / 16), nb = t % (SL / 16);
        f4 x = mm<DK, true, false>(sQh + mb * 16 * LK, LK, 1, sS + nb * 16, LS, 1, zero4());
        for (int kb = 0; kb <= mb; ++kb)
            x = mm<16, true, false>(sP + lt(mb, kb) * 256, 16, 1, sU + kb * 16 * LS + nb * 16, LS, 1, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = mb * 16 + 4 * j + e;
            if (r < len)
                store_out<OBF16>(P.o, (static_cast<size_t>(row0 + r) * H + h) * DV + s0 + nb * 16 + i, x[e]);
        }
    }
}

template <typename F>
hipError_t set_lds(F* kfn, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int DK, int DV, int C, bool ABF16, bool OBF16, int GATE>
hipError_t launch_typed(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    if (GRec<DK, DV, C>::END > pl.rec_bytes) return hipErrorInvalidValue;
    GParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.beta = a.beta;
    p.initial_state = a.initial_state; p.final_state = a.final_state; p.o = a.o;
    p.ctrl = reinterpret_cast<const int32_t*>(ws + pl.off_ctrl);
    p.first = reinterpret_cast<const int32_t*>(ws + pl.off_first);
    p.order = reinterpret_cast<const int32_t*>(ws + pl.off_order);
    p.table = reinterpret_cast<const int4*>(ws + pl.off_table);
    p.rec = ws + pl.off_rec;
    p.rec_bytes = pl.rec_bytes;
    p.gmax = pl.gmax;
    p.N = pl.N;
    p.H = pl.H;

    hipError_t e = launch_chunk_plan(pl, a.cu_seqlens, a.workspace, stream);
    if (e != hipSuccess) return e;
    const unsigned chunk_blocks = static_cast<unsigned>(pl.gmax * pl.H);
    const int64_t pairs = static_cast<int64_t>(pl.N) * pl.H;
    const unsigned chain_blocks = static_cast<unsigned>((pairs + 7) / 8 * 8 * (DV / 16));
    if (chunk_blocks > 0) {
        auto k1 = gprep_kernel<DK, DV, C, ABF16, GATE>;
        constexpr int l1 = GPrepB<C>::bytes;
        if ((e = set_lds(k1, l1)) != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(chunk_blocks), dim3(kThreads), l1, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (chain_blocks > 0) {
        auto k2 = gchain_kernel<DK, DV, C>;
        constexpr int l2 = GChainB<DK, C>::bytes;
        if ((e = set_lds(k2, l2)) != hipSuccess) return e;
        hipLaunchKernelGGL(k2, dim3(chain_blocks), dim3(kThreads), l2, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (chunk_blocks > 0) {
        auto k3 = gout_kernel<DK, DV, C, OBF16>;
        constexpr int l3 = GOutB<DK, C>::bytes;
        if ((e = set_lds(k3, l3)) != hipSuccess) return e;
        hipLaunchKernelGGL(k3, dim3(chunk_blocks * (DV / kSL)), dim3(kThreads), l3, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, int C, bool ABF16, bool OBF16>
hipError_t launch_gate(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (a.gate_kind == KDA_GATE_SOFTPLUS_BF16)
        return launch_typed<DK, DV, C, ABF16, OBF16, KDA_GATE_SOFTPLUS_BF16>(pl, a, stream);
    if (a.gate_kind == KDA_GATE_SCALAR) return launch_typed<DK, DV, C, ABF16, OBF16, KDA_GATE_SCALAR>(pl, a, stream);
    return launch_typed<DK, DV, C, ABF16, OBF16, KDA_GATE_ALPHA>(pl, a, stream);
}

template <int DK, int DV, int C>
hipError_t launch_types(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (!a.act_bf16) return launch_gate<DK, DV, C, false, false>(pl, a, stream);
    if (a.out_bf16) return launch_gate<DK, DV, C, true, true>(pl, a, stream);
    return launch_gate<DK, DV, C, true, false>(pl, a, stream);
}

template <int DK, int DV>
hipError_t launch_c(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (pl.C == 32) return launch_types<DK, DV, 32>(pl, a, stream);
    if (pl.C == 128) return launch_types<DK, DV, 128>(pl, a, stream);
    return hipErrorInvalidValue;
}

template <int DK, int DV>
size_t rec_end(int c) {
    return c == 32 ? GRec<DK, DV, 32>::END : c == 128 ? GRec<DK, DV, 128>::END : GRec<DK, DV, 64>::END;
}

}  // namespace

size_t generic_record_bytes(int Dk, int Dv, int chunk_size) {
    if (Dk == 128 && Dv == 128) return rec_end<128, 128>(chunk_size);
    if (Dk == 64 && Dv == 64) return rec_end<64, 64>(chunk_size);
    if (Dk == 128 && Dv == 64) return rec_end<128, 64>(chunk_size);
    return rec_end<64, 128>(chunk_size);
}

hipError_t launch_chunk_fwd_generic(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (pl.Dk == 128 && pl.Dv == 128) return launch_c<128, 128>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 64) return launch_c<64, 64>(pl, a, stream);
    if (pl.Dk == 128 && pl.Dv == 64) return launch_c<128, 64>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 128) return launch_c<64, 128>(pl, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
