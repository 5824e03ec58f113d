// Chunkwise KDA forward for chunk sizes other than 64 (C = 32 or 128), gfx950.
//
// The pages give the chunk size as 64 or 128 and tabulate 32 to 256 ("Linear
// Attention KDA Gating in a 3:1 Hybrid Architecture", section 3.1 and its
// chunk-size table); the result does not depend on C in exact arithmetic.
// The C = 64 kernels (kda_chunk.hip) are laid out for that one size; this
// path computes the same chunked algorithm for C in {32, 128} with every
// product on the fp32 matrix cores (the backward's building blocks), in
// three launches after the shared chunk-table kernel (two at C = 32):
//
//   gprep_kernel   one WG per (chunk, head), 512 threads (1024 at C = 128).  The key channels are
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
//                  chunks in order: U' = U - W S, then S <- Diag(gamma) S +
//                  Kt^T U'; the final state at the end.  At C = 128 the state
//                  entering each chunk and U' go to the record for gout; at
//                  C = 32 the chain forms O = Qh S + P U' itself.
//   gout_kernel    (C = 128) one 512-thread WG per (chunk, head, 32 value
//                  columns): O = Qh S + P U'.
#include <type_traits>

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

// Blk for an fp16 source (ROWS x NC, source row stride sld halves): four
// halves per 8-byte load, widened to fp32 on the way into LDS.
template <int ROWS, int NC, int NTH>
struct BlkH {
    static constexpr int V4 = NC / 4, N = ROWS * V4, IT = (N + NTH - 1) / NTH;
    h4 t[IT];
    __device__ __forceinline__ void load(const _Float16* src, int sld) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N)
                t[it] = *reinterpret_cast<const h4*>(src + static_cast<size_t>(idx / V4) * sld + (idx % V4) * 4);
        }
    }
    __device__ __forceinline__ void put(float* dst, int ld) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N)
                *reinterpret_cast<f4*>(dst + (idx / V4) * ld + (idx % V4) * 4) =
                    f4{static_cast<float>(t[it][0]), static_cast<float>(t[it][1]),
                       static_cast<float>(t[it][2]), static_cast<float>(t[it][3])};
        }
    }
};

// store_tile into fp16 memory
__device__ __forceinline__ void store_tile_h(_Float16* p, int ld, f4 v) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[(4 * j + e) * ld + i] = static_cast<_Float16>(v[e]);
}

// Per-(head, chunk) fp32 record (byte offsets); rows are chunk-local tokens.
// With 16-bit activations (H16) the state entering the chunk and U' -- the
// chain's outputs for the output pass -- are kept in fp16 (relative rounding
// 2^-11, against the 2e-2 x RMS bar of those inputs; 64 KiB less per (chunk,
// head) of state at d = 128).
template <int DK, int DV, int C, bool H16 = false> struct GRec {
    static constexpr size_t SE = H16 ? 2 : 4;    // bytes per element of SIN and UC
    static constexpr size_t CK = size_t(C) * DK * 4, CV = size_t(C) * DV * 4, CC = size_t(C) * C * 4;
    static constexpr size_t QH = 0;              // Gamma . Q                 [C][DK]
    static constexpr size_t KT = QH + CK;        // (gamma / Gamma) . K       [C][DK]
    static constexpr size_t W = KT + CK;         // T Diag(beta) (Gamma . K)  [C][DK]
    static constexpr size_t B = W + CK;          // b = cumsum(log2 alpha)     [C][DK]  (general form: its W pass reads it back)
    static constexpr size_t U = B + CK;          // T Diag(beta) V            [C][DV]
    static constexpr size_t P = U + CV;          // Tril(Qh Kb^T)             [C][C]
    static constexpr size_t GAM = P + CC;        // gamma                     [DK]
    // the chain's outputs for the output pass; at C = 32 the chain writes O
    // itself (FUSED) and the record ends before them
    static constexpr bool FUSED = C <= 32;
    static constexpr size_t SIN = GAM + size_t(DK) * 4;   // state entering  [DK][DV]
    static constexpr size_t UC = SIN + size_t(DK) * DV * SE;  // U - W S    [C][DV]
    static constexpr size_t END = FUSED ? SIN : UC + size_t(C) * DV * SE;
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
    int32_t* nslow;   // length of the general-form list (zeroed by the chunk table)
    int32_t* slow;    // general-form list: g * H + h of each (chunk, head) that takes it
};

__device__ __forceinline__ float* grec(const GParams& P, int h, int g, size_t off) {
    return reinterpret_cast<float*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
}

// ---------------------------------------------------------------------------
// gprep_kernel
// ---------------------------------------------------------------------------
// Threads of a preparation workgroup: at C = 128 its 140 KB of LDS leave one
// workgroup per CU, so it runs sixteen waves instead of eight.
template <int C> struct GPrepT {
    static constexpr int threads = C >= 128 ? 1024 : kThreads;
};

template <int C> struct GPrepB {
    static constexpr int NW = GPrepT<C>::threads / 64;
    static constexpr int NB = C / 16, NLT = NB * (NB + 1) / 2, NS = GPrepT<C>::threads / kSL;
    // the last region: the direct form's scan segment sums [NS][SL] and gamma
    // of the slice [SL], or the general form's tile totals [NB][SL]
    static constexpr int AUX = NS * kSL + kSL > NB * kSL ? NS * kSL + kSL : NB * kSL;
    static constexpr int bytes = (3 * C * kLS + 2 * NLT * 256 + NW * 256 + 2 * C + AUX) * 4;
};

// FAST: the direct form (one cumulative log2 sum per channel over the chunk;
// Kh = 2^b K, Kb = 2^-b K, Qh = 2^b Q in plain products), for every (chunk,
// head); one in which some channel decays below 2^-64 over the chunk is
// listed at the end for the general form (!FAST), whose decay factors are
// all 2^x with x <= 0.  Both write the same record.
template <int DK, int DV, int C, bool ABF16, int GATE, bool FAST>
__device__ __forceinline__ void gprep_body(const GParams& P, const int blk) {
    using R = GRec<DK, DV, C>;
    constexpr int NTH = GPrepT<C>::threads, NW = NTH / 64, SL = kSL, LS = kLS;
    constexpr int NB = GPrepB<C>::NB, NLT = GPrepB<C>::NLT;
    constexpr int NS = GPrepB<C>::NS, SEG = C / NS;   // direct form: scan segments
    constexpr int NTASK = 2 * NLT;        // direct form: A and P tiles as separate tasks
    constexpr int TW = FAST ? (NTASK + NW - 1) / NW : (NLT + NW - 1) / NW;
    constexpr bool GBF16 = GATE == KDA_GATE_SOFTPLUS_BF16;
    extern __shared__ float lds[];
    float* sK = lds;                     // K; pass 2: beta.Gamma.K, beta.V                      [C][LS]
    float* sB = sK + C * LS;             // gate -> b inside each 16-token tile; pass 2: b      [C][LS]
    float* sQ = sB + C * LS;             // Q                                                  [C][LS]
    float* sA = sQ + C * LS;             // A, packed lower tiles                                [NLT][256]
    float* sT = sA + NLT * 256;          // T, packed lower tiles                                [NLT][256]
    float* sX = sT + NLT * 256;          // T-solve scratch, one tile per wave                   [NW][256]
    float* sBeta = sX + NW * 256;        // [C]
    float* sGs = sBeta + C;              // scalar gate per row                                   [C]
    float* sTot = sGs + C;               // general: log2 alpha summed over each 16-token tile   [NB][SL]
    [[maybe_unused]] float* sPart = sGs + C;          // direct: scan segment sums   [NS][SL]
    [[maybe_unused]] float* sGam = sPart + NS * SL;   // direct: gamma of the slice  [SL]

    const int H = P.H;
    const int h = blk % H, g = blk / H;
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

    // direct form: log2 alpha of the gate slice staged in sB, per element
    // (padding rows: 0), and the sums of each thread's segment of rows into
    // sPart; b is then the running sum over the segments before and the rows
    // of the thread's own (the same operations in both passes, so the same b)
    [[maybe_unused]] auto log2_segments = [&]() {
        const int c = tid % SL, sg = tid / SL;
        float part = 0.f;
        for (int r = sg * SEG; r < sg * SEG + SEG; ++r) {
            float l2 = 0.f;
            if (r < len) {
                if constexpr (GATE == KDA_GATE_SCALAR) l2 = __builtin_amdgcn_logf(sGs[r]);
                else if constexpr (GBF16) l2 = log2_alpha_from_softplus_arg(sB[r * LS + c]);
                else l2 = __builtin_amdgcn_logf(sB[r * LS + c]);
            }
            sB[r * LS + c] = l2;
            part += l2;
        }
        sPart[sg * SL + c] = part;
        __syncthreads();
    };
    float* gP = grec(P, h, g, R::P);
    [[maybe_unused]] bool strong = false;   // direct form: some channel of this lane's decays below 2^-64
    if constexpr (FAST) {
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
                    tg.put(sB, LS);
                }
                tk.put(sK, LS);
                tq.put(sQ, LS);
            }
            __syncthreads();
            log2_segments();
            {   // b = cumsum(log2 alpha); Kh = 2^b K, Kb = 2^-b K, Qh = 2^b Q
                const int c = tid % SL, sg = tid / SL;
                float b = 0.f;
                for (int s2 = 0; s2 < sg; ++s2) b += sPart[s2 * SL + c];
                for (int r = sg * SEG; r < sg * SEG + SEG; ++r) {
                    b += sB[r * LS + c];
                    const float G = __builtin_amdgcn_exp2f(b), Gi = __builtin_amdgcn_exp2f(-b);
                    const float kv = sK[r * LS + c];
                    sK[r * LS + c] = G * kv;
                    sB[r * LS + c] = Gi * kv;
                    sQ[r * LS + c] *= G;
                }
                if (sg == NS - 1) {
                    gGam[cs + c] = sGam[c] = __builtin_amdgcn_exp2f(b);
                    strong = strong || b < -64.f;     // (NaN stays here and propagates)
                }
            }
            __syncthreads();
            for (int idx = tid; idx < C * SL; idx += NTH) {
                const int r = idx / SL, c = idx % SL;
                gKt[r * DK + cs + c] = sGam[c] * sB[r * LS + c];
                gQh[r * DK + cs + c] = sQ[r * LS + c];
            }
            // this slice's share of the A (Kh Kb^T) and P (Qh Kb^T) tiles
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int task = wave + NW * t;
                if (task >= NTASK) continue;
                int ti, tj;
                lt_decode(task % NLT, ti, tj);
                acc[t] = mm<SL, true, true>((task < NLT ? sK : sQ) + ti * 16 * LS, LS, 1, sB + tj * 16 * LS, 1, LS,
                                            acc[t]);
            }
            __syncthreads();
        }

        // ---- A tiles (strictly lower, row-scaled by beta) to LDS; P tiles to the record
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
    } else {
        // ---- pass 1: per 32-channel slice, decay, Gamma-scaled operands, A and P tiles.
        // Every decay factor is 2^x with x <= 0 (decayed_tile in kda_mm32.h):
        // cumulative sums restart at each 16-token tile, and products that cross
        // tiles add the totals of the tiles in between, so nothing overflows.
        f4 accA[TW], accP[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) accA[t] = accP[t] = zero4();
        for (int cs = 0; cs < DK; cs += SL) {
            {
                Tok<ABF16, DK, SL, NTH, C> tk, tq;
                tk.load(P.k, row0, len, h, H, cs);
                tq.load(P.q, row0, len, h, H, cs);
                if constexpr (GATE != KDA_GATE_SCALAR) {
                    Tok<GBF16, DK, SL, NTH, C> tg;
                    tg.load(P.gate, row0, len, h, H, cs);
                    tg.put(sB, LS);
                }
                tk.put(sK, LS);
                tq.put(sQ, LS);
            }
            __syncthreads();
            {   // b = cumulative log2 alpha inside each tile (padding rows add 0).  A
                // gate below 2^-150 counts as 2^-150: every fp32 factor that spans it
                // is zero either way.
                const int c = tid % SL, t = tid / SL;
                if (t < NB) {
                    float b = 0.f;
                    for (int r = 16 * t; r < 16 * t + 16; ++r) {
                        float l2 = 0.f;
                        if (r < len) {
                            if constexpr (GATE == KDA_GATE_SCALAR) l2 = __builtin_amdgcn_logf(sGs[r]);
                            else if constexpr (GBF16) l2 = log2_alpha_from_softplus_arg(sB[r * LS + c]);
                            else l2 = __builtin_amdgcn_logf(sB[r * LS + c]);
                            l2 = fmaxf(l2, -150.f);
                        }
                        b += l2;
                        sB[r * LS + c] = b;
                    }
                    sTot[t * SL + c] = b;
                }
            }
            __syncthreads();
            // record: b from the chunk start, Gamma.Q = 2^b Q, (gamma / Gamma).K and
            // gamma; with pre / suf the totals of the tiles before / after the row's:
            //   b = pre + b_t(r),  log2(gamma / Gamma_r) = T_t - b_t(r) + suf
            for (int idx = tid; idx < C * SL; idx += NTH) {
                const int r = idx / SL, c = idx % SL, t = r / 16;
                float pre = 0.f, suf = 0.f;
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const float x = sTot[u * SL + c];
                    if (u < t) pre += x;
                    else if (u > t) suf += x;
                }
                const float bl = sB[r * LS + c];
                const float b = pre + bl;
                gB[r * DK + cs + c] = b;
                gQh[r * DK + cs + c] = sQ[r * LS + c] * __builtin_amdgcn_exp2f(b);
                gKt[r * DK + cs + c] = sK[r * LS + c] * __builtin_amdgcn_exp2f(sTot[t * SL + c] - bl + suf);
            }
            if (tid < SL) {
                float tot = 0.f;
#pragma unroll
                for (int u = 0; u < NB; ++u) tot += sTot[u * SL + tid];
                gGam[cs + tid] = __builtin_amdgcn_exp2f(tot);
            }
            // this slice's share of the tiles of A (K-hat K-bar^T) and P (Q-hat K-bar^T)
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int task = wave + NW * t;
                if (task >= NLT) continue;
                int ti, tj;
                lt_decode(task, ti, tj);
                decayed_tile<SL / 16, true, true>(sK, sQ, sK, sB, sTot, LS, SL, ti, tj, accA[t], accP[t]);
            }
            __syncthreads();
        }

        // ---- A tiles (strictly lower, row-scaled by beta) to LDS; P tiles to the record
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int task = wave + NW * t;
            if (task >= NLT) continue;
            int ti, tj;
            lt_decode(task, ti, tj);
            f4 xa = accA[t], xp = accP[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = ti * 16 + 4 * j + e, s = tj * 16 + i;
                xa[e] = s < r ? sBeta[r] * xa[e] : 0.f;
                xp[e] = s <= r ? xp[e] : 0.f;
            }
            store_tile(sA + lt(ti, tj) * 256, 16, xa);
            store_tile(gP + ti * 16 * C + tj * 16, C, xp);
        }
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
            tk.load(P.k, row0, len, h, H, c0);
            if constexpr (FAST) {
                // b again from the gate (not stored: 16 bytes per token and
                // channel written and read back)
                if constexpr (GATE != KDA_GATE_SCALAR) {
                    Tok<GBF16, DK, SL, NTH, C> tg;
                    tg.load(P.gate, row0, len, h, H, c0);
                    tg.put(sB, LS);
                }
            } else {
                Blk<C, SL, NTH> bb;
                bb.load(gB + c0, DK);
                bb.put(sB, LS);
            }
            tk.put(sK, LS);
        } else {
            Tok<ABF16, DV, SL, NTH, C> tv;
            tv.load(P.v, row0, len, h, H, c0);
            tv.put(sK, LS);
        }
        __syncthreads();
        if (FAST && isw) {
            log2_segments();
            const int c = tid % SL, sg = tid / SL;
            float b = 0.f;
            for (int s2 = 0; s2 < sg; ++s2) b += sPart[s2 * SL + c];
            for (int r = sg * SEG; r < sg * SEG + SEG; ++r) {
                b += sB[r * LS + c];
                sK[r * LS + c] *= __builtin_amdgcn_exp2f(b) * sBeta[r];
            }
        } else {
            for (int idx = tid; idx < C * SL; idx += NTH) {
                const int r = idx / SL, c = idx % SL;
                const float sc = isw ? __builtin_amdgcn_exp2f(sB[r * LS + c]) * sBeta[r] : sBeta[r];
                sK[r * LS + c] *= sc;
            }
        }
        __syncthreads();
        for (int t = wave; t < NB * (SL / 16); t += NW) {
            const int mb = t / (SL / 16), nb = t % (SL / 16);
            f4 x = zero4();
            for (int kb = 0; kb <= mb; ++kb)
                x = mm<16, true, false>(sT + lt(mb, kb) * 256, 16, 1, sK + kb * 16 * LS + nb * 16, LS, 1, x);
            if (isw) store_tile(gW + mb * 16 * DK + c0 + nb * 16, DK, x);
            else store_tile(gU + mb * 16 * DV + c0 + nb * 16, DV, x);
        }
        __syncthreads();
    }
    if constexpr (FAST) {
        // the lanes that checked (the last scan segment: wave NW - 1, lanes 32..63)
        if (wave == NW - 1) {
            const bool any = __builtin_amdgcn_ballot_w64(strong) != 0;
            if (lane == 0 && any) P.slow[atomicAdd(P.nslow, 1)] = blk;
        }
    }
}

// One workgroup per (chunk, head): the direct form (listing the chunks that
// need the general one).
template <int DK, int DV, int C, bool ABF16, int GATE>
__global__ __launch_bounds__(GPrepT<C>::threads) void gprep_kernel(const GParams P) {
    gprep_body<DK, DV, C, ABF16, GATE, true>(P, blockIdx.x);
}

// Entry blockIdx.x of the general-form list, if the list is that long (one
// workgroup per (chunk, head), the list's largest length).
template <int DK, int DV, int C, bool ABF16, int GATE>
__global__ __launch_bounds__(GPrepT<C>::threads) void gprep_general_kernel(const GParams P) {
    if (static_cast<int>(blockIdx.x) >= *P.nslow) return;
    gprep_body<DK, DV, C, ABF16, GATE, false>(P, P.slow[blockIdx.x]);
}

// ---------------------------------------------------------------------------
// gchain_kernel: wave w holds state row block w (and w + 8); the C x 16
// product U' = U - W S is split over the waves: row block w % (C/16), part
// w / (C/16) of the d_k reduction, the parts handed to part 0 through LDS.
// At C = 128 a ninth wave pulls the record lines the chain reads (Kt, W, U,
// gamma) into L2 kGChainPrefetch chunks ahead, each of the d_v / 16 column
// tiles of a (sequence, head) every (d_v / 16)-th line, on its own wait
// counters (64K-token forward: 2.78 -> 2.38 ms; at C = 32, whose chunks'
// operands are a quarter as large, it cost 3.75 -> 3.98 ms).
// ---------------------------------------------------------------------------
template <int C> struct GChainPF {
    static constexpr bool on = C >= 128;
    static constexpr int threads = on ? kThreads + 64 : kThreads;
};
constexpr int kGChainPrefetch = 2;
// FUSED (C = 32): the chain also forms O = Gamma.Q S + P U' for its 16
// columns, so neither the state entering each chunk nor U' goes through the
// record and no output pass runs.  Gamma.Q S is split over the waves like
// W S (row block w % (C/16), part w / (C/16) of d_k, partial sums through
// LDS); the part-0 waves add them and P U' and store the rows.
template <int DK, int C> struct GChainB {
    static constexpr int LK = Ld<DK>::value, NSPLIT = kWaves / (C / 16), LP = C + 4;
    static constexpr bool FUSED = C <= 32;
    static constexpr int bytes = (2 * C * LK + DK * L16 + C * L16 + (NSPLIT - 1) * C * L16 + DK +
                                  (FUSED ? C * LK + (NSPLIT - 1) * C * L16 + C * LP : 0)) * 4;
};

template <int DK, int DV, int C, bool H16, bool OBF16>
__global__ __launch_bounds__(GChainPF<C>::threads) void gchain_kernel(const GParams P) {
    using R = GRec<DK, DV, C, H16>;
    constexpr int NTH = kThreads, NW = kWaves, LK = GChainB<DK, C>::LK, NT = DV / 16;
    constexpr int NB = C / 16, NSPLIT = GChainB<DK, C>::NSPLIT, KP = DK / NSPLIT;
    constexpr int NRB = DK / 16, RBW = (NRB + NW - 1) / NW;
    constexpr bool FUSED = GChainB<DK, C>::FUSED;
    constexpr int LP = GChainB<DK, C>::LP;
    static_assert(FUSED == R::FUSED, "the record and the chain agree on the fused output");
    extern __shared__ float lds[];
    float* sW = lds;                 // [C][LK]
    float* sKt = sW + C * LK;        // [C][LK]
    float* sS = sKt + C * LK;        // [DK][16]
    float* sU = sS + DK * L16;       // [C][16]
    float* sPart = sU + C * L16;     // [NSPLIT - 1][C][16]
    float* sGam = sPart + (NSPLIT - 1) * C * L16;   // [DK]
    [[maybe_unused]] float* sQh = sGam + DK;                       // FUSED: Gamma.Q [C][LK]
    [[maybe_unused]] float* sPartO = sQh + C * LK;                 // FUSED: [NSPLIT - 1][C][16]
    [[maybe_unused]] float* sPm = sPartO + (NSPLIT - 1) * C * L16; // FUSED: P [C][LP]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int n = P.order[pair / P.H], h = pair % P.H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = __builtin_amdgcn_readfirstlane(wave_id()), j = lane_id() >> 4;
    if (GChainPF<C>::on && wave == NW) {
        // the prefetch wave: matches the four barriers per chunk of the
        // others with bare ones (a fence would wait for these loads)
        __shared__ int s_pf[64];
        static_assert(R::W == R::KT + size_t(C) * DK * 4, "Kt and W are adjacent in the record");
        auto touch = [&](int gp) {
            l2_touch(grec(P, h, gp, R::KT), 2 * C * DK * 4, tile, NT, s_pf);
            l2_touch(grec(P, h, gp, R::U), C * DV * 4, tile, NT, s_pf);
            l2_touch(grec(P, h, gp, R::GAM), DK * 4, tile, NT, s_pf);
        };
        for (int gp = g0 + 1; gp < min(g0 + kGChainPrefetch, g1); ++gp) touch(gp);
        for (int g = g0; g < g1; ++g) {
            if (g + kGChainPrefetch < g1) touch(g + kGChainPrefetch);
#pragma unroll
            for (int b = 0; b < 4; ++b) __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);       // every load has landed before the wave ends
        return;
    }
    const int c0 = tile * 16;
    const int mb = wave % NB, part = wave / NB;
    const size_t sbase = (static_cast<size_t>(n) * P.H + h) * DK * DV;

    f4 S[RBW];
    for (int u = 0; u < RBW; ++u) {
        const int rb = wave + NW * u;
        S[u] = (P.initial_state && rb < NRB) ? load_tile(P.initial_state + sbase + rb * 16 * DV + c0, DV) : zero4();
    }
    Blk<C, DK, NTH> nW, nKt;
    [[maybe_unused]] Blk<C, FUSED ? DK : 4, NTH> nQh;
    [[maybe_unused]] Blk<C, FUSED ? C : 4, NTH> nP;
    f4 nU = zero4();
    float nGam = 0.f;
    auto fetch = [&](int g) {
        nW.load(grec(P, h, g, R::W), DK);
        nKt.load(grec(P, h, g, R::KT), DK);
        if constexpr (FUSED) {
            nQh.load(grec(P, h, g, R::QH), DK);
            nP.load(grec(P, h, g, R::P), C);
        }
        if (part == 0) nU = load_tile(grec(P, h, g, R::U) + mb * 16 * DV + c0, DV);
        if (threadIdx.x < DK) nGam = grec(P, h, g, R::GAM)[threadIdx.x];
    };
    if (g0 < g1) fetch(g0);
    for (int g = g0; g < g1; ++g) {
        nW.put(sW, LK);
        nKt.put(sKt, LK);
        if constexpr (FUSED) {
            nQh.put(sQh, LK);
            nP.put(sPm, LP);
        }
        const f4 uu = nU;
        if (threadIdx.x < DK) sGam[threadIdx.x] = nGam;
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(sS + rb * 16 * L16, L16, S[u]);
            if constexpr (!FUSED) {
                float* gS = grec(P, h, g, R::SIN);
                if constexpr (H16) store_tile_h(reinterpret_cast<_Float16*>(gS) + rb * 16 * DV + c0, DV, S[u]);
                else store_tile(gS + rb * 16 * DV + c0, DV, S[u]);
            }
        }
        __syncthreads();
        if (g + 1 < g1) fetch(g + 1);
        // U' = U - W S (and FUSED: Gamma.Q S), this wave's part of d_k
        const f4 x = mm<KP, true, false>(sW + mb * 16 * LK + part * KP, LK, 1, sS + part * KP * L16, L16, 1, zero4());
        if (part) store_tile(sPart + ((part - 1) * C + mb * 16) * L16, L16, x);
        [[maybe_unused]] f4 y = zero4();
        if constexpr (FUSED) {
            y = mm<KP, true, false>(sQh + mb * 16 * LK + part * KP, LK, 1, sS + part * KP * L16, L16, 1, zero4());
            if (part) store_tile(sPartO + ((part - 1) * C + mb * 16) * L16, L16, y);
        }
        __syncthreads();
        if (part == 0) {
            f4 uc = uu - x;
#pragma unroll
            for (int p2 = 1; p2 < NSPLIT; ++p2) uc -= load_tile(sPart + ((p2 - 1) * C + mb * 16) * L16, L16);
            store_tile(sU + mb * 16 * L16, L16, uc);
            if constexpr (FUSED) {
#pragma unroll
                for (int p2 = 1; p2 < NSPLIT; ++p2) y += load_tile(sPartO + ((p2 - 1) * C + mb * 16) * L16, L16);
            } else if constexpr (H16) {
                store_tile_h(reinterpret_cast<_Float16*>(grec(P, h, g, R::UC)) + mb * 16 * DV + c0, DV, uc);
            } else {
                store_tile(grec(P, h, g, R::UC) + mb * 16 * DV + c0, DV, uc);
            }
        }
        __syncthreads();
        if constexpr (FUSED) {
            // O rows of row block mb: Gamma.Q S + P U' (P lower triangular)
            if (part == 0) {
                for (int kb = 0; kb <= mb; ++kb)
                    y = mm<16, true, false>(sPm + mb * 16 * LP + kb * 16, LP, 1, sU + kb * 16 * L16, L16, 1, y);
                const int4 ent = P.table[g];
                const int i = lane_id() & 15;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mb * 16 + 4 * j + e;
                    if (r < ent.z)
                        store_out<OBF16>(P.o, (static_cast<size_t>(ent.y + r) * P.H + h) * DV + c0 + i, y[e]);
                }
            }
        }
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
// At C = 128 (QREG) output tile t is row block t % (C/16) and column block
// t / (C/16), so each wave owns one row block: it reads its 16 rows of
// Gamma.Q straight into registers at the start (the A operand of both its
// tiles) and only S, P and U' are staged in LDS (74 KB: two workgroups per
// CU; staging Gamma.Q too took 140 KB and 2.49 vs 1.89 ms).  At C = 32 the
// four tiles' two row blocks would be read by two waves each, and Gamma.Q is
// staged in LDS with the rest (1.57 vs 1.79 ms).
// ---------------------------------------------------------------------------
template <int DK, int C> struct GOutB {
    static constexpr bool QREG = C >= 128;
    static constexpr int LK = Ld<DK>::value, NB = C / 16, NLT = NB * (NB + 1) / 2;
    static constexpr int bytes = ((QREG ? 0 : C * LK) + DK * kLS + NLT * 256 + C * kLS) * 4;
};

template <int DK, int DV, int C, bool OBF16, bool H16>
__global__ __launch_bounds__(kThreads) void gout_kernel(const GParams P) {
    using R = GRec<DK, DV, C, H16>;
    constexpr int NTH = kThreads, NW = kWaves, SL = kSL, LS = kLS;
    constexpr int NB = GOutB<DK, C>::NB, NLT = GOutB<DK, C>::NLT, NSV = DV / SL;
    constexpr int PIT = (NLT * 256 + NTH - 1) / NTH;
    constexpr int NT = NB * (SL / 16);                 // output tiles
    constexpr int KG = DK / 16;                        // 16-deep groups of Qh S
    constexpr bool QREG = GOutB<DK, C>::QREG;
    constexpr int LK = GOutB<DK, C>::LK;
    static_assert(!QREG || NB == NW, "each wave's tiles share one row block");
    extern __shared__ float lds[];
    float* sQh = lds;                // Gamma.Q [C][LK] (not QREG)
    float* sS = lds + (QREG ? 0 : C * LK);   // S[:, slice]   [DK][LS]
    float* sP = sS + DK * LS;        // P, packed lower tiles [NLT][256]
    float* sU = sP + NLT * 256;      // U'[:, slice]  [C][LS]

    // Workgroups are dealt to the 8 XCDs round-robin: the NSV workgroups of
    // one (chunk, head) get block indices NSV consecutive slots apart on one
    // XCD, so its Gamma.Q and P are read into that XCD's L2 once. The grid is
    // padded to a multiple of 8 (chunk, head) pairs.
    const int H = P.H;
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    const int sv = slot % NSV, gh = (slot / NSV) * 8 + xcd;
    if (gh >= P.gmax * H) return;
    const int h = gh % H, g = gh / H;
    if (g >= P.ctrl[0]) return;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), i = lane_id() & 15, j = lane_id() >> 4;
    const int s0 = sv * SL;
    const int mb = wave % NB;        // QREG: this wave's row block

    // QREG: this wave's rows of Gamma.Q in the A layout of the 16-deep groups
    [[maybe_unused]] f4 aq[QREG ? KG : 1];
    if constexpr (QREG) {
        const float* gq = grec(P, h, g, R::QH) + static_cast<size_t>(mb * 16 + i) * DK + 4 * j;
#pragma unroll
        for (int gg = 0; gg < KG; ++gg) aq[gg] = *reinterpret_cast<const f4*>(gq + 16 * gg);
    }
    {
        Blk<C, QREG ? 4 : DK, NTH> bq;      // (QREG: unused)
        using BS = std::conditional_t<H16, BlkH<DK, SL, NTH>, Blk<DK, SL, NTH>>;
        using BU = std::conditional_t<H16, BlkH<C, SL, NTH>, Blk<C, SL, NTH>>;
        using SE = std::conditional_t<H16, _Float16, float>;
        BS bs;
        BU bu;
        float pv[PIT];
        if constexpr (!QREG) bq.load(grec(P, h, g, R::QH), DK);
        bs.load(reinterpret_cast<const SE*>(grec(P, h, g, R::SIN)) + s0, DV);
        bu.load(reinterpret_cast<const SE*>(grec(P, h, g, R::UC)) + s0, DV);
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
        if constexpr (!QREG) bq.put(sQh, LK);
        bs.put(sS, LS);
        bu.put(sU, LS);
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
            const int idx = tid + it * NTH;
            if (idx < NLT * 256) sP[idx] = pv[it];
        }
    }
    __syncthreads();
    for (int t = wave; t < NT; t += NW) {
        const int tmb = QREG ? mb : t / (SL / 16);
        const int nb = QREG ? t / NB : t % (SL / 16);
        f4 x = zero4();
        if constexpr (QREG) {
            const float* pb = sS + 4 * j * LS + nb * 16 + i;
#pragma unroll
            for (int gg = 0; gg < KG; ++gg) {
                const f4 b = f4{pb[16 * gg * LS], pb[(16 * gg + 1) * LS], pb[(16 * gg + 2) * LS], pb[(16 * gg + 3) * LS]};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) x = mfma4(aq[gg][s2], b[s2], x);
            }
        } else {
            x = mm<DK, true, false>(sQh + tmb * 16 * LK, LK, 1, sS + nb * 16, LS, 1, x);
        }
        for (int kb = 0; kb <= tmb; ++kb)
            x = mm<16, true, false>(sP + lt(tmb, kb) * 256, 16, 1, sU + kb * 16 * LS + nb * 16, LS, 1, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = tmb * 16 + 4 * j + e;
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
    if (GRec<DK, DV, C, ABF16>::END > pl.rec_bytes) return hipErrorInvalidValue;
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
    p.nslow = reinterpret_cast<int32_t*>(ws + pl.off_ctrl) + 1;
    p.slow = reinterpret_cast<int32_t*>(ws + pl.off_slow);

    hipError_t e = launch_chunk_plan(pl, a.cu_seqlens, a.workspace, stream);
    if (e != hipSuccess) return e;
    const unsigned chunk_blocks = static_cast<unsigned>(pl.gmax * pl.H);
    const int64_t pairs = static_cast<int64_t>(pl.N) * pl.H;
    const unsigned chain_blocks = static_cast<unsigned>((pairs + 7) / 8 * 8 * (DV / 16));
    if (chunk_blocks > 0) {
        constexpr int l1 = GPrepB<C>::bytes;
        for (auto k1 : {gprep_kernel<DK, DV, C, ABF16, GATE>, gprep_general_kernel<DK, DV, C, ABF16, GATE>}) {
            if ((e = set_lds(k1, l1)) != hipSuccess) return e;
            hipLaunchKernelGGL(k1, dim3(chunk_blocks), dim3(GPrepT<C>::threads), l1, stream, p);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (chain_blocks > 0) {
        auto k2 = gchain_kernel<DK, DV, C, ABF16, GChainB<DK, C>::FUSED && OBF16>;
        constexpr int l2 = GChainB<DK, C>::bytes;
        if ((e = set_lds(k2, l2)) != hipSuccess) return e;
        hipLaunchKernelGGL(k2, dim3(chain_blocks), dim3(GChainPF<C>::threads), l2, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (!GChainB<DK, C>::FUSED) {
        if (chunk_blocks > 0) {
            auto k3 = gout_kernel<DK, DV, C, OBF16, ABF16>;
            constexpr int l3 = GOutB<DK, C>::bytes;
            if ((e = set_lds(k3, l3)) != hipSuccess) return e;
            hipLaunchKernelGGL(k3, dim3((chunk_blocks + 7) / 8 * 8 * (DV / kSL)), dim3(kThreads), l3, stream, p);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
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
size_t rec_end(int c, bool h16) {
    if (h16) return c == 32 ? GRec<DK, DV, 32, true>::END : c == 128 ? GRec<DK, DV, 128, true>::END : GRec<DK, DV, 64, true>::END;
    return c == 32 ? GRec<DK, DV, 32>::END : c == 128 ? GRec<DK, DV, 128>::END : GRec<DK, DV, 64>::END;
}

}  // namespace

size_t generic_record_bytes(int Dk, int Dv, int chunk_size, bool act16) {
    if (Dk == 128 && Dv == 128) return rec_end<128, 128>(chunk_size, act16);
    if (Dk == 64 && Dv == 64) return rec_end<64, 64>(chunk_size, act16);
    if (Dk == 128 && Dv == 64) return rec_end<128, 64>(chunk_size, act16);
    return rec_end<64, 128>(chunk_size, act16);
}

hipError_t launch_chunk_fwd_generic(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (pl.Dk == 128 && pl.Dv == 128) return launch_c<128, 128>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 64) return launch_c<64, 64>(pl, a, stream);
    if (pl.Dk == 128 && pl.Dv == 64) return launch_c<128, 64>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 128) return launch_c<64, 128>(pl, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
