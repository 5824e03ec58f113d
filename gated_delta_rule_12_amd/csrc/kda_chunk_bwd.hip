// Chunkwise KDA backward for gfx950: the vector-Jacobian product of the
// chunked forward for L = sum(dO * o) + sum(dS_T * S_T).
//
// The pages present the chunk algorithm as the training form ("Hybrid Linear
// Attention Architectures...", Hardware-Aware Chunkwise Parallelism;
// "Linear Attention KDA Gating in a 3:1 Hybrid Architecture", section 3).
// Its backward is the chain rule through each line of that forward, chunk by
// chunk and last chunk first, with only the state gradient dS flowing from
// one chunk to the one before:
//
//   forward per chunk (state S entering it):
//     U' = U - W S,  O = Qh S + P U',  S_next = Diag(gamma) S + Kt^T U'
//   reverse per chunk (dS_next = gradient of the state leaving it):
//     dU' = P^T dO + Kt dS_next
//     dS  = Diag(gamma) dS_next + Qh^T dO - W^T dU'
//   then, per chunk and independent of the others,
//     M = Tril(dO U'^T), dQh = dO S^T + M Kb, dKb = M^T Qh + dR^T Kh,
//     dW = -dU' S^T, dKt = U' dS_next^T, dgamma = rowsum(dS_next .* S),
//     dT = dW Y^T + dU' Z^T, dY = T^T dW, dZ = T^T dU'  (Y = beta.Kh, Z = beta.V),
//     dA = -StrictTril(T^T dT T^T), dR = Diag(beta) dA  (R = Kh Kb^T),
//     dV = beta.dZ, dbeta = rowsum(dZ.V + dY.Kh + dA.R), dKh = beta.dY + dR Kb,
//     and the gate terms through Gamma = exp(b), b = cumsum(log alpha).
//
// Launches, on the caller's stream:
//   plan_kernel        the forward's chunk table (shared launcher; it also
//                      empties the general-form list)
//   bwd_prep_kernel    one WG per (chunk, head): b, Gamma.Q, (gamma/Gamma).K,
//                      A, T = (I + A)^-1, W, U, P, gamma -> record, in the
//                      direct form; a (chunk, head) that needs the general
//                      form is flagged, appended to the list, and left
//   bwd_prep_general_kernel   the same for each (chunk, head) of the list
//   bwd_ckpt_kernel    one WG per (sequence, head, 16 value columns),
//   (bwd_ckpt16)       chunks in order: the state entering each chunk and U'
//   bwd_rev_kernel     one WG per (sequence, head, 16 value columns),
//   (bwd_rev16)        chunks last to first: dS_next of each chunk and dU';
//                      dS_0 at the end
//   bwd_grad_kernel    one WG per (chunk, head) not flagged: every
//                      contraction over the value dimension (dO S^T, dU' S^T,
//                      U' dS_next^T, M, dU' V^T, dgamma), dv = beta . T^T dU',
//                      then dT, dA, R, dY, dKh, dQh, dKb, the gate chain rule,
//                      dq, dk, dgate, dbeta
//   bwd_grad_general_kernel   the same for each (chunk, head) of the list
//
// Two forms of the per-chunk work, chosen per (chunk, head) from its decay.
// Direct: when no channel decays below 2^-64 over the chunk, Gamma = 2^b and
// 1/Gamma are formed as fp32 factors (within 2^+-64) and Kh = Gamma.K,
// Kb = K/Gamma, Qh = Gamma.Q enter plain products.  General: no product ever
// forms Gamma or 1/Gamma of a whole chunk; the log decay is summed per
// 16-token tile and every decay factor is 2^x with x <= 0 (decayed_tile and
// decayed_lower_upper in kda_mm32.h), so any forget gate in (0, 1] is
// handled without overflow.  Both compute the same products up to rounding.
// They are separate kernels, so each is compiled (and its registers
// allocated) on its own; the general ones get one workgroup per possible
// list entry, and those past the list's length return at once.
//
// Numerics: with fp32 activations every product runs on the fp32 matrix
// cores (16x16x4) and every intermediate is stored in fp32.  With bf16
// activations the two state passes and the value-side contractions take
// fp16 operands (fp32 accumulation) and the record keeps S, dS_next, U', dU'
// and those operands in fp16; the key-side products keep fp32 operands (the
// five C x d_k ones split each into bf16 hi + lo for the bf16 matrix cores,
// which keeps fp32's exponent range and ~2^-16 relative accuracy).  No fp16
// operand holds a factor 1/Gamma: the 16-bit passes see Gamma.Q,
// (gamma/Gamma).K, P, W and T, whose decay factors are at most 1.
#include <type_traits>

#include "kda_chunk.h"
#include "kda_common.h"
#include "kda_mm32.h"

namespace kda {
namespace {

using namespace mm32;

constexpr int C = kChunk;
constexpr int LC = C + 4;          // LDS row stride of C x C fp32 tiles

// ---------------------------------------------------------------------------
// Per-(head, chunk) record of the backward (byte offsets).  Rows are
// chunk-local tokens; the tail of a partial chunk holds zeros (Qh, Kt, W, U,
// P, dU', ...).  With 16-bit activations (F16) the state passes read their A
// operands as fp16 fragments, so the fp32 Kt, W and P are absent, and S,
// dS_next, U' and dU' are stored in fp16; with fp32 activations the fragments
// are absent.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F16> struct BRec {
    static constexpr size_t CK = size_t(C) * DK * 4, CV = size_t(C) * DV * 4, CC = size_t(C) * C * 4;
    static constexpr size_t SE = F16 ? 2 : 4;    // bytes per element of S, dS_next, U', dU'
    static constexpr size_t QH = 0;              // Gamma . Q                 [C][DK]
    static constexpr size_t KT = QH + CK;        // (gamma / Gamma) . K       [C][DK]  (fp32 path)
    static constexpr size_t W = KT + (F16 ? 0 : CK);   // T Diag(beta) (Gamma . K)  [C][DK]  (fp32 path)
    static constexpr size_t U = W + (F16 ? 0 : CK);    // T Diag(beta) V            [C][DV]
    static constexpr size_t P = U + CV;          // Tril(Qh Kb^T)             [C][C]   (fp32 path)
    static constexpr size_t TT = P + (F16 ? 0 : CC);   // (I + A)^-1                [C][C]
    static constexpr size_t GAM = TT + CC;       // gamma                     [DK]
    static constexpr size_t SIN = GAM + size_t(DK) * 4;       // state entering   [DK][DV]
    static constexpr size_t DSO = SIN + size_t(DK) * DV * SE; // dL/d(state leaving) [DK][DV]
    static constexpr size_t UC = DSO + size_t(DK) * DV * SE;  // U' = U - W S      [C][DV]
    static constexpr size_t DUC = UC + size_t(C) * DV * SE;   // dL/dU'            [C][DV]
    // fp16 A fragments of the state passes' products (16-bit path)
    static constexpr size_t HK = F16 ? size_t(C) * DK * 2 : 0;
    static constexpr size_t FKT = DUC + size_t(C) * DV * SE;  // Kt                [C][DK]
    static constexpr size_t FKTT = FKT + HK;              // Kt^T              [DK][C]
    static constexpr size_t FQHT = FKTT + HK;             // Qh^T              [DK][C]
    static constexpr size_t FW = FQHT + HK;               // W                 [C][DK]
    static constexpr size_t FWT = FW + HK;                // W^T               [DK][C]
    static constexpr size_t FPT = FWT + HK;               // P^T               [C][C]
    static constexpr size_t END = FPT + (F16 ? size_t(C) * C * 2 : 0);
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* gate;
    const void* dout;
    const float* beta;
    const float* initial_state;
    const float* dfinal_state;
    void* dq;
    void* dk;
    void* dv;
    float* dgate;
    float* dbeta;
    float* dinitial_state;
    const int32_t* ctrl;
    int32_t* nslow;                     // length of the general list (zeroed by the chunk table)
    int32_t* slow;                      // general list: g * H + h of each chunk that takes it
    int32_t* flag;                      // per g * H + h: 1 when the chunk takes the general form
    const int32_t* first;
    const int32_t* order;
    const int4* table;
    unsigned char* rec;
    size_t rec_bytes;
    int64_t gmax;
    int N, H;
};

__device__ __forceinline__ float* rec_at(const BwdParams& P, int h, int g, size_t off) {
    return reinterpret_cast<float*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
}

// ---------------------------------------------------------------------------
// bwd_prep_kernel: one (chunk, head), 512 threads.
// ---------------------------------------------------------------------------
// b = cumsum over the chunk's rows of log2 alpha, per key channel; padding
// rows add 0.  On entry s[r * ld + c] holds the gate as given (for the scalar
// gate, sGs[r]); `each(r, c, b)` receives every b in row order per channel and
// may overwrite s[r * ld + c].  NTH / DK row segments per channel: segment
// sums first, then each segment's scan from the sum of the segments before
// it.  sPart holds NTH floats of scratch; one barrier inside, none at the end.
template <int DK, int NTH, int GATE, typename F>
__device__ __forceinline__ void gate_cumsum(float* s, int ld, const float* sGs, int len, float* sPart, F&& each) {
    constexpr int NS = NTH / DK, SEG = C / NS;
    static_assert(NS * SEG == C, "row segments tile the chunk");
    const int c = threadIdx.x % DK, sg = threadIdx.x / DK, r0 = sg * SEG;
    float l2[SEG];
#pragma unroll
    for (int r = 0; r < SEG; ++r) l2[r] = GATE == KDA_GATE_SCALAR ? sGs[r0 + r] : s[(r0 + r) * ld + c];
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < SEG; ++r) {
        float x = 0.f;
        if (r0 + r < len) {
            if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16) x = log2_alpha_from_softplus_arg(l2[r]);
            else x = __builtin_amdgcn_logf(l2[r]);
        }
        l2[r] = x;
        part += x;
    }
    sPart[sg * DK + c] = part;
    __syncthreads();
    float b = 0.f;
    for (int s2 = 0; s2 < sg; ++s2) b += sPart[s2 * DK + c];
#pragma unroll
    for (int r = 0; r < SEG; ++r) {
        b += l2[r];
        each(r0 + r, c, b);
    }
}

constexpr int kPrepThreads = 512, kPrepWaves = kPrepThreads / 64;

// A chunk in which no channel decays below 2^-64 (gamma >= kFastGammaMin)
// takes the direct form (Gamma and 1/Gamma as fp32 factors, each within
// 2^+-64); any other takes the general form, whose decay factors never
// exceed 1.
constexpr float kFastGammaMin = 0x1p-64f;

template <int DK, int DV> struct PrepB {
    static constexpr int LK = Ld<DK>::value, LV = Ld<DV>::value, LM = LK > LV ? LK : LV;
    static constexpr int bytes = (2 * C * LK + C * LM + 2 * C * LC + 2 * C + (C / 16) * DK) * 4;
};

// T = (I + A)^-1 (A strictly lower, fp32 [C][LC] in sA) into sT by 16 x 16
// blocks: each of waves 0..3 inverts one diagonal block by substitution (16
// lanes, one column each), then T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj for
// i - j = 1, 2, 3.  sX: one 16 x 16 fp32 tile of scratch per wave.  The
// caller's writes before the call are ordered by its first barrier; it ends
// with a barrier.
__device__ __forceinline__ void solve_t(const float* sA, float* sT, float* sX) {
    const int wave = wave_id(), lane = lane_id();
    // Column-oriented: once t[s] is final, every later row takes its term at
    // once (the same operations, in the same order per row, as row by row,
    // but a chain of 16 steps instead of 120).  Column s of the block is read
    // while column s - 1 is applied (not all 120 values first: that needs
    // more registers than two workgroups per CU leave).
    if (wave < 4 && lane < 16) {
        const int col = lane, o = 16 * wave;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = r == col ? 1.f : 0.f;
        float cur[16], nxt[16];
#pragma unroll
        for (int r = 1; r < 16; ++r) cur[r] = sA[(o + r) * LC + o];
#pragma unroll
        for (int s2 = 0; s2 < 15; ++s2) {
            if (s2 + 1 < 15) {
#pragma unroll
                for (int r = s2 + 2; r < 16; ++r) nxt[r] = sA[(o + r) * LC + o + s2 + 1];
            }
#pragma unroll
            for (int r = s2 + 1; r < 16; ++r) t[r] -= cur[r] * t[s2];
#pragma unroll
            for (int r = s2 + 2; r < 16; ++r) cur[r] = nxt[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(o + r) * LC + o + col] = t[r];
    }
    for (int idx = threadIdx.x; idx < 6 * 256; idx += kPrepThreads) {      // blocks above the diagonal
        const int blk = idx >> 8, e = idx & 255;
        const int mb = blk < 3 ? 0 : blk < 5 ? 1 : 2;
        const int nb = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
        sT[(mb * 16 + (e >> 4)) * LC + nb * 16 + (e & 15)] = 0.f;
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int bi = wave + d, bj = wave;
            f4 x = zero4();
            for (int bk = bj; bk < bi; ++bk)
                x = mm<16, true, false>(sA + 16 * bi * LC + 16 * bk, LC, 1, sT + 16 * bk * LC + 16 * bj, LC, 1, x);
            store_tile(sX + wave * 256, 16, x);
        }
        __syncthreads();
        if (wave < 4 - d) {
            const int bi = wave + d, bj = wave;
            const f4 y = mm<16, true, false>(sT + 16 * bi * LC + 16 * bi, LC, 1, sX + wave * 256, 16, 1, zero4());
            store_tile(sT + 16 * bi * LC + 16 * bj, LC, -y);
        }
        __syncthreads();
    }
}

// The general form for one listed (chunk, head): every decay factor formed
// from exponents <= 0, for any gate in [0, 1].  Channels are staged whole
// (137 KB of LDS: one workgroup per CU); it only runs on the listed chunks.
template <int DK, int DV, bool ABF16, int GATE>
__device__ __forceinline__ void prep_general_body(const BwdParams& P, const int h, const int g) {
    using R = BRec<DK, DV, ABF16>;
    constexpr int NTH = kPrepThreads, NW = kPrepWaves;
    constexpr int LK = PrepB<DK, DV>::LK, LV = PrepB<DK, DV>::LV;
    constexpr int NBLK = C / 16;
    constexpr bool GBF16 = GATE == KDA_GATE_SOFTPLUS_BF16;
    extern __shared__ float lds[];
    float* sKh = lds;                    // K -> Gamma.K -> beta.Gamma.K      [C][LK]
    float* sKb = sKh + C * LK;           // gate -> b (per tile) -> Kt -> T-solve scratch [C][LK]
    float* sQ = sKb + C * LK;            // Q -> Gamma.Q, later V -> beta.V    [C][LM]
    float* sA = sQ + C * PrepB<DK, DV>::LM;   // A                            [C][LC]
    float* sT = sA + C * LC;             // T                                  [C][LC]
    float* sBeta = sT + C * LC;          // [C]
    float* sGs = sBeta + C;              // scalar gate per row                [C]
    float* sTot = sGs + C;               // log2 alpha summed per 16-token tile [C/16][DK]

    const int H = P.H;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), lane = lane_id(), i = lane & 15, j = lane >> 4;

    Tok<ABF16, DV, DV, NTH> tv;          // V, held in registers until T is done
    {
        Tok<ABF16, DK, DK, NTH> tk, tq;
        tk.load(P.k, row0, len, h, H);
        tq.load(P.q, row0, len, h, H);
        tv.load(P.v, row0, len, h, H);
        if constexpr (GATE == KDA_GATE_SCALAR) {
            if (tid < C) sGs[tid] = tid < len ? static_cast<const float*>(P.gate)[(row0 + tid) * H + h] : 1.f;
        } else {
            Tok<GBF16, DK, DK, NTH> tg;
            tg.load(P.gate, row0, len, h, H);
            tg.put(sKb, LK);
        }
        if (tid < C) sBeta[tid] = tid < len ? P.beta[(row0 + tid) * H + h] : 0.f;
        tk.put(sKh, LK);
        tq.put(sQ, LK);
    }
    __syncthreads();

    float* gP = rec_at(P, h, g, R::P);
    float* gGam = rec_at(P, h, g, R::GAM);
    float* gKt = rec_at(P, h, g, R::KT);
    // A = StrictTril(Diag(beta) Kh Kb^T) -> sA;  P = Tril(Qh Kb^T) -> record.
    // Tile (mb, nb) of both shares its B operand; two tile positions per wave,
    // the ten below or on the diagonal spread so the waves sharing a SIMD
    // (w, w + 4) hold 3, 3, 2, 2 of them; the six above are only zeroed.
    constexpr unsigned kTiles[8] = {0x0010, 0x2030, 0x1101, 0x2102, 0x2203, 0x3112, 0x3213, 0x3323};
    // b per 16-token tile (sKb) and the tile totals; the tiles of A and P
    // from the raw K and Q with every decay factor <= 1 (decayed_tile)
    tile_gate_scan<DK, NTH, C, GATE>(sKb, LK, sGs, len, sTot, sA);
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
        const unsigned tt = (kTiles[wave] >> (8 * (1 - slot))) & 0xff;
        const int mb = tt >> 4, nb = tt & 15;
        f4 a = zero4(), pp = zero4();
        decayed_tile<DK / 16, true, true, ABF16>(sKh, sQ, sKh, sKb, sTot, LK, DK, mb, nb, a, pp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = mb * 16 + 4 * j + e, s2 = nb * 16 + i;
            a[e] = s2 < r ? sBeta[r] * a[e] : 0.f;
            pp[e] = s2 <= r ? pp[e] : 0.f;
        }
        store_tile(sA + mb * 16 * LC + nb * 16, LC, a);
        if constexpr (ABF16) store_tile(sT + mb * 16 * LC + nb * 16, LC, pp);   // P, for P^T fragments
        else store_tile(gP + mb * 16 * C + nb * 16, C, pp);
    }
    __syncthreads();
    // Kh = Gamma.K, Qh = Gamma.Q and Kt = (gamma / Gamma).K (into sKb), every
    // factor 2^x with x <= 0: with pre / suf the totals of the tiles
    // before / after the row's tile t,  log2 Gamma = pre + b,
    // log2(gamma / Gamma) = T_t - b + suf.
    for (int idx = tid; idx < C * DK; idx += NTH) {
        const int r = idx / DK, c = idx % DK, t = r / 16;
        const float bl = sKb[r * LK + c];
        const float pre = tot1(sTot, DK, c, 0, t), suf = tot1(sTot, DK, c, t + 1, NBLK);
        const float G = __builtin_amdgcn_exp2f(pre + bl);
        const float kv = sKh[r * LK + c];
        sKh[r * LK + c] = G * kv;
        sQ[r * LK + c] *= G;
        sKb[r * LK + c] = kv * __builtin_amdgcn_exp2f(sTot[t * DK + c] - bl + suf);
    }
    if (tid < DK) gGam[tid] = __builtin_amdgcn_exp2f(tot1(sTot, DK, tid, 0, NBLK));
    __syncthreads();
    if constexpr (!ABF16) {
        for (int idx = tid; idx < C * DK; idx += NTH) {
            const int r = idx / DK, c = idx % DK;
            gKt[r * DK + c] = sKb[r * LK + c];
        }
    }
    store_block<NTH>(rec_at(P, h, g, R::QH), DK, sQ, LK, C, DK);
    if constexpr (ABF16) {
        // fp16 fragments for the 16-bit state passes: Kt, Kt^T, Qh^T and P^T
        auto hrec = [&](size_t off) { return reinterpret_cast<_Float16*>(P.rec + (size_t(h) * P.gmax + g) * P.rec_bytes + off); };
        write_afrags<C, DK, NTH>(hrec(R::FKT), [&](int m, int k) { return sKb[m * LK + k]; });
        write_afrags<DK, C, NTH>(hrec(R::FKTT), [&](int m, int k) { return sKb[k * LK + m]; });
        write_afrags<DK, C, NTH>(hrec(R::FQHT), [&](int m, int k) { return sQ[k * LK + m]; });
        write_afrags<C, C, NTH>(hrec(R::FPT), [&](int m, int k) { return sT[k * LC + m]; });
        __syncthreads();
    }

    // Y = Diag(beta) Kh (in place), then T = (I + A)^-1 with sKb as scratch
    for (int idx = tid; idx < C * DK; idx += NTH) {
        const int r = idx / DK, c = idx % DK;
        sKh[r * LK + c] *= sBeta[r];
    }
    solve_t(sA, sT, sKb);
    store_block<NTH>(rec_at(P, h, g, R::TT), C, sT, LC, C, C);
    tv.put_scaled(sQ, LV, sBeta);        // Z = Diag(beta) V
    __syncthreads();

    // W = T Y, U = T Z (T lower triangular: row block mb reduces over 16 (mb + 1) tokens)
    float* gW = rec_at(P, h, g, R::W);
    float* gU = rec_at(P, h, g, R::U);
    // wave w: column blocks w, w + 8, ... of [W | U], all four row blocks
    // sharing each B read
    constexpr int NK = DK / 16, NV = DV / 16;
    for (int cb = wave; cb < NK + NV; cb += NW) {
        const bool isw = cb < NK;
        const int nb = isw ? cb : cb - NK;
        f4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
        mm_rows<4, C / 16, true, false>(sT, LC, 1, (isw ? sKh : sQ) + nb * 16, isw ? LK : LV, 1, 0, 1,
                                        [](int mb, int gg) { return gg <= mb; }, acc);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (isw) {
                if constexpr (ABF16) store_tile(sKb + mb * 16 * LK + nb * 16, LK, acc[mb]);   // W, for its fragments
                else store_tile(gW + mb * 16 * DK + nb * 16, DK, acc[mb]);
            } else {
                store_tile(gU + mb * 16 * DV + nb * 16, DV, acc[mb]);
            }
        }
    }
    if constexpr (ABF16) {
        __syncthreads();
        auto hrec = [&](size_t off) { return reinterpret_cast<_Float16*>(P.rec + (size_t(h) * P.gmax + g) * P.rec_bytes + off); };
        write_afrags<C, DK, NTH>(hrec(R::FW), [&](int m, int k) { return sKb[m * LK + k]; });
        write_afrags<DK, C, NTH>(hrec(R::FWT), [&](int m, int k) { return sKb[k * LK + m]; });
    }
}

// The direct form, channels 64 at a time.  Every channel's chunk decay is
// assumed within 2^-64 (Gamma and 1/Gamma as fp32 factors); the chunk is
// checked at the end and, when some channel decays further, flagged and
// appended to the general list (its values here are then never used).  The
// key channels are staged in slices of KSL, so the LDS holds four 64 x 68
// fp32 tiles (73 KB: two workgroups per CU): A and P accumulate in the
// waves' registers over the slices; after T, W = T Diag(beta) Gamma.K takes
// the last slice's Gamma.K still in LDS, and every other slice's formed again
// from k and the gate (the same scan, so the same values), each pass beside
// U = T Diag(beta) V for one value slice.
constexpr int KSL = 64, LH = KSL + 4;
static_assert(LH == LC, "the slice tiles and the C x C tiles share one row stride");

template <int DK> struct PrepDirB {
    static constexpr int bytes = (4 * C * LH + 2 * C + DK + kPrepThreads) * 4;
};

// write_afrags restricted to row blocks [mb0, mb0 + NMB) and reduction
// blocks [kb0, kb0 + NKS) of an M x K matrix (same fragment layout)
template <int M, int K, int NMB, int NKS, int NTH, typename F>
__device__ __forceinline__ void write_afrags_part(_Float16* dst, int mb0, int kb0, F elem) {
    constexpr int NKB = K / 32, N = NMB * NKS * 64;
    static_assert(NMB <= M / 16 && NKS <= NKB, "a part of the matrix");
    for (int idx = threadIdx.x; idx < N; idx += NTH) {
        const int f = idx >> 6, ln = idx & 63, mb = mb0 + f / NKS, kb = kb0 + f % NKS;
        const int m = 16 * mb + (ln & 15), k0 = 32 * kb + 8 * (ln >> 4);
        h8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<_Float16>(elem(m, k0 + e));
        *reinterpret_cast<h8*>(dst + afrag_off(mb, kb, NKB, ln)) = v;
    }
}

template <int DK, int DV, bool ABF16, int GATE>
__device__ __forceinline__ void prep_direct_body(const BwdParams& P, const int h, const int g) {
    using R = BRec<DK, DV, ABF16>;
    constexpr int NTH = kPrepThreads;
    constexpr int NKS = DK / KSL, NVS = DV / KSL, NIT = NKS > NVS ? NKS : NVS;
    constexpr bool GBF16 = GATE == KDA_GATE_SOFTPLUS_BF16;
    static_assert(DK % KSL == 0 && DV % KSL == 0, "whole slices");
    extern __shared__ float lds[];
    float* sX0 = lds;                    // K -> Gamma.K (kept for W); Diag(beta).Gamma.K        [C][LH]
    float* sX1 = sX0 + C * LH;           // gate -> K/Gamma; T-solve scratch; Diag(beta).V        [C][LH]
    float* sA = sX1 + C * LH;            // A; the gate (W pass); W, for its fragments           [C][LC]
    float* sT = sA + C * LC;             // Q -> Gamma.Q; P; T                                    [C][LC]
    float* sBeta = sT + C * LC;          // [C]
    float* sGs = sBeta + C;              // scalar gate per row [C]
    float* sGam = sGs + C;               // gamma = 2^b_last per channel [DK], kept to the end
    float* sPart = sGam + DK;            // scan scratch [NTH]

    const int H = P.H;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), lane = lane_id(), i = lane & 15, j = lane >> 4;
    auto hrec = [&](size_t off) { return reinterpret_cast<_Float16*>(P.rec + (size_t(h) * P.gmax + g) * P.rec_bytes + off); };

    Tok<ABF16, DK, KSL, NTH> tk, tq;     // the next key slice's k and q
    Tok<GBF16, DK, KSL, NTH> tg;         // and its gate (per-channel forms)
    auto load_slice = [&](int c0, bool withq) {
        tk.load(P.k, row0, len, h, H, c0);
        if (withq) tq.load(P.q, row0, len, h, H, c0);
        if constexpr (GATE != KDA_GATE_SCALAR) tg.load(P.gate, row0, len, h, H, c0);
    };
    load_slice(0, true);
    if constexpr (GATE == KDA_GATE_SCALAR) {
        if (tid < C) sGs[tid] = tid < len ? static_cast<const float*>(P.gate)[(row0 + tid) * H + h] : 1.f;
    }
    if (tid < C) sBeta[tid] = tid < len ? P.beta[(row0 + tid) * H + h] : 0.f;

    // A = StrictTril(Diag(beta) Kh Kb^T), P = Tril(Qh Kb^T), accumulated over
    // the slices: tile (mb, nb) of both shares its B operand; two tile
    // positions per wave, the ten below or on the diagonal spread so the
    // waves sharing a SIMD (w, w + 4) hold 3, 3, 2, 2 of them; the six above
    // are only zeroed.
    constexpr unsigned kTiles[8] = {0x0010, 0x2030, 0x1101, 0x2102, 0x2203, 0x3112, 0x3213, 0x3323};
    f4 accA[2] = {zero4(), zero4()}, accP[2] = {zero4(), zero4()};
#pragma unroll 1
    for (int ks = 0; ks < NKS; ++ks) {  // (kept rolled: unrolled, the slices' phases interleave and need ~200 registers)
        const int c0 = ks * KSL;
        tk.put(sX0, LH);
        tq.put(sT, LH);
        if constexpr (GATE != KDA_GATE_SCALAR) tg.put(sX1, LH);
        __syncthreads();
        // the next slice's loads fly during this slice's scan and products
        if (ks + 1 < NKS) load_slice(c0 + KSL, true);
        // b = cumsum(log2 alpha) per channel over the chunk;
        // Kh = 2^b K, Kb = 2^-b K, Qh = 2^b Q, gamma = 2^b_last
        gate_cumsum<KSL, NTH, GATE>(sX1, LH, sGs, len, sPart, [&](int r, int c, float b) {
            const float G = __builtin_amdgcn_exp2f(b), Gi = __builtin_amdgcn_exp2f(-b);
            const float kv = sX0[r * LH + c];
            sX0[r * LH + c] = G * kv;
            sX1[r * LH + c] = Gi * kv;
            sT[r * LH + c] *= G;
            if (r == C - 1) sGam[c0 + c] = G;
        });
        __syncthreads();
        if (tid < KSL) rec_at(P, h, g, R::GAM)[c0 + tid] = sGam[c0 + tid];
        if constexpr (!ABF16) {          // the 16-bit passes read Kt as fp16 fragments only
            float* gKt = rec_at(P, h, g, R::KT);
            for (int idx = tid; idx < C * KSL; idx += NTH) {
                const int r = idx / KSL, c = idx % KSL;
                gKt[r * DK + c0 + c] = sGam[c0 + c] * sX1[r * LH + c];
            }
        }
        store_block<NTH>(rec_at(P, h, g, R::QH) + c0, DK, sT, LH, C, KSL);
        if constexpr (ABF16) {
            // fp16 fragments of this slice for the 16-bit state passes: Kt
            // (its reduction blocks), Kt^T and Qh^T (their row blocks)
            write_afrags_part<C, DK, C / 16, KSL / 32, NTH>(hrec(R::FKT), 0, c0 / 32,
                [&](int m, int k) { return sGam[k] * sX1[m * LH + k - c0]; });
            write_afrags_part<DK, C, KSL / 16, C / 32, NTH>(hrec(R::FKTT), c0 / 16, 0,
                [&](int m, int k) { return sGam[m] * sX1[k * LH + m - c0]; });
            write_afrags_part<DK, C, KSL / 16, C / 32, NTH>(hrec(R::FQHT), c0 / 16, 0,
                [&](int m, int k) { return sT[k * LH + m - c0]; });
        }
#pragma unroll
        for (int slot = 0; slot < 2; ++slot) {
            const unsigned tt = (kTiles[wave] >> (8 * (1 - slot))) & 0xff;
            const int mb = tt >> 4, nb = tt & 15;
            if (nb <= mb)
                mm_two<KSL / 16, true, true>(sX0 + mb * 16 * LH, sT + mb * 16 * LH, LH, 1, sX1 + nb * 16 * LH, 1, LH,
                                             accA[slot], accP[slot]);
        }
        __syncthreads();                 // the slice tiles are read; the next slice (or P) may overwrite them
    }
    {
        float* gP = rec_at(P, h, g, R::P);
#pragma unroll
        for (int slot = 0; slot < 2; ++slot) {
            const unsigned tt = (kTiles[wave] >> (8 * (1 - slot))) & 0xff;
            const int mb = tt >> 4, nb = tt & 15;
            f4 a = accA[slot], pp = accP[slot];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = mb * 16 + 4 * j + e, s2 = nb * 16 + i;
                a[e] = s2 < r ? sBeta[r] * a[e] : 0.f;
                pp[e] = s2 <= r ? pp[e] : 0.f;
            }
            store_tile(sA + mb * 16 * LC + nb * 16, LC, a);
            if constexpr (ABF16) store_tile(sT + mb * 16 * LC + nb * 16, LC, pp);   // P, for P^T fragments
            else store_tile(gP + mb * 16 * C + nb * 16, C, pp);
        }
    }
    __syncthreads();
    if constexpr (ABF16) {
        write_afrags<C, C, NTH>(hrec(R::FPT), [&](int m, int k) { return sT[k * LC + m]; });
        __syncthreads();
    }
    // the W pass's inputs: V (read only here) and the key slices other than
    // the last, whose Gamma.K is still in sX0. bf16 tiles are issued before
    // the solve, which then hides their latency; fp32 tiles hold twice the
    // registers and would push the 16 x 16 substitution into scratch, so
    // they follow it
    Tok<ABF16, DV, KSL, NTH> tv[NVS];
    auto load_w_inputs = [&] {
        if (NKS > 1) load_slice(0, false);
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) tv[vs].load(P.v, row0, len, h, H, vs * KSL);
    };
    if constexpr (ABF16) load_w_inputs();
    solve_t(sA, sT, sX1);
    if constexpr (!ABF16) load_w_inputs();
    store_block<NTH>(rec_at(P, h, g, R::TT), C, sT, LC, C, C);

    // W = T Y, U = T Z (Y = Diag(beta) Gamma.K, Z = Diag(beta) V), one key
    // slice and one value slice per pass (key slices in the order NKS - 1,
    // 0, 1, ...): waves 0..3 the four 16-column blocks of W's slice, waves
    // 4..7 those of U's, all four row blocks sharing each B read (T lower
    // triangular: row block mb reduces over 16 (mb + 1) tokens).
    float* gW = rec_at(P, h, g, R::W);
    float* gU = rec_at(P, h, g, R::U);
#pragma unroll 1
    for (int it = 0; it < NIT; ++it) {
        const int c0 = (it == 0 ? NKS - 1 : it - 1) * KSL;   // this pass's key slice
        const int v0 = it * KSL;                             // and value slice
        if (it > 0 && it < NKS) {
            tk.put(sX0, LH);
            if constexpr (GATE != KDA_GATE_SCALAR) tg.put(sA, LH);
        }
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs)
            if (vs == it) tv[vs].put_scaled(sX1, LH, sBeta);
        __syncthreads();
        if (it > 0 && it + 1 < NKS) load_slice(it * KSL, false);
        if (it == 0) {
            for (int idx = tid; idx < C * KSL; idx += NTH) {
                const int r = idx / KSL, c = idx % KSL;
                sX0[r * LH + c] *= sBeta[r];
            }
        } else if (it < NKS) {
            gate_cumsum<KSL, NTH, GATE>(sA, LH, sGs, len, sPart, [&](int r, int c, float b) {
                sX0[r * LH + c] = (__builtin_amdgcn_exp2f(b) * sX0[r * LH + c]) * sBeta[r];
            });
        }
        __syncthreads();
        const bool isw = wave < 4;
        const int nb = wave & 3;
        if (isw ? it < NKS : it < NVS) {
            f4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
            mm_rows<4, C / 16, true, false>(sT, LC, 1, (isw ? sX0 : sX1) + nb * 16, LH, 1, 0, 1,
                                            [](int mb, int gg) { return gg <= mb; }, acc);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (isw) {
                    if constexpr (ABF16) store_tile(sA + mb * 16 * LC + nb * 16, LC, acc[mb]);   // W, for its fragments
                    else store_tile(gW + mb * 16 * DK + c0 + nb * 16, DK, acc[mb]);
                } else {
                    store_tile(gU + mb * 16 * DV + v0 + nb * 16, DV, acc[mb]);
                }
            }
        }
        if constexpr (ABF16) {
            if (it < NKS) {
                __syncthreads();
                write_afrags_part<C, DK, C / 16, KSL / 32, NTH>(hrec(R::FW), 0, c0 / 32,
                    [&](int m, int k) { return sA[m * LC + k - c0]; });
                write_afrags_part<DK, C, KSL / 16, C / 32, NTH>(hrec(R::FWT), c0 / 16, 0,
                    [&](int m, int k) { return sA[k * LC + m - c0]; });
            }
        }
        __syncthreads();                 // before the next pass overwrites the slice tiles
    }
    if (wave == 0) {                     // gamma (sGam) is left untouched since the scans
        bool bad = false;
#pragma unroll
        for (int c = lane; c < DK; c += 64) bad |= sGam[c] < kFastGammaMin;
        const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) {
            P.flag[g * H + h] = any;
            if (any) P.slow[atomicAdd(P.nslow, 1)] = g * H + h;
        }
    }
}

// One workgroup per (chunk, head): the direct form (two per CU).
template <int DK, int DV, bool ABF16, int GATE>
__global__ __launch_bounds__(kPrepThreads, 4) void bwd_prep_kernel(const BwdParams P) {
    const int g = blockIdx.x / P.H;
    if (g >= P.ctrl[0]) return;
    prep_direct_body<DK, DV, ABF16, GATE>(P, blockIdx.x % P.H, g);
}

// Entry blockIdx.x of the general list, if the list is that long (the grid
// has one workgroup per (chunk, head), the list's largest length; a loop over
// the entries would keep the body's loop-invariant values live throughout).
template <int DK, int DV, bool ABF16, int GATE>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_general_kernel(const BwdParams P) {
    if (static_cast<int>(blockIdx.x) >= *P.nslow) return;
    const int id = P.slow[blockIdx.x];
    prep_general_body<DK, DV, ABF16, GATE>(P, id % P.H, id / P.H);
}

// ---------------------------------------------------------------------------
// Sequential passes: one 512-thread WG per (sequence, head, 16 value
// columns).  The d_k x 16 state tile is kept in registers, row block rb in
// wave rb (and rb - 8 for d_k > 128); the C x 16 per-chunk product (U' or
// dU') is split over the two halves of the workgroup, waves 4..7 handing
// their partial sums to waves 0..3 through LDS.
// ---------------------------------------------------------------------------
constexpr int kChainThreads = 512, kChainWaves = kChainThreads / 64;

template <int DK> struct CkptB {
    static constexpr int LK = Ld<DK>::value;
    static constexpr int bytes = (2 * C * LK + DK * L16 + 2 * C * L16 + DK) * 4;
};

template <int DK, int DV>
__global__ __launch_bounds__(kChainThreads) void bwd_ckpt_kernel(const BwdParams P) {
    using R = BRec<DK, DV, false>;
    constexpr int NTH = kChainThreads, NW = kChainWaves;
    constexpr int LK = CkptB<DK>::LK, NT = DV / 16, NRB = DK / 16, RBW = (NRB + NW - 1) / NW;
    extern __shared__ float lds[];
    float* sW = lds;                 // [C][LK]
    float* sKt = sW + C * LK;        // [C][LK]
    float* sS = sKt + C * LK;        // [DK][16]
    float* sU = sS + DK * L16;       // [C][16]
    float* sPart = sU + C * L16;     // [C][16] partial W S from waves 4..7
    float* sGam = sPart + C * L16;   // [DK]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int n = P.order[pair / P.H], h = pair % P.H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = wave_id(), j = lane_id() >> 4;
    const int c0 = tile * 16;
    const int mb = wave & 3, khalf = wave >> 2;          // U' row block and half of the d_k reduction

    f4 S[RBW];
    for (int u = 0; u < RBW; ++u) {
        const int rb = wave + NW * u;
        S[u] = (P.initial_state && rb < NRB)
                   ? load_tile(P.initial_state + (static_cast<size_t>(n) * P.H + h) * DK * DV + rb * 16 * DV + c0, DV)
                   : zero4();
    }
    // the next chunk's operands, in flight while the current one computes
    Blk<C, DK, NTH> nW, nKt;
    f4 nU = zero4();
    float nGam = 0.f;
    auto fetch = [&](int g) {
        nW.load(rec_at(P, h, g, R::W), DK);
        nKt.load(rec_at(P, h, g, R::KT), DK);
        if (khalf == 0) nU = load_tile(rec_at(P, h, g, R::U) + mb * 16 * DV + c0, DV);
        if (threadIdx.x < DK) nGam = rec_at(P, h, g, R::GAM)[threadIdx.x];
    };
    if (g0 < g1) fetch(g0);
    for (int g = g0; g < g1; ++g) {
        nW.put(sW, LK);
        nKt.put(sKt, LK);
        const f4 uu = nU;
        if (threadIdx.x < DK) sGam[threadIdx.x] = nGam;
        float* gS = rec_at(P, h, g, R::SIN);
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(sS + rb * 16 * L16, L16, S[u]);
            store_tile(gS + rb * 16 * DV + c0, DV, S[u]);
        }
        __syncthreads();
        if (g + 1 < g1) fetch(g + 1);
        // U' = U - W S  (row block mb, d_k split over the two halves)
        const f4 x = mm<DK / 2, true, false>(sW + mb * 16 * LK + khalf * (DK / 2), LK, 1,
                                             sS + khalf * (DK / 2) * L16, L16, 1, zero4());
        if (khalf) store_tile(sPart + mb * 16 * L16, L16, x);
        __syncthreads();
        if (!khalf) {
            const f4 uc = uu - x - load_tile(sPart + mb * 16 * L16, L16);
            store_tile(sU + mb * 16 * L16, L16, uc);
            store_tile(rec_at(P, h, g, R::UC) + mb * 16 * DV + c0, DV, uc);
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
}

template <int DK> struct RevB {
    static constexpr int LK = Ld<DK>::value;
    static constexpr int bytes = (C * LC + 3 * C * LK + 3 * C * L16 + DK * L16 + DK) * 4;
};

// chunks last to first
template <int DK, int DV, bool ABF16>
__global__ __launch_bounds__(kChainThreads) void bwd_rev_kernel(const BwdParams P) {
    using R = BRec<DK, DV, false>;
    constexpr int NTH = kChainThreads, NW = kChainWaves;
    constexpr int LK = RevB<DK>::LK, NT = DV / 16, NRB = DK / 16, RBW = (NRB + NW - 1) / NW;
    extern __shared__ float lds[];
    float* sP = lds;                 // [C][LC]
    float* sKt = sP + C * LC;        // [C][LK]
    float* sQh = sKt + C * LK;       // [C][LK]
    float* sW = sQh + C * LK;        // [C][LK]
    float* sdO = sW + C * LK;        // [C][16]
    float* sdU = sdO + C * L16;      // [C][16]
    float* sPart = sdU + C * L16;    // [C][16] partial P^T dO from waves 4..7
    float* sdS = sPart + C * L16;    // [DK][16]
    float* sGam = sdS + DK * L16;    // [DK]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int H = P.H;
    const int n = P.order[pair / H], h = pair % H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = wave_id(), j = lane_id() >> 4;
    const int c0 = tile * 16;
    const int mb = wave & 3, half = wave >> 2;           // dU' row block; half 0: Kt dS, half 1: P^T dO
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;

    f4 dS[RBW];
    for (int u = 0; u < RBW; ++u) {
        const int rb = wave + NW * u;
        dS[u] = (P.dfinal_state && rb < NRB) ? load_tile(P.dfinal_state + sbase + rb * 16 * DV + c0, DV) : zero4();
    }
    // the next (earlier) chunk's operands, in flight while the current one computes
    Blk<C, C, NTH> nP;
    Blk<C, DK, NTH> nKt, nQh, nW;
    Tok<ABF16, DV, 16, NTH> ndO;
    float nGam = 0.f;
    auto fetch = [&](int g) {
        const int4 ent = P.table[g];
        nP.load(rec_at(P, h, g, R::P), C);
        nKt.load(rec_at(P, h, g, R::KT), DK);
        nQh.load(rec_at(P, h, g, R::QH), DK);
        nW.load(rec_at(P, h, g, R::W), DK);
        ndO.load(P.dout, ent.y, ent.z, h, H, c0);
        if (threadIdx.x < DK) nGam = rec_at(P, h, g, R::GAM)[threadIdx.x];
    };
    if (g1 > g0) fetch(g1 - 1);
    for (int g = g1 - 1; g >= g0; --g) {
        nP.put(sP, LC);
        nKt.put(sKt, LK);
        nQh.put(sQh, LK);
        nW.put(sW, LK);
        ndO.put(sdO, L16);
        if (threadIdx.x < DK) sGam[threadIdx.x] = nGam;
        float* gdS = rec_at(P, h, g, R::DSO);
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(sdS + rb * 16 * L16, L16, dS[u]);
            store_tile(gdS + rb * 16 * DV + c0, DV, dS[u]);
        }
        __syncthreads();
        if (g > g0) fetch(g - 1);
        // dU' = Kt dS + P^T dO  (row block mb; P^T[m][k] = P[k][m], zero for k < m)
        f4 acc;
        if (half == 0) {
            acc = mm<DK, true, false>(sKt + mb * 16 * LK, LK, 1, sdS, L16, 1, zero4());
        } else {
            acc = mm_n<false, false>(sP + mb * 16 * LC + mb * 16, 1, LC, sdO + mb * 16 * L16, L16, 1, C - mb * 16,
                                     zero4());
            store_tile(sPart + mb * 16 * L16, L16, acc);
        }
        __syncthreads();
        if (half == 0) {
            acc += load_tile(sPart + mb * 16 * L16, L16);
            store_tile(sdU + mb * 16 * L16, L16, acc);
            store_tile(rec_at(P, h, g, R::DUC) + mb * 16 * DV + c0, DV, acc);
        }
        __syncthreads();
        // dS <- Diag(gamma) dS + Qh^T dO - W^T dU'
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            f4 sv = dS[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] *= sGam[rb * 16 + 4 * j + e];
            sv = mm<C, false, false>(sQh + rb * 16, 1, LK, sdO, L16, 1, sv);
            const f4 x = mm<C, false, false>(sW + rb * 16, 1, LK, sdU, L16, 1, zero4());
            dS[u] = sv - x;
        }
        __syncthreads();
    }
    if (P.dinitial_state) {
        for (int u = 0; u < RBW; ++u) {
            const int rb = wave + NW * u;
            if (rb >= NRB) continue;
            store_tile(P.dinitial_state + sbase + rb * 16 * DV + c0, DV, dS[u]);
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit activations: the same two state passes on the fp16 matrix cores
// (16x16x32), as the forward's state pass does.  Each wave reads its A
// fragments (Kt, P^T, Qh^T, W^T; or W, Kt^T) straight from the record,
// fragment-major, ahead of the chain; the B operands (dO, dS, dU'; or S, U')
// pass through LDS as column-major fp16 tiles.  The states and their
// gradients stay fp32 in registers; the state entering each chunk, the
// state gradient, U' and dU' go to the record in fp16 (their one reader,
// the 16-bit value side of the gradient kernel, takes them as fp16 operands
// anyway).  Waves 0..3 compute the C x 16 product (row block = wave), every
// wave one 16-row block of the d_k x 16 state tile.
// ---------------------------------------------------------------------------
template <int DK> struct Chain16B {
    static constexpr int KPD = DK + 8, KPC = C + 8;      // column-major tile strides (halves)
    static constexpr int sink = (3 * 16 * KPC + 16 * KPD) * 2;   // byte offset of the prefetch sink
    static constexpr int bytes = sink + 64 * 4;
};
// Eight compute waves and one wave that brings the records (and dO rows) of
// the chunk kChainPrefetch steps ahead of the chain into the XCD's L2; the
// compute waves load each chunk's operands two (checkpoint pass) or one
// (reverse pass, whose operands take more registers) steps ahead.  The prefetch
// wave passes the same two barriers per chunk, bare (a fenced barrier would
// wait for its loads).
constexpr int kChain16Threads = kChainThreads + 64, kChainPrefetch = 3;

template <int DK, int DV>
__global__ __launch_bounds__(kChain16Threads) void bwd_rev16_kernel(const BwdParams P) {
    using R = BRec<DK, DV, true>;
    constexpr int NT = DV / 16, NRB = DK / 16;
    constexpr int KPD = Chain16B<DK>::KPD, KPC = Chain16B<DK>::KPC, NKD = DK / 32, NKC = C / 32;
    extern __shared__ float lds[];
    _Float16* sdO2 = reinterpret_cast<_Float16*>(lds);   // dO tile, column-major, by chunk parity  [2][16][KPC]
    _Float16* sdU = sdO2 + 2 * 16 * KPC;                 // dU'                   [16][KPC]
    _Float16* sdS = sdU + 16 * KPC;                      // dS                    [16][KPD]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int H = P.H;
    const int n = P.order[pair / H], h = pair % H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = wave_id(), lane = lane_id(), j = lane >> 4;
    const int c0 = tile * 16;
    const bool du = wave < 4, hasrb = wave < NRB;
    const int mb = wave & 3, rb = wave;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;

    f4 dS = (P.dfinal_state && hasrb) ? load_tile(P.dfinal_state + sbase + rb * 16 * DV + c0, DV) : zero4();
    auto hrec = [&](int g, size_t off) {
        return reinterpret_cast<const _Float16*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
    };
    auto hrec_w = [&](int g, size_t off) {
        return reinterpret_cast<_Float16*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
    };
    // gamma: one word per lane (a 16-byte load per lane of the four rows in
    // the accumulator layout asks the address path for 1 KiB per wave for 64
    // distinct bytes); the lanes then trade them into the tile's rows
    auto gam_word = [&](int g) { return rec_at(P, h, g, R::GAM)[rb * 16 + (lane & 15)]; };
    auto gam_rows = [&](float w) {
        f4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * j + i) << 2, __float_as_int(w)));
        return r;
    };
    // The next (earlier) chunk's operands, loaded while the current chunk
    // computes.  A sequence's chunks are consecutive rows of C tokens, so the
    // dO rows of chunk g follow from the sequence's first row and last
    // length (no per-chunk table load for a prefetch to wait on).
    const int row_first = g1 > g0 ? P.table[g0].y : 0;
    const int len_last = g1 > g0 ? P.table[g1 - 1].z : 0;
    if (wave == kChainWaves) {
        int* sink = reinterpret_cast<int*>(reinterpret_cast<unsigned char*>(lds) + Chain16B<DK>::sink);
        auto touch = [&](int gp) {
            l2_touch(hrec(gp, R::FKT), C * DK * 2, tile, NT, sink);
            l2_touch(hrec(gp, R::FPT), C * C * 2, tile, NT, sink);
            l2_touch(hrec(gp, R::FQHT), C * DK * 2, tile, NT, sink);
            l2_touch(hrec(gp, R::FWT), C * DK * 2, tile, NT, sink);
            l2_touch(rec_at(P, h, gp, R::GAM), DK * 4, tile, NT, sink);
            const int len = gp == g1 - 1 ? len_last : C;
            if (lane < len) {
                const size_t row = static_cast<size_t>(row_first) + (gp - g0) * C + lane;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(static_cast<const uint16_t*>(P.dout) +
                                                                    (row * H + h) * DV + c0),
                    (__attribute__((address_space(3))) void*)sink, 4, 0, 0);
            }
        };
        for (int gp = g1 - 2; gp >= max(g1 - kChainPrefetch, g0); --gp) touch(gp);
        for (int g = g1 - 1; g >= g0; --g) {
            if (g - kChainPrefetch >= g0) touch(g - kChainPrefetch);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);       // every load has landed before the wave ends
        return;
    }
    const int dr = threadIdx.x >> 2, dc = 4 * (threadIdx.x & 3);      // dO element rows / columns of this thread
    // Two operand stages: the operands of chunk g - 1 are loaded while chunk g
    // computes (the loop is unrolled by two so stage indices stay static; a
    // third stage would exceed the registers nine waves leave).  Each wave
    // role runs its own copy of the loop, so no load or store sits under a
    // per-wave branch and the compiler counts what is in flight instead of
    // draining every load each chunk.
    struct Stage {
        h8 kt[NKD], pt[NKC], qt[NKC], wt[NKC];
        u16x4 dO;
        float gam;                       // gamma of row rb * 16 + lane mod 16
        int len;
    };
    auto run = [&](auto du_c, auto rb_c) {
        constexpr bool DU = decltype(du_c)::value, RB = decltype(rb_c)::value;
        auto fetch = [&](Stage& st, int g) {
            const int row0 = row_first + (g - g0) * C, len = g == g1 - 1 ? len_last : C;
            st.len = len;
            if constexpr (RB) st.gam = gam_word(g);
            if constexpr (DU) {              // waves 0..3: dU' row block mb, and the dO tile (threads 0..4C-1)
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) st.kt[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FKT) + afrag_off(mb, kb, NKD, lane));
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) st.pt[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FPT) + afrag_off(mb, kb, NKC, lane));
                const int rr = dr < len ? dr : len - 1;
                st.dO = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(P.dout) +
                                                       (static_cast<size_t>(row0 + rr) * H + h) * DV + c0 + dc);
            }
            if constexpr (RB) {
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    st.qt[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FQHT) + afrag_off(rb, kb, NKC, lane));
                    st.wt[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FWT) + afrag_off(rb, kb, NKC, lane));
                }
            }
        };
        auto step = [&](const Stage& cur, Stage& nxt, int g) {
            _Float16* sdO = sdO2 + (g & 1) * 16 * KPC;
            if constexpr (DU) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sdO[(dc + e) * KPC + dr] = static_cast<_Float16>(dr < cur.len ? bf16_to_f32(cur.dO[e]) : 0.f);
            }
            if constexpr (RB) put_btile(sdS, KPD, rb * 16, dS);
            __syncthreads();
            fetch(nxt, max(g - 1, g0));          // unconditional (past the start: re-reads the first chunk)
            f4 gv = zero4();
            if constexpr (RB) gv = gam_rows(cur.gam);
            // dU' = Kt dS + P^T dO   (P^T[m][k] = P[k][m], zero for k < m); waves 4..7
            // meanwhile write dS to the record as 16-byte row words
            if constexpr (DU) {
                f4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) acc = mfma16(cur.kt[kb], bfrag(sdS, KPD, kb), acc);
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    if (32 * kb + 31 >= 16 * mb) acc = mfma16(cur.pt[kb], bfrag(sdO, KPC, kb), acc);
                put_btile(sdU, KPC, mb * 16, acc);
            } else {
                store_ctile16<DK, kChainThreads / 2>(hrec_w(g, R::DSO) + c0, DV, sdS, KPD, threadIdx.x - kChainThreads / 2);
            }
            __syncthreads();
            if constexpr (!DU)
                store_ctile16<C, kChainThreads / 2>(hrec_w(g, R::DUC) + c0, DV, sdU, KPC, threadIdx.x - kChainThreads / 2);
            // dS <- Diag(gamma) dS + Qh^T dO - W^T dU'.  No barrier after: the next
            // chunk writes dS and its own dO buffer before its first barrier, and
            // dU' after it.
            if constexpr (RB) {
                f4 x = dS * gv, y = zero4();
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    x = mfma16(cur.qt[kb], bfrag(sdO, KPC, kb), x);
                    y = mfma16(cur.wt[kb], bfrag(sdU, KPC, kb), y);
                }
                dS = x - y;
            }
        };
        if (g0 >= g1) return;
        Stage st0, st1;
        fetch(st0, g1 - 1);
        int g = g1 - 1;
        for (; g - 1 >= g0; g -= 2) {        // whole rounds: straight-line code
            step(st0, st1, g);
            step(st1, st0, g - 1);
        }
        if (g >= g0) step(st0, st1, g);
    };
    if (du) run(std::true_type{}, std::true_type{});            // waves 0..3 own a row block of dU' and of dS
    else if (hasrb) run(std::false_type{}, std::true_type{});
    else run(std::false_type{}, std::false_type{});
    if (P.dinitial_state && hasrb) store_tile(P.dinitial_state + sbase + rb * 16 * DV + c0, DV, dS);
}

template <int DK, int DV>
__global__ __launch_bounds__(kChain16Threads) void bwd_ckpt16_kernel(const BwdParams P) {
    using R = BRec<DK, DV, true>;
    constexpr int NT = DV / 16, NRB = DK / 16;
    constexpr int KPD = Chain16B<DK>::KPD, KPC = Chain16B<DK>::KPC, NKD = DK / 32, NKC = C / 32;
    extern __shared__ float lds[];
    _Float16* sU = reinterpret_cast<_Float16*>(lds);     // U', column-major        [16][KPC]
    _Float16* sS = sU + 2 * 16 * KPC;                    // S                       [16][KPD]

    int tile, pair;
    chain_coords<NT>(tile, pair);
    if (pair >= P.N * P.H) return;
    const int n = P.order[pair / P.H], h = pair % P.H;
    const int g0 = P.first[n], g1 = P.first[n + 1];
    const int wave = wave_id(), lane = lane_id(), j = lane >> 4;
    const int c0 = tile * 16;
    const bool du = wave < 4, hasrb = wave < NRB;
    const int mb = wave & 3, rb = wave;

    f4 S = (P.initial_state && hasrb)
               ? load_tile(P.initial_state + (static_cast<size_t>(n) * P.H + h) * DK * DV + rb * 16 * DV + c0, DV)
               : zero4();
    auto hrec = [&](int g, size_t off) {
        return reinterpret_cast<const _Float16*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
    };
    auto hrec_w = [&](int g, size_t off) {
        return reinterpret_cast<_Float16*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
    };
    // gamma: one word per lane (a 16-byte load per lane of the four rows in
    // the accumulator layout asks the address path for 1 KiB per wave for 64
    // distinct bytes); the lanes then trade them into the tile's rows
    auto gam_word = [&](int g) { return rec_at(P, h, g, R::GAM)[rb * 16 + (lane & 15)]; };
    auto gam_rows = [&](float w) {
        f4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * j + i) << 2, __float_as_int(w)));
        return r;
    };
    if (wave == kChainWaves) {
        int* sink = reinterpret_cast<int*>(reinterpret_cast<unsigned char*>(lds) + Chain16B<DK>::sink);
        auto touch = [&](int gp) {
            l2_touch(hrec(gp, R::FW), C * DK * 2, tile, NT, sink);
            l2_touch(hrec(gp, R::FKTT), C * DK * 2, tile, NT, sink);
            l2_touch(rec_at(P, h, gp, R::U), C * DV * 4, tile, NT, sink);
            l2_touch(rec_at(P, h, gp, R::GAM), DK * 4, tile, NT, sink);
        };
        for (int gp = g0 + 1; gp < min(g0 + kChainPrefetch, g1); ++gp) touch(gp);
        for (int g = g0; g < g1; ++g) {
            if (g + kChainPrefetch < g1) touch(g + kChainPrefetch);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);       // every load has landed before the wave ends
        return;
    }
    // A ring of three operand stages: the operands of chunk g + 2 are loaded
    // while chunk g computes (stage indices stay static: the loop is unrolled
    // by three).  Each wave role runs its own copy of the loop, so no load or
    // store sits under a per-wave branch and the compiler can count what is
    // still in flight instead of draining every load each chunk.
    struct Stage {
        h8 w[NKD], ktt[NKC];
        f4 u;
        float gam;                       // gamma of row rb * 16 + lane mod 16
    };
    auto run = [&](auto du_c, auto rb_c) {
        constexpr bool DU = decltype(du_c)::value, RB = decltype(rb_c)::value;
        auto fetch = [&](Stage& st, int g) {
            if constexpr (RB) st.gam = gam_word(g);
            if constexpr (DU) {
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) st.w[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FW) + afrag_off(mb, kb, NKD, lane));
                st.u = load_tile(rec_at(P, h, g, R::U) + mb * 16 * DV + c0, DV);
            }
            if constexpr (RB) {
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    st.ktt[kb] = *reinterpret_cast<const h8*>(hrec(g, R::FKTT) + afrag_off(rb, kb, NKC, lane));
            }
        };
        auto step = [&](const Stage& cur, Stage& nxt, int g) {
            if constexpr (RB) put_btile(sS, KPD, rb * 16, S);
            __syncthreads();
            fetch(nxt, min(g + 2, g1 - 1));      // unconditional (past the end: re-reads the last chunk)
            f4 gv = zero4();
            if constexpr (RB) gv = gam_rows(cur.gam);
            // U' = U - W S; waves 4..7 meanwhile write S to the record as 16-byte row words
            if constexpr (DU) {
                f4 x = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) x = mfma16(cur.w[kb], bfrag(sS, KPD, kb), x);
                const f4 uc = cur.u - x;
                put_btile(sU, KPC, mb * 16, uc);
            } else {
                store_ctile16<DK, kChainThreads / 2>(hrec_w(g, R::SIN) + c0, DV, sS, KPD, threadIdx.x - kChainThreads / 2);
            }
            __syncthreads();
            if constexpr (!DU)
                store_ctile16<C, kChainThreads / 2>(hrec_w(g, R::UC) + c0, DV, sU, KPC, threadIdx.x - kChainThreads / 2);
            // S <- Diag(gamma) S + Kt^T U'.  No barrier after: the next chunk
            // writes S before its first barrier (every read of S is before this
            // chunk's second one) and U' after it.
            if constexpr (RB) {
                f4 sv = S * gv;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) sv = mfma16(cur.ktt[kb], bfrag(sU, KPC, kb), sv);
                S = sv;
            }
        };
        if (g0 >= g1) return;
        Stage st0, st1, st2;
        fetch(st0, g0);
        fetch(st1, min(g0 + 1, g1 - 1));
        int g = g0;
        for (; g + 2 < g1; g += 3) {         // whole rounds: straight-line code
            step(st0, st2, g);
            step(st1, st0, g + 1);
            step(st2, st1, g + 2);
        }
        if (g < g1) step(st0, st2, g);
        if (g + 1 < g1) step(st1, st0, g + 1);
    };
    if (du) run(std::true_type{}, std::true_type{});            // waves 0..3 own a row block of U' and of S
    else if (hasrb) run(std::false_type{}, std::true_type{});
    else run(std::false_type{}, std::false_type{});
}

// ---------------------------------------------------------------------------
// bwd_grad_kernel: every per-chunk gradient, after the two state passes.  One
// 512-thread WG per (chunk, head), in two phases over the same LDS:
//
//   value side  every contraction over d_v (dO S^T, dU' S^T, U' dS_next^T,
//               M = Tril(dO U'^T), N = dU' V^T, dgamma), dZ = T^T dU' and
//               dv = beta . dZ; the products stay in the accumulators of the
//               waves that consume them below (only dW and M pass through LDS)
//   key side    dT, dA, R, dY, dKh, dQh, dKb, the gate chain rule, dq, dk,
//               dgate, dbeta
//
// Task numbering of the value-side products (t = wave + 8 k, accumulator k):
//   t < 12 NB            dO S^T, dU' S^T, U' dS_next^T: tile (mb, nb) of the
//                        which-th product at which * 4 NB + mb * NB + nb
//   12 NB + 4 mb + nb    M tile (mb, nb), zero above the diagonal
//   12 NB + 16 + ...     N tile (mb, nb)
// so with NB = d_k / 16 key column blocks the C x d_k tiles of wave w are
// column block w % NB, row blocks w / NB + r 8 / NB (r < NB / 2), and its
// C x C tiles are column block w % 4, row blocks w / 4 and w / 4 + 2: the
// ownership of the key-side phase.
// ---------------------------------------------------------------------------
constexpr int kGradThreads = 512, kGradWaves = kGradThreads / 64;

template <int DK> struct GradTasks {
    static constexpr int NB = DK / 16;          // key column blocks
    static constexpr int RW = NB / 2;           // tiles of one C x d_k product per wave
    static constexpr int MSTEP = 8 / NB;        // row-block step between them (= waves per column block)
    static constexpr int KM = 12 * NB / 8;      // accumulator of the wave's first M tile (then M, N, N)
    static constexpr int NTASK = 12 * NB + 32;
    static constexpr int KT = NTASK / 8;
    static_assert(NB == 4 || NB == 8, "d_k of 64 or 128");
};

// dA / R tiles of wave w in the gradient kernel: (mb, nb) of its first and
// second tile, 4 bits each.  Tile (mb, nb) below the diagonal costs
// 8 + nb + 1 product steps; the spread gives the waves sharing a SIMD
// (w, w + 4) 28, 28, 22, 22 steps; tiles above the diagonal are only zeroed.
constexpr unsigned grad_tiles(int w) {
    constexpr unsigned t[8] = {0x0010, 0x2030, 0x3301, 0x2202, 0x1103, 0x2112, 0x3113, 0x3223};
    return t[w];
}

template <int DK> struct GradB {
    static constexpr int LK = Ld<DK>::value;
    // key side: K, b, dW | three C x C tiles | beta, dbeta rows, Kt.dKt column sums, dgamma, rowsum(dZ.V),
    // tile totals of log2 alpha
    static constexpr int region = (3 * C * LK + 2 * C * LC) * 4;   // value-side scratch: everything before T
    static constexpr int bytes =
        (3 * C * LK + 3 * C * LC + C + kGradWaves * C + GradTasks<DK>::MSTEP * DK + DK + C + (C / 16) * DK) * 4;
};

// Decode value-side task t: operand rows of A and B (row-major, reduction
// along the row) and whether the tile is computed at all.
template <int NB, typename E>
__device__ __forceinline__ bool grad_task(int t, const E* sdO, const E* sdU, const E* sUc, const E* sS,
                                          const E* sdS, const E* sV, int ld, const E*& pa, const E*& pb) {
    if (t < 12 * NB) {
        const int which = t / (4 * NB), tt = t % (4 * NB), mb = tt / NB, nb = tt % NB;
        pa = (which == 0 ? sdO : which == 1 ? sdU : sUc) + mb * 16 * ld;
        pb = (which == 2 ? sdS : sS) + nb * 16 * ld;
        return true;
    }
    const int tt = (t - 12 * NB) & 15, mb = tt >> 2, nb = tt & 3;
    if (t < 12 * NB + 16) {
        pa = sdO + mb * 16 * ld;
        pb = sUc + nb * 16 * ld;
        return nb <= mb;
    }
    pa = sdU + mb * 16 * ld;
    pb = sV + nb * 16 * ld;
    return true;
}

// Value side, fp32 activations: the value dimension in slices of kSW
// columns, fp32 matrix cores; sT holds T (fp32), sBeta beta.
constexpr int kSW = 32, kLS = kSW + 4;

template <int DK, int DV>
__device__ __forceinline__ void vside_phase32(const BwdParams& P, int h, int g, int64_t row0, int len, float* region,
                                              float* sT, float* sBeta, f4 (&acc)[GradTasks<DK>::KT],
                                              float* sDgam, float* sDbz) {
    using R = BRec<DK, DV, false>;
    using GT = GradTasks<DK>;
    constexpr int NTH = kGradThreads, NB = GT::NB, KT = GT::KT;
    static_assert((2 * DK * kLS + 4 * C * kLS + 2 * C) * 4 <= GradB<DK>::region, "value-side scratch fits");
    float* sS = region;              // S[:, slice]        [DK][kLS]
    float* sdS = sS + DK * kLS;      // dS_next[:, slice]  [DK][kLS]
    float* sdO = sdS + DK * kLS;     // [C][kLS]
    float* sUc = sdO + C * kLS;      // [C][kLS]
    float* sdU = sUc + C * kLS;      // [C][kLS]
    float* sV = sdU + C * kLS;       // [C][kLS]
    float* sDbzP = sV + C * kLS;     // rowsum(dZ . V), one row per column half  [2][C]
    const int H = P.H, tid = threadIdx.x, wave = wave_id(), i = lane_id() & 15, j = lane_id() >> 4;

    // value slices, the next one in flight while the current one computes
    Blk<DK, kSW, NTH> nS, ndS;
    Blk<C, kSW, NTH> nUc, ndU;
    Tok<false, DV, kSW, NTH> ndO, nV;
    auto fetch = [&](int s0) {
        nS.load(rec_at(P, h, g, R::SIN) + s0, DV);
        ndS.load(rec_at(P, h, g, R::DSO) + s0, DV);
        nUc.load(rec_at(P, h, g, R::UC) + s0, DV);
        ndU.load(rec_at(P, h, g, R::DUC) + s0, DV);
        ndO.load(P.dout, row0, len, h, H, s0);
        nV.load(P.v, row0, len, h, H, s0);
    };
    fetch(0);
    load_block<C, C, NTH>(sT, LC, rec_at(P, h, g, R::TT), C);
    if (tid < C) sBeta[tid] = tid < len ? P.beta[(row0 + tid) * H + h] : 0.f;
#pragma unroll
    for (int k = 0; k < KT; ++k) acc[k] = zero4();
    float dgam = 0.f;
    float dbz[4] = {0.f, 0.f, 0.f, 0.f};
    const int zmb = wave >> 1, znb = wave & 1;      // this wave's block of dZ = T^T dU'[:, slice]

    for (int s0 = 0; s0 < DV; s0 += kSW) {
        nS.put(sS, kLS);
        ndS.put(sdS, kLS);
        nUc.put(sUc, kLS);
        ndU.put(sdU, kLS);
        ndO.put(sdO, kLS);
        nV.put(sV, kLS);
        __syncthreads();
        if (s0 + kSW < DV) fetch(s0 + kSW);
        if (tid < DK) {
#pragma unroll 8
            for (int c = 0; c < kSW; ++c) dgam += sdS[tid * kLS + c] * sS[tid * kLS + c];
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const float *pa, *pb;
            if (grad_task<NB>(wave + 8 * k, sdO, sdU, sUc, sS, sdS, sV, kLS, pa, pb))
                acc[k] = mm<kSW, true, true>(pa, kLS, 1, pb, 1, kLS, acc[k]);
        }
        // dZ = T^T dU'[:, slice] (T^T[m][k] = T[k][m], zero for k < m); dv = beta . dZ
        {
            const f4 z = mm_n<false, false>(sT + zmb * 16 * LC + zmb * 16, 1, LC, sdU + zmb * 16 * kLS + znb * 16, kLS, 1,
                              C - zmb * 16, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = zmb * 16 + 4 * j + e, col = s0 + znb * 16 + i;
                if (r < len) store_out<false>(P.dv, (static_cast<size_t>(row0 + r) * H + h) * DV + col, sBeta[r] * z[e]);
                dbz[e] += z[e] * sV[r * kLS + znb * 16 + i];
            }
        }
        __syncthreads();
    }
    if (tid < DK) sDgam[tid] = dgam;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x = row16_sum(dbz[e]);
        if (i == 0) sDbzP[znb * C + zmb * 16 + 4 * j + e] = x;
    }
    __syncthreads();
    if (tid < C) sDbz[tid] = sDbzP[tid] + sDbzP[C + tid];
}

// Value side, 16-bit activations: fp16 matrix cores, the value dimension in
// slices of 64 columns.  S, dS_next, U', dU' (fp16 in the record), dO and V
// are staged row-major in LDS, so both operands of every product read their
// 8 reduction indices as one 16-byte word; T^T and a transposed copy of dU'
// serve dZ = T^T dU'.
template <int DK, int DV> struct V16L {
    static constexpr int SW = DV < 64 ? DV : 64, RS = SW + 8, CS = C + 8, NZB = SW / 16;
    static constexpr int bytes = (2 * DK * RS + 4 * C * RS + SW * CS + C * CS) * 2 + NZB * C * 4 + C * RS * 2;
};

template <int DK, int DV>
__device__ __forceinline__ void vside_phase16(const BwdParams& P, int h, int g, int64_t row0, int len, float* region,
                                              float* sT, float* sBeta, f4 (&acc)[GradTasks<DK>::KT],
                                              float* sDgam, float* sDbz) {
    using R = BRec<DK, DV, true>;
    using VB = V16L<DK, DV>;
    using GT = GradTasks<DK>;
    constexpr int NTH = kGradThreads, SW = VB::SW, RS = VB::RS, CS = VB::CS, NZB = VB::NZB, NKS = SW / 32;
    constexpr int NB = GT::NB, KT = GT::KT;
    static_assert(VB::bytes <= GradB<DK>::region, "value-side scratch fits");
    _Float16* sS = reinterpret_cast<_Float16*>(region);   // S[:, slice]         [DK][RS]
    _Float16* sdS = sS + DK * RS;                          // dS_next[:, slice]   [DK][RS]
    _Float16* sdO = sdS + DK * RS;                         // [C][RS]
    _Float16* sUc = sdO + C * RS;                          // [C][RS]
    _Float16* sdU = sUc + C * RS;                          // [C][RS]
    _Float16* sV = sdU + C * RS;                           // [C][RS]
    _Float16* sdUt = sV + C * RS;                          // dU'[:, slice]^T     [SW][CS]
    _Float16* sTt = sdUt + SW * CS;                        // T^T                 [C][CS]
    float* sDbzP = reinterpret_cast<float*>(sTt + C * CS); // rowsum(dZ . V) per column block  [NZB][C]
    uint16_t* sDv = reinterpret_cast<uint16_t*>(sDbzP + NZB * C);   // dv of the slice, bf16   [C][RS]
    const int H = P.H, tid = threadIdx.x, wave = wave_id(), lane = lane_id(), i = lane & 15, j = lane >> 4;
    auto hrec = [&](size_t off) {
        return reinterpret_cast<const _Float16*>(P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes + off);
    };

    // Staged slices: every global load of a slice is issued before the first
    // LDS store, and the next slice's loads are in flight while the current
    // slice computes.  fp16 record rows ([rows][DV] halves) and activation rows
    // (clamped to the chunk, zeroed past its end) in 16-byte words.
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    constexpr int W8 = SW / 8, NSK = (DK * W8 + NTH - 1) / NTH, NSC = (C * W8 + NTH - 1) / NTH;
    h8 nS[NSK], ndS[NSK], nUc[NSC], ndU[NSC];
    u16x8 ndO[NSC], nV[NSC];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int it = 0; it < NSK; ++it) {
            const int idx = tid + it * NTH, r = idx / W8, c = (idx % W8) * 8;
            if (idx < DK * W8) {
                nS[it] = *reinterpret_cast<const h8*>(hrec(R::SIN) + static_cast<size_t>(r) * DV + s0 + c);
                ndS[it] = *reinterpret_cast<const h8*>(hrec(R::DSO) + static_cast<size_t>(r) * DV + s0 + c);
            }
        }
#pragma unroll
        for (int it = 0; it < NSC; ++it) {
            const int idx = tid + it * NTH, r = idx / W8, c = (idx % W8) * 8;
            if (idx < C * W8) {
                nUc[it] = *reinterpret_cast<const h8*>(hrec(R::UC) + static_cast<size_t>(r) * DV + s0 + c);
                ndU[it] = *reinterpret_cast<const h8*>(hrec(R::DUC) + static_cast<size_t>(r) * DV + s0 + c);
                const int rr = r < len ? r : len - 1;
                const size_t off = (static_cast<size_t>(row0 + rr) * H + h) * DV + s0 + c;
                ndO[it] = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(P.dout) + off);
                nV[it] = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(P.v) + off);
            }
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int it = 0; it < NSK; ++it) {
            const int idx = tid + it * NTH, r = idx / W8, c = (idx % W8) * 8;
            if (idx < DK * W8) {
                *reinterpret_cast<h8*>(sS + r * RS + c) = nS[it];
                *reinterpret_cast<h8*>(sdS + r * RS + c) = ndS[it];
            }
        }
#pragma unroll
        for (int it = 0; it < NSC; ++it) {
            const int idx = tid + it * NTH, r = idx / W8, c = (idx % W8) * 8;
            if (idx < C * W8) {
                *reinterpret_cast<h8*>(sUc + r * RS + c) = nUc[it];
                *reinterpret_cast<h8*>(sdU + r * RS + c) = ndU[it];
                h8 o, vv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[e] = static_cast<_Float16>(r < len ? bf16_to_f32(ndO[it][e]) : 0.f);
                    vv[e] = static_cast<_Float16>(r < len ? bf16_to_f32(nV[it][e]) : 0.f);
                }
                *reinterpret_cast<h8*>(sdO + r * RS + c) = o;
                *reinterpret_cast<h8*>(sV + r * RS + c) = vv;
            }
        }
    };
    fetch(0);
    // T (fp32, kept for the key side) and its fp16 transpose; beta
    {
        constexpr int NTT = C * C / 4 / NTH;
        f4 tv[NTT];
        const float* gT = rec_at(P, h, g, R::TT);
#pragma unroll
        for (int it = 0; it < NTT; ++it) tv[it] = *reinterpret_cast<const f4*>(gT + 4 * (tid + it * NTH));
        if (tid < C) sBeta[tid] = tid < len ? P.beta[(row0 + tid) * H + h] : 0.f;
#pragma unroll
        for (int it = 0; it < NTT; ++it) {
            const int idx = 4 * (tid + it * NTH), r = idx / C, c = idx % C;
            *reinterpret_cast<f4*>(sT + r * LC + c) = tv[it];
#pragma unroll
            for (int e = 0; e < 4; ++e) sTt[(c + e) * CS + r] = static_cast<_Float16>(tv[it][e]);
        }
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) acc[k] = zero4();
    float dgam = 0.f;
    float dbz[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

    for (int s0 = 0; s0 < DV; s0 += SW) {
        put();
        __syncthreads();
        if (s0 + SW < DV) fetch(s0 + SW);
        // dU'^T for dZ: eight tokens of one column per thread, one 16-byte store
        for (int idx = tid; idx < C * SW / 8; idx += NTH) {
            const int c = idx % SW, r0 = (idx / SW) * 8;
            h8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sdU[(r0 + e) * RS + c];
            *reinterpret_cast<h8*>(sdUt + c * CS + r0) = x;
        }
        // dgamma: NTH / DK threads per key row, 16-byte reads
        {
            constexpr int TPR = NTH / DK, CPT = SW / TPR;
            static_assert(CPT % 8 == 0, "whole 16-byte words per thread");
            const int r = tid / TPR, c0 = (tid % TPR) * CPT;
#pragma unroll
            for (int c = 0; c < CPT; c += 8) {
                const h8 a = *reinterpret_cast<const h8*>(sdS + r * RS + c0 + c);
                const h8 b = *reinterpret_cast<const h8*>(sS + r * RS + c0 + c);
#pragma unroll
                for (int e = 0; e < 8; ++e) dgam += static_cast<float>(a[e]) * static_cast<float>(b[e]);
            }
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const _Float16 *pa, *pb;
            if (grad_task<NB>(wave + 8 * k, sdO, sdU, sUc, sS, sdS, sV, RS, pa, pb)) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc[k] = mfma16(*reinterpret_cast<const h8*>(pa + i * RS + 32 * ks + 8 * j),
                                    *reinterpret_cast<const h8*>(pb + i * RS + 32 * ks + 8 * j), acc[k]);
            }
        }
        __syncthreads();
        // dZ = T^T dU'[:, slice] (T^T[m][k] = T[k][m], zero for k < m); dv = beta . dZ
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = wave + 8 * u, zmb = t / NZB, znb = t % NZB;
            if (zmb >= 4) continue;
            f4 z = zero4();
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb)
                if (32 * kb + 31 >= 16 * zmb)
                    z = mfma16(*reinterpret_cast<const h8*>(sTt + (16 * zmb + i) * CS + 32 * kb + 8 * j),
                               *reinterpret_cast<const h8*>(sdUt + (16 * znb + i) * CS + 32 * kb + 8 * j), z);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = zmb * 16 + 4 * j + e;
                sDv[r * RS + znb * 16 + i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sBeta[r] * z[e]));
                dbz[u][e] += z[e] * static_cast<float>(sV[r * RS + znb * 16 + i]);
            }
        }
        __syncthreads();
        // dv rows of the slice as 16-byte words
        for (int idx = tid; idx < C * W8; idx += NTH) {
            const int r = idx / W8, c = (idx % W8) * 8;
            if (r < len)
                *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(P.dv) + (static_cast<size_t>(row0 + r) * H + h) * DV + s0 + c) =
                    *reinterpret_cast<const u16x8*>(sDv + r * RS + c);
        }
    }
    {
        constexpr int TPR = NTH / DK;          // the threads of one key row are adjacent lanes
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) dgam += __shfl_xor(dgam, o, 64);
        if (tid % TPR == 0) sDgam[tid / TPR] = dgam;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = wave + 8 * u, zmb = t / NZB, znb = t % NZB;
        if (zmb >= 4) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = row16_sum(dbz[u][e]);
            if (i == 0) sDbzP[znb * C + zmb * 16 + 4 * j + e] = x;
        }
    }
    __syncthreads();
    if (tid < C) {
        float x = 0.f;
#pragma unroll
        for (int z = 0; z < NZB; ++z) x += sDbzP[z * C + tid];
        sDbz[tid] = x;
    }
}

template <int DK, int DV, bool ABF16, int GATE, bool FAST>
__device__ __forceinline__ void grad_body(const BwdParams& P, const int h, const int g) {
    using GT = GradTasks<DK>;
    using R = BRec<DK, DV, ABF16>;
    constexpr int NTH = kGradThreads, NW = kGradWaves, LK = GradB<DK>::LK;
    constexpr int NB = GT::NB, RW = GT::RW, MSTEP = GT::MSTEP, KM = GT::KM;
    constexpr int GC = C / 16, GK = DK / 16;
    constexpr bool GBF16 = GATE == KDA_GATE_SOFTPLUS_BF16;
    extern __shared__ float lds[];
    float* sKh = lds;                // K; later db                             [C][LK]
    float* sKb = sKh + C * LK;       // b per 16-token tile                     [C][LK]
    float* sW = sKb + C * LK;        // dW; later Q                             [C][LK]
    float* sX = sW + C * LK;         // dT; later dR                            [C][LC]
    float* sY = sX + C * LC;         // T^T dT                                  [C][LC]
    float* sT = sY + C * LC;         // T; later M                              [C][LC]
    float* sBeta = sT + C * LC;      // [C]
    float* sRow = sBeta + C;         // dbeta parts (A and Y), one row per wave [NW][C]
    float* sCol = sRow + NW * C;     // column sums of Kt . dKt, one row per wave sharing a column block [MSTEP][DK]
    float* sDgam = sCol + MSTEP * DK;   // dgamma                               [DK]
    float* sDbz = sDgam + DK;        // rowsum(dZ . V)                          [C]
    float* sTot = sDbz + C;          // log2 alpha summed per 16-token tile     [C/16][DK]
    float* sGs = sCol;               // scalar gate per row while b is formed  [C]
    static_assert(C <= MSTEP * DK, "scalar gate rows fit the column-sum buffer");
    static_assert(GradB<DK>::bytes <= 160 * 1024, "LDS of one CU");

    const int H = P.H;
    const int4 ent = P.table[g];
    const int64_t row0 = ent.y;
    const int len = ent.z;
    const int tid = threadIdx.x, wave = wave_id(), i = lane_id() & 15, j = lane_id() >> 4;
    for (int idx = tid; idx < NW * C; idx += NTH) sRow[idx] = 0.f;

    // ---- value side (LDS before T is its scratch) ----
    f4 acc[GT::KT];
    if constexpr (ABF16) vside_phase16<DK, DV>(P, h, g, row0, len, lds, sT, sBeta, acc, sDgam, sDbz);
    else vside_phase32<DK, DV>(P, h, g, row0, len, lds, sT, sBeta, acc, sDgam, sDbz);
    __syncthreads();

    // ---- key side ----
    constexpr int NS = NTH / DK, SEG = C / NS;   // reverse-cumsum split: NS row segments per channel
    Tok<GBF16, DK, DK, NTH> tg;
    float gs = 1.f, gam_t, dgam_t;
    if constexpr (FAST) {
            // Kh, Kb and Qh formed once (the direct form)
        const int tnb = wave & 3, tmb0 = wave >> 2;     // C x C tiles: column block tnb, row blocks tmb0, tmb0 + 2
        // C x d_k tiles: column block nb, row blocks cmb0 + r MSTEP (with one
        // column block per wave, cmb0 is 0 at compile time, so the triangular
        // skips inside the products fold away instead of branching)
        const int nb = wave % NB, cmb0 = NB == NW ? 0 : wave / NB;
        // dW -> sW; the gate, then b = cumsum(log2 alpha) as in the preparation
        // kernel; Kh = 2^b K, Kb = 2^-b K
        {
            Tok<ABF16, DK, DK, NTH> tk;
            Tok<GBF16, DK, DK, NTH> tg0;
            tk.load(P.k, row0, len, h, H);
            if constexpr (GATE == KDA_GATE_SCALAR) {
                if (tid < C) sGs[tid] = tid < len ? static_cast<const float*>(P.gate)[(row0 + tid) * H + h] : 1.f;
            } else {
                tg0.load(P.gate, row0, len, h, H);
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) store_tile(sW + (cmb0 + r * MSTEP) * 16 * LK + nb * 16, LK, -acc[RW + r]);
            tk.put(sKh, LK);
            if constexpr (GATE != KDA_GATE_SCALAR) tg0.put(sKb, LK);
        }
        __syncthreads();
        gate_cumsum<DK, NTH, GATE>(sKb, LK, sGs, len, sX, [&](int r, int c, float b) {
            const float kv = sKh[r * LK + c];
            sKh[r * LK + c] = __builtin_amdgcn_exp2f(b) * kv;
            sKb[r * LK + c] = __builtin_amdgcn_exp2f(-b) * kv;
        });
        __syncthreads();

        // dT = (dW Kh^T + N) Diag(beta)
        {
            f4 dt[2] = {acc[KM + 2], acc[KM + 3]};
            mm_rows<2, GK, true, true>(sW, LK, 1, sKh + tnb * 16 * LK, 1, LK, tmb0, 2,
                                       [](int, int) { return true; }, dt);
#pragma unroll
            for (int r = 0; r < 2; ++r) store_tile(sX + (tmb0 + 2 * r) * 16 * LC + tnb * 16, LC, dt[r] * sBeta[tnb * 16 + i]);
        }
        __syncthreads();
        // Y1 = T^T dT  (T^T[m][k] = T[k][m], zero for k < m).  One copy per
        // value of tmb0, so the triangular skips are known at compile time.
        {
            auto y1_rows = [&](auto m0c) {
                constexpr int M0 = decltype(m0c)::value;
                f4 y1[2] = {zero4(), zero4()};
                mm_rows<2, GC, false, false>(sT, 1, LC, sX + tnb * 16, LC, 1, M0, 2,
                                             [](int mb, int gg) { return gg >= mb; }, y1);
#pragma unroll
                for (int r = 0; r < 2; ++r) store_tile(sY + (M0 + 2 * r) * 16 * LC + tnb * 16, LC, y1[r]);
            };
            if (tmb0 == 0) y1_rows(std::integral_constant<int, 0>{});
            else y1_rows(std::integral_constant<int, 1>{});
        }
        __syncthreads();
        // dA = -StrictTril(Y1 T^T); R = Kh Kb^T; dbeta += rowsum(dA . R); dR = Diag(beta) dA -> sX,
        // two tiles per wave (grad_tiles).  The tiles are fixed at compile time
        // (one copy of the phase per wave), so the tile tests and the triangular
        // skips fold away.
        {
            auto tiles = [&](auto wc) {
                constexpr int WV = decltype(wc)::value;
#pragma unroll
                for (int slot = 0; slot < 2; ++slot) {
                    const unsigned tt = (grad_tiles(WV) >> (8 * (1 - slot))) & 0xff;
                    const int mb = tt >> 4, nb = tt & 15;
                    f4 dr = zero4();
                    if (nb <= mb) {
                        // (Y1 T^T)[m][n] = sum_k Y1[m][k] T[n][k], T[n][k] zero for k > n
                        f4 ya[1] = {zero4()}, rr[1] = {zero4()};
                        mm_rows<1, GC, true, true>(sY, LC, 1, sT + nb * 16 * LC, 1, LC, mb, 1,
                                                   [nb](int, int gg) { return gg <= nb; }, ya);
                        mm_rows<1, GK, true, true>(sKh, LK, 1, sKb + nb * 16 * LK, 1, LK, mb, 1,
                                                   [](int, int) { return true; }, rr);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = mb * 16 + 4 * j + e, s2 = nb * 16 + i;
                            const float da = s2 < r ? -ya[0][e] : 0.f;
                            const float part = row16_sum(da * rr[0][e]);
                            if (i == 0) sRow[wave * C + r] += part;
                            dr[e] = sBeta[r] * da;
                        }
                    }
                    store_tile(sX + mb * 16 * LC + nb * 16, LC, dr);
                }
            };
            switch (wave) {
                case 0: tiles(std::integral_constant<int, 0>{}); break;
                case 1: tiles(std::integral_constant<int, 1>{}); break;
                case 2: tiles(std::integral_constant<int, 2>{}); break;
                case 3: tiles(std::integral_constant<int, 3>{}); break;
                case 4: tiles(std::integral_constant<int, 4>{}); break;
                case 5: tiles(std::integral_constant<int, 5>{}); break;
                case 6: tiles(std::integral_constant<int, 6>{}); break;
                default: tiles(std::integral_constant<int, 7>{}); break;
            }
        }
        __syncthreads();

        // dY = T^T dW; dKh = beta.dY + dR Kb; dbeta += rowsum(dY . Kh).  (T, dR
        // and, below, M hold exact zeros above their diagonals, which the split
        // products' pair-wise skipping with bf16 activations relies on.)
        f4 dKh[RW], dKb[RW];
        {
            f4 dy[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) dy[r] = dKb[r] = zero4();
            mm_rows_k<ABF16, RW, GC, false, false>(sT, 1, LC, sW + nb * 16, LK, 1, cmb0, MSTEP,
                                          [](int mb, int gg) { return gg >= mb; }, dy);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int mb = cmb0 + r * MSTEP;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = mb * 16 + 4 * j + e, c = nb * 16 + i;
                    const float part = row16_sum(dy[r][e] * sKh[row * LK + c]);
                    if (i == 0) sRow[wave * C + row] += part;
                    dKh[r][e] = sBeta[row] * dy[r][e];
                }
            }
            // dR strictly lower: row block mb reduces over tokens < 16 (mb + 1)
            mm_rows_k<ABF16, RW, GC, true, false>(sX, LC, 1, sKb + nb * 16, LK, 1, cmb0, MSTEP,
                                         [](int mb, int gg) { return gg <= mb; }, dKh);
        }
        __syncthreads();
        // M -> sT (tiles above the diagonal were never accumulated), Qh -> sW
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const int mb = tmb0 + 2 * r2;
            f4 x = acc[KM + r2];
            if (tnb == mb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = i <= 4 * j + e ? x[e] : 0.f;
            }
            store_tile(sT + mb * 16 * LC + tnb * 16, LC, x);
        }
        load_block<C, DK, NTH>(sW, LK, rec_at(P, h, g, R::QH), DK);
        __syncthreads();

        // dQh = dO S^T + M Kb;  dKb = M^T Qh + dR^T Kh
        f4 dQh[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) dQh[r] = acc[r];
        mm_rows_k<ABF16, RW, GC, true, false>(sT, LC, 1, sKb + nb * 16, LK, 1, cmb0, MSTEP,
                                     [](int mb, int gg) { return gg <= mb; }, dQh);
        mm_rows_k<ABF16, RW, GC, false, false>(sT, 1, LC, sW + nb * 16, LK, 1, cmb0, MSTEP,
                                      [](int mb, int gg) { return gg >= mb; }, dKb);
        mm_rows_k<ABF16, RW, GC, false, false>(sX, 1, LC, sKh + nb * 16, LK, 1, cmb0, MSTEP,
                                      [](int mb, int gg) { return gg >= mb; }, dKb);
        __syncthreads();

        // bf16 dq and dk rows, staged in the (now free) dT / Y1 regions
        constexpr int LDQ = DK + 8;
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        uint16_t* sDq = reinterpret_cast<uint16_t*>(sX);
        uint16_t* sDk = sDq + C * LDQ;
        static_assert(2 * C * LDQ * 2 <= 2 * C * LC * 4, "dq and dk fit the dT and Y1 regions");
        // gate chain rule, dq, dk.  Every operand is staged in LDS first (the
        // regions are free now), so no load waits behind a store of dq or dk:
        // q -> sKh, k -> sKb, the gate -> sW (b after the scan); dKt is the
        // value-side accumulator of the same tile.
        const float* gGam = rec_at(P, h, g, R::GAM);
        float gam_c;
        {
            Tok<ABF16, DK, DK, NTH> tq, tk;
            tq.load(P.q, row0, len, h, H);
            tk.load(P.k, row0, len, h, H);
            if constexpr (GATE == KDA_GATE_SCALAR) {
                if (tid < C && tid < len) gs = static_cast<const float*>(P.gate)[(row0 + tid) * H + h];
            } else {
                tg.load(P.gate, row0, len, h, H);
            }
            gam_c = gGam[nb * 16 + i];
            gam_t = gGam[tid % DK];
            dgam_t = sDgam[tid % DK];
            tq.put(sKh, LK);
            tk.put(sKb, LK);
            if constexpr (GATE == KDA_GATE_SCALAR) {
                if (tid < C) sGs[tid] = tid < len ? gs : 1.f;
            } else {
                tg.put(sW, LK);
            }
        }
        __syncthreads();
        // b again (the same scan, so the same values as above) -> sW
        gate_cumsum<DK, NTH, GATE>(sW, LK, sGs, len, sT, [&](int r, int c, float b) { sW[r * LK + c] = b; });
        __syncthreads();
        {
            const int c = nb * 16 + i;
            float col = 0.f;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int mb = cmb0 + r * MSTEP;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = mb * 16 + 4 * j + e;
                    const float b = sW[row * LK + c];
                    const float G = __builtin_amdgcn_exp2f(b), Gi = __builtin_amdgcn_exp2f(-b);
                    const float qv = sKh[row * LK + c], kv = sKb[row * LK + c], dkt = acc[2 * RW + r][e];
                    const float qh = G * qv, kh = G * kv, kb = Gi * kv, kt = gam_c * kb;
                    const float dqh = dQh[r][e], dkh = dKh[r][e], dkb = dKb[r][e];
                    const float dqv = G * dqh, dkv = G * dkh + Gi * dkb + gam_c * Gi * dkt;
                    if constexpr (ABF16) {           // staged in LDS, written below as whole 16-byte words
                        sDq[row * LDQ + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dqv));
                        sDk[row * LDQ + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dkv));
                    } else if (row < len) {
                        const size_t ai = (static_cast<size_t>(row0 + row) * H + h) * DK + c;
                        store_out<false>(P.dq, ai, dqv);
                        store_out<false>(P.dk, ai, dkv);
                    }
                    sKh[row * LK + c] = qh * dqh + kh * dkh - kb * dkb - kt * dkt;   // db
                    col += kt * dkt;
                }
            }
            col += __shfl_xor(col, 16, 64);
            col += __shfl_xor(col, 32, 64);
            if (j == 0) sCol[cmb0 * DK + c] = col;
        }
        __syncthreads();
        if constexpr (ABF16) {
            constexpr int W8 = DK / 8;
            for (int idx = tid; idx < C * W8; idx += NTH) {
                const int r = idx / W8, c8 = (idx % W8) * 8;
                if (r < len) {
                    const size_t ai = (static_cast<size_t>(row0 + r) * H + h) * DK + c8;
                    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(P.dq) + ai) = *reinterpret_cast<const u16x8*>(sDq + r * LDQ + c8);
                    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(P.dk) + ai) = *reinterpret_cast<const u16x8*>(sDk + r * LDQ + c8);
                }
            }
        }
    } else {
            // Every product that the chunk form writes with Gamma.K, K/Gamma or
            // Gamma.Q (Kh, Kb, Qh) is taken on the raw K and Q with each decay
            // factor formed from exponents <= 0 (decayed_tile and
            // decayed_lower_upper in kda_mm32.h), and the gradients are carried
            // already multiplied by the factor the chain rule applies to them:
            //   dQh' = Gamma.dQh,  dKh' = Gamma.dKh,  dKb' = dKb / Gamma.
        constexpr int NBLK = C / 16;
        const int tnb = wave & 3, tmb0 = wave >> 2;     // C x C tiles: column block tnb, row blocks tmb0, tmb0 + 2
        // C x d_k tiles: column block nb, row blocks cmb0 + r MSTEP (with one
        // column block per wave, cmb0 is 0 at compile time)
        const int nb = wave % NB, cmb0 = NB == NW ? 0 : wave / NB;
        // Gamma of token row, channel c (b is per tile: add the earlier tiles' totals)
        auto gam_at = [&](int row, int c) {
            return __builtin_amdgcn_exp2f(tot1(sTot, DK, c, 0, row / 16) + sKb[row * LK + c]);
        };
        // dW -> sW; K -> sKh; the gate, then b per 16-token tile and the tile totals
        {
            Tok<ABF16, DK, DK, NTH> tk;
            Tok<GBF16, DK, DK, NTH> tg0;
            tk.load(P.k, row0, len, h, H);
            if constexpr (GATE == KDA_GATE_SCALAR) {
                if (tid < C) sGs[tid] = tid < len ? static_cast<const float*>(P.gate)[(row0 + tid) * H + h] : 1.f;
            } else {
                tg0.load(P.gate, row0, len, h, H);
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) store_tile(sW + (cmb0 + r * MSTEP) * 16 * LK + nb * 16, LK, -acc[RW + r]);
            tk.put(sKh, LK);
            if constexpr (GATE != KDA_GATE_SCALAR) tg0.put(sKb, LK);
        }
        __syncthreads();
        tile_gate_scan<DK, NTH, C, GATE>(sKb, LK, sGs, len, sTot, sX);

        // dT = (dW Kh^T + N) Diag(beta), Kh = Gamma.K formed per B operand
        {
            f4 dt[2] = {acc[KM + 2], acc[KM + 3]};
            const int st = tnb * 16 + i;
            {
#pragma unroll
                for (int gg = 0; gg < GK; ++gg) {
                    const int c0 = 16 * gg + 4 * j;
                    const f4 kk = *reinterpret_cast<const f4*>(sKh + st * LK + c0);
                    const f4 bl = *reinterpret_cast<const f4*>(sKb + st * LK + c0);
                    const f4 pr = tot4(sTot, DK, c0, 0, tnb);
                    f4 bv;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) bv[s2] = kk[s2] * __builtin_amdgcn_exp2f(pr[s2] + bl[s2]);
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const f4 a = *reinterpret_cast<const f4*>(sW + ((tmb0 + 2 * r) * 16 + i) * LK + c0);
#pragma unroll
                        for (int s2 = 0; s2 < 4; ++s2) dt[r] = mfma4(a[s2], bv[s2], dt[r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) store_tile(sX + (tmb0 + 2 * r) * 16 * LC + tnb * 16, LC, dt[r] * sBeta[tnb * 16 + i]);
        }
        __syncthreads();
        // Y1 = T^T dT  (T^T[m][k] = T[k][m], zero for k < m).  One copy per
        // value of tmb0, so the triangular skips are known at compile time.
        {
            auto y1_rows = [&](auto m0c) {
                constexpr int M0 = decltype(m0c)::value;
                f4 y1[2] = {zero4(), zero4()};
                mm_rows<2, GC, false, false>(sT, 1, LC, sX + tnb * 16, LC, 1, M0, 2,
                                             [](int mb, int gg) { return gg >= mb; }, y1);
#pragma unroll
                for (int r = 0; r < 2; ++r) store_tile(sY + (M0 + 2 * r) * 16 * LC + tnb * 16, LC, y1[r]);
            };
            if (tmb0 == 0) y1_rows(std::integral_constant<int, 0>{});
            else y1_rows(std::integral_constant<int, 1>{});
        }
        __syncthreads();
        // dA = -StrictTril(Y1 T^T); R = Kh Kb^T (decayed_tile); dbeta += rowsum(dA . R);
        // dR = Diag(beta) dA -> sX, two tiles per wave (grad_tiles).  The tiles are
        // fixed at compile time (one copy of the phase per wave).
        {
            auto tiles = [&](auto wc) {
                constexpr int WV = decltype(wc)::value;
#pragma unroll
                for (int slot = 0; slot < 2; ++slot) {
                    const unsigned tt = (grad_tiles(WV) >> (8 * (1 - slot))) & 0xff;
                    const int mb = tt >> 4, tb = tt & 15;
                    f4 dr = zero4();
                    if (tb <= mb) {
                        // (Y1 T^T)[m][n] = sum_k Y1[m][k] T[n][k], T[n][k] zero for k > n
                        f4 ya[1] = {zero4()}, rr[1] = {zero4()}, unused = zero4();
                        mm_rows<1, GC, true, true>(sY, LC, 1, sT + tb * 16 * LC, 1, LC, mb, 1,
                                                   [tb](int, int gg) { return gg <= tb; }, ya);
                        decayed_tile<GK, false, false, ABF16>(sKh, sKh, sKh, sKb, sTot, LK, DK, mb, tb, rr[0], unused);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = mb * 16 + 4 * j + e, s2 = tb * 16 + i;
                            const float da = s2 < r ? -ya[0][e] : 0.f;
                            const float part = row16_sum(da * rr[0][e]);
                            if (i == 0) sRow[wave * C + r] += part;
                            dr[e] = sBeta[r] * da;
                        }
                    }
                    store_tile(sX + mb * 16 * LC + tb * 16, LC, dr);
                }
            };
            switch (wave) {
                case 0: tiles(std::integral_constant<int, 0>{}); break;
                case 1: tiles(std::integral_constant<int, 1>{}); break;
                case 2: tiles(std::integral_constant<int, 2>{}); break;
                case 3: tiles(std::integral_constant<int, 3>{}); break;
                case 4: tiles(std::integral_constant<int, 4>{}); break;
                case 5: tiles(std::integral_constant<int, 5>{}); break;
                case 6: tiles(std::integral_constant<int, 6>{}); break;
                default: tiles(std::integral_constant<int, 7>{}); break;
            }
        }
        __syncthreads();

        // dY = T^T dW; dKh' = Gamma.(beta dY); dbeta += rowsum(dY . Kh)
        f4 dKh[RW], dKb[RW], dQh[RW];
        {
            f4 dy[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) dy[r] = dKb[r] = zero4();
            mm_rows_k<ABF16, RW, GC, false, false>(sT, 1, LC, sW + nb * 16, LK, 1, cmb0, MSTEP,
                                          [](int mb, int gg) { return gg >= mb; }, dy);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int mb = cmb0 + r * MSTEP;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = mb * 16 + 4 * j + e, c = nb * 16 + i;
                    const float G = gam_at(row, c);
                    const float part = row16_sum(dy[r][e] * sKh[row * LK + c] * G);
                    if (i == 0) sRow[wave * C + row] += part;
                    dKh[r][e] = sBeta[row] * dy[r][e] * G;
                    dQh[r][e] = acc[r][e] * G;                    // Gamma.(dO S^T)
                }
            }
        }
        __syncthreads();
        // M -> sT (tiles above the diagonal were never accumulated), Q -> sW
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const int mb = tmb0 + 2 * r2;
            f4 x = acc[KM + r2];
            if (tnb == mb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = i <= 4 * j + e ? x[e] : 0.f;
            }
            store_tile(sT + mb * 16 * LC + tnb * 16, LC, x);
        }
        {
            Tok<ABF16, DK, DK, NTH> tq;
            tq.load(P.q, row0, len, h, H);
            tq.put(sW, LK);
        }
        __syncthreads();

        // dKh' += Gamma.(dR Kb),  dQh' += Gamma.(M Kb)  (lower contractions);
        // dKb' = (M^T Qh + dR^T Kh) / Gamma  (upper contractions)
        decayed_lower_upper<RW, NBLK, ABF16>(sX, sT, LC, sKh, sW, sKb, sTot, LK, DK, cmb0, MSTEP, nb, dKh, dQh, dKb);
        __syncthreads();

        // bf16 dq and dk rows, staged in the (now free) dT / Y1 regions
        constexpr int LDQ = DK + 8;
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        uint16_t* sDq = reinterpret_cast<uint16_t*>(sX);
        uint16_t* sDk = sDq + C * LDQ;
        static_assert(2 * C * LDQ * 2 <= 2 * C * LC * 4, "dq and dk fit the dT and Y1 regions");
        // gate chain rule, dq, dk: dq = dQh', dk = dKh' + dKb' + (gamma/Gamma) dKt, and the
        // gradient of each token's log decay db = q dQh' + k dKh' - k dKb' - Kt dKt, written
        // over K (sKh) by the lane that owns the element; dKt is the value-side
        // accumulator of the same tile.
        gam_t = __builtin_amdgcn_exp2f(tot1(sTot, DK, tid % DK, 0, NBLK));
        dgam_t = sDgam[tid % DK];
        if constexpr (GATE == KDA_GATE_SCALAR) {
            if (tid < C && tid < len) gs = static_cast<const float*>(P.gate)[(row0 + tid) * H + h];
        } else {
            tg.load(P.gate, row0, len, h, H);
        }
        {
            const int c = nb * 16 + i;
            float col = 0.f;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int mb = cmb0 + r * MSTEP;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = mb * 16 + 4 * j + e, t = row / 16;
                    const float bl = sKb[row * LK + c];
                    const float ktf = __builtin_amdgcn_exp2f(sTot[t * DK + c] - bl + tot1(sTot, DK, c, t + 1, NBLK));
                    const float qv = sW[row * LK + c], kv = sKh[row * LK + c], dkt = acc[2 * RW + r][e];
                    const float dqv = dQh[r][e], dkv = dKh[r][e] + dKb[r][e] + ktf * dkt;
                    if constexpr (ABF16) {           // staged in LDS, written below as whole 16-byte words
                        sDq[row * LDQ + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dqv));
                        sDk[row * LDQ + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dkv));
                    } else if (row < len) {
                        const size_t ai = (static_cast<size_t>(row0 + row) * H + h) * DK + c;
                        store_out<false>(P.dq, ai, dqv);
                        store_out<false>(P.dk, ai, dkv);
                    }
                    const float kt = kv * ktf;
                    sKh[row * LK + c] = qv * dQh[r][e] + kv * dKh[r][e] - kv * dKb[r][e] - kt * dkt;   // db
                    col += kt * dkt;
                }
            }
            col += __shfl_xor(col, 16, 64);
            col += __shfl_xor(col, 32, 64);
            if (j == 0) sCol[cmb0 * DK + c] = col;
        }
        __syncthreads();
        if constexpr (ABF16) {
            constexpr int W8 = DK / 8;
            for (int idx = tid; idx < C * W8; idx += NTH) {
                const int r = idx / W8, c8 = (idx % W8) * 8;
                if (r < len) {
                    const size_t ai = (static_cast<size_t>(row0 + r) * H + h) * DK + c8;
                    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(P.dq) + ai) = *reinterpret_cast<const u16x8*>(sDq + r * LDQ + c8);
                    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(P.dk) + ai) = *reinterpret_cast<const u16x8*>(sDk + r * LDQ + c8);
                }
            }
        }
    }
    // the gate as given (b is no longer needed); partial sums of db per segment
    if constexpr (GATE == KDA_GATE_SCALAR) {
        if (tid < C) sW[tid] = gs;
    } else {
        tg.put(sW, LK);
    }
    float* sPart = sT;                       // [NS][DK]
    {
        const int c = tid % DK, sg = tid / DK;
        float part = 0.f;
        for (int r = sg * SEG; r < sg * SEG + SEG; ++r) part += sKh[r * LK + c];
        sPart[sg * DK + c] = part;
    }
    __syncthreads();

    // dlog(alpha)_r = sum_{s >= r} db_s (natural-log units), per channel; gamma's own
    // gradient and the Kt terms enter at the last row
    {
        const int c = tid % DK, sg = tid / DK;
        float acc2 = gam_t * dgam_t;
#pragma unroll
        for (int z = 0; z < MSTEP; ++z) acc2 += sCol[z * DK + c];
        for (int s2 = sg + 1; s2 < NS; ++s2) acc2 += sPart[s2 * DK + c];
        // the segment's db and gate values first (independent reads), then the scan
        float dbv[SEG], gv[SEG];
#pragma unroll
        for (int q = 0; q < SEG; ++q) {
            dbv[q] = sKh[(sg * SEG + q) * LK + c];
            if constexpr (GATE != KDA_GATE_SCALAR) gv[q] = sW[(sg * SEG + q) * LK + c];
        }
#pragma unroll
        for (int q = SEG - 1; q >= 0; --q) {
            const int r = sg * SEG + q;
            acc2 += dbv[q];
            if (r < len) {
                const size_t ai = (static_cast<size_t>(row0 + r) * H + h) * DK + c;
                if constexpr (GATE == KDA_GATE_ALPHA) {
                    P.dgate[ai] = acc2 / gv[q];
                } else if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16) {
                    // log alpha = -softplus(x): d/dx = -sigmoid(x)
                    const float sgm = 1.f / (1.f + __builtin_amdgcn_exp2f(-gv[q] * 1.4426950408889634f));
                    P.dgate[ai] = -acc2 * sgm;
                } else {
                    sKb[r * LK + c] = acc2;
                }
            }
        }
    }
    if constexpr (GATE == KDA_GATE_SCALAR) {
        __syncthreads();
        if (tid < len) {
            float s = 0.f;
            for (int c = 0; c < DK; ++c) s += sKb[tid * LK + c];
            P.dgate[static_cast<size_t>(row0 + tid) * H + h] = s / sW[tid];
        }
    }
    if (tid < len) {
        float db = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) db += sRow[w * C + tid];
        P.dbeta[(row0 + tid) * H + h] = sDbz[tid] + db;
    }
}

// One workgroup per (chunk, head) of the direct form (the preparation kernel
// set its flag).
template <int DK, int DV, bool ABF16, int GATE>
__global__ __launch_bounds__(kGradThreads) void bwd_grad_kernel(const BwdParams P) {
    const int g = blockIdx.x / P.H;
    if (g >= P.ctrl[0] || P.flag[blockIdx.x]) return;
    grad_body<DK, DV, ABF16, GATE, true>(P, blockIdx.x % P.H, g);
}

// Entry blockIdx.x of the general list, as for the preparation kernel.
template <int DK, int DV, bool ABF16, int GATE>
__global__ __launch_bounds__(kGradThreads) void bwd_grad_general_kernel(const BwdParams P) {
    if (static_cast<int>(blockIdx.x) >= *P.nslow) return;
    const int id = P.slow[blockIdx.x];
    grad_body<DK, DV, ABF16, GATE, false>(P, id % P.H, id / P.H);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }


template <typename F>
hipError_t set_lds(F* kfn, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int DK, int DV, bool ABF16, int GATE>
hipError_t launch_bwd_typed(const ChunkBwdPlan& bp, const ChunkBwdArgs& a, hipStream_t stream) {
    const ChunkPlan& pl = bp.fwd;
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    if (BRec<DK, DV, ABF16>::END > bp.rec_bytes) return hipErrorInvalidValue;
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.dout = a.dout; p.beta = a.beta;
    p.initial_state = a.initial_state; p.dfinal_state = a.dfinal_state;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dgate = a.dgate; p.dbeta = a.dbeta;
    p.dinitial_state = a.dinitial_state;
    p.ctrl = reinterpret_cast<const int32_t*>(ws + pl.off_ctrl);
    p.nslow = reinterpret_cast<int32_t*>(ws + pl.off_ctrl) + 1;
    p.slow = reinterpret_cast<int32_t*>(ws + bp.off_slow);
    p.flag = reinterpret_cast<int32_t*>(ws + bp.off_flag);
    p.first = reinterpret_cast<const int32_t*>(ws + pl.off_first);
    p.order = reinterpret_cast<const int32_t*>(ws + pl.off_order);
    p.table = reinterpret_cast<const int4*>(ws + pl.off_table);
    p.rec = ws + bp.off_rec;
    p.rec_bytes = bp.rec_bytes;
    p.gmax = pl.gmax;
    p.N = pl.N;
    p.H = pl.H;

    hipError_t e = launch_chunk_plan(pl, a.cu_seqlens, a.workspace, stream);
    if (e != hipSuccess) return e;
    const unsigned chunk_blocks = static_cast<unsigned>(pl.gmax * pl.H);
    // the general-form kernels: one workgroup per list entry that may exist;
    // those past the list's length return at once
    const unsigned general_blocks = chunk_blocks;
    const int64_t pairs = static_cast<int64_t>(pl.N) * pl.H;
    const unsigned chain_blocks = static_cast<unsigned>((pairs + 7) / 8 * 8 * (DV / 16));
    if (chunk_blocks > 0) {
        auto k1 = bwd_prep_kernel<DK, DV, ABF16, GATE>;
        constexpr int l1 = PrepDirB<DK>::bytes;
        if ((e = set_lds(k1, l1)) != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(chunk_blocks), dim3(kPrepThreads), l1, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto k1g = bwd_prep_general_kernel<DK, DV, ABF16, GATE>;
        constexpr int l1g = PrepB<DK, DV>::bytes;
        if ((e = set_lds(k1g, l1g)) != hipSuccess) return e;
        hipLaunchKernelGGL(k1g, dim3(general_blocks), dim3(kPrepThreads), l1g, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto k2 = ABF16 ? bwd_ckpt16_kernel<DK, DV> : bwd_ckpt_kernel<DK, DV>;
        constexpr int l2 = ABF16 ? Chain16B<DK>::bytes : CkptB<DK>::bytes;
        if ((e = set_lds(k2, l2)) != hipSuccess) return e;
        hipLaunchKernelGGL(k2, dim3(chain_blocks), dim3(ABF16 ? kChain16Threads : kChainThreads), l2, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (chain_blocks > 0) {
        auto k3 = ABF16 ? bwd_rev16_kernel<DK, DV> : bwd_rev_kernel<DK, DV, ABF16>;
        constexpr int l3 = ABF16 ? Chain16B<DK>::bytes : RevB<DK>::bytes;
        if ((e = set_lds(k3, l3)) != hipSuccess) return e;
        hipLaunchKernelGGL(k3, dim3(chain_blocks), dim3(ABF16 ? kChain16Threads : kChainThreads), l3, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (chunk_blocks > 0) {
        auto k4 = bwd_grad_kernel<DK, DV, ABF16, GATE>;
        constexpr int l4 = GradB<DK>::bytes;
        if ((e = set_lds(k4, l4)) != hipSuccess) return e;
        hipLaunchKernelGGL(k4, dim3(chunk_blocks), dim3(kGradThreads), l4, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto k4g = bwd_grad_general_kernel<DK, DV, ABF16, GATE>;
        if ((e = set_lds(k4g, l4)) != hipSuccess) return e;
        hipLaunchKernelGGL(k4g, dim3(general_blocks), dim3(kGradThreads), l4, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, bool ABF16>
hipError_t launch_bwd_gate(const ChunkBwdPlan& bp, const ChunkBwdArgs& a, hipStream_t stream) {
    if (a.gate_kind == KDA_GATE_SOFTPLUS_BF16)
        return launch_bwd_typed<DK, DV, ABF16, KDA_GATE_SOFTPLUS_BF16>(bp, a, stream);
    if (a.gate_kind == KDA_GATE_SCALAR) return launch_bwd_typed<DK, DV, ABF16, KDA_GATE_SCALAR>(bp, a, stream);
    return launch_bwd_typed<DK, DV, ABF16, KDA_GATE_ALPHA>(bp, a, stream);
}

template <int DK, int DV>
hipError_t launch_bwd_dims(const ChunkBwdPlan& bp, const ChunkBwdArgs& a, hipStream_t stream) {
    return a.act_bf16 ? launch_bwd_gate<DK, DV, true>(bp, a, stream) : launch_bwd_gate<DK, DV, false>(bp, a, stream);
}

}  // namespace

kda_status make_chunk_bwd_plan(int B, int64_t T, int H, int Dk, int Dv, bool varlen, int num_seqs,
                               int chunk_size, bool act_bf16, ChunkBwdPlan* plan) {
    if (chunk_size != kChunk) return KDA_ERROR_NOT_SUPPORTED;       // the backward runs at C = 64
    ChunkBwdPlan bp;
    const kda_status st = make_chunk_plan(B, T, H, Dk, Dv, varlen, num_seqs, chunk_size, act_bf16, &bp.fwd);
    if (st != KDA_SUCCESS) return st;
    // the forward's records are not used: the backward keeps its own record
    auto rec_end = [&](auto f16) -> size_t {
        constexpr bool F = decltype(f16)::value;
        if (Dk == 128 && Dv == 128) return BRec<128, 128, F>::END;
        if (Dk == 64 && Dv == 64) return BRec<64, 64, F>::END;
        if (Dk == 128 && Dv == 64) return BRec<128, 64, F>::END;
        return BRec<64, 128, F>::END;
    };
    const size_t end = act_bf16 ? rec_end(std::true_type{}) : rec_end(std::false_type{});
    bp.rec_bytes = align256(end);
    bp.off_rec = bp.fwd.off_rec;
    const size_t gh = static_cast<size_t>(bp.fwd.gmax) * H;
    bp.off_slow = align256(bp.off_rec + gh * bp.rec_bytes);
    bp.off_flag = align256(bp.off_slow + 4 * gh);
    bp.workspace_bytes = align256(bp.off_flag + 4 * gh);
    *plan = bp;
    return KDA_SUCCESS;
}

hipError_t launch_chunk_bwd(const ChunkBwdPlan& bp, const ChunkBwdArgs& a, hipStream_t stream) {
    const ChunkPlan& pl = bp.fwd;
    if (pl.Dk == 128 && pl.Dv == 128) return launch_bwd_dims<128, 128>(bp, a, stream);
    if (pl.Dk == 64 && pl.Dv == 64) return launch_bwd_dims<64, 64>(bp, a, stream);
    if (pl.Dk == 128 && pl.Dv == 64) return launch_bwd_dims<128, 64>(bp, a, stream);
    if (pl.Dk == 64 && pl.Dv == 128) return launch_bwd_dims<64, 128>(bp, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
