// Chunkwise KDA forward for gfx950.
//
// The chunked algorithm of "Linear Attention KDA Gating in a 3:1 Hybrid
// Architecture: Principles and Implementation Guide", section 3, carried out
// in three launches on the caller's stream:
//
//   plan_kernel   (integer)  chunk table: which sequence, first token row and
//                 length every 64-token chunk has; sequence order by length.
//   prep_kernel   (chunk-parallel, one workgroup per (chunk, head))
//                 log-domain cumulative decay b = cumsum(log alpha) over the
//                 chunk ("log-domain accumulation", "Designing and Deploying
//                 Hybrid MLA and Linear Attention Architectures", section 3);
//                 A = strictly-lower(Diag(beta)(Gamma.K)(K/Gamma)^T) and
//                 P = Tril((Gamma.Q)(K/Gamma)^T) on the matrix cores;
//                 T = (I + A)^-1 by blocked forward substitution;
//                 W = T Diag(beta)(Gamma.K), U = T Diag(beta) V on the matrix
//                 cores; Gamma.Q, ((gamma/Gamma).K)^T and gamma.
//   state_kernel  (sequential over the chunks of one sequence, one
//                 workgroup per (sequence, head, 16 value columns))
//                 U' = U - W S,  O = (Gamma.Q) S + P U',
//                 S <- Diag(gamma) S + ((gamma/Gamma).K)^T U'
//                 (inter-chunk transition of section 3.1, masked intra-chunk
//                 output of section 3.2), S kept in registers throughout.
//
// Reading of the garbled passages: Gamma_r is the inclusive per-channel
// product of alpha over the chunk's first r tokens; W and U are per-token
// rows obtained with the unit-lower-triangular inverse (I + A)^-1; Tril keeps
// the diagonal.  The padded tail of a partial chunk has alpha = 1, beta = 0
// and q = k = v = 0, which leaves every result unchanged.
//
// Numerics.  All accumulation is fp32.  With bf16 activations the matrix-core
// operands are fp16 (11-bit significand, 8x finer than bf16); with fp32
// activations every product runs on the fp32 matrix cores.  The decay factors
// are never formed as e^{+b} alone: products e^{b_r - b_s} (s <= r) are split
// as e^{b_r - ref} * e^{ref - b_s} around a reference token in the middle of
// each 16-token block ("chunk-wise normalization", same section), so every
// factor is bounded by the decay over at most 8 tokens.
#include "kda_chunk.h"
#include "kda_common.h"

namespace kda {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int C = kChunk;

// ---------------------------------------------------------------------------
// 16x16 matrix-core tile with a 32-deep reduction step.
//   A operand: lane l holds A[m = l%16][k = 8*(l/16) + e], e = 0..7
//   B operand: lane l holds B[k = 8*(l/16) + e][n = l%16]
//   C/D:       lane l holds D[4*(l/16) + i][l%16], i = 0..3
// The fp32 variant issues eight 16x16x4 steps; step e takes element e of the
// same eight values, so both variants reduce over the same 32 indices.
// ---------------------------------------------------------------------------
template <bool F16> struct Mx;

template <> struct Mx<true> {
    using E = _Float16;
    using V = h8;
    static __device__ __forceinline__ f4 mma(const V& a, const V& b, f4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ V load8(const E* p) { return *reinterpret_cast<const V*>(p); }
    // elements 0..3 from p0, 4..7 from p1 (each 8-byte aligned)
    static __device__ __forceinline__ V load4x2(const E* p0, const E* p1) {
        const h4 a = *reinterpret_cast<const h4*>(p0);
        const h4 b = *reinterpret_cast<const h4*>(p1);
        V v;
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
        return v;
    }
    static __device__ __forceinline__ E cvt(float x) { return static_cast<E>(x); }
    static __device__ __forceinline__ float tof(E x) { return static_cast<float>(x); }
    static __device__ __forceinline__ void store4(E* p, f4 x) {
        h4 h = {static_cast<E>(x[0]), static_cast<E>(x[1]), static_cast<E>(x[2]), static_cast<E>(x[3])};
        *reinterpret_cast<h4*>(p) = h;
    }
    static __device__ __forceinline__ void store8(E* p, const float* x) {
        h8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<E>(x[e]);
        *reinterpret_cast<h8*>(p) = h;
    }
};

template <> struct Mx<false> {
    using E = float;
    using V = f8;
    static __device__ __forceinline__ f4 mma(const V& a, const V& b, f4 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ V load8(const E* p) {
        const f4 lo = *reinterpret_cast<const f4*>(p);
        const f4 hi = *reinterpret_cast<const f4*>(p + 4);
        V v;
        v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
        v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
        return v;
    }
    static __device__ __forceinline__ V load4x2(const E* p0, const E* p1) {
        const f4 lo = *reinterpret_cast<const f4*>(p0);
        const f4 hi = *reinterpret_cast<const f4*>(p1);
        V v;
        v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
        v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
        return v;
    }
    static __device__ __forceinline__ E cvt(float x) { return x; }
    static __device__ __forceinline__ float tof(E x) { return x; }
    static __device__ __forceinline__ void store4(E* p, f4 x) { *reinterpret_cast<f4*>(p) = x; }
    static __device__ __forceinline__ void store8(E* p, const float* x) {
        f4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
        *reinterpret_cast<f4*>(p) = lo;
        *reinterpret_cast<f4*>(p + 4) = hi;
    }
};

// Eight consecutive activations (16-byte aligned) as fp32.
template <bool BF16> struct Load8;
template <> struct Load8<true> {
    static __device__ __forceinline__ void f(const uint16_t* p, float* out) {
        const u16x8 r = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32(r[e]);
    }
};
template <> struct Load8<false> {
    static __device__ __forceinline__ void f(const float* p, float* out) {
        const f4 lo = *reinterpret_cast<const f4*>(p);
        const f4 hi = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = lo[e]; out[4 + e] = hi[e]; }
    }
};

// Operand fragments in the workspace.  Every matrix-core operand that the
// state kernel loads is stored "fragment-major": fragment f of a matrix is
// the 16 rows x 32 reduction indices one MFMA step consumes, laid out as
// 64 lanes x 8 elements, so one wavefront load moves 1 KiB of contiguous
// bytes.  Within a fragment, lane (m, j) (m = lane % 16, j = lane / 16)
// holds row m at reduction indices frag_k(j, e), e = 0..7: two runs of four,
// 4j..4j+3 and 16+4j..16+4j+3.  Any bijection onto the 32 indices gives the
// same product as long as both operands of an MFMA use it; this one lets a
// 16x16 accumulator tile pair (rows 4j..4j+3 of each tile in lane (m, j))
// be written as a fragment without moving data between lanes.
__device__ __forceinline__ int frag_k(int j, int e) { return e < 4 ? 4 * j + e : 12 + 4 * j + e; }

__device__ __forceinline__ size_t frag_off(int f, int lane) { return (static_cast<size_t>(f) * 64 + lane) * 8; }

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// plan_kernel: chunk table, per-sequence first chunk, longest-first order.
// One workgroup of 1024 threads; every loop is spread over the threads.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kRankSortMax = 4096;   // above this, sequences keep their index order

__device__ __forceinline__ int seq_len(const int32_t* cu, int n, int64_t T) {
    return cu ? cu[n + 1] - cu[n] : static_cast<int>(T);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu, int N,
                                                            int64_t T, int64_t gmax,
                                                            int32_t* __restrict__ ctrl,
                                                            int32_t* __restrict__ first,
                                                            int32_t* __restrict__ order,
                                                            int4* __restrict__ table) {
    __shared__ int s_scan[kPlanThreads];
    __shared__ int s_len[kRankSortMax];
    __shared__ int s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    // first[n] = number of chunks of sequences 0..n-1 (block-wise inclusive scan)
    for (int base = 0; base < N; base += kPlanThreads) {
        const int n = base + tid;
        int cnt = 0;
        if (n < N) {
            const int len = seq_len(cu, n, T);
            cnt = len > 0 ? (len + C - 1) / C : 0;
            if (N <= kRankSortMax) s_len[n] = len;
        }
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        if (n < N) {
            const int f = s_carry + s_scan[tid] - cnt;
            first[n] = f < gmax ? f : static_cast<int>(gmax);
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) s_carry += s_scan[tid];
        __syncthreads();
    }
    // a malformed cu_seqlens cannot push work past the table's capacity
    const int total = s_carry < gmax ? s_carry : static_cast<int>(gmax);
    if (tid == 0) {
        first[N] = total;
        ctrl[0] = total;
    }
    __syncthreads();
    // one table entry per chunk: its sequence is the last n with first[n] <= g
    for (int g = tid; g < total; g += kPlanThreads) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first[mid] <= g) lo = mid; else hi = mid - 1;
        }
        const int n = lo;
        const int i = g - first[n];
        const int len = seq_len(cu, n, T);
        const int start = cu ? cu[n] : static_cast<int>(static_cast<int64_t>(n) * T);
        const int l = len - i * C;
        table[g] = make_int4(n, start + i * C, l < C ? l : C, 0);
    }
    // longest sequences first (ties by index), so long chains start early
    for (int n = tid; n < N; n += kPlanThreads) {
        int rank = n;
        if (N <= kRankSortMax) {
            const int len = s_len[n];
            rank = 0;
            for (int m = 0; m < N; ++m) {
                const int lm = s_len[m];
                rank += (lm > len) || (lm == len && m < n);
            }
        }
        order[rank] = n;
    }
}

// ---------------------------------------------------------------------------
// prep_kernel: everything of one (chunk, head) that does not depend on the
// state entering the chunk.  All global loads are issued first; the phases
// then work out of LDS.
// ---------------------------------------------------------------------------
struct PrepParams {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const int32_t* ctrl;
    const int4* table;
    unsigned char* rec;
    size_t rec_bytes;
    int64_t gmax;
    int H;
};

template <int a, int b> struct CMax { static constexpr int value = a > b ? a : b; };

// Byte offsets inside one (head, chunk) record of the workspace.
template <int DK, int DV, bool F16>
struct Rec {
    using E = typename Mx<F16>::E;
    static constexpr size_t QH = 0;
    static constexpr size_t W = QH + sizeof(E) * C * DK;
    static constexpr size_t KTT = W + sizeof(E) * C * DK;
    static constexpr size_t P = KTT + sizeof(E) * DK * C;
    static constexpr size_t UT = P + sizeof(E) * C * C;
    static constexpr size_t GAM = UT + 4 * DV * C;
    static constexpr size_t END = GAM + 4 * DK;
};

template <int DK, int DV, bool F16>
struct PrepLds {
    using A = typename Act<F16>::T;   // raw activation element
    using E = typename Mx<F16>::E;    // matrix-core operand element
    static constexpr int BP = DK + 4;        // fp32 row stride of b (log2 decay)
    static constexpr int KP = DK + 8;        // row stride of k / K-hat and of q
    static constexpr int VP = DV + 8;        // row stride of v
    static constexpr int AP = C + 1;         // fp32 row stride of A
    static constexpr int TP = C + 4;         // fp32 row stride of T
    static constexpr int TPP = C + 8;        // row stride of T Diag(beta) (operand type)
    static constexpr int kElem = sizeof(A) > sizeof(E) ? sizeof(A) : sizeof(E);
    // region 1: b, later T (fp32) followed by v
    static constexpr int R1 = CMax<C * BP * 4, C * TP * 4 + C * VP * (int)sizeof(A)>::value;
    // region 2: raw k, later K-hat in place
    static constexpr int R2 = C * KP * kElem;
    // region 3: raw q, later A (fp32), later T Diag(beta)
    static constexpr int R3 =
        CMax<C * KP * (int)sizeof(A), CMax<C * AP * 4, C * TPP * (int)sizeof(E)>::value>::value;
    static constexpr int PARTS = 256 / DK;
    static constexpr int R4 = (C + PARTS * DK) * 4;   // beta, cumsum part totals
    static constexpr int bytes = R1 + R2 + R3 + R4;
};

template <int DK, int DV, bool F16>
__global__ __launch_bounds__(256) void prep_kernel(const PrepParams P) {
    using L = PrepLds<DK, DV, F16>;
    using A = typename L::A;
    using M = Mx<F16>;
    using E = typename M::E;
    using V = typename M::V;
    constexpr int BP = L::BP, KP = L::KP, VP = L::VP, AP = L::AP, TP = L::TP, TPP = L::TPP;
    constexpr int PARTS = L::PARTS;
    constexpr int RP = C / PARTS;                          // cumsum rows per thread
    constexpr int EL16 = 16 / (int)sizeof(A);              // activations per 16 bytes
    constexpr int KROW16 = DK / EL16;                      // 16-byte pieces per k/q row
    constexpr int VROW16 = DV / EL16;
    constexpr int NK = C * KROW16 / 256;                   // pieces per thread
    constexpr int NV = C * VROW16 / 256;

    const int H = P.H;
    const int g = blockIdx.x / H;
    const int h = blockIdx.x - g * H;
    if (g >= P.ctrl[0]) return;
    const int4 ent = P.table[g];
    const int t0 = ent.y;
    const int len = ent.z;
    using R = Rec<DK, DV, F16>;
    unsigned char* rec = P.rec + (static_cast<size_t>(h) * P.gmax + g) * P.rec_bytes;

    extern __shared__ __align__(16) unsigned char lds[];
    float* s_b = reinterpret_cast<float*>(lds);
    float* s_T = reinterpret_cast<float*>(lds);                       // after b is dead
    A* s_v = reinterpret_cast<A*>(lds + C * TP * 4);                  // after b is dead
    A* s_kraw = reinterpret_cast<A*>(lds + L::R1);
    E* s_khat = reinterpret_cast<E*>(lds + L::R1);                    // K-hat, in place
    A* s_q = reinterpret_cast<A*>(lds + L::R1 + L::R2);
    float* s_A = reinterpret_cast<float*>(lds + L::R1 + L::R2);       // after q is dead
    E* s_Tp = reinterpret_cast<E*>(lds + L::R1 + L::R2);              // after A is dead
    float* s_beta = reinterpret_cast<float*>(lds + L::R1 + L::R2 + L::R3);
    float* s_part = s_beta + C;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lm = lane & 15;
    const int lg = lane >> 4;

    const A* __restrict__ q = static_cast<const A*>(P.q);
    const A* __restrict__ k = static_cast<const A*>(P.k);
    const A* __restrict__ v = static_cast<const A*>(P.v);
    auto row_k = [&](int r) { return (static_cast<size_t>(t0 + r) * H + h) * DK; };
    auto row_v = [&](int r) { return (static_cast<size_t>(t0 + r) * H + h) * DV; };

    // ---- (0) every global load of the chunk, up front ------------------------
    const int c_own = tid % DK;                 // cumsum: channel and row part
    const int part = tid / DK;
    float al[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const int r = part * RP + i;
        al[i] = r < len ? P.alpha[row_k(r) + c_own] : 1.f;
    }
    uint4 kreg[NK], qreg[NK], vreg[NV];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int id = tid + 256 * j;
        const int r = id / KROW16;
        const int cc = (id - r * KROW16) * EL16;
        kreg[j] = make_uint4(0, 0, 0, 0);
        qreg[j] = make_uint4(0, 0, 0, 0);
        if (r < len) {
            kreg[j] = *reinterpret_cast<const uint4*>(k + row_k(r) + cc);
            qreg[j] = *reinterpret_cast<const uint4*>(q + row_k(r) + cc);
        }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int id = tid + 256 * j;
        const int r = id / VROW16;
        const int cc = (id - r * VROW16) * EL16;
        vreg[j] = make_uint4(0, 0, 0, 0);
        if (r < len) vreg[j] = *reinterpret_cast<const uint4*>(v + row_v(r) + cc);
    }
    const float bet = (tid < C && tid < len) ? P.beta[static_cast<size_t>(t0 + tid) * H + h] : 0.f;

    // ---- (a) k, q to LDS; b = cumsum(log2 alpha) per key channel -------------
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int id = tid + 256 * j;
        const int r = id / KROW16;
        const int cc = (id - r * KROW16) * EL16;
        *reinterpret_cast<uint4*>(s_kraw + r * KP + cc) = kreg[j];
        *reinterpret_cast<uint4*>(s_q + r * KP + cc) = qreg[j];
    }
    if (tid < C) s_beta[tid] = bet;
    {
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            run += flog2(al[i]);
            al[i] = run;
        }
        s_part[part * DK + c_own] = run;
        __syncthreads();
        float off = 0.f;
        for (int pp = 0; pp < part; ++pp) off += s_part[pp * DK + c_own];
#pragma unroll
        for (int i = 0; i < RP; ++i) s_b[(part * RP + i) * BP + c_own] = al[i] + off;
        __syncthreads();
    }

    auto kraw = [&](int r, int c) -> float {
        if constexpr (F16) return bf16_to_f32(s_kraw[r * KP + c]);
        else return s_kraw[r * KP + c];
    };
    auto qraw = [&](int r, int c) -> float {
        if constexpr (F16) return bf16_to_f32(s_q[r * KP + c]);
        else return s_q[r * KP + c];
    };

    // ---- (b) gamma, Gamma.Q and ((gamma/Gamma).K)^T in fragment order --------
    {
        E* __restrict__ qh = reinterpret_cast<E*>(rec + R::QH);
        E* __restrict__ ktt = reinterpret_cast<E*>(rec + R::KTT);
        if (tid < DK) reinterpret_cast<float*>(rec + R::GAM)[tid] = fexp2(s_b[(C - 1) * BP + tid]);
        constexpr int KS = DK / 32;
        // Gamma.Q: fragment f = (token tile) * KS + (channel step)
        for (int id = tid; id < C * KS * 4; id += 256) {
            const int m = id & 15, j = (id >> 4) & 3, f = id >> 6;
            const int rt = f / KS, ks = f - rt * KS;
            const int r = 16 * rt + m;
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 32 * ks + frag_k(j, e);
                qv[e] = qraw(r, c) * fexp2(s_b[r * BP + c]);
            }
            M::store8(qh + frag_off(f, id & 63), qv);
        }
        // ((gamma/Gamma).K)^T: fragment f = (channel tile) * 2 + (token step)
        for (int id = tid; id < DK * 2 * 4; id += 256) {
            const int m = id & 15, j = (id >> 4) & 3, f = id >> 6;
            const int ct = f >> 1, ts = f & 1;
            const int c = 16 * ct + m;
            const float bl = s_b[(C - 1) * BP + c];
            float kv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 32 * ts + frag_k(j, e);
                kv[e] = kraw(t, c) * fexp2(bl - s_b[t * BP + c]);
            }
            M::store8(ktt + frag_off(f, id & 63), kv);
        }
    }

    // ---- (c) A and P on the matrix cores; wave I owns rows 16I..16I+15 -------
    {
        const int I = wave;
        const int rr = 16 * I + lm;                 // this lane's row (A operand)
        const int refr = 16 * I + 7;                // reference token of block I
        E* __restrict__ pout = reinterpret_cast<E*>(rec + R::P);
        constexpr int KS = DK / 32;
        V kr[KS], qr[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c0 = 32 * ks + 8 * lg;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = fexp2(s_b[rr * BP + c0 + e] - s_b[refr * BP + c0 + e]);
                kr[ks][e] = M::cvt(kraw(rr, c0 + e) * f);
                qr[ks][e] = M::cvt(qraw(rr, c0 + e) * f);
            }
        }
        __syncthreads();                            // q is dead; its region takes A
        // A in the accumulator layout (rows of A) for the solve; P as P^T tiles
        // so that its fragments can be stored straight from the accumulators.
        f4 accP[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            accP[J] = f4{0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
                const int s = 16 * J + lm;          // this lane's column token
                f4 accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c0 = 32 * ks + 8 * lg;
                    V kc;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        kc[e] = M::cvt(kraw(s, c0 + e) *
                                       fexp2(s_b[refr * BP + c0 + e] - s_b[s * BP + c0 + e]));
                    accA = M::mma(kr[ks], kc, accA);
                    accP[J] = M::mma(kc, qr[ks], accP[J]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * lg + i;
                    s_A[r * AP + s] = s < r ? s_beta[r] * accA[i] : 0.f;
                }
            }
        }
        // lane (lm, lg) of P^T tile J holds P[16I+lm][16J+4lg+i]
        const int r = 16 * I + lm;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s0 = 32 * ks + 4 * lg + e, s1 = s0 + 16;
                pv[e] = s0 <= r ? accP[2 * ks][e] : 0.f;
                pv[4 + e] = s1 <= r ? accP[2 * ks + 1][e] : 0.f;
            }
            M::store8(pout + frag_off(2 * I + ks, lane), pv);
        }
    }
    __syncthreads();

    // ---- (d) K-hat = Gamma.K in place (operand type); b dies here -----------
    for (int id = tid; id < C * DK; id += 256) {
        const int r = id / DK;
        const int c = id - r * DK;
        // each element is read and rewritten by the same thread
        const float kv = kraw(r, c) * fexp2(s_b[r * BP + c]);
        s_khat[r * KP + c] = M::cvt(kv);
    }
    __syncthreads();

    // ---- (e) v into LDS; T = (I + A)^-1 --------------------------------------
    {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int id = tid + 256 * j;
            const int r = id / VROW16;
            const int cc = (id - r * VROW16) * EL16;
            *reinterpret_cast<uint4*>(s_v + r * VP + cc) = vreg[j];
        }
        // diagonal 16x16 blocks by forward substitution; lane j owns column j
        if (lane < 16) {
            const int I = wave;
            const int j = lane;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= s_A[(16 * I + r) * AP + 16 * I + s] * x[s];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_T[(16 * I + r) * TP + 16 * I + j] = x[r];
        }
        __syncthreads();
        // blocks below the diagonal: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
        for (int I = 1; I < 4; ++I) {
            if (wave < I) {
                const int J = wave;
                f4 X = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const float a = s_A[(16 * I + lm) * AP + 16 * K + 4 * kk + lg];
                        const float b = s_T[(16 * K + 4 * kk + lg) * TP + 16 * J + lm];
                        X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, X, 0, 0, 0);
                    }
                }
                f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = -s_T[(16 * I + lm) * TP + 16 * I + 4 * lg + i];
                    Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, X[i], Y, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) s_T[(16 * I + 4 * lg + i) * TP + 16 * J + lm] = Y[i];
            }
            __syncthreads();
        }
        // T Diag(beta), zero above the diagonal, in the operand type
        for (int id = tid; id < C * C; id += 256) {
            const int r = id / C;
            const int s = id - r * C;
            s_Tp[r * TPP + s] = M::cvt(s <= r ? s_T[r * TP + s] * s_beta[s] : 0.f);
        }
        __syncthreads();
    }

    // ---- (f) W = T Diag(beta) K-hat and U = T Diag(beta) V ------------------
    {
        E* __restrict__ wout = reinterpret_cast<E*>(rec + R::W);
        float* __restrict__ uout = reinterpret_cast<float*>(rec + R::UT);
        constexpr int KS = DK / 32;
        // W^T tiles (channels x tokens): the pair of channel tiles of one
        // channel step gives a W fragment lane by lane.
        for (int item = wave; item < KS * 4; item += 4) {
            const int ksc = item >> 2;              // channel step
            const int I = item & 3;                 // token tile
            f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            const int kmax = (16 * I + 16 + 31) / 32;
            for (int kt = 0; kt < kmax; ++kt) {
                const int t = 32 * kt + 8 * lg;
                const V bT = M::load8(s_Tp + (16 * I + lm) * TPP + t);
                V a0, a1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a0[e] = s_khat[(t + e) * KP + 32 * ksc + lm];
                    a1[e] = s_khat[(t + e) * KP + 32 * ksc + 16 + lm];
                }
                acc0 = M::mma(a0, bT, acc0);
                acc1 = M::mma(a1, bT, acc1);
            }
            const float wv[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
            M::store8(wout + frag_off(I * KS + ksc, lane), wv);
        }
        // U in the accumulator layout the state kernel consumes directly
        for (int nt = wave; nt < DV / 16; nt += 4) {
            const int c = 16 * nt + lm;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                const int kmax = (16 * I + 16 + 31) / 32;
                for (int ks = 0; ks < kmax; ++ks) {
                    const int t = 32 * ks + 8 * lg;
                    const V a = M::load8(s_Tp + (16 * I + lm) * TPP + t);
                    V b;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if constexpr (F16) b[e] = M::cvt(bf16_to_f32(s_v[(t + e) * VP + c]));
                        else b[e] = s_v[(t + e) * VP + c];
                    }
                    acc = M::mma(a, b, acc);
                }
                *reinterpret_cast<f4*>(uout + (static_cast<size_t>(nt * 4 + I) * 64 + lane) * 4) = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// state_kernel: the sequential pass over the chunks of one sequence for one
// head and 16 value columns.  Wave w keeps state rows [w*DK/4, (w+1)*DK/4) of
// those 16 columns in registers; an fp16/fp32 copy of the whole 16-column
// state slice lives in LDS as the matrix-core operand of the next chunk.
// The operands of the next kDepth-1 chunks are in flight in a register ring
// while a chunk is computed, so the chain does not wait on memory latency.
// ---------------------------------------------------------------------------
struct StateParams {
    const int32_t* first;
    const int32_t* order;
    const int4* table;
    const unsigned char* rec;
    size_t rec_bytes;
    int64_t gmax;
    const float* initial_state;
    float* final_state;
    void* o;
    int N;
    int H;
};

template <int DK, bool F16>
struct StateStage {
    using V = typename Mx<F16>::V;
    static constexpr int KS = DK / 32;
    static constexpr int TPW = DK / 64;
    V w[KS], q[KS];          // rows 16w..16w+15 of W and Gamma.Q
    V p[2];                  // row 16w+lm of P, tokens 0..63
    V k[TPW][2];             // rows of ((gamma/Gamma).K)^T owned by this wave
    f4 u;                    // U^T: column `col`, tokens 16w+4lg..+3
    f4 gm[TPW];              // gamma for the owned state rows
    int t0, len;
};

template <bool F16> struct StateDepth { static constexpr int value = F16 ? 4 : 2; };

template <int DK, int DV, bool F16, bool OBF16>
__global__ __launch_bounds__(256) void state_kernel(const StateParams P) {
    using M = Mx<F16>;
    using E = typename M::E;
    using V = typename M::V;
    using Stage = StateStage<DK, F16>;
    using R = Rec<DK, DV, F16>;
    constexpr int D = StateDepth<F16>::value;   // chunks in flight
    constexpr int NTV = DV / 16;          // 16-column tiles per (sequence, head)
    constexpr int RPW = DK / 4;           // state rows per wave
    constexpr int TPW = RPW / 16;         // 16-row tiles per wave
    constexpr int KS = DK / 32;
    constexpr int SP = DK + 8;            // LDS row stride of the state operand
    constexpr int UP = C + 8;             // LDS row stride of U'

    // Workgroups are handed to the 8 XCDs round-robin; keep the NTV tiles of
    // one (sequence, head) on the same XCD so they share its L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int pair = (slot / NTV) * 8 + xcd;
    const int jt = slot - (slot / NTV) * NTV;
    const int H = P.H;
    if (pair >= P.N * H) return;
    const int n = P.order[pair / H];
    const int h = pair - (pair / H) * H;
    const int g0 = P.first[n];
    const int g1 = P.first[n + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lm = lane & 15;
    const int lg = lane >> 4;
    const int col = 16 * jt + lm;

    __shared__ __align__(16) E s_S[16 * SP];   // [value column][key row]
    __shared__ __align__(16) E s_U[16 * UP];   // [value column][token]

    const size_t sbase = (static_cast<size_t>(n) * H + h) * (DK * DV);
    f4 S[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = RPW * wave + 16 * t + 4 * lg + i;
            S[t][i] = P.initial_state ? P.initial_state[sbase + row * DV + col] : 0.f;
        }
        M::store4(s_S + lm * SP + RPW * wave + 16 * t + 4 * lg, S[t]);
    }

    const unsigned char* recs = P.rec + static_cast<size_t>(h) * P.gmax * P.rec_bytes;

    auto load = [&](Stage& st, int g) {
        const int4 ent = P.table[g];
        st.t0 = ent.y;
        st.len = ent.z;
        const unsigned char* rec = recs + static_cast<size_t>(g) * P.rec_bytes;
        const E* wr = reinterpret_cast<const E*>(rec + R::W);
        const E* qr = reinterpret_cast<const E*>(rec + R::QH);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            st.w[ks] = M::load8(wr + frag_off(wave * KS + ks, lane));
            st.q[ks] = M::load8(qr + frag_off(wave * KS + ks, lane));
        }
        const E* pr = reinterpret_cast<const E*>(rec + R::P);
        st.p[0] = M::load8(pr + frag_off(2 * wave, lane));
        st.p[1] = M::load8(pr + frag_off(2 * wave + 1, lane));
        const float* gam = reinterpret_cast<const float*>(rec + R::GAM);
        const E* kt = reinterpret_cast<const E*>(rec + R::KTT);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            st.k[t][0] = M::load8(kt + frag_off((TPW * wave + t) * 2, lane));
            st.k[t][1] = M::load8(kt + frag_off((TPW * wave + t) * 2 + 1, lane));
            st.gm[t] = *reinterpret_cast<const f4*>(gam + RPW * wave + 16 * t + 4 * lg);
        }
        st.u = *reinterpret_cast<const f4*>(reinterpret_cast<const float*>(rec + R::UT) +
                                            (static_cast<size_t>(jt * 4 + wave) * 64 + lane) * 4);
    };

    auto compute = [&](const Stage& st) {
        // (1) X = W S and O = (Gamma.Q) S for tokens 16w..16w+15
        f4 X = {0.f, 0.f, 0.f, 0.f}, O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const E* sb = s_S + lm * SP + 32 * ks + 4 * lg;
            const V bS = M::load4x2(sb, sb + 16);
            X = M::mma(st.w[ks], bS, X);
            O = M::mma(st.q[ks], bS, O);
        }
        // (2) U' = U - W S, shared through LDS
        M::store4(s_U + lm * UP + 16 * wave + 4 * lg, st.u - X);
        __syncthreads();
        // (3) O += Tril(...) U'  (tokens above this wave's rows are zero in P)
        const E* ub = s_U + lm * UP + 4 * lg;
        const V bU0 = M::load4x2(ub, ub + 16);
        const V bU1 = M::load4x2(ub + 32, ub + 48);
        O = M::mma(st.p[0], bU0, O);
        if (wave >= 2) O = M::mma(st.p[1], bU1, O);
        // (4) S <- Diag(gamma) S + ((gamma/Gamma).K)^T U'
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = M::mma(st.k[t][0], bU0, acc);
            acc = M::mma(st.k[t][1], bU1, acc);
            S[t] = st.gm[t] * S[t] + acc;
            M::store4(s_S + lm * SP + RPW * wave + 16 * t + 4 * lg, S[t]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * wave + 4 * lg + i;
            if (r < st.len) store_out<OBF16>(P.o, (static_cast<size_t>(st.t0 + r) * H + h) * DV + col, O[i]);
        }
        __syncthreads();
    };

    __syncthreads();
    // Ring loads are unconditional (clamped to the last chunk; the surplus
    // loads at the tail are never used) so that the loop body is straight-line
    // code and the hardware wait counters never have to drain the ring.
    Stage st[D];
    if (g0 < g1) {
#pragma unroll
        for (int j = 0; j < D - 1; ++j) load(st[j], min(g0 + j, g1 - 1));
    }
    for (int g = g0; g < g1; g += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            load(st[(j + D - 1) % D], min(g + j + D - 1, g1 - 1));
            if (g + j < g1) compute(st[j]);
        }
    }

    if (P.final_state) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = RPW * wave + 16 * t + 4 * lg + i;
                P.final_state[sbase + row * DV + col] = S[t][i];
            }
        }
    }
}


size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <int DK, int DV, bool F16, bool OBF16>
hipError_t launch_typed(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* ctrl = reinterpret_cast<int32_t*>(ws + pl.off_ctrl);
    int32_t* first = reinterpret_cast<int32_t*>(ws + pl.off_first);
    int32_t* order = reinterpret_cast<int32_t*>(ws + pl.off_order);
    int4* table = reinterpret_cast<int4*>(ws + pl.off_table);

    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.cu_seqlens, pl.N,
                       pl.varlen ? static_cast<int64_t>(0) : pl.T, pl.gmax, ctrl, first, order, table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (pl.gmax > 0) {
        PrepParams pp;
        pp.q = a.q; pp.k = a.k; pp.v = a.v; pp.alpha = a.alpha; pp.beta = a.beta;
        pp.ctrl = ctrl; pp.table = table;
        pp.rec = ws + pl.off_rec; pp.rec_bytes = pl.rec_bytes; pp.gmax = pl.gmax;
        pp.H = pl.H;
        constexpr int lds = PrepLds<DK, DV, F16>::bytes;
        auto kfn = prep_kernel<DK, DV, F16>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kfn, dim3(static_cast<unsigned>(pl.gmax * pl.H)), dim3(256), lds, stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    StateParams sp;
    sp.first = first; sp.order = order; sp.table = table;
    sp.rec = ws + pl.off_rec; sp.rec_bytes = pl.rec_bytes; sp.gmax = pl.gmax;
    sp.initial_state = a.initial_state;
    sp.final_state = a.final_state;
    sp.o = a.o;
    sp.N = pl.N;
    sp.H = pl.H;
    const int64_t pairs = static_cast<int64_t>(pl.N) * pl.H;
    const int64_t blocks = (pairs + 7) / 8 * 8 * (DV / 16);
    hipLaunchKernelGGL((state_kernel<DK, DV, F16, OBF16>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, stream, sp);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (!a.act_bf16) return launch_typed<DK, DV, false, false>(pl, a, stream);
    if (a.out_bf16) return launch_typed<DK, DV, true, true>(pl, a, stream);
    return launch_typed<DK, DV, true, false>(pl, a, stream);
}

}  // namespace

kda_status make_chunk_plan(int B, int64_t T, int H, int Dk, int Dv, bool varlen, int num_seqs,
                           int chunk_size, bool act_bf16, ChunkPlan* plan) {
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0) return KDA_ERROR_INVALID_VALUE;
    if ((Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128) || chunk_size != C)
        return KDA_ERROR_NOT_SUPPORTED;
    if (varlen && B != 1) return KDA_ERROR_INVALID_VALUE;
    ChunkPlan p;
    p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.varlen = varlen; p.f16 = act_bf16;
    p.N = varlen ? num_seqs : B;
    const int64_t tokens = static_cast<int64_t>(B) * T;
    if (tokens >= (static_cast<int64_t>(1) << 31)) return KDA_ERROR_NOT_SUPPORTED;
    const int64_t per_seq_chunks = (T + C - 1) / C;
    p.gmax = varlen ? per_seq_chunks + p.N : static_cast<int64_t>(B) * per_seq_chunks;
    if (p.gmax * H >= (static_cast<int64_t>(1) << 31)) return KDA_ERROR_NOT_SUPPORTED;
    const int64_t pairs = static_cast<int64_t>(p.N) * H;
    if ((pairs + 7) / 8 * 8 * (Dv / 16) >= (static_cast<int64_t>(1) << 31)) return KDA_ERROR_NOT_SUPPORTED;
    p.eb = act_bf16 ? 2 : 4;
    const size_t gh = static_cast<size_t>(p.gmax) * H;
    size_t off = 0;
    p.off_ctrl = off;  off = align256(off + 16);
    p.off_first = off; off = align256(off + 4 * (static_cast<size_t>(p.N) + 1));
    p.off_order = off; off = align256(off + 4 * static_cast<size_t>(p.N));
    p.off_table = off; off = align256(off + 16 * static_cast<size_t>(p.gmax));
    // per (head, chunk) record: qh, w, ktt, p (operand type), ut, gam (fp32)
    p.rec_bytes = align256(3 * static_cast<size_t>(C) * Dk * p.eb + static_cast<size_t>(C) * C * p.eb +
                           static_cast<size_t>(C) * Dv * 4 + static_cast<size_t>(Dk) * 4);
    p.off_rec = off;   off = align256(off + gh * p.rec_bytes);
    p.workspace_bytes = off;
    *plan = p;
    return KDA_SUCCESS;
}

hipError_t launch_chunk_fwd(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (pl.Dk == 128 && pl.Dv == 128) return launch_dims<128, 128>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 64) return launch_dims<64, 64>(pl, a, stream);
    if (pl.Dk == 128 && pl.Dv == 64) return launch_dims<128, 64>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 128) return launch_dims<64, 128>(pl, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
