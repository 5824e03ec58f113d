// Chunkwise KDA forward for gfx950.
//
// The chunked algorithm of "Linear Attention KDA Gating in a 3:1 Hybrid
// Architecture: Principles and Implementation Guide", section 3, carried out
// in four launches on the caller's stream:
//
//   plan_kernel   (integer)  chunk table: which sequence, first token row and
//                 length every 64-token chunk has; sequence order by length.
//   prep_kernel   (chunk-parallel, one workgroup per (chunk, head))
//                 the in-chunk decay ("log-domain accumulation", "Designing
//                 and Deploying Hybrid MLA and Linear Attention
//                 Architectures", section 3);
//                 A = strictly-lower(Diag(beta)(Gamma.K)(K/Gamma)^T) and
//                 P = Tril((Gamma.Q)(K/Gamma)^T) on the matrix cores;
//                 T = (I + A)^-1 by blocked forward substitution;
//                 W = T Diag(beta)(Gamma.K), U = T Diag(beta) V on the matrix
//                 cores; Gamma.Q, ((gamma/Gamma).K)^T and gamma -> record.
//                 Direct form; a (chunk, head) outside its range is listed
//                 for the next launch.
//   prep_general_kernel  the same for each listed (chunk, head), general form.
//   state_split_kernel (fp16 records) / state_kernel (fp32 records)
//                 (sequential over the chunks of one sequence, one
//                 workgroup per (sequence, head, 16 value columns))
//                 U' = U - W S,  O = (Gamma.Q) S + P U',
//                 S <- Diag(gamma) S + ((gamma/Gamma).K)^T U'
//                 (inter-chunk transition of section 3.1, masked intra-chunk
//                 output of section 3.2), S kept in registers throughout.
//
// Records are stored chunk-major ([chunk][head]): the sequential pass walks
// the chunks of all heads in step, and with head-major records the heads
// that share an XCD would sit a multiple of 2 MiB apart, on the same L2 sets.
//
// Reading of the garbled passages: Gamma_r is the inclusive per-channel
// product of alpha over the chunk's first r tokens; W and U are per-token
// rows obtained with the unit-lower-triangular inverse (I + A)^-1; Tril keeps
// the diagonal.  The padded tail of a partial chunk has alpha = 1, beta = 0
// and q = k = v = 0, which leaves every result unchanged.
//
// Numerics.  All accumulation is fp32.  With bf16 activations the matrix-core
// operands are fp16 (11-bit significand, 8x finer than bf16); with fp32
// activations every product runs on the fp32 matrix cores.  The decay between
// two tokens, e^{b_r - b_s} (s <= r), takes one of two forms ("chunk-wise
// normalization", same section):
//   direct   split as e^{b_r - ref} * e^{ref - b_s} around a reference token
//            in the middle of each 16-token block, so a factor spans at most
//            8 tokens of decay; used when every channel decays by at most
//            2^-64 over the chunk and, with fp16 operands, by at most 2^-14
//            over each 16-token block, with |k|, |q| <= 2 (every fp16 operand
//            then stays below 2^15);
//   general  every factor a product of alpha over a run of tokens, never
//            above 1, for any gate in [0, 1] (prep_general_kernel).
#include <type_traits>

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
    // four elements (8-byte aligned), converted where they are used
    using V4 = h4;
    static __device__ __forceinline__ V4 load4(const E* p) { return *reinterpret_cast<const h4*>(p); }
    static __device__ __forceinline__ f4 tof4(V4 a) {
        return f4{static_cast<float>(a[0]), static_cast<float>(a[1]), static_cast<float>(a[2]),
                  static_cast<float>(a[3])};
    }
    static __device__ __forceinline__ void store4(E* p, f4 x) {
        h4 h = {static_cast<E>(x[0]), static_cast<E>(x[1]), static_cast<E>(x[2]), static_cast<E>(x[3])};
        *reinterpret_cast<h4*>(p) = h;
    }
    static __device__ __forceinline__ void storeV(E* p, const V& v) { *reinterpret_cast<V*>(p) = v; }
    // Transposed operand read from a row-major LDS tile M (row stride ld):
    // element e of lane (j = l % 16) is M[ra + e][c0 + j] for e < 4 and
    // M[rb + e - 4][c0 + j] for e >= 4.  Within each 16-lane group, the
    // transposing LDS read hands lane j element j % 4 of the 64-bit words read
    // by lanes 4k + j / 4 (k = 0..3); lane s therefore points at row
    // (ra + s / 4), columns c0 + 4 (s % 4) .. + 3.
    static __device__ __forceinline__ V loadT(const E* M, int ld, int ra, int rb, int c0, int j) {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const int off = (j >> 2) * ld + c0 + 4 * (j & 3);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(M + ra * ld + off));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(M + rb * ld + off));
        const h4 l4 = __builtin_bit_cast(h4, lo), h4v = __builtin_bit_cast(h4, hi);
        V v;
        v[0] = l4[0]; v[1] = l4[1]; v[2] = l4[2]; v[3] = l4[3];
        v[4] = h4v[0]; v[5] = h4v[1]; v[6] = h4v[2]; v[7] = h4v[3];
        return v;
    }
    static __device__ __forceinline__ void store8(E* p, const float* x) {
        h8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<E>(x[e]);
        *reinterpret_cast<h8*>(p) = h;
    }
    // Record stores, non-temporal when `nt` (records too large to stay in the
    // caches until the next kernel reads them: 2.19 vs 2.21 ms on the 64K-token
    // forward; records that fit are read back faster when stored normally).
    static __device__ __forceinline__ void gstore8(E* p, const float* x, bool nt) {
        if (!nt) {
            store8(p, x);
            return;
        }
        h8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<E>(x[e]);
        __builtin_nontemporal_store(h, reinterpret_cast<h8*>(p));
    }
    static __device__ __forceinline__ void gstoreV(E* p, const V& v, bool nt) {
        if (nt) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
        else storeV(p, v);
    }
    static __device__ __forceinline__ void gstore4(E* p, f4 x, bool nt) {
        if (!nt) {
            store4(p, x);
            return;
        }
        h4 h = {static_cast<E>(x[0]), static_cast<E>(x[1]), static_cast<E>(x[2]), static_cast<E>(x[3])};
        __builtin_nontemporal_store(h, reinterpret_cast<h4*>(p));
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
    using V4 = f4;
    static __device__ __forceinline__ V4 load4(const E* p) { return *reinterpret_cast<const f4*>(p); }
    static __device__ __forceinline__ f4 tof4(V4 a) { return a; }
    static __device__ __forceinline__ void store4(E* p, f4 x) { *reinterpret_cast<f4*>(p) = x; }
    static __device__ __forceinline__ void storeV(E* p, const V& v) {
        *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f4*>(p + 4) = f4{v[4], v[5], v[6], v[7]};
    }
    // same element order as the 16-bit variant, by plain reads
    static __device__ __forceinline__ V loadT(const E* M, int ld, int ra, int rb, int c0, int j) {
        V v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = M[(ra + e) * ld + c0 + j];
            v[4 + e] = M[(rb + e) * ld + c0 + j];
        }
        return v;
    }
    static __device__ __forceinline__ void store8(E* p, const float* x) {
        f4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
        *reinterpret_cast<f4*>(p) = lo;
        *reinterpret_cast<f4*>(p + 4) = hi;
    }
    static __device__ __forceinline__ void gstore8(E* p, const float* x, bool nt) {
        if (!nt) {
            store8(p, x);
            return;
        }
        __builtin_nontemporal_store(f4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f4*>(p));
        __builtin_nontemporal_store(f4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f4*>(p + 4));
    }
    static __device__ __forceinline__ void gstoreV(E* p, const V& v, bool nt) {
        if (!nt) {
            storeV(p, v);
            return;
        }
        __builtin_nontemporal_store(f4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4*>(p));
        __builtin_nontemporal_store(f4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f4*>(p + 4));
    }
    static __device__ __forceinline__ void gstore4(E* p, f4 x, bool nt) {
        if (nt) __builtin_nontemporal_store(x, reinterpret_cast<f4*>(p));
        else store4(p, x);
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
// holds row m at reduction indices frag_k(j, e) = e < 4 ? 4j + e : 12 + 4j + e,
// e = 0..7: two runs of four, 4j..4j+3 and 16+4j..16+4j+3.  Any bijection onto the 32 indices gives the
// same product as long as both operands of an MFMA use it; this one lets a
// 16x16 accumulator tile pair (rows 4j..4j+3 of each tile in lane (m, j))
// be written as a fragment without moving data between lanes.
// With 16-bit records, Gamma.Q is the exception: it is written from the
// preparation pass's registers, whose lanes hold eight consecutive channels
// (8j..8j+7, the matrix core's own order), so its reader takes the state
// operand in that order.

__device__ __forceinline__ size_t frag_off(int f, int lane) { return (static_cast<size_t>(f) * 64 + lane) * 8; }

// P (C x C, lower triangular) in the record: fragment 2I + h holds token rows
// 16I..16I+15 and columns 32h..32h+31, and the fragments 1 and 3 (rows below
// 32, columns from 32 on) are all zero, so only the other six are stored.
constexpr int kPFrags = 6;
__device__ __forceinline__ int p_slot(int f) { return f == 0 ? 0 : f == 2 ? 1 : f - 2; }


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
                                                            int64_t T, int64_t gmax, int csize,
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
            cnt = len > 0 ? (len + csize - 1) / csize : 0;
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
        ctrl[1] = 0;              // the backward's general-form list starts empty
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
        const int l = len - i * csize;
        table[g] = make_int4(n, start + i * csize, l < csize ? l : csize, 0);
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
// state entering the chunk.  Wave I owns tokens 16I..16I+15 in the
// matrix-core lane layout; all global loads are issued first.
// ---------------------------------------------------------------------------
struct PrepParams {
    const void* q;
    const void* k;
    const void* v;
    const void* gate;         // forget gate in the form of the kernel's GATE (kda_gate)
    const float* beta;
    const int32_t* ctrl;
    const int4* table;
    unsigned char* rec;
    size_t rec_bytes;
    int64_t gmax;
    int H;
    int64_t T;     // tokens per sequence of a dense batch; 0 for varlen
    int cps;       // chunks per sequence of a dense batch
    int32_t* nslow;   // length of the general-form list (zeroed by the chunk table)
    int32_t* slow;    // general-form list: g * H + h of each (chunk, head) that takes it
    bool nt;          // records stored non-temporally (too large to stay in the caches)
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
    static constexpr size_t UT = P + sizeof(E) * kPFrags * 512;
    static constexpr size_t GAM = UT + sizeof(E) * DV * C;
    static constexpr size_t END = GAM + 4 * DK;
};

// Four consecutive activations: loaded raw, widened to fp32 where used.
template <bool BF16> struct Raw4;
template <> struct Raw4<true> {
    using T = uint2;
    static __device__ __forceinline__ T load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    static __device__ __forceinline__ f4 widen(T r) {
        return f4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                  __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    }
};
template <> struct Raw4<false> {
    using T = f4;
    static __device__ __forceinline__ T load(const float* p) { return *reinterpret_cast<const f4*>(p); }
    static __device__ __forceinline__ f4 widen(T r) { return r; }
};

template <int DK, int DV, bool F16>
struct PrepLds {
    using A = typename Act<F16>::T;   // raw activation element
    using E = typename Mx<F16>::E;    // matrix-core operand element
    static constexpr int KS = DK / 32;
    static constexpr int KXP = DK + 16;      // row stride of the token-major K-hat and K~
    static constexpr int VXP = DV + 16;      // row stride of the token-major V
    static constexpr int ATP = C + 4;        // fp32 row stride of A^T ([s][r])
    static constexpr int TP = C + 4;         // fp32 row stride of T
    static constexpr int TPP = C + 8;        // row stride of T Diag(beta) (operand type)
    // region a: column operands of the six blocks below the diagonal, later T (fp32)
    static constexpr int RA = CMax<6 * KS * 64 * 8 * (int)sizeof(E), C * TP * 4>::value;
    // region b: K~ [token][channel], later V [token][column] (operand type)
    static constexpr int RB = CMax<C * KXP, C * VXP>::value * (int)sizeof(E);
    // region c: K-hat [token][channel]
    static constexpr int RC = C * KXP * (int)sizeof(E);
    // region d: A^T (fp32), later T Diag(beta)
    static constexpr int RD = CMax<C * ATP * 4, C * TPP * (int)sizeof(E)>::value;
    // small: beta [64]
    static constexpr int RS = C * 4;
    // the block totals of the decay [4][DK] (general form) or the totals and
    // decay factors [4 + 16][DK] (direct form) live in region d until A^T is
    // written there
    static_assert(RD >= 20 * DK * 4, "region d holds the direct form's decay tables");
    static constexpr int bytes = RA + RB + RC + RD + RS;
};

__device__ __forceinline__ int frag_k(int j, int e) { return e < 4 ? 4 * j + e : 12 + 4 * j + e; }
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// Inclusive prefix sum over the 16 lanes of each DPP row (row_shr by 1, 2,
// 4, 8; lanes shifted in from outside the row read 0).
__device__ __forceinline__ float row_shr_f(float x, int n) {
    const int xi = __builtin_bit_cast(int, x);
    int y = 0;
    switch (n) {
        case 1: y = __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xf, 0xf, false); break;
        case 2: y = __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xf, 0xf, false); break;
        case 4: y = __builtin_amdgcn_update_dpp(0, xi, 0x114, 0xf, 0xf, false); break;
        default: y = __builtin_amdgcn_update_dpp(0, xi, 0x118, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float row_scan16(float x) {
    x += row_shr_f(x, 1);
    x += row_shr_f(x, 2);
    x += row_shr_f(x, 4);
    x += row_shr_f(x, 8);
    return x;
}

// Lanes of one 16-lane row hold 16 consecutive tokens.  Returns x of lane
// (lane ^ 2^p) | (2^p - 1): the last token of the other half of this token's
// aligned group of 2^(p+1) tokens.  p = 0, 1 stay inside a quad (DPP quad
// permutes [1,0,3,2] and [3,3,1,1]); p = 2, 3 go through the LDS crossbar.
__device__ __forceinline__ float other_half_last(int p, float x, int lane) {
    const int xi = __builtin_bit_cast(int, x);
    int y;
    if (p == 0) y = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xf, 0xf, false);
    else if (p == 1) y = __builtin_amdgcn_update_dpp(0, xi, 0x5F, 0xf, 0xf, false);
    else {
        const int src = (lane ^ (1 << p)) | ((1 << p) - 1);
        y = __builtin_amdgcn_ds_bpermute(src << 2, xi);
    }
    return __builtin_bit_cast(float, y);
}

// (I, J) with J < I -> index into the rescaling table
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <int DK, int DV, bool F16, int GATE, bool FAST>
__device__ __forceinline__ void prep_body(const PrepParams& P, const int blk) {
    using L = PrepLds<DK, DV, F16>;
    using A = typename L::A;
    using M = Mx<F16>;
    using E = typename M::E;
    using V = typename M::V;
    using R = Rec<DK, DV, F16>;
    constexpr int KS = L::KS, KXP = L::KXP, VXP = L::VXP, ATP = L::ATP, TP = L::TP, TPP = L::TPP;
    constexpr int EL16 = 16 / (int)sizeof(A);              // activations per 16 bytes
    constexpr int VROW16 = DV / EL16;
    constexpr int NV = C * VROW16 / 256;

    const int H = P.H;
    const int g = blk / H;
    const int h = blk - g * H;
    int t0, len;
    if (P.T > 0) {
        // dense batch: chunk g is chunk j of sequence n
        const int n = g / P.cps;
        const int j = g - n * P.cps;
        t0 = static_cast<int>(n * P.T) + C * j;
        len = min(C, static_cast<int>(P.T) - C * j);
    } else {
        if (g >= P.ctrl[0]) return;
        const int4 ent = P.table[g];
        t0 = ent.y;
        len = ent.z;
    }
    unsigned char* rec = P.rec + (static_cast<size_t>(g) * P.H + h) * P.rec_bytes;

    extern __shared__ __align__(16) unsigned char lds[];
    E* s_C = reinterpret_cast<E*>(lds);                                 // column fragments
    float* s_T = reinterpret_cast<float*>(lds);                         // after s_C is dead
    E* s_Kt = reinterpret_cast<E*>(lds + L::RA);                        // K~ [token][channel]
    E* s_v = reinterpret_cast<E*>(lds + L::RA);                         // V, after s_Kt is dead
    E* s_khat = reinterpret_cast<E*>(lds + L::RA + L::RB);              // K-hat [token][channel]
    float* s_AT = reinterpret_cast<float*>(lds + L::RA + L::RB + L::RC);
    E* s_Tp = reinterpret_cast<E*>(lds + L::RA + L::RB + L::RC);        // after A^T is dead
    float* s_F = s_AT;                                                  // [4][DK] block totals, until (c)
    float* s_beta = reinterpret_cast<float*>(lds + L::RA + L::RB + L::RC + L::RD);  // [C]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lm = lane & 15;
    const int lg = lane >> 4;
    const int I = wave;                       // this wave's 16-token block
    const int r = 16 * I + lm;                // this lane's token
    const bool valid = r < len;

    const A* __restrict__ q = static_cast<const A*>(P.q);
    const A* __restrict__ k = static_cast<const A*>(P.k);
    const A* __restrict__ v = static_cast<const A*>(P.v);
    auto row_v = [&](int rr) { return (static_cast<size_t>(t0 + rr) * H + h) * DV; };

    // Lane (lm, lg) owns token r and, in reduction step ks, eight channels:
    // with 16-bit activations the run 32ks + 8lg .. + 7, read as one 16-byte
    // word per tensor (8-byte reads of two runs of four made each load touch
    // 16 rows for 32 bytes each: 1.12 vs 1.00 ms on the 64K-token forward);
    // with fp32 activations two runs of four, at 32ks + 4lg and 32ks + 16 + 4lg
    // (frag_k).  Every operand built here uses the same channels, so the
    // products agree; the Gamma.Q record carries this order to the state pass.
    auto chan_h = [&](int ks, int half) { return F16 ? 32 * ks + 8 * lg + 4 * half : 32 * ks + frag_k(lg, 4 * half); };

    // ---- (0) global loads of alpha, k, q, beta (v follows in (b)) ---------------
    // Rows past the chunk's end re-read its last row (always in bounds) and
    // are replaced by the neutral values (alpha 1, k = q = v = beta = 0) where
    // used, so the loads carry no branches and nothing waits for them early.
    using R4 = Raw4<F16>;
    const int rl = len - 1;
    typename R4::T kraw[KS][2], qraw[KS][2];
    // the gate as given: fp32 alpha or bf16 pre-activation per channel, or one
    // fp32 alpha per token
    using GRaw = typename Raw4<GATE == KDA_GATE_SOFTPLUS_BF16>::T;
    GRaw graw[KS][2];
    float gscalar = 1.f;
    {
        const size_t rowt = static_cast<size_t>(t0 + min(r, rl)) * H + h;
        const size_t rowk = rowt * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int c = chan_h(ks, half);
                if constexpr (GATE == KDA_GATE_ALPHA)
                    graw[ks][half] = *reinterpret_cast<const f4*>(static_cast<const float*>(P.gate) + rowk + c);
                if constexpr (F16) {
                    // both runs of four in one 16-byte read
                    if (half == 1) continue;
                    auto split = [](uint4 w, uint2& lo, uint2& hi) { lo = uint2{w.x, w.y}; hi = uint2{w.z, w.w}; };
                    if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16)
                        split(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.gate) + rowk + c),
                              graw[ks][0], graw[ks][1]);
                    split(*reinterpret_cast<const uint4*>(k + rowk + c), kraw[ks][0], kraw[ks][1]);
                    split(*reinterpret_cast<const uint4*>(q + rowk + c), qraw[ks][0], qraw[ks][1]);
                } else {
                    if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16)
                        graw[ks][half] = Raw4<true>::load(static_cast<const uint16_t*>(P.gate) + rowk + c);
                    kraw[ks][half] = R4::load(k + rowk + c);
                    qraw[ks][half] = R4::load(q + rowk + c);
                }
            }
        if constexpr (GATE == KDA_GATE_SCALAR) gscalar = static_cast<const float*>(P.gate)[rowt];
    }
    const float bet_raw = P.beta[static_cast<size_t>(t0 + min(r, rl)) * H + h];
    const float bet = valid ? bet_raw : 0.f;

    // Two forms of (a) - (c), chosen per (chunk, head) from its decay:
    //   direct:  b = cumsum(log2 alpha) over the chunk; Gamma = 2^b and
    //            1/Gamma as fp32 factors, each 16 x 16 block rebased at its
    //            token 16I+7, so the 16-bit operands span at most 8 tokens of
    //            decay (checked below against the operand range);
    //   general: every decay factor a product of alpha over a run of tokens,
    //            never above 1, for any gate in [0, 1].
    // Both write the same record.
    V ra[KS], rq[KS];             // row operands of the blocks below the diagonal
    [[maybe_unused]] V Dc[KS];    // direct form: column operand of the diagonal block
    [[maybe_unused]] f4 dA = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};   // general form: diagonal blocks
    __shared__ int s_bad;         // direct form: some check failed (read at the end)
    if constexpr (FAST) {
        float* s_tot = s_AT;                                            // [4][DK], until (c)
        float* s_fac = s_AT + 4 * DK;                                   // [16][DK], until (c)
        auto chan = [&](int ks, int e) { return chan_h(ks, e >> 2) + (e & 3); };
        float b[KS][8];
        // ---- (a) b = inclusive cumsum of log2(alpha) over the chunk's tokens -----
        // scan over the 16 tokens of this wave's block (lanes of one 16-lane row),
        // then add the totals of the earlier blocks
        // log2(alpha) of this lane's elements (0 past the chunk's end), scanned
        if constexpr (GATE == KDA_GATE_SCALAR) {
            const float x = row_scan16(valid ? flog2(gscalar) : 0.f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) b[ks][e] = x;
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f4 lv;
                    if constexpr (GATE == KDA_GATE_ALPHA) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) lv[i] = flog2(graw[ks][half][i]);
                    } else {
                        const f4 xv = Raw4<true>::widen(graw[ks][half]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) lv[i] = log2_alpha_from_softplus_arg(xv[i]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) b[ks][4 * half + i] = row_scan16(valid ? lv[i] : 0.f);
                }
        }
        if (lm == 15) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_tot[I * DK + chan(ks, e)] = b[ks][e];
        }
        if (lg == 0) s_beta[r] = bet;
        __syncthreads();
        for (int Ip = 0; Ip < I; ++Ip)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) b[ks][e] += s_tot[Ip * DK + chan(ks, e)];
        // Gamma = 2^b and 1/Gamma for every element; every other decay factor is
        // one of them times a per-channel constant taken at the block's reference
        // token 16I+7 (lane 7 of the row) or its last token 16I+15 (lane 15):
        //   s_fac rows 0..3 2^ref_I, 4..7 2^-ref_I, 8..11 2^end_I, 12..15 2^-end_I
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) b[ks][e] = fexp2(b[ks][e]);
        if (lm == 7 || lm == 15) {
            float* d0 = s_fac + ((lm == 7 ? 0 : 8) + I) * DK;
            float* d1 = d0 + 4 * DK;
            auto rcp4 = [&](int ks, int o) {
                return f4{__builtin_amdgcn_rcpf(b[ks][o]), __builtin_amdgcn_rcpf(b[ks][o + 1]),
                          __builtin_amdgcn_rcpf(b[ks][o + 2]), __builtin_amdgcn_rcpf(b[ks][o + 3])};
            };
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                *reinterpret_cast<f4*>(d0 + chan_h(ks, 0)) = f4{b[ks][0], b[ks][1], b[ks][2], b[ks][3]};
                *reinterpret_cast<f4*>(d0 + chan_h(ks, 1)) = f4{b[ks][4], b[ks][5], b[ks][6], b[ks][7]};
                *reinterpret_cast<f4*>(d1 + chan_h(ks, 0)) = rcp4(ks, 0);
                *reinterpret_cast<f4*>(d1 + chan_h(ks, 1)) = rcp4(ks, 4);
            }
        }
        // (cleared here, once the loads above have landed: a store at the
        // kernel's start made the compiler wait for every load in flight)
        if (tid == 0) s_bad = 0;
        __syncthreads();
        // The direct form holds when, for every channel, the decay over the chunk
        // stays within 2^-64 (Gamma and 1/Gamma are fp32 factors) and, with
        // 16-bit operands, the decay over each 16-token block within 2^-14 and
        // |k|, |q| <= 2 (every operand below then stays within 2^15, inside fp16).
        // Otherwise the (chunk, head) joins the general-form list at the end
        // and the general kernel writes its whole record again (this
        // workgroup still runs to the end: its addressing does not depend on
        // the values, and an early exit here slowed every chunk down).
        {
            // branch-free (bitwise and / or); |k|, |q| are checked in derive
            int bad = 0;
            if (tid < DK) {
                const float* e = s_fac + 8 * DK + tid;      // 2^end_I, I = 0..3
                const float e0 = e[0], e1 = e[DK], e2 = e[2 * DK], e3 = e[3 * DK];
                bool ok = e3 >= 0x1p-64f;
                if constexpr (F16)
                    ok = ok & (e0 >= 0x1p-14f) & (e1 >= 0x1p-14f * e0) & (e2 >= 0x1p-14f * e1) & (e3 >= 0x1p-14f * e2);
                bad = !ok;
            }
            if (bad) atomicOr(&s_bad, 1);
        }
        float kqmax = 0.f;            // max |k|, |q| of this lane's elements (taken in derive)
        // gamma
        if (tid < DK) reinterpret_cast<float*>(rec + R::GAM)[tid] = s_fac[11 * DK + tid];

        // ---- (b) every decay-dependent quantity of this lane's elements -----------
        // A[r][s] and P[r][s] (s <= r) take 2^(b_r - b_s) = 2^(b_r - ref_I) 2^(ref_I - b_s)
        // for r in block I: the row operands (k, q) 2^(b - ref_I) are shared by
        // every column block; the column operand k_s 2^(ref_I - b_s) (<= 1 below
        // the diagonal block) is made by the wave that owns token s, for every
        // later block I, and handed over through LDS.
        // one copy per block index I (= the wave), so the tests of the later
        // blocks fold at compile time and the column operands of blocks that do
        // not exist take no registers (181 instead of 247)
        auto derive = [&](auto ic) {
            constexpr int I = decltype(ic)::value;
            E* __restrict__ qh = reinterpret_cast<E*>(rec + R::QH);
            auto fac4 = [&](int row, int ks, int half) {
                return *reinterpret_cast<const f4*>(s_fac + row * DK + chan_h(ks, half));
            };
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float qv[8], kh[8], kt[8], cl[3][8];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f4 kw = R4::widen(kraw[ks][half]);
                    const f4 qw = R4::widen(qraw[ks][half]);
                    const f4 ref = fac4(I, ks, half);          // 2^ref_I
                    const f4 rref = fac4(4 + I, ks, half);     // 2^-ref_I
                    const f4 gam = fac4(11, ks, half);         // gamma = 2^end_3
                    f4 refl[3];                                // 2^ref of the later blocks
#pragma unroll
                    for (int Il = 1; Il < 4; ++Il)
                        if (Il > I) refl[Il - 1] = fac4(Il, ks, half);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * half + i;
                        const float G = b[ks][e], rG = __builtin_amdgcn_rcpf(G);
                        const float kv = valid ? kw[i] : 0.f, qx = valid ? qw[i] : 0.f;
                        if constexpr (F16) kqmax = fmaxf(kqmax, fmaxf(__builtin_fabsf(kv), __builtin_fabsf(qx)));
                        const float e1 = G * rref[i];                      // 2^(b - ref_I)
                        ra[ks][e] = M::cvt(kv * e1);
                        rq[ks][e] = M::cvt(qx * e1);
                        Dc[ks][e] = M::cvt(kv * (rG * ref[i]));           // k 2^(ref_I - b)
#pragma unroll
                        for (int Il = 1; Il < 4; ++Il)
                            if (Il > I) cl[Il - 1][e] = kv * (rG * refl[Il - 1][i]);
                        kh[e] = kv * G;
                        qv[e] = qx * G;
                        kt[e] = kv * (rG * gam[i]);                        // k gamma / Gamma
                    }
                }
                M::gstore8(qh + frag_off(I * KS + ks, lane), qv, P.nt);
#pragma unroll
                for (int Il = 1; Il < 4; ++Il)
                    if (Il > I) M::store8(s_C + frag_off(pair_index(Il, I) * KS + ks, lane), cl[Il - 1]);
                const int c0 = chan_h(ks, 0), c1 = chan_h(ks, 1);
                M::store4(s_khat + r * KXP + c0, f4{kh[0], kh[1], kh[2], kh[3]});
                M::store4(s_khat + r * KXP + c1, f4{kh[4], kh[5], kh[6], kh[7]});
                M::store4(s_Kt + r * KXP + c0, f4{kt[0], kt[1], kt[2], kt[3]});
                M::store4(s_Kt + r * KXP + c1, f4{kt[4], kt[5], kt[6], kt[7]});
            }
            };
        switch (I) {
            case 0: derive(std::integral_constant<int, 0>{}); break;
            case 1: derive(std::integral_constant<int, 1>{}); break;
            case 2: derive(std::integral_constant<int, 2>{}); break;
            default: derive(std::integral_constant<int, 3>{}); break;
        }
        if constexpr (F16)
            if (!(kqmax <= 2.f)) atomicOr(&s_bad, 1);
    } else {
        // ---- (a) decay inside each 16-token block, as products of alpha -------------
        // No decay factor is ever formed above 1: every factor below is a product
        // of alpha over a run of tokens, in [0, 1], so no gate in [0, 1] can
        // overflow anything (strongly forgetting channels only underflow, towards
        // the exact limit 0).  This is the chunk-wise normalisation that keeps chunk
        // boundaries from overflowing ("Designing and Deploying Hybrid MLA and
        // Linear Attention Architectures", section 3), taken down to single tokens.
        // For this lane's token r and p = 0..4:
        //   pf_p(r) = product of alpha over r's aligned group of 2^p tokens, up to r
        //   sf_p(r) = product of alpha after r, to the end of that group.
        // From groups of 2^p to 2^(p+1) tokens, a token in the upper half takes the
        // lower half's total into pf, a token in the lower half the upper half's
        // total into sf; that total is pf_p of the other half's last token.
        constexpr bool SCAL = GATE == KDA_GATE_SCALAR;
        float pf[KS][8], sf[KS][8];
        auto PF = [&](int ks, int e) -> float& { return SCAL ? pf[0][0] : pf[ks][e]; };
        auto SF = [&](int ks, int e) -> float& { return SCAL ? sf[0][0] : sf[ks][e]; };
        if constexpr (SCAL) {
            pf[0][0] = valid ? gscalar : 1.f;
            sf[0][0] = 1.f;
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f4 av;
                    if constexpr (GATE == KDA_GATE_ALPHA) {
                        av = graw[ks][half];
                    } else {
                        const f4 xv = Raw4<true>::widen(graw[ks][half]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) av[i] = alpha_from_softplus_arg(xv[i]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[ks][4 * half + i] = valid ? av[i] : 1.f;
                        sf[ks][4 * half + i] = 1.f;
                    }
                }
        }
        if (lg == 0) s_beta[r] = bet;

        // Diagonal 16 x 16 blocks of A and P.  A pair of tokens s < r of this block
        // is taken at the level p of the highest bit in which r and s differ: both
        // lie in one aligned group of 2^(p+1) tokens, s in its lower half and r in
        // its upper half, and the decay between them factors exactly as
        //   prod_{t = s+1..r} alpha_t = pf_p(r) * sf_p(s),   both factors <= 1.
        // Level p is one matrix-core product of k (and q) scaled by pf_p on tokens
        // with bit p set and by sf_p on the others; only its own pairs are kept.
        // Lane (lm, lg) gathers A[16I + 4lg + i][16I + lm] in dA and
        // P[16I + lm][16I + 4lg + i] in dP (the layouts of the blocks below the
        // diagonal in (c)).
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const bool up = (lm >> p) & 1;
            f4 la = {0.f, 0.f, 0.f, 0.f}, lp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                V kc, qc;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f4 kw = R4::widen(kraw[ks][half]);
                    const f4 qw = R4::widen(qraw[ks][half]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * half + i;
                        const float f = up ? PF(ks, e) : SF(ks, e);
                        kc[e] = M::cvt((valid ? kw[i] : 0.f) * f);
                        qc[e] = M::cvt((valid ? qw[i] : 0.f) * f);
                    }
                }
                la = M::mma(kc, kc, la);      // rows r (A operand), columns s (B operand)
                lp = M::mma(kc, qc, lp);      // P^T: rows s, columns r
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra_ = 4 * lg + i;
                if (((ra_ ^ lm) >> p) == 1) {
                    if ((ra_ >> p) & 1) dA[i] = la[i];     // r = 4lg + i above s = lm
                    else dP[i] = lp[i];                    // r = lm above s = 4lg + i
                }
            }
            // pf_p, sf_p -> pf_{p+1}, sf_{p+1}
#pragma unroll
            for (int ks = 0; ks < (SCAL ? 1 : KS); ++ks)
#pragma unroll
                for (int e = 0; e < (SCAL ? 1 : 8); ++e) {
                    const float o = other_half_last(p, pf[ks][e], lane);
                    if (up) pf[ks][e] *= o;
                    else sf[ks][e] *= o;
                }
        }
        {   // the diagonal of P: q_r . k_r, no decay
            f4 pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                V kc, qc;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f4 kw = R4::widen(kraw[ks][half]);
                    const f4 qw = R4::widen(qraw[ks][half]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        kc[4 * half + i] = M::cvt(valid ? kw[i] : 0.f);
                        qc[4 * half + i] = M::cvt(valid ? qw[i] : 0.f);
                    }
                }
                pd = M::mma(kc, qc, pd);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i == lm) dP[i] = pd[i];
        }
        // block totals F_I (= pf_4 of the block's last token), [4][DK]
        if (lm == 15) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    *reinterpret_cast<f4*>(s_F + I * DK + chan_h(ks, half)) =
                        f4{PF(ks, 4 * half), PF(ks, 4 * half + 1), PF(ks, 4 * half + 2), PF(ks, 4 * half + 3)};
        }
        __syncthreads();
        // gamma = F_0 F_1 F_2 F_3
        if (tid < DK)
            reinterpret_cast<float*>(rec + R::GAM)[tid] =
                s_F[tid] * s_F[DK + tid] * s_F[2 * DK + tid] * s_F[3 * DK + tid];

        // ---- (b) every decay-dependent quantity of this lane's elements -----------
        // With E_I = F_0..F_{I-1} and X_I = F_{I+1}..F_3 (products, per channel):
        //   Gamma_r = E_I pf_4(r),  gamma / Gamma_r = sf_4(r) X_I.
        // Blocks below the diagonal (J < I) take 2^(b_r - b_s) as
        //   [pf_4(r)] * [sf_4(s) F_{J+1} .. F_{I-1}]
        // (split at the end of block I - 1): the row operands k pf_4, q pf_4 of
        // block I serve every J < I, and the column operand of block J for a later
        // block I is made by the wave that owns block J and handed over through LDS.
        // one copy per block index I (= the wave), so the tests of the later
        // blocks fold at compile time and the column operands of blocks that do
        // not exist take no registers
        auto derive = [&](auto ic) {
            constexpr int I = decltype(ic)::value;
            E* __restrict__ qh = reinterpret_cast<E*>(rec + R::QH);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float qv[8], kh[8], kt[8], cl[3][8];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f4 kw = R4::widen(kraw[ks][half]);
                    const f4 qw = R4::widen(qraw[ks][half]);
                    f4 Fb[4];
#pragma unroll
                    for (int K = 0; K < 4; ++K)
                        if (K != I) Fb[K] = *reinterpret_cast<const f4*>(s_F + K * DK + chan_h(ks, half));
                    f4 Eb = {1.f, 1.f, 1.f, 1.f}, Xb = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                    for (int K = 0; K < I; ++K) Eb = Eb * Fb[K];
#pragma unroll
                    for (int K = I + 1; K < 4; ++K) Xb = Xb * Fb[K];
                    f4 mid[3];                         // F_{I+1} .. F_{Il-1} for the later blocks Il
                    mid[0] = f4{1.f, 1.f, 1.f, 1.f};
                    if (I + 2 < 4) mid[1] = Fb[I + 1 < 4 ? I + 1 : 0];
                    if (I + 3 < 4) mid[2] = mid[1] * Fb[I + 2 < 4 ? I + 2 : 0];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * half + i;
                        const float kv = valid ? kw[i] : 0.f, qx = valid ? qw[i] : 0.f;
                        const float pfv = PF(ks, e), sfv = SF(ks, e);
                        const float G = Eb[i] * pfv;
                        ra[ks][e] = M::cvt(kv * pfv);
                        rq[ks][e] = M::cvt(qx * pfv);
#pragma unroll
                        for (int Il = 1; Il < 4; ++Il)
                            if (Il > I) cl[Il - 1][e] = kv * (sfv * mid[Il - I - 1][i]);
                        kh[e] = kv * G;
                        qv[e] = qx * G;
                        kt[e] = kv * (sfv * Xb[i]);
                    }
                }
                M::gstore8(qh + frag_off(I * KS + ks, lane), qv, P.nt);
#pragma unroll
                for (int Il = 1; Il < 4; ++Il)
                    if (Il > I) M::store8(s_C + frag_off(pair_index(Il, I) * KS + ks, lane), cl[Il - 1]);
                const int c0 = chan_h(ks, 0), c1 = chan_h(ks, 1);
                M::store4(s_khat + r * KXP + c0, f4{kh[0], kh[1], kh[2], kh[3]});
                M::store4(s_khat + r * KXP + c1, f4{kh[4], kh[5], kh[6], kh[7]});
                M::store4(s_Kt + r * KXP + c0, f4{kt[0], kt[1], kt[2], kt[3]});
                M::store4(s_Kt + r * KXP + c1, f4{kt[4], kt[5], kt[6], kt[7]});
            }
            };
        switch (I) {
            case 0: derive(std::integral_constant<int, 0>{}); break;
            case 1: derive(std::integral_constant<int, 1>{}); break;
            case 2: derive(std::integral_constant<int, 2>{}); break;
            default: derive(std::integral_constant<int, 3>{}); break;
        }
    }
    // v is first needed in (e); loading it here keeps it out of the
    // registers of the phases above
    uint4 vreg[NV];
#pragma unroll
    for (int jv = 0; jv < NV; ++jv) {
        const int id = tid + 256 * jv;
        const int rr = id / VROW16;
        const int cc = (id - rr * VROW16) * EL16;
        vreg[jv] = *reinterpret_cast<const uint4*>(v + row_v(min(rr, rl)) + cc);
    }
    __syncthreads();

    // ---- (c) A (as A^T) and P (as P^T tiles): blocks below the diagonal on
    // the matrix cores, diagonal blocks from (a) --------------------------------
    {
        E* __restrict__ pout = reinterpret_cast<E*>(rec + R::P);
        f4 accP[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            accP[J] = f4{0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
                f4 accA = {0.f, 0.f, 0.f, 0.f};
                if (FAST || J < I) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        V col;
                        if constexpr (FAST) col = J == I ? Dc[ks] : M::load8(s_C + frag_off(pair_index(I, J) * KS + ks, lane));
                        else col = M::load8(s_C + frag_off(pair_index(I, J) * KS + ks, lane));
                        accA = M::mma(ra[ks], col, accA);
                        accP[J] = M::mma(col, rq[ks], accP[J]);
                    }
                } else {
                    accA = dA;
                    accP[J] = dP;
                }
                // lane (lm, lg) holds A[16I + 4lg + i][16J + lm]; store A^T rows
                const int s = 16 * J + lm;
                f4 at;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * lg + i;
                    at[i] = s < rr ? s_beta[rr] * accA[i] : 0.f;
                }
                *reinterpret_cast<f4*>(s_AT + s * ATP + 16 * I + 4 * lg) = at;
            }
        }
        // lane (lm, lg) of P^T tile J holds P[16I+lm][16J+4lg+i]
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s0 = 32 * ks + 4 * lg + e, s1 = s0 + 16;
                pv[e] = s0 <= r ? accP[2 * ks][e] : 0.f;
                pv[4 + e] = s1 <= r ? accP[2 * ks + 1][e] : 0.f;
            }
            if (ks == 0 || I >= 2) M::gstore8(pout + frag_off(p_slot(2 * I + ks), lane), pv, P.nt);
        }
    }

    // ---- (d) ((gamma/Gamma).K)^T fragments from the staged K~ ------------------
    {
        E* __restrict__ ktt = reinterpret_cast<E*>(rec + R::KTT);
        for (int id = tid; id < DK * 2 * 4; id += 256) {
            const int jj = (id >> 4) & 3, f = id >> 6;
            const int ts = f & 1;
            // channel 16 (f >> 1) + lane % 16, tokens 32 ts + frag_k(jj, 0..7)
            M::gstoreV(ktt + frag_off(f, id & 63),
                       M::loadT(s_Kt, KXP, 32 * ts + 4 * jj, 32 * ts + 16 + 4 * jj, 16 * (f >> 1), lm), P.nt);
        }
    }
    __syncthreads();

    // ---- (e) v into LDS; T = (I + A)^-1 --------------------------------------
    {
#pragma unroll
        for (int jv = 0; jv < NV; ++jv) {
            const int id = tid + 256 * jv;
            const int rr = id / VROW16;
            const int cc = (id - rr * VROW16) * EL16;
            // V in the operand type, rows past the chunk's end as zeros
            const A* vv = reinterpret_cast<const A*>(&vreg[jv]);
            float x[EL16];
#pragma unroll
            for (int e = 0; e < EL16; ++e) {
                if constexpr (F16) x[e] = bf16_to_f32(vv[e]);
                else x[e] = vv[e];
                if (rr >= len) x[e] = 0.f;
            }
            if constexpr (F16) M::store8(s_v + rr * VXP + cc, x);
            else M::store4(s_v + rr * VXP + cc, f4{x[0], x[1], x[2], x[3]});
        }
        // diagonal 16x16 blocks, column-oriented forward substitution: once
        // x[s] is final, every later row takes its contribution
        if (lane < 16) {
            const int j = lane;
            // the block's strict lower triangle, every read issued before the
            // first use: a[rr(rr-1)/2 + s] = A[16I+rr][16I+s]
            float a[120];
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                const float* col = s_AT + (16 * I + s) * ATP + 16 * I;
#pragma unroll
                for (int rr = s + 1; rr < 16; ++rr) a[rr * (rr - 1) / 2 + s] = col[rr];
            }
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == j) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 15; ++s) {
#pragma unroll
                for (int rr = s + 1; rr < 16; ++rr) x[rr] -= a[rr * (rr - 1) / 2 + s] * x[s];
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) s_T[(16 * I + rr) * TP + 16 * I + j] = x[rr];
        }
        __syncthreads();
        // blocks below the diagonal: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
        for (int Ib = 1; Ib < 4; ++Ib) {
            if (wave < Ib) {
                const int J = wave;
                f4 X = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < Ib; ++K) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const float a = s_AT[(16 * K + 4 * kk + lg) * ATP + 16 * Ib + lm];
                        const float bv = s_T[(16 * K + 4 * kk + lg) * TP + 16 * J + lm];
                        X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, X, 0, 0, 0);
                    }
                }
                f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = -s_T[(16 * Ib + lm) * TP + 16 * Ib + 4 * lg + i];
                    Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, X[i], Y, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) s_T[(16 * Ib + 4 * lg + i) * TP + 16 * J + lm] = Y[i];
            }
            __syncthreads();
        }
        // T Diag(beta), zero above the diagonal, in the operand type
        for (int id = tid; id < C * C / 4; id += 256) {
            const int rr = id / (C / 4);
            const int s0 = 4 * (id - rr * (C / 4));
            const f4 t = *reinterpret_cast<const f4*>(s_T + rr * TP + s0);
            const f4 bt = *reinterpret_cast<const f4*>(s_beta + s0);
            f4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = s0 + i <= rr ? t[i] * bt[i] : 0.f;
            M::store4(s_Tp + rr * TPP + s0, x);
        }
        __syncthreads();
    }

    // ---- (f) W = T Diag(beta) K-hat and U = T Diag(beta) V ------------------
    {
        E* __restrict__ wout = reinterpret_cast<E*>(rec + R::W);
        E* __restrict__ uout = reinterpret_cast<E*>(rec + R::UT);
        // W^T tiles (channels x tokens): the pair of channel tiles of one
        // channel step gives a W fragment lane by lane.
        for (int item = wave; item < KS * 4; item += 4) {
            const int ksc = item >> 2;              // channel step
            const int Ib = item & 3;                // token tile
            f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            const int kmax = (16 * Ib + 16 + 31) / 32;
            for (int kt = 0; kt < kmax; ++kt) {
                const int t = 32 * kt + 8 * lg;
                const V bT = M::load8(s_Tp + (16 * Ib + lm) * TPP + t);
                const V a0 = M::loadT(s_khat, KXP, t, t + 4, 32 * ksc, lm);
                const V a1 = M::loadT(s_khat, KXP, t, t + 4, 32 * ksc + 16, lm);
                acc0 = M::mma(a0, bT, acc0);
                acc1 = M::mma(a1, bT, acc1);
            }
            const float wv[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
            M::gstore8(wout + frag_off(Ib * KS + ksc, lane), wv, P.nt);
        }
        // U in the accumulator layout the state kernel consumes directly
        for (int nt = wave; nt < DV / 16; nt += 4) {
#pragma unroll
            for (int Ib = 0; Ib < 4; ++Ib) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                const int kmax = (16 * Ib + 16 + 31) / 32;
                for (int ks = 0; ks < kmax; ++ks) {
                    const int t = 32 * ks + 8 * lg;
                    const V a = M::load8(s_Tp + (16 * Ib + lm) * TPP + t);
                    const V bv = M::loadT(s_v, VXP, t, t + 4, 16 * nt, lm);
                    acc = M::mma(a, bv, acc);
                }
                M::gstore4(uout + (static_cast<size_t>(nt * 4 + Ib) * 64 + lane) * 4, acc, P.nt);
            }
        }
    }
    if constexpr (FAST) {
        // s_bad was last written before the barrier that precedes (c)
        if (tid == 0 && s_bad) P.slow[atomicAdd(P.nslow, 1)] = blk;
    }
}

// One workgroup per (chunk, head): the direct form, or the (chunk, head)'s
// entry in the general-form list.
template <int DK, int DV, bool F16, int GATE>
__global__ __launch_bounds__(256, 2) void prep_kernel(const PrepParams P) {
    prep_body<DK, DV, F16, GATE, true>(P, blockIdx.x);
}

// Entry blockIdx.x of the general-form list, if the list is that long (one
// workgroup per (chunk, head), the list's largest length; those past its end
// return at once).
template <int DK, int DV, bool F16, int GATE>
__global__ __launch_bounds__(256, 2) void prep_general_kernel(const PrepParams P) {
    if (static_cast<int>(blockIdx.x) >= *P.nslow) return;
    prep_body<DK, DV, F16, GATE, false>(P, P.slow[blockIdx.x]);
}

// ---------------------------------------------------------------------------
// state_kernel (fp32 records; fp16 records take state_split_kernel below):
// the sequential pass over the chunks of one sequence for one
// head and 16*TW value columns.  Wave w keeps state rows [w*DK/4, (w+1)*DK/4)
// of those columns in fp32 registers; an operand-type copy of the state
// slice lives in LDS for the next chunk's products.  Every operand fragment a
// wave loads (W, Gamma.Q, P, ((gamma/Gamma).K)^T) serves all TW column tiles,
// whose chains are independent and interleave on the matrix cores.  The
// operands of the next kDepth-1 chunks are in flight in a register ring.
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

template <int DK, bool F16, int TW>
struct StateStage {
    using V = typename Mx<F16>::V;
    static constexpr int KS = DK / 32;
    static constexpr int TPW = DK / 64;
    V w[KS], q[KS];          // rows 16w..16w+15 of W and Gamma.Q
    V p[2];                  // row 16w+lm of P, tokens 0..63
    V k[TPW][2];             // rows of ((gamma/Gamma).K)^T owned by this wave
    typename Mx<F16>::V4 u[TW];   // U: tokens 16w+4lg..+3, one column per tile
    float gm;                // gamma of owned state row (lane mod DK/4); lanes trade them at use
};

// Four compute waves, plus one wave that prefetches records into L2 where
// the register budget of two waves per SIMD allows it (the fp32 d_k = 128
// variant needs more than 256 registers per wave).
template <int DK, bool F16> struct StateThreads { static constexpr int value = (F16 || DK == 64) ? 320 : 256; };
constexpr int kStatePrefetch = 2;       // chunks ahead that the prefetch wave touches
constexpr int kPrefetchShift = 7;       // log2 of the bytes per touched word (one per 128-B line)
constexpr int kStateDepth = 2;          // chunks of operands in the register ring
constexpr int kStateTiles = 1;          // value-column tiles (16 columns each) per workgroup

template <int DK, int DV, bool F16, bool OBF16>
__global__ __launch_bounds__((StateThreads<DK, F16>::value)) void state_kernel(const StateParams P) {
    using M = Mx<F16>;
    using E = typename M::E;
    using V = typename M::V;
    constexpr int TW = kStateTiles;
    using Stage = StateStage<DK, F16, TW>;
    using R = Rec<DK, DV, F16>;
    constexpr int D = kStateDepth;          // chunks in flight
    constexpr int NTV = DV / (16 * TW);   // workgroups per (sequence, head)
    constexpr int RPW = DK / 4;           // state rows per wave
    constexpr int TPW = RPW / 16;         // 16-row tiles per wave
    constexpr int KS = DK / 32;
    constexpr int SP = DK + 8;            // LDS row stride of the state operand
    constexpr int UP = C + 8;             // LDS row stride of U'
    static_assert(NTV >= 1 && NTV * 16 * TW == DV, "value tiling");
    static_assert((RPW & (RPW - 1)) == 0 && RPW <= 64, "a wave's gamma rows fit one word per lane");

    // Workgroups are handed to the 8 XCDs round-robin; keep the NTV
    // workgroups of one (sequence, head) on the same XCD so they share its L2.
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

    __shared__ __align__(16) E s_S[16 * TW * SP];   // [value column][key row]
    __shared__ __align__(16) E s_U[16 * TW * UP];   // [value column][token]
    __shared__ __align__(16) int s_pf[64];           // sink of the prefetch loads

    const size_t sbase = (static_cast<size_t>(n) * H + h) * (DK * DV);
    const bool pf_wave = StateThreads<DK, F16>::value > 256 && wave == 4;
    f4 S[TW][TPW];
#pragma unroll
    for (int c = 0; c < TW && !pf_wave; ++c) {
        const int col = 16 * (jt * TW + c) + lm;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = RPW * wave + 16 * t + 4 * lg + i;
                S[c][t][i] = P.initial_state ? P.initial_state[sbase + row * DV + col] : 0.f;
            }
            M::store4(s_S + (16 * c + lm) * SP + RPW * wave + 16 * t + 4 * lg, S[c][t]);
        }
    }

    // The chunks of a sequence are consecutive runs of C tokens from its
    // first row: the first and last table entries give every chunk's rows.
    int seq_t0 = 0, seq_end = 0;
    if (g0 < g1) {
        const int4 e0 = P.table[g0];
        const int4 e1 = P.table[g1 - 1];
        seq_t0 = e0.y;
        seq_end = e1.y + e1.z;
    }
    const unsigned char* recs = P.rec + static_cast<size_t>(h) * P.rec_bytes;
    const size_t gstride = static_cast<size_t>(H) * P.rec_bytes;
    // output rows of this lane: tokens 16w + 4lg + i of the chunk
    const size_t ostride = static_cast<size_t>(H) * DV;                 // elements per token row
    const size_t ocol = static_cast<size_t>(h) * DV + 16 * jt * TW + lm;

    // The next stage's loads are split into four groups issued between the
    // phases of the current chunk: a CU's vector-memory address path moves
    // about 64 B per clock, so issuing a whole stage at once would stall the
    // wave for ~1000 clocks while the matrix cores idle.  sched_barrier keeps
    // the compiler from regrouping them.
    // P2: the wave's rows reach tokens 32..63 of P (waves 2 and 3; the
    // second P fragment of waves 0 and 1 lies above the diagonal)
    auto load_part = [&](auto p2c, Stage& st, int g, int part) {
        constexpr bool P2 = decltype(p2c)::value;
        const unsigned char* rec = recs + static_cast<size_t>(g) * gstride;
        if (part == 0) {
            // W and U head the chain of the next chunk; gamma and the chunk's
            // table entry ride along
            const E* wr = reinterpret_cast<const E*>(rec + R::W);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.w[ks] = M::load8(wr + frag_off(wave * KS + ks, lane));
            const E* ut = reinterpret_cast<const E*>(rec + R::UT);
#pragma unroll
            for (int c = 0; c < TW; ++c)
                st.u[c] = M::load4(ut + (static_cast<size_t>((jt * TW + c) * 4 + wave) * 64 + lane) * 4);
            // one word per lane: the address path is paid per byte each lane
            // asks for, repeats included, and two 16-byte loads per lane of
            // the rows in the MFMA layout would ask 2 KiB for 128 bytes
            const float* gam = reinterpret_cast<const float*>(rec + R::GAM);
            st.gm = gam[RPW * wave + (lane & (RPW - 1))];
        } else if (part == 1) {
            const E* qr = reinterpret_cast<const E*>(rec + R::QH);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.q[ks] = M::load8(qr + frag_off(wave * KS + ks, lane));
        } else if (part == 2) {
            const E* kt = reinterpret_cast<const E*>(rec + R::KTT);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                st.k[t][0] = M::load8(kt + frag_off((TPW * wave + t) * 2, lane));
                st.k[t][1] = M::load8(kt + frag_off((TPW * wave + t) * 2 + 1, lane));
            }
        } else {
            const E* pr = reinterpret_cast<const E*>(rec + R::P);
            st.p[0] = M::load8(pr + frag_off(p_slot(2 * wave), lane));
            if constexpr (P2) st.p[1] = M::load8(pr + frag_off(p_slot(2 * wave + 1), lane));
        }
    };
    auto load = [&](auto p2c, Stage& st, int g) {
#pragma unroll
        for (int part = 0; part < 4; ++part) load_part(p2c, st, g, part);
    };

    // one chunk of the chain; `nx` / `gn` receive the loads of a later chunk
    auto compute = [&](auto p2c, const Stage& st, Stage& nx, int gn, int gc) {
        constexpr bool P2 = decltype(p2c)::value;
        // (1) X = W S and O = (Gamma.Q) S for tokens 16w..16w+15, every tile
        f4 X[TW], O[TW];
#pragma unroll
        for (int c = 0; c < TW; ++c) {
            X[c] = f4{0.f, 0.f, 0.f, 0.f};
            O[c] = f4{0.f, 0.f, 0.f, 0.f};
        }
        V bS[TW][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int c = 0; c < TW; ++c) {
                const E* sb = s_S + (16 * c + lm) * SP + 32 * ks + 4 * lg;
                bS[c][ks] = M::load4x2(sb, sb + 16);
            }
        __builtin_amdgcn_sched_barrier(0);
        load_part(p2c, nx, gn, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int c = 0; c < TW; ++c) {
                X[c] = M::mma(st.w[ks], bS[c][ks], X[c]);
                O[c] = M::mma(st.q[ks], bS[c][ks], O[c]);
            }
        // gamma of state rows 16t + 4lg + i from the lanes that loaded them
        // (needed in (4); the exchange rides under the barrier below)
        f4 gmv[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                gmv[t][i] = __int_as_float(__builtin_amdgcn_ds_bpermute((16 * t + 4 * lg + i) << 2, __float_as_int(st.gm)));
        __builtin_amdgcn_sched_barrier(0);
        load_part(p2c, nx, gn, 1);
        __builtin_amdgcn_sched_barrier(0);
        // (2) U' = U - W S, shared through LDS
#pragma unroll
        for (int c = 0; c < TW; ++c) M::store4(s_U + (16 * c + lm) * UP + 16 * wave + 4 * lg, M::tof4(st.u[c]) - X[c]);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        load_part(p2c, nx, gn, 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < TW; ++c) {
            const E* ub = s_U + (16 * c + lm) * UP + 4 * lg;
            const V bU0 = M::load4x2(ub, ub + 16);
            const V bU1 = M::load4x2(ub + 32, ub + 48);
            // (3) O += Tril(...) U'  (tokens above this wave's rows are zero in P)
            O[c] = M::mma(st.p[0], bU0, O[c]);
            if constexpr (P2) O[c] = M::mma(st.p[1], bU1, O[c]);
            // (4) S <- Diag(gamma) S + ((gamma/Gamma).K)^T U'
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = M::mma(st.k[t][0], bU0, acc);
                acc = M::mma(st.k[t][1], bU1, acc);
                S[c][t] = gmv[t] * S[c][t] + acc;
                M::store4(s_S + (16 * c + lm) * SP + RPW * wave + 16 * t + 4 * lg, S[c][t]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_part(p2c, nx, gn, 3);
        __builtin_amdgcn_sched_barrier(0);
        // outputs: full chunks take the branch-free path
        const int t0 = seq_t0 + C * (gc - g0);
        const int len = min(C, seq_end - t0);
        const size_t obase = (static_cast<size_t>(t0) + 16 * wave + 4 * lg) * ostride + ocol;
        if (len == C) {
#pragma unroll
            for (int c = 0; c < TW; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) store_out<OBF16>(P.o, obase + i * ostride + 16 * c, O[c][i]);
        } else {
#pragma unroll
            for (int c = 0; c < TW; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * wave + 4 * lg + i < len) store_out<OBF16>(P.o, obase + i * ostride + 16 * c, O[c][i]);
        }
        __syncthreads();
    };

    __syncthreads();
    if (pf_wave) {
        // Load one word of every 128-byte line of the record kStatePrefetch
        // chunks ahead (this workgroup takes every NTV-th line, so the NTV
        // workgroups of the pair cover the record once) to bring it into the
        // XCD's L2.  The words go straight to a scratch area of LDS and are
        // never waited on; they count on this wave's counters only.  The wave
        // passes the same barriers as the compute waves, two per chunk.
        const int nlines = static_cast<int>(P.rec_bytes >> kPrefetchShift);
        auto prefetch = [&](int gp) {
            const unsigned char* rec = recs + static_cast<size_t>(gp) * gstride;
            for (int line = jt + NTV * lane; line < nlines; line += NTV * 64)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(rec + (static_cast<size_t>(line) << kPrefetchShift)),
                    (__attribute__((address_space(3))) void*)s_pf, 4, 0, 0);
        };
        for (int gp = g0 + 1; gp < min(g0 + kStatePrefetch, g1); ++gp) prefetch(gp);
        // Bare barriers: a fence here would wait for the prefetches to land.
        for (int g = g0; g < g1; ++g) {
            if (g + kStatePrefetch < g1) prefetch(g + kStatePrefetch);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
        }
        // let the last loads land before the wave ends
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        return;
    }
    // Ring loads are unconditional (clamped to the last chunk; the surplus
    // loads at the tail are never used) and each wave role runs its own copy
    // of the loop, so the loop body is straight-line code and the hardware
    // wait counters never have to drain the ring.
    auto run = [&](auto p2c) {
        Stage st[D];
        if (g0 < g1) {
#pragma unroll
            for (int j = 0; j < D - 1; ++j) load(p2c, st[j], min(g0 + j, g1 - 1));
        }
        for (int g = g0; g < g1; g += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (g + j < g1) compute(p2c, st[j], st[(j + D - 1) % D], min(g + j + D - 1, g1 - 1), g + j);
            }
        }
    };
    if (wave >= 2) run(std::true_type{});
    else run(std::false_type{});

    if (P.final_state) {
#pragma unroll
        for (int c = 0; c < TW; ++c) {
            const int col = 16 * (jt * TW + c) + lm;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = RPW * wave + 16 * t + 4 * lg + i;
                    P.final_state[sbase + row * DV + col] = S[c][t][i];
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// state_split_kernel (fp16 records): the same sequential pass with the chain
// and the outputs on separate waves, two per SIMD.  Waves 0-3 carry the chain
// of each chunk (X = W S, U' = U - X, S <- Diag(gamma) S + K~^T U'), waves 4-7
// compute the outputs (O = (Gamma.Q) S + P U') beside them: their products
// and stores fill the matrix cores and the memory path while the chain waits
// on LDS and barriers.  With PF, wave 8 touches the records two chunks ahead
// into L2; records small enough to stay in the caches between the two passes
// (as for the non-temporal stores, up to 128 MB) need no prefetch, and
// without that wave two workgroups fit on a CU (B2 H8 T4096: 0.090 vs
// 0.092 ms; the 64K-token forward: 2.32 vs 2.11 ms the other way round).
// Per chunk, two barriers: after U' is in LDS, and after the new state is.
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 576;

template <int DK>
struct ChainStage {
    static constexpr int KS = DK / 32;
    static constexpr int TPW = DK / 64;
    h8 w[KS];        // rows 16c..16c+15 of W
    h8 k[TPW][2];    // rows of ((gamma/Gamma).K)^T owned by this wave
    h4 u;            // U: tokens 16c+4lg..+3 of this lane's column
    float gm;        // gamma of owned state row (lane mod DK/4)
};

template <int DK>
struct OutStage {
    static constexpr int KS = DK / 32;
    h8 q[KS];        // rows 16o..16o+15 of Gamma.Q
    h8 p[2];         // row 16o+lm of P, tokens 0..63
};

template <int DK, int DV, bool OBF16, bool PF>
__global__ __launch_bounds__(PF ? kSplitThreads : kSplitThreads - 64, PF ? 1 : 2) void state_split_kernel(const StateParams P) {
    using M = Mx<true>;
    using E = _Float16;
    using R = Rec<DK, DV, true>;
    constexpr int D = kStateDepth;
    constexpr int NTV = DV / 16;          // workgroups per (sequence, head)
    constexpr int RPW = DK / 4;           // state rows per chain wave
    constexpr int TPW = RPW / 16;
    constexpr int KS = DK / 32;
    constexpr int SP = DK + 8;            // LDS row stride of the state operand
    constexpr int UP = C + 8;             // LDS row stride of U'
    static_assert(NTV * 16 == DV, "value tiling");
    static_assert((RPW & (RPW - 1)) == 0 && RPW <= 64, "a wave's gamma rows fit one word per lane");

    // the NTV workgroups of one (sequence, head) on the same XCD
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // roles branch per wave
    const int lm = lane & 15;
    const int lg = lane >> 4;

    __shared__ __align__(16) E s_S[16 * SP];   // [value column][key row]
    __shared__ __align__(16) E s_U[16 * UP];   // [value column][token]
    __shared__ __align__(16) int s_pf[64];      // sink of the prefetch loads

    const size_t sbase = (static_cast<size_t>(n) * H + h) * (DK * DV);
    const int col = 16 * jt + lm;
    f4 S[TPW];
    if (wave < 4) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = RPW * wave + 16 * t + 4 * lg + i;
                S[t][i] = P.initial_state ? P.initial_state[sbase + row * DV + col] : 0.f;
            }
            M::store4(s_S + lm * SP + RPW * wave + 16 * t + 4 * lg, S[t]);
        }
    }

    int seq_t0 = 0, seq_end = 0;
    if (g0 < g1) {
        const int4 e0 = P.table[g0];
        const int4 e1 = P.table[g1 - 1];
        seq_t0 = e0.y;
        seq_end = e1.y + e1.z;
    }
    const unsigned char* recs = P.rec + static_cast<size_t>(h) * P.rec_bytes;
    const size_t gstride = static_cast<size_t>(H) * P.rec_bytes;
    __syncthreads();

    if (PF && wave == 8) {
        // one word of every 128-byte line, kStatePrefetch chunks ahead; this
        // workgroup takes every NTV-th line.  Never waited on; the barriers
        // carry no fence (a fence would wait for these loads to land).
        const int nlines = static_cast<int>(P.rec_bytes >> kPrefetchShift);
        auto prefetch = [&](int gp) {
            const unsigned char* rec = recs + static_cast<size_t>(gp) * gstride;
            for (int line = jt + NTV * lane; line < nlines; line += NTV * 64)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(rec + (static_cast<size_t>(line) << kPrefetchShift)),
                    (__attribute__((address_space(3))) void*)s_pf, 4, 0, 0);
        };
        for (int gp = g0 + 1; gp < min(g0 + kStatePrefetch, g1); ++gp) prefetch(gp);
        for (int g = g0; g < g1; ++g) {
            if (g + kStatePrefetch < g1) prefetch(g + kStatePrefetch);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        return;
    }

    if (wave < 4) {
        // ---- chain waves: c = wave owns tokens 16c..16c+15 of X and state rows RPW*c.. ----
        const int c = wave;
        using St = ChainStage<DK>;
        // the chain goes first on a SIMD it shares with an output wave
        __builtin_amdgcn_s_setprio(2);
        auto load_a = [&](St& st, int g) {
            const unsigned char* rec = recs + static_cast<size_t>(g) * gstride;
            const E* wr = reinterpret_cast<const E*>(rec + R::W);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.w[ks] = M::load8(wr + frag_off(c * KS + ks, lane));
            const E* ut = reinterpret_cast<const E*>(rec + R::UT);
            st.u = M::load4(ut + (static_cast<size_t>(jt * 4 + c) * 64 + lane) * 4);
            const float* gam = reinterpret_cast<const float*>(rec + R::GAM);
            st.gm = gam[RPW * c + (lane & (RPW - 1))];
        };
        auto load_b = [&](St& st, int g) {
            const unsigned char* rec = recs + static_cast<size_t>(g) * gstride;
            const E* kt = reinterpret_cast<const E*>(rec + R::KTT);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                st.k[t][0] = M::load8(kt + frag_off((TPW * c + t) * 2, lane));
                st.k[t][1] = M::load8(kt + frag_off((TPW * c + t) * 2 + 1, lane));
            }
        };
        auto step = [&](const St& st, St& nx, int gn) {
            h8 bS[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const E* sb = s_S + lm * SP + 32 * ks + 4 * lg;
                bS[ks] = M::load4x2(sb, sb + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
            load_a(nx, gn);
            __builtin_amdgcn_sched_barrier(0);
            f4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) X = M::mma(st.w[ks], bS[ks], X);
            M::store4(s_U + lm * UP + 16 * c + 4 * lg, M::tof4(st.u) - X);
            // gamma of state rows 16t + 4lg + i from the lanes that loaded them
            f4 gmv[TPW];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    gmv[t][i] = __int_as_float(__builtin_amdgcn_ds_bpermute((16 * t + 4 * lg + i) << 2, __float_as_int(st.gm)));
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            load_b(nx, gn);
            __builtin_amdgcn_sched_barrier(0);
            const E* ub = s_U + lm * UP + 4 * lg;
            const h8 bU0 = M::load4x2(ub, ub + 16);
            const h8 bU1 = M::load4x2(ub + 32, ub + 48);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = M::mma(st.k[t][0], bU0, acc);
                acc = M::mma(st.k[t][1], bU1, acc);
                S[t] = gmv[t] * S[t] + acc;
                M::store4(s_S + lm * SP + RPW * c + 16 * t + 4 * lg, S[t]);
            }
            __syncthreads();
        };
        St st[D];
        if (g0 < g1) {
#pragma unroll
            for (int j = 0; j < D - 1; ++j) {
                load_a(st[j], min(g0 + j, g1 - 1));
                load_b(st[j], min(g0 + j, g1 - 1));
            }
        }
        for (int g = g0; g < g1; g += D) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                if (g + j < g1) step(st[j], st[(j + D - 1) % D], min(g + j + D - 1, g1 - 1));
        }
        if (P.final_state) {
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = RPW * c + 16 * t + 4 * lg + i;
                    P.final_state[sbase + row * DV + col] = S[t][i];
                }
        }
        return;
    }

    // ---- output waves: o = wave - 4 owns tokens 16o..16o+15 ----
    const int o = wave - 4;
    using Os = OutStage<DK>;
    const size_t ostride = static_cast<size_t>(H) * DV;
    const size_t ocol = static_cast<size_t>(h) * DV + col;
    // P2: rows of wave o reach tokens 32..63 of P (o >= 2)
    auto run = [&](auto p2c) {
        constexpr bool P2 = decltype(p2c)::value;
        auto load_a = [&](Os& st, int g) {
            const E* qr = reinterpret_cast<const E*>(recs + static_cast<size_t>(g) * gstride + R::QH);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.q[ks] = M::load8(qr + frag_off(o * KS + ks, lane));
        };
        auto load_b = [&](Os& st, int g) {
            const E* pr = reinterpret_cast<const E*>(recs + static_cast<size_t>(g) * gstride + R::P);
            st.p[0] = M::load8(pr + frag_off(p_slot(2 * o), lane));
            if constexpr (P2) st.p[1] = M::load8(pr + frag_off(p_slot(2 * o + 1), lane));
        };
        auto step = [&](const Os& st, Os& nx, int gn, int gc) {
            // Gamma.Q comes in the preparation pass's channel order (eight
            // consecutive channels per lane group), W in two runs of four
            h8 bS[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) bS[ks] = M::load8(s_S + lm * SP + 32 * ks + 8 * lg);
            __builtin_amdgcn_sched_barrier(0);
            load_a(nx, gn);
            __builtin_amdgcn_sched_barrier(0);
            f4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) O = M::mma(st.q[ks], bS[ks], O);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            load_b(nx, gn);
            __builtin_amdgcn_sched_barrier(0);
            const E* ub = s_U + lm * UP + 4 * lg;
            const h8 bU0 = M::load4x2(ub, ub + 16);
            O = M::mma(st.p[0], bU0, O);
            if constexpr (P2) {
                const h8 bU1 = M::load4x2(ub + 32, ub + 48);
                O = M::mma(st.p[1], bU1, O);
            }
            const int t0 = seq_t0 + C * (gc - g0);
            const int len = min(C, seq_end - t0);
            const size_t obase = (static_cast<size_t>(t0) + 16 * o + 4 * lg) * ostride + ocol;
            if (len == C) {
#pragma unroll
                for (int i = 0; i < 4; ++i) store_out<OBF16>(P.o, obase + i * ostride, O[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * o + 4 * lg + i < len) store_out<OBF16>(P.o, obase + i * ostride, O[i]);
            }
            __syncthreads();
        };
        Os st[D];
        if (g0 < g1) {
#pragma unroll
            for (int j = 0; j < D - 1; ++j) {
                load_a(st[j], min(g0 + j, g1 - 1));
                load_b(st[j], min(g0 + j, g1 - 1));
            }
        }
        for (int g = g0; g < g1; g += D) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                if (g + j < g1) step(st[j], st[(j + D - 1) % D], min(g + j + D - 1, g1 - 1), g + j);
        }
    };
    if (o >= 2) run(std::true_type{});
    else run(std::false_type{});
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <int DK, int DV, bool F16, bool OBF16>
hipError_t launch_typed(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* ctrl = reinterpret_cast<int32_t*>(ws + pl.off_ctrl);
    int32_t* first = reinterpret_cast<int32_t*>(ws + pl.off_first);
    int32_t* order = reinterpret_cast<int32_t*>(ws + pl.off_order);
    int4* table = reinterpret_cast<int4*>(ws + pl.off_table);

    if (Rec<DK, DV, F16>::END > pl.rec_bytes) return hipErrorInvalidValue;
    hipError_t e = launch_chunk_plan(pl, a.cu_seqlens, a.workspace, stream);
    if (e != hipSuccess) return e;
    // records that stay in the caches until the state pass reads them: stored
    // normally and read without a prefetch wave
    const bool records_cached = static_cast<size_t>(pl.gmax) * pl.H * pl.rec_bytes <= (size_t(128) << 20);

    if (pl.gmax > 0) {
        PrepParams pp;
        pp.q = a.q; pp.k = a.k; pp.v = a.v; pp.gate = a.gate; pp.beta = a.beta;
        pp.ctrl = ctrl; pp.table = table;
        pp.rec = ws + pl.off_rec; pp.rec_bytes = pl.rec_bytes; pp.gmax = pl.gmax;
        pp.H = pl.H;
        pp.T = pl.varlen ? 0 : pl.T;
        pp.cps = static_cast<int>((pl.T + C - 1) / C);
        pp.nslow = ctrl + 1;
        pp.slow = reinterpret_cast<int32_t*>(ws + pl.off_slow);
        // records beyond about half the 256 MB memory-side cache are gone from
        // the caches before the state pass reads them
        pp.nt = !records_cached;
        constexpr int lds = PrepLds<DK, DV, F16>::bytes;
        auto kfn = a.gate_kind == KDA_GATE_SOFTPLUS_BF16 ? prep_kernel<DK, DV, F16, KDA_GATE_SOFTPLUS_BF16>
                 : a.gate_kind == KDA_GATE_SCALAR        ? prep_kernel<DK, DV, F16, KDA_GATE_SCALAR>
                                                         : prep_kernel<DK, DV, F16, KDA_GATE_ALPHA>;
        auto kgen = a.gate_kind == KDA_GATE_SOFTPLUS_BF16 ? prep_general_kernel<DK, DV, F16, KDA_GATE_SOFTPLUS_BF16>
                  : a.gate_kind == KDA_GATE_SCALAR        ? prep_general_kernel<DK, DV, F16, KDA_GATE_SCALAR>
                                                          : prep_general_kernel<DK, DV, F16, KDA_GATE_ALPHA>;
        const dim3 grid(static_cast<unsigned>(pl.gmax * pl.H));
        for (auto fn : {kfn, kgen}) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(fn, grid, dim3(256), lds, stream, pp);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
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
    const int64_t blocks = (pairs + 7) / 8 * 8 * (DV / (16 * kStateTiles));
    if constexpr (F16) {
        if (records_cached)
            hipLaunchKernelGGL((state_split_kernel<DK, DV, OBF16, false>), dim3(static_cast<unsigned>(blocks)),
                               dim3(kSplitThreads - 64), 0, stream, sp);
        else
            hipLaunchKernelGGL((state_split_kernel<DK, DV, OBF16, true>), dim3(static_cast<unsigned>(blocks)),
                               dim3(kSplitThreads), 0, stream, sp);
    }
    else
        hipLaunchKernelGGL((state_kernel<DK, DV, F16, OBF16>), dim3(static_cast<unsigned>(blocks)),
                           dim3(StateThreads<DK, F16>::value), 0, stream, sp);
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
    if ((Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128) ||
        (chunk_size != 32 && chunk_size != 64 && chunk_size != 128))
        return KDA_ERROR_NOT_SUPPORTED;
    if (varlen && B != 1) return KDA_ERROR_INVALID_VALUE;
    ChunkPlan p;
    p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.varlen = varlen; p.f16 = act_bf16;
    p.N = varlen ? num_seqs : B;
    const int64_t tokens = static_cast<int64_t>(B) * T;
    if (tokens >= (static_cast<int64_t>(1) << 31)) return KDA_ERROR_NOT_SUPPORTED;
    p.C = chunk_size;
    const int64_t per_seq_chunks = (T + chunk_size - 1) / chunk_size;
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
    p.off_slow = off;  off = align256(off + 4 * gh);    // general-form list of the preparation kernels
    // per (head, chunk) record: qh, w, ktt, p (its six lower fragments), ut
    // (operand type), gam (fp32)
    if (chunk_size == C)
        p.rec_bytes = align256(3 * static_cast<size_t>(C) * Dk * p.eb + static_cast<size_t>(kPFrags) * 512 * p.eb +
                               static_cast<size_t>(C) * Dv * p.eb + static_cast<size_t>(Dk) * 4);
    else
        p.rec_bytes = align256(generic_record_bytes(Dk, Dv, chunk_size, p.eb == 2));
    p.off_rec = off;   off = align256(off + gh * p.rec_bytes);
    p.workspace_bytes = off;
    *plan = p;
    return KDA_SUCCESS;
}

hipError_t launch_chunk_plan(const ChunkPlan& pl, const int32_t* cu_seqlens, void* workspace,
                             hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu_seqlens, pl.N,
                       pl.varlen ? static_cast<int64_t>(0) : pl.T, pl.gmax, pl.C,
                       reinterpret_cast<int32_t*>(ws + pl.off_ctrl),
                       reinterpret_cast<int32_t*>(ws + pl.off_first),
                       reinterpret_cast<int32_t*>(ws + pl.off_order),
                       reinterpret_cast<int4*>(ws + pl.off_table));
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkPlan& pl, const ChunkArgs& a, hipStream_t stream) {
    if (pl.C != C) return launch_chunk_fwd_generic(pl, a, stream);
    if (pl.Dk == 128 && pl.Dv == 128) return launch_dims<128, 128>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 64) return launch_dims<64, 64>(pl, a, stream);
    if (pl.Dk == 128 && pl.Dv == 64) return launch_dims<128, 64>(pl, a, stream);
    if (pl.Dk == 64 && pl.Dv == 128) return launch_dims<64, 128>(pl, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
