// Matrix-core building blocks shared by the chunkwise backward and the
// chunk-size-generic forward (gfx950): 16x16 fp32 MFMA tiles over LDS
// operands with arbitrary strides, the same products on the bf16 matrix
// cores with fp32 operands split into bf16 hi + lo, register-staged
// global -> LDS copies, DPP row sums, the XCD-aware chain grid, fp16 MFMA
// fragments and L2 prefetch touches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_chunk.h"
#include "kda_common.h"

namespace kda {
namespace mm32 {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int L16 = 16;            // LDS row stride of 16-column tiles

template <int D> struct Ld { static constexpr int value = D + 4; };   // LDS row stride, D columns

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------------------
// 16x16 fp32 matrix-core tile, 4-deep steps (v_mfma_f32_16x16x4f32):
//   A lane l holds A[l % 16][k], B lane l holds B[k][l % 16] for the step's
//   k, D lane l holds D[4 (l / 16) + e][l % 16], e = 0..3.
// mm: acc += sum_{k < K} A(m, k) B(k, n) with A(m, k) = pa[m am + k ak] and
// B(k, n) = pb[k bk + n bn]; the strides express any transpose.
// Within each 16-deep group of the reduction, lane group j = l / 16 takes
// the indices 4j..4j+3 in the group's four steps (any assignment gives the
// same product when both operands follow it), so an operand that is
// contiguous along the reduction (AV: ak == 1, BV: bk == 1) is read with one
// 16-byte LDS load per group instead of four.  mm keeps the operands of
// the next two groups in flight ahead of each group's products; mm_rows and
// mm_two read a group's operands just before its products and leave their
// interleaving to the compiler (with two waves per SIMD that measured
// faster than forcing the reads ahead).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool V>
__device__ __forceinline__ f4 grp4(const float* p, int stride) {
    if constexpr (V) return *reinterpret_cast<const f4*>(p);
    else return f4{p[0], p[stride], p[2 * stride], p[3 * stride]};
}

template <int K, bool AV, bool BV>
__device__ __forceinline__ f4 mm(const float* pa, int am, int ak, const float* pb, int bk, int bn, f4 acc) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    pa += i * am + 4 * j * ak;
    pb += 4 * j * bk + i * bn;
    constexpr int G = K / 16;
    f4 a[3], b[3];
    a[0] = grp4<AV>(pa, ak);
    b[0] = grp4<BV>(pb, bk);
    if constexpr (G > 1) {
        a[1] = grp4<AV>(pa + 16 * ak, ak);
        b[1] = grp4<BV>(pb + 16 * bk, bk);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g + 2 < G) {
            a[(g + 2) % 3] = grp4<AV>(pa + 16 * (g + 2) * ak, ak);
            b[(g + 2) % 3] = grp4<BV>(pb + 16 * (g + 2) * bk, bk);
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(a[g % 3][s2], b[g % 3][s2], acc);
    }
    return acc;
}

// Runtime depth K, a multiple of 16.
template <bool AV, bool BV>
__device__ __forceinline__ f4 mm_n(const float* pa, int am, int ak, const float* pb, int bk, int bn,
                                   int K, f4 acc) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    pa += i * am + 4 * j * ak;
    pb += 4 * j * bk + i * bn;
    if (K <= 0) return acc;
    f4 a0 = grp4<AV>(pa, ak), b0 = grp4<BV>(pb, bk), a1, b1;
    for (int k = 0; k < K; k += 32) {
        const bool more1 = k + 16 < K;
        if (more1) {
            a1 = grp4<AV>(pa + (k + 16) * ak, ak);
            b1 = grp4<BV>(pb + (k + 16) * bk, bk);
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(a0[s2], b0[s2], acc);
        if (!more1) break;
        if (k + 32 < K) {
            a0 = grp4<AV>(pa + (k + 32) * ak, ak);
            b0 = grp4<BV>(pb + (k + 32) * bk, bk);
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(a1[s2], b1[s2], acc);
    }
    return acc;
}

// D-layout tile <-> row-major memory (row stride ld, origin at the tile)
__device__ __forceinline__ void store_tile(float* p, int ld, f4 v) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[(4 * j + e) * ld + i] = v[e];
}
__device__ __forceinline__ f4 load_tile(const float* p, int ld) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p[(4 * j + e) * ld + i];
    return v;
}

// Sum over the 16 lanes of each DPP row (lanes 16r..16r+15), in every lane
// of the row: DPP adds, no trip through the LDS pipe.  Partners: quad xor 1,
// quad xor 2, half-row mirror (i <-> 7 - i), row mirror (i <-> 15 - i).
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);     // quad_perm [1, 0, 3, 2]
    x += dpp_f<0x4E>(x);     // quad_perm [2, 3, 0, 1]
    x += dpp_f<0x141>(x);    // row_half_mirror
    x += dpp_f<0x140>(x);    // row_mirror
    return x;
}

// Register-staged copies: load() issues every global load of a block before
// any is consumed, put() writes the block to LDS as fp32.  A block staged
// one step ahead keeps its loads in flight while the current step computes.
//
// Blk: ROWS x NC fp32 values, source row stride sld (floats).
template <int ROWS, int NC, int NTH>
struct Blk {
    static constexpr int V4 = NC / 4, N = ROWS * V4, IT = (N + NTH - 1) / NTH;
    f4 t[IT];
    __device__ __forceinline__ void load(const float* src, int sld) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N)
                t[it] = *reinterpret_cast<const f4*>(src + static_cast<size_t>(idx / V4) * sld + (idx % V4) * 4);
        }
    }
    __device__ __forceinline__ void put(float* dst, int ld) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N) *reinterpret_cast<f4*>(dst + (idx / V4) * ld + (idx % V4) * 4) = t[it];
        }
    }
};

template <bool B> struct RawT { using type = f4; };
template <> struct RawT<true> { using type = u16x4; };

// Tok: ROWS token rows x NC columns (from column c0) of a [rows, H, COLS]
// activation tensor, head h, first row row0; rows >= len (>= 1) read as
// zero.  The row index is clamped, so every load is issued unconditionally.
template <bool BF16, int COLS, int NC, int NTH, int ROWS = kChunk>
struct Tok {
    static constexpr int V4 = NC / 4, N = ROWS * V4, IT = (N + NTH - 1) / NTH;
    using Raw = typename RawT<BF16>::type;
    Raw t[IT];
    int len_ = 0;
    // the rows past len are zeroed in put(), so no load result is needed here
    __device__ __forceinline__ void load(const void* src, int64_t row0, int len, int h, int H, int c0 = 0) {
        len_ = len;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N) {
                const int r = idx / V4, c = (idx % V4) * 4;
                const int rr = r < len ? r : len - 1;
                const size_t off = (static_cast<size_t>(row0 + rr) * H + h) * COLS + c0 + c;
                if constexpr (BF16) t[it] = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(src) + off);
                else t[it] = *reinterpret_cast<const f4*>(static_cast<const float*>(src) + off);
            }
        }
    }
    __device__ __forceinline__ void put(float* dst, int ld) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N) {
                f4 x;
                if constexpr (BF16)
                    x = f4{bf16_to_f32(t[it][0]), bf16_to_f32(t[it][1]), bf16_to_f32(t[it][2]), bf16_to_f32(t[it][3])};
                else x = t[it];
                if (idx / V4 >= len_) x = zero4();
                *reinterpret_cast<f4*>(dst + (idx / V4) * ld + (idx % V4) * 4) = x;
            }
        }
    }
    // put() with every row r multiplied by scale[r]
    __device__ __forceinline__ void put_scaled(float* dst, int ld, const float* scale) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = threadIdx.x + it * NTH;
            if (N % NTH == 0 || idx < N) {
                f4 x;
                if constexpr (BF16)
                    x = f4{bf16_to_f32(t[it][0]), bf16_to_f32(t[it][1]), bf16_to_f32(t[it][2]), bf16_to_f32(t[it][3])};
                else x = t[it];
                const int r = idx / V4;
                x = r < len_ ? x * scale[r] : zero4();
                *reinterpret_cast<f4*>(dst + r * ld + (idx % V4) * 4) = x;
            }
        }
    }
};

template <int ROWS, int NC, int NTH>
__device__ __forceinline__ void load_block(float* dst, int ld, const float* src, int sld) {
    Blk<ROWS, NC, NTH> b;
    b.load(src, sld);
    b.put(dst, ld);
}

template <int NTH>
__device__ __forceinline__ void store_block(float* dst, int dld, const float* src, int ld, int rows, int ncols) {
    const int v4 = ncols / 4;
    for (int idx = threadIdx.x; idx < rows * v4; idx += NTH) {
        const int r = idx / v4, c = (idx % v4) * 4;
        *reinterpret_cast<f4*>(dst + static_cast<size_t>(r) * dld + c) = *reinterpret_cast<const f4*>(src + r * ld + c);
    }
}

// Sequential passes: one workgroup per (sequence-head pair, 16 value
// columns).  Workgroups are dealt to the 8 XCDs round-robin; the NT column
// tiles of one pair read the same per-chunk record, so they are kept on the
// same XCD (and its L2): block b = (group * NT + tile) * 8 + xcd serves
// pair group * 8 + xcd.  The grid is padded to a multiple of 8 pairs.
template <int NT>
__device__ __forceinline__ void chain_coords(int& tile, int& pair) {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    tile = slot % NT;
    pair = (slot / NT) * 8 + xcd;
}


// L2 prefetch by one wave: one word of every 128-byte line of
// [base, base + bytes) whose line index is part (mod parts) goes to an LDS
// sink of 64 words that nothing reads.  Only the issuing wave's counters see
// these loads, so a wave that does nothing else never waits for them.
__device__ __forceinline__ void l2_touch(const void* base, int bytes, int part, int parts, int* sink) {
    const int lines = bytes >> 7;
    const unsigned char* b = static_cast<const unsigned char*>(base);
    for (int line = part + parts * lane_id(); line < lines; line += parts * 64)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(b + (static_cast<size_t>(line) << 7)),
            (__attribute__((address_space(3))) void*)sink, 4, 0, 0);
}

// ---------------------------------------------------------------------------
// fp16 matrix-core operands (v_mfma_f32_16x16x32_f16) for the 16-bit paths.
//   A lane l holds A[l % 16][32 kb + 8 (l / 16) + e], e = 0..7
//   B lane l holds B[32 kb + 8 (l / 16) + e][l % 16]
//   D as for the fp32 tile.
// A operands live in memory fragment-major: fragment (mb, kb) of an M x K
// matrix is 64 lanes x 8 halves at ((mb * K / 32 + kb) * 64 + lane) * 8, so a
// wavefront reads 1 KiB of consecutive bytes.  B operands are staged in LDS
// column by column ([16][K + 8] halves), so a lane reads its 8 reduction
// indices as one 16-byte word.
// ---------------------------------------------------------------------------
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(const h8& a, const h8& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ size_t afrag_off(int mb, int kb, int nkb, int lane) {
    return (static_cast<size_t>(mb * nkb + kb) * 64 + lane) * 8;
}

// Write the fp16 A fragments of an M x K matrix whose element (m, k) is elem(m, k).
template <int M, int K, int NTH, typename F>
__device__ __forceinline__ void write_afrags(_Float16* dst, F elem) {
    constexpr int NKB = K / 32, N = (M / 16) * NKB * 64;
    for (int idx = threadIdx.x; idx < N; idx += NTH) {
        const int f = idx >> 6, lane = idx & 63, mb = f / NKB, kb = f % NKB;
        const int m = 16 * mb + (lane & 15), k0 = 32 * kb + 8 * (lane >> 4);
        h8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<_Float16>(elem(m, k0 + e));
        *reinterpret_cast<h8*>(dst + static_cast<size_t>(idx) * 8) = v;
    }
}

// B operand word of lane l from a column-major LDS tile (row stride KP halves)
__device__ __forceinline__ h8 bfrag(const _Float16* t, int kp, int kb) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    return *reinterpret_cast<const h8*>(t + i * kp + 32 * kb + 8 * j);
}

// D-layout fp32 tile holding rows k = k0 + 4 (l / 16) + e of B -> column-major fp16 LDS tile
__device__ __forceinline__ void put_btile(_Float16* t, int kp, int k0, f4 v) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    h4 h = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
            static_cast<_Float16>(v[3])};
    *reinterpret_cast<h4*>(t + i * kp + k0 + 4 * j) = h;
}

// A 16-column fp16 LDS tile stored column-major (element (r, c) at
// t[c * kp + r], as put_btile leaves it), rows 0..ROWS-1, to row-major memory
// (row stride ld halves) as 16-byte words, from threads tix = 0 .. NT-1.
template <int ROWS, int NT>
__device__ __forceinline__ void store_ctile16(_Float16* p, int ld, const _Float16* t, int kp, int tix) {
    for (int w = tix; w < ROWS * 2; w += NT) {
        const int r = w >> 1, c8 = (w & 1) * 8;
        h8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = t[(c8 + e) * kp + r];
        *reinterpret_cast<h8*>(p + static_cast<size_t>(r) * ld + c8) = x;
    }
}

// R output tiles that share their column block: tile r is row block
// mb0 + r * mstep, and acc[r] += sum over the 16-deep groups g of the
// reduction with inrange(row block, g) of A(m, k) B(k, n).  Each group's B
// operand is read once for all R tiles, and the R accumulators are
// independent chains, so their products overlap.
template <int R, int G, bool AV, bool BV, typename Range>
__device__ __forceinline__ void mm_rows(const float* pa, int am, int ak, const float* pb, int bk, int bn,
                                        int mb0, int mstep, Range inrange, f4 (&acc)[R]) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    pa += i * am + 4 * j * ak;
    pb += 4 * j * bk + i * bn;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        bool any = false;
#pragma unroll
        for (int r = 0; r < R; ++r) any |= inrange(mb0 + r * mstep, g);
        if (!any) continue;
        const f4 b = grp4<BV>(pb + 16 * g * bk, bk);
        f4 a[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (inrange(mb0 + r * mstep, g)) a[r] = grp4<AV>(pa + 16 * (mb0 + r * mstep) * am + 16 * g * ak, ak);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (inrange(mb0 + r * mstep, g)) acc[r] = mfma4(a[r][s2], b[s2], acc[r]);
    }
}

// mm_rows on the bf16 matrix cores with fp32 operands split in two: every
// operand x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (|x - hi - lo| <=
// 2^-18 |x|, fp32's exponent range), and A B ~ Ah Bh + Ah Bl + Al Bh (the
// dropped Al Bl is below 2^-16 of each term), accumulated in fp32.  One
// 16x16x32 step takes two 16-deep groups: lane group j feeds the reduction
// indices 16g + 4j + e and 16(g + 1) + 4j + e (e = 0..3) that the fp32 reads
// of mm_rows already hand it, so the operands are read exactly as there.  G
// is even; a pair of groups is taken when either is in range, so the skipped
// products must be of stored zeros.
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void split_bf16(const f4& x0, const f4& x1, bf8& hi, bf8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        const __bf16 h = static_cast<__bf16>(x);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(x - static_cast<float>(h));
    }
}
template <int R, int G, bool AV, bool BV, typename Range>
__device__ __forceinline__ void mm_rows_x3(const float* pa, int am, int ak, const float* pb, int bk, int bn,
                                           int mb0, int mstep, Range inrange, f4 (&acc)[R]) {
    static_assert(G % 2 == 0, "pairs of 16-deep groups");
    const int i = lane_id() & 15, j = lane_id() >> 4;
    pa += i * am + 4 * j * ak;
    pb += 4 * j * bk + i * bn;
#pragma unroll
    for (int g = 0; g < G; g += 2) {
        bool in[R], any = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            in[r] = inrange(mb0 + r * mstep, g) || inrange(mb0 + r * mstep, g + 1);
            any |= in[r];
        }
        if (!any) continue;
        bf8 bh, bl;
        split_bf16(grp4<BV>(pb + 16 * g * bk, bk), grp4<BV>(pb + 16 * (g + 1) * bk, bk), bh, bl);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (!in[r]) continue;
            const float* p = pa + 16 * (mb0 + r * mstep) * am + 16 * g * ak;
            bf8 ah, al;
            split_bf16(grp4<AV>(p, ak), grp4<AV>(p + 16 * ak, ak), ah, al);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[r], 0, 0, 0);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[r], 0, 0, 0);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[r], 0, 0, 0);
        }
    }
}

// mm_rows, or mm_rows_x3 when SPLIT
template <bool SPLIT, int R, int G, bool AV, bool BV, typename Range>
__device__ __forceinline__ void mm_rows_k(const float* pa, int am, int ak, const float* pb, int bk, int bn,
                                          int mb0, int mstep, Range inrange, f4 (&acc)[R]) {
    if constexpr (SPLIT) mm_rows_x3<R, G, AV, BV>(pa, am, ak, pb, bk, bn, mb0, mstep, inrange, acc);
    else mm_rows<R, G, AV, BV>(pa, am, ak, pb, bk, bn, mb0, mstep, inrange, acc);
}

// Two products that share their B operand: acc0 += A0 B, acc1 += A1 B over
// G groups of 16 reduction indices (pa0, pa1 at their tile's first row).
template <int G, bool AV, bool BV>
__device__ __forceinline__ void mm_two(const float* pa0, const float* pa1, int am, int ak, const float* pb, int bk,
                                       int bn, f4& acc0, f4& acc1) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    pa0 += i * am + 4 * j * ak;
    pa1 += i * am + 4 * j * ak;
    pb += 4 * j * bk + i * bn;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const f4 b = grp4<BV>(pb + 16 * g * bk, bk);
        const f4 a0 = grp4<AV>(pa0 + 16 * g * ak, ak), a1 = grp4<AV>(pa1 + 16 * g * ak, ak);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            acc0 = mfma4(a0[s2], b[s2], acc0);
            acc1 = mfma4(a1[s2], b[s2], acc1);
        }
    }
}

// ---------------------------------------------------------------------------
// Decay between tokens without overflow (chunk-wise normalisation, "Designing
// and Deploying Hybrid MLA and Linear Attention Architectures", section 3).
// The chunk's tokens fall in 16-token tiles; sB[r * ld + c] holds b, the
// cumulative log2 alpha of channel c restarted at every tile (so b <= 0), and
// sTot[t * ldt + c] the total of tile t.  The decay from token s to a later
// token r, 2^(b_r - b_s) over the chunk, is only ever formed from exponents
// <= 0, so no factor exceeds 1:
//   * tiles I > J:  2^(b_r) * 2^(tot of the tiles between) * 2^(tot_J - b_s)
//     (b is tile-local: the first factor runs from the start of tile I, the
//     last from s to the end of tile J);
//   * one tile: the pair (r, s) belongs to the level p of the highest bit in
//     which the tile-local indices differ; both lie in one aligned group of
//     2^(p+1) tokens, s in its lower and r in its upper half, and the decay
//     is pf_p(r) sf_p(s), with pf_p(x) = 2^(b_x - b_lo) (lo: the token before
//     x's aligned 2^p group) and sf_p(x) = 2^(b_hi - b_x) (hi: the last token
//     of that group).  A level is one matrix product with both factors
//     applied per token, of which only that level's pairs are kept.
// ---------------------------------------------------------------------------

// One 16-deep group of a 16x16 product, lane group j holding reduction
// indices 4j..4j+3 of A and B (the layout of mfma4's four steps): on the fp32
// matrix cores (four 16x16x4 steps), or with SPLIT on the bf16 ones with
// every operand split into bf16 hi + lo (as mm_rows_x3: fp32's exponent
// range, ~2^-16 relative; one 16x16x16 step per product).
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void split4_bf16(const f4& x, s4v& hi, s4v& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        hi[e] = __builtin_bit_cast(short, h);
        lo[e] = __builtin_bit_cast(short, static_cast<__bf16>(x[e] - static_cast<float>(h)));
    }
}
template <bool SPLIT>
__device__ __forceinline__ f4 mm16(f4 a, f4 b, f4 acc) {
    if constexpr (SPLIT) {
        s4v ah, al, bh, bl;
        split4_bf16(a, ah, al);
        split4_bf16(b, bh, bl);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
        return acc;
    } else {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(a[s2], b[s2], acc);
        return acc;
    }
}

// tile-local index of the token whose b enters pf_p (x has bit p set) / sf_p
__device__ __forceinline__ int lvl_lo(int x, int p) { return (x & ~((1 << p) - 1)) - 1; }
__device__ __forceinline__ int lvl_hi(int x, int p) { return x | ((1 << p) - 1); }

// pair (r, s) of one tile is taken at level p: p is the highest differing bit, r above s
__device__ __forceinline__ bool lvl_pair(int r, int s, int p) { return ((r ^ s) >> p) == 1 && ((r >> p) & 1); }

// sum of the tile totals of tiles lo .. hi-1 (4 channels from c)
__device__ __forceinline__ f4 tot4(const float* sTot, int ldt, int c, int lo, int hi) {
    f4 x = zero4();
    for (int u = lo; u < hi; ++u) x += *reinterpret_cast<const f4*>(sTot + u * ldt + c);
    return x;
}
__device__ __forceinline__ float tot1(const float* sTot, int ldt, int c, int lo, int hi) {
    float x = 0.f;
    for (int u = lo; u < hi; ++u) x += sTot[u * ldt + c];
    return x;
}

// Tile-local cumulative log2 alpha of a chunk of ROWS tokens and DK channels.
// On entry s[r * ld + c] holds the gate as given (the scalar gate: sGs[r]);
// on exit s holds b (restarted every 16 rows; padding rows add 0) and
// sTot[t * DK + c] the total of tile t.  A gate below 2^-150 counts as
// 2^-150: every fp32 factor that spans it is zero either way.  NTH / DK row
// segments per channel; sPart holds NTH floats of scratch.  Ends with a barrier.
template <int DK, int NTH, int ROWS, int GATE>
__device__ __forceinline__ void tile_gate_scan(float* s, int ld, const float* sGs, int len, float* sTot,
                                               float* sPart) {
    constexpr int NS = NTH / DK, SEG = ROWS / NS;
    static_assert(NS * SEG == ROWS && SEG <= 16 && 16 % SEG == 0, "row segments tile the 16-token tiles");
    const int c = threadIdx.x % DK, sg = threadIdx.x / DK, r0 = sg * SEG;
    float x[SEG];
#pragma unroll
    for (int r = 0; r < SEG; ++r) {
        const float g = GATE == KDA_GATE_SCALAR ? sGs[r0 + r] : s[(r0 + r) * ld + c];
        float l2 = 0.f;
        if (r0 + r < len) {
            if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16) l2 = log2_alpha_from_softplus_arg(g);
            else l2 = __builtin_amdgcn_logf(g);
            l2 = fmaxf(l2, -150.f);
        }
        x[r] = (r ? x[r - 1] : 0.f) + l2;
    }
    sPart[sg * DK + c] = x[SEG - 1];
    __syncthreads();
    const int first = (r0 / 16) * (16 / SEG);        // first segment of this tile
    float off = 0.f;
    for (int s2 = first; s2 < sg; ++s2) off += sPart[s2 * DK + c];
#pragma unroll
    for (int r = 0; r < SEG; ++r) s[(r0 + r) * ld + c] = off + x[r];
    if ((r0 + SEG) % 16 == 0) sTot[(r0 / 16) * DK + c] = off + x[SEG - 1];
    __syncthreads();
}

// Tile (mb, nb) of the C x C products over G groups of 16 channels
//   acc0 += (R0 . D) K^T,  acc1 += (R1 . D) K^T  (TWO),   D = decay from s to r,
// with R0, R1, K raw token-major rows (stride ld, reduction along the row), b
// in sB (same layout) and the tile totals in sTot (row stride ldt).  The
// tile is lower-triangular: tiles above the diagonal are not computed.  On the
// diagonal tile the strict lower part is formed; acc1 also gets its diagonal
// (r = s, no decay) when DIAG1.  D-layout: lane (i, j) holds rows 4j + e,
// column i of the tile.  SPLIT: the products on the bf16 matrix cores with
// split operands (mm16).
template <int G, bool TWO, bool DIAG1, bool SPLIT = false>
__device__ __forceinline__ void decayed_tile(const float* R0, const float* R1, const float* K, const float* sB,
                                             const float* sTot, int ld, int ldt, int mb, int nb, f4& acc0,
                                             f4& acc1) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    if (nb < mb) {
        const int r = 16 * mb + i, s = 16 * nb + i;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const int c0 = 16 * gg + 4 * j;
            const f4 br = *reinterpret_cast<const f4*>(sB + r * ld + c0);
            const f4 bs = *reinterpret_cast<const f4*>(sB + s * ld + c0);
            const f4 tt = *reinterpret_cast<const f4*>(sTot + nb * ldt + c0);
            const f4 mid = tot4(sTot, ldt, c0, nb + 1, mb);
            const f4 r0v = *reinterpret_cast<const f4*>(R0 + r * ld + c0);
            const f4 kv = *reinterpret_cast<const f4*>(K + s * ld + c0);
            f4 r1v;
            if constexpr (TWO) r1v = *reinterpret_cast<const f4*>(R1 + r * ld + c0);
            f4 fr, bk;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                fr[s2] = __builtin_amdgcn_exp2f(br[s2] + mid[s2]);
                bk[s2] = kv[s2] * __builtin_amdgcn_exp2f(tt[s2] - bs[s2]);
            }
            acc0 = mm16<SPLIT>(r0v * fr, bk, acc0);
            if constexpr (TWO) acc1 = mm16<SPLIT>(r1v * fr, bk, acc1);
        }
    } else if (nb == mb) {
        const int x = 16 * mb + i;
        f4 la[4], lb[4], pd = zero4();
#pragma unroll
        for (int p = 0; p < 4; ++p) la[p] = lb[p] = zero4();
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const int c0 = 16 * gg + 4 * j;
            const f4 kx = *reinterpret_cast<const f4*>(K + x * ld + c0);
            const f4 bx = *reinterpret_cast<const f4*>(sB + x * ld + c0);
            const f4 r0v = *reinterpret_cast<const f4*>(R0 + x * ld + c0);
            f4 r1v;
            if constexpr (TWO) r1v = *reinterpret_cast<const f4*>(R1 + x * ld + c0);
            if constexpr (TWO && DIAG1) pd = mm16<SPLIT>(r1v, kx, pd);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const bool up = (i >> p) & 1;
                const int ref = 16 * mb + (up ? lvl_lo(i, p) : lvl_hi(i, p));
                const f4 bref = *reinterpret_cast<const f4*>(sB + ref * ld + c0);
                f4 f;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) f[s2] = __builtin_amdgcn_exp2f(up ? bx[s2] - bref[s2] : bref[s2] - bx[s2]);
                const f4 kc = kx * f;
                la[p] = mm16<SPLIT>(r0v * f, kc, la[p]);
                if constexpr (TWO) lb[p] = mm16<SPLIT>(r1v * f, kc, lb[p]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * j + e;
            if (TWO && DIAG1 && row == i) acc1[e] += pd[e];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                if (lvl_pair(row, i, p)) {
                    acc0[e] += la[p][e];
                    if constexpr (TWO) acc1[e] += lb[p][e];
                }
        }
    }
}

// Decayed contractions over the tokens of a chunk (C x C by C x d_k) with b
// in sB and the tile totals in sTot as above:
//   lower:  Y[r, c] = sum_{s <= r} X[r, s] V[s, c] 2^(b_r - b_s)[c]
//   upper:  Z[s, c] = sum_{r >= s} X[r, s] V[r, c] 2^(b_r - b_s)[c]
// formed together, since they share every decay factor:
//   y0 += lower(X0, K),  y1 += lower(X1, K),  z += upper(X1, Q) + upper(X0, K)
// for the R row blocks mb0 + r * mstep and the 16 channels nb * 16 .. + 15
// (column i of the D layout).  X0 is strictly lower-triangular, X1 includes
// its diagonal (r = s, no decay); elements above the diagonal are never
// read.  X is row-major (stride ldx), K, Q and sB token-major (stride ld),
// sTot has row stride ldt.  Lane (i, j) holds the B operand rows 4j + s2 and
// the output rows 4j + e of every block, so the factors of those tokens in
// channel c serve both the operands and the outputs:
//   pf(x) = 2^(b_x)          decay from the start of x's tile to x
//   sf(x) = 2^(tot - b_x)    decay after x to the end of its tile
// Blocks below the diagonal use Horner's rule over the tiles in between (one
// multiply of the accumulator per block step, by the tile total 2^tot, a
// factor of the channel only); diagonal blocks go level by level.
template <int R, int NBLK, bool SPLIT = false>
__device__ __forceinline__ void decayed_lower_upper(const float* X0, const float* X1, int ldx, const float* K,
                                                    const float* Q, const float* sB, const float* sTot, int ld,
                                                    int ldt, int mb0, int mstep, int nb, f4 (&y0)[R],
                                                    f4 (&y1)[R], f4 (&z)[R]) {
    const int i = lane_id() & 15, j = lane_id() >> 4;
    const int c = 16 * nb + i;
    // the factors of this lane's four tokens of block t
    auto pf4 = [&](int t) {
        f4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_exp2f(sB[(16 * t + 4 * j + e) * ld + c]);
        return x;
    };
    auto sf4 = [&](int t) {
        const float tot = sTot[t * ldt + c];
        f4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_exp2f(tot - sB[(16 * t + 4 * j + e) * ld + c]);
        return x;
    };
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int I = mb0 + rr * mstep;
        __builtin_amdgcn_sched_barrier(0);
        // lower, blocks J < I: B = K[s] sf(s), Horner over J, rows times pf(r)
        if (I > 0) {
            f4 h0 = zero4(), h1 = zero4();
            for (int J = 0; J < I; ++J) {
                if (J > 0) {
                    const float F = __builtin_amdgcn_exp2f(sTot[J * ldt + c]);
                    h0 *= F;
                    h1 *= F;
                }
                const f4 x0 = *reinterpret_cast<const f4*>(X0 + (16 * I + i) * ldx + 16 * J + 4 * j);
                const f4 x1 = *reinterpret_cast<const f4*>(X1 + (16 * I + i) * ldx + 16 * J + 4 * j);
                const f4 sfj = sf4(J);
                f4 bk;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) bk[s2] = K[(16 * J + 4 * j + s2) * ld + c] * sfj[s2];
                h0 = mm16<SPLIT>(x0, bk, h0);
                h1 = mm16<SPLIT>(x1, bk, h1);
                __builtin_amdgcn_sched_barrier(0);
            }
            const f4 pfi = pf4(I);
            y0[rr] += h0 * pfi;
            y1[rr] += h1 * pfi;
        }
        __builtin_amdgcn_sched_barrier(0);
        // upper, blocks I2 > I (the output block is I): B = V[r] pf(r), Horner
        // over I2 from the last, rows times sf(s)
        if (I < NBLK - 1) {
            f4 h2 = zero4();
            for (int I2 = NBLK - 1; I2 > I; --I2) {
                if (I2 < NBLK - 1) h2 *= __builtin_amdgcn_exp2f(sTot[I2 * ldt + c]);
                const f4 pfi2 = pf4(I2);
                f4 a1, a0, bq, bk;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int rk = 16 * I2 + 4 * j + s2;
                    a1[s2] = X1[rk * ldx + 16 * I + i];
                    a0[s2] = X0[rk * ldx + 16 * I + i];
                    bq[s2] = Q[rk * ld + c] * pfi2[s2];
                    bk[s2] = K[rk * ld + c] * pfi2[s2];
                }
                h2 = mm16<SPLIT>(a1, bq, h2);
                h2 = mm16<SPLIT>(a0, bk, h2);
                __builtin_amdgcn_sched_barrier(0);
            }
            z[rr] += h2 * sf4(I);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the diagonal block I, level by level
        const f4 x0l = *reinterpret_cast<const f4*>(X0 + (16 * I + i) * ldx + 16 * I + 4 * j);
        const f4 x1l = *reinterpret_cast<const f4*>(X1 + (16 * I + i) * ldx + 16 * I + 4 * j);
        f4 x0u, x1u, kv, qv, bv;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int rk = 16 * I + 4 * j + s2;
            x0u[s2] = X0[rk * ldx + 16 * I + i];
            x1u[s2] = X1[rk * ldx + 16 * I + i];
            kv[s2] = K[rk * ld + c];
            qv[s2] = Q[rk * ld + c];
            bv[s2] = sB[rk * ld + c];
        }
        {   // the diagonal of X1 (r = s): lower X1[r][r] K[r], upper X1[s][s] Q[s]
            f4 m1, m2;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const bool on = i == 4 * j + s2;
                m1[s2] = on ? x1l[s2] : 0.f;
                m2[s2] = on ? x1u[s2] : 0.f;
            }
            y1[rr] = mm16<SPLIT>(m1, kv, y1[rr]);
            z[rr] = mm16<SPLIT>(m2, qv, z[rr]);
        }
        // (a loop at run time: unrolled, the four levels' operands crowd the registers)
#pragma unroll 1
        for (int p = 0; p < 4; ++p) {
            // pf_p (bit p set) and sf_p of this lane's four tokens 4j + e
            f4 pp, ss;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int xl = 4 * j + e;
                const int lo = lvl_lo(xl, p) < 0 ? 0 : lvl_lo(xl, p);   // in range even if read speculatively
                pp[e] = (xl >> p) & 1 ? __builtin_amdgcn_exp2f(bv[e] - sB[(16 * I + lo) * ld + c]) : 0.f;
                ss[e] = __builtin_amdgcn_exp2f(sB[(16 * I + lvl_hi(xl, p)) * ld + c] - bv[e]);
            }
            f4 a0, a1, u1, u0;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int kl = 4 * j + s2;                      // reduction token (B row)
                const bool lo = lvl_pair(i, kl, p);             // lower: r = i above s = kl
                const bool up = lvl_pair(kl, i, p);             // upper: r = kl above s = i
                a0[s2] = lo ? x0l[s2] : 0.f;
                a1[s2] = lo ? x1l[s2] : 0.f;
                u1[s2] = up ? x1u[s2] : 0.f;
                u0[s2] = up ? x0u[s2] : 0.f;
            }
            const f4 bk = kv * ss;
            f4 t0 = mm16<SPLIT>(a0, bk, zero4());
            f4 t1 = mm16<SPLIT>(a1, bk, zero4());
            f4 t2 = mm16<SPLIT>(u1, qv * pp, zero4());
            t2 = mm16<SPLIT>(u0, kv * pp, t2);
            y0[rr] += t0 * pp;
            y1[rr] += t1 * pp;
            z[rr] += t2 * ss;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace mm32
}  // namespace kda
