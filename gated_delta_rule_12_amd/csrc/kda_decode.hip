// KDA recurrent decode step: one token per (sequence, head), fp32 state
// updated in place.
//
// For one (sequence, head) with S~ = Diag(alpha) S (decay every key channel
// first), the KDA update (I - beta k k^T) S~ + beta k v^T and the read-out
// o = S_new^T q expand, by distributivity only, into
//     p     = S~^T k,   r = S~^T q,   delta = beta (v - p),
//     S_new = S~ + k delta^T,         o = r + (q . k) delta,
// so the state is read once and written once.  (KDA rule: "Hybrid Linear
// Attention Architectures...", Core Module Design, Stage 3; decode is the
// memory-bound token-by-token mode that "Linear Attention + Sparse
// Attention...", section 6, asks to benchmark apart from prefill.)
//
// Mapping: one 512-thread workgroup per (sequence, head, block of CB value
// columns), CB = 128: at d_v = 128 a workgroup owns a whole head, 64 KiB of
// contiguous state, held in registers between the read and the write (the
// columns of S evolve independently, since decay and write act on rows, and
// the projections p and r reduce over rows, so a column block is a
// self-contained task).  Thread (rg, cg) owns columns 4cg..4cg+3 of the block
// in rows rg, rg+RG, ...: one load instruction of the workgroup covers RG
// whole rows.  Column sums over the key channels are reduced with cross-lane
// shuffles inside a wavefront, then through LDS across the eight wavefronts.
// The state is read with ordinary loads and written with non-temporal
// stores.  Measured on the 256 x 32-head decode workload: 160 us per step
// (6.8 TB/s); the same tiling with non-temporal loads 199 us, with ordinary
// stores 213 us; half-head tiles (64 columns, 256 threads) 197 us; 256 or
// 1024 threads per whole head 168 / 194 us; one wavefront per 32 columns and
// no barriers 202 us.
#include "kda_common.h"

namespace kda {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// value columns and threads per workgroup
constexpr int kDecodeCols = 128;
constexpr int kDecodeThreads = 512;

// the forget gate of key channel c of task `pair`, in the form GATE (kda_gate)
template <int GATE, int DK>
__device__ __forceinline__ float gate_alpha(const void* __restrict__ gate, size_t pair, int c) {
    if constexpr (GATE == KDA_GATE_ALPHA) return static_cast<const float*>(gate)[pair * DK + c];
    else if constexpr (GATE == KDA_GATE_SOFTPLUS_BF16)
        return __builtin_amdgcn_exp2f(log2_alpha_from_softplus_arg(
            bf16_to_f32(static_cast<const uint16_t*>(gate)[pair * DK + c])));
    else return static_cast<const float*>(gate)[pair];
}

template <int DK, int DV, int CB, bool ABF16, bool OBF16, int GATE>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const typename Act<ABF16>::T* __restrict__ q, const typename Act<ABF16>::T* __restrict__ k,
    const typename Act<ABF16>::T* __restrict__ v, const void* __restrict__ gate,
    const float* __restrict__ beta, float* __restrict__ state, void* __restrict__ o) {
    constexpr int NCB = DV / CB;          // column blocks per (sequence, head)
    constexpr int CG = CB / 4;            // column groups of 4 floats
    constexpr int RG = kDecodeThreads / CG;   // row groups
    constexpr int RPT = DK / RG;          // rows per thread
    constexpr int NW = kDecodeThreads / 64;   // wavefronts per workgroup
    static_assert(NCB * CB == DV && RG * CG == kDecodeThreads && RPT * RG == DK && CG <= 64, "decode tiling");

    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t pair = blockIdx.x / NCB; // n * H + h
    const int col0 = (blockIdx.x - static_cast<int>(pair) * NCB) * CB;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f4 s_red[2][NW][CG];
    __shared__ float s_qk;

    // Issue the state loads first: they are the only HBM-heavy traffic.
    f4* sp = reinterpret_cast<f4*>(state + pair * (size_t)(DK * DV) + col0);
    f4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = sp[(i * RG + rg) * (DV / 4) + cg];

    for (int c = tid; c < DK; c += kDecodeThreads) {
        s_k[c] = Act<ABF16>::load(k, pair * DK + c);
        s_q[c] = Act<ABF16>::load(q, pair * DK + c);
        s_a[c] = gate_alpha<GATE, DK>(gate, pair, c);
    }
    __syncthreads();

    if (wave == 0) {
        float x = 0.f;
        for (int c = lane; c < DK; c += 64) x += s_q[c] * s_k[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (lane == 0) s_qk = x;
    }

    // Decay first, then the two projections of the decayed state.
    f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = i * RG + rg;
        s[i] *= s_a[r];
        pk += s[i] * s_k[r];
        pq += s[i] * s_q[r];
    }
    // Reduce over the row groups that share a wavefront.
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += __shfl_xor(pk[j], off);
            pq[j] += __shfl_xor(pq[j], off);
        }
    }
    if (lane < CG) {
        s_red[0][wave][cg] = pk;
        s_red[1][wave][cg] = pq;
    }
    __syncthreads();

    f4 p = s_red[0][0][cg], rr = s_red[1][0][cg];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        p += s_red[0][w][cg];
        rr += s_red[1][w][cg];
    }
    const float b = beta[pair];
    f4 vv;
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = Act<ABF16>::load(v, pair * DV + col0 + 4 * cg + j);
    const f4 d = b * (vv - p);

    if (rg == 0) {
        const f4 out = rr + s_qk * d;
#pragma unroll
        for (int j = 0; j < 4; ++j) store_out<OBF16>(o, pair * DV + col0 + 4 * cg + j, out[j]);
    }

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = i * RG + rg;
        s[i] += s_k[r] * d;
        __builtin_nontemporal_store(s[i], &sp[(i * RG + rg) * (DV / 4) + cg]);
    }
}

template <int DK, int DV, bool ABF16, bool OBF16, int GATE>
hipError_t launch(const void* q, const void* k, const void* v, const void* gate,
                  const float* beta, float* state, void* o, int pairs, hipStream_t stream) {
    using T = typename Act<ABF16>::T;
    constexpr int CB = kDecodeCols < DV ? kDecodeCols : DV;
    hipLaunchKernelGGL((decode_kernel<DK, DV, CB, ABF16, OBF16, GATE>), dim3(pairs * (DV / CB)),
                       dim3(kDecodeThreads), 0, stream, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), gate, beta, state, o);
    return hipGetLastError();
}

template <int DK, int DV, int GATE>
hipError_t dispatch_types(const void* q, const void* k, const void* v, const void* gate,
                          const float* beta, float* state, void* o, int pairs, bool abf16,
                          bool obf16, hipStream_t stream) {
    if (!abf16) return launch<DK, DV, false, false, GATE>(q, k, v, gate, beta, state, o, pairs, stream);
    if (obf16) return launch<DK, DV, true, true, GATE>(q, k, v, gate, beta, state, o, pairs, stream);
    return launch<DK, DV, true, false, GATE>(q, k, v, gate, beta, state, o, pairs, stream);
}

template <int DK, int DV>
hipError_t dispatch_gate(const void* q, const void* k, const void* v, const void* gate,
                         int gate_kind, const float* beta, float* state, void* o, int pairs,
                         bool abf16, bool obf16, hipStream_t stream) {
    if (gate_kind == KDA_GATE_ALPHA)
        return dispatch_types<DK, DV, KDA_GATE_ALPHA>(q, k, v, gate, beta, state, o, pairs, abf16, obf16, stream);
    if (gate_kind == KDA_GATE_SOFTPLUS_BF16)
        return dispatch_types<DK, DV, KDA_GATE_SOFTPLUS_BF16>(q, k, v, gate, beta, state, o, pairs, abf16, obf16, stream);
    return dispatch_types<DK, DV, KDA_GATE_SCALAR>(q, k, v, gate, beta, state, o, pairs, abf16, obf16, stream);
}

}  // namespace

hipError_t launch_recurrent_step(const void* q, const void* k, const void* v,
                                 const void* gate, int gate_kind, const float* beta, float* state,
                                 void* o, int N, int H, int Dk, int Dv, bool act_bf16,
                                 bool out_bf16, hipStream_t stream) {
    const int pairs = N * H;
    if (Dk == 128 && Dv == 128)
        return dispatch_gate<128, 128>(q, k, v, gate, gate_kind, beta, state, o, pairs, act_bf16, out_bf16, stream);
    if (Dk == 64 && Dv == 64)
        return dispatch_gate<64, 64>(q, k, v, gate, gate_kind, beta, state, o, pairs, act_bf16, out_bf16, stream);
    if (Dk == 128 && Dv == 64)
        return dispatch_gate<128, 64>(q, k, v, gate, gate_kind, beta, state, o, pairs, act_bf16, out_bf16, stream);
    if (Dk == 64 && Dv == 128)
        return dispatch_gate<64, 128>(q, k, v, gate, gate_kind, beta, state, o, pairs, act_bf16, out_bf16, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
