// Host side of the KDA C ABI: argument validation, workspace planning and
// kernel dispatch.  Every check runs before the first launch; a rejected call
// launches nothing.
#include <stdint.h>

#include <mutex>

#include "kda_chunk.h"
#include "kda_common.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool valid_gate(kda_gate g) {
    return g == KDA_GATE_ALPHA || g == KDA_GATE_SOFTPLUS_BF16 || g == KDA_GATE_SCALAR;
}

// alignment the kernels' gate loads need: 16 B (fp32 x 4), 8 B (bf16 x 4), 4 B
bool gate_aligned(const void* p, kda_gate g) {
    if (g == KDA_GATE_ALPHA) return aligned16(p);
    if (g == KDA_GATE_SOFTPLUS_BF16) return aligned8(p);
    return aligned4(p);
}

bool supported_head(int d) { return d == 64 || d == 128; }

// chunk sizes of the forward: 64 (the main kernels) and 32 / 128 (generic fp32 path)
bool supported_chunk(int c) { return c == 32 || c == 64 || c == 128; }

bool valid_dtype(kda_dtype d) { return d == KDA_DTYPE_F32 || d == KDA_DTYPE_BF16; }

// Output may be fp32 for any activation type, bf16 only for bf16 activations.
bool valid_out(kda_dtype act, kda_dtype out) {
    return out == KDA_DTYPE_F32 || (out == KDA_DTYPE_BF16 && act == KDA_DTYPE_BF16);
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH; }

// The workspace of kda_chunk_fwd_static: a file-scope device array, one copy
// per GPU the library's code is loaded on, held until the process ends.  Its
// name is only a host-side handle; the device address of each GPU's copy is
// looked up once, with that GPU current, and kept here.
static_assert(KDA_STATIC_WORKSPACE_BYTES % 256 == 0, "whole 256-byte lines");
__device__ __align__(256) unsigned char scratch[KDA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that `stream` belongs to (the
// current GPU for the null stream).
kda_status static_workspace(hipStream_t stream, void** out) {
    int dev = 0;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return KDA_ERROR_INVALID_VALUE;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return KDA_ERROR_LAUNCH;
    }
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERROR_NOT_SUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return KDA_ERROR_LAUNCH;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return KDA_ERROR_LAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return KDA_ERROR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_SUCCESS;
}

// Validation and dispatch of the chunkwise forward.  With `static_ws` the
// workspace arguments are ignored and the library's static array is used.
kda_status chunk_fwd(const void* q, const void* k, const void* v, const void* gate,
                     kda_gate gate_kind, const float* beta, const float* initial_state,
                     float* final_state, const int32_t* cu_seqlens, int num_seqs, void* o, int B,
                     int64_t T, int H, int Dk, int Dv, int chunk_size, kda_dtype act_dtype,
                     kda_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                     bool static_ws) {
    if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype) || !valid_gate(gate_kind))
        return KDA_ERROR_INVALID_VALUE;
    if (!valid_out(act_dtype, out_dtype)) return KDA_ERROR_NOT_SUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens != nullptr && (B != 1 || num_seqs < 0)) return KDA_ERROR_INVALID_VALUE;
    if (!supported_head(Dk) || !supported_head(Dv) || !supported_chunk(chunk_size))
        return KDA_ERROR_NOT_SUPPORTED;

    kda::ChunkPlan plan;
    const kda_status ps = kda::make_chunk_plan(B, T, H, Dk, Dv, cu_seqlens != nullptr, num_seqs,
                                               chunk_size, act_dtype == KDA_DTYPE_BF16, &plan);
    if (ps != KDA_SUCCESS) return ps;

    const bool has_tokens = (int64_t)B * T > 0;
    if (has_tokens) {
        if (!q || !k || !v || !gate || !beta || !o) return KDA_ERROR_INVALID_VALUE;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !gate_aligned(gate, gate_kind) ||
            !aligned4(beta) || !aligned16(o))
            return KDA_ERROR_INVALID_VALUE;
    }
    if (cu_seqlens && !aligned16(cu_seqlens)) return KDA_ERROR_INVALID_VALUE;
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERROR_INVALID_VALUE;
    if (static_ws) {
        if (plan.workspace_bytes > KDA_STATIC_WORKSPACE_BYTES) return KDA_ERROR_WORKSPACE_TOO_SMALL;
        if (plan.N == 0) return KDA_SUCCESS;
        const kda_status ws = static_workspace(static_cast<hipStream_t>(stream), &workspace);
        if (ws != KDA_SUCCESS) return ws;
    } else {
        if (plan.N == 0) return KDA_SUCCESS;             // nothing to compute or write
        if (plan.workspace_bytes > 0) {
            if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
                return KDA_ERROR_INVALID_VALUE;
            if (workspace_bytes < plan.workspace_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;
        }
    }

    kda::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.gate_kind = gate_kind; a.beta = beta;
    a.initial_state = initial_state; a.final_state = final_state;
    a.cu_seqlens = cu_seqlens; a.o = o; a.workspace = workspace;
    a.act_bf16 = act_dtype == KDA_DTYPE_BF16;
    a.out_bf16 = out_dtype == KDA_DTYPE_BF16;
    return from_hip(kda::launch_chunk_fwd(plan, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_SUCCESS: return "KDA_SUCCESS";
        case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
        case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
        case KDA_ERROR_WORKSPACE_TOO_SMALL: return "KDA_ERROR_WORKSPACE_TOO_SMALL";
        case KDA_ERROR_LAUNCH: return "KDA_ERROR_LAUNCH";
    }
    return "KDA_ERROR_UNKNOWN";
}

size_t kda_chunk_fwd_workspace_bytes(int B, int64_t T, int H, int Dk, int Dv, int varlen,
                                     int num_seqs, int chunk_size, kda_dtype act_dtype) {
    kda::ChunkPlan plan;
    if (kda::make_chunk_plan(B, T, H, Dk, Dv, varlen != 0, num_seqs, chunk_size,
                             act_dtype == KDA_DTYPE_BF16, &plan) != KDA_SUCCESS)
        return 0;
    if (!valid_dtype(act_dtype)) return 0;
    return plan.workspace_bytes;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* initial_state, float* final_state,
                         const int32_t* cu_seqlens, int num_seqs, void* o, int B, int64_t T,
                         int H, int Dk, int Dv, int chunk_size, kda_dtype act_dtype,
                         kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                         void* stream) {
    return kda_chunk_fwd_gated(q, k, v, alpha, KDA_GATE_ALPHA, beta, initial_state, final_state,
                               cu_seqlens, num_seqs, o, B, T, H, Dk, Dv, chunk_size, act_dtype,
                               out_dtype, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* gate,
                               kda_gate gate_kind, const float* beta, const float* initial_state,
                               float* final_state, const int32_t* cu_seqlens, int num_seqs,
                               void* o, int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                               kda_dtype act_dtype, kda_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return chunk_fwd(q, k, v, gate, gate_kind, beta, initial_state, final_state, cu_seqlens,
                     num_seqs, o, B, T, H, Dk, Dv, chunk_size, act_dtype, out_dtype, workspace,
                     workspace_bytes, stream, false);
}

kda_status kda_chunk_fwd_static(const void* q, const void* k, const void* v, const void* gate,
                                kda_gate gate_kind, const float* beta, const float* initial_state,
                                float* final_state, const int32_t* cu_seqlens, int num_seqs,
                                void* o, int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                                kda_dtype act_dtype, kda_dtype out_dtype, void* stream) {
    return chunk_fwd(q, k, v, gate, gate_kind, beta, initial_state, final_state, cu_seqlens,
                     num_seqs, o, B, T, H, Dk, Dv, chunk_size, act_dtype, out_dtype, nullptr, 0,
                     stream, true);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int64_t T, int H, int Dk, int Dv, int varlen,
                                     int num_seqs, int chunk_size, kda_dtype act_dtype) {
    if (!valid_dtype(act_dtype)) return 0;
    kda::ChunkBwdPlan plan;
    if (kda::make_chunk_bwd_plan(B, T, H, Dk, Dv, varlen != 0, num_seqs, chunk_size,
                                 act_dtype == KDA_DTYPE_BF16, &plan) != KDA_SUCCESS)
        return 0;
    return plan.workspace_bytes;
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* gate,
                         kda_gate gate_kind, const float* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int num_seqs, const void* dout,
                         const float* dfinal_state, void* dq, void* dk, void* dv, float* dgate,
                         float* dbeta, float* dinitial_state, int B, int64_t T, int H, int Dk,
                         int Dv, int chunk_size, kda_dtype act_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!valid_dtype(act_dtype) || !valid_gate(gate_kind)) return KDA_ERROR_INVALID_VALUE;
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens != nullptr && (B != 1 || num_seqs < 0)) return KDA_ERROR_INVALID_VALUE;
    if (!supported_head(Dk) || !supported_head(Dv) || chunk_size != 64) return KDA_ERROR_NOT_SUPPORTED;

    kda::ChunkBwdPlan plan;
    const kda_status ps = kda::make_chunk_bwd_plan(B, T, H, Dk, Dv, cu_seqlens != nullptr,
                                                   num_seqs, chunk_size,
                                                   act_dtype == KDA_DTYPE_BF16, &plan);
    if (ps != KDA_SUCCESS) return ps;

    if ((int64_t)B * T > 0) {
        if (!q || !k || !v || !gate || !beta || !dout || !dq || !dk || !dv || !dgate || !dbeta)
            return KDA_ERROR_INVALID_VALUE;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !gate_aligned(gate, gate_kind) ||
            !aligned4(beta) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
            !aligned16(dv) || !aligned4(dgate) || !aligned4(dbeta))
            return KDA_ERROR_INVALID_VALUE;
    }
    if (cu_seqlens && !aligned16(cu_seqlens)) return KDA_ERROR_INVALID_VALUE;
    if ((initial_state && !aligned16(initial_state)) || (dfinal_state && !aligned16(dfinal_state)) ||
        (dinitial_state && !aligned16(dinitial_state)))
        return KDA_ERROR_INVALID_VALUE;
    if (plan.fwd.N == 0) return KDA_SUCCESS;             // nothing to compute or write
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes < plan.workspace_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;

    kda::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.gate_kind = gate_kind; a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.dout = dout; a.dfinal_state = dfinal_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dgate = dgate; a.dbeta = dbeta;
    a.dinitial_state = dinitial_state; a.workspace = workspace;
    a.act_bf16 = act_dtype == KDA_DTYPE_BF16;
    return from_hip(kda::launch_chunk_bwd(plan, a, static_cast<hipStream_t>(stream)));
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, float* state, void* o, int N, int H, int Dk,
                              int Dv, kda_dtype act_dtype, kda_dtype out_dtype, void* stream) {
    return kda_recurrent_step_gated(q, k, v, alpha, KDA_GATE_ALPHA, beta, state, o, N, H, Dk, Dv,
                                    act_dtype, out_dtype, stream);
}

kda_status kda_recurrent_step_gated(const void* q, const void* k, const void* v, const void* gate,
                                    kda_gate gate_kind, const float* beta, float* state, void* o,
                                    int N, int H, int Dk, int Dv, kda_dtype act_dtype,
                                    kda_dtype out_dtype, void* stream) {
    if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype) || !valid_gate(gate_kind))
        return KDA_ERROR_INVALID_VALUE;
    if (!valid_out(act_dtype, out_dtype)) return KDA_ERROR_NOT_SUPPORTED;
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERROR_INVALID_VALUE;
    if (!supported_head(Dk) || !supported_head(Dv)) return KDA_ERROR_NOT_SUPPORTED;
    // one workgroup per (sequence, head, block of up to 64 value columns)
    if ((int64_t)N * H * 2 > 0x7fffffffLL) return KDA_ERROR_NOT_SUPPORTED;
    if (N == 0) return KDA_SUCCESS;
    if (!q || !k || !v || !gate || !beta || !state || !o) return KDA_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !gate_aligned(gate, gate_kind) ||
        !aligned4(beta) || !aligned16(state) || !aligned16(o))
        return KDA_ERROR_INVALID_VALUE;
    return from_hip(kda::launch_recurrent_step(q, k, v, gate, static_cast<int>(gate_kind), beta,
                                               state, o, N, H, Dk, Dv,
                                               act_dtype == KDA_DTYPE_BF16,
                                               out_dtype == KDA_DTYPE_BF16,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
