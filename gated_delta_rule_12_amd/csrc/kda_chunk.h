// Chunkwise forward: workspace plan and launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int kChunk = 64;      // tokens per chunk

// Where everything lives in the caller's workspace.  All offsets are bytes
// from the workspace base and 256-byte aligned.
//
//   ctrl       int32[4]            [0] = number of chunks actually used
//   first      int32[N+1]          first chunk of each sequence (prefix sums)
//   order      int32[N]            sequences by decreasing length (ties: index)
//   table      int32[Gmax][4]      per chunk: sequence, first token row, length
//   records    one per (head h, chunk g), at index h*Gmax + g, rec_bytes
//              each, so the chunks of one head follow each other.  With
//              E = fp16 (bf16 activations) or fp32 (fp32 activations):
//     qh       E[64][Dk]           Gamma (.) Q            (token-major)
//     w        E[64][Dk]           W = T Diag(beta) (Gamma (.) K)
//     ktt      E[Dk][64]           ((gamma/Gamma) (.) K)^T (channel-major)
//     p        E[64][64]           Tril((Gamma.Q)(K/Gamma)^T), zero above the diagonal
//     ut       E[Dv][64]           U^T, U = T Diag(beta) V (accumulator fragments)
//     gam      f32[Dk]             whole-chunk decay gamma
struct ChunkPlan {
    int B = 0, H = 0, Dk = 0, Dv = 0, N = 0;
    int C = kChunk;               // tokens per chunk: 64 (kernels above) or 32 / 128 (generic path)
    int64_t T = 0;
    bool varlen = false;
    bool f16 = false;             // bf16 activations -> fp16 matrix-core operands
    int64_t gmax = 0;             // chunk-table capacity
    size_t eb = 4;                // bytes per intermediate element
    size_t off_ctrl = 0, off_first = 0, off_order = 0, off_table = 0;
    size_t off_slow = 0;          // (chunk, head) list of the preparation kernels' general form
    size_t off_rec = 0, rec_bytes = 0;
    size_t workspace_bytes = 0;
};

struct ChunkArgs {
    const void *q = nullptr, *k = nullptr, *v = nullptr;
    const void* gate = nullptr;               // forget gate, in the form gate_kind
    kda_gate gate_kind = KDA_GATE_ALPHA;
    const float* beta = nullptr;
    const float* initial_state = nullptr;
    float* final_state = nullptr;
    const int32_t* cu_seqlens = nullptr;
    void* o = nullptr;
    void* workspace = nullptr;
    bool act_bf16 = false, out_bf16 = false;
};

kda_status make_chunk_plan(int B, int64_t T, int H, int Dk, int Dv, bool varlen, int num_seqs,
                           int chunk_size, bool act_bf16, ChunkPlan* plan);

hipError_t launch_chunk_fwd(const ChunkPlan& plan, const ChunkArgs& args, hipStream_t stream);

// Chunk sizes other than 64 (kda_chunk_generic.hip): an fp32 path with its
// own per-(head, chunk) record of generic_record_bytes bytes.
size_t generic_record_bytes(int Dk, int Dv, int chunk_size, bool act16);
hipError_t launch_chunk_fwd_generic(const ChunkPlan& plan, const ChunkArgs& args, hipStream_t stream);

// Enqueue the chunk-table kernel: fills ctrl, first, order and table of the
// plan's layout inside `workspace`.
hipError_t launch_chunk_plan(const ChunkPlan& plan, const int32_t* cu_seqlens, void* workspace,
                             hipStream_t stream);

// Backward: the forward's chunk table followed by one record per
// (head, chunk), at index h * gmax + g (layout in kda_chunk_bwd.hip), then
// the list of chunks that take the general form and a flag per chunk.
struct ChunkBwdPlan {
    ChunkPlan fwd;                // sizes and chunk-table offsets (its records are unused)
    size_t off_rec = 0, rec_bytes = 0;
    size_t off_slow = 0, off_flag = 0;
    size_t workspace_bytes = 0;
};

struct ChunkBwdArgs {
    const void *q = nullptr, *k = nullptr, *v = nullptr;
    const void* gate = nullptr;
    kda_gate gate_kind = KDA_GATE_ALPHA;
    const float* beta = nullptr;
    const float* initial_state = nullptr;
    const int32_t* cu_seqlens = nullptr;
    const void* dout = nullptr;
    const float* dfinal_state = nullptr;
    void *dq = nullptr, *dk = nullptr, *dv = nullptr;
    float* dgate = nullptr;
    float* dbeta = nullptr;
    float* dinitial_state = nullptr;
    void* workspace = nullptr;
    bool act_bf16 = false;
};

kda_status make_chunk_bwd_plan(int B, int64_t T, int H, int Dk, int Dv, bool varlen, int num_seqs,
                               int chunk_size, bool act_bf16, ChunkBwdPlan* plan);

hipError_t launch_chunk_bwd(const ChunkBwdPlan& plan, const ChunkBwdArgs& args, hipStream_t stream);

}  // namespace kda
