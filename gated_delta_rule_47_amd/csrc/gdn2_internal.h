// Host-side plumbing shared by the libgdn2 translation units: the workspace
// layout, the argument blocks passed to the kernels and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

// Per-chunk intermediates written by the chunk-factor kernel and consumed by
// the state-propagation kernel.  All arrays are indexed [chunk id][head][...].
struct WorkspaceLayout {
    size_t total = 0;
    int max_chunks = 0;
    size_t off_T = 0, off_W = 0, off_Qh = 0, off_KhT = 0, off_M = 0, off_U = 0, off_gl = 0,
           off_plan = 0;
    size_t plan_ints = 0;
};

// Returns false when the sizes overflow or are invalid.
bool workspace_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                      WorkspaceLayout *out);

struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *b, *w;
    const float *S0;
    void *o;
    float *S_final;
    const int32_t *cu_seqlens;
    int N, B, T, H;
    int NC;               // dense: chunks per sequence
    int max_chunks;       // chunk-id capacity (grid of the chunk-factor kernel)
    int32_t *plan;        // packed calls: chunk table (nullptr for dense calls)
    void *ws_T, *ws_W, *ws_Qh, *ws_KhT, *ws_M, *ws_U;
    float *ws_gl;
    int store_T;          // the chunk-factor kernel also stores T = (I + A)^-1
};

struct StepArgs {
    const void *q, *k, *v;
    const float *log_alpha, *b, *w;
    float *S;
    void *o;
    int B, H;
};

// Launchers (each enqueues on `stream` and returns hipGetLastError()).
hipError_t launch_plan(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_chunk_prep(const ChunkArgs &a, int Dk, bool bf16_io, hipStream_t stream);
hipError_t launch_chunk_prop(const ChunkArgs &a, int Dk, bool bf16_io, hipStream_t stream);
hipError_t launch_step(const StepArgs &a, int Dk, bool bf16_io, hipStream_t stream);

}  // namespace gdn2
