// Host-side plumbing shared by the libgdn2 translation units: the workspace
// layout, the argument blocks passed to the kernels and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

typedef __bf16 bf16_t;

// Offset of a workspace slot that a layout does not have.
constexpr size_t kNoSlot = ~(size_t)0;

// Per-chunk intermediates written by the chunk-factor kernel and consumed by
// the state-propagation kernel.  All arrays are indexed [chunk id][head][...].
// total covers every slot a forward call uses; total_T also covers T, which
// is stored only on request and sits after everything else.
struct WorkspaceLayout {
    size_t total = 0, total_T = 0;
    int max_chunks = 0;
    size_t off_T = 0, off_W = 0, off_Qh = 0, off_KhT = 0, off_M = 0, off_U = 0, off_gl = 0,
           off_plan = 0;
    size_t plan_ints = 0;
};

// Returns false when the sizes overflow or are invalid.  for_bwd: the layout
// a backward call needs (no T, Qhat or M slots; those offsets are kNoSlot).
bool workspace_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                      WorkspaceLayout *out, bool for_bwd = false);

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
    int gate_logits;      // log_alpha, b, w are bf16: log alpha and the logits of b and w
    long long ld_gate;    // with gate_logits: elements between consecutive tokens of
                          // log_alpha, b and w (H * Dk when they are separate arrays)
    const float *alpha_bias;  // with gate_logits: if set, log_alpha holds logits and
                              // log alpha = logsigmoid(log_alpha + alpha_bias[h][c])
    bf16_t *ws_Sc;        // if set, the propagation stores every chunk's incoming
                          // state here (bf16 [chunk id][head], layout of sc_index)
                          // and writes no o
    // If set (backward calls), the chunk-factor kernel also writes, in fragment
    // order: M^T [64][64], Qhat^T [Dk][64] and T^T [64][64].
    void *ws_Mt, *ws_Qt, *ws_Tt;
    float *ws_Sc32;       // if set (fp32 backward calls), the fp32 propagation stores
                          // every chunk's incoming state here, row-major
                          // [chunk id][head][Dk][Dv]; o may then be NULL
};

// The backward's workspace: the forward's layout without its T, Qhat and M
// slots, the transposed chunk factors M^T, Qhat^T, T^T (io dtype, fragment
// order), then arrays indexed [chunk id][head][...]: every chunk's incoming
// state Sc and the gradient dSc of its outgoing state (bf16 Dk x Dv, laid out
// by sc_index).  The per-chunk kernel's dKhat (bf16 [64][Dk]) goes over
// Qhat^T.
// Element (c, v) of a per-chunk bf16 state (Sc, dSc) of Dk rows: 32-column
// slabs [v / 32][c][v % 32], so that a slab is one contiguous block and a
// row's part of it is 64 contiguous bytes.
__host__ __device__ inline size_t sc_index(int c, int v, int Dk) {
    return ((size_t)(v >> 5) * Dk + c) * 32 + (v & 31);
}

struct BwdLayout {
    WorkspaceLayout fwd;
    size_t off_Mt = 0, off_Qt = 0, off_Tt = 0;
    size_t off_Sc = 0, off_dSc = 0, off_dKh = 0;
    size_t total = 0;
};

bool bwd_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                BwdLayout *out);

// The workspace of a forward whose chunk factors and chunk states a later
// backward reuses (gdn2_chunk_fwd_train, then gdn2_chunk_bwd_saved): the
// forward's layout without T, then the backward's slots as in BwdLayout,
// with dKhat in a slot of its own so that the saved data outlive a backward.
struct TrainLayout {
    WorkspaceLayout fwd;
    size_t off_Mt = 0, off_Qt = 0, off_Tt = 0;
    size_t off_Sc = 0, off_dSc = 0, off_dKh = 0;
    size_t total = 0;
};

bool train_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                  TrainLayout *out);

struct BwdArgs {
    ChunkArgs c;          // forward arguments and chunk factors (c.o unused)
    const void *dout;
    const float *dS_final;
    void *dq, *dk, *dv;
    float *dla, *db, *dw, *dS0;
    bf16_t *Sc, *dSc, *dKh;
};

// The fp32 backward's workspace: the forward's layout including T, then per
// chunk-head slot (all fp32, row-major): the incoming state Sc and the
// gradient dSp of the outgoing state [Dk][Dv]; [64][D] tiles: dU_eff, the
// gathered token rows Qg, Kg, Vg, Bg, Wg, dOg (zero past the chunk), the
// cumulative log-decay G, the midpoint-scaled Ep, Kp, Qp, U_eff and the
// products dQhat, dKhat, dW, dZ, dE, dEp, dQp, dKp; [64][64]: dM, dA.
struct BwdF32Layout {
    WorkspaceLayout fwd;
    size_t off_Sc = 0, off_dSp = 0, off_tiles = 0, off_sq = 0;  // tiles: 20 x [64][D]; sq: 2 x [64][64]
    size_t total = 0;
};

bool bwd_f32_layout(int N, int B, int T, int H, int Dk, int Dv, bool varlen, BwdF32Layout *out);

struct BwdF32Args {
    ChunkArgs c;          // forward arguments and chunk factors (c.o unused, c.ws_T set)
    const void *dout;
    const float *dS_final;
    void *dq, *dk, *dv;
    float *dla, *db, *dw, *dS0;
    float *Sc, *dSp, *dUeff;
    float *Qg, *Kg, *Vg, *Bg, *Wg, *dOg, *G, *Ep, *Kp, *Qp, *Ueff;
    float *dQhat, *dKhat, *dW, *dZ, *dE, *dEp, *dQp, *dKp, *dM, *dA;
};

// Token-mixer layer: the element-wise kernels around the core.
struct LayerArgs {
    const bf16_t *P;      // q | k | v projections [M][ldP], blocks of H*D columns
    long long ldP;
    const float *conv_w, *norm_w;
    bf16_t *q, *k, *v;    // mix_in outputs [M][H*D]
    const bf16_t *o;      // core output [M][H*D]
    const bf16_t *gate;   // output-gate logits [M][ldg] (the first H*D columns used)
    long long ldg;
    bf16_t *z;            // mix_out output [M][H*D]
    const int32_t *cu_seqlens;
    int M, H, T, N, L;
    float norm_eps;
};

// Sliding-window attention forward.
struct SwaArgs {
    const void *q, *k, *v;   // bf16 [tokens][H][D]
    void *o;                 // bf16 [tokens][H][D]
    float *lse;              // [B][H][T] or nullptr
    const int32_t *cu_seqlens;
    const int32_t *blk_start;  // packed calls: [N+1] prefix of H * query blocks per sequence
    int N, B, T, H, window;
    float scale;
    int n_items;             // grid work items (packed calls: an upper bound)
    long long ldq, ldkv;     // elements between consecutive tokens of q, and of k and v
                             // (H*D when contiguous; the layer reads its projections)
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
// Backward (bf16 only): reverse state-gradient pass, then the two per-chunk kernels.
hipError_t launch_chunk_bwd(const BwdArgs &a, int Dk, hipStream_t stream);
// fp32 backward (after the chunk factors with T and the state-storing propagation).
hipError_t launch_chunk_bwd_f32(const BwdF32Args &a, int Dk, hipStream_t stream);
hipError_t launch_swa_fwd(const SwaArgs &a, int D, hipStream_t stream);
hipError_t launch_swa_plan(const int32_t *cu, int N, int T, int H, int32_t *blk_start,
                           hipStream_t stream);
constexpr int kSwaBlockQueries = 128;  // queries per workgroup of the attention kernel
hipError_t launch_layer_mix_in(const LayerArgs &a, int D, hipStream_t stream);
hipError_t launch_layer_mix_out(const LayerArgs &a, int D, hipStream_t stream);
// Row-major C[M][N] = A[M][K] B[N][K]^T in bf16 (fp32 accumulation) by
// hipBLASLt; false if no algorithm fits ws_bytes or the library call fails.
bool gemm_bf16_nt(const bf16_t *A, long long lda, const bf16_t *B, long long ldb, bf16_t *C,
                  long long ldc, int M, int N, int K, void *ws, size_t ws_bytes, hipStream_t stream);

}  // namespace gdn2
