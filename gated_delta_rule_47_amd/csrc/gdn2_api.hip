// C ABI of libgdn2: argument validation, workspace carving and launches.
// The declarations and their contracts are in include/libgdn2.h.

#include <stdlib.h>
#include <string.h>

#include <climits>
#include <mutex>

#include "gdn2_device.h"
#include "gdn2_internal.h"
#include "libgdn2.h"

using namespace gdn2;

namespace {

constexpr int kAbiVersion = 3;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool debug_sync() {
    static const bool on = [] {
        const char *e = getenv("GDN2_DEBUG_SYNC");
        return e && e[0] == '1';
    }();
    return on;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool supported_dims(int Dk, int Dv) { return Dk == Dv && (Dk == 64 || Dk == 128); }

int finish(hipError_t launch_err, hipStream_t stream) {
    if (launch_err != hipSuccess) return GDN2_ERR_HIP;
    if (debug_sync()) {
        if (hipStreamSynchronize(stream) != hipSuccess) return GDN2_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return GDN2_ERR_HIP;
    }
    return GDN2_OK;
}

}  // namespace

namespace gdn2 {

bool workspace_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                      WorkspaceLayout *out, bool for_bwd) {
    if (N < 0 || B < 0 || T < 0 || H < 0 || !supported_dims(Dk, Dv)) return false;
    const long long nc_seq = (T + kChunk - 1) / kChunk;
    long long max_chunks = varlen ? nc_seq + N : (long long)B * nc_seq;
    if (max_chunks > INT_MAX / 2) return false;
    const size_t chd = (size_t)max_chunks * (size_t)H;  // chunk-heads
    if (H > 0 && chd / (size_t)H != (size_t)max_chunks) return false;
    WorkspaceLayout L;
    L.max_chunks = (int)max_chunks;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.off_W = take(chd * kChunk * Dk * io_bytes);
    // Qhat and M serve the output only: a backward call (no o) has no slots for them.
    L.off_Qh = for_bwd ? kNoSlot : take(chd * kChunk * Dk * io_bytes);
    L.off_KhT = take(chd * Dk * kChunk * io_bytes);
    L.off_M = for_bwd ? kNoSlot : take(chd * kChunk * kChunk * io_bytes);
    L.off_U = take(chd * kChunk * Dv * io_bytes);
    L.off_gl = take(chd * Dk * sizeof(float));
    L.plan_ints = varlen ? (size_t)N + 1 + 3 * (size_t)max_chunks : 0;
    L.off_plan = take(L.plan_ints * sizeof(int32_t));
    L.total = off;
    // T itself is kept only on request (GDN2_STAGE_STORE_T), after everything else.
    L.off_T = for_bwd ? kNoSlot : off;
    L.total_T = for_bwd ? off : align_up(off + chd * kChunk * kChunk * io_bytes);
    *out = L;
    return true;
}

bool bwd_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                BwdLayout *out) {
    BwdLayout L;
    if (!workspace_layout(N, B, T, H, Dk, Dv, io_bytes, varlen, &L.fwd, true)) return false;
    const size_t chd = (size_t)L.fwd.max_chunks * (size_t)H;
    size_t off = align_up(L.fwd.total);
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.off_Mt = take(chd * kChunk * kChunk * io_bytes);
    L.off_Qt = take(chd * Dk * kChunk * io_bytes);
    L.off_Tt = take(chd * kChunk * kChunk * io_bytes);
    L.off_Sc = take(chd * Dk * Dv * 2);
    L.off_dSc = take(chd * Dk * Dv * 2);
    // The per-chunk kernel hands dKhat from its state side to its factor side
    // through the slot of Qhat^T, which only the reverse pass (finished by
    // then) reads; same size (bf16, Dk == Dv).
    L.off_dKh = L.off_Qt;
    L.total = off;
    *out = L;
    return true;
}

bool train_layout(int N, int B, int T, int H, int Dk, int Dv, size_t io_bytes, bool varlen,
                  TrainLayout *out) {
    TrainLayout L;
    if (!workspace_layout(N, B, T, H, Dk, Dv, io_bytes, varlen, &L.fwd)) return false;
    const size_t chd = (size_t)L.fwd.max_chunks * (size_t)H;
    size_t off = align_up(L.fwd.total);  // (the T slot of the forward's layout is not used)
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.off_Mt = take(chd * kChunk * kChunk * io_bytes);
    L.off_Qt = take(chd * Dk * kChunk * io_bytes);
    L.off_Tt = take(chd * kChunk * kChunk * io_bytes);
    L.off_Sc = take(chd * Dk * Dv * 2);
    L.off_dSc = take(chd * Dk * Dv * 2);
    L.off_dKh = take(chd * kChunk * Dk * 2);
    L.total = off;
    *out = L;
    return true;
}

bool bwd_f32_layout(int N, int B, int T, int H, int Dk, int Dv, bool varlen, BwdF32Layout *out) {
    BwdF32Layout L;
    if (!workspace_layout(N, B, T, H, Dk, Dv, sizeof(float), varlen, &L.fwd)) return false;
    const size_t chd = (size_t)L.fwd.max_chunks * (size_t)H;
    size_t off = align_up(L.fwd.total_T);  // after the T slot, which this backward uses
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.off_Sc = take(chd * Dk * Dv * sizeof(float));
    L.off_dSp = take(chd * Dk * Dv * sizeof(float));
    L.off_tiles = take(20 * chd * kChunk * Dk * sizeof(float));
    L.off_sq = take(2 * chd * kChunk * kChunk * sizeof(float));
    L.total = off;
    *out = L;
    return true;
}

}  // namespace gdn2

extern "C" {

int gdn2_abi_version(void) { return kAbiVersion; }

const char *gdn2_status_string(int status) {
    switch (status) {
        case GDN2_OK: return "GDN2_OK";
        case GDN2_ERR_INVALID_ARGUMENT: return "GDN2_ERR_INVALID_ARGUMENT";
        case GDN2_ERR_UNSUPPORTED: return "GDN2_ERR_UNSUPPORTED";
        case GDN2_ERR_WORKSPACE: return "GDN2_ERR_WORKSPACE";
        case GDN2_ERR_HIP: return "GDN2_ERR_HIP";
        default: return "GDN2_ERR_UNKNOWN";
    }
}

int gdn2_device_info(int device, int *compute_units, int *peak_clock_khz) {
    int cus = 0, khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess)
        return GDN2_ERR_HIP;
    if (compute_units) *compute_units = cus;
    if (peak_clock_khz) *peak_clock_khz = khz;
    return GDN2_OK;
}

static size_t io_size(int io) { return io == GDN2_BF16 ? 2 : 4; }

size_t gdn2_chunk_fwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv, int io,
                                      int varlen) {
    if (io != GDN2_F32 && io != GDN2_BF16) return 0;
    WorkspaceLayout L;
    if (!workspace_layout(N, B, T, H, Dk, Dv, io_size(io), varlen != 0, &L)) return 0;
    return L.total;
}

int gdn2_chunk_fwd_workspace_layout(int N, int B, int T, int H, int Dk, int Dv, int io,
                                    int varlen, gdn2_workspace_layout *out) {
    if (!out) return GDN2_ERR_INVALID_ARGUMENT;
    if (io != GDN2_F32 && io != GDN2_BF16) return GDN2_ERR_INVALID_ARGUMENT;
    if (!supported_dims(Dk, Dv)) return GDN2_ERR_UNSUPPORTED;
    WorkspaceLayout L;
    if (!workspace_layout(N, B, T, H, Dk, Dv, io_size(io), varlen != 0, &L))
        return GDN2_ERR_INVALID_ARGUMENT;
    out->total_bytes = L.total;
    out->total_bytes_with_Tinv = L.total_T;
    out->max_chunks = L.max_chunks;
    out->off_Tinv = L.off_T;
    out->off_W = L.off_W;
    out->off_Qhat = L.off_Qh;
    out->off_KhatT = L.off_KhT;
    out->off_M = L.off_M;
    out->off_U = L.off_U;
    out->off_gamma_last = L.off_gl;
    out->off_plan = L.off_plan;
    return GDN2_OK;
}

}  // extern "C"

// The chunk forward; gate_logits selects bf16 gate inputs (log alpha and the
// logits of b and w) instead of fp32 gates.  train: the workspace has the
// TrainLayout, and the forward also keeps there what a later backward reads
// (the transposed factors and every chunk's incoming state).
static int chunk_fwd_impl(const void *q, const void *k, const void *v, const void *log_alpha,
                          const void *b, const void *w, const float *S0, void *o, float *S_final,
                          const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                          int io, void *workspace, size_t workspace_bytes, void *stream_ptr,
                          int stages, bool gate_logits, const float *alpha_bias = nullptr,
                          long long ld_gate = 0, bool train = false) {
    if (stages & ~(GDN2_STAGE_ALL | GDN2_STAGE_STORE_T)) return GDN2_ERR_INVALID_ARGUMENT;
    if (io != GDN2_F32 && io != GDN2_BF16) return GDN2_ERR_INVALID_ARGUMENT;
    if (N < 0 || B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDN2_ERR_INVALID_ARGUMENT;
    if (!supported_dims(Dk, Dv)) return GDN2_ERR_UNSUPPORTED;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? B != 1 : N != B) return GDN2_ERR_INVALID_ARGUMENT;
    if (N == 0 || H == 0) return GDN2_OK;  // nothing to compute
    // Dense sizes must fit the int indexing of the kernels.
    if ((long long)B * T > INT_MAX / 2) return GDN2_ERR_UNSUPPORTED;
    const bool need_tokens = T > 0;
    const void *tok_ptrs[] = {q, k, v, log_alpha, b, w, o};
    for (const void *p : tok_ptrs) {
        if (need_tokens && !p) return GDN2_ERR_INVALID_ARGUMENT;
        if (p && !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final)) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3)))
        return GDN2_ERR_INVALID_ARGUMENT;
    // (an empty call may pass o == NULL together with a NULL S0 or S_final)
    if (o && ((const void *)o == (const void *)S0 || (const void *)o == (const void *)S_final))
        return GDN2_ERR_INVALID_ARGUMENT;

    WorkspaceLayout L;
    TrainLayout TL;
    if (train) {
        if (!train_layout(N, B, T, H, Dk, Dv, io_size(io), varlen, &TL)) return GDN2_ERR_INVALID_ARGUMENT;
        L = TL.fwd;
    } else if (!workspace_layout(N, B, T, H, Dk, Dv, io_size(io), varlen, &L)) {
        return GDN2_ERR_INVALID_ARGUMENT;
    }
    const bool store_T = !train && (stages & GDN2_STAGE_STORE_T) && (stages & GDN2_STAGE_FACTORS);
    const size_t need = train ? TL.total : store_T ? L.total_T : L.total;
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN2_ERR_WORKSPACE;
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
        return GDN2_ERR_WORKSPACE;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();  // a stale error left by other code is not ours to report
    char *ws = static_cast<char *>(workspace);
    ChunkArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = static_cast<const float *>(log_alpha);  // bf16 when gate_logits
    a.b = static_cast<const float *>(b);
    a.w = static_cast<const float *>(w);
    a.gate_logits = gate_logits ? 1 : 0;
    a.ld_gate = ld_gate > 0 ? ld_gate : (long long)H * Dk;
    a.alpha_bias = gate_logits ? alpha_bias : nullptr;
    a.S0 = S0;
    a.o = o;
    a.S_final = S_final;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.B = B;
    a.T = T;
    a.H = H;
    a.NC = (T + kChunk - 1) / kChunk;
    a.max_chunks = L.max_chunks;
    a.plan = varlen ? reinterpret_cast<int32_t *>(ws + L.off_plan) : nullptr;
    a.ws_T = store_T ? ws + L.off_T : nullptr;
    a.ws_W = ws + L.off_W;
    a.ws_Qh = ws + L.off_Qh;
    a.ws_KhT = ws + L.off_KhT;
    a.ws_M = ws + L.off_M;
    a.ws_U = ws + L.off_U;
    a.store_T = store_T ? 1 : 0;
    a.ws_gl = reinterpret_cast<float *>(ws + L.off_gl);
    if (train) {  // both factor sets, and o together with every chunk's incoming state
        a.ws_Mt = ws + TL.off_Mt;
        a.ws_Qt = ws + TL.off_Qt;
        a.ws_Tt = ws + TL.off_Tt;
        a.ws_Sc = reinterpret_cast<bf16_t *>(ws + TL.off_Sc);
    }
    const bool bf = io == GDN2_BF16;

    hipError_t err = hipSuccess;
    if (varlen && (stages & GDN2_STAGE_PLAN)) err = launch_plan(a, stream);
    if (err == hipSuccess && (stages & GDN2_STAGE_FACTORS) && L.max_chunks > 0)
        err = launch_chunk_prep(a, Dk, bf, stream);
    if (err == hipSuccess && (stages & GDN2_STAGE_PROPAGATE) && (S_final || L.max_chunks > 0))
        err = launch_chunk_prop(a, Dk, bf, stream);
    return finish(err, stream);
}

extern "C" {

int gdn2_chunk_fwd_stages(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *b, const float *w, const float *S0, void *o,
                          float *S_final, const int32_t *cu_seqlens, int N, int B, int T, int H,
                          int Dk, int Dv, int io, void *workspace, size_t workspace_bytes,
                          void *stream_ptr, int stages) {
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk, Dv,
                          io, workspace, workspace_bytes, stream_ptr, stages, false);
}

int gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *b, const float *w, const float *S0, void *o, float *S_final,
                   const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk, int Dv, int io,
                   void *workspace, size_t workspace_bytes, void *stream_ptr) {
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk, Dv,
                          io, workspace, workspace_bytes, stream_ptr, GDN2_STAGE_ALL, false);
}

size_t gdn2_chunk_train_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv, int io,
                                        int varlen) {
    if (io != GDN2_BF16) return 0;
    TrainLayout L;
    if (!train_layout(N, B, T, H, Dk, Dv, io_size(io), varlen != 0, &L)) return 0;
    return L.total;
}

int gdn2_chunk_fwd_train(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *b, const float *w, const float *S0, void *o, float *S_final,
                         const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                         int io, void *workspace, size_t workspace_bytes, void *stream_ptr) {
    if (io == GDN2_F32) return GDN2_ERR_UNSUPPORTED;  // (fp32 I/O backs the reference path only)
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk, Dv,
                          io, workspace, workspace_bytes, stream_ptr, GDN2_STAGE_ALL, false, nullptr,
                          0, true);
}

}  // extern "C"

// ---- the chunk forward for callers that cannot allocate ------------------------

// Device memory of gdn2_chunk_fwd_noalloc: the chunk forward's intermediates,
// laid out as in a caller's workspace.  Each GPU holds its own copy from the
// library's first use of it until the process ends; every call on a GPU uses
// that copy, so calls that overlap on one GPU race.  In host code `scratch`
// names a host-side stand-in: only the address scratch_address() returns may
// reach a kernel.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

int gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *b, const float *w, const float *S0, void *o,
                           float *S_final, const int32_t *cu_seqlens, int N, int B, int T, int H,
                           int Dk, int Dv, int io, void *stream_ptr) {
    // A call whose intermediates do not fit the scratch is rejected first; a
    // call with invalid sizes gets its error from the common validation.
    void *ws = nullptr;
    size_t ws_bytes = 0;
    WorkspaceLayout L;
    if ((io == GDN2_F32 || io == GDN2_BF16) && N > 0 && H > 0 &&
        workspace_layout(N, B, T, H, Dk, Dv, io_size(io), cu_seqlens != nullptr, &L) &&
        L.total > 0) {
        if (L.total > kScratchBytes) return GDN2_ERR_WORKSPACE;
        ws = scratch_address();
        if (!ws) return GDN2_ERR_HIP;
        ws_bytes = kScratchBytes;
    }
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk, Dv,
                          io, ws, ws_bytes, stream_ptr, GDN2_STAGE_ALL, false);
}

int gdn2_chunk_fwd_gate_logits(const void *q, const void *k, const void *v,
                               const void *log_alpha, const void *b_logit, const void *w_logit,
                               const float *S0, void *o, float *S_final,
                               const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk,
                               int Dv, int io, void *workspace, size_t workspace_bytes,
                               void *stream_ptr) {
    if (io != GDN2_F32 && io != GDN2_BF16) return GDN2_ERR_INVALID_ARGUMENT;
    if (io != GDN2_BF16) return GDN2_ERR_UNSUPPORTED;
    return chunk_fwd_impl(q, k, v, log_alpha, b_logit, w_logit, S0, o, S_final, cu_seqlens, N, B,
                          T, H, Dk, Dv, io, workspace, workspace_bytes, stream_ptr, GDN2_STAGE_ALL,
                          true);
}

}  // extern "C"

// The fp32 backward (arguments already validated by gdn2_chunk_bwd): the chunk
// factors with T, the propagation storing every chunk's incoming state, then
// the fp32 reverse pass and per-chunk products.
static int chunk_bwd_f32(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *b, const float *w, const float *S0, const void *dout,
                         const float *dS_final, void *dq, void *dk, void *dv, float *dlog_alpha,
                         float *db, float *dw, float *dS0, const int32_t *cu_seqlens, int N, int B,
                         int T, int H, int Dk, int Dv, void *workspace, size_t workspace_bytes,
                         void *stream_ptr) {
    const bool varlen = cu_seqlens != nullptr;
    BwdF32Layout L;
    if (!bwd_f32_layout(N, B, T, H, Dk, Dv, varlen, &L)) return GDN2_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < L.total) return GDN2_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) return GDN2_ERR_WORKSPACE;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();  // a stale error left by other code is not ours to report
    char *ws = static_cast<char *>(workspace);
    const WorkspaceLayout &F = L.fwd;
    BwdF32Args f{};
    ChunkArgs &a = f.c;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.b = b;
    a.w = w;
    a.S0 = S0;
    a.o = nullptr;
    a.S_final = nullptr;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.B = B;
    a.T = T;
    a.H = H;
    a.NC = (T + kChunk - 1) / kChunk;
    a.max_chunks = F.max_chunks;
    a.plan = varlen ? reinterpret_cast<int32_t *>(ws + F.off_plan) : nullptr;
    a.ws_T = ws + F.off_T;
    a.store_T = 1;
    a.ws_W = ws + F.off_W;
    a.ws_Qh = ws + F.off_Qh;
    a.ws_KhT = ws + F.off_KhT;
    a.ws_M = ws + F.off_M;
    a.ws_U = ws + F.off_U;
    a.ws_gl = reinterpret_cast<float *>(ws + F.off_gl);
    a.ws_Sc32 = reinterpret_cast<float *>(ws + L.off_Sc);
    f.dout = dout;
    f.dS_final = dS_final;
    f.dq = dq;
    f.dk = dk;
    f.dv = dv;
    f.dla = dlog_alpha;
    f.db = db;
    f.dw = dw;
    f.dS0 = dS0;
    f.Sc = a.ws_Sc32;
    f.dSp = reinterpret_cast<float *>(ws + L.off_dSp);
    const size_t tile = (size_t)F.max_chunks * H * kChunk * Dk;  // floats per [64][D] array
    float *t = reinterpret_cast<float *>(ws + L.off_tiles);
    float **tiles[] = {&f.dUeff, &f.Qg, &f.Kg, &f.Vg, &f.Bg, &f.Wg, &f.dOg, &f.G, &f.Ep, &f.Kp,
                       &f.Qp, &f.Ueff, &f.dQhat, &f.dKhat, &f.dW, &f.dZ, &f.dE, &f.dEp, &f.dQp, &f.dKp};
    static_assert(sizeof(tiles) / sizeof(tiles[0]) == 20, "20 tile arrays");
    for (int i = 0; i < 20; ++i) *tiles[i] = t + i * tile;
    f.dM = reinterpret_cast<float *>(ws + L.off_sq);
    f.dA = f.dM + (size_t)F.max_chunks * H * kChunk * kChunk;

    hipError_t err = hipSuccess;
    if (varlen) err = launch_plan(a, stream);
    if (err == hipSuccess && F.max_chunks > 0) err = launch_chunk_prep(a, Dk, false, stream);
    if (err == hipSuccess) err = launch_chunk_prop(a, Dk, false, stream);
    if (err == hipSuccess) err = launch_chunk_bwd_f32(f, Dk, stream);
    return finish(err, stream);
}

// Argument checks shared by the backward entry points (S0 may be NULL);
// *empty is set when the call has nothing to compute.
static int check_bwd_args(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *b, const float *w, const float *S0, const void *dout,
                          const float *dS_final, void *dq, void *dk, void *dv, float *dlog_alpha,
                          float *db, float *dw, float *dS0, const int32_t *cu_seqlens, int N, int B,
                          int T, int H, int Dk, int Dv, int io, bool *empty) {
    *empty = false;
    if (io != GDN2_F32 && io != GDN2_BF16) return GDN2_ERR_INVALID_ARGUMENT;
    if (N < 0 || B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDN2_ERR_INVALID_ARGUMENT;
    if (!supported_dims(Dk, Dv)) return GDN2_ERR_UNSUPPORTED;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? B != 1 : N != B) return GDN2_ERR_INVALID_ARGUMENT;
    if (N == 0 || H == 0) {
        *empty = true;
        return GDN2_OK;
    }
    if ((long long)B * T > INT_MAX / 2) return GDN2_ERR_UNSUPPORTED;
    const void *ins[] = {q, k, v, log_alpha, b, w, dout};
    const void *outs[] = {dq, dk, dv, dlog_alpha, db, dw};
    for (const void *p : ins) {
        if (T > 0 && !p) return GDN2_ERR_INVALID_ARGUMENT;
        if (p && !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    }
    for (const void *p : outs) {
        if (T > 0 && !p) return GDN2_ERR_INVALID_ARGUMENT;
        if (p && !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    }
    if ((S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3)))
        return GDN2_ERR_INVALID_ARGUMENT;
    // Outputs must be distinct from each other and from every input.
    const void *all_out[] = {dq, dk, dv, dlog_alpha, db, dw, dS0};
    const void *all_in[] = {q, k, v, log_alpha, b, w, dout, S0, dS_final, cu_seqlens};
    for (int i = 0; i < 7; ++i) {
        if (!all_out[i]) continue;
        for (int j = i + 1; j < 7; ++j)
            if (all_out[i] == all_out[j]) return GDN2_ERR_INVALID_ARGUMENT;
        for (const void *p : all_in)
            if (all_out[i] == p) return GDN2_ERR_INVALID_ARGUMENT;
    }
    return GDN2_OK;
}

// Byte offsets of the backward's own slots in a workspace.
struct BwdSlots {
    size_t Mt, Qt, Tt, Sc, dSc, dKh;
};

// The bf16 backward on a checked call.  recompute: first rebuild the chunk
// table, the chunk factors (with their transposes) and every chunk's incoming
// state; otherwise they are read as a training forward left them.
static int chunk_bwd_bf16(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *b, const float *w, const float *S0, const void *dout,
                          const float *dS_final, void *dq, void *dk, void *dv, float *dlog_alpha,
                          float *db, float *dw, float *dS0, const int32_t *cu_seqlens, int N, int B,
                          int T, int H, int Dk, const WorkspaceLayout &F, const BwdSlots &sl, char *ws,
                          bool recompute, void *stream_ptr) {
    const bool varlen = cu_seqlens != nullptr;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();  // a stale error left by other code is not ours to report
    BwdArgs ba{};
    ChunkArgs &a = ba.c;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.b = b;
    a.w = w;
    a.S0 = S0;
    a.o = nullptr;
    a.S_final = nullptr;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.B = B;
    a.T = T;
    a.H = H;
    a.NC = (T + kChunk - 1) / kChunk;
    a.max_chunks = F.max_chunks;
    a.plan = varlen ? reinterpret_cast<int32_t *>(ws + F.off_plan) : nullptr;
    a.ws_T = nullptr;  // the backward kernels read neither T, Qhat nor M
    a.ws_W = ws + F.off_W;
    a.ws_Qh = nullptr;
    a.ws_KhT = ws + F.off_KhT;
    a.ws_M = nullptr;
    a.ws_U = ws + F.off_U;
    a.ws_gl = reinterpret_cast<float *>(ws + F.off_gl);
    a.store_T = 0;  // the backward kernels read T^T (ws_Tt) only
    a.ws_Sc = reinterpret_cast<bf16_t *>(ws + sl.Sc);
    a.ws_Mt = ws + sl.Mt;
    a.ws_Qt = ws + sl.Qt;
    a.ws_Tt = ws + sl.Tt;
    ba.dout = dout;
    ba.dS_final = dS_final;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dla = dlog_alpha;
    ba.db = db;
    ba.dw = dw;
    ba.dS0 = dS0;
    ba.Sc = a.ws_Sc;
    ba.dSc = reinterpret_cast<bf16_t *>(ws + sl.dSc);
    ba.dKh = reinterpret_cast<bf16_t *>(ws + sl.dKh);

    hipError_t err = hipSuccess;
    if (recompute) {
        if (varlen) err = launch_plan(a, stream);
        if (err == hipSuccess && F.max_chunks > 0) err = launch_chunk_prep(a, Dk, true, stream);
        if (err == hipSuccess && F.max_chunks > 0) err = launch_chunk_prop(a, Dk, true, stream);
    }
    if (err == hipSuccess) err = launch_chunk_bwd(ba, Dk, stream);
    return finish(err, stream);
}

extern "C" {

size_t gdn2_chunk_bwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv, int io,
                                      int varlen) {
    if (io != GDN2_F32 && io != GDN2_BF16) return 0;
    if (io == GDN2_F32) {
        BwdF32Layout L32;
        return bwd_f32_layout(N, B, T, H, Dk, Dv, varlen != 0, &L32) ? L32.total : 0;
    }
    BwdLayout L;
    if (!bwd_layout(N, B, T, H, Dk, Dv, io_size(io), varlen != 0, &L)) return 0;
    return L.total;
}

int gdn2_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *b, const float *w, const float *S0, const void *dout,
                   const float *dS_final, void *dq, void *dk, void *dv, float *dlog_alpha,
                   float *db, float *dw, float *dS0, const int32_t *cu_seqlens, int N, int B, int T,
                   int H, int Dk, int Dv, int io, void *workspace, size_t workspace_bytes,
                   void *stream_ptr) {
    bool empty = false;
    const int st = check_bwd_args(q, k, v, log_alpha, b, w, S0, dout, dS_final, dq, dk, dv,
                                  dlog_alpha, db, dw, dS0, cu_seqlens, N, B, T, H, Dk, Dv, io, &empty);
    if (st != GDN2_OK || empty) return st;
    const bool varlen = cu_seqlens != nullptr;
    if (io == GDN2_F32)
        return chunk_bwd_f32(q, k, v, log_alpha, b, w, S0, dout, dS_final, dq, dk, dv, dlog_alpha,
                             db, dw, dS0, cu_seqlens, N, B, T, H, Dk, Dv, workspace,
                             workspace_bytes, stream_ptr);
    BwdLayout L;
    if (!bwd_layout(N, B, T, H, Dk, Dv, io_size(io), varlen, &L)) return GDN2_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < L.total) return GDN2_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) return GDN2_ERR_WORKSPACE;
    const BwdSlots sl{L.off_Mt, L.off_Qt, L.off_Tt, L.off_Sc, L.off_dSc, L.off_dKh};
    return chunk_bwd_bf16(q, k, v, log_alpha, b, w, S0, dout, dS_final, dq, dk, dv, dlog_alpha, db,
                          dw, dS0, cu_seqlens, N, B, T, H, Dk, L.fwd, sl, static_cast<char *>(workspace),
                          true, stream_ptr);
}

int gdn2_chunk_bwd_saved(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *b, const float *w, const void *dout, const float *dS_final,
                         void *dq, void *dk, void *dv, float *dlog_alpha, float *db, float *dw,
                         float *dS0, const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk,
                         int Dv, int io, void *workspace, size_t workspace_bytes, void *stream_ptr) {
    bool empty = false;
    const int st = check_bwd_args(q, k, v, log_alpha, b, w, nullptr, dout, dS_final, dq, dk, dv,
                                  dlog_alpha, db, dw, dS0, cu_seqlens, N, B, T, H, Dk, Dv, io, &empty);
    if (st != GDN2_OK || empty) return st;
    if (io != GDN2_BF16) return GDN2_ERR_UNSUPPORTED;
    TrainLayout L;
    if (!train_layout(N, B, T, H, Dk, Dv, io_size(io), cu_seqlens != nullptr, &L))
        return GDN2_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < L.total) return GDN2_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) return GDN2_ERR_WORKSPACE;
    const BwdSlots sl{L.off_Mt, L.off_Qt, L.off_Tt, L.off_Sc, L.off_dSc, L.off_dKh};
    return chunk_bwd_bf16(q, k, v, log_alpha, b, w, nullptr, dout, dS_final, dq, dk, dv, dlog_alpha,
                          db, dw, dS0, cu_seqlens, N, B, T, H, Dk, L.fwd, sl,
                          static_cast<char *>(workspace), false, stream_ptr);
}

int gdn2_step(const void *q, const void *k, const void *v, const float *log_alpha, const float *b,
              const float *w, float *S, void *o, int B, int H, int Dk, int Dv, int io,
              void *stream_ptr) {
    if (io != GDN2_F32 && io != GDN2_BF16) return GDN2_ERR_INVALID_ARGUMENT;
    if (B < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDN2_ERR_INVALID_ARGUMENT;
    if (!supported_dims(Dk, Dv)) return GDN2_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return GDN2_OK;
    if ((long long)B * H > INT_MAX) return GDN2_ERR_UNSUPPORTED;
    const void *ptrs[] = {q, k, v, log_alpha, b, w, S, o};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    if ((const void *)o == (const void *)S) return GDN2_ERR_INVALID_ARGUMENT;
    StepArgs a{q, k, v, log_alpha, b, w, S, o, B, H};
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();  // a stale error left by other code is not ours to report
    return finish(launch_step(a, Dk, io == GDN2_BF16, stream), stream);
}

}  // extern "C"

// ---- token-mixer layer -----------------------------------------------------

namespace {

constexpr size_t kLayerGemmWs = 32u << 20;  // hipBLASLt workspace cap

struct LayerLayout {
    size_t off_P = 0, off_q = 0, off_k = 0, off_v = 0, off_o = 0, off_gemm = 0, off_core = 0,
           core_bytes = 0, total = 0;
};

bool layer_layout(int N, int B, int T, int H, int Dk, int Dv, int D, bool varlen, LayerLayout *out) {
    if (N < 0 || B < 0 || T < 0 || H < 0 || D <= 0 || (D & 7) || !supported_dims(Dk, Dv))
        return false;
    if (varlen ? B != 1 : N != B) return false;
    const long long M = (long long)B * T;
    if (M > INT_MAX / 2) return false;
    const size_t hd = (size_t)H * Dk, row = hd * sizeof(bf16_t);
    LayerLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    // all seven projections x W_in^T as one [M][7 H Dk] array, row blocks
    // q | k | v | alpha | output gate | b | w
    L.off_P = take((size_t)M * 7 * row);
    L.off_q = take((size_t)M * row);
    L.off_k = take((size_t)M * row);
    L.off_v = take((size_t)M * row);
    L.off_o = take((size_t)M * row);
    L.off_gemm = take(kLayerGemmWs);
    WorkspaceLayout C;
    if (!workspace_layout(N, B, T, H, Dk, Dv, 2, varlen, &C)) return false;
    L.core_bytes = C.total;
    L.off_core = take(C.total);
    L.total = off;
    *out = L;
    return true;
}

}  // namespace

extern "C" {

size_t gdn2_layer_fwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv, int D,
                                      int varlen) {
    LayerLayout L;
    return layer_layout(N, B, T, H, Dk, Dv, D, varlen != 0, &L) ? L.total : 0;
}

int gdn2_layer_fwd(const void *x, const gdn2_layer_weights *wt, int conv_len, float norm_eps,
                   const float *S0, void *y, float *S_final, const int32_t *cu_seqlens, int N,
                   int B, int T, int H, int Dk, int Dv, int D, void *workspace,
                   size_t workspace_bytes, void *stream_ptr) {
    if (N < 0 || B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0 || D <= 0)
        return GDN2_ERR_INVALID_ARGUMENT;
    if (!supported_dims(Dk, Dv) || (D & 7)) return GDN2_ERR_UNSUPPORTED;
    if (conv_len < 1 || conv_len > 8 || !(norm_eps >= 0.0f) || norm_eps > 3.0e38f || !wt)
        return GDN2_ERR_INVALID_ARGUMENT;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? B != 1 : N != B) return GDN2_ERR_INVALID_ARGUMENT;
    if (N == 0 || H == 0) return GDN2_OK;
    const long long M = (long long)B * T;
    if (M > INT_MAX / 2) return GDN2_ERR_UNSUPPORTED;
    const void *ptrs[] = {wt->W_in, wt->conv_w, wt->alpha_bias, wt->norm_w, wt->W_o};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!x || !y)) return GDN2_ERR_INVALID_ARGUMENT;
    if ((x && !aligned16(x)) || (y && !aligned16(y)) || (S0 && !aligned16(S0)) ||
        (S_final && !aligned16(S_final)) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3)))
        return GDN2_ERR_INVALID_ARGUMENT;
    if (y && (y == x || y == wt->W_in || y == wt->W_o || y == (const void *)S0 ||
              y == (void *)S_final))
        return GDN2_ERR_INVALID_ARGUMENT;

    LayerLayout L;
    if (!layer_layout(N, B, T, H, Dk, Dv, D, varlen, &L)) return GDN2_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < L.total) return GDN2_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) return GDN2_ERR_WORKSPACE;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    const int HD = H * Dk, m = (int)M;
    const bf16_t *X = static_cast<const bf16_t *>(x);
    const bf16_t *Win = static_cast<const bf16_t *>(wt->W_in);
    bf16_t *P = reinterpret_cast<bf16_t *>(ws + L.off_P);
    const long long ld7 = 7LL * HD;  // the gate logits are column blocks 3..6 of P
    const bf16_t *al = P + 3LL * HD, *gt = P + 4LL * HD, *bl = P + 5LL * HD, *wl = P + 6LL * HD;
    void *gws = ws + L.off_gemm;

    LayerArgs a{};
    a.P = P;
    a.ldP = ld7;
    a.conv_w = wt->conv_w;
    a.norm_w = wt->norm_w;
    a.q = reinterpret_cast<bf16_t *>(ws + L.off_q);
    a.k = reinterpret_cast<bf16_t *>(ws + L.off_k);
    a.v = reinterpret_cast<bf16_t *>(ws + L.off_v);
    a.o = reinterpret_cast<bf16_t *>(ws + L.off_o);
    a.gate = gt;
    a.ldg = ld7;
    a.z = a.q;  // q is dead once the core has run
    a.cu_seqlens = cu_seqlens;
    a.M = m;
    a.H = H;
    a.T = T;
    a.N = N;
    a.L = conv_len;
    a.norm_eps = norm_eps;

    if (m > 0) {
        // one GEMM for all seven projections: q | k | v feed the convolution
        // kernel, alpha, b and w go to the core as logits, the gate to the output
        if (!gemm_bf16_nt(X, D, Win, D, P, ld7, m, 7 * HD, D, gws, kLayerGemmWs, stream))
            return GDN2_ERR_HIP;
        if (launch_layer_mix_in(a, Dk, stream) != hipSuccess) return GDN2_ERR_HIP;
    }
    const int st = chunk_fwd_impl(a.q, a.k, a.v, al, bl, wl, S0, ws + L.off_o, S_final, cu_seqlens,
                                  N, B, T, H, Dk, Dv, GDN2_BF16, ws + L.off_core, L.core_bytes,
                                  stream_ptr, GDN2_STAGE_ALL, true, wt->alpha_bias, ld7);
    if (st != GDN2_OK) return st;
    if (m > 0) {
        if (launch_layer_mix_out(a, Dk, stream) != hipSuccess) return GDN2_ERR_HIP;
        if (!gemm_bf16_nt(a.z, HD, static_cast<const bf16_t *>(wt->W_o), HD,
                          static_cast<bf16_t *>(y), D, m, D, HD, gws, kLayerGemmWs, stream))
            return GDN2_ERR_HIP;
    }
    return finish(hipSuccess, stream);
}

}  // extern "C"

// ---- sliding-window attention ------------------------------------------------

namespace {

// q rows are ldq elements apart, k and v rows ldkv apart (H*D when contiguous).
int swa_fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse,
                 const int32_t *cu_seqlens, int N, int B, int T, int H, int D, int window,
                 float scale, long long ldq, long long ldkv, void *workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    const bool varlen = cu_seqlens != nullptr;
    const size_t need = varlen ? align_up((size_t)(N + 1) * sizeof(int32_t)) : 0;
    if (need && (!workspace || workspace_bytes < need)) return GDN2_ERR_WORKSPACE;
    if (need && (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) return GDN2_ERR_WORKSPACE;
    const long long nb = (T + kSwaBlockQueries - 1) / kSwaBlockQueries;
    const long long items = varlen ? (long long)H * (nb + N) : (long long)B * H * nb;
    if (items > INT_MAX / 2) return GDN2_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    SwaArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.cu_seqlens = cu_seqlens;
    a.blk_start = varlen ? static_cast<const int32_t *>(workspace) : nullptr;
    a.N = N;
    a.B = B;
    a.T = T;
    a.H = H;
    a.window = window;
    a.scale = scale;
    a.n_items = (int)items;
    a.ldq = ldq;
    a.ldkv = ldkv;
    hipError_t err = hipSuccess;
    if (varlen) err = launch_swa_plan(cu_seqlens, N, T, H, static_cast<int32_t *>(workspace), stream);
    if (err == hipSuccess) err = launch_swa_fwd(a, D, stream);
    return finish(err, stream);
}

bool swa_common_args_ok(int N, int B, int T, int H, int D, int window, float scale,
                        const int32_t *cu_seqlens, int *status) {
    *status = GDN2_OK;
    if (N < 0 || B < 0 || T < 0 || H < 0 || D <= 0) *status = GDN2_ERR_INVALID_ARGUMENT;
    else if (D != 64 && D != 128) *status = GDN2_ERR_UNSUPPORTED;
    else if (window < 1 || !(scale > 0.0f) || scale > 3.0e38f) *status = GDN2_ERR_INVALID_ARGUMENT;
    else if (cu_seqlens ? B != 1 : N != B) *status = GDN2_ERR_INVALID_ARGUMENT;
    else if ((long long)B * T > INT_MAX / 2) *status = GDN2_ERR_UNSUPPORTED;
    else if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3)) *status = GDN2_ERR_INVALID_ARGUMENT;
    return *status == GDN2_OK;
}

}  // namespace

extern "C" {

size_t gdn2_swa_fwd_workspace_bytes(int N, int varlen) {
    if (N < 0) return 0;
    return varlen ? align_up((size_t)(N + 1) * sizeof(int32_t)) : 0;
}

int gdn2_swa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 const int32_t *cu_seqlens, int N, int B, int T, int H, int D, int window,
                 float scale, void *workspace, size_t workspace_bytes, void *stream_ptr) {
    int st;
    if (!swa_common_args_ok(N, B, T, H, D, window, scale, cu_seqlens, &st)) return st;
    if (N == 0 || H == 0 || T == 0) return GDN2_OK;
    const void *ptrs[] = {q, k, v, o};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return GDN2_ERR_INVALID_ARGUMENT;
    if (o == q || o == k || o == v || (const void *)o == (const void *)lse)
        return GDN2_ERR_INVALID_ARGUMENT;
    return swa_fwd_impl(q, k, v, o, lse, cu_seqlens, N, B, T, H, D, window, scale,
                        (long long)H * D, (long long)H * D, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream_ptr));
}

}  // extern "C"

// ---- sliding-window attention layer --------------------------------------------

namespace {

struct SwaLayerLayout {
    size_t off_P = 0, off_O = 0, off_gemm = 0, off_plan = 0, plan_bytes = 0, total = 0;
};

bool swa_layer_layout(int N, int B, int T, int H, int D, int Dm, bool varlen, SwaLayerLayout *out) {
    if (N < 0 || B < 0 || T < 0 || H < 0 || Dm <= 0 || (Dm & 7) || (D != 64 && D != 128))
        return false;
    if (varlen ? B != 1 : N != B) return false;
    const long long M = (long long)B * T;
    if (M > INT_MAX / 2) return false;
    const size_t row = (size_t)H * D * sizeof(bf16_t);
    SwaLayerLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L.off_P = take((size_t)M * 3 * row);
    L.off_O = take((size_t)M * row);
    L.off_gemm = take(kLayerGemmWs);
    L.plan_bytes = varlen ? align_up((size_t)(N + 1) * sizeof(int32_t)) : 0;
    L.off_plan = take(L.plan_bytes);
    L.total = off;
    *out = L;
    return true;
}

}  // namespace

extern "C" {

size_t gdn2_swa_layer_fwd_workspace_bytes(int N, int B, int T, int H, int D, int Dm, int varlen) {
    SwaLayerLayout L;
    return swa_layer_layout(N, B, T, H, D, Dm, varlen != 0, &L) ? L.total : 0;
}

int gdn2_swa_layer_fwd(const void *x, const void *W_qkv, const void *W_o, void *y, float *lse,
                       const int32_t *cu_seqlens, int N, int B, int T, int H, int D, int Dm,
                       int window, float scale, void *workspace, size_t workspace_bytes,
                       void *stream_ptr) {
    int st;
    if (!swa_common_args_ok(N, B, T, H, D, window, scale, cu_seqlens, &st)) return st;
    if (Dm <= 0) return GDN2_ERR_INVALID_ARGUMENT;
    if (Dm & 7) return GDN2_ERR_UNSUPPORTED;
    if (N == 0 || H == 0 || T == 0) return GDN2_OK;
    const void *ptrs[] = {x, W_qkv, W_o, y};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return GDN2_ERR_INVALID_ARGUMENT;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return GDN2_ERR_INVALID_ARGUMENT;
    if (y == x || y == W_qkv || y == W_o || (const void *)y == (const void *)lse)
        return GDN2_ERR_INVALID_ARGUMENT;
    SwaLayerLayout L;
    if (!swa_layer_layout(N, B, T, H, D, Dm, cu_seqlens != nullptr, &L))
        return GDN2_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < L.total) return GDN2_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) return GDN2_ERR_WORKSPACE;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    const int HD = H * D, m = B * T;
    bf16_t *P = reinterpret_cast<bf16_t *>(ws + L.off_P);
    bf16_t *O = reinterpret_cast<bf16_t *>(ws + L.off_O);
    void *gws = ws + L.off_gemm;
    // q | k | v in one GEMM; the attention reads them as strided rows
    if (!gemm_bf16_nt(static_cast<const bf16_t *>(x), Dm, static_cast<const bf16_t *>(W_qkv), Dm, P,
                      3LL * HD, m, 3 * HD, Dm, gws, kLayerGemmWs, stream))
        return GDN2_ERR_HIP;
    st = swa_fwd_impl(P, P + HD, P + 2 * HD, O, lse, cu_seqlens, N, B, T, H, D, window, scale,
                      3LL * HD, 3LL * HD, ws + L.off_plan, L.plan_bytes, stream);
    if (st != GDN2_OK) return st;
    if (!gemm_bf16_nt(O, HD, static_cast<const bf16_t *>(W_o), HD, static_cast<bf16_t *>(y), Dm, m,
                      Dm, HD, gws, kLayerGemmWs, stream))
        return GDN2_ERR_HIP;
    return finish(hipSuccess, stream);
}

}  // extern "C"
