// Token-mixer layer around the core recurrence (forward): the element-wise
// kernels before and after the core, and the projection GEMMs.
//
// The layer follows the iplexlaw digest, section "Procesamiento del token y
// entrenamiento paralelo": q and k take a linear projection, a short causal
// convolution, SiLU and an L2 normalisation; v a projection, the convolution
// and SiLU; the core's output an RMS normalisation, an output gate of its own
// and a projection.  b and w are sigmoids of their own projections (section
// "Decisiones independientes en dos ejes").  Readings where the page is
// silent: the convolution is depthwise over the q, k and v channels with
// taps y_t = sum_j conv_w[c][j] x_{t-L+1+j} (zero before a sequence's first
// token); L2 normalisation per head, x / sqrt(|x|^2 + 1e-6); log alpha =
// logsigmoid(projection + per-channel bias); RMS normalisation per head with
// one weight vector shared by the heads; the output gate is a sigmoid.
//
// Data flow for M tokens (all bf16 in HBM, fp32 arithmetic in registers):
//   P   = x W_in^T                     [M, 7 HD]   (one GEMM), column blocks
//         q | k | v | al | gt | bl | wl (the last four are logits)
//   mix_in:  q, k, v                   [M, HD] each, from P
//   core:    o = the chunk forward with all three gates as logits: log alpha =
//            logsigmoid(al + alpha_bias), b = sigmoid(bl), w = sigmoid(wl),
//            taken in fp32 inside its chunk-factor kernel
//   mix_out: z = rmsnorm(o) * norm_w * sigmoid(gt)   [M, HD]
//   y   = z W_o^T                      [M, D]      (GEMM)
// The GEMMs are plain library GEMMs (hipBLASLt, bf16 in, fp32 accumulate,
// bf16 out).  The element-wise kernels stream HBM with 16-byte accesses:
// mix_in walks strips of consecutive tokens per wave with the convolution
// window in registers, mix_out takes 64/(D/8) (token, head) rows per wave.

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr float kL2Eps = 1e-6f;

constexpr float kLog2e = 1.4426950408889634f;

// 1 / (1 + e^-x) on the hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoidf_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + exp2_hw(-kLog2e * x));
}

__device__ __forceinline__ void load8(const bf16 *p, float (&x)[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
}

__device__ __forceinline__ void store8(bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(x[e]);
    *reinterpret_cast<bf16x8 *>(p) = v;
}

// Sum over the LPV lanes that hold one D-vector (LPV = D / 8, a power of 2).
template <int LPV>
__device__ __forceinline__ float vec_sum(float s) {
#pragma unroll
    for (int o = 1; o < LPV; o <<= 1) s += __shfl_xor(s, o);
    return s;
}

// Sequence bounds of token m: its sequence's first token and the first token
// of the next non-empty sequence.
__device__ __forceinline__ void seq_bounds(const LayerArgs &a, int m, int &start, int &next) {
    if (!a.cu_seqlens) {
        start = (m / a.T) * a.T;
        next = start + a.T;
        return;
    }
    int lo = 0, hi = a.N;  // cu[lo] <= m < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu_seqlens[mid] <= m) lo = mid;
        else hi = mid;
    }
    start = a.cu_seqlens[lo];
    next = a.cu_seqlens[lo + 1];
}

constexpr int kStrip = 32;  // consecutive tokens per wave in layer_mix_in

// One wave walks a strip of kStrip consecutive tokens for VPW of the 3H
// D-vectors of a token (q_0..q_{H-1}, k_0.., v_0..: the column blocks of P in
// order), each lane 8 channels.  The convolution window (the MAXL-1 inputs
// before the current block of four tokens) stays in registers, so every
// projection value is read from HBM once (plus MAXL-1 halo rows per strip).
// Waves are ordered vector-group-fastest so that concurrent waves stream
// neighbouring parts of the same rows.
template <int D, int MAXL>
__global__ __launch_bounds__(256) void layer_mix_in_kernel(LayerArgs a) {
    constexpr int LPV = D / 8, VPW = 64 / LPV;
    const int lane = threadIdx.x & 63;
    const int nvec = 3 * a.H, ngroups = (nvec + VPW - 1) / VPW;
    const long long wg = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int strip = (int)(wg / ngroups), vg = (int)(wg % ngroups);
    const int m0 = strip * kStrip;
    if (m0 >= a.M) return;
    const int m1 = min(m0 + kStrip, a.M);
    const int vi = vg * VPW + lane / LPV;
    if (vi >= nvec) return;  // a D-vector's lanes leave together
    const int grp = vi / a.H, h = vi - grp * a.H;
    const int c0 = 8 * (lane % LPV), HD = a.H * D, col = vi * D + c0;
    bf16 *dst = (grp == 0 ? a.q : grp == 1 ? a.k : a.v) + h * D + c0;
    const bf16 *src = a.P + col;

    // taps: wt[b][e] multiplies the input b tokens before the current one
    // (the loads are independent of the branch on b < L so they issue together;
    // the empty asm keeps the compiler from sinking each into a branch)
    float wt[MAXL][8], hist[MAXL - 1][8];
#pragma unroll
    for (int b = 0; b < MAXL; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) wt[b][e] = a.conv_w[(size_t)(col + e) * a.L + max(a.L - 1 - b, 0)];
#pragma unroll
    for (int b = 0; b < MAXL; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            asm volatile("" : "+v"(wt[b][e]));
            wt[b][e] = b < a.L ? wt[b][e] : 0.0f;
        }

    int start, next;
    seq_bounds(a, m0, start, next);
    // window: hist[j] = x_{mb-1-j} (j < MAXL-1), the inputs before the current
    // block of four tokens inside the same sequence (zero outside it)
#pragma unroll
    for (int j = 0; j + 1 < MAXL; ++j) {
        const int b = j + 1;
        const bool in = b < a.L && m0 - b >= start;
        float x[8];
        load8(src + (size_t)(in ? m0 - b : m0) * a.ldP, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[j][e] = in ? x[e] : 0.0f;
    }

    // four rows per block, the next block's rows in flight during this one's
    // math; rows past the strip repeat its last row
    float xr[4][8], xn[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(src + (size_t)min(m0 + u, m1 - 1) * a.ldP, xr[u]);
    for (int mb = m0; mb < m1; mb += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) load8(src + (size_t)min(mb + 4 + u, m1 - 1) * a.ldP, xn[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int m = mb + u;
            if (m >= m1) break;
            if (m >= next) {  // a new sequence starts at m: earlier inputs read as zero
                seq_bounds(a, m, start, next);
#pragma unroll
                for (int j = 0; j + 1 < MAXL; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) hist[j][e] = 0.0f;
#pragma unroll
                for (int v = 0; v < u; ++v)
#pragma unroll
                    for (int e = 0; e < 8; ++e) xr[v][e] = 0.0f;
            }
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float c = 0.0f;
#pragma unroll
                for (int b = 0; b < MAXL; ++b)
                    c += wt[b][e] * (b <= u ? xr[u - b][e] : hist[b - u - 1][e]);
                acc[e] = c * sigmoidf_fast(c);  // SiLU
            }
            if (grp < 2) {  // q, k: L2 normalisation over the head's D channels
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += acc[e] * acc[e];
                const float r = rsqrtf(vec_sum<LPV>(ss) + kL2Eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] *= r;
            }
            store8(dst + (size_t)m * HD, acc);
        }
        // slide the window past this block (only read if the strip goes on)
#pragma unroll
        for (int j = MAXL - 2; j >= 4; --j)
#pragma unroll
            for (int e = 0; e < 8; ++e) hist[j][e] = hist[j - 4][e];
#pragma unroll
        for (int j = (MAXL - 2 < 3 ? MAXL - 2 : 3); j >= 0; --j)
#pragma unroll
            for (int e = 0; e < 8; ++e) hist[j][e] = xr[3 - j][e];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[u][e] = xn[u][e];
    }
}

// z = o / sqrt(mean(o^2) + eps) * norm_w * sigmoid(gate), one D-vector per
// LPV lanes.
template <int D>
__global__ __launch_bounds__(256) void layer_mix_out_kernel(LayerArgs a) {
    constexpr int LPV = D / 8;
    const int lane = threadIdx.x & 63;
    const long long unit = ((long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * (64 / LPV) +
                           lane / LPV;
    if (unit >= (long long)a.M * a.H) return;
    const int m = (int)(unit / a.H), h = (int)(unit % a.H);
    const int c0 = 8 * (lane % LPV), HD = a.H * D;
    const size_t off = (size_t)m * HD + h * D + c0;
    float o[8], g[8];
    load8(a.o + off, o);
    load8(a.gate + (size_t)m * a.ldg + h * D + c0, g);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += o[e] * o[e];
    const float r = rsqrtf(vec_sum<LPV>(ss) * (1.0f / D) + a.norm_eps);
    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(a.norm_w + c0);
    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(a.norm_w + c0 + 4);
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = o[e] * r * (e < 4 ? w0[e] : w1[e - 4]) * sigmoidf_fast(g[e]);
    store8(a.z + off, z);
}

template <int D>
int blocks_for(const LayerArgs &a, int rows_per_wave) {
    const long long rows = (long long)a.M * a.H;
    const long long waves = (rows + rows_per_wave - 1) / rows_per_wave;
    return (int)((waves + 3) / 4);
}

// ---- hipBLASLt: one handle per device, algorithms cached per shape --------

constexpr int kMaxDevices = 64;

hipblasLtHandle_t lt_handle() {
    static std::mutex mu;
    static hipblasLtHandle_t handles[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> g(mu);
    if (!handles[dev] && hipblasLtCreate(&handles[dev]) != HIPBLAS_STATUS_SUCCESS)
        handles[dev] = nullptr;
    return handles[dev];
}

struct GemmPlan {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    bool ok = false;
};

// key: device, M, N, K, lda, ldb, ldc, workspace cap
typedef std::tuple<int, int, int, int, long long, long long, long long, size_t> GemmKey;

const GemmPlan *gemm_plan(hipblasLtHandle_t h, int M, int N, int K, long long lda, long long ldb,
                          long long ldc, size_t ws_cap) {
    static std::mutex mu;
    static std::map<GemmKey, GemmPlan> plans;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const GemmKey key(dev, M, N, K, lda, ldb, ldc, ws_cap);
    std::lock_guard<std::mutex> g(mu);
    auto it = plans.find(key);
    if (it != plans.end()) return it->second.ok ? &it->second : nullptr;
    GemmPlan &p = plans[key];
    // Row-major C[M][N] = A[M][K] B[N][K]^T is column-major C^T (N x M) =
    // op(B^T-as-stored) x A: matrix "A" of the library call is B (K x N,
    // transposed), matrix "B" is A (K x M).
    const hipblasOperation_t tA = HIPBLAS_OP_T, tB = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
        return nullptr;
    hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &tA, sizeof(tA));
    hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tB, sizeof(tB));
    if (hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, ldb) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, lda) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, M, ldc) != HIPBLAS_STATUS_SUCCESS)
        return nullptr;
    hipblasLtMatmulPreference_t pref;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return nullptr;
    uint64_t cap = ws_cap;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                          sizeof(cap));
    hipblasLtMatmulHeuristicResult_t res[1];
    int got = 0;
    const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.lc, p.lc, pref,
                                                               1, res, &got);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || got < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS)
        return nullptr;
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    p.ok = p.ws <= ws_cap;
    return p.ok ? &p : nullptr;
}

}  // namespace

hipError_t launch_layer_mix_in(const LayerArgs &a, int D, hipStream_t stream) {
    if ((long long)a.M * a.H == 0) return hipSuccess;
    const long long strips = (a.M + kStrip - 1) / kStrip;
    const int vpw = D == 128 ? 4 : 8;
    const long long waves = strips * ((3LL * a.H + vpw - 1) / vpw);
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (D == 128) {
        if (a.L <= 4) hipLaunchKernelGGL((layer_mix_in_kernel<128, 4>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((layer_mix_in_kernel<128, 8>), grid, block, 0, stream, a);
    } else {
        if (a.L <= 4) hipLaunchKernelGGL((layer_mix_in_kernel<64, 4>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((layer_mix_in_kernel<64, 8>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_layer_mix_out(const LayerArgs &a, int D, hipStream_t stream) {
    if ((long long)a.M * a.H == 0) return hipSuccess;
    if (D == 128)
        hipLaunchKernelGGL(layer_mix_out_kernel<128>, dim3(blocks_for<128>(a, 4)), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(layer_mix_out_kernel<64>, dim3(blocks_for<64>(a, 8)), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

bool gemm_bf16_nt(const bf16_t *A, long long lda, const bf16_t *B, long long ldb, bf16_t *C,
                  long long ldc, int M, int N, int K, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (M == 0 || N == 0) return true;
    hipblasLtHandle_t h = lt_handle();
    if (!h) return false;
    const GemmPlan *p = gemm_plan(h, M, N, K, lda, ldb, ldc, ws_bytes);
    if (!p) return false;
    const float one = 1.0f, zero = 0.0f;
    return hipblasLtMatmul(h, p->op, &one, B, p->la, A, p->lb, &zero, C, p->lc, C, p->lc, &p->algo,
                           p->ws ? ws : nullptr, p->ws, stream) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace gdn2
