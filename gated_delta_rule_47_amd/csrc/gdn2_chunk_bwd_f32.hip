// Chunkwise backward with fp32 I/O: the same chain rule as the bf16 backward
// (gdn2_chunk_bwd.hip; the gate-aware backward the gist.science summary names
// in part "3. Efficient chunkwise parallel training"), with every product an
// fp32 MFMA (16x16x4) and every intermediate in fp32, so that it agrees with
// the fp64 definition to fp32 rounding.  It is the precision reference of the
// backward rather than its fast path: the per-chunk products are batched GEMMs
// over all chunk-heads, each launch reading its operands where they lie.
//
// Per chunk (incoming state S, gradient dS' of the outgoing state, output
// gradient dO; T = (I + A)^-1, W = T E, U = T Z, E = gamma*b*k, Z = w*v, and the
// midpoint-scaled tiles Ep = b k e^{g-g_r}, Kp = k e^{g_r-g}, Qp = q e^{g-g_r}
// with A = strict_tril(Ep Kp^T), M = tril(Qp Kp^T)):
//   reverse pass  dU_eff = M^T dO + Khat dS',  dS = Diag(gl) dS' + Qhat^T dO - W^T dU_eff
//   state side    U_eff = U - W S,  dQhat = dO S^T,  dM = tril(dO U_eff^T),
//                 dKhat = U_eff dS'^T,  dW = -dU_eff S^T,  dZ = T^T dU_eff,
//                 dgl = rowsum(dS' * S)
//   factor side   dE = T^T dW,  dA = -strict_tril(dZ U^T + dE W^T),
//                 dEp = dA Kp,  dQp = dM Kp,  dKp = dA^T Ep + dM^T Qp
//   per token     dq = gamma dQhat + ex dQp,  db = k (gamma dE + ex dEp),
//                 dk = b (gamma dE + ex dEp) + ei dKp + eK dKhat,
//                 dv = w dZ,  dw = v dZ,
//                 dg = E dE + Ep dEp + Qhat dQhat + Qp dQp - Kp dKp - Khat dKhat,
//                 dlog_alpha_j = sum_{i>=j} dg_i + gl dgl + sum_i Khat_i dKhat_i
// (ex = e^{g-g_r}, ei = e^{g_r-g}, eK = e^{g_last-g}, gamma = e^g, g the
// within-chunk cumulative log-decay, g_r = g_last / 2).

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

// ---------------------------------------------------------------------------
// Operand views: element (r, c) of batch entry b of a matrix that lies in the
// workspace either row-major, in the chunk factors' fp32 fragment order, or in
// U's accumulator order.
// ---------------------------------------------------------------------------
enum : int { kRowMajor = 0, kFragOrder = 1, kAccOrder = 2 };

struct View {
    const float *p = nullptr;  // entry 0
    long long bs = 0;          // elements between batch entries
    int ld = 0;                // row pitch (row-major), or the stored column count
    int layout = kRowMajor;
    int trans = 0;             // logical (r, c) reads stored (c, r)
    int tri = 0;               // on stored (r, c): 1 keeps c <= r, 2 keeps c < r, else 0
};

View rm(const float *p, long long bs, int ld, int trans = 0) {
    View v;
    v.p = p;
    v.bs = bs;
    v.ld = ld;
    v.trans = trans;
    return v;
}

View frag(const void *p, long long bs, int K, int trans = 0, int tri = 0) {
    View v;
    v.p = static_cast<const float *>(p);
    v.bs = bs;
    v.ld = K;
    v.layout = kFragOrder;
    v.trans = trans;
    v.tri = tri;
    return v;
}

__device__ __forceinline__ float view_at(const View &v, long long b, int r, int c) {
    const int rr = v.trans ? c : r, cc = v.trans ? r : c;
    if ((v.tri == 1 && cc > rr) || (v.tri == 2 && cc >= rr)) return 0.0f;
    const float *p = v.p + b * v.bs;
    if (v.layout == kRowMajor) return p[(size_t)rr * v.ld + cc];
    if (v.layout == kFragOrder) return p[frag_index<float>(rr, cc, v.ld)];
    // accumulator order of a 64 x ld matrix: [I][cb][lane][r] holds
    // X[16 I + 4 (lane / 16) + r][16 cb + lane % 16]
    const int lane = 16 * ((rr & 15) >> 2) + (cc & 15);
    return p[((((size_t)(rr >> 4) * (v.ld / 16) + (cc >> 4)) * 64) + lane) * 4 + (rr & 3)];
}

// C(m, n) = alpha sum_k A(m, k) B(k, n) + beta Cin(m, n), row-major fp32
// output [batch][M][ldc]; tri_out 1 keeps n <= m, 2 keeps n < m (others 0).
struct Gemm {
    View A, B, Cin;
    float alpha = 1.0f, beta = 0.0f;
    float *C = nullptr;
    long long cbs = 0;
    int ldc = 0;
    int M = 0, N = 0, K = 0, tri_out = 0;
    int batch = 0;
};

constexpr int kGemmWaves = 4;

// One wave per 16 x 16 output tile; operands are gathered element by element
// (fp32 MFMA takes one value per lane and step).
__global__ __launch_bounds__(64 * kGemmWaves) void gemm_f32_kernel(Gemm g) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tiles_n = g.N / 16, tiles = (g.M / 16) * tiles_n;
    const int groups = (tiles + kGemmWaves - 1) / kGemmWaves;
    const long long b = blockIdx.x / groups;
    const int t = (blockIdx.x % groups) * kGemmWaves + wave;
    if (b >= g.batch || t >= tiles) return;
    const int m0 = (t / tiles_n) * 16, n0 = (t % tiles_n) * 16;
    f32x4 acc = zero4();
    for (int k0 = 0; k0 < g.K; k0 += 4) {
        const int k = k0 + (lane >> 4);
        const float x = view_at(g.A, b, m0 + (lane & 15), k);
        const float y = view_at(g.B, b, k, n0 + (lane & 15));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc, 0, 0, 0);
    }
    const int n = n0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * (lane >> 4) + r;
        float val = g.alpha * acc[r];
        if (g.Cin.p) val += g.beta * view_at(g.Cin, b, m, n);
        if ((g.tri_out == 1 && n > m) || (g.tri_out == 2 && n >= m)) val = 0.0f;
        g.C[b * g.cbs + (size_t)m * g.ldc + n] = val;
    }
}

hipError_t launch_gemm(const Gemm &g, hipStream_t stream) {
    const int tiles = (g.M / 16) * (g.N / 16);
    const long long blocks = (long long)g.batch * ((tiles + kGemmWaves - 1) / kGemmWaves);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)blocks), dim3(64 * kGemmWaves), 0, stream, g);
    return hipGetLastError();
}

__device__ __forceinline__ void chunk_of(const ChunkArgs &a, int cid, int &tok0, int &len) {
    if (a.plan) {  // entries clamped: a stale or malformed table stays in bounds
        const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
        tok0 = min(max(e[1], 0), a.T);
        len = min(max(e[2], 0), min(kChunk, a.T - tok0));
    } else {
        const int n = cid / a.NC, c = cid % a.NC;
        tok0 = n * a.T + c * kChunk;
        len = min(kChunk, a.T - c * kChunk);
    }
}

__device__ __forceinline__ bool chunk_exists(const ChunkArgs &a, int cid) {
    return !a.plan || cid < min(max(a.plan[a.N], 0), a.max_chunks);
}

// ---------------------------------------------------------------------------
// Gather: per chunk-head, the chunk's token rows of q, k, v, b, w and dO
// (zero past the chunk's end), the within-chunk cumulative log-decay g, and
// the midpoint-scaled tiles Ep, Kp, Qp, all row-major [64][D].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_gather_kernel(BwdF32Args f) {
    const ChunkArgs &a = f.c;
    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (!chunk_exists(a, cid)) return;
    int tok0, len;
    chunk_of(a, cid, tok0, len);
    const size_t ch = (size_t)cid * H + h, tile = ch * kChunk * D;
    const float *q = static_cast<const float *>(a.q), *k = static_cast<const float *>(a.k);
    const float *v = static_cast<const float *>(a.v), *dO = static_cast<const float *>(f.dout);
    for (int e = threadIdx.x; e < kChunk * D; e += kThreads) {
        const int i = e / D, c = e % D;
        const bool in = i < len;
        const size_t src = ((size_t)(tok0 + (in ? i : 0)) * H + h) * D + c;
        f.Qg[tile + e] = in ? q[src] : 0.0f;
        f.Kg[tile + e] = in ? k[src] : 0.0f;
        f.Vg[tile + e] = in ? v[src] : 0.0f;
        f.Bg[tile + e] = in ? a.b[src] : 0.0f;
        f.Wg[tile + e] = in ? a.w[src] : 0.0f;
        f.dOg[tile + e] = in ? dO[src] : 0.0f;
    }
    // cumulative log-decay per channel (padding tokens add 0), shared through
    // LDS with the threads that form the tiles
    __shared__ float sG[kChunk * D];
    for (int c = threadIdx.x; c < D; c += kThreads) {
        float g = 0.0f;
        for (int i = 0; i < kChunk; ++i) {
            if (i < len) g += a.log_alpha[((size_t)(tok0 + i) * H + h) * D + c];
            sG[i * D + c] = g;
            f.G[tile + (size_t)i * D + c] = g;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kChunk * D; e += kThreads) {
        const int c = e % D;
        const float g = sG[e], gr = 0.5f * sG[(kChunk - 1) * D + c];
        const float ex = __expf(g - gr), ei = __expf(gr - g);
        f.Ep[tile + e] = f.Bg[tile + e] * f.Kg[tile + e] * ex;
        f.Kp[tile + e] = f.Kg[tile + e] * ei;
        f.Qp[tile + e] = f.Qg[tile + e] * ex;
    }
}

// ---------------------------------------------------------------------------
// Reverse pass: one workgroup per (sequence, head), its chunks from last to
// first.  dS' (the gradient of the chunk's outgoing state) and dU_eff live in
// LDS; each chunk's dS' and dU_eff are also stored for the per-chunk products.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_f32_reverse_kernel(BwdF32Args f) {
    const ChunkArgs &a = f.c;
    const int chain = blockIdx.x, H = a.H;
    if (chain >= a.N * H) return;
    const int n = chain / H, h = chain % H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int LDD = D + 4;
    __shared__ float sdS[D * LDD];        // dS' [c][v]
    __shared__ float sdU[kChunk * LDD];   // dU_eff [i][v]
    for (int e = threadIdx.x; e < D * D; e += kThreads)
        sdS[(e / D) * LDD + e % D] = f.dS_final ? f.dS_final[(size_t)chain * D * D + e] : 0.0f;
    int cbeg, cend;
    if (a.plan) {
        cbeg = min(max(a.plan[n], 0), a.max_chunks);
        cend = min(max(a.plan[n + 1], cbeg), a.max_chunks);
    } else {
        cbeg = n * a.NC;
        cend = cbeg + a.NC;
    }
    const float *dO = static_cast<const float *>(f.dout);
    constexpr int NT = D / 16;
    __syncthreads();
    for (int cid = cend - 1; cid >= cbeg; --cid) {
        int tok0, len;
        chunk_of(a, cid, tok0, len);
        const size_t ch = (size_t)cid * H + h;
        const float *Mg = static_cast<const float *>(a.ws_M) + ch * kChunk * kChunk;
        const float *Kt = static_cast<const float *>(a.ws_KhT) + ch * D * kChunk;
        const float *Qh = static_cast<const float *>(a.ws_Qh) + ch * kChunk * D;
        const float *Wf = static_cast<const float *>(a.ws_W) + ch * kChunk * D;
        const float *gl = a.ws_gl + ch * D;
        auto dO_at = [&](int i, int vv) {  // rows past the chunk's end are zero
            return i < len ? dO[((size_t)(tok0 + i) * H + h) * D + vv] : 0.0f;
        };
        // dS' of this chunk, kept for the per-chunk products
        for (int e = threadIdx.x; e < D * D; e += kThreads)
            f.dSp[ch * D * D + e] = sdS[(e / D) * LDD + e % D];
        // dU_eff [64 x D] = M^T dO + Khat dS'
        for (int t = wave; t < 4 * NT; t += 4) {
            const int i0 = 16 * (t / NT), v0 = 16 * (t % NT);
            f32x4 acc = zero4();
            for (int k0 = 0; k0 < kChunk; k0 += 4) {  // M^T[i][j] = M[j][i] (M zero above the diagonal)
                const int j = k0 + (lane >> 4), i = i0 + (lane & 15);
                const float m = i <= j ? Mg[frag_index<float>(j, i, kChunk)] : 0.0f;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m, dO_at(j, v0 + (lane & 15)), acc, 0, 0, 0);
            }
            for (int k0 = 0; k0 < D; k0 += 4) {  // Khat[i][c] = Khat^T[c][i]
                const int c = k0 + (lane >> 4);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kt[frag_index<float>(c, i0 + (lane & 15), kChunk)],
                                                            sdS[c * LDD + v0 + (lane & 15)], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 4 * (lane >> 4) + r, vv = v0 + (lane & 15);
                sdU[i * LDD + vv] = acc[r];
                f.dUeff[ch * kChunk * D + (size_t)i * D + vv] = acc[r];
            }
        }
        __syncthreads();
        // dS [D x D] = Diag(gl) dS' + Qhat^T dO - W^T dU_eff   (in place: each
        // element reads only its own dS' value)
        for (int t = wave; t < NT * NT; t += 4) {
            const int c0 = 16 * (t / NT), v0 = 16 * (t % NT);
            f32x4 acc = zero4();
            for (int k0 = 0; k0 < kChunk; k0 += 4) {
                const int i = k0 + (lane >> 4), c = c0 + (lane & 15), vv = v0 + (lane & 15);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Qh[frag_index<float>(i, c, D)], dO_at(i, vv), acc,
                                                            0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-Wf[frag_index<float>(i, c, D)],
                                                            sdU[i * LDD + vv], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = c0 + 4 * (lane >> 4) + r, vv = v0 + (lane & 15);
                sdS[c * LDD + vv] = gl[c] * sdS[c * LDD + vv] + acc[r];
            }
        }
        __syncthreads();
    }
    if (f.dS0)
        for (int e = threadIdx.x; e < D * D; e += kThreads)
            f.dS0[(size_t)chain * D * D + e] = sdS[(e / D) * LDD + e % D];
}

// ---------------------------------------------------------------------------
// Per token: the element-wise gradients, dlog_alpha by a reverse cumulative
// sum over the chunk, written to the rows the chunk owns.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_final_kernel(BwdF32Args f) {
    const ChunkArgs &a = f.c;
    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (!chunk_exists(a, cid)) return;
    int tok0, len;
    chunk_of(a, cid, tok0, len);
    const size_t ch = (size_t)cid * H + h, tile = ch * kChunk * D;
    float *dq = static_cast<float *>(f.dq), *dk = static_cast<float *>(f.dk);
    float *dv = static_cast<float *>(f.dv);
    __shared__ float sdg[kChunk * (D + 1)];
    for (int e = threadIdx.x; e < kChunk * D; e += kThreads) {
        const int i = e / D, c = e % D;
        const float g = f.G[tile + e], gl_ = f.G[tile + (size_t)(kChunk - 1) * D + c], gr = 0.5f * gl_;
        const float gam = __expf(g), ex = __expf(g - gr), ei = __expf(gr - g), eK = __expf(gl_ - g);
        const float q = f.Qg[tile + e], k = f.Kg[tile + e], b = f.Bg[tile + e];
        const float dQh = f.dQhat[tile + e], dQp = f.dQp[tile + e], dE = f.dE[tile + e];
        const float dEp = f.dEp[tile + e], dKp = f.dKp[tile + e], dKh = f.dKhat[tile + e];
        const float dEt = gam * dE + ex * dEp;
        // dg = E dE + Ep dEp + Qhat dQhat + Qp dQp - Kp dKp - Khat dKhat
        sdg[i * (D + 1) + c] = gam * b * k * dE + ex * b * k * dEp + gam * q * dQh + ex * q * dQp -
                               ei * k * dKp - eK * k * dKh;
        if (i < len) {
            const size_t o = ((size_t)(tok0 + i) * H + h) * D + c;
            const float dZ = f.dZ[tile + e];
            dq[o] = gam * dQh + ex * dQp;
            f.db[o] = k * dEt;
            dk[o] = b * dEt + ei * dKp + eK * dKh;
            dv[o] = f.Wg[tile + e] * dZ;
            f.dw[o] = f.Vg[tile + e] * dZ;
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += kThreads) {
        // the chunk-wide terms: gamma_last dgl (dgl = rowsum(dS' * S)) and
        // sum_i Khat_i dKhat_i, both through g_last
        const float gl_ = f.G[tile + (size_t)(kChunk - 1) * D + c];
        float dgl = 0.0f;
        for (int vv = 0; vv < D; ++vv)
            dgl += f.dSp[ch * D * D + (size_t)c * D + vv] * f.Sc[ch * D * D + (size_t)c * D + vv];
        float kd = 0.0f;
        for (int i = 0; i < kChunk; ++i)
            kd += __expf(gl_ - f.G[tile + (size_t)i * D + c]) * f.Kg[tile + (size_t)i * D + c] *
                  f.dKhat[tile + (size_t)i * D + c];
        float run = __expf(gl_) * dgl + kd;
        for (int i = kChunk - 1; i >= 0; --i) {
            run += sdg[i * (D + 1) + c];
            if (i < len) f.dla[((size_t)(tok0 + i) * H + h) * D + c] = run;
        }
    }
}

}  // namespace

// The per-chunk products, as batched GEMMs over every chunk-head slot.
template <int D>
static hipError_t chunk_products(const BwdF32Args &f, hipStream_t stream) {
    const ChunkArgs &a = f.c;
    const int batch = a.max_chunks * a.H;
    const long long t64 = (long long)kChunk * D, tDD = (long long)D * D, t4k = kChunk * kChunk;
    hipError_t err = hipSuccess;
    auto run = [&](Gemm g, int M, int N, int K, float *C, long long cbs, int ldc) {
        if (err != hipSuccess) return;
        g.M = M;
        g.N = N;
        g.K = K;
        g.C = C;
        g.cbs = cbs;
        g.ldc = ldc;
        g.batch = batch;
        err = launch_gemm(g, stream);
    };
    const View W = frag(a.ws_W, t64, D), Sc = rm(f.Sc, tDD, D);
    const View dO = rm(f.dOg, t64, D), dUe = rm(f.dUeff, t64, D);
    const View T = rm(static_cast<const float *>(a.ws_T), t4k, kChunk);
    View U;
    U.p = static_cast<const float *>(a.ws_U);
    U.bs = t64;
    U.ld = D;
    U.layout = kAccOrder;
    {  // U_eff = U - W S
        Gemm g;
        g.A = W;
        g.B = Sc;
        g.Cin = U;
        g.alpha = -1.0f;
        g.beta = 1.0f;
        run(g, kChunk, D, D, f.Ueff, t64, D);
    }
    {  // dQhat = dO S^T
        Gemm g;
        g.A = dO;
        g.B = rm(f.Sc, tDD, D, 1);
        run(g, kChunk, D, D, f.dQhat, t64, D);
    }
    {  // dM = tril(dO U_eff^T)
        Gemm g;
        g.A = dO;
        g.B = rm(f.Ueff, t64, D, 1);
        g.tri_out = 1;
        run(g, kChunk, kChunk, D, f.dM, t4k, kChunk);
    }
    {  // dKhat = U_eff dS'^T
        Gemm g;
        g.A = rm(f.Ueff, t64, D);
        g.B = rm(f.dSp, tDD, D, 1);
        run(g, kChunk, D, D, f.dKhat, t64, D);
    }
    {  // dW = -dU_eff S^T
        Gemm g;
        g.A = dUe;
        g.B = rm(f.Sc, tDD, D, 1);
        g.alpha = -1.0f;
        run(g, kChunk, D, D, f.dW, t64, D);
    }
    {  // dZ = T^T dU_eff
        Gemm g;
        g.A = rm(T.p, t4k, kChunk, 1);
        g.B = dUe;
        run(g, kChunk, D, kChunk, f.dZ, t64, D);
    }
    {  // dE = T^T dW
        Gemm g;
        g.A = rm(T.p, t4k, kChunk, 1);
        g.B = rm(f.dW, t64, D);
        run(g, kChunk, D, kChunk, f.dE, t64, D);
    }
    {  // dA = dZ U^T, then dA = -strict_tril(dA + dE W^T)
        Gemm g;
        g.A = rm(f.dZ, t64, D);
        View Ut = U;
        Ut.trans = 1;
        g.B = Ut;
        run(g, kChunk, kChunk, D, f.dA, t4k, kChunk);
        Gemm g2;
        g2.A = rm(f.dE, t64, D);
        g2.B = frag(a.ws_W, t64, D, 1);
        g2.Cin = rm(f.dA, t4k, kChunk);
        g2.alpha = -1.0f;
        g2.beta = -1.0f;
        g2.tri_out = 2;
        run(g2, kChunk, kChunk, D, f.dA, t4k, kChunk);
    }
    {  // dEp = dA Kp,  dQp = dM Kp
        Gemm g;
        g.A = rm(f.dA, t4k, kChunk);
        g.B = rm(f.Kp, t64, D);
        run(g, kChunk, D, kChunk, f.dEp, t64, D);
        Gemm g2;
        g2.A = rm(f.dM, t4k, kChunk);
        g2.B = rm(f.Kp, t64, D);
        run(g2, kChunk, D, kChunk, f.dQp, t64, D);
    }
    {  // dKp = dA^T Ep + dM^T Qp
        Gemm g;
        g.A = rm(f.dA, t4k, kChunk, 1);
        g.B = rm(f.Ep, t64, D);
        run(g, kChunk, D, kChunk, f.dKp, t64, D);
        Gemm g2;
        g2.A = rm(f.dM, t4k, kChunk, 1);
        g2.B = rm(f.Qp, t64, D);
        g2.Cin = rm(f.dKp, t64, D);
        g2.beta = 1.0f;
        run(g2, kChunk, D, kChunk, f.dKp, t64, D);
    }
    return err;
}

template <int D>
static hipError_t bwd_f32_d(const BwdF32Args &f, hipStream_t stream) {
    const ChunkArgs &a = f.c;
    const unsigned items = (unsigned)((size_t)a.max_chunks * a.H);
    if (items > 0) {
        hipLaunchKernelGGL((bwd_f32_gather_kernel<D>), dim3(items), dim3(kThreads), 0, stream, f);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (a.N * a.H > 0) {
        hipLaunchKernelGGL((bwd_f32_reverse_kernel<D>), dim3((unsigned)(a.N * a.H)), dim3(kThreads), 0,
                           stream, f);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (items == 0) return hipSuccess;
    const hipError_t err = chunk_products<D>(f, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_f32_final_kernel<D>), dim3(items), dim3(kThreads), 0, stream, f);
    return hipGetLastError();
}

hipError_t launch_chunk_bwd_f32(const BwdF32Args &f, int Dk, hipStream_t stream) {
    return Dk == 128 ? bwd_f32_d<128>(f, stream) : bwd_f32_d<64>(f, stream);
}

}  // namespace gdn2
