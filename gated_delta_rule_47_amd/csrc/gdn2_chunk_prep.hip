// Chunk-factor kernel: everything of a 64-token chunk that does not depend on
// the incoming state, for one (chunk, head) per workgroup.
//
// The chunk form follows the WY description of the iplexlaw digest (section
// "Procesamiento del token y entrenamiento paralelo": 64-token chunks, the
// cumulative per-channel decay folded into asymmetric erase factors, a
// triangular solve and dense products inside the chunk, decay in fp32) and of
// the gist.science summary (part "3. Efficient chunkwise parallel training":
// decay absorbed into the erase and write matrices, the lower-triangular
// system (I+T)^-1, erase-side and write-side auxiliaries).  With the local
// cumulative log-decay g_i = sum_{j<=i} log alpha_j and gamma_i = exp(g_i):
//
//   stage 1  g = inclusive cumsum of log alpha over the chunk (fp32)
//   stage 2  A_ij = sum_c b_i k_i k_j exp(g_i - g_j)   (j < i),  T = (I + A)^-1
//   stage 3  W = T (gamma * b * k),  M_ij = sum_c q_i k_j exp(g_i - g_j) (j <= i),
//            Qhat = gamma * q,  Khat = exp(g_last - g) * k,  gamma_last = exp(g_last)
//
// Numerics.  A and M are products of two scaled tiles referenced to the
// per-channel midpoint g_r = g_last / 2: (b k e^{g-g_r}) and (k e^{g_r-g}), so
// every factor lies within e^{|g_last|/2}; their bf16 MFMA products keep bf16
// relative precision.  T is solved in fp32: the four 16x16 diagonal blocks by
// forward substitution, the off-diagonal blocks by fp32 MFMA block products,
// level by level.  The contraction W uses bf16 (or fp32) MFMA with fp32
// accumulation.
//
// Work split (256 threads = 4 waves): thread (p, tg) owns channels 2p, 2p+1 of
// tokens tg*TPG .. tg*TPG+TPG-1, so global loads of a token row are coalesced.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <typename E, int DK>
struct PrepCfg {
    static constexpr int NPAIR = DK / 2;
    static constexpr int NTG = kThreads / NPAIR;     // token groups
    static constexpr int TPG = kChunk / NTG;         // tokens per group
    static constexpr int PAD = (sizeof(E) == 2) ? 8 : 4;
    static constexpr int LDT = DK + PAD;             // token-major tiles [64][LDT]
    static constexpr int LDC = kChunk + PAD;         // channel-major tiles [DK][LDC]
    static constexpr int LDA = kChunk + 4;           // fp32 64x64 matrices
    static constexpr int LDX = 16 + 4;               // fp32 16x16 scratch
    // Region 1: three token-major tiles, later reused for A, T, T (as E), scratch.
    static constexpr size_t R1_TILES = 3 * size_t(kChunk) * LDT * sizeof(E);
    static constexpr size_t SZ_A = size_t(kChunk) * LDA * 4;
    static constexpr size_t SZ_TB = size_t(kChunk) * LDC * sizeof(E);
    static constexpr size_t SZ_X = 4 * 16 * LDX * 4;
    static constexpr size_t R1_SOLVE = 2 * SZ_A + SZ_TB + SZ_X;
    static constexpr size_t R1 = R1_TILES > R1_SOLVE ? R1_TILES : R1_SOLVE;
    static constexpr size_t SZ_ET = size_t(DK) * LDC * sizeof(E);
    static constexpr size_t SZ_TOT = size_t(NTG) * DK * 4;
    static constexpr size_t SMEM = R1 + SZ_ET + SZ_TOT;
    static_assert(NTG * NPAIR == kThreads && TPG * NTG == kChunk, "thread map");
};

// acc += X[16x16] * Y[16x16], both fp32 row-major (Y indexed [k][n]).
__device__ __forceinline__ f32x4 mma16_f32_nn(f32x4 acc, const float *X, int ldx, const float *Y,
                                              int ldy, int lane) {
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4) {
        const float a = X[(lane & 15) * ldx + kk + (lane >> 4)];
        const float b = Y[(kk + (lane >> 4)) * ldy + (lane & 15)];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

template <typename E>
__device__ __forceinline__ void store2(E *p, float x0, float x1) {
    if constexpr (sizeof(E) == 2) {
        bf16x2 v;
        v[0] = static_cast<bf16>(x0);
        v[1] = static_cast<bf16>(x1);
        *reinterpret_cast<bf16x2 *>(p) = v;
    } else {
        *reinterpret_cast<f32x2 *>(p) = f32x2{x0, x1};
    }
}

template <typename E>
__device__ __forceinline__ void load2(const E *p, float &x0, float &x1) {
    if constexpr (sizeof(E) == 2) {
        const bf16x2 v = *reinterpret_cast<const bf16x2 *>(p);
        x0 = static_cast<float>(v[0]);
        x1 = static_cast<float>(v[1]);
    } else {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        x0 = v[0];
        x1 = v[1];
    }
}

// Store n (a multiple of 4) consecutive values as E.
template <typename E, int n>
__device__ __forceinline__ void store_run(E *p, const float *x) {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
        if constexpr (sizeof(E) == 2) {
            bf16x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = static_cast<bf16>(x[i + j]);
            *reinterpret_cast<bf16x4 *>(p + i) = v;
        } else {
            *reinterpret_cast<f32x4 *>(p + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
        }
    }
}

template <typename E, int DK>
__global__ __launch_bounds__(kThreads, 2) void chunk_prep_kernel(ChunkArgs a) {
    using C = PrepCfg<E, DK>;
    constexpr int TPG = C::TPG, LDT = C::LDT, LDC = C::LDC, LDA = C::LDA, LDX = C::LDX;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    E *sEp = reinterpret_cast<E *>(smem);                  // [64][LDT] b k e^{g-g_r}
    E *sKp = sEp + kChunk * LDT;                           // [64][LDT] k e^{g_r-g}
    E *sQp = sKp + kChunk * LDT;                           // [64][LDT] q e^{g-g_r}
    float *sA = reinterpret_cast<float *>(smem);           // [64][LDA]  (after the tiles die)
    float *sT = sA + kChunk * LDA;                         // [64][LDA]
    E *sTb = reinterpret_cast<E *>(sT + kChunk * LDA);     // [64][LDC]  T as E
    float *sX = reinterpret_cast<float *>(smem + 2 * C::SZ_A + C::SZ_TB);  // [4][16][LDX]
    E *sEt = reinterpret_cast<E *>(smem + C::R1);          // [DK][LDC]  (gamma b k)^T
    float *sTot = reinterpret_cast<float *>(smem + C::R1 + C::SZ_ET);  // [NTG][DK]

    const int cid = blockIdx.x, h = blockIdx.y, H = a.H;
    int tok0, len;
    if (a.plan) {
        if (cid >= a.plan[a.N]) return;
        // Entries are clamped so that a stale or malformed table stays in bounds.
        const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
        tok0 = min(max(e[1], 0), a.T);
        len = min(max(e[2], 0), min(kChunk, a.T - tok0));
    } else {
        const int n = cid / a.NC, c = cid % a.NC;
        tok0 = n * a.T + c * kChunk;
        len = min(kChunk, a.T - c * kChunk);
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = tid % C::NPAIR, tg = tid / C::NPAIR;
    const int c0 = 2 * p;
    const size_t ch = (size_t)cid * H + h;  // chunk-head index into the workspace

    const E *q = reinterpret_cast<const E *>(a.q);
    const E *k = reinterpret_cast<const E *>(a.k);

    // ---- stage 1: load and cumulative log-decay ---------------------------
    float g0[TPG], g1[TPG], b0[TPG], b1[TPG], k0[TPG], k1[TPG], q0[TPG], q1[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        if (i < len) {
            const size_t off = ((size_t)(tok0 + i) * H + h) * DK + c0;
            const f32x2 la = *reinterpret_cast<const f32x2 *>(a.log_alpha + off);
            const f32x2 bb = *reinterpret_cast<const f32x2 *>(a.b + off);
            g0[j] = la[0];
            g1[j] = la[1];
            b0[j] = bb[0];
            b1[j] = bb[1];
            load2<E>(k + off, k0[j], k1[j]);
            load2<E>(q + off, q0[j], q1[j]);
        } else {  // padding token: k = q = b = 0, log alpha = 0 (an exact no-op)
            g0[j] = g1[j] = b0[j] = b1[j] = k0[j] = k1[j] = q0[j] = q1[j] = 0.0f;
        }
    }
#pragma unroll
    for (int j = 1; j < TPG; ++j) {
        g0[j] += g0[j - 1];
        g1[j] += g1[j - 1];
    }
    sTot[tg * DK + c0] = g0[TPG - 1];
    sTot[tg * DK + c0 + 1] = g1[TPG - 1];
    __syncthreads();
    float off0 = 0.0f, off1 = 0.0f, gl0 = 0.0f, gl1 = 0.0f;
#pragma unroll
    for (int t = 0; t < C::NTG; ++t) {
        const float t0 = sTot[t * DK + c0], t1 = sTot[t * DK + c0 + 1];
        if (t < tg) {
            off0 += t0;
            off1 += t1;
        }
        gl0 += t0;
        gl1 += t1;
    }
    // Per-channel constants: midpoint reference g_r = g_last/2 and e^{g_r}.
    const float gr0 = 0.5f * gl0, gr1 = 0.5f * gl1;
    const float egr0 = __expf(gr0), egr1 = __expf(gr1);

    // ---- scaled tiles ------------------------------------------------------
    E *Qh = reinterpret_cast<E *>(a.ws_Qh) + ch * kChunk * DK;
    E *KhT = reinterpret_cast<E *>(a.ws_KhT) + ch * DK * kChunk;
    float et0[TPG], et1[TPG], kh0[TPG], kh1[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        const float ga = g0[j] + off0, gb = g1[j] + off1;
        const float ex0 = __expf(ga - gr0), ex1 = __expf(gb - gr1);     // e^{g - g_r}
        const float ei0 = __expf(gr0 - ga), ei1 = __expf(gr1 - gb);     // e^{g_r - g}
        store2<E>(sEp + i * LDT + c0, b0[j] * k0[j] * ex0, b1[j] * k1[j] * ex1);
        store2<E>(sKp + i * LDT + c0, k0[j] * ei0, k1[j] * ei1);
        store2<E>(sQp + i * LDT + c0, q0[j] * ex0, q1[j] * ex1);
        // gamma = e^{g} = e^{g-g_r} e^{g_r};  e^{g_last-g} = e^{g_r-g} e^{g_r}
        const float gm0 = ex0 * egr0, gm1 = ex1 * egr1;
        store2<E>(Qh + i * DK + c0, q0[j] * gm0, q1[j] * gm1);
        et0[j] = gm0 * b0[j] * k0[j];
        et1[j] = gm1 * b1[j] * k1[j];
        kh0[j] = ei0 * egr0 * k0[j];
        kh1[j] = ei1 * egr1 * k1[j];
    }
    store_run<E, TPG>(sEt + c0 * LDC + tg * TPG, et0);
    store_run<E, TPG>(sEt + (c0 + 1) * LDC + tg * TPG, et1);
    store_run<E, TPG>(KhT + (size_t)c0 * kChunk + tg * TPG, kh0);
    store_run<E, TPG>(KhT + (size_t)(c0 + 1) * kChunk + tg * TPG, kh1);
    if (tg == 0) {
        float *gl = a.ws_gl + ch * DK;
        *reinterpret_cast<f32x2 *>(gl + c0) = f32x2{__expf(gl0), __expf(gl1)};
    }
    __syncthreads();

    // ---- stage 2a: A (waves 0,1) and M (waves 2,3) by MFMA ----------------
    // Tile (I, J), I >= J, is formed transposed: D[j][i] = sum_c Kp[j][c] Y[i][c],
    // so each lane ends up with 4 consecutive columns j of one row i.
    // Waves pair row blocks {0,3} and {1,2} to balance the triangle.
    const int rb_a = (wave & 1) ? 1 : 0, rb_b = (wave & 1) ? 2 : 3;
    f32x4 accA[5];
    E *Mg = reinterpret_cast<E *>(a.ws_M) + ch * kChunk * kChunk;
    {
        const bool isA = wave < 2;
        const E *Y = isA ? sEp : sQp;
        int t = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int I = s == 0 ? rb_a : rb_b;
            for (int J = 0; J <= I; ++J, ++t) {
                f32x4 acc = mma_tile<E, DK>(zero4(), sKp + 16 * J * LDT, LDT, Y + 16 * I * LDT,
                                            LDT, lane);
                const int i = 16 * I + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J + 4 * (lane >> 4) + r;
                    const bool keep = isA ? (j < i) : (j <= i);
                    acc[r] = keep ? acc[r] : 0.0f;
                }
                if (isA) {
#pragma unroll
                    for (int u = 0; u < 5; ++u)
                        if (u == t) accA[u] = acc;
                } else {
                    store_tile_t<E>(Mg + 16 * I * kChunk + 16 * J, kChunk, acc, lane);
                }
            }
        }
        if (!isA) {  // the zero upper blocks of M (read by the propagation kernel)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int I = s == 0 ? rb_a : rb_b;
                for (int J = I + 1; J < 4; ++J)
                    store_tile_t<E>(Mg + 16 * I * kChunk + 16 * J, kChunk, zero4(), lane);
            }
        }
    }
    __syncthreads();  // the scaled token-major tiles are dead from here on

    if (wave < 2) {
        int t = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int I = s == 0 ? rb_a : rb_b;
            for (int J = 0; J <= I; ++J, ++t) {
                f32x4 acc = accA[0];
#pragma unroll
                for (int u = 1; u < 5; ++u)
                    if (u == t) acc = accA[u];
                store_tile_t<float>(sA + 16 * I * LDA + 16 * J, LDA, acc, lane);
            }
        }
    } else {  // zero the strictly upper 16x16 blocks of T
        for (int blk = tid - 128; blk < 6 * 256; blk += 128) {
            const int which = blk / 256, e = blk % 256;
            const int I = which < 3 ? 0 : (which < 5 ? 1 : 2);
            const int J = which < 3 ? which + 1 : (which < 5 ? which - 1 : 3);
            sT[(16 * I + e / 16) * LDA + 16 * J + (e % 16)] = 0.0f;
        }
    }
    __syncthreads();

    // ---- stage 2b: T = (I + A)^-1 in fp32 ----------------------------------
    // Diagonal blocks: wave 0, lane = (block, column); forward substitution.
    if (wave == 0) {
        const int I = lane >> 4, c = lane & 15;
        const float *Ab = sA + 16 * I * LDA + 16 * I;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == c) ? 1.0f : 0.0f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= Ab[i * LDA + j] * x[j];
            x[i] = s;
        }
        float *Tb = sT + 16 * I * LDA + 16 * I;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * LDA + c] = x[i];
    }
    __syncthreads();
    // Off-diagonal blocks, level s = I - J:  T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.
#pragma unroll
    for (int s = 1; s < 4; ++s) {
        const int J = wave, I = wave + s;
        if (I < 4) {
            f32x4 acc = zero4();
            for (int K = J; K < I; ++K)
                acc = mma16_f32_nn(acc, sA + 16 * I * LDA + 16 * K, LDA, sT + 16 * K * LDA + 16 * J,
                                   LDA, lane);
            float *X = sX + wave * 16 * LDX;
            store_tile<float>(X, LDX, acc, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 t = mma16_f32_nn(zero4(), sT + 16 * I * LDA + 16 * I, LDA, X, LDX, lane);
            store_tile<float>(sT + 16 * I * LDA + 16 * J, LDA, -t, lane);
        }
        __syncthreads();
    }

    // ---- T out: E copy in LDS for the W product, and to the workspace ------
    {
        E *Tg = reinterpret_cast<E *>(a.ws_T) + ch * kChunk * kChunk;
        const int row = tid >> 2, col = 16 * (tid & 3);
        float tv[16];
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sT + row * LDA + col + j);
            tv[j] = v[0];
            tv[j + 1] = v[1];
            tv[j + 2] = v[2];
            tv[j + 3] = v[3];
        }
        store_run<E, 16>(sTb + row * LDC + col, tv);
        store_run<E, 16>(Tg + row * kChunk + col, tv);
    }
    __syncthreads();

    // ---- stage 3: W = T (gamma b k), formed transposed --------------------
    // D[c][i] = sum_j Et[c][j] T[i][j]; lane holds W[i][c..c+3].
    {
        using M = Mma<E>;
        E *Wg = reinterpret_cast<E *>(a.ws_W) + ch * kChunk * DK;
        constexpr int CB = DK / 16;          // channel blocks
        constexpr int CB_PER_WAVE = CB / 4;
#pragma unroll
        for (int cb = 0; cb < CB_PER_WAVE; ++cb) {
            const int cblk = wave * CB_PER_WAVE + cb;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                constexpr int KS = M::KS;
                const int K = ((16 * (I + 1) + KS - 1) / KS) * KS;
                f32x4 acc = mma_tile_k<E>(zero4(), sEt + 16 * cblk * LDC, LDC, sTb + 16 * I * LDC,
                                          LDC, K, lane);
                store_tile_t<E>(Wg + 16 * I * DK + 16 * cblk, DK, acc, lane);
            }
        }
    }
}

hipError_t launch_chunk_prep(const ChunkArgs &a, int Dk, bool bf16_io, hipStream_t stream) {
    const dim3 grid((unsigned)a.max_chunks, (unsigned)a.H), block(kThreads);
    if (bf16_io) {
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64>), grid, block, 0, stream, a);
    } else {
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<float, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<float, 64>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gdn2
