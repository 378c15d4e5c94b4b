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
//   stage 3  W = T (gamma * b * k)   (erase side),   U = T (w * v)   (write side),
//            M_ij = sum_c q_i k_j exp(g_i - g_j) (j <= i),
//            Qhat = gamma * q,  Khat = exp(g_last - g) * k,  gamma_last = exp(g_last)
//
// Numerics.  A and M are products of two scaled tiles referenced to the
// per-channel midpoint g_r = g_last / 2: (b k e^{g-g_r}) and (k e^{g_r-g}), so
// every factor lies within e^{|g_last|/2}; their bf16 MFMA products keep bf16
// relative precision.  T is solved in fp32: the four 16x16 diagonal blocks by
// forward substitution, the off-diagonal blocks by fp32 MFMA block products,
// level by level.  W and U use bf16 (or fp32) MFMA with fp32 accumulation.
//
// Work split (256 threads = 4 waves): thread (qd, tg) owns channels 4qd..4qd+3
// of tokens tg*TPG .. tg*TPG+TPG-1, so each wave load instruction reads whole
// token rows of one head.  LDS is reused phase by phase (68 KB for bf16 with
// 128-wide heads; two workgroups per CU).  W, M and U leave the accumulators
// as 512 contiguous bytes per wave store; Qhat and Khat^T, whose fragment order
// does not match the thread map, go through an LDS image and leave in 1 KiB
// contiguous wave stores.

#include <type_traits>

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <typename E, int DK>
struct PrepCfg {
    static constexpr int NQUAD = DK / 4;             // 4-channel groups
    static constexpr int NTG = kThreads / NQUAD;     // token groups
    static constexpr int TPG = kChunk / NTG;         // tokens per group
    static constexpr int PAD = (sizeof(E) == 2) ? 8 : 4;
    static constexpr int LDT = DK + PAD;             // token-major tiles [64][LDT]
    static constexpr int LDC = kChunk + PAD;         // channel-major tiles [DK][LDC]
    static constexpr int LDA = kChunk + 4;           // fp32 64x64 (A, then T in place)
    static constexpr int LDX = 16 + 4;               // fp32 16x16 scratch
    // Region 1: token-major tiles Kp and X (X holds Ep, then Qp); later the
    // solve buffers A/T, T as E, and the per-wave scratch.
    static constexpr size_t SZ_TILE = size_t(kChunk) * LDT * sizeof(E);
    static constexpr size_t SZ_A = size_t(kChunk) * LDA * 4;
    static constexpr size_t SZ_TB = size_t(kChunk) * LDC * sizeof(E);
    static constexpr size_t SZ_X = 4 * 16 * LDX * 4;
    static constexpr size_t R1_SOLVE = SZ_A + SZ_TB + SZ_X;
    static constexpr size_t R1 = 2 * SZ_TILE > R1_SOLVE ? 2 * SZ_TILE : R1_SOLVE;
    // Region 2: channel-major (gamma b k)^T, later (w v)^T.
    static constexpr size_t SZ_ET = size_t(DK) * LDC * sizeof(E);
    // Region 3: fragment-order image of Khat^T, then of Qhat, copied out in
    // 16-byte granules (NG of them).
    static constexpr size_t SZ_STG = size_t(kChunk) * DK * sizeof(E);
    static constexpr int NG = int(SZ_STG / 16);
    static constexpr size_t SMEM = R1 + SZ_ET + SZ_STG;
    static_assert(NTG * NQUAD == kThreads && TPG * NTG == kChunk && TPG % 4 == 0, "thread map");
    static_assert(size_t(NTG) * DK * 4 <= R1, "group totals fit in region 1");
    static_assert(NG % kThreads == 0 && SMEM <= 160 * 1024, "staging image");
};

// The staging image keeps the fragment order in 16-byte granules, with granule
// g held at slot g ^ ((g/16 ^ g/128) mod 16).  The XOR only permutes the slots
// inside each aligned run of 16 granules (one pass over all LDS banks), so the
// contiguous copy-out reads without bank conflicts, and it spreads the
// scattered writes of the thread map below over distinct banks.
__device__ __forceinline__ int stage_slot(int g) { return g ^ (((g >> 4) ^ (g >> 7)) & 15); }

template <typename E>
__device__ __forceinline__ E *stage_ptr(E *img, size_t e) {  // element e of the fragment order
    constexpr int G = 16 / sizeof(E);
    return img + (size_t)stage_slot(int(e / G)) * G + e % G;
}

// Copy the whole image to its fragment-ordered destination: each wave store
// instruction writes 1 KiB of consecutive bytes.  The chunk factors are
// stored non-temporally (as W, M and U below): the next kernel reads them
// from HBM anyway, and keeping them out of the caches measured ~3% faster.
template <typename E, int NG>
__device__ __forceinline__ void stage_copy_out(E *dst, const E *img, int tid) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const char *src = reinterpret_cast<const char *>(img);
    char *d = reinterpret_cast<char *>(dst);
#pragma unroll
    for (int t = tid; t < NG; t += kThreads)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src + (size_t)stage_slot(t) * 16),
                                    reinterpret_cast<u32x4 *>(d + (size_t)t * 16));
}

// acc += X[16x16] * Y[16x16] in fp32, with X[m][k] read at X[m*xsm + k*xsk] and
// Y[k][n] at Y[k*ysk + n*ysn] (either operand may be stored transposed).
__device__ __forceinline__ f32x4 mma16_f32(f32x4 acc, const float *X, int xsm, int xsk,
                                           const float *Y, int ysk, int ysn, int lane) {
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4) {
        const float a = X[(lane & 15) * xsm + (kk + (lane >> 4)) * xsk];
        const float b = Y[(kk + (lane >> 4)) * ysk + (lane & 15) * ysn];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

// The channel-major tile (rows = channels, columns = the chunk's tokens) keeps
// the 16-byte token granule g of channel row c at granule g ^ ((c / 16) mod 8).
// The XOR is uniform over each 16-row MFMA tile, so operand reads see the plain
// padded layout, and it spreads the transposing stores of the thread map
// (32 lanes on 32 different channels, one granule each) over all banks.
template <typename E>
__device__ __forceinline__ int et_col(int c, int t) {
    constexpr int G = 16 / sizeof(E);
    return (((t / G) ^ ((c >> 4) & 7)) * G) + t % G;
}

// acc += A[16 x K] * B[16 x K]^T from row-major tiles with k contiguous, where
// an operand with swizzle s != 0 is a channel-major tile row block whose
// granules are permuted by XOR with s (see et_col).
template <typename E>
__device__ __forceinline__ f32x4 mma_tile_swz(f32x4 acc, const E *A, int lda, int swa, const E *B,
                                              int ldb, int swb, int K, int lane) {
    using M = Mma<E>;
    constexpr int G = 16 / sizeof(E);
    for (int kk = 0; kk < K; kk += M::KS) {
        const int k = kk + M::KPL * (lane >> 4);
        const int ka = (((k / G) ^ swa) * G) + k % G, kb = (((k / G) ^ swb) * G) + k % G;
        acc = M::mma(*reinterpret_cast<const typename M::frag *>(A + (lane & 15) * lda + ka),
                     *reinterpret_cast<const typename M::frag *>(B + (lane & 15) * ldb + kb), acc);
    }
    return acc;
}

template <typename E>
__device__ __forceinline__ void store4(E *p, f32x4 x) {
    if constexpr (sizeof(E) == 2) {
        bf16x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = static_cast<bf16>(x[j]);
        *reinterpret_cast<bf16x4 *>(p) = v;
    } else {
        *reinterpret_cast<f32x4 *>(p) = x;
    }
}

template <typename E>
__device__ __forceinline__ f32x4 load4(const E *p) {
    if constexpr (sizeof(E) == 2) {
        const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
        return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                     static_cast<float>(v[3])};
    } else {
        return *reinterpret_cast<const f32x4 *>(p);
    }
}

// store4_frag with a non-temporal store (bf16)
template <typename E>
__device__ __forceinline__ void store4_frag_nt(E *X, int K, int r, int k, f32x4 v) {
    if constexpr (sizeof(E) == 2) {
        bf16x4 b;
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = static_cast<bf16>(v[j]);
        __builtin_nontemporal_store(b, reinterpret_cast<bf16x4 *>(X + frag_index<E>(r, k, K)));
    } else {
        store4_frag<E>(X, K, r, k, v);
    }
}

// Four values kept in the element type between phases (halves the registers for bf16).
template <typename E>
using Vec4 = typename std::conditional<sizeof(E) == 2, bf16x4, f32x4>::type;

template <typename E>
__device__ __forceinline__ Vec4<E> pack4(f32x4 x) {
    if constexpr (sizeof(E) == 2) {
        bf16x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = static_cast<bf16>(x[j]);
        return v;
    } else {
        return x;
    }
}

template <typename E>
__device__ __forceinline__ float elem(Vec4<E> x, int j) { return to_f32(x[j]); }

__device__ __forceinline__ f32x4 to4(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 to4(bf16x4 x) {
    return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                 static_cast<float>(x[3])};
}

// Store the n (a multiple of 4) tokens t0.. of channel c into the channel-major
// tile (row pointer `row`), in the granule order of et_col.
template <typename E, int n>
__device__ __forceinline__ void store_run_et(E *row, int c, int t0, const float *x) {
    if constexpr (sizeof(E) == 2 && n % 8 == 0) {  // whole granules: one 16-byte store each
#pragma unroll
        for (int i = 0; i < n; i += 8) {
            bf16x8 v;
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = static_cast<bf16>(x[i + u]);
            *reinterpret_cast<bf16x8 *>(row + et_col<E>(c, t0 + i)) = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < n; i += 4)
            store4<E>(row + et_col<E>(c, t0 + i), f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]});
    }
}

// Lower-triangle 16x16 tiles (I >= J) in a fixed order, dealt to the 4 waves
// round-robin; upper tiles likewise.
__device__ __forceinline__ void lower_tile(int t, int &I, int &J) {
    // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
    I = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
    J = t - (I * (I + 1)) / 2;
}
__device__ __forceinline__ void upper_tile(int t, int &I, int &J) {
    // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    I = t < 3 ? 0 : t < 5 ? 1 : 2;
    J = t < 3 ? t + 1 : t < 5 ? t - 1 : 3;
}

// Token span of chunk `cid`: dense arithmetic, or the device chunk table
// (entries clamped so that a stale or malformed table stays in bounds).
__device__ __forceinline__ void chunk_span(const ChunkArgs &a, int cid, int &tok0, int &len) {
    if (a.plan) {
        const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
        tok0 = min(max(e[1], 0), a.T);
        len = min(max(e[2], 0), min(kChunk, a.T - tok0));
    } else {
        const int n = cid / a.NC, c = cid % a.NC;
        tok0 = n * a.T + c * kChunk;
        len = min(kChunk, a.T - c * kChunk);
    }
}

// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp; the operands are bf16).
__device__ __forceinline__ float sigmoid1(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// kBwd: also write the transposed factors a backward call needs (a.ws_Mt,
// ws_Qt, ws_Tt), and not Qhat or M, which only o needs (its kernels read
// Khat and W^T from Khat^T and W with transposing LDS reads).  kBoth (with
// kBwd): write both sets, for a forward whose factors a later backward reuses.
// kLogits: the gates arrive as bf16 -- log alpha itself and the logits of b
// and w, whose sigmoid is taken here.  kAlphaLogit (with kLogits): log_alpha
// holds logits too, and log alpha = logsigmoid(logit + a.alpha_bias).
// Two workgroups per CU where their LDS fits (fp32 with 128-wide heads needs
// over 80 KB, so one workgroup runs per CU and may use all of its registers).
template <typename E, int DK, bool kBwd, bool kLogits = false, bool kAlphaLogit = false, bool kBoth = false>
__global__ __launch_bounds__(kThreads, (PrepCfg<E, DK>::SMEM <= 80 * 1024 ? 2 : 1)) void chunk_prep_kernel(ChunkArgs a) {
    using C = PrepCfg<E, DK>;
    constexpr bool kFwdOut = !kBwd || kBoth;  // Qhat and M (for o)
    constexpr bool kBwdOut = kBwd || kBoth;   // M^T, Qhat^T, T^T (for a backward)
    using M = Mma<E>;
    constexpr int TPG = C::TPG, LDT = C::LDT, LDC = C::LDC, LDA = C::LDA, LDX = C::LDX;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    E *sKp = reinterpret_cast<E *>(smem);                  // [64][LDT] k e^{g_r-g}
    E *sX = sKp + kChunk * LDT;                            // [64][LDT] b k e^{g-g_r}, then q e^{g-g_r}
    float *sTot = reinterpret_cast<float *>(smem);         // [NTG][DK] group totals (first)
    float *sA = reinterpret_cast<float *>(smem);           // [64][LDA] A, T solved in place
    E *sTb = reinterpret_cast<E *>(smem + C::SZ_A);        // [64][LDC] T as E, row-major
    float *sS = reinterpret_cast<float *>(smem + C::SZ_A + C::SZ_TB);  // [4][16][LDX]
    E *sEt = reinterpret_cast<E *>(smem + C::R1);          // [DK][LDC] (gamma b k)^T, then (w v)^T
    E *sStg = reinterpret_cast<E *>(smem + C::R1 + C::SZ_ET);  // Khat^T, then Qhat image

    // Heads vary fastest across workgroup ids, so that workgroups running at the
    // same time read neighbouring head slices of the same token rows.
    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    chunk_span(a, cid, tok0, len);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qd = tid % C::NQUAD, tg = tid / C::NQUAD;
    const int c0 = 4 * qd;                  // this thread's 4 channels
    const size_t ch = (size_t)cid * H + h;  // chunk-head index into the workspace
    const E *q = reinterpret_cast<const E *>(a.q);
    const E *k = reinterpret_cast<const E *>(a.k);
    const E *v = reinterpret_cast<const E *>(a.v);

    // ---- stage 1: load, cumulative log-decay -------------------------------
    // Every token slot loads unconditionally (from the chunk's last token when
    // the slot is past its length) and padding slots are zeroed afterwards
    // (k = q = b = v = 0, log alpha = 0: an exact no-op).  A load under a
    // per-token branch makes the merge with the other branch's zero wait for
    // the load, which turned the loads into one memory round trip per token.
    // The raw values (bf16 gate logits still bf16) are converted only after
    // every load has been issued.  q and k stay in their input type (exact)
    // until used.
    using GR = typename std::conditional<kLogits, bf16x4, f32x4>::type;  // a gate as loaded
    GR rla[TPG], rb[TPG];
    Vec4<E> kk[TPG], qq[TPG];
    size_t src[TPG];  // element offset of each slot's token row (head h, channel c0)
#pragma unroll
    for (int j = 0; j < TPG; ++j) src[j] = (size_t)(tok0 + max(min(tg * TPG + j, len - 1), 0));
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const size_t off = (src[j] * H + h) * DK + c0;
        if constexpr (kLogits) {
            const size_t offg = src[j] * a.ld_gate + (size_t)h * DK + c0;
            rla[j] = *reinterpret_cast<const GR *>(reinterpret_cast<const bf16 *>(a.log_alpha) + offg);
            rb[j] = *reinterpret_cast<const GR *>(reinterpret_cast<const bf16 *>(a.b) + offg);
        } else {
            rla[j] = *reinterpret_cast<const GR *>(a.log_alpha + off);
            rb[j] = *reinterpret_cast<const GR *>(a.b + off);
        }
        kk[j] = *reinterpret_cast<const Vec4<E> *>(k + off);
        qq[j] = *reinterpret_cast<const Vec4<E> *>(q + off);
    }
    // w and v are multiplied only when (w v)^T is staged, after W: their loads
    // stay in flight through the following phases.
    using GW = GR;  // w, or its logit
    GW zw[TPG];
    Vec4<E> zv[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const size_t off = (src[j] * H + h) * DK + c0;  // Dv == Dk
        if constexpr (kLogits)
            zw[j] = *reinterpret_cast<const GW *>(reinterpret_cast<const bf16 *>(a.w) +
                                                  src[j] * a.ld_gate + (size_t)h * DK + c0);
        else
            zw[j] = *reinterpret_cast<const GW *>(a.w + off);
        zv[j] = *reinterpret_cast<const Vec4<E> *>(v + off);
    }
    f32x4 g[TPG], bk[TPG];
    f32x4 abias = zero4();
    if constexpr (kAlphaLogit) abias = *reinterpret_cast<const f32x4 *>(a.alpha_bias + h * DK + c0);
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const bool pad = tg * TPG + j >= len;
        g[j] = to4(rla[j]);
        if constexpr (kAlphaLogit) {
#pragma unroll
            for (int c = 0; c < 4; ++c) g[j][c] = logsigmoid_fast(g[j][c] + abias[c]);
        }
        bk[j] = to4(rb[j]);
        if constexpr (kLogits) {
#pragma unroll
            for (int c = 0; c < 4; ++c) bk[j][c] = sigmoid1(bk[j][c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            g[j][c] = pad ? 0.0f : g[j][c];
            bk[j][c] = pad ? 0.0f : bk[j][c];
        }
    }
#pragma unroll
    for (int j = 1; j < TPG; ++j) g[j] += g[j - 1];
    *reinterpret_cast<f32x4 *>(sTot + tg * DK + c0) = g[TPG - 1];
    __syncthreads();
    f32x4 goff = zero4(), glast = zero4();
#pragma unroll
    for (int t = 0; t < C::NTG; ++t) {
        const f32x4 tt = *reinterpret_cast<const f32x4 *>(sTot + t * DK + c0);
        if (t < tg) goff += tt;
        glast += tt;
    }
    __syncthreads();  // region 1 is overwritten below
    // Per-channel constants: midpoint reference g_r = g_last/2 and e^{g_r}.
    const f32x4 gr = 0.5f * glast;
    f32x4 egr;
#pragma unroll
    for (int c = 0; c < 4; ++c) egr[c] = __expf(gr[c]);

    // ---- scaled tiles --------------------------------------------------------
    E *Qh = kFwdOut ? reinterpret_cast<E *>(a.ws_Qh) + ch * kChunk * DK : nullptr;
    E *KhT = reinterpret_cast<E *>(a.ws_KhT) + ch * DK * kChunk;
    Vec4<E> qp[TPG], qh[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        const f32x4 gg = g[j] + goff;
        f32x4 ex, ei;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ex[c] = __expf(gg[c] - gr[c]);   // e^{g - g_r}
            ei[c] = __expf(gr[c] - gg[c]);   // e^{g_r - g}
        }
        const bool pad = i >= len;  // padding: k = q = 0
        f32x4 kf = to4(kk[j]), qf = to4(qq[j]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kf[c] = pad ? 0.0f : kf[c];
            qf[c] = pad ? 0.0f : qf[c];
        }
        bk[j] *= kf;
        store4<E>(sX + i * LDT + c0, bk[j] * ex);
        store4<E>(sKp + i * LDT + c0, kf * ei);
        // gamma = e^{g} = e^{g-g_r} e^{g_r};  e^{g_last-g} = e^{g_r-g} e^{g_r}
        const f32x4 gm = ex * egr;
        qh[j] = pack4<E>(qf * gm);    // Qhat, staged once the image region is free
        qp[j] = pack4<E>(qf * ex);    // q e^{g-g_r}, kept for M
        bk[j] *= gm;                  // gamma b k, stored channel-major below
        g[j] = kf * ei * egr;         // e^{g_last-g} k, staged below
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float et[TPG];
#pragma unroll
        for (int j = 0; j < TPG; ++j) et[j] = bk[j][c];
        store_run_et<E, TPG>(sEt + (c0 + c) * LDC, c0 + c, tg * TPG, et);
    }
    if constexpr (kBwdOut) {  // backward calls: Qhat^T, fragment order
        E *QtG = reinterpret_cast<E *>(a.ws_Qt) + ch * DK * kChunk;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int m = 0; m < TPG; m += 4)
                store4_frag<E>(QtG, kChunk, c0 + c, tg * TPG + m,
                               f32x4{elem<E>(qh[m], c), elem<E>(qh[m + 1], c), elem<E>(qh[m + 2], c),
                                     elem<E>(qh[m + 3], c)});
    }
    // Khat^T image: row = channel, column = token.
    if constexpr (sizeof(E) == 2) {  // a granule is 8 tokens of one channel
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float kh[TPG];
#pragma unroll
            for (int j = 0; j < TPG; ++j) kh[j] = g[j][c];
            if constexpr (TPG % 8 == 0) {
#pragma unroll
                for (int m = 0; m < TPG; m += 8) {
                    bf16x8 x;
#pragma unroll
                    for (int u = 0; u < 8; ++u) x[u] = static_cast<bf16>(kh[m + u]);
                    *reinterpret_cast<bf16x8 *>(
                        stage_ptr(sStg, frag_index<E>(c0 + c, tg * TPG + m, kChunk))) = x;
                }
            } else {
#pragma unroll
                for (int m = 0; m < TPG; m += 4)
                    store4<E>(stage_ptr(sStg, frag_index<E>(c0 + c, tg * TPG + m, kChunk)),
                              f32x4{kh[m], kh[m + 1], kh[m + 2], kh[m + 3]});
            }
        }
    } else {  // a granule is 4 channels of one token
#pragma unroll
        for (int j = 0; j < TPG; ++j)
            *reinterpret_cast<f32x4 *>(stage_ptr(sStg, frag_index<E>(c0, tg * TPG + j, kChunk))) =
                g[j];
    }
    if (tg == 0) {
        f32x4 gl;
#pragma unroll
        for (int c = 0; c < 4; ++c) gl[c] = __expf(glast[c]);
        *reinterpret_cast<f32x4 *>(a.ws_gl + ch * DK + c0) = gl;
    }
    __syncthreads();

    // ---- stage 2a: A (then M) by MFMA over the channels -------------------
    // Tile (I, J), I >= J, is formed transposed: D[j][i] = sum_c Kp[j][c] Y[i][c],
    // so each lane ends up with 4 consecutive columns j of one row i.
    stage_copy_out<E, C::NG>(KhT, sStg, tid);
    f32x4 accA[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int t = wave + 4 * u;
        accA[u] = zero4();
        if (t < 10) {
            int I, J;
            lower_tile(t, I, J);
            f32x4 acc = mma_tile<E, DK>(zero4(), sKp + 16 * J * LDT, LDT, sX + 16 * I * LDT, LDT,
                                        lane);
            const int i = 16 * I + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J + 4 * (lane >> 4) + r;
                acc[r] = j < i ? acc[r] : 0.0f;
            }
            accA[u] = acc;
        }
    }
    __syncthreads();  // Ep and the Khat^T image are dead: X receives q e^{g-g_r}, the image Qhat
#pragma unroll
    for (int j = 0; j < TPG; ++j) *reinterpret_cast<Vec4<E> *>(sX + (tg * TPG + j) * LDT + c0) = qp[j];
    // (A backward call needs neither Qhat nor M: its propagation forms no o.)
    if constexpr (!kFwdOut) {
    } else if constexpr (sizeof(E) == 2) {  // a granule is 8 channels of one token
#pragma unroll
        for (int j = 0; j < TPG; ++j)
            *reinterpret_cast<Vec4<E> *>(stage_ptr(sStg, frag_index<E>(tg * TPG + j, c0, DK))) = qh[j];
    } else {  // a granule is 4 tokens of one channel
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int m = 0; m < TPG; m += 4)
                *reinterpret_cast<f32x4 *>(stage_ptr(sStg, frag_index<E>(tg * TPG + m, c0 + c, DK))) =
                    f32x4{qh[m][c], qh[m + 1][c], qh[m + 2][c], qh[m + 3][c]};
    }
    __syncthreads();
    if constexpr (kFwdOut) stage_copy_out<E, C::NG>(Qh, sStg, tid);
    E *Mg = kFwdOut ? reinterpret_cast<E *>(a.ws_M) + ch * kChunk * kChunk : nullptr;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int t = wave + 4 * u;
        if (t < 10) {
            int I, J;
            lower_tile(t, I, J);
            if constexpr (kFwdOut) {
                f32x4 acc = mma_tile<E, DK>(zero4(), sKp + 16 * J * LDT, LDT, sX + 16 * I * LDT, LDT,
                                            lane);
                const int i = 16 * I + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J + 4 * (lane >> 4) + r;
                    acc[r] = j <= i ? acc[r] : 0.0f;
                }
                store4_frag_nt<E>(Mg, kChunk, i, 16 * J + 4 * (lane >> 4), acc);
            }
            if constexpr (kBwdOut) {  // M^T[j][i] = M[i][j]: the same tile with the operands swapped
                f32x4 t = mma_tile<E, DK>(zero4(), sX + 16 * I * LDT, LDT, sKp + 16 * J * LDT, LDT, lane);
                const int jj = 16 * J + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) t[r] = jj <= 16 * I + 4 * (lane >> 4) + r ? t[r] : 0.0f;
                store4_frag<E>(reinterpret_cast<E *>(a.ws_Mt) + ch * kChunk * kChunk, kChunk, jj,
                               16 * I + 4 * (lane >> 4), t);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // zero blocks of M above the diagonal
        const int t = wave + 4 * u;
        if (t < 6) {
            int I, J;
            upper_tile(t, I, J);
            // Only the zero blocks inside an operand fragment that also holds
            // elements on or below the diagonal are written (and read): the
            // fragments wholly above it are skipped by the propagation.
            if constexpr (kFwdOut) {
                if (m_frag_used<E>(I, 16 * J)) {
                    // A zero made here: a loop-invariant zero register would be
                    // spilled, and its reload waits for every load in flight.
                    float z;
                    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
                    store4_frag<E>(Mg, kChunk, 16 * I + (lane & 15), 16 * J + 4 * (lane >> 4),
                                   f32x4{z, z, z, z});
                }
            }
            if constexpr (kBwdOut) {  // the zero lower blocks of M^T
                store4_frag<E>(reinterpret_cast<E *>(a.ws_Mt) + ch * kChunk * kChunk, kChunk,
                               16 * J + (lane & 15), 16 * I + 4 * (lane >> 4), zero4());
            }
        }
    }
    __syncthreads();  // the token-major tiles are dead: region 1 becomes the solve buffers
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int t = wave + 4 * u;
        if (t < 10) {
            int I, J;
            lower_tile(t, I, J);
            // A_IJ row-major below the diagonal; the diagonal blocks transposed
            // (A_II^T), so that the substitution below reads columns as rows.
            if (I == J) store_tile<float>(sA + 16 * I * LDA + 16 * I, LDA, accA[u], lane);
            else store_tile_t<float>(sA + 16 * I * LDA + 16 * J, LDA, accA[u], lane);
        }
    }
    // T as E (sTb, row-major) is written block by block by the solve below;
    // its strictly upper blocks are zero.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = wave + 4 * u;
        if (t < 6) {
            int I, J;
            upper_tile(t, I, J);
            store_tile<E>(sTb + 16 * I * LDC + 16 * J, LDC, zero4(), lane);
        }
    }
    __syncthreads();

    // ---- stage 2b: T = (I + A)^-1 in fp32, in place ------------------------
    // Diagonal blocks: forward substitution, one column c of T_II per lane,
    // eliminating one unknown at a time (so the updates of the later rows are
    // independent of each other); column j of A_II is row j of the stored
    // A_II^T.  T_II then overwrites the block, row-major.
    if (wave == 0) {
        const int I = lane >> 4, c = lane & 15;
        float *Ab = sA + 16 * I * LDA + 16 * I;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
            const float *colj = Ab + j * LDA;  // A_II[i][j] at colj[i]
#pragma unroll
            for (int i = j + 1; i < 16; ++i) x[i] -= colj[i] * x[j];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Ab[i * LDA + c] = x[i];
            sTb[(16 * I + i) * LDC + 16 * I + c] = from_f32<E>(x[i]);
        }
    }
    __syncthreads();
    // Off-diagonal blocks, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, grouped as
    // 2x2 super-blocks T = [[Ta, 0], [Tc, Tb]] with Tc = -Tb (Ac Ta): three
    // dependent phases of at most two 16x16 products per wave.  T_IJ (I > J)
    // is stored transposed in the free upper block (J, I); sS slot w holds
    // wave w's intermediate X blocks.
    {
        auto blk = [&](int I, int J) { return sA + 16 * I * LDA + 16 * J; };
        const float *T10 = blk(0, 1), *T32 = blk(2, 3);  // transposed: X[m][k] at X[k*LDA + m]
        auto slot = [&](int w) { return sS + w * 16 * LDX; };
        auto put_T = [&](int I, int J, f32x4 t) {
            store_tile_t<float>(sA + 16 * J * LDA + 16 * I, LDA, t, lane);
            store_tile<E>(sTb + 16 * I * LDC + 16 * J, LDC, t, lane);
        };
        if (wave < 2) {  // T_10 (wave 0), T_32 (wave 1) = -T_II (A_IJ T_JJ)
            const int J = 2 * wave, I = J + 1;
            store_tile<float>(slot(wave), LDX, mma16_f32(zero4(), blk(I, J), LDA, 1, blk(J, J), LDA, 1, lane),
                              lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            put_T(I, J, -mma16_f32(zero4(), blk(I, I), LDA, 1, slot(wave), LDX, 1, lane));
        } else {  // X_21 (wave 2), X_31 (wave 3) = A_I1 T_11
            store_tile<float>(slot(wave), LDX, mma16_f32(zero4(), blk(wave, 1), LDA, 1, blk(1, 1), LDA, 1, lane),
                              lane);
        }
        __syncthreads();
        if (wave < 2) {  // X_20 (wave 0), X_30 (wave 1) = A_I0 T_00 + A_I1 T_10
            const int I = 2 + wave;
            f32x4 x = mma16_f32(zero4(), blk(I, 0), LDA, 1, blk(0, 0), LDA, 1, lane);
            x = mma16_f32(x, blk(I, 1), LDA, 1, T10, 1, LDA, lane);
            store_tile<float>(slot(wave), LDX, x, lane);
        } else if (wave == 2) {  // T_21 = -T_22 X_21
            put_T(2, 1, -mma16_f32(zero4(), blk(2, 2), LDA, 1, slot(2), LDX, 1, lane));
        } else {  // T_31 = -(T_32 X_21 + T_33 X_31)
            f32x4 t = mma16_f32(zero4(), T32, 1, LDA, slot(2), LDX, 1, lane);
            t = mma16_f32(t, blk(3, 3), LDA, 1, slot(3), LDX, 1, lane);
            put_T(3, 1, -t);
        }
        __syncthreads();
        if (wave == 0) {  // T_20 = -T_22 X_20
            put_T(2, 0, -mma16_f32(zero4(), blk(2, 2), LDA, 1, slot(0), LDX, 1, lane));
        } else if (wave == 1) {  // T_30 = -(T_32 X_20 + T_33 X_30)
            f32x4 t = mma16_f32(zero4(), T32, 1, LDA, slot(0), LDX, 1, lane);
            t = mma16_f32(t, blk(3, 3), LDA, 1, slot(1), LDX, 1, lane);
            put_T(3, 0, -t);
        }
        __syncthreads();
    }

    // ---- optionally T itself (row-major, from its E copy) ---------------
    if (a.store_T) {
        const int row = tid >> 2, col0 = 16 * (tid & 3);
        E *Tg = reinterpret_cast<E *>(a.ws_T) + ch * kChunk * kChunk + row * kChunk + col0;
#pragma unroll
        for (int j = 0; j < 16; j += 4)
            *reinterpret_cast<Vec4<E> *>(Tg + j) = *reinterpret_cast<const Vec4<E> *>(sTb + row * LDC + col0 + j);
    }
    if constexpr (kBwdOut && sizeof(E) == 2) {  // T^T in fragment order: rows i, columns j = T[j][i]
        E *TtG = reinterpret_cast<E *>(a.ws_Tt) + ch * kChunk * kChunk;
        for (int gi = tid; gi < kChunk * kChunk / 8; gi += kThreads) {
            const int blk = gi >> 6, lp = gi & 63;
            const int i = (blk >> 1) * 16 + (lp & 15), j0 = (blk & 1) * 32 + (lp >> 4) * 8;
            bf16x8 x;
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = sTb[(j0 + t) * LDC + i];
            *reinterpret_cast<bf16x8 *>(TtG + (size_t)gi * 8) = x;
        }
    }

    // ---- stage 3: W = T (gamma b k), formed transposed ---------------------
    // D[c][i] = sum_j Et[c][j] T[i][j]; lane holds W[i][c..c+3].
    {
        E *Wg = reinterpret_cast<E *>(a.ws_W) + ch * kChunk * DK;
        constexpr int CBW = DK / 64;  // channel blocks per wave
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) {
            const int cblk = wave * CBW + cb;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                constexpr int KS = M::KS;
                const int K = ((16 * (I + 1) + KS - 1) / KS) * KS;
                f32x4 acc = mma_tile_swz<E>(zero4(), sEt + 16 * cblk * LDC, LDC, cblk & 7,
                                            sTb + 16 * I * LDC, LDC, 0, K, lane);
                store4_frag_nt<E>(Wg, DK, 16 * I + (lane & 15), 16 * cblk + 4 * (lane >> 4), acc);
            }
        }
    }

    __syncthreads();  // (gamma b k)^T is dead: region 2 receives (w v)^T
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float zt[TPG];
#pragma unroll
        for (int j = 0; j < TPG; ++j) {
            float wv;
            if constexpr (kLogits) wv = sigmoid1(static_cast<float>(zw[j][c]));
            else wv = zw[j][c];
            zt[j] = tg * TPG + j < len ? wv * elem<E>(zv[j], c) : 0.0f;  // padding: v = 0
        }
        store_run_et<E, TPG>(sEt + (c0 + c) * LDC, c0 + c, tg * TPG, zt);
    }
    __syncthreads();

    // ---- stage 3: U = T (w v) in MFMA accumulator order -------------------
    // D[i][col] = sum_j T[i][j] Z^T[col][j]; tile (I, cb) is stored as
    // U[ch][I][cb][lane][r] = U[16I + 4(lane/16) + r][16cb + lane%16].
    {
        E *Ug = reinterpret_cast<E *>(a.ws_U) + ch * kChunk * DK;
        constexpr int NCBU = DK / 16;
        const int I = wave;
        constexpr int KS = M::KS;
        const int K = ((16 * (I + 1) + KS - 1) / KS) * KS;
#pragma unroll
        for (int cb = 0; cb < NCBU; ++cb) {
            f32x4 acc = mma_tile_swz<E>(zero4(), sTb + 16 * I * LDC, LDC, 0, sEt + 16 * cb * LDC, LDC,
                                        cb & 7, K, lane);
            if constexpr (sizeof(E) == 2) {
                bf16x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = static_cast<bf16>(acc[j]);
                __builtin_nontemporal_store(b, reinterpret_cast<bf16x4 *>(Ug + ((I * NCBU + cb) * 64 + lane) * 4));
            } else {
                store4<E>(Ug + ((I * NCBU + cb) * 64 + lane) * 4, acc);
            }
        }
    }
}

hipError_t launch_chunk_prep(const ChunkArgs &a, int Dk, bool bf16_io, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)a.max_chunks * a.H)), block(kThreads);
    if (bf16_io && a.gate_logits && a.alpha_bias) {  // all three gates as logits
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128, false, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64, false, true, true>), grid, block, 0, stream, a);
    } else if (bf16_io && a.gate_logits) {  // bf16 gates, sigmoid in the kernel (forward only)
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64, false, true>), grid, block, 0, stream, a);
    } else if (bf16_io && a.ws_Mt && a.ws_Qh) {  // forward for a later backward: both factor sets
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128, true, false, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64, true, false, false, true>), grid, block, 0, stream, a);
    } else if (bf16_io && a.ws_Mt) {  // backward calls (bf16 only)
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64, true>), grid, block, 0, stream, a);
    } else if (bf16_io) {
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<bf16, 128, false>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<bf16, 64, false>), grid, block, 0, stream, a);
    } else {
        if (Dk == 128) hipLaunchKernelGGL((chunk_prep_kernel<float, 128, false>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((chunk_prep_kernel<float, 64, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gdn2
