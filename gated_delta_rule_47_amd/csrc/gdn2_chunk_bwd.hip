// Chunkwise backward of the chunk forward (bf16 I/O).
//
// The pages name a gate-aware backward as one of the method's contributions
// (gist.science summary, part "3. Efficient chunkwise parallel training", item
// on the backward pass: the channel-wise gates b and w enter the gradients of
// the chunk's auxiliary matrices directly) without printing it; what follows
// is the chain rule of the chunk form used by the forward.  Per chunk, with
// incoming state S, gradient dS' of the outgoing state and output gradient dO:
//
//   forward   U_eff = U - W S,  O = Qhat S + M U_eff,  S' = Diag(gl) S + Khat^T U_eff
//   reverse   dU_eff = M^T dO + Khat dS'
//             dS     = Diag(gl) dS' + Qhat^T dO - W^T dU_eff        (carried to the previous chunk)
//   state side   dQhat = dO S^T,  dW = -dU_eff S^T,  dKhat = U_eff dS'^T,
//                dM = tril(dO U_eff^T),  dgl = rowsum(dS' * S),  dZ = T^T dU_eff,
//                dv = w * dZ,  dw = v * dZ
//   factor side  dE = T^T dW,  dA = -strict_tril(dZ U^T + dE W^T),
//                dEp = dA Kp,  dQp = dM Kp,  dKp = dA^T Ep + dM^T Qp
// where T = (I + A)^-1, W = T E, U = T Z, E = gamma*b*k, Z = w*v, and Ep, Kp, Qp
// are the midpoint-scaled tiles of the forward (A = strict_tril(Ep Kp^T),
// M = tril(Qp Kp^T)).  Per token i and key channel c (ex = e^{g-g_r},
// ei = e^{g_r-g}, eK = e^{g_last-g}, gamma = e^g):
//   dq = gamma dQhat + ex dQp,   db = k (gamma dE + ex dEp),
//   dk = b (gamma dE + ex dEp) + ei dKp + eK dKhat,
//   dg = E dE + Ep dEp + Qhat dQhat + Qp dQp - Kp dKp - Khat dKhat,
//   dlog_alpha_j = sum_{i>=j} dg_i + gl dgl + sum_i Khat_i dKhat_i.
//
// Three kernels after the forward (chunk factors with T, and the propagation
// storing every chunk's incoming state):
//   chunk_bwd_rev_kernel     sequential over the chunks of a sequence, in
//                            reverse: dU_eff and dS, storing each chunk's dS'
//   chunk_bwd_state_kernel   per chunk: the state-side products, dv and dw
//   chunk_bwd_factor_kernel  per chunk: the factor side, dq, dk, db, dlog_alpha
// The products are fp32 MFMA (16x16x4) with operands read element by element
// from LDS, so every operand can keep the layout it was stored in.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

typedef unsigned int granule_t __attribute__((ext_vector_type(4)));

// Element (r, k) of a fragment-ordered bf16 matrix with K columns.
__device__ __forceinline__ float fe(const bf16 *X, int K, int r, int k) {
    return static_cast<float>(X[frag_index<bf16>(r, k, K)]);
}

// acc += A B^T over K (a multiple of 4) for one 16x16 tile with fp32 MFMA:
// a(m, k) = A[m][k], b(n, k) = B[n][k] for the tile's rows m and columns n.
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 mma_f32(f32x4 acc, int lane, const FA &a, const FB &b) {
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll 8
    for (int kk = 0; kk < K; kk += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m, kk + kq), b(m, kk + kq), acc, 0, 0, 0);
    return acc;
}

// Copy `bytes` (a multiple of 16) from global to LDS, 16 bytes per thread.
__device__ __forceinline__ void copy16(void *dst, const void *src, int bytes, int tid, int nthr) {
    const granule_t *s = reinterpret_cast<const granule_t *>(src);
    granule_t *d = reinterpret_cast<granule_t *>(dst);
    for (int i = tid; i < bytes / 16; i += nthr) d[i] = s[i];
}

__device__ __forceinline__ void chunk_span_of(const ChunkArgs &a, int cid, int cbeg, int n, int &tok0,
                                              int &len) {
    if (a.plan) {
        const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
        tok0 = min(max(e[1], 0), a.T);
        len = min(max(e[2], 0), min(kChunk, a.T - tok0));
    } else {
        const int c = cid - cbeg;
        tok0 = n * a.T + c * kChunk;
        len = min(kChunk, a.T - c * kChunk);
    }
}

__device__ __forceinline__ void seq_chunks(const ChunkArgs &a, int n, int &cbeg, int &cend) {
    if (a.plan) {
        cbeg = min(max(a.plan[n], 0), a.max_chunks);
        cend = min(max(a.plan[n + 1], cbeg), a.max_chunks);
    } else {
        cbeg = n * a.NC;
        cend = cbeg + a.NC;
    }
}

__device__ __forceinline__ void dense_span(const ChunkArgs &a, int cid, int &tok0, int &len) {
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

}  // namespace

// ---------------------------------------------------------------------------
// Reverse pass: one workgroup per (sequence, head, DVS-column slab), the
// chunks of the sequence from last to first, bf16 MFMA.  dS' lives in fp32
// accumulators (wave w owns state rows 16 (w*KB_W + b) .. of the slab, like
// the forward); its bf16 transpose in LDS is the operand of Khat dS'.  The
// factors are the transposed copies the chunk-factor kernel writes for
// backward calls (M^T, Khat, Qhat^T, W^T), loaded as fragments.
// ---------------------------------------------------------------------------
template <int DK, int DVS>
struct RevCfg {
    static constexpr int DV = DK, NS = DV / DVS, NCB = DVS / 16, NKB = DK / 16;
    static constexpr int KB_W = NKB / 4, S_TPW = KB_W * NCB;
    static constexpr int LDKP = DK + 8, L64 = kChunk + 8;
};

template <int DK, int DVS>
__global__ __launch_bounds__(kThreads, 1) void chunk_bwd_rev_kernel(BwdArgs ba) {
    using C = RevCfg<DK, DVS>;
    using MB = Mma<bf16>;
    constexpr int DV = C::DV, NCB = C::NCB, LDKP = C::LDKP, L64 = C::L64, NKD = DK / 32;
    const ChunkArgs &a = ba.c;
    __shared__ __attribute__((aligned(16))) bf16 sdSt[DVS * LDKP];  // [v][c] = dS'[c][v]
    __shared__ __attribute__((aligned(16))) bf16 sdOt[DVS * L64];   // [v][i] = dO[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdUt[DVS * L64];   // [v][i] = dU_eff[i][v]

    const int H = a.H;
    const int x = blockIdx.x, xcd = x & 7, rest = x >> 3;
    const int slab = rest % C::NS, chain = (rest / C::NS) * 8 + xcd;
    if (chain >= a.N * H) return;
    const int n = chain / H, h = chain % H, col0 = slab * DVS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int cbeg, cend;
    seq_chunks(a, n, cbeg, cend);

    f32x4 dS[C::S_TPW];
#pragma unroll
    for (int u = 0; u < C::S_TPW; ++u) {
        const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * cblk + 4 * (lane >> 4) + r, col = col0 + 16 * colb + (lane & 15);
            dS[u][r] = ba.dS_final ? ba.dS_final[((size_t)chain * DK + row) * DV + col] : 0.0f;
        }
    }
    const bf16 *dout = reinterpret_cast<const bf16 *>(ba.dout);
    for (int cid = cend - 1; cid >= cbeg; --cid) {
        const size_t ch = (size_t)cid * H + h;
        int tok0, len;
        chunk_span_of(a, cid, cbeg, n, tok0, len);
        // Fragments of this chunk: M^T and Khat rows of block `wave`, Qhat^T
        // and W^T rows of this wave's state row blocks; gamma_last.
        const bf16 *Mt = reinterpret_cast<const bf16 *>(a.ws_Mt) + ch * kChunk * kChunk;
        const bf16 *Kh = reinterpret_cast<const bf16 *>(a.ws_Kh) + ch * kChunk * DK;
        const bf16 *Qt = reinterpret_cast<const bf16 *>(a.ws_Qt) + ch * DK * kChunk;
        const bf16 *Wt = reinterpret_cast<const bf16 *>(a.ws_Wt) + ch * DK * kChunk;
        MB::frag fM[2], fK[NKD], fQ[C::KB_W][2], fW[C::KB_W][2];
        f32x4 gl[C::KB_W];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) fM[kk] = load_frag_packed<bf16>(Mt, kChunk, wave, kk, lane);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) fK[kk] = load_frag_packed<bf16>(Kh, DK, wave, kk, lane);
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b) {
            const int cblk = wave * C::KB_W + b;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                fQ[b][kk] = load_frag_packed<bf16>(Qt, kChunk, cblk, kk, lane);
                fW[b][kk] = load_frag_packed<bf16>(Wt, kChunk, cblk, kk, lane);
            }
            gl[b] = *reinterpret_cast<const f32x4 *>(a.ws_gl + ch * DK + 16 * cblk + 4 * (lane >> 4));
        }
        // dS' of this chunk: to the workspace (fp32, for the per-chunk kernels)
        // and, transposed, to LDS.
        float *dSc = ba.dSc + ch * DK * DV;
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dSc[(size_t)(16 * cblk + 4 * (lane >> 4) + r) * DV + col0 + 16 * colb + (lane & 15)] = dS[u][r];
            store_tile_t<bf16>(sdSt + 16 * colb * LDKP + 16 * cblk, LDKP, dS[u], lane);
        }
        // dO rows of the chunk (zero past its end), transposed.
        for (int e = tid; e < kChunk * DVS / 4; e += kThreads) {
            const int i = e / (DVS / 4), c4 = 4 * (e % (DVS / 4));
            bf16x4 v4;
            if (i < len) {
                v4 = *reinterpret_cast<const bf16x4 *>(dout + ((size_t)(tok0 + i) * H + h) * DV + col0 + c4);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) v4[t] = static_cast<bf16>(0.0f);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) sdOt[(c4 + t) * L64 + i] = v4[t];
        }
        __syncthreads();

        // dU_eff rows of block `wave`:  M^T dO + Khat dS'.
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                acc = MB::mma(fM[kk], load_frag<bf16>(sdOt + 16 * cb * L64 + 32 * kk, L64, lane), acc);
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)
                acc = MB::mma(fK[kk], load_frag<bf16>(sdSt + 16 * cb * LDKP + 32 * kk, LDKP, lane), acc);
            store_tile_t<bf16>(sdUt + 16 * cb * L64 + 16 * wave, L64, acc, lane);
        }
        __syncthreads();

        // dS <- Diag(gl) dS' + Qhat^T dO - W^T dU_eff.
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int b = u / NCB, colb = u % NCB;
            f32x4 q = zero4(), wu = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                q = MB::mma(fQ[b][kk], load_frag<bf16>(sdOt + 16 * colb * L64 + 32 * kk, L64, lane), q);
                wu = MB::mma(fW[b][kk], load_frag<bf16>(sdUt + 16 * colb * L64 + 32 * kk, L64, lane), wu);
            }
            dS[u] = gl[b] * dS[u] + q - wu;
        }
        __syncthreads();
    }
    if (ba.dS0) {
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * cblk + 4 * (lane >> 4) + r, col = col0 + 16 * colb + (lane & 15);
                ba.dS0[((size_t)chain * DK + row) * DV + col] = dS[u][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// State side, one workgroup per (chunk, head): the products with S and dS',
// taken over 32-column slabs of the value axis with bf16 MFMA (16x16x32).
// Every operand is staged in LDS in the orientation its fragment load wants
// (k contiguous), transposing on the way in where needed.  Wave w owns token
// rows 16w .. 16w+15 of every 64-row result.
// ---------------------------------------------------------------------------
template <int DK>
struct StateCfg {
    static constexpr int DV = DK, SW = 32, NSL = DV / SW, NKB = DK / 16;
    static constexpr int LSW = SW + 8;     // [..][SW] bf16 rows
    static constexpr int LDKP = DK + 8;    // [..][DK] bf16 rows
    static constexpr int L64 = kChunk + 8; // [..][64] bf16 rows
};

// Scatter 8 consecutive elements of row r (columns k..k+7) of a fragment-ordered
// source into a transposed LDS array: dst[(k + t) * ld + r].
__device__ __forceinline__ void scatter_t8(bf16 *dst, int ld, int r, int k, granule_t g8) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(&g8);
#pragma unroll
    for (int t = 0; t < 8; ++t) dst[(k + t) * ld + r] = v[t];
}

// Row and first column of granule `gi` (8 elements) of a fragment-ordered bf16
// matrix with K columns.
__device__ __forceinline__ void frag_granule_pos(int gi, int K, int &r, int &k) {
    const int blk = gi >> 6, lp = gi & 63, nkb = K / 32;
    r = (blk / nkb) * 16 + (lp & 15);
    k = (blk % nkb) * 32 + (lp >> 4) * 8;
}

template <int DK>
__global__ __launch_bounds__(kThreads, 1) void chunk_bwd_state_kernel(BwdArgs ba) {
    using C = StateCfg<DK>;
    using MB = Mma<bf16>;
    constexpr int DV = C::DV, SW = C::SW, NKB = C::NKB, LSW = C::LSW, LDKP = C::LDKP, L64 = C::L64;
    constexpr int NKD = DK / 32;
    const ChunkArgs &a = ba.c;
    // persistent
    __shared__ __attribute__((aligned(16))) bf16 sW[kChunk * DK];    // W, fragment order
    __shared__ __attribute__((aligned(16))) bf16 sMt[kChunk * L64];  // [i][j] = M[j][i]
    __shared__ __attribute__((aligned(16))) bf16 sKh[kChunk * LDKP]; // [i][c] = Khat[i][c]
    __shared__ __attribute__((aligned(16))) bf16 sTt[kChunk * L64];  // [i][j] = T[j][i]
    // per slab
    __shared__ __attribute__((aligned(16))) bf16 sSt[SW * LDKP];     // [v][c] = S[c][v]
    __shared__ __attribute__((aligned(16))) bf16 sS[DK * LSW];       // [c][v]
    __shared__ __attribute__((aligned(16))) bf16 sdSt[SW * LDKP];    // [v][c] = dS'[c][v]
    __shared__ __attribute__((aligned(16))) bf16 sdS[DK * LSW];      // [c][v]
    __shared__ __attribute__((aligned(16))) bf16 sdOt[SW * L64];     // [v][j] = dO[j][v]
    __shared__ __attribute__((aligned(16))) bf16 sdO[kChunk * LSW];  // [i][v]
    __shared__ __attribute__((aligned(16))) bf16 sU[kChunk * LSW];   // [j][v] = U[j][v]
    __shared__ __attribute__((aligned(16))) bf16 sUe[kChunk * LSW];  // [i][v] = U_eff
    __shared__ __attribute__((aligned(16))) bf16 sdUt[SW * L64];     // [v][i] = dU_eff[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdU[kChunk * LSW];  // [i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdZ[kChunk * LSW];  // [i][v]

    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    dense_span(a, cid, tok0, len);
    const size_t ch = (size_t)cid * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, I = wave;
    const bf16 *dout = reinterpret_cast<const bf16 *>(ba.dout);
    const bf16 *vin = reinterpret_cast<const bf16 *>(a.v);
    const bf16 *Ug = reinterpret_cast<const bf16 *>(a.ws_U) + ch * kChunk * DV;
    bf16 *dv = reinterpret_cast<bf16 *>(ba.dv);

    // ---- persistent operands ---------------------------------------------
    copy16(sW, reinterpret_cast<const bf16 *>(a.ws_W) + ch * kChunk * DK, kChunk * DK * 2, tid, kThreads);
    {
        const granule_t *Mg = reinterpret_cast<const granule_t *>(a.ws_M) + ch * (kChunk * kChunk / 8);
        for (int gi = tid; gi < kChunk * kChunk / 8; gi += kThreads) {
            int r, k;
            frag_granule_pos(gi, kChunk, r, k);   // M[r][k..k+7] -> sMt[k+t][r]
            scatter_t8(sMt, L64, r, k, Mg[gi]);
        }
        const granule_t *Kg = reinterpret_cast<const granule_t *>(a.ws_KhT) + ch * (DK * kChunk / 8);
        for (int gi = tid; gi < DK * kChunk / 8; gi += kThreads) {
            int r, k;
            frag_granule_pos(gi, kChunk, r, k);   // KhT[c = r][i = k..k+7] -> sKh[i][c]
            scatter_t8(sKh, LDKP, r, k, Kg[gi]);
        }
        const granule_t *Tg = reinterpret_cast<const granule_t *>(a.ws_T) + ch * (kChunk * kChunk / 8);
        for (int gi = tid; gi < kChunk * kChunk / 8; gi += kThreads)  // T row-major [j][i..i+7]
            scatter_t8(sTt, L64, gi / 8, 8 * (gi % 8), Tg[gi]);
    }

    f32x4 dQh[NKB], dWt[NKB], dKh[NKB], dMa[4], dAp[4];
#pragma unroll
    for (int j = 0; j < NKB; ++j) dQh[j] = dWt[j] = dKh[j] = zero4();
#pragma unroll
    for (int j = 0; j < 4; ++j) dMa[j] = dAp[j] = zero4();
    const float *Sc = ba.Sc + ch * DK * DV;
    const float *dSc = ba.dSc + ch * DK * DV;

    for (int sl = 0; sl < C::NSL; ++sl) {
        const int v0 = sl * SW;
        // S and dS' columns v0..v0+SW: [c][v] and transposed [v][c].
        for (int e = tid; e < DK * SW / 4; e += kThreads) {
            const int c = e / (SW / 4), v4 = 4 * (e % (SW / 4));
            const f32x4 s4 = *reinterpret_cast<const f32x4 *>(Sc + (size_t)c * DV + v0 + v4);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dSc + (size_t)c * DV + v0 + v4);
            bf16x4 sb, db;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sb[t] = static_cast<bf16>(s4[t]);
                db[t] = static_cast<bf16>(d4[t]);
                sSt[(v4 + t) * LDKP + c] = sb[t];
                sdSt[(v4 + t) * LDKP + c] = db[t];
            }
            *reinterpret_cast<bf16x4 *>(sS + c * LSW + v4) = sb;
            *reinterpret_cast<bf16x4 *>(sdS + c * LSW + v4) = db;
        }
        // dO rows (zero past the chunk) and U, [i][v] and transposed.
        for (int e = tid; e < kChunk * SW / 4; e += kThreads) {
            const int i = e / (SW / 4), v4 = 4 * (e % (SW / 4));
            bf16x4 o4;
            if (i < len) {
                o4 = *reinterpret_cast<const bf16x4 *>(dout + ((size_t)(tok0 + i) * H + h) * DV + v0 + v4);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) o4[t] = static_cast<bf16>(0.0f);
            }
            *reinterpret_cast<bf16x4 *>(sdO + i * LSW + v4) = o4;
#pragma unroll
            for (int t = 0; t < 4; ++t) sdOt[(v4 + t) * L64 + i] = o4[t];
            // U in accumulator order: [I][cb][lane][r] = U[16I + 4(lane/16) + r][16cb + lane%16]
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int col = v0 + v4 + t, ul = 16 * ((i & 15) >> 2) + (col & 15);
                sU[i * LSW + v4 + t] = Ug[(((size_t)(i >> 4) * (DV / 16) + (col >> 4)) * 64 + ul) * 4 + (i & 3)];
            }
        }
        __syncthreads();

        // U_eff = U - W S and dU_eff = M^T dO + Khat dS' on this slab (rows of block I).
#pragma unroll
        for (int cb = 0; cb < SW / 16; ++cb) {
            f32x4 ws = zero4(), du = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                ws = MB::mma(load_frag_packed<bf16>(sW, DK, I, kk, lane),
                             load_frag<bf16>(sSt + 16 * cb * LDKP + 32 * kk, LDKP, lane), ws);
                du = MB::mma(load_frag<bf16>(sKh + 16 * I * LDKP + 32 * kk, LDKP, lane),
                             load_frag<bf16>(sdSt + 16 * cb * LDKP + 32 * kk, LDKP, lane), du);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                du = MB::mma(load_frag<bf16>(sMt + 16 * I * L64 + 32 * kk, L64, lane),
                             load_frag<bf16>(sdOt + 16 * cb * L64 + 32 * kk, L64, lane), du);
            // U tile in accumulator order straight from the workspace.
            const bf16x4 u4 = *reinterpret_cast<const bf16x4 *>(
                Ug + (((size_t)I * (DV / 16) + (v0 / 16 + cb)) * 64 + lane) * 4);
            f32x4 ue;
#pragma unroll
            for (int r = 0; r < 4; ++r) ue[r] = static_cast<float>(u4[r]) - ws[r];
            store_tile<bf16>(sUe + 16 * I * LSW + 16 * cb, LSW, ue, lane);
            store_tile<bf16>(sdU + 16 * I * LSW + 16 * cb, LSW, du, lane);
            store_tile_t<bf16>(sdUt + 16 * cb * L64 + 16 * I, L64, du, lane);
        }
        __syncthreads();

        // dZ = T^T dU_eff; dv = w dZ, dw = v dZ.
#pragma unroll
        for (int cb = 0; cb < SW / 16; ++cb) {
            f32x4 dz = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                dz = MB::mma(load_frag<bf16>(sTt + 16 * I * L64 + 32 * kk, L64, lane),
                             load_frag<bf16>(sdUt + 16 * cb * L64 + 32 * kk, L64, lane), dz);
            store_tile<bf16>(sdZ + 16 * I * LSW + 16 * cb, LSW, dz, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * (lane >> 4) + r, vv = 16 * cb + (lane & 15);
                if (i < len) {
                    const size_t o = ((size_t)(tok0 + i) * H + h) * DV + v0 + vv;
                    dv[o] = static_cast<bf16>(a.w[o] * dz[r]);
                    ba.dw[o] = static_cast<float>(vin[o]) * dz[r];
                }
            }
        }
        // Products accumulated over the slabs (k = the slab's 32 columns).
        {
            const MB::frag fdO = load_frag<bf16>(sdO + 16 * I * LSW, LSW, lane);
            const MB::frag fdU = load_frag<bf16>(sdU + 16 * I * LSW, LSW, lane);
            const MB::frag fUe = load_frag<bf16>(sUe + 16 * I * LSW, LSW, lane);
#pragma unroll
            for (int cb = 0; cb < NKB; ++cb) {
                const MB::frag fS = load_frag<bf16>(sS + 16 * cb * LSW, LSW, lane);
                dQh[cb] = MB::mma(fdO, fS, dQh[cb]);
                dWt[cb] = MB::mma(fdU, fS, dWt[cb]);
                dKh[cb] = MB::mma(fUe, load_frag<bf16>(sdS + 16 * cb * LSW, LSW, lane), dKh[cb]);
            }
#pragma unroll
            for (int J = 0; J < 4; ++J)
                dMa[J] = MB::mma(fdO, load_frag<bf16>(sUe + 16 * J * LSW, LSW, lane), dMa[J]);
        }
        __syncthreads();  // dZ complete
        {
            const MB::frag fdZ = load_frag<bf16>(sdZ + 16 * I * LSW, LSW, lane);
#pragma unroll
            for (int J = 0; J < 4; ++J)
                dAp[J] = MB::mma(fdZ, load_frag<bf16>(sU + 16 * J * LSW, LSW, lane), dAp[J]);
        }
        __syncthreads();  // before the next slab is staged
    }

    float *oQ = ba.dQh + ch * kChunk * DK, *oW = ba.dW + ch * kChunk * DK, *oK = ba.dKh + ch * kChunk * DK;
    float *oM = ba.dM + ch * kChunk * kChunk, *oA = ba.dAp + ch * kChunk * kChunk;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * (lane >> 4) + r;
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb) {
            const int c = 16 * cb + (lane & 15);
            oQ[i * DK + c] = dQh[cb][r];
            oW[i * DK + c] = -dWt[cb][r];
            oK[i * DK + c] = dKh[cb][r];
        }
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const int j = 16 * J + (lane & 15);
            oM[i * kChunk + j] = j <= i ? dMa[J][r] : 0.0f;
            oA[i * kChunk + j] = dAp[J][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Factor side, one workgroup per (chunk, head).  Thread (qd, tg) owns key
// channels 4qd..4qd+3 of tokens tg*TPG .. for the element-wise parts; wave w
// owns token rows 16w .. of the 64-row products.
// ---------------------------------------------------------------------------
template <int DK>
struct FacCfg {
    static constexpr int NQUAD = DK / 4, NTG = kThreads / NQUAD, TPG = kChunk / NTG;
    static constexpr int LDT = DK + 8;    // bf16 tiles [64][LDT]
    static constexpr int LDF = DK + 4;    // fp32 [64][LDF]
    static constexpr int LDA = kChunk + 4;
    static constexpr size_t SZ_RT = size_t(3) * kChunk * LDT * 2;
    static constexpr size_t SZ_F = size_t(kChunk) * LDF * 4;
    static constexpr size_t SZ_A = size_t(kChunk) * LDA * 4;
    static constexpr size_t SZ_RED = size_t(2) * NTG * DK * 4;
    static constexpr size_t OFF_RD = SZ_RT, OFF_RA = OFF_RD + SZ_F, OFF_RM = OFF_RA + SZ_A,
                            OFF_RW = OFF_RM + SZ_A, OFF_RED = OFF_RW + SZ_F;
    static constexpr size_t SMEM = OFF_RED + SZ_RED;
    static_assert(SZ_F <= 2 * SZ_A && SZ_F <= SZ_RT && size_t(kChunk) * kChunk * 2 <= SZ_RT, "reuse");
    static_assert(size_t(NTG) * DK * 4 <= SZ_F && size_t(kChunk) * DK * 2 <= SZ_F, "reuse");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

template <int DK>
__global__ __launch_bounds__(kThreads, 1) void chunk_bwd_factor_kernel(BwdArgs ba) {
    using C = FacCfg<DK>;
    constexpr int LDT = C::LDT, LDF = C::LDF, LDA = C::LDA, TPG = C::TPG, NKB = DK / 16;
    const ChunkArgs &a = ba.c;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    bf16 *sKp = reinterpret_cast<bf16 *>(smem);           // [64][LDT] k e^{g_r-g}
    bf16 *sEp = sKp + kChunk * LDT;                        // [64][LDT] b k e^{g-g_r}
    bf16 *sQp = sEp + kChunk * LDT;                        // [64][LDT] q e^{g-g_r}
    bf16 *sT = reinterpret_cast<bf16 *>(smem);             // T [64][64] (before the tiles)
    float *sdKp = reinterpret_cast<float *>(smem);         // dKp [64][LDF] (after the products)
    float *sdE = reinterpret_cast<float *>(smem + C::OFF_RD);   // dE [64][LDF]
    float *sA = reinterpret_cast<float *>(smem + C::OFF_RA);    // dZ U^T, then dA [64][LDA]
    float *sMm = reinterpret_cast<float *>(smem + C::OFF_RM);   // dM [64][LDA]
    float *sdQp = reinterpret_cast<float *>(smem + C::OFF_RA);  // dQp [64][LDF] (after the products)
    float *sRw = reinterpret_cast<float *>(smem + C::OFF_RW);   // dW, then W, then totals, then dEp
    bf16 *sWf = reinterpret_cast<bf16 *>(smem + C::OFF_RW);
    float *sRed = reinterpret_cast<float *>(smem + C::OFF_RED);  // [2][NTG][DK]

    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    dense_span(a, cid, tok0, len);
    const size_t ch = (size_t)cid * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, I = wave;
    const int qd = tid % C::NQUAD, tg = tid / C::NQUAD, c0 = 4 * qd;

    // ---- stage dW, T, dZ U^T, dM ------------------------------------------
    {
        const float *dWg = ba.dW + ch * kChunk * DK;
        for (int e = tid; e < kChunk * DK / 4; e += kThreads) {
            const int i = e / (DK / 4), c4 = 4 * (e % (DK / 4));
            *reinterpret_cast<f32x4 *>(sRw + i * LDF + c4) =
                *reinterpret_cast<const f32x4 *>(dWg + (size_t)i * DK + c4);
        }
        copy16(sT, reinterpret_cast<const bf16 *>(a.ws_T) + ch * kChunk * kChunk, kChunk * kChunk * 2, tid,
               kThreads);
        const float *Ap = ba.dAp + ch * kChunk * kChunk, *Mg = ba.dM + ch * kChunk * kChunk;
        for (int e = tid; e < kChunk * kChunk / 4; e += kThreads) {
            const int i = e / (kChunk / 4), c4 = 4 * (e % (kChunk / 4));
            *reinterpret_cast<f32x4 *>(sA + i * LDA + c4) =
                *reinterpret_cast<const f32x4 *>(Ap + (size_t)i * kChunk + c4);
            *reinterpret_cast<f32x4 *>(sMm + i * LDA + c4) =
                *reinterpret_cast<const f32x4 *>(Mg + (size_t)i * kChunk + c4);
        }
    }
    __syncthreads();
    // dE = T^T dW (rows of block I).
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb) {
        const f32x4 d = mma_f32<kChunk>(
            zero4(), lane, [&](int m, int k) { return static_cast<float>(sT[k * kChunk + 16 * I + m]); },
            [&](int nn, int k) { return sRw[k * LDF + 16 * cb + nn]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) sdE[(16 * I + 4 * (lane >> 4) + r) * LDF + 16 * cb + (lane & 15)] = d[r];
    }
    __syncthreads();  // dW is dead: the region receives W
    copy16(sWf, reinterpret_cast<const bf16 *>(a.ws_W) + ch * kChunk * DK, kChunk * DK * 2, tid, kThreads);
    __syncthreads();
    // dA = -strict_tril(dZ U^T + dE W^T), in place of dZ U^T.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        const f32x4 d = mma_f32<DK>(
            zero4(), lane, [&](int m, int k) { return sdE[(16 * I + m) * LDF + k]; },
            [&](int nn, int k) { return fe(sWf, DK, 16 * J + nn, k); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * (lane >> 4) + r, j = 16 * J + (lane & 15);
            float &x = sA[i * LDA + j];
            x = j < i ? -(x + d[r]) : 0.0f;
        }
    }
    __syncthreads();  // W is dead: the region receives the scan totals

    // ---- cumulative log-decay and the scaled tiles --------------------------
    f32x4 g[TPG];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        g[j] = i < len ? *reinterpret_cast<const f32x4 *>(a.log_alpha + ((size_t)(tok0 + i) * H + h) * DK + c0)
                       : zero4();
    }
#pragma unroll
    for (int j = 1; j < TPG; ++j) g[j] += g[j - 1];
    *reinterpret_cast<f32x4 *>(sRw + tg * DK + c0) = g[TPG - 1];
    __syncthreads();
    f32x4 goff = zero4(), glast = zero4();
#pragma unroll
    for (int t = 0; t < C::NTG; ++t) {
        const f32x4 tt = *reinterpret_cast<const f32x4 *>(sRw + t * DK + c0);
        if (t < tg) goff += tt;
        glast += tt;
    }
#pragma unroll
    for (int j = 0; j < TPG; ++j) g[j] += goff;
    const f32x4 gr = 0.5f * glast;
    const bf16 *kin = reinterpret_cast<const bf16 *>(a.k), *qin = reinterpret_cast<const bf16 *>(a.q);
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        f32x4 kf = zero4(), qf = zero4(), bf = zero4();
        if (i < len) {
            const size_t off = ((size_t)(tok0 + i) * H + h) * DK + c0;
            const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(kin + off);
            const bf16x4 q4 = *reinterpret_cast<const bf16x4 *>(qin + off);
            bf = *reinterpret_cast<const f32x4 *>(a.b + off);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kf[c] = static_cast<float>(k4[c]);
                qf[c] = static_cast<float>(q4[c]);
            }
        }
        bf16x4 kp, ep, qp;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float ex = __expf(g[j][c] - gr[c]), ei = __expf(gr[c] - g[j][c]);
            kp[c] = static_cast<bf16>(kf[c] * ei);
            ep[c] = static_cast<bf16>(bf[c] * kf[c] * ex);
            qp[c] = static_cast<bf16>(qf[c] * ex);
        }
        *reinterpret_cast<bf16x4 *>(sKp + i * LDT + c0) = kp;
        *reinterpret_cast<bf16x4 *>(sEp + i * LDT + c0) = ep;
        *reinterpret_cast<bf16x4 *>(sQp + i * LDT + c0) = qp;
    }
    __syncthreads();

    // ---- dEp = dA Kp, dQp = dM Kp, dKp = dA^T Ep + dM^T Qp ------------------
    f32x4 dEp[NKB], dQp[NKB], dKp[NKB];
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb) {
        auto kp = [&](int nn, int k) { return static_cast<float>(sKp[k * LDT + 16 * cb + nn]); };
        dEp[cb] = mma_f32<kChunk>(zero4(), lane, [&](int m, int k) { return sA[(16 * I + m) * LDA + k]; }, kp);
        dQp[cb] = mma_f32<kChunk>(zero4(), lane, [&](int m, int k) { return sMm[(16 * I + m) * LDA + k]; }, kp);
        f32x4 d = mma_f32<kChunk>(zero4(), lane, [&](int m, int k) { return sA[k * LDA + 16 * I + m]; },
                                  [&](int nn, int k) { return static_cast<float>(sEp[k * LDT + 16 * cb + nn]); });
        dKp[cb] = mma_f32<kChunk>(d, lane, [&](int m, int k) { return sMm[k * LDA + 16 * I + m]; },
                                  [&](int nn, int k) { return static_cast<float>(sQp[k * LDT + 16 * cb + nn]); });
    }
    __syncthreads();  // tiles, dA and dM are dead
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = (16 * I + 4 * (lane >> 4) + r) * LDF + 16 * cb + (lane & 15);
            sRw[o] = dEp[cb][r];
            sdQp[o] = dQp[cb][r];
            sdKp[o] = dKp[cb][r];
        }
    __syncthreads();

    // ---- element-wise gradients, thread (qd, tg) ---------------------------
    const float *dQg = ba.dQh + ch * kChunk * DK, *dKg = ba.dKh + ch * kChunk * DK;
    f32x4 dgv[TPG];
    f32x4 kdk = zero4();
    bf16 *dqo = reinterpret_cast<bf16 *>(ba.dq), *dko = reinterpret_cast<bf16 *>(ba.dk);
    f32x4 egr;
#pragma unroll
    for (int c = 0; c < 4; ++c) egr[c] = __expf(gr[c]);
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        dgv[j] = zero4();
        if (i >= len) continue;
        const size_t off = ((size_t)(tok0 + i) * H + h) * DK + c0;
        const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(kin + off);
        const bf16x4 q4 = *reinterpret_cast<const bf16x4 *>(qin + off);
        const f32x4 bf = *reinterpret_cast<const f32x4 *>(a.b + off);
        const f32x4 dQh = *reinterpret_cast<const f32x4 *>(dQg + i * DK + c0);
        const f32x4 dKh = *reinterpret_cast<const f32x4 *>(dKg + i * DK + c0);
        const f32x4 dE = *reinterpret_cast<const f32x4 *>(sdE + i * LDF + c0);
        const f32x4 dEpv = *reinterpret_cast<const f32x4 *>(sRw + i * LDF + c0);
        const f32x4 dQpv = *reinterpret_cast<const f32x4 *>(sdQp + i * LDF + c0);
        const f32x4 dKpv = *reinterpret_cast<const f32x4 *>(sdKp + i * LDF + c0);
        f32x4 dq, dk, db;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float kf = static_cast<float>(k4[c]), qf = static_cast<float>(q4[c]);
            const float ex = __expf(g[j][c] - gr[c]), ei = __expf(gr[c] - g[j][c]);
            const float gam = ex * egr[c], eK = ei * egr[c];
            const float t1 = gam * dE[c] + ex * dEpv[c];
            dq[c] = gam * dQh[c] + ex * dQpv[c];
            db[c] = kf * t1;
            dk[c] = bf[c] * t1 + ei * dKpv[c] + eK * dKh[c];
            dgv[j][c] = bf[c] * kf * t1 + qf * dq[c] - kf * (ei * dKpv[c] + eK * dKh[c]);
            kdk[c] += kf * eK * dKh[c];
        }
        bf16x4 dq4, dk4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            dq4[c] = static_cast<bf16>(dq[c]);
            dk4[c] = static_cast<bf16>(dk[c]);
        }
        *reinterpret_cast<bf16x4 *>(dqo + off) = dq4;
        *reinterpret_cast<bf16x4 *>(dko + off) = dk4;
        *reinterpret_cast<f32x4 *>(ba.db + off) = db;
    }
    // dlog_alpha_j = sum_{i>=j} dg_i + gl dgl + sum_i Khat_i dKhat_i.
#pragma unroll
    for (int j = TPG - 2; j >= 0; --j) dgv[j] += dgv[j + 1];   // suffix sums inside the group
    *reinterpret_cast<f32x4 *>(sRed + tg * DK + c0) = dgv[0];
    *reinterpret_cast<f32x4 *>(sRed + (C::NTG + tg) * DK + c0) = kdk;
    __syncthreads();
    f32x4 after = zero4(), kdk_all = zero4();
#pragma unroll
    for (int t = 0; t < C::NTG; ++t) {
        if (t > tg) after += *reinterpret_cast<const f32x4 *>(sRed + t * DK + c0);
        kdk_all += *reinterpret_cast<const f32x4 *>(sRed + (C::NTG + t) * DK + c0);
    }
    // dgl[c] = sum_v dS'[c][v] S[c][v]: this thread takes v in [tg*DV/NTG, ..), the
    // group partials meet in LDS.
    {
        constexpr int VPT = DK / C::NTG;
        const float *Sc = ba.Sc + ch * DK * DK, *dSc = ba.dSc + ch * DK * DK;
        f32x4 part = zero4();
#pragma unroll
        for (int c = 0; c < 4; ++c)
            for (int v = tg * VPT; v < (tg + 1) * VPT; v += 4) {
                const f32x4 s4 = *reinterpret_cast<const f32x4 *>(Sc + (size_t)(c0 + c) * DK + v);
                const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dSc + (size_t)(c0 + c) * DK + v);
                part[c] += s4[0] * d4[0] + s4[1] * d4[1] + s4[2] * d4[2] + s4[3] * d4[3];
            }
        __syncthreads();  // the totals above have been read
        *reinterpret_cast<f32x4 *>(sRed + tg * DK + c0) = part;
    }
    __syncthreads();
    f32x4 dG = zero4();
#pragma unroll
    for (int t = 0; t < C::NTG; ++t) dG += *reinterpret_cast<const f32x4 *>(sRed + t * DK + c0);
    f32x4 dglast;
#pragma unroll
    for (int c = 0; c < 4; ++c) dglast[c] = __expf(glast[c]) * dG[c] + kdk_all[c];
#pragma unroll
    for (int j = 0; j < TPG; ++j) {
        const int i = tg * TPG + j;
        if (i < len)
            *reinterpret_cast<f32x4 *>(ba.dla + ((size_t)(tok0 + i) * H + h) * DK + c0) =
                dgv[j] + after + dglast;
    }
}

template <int D>
static void launch_bwd_d(const BwdArgs &a, hipStream_t stream) {
    const int chains = a.c.N * a.c.H, groups = (chains + 7) / 8;
    const int dvs = (D >= 64 && chains >= 128) ? 64 : (chains >= 64 ? 32 : 16);
    const dim3 block(kThreads);
    if (dvs == 64)
        hipLaunchKernelGGL((chunk_bwd_rev_kernel<D, 64>), dim3(groups * 8 * (D / 64)), block, 0, stream, a);
    else if (dvs == 32)
        hipLaunchKernelGGL((chunk_bwd_rev_kernel<D, 32>), dim3(groups * 8 * (D / 32)), block, 0, stream, a);
    else
        hipLaunchKernelGGL((chunk_bwd_rev_kernel<D, 16>), dim3(groups * 8 * (D / 16)), block, 0, stream, a);
    if (a.c.max_chunks == 0) return;
    const dim3 grid((unsigned)((size_t)a.c.max_chunks * a.c.H));
    hipLaunchKernelGGL((chunk_bwd_state_kernel<D>), grid, block, 0, stream, a);
    hipLaunchKernelGGL((chunk_bwd_factor_kernel<D>), grid, block, 0, stream, a);
}

hipError_t launch_chunk_bwd(const BwdArgs &a, int Dk, hipStream_t stream) {
    if (Dk == 128) launch_bwd_d<128>(a, stream);
    else launch_bwd_d<64>(a, stream);
    return hipGetLastError();
}

}  // namespace gdn2
