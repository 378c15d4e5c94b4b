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
//   state side   dW = -dU_eff S^T,  dKhat = U_eff dS'^T,  dM = tril(dO U_eff^T),
//                dgl = rowsum(dS' * S),  dZ = T^T dU_eff,  dv = w * dZ,  dw = v * dZ
//   factor side  dQhat = dO S^T,  dE = T^T dW,  dA = -strict_tril(dZ U^T + dE W^T),
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
// Two kernels after the forward (the chunk factors a backward call needs:
// W, Khat^T, U, gamma_last and the transposes M^T, Qhat^T, T^T; the
// propagation storing every chunk's incoming state and forming no o):
//   chunk_bwd_rev2_kernel    sequential over the chunks of a sequence, in
//   (chunk_bwd_rev_kernel    reverse: dU_eff and dS, storing each chunk's dS'
//    with 256+ chains)
//   chunk_bwd_local_kernel   per chunk: the state-side products with dv and dw,
//                            then the factor side with dq, dk, db, dlog_alpha
// All products are bf16 MFMA (16x16x32) with fp32 accumulation; each operand is
// either a fragment-ordered factor from the workspace or staged in LDS with its
// contraction index contiguous.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

typedef unsigned int granule_t __attribute__((ext_vector_type(4)));

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

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// Operand fragment of the transpose of a row-major bf16 tile X in LDS (pitch
// ld, 8-byte aligned rows): lane l receives X[r0 + 8 (l/16) + t][c0 + l%16],
// t = 0..7, i.e. the fragment of X^T at rows c0.., contraction index r0...
// Two transposing 8-byte reads: in each group of 16 lanes, lane j points at
// row r0 + 8 (l/16) + j/4 (+4), columns c0 + 4 (j%4) .. +3, and lane i then
// receives column c0 + i of those 4 rows.
__device__ __forceinline__ Mma<bf16>::frag load_frag_tr(const bf16 *X, int ld, int r0, int c0, int lane) {
    const int j = lane & 15, row = r0 + 8 * (lane >> 4) + (j >> 2), col = c0 + 4 * (j & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(X + row * ld + col));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(X + (row + 4) * ld + col));
    const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(Mma<bf16>::frag, both);
}

// LDS slot of 16-byte granule g of a fragment-ordered image that is read
// transposed: granules whose bit 4 is set trade places with the granule 4
// away, so that a transposing read's two column groups of the same rows (16
// granules apart) land on different banks.
__device__ __forceinline__ int fo_slot(int g) { return g ^ (((g >> 4) & 1) << 2); }

// Operand fragment of X^T where X (K columns) lies in LDS in the chunk
// factors' fragment order, granules placed by fo_slot: lane l receives
// X[r0 + 8 (l/16) + t][c0 + l%16], t = 0..7, i.e. the fragment of X^T at rows
// c0.., contraction index r0...  Four consecutive columns of an X row are 8
// contiguous bytes of that order, so the two transposing reads work on it as
// on a row-major tile.
__device__ __forceinline__ const bf16 *fo_at(const bf16 *X, int r, int k, int K) {
    const int e = (int)frag_index<bf16>(r, k, K);
    return X + fo_slot(e >> 3) * 8 + (e & 7);
}
__device__ __forceinline__ Mma<bf16>::frag load_frag_tr_fo(const bf16 *X, int K, int r0, int c0, int lane) {
    const int j = lane & 15, row = r0 + 8 * (lane >> 4) + (j >> 2), col = c0 + 4 * (j & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)fo_at(X, row, col, K));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)fo_at(X, row + 4, col, K));
    const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(Mma<bf16>::frag, both);
}

}  // namespace

// ---------------------------------------------------------------------------
// Reverse pass: one workgroup per (sequence, head, DVS-column slab), the
// chunks of the sequence from last to first, bf16 MFMA.  dS' lives in fp32
// accumulators (wave w owns state rows 16 (w*KB_W + b) .. of the slab, like
// the forward); its bf16 copy in LDS, read through transposing LDS reads, is
// the operand of Khat dS'.  M^T and Qhat^T (written for backward calls) are
// loaded as fragments; Khat and W^T come from the Khat^T and W images the
// forward propagation reads, staged in LDS and read transposed.
// ---------------------------------------------------------------------------
template <int DK, int DVS>
struct RevCfg {
    static constexpr int DV = DK, NS = DV / DVS, NCB = DVS / 16, NKB = DK / 16;
    static constexpr int KB_W = NKB / 4, S_TPW = KB_W * NCB;
    static constexpr int L64 = kChunk + 8, LDV = DVS + 8;
    static constexpr int NP = DK * DVS / 8;                   // 16-byte pieces of dS'
    static constexpr int NPC = (NP + kThreads - 1) / kThreads;  // per thread
    static constexpr int GK = kChunk * DK / 8;                 // 16-byte granules of Khat^T, of W
    static constexpr int NKW = 2 * GK / kThreads;              // per thread
    static_assert(NKW * kThreads == 2 * GK, "Khat^T and W split");
};

template <int DK, int DVS>
__global__ __launch_bounds__(kThreads, 1) void chunk_bwd_rev_kernel(BwdArgs ba) {
    using C = RevCfg<DK, DVS>;
    using MB = Mma<bf16>;
    constexpr int DV = C::DV, NCB = C::NCB, L64 = C::L64, NKD = DK / 32;
    const ChunkArgs &a = ba.c;
    __shared__ __attribute__((aligned(16))) bf16 sKW[2 * C::GK * 8];  // Khat^T | W, fragment order
    __shared__ __attribute__((aligned(16))) bf16 sdO[kChunk * C::LDV];  // [i][v] = dO[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdUt[DVS * L64];   // [v][i] = dU_eff[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdS[DK * C::LDV];  // [c][v] = dS'[c][v]
    const bf16 *sKt = sKW, *sW = sKW + C::GK * 8;

    const int H = a.H;
    const int x = blockIdx.x, xcd = x & 7, rest = x >> 3;
    const int slab = rest % C::NS, chain = (rest / C::NS) * 8 + xcd;
    if (chain >= a.N * H) return;
    const int n = chain / H, h = chain % H, col0 = slab * DVS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int cbeg, cend;
    seq_chunks(a, n, cbeg, cend);

    f32x4 dS[C::S_TPW];
    load_state_tiles<DK, DV, C::KB_W, NCB>(dS, ba.dS_final, chain, wave, col0, lane);
    const bf16 *dout = reinterpret_cast<const bf16 *>(ba.dout);
    // Everything a chunk reads from global memory: M^T rows of block `wave`,
    // Qhat^T rows of this wave's state row blocks, this thread's granules of
    // the Khat^T and W images, gamma_last, and this thread's dO pieces (raw;
    // rows past the chunk's end read row 0, zeroed at use).
    constexpr int NE = kChunk * DVS / 4 / kThreads;
    static_assert(NE * kThreads * 4 == kChunk * DVS, "dO split");
    struct RevIn {
        MB::frag fM[2], fQ[C::KB_W][2];
        granule_t kw[C::NKW];
        f32x4 gl[C::KB_W];
        bf16x4 o[NE];
        int len;
    };
    auto load_in = [&](RevIn &x, int cid) {
        const size_t ch = (size_t)cid * H + h;
        int tok0, len;
        chunk_span_of(a, cid, cbeg, n, tok0, len);
        x.len = len;
        const bf16 *Mt = reinterpret_cast<const bf16 *>(a.ws_Mt) + ch * kChunk * kChunk;
        const bf16 *Qt = reinterpret_cast<const bf16 *>(a.ws_Qt) + ch * DK * kChunk;
        const granule_t *Kt = reinterpret_cast<const granule_t *>(a.ws_KhT) + ch * C::GK;
        const granule_t *Wg = reinterpret_cast<const granule_t *>(a.ws_W) + ch * C::GK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) x.fM[kk] = load_frag_packed<bf16>(Mt, kChunk, wave, kk, lane);
#pragma unroll
        for (int j = 0; j < C::NKW; ++j) {
            const int g = j * kThreads + tid;
            x.kw[j] = g < C::GK ? Kt[g] : Wg[g - C::GK];
        }
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b) {
            const int cblk = wave * C::KB_W + b;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) x.fQ[b][kk] = load_frag_packed<bf16>(Qt, kChunk, cblk, kk, lane);
            x.gl[b] = *reinterpret_cast<const f32x4 *>(a.ws_gl + ch * DK + 16 * cblk + 4 * (lane >> 4));
        }
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = tid + q * kThreads, i = e / (DVS / 4), c4 = 4 * (e % (DVS / 4));
            const size_t off = len > 0 ? ((size_t)(tok0 + (i < len ? i : 0)) * H + h) * DV + col0 + c4 : 0;
            x.o[q] = *reinterpret_cast<const bf16x4 *>(dout + off);
        }
    };
    // (A second register set, to load a chunk ahead, would drop 128-wide heads
    // to one wave per SIMD: each chunk's operands are loaded at its start.)
    RevIn cur;
    for (int cid = cend - 1; cid >= cbeg; --cid) {
        const size_t ch = (size_t)cid * H + h;
        load_in(cur, cid);
        const int len = cur.len;
        // dS' of this chunk to LDS (bf16); the copy goes on to the workspace
        // for the per-chunk kernels in 16-byte row pieces (2-byte stores
        // straight from the accumulators cost more than the rest of the
        // chunk's work).  The chunk's Khat^T and W images to LDS.
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
            store_tile<bf16>(sdS + 16 * cblk * C::LDV + 16 * colb, C::LDV, dS[u], lane);
        }
#pragma unroll
        for (int j = 0; j < C::NKW; ++j)
            *reinterpret_cast<granule_t *>(sKW + fo_slot(j * kThreads + tid) * 8) = cur.kw[j];
        // dO rows of the chunk (zero past its end), read through transposing
        // LDS reads.
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = tid + q * kThreads, i = e / (DVS / 4), c4 = 4 * (e % (DVS / 4));
            bf16x4 v4 = cur.o[q];
            if (i >= len) {
#pragma unroll
                for (int t = 0; t < 4; ++t) v4[t] = static_cast<bf16>(0.0f);
            }
            *reinterpret_cast<bf16x4 *>(sdO + i * C::LDV + c4) = v4;
        }
        __syncthreads();
        bf16 *dSc = ba.dSc + ch * DK * DV;
#pragma unroll
        for (int p = 0; p < C::NPC; ++p) {
            const int e = tid + p * kThreads, c = e / (DVS / 8), v8 = 8 * (e % (DVS / 8));
            if (C::NP % kThreads == 0 || e < C::NP)
                *reinterpret_cast<bf16x8 *>(dSc + sc_index(c, col0 + v8, DK)) =
                    *reinterpret_cast<const bf16x8 *>(sdS + c * C::LDV + v8);
        }

        // dU_eff rows of block `wave`:  M^T dO + Khat dS'.
        {
            MB::frag fK[NKD];  // Khat rows of block `wave` = columns of Khat^T
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) fK[kk] = load_frag_tr_fo(sKt, kChunk, 32 * kk, 16 * wave, lane);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc = MB::mma(cur.fM[kk], load_frag_tr(sdO, C::LDV, 32 * kk, 16 * cb, lane), acc);
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk)
                    acc = MB::mma(fK[kk], load_frag_tr(sdS, C::LDV, 32 * kk, 16 * cb, lane), acc);
                store_tile_t<bf16>(sdUt + 16 * cb * L64 + 16 * wave, L64, acc, lane);
            }
        }
        __syncthreads();

        // dS <- Diag(gl) dS' + Qhat^T dO - W^T dU_eff.
        MB::frag fW[C::KB_W][2];  // W^T rows of the wave's state row blocks = columns of W
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                fW[b][kk] = load_frag_tr_fo(sW, DK, 32 * kk, 16 * (wave * C::KB_W + b), lane);
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int b = u / NCB, colb = u % NCB;
            f32x4 q = zero4(), wu = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                q = MB::mma(cur.fQ[b][kk], load_frag_tr(sdO, C::LDV, 32 * kk, 16 * colb, lane), q);
                wu = MB::mma(fW[b][kk], load_frag<bf16>(sdUt + 16 * colb * L64 + 32 * kk, L64, lane), wu);
            }
            dS[u] = cur.gl[b] * dS[u] + q - wu;
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
// Reverse pass with shared factor reads: one workgroup of 8 waves per
// (sequence, head, 2*SUB-column slab).  Waves 0-3 and 4-7 each run the form
// above on SUB columns.  The chunk's factors (M^T, Khat^T, Qhat^T, W in
// fragment order) are read from the workspace once per workgroup, by all
// 512 threads, into registers one chunk ahead, and staged in LDS at the
// chunk's start; the four waves of a half read their fragments from there
// (those of Khat and W^T through transposing reads).
// The per-CU vector-memory path bounds this pass, and the two halves now
// share one read of the factors.
// ---------------------------------------------------------------------------
template <int DK, int SUB>
struct Rev2Cfg {
    static constexpr int DV = DK, WC = 2 * SUB, NS = DV / WC, NCB = SUB / 16, NKB = DK / 16;
    static constexpr int KB_W = NKB / 4, S_TPW = KB_W * NCB;
    static constexpr int LDKP = DK + 8, L64 = kChunk + 8, LDV = WC + 8;
    static constexpr int NT = 2 * kThreads;
    // 16-byte granules of M^T, and of each of Khat^T, Qhat^T, W
    static constexpr int GM = kChunk * kChunk / 8, GK = kChunk * DK / 8;
    static constexpr int NG = GM + 3 * GK, NJ = NG / NT;
    static constexpr int NGO = kChunk * WC / 8, NJO = (NGO + NT - 1) / NT;  // dO granules
    static constexpr int NP = DK * WC / 8, NPC = (NP + NT - 1) / NT;       // dS' pieces
    static_assert(GM % NT == 0 && GK % NT == 0, "factor granules split");
};

template <int DK, int SUB>
__global__ __launch_bounds__(2 * kThreads, 1) void chunk_bwd_rev2_kernel(BwdArgs ba) {
    using C = Rev2Cfg<DK, SUB>;
    using MB = Mma<bf16>;
    constexpr int DV = C::DV, WC = C::WC, NCB = C::NCB, LDKP = C::LDKP, L64 = C::L64, LDV = C::LDV;
    constexpr int NKD = DK / 32, NT = C::NT;
    const ChunkArgs &a = ba.c;
    __shared__ __attribute__((aligned(16))) bf16 sF[C::NG * 8];     // M^T | Khat^T | Qhat^T | W
    __shared__ __attribute__((aligned(16))) bf16 sdSt[WC * LDKP];   // [v][c] = dS'[c][v]
    __shared__ __attribute__((aligned(16))) bf16 sdO[kChunk * LDV];  // [i][v] = dO[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdUt[WC * L64];    // [v][i] = dU_eff[i][v]
    __shared__ __attribute__((aligned(16))) bf16 sdS[DK * LDV];     // [c][v] = dS'[c][v]
    const bf16 *sMt = sF, *sKt = sF + C::GM * 8, *sQt = sKt + C::GK * 8, *sW = sQt + C::GK * 8;

    const int H = a.H;
    const int x = blockIdx.x, xcd = x & 7, rest = x >> 3;
    const int slab = rest % C::NS, chain = (rest / C::NS) * 8 + xcd;
    if (chain >= a.N * H) return;
    const int n = chain / H, h = chain % H, col0 = slab * WC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wl = wave & 3;
    const int hc = (wave >> 2) * SUB;  // the half's first column within the slab
    int cbeg, cend;
    seq_chunks(a, n, cbeg, cend);

    f32x4 dS[C::S_TPW];
    load_state_tiles<DK, DV, C::KB_W, NCB>(dS, ba.dS_final, chain, wl, col0 + hc, lane);
    const bf16 *dout = reinterpret_cast<const bf16 *>(ba.dout);
    // One chunk's global operands: its factor granules (thread t holds
    // granules t, t + 512, ...), dO granules (8 columns of one token row; rows
    // past the chunk's end read row 0, zeroed at use) and gamma_last of the
    // wave's state rows.  Two sets alternate, so each is requested two chunks
    // before its use: one chunk ahead left the pass waiting on those loads.
    struct In {
        granule_t f[C::NJ], o[C::NJO];
        f32x4 gl[C::KB_W];
    };
    auto load_f = [&](In &x, int cid) {
        const size_t ch = (size_t)cid * H + h;
        const granule_t *Mt = reinterpret_cast<const granule_t *>(a.ws_Mt) + ch * C::GM;
        const granule_t *Kt = reinterpret_cast<const granule_t *>(a.ws_KhT) + ch * C::GK;
        const granule_t *Qt = reinterpret_cast<const granule_t *>(a.ws_Qt) + ch * C::GK;
        const granule_t *Wg = reinterpret_cast<const granule_t *>(a.ws_W) + ch * C::GK;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
            const int g = j * NT + tid;
            if (j * NT < C::GM) x.f[j] = Mt[g];
            else if (j * NT < C::GM + C::GK) x.f[j] = Kt[g - C::GM];
            else if (j * NT < C::GM + 2 * C::GK) x.f[j] = Qt[g - C::GM - C::GK];
            else x.f[j] = Wg[g - C::GM - 2 * C::GK];
        }
    };
    auto load_o = [&](In &x, int cid) {
        int tok0, len;
        chunk_span_of(a, cid, cbeg, n, tok0, len);
#pragma unroll
        for (int q = 0; q < C::NJO; ++q) {
            const int e = tid + q * NT, i = e / (WC / 8), c8 = 8 * (e % (WC / 8));
            if (C::NGO % NT == 0 || e < C::NGO) {
                const size_t off = len > 0 ? ((size_t)(tok0 + (i < len ? i : 0)) * H + h) * DV + col0 + c8 : 0;
                x.o[q] = *reinterpret_cast<const granule_t *>(dout + off);
            }
        }
    };
    auto load_gl = [&](In &x, int cid) {
        const size_t ch = (size_t)cid * H + h;
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b)
            x.gl[b] = *reinterpret_cast<const f32x4 *>(a.ws_gl + ch * DK + 16 * (wl * C::KB_W + b) +
                                                       4 * (lane >> 4));
    };
    // Chunk cid with its operands in x; x is refilled with chunk cid - 2 as
    // each part of it is consumed.
    auto step = [&](int cid, In &x) {
        const size_t ch = (size_t)cid * H + h;
        const int nxt2 = max(cid - 2, cbeg);
        int tok0, len;
        chunk_span_of(a, cid, cbeg, n, tok0, len);
        // This chunk's factors, dS' (as it is and transposed) and dO (rows,
        // zero past the chunk's end; read through transposing LDS reads)
        // into LDS.
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {  // Khat^T and W (read transposed) placed by fo_slot
            const int g = j * NT + tid;
            const bool tr = (j * NT >= C::GM && j * NT < C::GM + C::GK) || j * NT >= C::GM + 2 * C::GK;
            *reinterpret_cast<granule_t *>(sF + (tr ? fo_slot(g) : g) * 8) = x.f[j];
        }
        load_f(x, nxt2);
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wl * C::KB_W + u / NCB, colb = u % NCB;
            store_tile<bf16>(sdS + 16 * cblk * LDV + hc + 16 * colb, LDV, dS[u], lane);
            store_tile_t<bf16>(sdSt + (hc + 16 * colb) * LDKP + 16 * cblk, LDKP, dS[u], lane);
        }
#pragma unroll
        for (int q = 0; q < C::NJO; ++q) {
            const int e = tid + q * NT, i = e / (WC / 8), c8 = 8 * (e % (WC / 8));
            if (C::NGO % NT == 0 || e < C::NGO) {
                bf16x8 v8 = __builtin_bit_cast(bf16x8, x.o[q]);
                if (i >= len) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) v8[t] = static_cast<bf16>(0.0f);
                }
                *reinterpret_cast<bf16x8 *>(sdO + i * LDV + c8) = v8;
            }
        }
        load_o(x, nxt2);
        __syncthreads();
        // dS' to the workspace.
        bf16 *dSc = ba.dSc + ch * DK * DV;
#pragma unroll
        for (int p = 0; p < C::NPC; ++p) {
            const int e = tid + p * NT, c = e / (WC / 8), v8 = 8 * (e % (WC / 8));
            if (C::NP % NT == 0 || e < C::NP)
                *reinterpret_cast<granule_t *>(dSc + sc_index(c, col0 + v8, DK)) =
                    *reinterpret_cast<const granule_t *>(sdS + c * LDV + v8);
        }

        // dU_eff rows of block wl, the half's columns:  M^T dO + Khat dS'.
        {
            MB::frag fM[2], fK[NKD];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) fM[kk] = load_frag_packed<bf16>(sMt, kChunk, wl, kk, lane);
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) fK[kk] = load_frag_tr_fo(sKt, kChunk, 32 * kk, 16 * wl, lane);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int v = hc + 16 * cb;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc = MB::mma(fM[kk], load_frag_tr(sdO, LDV, 32 * kk, v, lane), acc);
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk)
                    acc = MB::mma(fK[kk], load_frag<bf16>(sdSt + v * LDKP + 32 * kk, LDKP, lane), acc);
                store_tile_t<bf16>(sdUt + v * L64 + 16 * wl, L64, acc, lane);
            }
        }
        __syncthreads();

        // dS <- Diag(gl) dS' + Qhat^T dO - W^T dU_eff.
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b) {
            const int cblk = wl * C::KB_W + b;
            MB::frag fQ[2], fW[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                fQ[kk] = load_frag_packed<bf16>(sQt, kChunk, cblk, kk, lane);
                fW[kk] = load_frag_tr_fo(sW, DK, 32 * kk, 16 * cblk, lane);
            }
#pragma unroll
            for (int colb = 0; colb < NCB; ++colb) {
                const int v = hc + 16 * colb;
                f32x4 q = zero4(), wu = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    q = MB::mma(fQ[kk], load_frag_tr(sdO, LDV, 32 * kk, v, lane), q);
                    wu = MB::mma(fW[kk], load_frag<bf16>(sdUt + v * L64 + 32 * kk, L64, lane), wu);
                }
                const int u = b * NCB + colb;
                dS[u] = x.gl[b] * dS[u] + q - wu;
            }
        }
        load_gl(x, nxt2);
        __syncthreads();
    };
    In inA, inB;
    if (cend > cbeg) {
        load_f(inA, cend - 1);
        load_o(inA, cend - 1);
        load_gl(inA, cend - 1);
        load_f(inB, max(cend - 2, cbeg));
        load_o(inB, max(cend - 2, cbeg));
        load_gl(inB, max(cend - 2, cbeg));
    }
    for (int cid = cend - 1; cid >= cbeg; cid -= 2) {
        step(cid, inA);
        if (cid - 1 >= cbeg) step(cid - 1, inB);
    }
    if (ba.dS0) {
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wl * C::KB_W + u / NCB, colb = u % NCB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * cblk + 4 * (lane >> 4) + r, col = col0 + hc + 16 * colb + (lane & 15);
                ba.dS0[((size_t)chain * DK + row) * DV + col] = dS[u][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// State side, one workgroup per (chunk, head): the products with S and dS'
// (except dQhat = dO S^T, which the factor side forms),
// taken over 32-column slabs of the value axis with bf16 MFMA (16x16x32).
// Every operand is staged in LDS in the orientation its fragment load wants
// (k contiguous), transposing on the way in where needed; S and dS' are
// staged once, [c][v], and read through transposing LDS reads where the
// contraction runs over c.  A slab's global operands are loaded during the
// previous slab.  Wave w owns token rows 16w .. 16w+15 of every 64-row
// result.
// ---------------------------------------------------------------------------
template <int DK>
struct StateCfg {
    static constexpr int DV = DK, SW = 32, NSL = DV / SW, NKB = DK / 16;
    static constexpr int LSW = SW + 8;     // [..][SW] bf16 rows
    static constexpr int L64 = kChunk + 8; // [..][64] bf16 rows
    // LDS (bf16 elements): Khat^T image, S and dS' [c][v], dO, U, U_eff, dU_eff
    // and dZ [i][v], dU_eff^T [v][i]
    static constexpr int E_KT = DK * kChunk, E_S = DK * LSW, E_R = kChunk * LSW, E_UT = SW * L64;
    static constexpr size_t SMEM = size_t(E_KT + 2 * E_S + 5 * E_R + E_UT) * 2;
    static_assert(E_KT % 8 == 0 && E_S % 8 == 0 && E_R % 8 == 0, "16-byte aligned arrays");
};

template <int DK>
struct FacCfg {
    static constexpr int DH = DK / 2;                 // channels per half
    static constexpr int NQUAD = DH / 4, NTG = kThreads / NQUAD, TPG = kChunk / NTG;
    // the loops over the NTG token groups' partial sums: fully unrolled for
    // 128-wide heads; by 4 for 64-wide ones, whose 32 groups would otherwise
    // hold 32 LDS reads in flight and spill
    static constexpr int NTG_UNROLL = NTG > 16 ? 4 : NTG;
    static constexpr int L64 = kChunk + 8;            // bf16 [..][64]
    static constexpr int LDKP = DK + 8;               // bf16 [..][DK]
    static constexpr int LDG = DH + 4;                // fp32 [64][LDG]
    static constexpr size_t SZ_CT = size_t(DH) * L64 * 2;       // [DH][64] bf16
    static constexpr size_t SZ_64 = size_t(kChunk) * L64 * 2;    // [64][64] bf16
    static constexpr size_t SZ_DE = size_t(kChunk) * LDKP * 2;   // dE bf16 [64][LDKP]
    static constexpr size_t SZ_T3 = 3 * SZ_CT;                   // Kp^T, Ep^T, Qp^T of a half
    static constexpr size_t OFF_T = 0;                           // dE, then the half's tiles
    static constexpr size_t OFF_A = OFF_T + (SZ_DE > SZ_T3 ? SZ_DE : SZ_T3);  // dA, dA^T
    static constexpr size_t OFF_G = OFF_A + 2 * SZ_64;           // g, then dg of a half (fp32)
    static constexpr size_t OFF_R = OFF_G + size_t(kChunk) * LDG * 4;
    static constexpr size_t SZ_R = size_t(2 * NTG + 4) * DH * 4 + size_t(2) * DK * 4;
    static constexpr size_t OFF_DG = OFF_R + size_t(2 * NTG + 4) * DH * 4;  // dgl [DK] (in the R region)
    static constexpr size_t SMEM = OFF_R + SZ_R;
    static_assert(SMEM <= 80 * 1024, "two workgroups per CU");
};

// What the state side hands to the factor side in registers, per wave (rows
// of block I, MFMA accumulator order): dU_eff S^T (= -dW), dO U_eff^T (dM
// before its mask), dZ U^T, and the wave's T^T fragments; also the factor
// side's first global operands (every row block of W, the wave's dO rows),
// issued by the state side as it finishes so that they arrive during the
// hand-over.  Its gamma_last gradient goes to the factor side's LDS slot
// directly, and dKhat through the workspace.
template <int DK>
struct StateOut {
    f32x4 dWn[DK / 16], dM[4], dAp[4];
    Mma<bf16>::frag fTt[2], fWd[4][DK / 32], fdO[DK / 32];
};

// LDS of the per-chunk kernel, sized for 128-wide heads (the larger): the
// state side's tiles, then the factor side's in the same bytes.
constexpr size_t kBwdSmem = StateCfg<128>::SMEM > FacCfg<128>::SMEM ? StateCfg<128>::SMEM : FacCfg<128>::SMEM;
static_assert(kBwdSmem <= 80 * 1024, "two workgroups per CU");
__shared__ __attribute__((aligned(16))) char bwd_smem[kBwdSmem];

// The state side of one (chunk, head), the first part of
// chunk_bwd_local_kernel, in bwd_smem (StateCfg<DK>::SMEM bytes).
template <int DK>
__device__ __forceinline__ void bwd_state_side(const BwdArgs &ba, StateOut<DK> &out) {
    char *smem = bwd_smem;
    static_assert(FacCfg<DK>::OFF_DG >= StateCfg<DK>::SMEM, "the gamma_last gradient slot is clear of the state side's tiles");
    using C = StateCfg<DK>;
    using MB = Mma<bf16>;
    constexpr int DV = C::DV, SW = C::SW, NKB = C::NKB, LSW = C::LSW, L64 = C::L64;
    constexpr int NKD = DK / 32;
    const ChunkArgs &a = ba.c;
    // per slab (W, M^T and T^T are loaded as fragments from the workspace,
    // Khat through the Khat^T image in sKt)
    bf16 *sKt = reinterpret_cast<bf16 *>(smem);  // Khat^T, fragment order
    bf16 *sS = sKt + C::E_KT;                     // [c][v]
    bf16 *sdS = sS + C::E_S;                      // [c][v]
    bf16 *sdO = sdS + C::E_S;                     // [i][v]
    bf16 *sU = sdO + C::E_R;                      // [j][v] = U[j][v]
    bf16 *sUe = sU + C::E_R;                      // [i][v] = U_eff
    bf16 *sdU = sUe + C::E_R;                     // [i][v]
    bf16 *sdZ = sdU + C::E_R;                     // [i][v]
    bf16 *sdUt = sdZ + C::E_R;                    // [v][i] = dU_eff[i][v]

    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    dense_span(a, cid, tok0, len);
    if (len <= 0) return;  // (a malformed table only) no token; the factor side skips it too
    const size_t ch = (size_t)cid * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, I = wave;
    const bf16 *dout = reinterpret_cast<const bf16 *>(ba.dout);
    const bf16 *vin = reinterpret_cast<const bf16 *>(a.v);
    const bf16 *Ug = reinterpret_cast<const bf16 *>(a.ws_U) + ch * kChunk * DV;
    bf16 *dv = reinterpret_cast<bf16 *>(ba.dv);

    const bf16 *Wg = reinterpret_cast<const bf16 *>(a.ws_W) + ch * kChunk * DK;
    const bf16 *Mtg = reinterpret_cast<const bf16 *>(a.ws_Mt) + ch * kChunk * kChunk;
    const granule_t *Ktg = reinterpret_cast<const granule_t *>(a.ws_KhT) + ch * (DK * kChunk / 8);
    const bf16 *Ttg = reinterpret_cast<const bf16 *>(a.ws_Tt) + ch * kChunk * kChunk;

    f32x4 dWt[NKB], dKh[NKB], dMa[4], dAp[4];
#pragma unroll
    for (int j = 0; j < NKB; ++j) dWt[j] = dKh[j] = zero4();
#pragma unroll
    for (int j = 0; j < 4; ++j) dMa[j] = dAp[j] = zero4();
    const bf16 *Sc = ba.Sc + ch * DK * DV;
    const bf16 *dSc = ba.dSc + ch * DK * DV;
    // The wave's rows of W, M^T and T^T, held in registers across the slabs
    // (reloading them per slab re-reads them from HBM once the working set of
    // the resident workgroups has left L2).  Khat's rows are columns of the
    // Khat^T image, staged in LDS once and read per use.
    constexpr int NKG = DK * kChunk / 8 / kThreads;  // granules of Khat^T per thread
    MB::frag fW[NKD], fMt[2], fTt[2];
    {
        granule_t kg[NKG];
#pragma unroll
        for (int j = 0; j < NKG; ++j) kg[j] = Ktg[j * kThreads + tid];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) fW[kk] = load_frag_packed<bf16>(Wg, DK, I, kk, lane);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            fMt[kk] = load_frag_packed<bf16>(Mtg, kChunk, I, kk, lane);
            fTt[kk] = load_frag_packed<bf16>(Ttg, kChunk, I, kk, lane);
        }
#pragma unroll
        for (int j = 0; j < NKG; ++j) *reinterpret_cast<granule_t *>(sKt + fo_slot(j * kThreads + tid) * 8) = kg[j];
        // (the first slab's staging barrier orders these stores before their reads)
    }
    // Thread t stages row c = t / TPR of S and dS' (columns CPT (t % TPR) .. of
    // each slab) and accumulates dgl[c] = sum_v dS'[c][v] S[c][v] over the slabs.
    constexpr int TPR = kThreads / DK, CPT = SW / TPR;
    static_assert(CPT % 8 == 0, "16-byte row pieces");
    const int srow = tid / TPR, scol = CPT * (tid % TPR);
    float dgp = 0.0f;

    constexpr int NCS = SW / 16;
    // This lane's row piece (token iq, columns 4 lq4 .. +3 of each 16-column
    // block) of w and v, and of the dv and dw it writes.
    const int iq = 16 * I + 4 * (lane >> 4) + (lane & 3), lq4 = 4 * ((lane >> 2) & 3);
    const size_t oq = ((size_t)(tok0 + (iq < len ? iq : 0)) * H + h) * DV + lq4;

    // A slab's global operands, loaded one slab ahead: the next slab's are
    // issued as soon as this slab's are staged in LDS, so their latency
    // overlaps this slab's products.  Thread t holds CPT columns of row
    // t / TPR of S and dS', NDO dO row pieces (row e / (SW/4), e = t + 256 p;
    // rows past the chunk read row 0 and are zeroed when staged), and its
    // lane's U tiles (accumulator order).
    constexpr int NP8 = CPT / 8, NDO = kChunk * SW / 4 / kThreads;
    static_assert(NDO * kThreads == kChunk * SW / 4, "dO row pieces split evenly");
    struct SlabIn {
        bf16x8 sb[NP8], db[NP8];
        bf16x4 o4[NDO], u4[NCS];
    };
    auto load_slab = [&](SlabIn &x, int v0) {
#pragma unroll
        for (int p = 0; p < NP8; ++p) {
            x.sb[p] = *reinterpret_cast<const bf16x8 *>(Sc + sc_index(srow, v0 + scol + 8 * p, DK));
            x.db[p] = *reinterpret_cast<const bf16x8 *>(dSc + sc_index(srow, v0 + scol + 8 * p, DK));
        }
#pragma unroll
        for (int p = 0; p < NDO; ++p) {
            const int e = tid + kThreads * p, i = e / (SW / 4), v4 = 4 * (e % (SW / 4));
            x.o4[p] = *reinterpret_cast<const bf16x4 *>(dout + ((size_t)(tok0 + (i < len ? i : 0)) * H + h) * DV +
                                                        v0 + v4);
        }
#pragma unroll
        for (int cb = 0; cb < NCS; ++cb) {
            x.u4[cb] = *reinterpret_cast<const bf16x4 *>(Ug + (((size_t)I * (DV / 16) + (v0 / 16 + cb)) * 64 + lane) * 4);
        }
    };
    SlabIn cur;
    load_slab(cur, 0);

    for (int sl = 0; sl < C::NSL; ++sl) {
        const int v0 = sl * SW;
        // w and v row pieces of the slab (rows past the chunk read row 0 and
        // are not stored), used after the dZ product
        f32x4 wq[NCS];
        bf16x4 vq[NCS];
#pragma unroll
        for (int cb = 0; cb < NCS; ++cb) {
            wq[cb] = *reinterpret_cast<const f32x4 *>(a.w + oq + v0 + 16 * cb);
            vq[cb] = *reinterpret_cast<const bf16x4 *>(vin + oq + v0 + 16 * cb);
        }
        // S and dS' columns v0..v0+SW, [c][v] (products contracting over c
        // read them with transposing LDS reads); dO rows [i][v].
#pragma unroll
        for (int p = 0; p < NP8; ++p) {
            const int v = scol + 8 * p;
            const bf16x8 sb = cur.sb[p], db = cur.db[p];
#pragma unroll
            for (int t = 0; t < 8; ++t) dgp += static_cast<float>(sb[t]) * static_cast<float>(db[t]);
            *reinterpret_cast<bf16x4 *>(sS + srow * LSW + v) = bf16x4{sb[0], sb[1], sb[2], sb[3]};
            *reinterpret_cast<bf16x4 *>(sS + srow * LSW + v + 4) = bf16x4{sb[4], sb[5], sb[6], sb[7]};
            *reinterpret_cast<bf16x4 *>(sdS + srow * LSW + v) = bf16x4{db[0], db[1], db[2], db[3]};
            *reinterpret_cast<bf16x4 *>(sdS + srow * LSW + v + 4) = bf16x4{db[4], db[5], db[6], db[7]};
        }
#pragma unroll
        for (int p = 0; p < NDO; ++p) {
            const int e = tid + kThreads * p, i = e / (SW / 4), v4 = 4 * (e % (SW / 4));
            bf16x4 o4 = cur.o4[p];
            if (i >= len) {
#pragma unroll
                for (int t = 0; t < 4; ++t) o4[t] = static_cast<bf16>(0.0f);
            }
            *reinterpret_cast<bf16x4 *>(sdO + i * LSW + v4) = o4;
        }
        __syncthreads();
        SlabIn nxt;
        if (sl + 1 < C::NSL) load_slab(nxt, v0 + SW);

        // U_eff = U - W S and dU_eff = M^T dO + Khat dS' on this slab (rows of block I).
#pragma unroll
        for (int cb = 0; cb < SW / 16; ++cb) {
            f32x4 ws = zero4(), du = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                ws = MB::mma(fW[kk], load_frag_tr(sS, LSW, 32 * kk, 16 * cb, lane), ws);
                du = MB::mma(load_frag_tr_fo(sKt, kChunk, 32 * kk, 16 * I, lane),
                             load_frag_tr(sdS, LSW, 32 * kk, 16 * cb, lane), du);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                du = MB::mma(fMt[kk], load_frag_tr(sdO, LSW, 32 * kk, 16 * cb, lane), du);
            // U tile in accumulator order straight from the workspace (also
            // kept as rows [j][v] for dZ U^T).
            const bf16x4 u4 = cur.u4[cb];
            f32x4 ue, uf;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uf[r] = static_cast<float>(u4[r]);
                ue[r] = uf[r] - ws[r];
            }
            store_tile<bf16>(sU + 16 * I * LSW + 16 * cb, LSW, uf, lane);
            store_tile<bf16>(sUe + 16 * I * LSW + 16 * cb, LSW, ue, lane);
            store_tile<bf16>(sdU + 16 * I * LSW + 16 * cb, LSW, du, lane);
            store_tile_t<bf16>(sdUt + 16 * cb * L64 + 16 * I, L64, du, lane);
        }
        __syncthreads();

        // dZ = T^T dU_eff; dv = w dZ, dw = v dZ as row pieces (dZ quad
        // transposed: 4 columns of one token per lane, the layout of w and v).
#pragma unroll
        for (int cb = 0; cb < NCS; ++cb) {
            f32x4 dz = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                dz = MB::mma(fTt[kk], load_frag<bf16>(sdUt + 16 * cb * L64 + 32 * kk, L64, lane), dz);
            store_tile<bf16>(sdZ + 16 * I * LSW + 16 * cb, LSW, dz, lane);
            const f32x4 zt = quad_transpose(dz, lane);
            f32x4 dvv, dwv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dvv[r] = wq[cb][r] * zt[r];
                dwv[r] = static_cast<float>(vq[cb][r]) * zt[r];
            }
            if (iq < len) {
                const size_t o = oq + v0 + 16 * cb;
                *reinterpret_cast<bf16x4 *>(dv + o) =
                    bf16x4{static_cast<bf16>(dvv[0]), static_cast<bf16>(dvv[1]), static_cast<bf16>(dvv[2]),
                           static_cast<bf16>(dvv[3])};
                *reinterpret_cast<f32x4 *>(ba.dw + o) = dwv;
            }
        }
        // Products accumulated over the slabs (k = the slab's 32 columns).
        {
            const MB::frag fdO = load_frag<bf16>(sdO + 16 * I * LSW, LSW, lane);
            const MB::frag fdU = load_frag<bf16>(sdU + 16 * I * LSW, LSW, lane);
            const MB::frag fUe = load_frag<bf16>(sUe + 16 * I * LSW, LSW, lane);
#pragma unroll
            for (int cb = 0; cb < NKB; ++cb) {
                dWt[cb] = MB::mma(fdU, load_frag<bf16>(sS + 16 * cb * LSW, LSW, lane), dWt[cb]);
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
        cur = nxt;
    }

    // dgl: the TPR threads staging a row are consecutive lanes.
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) dgp += __shfl_xor(dgp, o, TPR);
    if ((tid % TPR) == 0) reinterpret_cast<float *>(smem + FacCfg<DK>::OFF_DG)[srow] = dgp;
    // dKhat leaves as row pieces after a quad transpose (row it, columns 4 lq ..).
    bf16 *oK = ba.dKh + ch * kChunk * DK;
    const int it = 16 * I + 4 * (lane >> 4) + (lane & 3), lq = (lane >> 2) & 3;
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb) {
        const f32x4 kt = quad_transpose(dKh[cb], lane);
        *reinterpret_cast<bf16x4 *>(oK + it * DK + 16 * cb + 4 * lq) =
            bf16x4{static_cast<bf16>(kt[0]), static_cast<bf16>(kt[1]), static_cast<bf16>(kt[2]),
                   static_cast<bf16>(kt[3])};
    }
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb) out.dWn[cb] = dWt[cb];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        out.dM[J] = dMa[J];
        out.dAp[J] = dAp[J];
    }
    out.fTt[0] = fTt[0];
    out.fTt[1] = fTt[1];
    // The factor side's operands of dA (W, every row block) and of dQhat (the
    // wave's dO rows; rows past the chunk's end read row 0, zeroed at use).
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) out.fWd[J][kk] = load_frag_packed<bf16>(Wg, DK, J, kk, lane);
    {
        const int row = 16 * I + (lane & 15);
        const bf16 *src = dout + ((size_t)(tok0 + (row < len ? row : 0)) * H + h) * DV + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) out.fdO[kk] = *reinterpret_cast<const MB::frag *>(src + 32 * kk);
    }
}

// ---------------------------------------------------------------------------
// Factor side, one workgroup per (chunk, head), bf16 MFMA.  Wave w owns token
// rows 16w .. 16w+15 of every 64-row result; the element-wise step runs in the
// same accumulator layout (lane holds rows 16w + 4(l/16) + r, column l%16 of
// each 16-column block), so dE, dEp, dQp and dKp never leave registers.
// After dE and dA (which contract over all channels), the key channels are
// processed in two halves of DK/2: the decay scan, the scaled tiles, dEp, dQp,
// dKp, dQhat, the element-wise gradients and d log alpha of one half share
// LDS with the other's, which keeps the workgroup under 80 KB of LDS (two per
// CU).
// ---------------------------------------------------------------------------
// The half's channel-major tiles (rows = channels, columns = the chunk's
// tokens) keep the 16-byte token granule g of row c at granule
// g ^ ((c / 16) mod 8): uniform over each 16-row MFMA tile, so operand reads
// keep the padded layout's bank spread, while the stores of a thread's token
// run for 16 different channels land on different banks.
__device__ __forceinline__ int fac_col(int c, int t) { return (((t >> 3) ^ ((c >> 4) & 7)) << 3) + (t & 7); }

// Operand fragment kk (tokens 32kk ..) of the 16-row block starting at `tile`
// (row block rb of a swizzled half tile).
__device__ __forceinline__ bf16x8 load_frag_fac(const bf16 *tile, int ld, int rb, int kk, int lane) {
    return *reinterpret_cast<const bf16x8 *>(tile + (lane & 15) * ld + (((4 * kk + (lane >> 4)) ^ (rb & 7)) << 3));
}


// The factor side of one (chunk, head), the second part of
// chunk_bwd_local_kernel, in bwd_smem (FacCfg<DK>::SMEM bytes).
template <int DK>
__device__ __forceinline__ void bwd_factor_side(const BwdArgs &ba, const StateOut<DK> &st) {
    char *smem = bwd_smem;
    using C = FacCfg<DK>;
    using MB = Mma<bf16>;
    constexpr int DH = C::DH, L64 = C::L64, LDKP = C::LDKP, LDG = C::LDG, TPG = C::TPG;
    constexpr int NKB = DK / 16, NKD = DK / 32, NHB = DH / 16;
    const ChunkArgs &a = ba.c;
    bf16 *sdE = reinterpret_cast<bf16 *>(smem + C::OFF_T);     // [i][c] (until dA is formed)
    bf16 *sKpt = reinterpret_cast<bf16 *>(smem + C::OFF_T);    // [c][j] = Kp[j][c], half
    bf16 *sEpt = sKpt + DH * L64;                               // [c][i] = Ep[i][c]
    bf16 *sQpt = sEpt + DH * L64;                               // [c][i] = Qp[i][c]
    bf16 *sdA = reinterpret_cast<bf16 *>(smem + C::OFF_A);     // [i][j]
    bf16 *sdAt = sdA + kChunk * L64;                            // [j][i]
    float *sG = reinterpret_cast<float *>(smem + C::OFF_G);    // g, then dg [64][LDG], half
    float *sR = reinterpret_cast<float *>(smem + C::OFF_R);    // [2*NTG][DH] scan partials
    float *sGl = sR + 2 * C::NTG * DH;                          // g_last [DH]
    float *sKdk = sGl + DH;                                     // [3][DH] per-wave sums (waves 1..3)
    float *sDG = sKdk + 3 * DH;                                 // dgl [DK]
    float *sKdk0 = sDG + DK;                                    // wave 0's sums [DK]

    const int H = a.H, cid = blockIdx.x / H, h = blockIdx.x % H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    dense_span(a, cid, tok0, len);
    if (len <= 0) return;  // (a malformed table only) no token: nothing to write
    const size_t ch = (size_t)cid * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, I = wave;
    const int qd = tid % C::NQUAD, tg = tid / C::NQUAD, cq = 4 * qd;  // channel quad within a half
    const bf16 *kin = reinterpret_cast<const bf16 *>(a.k), *qin = reinterpret_cast<const bf16 *>(a.q);

    // (sDG holds the state side's gamma_last gradient; the dW^T image lies in
    // the dA region and the dM image in the g region until they are read)
    const bf16 *sWt = reinterpret_cast<const bf16 *>(smem + C::OFF_A);
    const bf16 *sMi = reinterpret_cast<const bf16 *>(smem + C::OFF_G);

    // W (every row block, for dA) and the wave's dO rows (for dQhat), loaded
    // by the state side as it finished.
    const auto &fWd = st.fWd;
    MB::frag fdO[NKD];
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) fdO[kk] = st.fdO[kk];

    // ---- dE = T^T dW (rows of block I), kept in registers and as bf16 --------
    f32x4 dE[NKB];
#pragma unroll
    for (int cb = 0; cb < NKB; ++cb) {
        f32x4 d = MB::mma(st.fTt[0], load_frag_packed<bf16>(sWt, kChunk, cb, 0, lane), zero4());
        d = MB::mma(st.fTt[1], load_frag_packed<bf16>(sWt, kChunk, cb, 1, lane), d);
        dE[cb] = d;
        store_tile<bf16>(sdE + 16 * I * LDKP + 16 * cb, LDKP, d, lane);
    }
    // (each wave reads back only its own rows of dE; the barrier orders the
    // reads of the dW^T image before dA overwrites it)
    __syncthreads();
    MB::frag fM[2], fMt[2];  // dM and dM^T rows of block I
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        fM[kk] = *reinterpret_cast<const MB::frag *>(sMi + fo_slot((2 * I + kk) * 64 + lane) * 8);
        fMt[kk] = load_frag_tr_fo(sMi, kChunk, 32 * kk, 16 * I, lane);
    }
    // ---- dA = -strict_tril(dZ U^T + dE W^T), both orientations --------------
    {
        MB::frag fe_[NKD];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) fe_[kk] = load_frag<bf16>(sdE + 16 * I * LDKP + 32 * kk, LDKP, lane);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            f32x4 d = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) d = MB::mma(fe_[kk], fWd[J][kk], d);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * (lane >> 4) + r, j = 16 * J + (lane & 15);
                d[r] = j < i ? -(st.dAp[J][r] + d[r]) : 0.0f;
            }
            store_tile<bf16>(sdA + 16 * I * L64 + 16 * J, L64, d, lane);
            store_tile_t<bf16>(sdAt + 16 * I + 16 * J * L64, L64, d, lane);
        }
    }
    __syncthreads();  // dE (bf16) is dead: its region receives the half's tiles

    // operands of the whole chunk, loaded once
    MB::frag fA[2], fAt[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        fA[kk] = load_frag<bf16>(sdA + 16 * I * L64 + 32 * kk, L64, lane);
        fAt[kk] = load_frag<bf16>(sdAt + 16 * I * L64 + 32 * kk, L64, lane);
    }
    if (16 * I + (lane & 15) >= len) {  // dO rows past the chunk's end are zero
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) fdO[kk] = MB::zero();
    }
    const bf16 *Sc = ba.Sc + ch * DK * DK;
    const bf16 *dKg = ba.dKh + ch * kChunk * DK;
    bf16 *dqo = reinterpret_cast<bf16 *>(ba.dq), *dko = reinterpret_cast<bf16 *>(ba.dk);

#pragma unroll
    for (int half = 0; half < 2; ++half) {  // unrolled: dE is indexed by half
        const int cbase = half * DH;
        // ---- cumulative log-decay of the half's channels, the scaled tiles ----
        {
            f32x4 g[TPG], bf[TPG];
            bf16x4 k4[TPG], q4[TPG];
#pragma unroll
            for (int j = 0; j < TPG; ++j) {  // every load first (rows past the end read row 0)
                const int i = tg * TPG + j;
                const size_t off = ((size_t)(tok0 + (i < len ? i : 0)) * H + h) * DK + cbase + cq;
                g[j] = *reinterpret_cast<const f32x4 *>(a.log_alpha + off);
                k4[j] = *reinterpret_cast<const bf16x4 *>(kin + off);
                q4[j] = *reinterpret_cast<const bf16x4 *>(qin + off);
                bf[j] = *reinterpret_cast<const f32x4 *>(a.b + off);
            }
#pragma unroll
            for (int j = 0; j < TPG; ++j)  // padding tokens: k = q = b = 0, log alpha = 0
                if (tg * TPG + j >= len) g[j] = bf[j] = zero4();
#pragma unroll
            for (int j = 1; j < TPG; ++j) g[j] += g[j - 1];
            *reinterpret_cast<f32x4 *>(sR + tg * DH + cq) = g[TPG - 1];
            __syncthreads();
            f32x4 goff = zero4(), glast = zero4();
#pragma unroll C::NTG_UNROLL
            for (int t = 0; t < C::NTG; ++t) {
                const f32x4 tt = *reinterpret_cast<const f32x4 *>(sR + t * DH + cq);
                if (t < tg) goff += tt;
                glast += tt;
            }
            const f32x4 gr = 0.5f * glast;
            if (tg == 0) *reinterpret_cast<f32x4 *>(sGl + cq) = glast;
            float kp[4][TPG], ep[4][TPG], qp[4][TPG];
#pragma unroll
            for (int j = 0; j < TPG; ++j) {
                const int i = tg * TPG + j;
                g[j] += goff;
                *reinterpret_cast<f32x4 *>(sG + i * LDG + cq) = g[j];
                const bool ok = i < len;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float kf = ok ? static_cast<float>(k4[j][c]) : 0.0f;
                    const float qf = ok ? static_cast<float>(q4[j][c]) : 0.0f;
                    const float ex = __expf(g[j][c] - gr[c]), ei = __expf(gr[c] - g[j][c]);
                    kp[c][j] = kf * ei;
                    ep[c][j] = bf[j][c] * kf * ex;
                    qp[c][j] = qf * ex;
                }
            }
            // each channel's TPG tokens as one store per tile
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int at = (cq + c) * L64 + fac_col(cq + c, tg * TPG);
                if constexpr (TPG == 4) {
                    *reinterpret_cast<bf16x4 *>(sKpt + at) = bf16x4{static_cast<bf16>(kp[c][0]), static_cast<bf16>(kp[c][1]),
                                                                    static_cast<bf16>(kp[c][2]), static_cast<bf16>(kp[c][3])};
                    *reinterpret_cast<bf16x4 *>(sEpt + at) = bf16x4{static_cast<bf16>(ep[c][0]), static_cast<bf16>(ep[c][1]),
                                                                    static_cast<bf16>(ep[c][2]), static_cast<bf16>(ep[c][3])};
                    *reinterpret_cast<bf16x4 *>(sQpt + at) = bf16x4{static_cast<bf16>(qp[c][0]), static_cast<bf16>(qp[c][1]),
                                                                    static_cast<bf16>(qp[c][2]), static_cast<bf16>(qp[c][3])};
                } else {
                    static_assert(TPG == 2, "token runs of 2 or 4");
                    *reinterpret_cast<bf16x2 *>(sKpt + at) = bf16x2{static_cast<bf16>(kp[c][0]), static_cast<bf16>(kp[c][1])};
                    *reinterpret_cast<bf16x2 *>(sEpt + at) = bf16x2{static_cast<bf16>(ep[c][0]), static_cast<bf16>(ep[c][1])};
                    *reinterpret_cast<bf16x2 *>(sQpt + at) = bf16x2{static_cast<bf16>(qp[c][0]), static_cast<bf16>(qp[c][1])};
                }
            }
        }
        __syncthreads();

        // Per 16-channel block hb: dEp = dA Kp, dQp = dM Kp, dKp = dA^T Ep +
        // dM^T Qp and dQhat = dO S^T, then the element-wise gradients in the
        // accumulator layout (one block's results live at a time).
        // The global operands of block hb (S^T fragments and the element-wise
        // inputs, raw as loaded) are issued one block ahead.
        struct HbIn {
            MB::frag s[NKD];
            bf16 k[4], q[4], dk[4];
            float b[4];
        };
        auto load_hb = [&](HbIn &x, int hb) {
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)  // rows cbase+16hb.., columns 32kk..: one 32-column slab
                x.s[kk] = load_frag<bf16>(Sc + sc_index(cbase + 16 * hb, 32 * kk, DK), 32, lane);
            const int c = cbase + 16 * hb + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * (lane >> 4) + r, ic = i < len ? i : 0;
                const size_t off = ((size_t)(tok0 + ic) * H + h) * DK + c;
                x.k[r] = kin[off];
                x.q[r] = qin[off];
                x.b[r] = a.b[off];
                x.dk[r] = dKg[(size_t)ic * DK + c];
            }
        };
        HbIn hin[2];
        load_hb(hin[0], 0);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            if (hb + 1 < NHB) load_hb(hin[(hb + 1) & 1], hb + 1);
            const HbIn &x = hin[hb & 1];
            f32x4 dEp = zero4(), dQp = zero4(), dKp = zero4(), dQh = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const MB::frag kp = load_frag_fac(sKpt + 16 * hb * L64, L64, hb, kk, lane);
                dEp = MB::mma(fA[kk], kp, dEp);
                dQp = MB::mma(fM[kk], kp, dQp);
                dKp = MB::mma(fAt[kk], load_frag_fac(sEpt + 16 * hb * L64, L64, hb, kk, lane), dKp);
                dKp = MB::mma(fMt[kk], load_frag_fac(sQpt + 16 * hb * L64, L64, hb, kk, lane), dKp);
            }
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) dQh = MB::mma(fdO[kk], x.s[kk], dQh);
            const int cl = 16 * hb + (lane & 15), c = cbase + cl;
            const float gl_c = sGl[cl], gr_c = 0.5f * gl_c, egr = __expf(gr_c);
            const f32x4 dEc = dE[half * NHB + hb];
            float kdk = 0.0f;
            f32x4 dqv, dkv, dbv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * (lane >> 4) + r;
                float dg = 0.0f;
                dqv[r] = dkv[r] = dbv[r] = 0.0f;
                if (i < len) {
                    const float kf = static_cast<float>(x.k[r]), qf = static_cast<float>(x.q[r]);
                    const float bf = x.b[r];
                    const float dKh = static_cast<float>(x.dk[r]);
                    const float gg = sG[i * LDG + cl];
                    const float ex = __expf(gg - gr_c), ei = __expf(gr_c - gg);
                    const float gam = ex * egr, eK = ei * egr;
                    const float t1 = gam * dEc[r] + ex * dEp[r];
                    const float dq = gam * dQh[r] + ex * dQp[r];
                    const float kpart = ei * dKp[r] + eK * dKh;
                    dqv[r] = dq;
                    dkv[r] = bf * t1 + kpart;
                    dbv[r] = kf * t1;
                    dg = bf * kf * t1 + qf * dq - kf * kpart;
                    kdk += kf * eK * dKh;
                }
                sG[i * LDG + cl] = dg;  // each element is read, then overwritten, by this lane only
            }
            // dq, dk, db leave as row pieces (4 channels of one token per lane)
            // after a transpose inside each lane quad: one 8- or 16-byte store
            // per lane instead of four 2- or 4-byte ones.
            dqv = quad_transpose(dqv, lane);
            dkv = quad_transpose(dkv, lane);
            dbv = quad_transpose(dbv, lane);
            {
                const int i = 16 * I + 4 * (lane >> 4) + (lane & 3);
                if (i < len) {
                    const size_t off = ((size_t)(tok0 + i) * H + h) * DK + cbase + 16 * hb + 4 * ((lane >> 2) & 3);
                    *reinterpret_cast<bf16x4 *>(dqo + off) =
                        bf16x4{static_cast<bf16>(dqv[0]), static_cast<bf16>(dqv[1]), static_cast<bf16>(dqv[2]),
                               static_cast<bf16>(dqv[3])};
                    *reinterpret_cast<bf16x4 *>(dko + off) =
                        bf16x4{static_cast<bf16>(dkv[0]), static_cast<bf16>(dkv[1]), static_cast<bf16>(dkv[2]),
                               static_cast<bf16>(dkv[3])};
                    *reinterpret_cast<f32x4 *>(ba.db + off) = dbv;
                }
            }
            // sum over this wave's 16 tokens: 4 per lane, then the 4 lane groups
            kdk += __shfl_xor(kdk, 16);
            kdk += __shfl_xor(kdk, 32);
            if (lane < 16) {
                if (wave == 0) sKdk0[c] = kdk;
                else sKdk[(wave - 1) * DH + cl] = kdk;
            }
        }
        __syncthreads();

        // ---- dlog_alpha_j = sum_{i>=j} dg_i + gl dgl + sum_i Khat_i dKhat_i -------
        {
            f32x4 dgv[TPG];
#pragma unroll
            for (int j = 0; j < TPG; ++j) dgv[j] = *reinterpret_cast<const f32x4 *>(sG + (tg * TPG + j) * LDG + cq);
#pragma unroll
            for (int j = TPG - 2; j >= 0; --j) dgv[j] += dgv[j + 1];  // suffix sums inside the group
            *reinterpret_cast<f32x4 *>(sR + (C::NTG + tg) * DH + cq) = dgv[0];
            __syncthreads();
            f32x4 after = zero4();
#pragma unroll C::NTG_UNROLL
            for (int t = 0; t < C::NTG; ++t)
                if (t > tg) after += *reinterpret_cast<const f32x4 *>(sR + (C::NTG + t) * DH + cq);
            f32x4 dglast;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int cl = cq + c, cc = cbase + cl;
                dglast[c] = __expf(sGl[cl]) * sDG[cc] + sKdk0[cc] + sKdk[cl] + sKdk[DH + cl] + sKdk[2 * DH + cl];
            }
#pragma unroll
            for (int j = 0; j < TPG; ++j) {
                const int i = tg * TPG + j;
                if (i < len)
                    *reinterpret_cast<f32x4 *>(ba.dla + ((size_t)(tok0 + i) * H + h) * DK + cbase + cq) =
                        dgv[j] + after + dglast;
            }
        }
        __syncthreads();  // the next half reuses the tiles, g and the partials
    }
}

// Both per-chunk sides of one (chunk, head) on one workgroup, one after the
// other.  The state side's partial gradients reach the factor side in
// registers (dU_eff S^T, dO U_eff^T, dZ U^T, T^T fragments), through LDS (the
// gamma_last gradient; dW^T and dM as fragment-ordered images written between
// the two sides) or, for dKhat, through the workspace; the operands both
// sides read (S, dO, W) come back from the caches.
template <int DK>
__global__ __launch_bounds__(kThreads, 2) void chunk_bwd_local_kernel(BwdArgs ba) {
    const ChunkArgs &a = ba.c;
    const int cid = blockIdx.x / a.H;
    if (a.plan && cid >= a.plan[a.N]) return;
    int tok0, len;
    dense_span(a, cid, tok0, len);
    if (len <= 0) return;  // (a malformed table only) no token: nothing to write
    StateOut<DK> st;
    bwd_state_side<DK>(ba, st);
    __syncthreads();  // the state side's tiles are dead
    {
        bf16 *sWt = reinterpret_cast<bf16 *>(bwd_smem + FacCfg<DK>::OFF_A);  // dW^T [DK][64]
        bf16 *sMi = reinterpret_cast<bf16 *>(bwd_smem + FacCfg<DK>::OFF_G);  // dM [64][64], fo_slot
        const int lane = threadIdx.x & 63, I = threadIdx.x >> 6;
        const int i0 = 16 * I + 4 * (lane >> 4), it = i0 + (lane & 3), lq = (lane >> 2) & 3;
#pragma unroll
        for (int cb = 0; cb < DK / 16; ++cb) store4_frag<bf16>(sWt, kChunk, 16 * cb + (lane & 15), i0, -st.dWn[cb]);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const int j = 16 * J + (lane & 15);
            f32x4 m;
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = j <= i0 + r ? st.dM[J][r] : 0.0f;  // dM is zero above the diagonal
            m = quad_transpose(m, lane);
            *reinterpret_cast<bf16x4 *>(const_cast<bf16 *>(fo_at(sMi, it, 16 * J + 4 * lq, kChunk))) =
                bf16x4{static_cast<bf16>(m[0]), static_cast<bf16>(m[1]), static_cast<bf16>(m[2]),
                       static_cast<bf16>(m[3])};
        }
    }
    __syncthreads();
    bwd_factor_side<DK>(ba, st);
}

template <int D>
static void launch_bwd_d(const BwdArgs &a, hipStream_t stream) {
    const int chains = a.c.N * a.c.H, groups = (chains + 7) / 8;
    const dim3 block(kThreads);
    if (chains >= 256)  // 64-column slabs, 4 waves: two workgroups per CU
        hipLaunchKernelGGL((chunk_bwd_rev_kernel<D, 64>), dim3(groups * 8 * (D / 64)), block, 0, stream, a);
    else if (chains >= 64)  // 64-column slabs, two 32-column halves
        hipLaunchKernelGGL((chunk_bwd_rev2_kernel<D, 32>), dim3(groups * 8 * (D / 64)), dim3(2 * kThreads),
                           0, stream, a);
    else  // 32-column slabs, two 16-column halves
        hipLaunchKernelGGL((chunk_bwd_rev2_kernel<D, 16>), dim3(groups * 8 * (D / 32)), dim3(2 * kThreads),
                           0, stream, a);
    if (a.c.max_chunks == 0) return;
    const dim3 grid((unsigned)((size_t)a.c.max_chunks * a.c.H));
    hipLaunchKernelGGL((chunk_bwd_local_kernel<D>), grid, block, 0, stream, a);
}

hipError_t launch_chunk_bwd(const BwdArgs &a, int Dk, hipStream_t stream) {
    if (Dk == 128) launch_bwd_d<128>(a, stream);
    else launch_bwd_d<64>(a, stream);
    return hipGetLastError();
}

}  // namespace gdn2
