// State-propagation kernel: the only sequential part of the chunk forward.
//
// For each (sequence, head) the fp32 state is carried across the chunks of
// the sequence in order.  With the chunk factors of the chunk-factor kernel
// (U = T (w*v), W, Qhat, Khat, M, gamma_last), one chunk is
//
//   U_eff = U - W S                  per-token corrected values
//   O     = Qhat S + M U_eff         the query reads the updated state
//   S    <- Diag(gamma_last) S + Khat^T U_eff
//
// which is the unrolled recurrence of the pages' update (see the chunk-factor
// kernel for the sources).  Every step acts on the columns of S (the value
// axis) independently, so each (sequence, head) is split into Dv / DVS
// column slabs, one workgroup per slab.  The slab's fp32 state lives in MFMA
// accumulator registers for the whole sequence; a bf16 (or fp32) copy of it,
// transposed and double-buffered, is kept in LDS as the MFMA operand.  All
// loads of chunk c+1 (operand fragments straight from the workspace into
// registers) are issued before chunk c is computed.  Workgroup ids are mapped
// so that all slabs of one (sequence, head) land on the same XCD (ids are
// dispatched round-robin over the 8 XCDs), where they share the chunk
// factors through that XCD's L2.

#include <type_traits>

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <typename E, int DK, int DVS>
struct PropCfg {
    static constexpr int PAD = (sizeof(E) == 2) ? 8 : 4;
    static constexpr int LDS_ = DK + PAD;       // S^T     [DVS][LDS_]
    static constexpr int LDU = kChunk + PAD;    // U_eff^T [DVS][LDU]
    static constexpr int NCB = DVS / 16;        // 16-column blocks of the slab
    static constexpr int NKB = DK / 16;         // 16-row blocks of the state
    static constexpr int S_TPW = NKB * NCB / 4; // state tiles per wave
    static constexpr int KB_W = NKB / 4;        // state row blocks per wave
    static constexpr size_t SZ_S = size_t(DVS) * LDS_ * sizeof(E);
    static constexpr size_t SMEM = 2 * SZ_S + size_t(DVS) * LDU * sizeof(E);
    static_assert(S_TPW * 4 == NKB * NCB && KB_W * 4 == NKB, "state tiles split over 4 waves");
};

// Everything one wave reads from memory for one chunk: the operand fragments of
// its row blocks (W, Qhat, M, the state rows of Khat^T, gamma_last) and its U
// tiles (already in accumulator order).
template <typename E, int DK, int DVS>
struct ChunkFrags {
    using M = Mma<E>;
    using C = PropCfg<E, DK, DVS>;
    using V4 = typename std::conditional<sizeof(E) == 2, bf16x4, f32x4>::type;
    static constexpr int NK64 = kChunk / M::KS;
    static constexpr int NKD = DK / M::KS;
    typename M::frag w[NKD], qh[NKD], m[NK64], kh[C::KB_W][NK64];
    V4 u[C::NCB];
    f32x4 gl[C::KB_W];
    int tok0, len;
};

template <typename E, int DK, int DV, int DVS>
__device__ __forceinline__ void load_chunk(ChunkFrags<E, DK, DVS> &f, const ChunkArgs &a, int n,
                                           int h, int cid, int cbeg, int col0, int wave,
                                           int lane) {
    using M = Mma<E>;
    using C = PropCfg<E, DK, DVS>;
    using F = ChunkFrags<E, DK, DVS>;
    if (a.plan) {
        // Entries are clamped so that a stale or malformed table stays in bounds.
        const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
        f.tok0 = min(max(e[1], 0), a.T);
        f.len = min(max(e[2], 0), min(kChunk, a.T - f.tok0));
    } else {
        const int c = cid - cbeg;
        f.tok0 = n * a.T + c * kChunk;
        f.len = min(kChunk, a.T - c * kChunk);
    }
    const size_t ch = (size_t)cid * a.H + h;
    // W, Qhat, M and Khat^T are stored in fragment order (see frag_index).
    const E *Wg = reinterpret_cast<const E *>(a.ws_W) + ch * kChunk * DK;
    const E *Qg = reinterpret_cast<const E *>(a.ws_Qh) + ch * kChunk * DK;
    const E *Mg = reinterpret_cast<const E *>(a.ws_M) + ch * kChunk * kChunk;
    const E *Kg = reinterpret_cast<const E *>(a.ws_KhT) + ch * DK * kChunk;
    const E *Ug = reinterpret_cast<const E *>(a.ws_U) + ch * kChunk * DV +
                  ((wave * (DV / 16) + col0 / 16) * 64 + lane) * 4;
    const float *gl = a.ws_gl + ch * DK;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
        f.u[cb] = *reinterpret_cast<const typename F::V4 *>(Ug + cb * 64 * 4);
#pragma unroll
    for (int kk = 0; kk < F::NKD; ++kk) f.w[kk] = load_frag_packed<E>(Wg, DK, wave, kk, lane);
#pragma unroll
    for (int kk = 0; kk < F::NK64; ++kk) f.m[kk] = load_frag_packed<E>(Mg, kChunk, wave, kk, lane);
#pragma unroll
    for (int kk = 0; kk < F::NKD; ++kk) f.qh[kk] = load_frag_packed<E>(Qg, DK, wave, kk, lane);
#pragma unroll
    for (int b = 0; b < C::KB_W; ++b) {
        const int cblk = wave * C::KB_W + b;
#pragma unroll
        for (int kk = 0; kk < F::NK64; ++kk)
            f.kh[b][kk] = load_frag_packed<E>(Kg, kChunk, cblk, kk, lane);
        f.gl[b] = *reinterpret_cast<const f32x4 *>(gl + 16 * cblk + 4 * (lane >> 4));
    }
}

template <typename E, typename V4>
__device__ __forceinline__ f32x4 to_f32x4(V4 x) {
    return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kThreads, 2) void chunk_prop_kernel(ChunkArgs a) {
    using C = PropCfg<E, DK, DVS>;
    using M = Mma<E>;
    using F = ChunkFrags<E, DK, DVS>;
    constexpr int NS = DV / DVS, LDS_ = C::LDS_, LDU = C::LDU, NCB = C::NCB;
    // Double-buffer the fragments in registers for bf16; fp32 fragments are
    // 4x larger, so the fp32 path loads each chunk just before using it.
    constexpr bool kPrefetch = sizeof(E) == 2;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    E *sS0 = reinterpret_cast<E *>(smem);               // S^T of the slab, two buffers
    E *sU = reinterpret_cast<E *>(smem + 2 * C::SZ_S);   // U_eff^T

    const int H = a.H;
    const int x = blockIdx.x, xcd = x & 7, rest = x >> 3;
    const int slab = rest % NS, chain = (rest / NS) * 8 + xcd;
    if (chain >= a.N * H) return;
    const int n = chain / H, h = chain % H;
    const int col0 = slab * DVS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int cbeg, cend;
    if (a.plan) {
        cbeg = min(max(a.plan[n], 0), a.max_chunks);
        cend = min(max(a.plan[n + 1], cbeg), a.max_chunks);
    } else {
        cbeg = n * a.NC;
        cend = cbeg + a.NC;
    }

    F cur, nxt;
    if (cbeg < cend) load_chunk<E, DK, DV, DVS>(cur, a, n, h, cbeg, cbeg, col0, wave, lane);

    // Initial state (fp32 accumulators) and its operand copy.
    f32x4 Sacc[C::S_TPW];
#pragma unroll
    for (int u = 0; u < C::S_TPW; ++u) {
        const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
        const int col = col0 + 16 * colb + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cblk + 4 * (lane >> 4) + r;
            Sacc[u][r] = a.S0 ? a.S0[((size_t)chain * DK + c) * DV + col] : 0.0f;
        }
        store_tile_t<E>(sS0 + 16 * colb * LDS_ + 16 * cblk, LDS_, Sacc[u], lane);
    }
    __syncthreads();

    E *out = reinterpret_cast<E *>(a.o);
    int buf = 0;
    for (int cid = cbeg; cid < cend; ++cid) {
        if constexpr (kPrefetch) {
            if (cid + 1 < cend)
                load_chunk<E, DK, DV, DVS>(nxt, a, n, h, cid + 1, cbeg, col0, wave, lane);
        }
        const E *sS = sS0 + buf * (DVS * LDS_);
        E *sSn = sS0 + (buf ^ 1) * (DVS * LDS_);

        // U_eff rows of block `wave`:  U - W S.
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            f32x4 ws = zero4();
#pragma unroll
            for (int kk = 0; kk < F::NKD; ++kk)
                ws = M::mma(cur.w[kk], load_frag<E>(sS + 16 * cb * LDS_ + kk * M::KS, LDS_, lane),
                            ws);
            store_tile_t<E>(sU + 16 * cb * LDU + 16 * wave, LDU, to_f32x4<E>(cur.u[cb]) - ws, lane);
        }
        __syncthreads();

        // O^T rows of block `wave`:  D[col][i] = S^T Qhat^T + U_eff^T M^T.
        {
            const int i = 16 * wave + (lane & 15);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < F::NKD; ++kk)
                    acc = M::mma(load_frag<E>(sS + 16 * cb * LDS_ + kk * M::KS, LDS_, lane),
                                 cur.qh[kk], acc);
#pragma unroll
                for (int kk = 0; kk < F::NK64; ++kk)
                    acc = M::mma(load_frag<E>(sU + 16 * cb * LDU + kk * M::KS, LDU, lane),
                                 cur.m[kk], acc);
                if (i < cur.len) {
                    E *dst = out + ((size_t)(cur.tok0 + i) * H + h) * DV + col0 + 16 * cb +
                             4 * (lane >> 4);
                    if constexpr (sizeof(E) == 2) {
                        bf16x4 ov;
#pragma unroll
                        for (int r = 0; r < 4; ++r) ov[r] = static_cast<bf16>(acc[r]);
                        *reinterpret_cast<bf16x4 *>(dst) = ov;
                    } else {
                        *reinterpret_cast<f32x4 *>(dst) = acc;
                    }
                }
            }
        }
        // S <- Diag(gamma_last) S + Khat^T U_eff, and its operand copy for the next chunk.
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int b = u / NCB, colb = u % NCB;
            f32x4 d = zero4();
#pragma unroll
            for (int kk = 0; kk < F::NK64; ++kk)
                d = M::mma(cur.kh[b][kk], load_frag<E>(sU + 16 * colb * LDU + kk * M::KS, LDU, lane),
                           d);
            Sacc[u] = cur.gl[b] * Sacc[u] + d;
            const int cblk = wave * C::KB_W + b;
            store_tile_t<E>(sSn + 16 * colb * LDS_ + 16 * cblk, LDS_, Sacc[u], lane);
        }
        __syncthreads();
        buf ^= 1;
        if constexpr (kPrefetch) {
            cur = nxt;
        } else {
            if (cid + 1 < cend)
                load_chunk<E, DK, DV, DVS>(cur, a, n, h, cid + 1, cbeg, col0, wave, lane);
        }
    }

    if (a.S_final) {
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
            const int col = col0 + 16 * colb + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * cblk + 4 * (lane >> 4) + r;
                a.S_final[((size_t)chain * DK + c) * DV + col] = Sacc[u][r];
            }
        }
    }
}

// Slab width.  Every slab workgroup of a (sequence, head) reads all of that
// chunk's factors through its CU's vector memory path, which bounds the time
// per chunk; wide slabs cut that re-reading, narrow slabs give parallelism
// when there are few (sequence, head) chains.
static int choose_dvs(int chains, int Dv) {
    if (Dv >= 64 && chains >= 128) return 64;
    if (Dv >= 32 && chains >= 64) return 32;
    return 16;
}

template <typename E, int D>
static void launch_prop_d(const ChunkArgs &a, int dvs, hipStream_t stream) {
    const int chains = a.N * a.H;
    const int groups = (chains + 7) / 8;
    const dim3 block(kThreads);
    if (dvs == 64) {
        hipLaunchKernelGGL((chunk_prop_kernel<E, D, D, 64>), dim3(groups * 8 * (D / 64)), block, 0,
                           stream, a);
    } else if (dvs == 32) {
        hipLaunchKernelGGL((chunk_prop_kernel<E, D, D, 32>), dim3(groups * 8 * (D / 32)), block, 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((chunk_prop_kernel<E, D, D, 16>), dim3(groups * 8 * (D / 16)), block, 0,
                           stream, a);
    }
}

hipError_t launch_chunk_prop(const ChunkArgs &a, int Dk, bool bf16_io, hipStream_t stream) {
    const int dvs = choose_dvs(a.N * a.H, Dk);
    if (bf16_io) {
        if (Dk == 128) launch_prop_d<bf16, 128>(a, dvs, stream);
        else launch_prop_d<bf16, 64>(a, dvs, stream);
    } else {
        if (Dk == 128) launch_prop_d<float, 128>(a, dvs, stream);
        else launch_prop_d<float, 64>(a, dvs, stream);
    }
    return hipGetLastError();
}

}  // namespace gdn2
