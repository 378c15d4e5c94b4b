// State-propagation kernel: the only sequential part of the chunk forward.
//
// For each (sequence, head) the fp32 state is carried across the chunks of
// the sequence in order.  With the chunk factors of the chunk-factor kernel
// (T = (I + A)^-1, W, Qhat, Khat, M, gamma_last) and Z = w * v, one chunk is
//
//   U     = T Z                      write-side auxiliary
//   U_eff = U - W S                  per-token corrected values
//   O     = Qhat S + M U_eff         the query reads the updated state
//   S    <- Diag(gamma_last) S + Khat^T U_eff
//
// which is the unrolled recurrence of the pages' update (see the chunk-factor
// kernel for the sources).  Every step acts on the columns of S (the value
// axis) independently, so each (sequence, head) is split into Dv / DVS
// column slabs, one workgroup per slab.  The slab's fp32 state lives in MFMA
// accumulator registers for the whole sequence; a bf16 (or fp32) copy of it,
// transposed, is kept in LDS as the MFMA operand.  Workgroup ids are mapped
// so that all slabs of one (sequence, head) land on the same XCD (ids are
// dispatched round-robin over the 8 XCDs), where they share the chunk
// factors through that XCD's L2.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <typename E, int DK, int DVS>
struct PropCfg {
    static constexpr int PAD = (sizeof(E) == 2) ? 8 : 4;
    static constexpr int LDS_ = DK + PAD;       // S^T     [DVS][LDS_]
    static constexpr int LDZ = kChunk + PAD;    // Z^T, U_eff^T [DVS][LDZ]
    static constexpr int NCB = DVS / 16;        // 16-column blocks of the slab
    static constexpr int NKB = DK / 16;         // 16-row blocks of the state
    static constexpr int S_TPW = NKB * NCB / 4; // state tiles per wave
    static constexpr size_t SMEM = (size_t(DVS) * LDS_ + 2 * size_t(DVS) * LDZ) * sizeof(E);
    static_assert(S_TPW * 4 == NKB * NCB, "state tiles split over 4 waves");
};

template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kThreads, 2) void chunk_prop_kernel(ChunkArgs a) {
    using C = PropCfg<E, DK, DVS>;
    using M = Mma<E>;
    constexpr int NS = DV / DVS, LDS_ = C::LDS_, LDZ = C::LDZ, NCB = C::NCB;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    E *sS = reinterpret_cast<E *>(smem);   // S^T of the slab
    E *sZ = sS + DVS * LDS_;               // Z^T
    E *sU = sZ + DVS * LDZ;                // U_eff^T

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

    // Initial state (fp32 accumulators) and its operand copy.
    f32x4 Sacc[C::S_TPW];
#pragma unroll
    for (int u = 0; u < C::S_TPW; ++u) {
        const int t = wave * C::S_TPW + u, cblk = t / NCB, colb = t % NCB;
        const int col = col0 + 16 * colb + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cblk + 4 * (lane >> 4) + r;
            Sacc[u][r] = a.S0 ? a.S0[((size_t)chain * DK + c) * DV + col] : 0.0f;
        }
        store_tile_t<E>(sS + 16 * colb * LDS_ + 16 * cblk, LDS_, Sacc[u], lane);
    }

    const E *vin = reinterpret_cast<const E *>(a.v);
    E *out = reinterpret_cast<E *>(a.o);
    constexpr int ZC = DVS / 4;  // columns of Z per thread
    const int zi = tid & 63, zc0 = (tid >> 6) * ZC;

    for (int cid = cbeg; cid < cend; ++cid) {
        int tok0, len;
        if (a.plan) {
            const int32_t *e = a.plan + a.N + 1 + 3 * (size_t)cid;
            tok0 = min(max(e[1], 0), a.T);
            len = min(max(e[2], 0), min(kChunk, a.T - tok0));
        } else {
            const int c = cid - cbeg;
            tok0 = n * a.T + c * kChunk;
            len = min(kChunk, a.T - c * kChunk);
        }
        const size_t ch = (size_t)cid * H + h;
        const E *Tg = reinterpret_cast<const E *>(a.ws_T) + ch * kChunk * kChunk;
        const E *Wg = reinterpret_cast<const E *>(a.ws_W) + ch * kChunk * DK;
        const E *Qg = reinterpret_cast<const E *>(a.ws_Qh) + ch * kChunk * DK;
        const E *Kg = reinterpret_cast<const E *>(a.ws_KhT) + ch * DK * kChunk;
        const E *Mg = reinterpret_cast<const E *>(a.ws_M) + ch * kChunk * kChunk;
        const float *gl = a.ws_gl + ch * DK;

        // Z^T = (w * v)^T of the slab (zero past the chunk's length).
        {
            float zv[ZC];
            if (zi < len) {
                const size_t off = ((size_t)(tok0 + zi) * H + h) * DV + col0 + zc0;
#pragma unroll
                for (int j = 0; j < ZC; ++j) zv[j] = a.w[off + j] * to_f32(vin[off + j]);
            } else {
#pragma unroll
                for (int j = 0; j < ZC; ++j) zv[j] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < ZC; ++j) sZ[(zc0 + j) * LDZ + zi] = from_f32<E>(zv[j]);
        }
        __syncthreads();

        // U_eff rows of block `wave`:  T Z - W S.
        {
            const int KT = ((16 * (wave + 1) + M::KS - 1) / M::KS) * M::KS;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 u = mma_tile_k<E>(zero4(), Tg + 16 * wave * kChunk, kChunk,
                                        sZ + 16 * cb * LDZ, LDZ, KT, lane);
                f32x4 ws = mma_tile<E, DK>(zero4(), Wg + 16 * wave * DK, DK,
                                           sS + 16 * cb * LDS_, LDS_, lane);
                store_tile_t<E>(sU + 16 * cb * LDZ + 16 * wave, LDZ, u - ws, lane);
            }
        }
        __syncthreads();

        // O^T rows of block `wave`:  D[col][i] = S^T Qhat^T + U_eff^T M^T.
        {
            const int KM = ((16 * (wave + 1) + M::KS - 1) / M::KS) * M::KS;
            const int i = 16 * wave + (lane & 15);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 acc = mma_tile<E, DK>(zero4(), sS + 16 * cb * LDS_, LDS_,
                                            Qg + 16 * wave * DK, DK, lane);
                acc = mma_tile_k<E>(acc, sU + 16 * cb * LDZ, LDZ, Mg + 16 * wave * kChunk, kChunk,
                                    KM, lane);
                if (i < len) {
                    E *dst = out + ((size_t)(tok0 + i) * H + h) * DV + col0 + 16 * cb +
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
        // S <- Diag(gamma_last) S + Khat^T U_eff.
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int t = wave * C::S_TPW + u, cblk = t / NCB, colb = t % NCB;
            const f32x4 g = *reinterpret_cast<const f32x4 *>(gl + 16 * cblk + 4 * (lane >> 4));
            const f32x4 d = mma_tile<E, kChunk>(zero4(), Kg + 16 * cblk * kChunk, kChunk,
                                                sU + 16 * colb * LDZ, LDZ, lane);
            Sacc[u] = g * Sacc[u] + d;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int t = wave * C::S_TPW + u, cblk = t / NCB, colb = t % NCB;
            store_tile_t<E>(sS + 16 * colb * LDS_ + 16 * cblk, LDS_, Sacc[u], lane);
        }
    }

    if (a.S_final) {
#pragma unroll
        for (int u = 0; u < C::S_TPW; ++u) {
            const int t = wave * C::S_TPW + u, cblk = t / NCB, colb = t % NCB;
            const int col = col0 + 16 * colb + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * cblk + 4 * (lane >> 4) + r;
                a.S_final[((size_t)chain * DK + c) * DV + col] = Sacc[u][r];
            }
        }
    }
}

// Slab width: the widest of 64/32/16 columns that still gives >= 512 workgroups.
static int choose_dvs(int chains, int Dv) {
    for (int dvs = 64; dvs >= 16; dvs >>= 1)
        if (dvs <= Dv && (long long)chains * (Dv / dvs) >= 512) return dvs;
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
