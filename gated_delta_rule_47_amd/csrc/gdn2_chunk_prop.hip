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
// transposed, is kept in LDS as the MFMA operand.  Workgroup ids are mapped
// so that all slabs of one (sequence, head) land on the same XCD (ids are
// dispatched round-robin over the 8 XCDs), where they share the chunk
// factors through that XCD's L2.
//
// Two implementations: for bf16, 4 compute waves fed through LDS by 4 loader
// waves (chunk_prop_ws_kernel); for fp32, whose fragments are twice as large,
// 4 waves that load their own operand fragments (chunk_prop_kernel).

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
    for (int kk = 0; kk < F::NK64; ++kk)  // fragments wholly above the diagonal are not stored
        f.m[kk] = m_frag_used<E>(wave, kk * M::KS) ? load_frag_packed<E>(Mg, kChunk, wave, kk, lane)
                                                   : M::zero();
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

// Two workgroups per CU where their LDS fits (fp32 with 64-column slabs of
// 128-wide heads needs 85 KB: one workgroup per CU, all registers).
template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kThreads, (PropCfg<E, DK, DVS>::SMEM <= 80 * 1024 ? 2 : 1)) void chunk_prop_kernel(ChunkArgs a) {
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
    load_state_tiles<DK, DV, C::KB_W, NCB>(Sacc, a.S0, chain, wave, col0, lane);
#pragma unroll
    for (int u = 0; u < C::S_TPW; ++u) {
        const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
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
        if (a.ws_Sc32) {  // fp32 backward calls: this chunk's incoming state, row-major
#pragma unroll
            for (int u = 0; u < C::S_TPW; ++u) {
                const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
                const int col = col0 + 16 * colb + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int c = 16 * cblk + 4 * (lane >> 4) + r;
                    a.ws_Sc32[(((size_t)cid * H + h) * DK + c) * DV + col] = Sacc[u][r];
                }
            }
        }

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
                    if (m_frag_used<E>(wave, kk * M::KS))
                        acc = M::mma(load_frag<E>(sU + 16 * cb * LDU + kk * M::KS, LDU, lane),
                                     cur.m[kk], acc);
                if (out && i < cur.len) {
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

// ---------------------------------------------------------------------------
// bf16 path with producer waves.
//
// A compute wave that issues its own prefetch stalls in the issue of those
// loads for as long as the memory pipeline takes to return earlier ones, and
// cannot do MFMA work meanwhile.  Here each workgroup has 4 compute waves and
// 4 loader waves.  The loader waves copy the fragment-ordered W, Qhat, M and
// Khat^T of a chunk (a byte-for-byte image of the workspace, so every fragment
// is one conflict-free 16-byte-per-lane LDS read) into one of two LDS stages,
// two chunks ahead: during chunk c they write chunk c+1 (loaded during chunk
// c-1) into the free stage and then issue the loads of chunk c+2.  The compute
// waves read the factors from the stage and load only their own U tiles and
// gamma_last.  Qhat S does not depend on U_eff, so it is formed before the
// mid-chunk barrier, together with W S.
// ---------------------------------------------------------------------------
template <int DK, int DVS>
struct WsCfg {
    static constexpr int PAD = 8;
    static constexpr int LDS_ = DK + PAD;       // S^T     [DVS][LDS_]
    static constexpr int LDU = kChunk + PAD;    // U_eff^T [DVS][LDU]
    static constexpr int NCB = DVS / 16;
    static constexpr int NKB = DK / 16;
    static constexpr int S_TPW = NKB * NCB / 4;
    static constexpr int KB_W = NKB / 4;
    static constexpr int NG_W = kChunk * DK * 2 / 16;      // 16-byte granules of W, Qhat, Khat^T
    static constexpr int NG_M = kChunk * kChunk * 2 / 16;  // of M
    static constexpr int NG = 3 * NG_W + NG_M;             // one chunk's stage: W | Qhat | M | Khat^T
    static constexpr int NJ = NG / kThreads;               // loads per loader thread
    static constexpr size_t SZ_STAGE = size_t(NG) * 16;
    static constexpr size_t SZ_S = size_t(DVS) * LDS_ * 2;
    static constexpr int LDO = DVS + 8;         // O staging [64][LDO]
    static constexpr int GPR_O = DVS / 8;       // 16-byte granules per token row of O
    static constexpr size_t SZ_U = size_t(DVS) * LDU * 2;
    static constexpr size_t SZ_O = size_t(kChunk) * LDO * 2;
    static constexpr size_t SMEM = 2 * SZ_STAGE + SZ_S + SZ_U + SZ_O;
    static_assert(NG % kThreads == 0 && NG_W % kThreads == 0 && NG_M % kThreads == 0, "loader split");
    static_assert(S_TPW * 4 == NKB * NCB && KB_W * 4 == NKB, "state tiles split over 4 waves");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

typedef unsigned int granule_t __attribute__((ext_vector_type(4)));

// A states-only call stages each chunk's incoming state, bf16 [Dk][DVS], in
// the Qhat part of stage 0 (unused by such a call) so that it leaves in
// 16-byte pieces.  Unpadded rows; the 16-byte granules of row c are permuted
// by an even XOR key taken from c / 4, which puts the four row groups of an
// accumulator tile store on different banks.
template <int DVS>
__device__ __forceinline__ int sr_index(int c, int v) {
    constexpr int NGR = DVS / 8;
    const int key = 2 * ((c >> 2) & (NGR / 2 - 1));
    return c * DVS + (((v >> 3) ^ key) << 3) + (v & 7);
}

// Accumulator tile (state rows 16 cblk.., columns 16 colb.. of the slab) into
// that order.
// kSaveSc: state tile (rows 16 cblk.., columns 16 colb.. of the slab) of a
// chunk's incoming state straight to its workspace copy, as 8-byte row pieces
// after a quad transpose (row 16 cblk + 4 (lane/16) + lane%4, four
// consecutive columns), in the sc_index layout.
template <int DK>
__device__ __forceinline__ void store_state_pieces(bf16 *Sc, int cblk, int colb, int col0, f32x4 acc,
                                                   int lane) {
    const f32x4 t = quad_transpose(acc, lane);
    const int c = 16 * cblk + 4 * (lane >> 4) + (lane & 3), v = col0 + 16 * colb + 4 * ((lane >> 2) & 3);
    *reinterpret_cast<bf16x4 *>(Sc + sc_index(c, v, DK)) =
        bf16x4{static_cast<bf16>(t[0]), static_cast<bf16>(t[1]), static_cast<bf16>(t[2]), static_cast<bf16>(t[3])};
}

template <int DVS>
__device__ __forceinline__ void store_state_rows(bf16 *sSr, int cblk, int colb, f32x4 acc, int lane) {
    const int v = 16 * colb + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        sSr[sr_index<DVS>(16 * cblk + 4 * (lane >> 4) + r, v)] = static_cast<bf16>(acc[r]);
}

template <int NJ>
struct StageRegs {
    granule_t v[NJ];
};

// Loader thread t (0..255) moves granules t, t+256, ... of a chunk's stage;
// load j covers granules 256j .. 256j+255, which lie in one of the four arrays.
template <int DK, int DVS, int J>
__device__ __forceinline__ granule_t ws_load(const ChunkArgs &a, size_t ch, int t) {
    using C = WsCfg<DK, DVS>;
    constexpr int g = J * kThreads;
    if constexpr (g < C::NG_W)
        return reinterpret_cast<const granule_t *>(a.ws_W)[ch * C::NG_W + g + t];
    else if constexpr (g < 2 * C::NG_W)
        return reinterpret_cast<const granule_t *>(a.ws_Qh)[ch * C::NG_W + g - C::NG_W + t];
    else if constexpr (g < 2 * C::NG_W + C::NG_M)
        return reinterpret_cast<const granule_t *>(a.ws_M)[ch * C::NG_M + g - 2 * C::NG_W + t];
    else
        return reinterpret_cast<const granule_t *>(a.ws_KhT)[ch * C::NG_W + g - 2 * C::NG_W - C::NG_M + t];
}

// Loads J .. J1-1: store each register of the chunk already loaded into
// `stage`, then reuse it for the same load of chunk-head `ch_next`, so that the
// loads stay in flight one after another.  The sequence has no branches, which
// lets every store wait for its own load only.  kStates (no output) moves
// only W and Khat^T: Qhat and M serve o alone.
template <int DK, int DVS, int J, int J1, bool kStates = false>
__device__ __forceinline__ void ws_pipe(StageRegs<WsCfg<DK, DVS>::NJ> &buf, char *stage,
                                        const ChunkArgs &a, size_t ch_next, int t) {
    if constexpr (J < J1) {
        using C = WsCfg<DK, DVS>;
        constexpr int g = J * kThreads;
        constexpr bool skip = kStates && g >= C::NG_W && g < 2 * C::NG_W + C::NG_M;
        if constexpr (!skip) {
            *reinterpret_cast<granule_t *>(stage + ((size_t)J * kThreads + t) * 16) = buf.v[J];
            buf.v[J] = ws_load<DK, DVS, J>(a, ch_next, t);
        }
        ws_pipe<DK, DVS, J + 1, J1, kStates>(buf, stage, a, ch_next, t);
    }
}

// Loader side: the O rows of one chunk (staged in LDS by the compute waves)
// to global memory, 16 bytes per lane, the slab's part of each token row
// contiguous, stored non-temporally (o is not read again by this call).
template <int DK, int DV, int DVS>
__device__ __forceinline__ void ws_store_o(const ChunkArgs &a, const bf16 *sO, int h, int tok0, int len,
                                           int col0, int t) {
    using C = WsCfg<DK, DVS>;
    bf16 *out = reinterpret_cast<bf16 *>(a.o);
#pragma unroll
    for (int g = t; g < kChunk * C::GPR_O; g += kThreads) {
        const int row = g / C::GPR_O, piece = g % C::GPR_O;
        if (row < len)
            __builtin_nontemporal_store(*reinterpret_cast<const granule_t *>(sO + row * C::LDO + 8 * piece),
                                        reinterpret_cast<granule_t *>(out + ((size_t)(tok0 + row) * a.H + h) * DV + col0 + 8 * piece));
    }
}

// kStates: also store every chunk's incoming state in a.ws_Sc (for the
// backward) and write no o.  kSaveSc (without kStates): write o and also
// store every chunk's incoming state in a.ws_Sc, from the compute waves'
// accumulators (the stage region that kStates uses for them holds Qhat).
template <int DK, int DV, int DVS, bool kStates, bool kSaveSc = false>
__global__ __launch_bounds__(2 * kThreads, 1) void chunk_prop_ws_kernel(ChunkArgs a) {
    static_assert(!(kStates && kSaveSc), "one way of storing the chunk states");
    using C = WsCfg<DK, DVS>;
    using M = Mma<bf16>;
    constexpr int NS = DV / DVS, LDS_ = C::LDS_, LDU = C::LDU, NCB = C::NCB;
    constexpr int NKD = DK / M::KS, NK64 = kChunk / M::KS;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    // S^T as the MFMA operand: read only before the mid-chunk barrier and
    // rewritten only after it, so one buffer serves.
    bf16 *sS = reinterpret_cast<bf16 *>(smem + 2 * C::SZ_STAGE);
    bf16 *sU = reinterpret_cast<bf16 *>(smem + 2 * C::SZ_STAGE + C::SZ_S);  // U_eff^T
    bf16 *sO = reinterpret_cast<bf16 *>(smem + 2 * C::SZ_STAGE + C::SZ_S + C::SZ_U);  // O, row-major
    bf16 *sSr = reinterpret_cast<bf16 *>(smem + (size_t)C::NG_W * 16);  // kStates: S, sr_index order
    static_assert(!kStates || DK * DVS * 2 <= C::NG_W * 16, "state rows fit the Qhat stage part");

    const int H = a.H;
    const int x = blockIdx.x, xcd = x & 7, rest = x >> 3;
    const int slab = rest % NS, chain = (rest / NS) * 8 + xcd;
    if (chain >= a.N * H) return;  // uniform over the workgroup
    const int n = chain / H, h = chain % H;
    const int col0 = slab * DVS;
    const int tid = threadIdx.x;

    int cbeg, cend;
    if (a.plan) {
        cbeg = min(max(a.plan[n], 0), a.max_chunks);
        cend = min(max(a.plan[n + 1], cbeg), a.max_chunks);
    } else {
        cbeg = n * a.NC;
        cend = cbeg + a.NC;
    }

    if (cbeg == cend) {  // nothing to propagate: S_final = S0, no barriers in either role
        if (tid >= kThreads || !a.S_final) return;
        for (int e = tid; e < DK * DVS; e += kThreads) {
            const size_t o = ((size_t)chain * DK + e / DVS) * DV + col0 + e % DVS;
            a.S_final[o] = a.S0 ? a.S0[o] : 0.0f;
        }
        return;
    }

    if (tid >= kThreads) {
        // ---- loader waves ----------------------------------------------------
        // Step `it` runs beside the compute of chunk cbeg+it-2, with the same
        // two barriers.  It first writes out the O rows of chunk cbeg+it-3
        // (staged by the compute waves during the previous step), then stores
        // the registers holding chunk cbeg+it-1 into that chunk's stage and
        // reuses them for chunk cbeg+it+1 (clamped to the last chunk; stages
        // written past the end are never read).  Two register sets alternate,
        // so a chunk's loads have two steps to arrive.  The loop is unrolled
        // by two and always runs an even number of steps; the stage traffic
        // has no branches, so the loads in flight at its head always come in
        // the same order and each store waits only for its own load.
        constexpr int NJ = C::NJ, NJ2 = NJ / 2;
        const int t = tid - kThreads, col0_ = col0, nch = cend - cbeg;
        // Token span of chunk k of this sequence, from its first token and end.
        int tok_first, seq_end;
        if (a.plan) {
            const int32_t *e0 = a.plan + a.N + 1 + 3 * (size_t)cbeg;
            const int32_t *e1 = a.plan + a.N + 1 + 3 * (size_t)(cend - 1);
            tok_first = min(max(e0[1], 0), a.T);
            seq_end = min(max(e1[1] + e1[2], tok_first), a.T);
        } else {
            tok_first = n * a.T;
            seq_end = tok_first + a.T;
        }
        auto store_o = [&](int k) {
            if constexpr (!kStates) {
                const int tok0 = min(tok_first + k * kChunk, a.T * (a.plan ? 1 : a.N));
                ws_store_o<DK, DV, DVS>(a, sO, h, tok0, min(kChunk, seq_end - tok0), col0_, t);
            }
        };
        // kStates: the incoming state of chunk k, staged by the compute waves
        // before the barrier that ends chunk k-1 and rewritten only after the
        // mid-chunk barrier of chunk k, to the workspace.
        auto store_sc = [&](int k) {
            if constexpr (kStates) {
                bf16 *Sc = a.ws_Sc + ((size_t)(cbeg + k) * H + h) * DK * DV;
                constexpr int NP = DK * DVS / 8, NPC = (NP + kThreads - 1) / kThreads;
#pragma unroll
                for (int p = 0; p < NPC; ++p) {
                    const int e = t + p * kThreads, c = e / (DVS / 8), v8 = 8 * (e % (DVS / 8));
                    if (NP % kThreads == 0 || e < NP)
                        *reinterpret_cast<granule_t *>(Sc + sc_index(c, col0_ + v8, DK)) =
                            *reinterpret_cast<const granule_t *>(sSr + sr_index<DVS>(c, v8));
                }
            }
        };
        auto chunk_head = [&](int k) { return (size_t)(cbeg + min(k, nch - 1)) * H + h; };
        StageRegs<NJ> buf0, buf1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) buf0.v[j] = granule_t{0u, 0u, 0u, 0u};
        // chunk 0 into buf1 (stored at step 1); buf0 receives chunk 1 at step 0
#pragma unroll
        for (int j = 0; j < NJ; ++j) buf1.v[j] = granule_t{0u, 0u, 0u, 0u};
        ws_pipe<DK, DVS, 0, NJ, kStates>(buf1, smem + C::SZ_STAGE, a, chunk_head(0), t);
        const int nsteps = (nch + 3) & ~1;  // nch + 2, rounded up to even
        for (int it = 0; it < nsteps; it += 2) {
            if (it >= 3 && it - 3 < nch) store_o(it - 3);
            if (kStates && it >= 2 && it - 2 < nch) store_sc(it - 2);
            ws_pipe<DK, DVS, 0, NJ2, kStates>(buf0, smem + C::SZ_STAGE, a, chunk_head(it + 1), t);
            __syncthreads();
            ws_pipe<DK, DVS, NJ2, NJ, kStates>(buf0, smem + C::SZ_STAGE, a, chunk_head(it + 1), t);
            __syncthreads();
            if (it + 1 >= 3 && it - 2 < nch) store_o(it - 2);
            if (kStates && it + 1 >= 2 && it - 1 < nch) store_sc(it - 1);
            ws_pipe<DK, DVS, 0, NJ2, kStates>(buf1, smem, a, chunk_head(it + 2), t);
            __syncthreads();
            ws_pipe<DK, DVS, NJ2, NJ, kStates>(buf1, smem, a, chunk_head(it + 2), t);
            __syncthreads();
        }
        if (nsteps - 3 < nch) store_o(nch - 1);  // the last chunk when no step after it remained
        return;
    }

    // ---- compute waves ----------------------------------------------------
    const int lane = tid & 63, wave = tid >> 6;
    // Per chunk: this wave's U tiles (accumulator order) and gamma_last of its
    // state rows, loaded two chunks ahead.
    struct Own {
        bf16x4 u[NCB];
        f32x4 gl[C::KB_W];
    };
    auto load_own = [&](Own &f, int cid) {
        const size_t ch = (size_t)cid * H + h;
        const bf16 *Ug = reinterpret_cast<const bf16 *>(a.ws_U) + ch * kChunk * DV +
                         ((wave * (DV / 16) + col0 / 16) * 64 + lane) * 4;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) f.u[cb] = *reinterpret_cast<const bf16x4 *>(Ug + cb * 64 * 4);
#pragma unroll
        for (int b = 0; b < C::KB_W; ++b)
            f.gl[b] = *reinterpret_cast<const f32x4 *>(a.ws_gl + ch * DK + 16 * (wave * C::KB_W + b) +
                                                       4 * (lane >> 4));
    };
    Own cur, nxt, nxt2;
    load_own(cur, cbeg);
    load_own(nxt, min(cbeg + 1, cend - 1));

    f32x4 Sacc[C::S_TPW];
    load_state_tiles<DK, DV, C::KB_W, NCB>(Sacc, a.S0, chain, wave, col0, lane);
#pragma unroll
    for (int u = 0; u < C::S_TPW; ++u) {
        const int cblk = wave * C::KB_W + u / NCB, colb = u % NCB;
        store_tile_t<bf16>(sS + 16 * colb * LDS_ + 16 * cblk, LDS_, Sacc[u], lane);
        if constexpr (kStates) store_state_rows<DVS>(sSr, cblk, colb, Sacc[u], lane);
        if constexpr (kSaveSc)
            store_state_pieces<DK>(a.ws_Sc + ((size_t)cbeg * H + h) * DK * DV, cblk, colb, col0, Sacc[u], lane);
    }
    // The loader's steps 0 and 1 (the first chunk reaches stage 0).
#pragma unroll
    for (int j = 0; j < 4; ++j) __syncthreads();

    for (int cid = cbeg; cid < cend; ++cid) {
        load_own(nxt2, min(cid + 2, cend - 1));
        const bf16 *stage = reinterpret_cast<const bf16 *>(smem + ((cid - cbeg) & 1) * C::SZ_STAGE);
        const bf16 *Wf = stage;
        const bf16 *Qf = stage + C::NG_W * 8;
        const bf16 *Mf = stage + 2 * C::NG_W * 8;
        const bf16 *Kf = stage + (2 * C::NG_W + C::NG_M) * 8;

        // Phase 1: U_eff rows of block `wave` (U - W S) and the state part of
        // O^T (S^T Qhat^T).  All operands are read first, then the products run
        // as 2*NCB independent accumulation chains.
        f32x4 oacc[NCB];
        {
            M::frag wf[NKD], qf[NKD], sf[NCB][NKD];
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                wf[kk] = load_frag_packed<bf16>(Wf, DK, wave, kk, lane);
                if constexpr (!kStates) qf[kk] = load_frag_packed<bf16>(Qf, DK, wave, kk, lane);
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk)
                    sf[cb][kk] = load_frag<bf16>(sS + 16 * cb * LDS_ + kk * M::KS, LDS_, lane);
            f32x4 ws[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) ws[cb] = oacc[cb] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    ws[cb] = M::mma(wf[kk], sf[cb][kk], ws[cb]);
                    if constexpr (!kStates) oacc[cb] = M::mma(sf[cb][kk], qf[kk], oacc[cb]);
                }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store_tile_t<bf16>(sU + 16 * cb * LDU + 16 * wave, LDU,
                                   to_f32x4<bf16>(cur.u[cb]) - ws[cb], lane);
        }
        __syncthreads();  // U_eff complete; S^T is no longer read this chunk

        // Phase 2: O^T += U_eff^T M^T;  S <- Diag(gamma_last) S + Khat^T U_eff.
        {
            M::frag uf[NCB][NK64], mf[NK64], kf[C::KB_W][NK64];
#pragma unroll
            for (int kk = 0; kk < NK64; ++kk) {
                if (!kStates && m_frag_used<bf16>(wave, kk * M::KS))
                    mf[kk] = load_frag_packed<bf16>(Mf, kChunk, wave, kk, lane);
#pragma unroll
                for (int b = 0; b < C::KB_W; ++b)
                    kf[b][kk] = load_frag_packed<bf16>(Kf, kChunk, wave * C::KB_W + b, kk, lane);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    uf[cb][kk] = load_frag<bf16>(sU + 16 * cb * LDU + kk * M::KS, LDU, lane);
            }
            f32x4 d[C::S_TPW];
#pragma unroll
            for (int u = 0; u < C::S_TPW; ++u) d[u] = zero4();
#pragma unroll
            for (int kk = 0; kk < NK64; ++kk) {
                if (!kStates && m_frag_used<bf16>(wave, kk * M::KS)) {  // M is zero above the diagonal
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) oacc[cb] = M::mma(uf[cb][kk], mf[kk], oacc[cb]);
                }
#pragma unroll
                for (int u = 0; u < C::S_TPW; ++u)
                    d[u] = M::mma(kf[u / NCB][kk], uf[u % NCB][kk], d[u]);
            }
            // O rows to the staging buffer; the loader waves write them out.
#pragma unroll
            for (int cb = 0; cb < (kStates ? 0 : NCB); ++cb) {
                bf16x4 ov;
#pragma unroll
                for (int r = 0; r < 4; ++r) ov[r] = static_cast<bf16>(oacc[cb][r]);
                *reinterpret_cast<bf16x4 *>(sO + (16 * wave + (lane & 15)) * C::LDO + 16 * cb +
                                            4 * (lane >> 4)) = ov;
            }
#pragma unroll
            for (int u = 0; u < C::S_TPW; ++u) {
                const int b = u / NCB, colb = u % NCB;
                Sacc[u] = cur.gl[b] * Sacc[u] + d[u];
                store_tile_t<bf16>(sS + 16 * colb * LDS_ + 16 * (wave * C::KB_W + b), LDS_, Sacc[u],
                                   lane);
                if constexpr (kStates) store_state_rows<DVS>(sSr, wave * C::KB_W + b, colb, Sacc[u], lane);
                if constexpr (kSaveSc) {  // the incoming state of the next chunk
                    if (cid + 1 < cend)
                        store_state_pieces<DK>(a.ws_Sc + ((size_t)(cid + 1) * H + h) * DK * DV,
                                               wave * C::KB_W + b, colb, col0, Sacc[u], lane);
                }
            }
        }
        __syncthreads();
        cur = nxt;
        nxt = nxt2;
    }
    if ((cend - cbeg) & 1) {  // the loader's padding step
        __syncthreads();
        __syncthreads();
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
    if constexpr (sizeof(E) == 2) {  // compute + loader waves
        const dim3 block(2 * kThreads);
        if (a.ws_Sc && a.o) {  // o and every chunk's incoming state (a forward for a later backward)
            if (dvs == 64)
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 64, false, true>), dim3(groups * 8 * (D / 64)),
                                   block, 0, stream, a);
            else if (dvs == 32)
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 32, false, true>), dim3(groups * 8 * (D / 32)),
                                   block, 0, stream, a);
            else
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 16, false, true>), dim3(groups * 8 * (D / 16)),
                                   block, 0, stream, a);
        } else if (a.ws_Sc) {
            if (dvs == 64)
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 64, true>), dim3(groups * 8 * (D / 64)),
                                   block, 0, stream, a);
            else if (dvs == 32)
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 32, true>), dim3(groups * 8 * (D / 32)),
                                   block, 0, stream, a);
            else
                hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 16, true>), dim3(groups * 8 * (D / 16)),
                                   block, 0, stream, a);
        } else if (dvs == 64) {
            hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 64, false>), dim3(groups * 8 * (D / 64)), block,
                               0, stream, a);
        } else if (dvs == 32) {
            hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 32, false>), dim3(groups * 8 * (D / 32)), block,
                               0, stream, a);
        } else {
            hipLaunchKernelGGL((chunk_prop_ws_kernel<D, D, 16, false>), dim3(groups * 8 * (D / 16)), block,
                               0, stream, a);
        }
    } else {
        const dim3 block(kThreads);
        if (dvs == 64)
            hipLaunchKernelGGL((chunk_prop_kernel<E, D, D, 64>), dim3(groups * 8 * (D / 64)), block, 0,
                               stream, a);
        else if (dvs == 32)
            hipLaunchKernelGGL((chunk_prop_kernel<E, D, D, 32>), dim3(groups * 8 * (D / 32)), block, 0,
                               stream, a);
        else
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
