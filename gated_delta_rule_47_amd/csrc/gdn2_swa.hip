// Sliding-window softmax attention, forward (the hybrid model's local
// attention: iplexlaw digest, section "Condiciones de comparación", 2K
// window; gist.science summary, part "4. Architecture", SWA interleaved with
// the Gated DeltaNet-2 mixer).  Query i of a sequence attends to keys
// i - window < j <= i of the same sequence:
//   o_i = sum_j softmax_j(scale q_i . k_j) v_j,   lse_i = log sum_j e^{scale q_i . k_j}.
//
// One workgroup (4 waves) takes 128 consecutive queries of one (sequence,
// head); wave w owns queries 32w .. 32w+31 as two 16-query tiles.  The keys
// of the window are walked in tiles of 64, double-buffered in LDS (K
// row-major, V transposed), with an online softmax in base 2.  Everything is
// computed transposed so that each lane owns one query column:
//   S^T = K Q^T      (16x16x32 bf16 MFMA; A = K rows from LDS, B = Q in registers)
//   O^T += V^T P^T   (A = V^T rows from LDS, B = P straight from the S^T
//                     accumulator registers, with the keys of each 32-wide
//                     contraction taken in the order the accumulator holds them)
// so the rescaling of O and the row sums need no cross-lane traffic; the row
// max is reduced across lanes only when it grows (lazy rescaling).
// Workgroups are mapped XCD-contiguously: consecutive query blocks of one
// head share most of their key window and run on the same XCD's L2.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // base-2 headroom before the running max is raised

template <int D>
struct SwaCfg {
    static constexpr int BM = kSwaBlockQueries, BN = 64, NC = D / 32, NDT = D / 16, NKT = BN / 16;
    static constexpr int LDK = D + 8;   // K tile [BN][LDK] bf16
    // V^T tile [D][LDV] bf16.  LDV = BN + 4 (34 dwords per row) puts the 16 rows
    // a fragment read touches on distinct bank pairs, and the transposing
    // stores (key group fastest across lanes) on distinct banks too.
    static constexpr int LDV = BN + 4;
    static constexpr int SZ_K = BN * LDK, SZ_V = D * LDV;  // elements
    static constexpr int KG = BN * D / 8;                  // 16-byte granules of a K tile
    static constexpr int VG = (D / 8) * (BN / 4);          // (8 dims x 4 keys) groups of a V tile
    static constexpr int KPT = (KG + kThreads - 1) / kThreads;
    static constexpr size_t SMEM = 2 * size_t(SZ_K + SZ_V) * 2;
    static_assert(VG <= kThreads, "one V group per thread");
};

template <int D>
struct SwaStage {
    bf16x8 kx[SwaCfg<D>::KPT];
    bf16x8 vx[4];
};

template <int D>
__device__ __forceinline__ void swa_load(const SwaArgs &a, int h, int s0, int s1, int k0, int tid,
                                         SwaStage<D> &st) {
    using C = SwaCfg<D>;
    const bf16 *K = reinterpret_cast<const bf16 *>(a.k);
    const bf16 *V = reinterpret_cast<const bf16 *>(a.v);
    const size_t ld = (size_t)a.H * D;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        const int id = tid + i * kThreads;
        const int key = min(id / (D / 8), C::BN - 1), dc = id % (D / 8);
        const int t = min(max(k0 + key, s0), s1 - 1);
        st.kx[i] = *reinterpret_cast<const bf16x8 *>(K + (size_t)t * ld + h * D + 8 * dc);
    }
    // V: thread -> (key group kg, fastest across lanes; 8-dim chunk dc)
    const int g = min(tid, C::VG - 1), kg = g % (C::BN / 4), dc = g / (C::BN / 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = min(max(k0 + 4 * kg + u, s0), s1 - 1);
        st.vx[u] = *reinterpret_cast<const bf16x8 *>(V + (size_t)t * ld + h * D + 8 * dc);
    }
}

template <int D>
__device__ __forceinline__ void swa_store(bf16 *sK, bf16 *sV, int tid, const SwaStage<D> &st) {
    using C = SwaCfg<D>;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        const int id = tid + i * kThreads;
        if (id < C::KG) {
            const int key = id / (D / 8), dc = id % (D / 8);
            *reinterpret_cast<bf16x8 *>(sK + key * C::LDK + 8 * dc) = st.kx[i];
        }
    }
    if (tid < C::VG) {  // 4 keys x 8 dims -> 8 rows of V^T, 4 keys each
        const int kg = tid % (C::BN / 4), dc = tid / (C::BN / 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 w;
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = st.vx[u][e];
            *reinterpret_cast<bf16x4 *>(sV + (8 * dc + e) * C::LDV + 4 * kg) = w;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void swa_fwd_kernel(SwaArgs a) {
    using C = SwaCfg<D>;
    using MB = Mma<bf16>;
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * (C::SZ_K + C::SZ_V)];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;

    // XCD-contiguous work mapping: work item w = (sequence, head, query block)
    // with query blocks fastest; XCD x takes items [x*per, (x+1)*per).
    // (packed calls: n_items is an upper bound, the real count is blk_start[N])
    const int per = (a.n_items + 7) / 8;
    const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (item >= (a.cu_seqlens ? a.blk_start[a.N] : a.n_items)) return;
    // locate the item: sequences in order, each with H * nblk(seq) items
    int n, s0, s1, rem = item;
    if (!a.cu_seqlens) {
        const int nb = (a.T + C::BM - 1) / C::BM, ph = nb * a.H;
        n = rem / ph;
        rem -= n * ph;
        s0 = n * a.T;
        s1 = s0 + a.T;
    } else {
        const int32_t *bs = a.blk_start;  // [N+1] prefix of H * nblk(seq)
        int lo = 0, hi = a.N;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (bs[mid] <= rem) lo = mid;
            else hi = mid;
        }
        n = lo;
        rem -= bs[lo];
        s0 = min(max(a.cu_seqlens[lo], 0), a.T);
        s1 = min(max(a.cu_seqlens[lo + 1], s0), a.T);
        if (s1 == s0) return;  // only reachable with inconsistent offsets
    }
    const int nb = (s1 - s0 + C::BM - 1) / C::BM;
    const int h = rem / nb, qb = rem % nb;
    const int q0 = s0 + qb * C::BM;               // first query (flat token index)
    const int qlast = min(q0 + C::BM, s1) - 1;
    const int W = a.window;
    const int kstart = max(s0, q0 - W + 1), kend = qlast;
    const int ntiles = (kend - kstart) / C::BN + 1;

    // buffer b: K tile at smem + b * (SZ_K + SZ_V), V^T tile right after it
    constexpr int BUF = C::SZ_K + C::SZ_V;

    // Q fragments (B operand of S^T = K Q^T): lane holds query col of tile rt,
    // dims 32c + 8 grp .. + 8
    const bf16 *Q = reinterpret_cast<const bf16 *>(a.q);
    const size_t ld = (size_t)a.H * D;
    const int wq0 = q0 + 32 * wave;  // this wave's first query
    MB::frag qf[2][C::NC];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int t = min(wq0 + 16 * rt + col, s1 - 1);
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
            qf[rt][c] = *reinterpret_cast<const bf16x8 *>(Q + (size_t)t * ld + h * D + 32 * c + 8 * grp);
    }

    f32x4 acc[2][C::NDT];  // O^T: [dim 16 dt + 4 grp + r][query col]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) acc[rt][dt] = zero4();
    float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.0f, 0.0f};
    const float cs = a.scale * kLog2eF;  // scores in base-2 units

    SwaStage<D> st;
    swa_load<D>(a, h, s0, s1, kstart, tid, st);
    swa_store<D>(smem, smem + C::SZ_K, tid, st);
    __syncthreads();

    const int wq_hi = min(wq0 + 31, s1 - 1);
    for (int j = 0; j < ntiles; ++j) {
        const int k0 = kstart + j * C::BN;
        if (j + 1 < ntiles) swa_load<D>(a, h, s0, s1, k0 + C::BN, tid, st);
        const bf16 *cK = smem + (j & 1) * BUF, *cV = cK + C::SZ_K;

        // ---- S^T = K Q^T: s[rt][kt] = [key 16 kt + 4 grp + r][query col] ----
        // The K fragments of key tile kt+1 are read while the MFMAs of tile kt
        // run (the scheduling fences keep that order).
        f32x4 s[2][C::NKT];
        MB::frag kf[2][C::NC];
#pragma unroll
        for (int c = 0; c < C::NC; ++c) kf[0][c] = load_frag<bf16>(cK + 32 * c, C::LDK, lane);
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) {
            if (kt + 1 < C::NKT) {
#pragma unroll
                for (int c = 0; c < C::NC; ++c)
                    kf[(kt + 1) & 1][c] = load_frag<bf16>(cK + 16 * (kt + 1) * C::LDK + 32 * c, C::LDK, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
            for (int c = 0; c < C::NC; ++c) {
                d0 = MB::mma(kf[kt & 1][c], qf[0][c], d0);
                d1 = MB::mma(kf[kt & 1][c], qf[1][c], d1);
            }
            __builtin_amdgcn_sched_barrier(0);
            s[0][kt] = d0;  // raw q.k; the scale enters the exponent below
            s[1][kt] = d1;
        }
        // V^T fragments of the first two dim tiles, in flight through the softmax
        // (keys in the order the S^T accumulator holds them: 4 grp .. +3 of each
        // 16-key half of a 32-key contraction)
        MB::frag vf[3][C::BN / 32];
        auto load_v = [&](int dt, MB::frag (&dst)[C::BN / 32]) {
#pragma unroll
            for (int jj = 0; jj < C::BN / 32; ++jj) {
                const bf16 *vr = cV + (16 * dt + col) * C::LDV + 32 * jj + 4 * grp;
                const bf16x4 lo4 = *reinterpret_cast<const bf16x4 *>(vr);
                const bf16x4 hi4 = *reinterpret_cast<const bf16x4 *>(vr + 16);
                dst[jj] = MB::frag{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            }
        };
        load_v(0, vf[0]);
        load_v(1, vf[1]);
        // mask the tile unless every key is inside every query's window
        const bool full = (k0 + C::BN - 1 <= wq0) && (k0 > wq_hi - W);
        if (!full) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int qq = wq0 + 16 * rt + col;
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = k0 + 16 * kt + 4 * grp + r;
                        if (kk > qq || kk <= qq - W || kk > kend) s[rt][kt][r] = -INFINITY;
                    }
            }
        }
        // ---- online softmax; P packed as the B operand of O^T += V^T P^T ----
        // The running max m (base-2 units) is raised only when a row's tile max
        // exceeds it by more than kLazy; otherwise p = 2^(cs s - m) <= 2^kLazy,
        // which fp32 sums and bf16 probabilities carry without loss, and the
        // O rescaling is skipped for the whole wave.
        MB::frag pf[2][C::BN / 32];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // this lane's max over its 16 keys; the row max across the four
            // lane groups is only needed when some lane would exceed the headroom
            float mx = s[rt][0][0];
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[rt][kt][r]);
            if (__any(mx * cs > m_run[rt] + kLazy)) {
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[rt], mx * cs);
                const float alpha = exp2_hw(m_run[rt] - m_new);
                m_run[rt] = m_new;
                l_run[rt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) acc[rt][dt] *= alpha;
            }
            const float nm = -m_run[rt];
            float ls = 0.0f;
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = exp2_hw(fmaf(s[rt][kt][r], cs, nm));
                    s[rt][kt][r] = p;
                    ls += p;
                }
            l_run[rt] += ls;
#pragma unroll
            for (int jj = 0; jj < C::BN / 32; ++jj) {
                bf16x8 p8;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p8[r] = static_cast<bf16>(s[rt][2 * jj][r]);
                    p8[4 + r] = static_cast<bf16>(s[rt][2 * jj + 1][r]);
                }
                pf[rt][jj] = p8;
            }
        }
        // ---- O^T += V^T P^T, the V^T fragments two dim tiles ahead ----
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            if (dt + 2 < C::NDT) load_v(dt + 2, vf[(dt + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < C::BN / 32; ++jj) {
                acc[0][dt] = MB::mma(vf[dt % 3][jj], pf[0][jj], acc[0][dt]);
                acc[1][dt] = MB::mma(vf[dt % 3][jj], pf[1][jj], acc[1][dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (j + 1 < ntiles) {
            bf16 *nK = smem + ((j + 1) & 1) * BUF;
            swa_store<D>(nK, nK + C::SZ_K, tid, st);
        }
        __syncthreads();
    }

    // ---- normalise and store: lane holds dims 16 dt + 4 grp .. +3 of query col ----
    bf16 *O = reinterpret_cast<bf16 *>(a.o);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float l = l_run[rt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int qq = wq0 + 16 * rt + col;
        if (qq < s1) {
            const float inv = __builtin_amdgcn_rcpf(l);
            bf16 *orow = O + (size_t)qq * ld + h * D + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = static_cast<bf16>(acc[rt][dt][r] * inv);
                *reinterpret_cast<bf16x4 *>(orow + 16 * dt) = w;
            }
            if (a.lse && grp == 0) {
                const int b = a.cu_seqlens ? 0 : n, t = a.cu_seqlens ? qq : qq - s0;
                a.lse[((size_t)b * a.H + h) * a.T + t] = (m_run[rt] + __log2f(l)) * kLn2F;
            }
        }
    }
}

// Packed calls: prefix over sequences of H * (number of 128-query blocks).
// Offsets are clamped into [0, T] as the attention kernel clamps them.
__global__ void swa_plan_kernel(const int32_t *cu, int N, int T, int H, int BM, int32_t *blk_start) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0;
    blk_start[0] = 0;
    for (int n = 0; n < N; ++n) {
        const int a0 = min(max(cu[n], 0), T), a1 = min(max(cu[n + 1], a0), T);
        const int len = a1 - a0;
        acc += H * ((len + BM - 1) / BM);
        blk_start[n + 1] = acc;
    }
}

}  // namespace

hipError_t launch_swa_fwd(const SwaArgs &a, int D, hipStream_t stream) {
    if (a.n_items <= 0) return hipSuccess;
    const int per = (a.n_items + 7) / 8;
    const dim3 grid(8u * (unsigned)per), block(kThreads);
    if (D == 128) hipLaunchKernelGGL(swa_fwd_kernel<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(swa_fwd_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_swa_plan(const int32_t *cu, int N, int T, int H, int32_t *blk_start,
                           hipStream_t stream) {
    hipLaunchKernelGGL(swa_plan_kernel, dim3(1), dim3(64), 0, stream, cu, N, T, H, SwaCfg<128>::BM,
                       blk_start);
    return hipGetLastError();
}

}  // namespace gdn2
