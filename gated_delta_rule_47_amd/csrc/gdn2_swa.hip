// Sliding-window softmax attention, forward (the hybrid model's local
// attention: iplexlaw digest, section "Condiciones de comparación", 2K
// window; gist.science summary, part "4. Architecture", SWA interleaved with
// the Gated DeltaNet-2 mixer).  Query i of a sequence attends to keys
// i - window < j <= i of the same sequence:
//   o_i = sum_j softmax_j(scale q_i . k_j) v_j,   lse_i = log sum_j e^{scale q_i . k_j}.
//
// One workgroup (4 waves) takes 128 consecutive queries of one (sequence,
// head); wave w owns queries 32w .. 32w+31 as two 16-query tiles.  The keys
// of the window are walked in tiles of 64, double-buffered in LDS (both
// row-major, filled by direct global->LDS loads), with an online softmax in
// base 2.  Everything is
// computed transposed so that each lane owns one query column:
//   S^T = K Q^T      (16x16x32 bf16 MFMA; A = K rows from LDS, B = Q in registers)
//   O^T += V^T P^T   (A = V^T fragments by LDS transposing reads, B = P straight from the S^T
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
    // K and V tiles are row-major [BN][D] bf16 without padding (the direct
    // global->LDS loads fill 1 KB contiguously per wave instruction); bank
    // conflicts are avoided by XOR-swizzling the 16-byte chunks of each row.
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int SZ = BN * D;                  // elements per tile
    static constexpr int LOADS = BN * CPR / 64 / 4;    // wave instructions per tile, per wave
    static_assert(BN * CPR % 256 == 0, "tile splits evenly over 4 waves");
};

// Physical chunk of logical chunk c in row r.  K rows are read as 16-byte
// fragments of 16 consecutive rows (c ^ (r mod CPR) keeps each phase of 8 or
// 16 lanes on distinct banks); V rows are read by the transposing 8-byte loads,
// 4 rows x 2 chunks per 16 lanes (c ^ 2(r mod 8) spreads them).
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (SwaCfg<D>::CPR - 1)); }
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((2 * r) & (SwaCfg<D>::CPR - 2)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// The direct global->LDS loads of key tile [k0, k0+BN).  Wave w fills
// chunks [(w*LOADS + i)*64, +64) of each tile, lane t chunk +t.  A lane's
// element offsets from the tile's first key row do not change from tile to
// tile, so they are formed once; a tile that runs past the sequence's end
// (its last one) takes the rows clamped to the sequence instead (rows past
// it are masked by the caller).
template <int D>
struct SwaFeed {
    unsigned offK[SwaCfg<D>::LOADS], offV[SwaCfg<D>::LOADS];
};

template <int D>
__device__ __forceinline__ SwaFeed<D> swa_feed(const SwaArgs &a, int h, int wave, int lane) {
    using C = SwaCfg<D>;
    SwaFeed<D> f;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int p = (wave * C::LOADS + i) * 64 + lane, row = p / C::CPR, pc = p % C::CPR;
        const unsigned r0 = (unsigned)row * (unsigned)a.ldkv + (unsigned)(h * D);
        f.offK[i] = r0 + 8 * k_chunk<D>(row, pc);
        f.offV[i] = r0 + 8 * v_chunk<D>(row, pc);
    }
    return f;
}

template <int D>
__device__ __forceinline__ void swa_issue(const SwaArgs &a, const SwaFeed<D> &f, int h, int s0, int s1,
                                          int k0, bf16 *tK, bf16 *tV, int wave, int lane) {
    using C = SwaCfg<D>;
    const bf16 *K = reinterpret_cast<const bf16 *>(a.k);
    const bf16 *V = reinterpret_cast<const bf16 *>(a.v);
    const size_t ld = (size_t)a.ldkv;
    if (k0 + C::BN <= s1) {  // every row inside the sequence
        const bf16 *Kb = K + (size_t)k0 * ld, *Vb = V + (size_t)k0 * ld;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int base = (wave * C::LOADS + i) * 64;
            __builtin_amdgcn_global_load_lds(Kb + f.offK[i], (lds_void *)(tK + 8 * base), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(Vb + f.offV[i], (lds_void *)(tV + 8 * base), 16, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int base = (wave * C::LOADS + i) * 64, p = base + lane;
        const int row = p / C::CPR, pc = p % C::CPR;
        const int t = min(max(k0 + row, s0), s1 - 1);
        const size_t g = (size_t)t * ld + h * D;
        __builtin_amdgcn_global_load_lds(K + g + 8 * k_chunk<D>(row, pc),
                                         (lds_void *)(tK + 8 * base), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(V + g + 8 * v_chunk<D>(row, pc),
                                         (lds_void *)(tV + 8 * base), 16, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void swa_fwd_kernel(SwaArgs a) {
    using C = SwaCfg<D>;
    using MB = Mma<bf16>;
    // two stages, each a K tile followed by a V tile, as distinct arrays so
    // that the compiler can tell the stage being read from the one the direct
    // loads write
    __shared__ __attribute__((aligned(16))) bf16 smemA[2 * C::SZ];
    __shared__ __attribute__((aligned(16))) bf16 smemB[2 * C::SZ];
    // (the wave index as a uniform value: the LDS addresses of the direct
    // loads are then formed in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Q fragments (B operand of S^T = K Q^T): lane holds query col of tile rt,
    // dims 32c + 8 grp .. + 8
    const bf16 *Q = reinterpret_cast<const bf16 *>(a.q);
    const size_t ldq = (size_t)a.ldq, ld = (size_t)a.H * D;  // ld: o
    const int wq0 = q0 + 32 * wave;  // this wave's first query
    MB::frag qf[2][C::NC];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int t = min(wq0 + 16 * rt + col, s1 - 1);
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
            qf[rt][c] = *reinterpret_cast<const bf16x8 *>(Q + (size_t)t * ldq + h * D + 32 * c + 8 * grp);
    }

    f32x4 acc[2][C::NDT];  // O^T: [dim 16 dt + 4 grp + r][query col]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) acc[rt][dt] = zero4();
    float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.0f, 0.0f};
    const float cs = a.scale * kLog2eF;  // scores in base-2 units

    const SwaFeed<D> feed = swa_feed<D>(a, h, wave, lane);
    swa_issue<D>(a, feed, h, s0, s1, kstart, smemA, smemA + C::SZ, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int wq_hi = min(wq0 + 31, s1 - 1);
    // one key tile: read stage cK, fill stage nK with the next tile
    auto tile = [&](int j, const bf16 *cK, bf16 *nK) {
        const int k0 = kstart + j * C::BN;
        const bf16 *cV = cK + C::SZ;

        // ---- S^T = K Q^T: s[rt][kt] = [key 16 kt + 4 grp + r][query col] ----
        // Contraction chunk c outermost: the 8 accumulators advance together,
        // so consecutive MFMAs are independent.  The K fragments of chunk c+1
        // are read while the MFMAs of chunk c run (the fences keep the order).
        f32x4 s[2][C::NKT];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) s[0][kt] = s[1][kt] = zero4();
        // K fragment (rows 16 kt .. +15, dims 32 cc .. +31): lane reads row
        // 16 kt + col, logical chunk 4 cc + grp
        auto load_k = [&](int kt, int cc) {
            const int row = 16 * kt + col;
            return *reinterpret_cast<const MB::frag *>(cK + row * D + 8 * k_chunk<D>(row, 4 * cc + grp));
        };
        MB::frag kf[2][C::NKT];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) kf[0][kt] = load_k(kt, 0);
#pragma unroll
        for (int c = 0; c < C::NC; ++c) {
            if (c + 1 < C::NC) {
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
                    kf[(c + 1) & 1][kt] = load_k(kt, c + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt) {
                s[0][kt] = MB::mma(kf[c & 1][kt], qf[0][c], s[0][kt]);
                s[1][kt] = MB::mma(kf[c & 1][kt], qf[1][c], s[1][kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // (s holds raw q.k; the scale enters the exponent below)
        // V^T fragments (keys in the order the S^T accumulator holds them: 4 grp
        // .. +3 of each 16-key half of a 32-key contraction); the first group
        // is read before the softmax so it is in flight meanwhile
        // V^T fragment (dims 16 dt .. +15, keys of contraction jj): two
        // transposing 8-byte reads of the row-major V tile.  In each group of 16
        // lanes, lane j points at row (key) 32 jj + 4 grp + j/4 (+16), dims
        // 16 dt + 4 (j%4) .. +3; lane i then receives dim 16 dt + i of those 4 rows.
        auto load_v = [&](int dt, int jj) {
            const int row = 32 * jj + 4 * grp + ((lane & 15) >> 2);
            const int c = 2 * dt + ((lane & 3) >> 1), half = lane & 1;
            const bf16 *p0 = cV + row * D + 8 * v_chunk<D>(row, c) + 4 * half;
            const bf16 *p1 = cV + (row + 16) * D + 8 * v_chunk<D>(row + 16, c) + 4 * half;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)(p0));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)(p1));
            typedef short v8i16 __attribute__((ext_vector_type(8)));
            const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(MB::frag, both);
        };
        constexpr int VGRP = 4;  // dim tiles per read group
        MB::frag vf[2][VGRP];
#pragma unroll
        for (int u = 0; u < VGRP; ++u) vf[0][u] = load_v(u, 0);
        // The next tile's direct loads go out now, into the other stage's
        // array: they land during the softmax and the V^T P^T products.  The
        // two stages are distinct arrays and the tile loop is unrolled by two,
        // so every LDS read names its stage and the compiler's wait
        // insertion can tell it apart from the direct loads in flight (with
        // one array and a runtime stage offset, every read after the issue
        // waited for all of them).  Issuing before the S^T products, or
        // before the first V^T reads, measured slower.
        if (j + 1 < ntiles) swa_issue<D>(a, feed, h, s0, s1, k0 + C::BN, nK, nK + C::SZ, wave, lane);
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
        // ---- O^T += V^T P^T: 32-key half jj outermost, 16 independent
        // accumulators; V^T fragments read one group of 4 dim tiles ahead ----
        constexpr int NG = (C::BN / 32) * (C::NDT / VGRP);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int jj = gi / (C::NDT / VGRP), d0 = (gi % (C::NDT / VGRP)) * VGRP;
            if (gi + 1 < NG) {
                const int jn = (gi + 1) / (C::NDT / VGRP), dn = ((gi + 1) % (C::NDT / VGRP)) * VGRP;
#pragma unroll
                for (int u = 0; u < VGRP; ++u) vf[(gi + 1) & 1][u] = load_v(dn + u, jn);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < VGRP; ++u) {
                acc[0][d0 + u] = MB::mma(vf[gi & 1][u], pf[0][jj], acc[0][d0 + u]);
                acc[1][d0 + u] = MB::mma(vf[gi & 1][u], pf[1][jj], acc[1][d0 + u]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the next tile has landed
        __syncthreads();
    };
    for (int j = 0; j < ntiles; j += 2) {
        tile(j, smemA, smemB);
        if (j + 1 < ntiles) tile(j + 1, smemB, smemA);
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
