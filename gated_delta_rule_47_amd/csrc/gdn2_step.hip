// Decode step: one token for every (batch, head), state updated in place.
//
// Per (b, h) the Dk x Dv fp32 state is streamed through registers exactly
// once: one read pass forms both reductions the token needs,
//   r = sum_c alpha_c b_c k_c S[c,:]   (read of the decayed state with e = b*k)
//   p = sum_c alpha_c q_c S[c,:]
// and one write pass stores S[c,:] <- alpha_c S[c,:] + k_c (z - r) with
// z = w*v.  The output o = S_t^T q_t is recovered as p + (q.k)(z - r), since
// S_t^T q = Sbar^T q + (k.q)(z - r).  The order (decay, read, write, query the
// updated state) follows the iplexlaw digest, section "Decisiones
// independientes en dos ejes"; constant memory per decoded token is the
// gist.science summary's problem statement.
//
// Layout: S [B, H, Dk, Dv] row-major (rows = key channels).  One workgroup
// of 256 threads owns one (b, h); thread (cq, rg) owns columns 4cq..4cq+3 of
// rows rg, rg + NRG, rg + 2 NRG, ..., so each wave load instruction reads
// whole 512-byte rows (coalesced 16-byte accesses).

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
    constexpr int NQ = DV / 4;          // column quads
    constexpr int NRG = 256 / NQ;       // row groups
    constexpr int RPT = DK / NRG;       // rows per thread
    constexpr int NW = 4;               // waves
    static_assert(NRG * NQ == 256 && RPT * NRG == DK, "thread map");

    __shared__ f32x4 coef[DK];               // (alpha, alpha*b*k, alpha*q, k) per row
    __shared__ float part_qk[NW];
    __shared__ f32x4 red[NW][NQ][2];         // per-wave partial (r, p) per column quad

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cq = tid % NQ, rg = tid / NQ;
    const size_t bh = blockIdx.x;

    // Issue the state loads first: they are the whole cost of the kernel.
    float *S = a.S + bh * DK * DV;
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = *reinterpret_cast<const f32x4 *>(S + (size_t)(rg + NRG * m) * DV + 4 * cq);

    const IO *vv = reinterpret_cast<const IO *>(a.v) + bh * DV + 4 * cq;
    const float *ww = a.w + bh * DV + 4 * cq;
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = ww[j] * to_f32(vv[j]);

    float qk_part = 0.0f;
    if (tid < DK) {
        const IO *qq = reinterpret_cast<const IO *>(a.q) + bh * DK;
        const IO *kk = reinterpret_cast<const IO *>(a.k) + bh * DK;
        const float kc = to_f32(kk[tid]), qc = to_f32(qq[tid]);
        const float alpha = __expf(a.log_alpha[bh * DK + tid]);
        const float bc = a.b[bh * DK + tid];
        coef[tid] = f32x4{alpha, alpha * bc * kc, alpha * qc, kc};
        qk_part = qc * kc;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qk_part += __shfl_xor(qk_part, off);
    if (lane == 0) part_qk[wave] = qk_part;
    __syncthreads();
    float qk = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) qk += part_qk[i];

    f32x4 r = zero4(), p = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const f32x4 cf = coef[rg + NRG * m];
        r += cf[1] * s[m];
        p += cf[2] * s[m];
    }
    // Reduce over the row groups inside the wave (lanes that share cq).
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] += __shfl_xor(r[j], off);
            p[j] += __shfl_xor(p[j], off);
        }
    }
    if (lane < NQ) {
        red[wave][cq][0] = r;
        red[wave][cq][1] = p;
    }
    __syncthreads();
    r = zero4();
    p = zero4();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        r += red[i][cq][0];
        p += red[i][cq][1];
    }

    f32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = z[j] - r[j];

    if (rg == 0) {
        IO *oo = reinterpret_cast<IO *>(a.o) + bh * DV + 4 * cq;
#pragma unroll
        for (int j = 0; j < 4; ++j) oo[j] = from_f32<IO>(p[j] + qk * u[j]);
    }

    // The new state is stored non-temporally: it is read again only by the
    // next step's launch, and keeping it out of the caches measured 6.5% more
    // bandwidth at B = 256, H = 16 (non-temporal loads measured slower).
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const f32x4 cf = coef[rg + NRG * m];
        const f32x4 snew = cf[0] * s[m] + cf[3] * u;
        __builtin_nontemporal_store(snew, reinterpret_cast<f32x4 *>(S + (size_t)(rg + NRG * m) * DV + 4 * cq));
    }
}

hipError_t launch_step(const StepArgs &a, int Dk, bool bf16_io, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H)), block(256);
    if (bf16_io) {
        if (Dk == 128) hipLaunchKernelGGL((step_kernel<bf16, 128, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((step_kernel<bf16, 64, 64>), grid, block, 0, stream, a);
    } else {
        if (Dk == 128) hipLaunchKernelGGL((step_kernel<float, 128, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((step_kernel<float, 64, 64>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gdn2
