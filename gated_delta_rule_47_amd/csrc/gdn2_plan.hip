// Chunk table of a packed variable-length call, built on the device so that
// the host never reads cu_seqlens.
//
// Each sequence is cut into 64-token chunks from its own first token; its
// last chunk may be shorter.  Output (int32, inside the workspace):
//   plan[n], n = 0..N-1 : id of the first chunk of sequence n
//   plan[N]             : number of chunks in the call
//   plan[N+1 + 3c ...]  : (sequence, first token, length) of chunk c
// Offsets are clamped into [0, T] and the table is capped at its capacity,
// so malformed offsets cannot cause out-of-bounds accesses.

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t *__restrict__ cu, int N,
                                                             int T, int cap,
                                                             int32_t *__restrict__ plan) {
    __shared__ int wave_tot[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < N; base += kPlanThreads) {
        const int n = base + tid;
        int s = 0, len = 0;
        if (n < N) {
            s = min(max(cu[n], 0), T);
            const int e = min(max(cu[n + 1], s), T);
            len = e - s;
        }
        const int nch = (len + kChunk - 1) / kChunk;
        // Block-wide inclusive scan of nch.
        int x = nch;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        int before = 0, total = 0;
        for (int i = 0; i < kPlanThreads / 64; ++i) {
            const int t = wave_tot[i];
            before += (i < wave) ? t : 0;
            total += t;
        }
        const int first = carry + before + x - nch;
        if (n < N) {
            plan[n] = min(first, cap);
            for (int j = 0; j < nch; ++j) {
                const int c = first + j;
                if (c >= cap) break;
                int32_t *e = plan + N + 1 + 3 * (size_t)c;
                e[0] = n;
                e[1] = s + kChunk * j;
                e[2] = min(kChunk, len - kChunk * j);
            }
        }
        carry += total;
        __syncthreads();  // wave_tot is rewritten by the next round
    }
    if (tid == 0) plan[N] = min(carry, cap);
}

hipError_t launch_plan(const ChunkArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.cu_seqlens, a.N, a.T,
                       a.max_chunks, a.plan);
    return hipGetLastError();
}

}  // namespace gdn2
