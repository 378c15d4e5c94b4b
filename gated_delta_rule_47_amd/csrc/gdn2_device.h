// Device-side building blocks shared by the libgdn2 kernels (gfx950 only).
//
// MFMA conventions used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, wave64):
//   D[m][n] += sum_k A[m][k] * B[n][k]          ("NT" form)
// Operands are read from row-major tiles with k contiguous:
//   lane l supplies A[m0 + l%16][k0 + KPL*(l/16) .. + KPL-1] and the same for B,
// where KPL = 8 (bf16) or 1 (f32).  The 16x16 fp32 result is held as
//   lane l: D[4*(l/16) + r][l%16], r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

constexpr int kChunk = 64;        // tokens per chunk
constexpr int kThreads = 256;     // threads per workgroup of the chunk kernels (4 waves)

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 2^x on the hardware exp2 (results outside the fp32 range saturate to 0 or
// inf, which every caller absorbs).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log(1 + u) for u in [0, 1] from the hardware logarithm, with Goldberg's
// correction log(w) * u / (w - 1), w = fl(1 + u) (D. Goldberg, "What every
// computer scientist should know about floating-point arithmetic", 1991,
// theorem 4), which keeps the relative accuracy for small u.
__device__ __forceinline__ float log1p_unit(float u) {
    const float w = 1.0f + u;
    return w == 1.0f ? u : __logf(w) * u * __builtin_amdgcn_rcpf(w - 1.0f);
}

// log(1 / (1 + e^-z)) = min(z, 0) - log1p(e^-|z|), finite for every finite z.
__device__ __forceinline__ float logsigmoid_fast(float z) {
    return fminf(z, 0.0f) - log1p_unit(exp2_hw(-1.4426950408889634f * fabsf(z)));
}

// Value of lane l ^ kXor (kXor = 1 or 2) inside each group of four lanes
// (DPP quad permutation [1,0,3,2] or [2,3,0,1]).
template <int kXor>
__device__ __forceinline__ float quad_xor(float x) {
    static_assert(kXor == 1 || kXor == 2, "quad partner");
    constexpr int ctrl = kXor == 1 ? 0xB1 : 0x4E;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
}

// 4x4 transpose inside each group of four lanes: lane 4m + j enters with
// x[r] = X[r][j] of its group's block and leaves with x[c] = X[j][c].  On an
// MFMA accumulator tile (lane l: D[4(l/16) + r][l%16]) this leaves lane l
// with row 4(l/16) + l%4, columns 4((l/4)%4) .. +3.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int lane) {
    const bool odd = lane & 1, hi = lane & 2;
    // the off-diagonal elements of each 2x2 block, with lane j ^ 1
    float r0 = quad_xor<1>(odd ? x[0] : x[1]), r1 = quad_xor<1>(odd ? x[2] : x[3]);
    const f32x4 y = odd ? f32x4{r0, x[1], r1, x[3]} : f32x4{x[0], r0, x[2], r1};
    // the off-diagonal 2x2 blocks, with lane j ^ 2
    r0 = quad_xor<2>(hi ? y[0] : y[2]);
    r1 = quad_xor<2>(hi ? y[1] : y[3]);
    return hi ? f32x4{r0, r1, y[2], y[3]} : f32x4{y[0], y[1], r0, r1};
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---------------------------------------------------------------------------
// MFMA traits: one 16x16 output tile per instruction, K = KS per instruction.
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<bf16> {
    using elem = bf16;
    typedef bf16x8 frag;
    static constexpr int KS = 32;
    static constexpr int KPL = 8;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag zero() {
        frag z;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = static_cast<bf16>(0.0f);
        return z;
    }
};

template <> struct Mma<float> {
    using elem = float;
    typedef float frag;
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag zero() { return 0.0f; }
};

// Operand fragment of a row-major tile (rows r0.., k0..) with leading dim ld.
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag load_frag(const E *tile, int ld, int lane) {
    using M = Mma<E>;
    return *reinterpret_cast<const typename M::frag *>(tile + (lane & 15) * ld + M::KPL * (lane >> 4));
}

// acc += A[16 x K] * B[16 x K]^T, both row-major with k contiguous.
template <typename E, int K>
__device__ __forceinline__ f32x4 mma_tile(f32x4 acc, const E *A, int lda, const E *B, int ldb,
                                          int lane) {
    using M = Mma<E>;
#pragma unroll
    for (int kk = 0; kk < K; kk += M::KS)
        acc = M::mma(load_frag<E>(A + kk, lda, lane), load_frag<E>(B + kk, ldb, lane), acc);
    return acc;
}

// Same with a runtime K (a multiple of KS).
template <typename E>
__device__ __forceinline__ f32x4 mma_tile_k(f32x4 acc, const E *A, int lda, const E *B, int ldb,
                                            int K, int lane) {
    using M = Mma<E>;
    for (int kk = 0; kk < K; kk += M::KS)
        acc = M::mma(load_frag<E>(A + kk, lda, lane), load_frag<E>(B + kk, ldb, lane), acc);
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// Operand-fragment order of a matrix X with K columns (used for the chunk
// factors kept in the workspace): 16-row blocks by KS-column blocks, each
// block stored as 64 lanes x KPL elements exactly as load_frag would gather
// it, so that one wave reads a fragment as one contiguous 64*KPL-element run.
template <typename E>
__device__ __forceinline__ size_t frag_index(int r, int k, int K) {
    using M = Mma<E>;
    return ((size_t)(r >> 4) * (K / M::KS) + k / M::KS) * (64 * M::KPL) +
           ((r & 15) + 16 * ((k % M::KS) / M::KPL)) * M::KPL + (k % M::KPL);
}

// The causal query-key matrix M of a chunk (64 x 64, zero above the diagonal)
// is kept in fragment order without its fragments that lie wholly above the
// diagonal: is the fragment of row block I (16 rows) holding column col used?
template <typename E>
__host__ __device__ constexpr bool m_frag_used(int I, int col) {
    return (col / Mma<E>::KS) * Mma<E>::KS <= 16 * I + 15;
}

// Fragment (row block rb, column block kb) of a matrix stored in fragment order.
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag load_frag_packed(const E *X, int K, int rb, int kb,
                                                                   int lane) {
    using M = Mma<E>;
    return *reinterpret_cast<const typename M::frag *>(
        X + ((size_t)rb * (K / M::KS) + kb) * (64 * M::KPL) + lane * M::KPL);
}

// X[r][k..k+3] = v (k a multiple of 4) into fragment order.
template <typename E>
__device__ __forceinline__ void store4_frag(E *X, int K, int r, int k, f32x4 v) {
    if constexpr (sizeof(E) == 2) {  // the 4 values are adjacent within a lane's 8
        bf16x4 b;
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = static_cast<bf16>(v[j]);
        *reinterpret_cast<bf16x4 *>(X + frag_index<E>(r, k, K)) = b;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) X[frag_index<E>(r, k + j, K)] = v[j];
    }
}

// Store the 4 results a lane holds as 4 consecutive elements of row (l%16)
// of a row-major destination: dst[(l%16)*ld + 4*(l/16) + r] = acc[r].
// (This writes the TRANSPOSE of the D tile: Dt[n][m].)
template <typename E>
__device__ __forceinline__ void store_tile_t(E *dst, int ld, f32x4 acc, int lane) {
    E *p = dst + (lane & 15) * ld + 4 * (lane >> 4);
    if constexpr (sizeof(E) == 2) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<bf16>(acc[r]);
        *reinterpret_cast<bf16x4 *>(p) = v;
    } else {
        *reinterpret_cast<f32x4 *>(p) = acc;
    }
}

// Store the D tile in its natural orientation: dst[(4*(l/16)+r)*ld + l%16] = acc[r].
template <typename E>
__device__ __forceinline__ void store_tile(E *dst, int ld, f32x4 acc, int lane) {
    E *p = dst + (4 * (lane >> 4)) * ld + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r * ld] = from_f32<E>(acc[r]);
}

// The state tiles a wave owns, in accumulator order, from an fp32 [chains, DK,
// DV] array (or zeros when src is NULL): tile u covers rows 16 (w KB_W + u/NCB)
// .. +15 and columns col0 + 16 (u%NCB) .. +15 of chain `chain`.  The NULL test
// is one branch around every load: a per-element select makes the compiler
// wait for each load before issuing the next.
template <int DK, int DV, int KB_W, int NCB>
__device__ __forceinline__ void load_state_tiles(f32x4 (&acc)[KB_W * NCB], const float *src, int chain,
                                                 int w, int col0, int lane) {
    if (src) {
#pragma unroll
        for (int u = 0; u < KB_W * NCB; ++u) {
            const int cblk = w * KB_W + u / NCB, col = col0 + 16 * (u % NCB) + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[u][r] = src[((size_t)chain * DK + 16 * cblk + 4 * (lane >> 4) + r) * DV + col];
        }
    } else {
#pragma unroll
        for (int u = 0; u < KB_W * NCB; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

}  // namespace gdn2
