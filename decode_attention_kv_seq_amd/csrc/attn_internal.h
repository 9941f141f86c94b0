// attn_internal.h -- declarations shared by the library's translation units
// (decode attention and its neighbours in attn_decode.hip, the row softmax in
// attn_softmax.hip).  Not part of the public interface (include/attn_decode.h).
#ifndef ATTN_INTERNAL_H
#define ATTN_INTERNAL_H

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "attn_decode.h"

namespace attn {

// ------------------------------------------------------ workgroup reductions
// Max and sum over a workgroup of NT threads (NT a multiple of 64): xor
// shuffles inside each wave, then the per-wave results through LDS, read in a
// fixed order so every thread gets the same bits.  Every thread must call;
// sm_red holds NT/64 floats and may be reused only after a barrier.

template <int NT>
__device__ __forceinline__ float block_max(float x, float *sm_red) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    if ((threadIdx.x & 63) == 0) sm_red[threadIdx.x >> 6] = x;
    __syncthreads();
    float M = sm_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_red[w]);
    return M;
}

template <int NT>
__device__ __forceinline__ float block_sum(float x, float *sm_red) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) sm_red[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = sm_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += sm_red[w];
    return t;
}

// --------------------------------------------------------------- host side

// Records the detail text for attn_last_error() and returns s.
attn_status_t fail(attn_status_t s, const char *fmt, ...);
inline attn_status_t ok() { return ATTN_OK; }
// ATTN_ERR_HIP with the runtime's text if the last launch was refused.
attn_status_t hip_check(const char *what);

inline uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace attn

#endif  // ATTN_INTERNAL_H
