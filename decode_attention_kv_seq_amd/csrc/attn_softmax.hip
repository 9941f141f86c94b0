// attn_softmax.hip -- softmax over the last dimension of an fp32 tensor, for
// gfx950 (MI355X): one read and one write per element when a row fits in a
// workgroup's registers, a two-launch chunked path otherwise.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn_internal.h"

namespace {

using namespace attn;

// ------------------------------------------------------------ row softmax
// Softmax over the last dimension of an fp32 [rows, cols] tensor: the
// Foundry notes' fm_softmax (section "API Reference"), max-shifted as the
// page "Developing Apple Metal Kernels in Rust - A Deep Dive Through
// Attention" does it in attention_pv_f16 (section "The MSL, briefly"):
// m = max x, e = exp(x - m) (as 2^((x - m) log2 e)), out = e / sum e.  A row
// of -inf only gives NaN, as the definition does.
//
// Row kernel: one workgroup of NT threads per row, the whole row in
// registers (VPT values per thread), so x is read once and out written once.
// Split path, for rows longer than a workgroup holds or too few rows to fill
// the chip: a stats launch leaves (max, sum of 2^(x - max)) per chunk of CH =
// NT*VPT columns; an apply launch merges a row's chunk stats and rewrites its
// chunk (x read twice: the first launch reads it with ordinary loads, so the
// second read mostly hits the caches; plain loads there measured 14% faster
// than non-temporal ones on a [64, 131072] input).

constexpr float kLog2e = 1.4426950408889634f;

// NTL: non-temporal loads (the last read of x); plain loads leave x in the
// caches for a second read.
template <int NT, int VPT, bool V4, bool NTL = true>
__device__ __forceinline__ void sm_load(const float *xr, uint32_t c0, uint32_t c_end, float (&v)[VPT]) {
    const uint32_t tid = threadIdx.x;
    if constexpr (V4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) {
            const uint32_t c = c0 + (tid + (uint32_t)k * NT) * 4u;
            f4 f = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (c < c_end)
                f = NTL ? __builtin_nontemporal_load(reinterpret_cast<const f4 *>(xr + c))
                        : *reinterpret_cast<const f4 *>(xr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * k + e] = f[e];
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const uint32_t c = c0 + tid + (uint32_t)k * NT;
            v[k] = c < c_end ? (NTL ? __builtin_nontemporal_load(xr + c) : xr[c]) : -INFINITY;
        }
    }
}

template <int NT, int VPT, bool V4>
__device__ __forceinline__ void sm_store(float *orow, uint32_t c0, uint32_t c_end, const float (&v)[VPT]) {
    const uint32_t tid = threadIdx.x;
    if constexpr (V4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) {
            const uint32_t c = c0 + (tid + (uint32_t)k * NT) * 4u;
            if (c < c_end) {
                f4 f = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
                __builtin_nontemporal_store(f, reinterpret_cast<f4 *>(orow + c));
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const uint32_t c = c0 + tid + (uint32_t)k * NT;
            if (c < c_end) __builtin_nontemporal_store(v[k], orow + c);
        }
    }
}

// v <- 2^((v - m) log2 e); returns this thread's sum.  Padding (-inf) gives 0.
template <int VPT>
__device__ __forceinline__ float sm_exp(float (&v)[VPT], float m) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        v[k] = __builtin_amdgcn_exp2f((v[k] - m) * kLog2e);
        s += v[k];
    }
    return s;
}

template <int NT, int VPT, bool V4>
__global__ __launch_bounds__(NT) void attn_softmax_row_kernel(const float *x, float *out, uint32_t cols) {
    __shared__ float sm_max[NT / 64];
    __shared__ float sm_sum[NT / 64];
    const size_t row = blockIdx.x;
    float v[VPT];
    sm_load<NT, VPT, V4>(x + row * cols, 0, cols, v);
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < VPT; ++k) m = fmaxf(m, v[k]);
    m = block_max<NT>(m, sm_max);
    const float s = block_sum<NT>(sm_exp<VPT>(v, m), sm_sum);
    const float inv = 1.f / s;
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] *= inv;
    sm_store<NT, VPT, V4>(out + row * cols, 0, cols, v);
}

// Split path, first launch: workgroup w takes chunk w % n_chunks of row
// w / n_chunks and writes its (max, sum of 2^(x - max) in base-2 units).  An
// all -inf chunk leaves (-inf, 0).
template <int NT, int VPT, bool V4>
__global__ __launch_bounds__(NT) void attn_softmax_stats_kernel(const float *x, float *stats,
                                                                uint32_t cols, uint32_t n_chunks) {
    __shared__ float sm_max[NT / 64];
    __shared__ float sm_sum[NT / 64];
    constexpr uint32_t CH = NT * VPT;
    const size_t row = blockIdx.x / n_chunks;
    const uint32_t chunk = blockIdx.x % n_chunks;
    const uint32_t c0 = chunk * CH;
    const uint32_t c_end = cols - c0 < CH ? cols : c0 + CH;
    float v[VPT];
    sm_load<NT, VPT, V4, false>(x + row * cols, c0, c_end, v);   // x is read again
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < VPT; ++k) m = fmaxf(m, v[k]);
    m = block_max<NT>(m, sm_max);
    const float s = block_sum<NT>(sm_exp<VPT>(v, m == -INFINITY ? 0.f : m), sm_sum);
    if (threadIdx.x == 0) {
        stats[((size_t)row * n_chunks + chunk) * 2] = m;
        stats[((size_t)row * n_chunks + chunk) * 2 + 1] = s;
    }
}

// Split path, second launch: every workgroup of a row merges the row's chunk
// stats the same way (M = max m_c, L = sum s_c 2^((m_c - M) log2 e), a fixed
// order), then rewrites its chunk as 2^((x - M) log2 e) / L.
template <int NT, int VPT, bool V4>
__global__ __launch_bounds__(NT) void attn_softmax_apply_kernel(const float *x, float *out,
                                                                const float *stats, uint32_t cols,
                                                                uint32_t n_chunks, uint32_t reverse) {
    __shared__ float sm_max[NT / 64];
    __shared__ float sm_sum[NT / 64];
    constexpr uint32_t CH = NT * VPT;
    const uint32_t w = reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const size_t row = w / n_chunks;
    const uint32_t chunk = w % n_chunks;
    const uint32_t c0 = chunk * CH;
    const uint32_t c_end = cols - c0 < CH ? cols : c0 + CH;
    float v[VPT];
    sm_load<NT, VPT, V4>(x + row * cols, c0, c_end, v);
    const float *st = stats + (size_t)row * n_chunks * 2;
    float mc = -INFINITY;
    for (uint32_t c = threadIdx.x; c < n_chunks; c += NT) mc = fmaxf(mc, st[2 * c]);
    const float M = block_max<NT>(mc, sm_max);
    float l = 0.f;
    // a chunk of -inf only adds 0 * 2^-inf = 0; a row of -inf only gives NaN
    for (uint32_t c = threadIdx.x; c < n_chunks; c += NT)
        l += st[2 * c + 1] * __builtin_amdgcn_exp2f((st[2 * c] - M) * kLog2e);
    const float L = block_sum<NT>(l, sm_sum);
    sm_exp<VPT>(v, M);
    const float inv = 1.f / L;
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] *= inv;
    sm_store<NT, VPT, V4>(out + row * cols, c0, c_end, v);
}

// Row softmax plan.  Rows of up to 1024 columns take one wave each; up to
// 32768 columns, one workgroup holds the row in registers when there are
// enough rows to fill the chip or too little data for a second launch to pay;
// otherwise the split path with 4096-column chunks.
constexpr uint32_t kSmChunk = 256 * 16;            // split-path chunk (NT 256, VPT 16)
constexpr uint32_t kSmRowMax = 1024 * 32;          // longest row held by one workgroup
constexpr uint32_t kSmMinRows = 256;               // rows that fill the chip one per CU
constexpr uint64_t kSmSmallElems = 1u << 21;       // below this, one launch even with few rows

enum class SmPath { wave, row256, row512, row1024, split };

// Tuning sweeps only: ATTN_SOFTMAX_TUNE="ch=N,nt=N,rev=1" picks the split
// path's chunk (4096, 8192 or 16384 columns: never more chunks than the
// workspace holds), its threads, and the apply launch's chunk order.  Read
// once per process.
struct SmTune {
    uint32_t ch = 0, nt = 0, rev = 0;
};
const SmTune &sm_tune() {
    static const SmTune t = [] {
        SmTune r;
        const char *e = getenv("ATTN_SOFTMAX_TUNE");
        if (e) {
            char buf[128];
            snprintf(buf, sizeof buf, "%s", e);
            for (char *tok = strtok(buf, ","); tok; tok = strtok(nullptr, ",")) {
                unsigned v = 0;
                if (sscanf(tok, "ch=%u", &v) == 1 && (v == 4096 || v == 8192 || v == 16384)) r.ch = v;
                else if (sscanf(tok, "nt=%u", &v) == 1) r.nt = v;
                else if (sscanf(tok, "rev=%u", &v) == 1) r.rev = v ? 1u : 0u;
            }
        }
        return r;
    }();
    return t;
}

SmPath softmax_path(uint32_t rows, uint32_t cols) {
    static const int forced = [] {
        const char *e = getenv("ATTN_SOFTMAX_PATH");   // tuning sweeps: "split" or "row"
        return e ? (strcmp(e, "split") == 0 ? 1 : strcmp(e, "row") == 0 ? 2 : 0) : 0;
    }();
    if (cols <= 1024 && forced != 1) return SmPath::wave;
    const bool fits = cols <= kSmRowMax;
    const bool row_ok = fits && (forced == 2 || (forced == 0 && ((uint64_t)rows >= kSmMinRows ||
                                                                 (uint64_t)rows * cols <= kSmSmallElems)));
    if (!row_ok) return SmPath::split;
    return cols <= 256 * 32 ? SmPath::row256 : cols <= 512 * 32 ? SmPath::row512 : SmPath::row1024;
}

size_t softmax_ws_bytes(uint32_t rows, uint32_t cols) {
    const uint64_t n_chunks = cdiv(cols, kSmChunk);
    const uint64_t b = (uint64_t)rows * n_chunks * 2 * sizeof(float);
    return (size_t)((b + 255) / 256 * 256);
}

template <bool V4>
void launch_softmax(SmPath path, const float *x, float *out, uint32_t rows, uint32_t cols,
                    float *stats, hipStream_t st) {
    switch (path) {
    case SmPath::wave:
        hipLaunchKernelGGL((attn_softmax_row_kernel<64, 16, V4>), dim3(rows), dim3(64), 0, st, x, out, cols);
        break;
    case SmPath::row256:
        hipLaunchKernelGGL((attn_softmax_row_kernel<256, 32, V4>), dim3(rows), dim3(256), 0, st, x, out, cols);
        break;
    case SmPath::row512:
        hipLaunchKernelGGL((attn_softmax_row_kernel<512, 32, V4>), dim3(rows), dim3(512), 0, st, x, out, cols);
        break;
    case SmPath::row1024:
        hipLaunchKernelGGL((attn_softmax_row_kernel<1024, 32, V4>), dim3(rows), dim3(1024), 0, st, x, out, cols);
        break;
    case SmPath::split: {
        const SmTune &t = sm_tune();
        const uint32_t ch = t.ch ? t.ch : kSmChunk;
        const uint32_t n_chunks = (uint32_t)cdiv(cols, ch);
        const dim3 grid((unsigned)((uint64_t)rows * n_chunks));
        if (ch == 8192 && t.nt == 512) {
            hipLaunchKernelGGL((attn_softmax_stats_kernel<512, 16, V4>), grid, dim3(512), 0, st, x, stats, cols, n_chunks);
            hipLaunchKernelGGL((attn_softmax_apply_kernel<512, 16, V4>), grid, dim3(512), 0, st, x, out, stats, cols, n_chunks, t.rev);
        } else if (ch == 8192) {
            hipLaunchKernelGGL((attn_softmax_stats_kernel<256, 32, V4>), grid, dim3(256), 0, st, x, stats, cols, n_chunks);
            hipLaunchKernelGGL((attn_softmax_apply_kernel<256, 32, V4>), grid, dim3(256), 0, st, x, out, stats, cols, n_chunks, t.rev);
        } else if (ch == 16384 && t.nt == 1024) {
            hipLaunchKernelGGL((attn_softmax_stats_kernel<1024, 16, V4>), grid, dim3(1024), 0, st, x, stats, cols, n_chunks);
            hipLaunchKernelGGL((attn_softmax_apply_kernel<1024, 16, V4>), grid, dim3(1024), 0, st, x, out, stats, cols, n_chunks, t.rev);
        } else if (ch == 16384) {
            hipLaunchKernelGGL((attn_softmax_stats_kernel<512, 32, V4>), grid, dim3(512), 0, st, x, stats, cols, n_chunks);
            hipLaunchKernelGGL((attn_softmax_apply_kernel<512, 32, V4>), grid, dim3(512), 0, st, x, out, stats, cols, n_chunks, t.rev);
        } else {
            hipLaunchKernelGGL((attn_softmax_stats_kernel<256, 16, V4>), grid, dim3(256), 0, st, x, stats, cols, n_chunks);
            hipLaunchKernelGGL((attn_softmax_apply_kernel<256, 16, V4>), grid, dim3(256), 0, st, x, out, stats, cols, n_chunks, t.rev);
        }
        break;
    }
    }
}

}  // namespace

extern "C" {

size_t attn_softmax_workspace_bytes(uint32_t rows, uint32_t cols) {
    if (rows == 0 || cols == 0 || (uint64_t)rows * cdiv(cols, kSmChunk) > 0x7fffffffull) return 0;
    return softmax_ws_bytes(rows, cols);
}

attn_status_t attn_softmax_f32(const float *x, float *out, uint32_t rows, uint32_t cols,
                               void *workspace, size_t workspace_bytes, void *stream) {
    if (!x || !out) return fail(ATTN_ERR_NULL, "x and out must be non-NULL");
    if (rows == 0 || cols == 0)
        return fail(ATTN_ERR_DIM, "rows=%u and cols=%u must be nonzero", rows, cols);
    if ((uint64_t)rows * cdiv(cols, kSmChunk) > 0x7fffffffull)
        return fail(ATTN_ERR_DIM, "rows=%u x cols=%u is too large", rows, cols);
    if (!aligned(x, 4) || !aligned(out, 4)) return fail(ATTN_ERR_ALIGN, "x and out must be 4-byte aligned");
    const size_t need = softmax_ws_bytes(rows, cols);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    workspace_bytes, need);
    const SmPath path = softmax_path(rows, cols);
    // a dispatch holds its grid size in work-items, 32 bits per dimension
    const uint64_t items = path == SmPath::wave     ? (uint64_t)rows * 64
                         : path == SmPath::row256   ? (uint64_t)rows * 256
                         : path == SmPath::row512   ? (uint64_t)rows * 512
                         : path == SmPath::row1024  ? (uint64_t)rows * 1024
                                                    : (uint64_t)rows * cdiv(cols, kSmChunk) * 256;
    if (items > 0xFFFFFFFFull)
        return fail(ATTN_ERR_DIM, "rows=%u x cols=%u exceeds the dispatch limit", rows, cols);
    const bool v4 = cols % 4 == 0 && aligned(x, 16) && aligned(out, 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *stats = static_cast<float *>(workspace);
    if (v4) launch_softmax<true>(path, x, out, rows, cols, stats, st);
    else launch_softmax<false>(path, x, out, rows, cols, stats, st);
    return hip_check("softmax kernel launch");
}

}  // extern "C"
