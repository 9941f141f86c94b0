// attn_table.hip -- a check of a paged cache's block table, for gfx950
// (MI355X).  The paged decode reads only the table entries of positions up to
// each sequence's current_pos and, rather than trust an entry past the pool,
// reads the last page instead (in bounds, output meaningless).  This check
// lets a caller find such entries on the device without a host copy of the
// table: it counts the entries the decode would read that name no page of
// the pool, and finds the first sequence holding one.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "attn_internal.h"

namespace {

using namespace attn;

// result[0] = 0 (entries past the pool), result[1] = UINT32_MAX (first
// sequence holding one).  A kernel, not a memset, so a captured graph
// replays it like any other node.
__global__ __launch_bounds__(64) void attn_table_check_init_kernel(uint32_t *result) {
    if (threadIdx.x == 0) {
        result[0] = 0u;
        result[1] = 0xFFFFFFFFu;
    }
}

// Entry i = b * max_blocks + j is read by a decode of sequence b when block j
// holds a position <= current_pos[b] (clamped to the capacity), i.e. when
// j * page_size <= pos.  Each such entry >= num_blocks adds one to
// result[0] and offers b to result[1] (vector atomics, any order: the
// results do not depend on it).
__global__ __launch_bounds__(256) void attn_table_check_kernel(const uint32_t *table, const uint32_t *cp,
                                                               uint32_t batch, uint32_t page_shift,
                                                               uint32_t max_blocks, uint32_t num_blocks,
                                                               uint32_t *result) {
    const uint64_t total = (uint64_t)batch * max_blocks;
    const uint64_t cap_minus_1 = ((uint64_t)max_blocks << page_shift) - 1;
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * 256u) {
        const uint32_t b = (uint32_t)(i / max_blocks);
        const uint64_t j = i - (uint64_t)b * max_blocks;
        const uint64_t pos = cp[b] < cap_minus_1 ? cp[b] : cap_minus_1;
        if ((j << page_shift) <= pos && table[i] >= num_blocks) {
            atomicAdd(&result[0], 1u);
            atomicMin(&result[1], b);
        }
    }
}

}  // namespace

extern "C" {

attn_status_t attn_paged_table_check(const uint32_t *block_table, const uint32_t *current_pos,
                                     uint32_t batch, uint32_t page_size, uint32_t max_blocks,
                                     uint32_t num_blocks, uint32_t *result, void *stream) {
    if (!block_table || !current_pos || !result)
        return fail(ATTN_ERR_NULL, "block_table, current_pos and result must be non-NULL");
    if (!aligned(block_table, 4) || !aligned(current_pos, 4) || !aligned(result, 4))
        return fail(ATTN_ERR_ALIGN, "block_table, current_pos and result must be 4-byte aligned");
    if (batch == 0 || max_blocks == 0 || num_blocks == 0)
        return fail(ATTN_ERR_DIM, "batch, max_blocks and num_blocks must be nonzero");
    if (page_size == 0 || (page_size & (page_size - 1)) || page_size > 65536u)
        return fail(ATTN_ERR_DIM, "page_size=%u must be a power of two <= 65536", page_size);
    if ((uint64_t)max_blocks * page_size > (1ull << 31))
        return fail(ATTN_ERR_DIM, "max_blocks*page_size exceeds 2^31");
    if ((uint64_t)batch * max_blocks > (1ull << 40))
        return fail(ATTN_ERR_DIM, "block table too large");
    uint32_t shift = 0;
    while ((1u << shift) < page_size) ++shift;
    const uint64_t total = (uint64_t)batch * max_blocks;
    const uint64_t blocks = cdiv(total, 256) < 8192 ? cdiv(total, 256) : 8192;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(attn_table_check_init_kernel, dim3(1), dim3(64), 0, st, result);
    attn_status_t s = hip_check("table check init launch");
    if (s != ATTN_OK) return s;
    hipLaunchKernelGGL(attn_table_check_kernel, dim3((unsigned)blocks), dim3(256), 0, st, block_table,
                       current_pos, batch, shift, max_blocks, num_blocks, result);
    return hip_check("table check launch");
}

}  // extern "C"
