// attn_decode.hip -- split-sequence decode attention for gfx950 (MI355X).
//
// The computation is the masked, scaled Q.K^T followed by softmax and the
// probability-weighted sum of V that the page "Developing Apple Metal Kernels
// in Rust - A Deep Dive Through Attention" defines in section "The MSL,
// briefly".  The page runs it as two dispatches with an fp16 score buffer in
// between; here the cache is read once:
//
//   split kernel    one workgroup streams one chunk of positions for one or
//                   more heads with 16-byte loads, takes fp32 dot products
//                   (v_dot2 on the fp16 inputs), reduces them inside a lane
//                   group with DPP, and keeps an online softmax state
//                   (running max m, running sum l, weighted V sum o) in
//                   registers, in base-2 units.  Lane groups that share a
//                   head merge through LDS; the workgroup writes one partial
//                   (m, l, o[D]) per head, or the final fp16 row when a single
//                   chunk covers the sequence.
//   combine kernel  one workgroup per (sequence, head) merges the chunk
//                   partials: M = max m_c, l = sum l_c 2^(m_c-M),
//                   out = sum o_c 2^(m_c-M) / l, rounded to fp16.
//
// Positions after current_pos are never loaded.  MFMA is not used: one query
// row per head makes this a matrix-vector product bound by HBM bandwidth.
//
// The same split kernel, in other modes, also serves the page's own two
// dispatches (scores written as fp16, then softmax.V from a stored score
// row), a paged cache read through a block table, and the decode step of the
// page "Tutorial 16: Writing Custom Metal Kernels" (q rotated at the new
// token's position; the combine folds in the new token and appends its K/V
// rows, or the split kernel itself when one chunk covers each head block).
// File layout: device helpers (packs, lane-group sums, rotation),
// split kernels, combine kernel, dump fill, standalone rotation; then the
// host planner, kernel selection, launchers and the C ABI.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attn_internal.h"

namespace {

using namespace attn;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;            // waves per split workgroup
constexpr int kThreads = kWaves * 64;
constexpr uint32_t kBalancedMaxBatch = 1024;   // sequences the balanced grid handles
constexpr uint32_t kCombineWide = 512;    // (sequence, head) pairs from which the combine uses 256 threads
constexpr uint32_t kCombineWave = 2048;   // ... and from which it takes one wave per pair
constexpr uint32_t kScoreWindow = 8192;   // fp16 scores a scores-mode workgroup holds in LDS

// ------------------------------------------------------------------ packs
// A pack is VEC consecutive fp16 values of one row held by one lane.

template <int VEC> struct Pack;
template <> struct Pack<8> { u32x4 w; };
template <> struct Pack<4> { u32x2 w; };
template <> struct Pack<2> { uint32_t w; };
template <> struct Pack<1> { uint16_t w; };

template <int VEC>
__device__ __forceinline__ Pack<VEC> load_pack(const uint16_t *p) {
    Pack<VEC> r;
    if constexpr (VEC == 8) r.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else if constexpr (VEC == 4) r.w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    else if constexpr (VEC == 2) r.w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    else r.w = __builtin_nontemporal_load(p);
    return r;
}

template <int VEC>
__device__ __forceinline__ Pack<VEC> zero_pack() {
    Pack<VEC> r;
    if constexpr (VEC == 8) r.w = u32x4{0u, 0u, 0u, 0u};
    else if constexpr (VEC == 4) r.w = u32x2{0u, 0u};
    else r.w = 0;
    return r;
}

template <int VEC>
__device__ __forceinline__ Pack<VEC> make_pack(const uint16_t (&hv)[VEC]) {
    Pack<VEC> r;
    if constexpr (VEC == 1) {
        r.w = hv[0];
    } else if constexpr (VEC == 2) {
        r.w = (uint32_t)hv[0] | (uint32_t)hv[1] << 16;
    } else {
#pragma unroll
        for (int j = 0; j < VEC / 2; ++j) r.w[j] = (uint32_t)hv[2 * j] | (uint32_t)hv[2 * j + 1] << 16;
    }
    return r;
}

template <int VEC>
__device__ __forceinline__ uint32_t pack_word(const Pack<VEC> &p, int j) {
    if constexpr (VEC == 8) return p.w[j];
    else if constexpr (VEC == 4) return p.w[j];
    else return p.w;
}

// Store N fp16 values to N consecutive elements in one write; dst must be
// aligned to 2N bytes.
template <int N>
__device__ __forceinline__ void store_halves(uint16_t *dst, const uint16_t (&hv)[N]) {
    const Pack<N> pk = make_pack<N>(hv);
    if constexpr (N == 8) *reinterpret_cast<u32x4 *>(dst) = pk.w;
    else if constexpr (N == 4) *reinterpret_cast<u32x2 *>(dst) = pk.w;
    else if constexpr (N == 2) *reinterpret_cast<uint32_t *>(dst) = pk.w;
    else *dst = pk.w;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// element e (0..VEC-1) of a pack as fp32
template <int VEC>
__device__ __forceinline__ float pack_elem(const Pack<VEC> &p, int e) {
    if constexpr (VEC == 1) return h2f(p.w);
    else {
        uint32_t w = pack_word<VEC>(p, e >> 1);
        return h2f((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
}

// acc + sum_e a[e]*b[e] with fp32 accumulation of exact fp16 products
template <int VEC>
__device__ __forceinline__ float dot_pack(const Pack<VEC> &a, const Pack<VEC> &b, float acc) {
    if constexpr (VEC == 1) {
        return fmaf(h2f(a.w), h2f(b.w), acc);
    } else {
#pragma unroll
        for (int j = 0; j < VEC / 2; ++j)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, pack_word<VEC>(a, j)),
                                         __builtin_bit_cast(half2v, pack_word<VEC>(b, j)), acc,
                                         false);
        return acc;
    }
}

// ------------------------------------------------------- lane-group sums
// Sum over aligned groups of GL lanes; every lane of a group ends with the
// same bits (each step adds a pair of values in both orders' common result).

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

template <int GL>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (GL >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (GL >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (GL >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (GL >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (GL >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (GL >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

__device__ __forceinline__ uint32_t valid_len(uint32_t cp, uint32_t S) {
    return (cp < S - 1u ? cp : S - 1u) + 1u;
}

__device__ __forceinline__ uint16_t f2h_rne(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ------------------------------------------------------- rotary embedding
// The rotation of the page "Tutorial 16: Writing Custom Metal Kernels"
// (section "5. Example: Fused RoPE Kernel"): pair i of the first `dims`
// values turns by pos * base^(-2i/dims); pairs are (i, i + dims/2), or
// (2i, 2i+1) when `traditional`; values past dims pass through.  The page
// loads precomputed cos/sin; here the frequencies come precomputed (fp64,
// from the host) and cos/sin of the angle are evaluated in the kernel: the
// angle and its reduction to [-pi/4, pi/4] are fp64, so positions in the
// billions keep a full fp32 cos/sin, and the rotation itself is fp32.

constexpr uint32_t kRopeMaxPairs = ATTN_MAX_HEAD_DIM / 2;

struct RopeArgs {
    const uint16_t *k_new;   // [B, H, D] new key rows, before rotation
    const uint16_t *v_new;   // [B, H, D] new value rows
    uint16_t *k_cache;       // caches the new rows are written into
    uint16_t *v_cache;
    uint32_t dims;           // rotated leading values (even, <= D)
    uint32_t traditional;
    double theta[kRopeMaxPairs];   // base^(-2i/dims) for i < dims/2
};

// cos and sin of pos * theta_i.  The angle t is split as n pi/2 + x with n
// the nearest integer to t 2/pi and x = t - n pi/2 taken with pi/2 in two
// parts (Cody and Waite's reduction), |x| <= pi/4; sin x and cos x come from
// their Taylor series (through x^9 and x^10: truncation below 2e-9), and the
// quadrant n mod 4 picks signs and order.
__device__ __forceinline__ void rope_cos_sin(uint32_t i, uint32_t pos, const RopeArgs &r, float *c,
                                             float *s) {
    constexpr double kPio2Hi = 1.5707963267948966;      // pi/2 rounded to fp64
    constexpr double kPio2Lo = 6.123233995736766e-17;   // pi/2 - kPio2Hi
    constexpr double kTwoOverPi = 0.6366197723675814;
    const double t = (double)pos * r.theta[i];
    const double n = rint(t * kTwoOverPi);
    const float x = (float)fma(-n, kPio2Lo, fma(-n, kPio2Hi, t));
    const float x2 = x * x;
    const float sx = x * (1.f + x2 * (-1.f / 6.f + x2 * (1.f / 120.f + x2 * (-1.f / 5040.f +
                                                                             x2 * (1.f / 362880.f)))));
    const float cx = 1.f + x2 * (-0.5f + x2 * (1.f / 24.f + x2 * (-1.f / 720.f +
                                                                x2 * (1.f / 40320.f +
                                                                      x2 * (-1.f / 3628800.f)))));
    const uint32_t quad = (uint32_t)((uint64_t)n & 3u);   // t >= 0, so n >= 0
    const float cq = (quad & 1u) ? sx : cx;
    const float sq = (quad & 1u) ? cx : sx;
    *c = (quad == 1u || quad == 2u) ? -cq : cq;
    *s = (quad >= 2u) ? -sq : sq;
}

// The element that element d is paired with (d itself past dims).
__device__ __forceinline__ uint32_t rope_partner(uint32_t d, const RopeArgs &r) {
    if (d >= r.dims) return d;
    const uint32_t half = r.dims >> 1;
    return r.traditional ? (d ^ 1u) : (d < half ? d + half : d - half);
}

// Element d of a rotated row, from its value x and its partner's value y.
__device__ __forceinline__ float rope_apply(float x, float y, uint32_t d, const RopeArgs &r,
                                            uint32_t pos) {
#pragma clang fp contract(off)
    if (d >= r.dims) return x;
    const uint32_t half = r.dims >> 1;
    const bool first = r.traditional ? (d & 1u) == 0 : d < half;
    const uint32_t i = r.traditional ? d >> 1 : (first ? d : d - half);
    float c, s;
    rope_cos_sin(i, pos, r, &c, &s);
    // pair (a, b) -> (a c - b s, a s + b c); x is a when first, b otherwise
    return first ? fmaf(x, c, -(y * s)) : fmaf(y, s, x * c);
}

__device__ __forceinline__ float rope_elem(const uint16_t *row, uint32_t d, const RopeArgs &r,
                                           uint32_t pos) {
    return rope_apply(h2f(row[d]), h2f(row[rope_partner(d, r)]), d, r, pos);
}

// ------------------------------------------------------------ split kernel

struct SplitArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const uint32_t *cp_dev;   // per-sequence current_pos, or null
    uint32_t cp_host;         // used when cp_dev is null
    uint32_t H, D, S;         // heads, head_dim, cache length per sequence
    uint32_t chunk;           // positions per workgroup (chunked grid)
    uint32_t n_hb;            // head blocks (H / hpb)
    uint32_t hpb;             // heads per workgroup
    uint32_t nc_stride;       // chunk stride of the partial arrays (chunked grid)
    float scale_log2;         // log2(e) / sqrt(D)
    float scale;              // 1 / sqrt(D)
    float *part_o;            // partial o rows (layout: see the kernels)
    float *part_ml;           // partial (m, l) pairs
    uint16_t *out;            // final rows when `direct`
    float *dump;              // [B, H, S] or null
    int direct;               // 1: one chunk per sequence, write fp16 rows
    uint32_t batch;           // sequences (balanced grid)
    uint32_t grid;            // workgroups launched (balanced grid)
    uint32_t *header;         // workspace header: how the partials are laid out
    const uint16_t *scores_in;    // second dispatch: stored fp16 scores [B, H, S]
    uint16_t *scores_out;         // first dispatch: fp16 scores [H, S]
    const uint32_t *block_table;  // paged cache: [batch, max_blocks] page ids, or null
    uint32_t max_blocks;      // block-table row length
    uint32_t num_blocks;      // pages in the pool
    uint32_t page_shift;      // log2(positions per page)
    RopeArgs rope;            // decode step: q is rotated, the new token's slot is skipped
};

// Workspace header written by the split launch and read by the combine.
enum : uint32_t { kHdrBalanced = 0, kHdrChunk, kHdrNcStride, kHdrNHb, kHdrHpb, kHdrGrid, kHdrWords };
constexpr uint32_t kHdrPrefixWord = 64;   // balanced grid: uint64 length prefix [batch + 1] from byte 256
constexpr size_t kHeaderBytes = 256 + ((size_t)kBalancedMaxBatch + 1) * 8 + 248;   // 256-byte multiple

__device__ __forceinline__ void write_header(const SplitArgs &a, uint32_t balanced) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        a.header[kHdrBalanced] = balanced;
        a.header[kHdrChunk] = a.chunk;
        a.header[kHdrNcStride] = a.nc_stride;
        a.header[kHdrNHb] = a.n_hb;
        a.header[kHdrHpb] = a.hpb;
        a.header[kHdrGrid] = a.grid;
    }
}

// Where one workgroup's merged result for head ho of its head block goes:
// o row at po + ho*po_hs, (m, l) at pml + ho*pml_hs; or, when direct, the
// fp16 row at out + ho*D.
struct PieceDst {
    float *po;
    size_t po_hs;
    float *pml;
    size_t pml_hs;
    uint16_t *out;
};

// What a split launch computes: the one-pass decode; softmax.V from stored
// fp16 scores (the page's second dispatch); the decode step (q rotated, the
// new token's slot left to the combine, or merged and appended here when one
// chunk covers each head block); or only the scores, written as fp16 (the
// page's first dispatch).
enum : int { kModeDecode = 0, kModePv = 1, kModeStep = 2, kModeQk = 3 };

// Stream positions [c0, c_end) of head block hb of sequence b through the
// online softmax and leave one merged state per head at `dst` (kModeQk: write
// the scores of those positions instead).  The caller
// guarantees c0 < c_end, except for a one-launch decode step at position 0
// (c0 == c_end: nothing is streamed, and the new token alone is merged).  LDS is free again when this returns.
template <int VEC, int GL, int NV, bool FULL, int U, bool PF, bool DUMP, bool PAGED, int MODE>
__device__ __forceinline__ void split_piece(const SplitArgs &a, uint32_t b, uint32_t hb,
                                            uint32_t c0, uint32_t c_end, const PieceDst &dst,
                                            float *sm_o, float *sm_m, float *sm_l,
                                            uint16_t *sm_sc = nullptr) {
    constexpr int RG = 64 / GL;              // row groups per wave
    constexpr int NG = kWaves * RG;          // row groups per workgroup
    constexpr int DPAD = VEC * GL * NV;      // padded row length in LDS
    constexpr bool SC = MODE == kModePv;
    constexpr bool ROPE = MODE == kModeStep;
    constexpr bool QK = MODE == kModeQk;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = (tid >> 6) * RG + lane / GL;   // row group in the workgroup
    const int gl = lane % GL;                    // lane inside the row group
    const uint32_t hg = (uint32_t)g % a.hpb;     // head inside the head block
    const uint32_t pg = (uint32_t)g / a.hpb;     // position lane
    const uint32_t pps = NG / a.hpb;             // positions per step
    const uint32_t h = hb * a.hpb + hg;
    const size_t D = a.D;
    const size_t HD = (size_t)a.H * D;

    // element offsets of this lane's packs and their validity
    int eoff[NV];
    bool eok[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        eoff[j] = (gl + GL * j) * VEC;
        eok[j] = FULL || eoff[j] < (int)a.D;
    }

    // one-launch decode step: the new token's score per head, and v_new
    __shared__ float sm_tnew[ROPE ? NG : 1];
    __shared__ uint16_t sm_vnew[ROPE ? NG * DPAD : 1];
    Pack<VEC> qp[NV];
    if constexpr (ROPE) {
        // Decode step: the head block's query rows, rotated at the new
        // token's position and rounded to fp16 (the combine rotates them the
        // same way), one element per thread into LDS, which is free here.
        // Done before the first K/V loads: overlapping the two costs the main
        // loop registers, which is worse.
        uint16_t *sq = reinterpret_cast<uint16_t *>(sm_o);
        const uint32_t pos = valid_len(a.cp_dev ? a.cp_dev[b] : a.cp_host, a.S) - 1u;
        const size_t bh0 = (size_t)b * a.H + (size_t)hb * a.hpb;
        const uint16_t *qblk = a.q + bh0 * D;
        const uint32_t n_q = a.hpb * a.D;
        // One chunk per head block (dst.out: the step is one launch): the new
        // token too, which the merge launch takes otherwise.  Its key rows are
        // rotated alongside q (their loads share q's round trip), both rows
        // are appended at slot pos (no streamed position reads that slot),
        // and v_new waits in LDS for the final merge.
        uint16_t *sk = sq + n_q;
        size_t slot = (size_t)b * a.S + pos;
        bool keep = true;
        if constexpr (PAGED) {
            if (dst.out) {
                const uint32_t page = a.block_table[(size_t)b * a.max_blocks + (pos >> a.page_shift)];
                keep = page < a.num_blocks;   // an entry past the pool: nothing is written
                slot = (size_t)page << a.page_shift | (pos & ((1u << a.page_shift) - 1u));
            }
        }
#pragma unroll 1
        for (uint32_t idx = tid; idx < n_q; idx += kThreads) {
            const uint32_t ho = idx / a.D;
            const uint32_t d = idx - ho * a.D;
            sq[idx] = f2h_rne(rope_elem(qblk + (size_t)ho * D, d, a.rope, pos));
            if (dst.out) {
                const uint16_t k16 = f2h_rne(rope_elem(a.rope.k_new + (bh0 + ho) * D, d, a.rope, pos));
                const uint16_t v16 = a.rope.v_new[(bh0 + ho) * D + d];
                sk[idx] = k16;
                sm_vnew[idx] = v16;
                if (keep) {
                    const size_t crow = (slot * a.H + (size_t)hb * a.hpb + ho) * D + d;
                    a.rope.k_cache[crow] = k16;
                    a.rope.v_cache[crow] = v16;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            uint16_t hv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) hv[e] = eok[j] ? sq[hg * a.D + eoff[j] + e] : 0;
            qp[j] = make_pack<VEC>(hv);
        }
        if (dst.out) {   // the new token's base-2 score: wave w takes heads w, w + 4, ...
            for (uint32_t ho = (uint32_t)tid >> 6; ho < a.hpb; ho += kWaves) {
                float prod = 0.f;
                for (uint32_t d = lane; d < a.D; d += 64)   // exact products of fp16 values
                    prod += h2f(sq[ho * a.D + d]) * h2f(sk[ho * a.D + d]);
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) prod += __shfl_xor(prod, off, 64);
                if (lane == 0) sm_tnew[ho] = prod * a.scale_log2;
            }
        }
        __syncthreads();   // LDS is written again by the merge below
    } else if constexpr (!SC) {
        const uint16_t *qrow = a.q + ((size_t)b * a.H + h) * D;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            qp[j] = eok[j] ? load_pack<VEC>(qrow + eoff[j]) : zero_pack<VEC>();
    }
    // stored scores (second dispatch of the two-launch form): row (b, h) of [B, H, S]
    const uint16_t *srow = SC ? a.scores_in + ((size_t)b * a.H + h) * a.S : nullptr;

    // dense: sequence b's rows start at b*S*H*D; paged: rows live in pool
    // pages [num_blocks, page, H, D] named by the sequence's block-table row
    const uint32_t *bt = PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr;
    const size_t seq_base = (PAGED ? 0 : (size_t)b * a.S * HD) + (size_t)h * D;
    const uint16_t *kbase = a.k + seq_base;
    const uint16_t *vbase = a.v + seq_base;
    auto row_of = [&](uint32_t p) -> size_t { return (size_t)p * HD; };
    // paged rows: any table entry >= num_blocks reads the last page (in bounds)

    float m = -INFINITY, l = 0.f;
    float acc[NV][VEC];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;

    // Position of block slot u of this lane's row group.  Row groups
    // interleave (slot u of every row group, then slot u + 1), except in
    // scores mode, where a row group takes U adjacent positions so that its
    // leader writes their scores to LDS with one packed store.  Each load
    // instruction still reads whole head blocks of single positions.
    auto pos_at = [&](uint32_t base, int u) -> uint32_t {
        return QK ? base + pg * U + u : base + u * pps + pg;
    };

    // One block = U positions per row group.  Slots past the chunk end load
    // the chunk's first row (always valid) and get weight 0.
    struct Block {
        Pack<VEC> k[U][NV], v[U][NV];
        uint16_t sc[U];   // stored scores (SC)
    };
    // Page ids of a block's positions (paged caches).  They are fetched one
    // block ahead of the K/V loads that need them, and before the K/V loads of
    // the block in between, so waiting for them never waits for K/V data.
    struct Pids {
        uint32_t id[U];
    };
    auto fetch_pids = [&](Pids &pi, uint32_t base) {
        if constexpr (PAGED) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t p = pos_at(base, u);
                pi.id[u] = bt[(p < c_end ? p : c0) >> a.page_shift];
            }
        }
    };
    auto load_rows = [&](Block &blk, uint32_t base, const Pids &pi) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = pos_at(base, u);
            const uint32_t pc = p < c_end ? p : c0;
            size_t row;
            if constexpr (PAGED) {
                const uint32_t page = pi.id[u] < a.num_blocks ? pi.id[u] : a.num_blocks - 1;
                row = ((size_t)page << a.page_shift | (pc & ((1u << a.page_shift) - 1u))) * HD;
            } else {
                row = row_of(pc);
            }
            if constexpr (SC) blk.sc[u] = srow[pc];
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if constexpr (!SC)
                    blk.k[u][j] = eok[j] ? load_pack<VEC>(kbase + row + eoff[j]) : zero_pack<VEC>();
                if constexpr (!QK)
                    blk.v[u][j] = eok[j] ? load_pack<VEC>(vbase + row + eoff[j]) : zero_pack<VEC>();
            }
        }
    };
    // Scores mode: the scores of a window of qk_w positions per head collect
    // in LDS (sm_sc, kScoreWindow values) and leave in 16-byte stores when
    // the window is full or the piece ends.  Stores and loads share one
    // completion counter, so a store per block would put a write
    // acknowledgement into every block's wait.  qk_w is a power of two and
    // a multiple of the block's positions, so blocks never straddle windows.
    const uint32_t qk_w = QK ? kScoreWindow / a.hpb : 0;
    auto flush_scores = [&](uint32_t w0, uint32_t wn) {
        const uint32_t n8 = (wn + 7) / 8;
        for (uint32_t idx = tid; idx < a.hpb * n8; idx += kThreads) {
            const uint32_t ho = idx / n8;
            const uint32_t j = idx - ho * n8;
            const uint16_t *src = sm_sc + ho * qk_w + j * 8;
            uint16_t *out = a.scores_out + ((size_t)b * a.H + (size_t)hb * a.hpb + ho) * a.S + w0 + j * 8;
            const uint32_t cnt = min(8u, wn - j * 8);
            if (cnt == 8 && ((uintptr_t)out & 15) == 0) {
                *reinterpret_cast<u32x4 *>(out) = *reinterpret_cast<const u32x4 *>(src);
            } else {
                for (uint32_t e = 0; e < cnt; ++e) out[e] = src[e];
            }
        }
    };
    auto consume = [&](const Block &blk, uint32_t base) {
        if constexpr (QK) {   // first dispatch: the fp16 score of each position
            uint16_t s16[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = 0.f;
#pragma unroll
                for (int j = 0; j < NV; ++j) dot = dot_pack<VEC>(qp[j], blk.k[u][j], dot);
                s16[u] = f2h_rne(group_sum<GL>(dot) * a.scale);
            }
            const uint32_t w0 = c0 + (base - c0) / qk_w * qk_w;
            // slots past the piece's end land inside the window, unflushed
            if (gl == 0) store_halves<U>(sm_sc + hg * qk_w + (pos_at(base, 0) - w0), s16);
            const uint32_t next = base + pps * U;
            if (next == w0 + qk_w || next >= c_end) {   // the same for every thread
                __syncthreads();
                flush_scores(w0, min(qk_w, c_end - w0));
                __syncthreads();
            }
            return;
        }
        float t[U];
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = pos_at(base, u);
            float dot = 0.f;
            if constexpr (SC) {
                // natural-log score from the buffer, in base-2 units
                t[u] = p < c_end ? h2f(blk.sc[u]) * 1.4426950408889634f : -INFINITY;
            } else {
#pragma unroll
                for (int j = 0; j < NV; ++j) dot = dot_pack<VEC>(qp[j], blk.k[u][j], dot);
                dot = group_sum<GL>(dot);
                t[u] = p < c_end ? dot * a.scale_log2 : -INFINITY;
            }
            tmax = fmaxf(tmax, t[u]);
            if constexpr (DUMP) {
                if (p < c_end && gl == 0) a.dump[((size_t)b * a.H + h) * a.S + p] = dot * a.scale;
            }
        }
        const float m_new = fmaxf(m, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // group saw no position yet
        const float corr = __builtin_amdgcn_exp2f(m - m_use);
        l *= corr;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[j][e] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float pw = __builtin_amdgcn_exp2f(t[u] - m_use);   // 0 for masked slots
            l += pw;
            // a stored -inf score weighs nothing, whatever V holds at that row
            const bool live = !SC || t[u] != -INFINITY;
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    acc[j][e] = fmaf(pw, live ? pack_elem<VEC>(blk.v[u][j], e) : 0.f, acc[j][e]);
        }
        m = m_new;
    };

    const uint32_t step = pps * U;
    // An empty piece (a one-launch decode step at position 0) streams nothing;
    // other modes never get one, and their code keeps no test for it.
    if (!ROPE || c0 < c_end) {
    if constexpr (PF) {
        // Two register blocks: the next block's loads are in flight while the
        // current one is reduced.  The steady-state loop issues its loads
        // unconditionally (the last one or two blocks are peeled off), so the
        // compiler's wait counts cover only the block being reduced.
        Block A, B;
        Pids P0{}, P1{};
        const uint32_t n = (c_end - c0 + step - 1) / step;   // blocks, >= 1
        uint32_t base = c0;
        fetch_pids(P0, base);
        fetch_pids(P1, base + step);
        load_rows(A, base, P0);
        uint32_t i = 0;
        for (; i + 2 < n; i += 2) {
            fetch_pids(P0, base + 2 * step);
            load_rows(B, base + step, P1);
            consume(A, base);
            fetch_pids(P1, base + 3 * step);
            load_rows(A, base + 2 * step, P0);
            consume(B, base + step);
            base += 2 * step;
        }
        if (i + 1 < n) {
            load_rows(B, base + step, P1);
            consume(A, base);
            consume(B, base + step);
        } else {
            consume(A, base);
        }
    } else {
        Pids P0{}, P1{};
        fetch_pids(P0, c0);
        for (uint32_t base = c0; base < c_end; base += step) {
            Block A;
            fetch_pids(P1, base + step);
            load_rows(A, base, P0);
            consume(A, base);
            P0 = P1;
        }
    }
    }

    if constexpr (QK) return;   // no softmax state to merge

    // ---- merge the row groups that share a head
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_o[g * DPAD + eoff[j] + e] = acc[j][e];
    if (gl == 0) {
        sm_m[g] = m;
        sm_l[g] = l;
    }
    __syncthreads();

    const uint32_t n_out = a.hpb * a.D;
    for (uint32_t idx = tid; idx < n_out; idx += kThreads) {
        const uint32_t ho = idx / a.D;
        const uint32_t d = idx % a.D;
        float M = -INFINITY;
        for (uint32_t r = 0; r < pps; ++r) M = fmaxf(M, sm_m[r * a.hpb + ho]);
        float t_new = -INFINITY;   // the new token's score (one-launch decode step)
        if constexpr (ROPE) {
            if (dst.out) {
                t_new = sm_tnew[ho];
                M = fmaxf(M, t_new);
            }
        }
        // Position lane 0 always saw position c0, so M is finite unless every
        // score here is a stored -inf (softmax.V from a masked stretch of the
        // row); such a head merges to (-inf, 0, 0), which the combine weighs
        // exactly 0, rather than to the NaN that 2^(-inf - -inf) would give.
        const float Mu = M == -INFINITY ? 0.f : M;
        float o = 0.f, lsum = 0.f;
        for (uint32_t r = 0; r < pps; ++r) {
            const int gg = r * a.hpb + ho;
            const float w = __builtin_amdgcn_exp2f(sm_m[gg] - Mu);
            o = fmaf(sm_o[gg * DPAD + d], w, o);
            lsum = fmaf(sm_l[gg], w, lsum);
        }
        if (dst.out) {
            if constexpr (ROPE) {   // the new token joins with l term 1
                const float w = __builtin_amdgcn_exp2f(t_new - Mu);
                o = fmaf(h2f(sm_vnew[ho * a.D + d]), w, o);
                lsum = fmaf(1.f, w, lsum);
            }
            dst.out[ho * a.D + d] = f2h_rne(o / lsum);
        } else {
            dst.po[ho * dst.po_hs + d] = o;
            if (d == 0) {
                dst.pml[ho * dst.pml_hs] = M;
                dst.pml[ho * dst.pml_hs + 1] = lsum;
            }
        }
    }
    __syncthreads();   // LDS may be reused by the caller's next piece
}

// VEC: fp16 values per lane load; GL: lanes per row (power of two);
// NV: packs per lane per row; FULL: D == VEC*GL*NV (no element guards);
// U: positions per row group per block; PF: double-buffered blocks.
#define ATTN_SPLIT_LDS                                                                   \
    constexpr int NG_ = kWaves * (64 / GL);                                              \
    __shared__ float sm_o[NG_ * VEC * GL * NV];                                          \
    __shared__ float sm_m[NG_];                                                          \
    __shared__ float sm_l[NG_];

// Chunked grid: workgroup (hb + n_hb*chunk, b) takes positions
// [chunk*C, (chunk+1)*C) of head block hb.  Partials: o [B, H, nc_stride, D],
// (m, l) [B, H, nc_stride, 2].
template <int VEC, int GL, int NV, bool FULL, int U, bool PF, bool DUMP, bool PAGED, int MODE, int WAVES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, WAVES)))
void attn_split_kernel(SplitArgs a) {
    ATTN_SPLIT_LDS
    constexpr bool ROPE = MODE == kModeStep;
    if constexpr (MODE == kModeQk) {
        // workgroups past the reading grid write -inf over the masked
        // positions [L, S) of every head (their rows are never read)
        if (blockIdx.x >= a.grid) {
            constexpr uint16_t kNegInfHalf = 0xFC00;
            const uint32_t L = valid_len(a.cp_host, a.S);
            const uint64_t span = a.S - L;
            const uint64_t total = (uint64_t)a.H * span;
            const uint64_t n_fill = gridDim.x - a.grid;
            for (uint64_t i = (uint64_t)(blockIdx.x - a.grid) * kThreads + threadIdx.x; i < total;
                 i += n_fill * kThreads) {
                const uint64_t h = i / span;
                a.scores_out[h * a.S + L + (i - h * span)] = kNegInfHalf;
            }
            return;
        }
    } else {
        write_header(a, 0);
    }
    const uint32_t b = blockIdx.y;
    const uint32_t hb = blockIdx.x % a.n_hb;
    const uint32_t chunk = blockIdx.x / a.n_hb;
    const uint32_t cp = a.cp_dev ? a.cp_dev[b] : a.cp_host;
    // a decode step streams the positions before the new token's slot
    const uint32_t L = valid_len(cp, a.S) - (ROPE ? 1u : 0u);
    const uint32_t c0 = chunk * a.chunk;
    // whole workgroup: nothing to read (a one-launch decode step at position
    // 0 still merges the new token)
    if (c0 >= L && !(ROPE && a.direct)) return;
    const uint32_t c_end = min(c0 + a.chunk, L);
    const size_t bh0 = (size_t)b * a.H + (size_t)hb * a.hpb;
    PieceDst dst;
    dst.po = a.part_o + (bh0 * a.nc_stride + chunk) * a.D;
    dst.po_hs = (size_t)a.nc_stride * a.D;
    dst.pml = a.part_ml + (bh0 * a.nc_stride + chunk) * 2;
    dst.pml_hs = (size_t)a.nc_stride * 2;
    dst.out = a.direct ? a.out + bh0 * a.D : nullptr;
    __shared__ __align__(16) uint16_t sm_sc[MODE == kModeQk ? kScoreWindow : 8];
    split_piece<VEC, GL, NV, FULL, U, PF, DUMP, PAGED, MODE>(a, b, hb, c0, c_end, dst, sm_o, sm_m,
                                                                 sm_l, sm_sc);
}

// Inclusive prefix of the streamed lengths (valid length minus `excl`):
// pref[0] = 0, pref[b+1] = sum of L_0..L_b, for batch <= kBalancedMaxBatch.  Hillis-Steele scan in LDS over
// per-thread sums of consecutive sequences.  Every thread must call it.
template <int NT>
__device__ __forceinline__ void length_prefix(const uint32_t *cp, uint32_t cp_host, uint32_t S,
                                              uint32_t excl, uint32_t batch, uint64_t *pref,
                                              uint64_t *tmp) {
    const uint32_t tid = threadIdx.x;
    const uint32_t per = (batch + NT - 1) / NT;   // <= kBalancedMaxBatch / NT
    const uint32_t b0 = tid * per;
    uint64_t sum = 0;
    for (uint32_t i = 0; i < per; ++i)
        if (b0 + i < batch) sum += valid_len(cp ? cp[b0 + i] : cp_host, S) - excl;
    tmp[tid] = sum;
    __syncthreads();
    for (uint32_t off = 1; off < NT; off <<= 1) {
        const uint64_t add = tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        tmp[tid] += add;
        __syncthreads();
    }
    uint64_t run = tid ? tmp[tid - 1] : 0;
    if (tid == 0) pref[0] = 0;
    for (uint32_t i = 0; i < per; ++i)
        if (b0 + i < batch) {
            run += valid_len(cp ? cp[b0 + i] : cp_host, S) - excl;
            pref[b0 + i + 1] = run;
        }
    __syncthreads();
}

// Sequence b with pref[b] <= key < pref[b+1], for key < pref[batch]; such a
// sequence has at least one position (empty ones are never returned).
__device__ __forceinline__ uint32_t find_sequence(const uint64_t *pref, uint32_t batch, uint64_t key) {
    uint32_t lo = 0, hi = batch;   // pref[lo] <= key < pref[hi]
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (pref[mid] <= key) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Balanced grid for per-sequence lengths: the batch's work, laid out as
// segments (b, hb) of L_b positions each in order s = b*n_hb + hb, is cut into
// `grid` equal ranges, one per workgroup.  A workgroup writes one partial per
// segment piece it covers, at slot w + s; o [slots, hpb, D], (m, l)
// [slots, hpb, 2] with slots = grid + batch*n_hb.
template <int VEC, int GL, int NV, bool FULL, int U, bool PF, bool DUMP, bool PAGED, int MODE, int WAVES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, WAVES)))
void attn_split_balanced_kernel(SplitArgs a) {
    ATTN_SPLIT_LDS
    constexpr bool ROPE = MODE == kModeStep;
    write_header(a, 1);
    __shared__ uint64_t sm_pref[kBalancedMaxBatch + 1];
    __shared__ uint64_t sm_tmp[kThreads];
    length_prefix<kThreads>(a.cp_dev, a.cp_host, a.S, ROPE ? 1u : 0u, a.batch, sm_pref, sm_tmp);
    if (blockIdx.x == 0) {   // publish the prefix for the combine launch
        uint64_t *hp = reinterpret_cast<uint64_t *>(a.header + kHdrPrefixWord);
        for (uint32_t i = threadIdx.x; i <= a.batch; i += kThreads) hp[i] = sm_pref[i];
    }
    const uint64_t n_hb = a.n_hb;
    const uint64_t W = n_hb * sm_pref[a.batch];
    // at most one workgroup per unit of work, so every range is non-empty
    const uint64_t G = a.grid < W ? a.grid : W;
    const uint64_t w = blockIdx.x;
    if (w >= G) return;
    // the host only picks this grid when W * grid < 2^63
    const uint64_t lo = w * W / G;
    const uint64_t hi = (w + 1) * W / G;
    uint64_t x = lo;
    while (x < hi) {
        const uint32_t b = find_sequence(sm_pref, a.batch, x / n_hb);
        const uint64_t L = sm_pref[b + 1] - sm_pref[b];
        const uint64_t off = x - n_hb * sm_pref[b];
        const uint32_t hb = (uint32_t)(off / L);
        const uint64_t seg_end = n_hb * sm_pref[b] + (hb + 1) * L;
        const uint64_t x_end = hi < seg_end ? hi : seg_end;
        const uint32_t c0 = (uint32_t)(off % L);
        const uint32_t c_end = c0 + (uint32_t)(x_end - x);
        const uint64_t slot = w + (uint64_t)b * n_hb + hb;
        PieceDst dst;
        dst.po = a.part_o + slot * a.hpb * a.D;
        dst.po_hs = a.D;
        dst.pml = a.part_ml + slot * a.hpb * 2;
        dst.pml_hs = 2;
        dst.out = nullptr;
        split_piece<VEC, GL, NV, FULL, U, PF, DUMP, PAGED, MODE>(a, b, hb, c0, c_end, dst, sm_o, sm_m,
                                                                 sm_l);
        x = x_end;
    }
}

// ---------------------------------------------------------- combine kernel

struct CombineArgs {
    const float *part_o;
    const float *part_ml;
    const uint32_t *cp_dev;
    uint32_t cp_host;
    uint32_t H, D, S, batch;
    const uint32_t *header;   // written by the split launch
    uint16_t *out;
    // decode step: the new token (rotated q and k_new, v_new) joins as one
    // more partial, and its k and v rows are appended to the caches
    const uint16_t *q;
    float scale_log2;         // log2(e) / sqrt(D)
    RopeArgs rope;
    // paged caches: the appended rows go to the page the block table names
    // for slot pos (nothing is written for an entry >= num_blocks)
    const uint32_t *block_table;
    uint32_t max_blocks, num_blocks, page_shift;
};

// One workgroup per (sequence, head); thread (cg, d) handles element d of
// chunks cg, cg+G, ...  When every chunk fits in registers (the usual case)
// all partials are loaded in one round before any arithmetic: M = max m_c
// across the workgroup, weights 2^(m_c - M) go through LDS, and each thread
// sums its o_c[d]*w and l_c*w.  More chunks take a tiled loop.  o and l go
// through the same operations in the same order, so all-equal V rows give
// exactly 1.
constexpr int kCombineRegs = 8;   // chunk values per thread held in registers

// Where the split launch left the partials of (sequence b, head h): nc of
// them, the first at (ml, po), consecutive ones ml_cs and po_cs floats apart.
// `excl` positions at the end of the sequence are not in the partials (a
// decode step's new token).
struct PartialSpan {
    uint32_t nc;
    const float *ml, *po;
    size_t ml_cs, po_cs;
};

__device__ __forceinline__ PartialSpan locate_partials(const CombineArgs &a, uint32_t b, uint32_t h,
                                                       uint32_t cp, uint32_t excl) {
    PartialSpan r{0, nullptr, nullptr, 0, 0};
    const size_t bh = (size_t)b * a.H + h;
    if (!a.header[kHdrBalanced]) {
        const uint32_t L = valid_len(cp, a.S) - excl;
        const uint32_t chunk = a.header[kHdrChunk];
        const size_t nc_stride = a.header[kHdrNcStride];
        r.nc = (L + chunk - 1) / chunk;
        r.ml = a.part_ml + bh * nc_stride * 2;
        r.po = a.part_o + bh * nc_stride * a.D;
        r.ml_cs = 2;
        r.po_cs = a.D;
    } else {
        // the split grid's workgroups w_first..w_last covered segment
        // s = b*n_hb + hb; workgroup w left its piece at slot w + s
        const uint64_t *pref = reinterpret_cast<const uint64_t *>(a.header + kHdrPrefixWord);
        const uint32_t hpb = a.header[kHdrHpb];
        const uint64_t n_hb = a.header[kHdrNHb];
        const uint64_t W = n_hb * pref[a.batch];
        const uint64_t G = a.header[kHdrGrid] < W ? a.header[kHdrGrid] : W;   // as the split did
        const uint32_t hb = h / hpb, ho = h % hpb;
        const uint64_t L = pref[b + 1] - pref[b];
        if (L > 0) {   // (a decode step at position 0 has no earlier positions)
            const uint64_t first = n_hb * pref[b] + hb * L;
            const uint64_t last = first + L - 1;
            const uint64_t w_first = ((first + 1) * G - 1) / W;   // W * G < 2^63
            const uint64_t w_last = ((last + 1) * G - 1) / W;
            r.nc = (uint32_t)(w_last - w_first + 1);
            const uint64_t slot0 = w_first + (uint64_t)b * n_hb + hb;
            r.ml = a.part_ml + (slot0 * hpb + ho) * 2;
            r.po = a.part_o + (slot0 * hpb + ho) * a.D;
            r.ml_cs = (size_t)hpb * 2;
            r.po_cs = (size_t)hpb * a.D;
        }
    }
    return r;
}

// Decode step: element d of the new token's rotated key and value row into
// slot pos of sequence b's caches (dense, or the page the block table names;
// nothing for a table entry past the pool).
__device__ __forceinline__ void append_elem(const CombineArgs &a, uint32_t b, uint32_t h,
                                            uint32_t pos, uint32_t d, uint16_t k16, uint16_t v16) {
    size_t slot = (size_t)b * a.S + pos;
    if (a.block_table) {
        const uint32_t page = a.block_table[(size_t)b * a.max_blocks + (pos >> a.page_shift)];
        if (page >= a.num_blocks) return;
        slot = (size_t)page << a.page_shift | (pos & ((1u << a.page_shift) - 1u));
    }
    const size_t row = (slot * a.H + h) * a.D + d;
    a.rope.k_cache[row] = k16;
    a.rope.v_cache[row] = v16;
}

// NT threads per workgroup: 1024 when there are few (sequence, head) pairs,
// each of which may have many partials; 256 from kCombineWide pairs, so the
// grid fills the chip in one round; larger batches take
// attn_combine_wave_kernel below.  STEP: the second launch of a decode step
// (see CombineArgs).
template <int NT, bool STEP>
__global__ __launch_bounds__(NT) void attn_combine_kernel(CombineArgs a) {
    __shared__ float sm_w[NT];
    __shared__ float sm_lc[NT];
    __shared__ float sm_red[NT / 64];
    __shared__ float sm_o[NT];
    __shared__ float sm_l[NT];

    const uint32_t h = blockIdx.x;
    const uint32_t b = blockIdx.y;
    const size_t bh = (size_t)b * a.H + h;
    const uint32_t tid = threadIdx.x;
    const uint32_t cp = a.cp_dev ? a.cp_dev[b] : a.cp_host;

    // The new token (STEP): element tid < D of its q, k_new (each with its
    // pair partner) and v_new rows, loaded before the partials so the two
    // sets of loads overlap.
    float qx = 0.f, qy = 0.f, kx = 0.f, ky = 0.f;
    uint16_t v16 = 0;
    if constexpr (STEP) {
        if (tid < a.D) {
            const uint32_t pd = rope_partner(tid, a.rope);
            const uint16_t *qrow = a.q + bh * a.D;
            const uint16_t *krow = a.rope.k_new + bh * a.D;
            qx = h2f(qrow[tid]);
            qy = h2f(qrow[pd]);
            kx = h2f(krow[tid]);
            ky = h2f(krow[pd]);
            v16 = a.rope.v_new[bh * a.D + tid];
        }
    }
    // Its score: the rotated q against the rotated k_new, both rounded to
    // fp16 as the split kernel and the cache hold them (base-2 units), and
    // the append of its rows at slot pos.  Every thread must call it.
    __shared__ float sm_dot[NT / 64];
    auto new_token_score = [&]() -> float {
        const uint32_t pos = valid_len(cp, a.S) - 1u;
        float prod = 0.f;
        if (tid < a.D) {
            const uint16_t q16 = f2h_rne(rope_apply(qx, qy, tid, a.rope, pos));
            const uint16_t k16 = f2h_rne(rope_apply(kx, ky, tid, a.rope, pos));
            prod = h2f(q16) * h2f(k16);   // exact: both factors are fp16
            append_elem(a, b, h, pos, tid, k16, v16);
        }
        return block_sum<NT>(prod, sm_dot) * a.scale_log2;
    };
    float t_new = -INFINITY;

    const PartialSpan ps = locate_partials(a, b, h, cp, STEP ? 1u : 0u);
    const uint32_t nc = ps.nc;
    const float *ml = ps.ml, *po = ps.po;
    const size_t ml_cs = ps.ml_cs, po_cs = ps.po_cs;
    const uint32_t G = NT / a.D;   // chunk groups (D <= 256)
    const uint32_t cg = tid / a.D;
    const uint32_t d = tid % a.D;
    const bool active = cg < G;
    float o = 0.f, lsum = 0.f;
    float M_all;   // the largest m over all partials (and the new token)

    if (nc <= G * kCombineRegs && nc <= (uint32_t)NT) {
        // one round of loads
        const float mc = tid < nc ? ml[tid * ml_cs] : -INFINITY;
        const float lc = tid < nc ? ml[tid * ml_cs + 1] : 0.f;
        float ov[kCombineRegs];
#pragma unroll
        for (int j = 0; j < kCombineRegs; ++j) {
            const uint32_t c = cg + j * G;
            ov[j] = (active && c < nc) ? po[c * po_cs + d] : 0.f;
        }
        if constexpr (STEP) t_new = new_token_score();
        float M = block_max<NT>(mc, sm_red);
        if constexpr (STEP) M = fmaxf(M, t_new);
        M_all = M;
        if (tid < nc) {
            sm_w[tid] = __builtin_amdgcn_exp2f(mc - M);
            sm_lc[tid] = lc;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kCombineRegs; ++j) {
            const uint32_t c = cg + j * G;
            if (active && c < nc) {
                const float w = sm_w[c];
                o = fmaf(ov[j], w, o);
                lsum = fmaf(sm_lc[c], w, lsum);
            }
        }
    } else {
        float mx = -INFINITY;
        for (uint32_t c = tid; c < nc; c += NT) mx = fmaxf(mx, ml[c * ml_cs]);
        if constexpr (STEP) t_new = new_token_score();
        float M = block_max<NT>(mx, sm_red);
        if constexpr (STEP) M = fmaxf(M, t_new);
        M_all = M;
        for (uint32_t t0 = 0; t0 < nc; t0 += NT) {
            const uint32_t tn = min(nc - t0, (uint32_t)NT);
            __syncthreads();   // previous tile's weights are consumed
            if (tid < tn) {
                sm_w[tid] = __builtin_amdgcn_exp2f(ml[(t0 + tid) * ml_cs] - M);
                sm_lc[tid] = ml[(t0 + tid) * ml_cs + 1];
            }
            __syncthreads();
            if (active) {
                uint32_t c = cg;
                for (; c + 3 * G < tn; c += 4 * G) {
                    float ov[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) ov[u] = po[(t0 + c + u * G) * po_cs + d];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float w = sm_w[c + u * G];
                        o = fmaf(ov[u], w, o);
                        lsum = fmaf(sm_lc[c + u * G], w, lsum);
                    }
                }
                for (; c < tn; c += G) {
                    const float w = sm_w[c];
                    o = fmaf(po[(t0 + c) * po_cs + d], w, o);
                    lsum = fmaf(sm_lc[c], w, lsum);
                }
            }
        }
    }
    if constexpr (STEP) {
        if (tid < a.D) {   // the new token, with weight 2^(t_new - M) and l term 1
            const float w = __builtin_amdgcn_exp2f(t_new - M_all);
            o = fmaf(h2f(v16), w, o);
            lsum = fmaf(1.f, w, lsum);
        }
    } else {
        (void)M_all;
        (void)t_new;
        (void)new_token_score;
    }
    sm_o[tid] = o;
    sm_l[tid] = lsum;
    __syncthreads();
    if (tid < a.D) {
        float os = 0.f, ls = 0.f;
        for (uint32_t r = 0; r < G; ++r) {
            os += sm_o[r * a.D + tid];
            ls += sm_l[r * a.D + tid];
        }
        a.out[bh * a.D + tid] = f2h_rne(os / ls);
    }
}

// Many (sequence, head) pairs, each with a few partials (batches): one wave
// per pair, four pairs per workgroup, so the launch is a quarter of the
// workgroups and no barrier is needed.  Lane i holds output elements
// i, i+64, ...; the partials are merged in chunk order (the max first, then
// the weighted sums of o and l through the same operations, so all-equal V
// rows still give exactly 1).  STEP as in attn_combine_kernel.
template <bool STEP>
__global__ __launch_bounds__(256) void attn_combine_wave_kernel(CombineArgs a) {
    constexpr int EPL = ATTN_MAX_HEAD_DIM / 64;   // output elements per lane, at most
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t pair = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (uint64_t)a.batch * a.H) return;   // the whole wave
    const uint32_t b = (uint32_t)(pair / a.H), h = (uint32_t)(pair % a.H);
    const uint32_t cp = a.cp_dev ? a.cp_dev[b] : a.cp_host;

    float qx[EPL], qy[EPL], kx[EPL], ky[EPL];
    uint16_t v16[EPL];
    if constexpr (STEP) {   // the new token's rows, loaded before the partials
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint32_t d = lane + 64u * j;
            qx[j] = qy[j] = kx[j] = ky[j] = 0.f;
            v16[j] = 0;
            if (d < a.D) {
                const uint32_t pd = rope_partner(d, a.rope);
                const uint16_t *qrow = a.q + pair * a.D;
                const uint16_t *krow = a.rope.k_new + pair * a.D;
                qx[j] = h2f(qrow[d]);
                qy[j] = h2f(qrow[pd]);
                kx[j] = h2f(krow[d]);
                ky[j] = h2f(krow[pd]);
                v16[j] = a.rope.v_new[pair * a.D + d];
            }
        }
    }
    const PartialSpan ps = locate_partials(a, b, h, cp, STEP ? 1u : 0u);
    float M = -INFINITY;
    for (uint32_t c = lane; c < ps.nc; c += 64) M = fmaxf(M, ps.ml[c * ps.ml_cs]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float t_new = -INFINITY;
    if constexpr (STEP) {
        const uint32_t pos = valid_len(cp, a.S) - 1u;
        float prod = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint32_t d = lane + 64u * j;
            if (d < a.D) {
                const uint16_t q16 = f2h_rne(rope_apply(qx[j], qy[j], d, a.rope, pos));
                const uint16_t k16 = f2h_rne(rope_apply(kx[j], ky[j], d, a.rope, pos));
                prod += h2f(q16) * h2f(k16);   // exact products, fp32 sum
                append_elem(a, b, h, pos, d, k16, v16[j]);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) prod += __shfl_xor(prod, off, 64);
        t_new = prod * a.scale_log2;
        M = fmaxf(M, t_new);
    }
    float o[EPL], l = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) o[j] = 0.f;
#pragma unroll 4
    for (uint32_t c = 0; c < ps.nc; ++c) {
        const float w = __builtin_amdgcn_exp2f(ps.ml[c * ps.ml_cs] - M);
        l = fmaf(ps.ml[c * ps.ml_cs + 1], w, l);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint32_t d = lane + 64u * j;
            if (d < a.D) o[j] = fmaf(ps.po[c * ps.po_cs + d], w, o[j]);
        }
    }
    if constexpr (STEP) {   // the new token, with weight 2^(t_new - M) and l term 1
        const float w = __builtin_amdgcn_exp2f(t_new - M);
        l = fmaf(1.f, w, l);
#pragma unroll
        for (int j = 0; j < EPL; ++j) o[j] = fmaf(h2f(v16[j]), w, o[j]);
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const uint32_t d = lane + 64u * j;
        if (d < a.D) a.out[pair * a.D + d] = f2h_rne(o[j] / l);
    }
}

// ------------------------------------------------------------- dump fill

__global__ __launch_bounds__(256) void attn_dump_fill_kernel(float *dump, const uint32_t *cp_dev,
                                                             uint32_t cp_host, uint32_t H,
                                                             uint32_t S, uint64_t total) {
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * 256u) {
        const uint64_t bh = i / S;
        const uint32_t p = (uint32_t)(i - bh * S);
        const uint32_t cp = cp_dev ? cp_dev[bh / H] : cp_host;
        if (p >= valid_len(cp, S)) dump[i] = -INFINITY;
    }
}

// ------------------------------------------------------ standalone rotation

// x, y [rows, D]; row r is at position pos[r / rows_per_pos].
__global__ __launch_bounds__(256) void attn_rope_kernel(const uint16_t *x, uint16_t *y,
                                                        const uint32_t *pos, uint32_t rows_per_pos,
                                                        uint32_t D, uint64_t total, RopeArgs r) {
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * 256u) {
        const uint64_t row = i / D;
        const uint32_t d = (uint32_t)(i - row * D);
        y[i] = f2h_rne(rope_elem(x + row * D, d, r, pos[row / rows_per_pos]));
    }
}

// =============================================================== host side

// Planner knobs, sized for 256 compute units and measured on MI355X: the
// best head blocking makes each position's read 512 contiguous bytes or
// more, and about 1024 workgroups (4 per CU) keep enough loads in flight.
// The ATTN_DECODE_TUNE environment variable
// ("wgs=N,cmax=N,hpb=N,unroll=N,pf=N,bal=N,wfloor=N,waves=N") overrides them for
// tuning sweeps; it is read once per process.
struct Knobs {
    uint32_t wgs;      // target workgroups per call
    uint32_t cmax;     // largest chunk, positions
    uint32_t hpb;      // requested heads per workgroup
    uint32_t unroll;   // positions per row group per block (2, 4, 8)
    uint32_t pf;       // double-buffered blocks
    uint32_t bal;      // per-sequence lengths: balanced grid (equal work per workgroup)
    uint32_t wfloor = 2;   // chunks per head block from wgs / head blocks: 0 rounded up,
                           // 1 rounded down, 2 down for targets of <= 512 workgroups
    uint32_t waves = 0;    // 2: the instantiation compiled for at most two waves per
                           // SIMD (decodes and steps, U = 2 or 8, double-buffered); 0: none
};
constexpr uint32_t kChunkGranule = 16;
constexpr uint32_t kMaxHeadsPerWG = kWaves * 64 / 8;   // row groups at 8 lanes per row

const Knobs &env_knobs() {
    static const Knobs t = [] {
        Knobs r{0, 0, 0, 0, 2, 2, 3};
        const char *env = getenv("ATTN_DECODE_TUNE");
        if (env) {
            char buf[256];
            snprintf(buf, sizeof buf, "%s", env);
            for (char *tok = strtok(buf, ","); tok; tok = strtok(nullptr, ",")) {
                unsigned v = 0;
                if (sscanf(tok, "wgs=%u", &v) == 1 && v > 0) r.wgs = v;
                else if (sscanf(tok, "cmax=%u", &v) == 1 && v >= kChunkGranule)
                    r.cmax = v / kChunkGranule * kChunkGranule;
                else if (sscanf(tok, "hpb=%u", &v) == 1 && v > 0) r.hpb = v;
                else if (sscanf(tok, "unroll=%u", &v) == 1 && (v == 2 || v == 4 || v == 8))
                    r.unroll = v;
                else if (sscanf(tok, "pf=%u", &v) == 1) r.pf = v ? 1 : 0;
                else if (sscanf(tok, "bal=%u", &v) == 1) r.bal = v ? 1 : 0;
                else if (sscanf(tok, "wfloor=%u", &v) == 1 && v <= 2) r.wfloor = v;
                else if (sscanf(tok, "waves=%u", &v) == 1 && (v == 2 || v == 8)) r.waves = v;
            }
        }
        return r;
    }();
    return t;
}

// Defaults by row size (head_dim) and by call kind: one sequence (host
// current_pos), a batch with per-sequence lengths, a paged batch, or one
// sequence streaming a single tensor per position (the page's two
// dispatches: V alone for softmax.V, K alone for the scores), which needs
// double buffering to keep as many bytes in flight.  The scores pass has its
// own row: it writes as it reads, and its best head blocking and unroll
// differ.
// A single sequence of head_dim > 64 that streams at most kShortSpan
// positions takes one head per workgroup: with so few positions per chunk
// the narrower head block wins (4096 positions: 16.5 against 18.6 us; 8192:
// 27.2 against 27.9; from 16384 on it loses).
// A decode step over more positions than that, with 256-byte rows (head_dim
// 128), wants one workgroup per CU (32 heads x 32768 positions: 83.4
// against 87.5 us with two; 64 x 16384: 88.9 against 94.9); at head_dim 192
// it loses (82.4 against 73.2 us), and head_dim 256 does as well on its own
// row.  The plain decode takes one per CU only in the instantiation bounded
// to two waves per SIMD, which plan_split picks for it at head_dim 128.
// A single sequence short enough that one workgroup per head block streams
// its whole span in about the time a combine launch costs (<= 256 KiB of K+V
// per workgroup) takes one chunk per head block, double-buffered so that its
// blocks' loads are in flight together: the split launch then writes the
// output itself (4 heads x 101 positions: 3.7 us with the cache in the
// caches, 4.9 us from DRAM, against 9.0 us for 16-position chunks and a
// combine).
// A batch (device lengths, contiguous or paged) whose capacity is that short
// for one 256-byte head block takes the same plan: one chunk per sequence and
// head block on the chunked grid, written out directly.  The balanced grid's
// workgroups walk many short pieces one after another there, each with its
// own query load and partial, and a combine follows (64 sequences x 32 heads
// x 128 positions: 36.5 -> 15.9 us; 1024 x 32 x 32: 161.7 -> 50.7; 2 x 8 x
// 512: 12.7 -> 4.9).  Many head blocks want wider blocks: at most
// kShortGroups workgroups (1024 x 32 heads x 32 positions: 72.5 us at 32768,
// 50.7 at 16384, 50.3 at 8192).  Up to twice that capacity the plan still
// wins for head_dim <= 128 once the workgroups cover every CU (8 x 32 x
// 1024: 27.4 -> 21.3 us; 48 x 8 x 1024: 29.4 -> 23.9); with fewer it is a
// toss-up, and at head_dim 256 it loses.  A paged cache needs more
// workgroups than CUs there: at exactly one per CU it lost 8-28% on four of
// five shapes, from 300 workgroups on it won 3-43%.
// Other batches whose caches hold at most kMidBatchBytes of K+V take the
// chunked grid aimed at 512 workgroups, with a combine: the balanced grid's
// length scan and piece walk are not repaid at that size (16 x 8 heads x
// 1024 positions: 18.7 -> 13.8 us; 4 x 32 x 1024: 19.5 -> 14.8; paged and
// decode steps alike), while from 256 MiB on it is level or ahead.
enum class Kind { single, batched, paged, stream, batched_chunked, scores, single_short, single_step,
                  single_tiny, batched_short, batched_mid };
constexpr uint32_t kShortSpan = 8192;
constexpr uint64_t kOneChunkBytes = 256u << 10;
constexpr uint64_t kShortGroups = 8192;
constexpr uint64_t kShortMinGroups = 256;   // the CU count
constexpr uint64_t kShortU8MinGroups = 128;  // from here to the CU count, one-chunk batches take U = 8
constexpr uint64_t kMidBatchBytes = 128ull << 20;
// A dispatch holds its grid size in work-items, 32 bits per dimension.
constexpr uint64_t kMaxGridItems = 0xFFFFFFFFull;

Knobs knobs(uint32_t D, Kind kind) {
    Knobs k;
    if (kind == Kind::batched || kind == Kind::paged) k = Knobs{256, 8192, 8, 4, 1, 1};
    // batches the balanced grid does not take (more than its sequences): one
    // workgroup per sequence, head block and chunk of at most 8192 positions
    // (one chunk, and one launch, up to that capacity).  Eight positions per
    // block keep more bytes in flight per workgroup (ragged 1200 x 4 x 128 x
    // 8192: 1951 -> 1597 us; 1030 x 8 x 64 x 4096: 786 -> 726); two 256-byte
    // heads per workgroup balance ragged lengths better than four (1100 x 8 x
    // 128 x 4096: 1471 -> 1386), four 128-byte ones stream faster than two
    // (1025 x 32 x 64 x 2048: 1214 with four, 1300 with two)
    else if (kind == Kind::batched_chunked) k = D <= 64 ? Knobs{256, 8192, 4, 8, 1, 0} : Knobs{256, 8192, 2, 8, 1, 0};
    // mid-size batches: two 256-byte heads per workgroup (16 x 8 heads x
    // 1024 positions: 14.2 -> 13.7 us; 2 x 32 x 4096: 21.0 -> 20.6), four
    // 128-byte ones (with two, 16 x 16 x 2048: 21.1 -> 21.4)
    else if (kind == Kind::batched_mid) k = D <= 64 ? Knobs{512, 8192, 4, 2, 1, 0} : Knobs{512, 8192, 2, 2, 1, 0};
    else if (kind == Kind::stream) k = D <= 64 ? Knobs{1024, 8192, 8, 2, 1, 0} : Knobs{1024, 8192, 2, 2, 1, 0};
    else if (kind == Kind::scores) k = D <= 64 ? Knobs{1024, 8192, 4, 2, 1, 0} : Knobs{1024, 8192, 4, 8, 1, 0};
    else if (kind == Kind::single_short && D > 64) k = Knobs{512, 8192, 1, 2, 0, 0};
    else if (kind == Kind::single_step && D > 64) k = Knobs{256, 8192, 2, 2, 1, 0};
    else if (kind == Kind::single_tiny) k = D <= 64 ? Knobs{1024, 8192, 4, 8, 1, 0} : Knobs{512, 8192, 1, 2, 1, 0};
    else if (kind == Kind::batched_short) k = D <= 64 ? Knobs{256, 8192, 2, 2, 1, 0} : Knobs{256, 8192, 1, 2, 1, 0};
    else if (D <= 64) k = Knobs{1024, 8192, 4, 8, 0, 0};               // 128-byte rows
    else if (D < 256) k = Knobs{512, 8192, 2, 2, 1, 0};                // 256- to 510-byte rows
    // 512-byte rows (head_dim 256): one head is already a 512-byte read, and
    // one head per workgroup with more workgroups beats wider blocks (16
    // heads x 32768 positions: 84.0 against 110.9 us; at head_dim 192 two
    // heads per workgroup stay better, 70.2 against 73.3 us).
    else k = Knobs{1024, 8192, 1, 2, 1, 0};
    // Head blocks on whole 128-byte cache lines: a block that ends mid-line
    // shares that line with the next head block, whose workgroup (on another
    // XCD, so another L2) fetches it again.  Rows of 64, 96, 128 or 256
    // values already fit; head_dim 80 moves from 2 heads (320 bytes) to 4
    // (640 bytes): 32 heads x 32768 positions 70.0 -> 58.5 us.
    while (k.hpb < kMaxHeadsPerWG && (k.hpb * D * 2) % 128 != 0) k.hpb <<= 1;
    const Knobs &e = env_knobs();
    if (e.wgs) k.wgs = e.wgs;
    if (e.cmax) k.cmax = e.cmax;
    if (e.hpb) k.hpb = e.hpb;
    if (e.unroll) k.unroll = e.unroll;
    if (e.pf != 2) k.pf = e.pf;
    if (e.bal != 2) k.bal = e.bal;
    if (e.wfloor != 3) k.wfloor = e.wfloor;
    if (e.waves) k.waves = e.waves == 2 ? 2 : 0;
    return k;
}

uint32_t pow2ceil(uint32_t x) {
    uint32_t r = 1;
    while (r < x) r <<= 1;
    return r;
}

// Lane layout of one cache row: VEC fp16 values per load, GL lanes per row
// (power of two, >= 8), NV loads per lane.
struct Layout {
    int vec, gl, nv;
    bool full;
};

Layout choose_layout(uint32_t D, const void *q, const void *k, const void *v) {
    int vec = 1;
    for (int c : {8, 4, 2}) {
        const uintptr_t bytes = 2u * c;
        if (D % c == 0 && aligned(q, bytes) && aligned(k, bytes) && aligned(v, bytes)) {
            vec = c;
            break;
        }
    }
    const uint32_t nvec = D / vec;
    uint32_t gl = pow2ceil(nvec);
    if (gl > 64) gl = 64;
    if (gl < 8) gl = 8;
    const uint32_t nv = (uint32_t)cdiv(nvec, gl);
    // only the 16-byte layouts have guard-free instantiations
    Layout L{vec, (int)gl, (int)nv, vec == 8 && (uint32_t)(vec * gl * nv) == D};
    return L;
}

// Heads per workgroup: the largest power of two <= the request that divides
// H and fits the layout's row groups.
uint32_t heads_per_wg(uint32_t H, const Layout &ly, uint32_t want) {
    const uint32_t ng = kWaves * (64 / ly.gl);
    uint32_t hpb = 1;
    for (uint32_t c = 1; c <= want && c <= ng && c <= H; c <<= 1)
        if (H % c == 0) hpb = c;
    return hpb;
}

struct Plan {
    uint32_t chunk;       // positions per workgroup
    uint32_t n_chunks;    // chunks launched per (sequence, head block)
    uint32_t nc_stride;   // chunk stride in the workspace (an upper bound)
};

// Chunk count bound of one knob set for the workspace layout.
uint32_t chunk_bound_for(const Knobs &k, uint32_t batch, uint32_t H, uint32_t S) {
    const uint64_t nhb_min = cdiv(H, kMaxHeadsPerWG);
    const uint64_t nt = cdiv(k.wgs, (uint64_t)batch * nhb_min);
    const uint64_t hi = nt > cdiv(S, k.cmax) ? nt : cdiv(S, k.cmax);
    const uint64_t lo = cdiv(S, kChunkGranule);
    return (uint32_t)(hi < lo ? hi : lo);
}

// Workspace chunk stride: covers single-sequence and batched plans, so it
// depends on sizes only.
uint32_t chunk_bound(uint32_t batch, uint32_t H, uint32_t D, uint32_t S) {
    uint32_t m = 0;
    for (Kind kd : {Kind::single, Kind::single_short, Kind::single_step, Kind::single_tiny, Kind::batched,
                    Kind::paged, Kind::stream, Kind::batched_chunked, Kind::batched_short,
                    Kind::batched_mid}) {
        const uint32_t c = chunk_bound_for(knobs(D, kd), batch, H, S);
        if (c > m) m = c;
    }
    return m;
}

// Chunk size for `span` positions.  The head blocking assumed here is the
// one of the widest-load layout for this head_dim, so the plan depends on
// sizes only (the combine launch recomputes it without the cache pointers).
Plan make_plan(uint32_t batch, uint32_t H, uint32_t D, uint32_t S, uint32_t span, Kind kind,
               const Knobs &k) {
    const Layout best = choose_layout(D, nullptr, nullptr, nullptr);
    const uint64_t n_hb = H / heads_per_wg(H, best, k.hpb);
    // Chunks per (sequence, head block): about wgs workgroups in all.  With
    // a target of at most two workgroups per CU (wgs <= 512), never more
    // than the target: a few workgroups past a multiple of the CU count put
    // a third chunk on some CUs, and the launch waits for them (40 heads x
    // 32768 positions, head_dim 128: 520 workgroups 124.5 us, 500 103.8 us).
    // With four per CU, one or two past the target cost less than the
    // longer chunks of fewer workgroups (12 heads x 65536, head_dim 64: 1026
    // workgroups 38.2 us, 948 42.1 us).
    const uint64_t per = (uint64_t)batch * n_hb;
    const bool at_most = k.wfloor == 1 || (k.wfloor == 2 && k.wgs <= 512);
    const uint64_t nt = at_most ? (k.wgs / per > 0 ? k.wgs / per : 1) : cdiv(k.wgs, per);
    uint64_t c = cdiv(cdiv(span, nt), kChunkGranule) * kChunkGranule;
    if (kind == Kind::single_tiny || kind == Kind::batched_short)   // one chunk
        c = cdiv(span, kChunkGranule) * kChunkGranule;
    if (c > k.cmax) c = k.cmax;
    if (c < kChunkGranule) c = kChunkGranule;
    Plan p;
    p.chunk = (uint32_t)c;
    p.n_chunks = (uint32_t)cdiv(span, c);
    p.nc_stride = chunk_bound(batch, H, D, S);
    return p;
}

// Workspace: [header: kHeaderBytes][o rows fp32][(m, l) pairs fp32], each region
// 256-byte aligned.  It holds whichever partial layout the split launch
// picks: chunked, B*H*nc_stride slots, or balanced, grid*hpb + B*H slots
// (per-sequence lengths, batch <= kBalancedMaxBatch).
struct WsLayout {
    size_t o_off, ml_off, total;
    size_t slots;   // partial states the workspace holds
};

size_t balanced_slots(uint32_t batch, uint32_t H, uint32_t D) {
    if (batch > kBalancedMaxBatch) return 0;
    const Layout best = choose_layout(D, nullptr, nullptr, nullptr);
    size_t m = 0;
    for (Kind kd : {Kind::single, Kind::single_short, Kind::single_step, Kind::single_tiny, Kind::batched,
                    Kind::paged, Kind::stream, Kind::batched_chunked, Kind::batched_short,
                    Kind::batched_mid}) {
        const Knobs k = knobs(D, kd);
        const size_t n = (size_t)k.wgs * heads_per_wg(H, best, k.hpb) + (size_t)batch * H;
        if (n > m) m = n;
    }
    return m;
}

WsLayout workspace_layout(uint32_t batch, uint32_t H, uint32_t D, uint32_t S) {
    size_t slots = (size_t)batch * H * chunk_bound(batch, H, D, S);
    const size_t bal = balanced_slots(batch, H, D);
    if (bal > slots) slots = bal;
    const size_t hdr = kHeaderBytes;
    const size_t o_bytes = (slots * D * sizeof(float) + 255) / 256 * 256;
    const size_t ml_bytes = (slots * 2 * sizeof(float) + 255) / 256 * 256;
    return WsLayout{hdr, hdr + o_bytes, hdr + o_bytes + ml_bytes, slots};
}

attn_status_t check_sizes(uint32_t batch, uint32_t H, uint32_t D, uint32_t S) {
    if (batch == 0 || H == 0 || D == 0 || S == 0)
        return fail(ATTN_ERR_DIM, "sizes must be nonzero (batch=%u n_heads=%u head_dim=%u seq_len=%u)",
                    batch, H, D, S);
    if (D > ATTN_MAX_HEAD_DIM)
        return fail(ATTN_ERR_DIM, "head_dim=%u exceeds %u", D, ATTN_MAX_HEAD_DIM);
    const unsigned __int128 elems = (unsigned __int128)batch * S * H * D;
    if (elems > ((unsigned __int128)1 << 60))
        return fail(ATTN_ERR_DIM, "cache of %llu x %u x %u x %u elements is too large",
                    (unsigned long long)batch, S, H, D);
    if (S > (1u << 31))
        return fail(ATTN_ERR_DIM, "seq_len=%u exceeds 2^31", S);
    if (batch > 65535u)
        return fail(ATTN_ERR_DIM, "batch=%u exceeds 65535", batch);
    if (cdiv((uint64_t)batch * H, 4) * 256 > kMaxGridItems)   // the combine's wave grid
        return fail(ATTN_ERR_DIM, "batch*n_heads=%llu exceeds %llu", (unsigned long long)batch * H,
                    (unsigned long long)(kMaxGridItems / 256 * 4));
    return ok();
}

// -------------------------------------------------------- kernel selection

using SplitFn = void (*)(SplitArgs);

template <int V, int G, int N, bool F, int U, bool PF, bool DUMP, bool PAGED, int MODE, int WAVES = 8>
SplitFn kernel_for(bool bal) {
    if constexpr (MODE == kModeQk || MODE == kModePv)   // single sequence: chunked grid
        return attn_split_kernel<V, G, N, F, U, PF, DUMP, PAGED, MODE, WAVES>;
    else
        return bal ? attn_split_balanced_kernel<V, G, N, F, U, PF, DUMP, PAGED, MODE, WAVES>
                   : attn_split_kernel<V, G, N, F, U, PF, DUMP, PAGED, MODE, WAVES>;
}

// Double-buffered blocks.  A grid of at most one workgroup per CU runs one
// wave per SIMD, but the compiler schedules for the occupancy the registers
// would allow: at U = 2 and U = 8 it moved V loads down to their use, so
// that iterations waited for all loads in flight.  Compiled for at most two
// waves per SIMD (amdgpu_waves_per_eu), it issues each block's loads a block
// ahead.  The plan asks for that instantiation (knob waves = 2) where it
// measured faster; decodes and decode steps have it.
template <int V, int G, int N, bool F, int U, bool DUMP, bool PAGED, int MODE>
SplitFn kernel_pf(const Knobs &t, bool bal) {
    if constexpr ((MODE == kModeDecode || MODE == kModeStep) && (U == 2 || U == 8))
        if (t.waves == 2) return kernel_for<V, G, N, F, U, true, DUMP, PAGED, MODE, 2>(bal);
    return kernel_for<V, G, N, F, U, true, DUMP, PAGED, MODE>(bal);
}

// Dense caches honour the unroll/prefetch knobs on the fast layouts; paged
// caches are double-buffered at U=4 and U=8, and honour the prefetch knob at
// U=2.  kernel_shape (below) restates these choices for attn_decode_plan:
// a change here changes it too.
template <int V, int G, int N, bool F, bool DUMP, bool PAGED, int MODE>
SplitFn pick_unroll(const Knobs &t, bool bal) {
    if constexpr (PAGED) {
        if (t.unroll == 8) return kernel_pf<V, G, N, F, 8, DUMP, PAGED, MODE>(t, bal);
        if (t.unroll == 4) return kernel_for<V, G, N, F, 4, true, DUMP, PAGED, MODE>(bal);
        return t.pf ? kernel_pf<V, G, N, F, 2, DUMP, PAGED, MODE>(t, bal)
                    : kernel_for<V, G, N, F, 2, false, DUMP, PAGED, MODE>(bal);
    } else {
        if (t.unroll == 2) return t.pf ? kernel_pf<V, G, N, F, 2, DUMP, PAGED, MODE>(t, bal)
                                       : kernel_for<V, G, N, F, 2, false, DUMP, PAGED, MODE>(bal);
        if (t.unroll == 8) return t.pf ? kernel_pf<V, G, N, F, 8, DUMP, PAGED, MODE>(t, bal)
                                       : kernel_for<V, G, N, F, 8, false, DUMP, PAGED, MODE>(bal);
        return t.pf ? kernel_for<V, G, N, F, 4, true, DUMP, PAGED, MODE>(bal)
                    : kernel_for<V, G, N, F, 4, false, DUMP, PAGED, MODE>(bal);
    }
}

template <bool DUMP, bool PAGED, int MODE>
SplitFn pick_split(const Layout &ly, const Knobs &k, bool bal) {
    // fast paths: head_dim 64 and 128 with 16-byte rows
    if (ly.vec == 8 && ly.nv == 1 && ly.full && ly.gl == 8) return pick_unroll<8, 8, 1, true, DUMP, PAGED, MODE>(k, bal);
    if (ly.vec == 8 && ly.nv == 1 && ly.full && ly.gl == 16) return pick_unroll<8, 16, 1, true, DUMP, PAGED, MODE>(k, bal);
#define ATTN_CASE(V, G, N, F)                                                          \
    if (ly.vec == V && ly.gl == G && ly.nv == N && ly.full == F)                       \
        return kernel_for<V, G, N, F, 4, true, DUMP, PAGED, MODE>(bal);
    ATTN_CASE(8, 32, 1, true)
    ATTN_CASE(8, 8, 1, false)
    ATTN_CASE(8, 16, 1, false)
    ATTN_CASE(8, 32, 1, false)
    ATTN_CASE(4, 8, 1, false)
    ATTN_CASE(4, 16, 1, false)
    ATTN_CASE(4, 32, 1, false)
    ATTN_CASE(4, 64, 1, false)
    ATTN_CASE(2, 8, 1, false)
    ATTN_CASE(2, 16, 1, false)
    ATTN_CASE(2, 32, 1, false)
    ATTN_CASE(2, 64, 1, false)
    ATTN_CASE(2, 64, 2, false)
    ATTN_CASE(1, 8, 1, false)
    ATTN_CASE(1, 16, 1, false)
    ATTN_CASE(1, 32, 1, false)
    ATTN_CASE(1, 64, 1, false)
    ATTN_CASE(1, 64, 2, false)
    ATTN_CASE(1, 64, 3, false)
    ATTN_CASE(1, 64, 4, false)
#undef ATTN_CASE
    return nullptr;
}

// The unroll and wave bound of the split kernel pick_split runs for these
// knobs (reported by attn_decode_plan; it follows pick_unroll, kernel_pf and
// pick_split, and changes with them): the two 16-byte layouts honour the
// unroll knob (paged caches: 2, 4 or 8; dense: 2, 4 or 8, else 4), every
// other layout runs U = 4; the two-wave instantiation exists for decodes
// and steps, double-buffered, at U = 2 and U = 8.
struct KernelShape {
    uint32_t unroll, waves;
};
KernelShape kernel_shape(const Layout &ly, const Knobs &k, bool paged, int mode) {
    const bool fast = ly.vec == 8 && ly.nv == 1 && ly.full && (ly.gl == 8 || ly.gl == 16);
    if (!fast) return {4, 8};
    const uint32_t u = paged ? (k.unroll == 8 ? 8u : k.unroll == 4 ? 4u : 2u)
                             : (k.unroll == 2 || k.unroll == 8 ? k.unroll : 4u);
    const bool pf = paged ? (u != 2 || k.pf) : k.pf != 0;
    const bool bounded = pf && (u == 2 || u == 8) && k.waves == 2 &&
                         (mode == kModeDecode || mode == kModeStep);
    return {u, bounded ? 2u : 8u};
}

// Shared argument checks of the split phase.
attn_status_t check_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const uint32_t *cp_dev, uint32_t batch, uint32_t H, uint32_t D,
                          uint32_t S, const float *dump) {
    if (!q || !k || !v) return fail(ATTN_ERR_NULL, "q, k_cache and v_cache must be non-NULL");
    attn_status_t s = check_sizes(batch, H, D, S);
    if (s != ATTN_OK) return s;
    if (!aligned(q, 2) || !aligned(k, 2) || !aligned(v, 2))
        return fail(ATTN_ERR_ALIGN, "fp16 tensors must be 2-byte aligned");
    if (dump && !aligned(dump, 4)) return fail(ATTN_ERR_ALIGN, "scores_dump must be 4-byte aligned");
    if (cp_dev && !aligned(cp_dev, 4)) return fail(ATTN_ERR_ALIGN, "current_pos must be 4-byte aligned");
    return ok();
}

attn_status_t check_workspace(const void *ws, size_t ws_bytes, uint32_t batch, uint32_t H,
                              uint32_t D, uint32_t S) {
    const size_t need = workspace_layout(batch, H, D, S).total;
    if (!ws) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(ws, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, need);
    return ok();
}

// Enqueue the split kernel (and the dump fill).  `out` non-null and a single
// chunk per sequence: the split kernel writes the final rows itself.
// A paged cache: pool pages [num_blocks, page, H, D] and a device block table.
struct Paging {
    const uint32_t *block_table;
    uint32_t max_blocks, num_blocks, page_shift;
};

// Everything a split launch decides from the sizes and the tensors' lane
// layout: the knob row, heads per workgroup, the grid and the chunking.
struct SplitPlan {
    Kind kind;
    Knobs kn;
    uint32_t hpb;
    bool bal;   // balanced grid
    Plan plan;
};

// Positions one block of a workgroup covers: its row groups per head block
// (64 / gl per wave) times U.
uint32_t block_positions(const Layout &ly, uint32_t hpb, uint32_t U) {
    return (uint32_t)(kWaves * 64 / ly.gl) / hpb * U;
}

// dev_pos: per-sequence current_pos on the device (batched or paged);
// paged: a paged cache; rope: a decode step; scores: softmax.V from stored
// scores (the second dispatch).
SplitPlan plan_split(const Layout &ly, bool dev_pos, uint32_t cp_host, bool paged, bool rope,
                     bool scores, uint32_t batch, uint32_t H, uint32_t D, uint32_t S) {
    // host current_pos: plan the exact span (a decode step streams one
    // position less; at least one chunk is launched, so the header is
    // written); device array: plan the capacity
    uint32_t span = dev_pos ? S : (cp_host < S - 1 ? cp_host : S - 1) + 1 - (rope ? 1u : 0u);
    if (span == 0) span = 1;
    Kind kind = scores ? Kind::stream : paged ? Kind::paged : dev_pos ? Kind::batched
              : (D > 64 && span <= kShortSpan) ? Kind::single_short
              : (D > 64 && D <= 128 && rope) ? Kind::single_step : Kind::single;
    if (!scores && !paged && !dev_pos) {
        const uint32_t tiny_hpb = heads_per_wg(H, choose_layout(D, nullptr, nullptr, nullptr),
                                               knobs(D, Kind::single_tiny).hpb);
        if ((uint64_t)span * tiny_hpb * D * 4 <= kOneChunkBytes) kind = Kind::single_tiny;
    }
    if (kind == Kind::batched || kind == Kind::paged) {
        const uint32_t short_hpb = heads_per_wg(H, choose_layout(D, nullptr, nullptr, nullptr),
                                                knobs(D, Kind::batched_short).hpb);
        const uint64_t wg_bytes = (uint64_t)S * short_hpb * D * 4;
        const uint64_t groups = (uint64_t)batch * (H / short_hpb);
        if (wg_bytes <= kOneChunkBytes ||
            (D <= 128 && wg_bytes <= 2 * kOneChunkBytes &&
             (paged ? groups > kShortMinGroups : groups >= kShortMinGroups)))
            kind = Kind::batched_short;
        else if ((uint64_t)batch * S * H * D * 4 <= kMidBatchBytes)
            kind = Kind::batched_mid;
    }
    Knobs kn = knobs(D, kind);
    uint32_t hpb = heads_per_wg(H, ly, kn.hpb);
    // mid-size batches (about 512 workgroups, two per CU): decodes in the
    // instantiation bounded to two waves per SIMD (ragged 1 x 32 x 8192:
    // 16.4 -> 14.8 us, paged 18.4 -> 16.4; 8 x 8 x 4096: 21.1 -> 19.6; full
    // lengths level).  Dense steps measured mixed (-0.4% to +3.7%).
    if (kind == Kind::batched_mid && !rope && env_knobs().waves == 0) kn.waves = 2;
    // Single sequences of head_dim 128 (the 16-byte layout) whose head blocks
    // are a power of two: one workgroup per CU in the bounded instantiation
    // rather than two in the unbounded one (32 heads x 20001 of 32768
    // positions: 53.6 -> 52.6 us; 8 x 131072: 83.6 -> 82.0; 16 x 16384: 28.2
    // -> 26.7).  Unbounded, 256 workgroups lost 8-17%; with six head blocks
    // (12 heads) the bounded grid lost 3-8%.
    // Single sequences of one chunk per head block at head_dim 128 (U = 2,
    // one workgroup per head): the bounded instantiation (16 heads x 512
    // positions: 11.95 -> 10.34 us; 64 x 256: 7.6 -> 7.4; 4 x 512: 11.6 ->
    // 9.8).  The step measured 2% slower with it.
    if (kind == Kind::single_tiny && !rope && D > 64 && env_knobs().waves == 0) kn.waves = 2;
    if (kind == Kind::single && !rope && ly.vec == 8 && ly.gl == 16 && ly.full && ly.nv == 1 &&
        ((H / hpb) & (H / hpb - 1)) == 0 && env_knobs().wgs == 0 && env_knobs().waves == 0) {
        kn.wgs = 256;
        kn.waves = 2;
    }
    if (kind == Kind::batched_short) {
        for (uint32_t w = hpb * 2; (uint64_t)batch * (H / hpb) > kShortGroups && w <= H; w *= 2) {
            const uint32_t h = heads_per_wg(H, ly, w);
            if (h == hpb) break;
            hpb = h;
        }
        // At most one workgroup per CU, each streaming its whole span: U = 8
        // keeps four times the bytes in flight (4 x 32 heads x 512 positions:
        // 11.2 -> 9.7 us; 128 x 2 x 512: 13.5 -> 11.4; 8 x 32 x 1024: 21.8 ->
        // 19.3).  With fewer workgroups the longer blocks cost latency (1 x
        // 32 x 256: 3.8 -> 4.4), with more they are not needed.
        const uint64_t groups = (uint64_t)batch * (H / hpb);
        if (groups >= kShortU8MinGroups && groups <= kShortMinGroups && env_knobs().unroll == 0) {
            kn.unroll = 8;
            // and, for dense decodes whose spans hold four blocks or more,
            // the instantiation bounded to two waves per SIMD (8 x 32 heads
            // x 1024 positions: 19.7 -> 18.5 us; 4 x 32 x 512: 9.70 ->
            // 9.33).  At two blocks it lost (64 x 4 x 256: 7.04 -> 7.36).
            if (!rope && !paged && S >= 4 * block_positions(ly, hpb, 8) && env_knobs().waves == 0)
                kn.waves = 2;
        }
        // Decode steps whose spans hold at most four blocks of U = 2: one
        // block at a time (the rotation prologue and two register blocks
        // cost occupancy that many small workgroups need: 256 x 32 heads x
        // 64 positions 43.6 -> 37.3 us, paged 47.8 -> 41.8; 1024 x 32 x 32
        // 77.9 -> 66.7; 64 x 32 x 128 21.1 -> 18.7); at eight blocks double
        // buffering wins (16 x 32 x 256: 12.0 against 12.8, paged 13.9
        // against 17.3).  Decodes keep it (paged ones lost 3-12% without).
        if (rope && kn.unroll == 2 && S <= 4 * block_positions(ly, hpb, 2) && env_knobs().pf == 2)
            kn.pf = 0;
    }
    // balanced grid: its 64-bit range arithmetic needs n_hb*batch*S*grid < 2^63
    const bool bal = !scores && kn.bal && batch <= kBalancedMaxBatch &&
                     (unsigned __int128)(H / hpb) * batch * S * kn.wgs < ((unsigned __int128)1 << 63);
    // Dense head_dim 65-128 on the balanced grid with fewer than four head
    // blocks: four heads per workgroup where that makes four blocks (16
    // heads), so that the next rule applies (32 x 16 heads x 16384
    // positions: 351 -> 346 us, full 642 -> 621; steps 356 -> 351).  At 32
    // heads four per workgroup lost (the 64 x 32 x 8192 ragged batch: 607 ->
    // 615 us).
    if (bal && kind == Kind::batched && D > 64 && D <= 128 && H / hpb < 4 && env_knobs().hpb == 0) {
        const uint32_t h4 = heads_per_wg(H, ly, hpb / 2);
        if (h4 >= 4 && H / h4 >= 4 &&
            (unsigned __int128)(H / h4) * batch * S * kn.wgs < ((unsigned __int128)1 << 63))
            hpb = h4;
    }
    // Dense decodes and steps on the balanced grid, at least 16 sequences of
    // at least four head blocks: two positions per block, in the
    // instantiation bounded to two waves per SIMD (64 x 32 heads x 8192
    // positions, ragged: 636 -> 625 us, step 646 -> 638; 48 x 32 x 8192: 477
    // -> 465; 32 x 32 x 16384 at head_dim 64: 345 -> 339).  With one or two
    // head blocks (8 or 16 heads) it lost up to 4% (32 x 16 x 16384: 356 ->
    // 369), with 4-8 sequences it gained nothing or lost (8 x 64 x 32768: 789
    // -> 801).  Paged caches keep four (at two: paged 2-3% slower, the paged
    // step 4-10%).
    if (bal && kind == Kind::batched && batch >= 16 && H / hpb >= 4 && env_knobs().unroll == 0) {
        kn.unroll = 2;
        if (env_knobs().waves == 0) kn.waves = 2;
    }
    if (!bal && (kind == Kind::batched || kind == Kind::paged)) {   // a batch on the chunked grid
        kind = Kind::batched_chunked;
        kn = knobs(D, kind);
        hpb = heads_per_wg(H, ly, kn.hpb);
        // the instantiation bounded to two waves per SIMD where a chunk holds
        // four blocks or more (1030 x 8 x 64 x 4096: 718 -> 703 us, paged
        // 728 -> 713, decode step 698 -> 684; 1200 x 4 x 128 x 8192: 1616
        // -> 1581)
        if ((S < kn.cmax ? S : kn.cmax) >= 4 * block_positions(ly, hpb, kn.unroll) &&
            env_knobs().waves == 0)
            kn.waves = 2;
    }
    return SplitPlan{kind, kn, hpb, bal, make_plan(batch, H, D, S, span, kind, kn)};
}

attn_status_t launch_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const uint32_t *cp_dev, uint32_t cp_host, uint32_t batch, uint32_t H,
                           uint32_t D, uint32_t S, float *dump, void *ws, uint16_t *out,
                           const Paging *pg, hipStream_t stream, bool *wrote_out,
                           const uint16_t *scores_in = nullptr, const RopeArgs *rope = nullptr) {
    const Layout ly = scores_in ? choose_layout(D, v, v, v) : choose_layout(D, q, k, v);
    const SplitPlan sp = plan_split(ly, cp_dev != nullptr, cp_host, pg != nullptr, rope != nullptr,
                                    scores_in != nullptr, batch, H, D, S);
    const Knobs &kn = sp.kn;
    const uint32_t hpb = sp.hpb;
    const bool bal = sp.bal;
    const Plan &plan = sp.plan;
    const uint64_t grid_x = bal ? kn.wgs : (uint64_t)(H / hpb) * plan.n_chunks;
    if (grid_x * kThreads > kMaxGridItems)
        return fail(ATTN_ERR_DIM, "%llu workgroups per sequence exceed the dispatch limit of %llu",
                    (unsigned long long)grid_x, (unsigned long long)(kMaxGridItems / kThreads));
    const SplitFn fn =
        scores_in ? pick_split<false, false, kModePv>(ly, kn, false)
        : rope    ? (pg ? pick_split<false, true, kModeStep>(ly, kn, bal)
                        : pick_split<false, false, kModeStep>(ly, kn, bal))
        : pg ? (dump ? pick_split<true, true, kModeDecode>(ly, kn, bal)
                     : pick_split<false, true, kModeDecode>(ly, kn, bal))
             : (dump ? pick_split<true, false, kModeDecode>(ly, kn, bal)
                     : pick_split<false, false, kModeDecode>(ly, kn, bal));
    if (!fn) return fail(ATTN_ERR_DIM, "no kernel for head_dim=%u", D);
    const WsLayout wl = workspace_layout(batch, H, D, S);

    SplitArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.cp_dev = cp_dev;
    a.cp_host = cp_host;
    a.H = H;
    a.D = D;
    a.S = S;
    a.chunk = plan.chunk;
    a.n_hb = H / hpb;
    a.hpb = hpb;
    a.nc_stride = plan.nc_stride;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    a.scale = (float)(1.0 / sqrt((double)D));
    a.header = static_cast<uint32_t *>(ws);
    a.part_o = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.o_off);
    a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.ml_off);
    a.direct = (!bal && out && plan.n_chunks == 1) ? 1 : 0;
    a.out = out;
    a.dump = dump;
    a.batch = batch;
    a.grid = bal ? kn.wgs : 0;
    a.scores_in = scores_in;
    a.scores_out = nullptr;
    a.block_table = pg ? pg->block_table : nullptr;
    a.max_blocks = pg ? pg->max_blocks : 0;
    a.num_blocks = pg ? pg->num_blocks : 0;
    a.page_shift = pg ? pg->page_shift : 0;
    a.rope = rope ? *rope : RopeArgs{};
    *wrote_out = a.direct != 0;

    if (dump) {
        const uint64_t total = (uint64_t)batch * H * S;
        const uint64_t blocks = cdiv(total, 256) < 4096 ? cdiv(total, 256) : 4096;
        hipLaunchKernelGGL(attn_dump_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           dump, cp_dev, cp_host, H, S, total);
        attn_status_t s = hip_check("dump fill launch");
        if (s != ATTN_OK) return s;
    }
    const dim3 grid = bal ? dim3(a.grid) : dim3(a.n_hb * plan.n_chunks, batch);
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), 0, stream, a);
    return hip_check("split kernel launch");
}

attn_status_t launch_combine(uint16_t *out, const uint32_t *cp_dev, uint32_t cp_host,
                             uint32_t batch, uint32_t H, uint32_t D, uint32_t S, const void *ws,
                             hipStream_t stream, const RopeArgs *rope = nullptr,
                             const uint16_t *q = nullptr, const Paging *pg = nullptr) {
    const WsLayout wl = workspace_layout(batch, H, D, S);
    CombineArgs c;
    c.header = static_cast<const uint32_t *>(ws);
    c.part_o = reinterpret_cast<const float *>(static_cast<const char *>(ws) + wl.o_off);
    c.part_ml = reinterpret_cast<const float *>(static_cast<const char *>(ws) + wl.ml_off);
    c.cp_dev = cp_dev;
    c.cp_host = cp_host;
    c.H = H;
    c.D = D;
    c.S = S;
    c.batch = batch;
    c.out = out;
    c.q = q;
    c.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    c.rope = rope ? *rope : RopeArgs{};
    c.block_table = pg ? pg->block_table : nullptr;
    c.max_blocks = pg ? pg->max_blocks : 0;
    c.num_blocks = pg ? pg->num_blocks : 0;
    c.page_shift = pg ? pg->page_shift : 0;
    const uint64_t pairs = (uint64_t)batch * H;
    const dim3 grid(H, batch);
    const dim3 wave_grid((unsigned)cdiv(pairs, 4));
    if (pairs < kCombineWide) {   // few pairs, possibly many partials each
        if (rope) hipLaunchKernelGGL((attn_combine_kernel<1024, true>), grid, dim3(1024), 0, stream, c);
        else hipLaunchKernelGGL((attn_combine_kernel<1024, false>), grid, dim3(1024), 0, stream, c);
    } else if (pairs < kCombineWave) {
        if (rope) hipLaunchKernelGGL((attn_combine_kernel<256, true>), grid, dim3(256), 0, stream, c);
        else hipLaunchKernelGGL((attn_combine_kernel<256, false>), grid, dim3(256), 0, stream, c);
    } else {                      // many pairs, a few partials each
        if (rope) hipLaunchKernelGGL((attn_combine_wave_kernel<true>), wave_grid, dim3(256), 0, stream, c);
        else hipLaunchKernelGGL((attn_combine_wave_kernel<false>), wave_grid, dim3(256), 0, stream, c);
    }
    return hip_check("combine kernel launch");
}

// Rotation parameters: the frequencies base^(-2i/dims) in fp64; no pointers.
void fill_rope(RopeArgs *r, uint32_t dims, double base, int traditional) {
    memset(r, 0, sizeof *r);
    r->dims = dims;
    r->traditional = traditional ? 1u : 0u;
    for (uint32_t i = 0; i < dims / 2; ++i) r->theta[i] = pow(base, -(2.0 * i) / (double)dims);
}

// One decode step: rotate q and k_new at pos = min(current_pos, S - 1),
// stream positions 0..pos-1 (split launch), then merge them with the new
// token and append its k and v rows at slot pos (combine launch).  When the
// plan gives each head block one chunk, the split launch does the merge and
// the append itself, and the step is one launch.
attn_status_t decode_step(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                          uint16_t *k_cache, uint16_t *v_cache, uint16_t *out,
                          const uint32_t *cp_dev, uint32_t cp_host, uint32_t batch, uint32_t H,
                          uint32_t D, uint32_t S, uint32_t dims, double base, int traditional,
                          void *ws, size_t ws_bytes, void *stream, const Paging *pg = nullptr) {
    attn_status_t s = check_split(q, k_cache, v_cache, cp_dev, batch, H, D, S, nullptr);
    if (s != ATTN_OK) return s;
    if (!k_new || !v_new || !out) return fail(ATTN_ERR_NULL, "k_new, v_new and out must be non-NULL");
    if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(out, 2))
        return fail(ATTN_ERR_ALIGN, "fp16 tensors must be 2-byte aligned");
    if ((dims & 1u) || dims > D)
        return fail(ATTN_ERR_DIM, "rope_dims=%u must be even and <= head_dim=%u", dims, D);
    if (!(base > 0.0) || !isfinite(base))
        return fail(ATTN_ERR_DIM, "rope_base must be positive and finite");
    if (!cp_dev && cp_host >= S)
        return fail(ATTN_ERR_DIM, "current_pos=%u must be < seq_len=%u (the new token's slot)", cp_host, S);
    s = check_workspace(ws, ws_bytes, batch, H, D, S);
    if (s != ATTN_OK) return s;
    RopeArgs r;
    fill_rope(&r, dims, base, traditional);
    r.k_new = k_new;
    r.v_new = v_new;
    r.k_cache = k_cache;
    r.v_cache = v_cache;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool wrote = false;
    s = launch_split(q, k_cache, v_cache, cp_dev, cp_host, batch, H, D, S, nullptr, ws, out,
                     pg, st, &wrote, nullptr, &r);
    if (s != ATTN_OK || wrote) return s;   // one chunk per head block: the split launch did it all
    return launch_combine(out, cp_dev, cp_host, batch, H, D, S, ws, st, &r, q, pg);
}

attn_status_t decode_full(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                          const uint32_t *cp_dev, uint32_t cp_host, uint32_t batch, uint32_t H,
                          uint32_t D, uint32_t S, float *dump, void *ws, size_t ws_bytes,
                          const Paging *pg, void *stream) {
    attn_status_t s = check_split(q, k, v, cp_dev, batch, H, D, S, dump);
    if (s != ATTN_OK) return s;
    if (!out) return fail(ATTN_ERR_NULL, "out must be non-NULL");
    if (!aligned(out, 2)) return fail(ATTN_ERR_ALIGN, "out must be 2-byte aligned");
    s = check_workspace(ws, ws_bytes, batch, H, D, S);
    if (s != ATTN_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool wrote = false;
    s = launch_split(q, k, v, cp_dev, cp_host, batch, H, D, S, dump, ws, out, pg, st, &wrote);
    if (s != ATTN_OK || wrote) return s;
    return launch_combine(out, cp_dev, cp_host, batch, H, D, S, ws, st);
}

// Checks of a paged cache's description; fills `pg` and the capacity.
attn_status_t check_paging(const uint32_t *block_table, const uint32_t *cp_dev, uint32_t batch,
                           uint32_t H, uint32_t D, uint32_t page_size, uint32_t max_blocks,
                           uint32_t num_blocks, Paging *pg, uint32_t *capacity) {
    if (!block_table || !cp_dev)
        return fail(ATTN_ERR_NULL, "block_table and current_pos must be non-NULL");
    if (!aligned(block_table, 4)) return fail(ATTN_ERR_ALIGN, "block_table must be 4-byte aligned");
    if (page_size == 0 || (page_size & (page_size - 1)) || page_size > 65536u)
        return fail(ATTN_ERR_DIM, "page_size=%u must be a power of two <= 65536", page_size);
    if (max_blocks == 0 || num_blocks == 0)
        return fail(ATTN_ERR_DIM, "max_blocks and num_blocks must be nonzero");
    const uint64_t cap = (uint64_t)max_blocks * page_size;
    if (cap > (1ull << 31)) return fail(ATTN_ERR_DIM, "max_blocks*page_size exceeds 2^31");
    const unsigned __int128 pool = (unsigned __int128)num_blocks * page_size * H * D;
    if (pool > ((unsigned __int128)1 << 60)) return fail(ATTN_ERR_DIM, "page pool too large");
    if ((uint64_t)batch * max_blocks > (1ull << 40)) return fail(ATTN_ERR_DIM, "block table too large");
    uint32_t shift = 0;
    while ((1u << shift) < page_size) ++shift;
    *pg = Paging{block_table, max_blocks, num_blocks, shift};
    *capacity = (uint32_t)cap;
    return ok();
}

}  // namespace

// ------------------------------------------------- allocation-free calls
// The workspace of attn_decode_f16_batched_noalloc: a fixed array on every
// GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (in host code it stands in for the
// symbol, not for a device address): it looks up the device address once per
// device with hipGetSymbolAddress and passes that.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch`, per device

// The current device's `scratch`, looked up on its first use there.  A
// stream of another device is refused: its kernels would be handed this
// device's address.
attn_status_t scratch_of_current_device(void **ptr, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(ATTN_ERR_HIP, "device %d is past the %d the library keeps scratch for", dev,
                    kMaxScratchDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(ATTN_ERR_DIM, "the stream belongs to device %d, the current device is %d", sdev,
                        dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

// ============================================================== C ABI

extern "C" {

size_t attn_decode_workspace_bytes(uint32_t batch, uint32_t n_heads, uint32_t head_dim,
                                   uint32_t seq_len) {
    if (check_sizes(batch, n_heads, head_dim, seq_len) != ATTN_OK) return 0;
    return workspace_layout(batch, n_heads, head_dim, seq_len).total;
}

attn_status_t attn_decode_plan(uint32_t batch, uint32_t n_heads, uint32_t head_dim,
                               uint32_t seq_len, uint32_t current_pos, uint32_t flags,
                               attn_plan_info *info) {
    if (!info) return fail(ATTN_ERR_NULL, "info must be non-NULL");
    attn_status_t s = check_sizes(batch, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    if (flags & ~(ATTN_PLAN_DEVICE_POS | ATTN_PLAN_PAGED | ATTN_PLAN_STEP | ATTN_PLAN_FROM_SCORES))
        return fail(ATTN_ERR_DIM, "unknown plan flags 0x%x", flags);
    const bool paged = flags & ATTN_PLAN_PAGED;
    const bool dev_pos = paged || (flags & ATTN_PLAN_DEVICE_POS);
    const bool step = flags & ATTN_PLAN_STEP;
    const bool scores = flags & ATTN_PLAN_FROM_SCORES;
    if (scores && (dev_pos || step || batch != 1))
        return fail(ATTN_ERR_DIM, "softmax.V from stored scores is a single-sequence call");
    if (step && !dev_pos && current_pos >= seq_len)
        return fail(ATTN_ERR_DIM, "current_pos=%u must be < seq_len=%u (the new token's slot)",
                    current_pos, seq_len);
    const Layout ly = choose_layout(head_dim, nullptr, nullptr, nullptr);
    const SplitPlan sp = plan_split(ly, dev_pos, current_pos, paged, step, scores, batch, n_heads,
                                    head_dim, seq_len);
    const uint64_t n_hb = n_heads / sp.hpb;
    const uint64_t grid_x = sp.bal ? sp.kn.wgs : n_hb * sp.plan.n_chunks;
    if (grid_x * kThreads > kMaxGridItems)
        return fail(ATTN_ERR_DIM, "%llu workgroups per sequence exceed the dispatch limit of %llu",
                    (unsigned long long)grid_x, (unsigned long long)(kMaxGridItems / kThreads));
    // one launch: a one-call entry point (a batch with one host current_pos
    // exists only as the split / combine pair) whose plan has one chunk
    const bool direct = !sp.bal && sp.plan.n_chunks == 1 && (dev_pos || batch == 1);
    info->balanced = sp.bal ? 1u : 0u;
    info->heads_per_workgroup = sp.hpb;
    info->workgroups = sp.bal ? (uint64_t)sp.kn.wgs : grid_x * batch;
    info->chunk = sp.bal ? 0u : sp.plan.chunk;
    info->chunks = sp.bal ? 0u : sp.plan.n_chunks;
    info->launches = direct ? 1u : 2u;
    // one past the highest partial slot the split launch writes: balanced,
    // (w + segment) * hpb + head for w < grid; chunked, (b*H + h) * stride + c
    info->partial_slots = direct ? 0
                        : sp.bal ? ((uint64_t)sp.kn.wgs + (uint64_t)batch * n_hb - 1) * sp.hpb
                                 : ((uint64_t)batch * n_heads - 1) * sp.plan.nc_stride + sp.plan.n_chunks;
    info->workspace_slots = workspace_layout(batch, n_heads, head_dim, seq_len).slots;
    const KernelShape ks = kernel_shape(ly, sp.kn, paged, scores ? kModePv : step ? kModeStep : kModeDecode);
    info->unroll = ks.unroll;
    info->max_waves = ks.waves;
    return ok();
}

attn_status_t attn_decode_f16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                              uint16_t *out, uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                              uint32_t current_pos, float *scores_dump, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return decode_full(q, k_cache, v_cache, out, nullptr, current_pos, 1, n_heads, head_dim,
                       seq_len, scores_dump, workspace, workspace_bytes, nullptr, stream);
}

attn_status_t attn_decode_f16_batched(const uint16_t *q, const uint16_t *k_cache,
                                      const uint16_t *v_cache, uint16_t *out,
                                      const uint32_t *current_pos, uint32_t batch,
                                      uint32_t n_heads, uint32_t head_dim, uint32_t capacity,
                                      float *scores_dump, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    if (!current_pos) return fail(ATTN_ERR_NULL, "current_pos must be non-NULL");
    return decode_full(q, k_cache, v_cache, out, current_pos, 0, batch, n_heads, head_dim,
                       capacity, scores_dump, workspace, workspace_bytes, nullptr, stream);
}

attn_status_t attn_decode_f16_batched_noalloc(const uint16_t *q, const uint16_t *k_cache,
                                              const uint16_t *v_cache, uint16_t *out,
                                              const uint32_t *current_pos, uint32_t batch,
                                              uint32_t n_heads, uint32_t head_dim,
                                              uint32_t capacity, float *scores_dump,
                                              void *stream) {
    // every argument check before the first HIP call, as elsewhere
    if (!current_pos) return fail(ATTN_ERR_NULL, "current_pos must be non-NULL");
    attn_status_t s = check_split(q, k_cache, v_cache, current_pos, batch, n_heads, head_dim,
                                  capacity, scores_dump);
    if (s != ATTN_OK) return s;
    if (!out) return fail(ATTN_ERR_NULL, "out must be non-NULL");
    if (!aligned(out, 2)) return fail(ATTN_ERR_ALIGN, "out must be 2-byte aligned");
    const size_t need = workspace_layout(batch, n_heads, head_dim, capacity).total;
    if (need > ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_WORKSPACE,
                    "these sizes need %zu bytes of workspace; the allocation-free call holds %zu",
                    need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    s = scratch_of_current_device(&ws, static_cast<hipStream_t>(stream));
    if (s != ATTN_OK) return s;
    return decode_full(q, k_cache, v_cache, out, current_pos, 0, batch, n_heads, head_dim,
                       capacity, scores_dump, ws, ATTN_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}

attn_status_t attn_decode_f16_split(const uint16_t *q, const uint16_t *k_cache,
                                    const uint16_t *v_cache, const uint32_t *current_pos_dev,
                                    uint32_t current_pos, uint32_t batch, uint32_t n_heads,
                                    uint32_t head_dim, uint32_t seq_len, float *scores_dump,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    attn_status_t s = check_split(q, k_cache, v_cache, current_pos_dev, batch, n_heads, head_dim,
                                  seq_len, scores_dump);
    if (s != ATTN_OK) return s;
    s = check_workspace(workspace, workspace_bytes, batch, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    bool wrote = false;
    return launch_split(q, k_cache, v_cache, current_pos_dev, current_pos, batch, n_heads,
                        head_dim, seq_len, scores_dump, workspace, nullptr, nullptr,
                        static_cast<hipStream_t>(stream), &wrote);
}

attn_status_t attn_decode_f16_combine(uint16_t *out, const uint32_t *current_pos_dev,
                                      uint32_t current_pos, uint32_t batch, uint32_t n_heads,
                                      uint32_t head_dim, uint32_t seq_len, const void *workspace,
                                      size_t workspace_bytes, void *stream) {
    if (!out) return fail(ATTN_ERR_NULL, "out must be non-NULL");
    attn_status_t s = check_sizes(batch, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    if (!aligned(out, 2)) return fail(ATTN_ERR_ALIGN, "out must be 2-byte aligned");
    if (current_pos_dev && !aligned(current_pos_dev, 4))
        return fail(ATTN_ERR_ALIGN, "current_pos must be 4-byte aligned");
    s = check_workspace(workspace, workspace_bytes, batch, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    return launch_combine(out, current_pos_dev, current_pos, batch, n_heads, head_dim, seq_len,
                          workspace, static_cast<hipStream_t>(stream));
}

attn_status_t attn_decode_f16_paged(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    uint16_t *out, const uint32_t *block_table,
                                    const uint32_t *current_pos, uint32_t batch, uint32_t n_heads,
                                    uint32_t head_dim, uint32_t page_size, uint32_t max_blocks,
                                    uint32_t num_blocks, float *scores_dump, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    attn_status_t s = check_sizes(batch, n_heads, head_dim, 1);
    if (s != ATTN_OK) return s;
    Paging pg;
    uint32_t cap = 0;
    s = check_paging(block_table, current_pos, batch, n_heads, head_dim, page_size, max_blocks,
                     num_blocks, &pg, &cap);
    if (s != ATTN_OK) return s;
    return decode_full(q, k_pool, v_pool, out, current_pos, 0, batch, n_heads, head_dim, cap,
                       scores_dump, workspace, workspace_bytes, &pg, stream);
}

attn_status_t attn_decode_f16_paged_split(const uint16_t *q, const uint16_t *k_pool,
                                          const uint16_t *v_pool, const uint32_t *block_table,
                                          const uint32_t *current_pos, uint32_t batch,
                                          uint32_t n_heads, uint32_t head_dim, uint32_t page_size,
                                          uint32_t max_blocks, uint32_t num_blocks,
                                          float *scores_dump, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    attn_status_t s = check_sizes(batch, n_heads, head_dim, 1);
    if (s != ATTN_OK) return s;
    Paging pg;
    uint32_t cap = 0;
    s = check_paging(block_table, current_pos, batch, n_heads, head_dim, page_size, max_blocks,
                     num_blocks, &pg, &cap);
    if (s != ATTN_OK) return s;
    s = check_split(q, k_pool, v_pool, current_pos, batch, n_heads, head_dim, cap, scores_dump);
    if (s != ATTN_OK) return s;
    s = check_workspace(workspace, workspace_bytes, batch, n_heads, head_dim, cap);
    if (s != ATTN_OK) return s;
    bool wrote = false;
    return launch_split(q, k_pool, v_pool, current_pos, 0, batch, n_heads, head_dim, cap,
                        scores_dump, workspace, nullptr, &pg, static_cast<hipStream_t>(stream),
                        &wrote);
}

attn_status_t attn_qk_f16(const uint16_t *q, const uint16_t *k_cache, uint16_t *scores,
                          uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                          uint32_t current_pos, void *stream) {
    if (!q || !k_cache || !scores) return fail(ATTN_ERR_NULL, "q, k_cache and scores must be non-NULL");
    attn_status_t s = check_sizes(1, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    if (!aligned(q, 2) || !aligned(k_cache, 2) || !aligned(scores, 2))
        return fail(ATTN_ERR_ALIGN, "fp16 tensors must be 2-byte aligned");
    const Layout ly = choose_layout(head_dim, q, k_cache, k_cache);
    const Knobs kn = knobs(head_dim, Kind::scores);
    const SplitFn fn = pick_split<false, false, kModeQk>(ly, kn, false);
    if (!fn) return fail(ATTN_ERR_DIM, "no kernel for head_dim=%u", head_dim);
    const uint32_t hpb = heads_per_wg(n_heads, ly, kn.hpb);
    // the reading grid covers positions 0..current_pos; a few more
    // workgroups write -inf over the rest
    const uint32_t L = (current_pos < seq_len - 1 ? current_pos : seq_len - 1) + 1;
    const Plan plan = make_plan(1, n_heads, head_dim, seq_len, L, Kind::scores, kn);
    SplitArgs a = {};
    a.q = q;
    a.k = k_cache;
    a.cp_host = current_pos;
    a.H = n_heads;
    a.D = head_dim;
    a.S = seq_len;
    a.chunk = plan.chunk;
    a.n_hb = n_heads / hpb;
    a.hpb = hpb;
    a.scale = (float)(1.0 / sqrt((double)head_dim));
    a.scores_out = scores;
    a.batch = 1;
    const uint64_t masked = (uint64_t)(seq_len - L) * n_heads;
    const uint64_t fill = masked ? cdiv(masked, (uint64_t)kThreads * 16) : 0;
    const uint32_t n_fill = (uint32_t)(fill < 1024 ? fill : 1024);
    const uint64_t grid_x = (uint64_t)a.n_hb * plan.n_chunks;
    if ((grid_x + n_fill) * kThreads > kMaxGridItems)
        return fail(ATTN_ERR_DIM, "%llu workgroups exceed the dispatch limit of %llu",
                    (unsigned long long)(grid_x + n_fill), (unsigned long long)(kMaxGridItems / kThreads));
    a.grid = (uint32_t)grid_x;
    hipLaunchKernelGGL(fn, dim3(a.grid + n_fill), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return hip_check("score kernel launch");
}

attn_status_t attn_pv_f16(const uint16_t *scores, const uint16_t *v_cache, uint16_t *out,
                          uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                          uint32_t current_pos, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (!scores || !v_cache || !out)
        return fail(ATTN_ERR_NULL, "scores, v_cache and out must be non-NULL");
    attn_status_t s = check_sizes(1, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    if (!aligned(scores, 2) || !aligned(v_cache, 2) || !aligned(out, 2))
        return fail(ATTN_ERR_ALIGN, "fp16 tensors must be 2-byte aligned");
    s = check_workspace(workspace, workspace_bytes, 1, n_heads, head_dim, seq_len);
    if (s != ATTN_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool wrote = false;
    s = launch_split(nullptr, nullptr, v_cache, nullptr, current_pos, 1, n_heads, head_dim,
                     seq_len, nullptr, workspace, out, nullptr, st, &wrote, scores);
    if (s != ATTN_OK || wrote) return s;
    return launch_combine(out, nullptr, current_pos, 1, n_heads, head_dim, seq_len, workspace, st);
}

attn_status_t attn_decode_step_f16(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                   uint16_t *k_cache, uint16_t *v_cache, uint16_t *out,
                                   uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                                   uint32_t current_pos, uint32_t rope_dims, double rope_base,
                                   int rope_traditional, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    return decode_step(q, k_new, v_new, k_cache, v_cache, out, nullptr, current_pos, 1, n_heads,
                       head_dim, seq_len, rope_dims, rope_base, rope_traditional, workspace,
                       workspace_bytes, stream);
}

attn_status_t attn_decode_step_f16_batched(const uint16_t *q, const uint16_t *k_new,
                                           const uint16_t *v_new, uint16_t *k_cache,
                                           uint16_t *v_cache, uint16_t *out,
                                           const uint32_t *current_pos, uint32_t batch,
                                           uint32_t n_heads, uint32_t head_dim, uint32_t capacity,
                                           uint32_t rope_dims, double rope_base,
                                           int rope_traditional, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    if (!current_pos) return fail(ATTN_ERR_NULL, "current_pos must be non-NULL");
    return decode_step(q, k_new, v_new, k_cache, v_cache, out, current_pos, 0, batch, n_heads,
                       head_dim, capacity, rope_dims, rope_base, rope_traditional, workspace,
                       workspace_bytes, stream);
}

attn_status_t attn_decode_step_f16_paged(const uint16_t *q, const uint16_t *k_new,
                                         const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                                         uint16_t *out, const uint32_t *block_table,
                                         const uint32_t *current_pos, uint32_t batch,
                                         uint32_t n_heads, uint32_t head_dim, uint32_t page_size,
                                         uint32_t max_blocks, uint32_t num_blocks,
                                         uint32_t rope_dims, double rope_base, int rope_traditional,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    attn_status_t s = check_sizes(batch, n_heads, head_dim, 1);
    if (s != ATTN_OK) return s;
    Paging pg;
    uint32_t cap = 0;
    s = check_paging(block_table, current_pos, batch, n_heads, head_dim, page_size, max_blocks,
                     num_blocks, &pg, &cap);
    if (s != ATTN_OK) return s;
    return decode_step(q, k_new, v_new, k_pool, v_pool, out, current_pos, 0, batch, n_heads,
                       head_dim, cap, rope_dims, rope_base, rope_traditional, workspace,
                       workspace_bytes, stream, &pg);
}

attn_status_t attn_rope_f16(const uint16_t *x, uint16_t *out, const uint32_t *positions,
                            uint32_t batch, uint32_t n_heads, uint32_t head_dim, uint32_t rope_dims,
                            double rope_base, int rope_traditional, void *stream) {
    if (!x || !out || !positions) return fail(ATTN_ERR_NULL, "x, out and positions must be non-NULL");
    attn_status_t s = check_sizes(batch, n_heads, head_dim, 1);
    if (s != ATTN_OK) return s;
    if (!aligned(x, 2) || !aligned(out, 2)) return fail(ATTN_ERR_ALIGN, "fp16 tensors must be 2-byte aligned");
    if (!aligned(positions, 4)) return fail(ATTN_ERR_ALIGN, "positions must be 4-byte aligned");
    if ((rope_dims & 1u) || rope_dims > head_dim)
        return fail(ATTN_ERR_DIM, "rope_dims=%u must be even and <= head_dim=%u", rope_dims, head_dim);
    if (!(rope_base > 0.0) || !isfinite(rope_base))
        return fail(ATTN_ERR_DIM, "rope_base must be positive and finite");
    RopeArgs r;
    fill_rope(&r, rope_dims, rope_base, rope_traditional);
    const uint64_t total = (uint64_t)batch * n_heads * head_dim;
    const uint64_t blocks = cdiv(total, 256) < 8192 ? cdiv(total, 256) : 8192;
    hipLaunchKernelGGL(attn_rope_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), x, out, positions, n_heads, head_dim,
                       total, r);
    return hip_check("rope kernel launch");
}

}  // extern "C"
