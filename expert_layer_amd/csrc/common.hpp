// common.hpp -- device types, MFMA fragments and launch helpers shared by the
// HIP kernels of the MoE layer (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Four fp32 -> OCP e4m3 codes (nearest-even, saturating at +-448), packed
// little-endian into a word: gfx950's v_cvt_pk_fp8_f32 rounds to nearest-even
// in the OCP format; finite values are first clamped to [-448, 448] (the
// instruction itself does not saturate), a NaN becomes the positive NaN code
// 0x7F, and a negative value that rounds to zero gets the code 0x00 rather
// than the instruction's negative zero 0x80.
__device__ __forceinline__ uint32_t e4m3x4_rne_sat(float a, float b, float c, float d) {
    auto prep = [](float v) { return v != v ? __builtin_nanf("") : __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(prep(a), prep(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(prep(c), prep(d), w, true);
    const uint32_t u = (uint32_t)w;
    const uint32_t mag = u & 0x7F7F7F7Fu;
    const uint32_t nonzero = (mag + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7 of a byte: its magnitude is not 0
    return mag | (u & nonzero);
}

// The tiled bf16 layout of the grouped FFN's operands: 1 KiB blocks of 16 rows
// x 32 k, block (row / 16, k / 32) at 16-byte chunk (row / 16 * KS + k / 32) * 64,
// and inside a block chunk c (8 k values) of row r at r * 4 + (c ^ tile_swz(r)).
// The XOR makes any 16 consecutive rows of one chunk column land on 16
// distinct LDS bank groups once the block is copied to LDS verbatim.
__device__ __forceinline__ int tile_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ size_t tiled_chunk(int64_t row, int chunk, int KS) {
    const int r = (int)(row & 15);
    return ((size_t)(row >> 4) * (size_t)KS + (size_t)(chunk >> 2)) * 64 + (size_t)(r * 4 + ((chunk & 3) ^ tile_swz(r)));
}

// silu(z) = z / (1 + e^-z) in fp32, the quotient through the hardware reciprocal
// (about one ulp) rather than the correctly rounded division sequence: every
// consumer rounds the product silu * u to bf16 or e4m3 or holds fp32 to 1e-4.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16: A fragment = 8 bf16 of one row (lane % 32) at
// k-half (lane / 32); B fragment = 8 bf16 of one column; C/D 16 fp32 per lane:
// column = lane % 32, row = (i / 4) * 8 + (lane / 32) * 4 + (i % 4).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 with both operands e4m3 (format code 0): A/B
// fragment = 32 e4m3 bytes of one row/column at k-half (lane / 32).
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int c_row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// Remaps a linear block id so that consecutive logical tiles run on the same
// XCD: the dispatcher hands block b to XCD b % 8, so logical tile
// L = (b % 8) * per_xcd + b / 8 keeps a contiguous run of tiles (sharing an A
// panel or a weight panel) inside one XCD's L2.  Returns -1 for idle blocks.
// Every L < n_valid is reached exactly once when the grid is a multiple of 8
// of at least n_valid blocks (then each XCD has grid / 8 >= per_xcd blocks):
// launches size their grids with xcd_grid.
__host__ __device__ __forceinline__ int xcd_remap(int b, int n_valid) {
    constexpr int kXcd = 8;
    int per = (n_valid + kXcd - 1) / kXcd;
    int x = b % kXcd, i = b / kXcd;
    if (i >= per) return -1;
    int L = x * per + i;
    return L < n_valid ? L : -1;
}
// Grid of a launch whose blocks go through xcd_remap for up to `items`
// logical tiles: `items` rounded up to a multiple of 8.
__host__ __device__ __forceinline__ int64_t xcd_grid(int64_t items) { return (items + 7) / 8 * 8; }

// The same with runs: above 256 tiles, XCD x takes runs x, x + 8, x + 16, ...
// of 32 consecutive logical tiles (up to 256, xcd_remap's even split, so a
// small launch still spreads over every XCD).  A run fills one XCD's CUs and
// shares its L2; at any time the eight XCDs work on eight neighbouring runs,
// whose common panels (the weights of one expert, the row panels of its M
// tiles) the whole chip then reads from the memory-side cache instead of HBM.
// The last, partial round of eight runs is split evenly over the XCDs, so that
// their shares differ by at most one tile.  Every L < n_valid is reached
// exactly once for a grid of xcd_grid_runs(items) blocks, n_valid <= items; -1
// for idle blocks.
__host__ __device__ __forceinline__ int xcd_remap_runs(int b, int n_valid) {
    constexpr int kXcd = 8, kRun = 32, kRound = kXcd * kRun;
    if (n_valid <= kRound) return xcd_remap(b, n_valid);
    const int x = b % kXcd, i = b / kXcd, r = i / kRun, full = n_valid / kRound;
    if (r < full) return (r * kXcd + x) * kRun + i % kRun;
    const int rem = n_valid - full * kRound, per = (rem + kXcd - 1) / kXcd, j = i - r * kRun;
    const int L = full * kRound + x * per + j;
    return r == full && j < per && L < n_valid ? L : -1;
}
__host__ __device__ __forceinline__ int64_t xcd_grid_runs(int64_t items) { return (items + 255) / 256 * 256; }

// The tiles of XCD x's share in xcd_remap_runs order: its block i = b / 8
// takes the share's i-th tile for i < xcd_share(x, n_valid).
__host__ __device__ __forceinline__ int xcd_share(int x, int n_valid) {
    constexpr int kXcd = 8, kRun = 32, kRound = kXcd * kRun;
    const bool small = n_valid <= kRound;
    const int full = small ? 0 : n_valid / kRound, rem = n_valid - full * kRound;
    const int per = (rem + kXcd - 1) / kXcd, left = rem - x * per;
    return full * kRun + (left < 0 ? 0 : (left < per ? left : per));
}

// Work queues.  The XCDs of one chip do not run equally fast (their clocks and
// their share of the memory traffic differ), so a static split of a grouped
// GEMM's work items leaves the faster XCDs idle at the end.  The grouped GEMMs
// therefore hand out the last kQueueTail tiles of each XCD's share at run
// time: block i = b / 8 of XCD x = b % 8 takes the i-th tile of its share while
// i < S = xcd_share(7, n) - kQueueTail (the smallest share less the tail; no
// atomics), and the blocks after that draw tiles S, S + 1, ... of a share from
// that share's counter -- their own XCD's first, then the other XCDs' -- so an
// XCD whose workgroups finish sooner takes more of the last tiles.  A queue is
// 8 counters and a mask of the shares found empty; the tile builder zeroes
// them.  The grid is xcd_queue_grid(items): xcd_grid_runs plus 8 kQueueTail
// blocks, which gives every XCD at least S + kQueueTail blocks, so that a fast
// XCD can take up to twice its own tail.  Each tile is taken exactly once:
// tiles below S by the one block that owns them, the others by the one counter
// value that names them.  A block makes at most nine atomic accesses, so every
// block ends.
constexpr int kQueueTail = 64;
constexpr int kQueueWords = 9;
constexpr int kQueueSets = 3;  // GEMM1, GEMM2 (routed groups or all), GEMM2 of the shared group
__host__ __device__ __forceinline__ int64_t xcd_queue_grid(int64_t items) {
    return items > 0 ? xcd_grid_runs(items) + 8 * kQueueTail : 0;
}
__host__ __device__ __forceinline__ int xcd_queue_static(int n_valid) {
    const int s = xcd_share(7, n_valid) - kQueueTail;
    return s > 0 ? s : 0;
}
// The logical tile of block b (-1: none).  Q gives the queue's three atomic
// accesses: empty() reads the mask, draw(y) takes the next value of counter y,
// mark(y) sets bit y of the mask.
template <class Q>
__host__ __device__ __forceinline__ int xcd_queue_pick(int b, int n_valid, Q& q) {
    const int x = b & 7, i = b >> 3, S = xcd_queue_static(n_valid);
    if (i < S) return xcd_remap_runs(b, n_valid);
    const int empty = q.empty();
    for (int d = 0; d < 8; ++d) {
        const int y = (x + d) & 7;
        if ((empty >> y) & 1) continue;
        const int j = q.draw(y) + S;
        if (j < xcd_share(y, n_valid)) return xcd_remap_runs(j * 8 + y, n_valid);
        q.mark(y);
    }
    return -1;
}
#if defined(__HIP__)
// A queue in device memory, used by every lane of one wave: lane 0 makes the
// accesses (device scope, so the XCDs' L2s see one counter) and the wave
// shares their results.
struct XcdQueue {
    int* c;
    bool lane0;
    __device__ int empty() {
        int e = 0;
        if (lane0) e = __hip_atomic_load(&c[8], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_amdgcn_readfirstlane(e);
    }
    __device__ int draw(int y) {
        int j = 0;
        if (lane0) j = atomicAdd(&c[y], 1);
        return __builtin_amdgcn_readfirstlane(j);
    }
    __device__ void mark(int y) {
        if (lane0) atomicOr(&c[8], 1 << y);
    }
};
// The tile of the calling workgroup: wave 0 picks it, and every thread
// returns it.  Call at the top of the kernel (it uses __syncthreads).
__device__ __forceinline__ int xcd_queue_tile(int n_valid, int* queue) {
    __shared__ int s_tile;
    if (threadIdx.x < 64) {
        XcdQueue q{queue, threadIdx.x == 0};
        const int L = xcd_queue_pick((int)blockIdx.x, n_valid, q);
        if (threadIdx.x == 0) s_tile = L;
    }
    __syncthreads();
    return s_tile;
}
#endif

}  // namespace moe

// ---------------------------------------------------------------- launchers
// Implemented in the .hip files; called by the C ABI layer (capi.cpp) after
// argument checks.  Each returns hipSuccess or the launch error.
namespace moe {

// The router writes router_splits(c) K-split partial logits [split][T][E]
// (one for fp32); route_select sums them in split order.  With x_q (bf16 x,
// H a multiple of 128) it also writes x's per-token e4m3 codes and 1 x 128
// scales (the rule of launch_quant_rows_e4m3) from the same pass over x.
int router_splits(const moe_cfg& c);
hipError_t launch_router_logits(const moe_cfg& c, const void* x, const void* w_router,
                                float* partial_logits, hipStream_t s, uint8_t* x_q = nullptr,
                                float* x_scale = nullptr);
hipError_t launch_route_select(const moe_cfg& c, const float* logits, int nsplit, const float* bias,
                               float* logits_copy, int32_t* ids, float* w, hipStream_t s);

struct PermuteWs {
    int32_t* hist;   // [nblk][E] per-block expert counts
    int32_t* base;   // [nblk][E] first row of block b's segment of expert e
};
int permute_blocks(int T);
// Layout of the permuted rows: row-major [max_rows][H], or (bf16 only) tiled
// with KS = ceil(H / 32); with shared_row0 >= 0 the tiled output also holds
// token t at row shared_row0 + t (the shared expert's operand).
struct PermuteLayout {
    int tiled;
    int64_t shared_row0;
    int payload;  // 0: the maps only (indexed layout), no x_perm
};
hipError_t launch_permute(const moe_cfg& c, const void* x, const float* x_scale, const int32_t* ids,
                          int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t* tok_row,
                          void* x_perm, float* x_perm_scale, int64_t max_rows, PermuteWs ws,
                          PermuteLayout lay, hipStream_t s);

// The allocation-free permute's scratch: a static device array of this many
// int32 (4 MiB), whose address on the current device noalloc_permute_scratch
// returns (looked up once per device).
constexpr int64_t kNoAllocPermuteInts = (int64_t)1 << 20;
hipError_t noalloc_permute_scratch(int32_t** ptr);

// bf16 rows [T][H] -> e4m3 codes [T][H] and fp32 scales [T][H / 128], one
// scale per 1 x 128 block (H a multiple of 128; x, q 16- and 8-byte aligned).
hipError_t launch_quant_rows_e4m3(const void* x, int T, int H, uint8_t* q, float* sc, hipStream_t s);
// offsets = {0, n}: one expert group covering rows [0, n) (two fill kernels,
// no memset, so the sequence can be captured in a graph).
hipError_t launch_offsets_one_group(int32_t* offsets, int n, hipStream_t s);

// Grouped FFN building blocks (gemm_bf16.hip, gemm_fp8.hip, gemm_f32.hip).
// Tile heights (rows) and the h / output columns one tile covers in GEMM1 /
// GEMM2; fp8 tiles cover the bf16 tiles' columns.
constexpr int kFfnBmBf16 = 288, kFfnN1Bf16 = 128, kFfnN2Bf16 = 256;
constexpr int kFfnBmFp8 = 224, kFfnBmFp8Small = 128, kFfnBmE4m3 = 256;
constexpr int kFfnBmF32 = 64, kFfnN1F32 = 64, kFfnN2F32 = 64;

// Device work lists of the grouped FFN, carved from the workspace.
constexpr int kFfnCtlWords = 2 + kQueueSets * kQueueWords;
struct FfnWork {
    int32_t* tiles;    // [max_tiles] x int4 {group, row_begin, row_end, 0}
    int32_t* n_tiles;  // [kFfnCtlWords]: M tiles written; of them the routed groups' (first in the
                       // list); then the kQueueSets work queues of the launches (kQueueWords each)
    int32_t* work1;    // [max_tiles * nt1] x int2 {M tile, N tile} of GEMM1
    int32_t* work2;    // [max_tiles * nt2] x int2 {M tile, N tile} of GEMM2
    int nt1, nt2;      // N tiles per M tile of GEMM1 / GEMM2
};
hipError_t launch_build_tiles(const moe_cfg& c, const int32_t* offsets, int bm, int64_t rows_cap,
                              const FfnWork& wk, hipStream_t s);
// Pointer-table weights (moe_weights.table): entry
// ((layer * row + first + g) * 6 + slot) holds group g's matrix `slot` (0 gate
// or tiled gate+up, 1 up, 2 down, 3 .. 5 their fp8 block scales) of the layer
// *layer, which the kernels read when they run.  tab == NULL: contiguous
// weights.
struct WTab {
    const void* const* tab;
    const int32_t* layer;
    int n_layers;
    int row;    // entries per layer / 6: E + has_shared of the caller's cfg
    int first;  // entry of the launch's group 0 (the shared expert's own launch: E)
};
// The layer a launch reads, or -1 when *layer is outside [0, n_layers) (the
// launch then does nothing).  Uniform: a scalar load.
__device__ __forceinline__ int wtab_layer(const WTab& t) {
    const int L = *t.layer;
    return (L >= 0 && L < t.n_layers) ? L : -1;
}
__device__ __forceinline__ const void* wtab_ptr(const WTab& t, int layer, int g, int slot) {
    return t.tab[((size_t)layer * (size_t)t.row + (size_t)(t.first + g)) * 6 + (size_t)slot];
}

// Row operands of the grouped FFN: GEMM1 inputs (routed rows, shared-expert
// tokens; row-major or tiled) and GEMM2 outputs.
struct FfnOperands {
    const void* x_rows;
    const void* x_tokens;
    int x_rows_tiled, x_tokens_tiled;
    void* y_rows;
    void* y_shared;
    const int32_t* row_src;  // non-NULL: x_rows is x [T][H], row r is token row_src[r] / k
    // comb_out non-NULL (bf16 y, a shared expert): the shared expert's GEMM2
    // also combines -- out [T][H] (cfg out_dtype) = sum_j topk_w[t][j] *
    // y_rows[tok_row[t][j]] + the shared expert's y, rounded to bf16 -- and
    // y_shared is not written
    void* comb_out;
    const int32_t* tok_row;
    const float* topk_w;
};
hipError_t launch_gemm_bf16(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const FfnOperands& op,
                            const int32_t* offsets, const moe_weights& w, const WTab& wt, const FfnWork& wk,
                            void* h_tiles, hipStream_t s);
// Bytes of one h tile slot (kFfnBmBf16 rows) of the bf16 path.
inline size_t h_slot_bytes(const moe_cfg& c) {
    const int imax = c.has_shared && c.I_shared > c.I ? c.I_shared : c.I;
    return (size_t)kFfnBmBf16 * ((imax + 31) / 32) * 32 * 2;
}
struct TiledSizes {
    size_t w13, w2, sh13, sh2;  // bytes of the tiled routed and shared matrices
};
TiledSizes tiled_sizes(const moe_cfg& c);
hipError_t launch_tile_weights(const moe_cfg& c, const moe_weights& src, void* w13, void* w2, void* sh13, void* sh2,
                               hipStream_t s);
// fp8 (e4m3) grouped FFN: x_rows [n_rows_cap][H] with x_scale [n_rows_cap][H/128]
// (row_src non-NULL: x_rows is x [T][H] and x_scale [T][H/128], row r being token
// row_src[r] / k); h [n_rows_cap][I] e4m3 and h_scale [n_rows_cap][I/128] are workspace.
hipError_t launch_gemm_fp8(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                           const float* x_scale, const int32_t* row_src, const int32_t* offsets,
                           const moe_weights& w, const WTab& wt, void* y_rows, const FfnWork& wk, void* h,
                           float* h_scale, hipStream_t s);
// The e4m3-weight path of launch_gemm_fp8 (same arguments): weights row-major
// or in the tiled e4m3 layout, streamed into registers.
hipError_t launch_gemm_e4m3(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                            const float* x_scale, const int32_t* row_src, const int32_t* offsets,
                            const moe_weights& w, const WTab& wt, void* y_rows, const FfnWork& wk, void* h,
                            float* h_scale, hipStream_t s);
hipError_t launch_tile_weights_e4m3(const moe_cfg& c, const moe_weights& src, void* w13, void* w2, void* sh13,
                                    void* sh2, hipStream_t s);
hipError_t launch_gemm_f32(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                           const int32_t* offsets, const moe_weights& w, const void* x_tokens, void* y_rows,
                           void* y_shared, const FfnWork& wk, void* h, void* h_sh, hipStream_t s);

hipError_t launch_combine(const moe_cfg& c, const void* y_rows, const int32_t* tok_row,
                          const float* topk_w, const void* y_shared, void* out, hipStream_t s);

}  // namespace moe
