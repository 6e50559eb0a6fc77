// gemm_e4m3.hip -- the grouped SwiGLU FFN on e4m3 rows and e4m3 weights with
// fp32 block scales ("ASAP", section 3.4.2: the MoE kernel is a grouped matrix
// multiplication of hidden states by the layer's expert weights; the fp8 expert
// GEMMs of the AFD page, figure 1 caption, and its W8A8 setting, section 7).
// Operands are e4m3 codes with one fp32 scale per 1 x 128 block of a row (x,
// h) and per 128 x 128 block of a weight matrix; a dequantised value is
// code * scale.
//
// Scale promotion.  A K block of 128 is exactly one
// v_mfma_scale_f32_16x16x128_f8f6f4, so every MFMA result t is the unscaled
// partial sum of one scale block and is folded in as acc += t * (s_row *
// s_weight) on the VALU (the MFMAs write VGPRs: this file is compiled in the
// VGPR form).  The weight fragment is the MFMA's first operand and the row
// fragment its second, so a 16 x 16 result comes out transposed: lane l holds
// row l % 16 and the four weight rows 4 (l / 16) + [0, 4), and one product
// s_row * s_weight serves all four.  Both operands give lane l the 32 bytes
// 32 (l / 16) + [0, 32) of the K block: the same K order on both sides, so
// the MFMA sums the same products.
//
// Tile.  Up to 256 rows x 256 weight rows, 8 waves (two per SIMD).  Wave w owns
// every row of the tile and 32 weight rows, two column blocks of 16:
//   GEMM1: the 16 gate rows and the 16 up rows of h columns 16 w .. 16 w + 15
//          of the tile's 128, so h = silu(g) * u forms in registers;
//   GEMM2: output columns 32 w .. 32 w + 31 of the tile's 256.
// A tile is specialised on its number of 32-row units, so a short tile (a
// small group, the last tile of a group) issues only the MFMAs of its rows.
//
// Operand paths.  The rows (A) are shared by the eight waves and move HBM ->
// LDS by buffer_load ... lds (no staging registers); a wave's weight rows are
// read by that wave alone, so they skip LDS and stream from HBM into a ring of
// three register sets (16 VGPRs each).  With the tiled weight layout (below)
// a wave's stage is one contiguous 4 KiB read; row-major weights take the same
// loads at row-strided addresses.
// Pipeline.  K advances in stages of 128 (one MFMA per row block and column
// block).  Three LDS buffers of [256 rows x 128 B | 256 row scales] hold A,
// loaded two stages ahead; the B register set of a stage is reloaded with the
// stage three ahead as soon as the stage's last MFMA has issued.  One barrier
// a stage: after it the stage's A has landed for every wave and the buffer of
// the previous stage is free for the next DMA.  Chunks outside the tile (rows
// past the group's end, weight rows past N, stages past the end) carry an
// offset past their buffer descriptor and load zeros with no memory traffic.
// LDS chunks of 16 B are XOR-swizzled by (row & 7) ^ ((row >> 3) & 1): the 16
// rows of a fragment read at one logical chunk land on 16 distinct bank groups.
// GEMM1 epilogue: h is requantised per row and 128 columns (the tile's h
// columns are one scale block): s = max|h| / 448 (1 for an all-zero block),
// q = e4m3_rne_sat(h / s), staged through LDS and stored as 16-byte chunks.
// GEMM2 epilogue: bf16 y is staged through LDS one 32-row unit at a time and
// stored as whole 512-byte rows of the tile (fp32 y straight from registers).
//
// Tiled e4m3 weights (written by tile_matrices_e4m3, once): a matrix of R rows
// and K columns (K a multiple of 128) becomes 4 KiB blocks of 32 rows x 128
// columns, block (r / 32, k / 128) at byte ((r / 32) * (K / 128) + k / 128) *
// 4096; inside, byte 1024 i + 16 l + b (i < 4, l < 64, b < 16) holds row
// 16 (i / 2) + l % 16 and column 32 (l / 16) + 16 (i % 2) + b -- load i of lane
// l is half i % 2 of the lane's fragment of column block i / 2.  Gate and up
// merge into one matrix of 2 I rows: 32-row group q holds gate rows 16 q ..
// 16 q + 15, then the up rows of the same h columns.  Down keeps its H rows.
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

constexpr int TB = kFfnBmE4m3, BN = 256, BK = 128, NWAVES = 8, NTH = NWAVES * 64, NS = 3;
constexpr int kRB = TB / 16;             // 16-row MFMA blocks of a full tile
constexpr int kChunks = TB * 8;          // 16-byte chunks of a stage's rows
constexpr int kStage = kChunks + TB / 4; // then the stage's TB fp32 row scales
static_assert(TB == 256, "the load slots below cover 256 rows: 4 chunk loads and 1 scale load per wave");
constexpr int kLoadsB = 4;  // B vector-memory instructions per wave per stage
// A instructions per wave per stage: the four row-chunk loads of rows 32 w ..
// 32 w + 31 while they are rows of the tile (w < NRB 32-row units), and the
// row-scale load of rows 64 w .. 64 w + 63 for waves w < 4 while those are
// (2 w < NRB).  The tile body is specialised on both, so a wave issues only
// real loads and waits on exact counts.
template <bool CHUNKS, bool SCALES>
constexpr int kLoadsAOf = (CHUNKS ? 4 : 0) + (SCALES ? 1 : 0);
// vmcnt at the top of stage s: this wave's NA A loads of stage s (issued
// during stage s - 2) have landed when at most the B loads of stage s + 1, the
// A loads of stage s + 1 and the B loads of stage s + 2 are outstanding.
template <int NA>
constexpr int kWaitStage = kLoadsB + NA + kLoadsB;
constexpr uint32_t kOOB = 0x80000000u;   // past every descriptor (all are < 2 GiB): the load returns zero

typedef __attribute__((address_space(3))) void* lds_t;

// The A stage buffers: distinct objects, so that the compiler can tell which
// buffer an in-flight LDS DMA writes and never waits for a load into another.
__shared__ i32x4 ring0[kStage];
__shared__ i32x4 ring1[kStage];
__shared__ i32x4 ring2[kStage];

template <int BUF>
__device__ __forceinline__ i32x4* ring() {
    static_assert(BUF < NS, "ring buffer index");
    if constexpr (BUF == 0) return ring0;
    else if constexpr (BUF == 1) return ring1;
    else return ring2;
}

__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma_e4m3(i32x8 w, i32x8 a) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

struct E4m3Args {
    const uint8_t* a;       // GEMM1: x rows [rows][H]; GEMM2: h [rows][I]
    const float* a_scale;   // [rows][K / 128]
    const uint8_t* w0;      // GEMM1: w_gate [E][I][H] or tiled gate+up; GEMM2: w_down [E][H][I] or tiled
    const uint8_t* w1;      // GEMM1: w_up [E][I][H] (row-major only)
    const float* s0;        // GEMM1: s_gate [E][I/128][H/128]; GEMM2: s_down [E][H/128][I/128]
    const float* s1;        // GEMM1: s_up
    void* out;              // GEMM1: h [rows][I] e4m3; GEMM2: y [rows][H]
    float* out_scale;       // GEMM1: h scales [rows][I / 128]
    const int4* tiles;
    const int32_t* n_tiles;
    int32_t* queue;  // the launch's work queue (see xcd_queue_pick)
    const int2* work;       // {M tile, N tile} in launch order
    int NT;                 // N tiles per M tile
    int K, N;               // GEMM1: K = H, N = I; GEMM2: K = I, N = H
    int out_f32;            // GEMM2 output dtype
    int w_tiled;            // weights in the tiled e4m3 layout
    WTab wt;                // wt.tab != NULL: w0, w1, s0, s1 of group g are table entries
    int slot0, slot1;       //   slot0, slot1, slot0 + 3, slot1 + 3
    const int32_t* a_row_src;  // GEMM1: non-NULL -> a is x [a_rows][K], row r of A is x row a_row_src[r] / a_row_k
    int a_row_k, a_rows;
};

// Per-tile load state.  A: descriptors of the rows and their scales and this
// lane's offsets in stage 0 (a stage moves them 128 B and 4 B).  B: the
// descriptors of the wave's two column blocks, this lane's offset of each in
// stage 0, the move of a fragment's second half and of a stage (tiled: 1 KiB
// and 4 KiB; row-major: 16 B and 128 B).
struct Dma {
    __amdgpu_buffer_rsrc_t ra, rs, rb0, rb1;
    uint32_t va[4], vs, vb[2], bh, bt;
    int nsteps;
};

// A load J (0..4) of stage t into buffer BUF, issued when this wave has it
// (CHUNKS for J < 4, SCALES for J = 4): J < 4 fills LDS chunks (4 w + J) * 64
// + lane (rows (4 w + J) * 8 + lane / 8); J = 4 the row scales of waves w < 4,
// positions 64 w + [0, 64) (position 64 c + 4 l + j holds row 64 c + 16 j + l,
// so a lane's scales of row blocks 4 c .. 4 c + 3 are one 16-byte chunk).
template <int BUF, int J, bool CHUNKS, bool SCALES>
__device__ __forceinline__ void dma_a1(const Dma& d, int t, int wave) {
    const bool real = t < d.nsteps;
    if constexpr (J < 4) {
        if constexpr (!CHUNKS) return;
        const uint32_t off = (!real || d.va[J] == kOOB) ? kOOB : d.va[J] + (uint32_t)t * BK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_t)(ring<BUF>() + (wave * 4 + J) * 64), 16, off, 0, 0, 0);
    } else {
        if constexpr (!SCALES) return;
        const uint32_t off = (!real || d.vs == kOOB) ? kOOB : d.vs + (uint32_t)t * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_t)(ring<BUF>() + kChunks + (wave & 3) * 16), 4, off, 0,
                                                 0, 0);
    }
}

// The B fragments of stage t into register set b: fragment cb = loads 2 cb and
// 2 cb + 1.  Selects only (a branch would cost the wait counters their
// precision).
__device__ __forceinline__ void load_b(const Dma& d, int t, i32x8 (&b)[2]) {
    const bool real = t < d.nsteps;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const __amdgpu_buffer_rsrc_t r = cb ? d.rb1 : d.rb0;
        const uint32_t o0 = (!real || d.vb[cb] == kOOB) ? kOOB : d.vb[cb] + (uint32_t)t * d.bt;
        const uint32_t o1 = o0 == kOOB ? kOOB : o0 + d.bh;
        const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, o0, 0, 0);
        const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, o1, 0, 0);
        b[cb] = cat(lo, hi);
    }
}

// acc += t * s_row * s_weight for one row block: sa is this lane's row scale,
// p0 the weight scale of column block 0 (gate or down) and p1 of block 1.
__device__ __forceinline__ void promote(const f32x4 (&t)[2], float sa, float p0, float p1, f32x4 (&acc)[2]) {
    const float q0 = sa * p0, q1 = sa * p1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[0][j] = __builtin_fmaf(t[0][j], q0, acc[0][j]);
        acc[1][j] = __builtin_fmaf(t[1][j], q1, acc[1][j]);
    }
}

// One K stage s on A buffer BUF and B register set BUF, RB row blocks.  The
// fragment of row block rb + 1 is read just before the two MFMAs of rb issue
// (a whole row block ahead of its use), and rb - 1 is promoted while they
// run; the stage's five A loads (stage s + 2, into the buffer stage s - 1
// used) follow the MFMAs of the first row blocks; the register set is
// reloaded with stage s + 3 after the last MFMA.
template <int RB, int BUF, bool CH, bool SC>
__device__ __forceinline__ void stage(const Dma& d, int s, int wave, int lane, i32x8 (&b)[NS][2], float p0,
                                      float p1, f32x4 (&acc)[kRB][2]) {
    constexpr int NA = (BUF + 2) % NS;
    // every access indexes the buffer object itself (an integer base plus a
    // constant), so the compiler tells it from the DMA in flight into the others
    const i32x4* buf = ring<BUF>();
    const int l16 = lane & 15;
    const int plo = (2 * (lane >> 4)) ^ swz8(l16), phi = plo ^ 1;
    const int ia = l16 * 8;  // row block rb: + rb * 128
    const int is = kChunks + l16;  // row scales of row blocks 4 c .. 4 c + 3: + 16 c
    wait_vm<kWaitStage<kLoadsAOf<CH, SC>>>();  // this wave's A loads of stage s have landed
    barrier_lds();          // ... every wave's, and every wave is done with stage s - 1
    i32x8 a[2];
    f32x4 t[2][2];
    f32x4 sa[2];
    sa[0] = __builtin_bit_cast(f32x4, buf[is]);
    a[0] = cat(buf[ia + plo], buf[ia + phi]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        // the fragment of rb + 1 goes to the register the MFMAs of rb - 1 read
        if (rb + 1 < RB) {
            a[(rb + 1) & 1] = cat(buf[ia + (rb + 1) * 128 + plo], buf[ia + (rb + 1) * 128 + phi]);
            if ((rb + 1) % 4 == 0) sa[((rb + 1) / 4) & 1] = __builtin_bit_cast(f32x4, buf[is + 16 * ((rb + 1) / 4)]);
        }
        t[rb & 1][0] = mfma_e4m3(b[BUF][0], a[rb & 1]);
        t[rb & 1][1] = mfma_e4m3(b[BUF][1], a[rb & 1]);
        switch (rb) {  // a constant: the loop is unrolled
            case 0: dma_a1<NA, 0, CH, SC>(d, s + 2, wave); break;
            case 1: dma_a1<NA, 1, CH, SC>(d, s + 2, wave); break;
            case 2: dma_a1<NA, 2, CH, SC>(d, s + 2, wave); break;
            case 3: dma_a1<NA, 3, CH, SC>(d, s + 2, wave); break;
            case 4: dma_a1<NA, 4, CH, SC>(d, s + 2, wave); break;
            default: break;
        }
        if (rb > 0) promote(t[(rb - 1) & 1], sa[((rb - 1) / 4) & 1][(rb - 1) & 3], p0, p1, acc[rb - 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (RB < 2) dma_a1<NA, 1, CH, SC>(d, s + 2, wave);
    if constexpr (RB < 3) dma_a1<NA, 2, CH, SC>(d, s + 2, wave);
    if constexpr (RB < 4) dma_a1<NA, 3, CH, SC>(d, s + 2, wave);
    if constexpr (RB < 5) dma_a1<NA, 4, CH, SC>(d, s + 2, wave);
    promote(t[(RB - 1) & 1], sa[((RB - 1) / 4) & 1][(RB - 1) & 3], p0, p1, acc[RB - 1]);
    __builtin_amdgcn_sched_barrier(0);
    load_b(d, s + NS, b[BUF]);  // the set is free once its MFMAs have issued
    __builtin_amdgcn_sched_barrier(0);
}

// Rows of a tile past the group's end load as zero and are computed with the
// rest of their 32-row unit.
template <int MODE, int NRB, bool CH, bool SC>
__device__ __forceinline__ void run_tile(const E4m3Args& p, int g, int row0, int M, int nt) {
    constexpr int RB = 2 * NRB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = p.K, N = p.N;
    const int KB = K / BK;  // K and N are multiples of 128
    const int NBn = N / BK;
    const int n0 = MODE == 0 ? nt * (BN / 2) : nt * BN;  // first h column / output column of the tile
    Dma d;
    d.nsteps = KB;
    // ---- A rows row0 .. row0 + M and their scales; indexed (GEMM1 of the
    // layer): the descriptors span all of x and its scales, and row r of the
    // tile is token row_src[row0 + r] / k (rows with row_src -1 load zeros)
    const bool a_idx = MODE == 0 && p.a_row_src != nullptr;
    auto a_row = [&](int r) {  // the row of the descriptor's array holding tile row r, or -1
        if (r >= M) return -1;
        if (!a_idx) return r;
        const int src = p.a_row_src[row0 + r];
        return src >= 0 ? src / p.a_row_k : -1;
    };
    if (a_idx) {
        d.ra = make_rsrc(p.a, (uint32_t)p.a_rows * (uint32_t)K);
        d.rs = make_rsrc(p.a_scale, (uint32_t)p.a_rows * (uint32_t)KB * 4u);
    } else {
        d.ra = make_rsrc(p.a + (size_t)row0 * K, (uint32_t)M * (uint32_t)K);
        d.rs = make_rsrc(p.a_scale + (size_t)row0 * KB, (uint32_t)M * (uint32_t)KB * 4u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (wave * 4 + i) * 8 + (lane >> 3);
        const int ar = a_row(row);
        d.va[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)K + (uint32_t)(((lane & 7) ^ swz8(row)) * 16) : kOOB;
    }
    {
        const int row = 64 * (wave & 3) + 16 * (lane & 3) + (lane >> 2);
        const int ar = a_row(row);
        d.vs = ar >= 0 ? (uint32_t)ar * (uint32_t)KB * 4u : kOOB;
    }
    // ---- B: this group's matrices and block scales
    const uint8_t *w0 = p.w0, *w1 = p.w1;
    const float *s0 = p.s0, *s1 = p.s1;
    int ge = g;
    if (p.wt.tab) {
        const int lay = *p.wt.layer;
        w0 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot0));
        s0 = static_cast<const float*>(wtab_ptr(p.wt, lay, g, p.slot0 + 3));
        if (MODE == 0) {
            if (!p.w_tiled) w1 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot1));
            s1 = static_cast<const float*>(wtab_ptr(p.wt, lay, g, p.slot1 + 3));
        }
        ge = 0;
    }
    // the wave's weight rows: GEMM1 gate / up rows n0 + 16 w + [0, 16) (h
    // columns), GEMM2 rows n0 + 32 w + [0, 32); a wave past N (GEMM2 with N not
    // a multiple of 256) loads zeros and stores nothing
    const int wrow = MODE == 0 ? n0 + 16 * wave : n0 + 32 * wave;
    const bool wvalid = wrow < N;
    const int l16 = lane & 15, g4 = lane >> 4;
    if (p.w_tiled) {
        // one matrix of 32-row groups: GEMM1 group n0 / 16 + w of the gate+up
        // matrix (2 N rows), GEMM2 group n0 / 32 + w of the down matrix
        const size_t mrows = MODE == 0 ? 2 * (size_t)N : (size_t)N;
        const uint8_t* W = w0 + (size_t)ge * mrows * K;
        d.rb0 = d.rb1 = make_rsrc(W, (uint32_t)(mrows * (size_t)K));
        const uint32_t grp = (uint32_t)(MODE == 0 ? n0 / 16 + wave : n0 / 32 + wave);
        const uint32_t base = grp * (uint32_t)KB * 4096u + (uint32_t)lane * 16u;
        d.vb[0] = wvalid ? base : kOOB;
        d.vb[1] = wvalid ? base + 2048u : kOOB;
        d.bh = 1024u;
        d.bt = 4096u;
    } else {
        const size_t mat = (size_t)N * K;
        d.rb0 = make_rsrc(w0 + (size_t)ge * mat, (uint32_t)mat);
        d.rb1 = MODE == 0 ? make_rsrc(w1 + (size_t)ge * mat, (uint32_t)mat) : d.rb0;
        const int r0 = wrow + l16, r1 = MODE == 0 ? r0 : r0 + 16;  // GEMM1: the same row of gate and up
        d.vb[0] = wvalid ? (uint32_t)r0 * (uint32_t)K + (uint32_t)(32 * g4) : kOOB;
        d.vb[1] = wvalid ? (uint32_t)r1 * (uint32_t)K + (uint32_t)(32 * g4) : kOOB;
        d.bh = 16u;
        d.bt = (uint32_t)BK;
    }
    // weight-block scales of this wave's columns for every K block, lane kb % 64
    // of register kb / 64 holding block kb (K <= 16384): loaded once, then read
    // with readlane
    const int wbase = !wvalid ? -1 : (ge * NBn + wrow / BK) * KB;
    float ws0[2] = {0.f, 0.f}, ws1[2] = {0.f, 0.f};
    if (wbase >= 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kb = h * 64 + lane;
            if (kb < KB) {
                ws0[h] = s0[wbase + kb];
                ws1[h] = MODE == 0 ? s1[wbase + kb] : ws0[h];
            }
        }
    }
    auto wscale = [&](int kb, float& p0, float& p1) {
        const int h = kb >> 6, l = kb & 63;
        p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h ? ws0[1] : ws0[0]), l));
        p1 = MODE == 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h ? ws1[1] : ws1[0]), l)) : p0;
    };

    f32x4 acc[kRB][2];
#pragma unroll
    for (int i = 0; i < kRB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Prologue, in the steady state's issue order: B(0), A(0), B(1), A(1), B(2).
    i32x8 b[NS][2];
    load_b(d, 0, b[0]);
    dma_a1<0, 0, CH, SC>(d, 0, wave);
    dma_a1<0, 1, CH, SC>(d, 0, wave);
    dma_a1<0, 2, CH, SC>(d, 0, wave);
    dma_a1<0, 3, CH, SC>(d, 0, wave);
    dma_a1<0, 4, CH, SC>(d, 0, wave);
    load_b(d, 1, b[1]);
    dma_a1<1, 0, CH, SC>(d, 1, wave);
    dma_a1<1, 1, CH, SC>(d, 1, wave);
    dma_a1<1, 2, CH, SC>(d, 1, wave);
    dma_a1<1, 3, CH, SC>(d, 1, wave);
    dma_a1<1, 4, CH, SC>(d, 1, wave);
    load_b(d, 2, b[2]);
    // Stage s uses A buffer and B register set s % 3.  The loop body is one
    // period of the ring, entered at stage 1: at the loop head the compiler
    // no longer tells the ring buffers apart and, before the first LDS read,
    // waits for the A loads issued in the previous stage as well (a longer
    // body spills registers).
    int s = 0;
    {
        float p0, p1;
        wscale(s, p0, p1);
        stage<RB, 0, CH, SC>(d, s, wave, lane, b, p0, p1, acc);
    }
    for (;;) {
        float p0, p1;
        if (++s >= KB) break;
        wscale(s, p0, p1);
        stage<RB, 1, CH, SC>(d, s, wave, lane, b, p0, p1, acc);
        if (++s >= KB) break;
        wscale(s, p0, p1);
        stage<RB, 2, CH, SC>(d, s, wave, lane, b, p0, p1, acc);
        if (++s >= KB) break;
        wscale(s, p0, p1);
        stage<RB, 0, CH, SC>(d, s, wave, lane, b, p0, p1, acc);
    }
    wait_vm<0>();  // the zero loads of the stages past the end land before the buffers are reused
    barrier_lds();

    // A lane holds row 16 rb + l16 of the tile and, in column block cb, the
    // weight rows 16 cb + 4 g4 + [0, 4) of its 32.
    if constexpr (MODE == 0) {
        // h = silu(g) * u for h columns n0 + 16 w + 4 g4 + j, into acc[rb][0]
        float* red = reinterpret_cast<float*>(ring<0>());  // [8 waves][256 rows] row maxima
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[rb][0][j] = silu_f(acc[rb][0][j]) * acc[rb][1][j];
                m = fmaxf(m, fabsf(acc[rb][0][j]));
            }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (lane < 16) red[wave * TB + rb * 16 + l16] = m;
        }
        __syncthreads();
        float* rsc = reinterpret_cast<float*>(ring<1>());  // [256] the rows' scales
        const int tid = threadIdx.x;
        if (tid < 32 * NRB) {
            float amax = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) amax = fmaxf(amax, red[w * TB + tid]);
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            rsc[tid] = sc;
            if (tid < M) p.out_scale[(size_t)(row0 + tid) * NBn + n0 / BK] = sc;
        }
        __syncthreads();
        // [256 rows][128 columns] e4m3, 32 words a row; the 16-byte chunk c of
        // row r at chunk c ^ ((r >> 1) & 7): the 16 rows x 4 words of one
        // store touch 64 distinct banks
        uint32_t* qs = reinterpret_cast<uint32_t*>(ring<2>());
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = rb * 16 + l16;
            const float sc = rsc[row];
            const uint32_t w = e4m3x4_rne_sat(acc[rb][0][0] / sc, acc[rb][0][1] / sc, acc[rb][0][2] / sc,
                                              acc[rb][0][3] / sc);
            qs[row * 32 + ((wave ^ ((row >> 1) & 7)) << 2) + g4] = w;
        }
        __syncthreads();
        // coalesced 16-byte stores of the tile's M rows x 128 h columns
        uint8_t* h = static_cast<uint8_t*>(p.out);
        const i32x4* qv = reinterpret_cast<const i32x4*>(qs);
        for (int c = tid; c < M * 8; c += NTH) {
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<i32x4*>(h + (size_t)(row0 + row) * N + n0 + ch * 16) = qv[row * 8 + (ch ^ ((row >> 1) & 7))];
        }
    } else if (!p.out_f32) {
        // y in bf16, staged through LDS one 32-row unit at a time (two
        // buffers, one barrier a unit) and stored as whole rows of the tile.
        // The 16-byte chunk c of a staged row r sits at chunk c ^ (r & 15): a
        // wave's write (16 rows x 2 chunks) and its read (2 whole rows) both
        // spread over every bank.
        uint16_t* y = static_cast<uint16_t*>(p.out);
        const int tid = threadIdx.x;
        const int ncols = min(BN, N - n0);  // columns of the tile inside y
#pragma unroll
        for (int u = 0; u < NRB; ++u) {
            uint32_t* st = reinterpret_cast<uint32_t*>(u & 1 ? ring<1>() : ring<0>());
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int r = 16 * hb + l16;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const f32x4 v = acc[2 * u + hb][cb];
                    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                    const int c = 4 * wave + 2 * cb + (g4 >> 1);
                    *reinterpret_cast<uint2*>(st + r * 128 + ((c ^ (r & 15)) << 2) + (g4 & 1) * 2) =
                        make_uint2(lo, hi);
                }
            }
            // the unit is staged; the other buffer's reads (unit u - 1) came
            // before every thread's writes above, so it is free for unit u + 1
            __syncthreads();
            const i32x4* sv = reinterpret_cast<const i32x4*>(st);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int id = i * NTH + tid;
                const int r = id >> 5, c = id & 31, row = 32 * u + r;
                // non-temporal: y is read again only by the combine, after the launch
                if (row < M && c * 8 < ncols)
                    __builtin_nontemporal_store(sv[r * 32 + (c ^ (r & 15))],
                                                reinterpret_cast<i32x4*>(y + (size_t)(row0 + row) * N + n0 + c * 8));
            }
        }
    } else {
        // fp32 y: lane stores 4 consecutive columns of its row per column block
        if (!wvalid) return;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = rb * 16 + l16;
            if (row >= M) continue;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const size_t o = (size_t)(row0 + row) * N + (size_t)(wrow + 16 * cb + 4 * g4);
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = acc[rb][cb];
            }
        }
    }
}

// The tile body of this wave: whether it loads row chunks (w < NRB) and row
// scales (w < 4 and 2 w < NRB) is uniform per wave.  A wave that loads scales
// also loads chunks.
template <int MODE, int NRB>
__device__ __forceinline__ void tile_of_wave(const E4m3Args& p, int g, int row0, int M, int nt) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4 && 2 * wave < NRB) run_tile<MODE, NRB, true, true>(p, g, row0, M, nt);
    else if constexpr (NRB < NWAVES) {
        if (wave < NRB) run_tile<MODE, NRB, true, false>(p, g, row0, M, nt);
        else run_tile<MODE, NRB, false, false>(p, g, row0, M, nt);
    } else {
        run_tile<MODE, NRB, true, false>(p, g, row0, M, nt);
    }
}

template <int MODE>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
ffn_gemm_e4m3(E4m3Args p) {
    const int L = xcd_queue_tile(p.n_tiles[0] * p.NT, p.queue);
    if (L < 0) return;
    if (p.wt.tab && wtab_layer(p.wt) < 0) return;
    const int2 wl = p.work[L];
    const int4 td = p.tiles[wl.x];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const int n0 = MODE == 0 ? wl.y * (BN / 2) : wl.y * BN;
    if (n0 >= p.N || M <= 0) return;
    switch ((M + 31) / 32) {  // tile heights are multiples of 32 rows, at most 256
        case 1: tile_of_wave<MODE, 1>(p, g, row0, M, wl.y); break;
        case 2: tile_of_wave<MODE, 2>(p, g, row0, M, wl.y); break;
        case 3: tile_of_wave<MODE, 3>(p, g, row0, M, wl.y); break;
        case 4: tile_of_wave<MODE, 4>(p, g, row0, M, wl.y); break;
        case 5: tile_of_wave<MODE, 5>(p, g, row0, M, wl.y); break;
        case 6: tile_of_wave<MODE, 6>(p, g, row0, M, wl.y); break;
        case 7: tile_of_wave<MODE, 7>(p, g, row0, M, wl.y); break;
        default: tile_of_wave<MODE, 8>(p, g, row0, M, wl.y); break;
    }
}

// ------------------------------------------------------------- weight tiling
// Rewrites E row-major e4m3 matrices [rows][K] into the tiled layout above, one
// thread per destination 16-byte chunk.  With `pair`, 32-row group q holds gate
// rows 16 q .. 16 q + 15 (src0) and then the up rows (src1) of the same h
// columns.
__global__ void __launch_bounds__(256)
tile_matrices_e4m3(const uint8_t* __restrict__ src0, const uint8_t* __restrict__ src1, int E, int rows, int K,
                   int pair, uint8_t* __restrict__ dst, int groups) {
    const int KB = K / BK;
    const size_t per = (size_t)groups * KB * 256;  // 16-byte chunks of one matrix
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= per * E) return;
    const int e = (int)(idx / per);
    const size_t rem = idx % per;
    const int lane = (int)(rem & 63), i = (int)((rem >> 6) & 3);
    const size_t blk = rem >> 8;
    const int kb = (int)(blk % KB), q = (int)(blk / KB);
    const int cb = i >> 1;
    const int k0 = kb * BK + 32 * (lane >> 4) + 16 * (i & 1);
    const uint8_t* src = pair ? (cb ? src1 : src0) : src0;
    const int srow = pair ? 16 * q + (lane & 15) : 32 * q + 16 * cb + (lane & 15);
    i32x4 v = {0, 0, 0, 0};
    if (srow < rows) v = *reinterpret_cast<const i32x4*>(src + ((size_t)e * rows + srow) * K + k0);
    reinterpret_cast<i32x4*>(dst)[idx] = v;
}

}  // namespace

hipError_t launch_gemm_e4m3(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                            const float* x_scale, const int32_t* row_src, const int32_t* offsets,
                            const moe_weights& w, const WTab& wt, void* y_rows, const FfnWork& wk, void* h,
                            float* h_scale, hipStream_t s) {
    hipError_t e0 = launch_build_tiles(c, offsets, TB, n_rows_cap, wk, s);
    if (e0 != hipSuccess) return e0;
    E4m3Args a{};
    a.wt = wt;
    a.w_tiled = w.layout == MOE_LAYOUT_TILED ? 1 : 0;
    a.slot0 = 0;
    a.slot1 = 1;
    a.tiles = reinterpret_cast<const int4*>(wk.tiles);
    a.n_tiles = wk.n_tiles;
    // GEMM1: gate/up + SwiGLU -> h (e4m3) and its row-block scales
    a.work = reinterpret_cast<const int2*>(wk.work1);
    a.NT = wk.nt1;
    a.a = static_cast<const uint8_t*>(x_rows);
    a.a_scale = x_scale;
    a.a_row_src = row_src;  // indexed: x_rows is x [T][H], x_scale its [T][H / 128]
    a.a_row_k = c.k;
    a.a_rows = c.T;
    a.w0 = static_cast<const uint8_t*>(w.w_gate);
    a.w1 = static_cast<const uint8_t*>(w.w_up);
    a.s0 = w.s_gate;
    a.s1 = w.s_up;
    a.out = h;
    a.out_scale = h_scale;
    a.K = c.H;
    a.N = c.I;
    a.queue = wk.n_tiles + 2;  // queue 0
    hipLaunchKernelGGL(ffn_gemm_e4m3<0>, dim3((unsigned)xcd_queue_grid(max_tiles * wk.nt1)), dim3(NTH), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // GEMM2: down projection of h
    a.work = reinterpret_cast<const int2*>(wk.work2);
    a.NT = wk.nt2;
    a.a = static_cast<const uint8_t*>(h);
    a.a_scale = h_scale;
    a.a_row_src = nullptr;
    a.w0 = static_cast<const uint8_t*>(w.w_down);
    a.w1 = nullptr;
    a.slot0 = 2;
    a.s0 = w.s_down;
    a.s1 = nullptr;
    a.out = y_rows;
    a.out_scale = nullptr;
    a.K = c.I;
    a.N = c.H;
    a.out_f32 = c.y_dtype == MOE_F32 ? 1 : 0;
    a.queue = wk.n_tiles + 2 + kQueueWords;  // queue 1
    hipLaunchKernelGGL(ffn_gemm_e4m3<1>, dim3((unsigned)xcd_queue_grid(max_tiles * wk.nt2)), dim3(NTH), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tile_weights_e4m3(const moe_cfg& c, const moe_weights& src, void* w13, void* w2, void* sh13,
                                    void* sh2, hipStream_t s) {
    auto go = [&](const void* a, const void* b, int E, int rows, int K, int pair, void* dst) {
        const int groups = pair ? rows / 16 : rows / 32;  // rows: I (pair) or H, multiples of 128
        const size_t n = (size_t)E * groups * (K / BK) * 256;
        hipLaunchKernelGGL(tile_matrices_e4m3, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b), E, rows, K, pair,
                           static_cast<uint8_t*>(dst), groups);
    };
    go(src.w_gate, src.w_up, c.E, c.I, c.H, 1, w13);
    go(src.w_down, nullptr, c.E, c.H, c.I, 0, w2);
    if (c.has_shared) {
        go(src.sh_gate, src.sh_up, 1, c.I_shared, c.H, 1, sh13);
        go(src.sh_down, nullptr, 1, c.H, c.I_shared, 0, sh2);
    }
    return hipGetLastError();
}

}  // namespace moe
