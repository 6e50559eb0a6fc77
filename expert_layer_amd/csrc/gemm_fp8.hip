// gemm_fp8.hip -- the grouped SwiGLU FFN on fp8 (OCP e4m3) MFMA with fp32 block
// scales ("ASAP", section 3.4.2: the MoE kernel is a grouped matrix
// multiplication of hidden states by the layer's expert weights).  The operands
// are e4m3 codes with one fp32 scale per 1 x 128 block of a row (activations,
// h) and per 128 x 128 block (weights); a dequantised value is code * scale.
//
// Scale promotion.  A K block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4,
// so every MFMA result t is the unscaled partial sum of one scale block and is
// folded in as acc += t * (s_row * s_weight) on the VALU.  The MFMAs write VGPRs
// (this file is compiled in the VGPR form), so the promotion reads t directly.
//
// Tile.  256 rows x 256 weight rows, 8 waves (two per SIMD); wave w owns rows
// 128 (w / 4) + [0, 128) and weight rows 64 (w % 4) + [0, 64): 8 x 4 MFMA blocks
// of 16 x 16 and their fp32 accumulators (128 VGPRs -- the promotion FMAs need
// them in VALU registers, so a wave cannot hold more).  GEMM1: the 64 weight
// rows of a wave are 32 gate rows then the 32 up rows of the same h columns, so
// h = silu(g) * u forms in registers; GEMM2: 64 output columns.
// Pipeline.  K advances in stages of 128 through two A buffers [256 x 128 B |
// 256 row scales] and two B buffers [256 x 128 B]; operands move HBM -> LDS by
// buffer_load ... lds.  A wave reads all its B fragments of a stage first, so
// B of stage s+2 is issued as soon as every wave has them (almost two stages
// ahead of use) and A of stage s+1 at the start of stage s (one stage ahead).  Chunks outside the tile (rows past the
// group's end, weight rows past N) carry an offset beyond their buffer
// descriptor and load as zero.  LDS chunks of 16 B are XOR-swizzled by
// (row >> 1) & 7, so a fragment read of 16 rows at one logical chunk touches
// 16 distinct 16-byte bank groups of the 64 banks.
// GEMM1 epilogue: h is requantised per row and 128 columns -- the tile's 128 h
// columns are one scale block: s = max|h| / 448 (1 for an all-zero block),
// q = e4m3_rne_sat(h / s) -- staged through LDS and stored as 16-byte chunks.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 128, NTH = 512;
constexpr int kChunks = 256 * 8;               // 16-byte chunks of one operand in one stage
constexpr int kStageA = kChunks + 128;         // A, 256 fp32 row scales, a 1 KiB sink
constexpr uint32_t kOOB = 0x40000000u;         // past every descriptor: the load returns zero

typedef __attribute__((address_space(3))) void* lds_t;

__shared__ i32x4 stgA0[kStageA];
__shared__ i32x4 stgA1[kStageA];
__shared__ i32x4 stgB0[kChunks];
__shared__ i32x4 stgB1[kChunks];

template <int BUF>
__device__ __forceinline__ i32x4* stgA() {
    if constexpr (BUF == 0) return stgA0;
    else return stgA1;
}
template <int BUF>
__device__ __forceinline__ i32x4* stgB() {
    if constexpr (BUF == 0) return stgB0;
    else return stgB1;
}

__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
}

struct Fp8Args {
    const uint8_t* a;       // GEMM1: x rows [rows][H]; GEMM2: h [rows][I]
    const float* a_scale;   // [rows][K / 128]
    const uint8_t* w0;      // GEMM1: w_gate [E][I][H]; GEMM2: w_down [E][H][I]
    const uint8_t* w1;      // GEMM1: w_up [E][I][H]
    const float* s0;        // GEMM1: s_gate [E][I/128][H/128]; GEMM2: s_down [E][H/128][I/128]
    const float* s1;        // GEMM1: s_up
    void* out;              // GEMM1: h [rows][I] e4m3; GEMM2: y [rows][H]
    float* out_scale;       // GEMM1: h scales [rows][I / 128]
    const int4* tiles;
    const int32_t* n_tiles;
    const int2* work;       // {M tile, N tile} in launch order
    int NT;                 // N tiles per M tile
    int K, N;               // GEMM1: K = H, N = I; GEMM2: K = I, N = H
    int out_f32;            // GEMM2 output dtype
};

struct Dma {
    __amdgpu_buffer_rsrc_t ra, rs, rb0, rb1;
    uint32_t va[4], vb[4], vs;
    int nsteps;  // K blocks
};

// A loads of stage t into A buffer BUF: 4 chunk loads per lane (8 LDS rows
// each) and one row-scale load -- waves 0..3 load the scales of 64 rows each,
// waves 4..7 an out-of-range (zero) load into the sink, so every wave has the
// same 5 A loads per stage.
template <int BUF>
__device__ __forceinline__ void dma_a(const Dma& d, int t, int wave) {
    i32x4* buf = stgA<BUF>();
    const uint32_t k = (uint32_t)t * BK;
    const bool real = t < d.nsteps;  // stages past the end load zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t off = (!real || d.va[i] == kOOB) ? kOOB : d.va[i] + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_t)(buf + (wave * 4 + i) * 64), 16, off, 0, 0, 0);
    }
    const uint32_t so = (!real || d.vs == kOOB) ? kOOB : d.vs + (uint32_t)t * 4u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_t)(buf + kChunks + wave * 16), 4, so, 0, 0, 0);
}

// B loads of stage t into B buffer BUF: 4 chunk loads per lane.
template <int MODE, int BUF>
__device__ __forceinline__ void dma_b(const Dma& d, int t, int wave) {
    i32x4* buf = stgB<BUF>();
    const uint32_t k = (uint32_t)t * BK;
    const bool real = t < d.nsteps;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t off = (!real || d.vb[i] == kOOB) ? kOOB : d.vb[i] + k;
        // GEMM1: wave w fills LDS rows 32 w + [0, 32): gate rows of quarter w / 2
        // on even waves, up rows on odd waves
        const __amdgpu_buffer_rsrc_t r = (MODE == 0 && (wave & 1)) ? d.rb1 : d.rb0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t)(buf + (wave * 4 + i) * 64), 16, off, 0, 0, 0);
    }
}

// vmcnt(4) with the other counters at zero: a stage's A loads and everything
// before them have landed (the 4 B loads issued after them may be in flight),
// and every LDS read of this wave has returned.
__device__ __forceinline__ void wait_stage() { __builtin_amdgcn_s_waitcnt(4 | 0x0070); }

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void promote(const f32x4 (&t)[4], const f32x4& sa, float p0, float p1,
                                        f32x4 (&acc)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float q0 = sa[j] * p0, q1 = sa[j] * p1;
        acc[0][j] = __builtin_fmaf(t[0][j], q0, acc[0][j]);
        acc[1][j] = __builtin_fmaf(t[1][j], q0, acc[1][j]);
        acc[2][j] = __builtin_fmaf(t[2][j], q1, acc[2][j]);
        acc[3][j] = __builtin_fmaf(t[3][j], q1, acc[3][j]);
    }
}

// The B fragments of this wave (column blocks of 16 rows of weight rows
// q * 64 ..) in stage buffer BUF.  A lane reads row (16 i + lane % 16) at
// logical chunks 2 (lane / 16) and 2 (lane / 16) + 1; the swizzle of a row
// depends on row % 16 only, so every fragment address is one of two per-lane
// bases plus a constant.
template <int BUF>
__device__ __forceinline__ void read_b(int q, int lane, i32x8 (&b)[4]) {
    const i32x4* buf = stgB<BUF>();
    const int l16 = lane & 15;
    const int plo = (2 * (lane >> 4)) ^ swz8(l16), phi = plo ^ 1;
    const int ib = ((q & 3) * 64 + l16) * 8;  // column block cb: + cb * 128
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) b[cb] = cat(buf[ib + cb * 128 + plo], buf[ib + cb * 128 + phi]);
}

// One K stage for the 8 row blocks of 16 starting at tile row r0: every (row
// block, column block) MFMA of this wave, promoted with the stage's row scales
// and the wave's weight-block scales p0 (gate or down columns) and p1 (up
// columns).  Software-pipelined over row blocks: while the four MFMAs of row
// block rb run, the fragments of rb + 1 are read and rb - 1 is promoted.
template <int BUF>
__device__ __forceinline__ void kstep(int r0, int lane, const i32x8 (&b)[4], float p0, float p1,
                                      f32x4 (&acc)[8][4]) {
    constexpr int RB = 8;
    // Every access indexes the stage buffer itself (an integer base plus a
    // constant), so the compiler can tell it from the DMA in flight into the
    // other buffers and adds no wait for it.
    const i32x4* buf = stgA<BUF>();
    const int l16 = lane & 15;
    const int plo = (2 * (lane >> 4)) ^ swz8(l16), phi = plo ^ 1;
    const int ia = ((r0 & 128) + l16) * 8;              // row block rb: + rb * 128
    const int is = kChunks + (r0 & 128) / 4 + (lane >> 4);  // row block rb: + rb * 4
    i32x8 a[2];
    f32x4 sa[3];
    f32x4 t[2][4];
    a[0] = cat(buf[ia + plo], buf[ia + phi]);
    sa[0] = __builtin_bit_cast(f32x4, buf[is]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) t[rb & 1][cb] = mfma16x16x128_fp8(a[rb & 1], b[cb]);
        if (rb + 1 < RB) {
            a[(rb + 1) & 1] = cat(buf[ia + (rb + 1) * 128 + plo], buf[ia + (rb + 1) * 128 + phi]);
            sa[(rb + 1) % 3] = __builtin_bit_cast(f32x4, buf[is + (rb + 1) * 4]);
        }
        if (rb > 0) promote(t[(rb - 1) & 1], sa[(rb - 1) % 3], p0, p1, acc[rb - 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    promote(t[(RB - 1) & 1], sa[(RB - 1) % 3], p0, p1, acc[RB - 1]);
}

// Rows of a tile past the group's end load as zero and are computed like the
// others; a wave whose half of the tile holds no row skips the MFMAs.
template <int MODE>
__device__ __forceinline__ void run_tile(const Fp8Args& p, int g, int row0, int M, int n0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mh = wave >> 2, q = wave & 3, r0 = mh * 128;
    const int K = p.K, N = p.N;
    const int KB = K / BK;  // K and N are multiples of 128
    const int NB = N / BK;
    Dma d;
    d.nsteps = KB;
    // ---- A rows row0 .. row0 + M and their row scales
    d.ra = make_rsrc(p.a + (size_t)row0 * K, (uint32_t)M * (uint32_t)K);
    d.rs = make_rsrc(p.a_scale + (size_t)row0 * KB, (uint32_t)M * (uint32_t)KB * 4u);
    {
        const int r = wave * 64 + lane;
        d.vs = (wave < 4 && r < M) ? (uint32_t)r * (uint32_t)KB * 4u : kOOB;
    }
    // ---- B: GEMM1 the gate and up rows n0 + [0, 128) (LDS quarter j holds gate
    // rows 32 j + [0, 32) then the up rows of the same h columns); GEMM2 the
    // weight rows n0 + [0, 256)
    const int nlim = MODE == 0 ? min(N - n0, 128) : min(N - n0, BN);
    if (MODE == 0) {
        const size_t mat = (size_t)N * K;
        d.rb0 = make_rsrc(p.w0 + (size_t)g * mat + (size_t)n0 * K, (uint32_t)nlim * (uint32_t)K);
        d.rb1 = make_rsrc(p.w1 + (size_t)g * mat + (size_t)n0 * K, (uint32_t)nlim * (uint32_t)K);
    } else {
        d.rb0 = make_rsrc(p.w0 + (size_t)g * N * K + (size_t)n0 * K, (uint32_t)nlim * (uint32_t)K);
        d.rb1 = d.rb0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wave * 32 + i * 8 + (lane >> 3);  // LDS row this lane fills (A and B)
        const uint32_t logical = (uint32_t)(((lane & 7) ^ swz8(row)) * 16);
        d.va[i] = row < M ? (uint32_t)row * (uint32_t)K + logical : kOOB;
        const int wrow = MODE == 0 ? (wave >> 1) * 32 + i * 8 + (lane >> 3) : row;  // relative to n0
        d.vb[i] = wrow < nlim ? (uint32_t)wrow * (uint32_t)K + logical : kOOB;
    }
    // weight-block scales of this wave's columns for every K block, lane kb % 64
    // of register kb / 64 holding block kb (K <= 16384): loaded once, then read
    // with readlane, so no vector-memory load besides the DMA runs in the K loop
    int wbase = -1;
    if (MODE == 0) {
        wbase = (g * NB + n0 / BK) * KB;
    } else {
        // a wave whose 64 columns lie past N (N not a multiple of 256) reads no scale
        const int cbk = (n0 + q * 64) / BK;
        if (cbk < NB) wbase = (g * NB + cbk) * KB;
    }
    float ws0[2] = {0.f, 0.f}, ws1[2] = {0.f, 0.f};
    if (wbase >= 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kb = h * 64 + lane;
            if (kb < KB) {
                ws0[h] = p.s0[wbase + kb];
                ws1[h] = MODE == 0 ? p.s1[wbase + kb] : ws0[h];
            }
        }
    }
    auto wscale = [&](int kb, float& p0, float& p1) {
        const int h = kb >> 6, l = kb & 63;
        p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h ? ws0[1] : ws0[0]), l));
        p1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h ? ws1[1] : ws1[0]), l));
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The loop runs whole pairs of stages and always issues the next loads
    // (zeros past the end; an odd last stage computes on zeros with zero
    // scales).  Per stage, in issue order: A of stage s+1 (5 loads), then B of
    // stage s+2 (4 loads), so at the start of a stage vmcnt(4) covers its A and
    // B.  Prologue: B0, A0, B1.
    dma_b<MODE, 0>(d, 0, wave);
    dma_a<0>(d, 0, wave);
    dma_b<MODE, 1>(d, 1, wave);
    i32x8 b[4];
    for (int s = 0; s < KB; s += 2) {
        float p0, p1;
        wscale(s, p0, p1);
        wait_stage();       // stage s (buffers 0) has landed; this wave's reads of stage s-1 are done
        barrier_lds();      // ... everybody's: the buffers 1 are free
        dma_a<1>(d, s + 1, wave);
        read_b<0>(q, lane, b);
        wait_lgkm0();
        barrier_lds();      // every wave holds its B fragments of stage s
        dma_b<MODE, 0>(d, s + 2, wave);
        if (r0 < M) kstep<0>(r0, lane, b, p0, p1, acc);
        wscale(s + 1, p0, p1);
        wait_stage();
        barrier_lds();
        dma_a<0>(d, s + 2, wave);
        read_b<1>(q, lane, b);
        wait_lgkm0();
        barrier_lds();
        dma_b<MODE, 1>(d, s + 3, wave);
        if (r0 < M) kstep<1>(r0, lane, b, p0, p1, acc);
    }
    wait_vm0();  // no LDS DMA may outlive the workgroup
    barrier_lds();

    const int l16 = lane & 15, rq = 4 * (lane >> 4);
    if (MODE == 0) {
        // h = silu(g) * u for h columns n0 + 32 q + 16 c + l16, c = 0, 1
        float rmax[8][4];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[rb][0][j] = silu_f(acc[rb][0][j]) * acc[rb][2][j];
                acc[rb][1][j] = silu_f(acc[rb][1][j]) * acc[rb][3][j];
                float m = fmaxf(fabsf(acc[rb][0][j]), fabsf(acc[rb][1][j]));
                m = fmaxf(m, __shfl_xor(m, 1, 16));
                m = fmaxf(m, __shfl_xor(m, 2, 16));
                m = fmaxf(m, __shfl_xor(m, 4, 16));
                m = fmaxf(m, __shfl_xor(m, 8, 16));
                rmax[rb][j] = m;
            }
        // per-row maxima of the four quarters' 32 columns -> LDS [4][256]
        float* red = reinterpret_cast<float*>(stgA0);
        if (l16 == 0)
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int j = 0; j < 4; ++j) red[q * 256 + r0 + rb * 16 + rq + j] = rmax[rb][j];
        __syncthreads();
        uint8_t* qs = reinterpret_cast<uint8_t*>(stgB0);  // [256 rows][128 columns] e4m3
        const int qc = q * 32 + l16;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = r0 + rb * 16 + rq + j;
                const float amax = fmaxf(fmaxf(red[row], red[256 + row]), fmaxf(red[512 + row], red[768 + row]));
                const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
                qs[row * 128 + qc] = f32_to_e4m3(acc[rb][0][j] / sc);
                qs[row * 128 + qc + 16] = f32_to_e4m3(acc[rb][1][j] / sc);
                if (q == 0 && l16 == 0 && row < M) p.out_scale[(size_t)(row0 + row) * NB + n0 / BK] = sc;
            }
        __syncthreads();
        // coalesced 16-byte stores of the tile's M rows x 128 h columns
        uint8_t* h = static_cast<uint8_t*>(p.out);
        const i32x4* qv = reinterpret_cast<const i32x4*>(qs);
        for (int c = threadIdx.x; c < M * 8; c += NTH) {
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<i32x4*>(h + (size_t)(row0 + row) * N + n0 + ch * 16) = qv[c];
        }
    } else {
        // y through LDS, 16 rows at a time: each wave stages its 16 x 64 block
        // (fp32, 4 KiB of B buffer 0) with the 16-column groups of a row
        // XOR-ed by bits 2..3 of the row, so the four row groups of a store
        // instruction and the 16 lanes of a row's read touch distinct banks;
        // then every lane stores 4 columns (8 B bf16 / 16 B fp32).  LDS
        // operations of one wave are processed in order.
        float* st = reinterpret_cast<float*>(stgB0 + wave * 256);
        const int cw = n0 + q * 64;  // first output column of this wave
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int row = rq + j;  // bits 2..3 of row are lane / 16
                    st[row * 64 + ((cb * 16 + l16) ^ (((row >> 2) & 3) << 4))] = acc[rb][cb][j];
                }
            // the staged values are read by other lanes of this wave: keep the
            // compiler from moving the reads above the writes (no wait is needed)
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int qq = it * 64 + lane;  // chunk qq: row qq / 16, columns 4 (qq % 16) .. + 3
                const int row = qq >> 4, c4 = (qq & 15) * 4;
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * 64 + (c4 ^ (((row >> 2) & 3) << 4)));
                const int grow = r0 + rb * 16 + row, col = cw + c4;
                if (grow < M && col < N) {
                    const size_t o = (size_t)(row0 + grow) * N + col;
                    if (p.out_f32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = v;
                    } else {
                        const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                        const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(lo, hi);
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // reads before the next block's writes
        }
    }
}

template <int MODE>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
ffn_gemm_fp8(Fp8Args p) {
    const int L = xcd_remap(blockIdx.x, p.n_tiles[0] * p.NT);
    if (L < 0) return;
    const int2 wl = p.work[L];
    const int4 td = p.tiles[wl.x];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const int n0 = MODE == 0 ? wl.y * (BN / 2) : wl.y * BN;
    if (n0 >= p.N || M <= 0) return;
    run_tile<MODE>(p, g, row0, M, n0);
}

}  // namespace

hipError_t launch_gemm_fp8(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                           const float* x_scale, const int32_t* offsets, const moe_weights& w, void* y_rows,
                           const FfnWork& wk, void* h, float* h_scale, hipStream_t s) {
    hipError_t e0 = launch_build_tiles(c, offsets, BM, n_rows_cap, wk, s);
    if (e0 != hipSuccess) return e0;
    Fp8Args a{};
    a.tiles = reinterpret_cast<const int4*>(wk.tiles);
    a.n_tiles = wk.n_tiles;
    // GEMM1: gate/up + SwiGLU -> h (e4m3) and its row-block scales
    a.work = reinterpret_cast<const int2*>(wk.work1);
    a.NT = wk.nt1;
    a.a = static_cast<const uint8_t*>(x_rows);
    a.a_scale = x_scale;
    a.w0 = static_cast<const uint8_t*>(w.w_gate);
    a.w1 = static_cast<const uint8_t*>(w.w_up);
    a.s0 = w.s_gate;
    a.s1 = w.s_up;
    a.out = h;
    a.out_scale = h_scale;
    a.K = c.H;
    a.N = c.I;
    const int64_t grid1 = max_tiles * wk.nt1;
    hipLaunchKernelGGL(ffn_gemm_fp8<0>, dim3((unsigned)grid1), dim3(NTH), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // GEMM2: down projection of h
    a.work = reinterpret_cast<const int2*>(wk.work2);
    a.NT = wk.nt2;
    a.a = static_cast<const uint8_t*>(h);
    a.a_scale = h_scale;
    a.w0 = static_cast<const uint8_t*>(w.w_down);
    a.w1 = nullptr;
    a.s0 = w.s_down;
    a.s1 = nullptr;
    a.out = y_rows;
    a.out_scale = nullptr;
    a.K = c.I;
    a.N = c.H;
    a.out_f32 = c.y_dtype == MOE_F32 ? 1 : 0;
    const int64_t grid2 = max_tiles * wk.nt2;
    hipLaunchKernelGGL(ffn_gemm_fp8<1>, dim3((unsigned)grid2), dim3(NTH), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
