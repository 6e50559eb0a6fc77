// gemm_fp8.hip -- the grouped SwiGLU FFN on e4m3 rows with MXFP4 expert weights
// ("ASAP", section 3.4.2: the MoE kernel is a grouped matrix multiplication of
// hidden states by the layer's expert weights; the 4-bit expert weights of
// "DWDP", appendix A4).  Rows are e4m3 codes with one fp32 scale per 1 x 128
// block of a row (x, h); weights are OCP MX: E2M1 codes, one E8M0 scale per 32
// elements of a row.  (e4m3 weights run in gemm_e4m3.hip.)
//
// MFMA.  v_mfma_scale_f32_16x16x128_f8f6f4 in its FP4 x e4m3 form applies each
// lane's E8M0 weight scale itself; a K block of 128 is one MFMA and one row
// scale block, so every MFMA result t is folded in as acc += t * s_row on the
// VALU (this file is compiled in the VGPR form).  The weight fragment is the
// first operand and the row fragment the second, so a 16 x 16 result comes out
// transposed: lane l holds row l % 16 and the four weight rows 4 (l / 16) +
// [0, 4).
//
// Tile.  256 rows (128 for launches of small groups) x 256 weight rows, 8 waves
// (two per SIMD); wave w owns rows TB / 2 (w / 4) + [0, TB / 2) and weight rows
// 64 (w % 4) + [0, 64): TB / 32 x 4 MFMA blocks of 16 x 16 and their fp32
// accumulators.  GEMM1: the 64 weight rows of a wave are 32 gate rows then the
// 32 up rows of the same h columns, so h = silu(g) * u forms in registers;
// GEMM2: 64 output columns.  A wave issues MFMAs only for the 32-row units of
// its half that hold rows of the group (the tile body is specialised on their
// count); the rest of its accumulators stay zero.
// Pipeline.  K advances in stages of 128 through three A buffers [256 x 128 B |
// 288 row scales] and two weight buffers [256 x 64 B | 8 x 256 B of E8M0
// scales]; operands move HBM -> LDS by buffer_load ... lds, both two stages
// ahead: A of stage s+2 at the start of stage s (its buffer held stage s-1),
// the weights of stage s+2 as soon as every wave has read its fragments of
// stage s into registers.  Chunks outside the tile (rows past the group's end,
// weight rows past N) carry an offset beyond their buffer descriptor and load
// as zero.  A rows in LDS: 16-byte chunks XOR-swizzled by (row & 7) ^ ((row >>
// 3) & 1), so a 16-byte read served eight lanes (128 B) at a time lands the
// eight rows of a group, at one logical chunk, on eight distinct 16-byte bank
// groups (so do the two row parities of 16 lanes).
// GEMM1 epilogue: h is requantised per row and 128 columns -- the tile's 128 h
// columns are one scale block: s = max|h| / 448 (1 for an all-zero block),
// q = e4m3_rne_sat(h / s) -- staged through LDS and stored as 16-byte chunks.
#include "common.hpp"

namespace moe {
namespace {

// kBig: the tallest tile (it sizes the LDS); a launch runs tiles of TB = kBig
// or kFfnBmFp8Small rows (the template parameter TB below), a wave owning
// TB / 32 row blocks of 16.
constexpr int kBig = 256, BN = 256, BK = 128, NTH = 512;
constexpr int kChunksA = kBig * 8;             // 16-byte chunks of A in one stage
constexpr int kStageA = kChunksA + 72;         // A, then 288 fp32 row scales (see scale_row)
constexpr int kScaleB4 = BN * 4;               // chunks of a stage's weight codes; then 8 x 256 B of scales
constexpr int kChunksB = kScaleB4 + 128;
static_assert(kFfnBmFp8Small == 128, "the load slots below are laid out for 4 and 8 row blocks");
constexpr uint32_t kOOB = 0x80000000u;         // past every descriptor (all are < 2 GiB): the load returns zero

typedef __attribute__((address_space(3))) void* lds_t;

// The stage buffers (distinct objects, so that the compiler can tell which
// buffer an in-flight LDS DMA writes); both tile heights use them.
__shared__ i32x4 stgA0[kStageA];
__shared__ i32x4 stgA1[kStageA];
__shared__ i32x4 stgA2[kStageA];
__shared__ i32x4 stgB0[kChunksB];
__shared__ i32x4 stgB1[kChunksB];

template <int BUF>
__device__ __forceinline__ i32x4* stgA() {
    if constexpr (BUF == 0) return stgA0;
    else if constexpr (BUF == 1) return stgA1;
    else return stgA2;
}
template <int BUF>
__device__ __forceinline__ i32x4* stgB() {
    if constexpr (BUF == 0) return stgB0;
    else return stgB1;
}

__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// FP4 (E2M1) first operand with the lane's E8M0 scale sw, e4m3 second operand
// at scale 1 (E8M0 127).  The FP4 operand of lane l holds row l % 16, elements
// 32 (l / 16) + [0, 32) of the K block (low nibble first); the matching e4m3
// operand of lane l holds column l % 16 at elements 16 (l / 16) + [0, 16) in
// its first 16 bytes and 64 + 16 (l / 16) + [0, 16) in the last 16 (measured:
// an in-bounds probe of one MFMA against a host product).
__device__ __forceinline__ f32x4 mfma16x16x128_fp4_fp8(i32x8 w4, i32x8 a8, int sw) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w4, a8, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, sw, 0, 127);
}

struct Fp8Args {
    const uint8_t* a;       // GEMM1: x rows [rows][H]; GEMM2: h [rows][I]
    const float* a_scale;   // [rows][K / 128]
    const uint8_t* w0;      // GEMM1: w_gate [E][I][H/2]; GEMM2: w_down [E][H][I/2] (E2M1 pairs)
    const uint8_t* w1;      // GEMM1: w_up [E][I][H/2]
    const uint8_t* s0;      // E8M0: GEMM1 s_gate [E][I][H/32]; GEMM2 s_down [E][H][I/32]
    const uint8_t* s1;      // GEMM1: s_up
    void* out;              // GEMM1: h [rows][I] e4m3; GEMM2: y [rows][H]
    float* out_scale;       // GEMM1: h scales [rows][I / 128]
    const int4* tiles;
    const int32_t* n_tiles;
    const int2* work;       // {M tile, N tile} in launch order
    int NT;                 // N tiles per M tile
    int K, N;               // GEMM1: K = H, N = I; GEMM2: K = I, N = H
    int out_f32;            // GEMM2 output dtype
    WTab wt;                // wt.tab != NULL: w0, w1, s0, s1 of group g are table entries
    int slot0, slot1;       //   slot0, slot1, slot0 + 3, slot1 + 3
    const int32_t* a_row_src;  // GEMM1: non-NULL -> a is x [a_rows][K], row r of A is x row a_row_src[r] / a_row_k
    int a_row_k, a_rows;
};

// Row scales of a stage in LDS: position P = 128 h + 64 (rb / 4) + 4 l + rb % 4
// holds the scale of tile row scale_row(P) = (TB / 2) h + 16 rb + l, so the
// scales a lane needs (rows 16 rb + lane % 16 of its half h) are at most two
// 16-byte chunks, and the 16 lanes of a row group read 16 consecutive chunks.
// Positions whose row lies past the tile (the second half's rb >= TB / 32,
// P >= 256) hold zeros; in the first half such positions repeat rows of the
// second.
template <int TB>
__device__ __forceinline__ int scale_row(int pos) {
    const int rb = ((pos >> 6) & 1) * 4 + (pos & 3), l = (pos >> 2) & 15;
    return (TB / 2) * (pos >> 7) + 16 * rb + l;
}

struct Dma {
    __amdgpu_buffer_rsrc_t ra, rs, rb0, rb1;
    __amdgpu_buffer_rsrc_t rsb0, rsb1;  // MXFP4: the weight rows' E8M0 scales
    uint32_t va[4], vb[4], vs, vbs;
    int nsteps;  // K blocks
};

// Loads a wave issues per stage: 4 A chunk loads, the row scales, then 2
// weight chunk loads and the weight scales.
constexpr int kLoads = 8;

// A loads of stage t into A buffer BUF: 4 chunk loads per lane (8 LDS rows
// each) and one row-scale load, the same 5 for every wave.  The tile's TB rows
// take TB / 8 chunk loads (32 or 16); in 128-row tiles the second four waves
// repeat the first four's loads, writing the same bytes to the same place.
// Wave w loads the scales of rows 32 w + [0, 64): each row's scale is written
// by two waves, again the same value, and rows past the tile load zeros.
// Every destination is an offset into the buffer itself, so the compiler can
// tell the buffers apart while the loads are in flight.
//
// Load J (0..7) of the 8 a wave issues per stage t: J < 4 the A chunk loads,
// J = 4 the row-scale load (both into A buffer ABUF); J = 5, 6 fill the wave's
// 32 weight rows of B buffer BBUF (a weight row of a stage is 64 bytes: four
// chunks, swizzled by (row >> 2) & 3), 16 rows at a time, and J = 7 loads the
// rows' E8M0 scales of the stage (one dword a row: the four 32-element blocks)
// into the wave's 256-byte slot after the codes, lanes 32 .. 63 loading zeros
// into its unused half.  A load that is not real (a stage past the end, rows
// past the tile) carries an offset past its descriptor and loads zeros.
template <int MODE, int ABUF, int BBUF, int J, int TB>
__device__ __forceinline__ void dma1(const Dma& d, int t, int wave) {
    const uint32_t k = (uint32_t)t * BK;
    const bool real = t < d.nsteps;
    if constexpr (J < 4) {
        const uint32_t off = (!real || d.va[J] == kOOB) ? kOOB : d.va[J] + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_t)(stgA<ABUF>() + ((wave * 4 + J) % (TB / 8)) * 64), 16,
                                                 off, 0, 0, 0);
    } else if constexpr (J == 4) {
        const uint32_t so = (!real || d.vs == kOOB) ? kOOB : d.vs + (uint32_t)t * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_t)(stgA<ABUF>() + kChunksA + wave * 8), 4, so, 0, 0, 0);
    } else if constexpr (J < 7) {
        // GEMM1: even waves fill gate rows, odd waves the up rows of the same h columns
        const __amdgpu_buffer_rsrc_t r = (MODE == 0 && (wave & 1)) ? d.rb1 : d.rb0;
        constexpr int i = J - 5;
        const uint32_t off = (!real || d.vb[i] == kOOB) ? kOOB : d.vb[i] + k / 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t)(stgB<BBUF>() + (wave * 2 + i) * 64), 16, off, 0, 0, 0);
    } else {
        const __amdgpu_buffer_rsrc_t rs = (MODE == 0 && (wave & 1)) ? d.rsb1 : d.rsb0;
        const uint32_t off = (!real || d.vbs == kOOB) ? kOOB : d.vbs + (uint32_t)t * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t)(stgB<BBUF>() + kScaleB4 + wave * 16), 4, off, 0, 0, 0);
    }
}

// The A loads (J = 0..4) of stage t into A buffer BUF.
template <int MODE, int BUF, int TB>
__device__ __forceinline__ void dma_a(const Dma& d, int t, int wave) {
    dma1<MODE, BUF, 0, 0, TB>(d, t, wave);
    dma1<MODE, BUF, 0, 1, TB>(d, t, wave);
    dma1<MODE, BUF, 0, 2, TB>(d, t, wave);
    dma1<MODE, BUF, 0, 3, TB>(d, t, wave);
    dma1<MODE, BUF, 0, 4, TB>(d, t, wave);
}

// The B loads (J = 5 .. kLoads - 1) of stage t into B buffer BUF.
template <int MODE, int BUF, int TB>
__device__ __forceinline__ void dma_b(const Dma& d, int t, int wave) {
    dma1<MODE, 0, BUF, 5, TB>(d, t, wave);
    dma1<MODE, 0, BUF, 6, TB>(d, t, wave);
    dma1<MODE, 0, BUF, 7, TB>(d, t, wave);
}

// vmcnt(kLoads) with the other counters at zero: a stage's A and B loads and
// everything before them have landed (the loads of the next stage may be in
// flight), and every LDS read of this wave has returned.
__device__ __forceinline__ void wait_stage() { __builtin_amdgcn_s_waitcnt(kLoads | 0x0070); }

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// acc += t * s_row for one row block (the weight scales are applied by the
// MFMA): sa is this lane's row scale.
__device__ __forceinline__ void promote(const f32x4 (&t)[4], float sa, f32x4 (&acc)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[0][j] = __builtin_fmaf(t[0][j], sa, acc[0][j]);
        acc[1][j] = __builtin_fmaf(t[1][j], sa, acc[1][j]);
        acc[2][j] = __builtin_fmaf(t[2][j], sa, acc[2][j]);
        acc[3][j] = __builtin_fmaf(t[3][j], sa, acc[3][j]);
    }
}

// The FP4 fragment of column block cb is the lane's 32 elements of
// row (16 cb + lane % 16), K block lane / 16 of the stage: logical chunk
// lane / 16 of the 64-byte LDS row, the low four dwords of the operand; its
// E8M0 scale is byte lane / 16 of the row's scale dword.
template <int BUF, int TB>
__device__ __forceinline__ void read_b4(int q, int lane, i32x8 (&b)[4], int (&bs)[4]) {
    const i32x4* buf = stgB<BUF>();
    const int l16 = lane & 15, g = lane >> 4;
    const int ib = ((q & 3) * 64 + l16) * 4 + (g ^ ((l16 >> 2) & 3));  // column block cb: + cb * 64
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(buf + kScaleB4);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const i32x4 v = buf[ib + cb * 64];
        b[cb] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        const int row = (q & 3) * 64 + cb * 16 + l16;  // LDS row; its dword in slot row / 32
        bs[cb] = (int)((sc[(row >> 5) * 64 + (row & 31)] >> (8 * g)) & 0xFFu);
    }
}

// The loads of stage t spread over the row blocks of a K stage, J after the
// MFMAs of row block rb -- 8 row blocks: two after each of the first three,
// one after each of the next two; 4 row blocks: three, two, two, one.  A wave that issues all 8 at once stalls until the texture unit has
// taken them, and the other waves' loads are queued there too.
template <int RBN, int NJ>
constexpr int slot_start(int r) {
    const int j = RBN >= 6 ? (r < 3 ? 2 * r : r + 3) : (r == 0 ? 0 : 1 + 2 * r);
    return j < NJ ? j : NJ;
}
template <int MODE, int NA, int NB, int RBI, int TB>
__device__ __forceinline__ void dma_slot(const Dma& d, int t, int wave) {
    constexpr int j0 = slot_start<TB / 32, kLoads>(RBI), j1 = slot_start<TB / 32, kLoads>(RBI + 1);
    if constexpr (j0 < j1) dma1<MODE, NA, NB, j0, TB>(d, t, wave);
    if constexpr (j0 + 1 < j1) dma1<MODE, NA, NB, j0 + 1, TB>(d, t, wave);
    if constexpr (j0 + 2 < j1) dma1<MODE, NA, NB, j0 + 2, TB>(d, t, wave);
}

// One K stage for the RB row blocks of 16 starting at tile row r0: every (row
// block, column block) MFMA of this wave's first LRB row blocks (those that
// hold rows of the tile), promoted with the stage's row scales, with the
// loads of stage t into A buffer NA and B buffer NB issued between them (at
// the slots of all RB row blocks, the MFMAs of the rest left out).
// Software-pipelined over row blocks: the fragments of rb + 1 are read just
// before the four MFMAs of rb issue, and rb - 1 is promoted while they run.
// The weight operand is FP4 with its E8M0 scales bs applied by the MFMA; the
// row fragment takes chunks lane / 16 and lane / 16 + 4 of the row (the K
// order the FP4 x e4m3 form expects).
template <int MODE, int BUF, int NA, int NB, int TB, int LRB>
__device__ __forceinline__ void kstep(const Dma& d, int t_stage, int wave, int r0, int lane, const i32x8 (&b)[4],
                                      const int (&bs)[4], f32x4 (&acc)[TB / 32][4]) {
    constexpr int RB = TB / 32;
    static_assert(LRB >= 0 && LRB <= RB, "live row blocks");
    // Every access indexes the stage buffer itself (an integer base plus a
    // constant), so the compiler can tell it from the DMA in flight into the
    // other buffers and adds no wait for it.
    const i32x4* buf = stgA<BUF>();
    const int l16 = lane & 15;
    const int plo = (lane >> 4) ^ swz8(l16);
    const int phi = ((lane >> 4) + 4) ^ swz8(l16);
    const int ia = (r0 + l16) * 8;                      // row block rb: + rb * 128
    // this lane's row scales: row blocks 0..3 in chunk 32 h + l16, 4..7 in 32 h + 16 + l16
    const int is = kChunksA + (r0 / (TB / 2)) * 32 + l16;
    const f32x4 sa_lo = __builtin_bit_cast(f32x4, buf[is]), sa_hi = __builtin_bit_cast(f32x4, buf[is + 16]);
    auto sa = [&](int rb) { return rb < 4 ? sa_lo[rb & 3] : sa_hi[rb & 3]; };
    i32x8 a[2];
    f32x4 t[2][4];
    if constexpr (LRB > 0) a[0] = cat(buf[ia + plo], buf[ia + phi]);
    __builtin_amdgcn_sched_barrier(0);
    static_assert(RB == 4 || RB == 8, "the load slots are laid out for 4 and 8 row blocks");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        // the fragment of rb + 1 goes to the register the MFMAs of rb - 1 read
        if (rb + 1 < LRB) a[(rb + 1) & 1] = cat(buf[ia + (rb + 1) * 128 + plo], buf[ia + (rb + 1) * 128 + phi]);
        if (rb < LRB) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) t[rb & 1][cb] = mfma16x16x128_fp4_fp8(b[cb], a[rb & 1], bs[cb]);
        }
        switch (rb) {  // rb is a constant here: the loop is unrolled
            case 0: dma_slot<MODE, NA, NB, 0, TB>(d, t_stage, wave); break;
            case 1: dma_slot<MODE, NA, NB, 1, TB>(d, t_stage, wave); break;
            case 2: dma_slot<MODE, NA, NB, 2, TB>(d, t_stage, wave); break;
            case 3: dma_slot<MODE, NA, NB, 3, TB>(d, t_stage, wave); break;
            case 4: dma_slot<MODE, NA, NB, 4, TB>(d, t_stage, wave); break;
            case 5: dma_slot<MODE, NA, NB, 5, TB>(d, t_stage, wave); break;
            default: break;
        }
        if (rb > 0 && rb - 1 < LRB) promote(t[(rb - 1) & 1], sa(rb - 1), acc[rb - 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LRB == RB) promote(t[(RB - 1) & 1], sa(RB - 1), acc[RB - 1]);
}

// Rows of a tile past the group's end load as zero.  A wave computes the 32-row
// units of its half of the tile that hold rows (LU of them; a wave whose half
// holds none issues no MFMA) and accumulates zeros for the rest, while every
// wave keeps the full load schedule, so the compiler's count of loads in
// flight stays exact.
template <int MODE, int TB, int LU>
__device__ __forceinline__ void run_tile(const Fp8Args& p, int g, int row0, int M, int n0) {
    constexpr int RB = TB / 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mh = wave >> 2, q = wave & 3, r0 = mh * (TB / 2);
    const int K = p.K, N = p.N;
    const int KB = K / BK;  // K and N are multiples of 128
    Dma d;
    d.nsteps = KB;
    // ---- A rows row0 .. row0 + M and their row scales; indexed (GEMM1 of the
    // layer): the descriptors span all of x and its scales, and row r of the
    // tile is token row_src[row0 + r] / k (rows with row_src -1, the segment
    // padding, load as zero)
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
    {
        const int pos = wave * 32 + lane;  // < 288: the scale area of a stage
        const int r = a_row(pos < 256 ? scale_row<TB>(pos) : TB);
        d.vs = r >= 0 ? (uint32_t)r * (uint32_t)KB * 4u : kOOB;
    }
    // ---- B: GEMM1 the gate and up rows n0 + [0, 128) (LDS quarter j holds gate
    // rows 32 j + [0, 32) then the up rows of the same h columns); GEMM2 the
    // weight rows n0 + [0, 256)
    const int nlim = MODE == 0 ? min(N - n0, 128) : min(N - n0, BN);
    // this group's codes and E8M0 scales, and its index in them
    const uint8_t *w0 = p.w0, *w1 = p.w1;
    const uint8_t *s0 = p.s0, *s1 = p.s1;
    int ge = g;
    if (p.wt.tab) {
        const int lay = *p.wt.layer;
        w0 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot0));
        s0 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot0 + 3));
        if (MODE == 0) {
            w1 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot1));
            s1 = static_cast<const uint8_t*>(wtab_ptr(p.wt, lay, g, p.slot1 + 3));
        }
        ge = 0;
    }
    const int KW = K / 2;  // bytes of a weight row
    const size_t mat = (size_t)N * KW;
    d.rb0 = make_rsrc(w0 + (size_t)ge * mat + (size_t)n0 * KW, (uint32_t)nlim * (uint32_t)KW);
    d.rb1 = MODE == 0 ? make_rsrc(w1 + (size_t)ge * mat + (size_t)n0 * KW, (uint32_t)nlim * (uint32_t)KW) : d.rb0;
    // A loads i: LDS row 32 wave + 8 i + lane / 8 (modulo TB), physical chunk
    // lane % 8 holding logical chunk (lane % 8) ^ swz8(row)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int arow = (wave * 32 + i * 8 + (lane >> 3)) % TB;
        const int ar = a_row(arow);
        d.va[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)K + (uint32_t)(((lane & 7) ^ swz8(arow)) * 16) : kOOB;
    }
    // B loads i = 0, 1: LDS rows 32 wave + 16 i + lane / 4, physical chunk
    // lane % 4 holding logical chunk (lane % 4) ^ ((row >> 2) & 3); GEMM1: even
    // waves the gate rows, odd waves the up rows of h columns 32 (wave / 2) ..
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = wave * 32 + i * 16 + (lane >> 2);
        const int wrow = MODE == 0 ? (wave >> 1) * 32 + i * 16 + (lane >> 2) : row;  // relative to n0
        const uint32_t logical = (uint32_t)(((lane & 3) ^ ((row >> 2) & 3)) * 16);
        d.vb[i] = wrow < nlim ? (uint32_t)wrow * (uint32_t)KW + logical : kOOB;
    }
    // E8M0 scales [rows][K / 32]: lane < 32 loads the stage's dword of LDS row 32 wave + lane
    {
        const uint8_t* sb1 = MODE == 0 ? s1 : s0;
        const size_t smat = (size_t)N * (K / 32);
        d.rsb0 = make_rsrc(s0 + (size_t)ge * smat + (size_t)n0 * (K / 32), (uint32_t)nlim * (uint32_t)(K / 32));
        d.rsb1 = MODE == 0 ? make_rsrc(sb1 + (size_t)ge * smat + (size_t)n0 * (K / 32),
                                       (uint32_t)nlim * (uint32_t)(K / 32))
                           : d.rsb0;
        const int wrow = MODE == 0 ? (wave >> 1) * 32 + lane : wave * 32 + lane;
        d.vbs = (lane < 32 && wrow < nlim) ? (uint32_t)wrow * (uint32_t)(K / 32) : kOOB;
    }

    f32x4 acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Stage s uses A buffer s % 3 and B buffer s % 2; the loop body is the six
    // stages of one period of both rings and leaves after stage KB - 1.  Loads
    // of stages past the end carry zeros.  Issue order: A0, B0, A1, B1, then per
    // stage s, during its MFMAs: A(s+2) (5 loads), B(s+2) (3).
    dma_a<MODE, 0, TB>(d, 0, wave);
    dma_b<MODE, 0, TB>(d, 0, wave);
    dma_a<MODE, 1, TB>(d, 1, wave);
    dma_b<MODE, 1, TB>(d, 1, wave);
    i32x8 b[4];
    int bs[4] = {127, 127, 127, 127};
    int s = 0;
    auto stage = [&](auto ab, auto bb) {
        constexpr int AB = decltype(ab)::value, BB = decltype(bb)::value;
        wait_stage();  // stage s has landed (this wave's loads); this wave's reads of stage s-1 are done
        barrier_lds();     // ... every wave's: A buffer (s+2) % 3 is free
        read_b4<BB, TB>(q, lane, b, bs);
        wait_lgkm0();
        barrier_lds();  // every wave holds its B fragments of stage s: B buffer s % 2 is free
        kstep<MODE, AB, (AB + 2) % 3, BB, TB, 2 * LU>(d, s + 2, wave, r0, lane, b, bs, acc);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    stage(C0{}, C0{});
    while (++s < KB) {
        stage(C1{}, C1{});
        if (++s >= KB) break;
        stage(C2{}, C0{});
        if (++s >= KB) break;
        stage(C0{}, C1{});
        if (++s >= KB) break;
        stage(C1{}, C0{});
        if (++s >= KB) break;
        stage(C2{}, C1{});
        if (++s >= KB) break;
        stage(C0{}, C0{});
    }
    wait_vm0();  // no LDS DMA may outlive the workgroup
    barrier_lds();

    // A lane holds row r0 + 16 rb + l16 of its row blocks and, in column block
    // cb, the four columns 16 cb + g4 + [0, 4) of its 64 weight rows.
    const int l16 = lane & 15;
    if (MODE == 0) {
        // h = silu(g) * u for h columns n0 + 32 q + 16 c + g4 + j, c = 0, 1
        float rmax[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[rb][0][j] = silu_f(acc[rb][0][j]) * acc[rb][2][j];
                acc[rb][1][j] = silu_f(acc[rb][1][j]) * acc[rb][3][j];
                m = fmaxf(m, fmaxf(fabsf(acc[rb][0][j]), fabsf(acc[rb][1][j])));
            }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            rmax[rb] = m;
        }
        // per-row maxima of the four quarters' 32 columns -> LDS [4][256]
        float* red = reinterpret_cast<float*>(stgA<0>());
        if (lane < 16)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) red[q * 256 + r0 + rb * 16 + l16] = rmax[rb];
        __syncthreads();
        // [TB rows][128 columns] e4m3, 32 words a row, the 16-byte chunk c of row r
        // at chunk c ^ ((r >> 1) & 7): a 4-byte store of 16 rows x 4 words then
        // touches 64 distinct banks
        uint32_t* qs = reinterpret_cast<uint32_t*>(stgA<1>());
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = r0 + rb * 16 + l16;
            const float amax = fmaxf(fmaxf(red[row], red[256 + row]), fmaxf(red[512 + row], red[768 + row]));
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t w = e4m3x4_rne_sat(acc[rb][c][0] / sc, acc[rb][c][1] / sc, acc[rb][c][2] / sc,
                                                  acc[rb][c][3] / sc);
                qs[row * 32 + (((q * 2 + c) ^ ((row >> 1) & 7)) << 2) + (lane >> 4)] = w;
            }
            if (q == 0 && lane < 16 && row < M) p.out_scale[(size_t)(row0 + row) * (N / BK) + n0 / BK] = sc;
        }
        __syncthreads();
        // coalesced 16-byte stores of the tile's M rows x 128 h columns
        uint8_t* h = static_cast<uint8_t*>(p.out);
        const i32x4* qv = reinterpret_cast<const i32x4*>(qs);
        for (int c = threadIdx.x; c < M * 8; c += NTH) {
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<i32x4*>(h + (size_t)(row0 + row) * N + n0 + ch * 16) = qv[row * 8 + (ch ^ ((row >> 1) & 7))];
        }
    } else if (!p.out_f32) {
        // bf16 y through LDS, 32 rows of each half of the tile at a time, by all
        // eight waves into one [64 rows][256 columns] image (image row 32 h + i
        // is tile row TB / 2 * h + 32 u + i; two A buffers, one barrier a
        // round), then stored as whole rows of the tile.  The 16-byte chunk c
        // of image row r sits at chunk c ^ (r & 15): a wave's writes (16 rows x
        // 2 chunks) and its reads (two whole rows) both spread over every bank.
        uint16_t* y = static_cast<uint16_t*>(p.out);
        const int tid = threadIdx.x, g4 = lane >> 4;
#pragma unroll
        for (int u = 0; u < RB / 2; ++u) {
            uint32_t* st = reinterpret_cast<uint32_t*>(u & 1 ? stgA<1>() : stgA<0>());
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int r = 32 * mh + 16 * hb + l16;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const f32x4 v = acc[2 * u + hb][cb];
                    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                    const int c = 8 * q + 2 * cb + (g4 >> 1);
                    *reinterpret_cast<uint2*>(st + r * 128 + ((c ^ (r & 15)) << 2) + (g4 & 1) * 2) =
                        make_uint2(lo, hi);
                }
            }
            // the round is staged; the other buffer's reads (round u - 1) came
            // before every thread's writes above, so it is free for round u + 1
            __syncthreads();
            const i32x4* sv = reinterpret_cast<const i32x4*>(st);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int id = k * NTH + tid;
                const int r = id >> 5, c = id & 31;
                const int row = (r >> 5) * (TB / 2) + 32 * u + (r & 31), col = n0 + c * 8;
                // non-temporal: y is read again only by the combine, after the launch
                if (row < M && col < N)
                    __builtin_nontemporal_store(sv[r * 32 + (c ^ (r & 15))],
                                                reinterpret_cast<i32x4*>(y + (size_t)(row0 + row) * N + col));
            }
        }
    } else {
        // fp32 y through LDS, 16 rows at a time: each wave stages its 16 x 64 block
        // (fp32, 4 KiB of B buffer 0; of A buffer 1 in 256-row tiles, whose B
        // buffers are smaller), row r's 16-byte chunk c at chunk c ^ r,
        // so the eight rows of a store group and the eight chunks of a row's
        // read group touch distinct banks; then every lane stores 4 columns
        // (8 B bf16 / 16 B fp32).  LDS operations of one wave are processed in
        // order.
        float* st = reinterpret_cast<float*>(stgA<1>() + wave * 256);
        const int cw = n0 + q * 64;  // first output column of this wave
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j)  // element stores: a whole-vector store here makes the compiler spill acc
                    st[l16 * 64 + ((4 * cb + (lane >> 4)) ^ l16) * 4 + j] = acc[rb][cb][j];
            // the staged values are read by other lanes of this wave: keep the
            // compiler from moving the reads above the writes (no wait is needed)
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int qq = it * 64 + lane;  // chunk qq: row qq / 16, columns 4 (qq % 16) .. + 3
                const int row = qq >> 4, c = qq & 15;
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * 64 + (c ^ row) * 4);
                const int grow = r0 + rb * 16 + row, col = cw + c * 4;
                if (grow < M && col < N)
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + (size_t)(row0 + grow) * N + col) = v;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // reads before the next block's writes
        }
    }
}

template <int MODE, int TB>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
ffn_gemm_fp8(Fp8Args p) {
    const int L = xcd_remap_runs(blockIdx.x, p.n_tiles[0] * p.NT);
    if (L < 0) return;
    if (p.wt.tab && wtab_layer(p.wt) < 0) return;
    const int2 wl = p.work[L];
    const int4 td = p.tiles[wl.x];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const int n0 = MODE == 0 ? wl.y * (BN / 2) : wl.y * BN;
    if (n0 >= p.N || M <= 0) return;
    // the 32-row units of this wave's half of the tile (rows TB / 2 * (w / 4) ..)
    // that hold rows of the group: a uniform branch per wave
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int live = M - (wave >> 2) * (TB / 2);
    const int lu = live <= 0 ? 0 : min((live + 31) >> 5, TB / 64);
    switch (lu) {
    case 0: run_tile<MODE, TB, 0>(p, g, row0, M, n0); break;
    case 1: run_tile<MODE, TB, 1>(p, g, row0, M, n0); break;
    case 2: run_tile<MODE, TB, 2>(p, g, row0, M, n0); break;
    default:
        if constexpr (TB / 64 >= 4) {
            if (lu == 3) run_tile<MODE, TB, 3>(p, g, row0, M, n0);
            else run_tile<MODE, TB, TB / 64>(p, g, row0, M, n0);
        }
        break;
    }
}

template <int MODE>
void launch_one(int tb, int64_t grid, const Fp8Args& a, hipStream_t s) {
    const dim3 gr((unsigned)grid), bl(NTH);
    if (tb == kFfnBmFp8Small) hipLaunchKernelGGL((ffn_gemm_fp8<MODE, kFfnBmFp8Small>), gr, bl, 0, s, a);
    else hipLaunchKernelGGL((ffn_gemm_fp8<MODE, kBig>), gr, bl, 0, s, a);
}

}  // namespace

hipError_t launch_gemm_fp8(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                           const float* x_scale, const int32_t* row_src, const int32_t* offsets,
                           const moe_weights& w, const WTab& wt, void* y_rows, const FfnWork& wk, void* h,
                           float* h_scale, hipStream_t s) {
    if (c.w_dtype != MOE_FP4_E2M1)  // e4m3 weights
        return launch_gemm_e4m3(c, max_tiles, n_rows_cap, x_rows, x_scale, row_src, offsets, w, wt, y_rows, wk, h,
                                h_scale, s);
    // Tile height: 256 rows, so a group of about 256 rows (the DeepSeek-V3
    // layer's 256 experts, 8 rows a token) streams its weights once; launches
    // whose groups average under about 136 rows take 128-row tiles.
    const int G = c.E + (c.has_shared ? 1 : 0);
    const bool small = n_rows_cap <= (int64_t)G * 136;
    const int tb = small ? kFfnBmFp8Small : kBig;
    hipError_t e0 = launch_build_tiles(c, offsets, tb, n_rows_cap, wk, s);
    if (e0 != hipSuccess) return e0;
    Fp8Args a{};
    a.wt = wt;
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
    a.s0 = reinterpret_cast<const uint8_t*>(w.s_gate);
    a.s1 = reinterpret_cast<const uint8_t*>(w.s_up);
    a.out = h;
    a.out_scale = h_scale;
    a.K = c.H;
    a.N = c.I;
    const int64_t grid1 = xcd_grid_runs(max_tiles * wk.nt1);
    launch_one<0>(tb, grid1, a, s);
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
    a.s0 = reinterpret_cast<const uint8_t*>(w.s_down);
    a.s1 = nullptr;
    a.out = y_rows;
    a.out_scale = nullptr;
    a.K = c.I;
    a.N = c.H;
    a.out_f32 = c.y_dtype == MOE_F32 ? 1 : 0;
    const int64_t grid2 = xcd_grid_runs(max_tiles * wk.nt2);
    launch_one<1>(tb, grid2, a, s);
    return hipGetLastError();
}

}  // namespace moe
