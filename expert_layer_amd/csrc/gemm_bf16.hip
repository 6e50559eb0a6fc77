// gemm_bf16.hip -- the grouped SwiGLU FFN on bf16 MFMA ("ASAP", section
// 3.4.2: the MoE kernel is a grouped matrix multiplication, hidden states on
// the left, the layer's expert weights on the right).
//
// Work list.  ffn_build_tiles turns the expert offsets into a device-side list
// of M tiles {group, row_begin, row_end}: an expert with n rows gets
// ceil(n / 288) tiles of equal height (rounded up to 32 rows), so a skewed
// expert spreads over many workgroups and a cold one costs one short tile.  The
// shared expert is one more group over all T tokens.  Nothing returns to the
// host: the grid is sized from the host-known bound and blocks past the
// device-side count exit at once.
//
// Tile.  Up to 288 rows x 256 weight rows, 8 waves, two per SIMD.  Each wave
// owns all rows of the tile and one 32-column MFMA block of weight rows
// (v_mfma_f32_32x32x16_bf16), so an expert of up to 288 rows -- nearly every
// expert of a DeepSeek-V3-sized layer at 8 192 tokens -- streams each weight
// panel in one tile, a short tile drops whole 32-row blocks, and the SIMDs stay
// equally loaded; the tile body is specialised on the number of 32-row blocks.
// The second wave on a SIMD issues its MFMAs while the first waits on LDS or
// the stage barrier.
//   GEMM1: wave w holds the gate (w < 4) or the up (w >= 4) rows of h columns
//          32 (w % 4) .. +31 of the tile; the pair meets through LDS at the
//          end and the gate wave forms h = silu(g) * u.
//   GEMM2: 256 output columns of y = h . w_down^T, fp32 or bf16.
//   GEMM2 with the combine (MODE 2, the layer's shared group, launched after
//          the routed groups' GEMM2): the shared expert's tile rows are token
//          rows, so the epilogue writes out = sum_j w_j y_j + y_shared itself
//          (the dispatch's counterpart of the fused row gather in GEMM1).
// Operand paths.  The rows (A) are shared by the eight waves and go through
// LDS; the weight rows of a wave are read by that wave alone, so they skip LDS
// and stream from HBM straight into a ring of register sets, one per stage, in
// MFMA fragment order (the tiled weight layout below makes each wave's stage
// one contiguous 2 KiB read).
// Pipeline.  K advances in 32-wide stages; NS stages are in flight: NS LDS
// buffers of 18 KiB for A, filled by buffer_load ... lds (no staging
// registers), and NS register sets of 8 VGPRs for B.  A stage's loads are
// issued NS - 1 stages ahead; a chunk outside the tile (rows past the expert's
// end, columns past N, the K tail, stages past the end) carries an offset
// beyond its buffer descriptor and loads as zero with no memory traffic.  Each
// stage has two 16-wide k steps; the A fragments of a row block are re-read
// for the next k step right after its MFMA has issued, so each read has a
// whole k step (of both waves on the SIMD) to land.  Between a stage's two k
// steps: wait for the next stage's A, one s_barrier, and reissue the drained A
// buffer; after a stage's last MFMA its B register set is reloaded.
// LDS chunks of 16 B are XOR-swizzled by row, physical chunk = logical ^
// ((row >> 1) & 3) ^ ((row >> 3) & 1): a fragment read of 16 consecutive rows
// (one pass of ds_read_b128 through the 64 banks of gfx950's LDS) touches 16
// distinct 16-byte bank groups, and so does any 8 consecutive rows.
// Launch order: the work list (see ffn_build_tiles) remapped so that runs of
// 32 consecutive items live on one XCD and share its L2, the eight XCDs
// working on neighbouring runs at any time (xcd_remap_runs).
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = kFfnBmBf16, BN = 256, BK = 32, NWAVES = 8, NTH = NWAVES * 64;
#ifndef MOE_GEMM1_STAGES
#define MOE_GEMM1_STAGES 4
#endif
#ifndef MOE_GEMM2_STAGES
#define MOE_GEMM2_STAGES 4
#endif
// Stages in flight (A: LDS buffers, B: register sets), per GEMM.  The loop
// runs in whole turns of the ring (stages past the end load zeros and still
// issue their MFMAs), so a depth that divides the stage count of the usual K
// (7168, 4096, 2048, 1536 are all multiples of 4 stages of 32) runs no zero
// stage; three stages of loads ahead cover the latency at every T measured.
template <int MODE>
constexpr int kStages = MODE == 0 ? MOE_GEMM1_STAGES : MOE_GEMM2_STAGES;
static_assert(kStages<0> >= 3 && kStages<0> <= 7 && kStages<1> >= 3 && kStages<1> <= 7,
              "ring depth: LDS holds up to seven A stages");
constexpr int kRowBlocks = BM / 32;      // 32-row MFMA blocks of a full tile
constexpr int kBlocks16 = BM / 16;       // 16-row DMA blocks of one A stage
static_assert(BM % 32 == 0 && kRowBlocks <= 9 && kBlocks16 <= 3 * NWAVES, "tile height");
// A stage buffer: the tile's rows, 64 B each.
constexpr int kSlots = kBlocks16 * 64;
// vector-memory instructions per wave per stage: up to three A blocks (blocks
// w, w + 8, w + 16 of the tile's) and two B fragments
constexpr int kLoadsA = 3, kLoadsB = 2;
constexpr uint32_t kOOB = 0x80000000u;   // past every descriptor (all are < 2 GiB): the load returns zero

typedef __attribute__((address_space(3))) void* lds_t;

// The A stage buffers.  They are distinct objects so that the compiler can
// tell which buffer an in-flight LDS DMA writes and never waits for a load
// into another buffer.
__shared__ i32x4 ring0[kSlots];
__shared__ i32x4 ring1[kSlots];
__shared__ i32x4 ring2[kSlots];
__shared__ i32x4 ring3[kSlots];
__shared__ i32x4 ring4[kSlots];
__shared__ i32x4 ring5[kSlots];
__shared__ i32x4 ring6[kSlots];

template <int BUF>
__device__ __forceinline__ i32x4* ring() {
    static_assert(BUF < 7, "ring buffer index");
    if constexpr (BUF == 0) return ring0;
    else if constexpr (BUF == 1) return ring1;
    else if constexpr (BUF == 2) return ring2;
    else if constexpr (BUF == 3) return ring3;
    else if constexpr (BUF == 4) return ring4;
    else if constexpr (BUF == 5) return ring5;
    else return ring6;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Workgroup barrier without a memory fence (a fence would wait for every
// in-flight LDS DMA); the clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 7 and lgkmcnt 15 mean no wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// lgkmcnt(0): every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// XOR pattern of the 16-byte chunks of an LDS row (only bits 1..3 of the row
// matter, so rows 16 apart share it): the tiled row layout's pattern.
__device__ __forceinline__ int swz_of_row(int row) { return tile_swz(row); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Operand layouts.
//  Row-major: [rows][K], K contiguous.
//  Tiled rows (x_perm, the shared expert's tokens, the h tile slots): 1 KiB
//    blocks of 16 rows x 32 k, block (rb, ks) at byte (rb * KS + ks) * 1024
//    with KS = ceil(K / 32), the 16-byte chunks inside a block already in the
//    LDS order (chunk c of row r at slot r * 4 + (c ^ swz_of_row(r))), zero
//    padded.  A tiled stage of 16 rows is one contiguous 1 KiB read.
//  Tiled weights (fragment order): the rows in groups of 64 (GEMM1: the 32
//    gate rows and the 32 up rows of 32 h columns; GEMM2: 64 rows of w_down),
//    group q, stage ks at byte (q * KS + ks) * 4096; inside, four 1 KiB MFMA
//    B fragments j = 2 * c + kk (c: 32-row half, kk: 16-wide k step), lane l's
//    16 bytes at l * 16 = row 32 c + l % 32, k = 32 ks + 16 kk + 8 (l / 32)
//    .. + 7.  Zero padded in rows and k.  A wave reads half c of a group: its
//    stage is the 2 KiB at byte (q * KS + ks) * 4096 + c * 2048.
struct GemmArgs {
    const uint16_t* a_routed;  // GEMM1: x rows (row-major or tiled); GEMM2: h tile slots (tiled)
    const uint16_t* a_shared;  // GEMM1: shared-expert tokens (row-major or tiled); GEMM2: h tile slots
    const uint16_t* w0_routed; // GEMM1: w_gate [E][I][H] or tiled w13; GEMM2: w_down [E][H][I] or tiled
    const uint16_t* w1_routed; // GEMM1: w_up (row-major only)
    const uint16_t* w0_shared;
    const uint16_t* w1_shared;
    void* out_routed;          // GEMM1: h tile slots; GEMM2: y_rows
    void* out_shared;          // GEMM1: h tile slots; GEMM2: y_shared
    const int4* tiles;
    const int32_t* n_tiles;
    int32_t* queue;            // the launch's work queue (see xcd_queue_pick)
    const int2* work;          // {M tile, N tile} in launch order
    int E;
    int NT;                    // N tiles per M tile in the launch grid
    int K_routed, K_shared;    // reduction length
    int N_routed, N_shared;    // GEMM1: h columns (I, I_sh); GEMM2: H
    int out_f32;               // GEMM2 output dtype
    int a_tiled_routed, a_tiled_shared;  // A operand layout of the two groups
    const int32_t* a_row_src;  // GEMM1, routed groups: non-NULL -> A row r is x row a_row_src[r] / a_row_k
    int a_row_k;
    int a_rows;                // rows of x (the indexed A operand)
    int w_tiled;               // weights tiled (fragment order)
    int h_slot_ks;             // k blocks of one h tile slot (ceil(max(I, I_sh) / 32))
    WTab wt;                   // wt.tab != NULL: w0 / w1 of group g are table entries slot0 / slot1
    int slot0, slot1;
    int part;                  // work items: 0 all, 1 the routed groups', 2 the shared group's
    // MODE 2 (the shared group's GEMM2 with the combine): out[t] = sum_j w[t][j] *
    // y_rows[tok_row[t][j]] + y_shared[t], y_shared the tile's own result
    // rounded to bf16, and y_rows the routed GEMM2's bf16 output
    const uint16_t* y_routed;
    const int32_t* tok_row;
    const float* topk_w;
    void* comb_out;
    int comb_k, comb_out_f32;
};

// Per-tile load state.  A: the buffer descriptor, the byte offsets of this
// lane's three 16-byte chunks in stage 0 and how far a stage moves them (64 B
// row-major, 1 KiB tiled).  B: the descriptor of the wave's 32 weight rows,
// this lane's offset in stage 0, and the per-stage and per-k-step moves
// (tiled: 4 KiB and 1 KiB; row-major: 64 B and 32 B).
struct Dma {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[kLoadsA];
    uint32_t vb;
    uint32_t sa, sb, kb;    // bytes per stage (A, B), bytes per k step (B)
    uint32_t kvalid_last;   // valid K columns in the last stage (multiple of 8)
    int nsteps;             // real stages
    int klim;               // B: this lane's loads of k step kk in stage t are real while 32 t + 16 kk < klim
    bool a_rm;              // row-major A: the K tail must be masked
};

// The 16-row block of an A stage that instruction i of wave w fills: blocks
// w, w + 8 and w + 16.  A tile of NRB row blocks has L = min(kBlocks16, 2 NRB)
// 16-row blocks, so wave w issues a_loads(NRB, w) = L / 8 + (w < L % 8) A
// instructions a stage, the first that many of its three; the tile body is
// specialised on whether the wave has the extra one, so every load it issues
// is real and its wait counts are exact.
__device__ __forceinline__ int a_block(int wave, int i) { return wave + NWAVES * i; }
template <int NRB>
constexpr int kTileBlocks16 = 2 * NRB < kBlocks16 ? 2 * NRB : kBlocks16;
template <int NRB, bool EXTRA>
constexpr int kLoadsAOf = kTileBlocks16<NRB> / NWAVES + (EXTRA ? 1 : 0);

// A load of stage t into buffer BUF, one instruction (i of the wave's A
// loads): row-major chunks of the K tail load zero (tiled operands are zero
// padded).
template <int BUF>
__device__ __forceinline__ void dma_a1(const Dma& d, int t, int lane, int i) {
    i32x4* buf = ring<BUF>();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool real = t < d.nsteps;
    const bool last = t == d.nsteps - 1;
    const uint32_t logical8 = (uint32_t)(((lane & 3) ^ swz_of_row(lane >> 2)) * 8);
    const bool a_ok = real & (!d.a_rm | !last | (logical8 < d.kvalid_last)) & (d.va[i] != kOOB);
    const uint32_t off = a_ok ? d.va[i] + (uint32_t)t * d.sa : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_t)(buf + a_block(wave, i) * 64), 16, off, 0, 0, 0);
}

// All NA A loads of stage t into buffer BUF.
template <int BUF, int NA>
__device__ __forceinline__ void dma_a(const Dma& d, int t, int lane) {
#pragma unroll
    for (int i = 0; i < NA; ++i) dma_a1<BUF>(d, t, lane, i);
}

// The cache policy of a buffer load with its non-temporal bit set.
constexpr int kCpolNT = 2;

// B fragments of stage t: q[kk] = k step kk of the wave's 32 weight rows.  A
// load is real while kk * 16 is below the lane's limit for the stage (no limit
// for the zero-padded tiled weights, the K tail for row-major ones, none at
// all past the last stage); the rest carry kOOB.  Selects only: a branch here
// would cost the wait counters their precision.  STREAM: non-temporal loads,
// for launches whose weight panels are each read by about one M tile.
template <bool STREAM>
__device__ __forceinline__ void load_b(const Dma& d, int t, i32x4 (&q)[2]) {
    const int lim = t < d.nsteps ? d.klim - t * BK : -1;
    const uint32_t base = (uint32_t)t * d.sb;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const uint32_t off = kk * 16 < lim ? d.vb + base + (uint32_t)kk * d.kb : kOOB;
        q[kk] = __builtin_amdgcn_raw_buffer_load_b128(d.rb, off, 0, STREAM ? kCpolNT : 0);
    }
}

// One fragment read of A: row block r of k step KK in buffer BUF (rows
// r * 32 + lane % 32 at logical chunk 2 * KK + lane / 32).
template <int BUF, int KK>
__device__ __forceinline__ i32x4 read_a1(int lane, int r) {
    const i32x4* buf = ring<BUF>();
    const int l32 = lane & 31, half = lane >> 5;
    return buf[(r * 32 + l32) * 4 + ((KK * 2 + half) ^ swz_of_row(l32))];
}

// vmcnt after which this wave's NA A loads of the next stage have landed: the
// loads issued after them are that stage's B loads and the A and B loads of
// the NS - 2 stages after it.
template <int NS, int NA>
constexpr int kWaitNextA = kLoadsB + (NA + kLoadsB) * (NS - 2);
// ... and, in the prologue, stage 0's A loads: every later load of NS stages.
template <int NS, int NA>
constexpr int kWaitFirstA = kLoadsB + (NA + kLoadsB) * (NS - 1);
static_assert(kWaitFirstA<kStages<0>, kLoadsA> < 64 && kWaitFirstA<kStages<1>, kLoadsA> < 64, "vmcnt is 6 bits");

// MFMA row blocks of k step 1 issued before the stage's barrier (they read
// registers only), so the MFMA pipe has work while the waves meet.
#ifndef MOE_GEMM1_PRE_ROWS
#define MOE_GEMM1_PRE_ROWS 2
#endif
#ifndef MOE_GEMM2_PRE_ROWS
#define MOE_GEMM2_PRE_ROWS 2
#endif
template <int MODE>
constexpr int kPreBarrierRows = MODE == 0 ? MOE_GEMM1_PRE_ROWS : MOE_GEMM2_PRE_ROWS;

__device__ __forceinline__ void mma1(const i32x4& a, const i32x4& b, f32x16& c) {
    c = mfma32x32x16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c);
}

// One pipeline stage (two 16-wide k steps) on stage s, A in buffer BUF, B in
// register set BUF.  Entering, fa[r] holds row block r of stage s, k step 0.
// Each MFMA is followed by the read that refills its A register for the next
// k step (k step 1 of this stage, then k step 0 of stage s + 1 once the
// barrier has made that buffer safe), so every read has a whole k step to
// land; the stage's A DMA for stage s + NS is spread over the second k step.
template <int MODE, int NRB, int NA, int BUF, bool STREAM>
__device__ __forceinline__ void stage(const Dma& d, int s, int lane, i32x4 (&fa)[NRB],
                                      i32x4 (&bq)[kStages<MODE>][2], f32x16 (&acc)[kRowBlocks]) {
    constexpr int NS = kStages<MODE>;
    constexpr int NB = (BUF + 1) % NS;
    constexpr int PRE = NRB < kPreBarrierRows<MODE> ? NRB : kPreBarrierRows<MODE>;
    // k step 0, refilling each A register with k step 1 of this stage
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        mma1(fa[r], bq[BUF][0], acc[r]);
        __builtin_amdgcn_sched_barrier(0);
        fa[r] = read_a1<BUF, 1>(lane, r);
        __builtin_amdgcn_sched_barrier(0);
    }
    // k step 1, first row blocks: registers only
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        mma1(fa[r], bq[BUF][1], acc[r]);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();             // every read of buffer BUF by this wave has returned
    wait_vm<kWaitNextA<NS, NA>>();  // this wave's A loads of stage s+1 have landed
    barrier_lds();            // ... everybody's have, and everybody is done with buffer BUF
#pragma unroll
    for (int r = 0; r < PRE; ++r) fa[r] = read_a1<NB, 0>(lane, r);
    __builtin_amdgcn_sched_barrier(0);
    // the rest of k step 1, each MFMA followed by the read of stage s+1's k
    // step 0 into its register, with the A loads NS ahead into buffer BUF
    int issued_dma = 0;
#pragma unroll
    for (int r = PRE; r < NRB; ++r) {
        mma1(fa[r], bq[BUF][1], acc[r]);
        __builtin_amdgcn_sched_barrier(0);
        fa[r] = read_a1<NB, 0>(lane, r);
        __builtin_amdgcn_sched_barrier(0);
        if (issued_dma < NA) {
            dma_a1<BUF>(d, s + NS, lane, issued_dma);
            ++issued_dma;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
        if (i >= issued_dma) dma_a1<BUF>(d, s + NS, lane, i);
    __builtin_amdgcn_sched_barrier(0);
    load_b<STREAM>(d, s + NS, bq[BUF]);  // register set BUF is free once its MFMAs have issued
    __builtin_amdgcn_sched_barrier(0);
}

template <int NRB, int J>
__device__ __forceinline__ float* xchg_slot(int g) {
    return reinterpret_cast<float*>(ring<J>()) + g * 1024;
}

template <int MODE, int NRB, bool EXTRA, bool STREAM>
__device__ __forceinline__ void run_tile(const GemmArgs& p, int mt, int g, int row0, int M, int n0, int K, int N,
                                         bool shared, int nt) {
    constexpr int NA = kLoadsAOf<NRB, EXTRA>;  // this wave's A loads a stage
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int KS = (K + BK - 1) / BK;
    const int wg = wave & 3, wc = wave >> 2;  // the wave's 64-row weight group of the tile and its 32-row half

    Dma d;
    d.nsteps = KS;
    d.kvalid_last = (uint32_t)(K - (KS - 1) * BK);
    // ---- A: rows row0 .. row0+M of this group
    const bool a_tiled = MODE != 0 || (shared ? p.a_tiled_shared : p.a_tiled_routed);
    d.a_rm = !a_tiled;
    if (MODE != 0) {
        // GEMM2 reads the h tile slot of this M tile, written tiled by GEMM1
        const uint16_t* A = (shared ? p.a_shared : p.a_routed) + (size_t)mt * kBlocks16 * p.h_slot_ks * 512;
        d.ra = make_rsrc(A, (uint32_t)((NRB * 2) * KS * 1024));
    } else if (a_tiled) {
        // row0 is a multiple of 16 here (the caller aligns expert segments)
        const uint16_t* A = (shared ? p.a_shared : p.a_routed) + (size_t)(row0 / 16) * KS * 512;
        d.ra = make_rsrc(A, (uint32_t)(((M + 15) / 16) * KS * 1024));
    } else if (!shared && p.a_row_src) {
        // indexed: the rows of x named by row_src (the descriptor spans all of x)
        d.ra = make_rsrc(p.a_routed, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    } else {
        const uint16_t* A = (shared ? p.a_shared : p.a_routed) + (size_t)row0 * K;
        d.ra = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
    }
    const bool a_indexed = MODE == 0 && !shared && p.a_row_src != nullptr;
    d.sa = a_tiled ? 1024u : (uint32_t)(BK * 2);
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
        const int blk = a_block(wave, i);       // 16-row block of the tile this instruction fills
        const int row = blk * 16 + (lane >> 2);
        const uint32_t logical8 = (uint32_t)(((lane & 3) ^ swz_of_row(row)) * 8);
        if (i >= NA) {
            d.va[i] = kOOB;                     // not issued
        } else if (a_tiled) {
            d.va[i] = (uint32_t)blk * (uint32_t)KS * 1024u + (uint32_t)lane * 16u;
        } else if (a_indexed) {
            const int src = row < M ? p.a_row_src[row0 + row] : -1;
            d.va[i] = src >= 0 ? ((uint32_t)(src / p.a_row_k) * (uint32_t)K + logical8) * 2u : kOOB;
        } else {
            d.va[i] = row < M ? ((uint32_t)row * (uint32_t)K + logical8) * 2u : kOOB;
        }
    }
    // ---- B: the 32 weight rows of this wave (GEMM1: the gate (wc = 0) or up
    // (wc = 1) rows of h columns n0 + 32 wg .. +31; GEMM2: rows n0 + 64 wg +
    // 32 wc .. +31)
    if (p.w_tiled) {
        d.klim = 1 << 30;  // zero padded
        // fragment-order groups of 64 rows: GEMM1 2 * roundup(N, 128) rows, GEMM2 N rows
        const int groups = MODE == 0 ? ((N + 127) / 128) * 4 : (N + 63) / 64;
        const size_t mat = (size_t)groups * KS * 2048;  // elements of one expert's matrix
        const uint16_t* W = p.wt.tab ? static_cast<const uint16_t*>(wtab_ptr(p.wt, *p.wt.layer, g, p.slot0))
                            : shared ? p.w0_shared : p.w0_routed + (size_t)g * mat;
        const int q0 = nt * 4;                          // first group of the N tile
        d.rb = make_rsrc(W + (size_t)q0 * KS * 2048, (uint32_t)((groups - q0) * KS * 4096));
        d.vb = (uint32_t)wg * (uint32_t)KS * 4096u + (uint32_t)wc * 2048u + (uint32_t)lane * 16u;
        d.sb = 4096u;
        d.kb = 1024u;
    } else {
        const int ncols = MODE == 0 ? min(BN / 2, N - n0) : min(BN, N - n0);
        const size_t wmat = (size_t)K * (size_t)N;
        const uint16_t* W;
        if (p.wt.tab) {
            const int lay = *p.wt.layer;
            W = static_cast<const uint16_t*>(wtab_ptr(p.wt, lay, g, MODE == 0 && wc ? p.slot1 : p.slot0));
        } else if (MODE == 0 && wc) {
            W = shared ? p.w1_shared : p.w1_routed + (size_t)g * wmat;
        } else {
            W = shared ? p.w0_shared : p.w0_routed + (size_t)g * wmat;
        }
        W += (size_t)n0 * K;
        d.rb = make_rsrc(W, (uint32_t)ncols * (uint32_t)K * 2u);
        // the B row of this lane relative to n0 (GEMM1: same row of gate or up)
        const int br = MODE == 0 ? wg * 32 + l32 : wg * 64 + wc * 32 + l32;
        d.vb = br < ncols ? ((uint32_t)br * (uint32_t)K + (uint32_t)(lane >> 5) * 8u) * 2u : kOOB;
        d.sb = (uint32_t)(BK * 2);
        d.kb = 32u;
        d.klim = br < ncols ? K - (lane >> 5) * 8 : -1;  // the lane's chunk starts 8 (lane / 32) into the k step
    }

    f32x16 acc[kRowBlocks];
#pragma unroll
    for (int i = 0; i < kRowBlocks; ++i) acc[i] = f32x16{};
    i32x4 fa[NRB];
    constexpr int NS = kStages<MODE>;
    i32x4 bq[NS][2];

    static_for<0, NS>([&](auto c) {
        constexpr int t = decltype(c)::value;
        dma_a<t, NA>(d, t, lane);
        load_b<STREAM>(d, t, bq[t]);
    });
    wait_vm<kWaitFirstA<NS, NA>>();
    barrier_lds();
#pragma unroll
    for (int r = 0; r < NRB; ++r) fa[r] = read_a1<0, 0>(lane, r);
    // stages past the end load zeros, so the loop runs in whole turns of the ring
    const int nturns = (d.nsteps + NS - 1) / NS;
    for (int s = 0; s < nturns * NS; s += NS) {
        static_for<0, NS>([&](auto c) {
            constexpr int b = decltype(c)::value;
            stage<MODE, NRB, NA, b, STREAM>(d, s + b, lane, fa, bq, acc);
        });
    }
    wait_vm<0>();  // no LDS DMA may outlive the workgroup
    wait_lgkm0();
    void* out = shared ? p.out_shared : p.out_routed;
    barrier_lds();  // every wave has left the main loop: the ring is free
    if (MODE == 0) {
        // h = silu(g) * u into this M tile's slot, tiled with the slot's own KS
        // (the K of GEMM2), so GEMM2 streams it with contiguous 1 KiB reads.
        // Columns in [N, roundup(N, 32)) are GEMM2's K padding: they get zeros.
        // The pair's 32 h columns are one k block of the slot.  A lane's 16
        // accumulators of a row block are rows c_row(i): i < 8 the block's
        // rows 0..15, i >= 8 rows 16..31.  Round by round, the gate wave hands
        // the up wave its g of rows 16..31 and the up wave hands the gate wave
        // its u of rows 0..15 (lane-major through one ring buffer per row
        // block, so writes and reads are contiguous); after a barrier each
        // wave forms h of its 16 rows.  They go through the wave's private
        // 2 KiB slice of the last ring buffer, fp32, row r at r * 128 B with
        // rows r and r ^ 1 exchanged when bit 2 of r is set, so the writes
        // (rows r and r + 4 in the two half-waves) touch 64 distinct banks;
        // read back in the tiled block's own order -- lane q takes slot q, 8
        // columns of one row, two 16-byte reads on distinct banks -- each
        // 16-row block is one contiguous 1 KiB store.  Rows of the slot past M
        // hold zeros (their A rows loaded as zeros).  LDS operations of one
        // wave are processed in order.
        constexpr int R = kStages<0> - 1;  // row blocks per round
        const int ksh = (N + BK - 1) / BK;
        const int kb = (n0 >> 5) + wg;  // n0 is a multiple of 32
        const bool pair_live = kb < ksh;
        const bool live = pair_live && kb * 32 + l32 < N;
        uint16_t* h = static_cast<uint16_t*>(out) + (size_t)mt * kBlocks16 * p.h_slot_ks * 512;
        float* st = reinterpret_cast<float*>(ring<kStages<0> - 1>()) + wg * 1024 + wc * 512;
        const int rr = lane >> 2, c8 = (lane & 3) ^ swz_of_row(rr);  // the slot this lane stores
        const int mine = wc * 8;  // the accumulators whose rows this wave finishes
        static_for<0, (NRB + R - 1) / R>([&](auto rc) {
            constexpr int r0 = decltype(rc)::value * R;
            // hand over the other half: the gate wave its g of i >= 8 (slot
            // half 0), the up wave its u of i < 8 (slot half 1)
            static_for<0, R>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (r0 + j < NRB) {
                    float* x = xchg_slot<NRB, j>(wg) + wc * 512;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i * 64 + lane] = acc[r0 + j][8 - mine + i];
                }
            });
            barrier_lds();
            if (pair_live) {
                static_for<0, R>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int r = r0 + j;
                    if constexpr (r < NRB) {
                        const float* x = xchg_slot<NRB, j>(wg) + (1 - wc) * 512;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float mv = acc[r][mine + i], ov = x[i * 64 + lane];
                            const float g = wc ? ov : mv, u = wc ? mv : ov;
                            const int row = c_row(mine + i, lane) - wc * 16;  // bit 2 of row is lane / 32
                            st[(row ^ ((row >> 2) & 1)) * 32 + l32] = live ? silu_f(g) * u : 0.0f;
                        }
                        // the staged values are read by other lanes of this wave:
                        // keep the compiler from moving the reads above the writes
                        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                        const float* src = st + (rr ^ ((rr >> 2) & 1)) * 32 + c8 * 8;
                        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
                        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
                        uint4 q;
                        q.x = (uint32_t)f32_to_bf16(v0[0]) | ((uint32_t)f32_to_bf16(v0[1]) << 16);
                        q.y = (uint32_t)f32_to_bf16(v0[2]) | ((uint32_t)f32_to_bf16(v0[3]) << 16);
                        q.z = (uint32_t)f32_to_bf16(v1[0]) | ((uint32_t)f32_to_bf16(v1[1]) << 16);
                        q.w = (uint32_t)f32_to_bf16(v1[2]) | ((uint32_t)f32_to_bf16(v1[3]) << 16);
                        if (r * 32 + wc * 16 < M)
                            *reinterpret_cast<uint4*>(h + ((size_t)(r * 2 + wc) * ksh + kb) * 512 + lane * 8) = q;
                        // reads before the next block's writes
                        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    }
                });
            }
            barrier_lds();  // the round's slots are read before the next round writes them
        });
    } else if (MODE == 2) {
        // The combine, for the tile's tokens (the shared group's tile row r is
        // token row0 + r) and columns n0 .. n0 + 255: the shared term is staged
        // one 32-row block at a time by all eight waves as bf16 -- the value
        // the GEMM2 store of y_shared would hold -- into a [32 rows][256
        // columns] image (as the bf16 y store below: chunk c of row r at
        // c ^ (((r >> 2) & 3) << 2), two buffers, one barrier a block); then
        // each thread takes two 8-column chunks of the block, issues the loads
        // of the token's k routed rows, sums w_j * y_j in slot order with fp32
        // multiply-adds, adds the shared term last and stores the output row
        // chunk: the arithmetic of combine_kernel, so the result is the same.
        const int cl = wg * 64 + wc * 32 + l32;
        const int tid = threadIdx.x;
        const int K8 = p.comb_k;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            uint16_t* st = reinterpret_cast<uint16_t*>(r & 1 ? ring<1>() : ring<0>());
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = c_row(i, lane);
                st[row * 256 + (((cl >> 3) ^ (((row >> 2) & 3) << 2)) << 3) + (cl & 7)] = f32_to_bf16(acc[r][i]);
            }
            __syncthreads();
            const i32x4* sv = reinterpret_cast<const i32x4*>(st);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int id = h2 * NTH + tid;
                const int row = id >> 5, c = id & 31, grow = r * 32 + row, col = n0 + c * 8;
                if (grow >= M || col >= N) continue;
                const int t = row0 + grow;
                float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (K8 == 8) {
                    i32x4 ys[8];
                    float wj[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int yr = p.tok_row[(size_t)t * 8 + j];
                        wj[j] = p.topk_w[(size_t)t * 8 + j];
                        ys[j] = __builtin_nontemporal_load(
                            reinterpret_cast<const i32x4*>(p.y_routed + (size_t)yr * N + col));
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t u = (uint32_t)ys[j][q];
                            a[2 * q] = fmaf(wj[j], __uint_as_float(u << 16), a[2 * q]);
                            a[2 * q + 1] = fmaf(wj[j], __uint_as_float(u & 0xFFFF0000u), a[2 * q + 1]);
                        }
                } else {
                    for (int j = 0; j < K8; ++j) {
                        const int yr = p.tok_row[(size_t)t * K8 + j];
                        const float w = p.topk_w[(size_t)t * K8 + j];
                        const i32x4 y = __builtin_nontemporal_load(
                            reinterpret_cast<const i32x4*>(p.y_routed + (size_t)yr * N + col));
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t u = (uint32_t)y[q];
                            a[2 * q] = fmaf(w, __uint_as_float(u << 16), a[2 * q]);
                            a[2 * q + 1] = fmaf(w, __uint_as_float(u & 0xFFFF0000u), a[2 * q + 1]);
                        }
                    }
                }
                const i32x4 sh = sv[row * 32 + (c ^ (((row >> 2) & 3) << 2))];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t u = (uint32_t)sh[q];
                    a[2 * q] += __uint_as_float(u << 16);
                    a[2 * q + 1] += __uint_as_float(u & 0xFFFF0000u);
                }
                if (p.comb_out_f32) {
                    f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(p.comb_out) + (size_t)t * N + col);
                    o[0] = f32x4{a[0], a[1], a[2], a[3]};
                    o[1] = f32x4{a[4], a[5], a[6], a[7]};
                } else {
                    i32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = (int)((uint32_t)f32_to_bf16(a[2 * q]) | ((uint32_t)f32_to_bf16(a[2 * q + 1]) << 16));
                    *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.comb_out) + (size_t)t * N + col) = o;
                }
            }
        }
    } else if (!p.out_f32) {
        // bf16 y through LDS, one 32-row block at a time, by all eight waves
        // into one [32 rows][256 columns] image (two buffers, one barrier a
        // block), then stored as whole rows of the tile.  The 16-byte chunk c
        // of image row r sits at chunk c ^ (((r >> 2) & 3) << 2): a wave's
        // element writes (rows r and r + 4, 32 columns each) and its 16-byte
        // reads (two whole rows) both spread over every bank.
        const int cl = wg * 64 + wc * 32 + l32;  // this lane's column of the tile
        const int tid = threadIdx.x;
        uint16_t* y = static_cast<uint16_t*>(out);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            uint16_t* st = reinterpret_cast<uint16_t*>(r & 1 ? ring<1>() : ring<0>());
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = c_row(i, lane);
                st[row * 256 + (((cl >> 3) ^ (((row >> 2) & 3) << 2)) << 3) + (cl & 7)] = f32_to_bf16(acc[r][i]);
            }
            // the block is staged; the other buffer's reads (block r - 1) came
            // before every thread's writes above, so it is free for block r + 1
            __syncthreads();
            const i32x4* sv = reinterpret_cast<const i32x4*>(st);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int id = k * NTH + tid;
                const int row = id >> 5, c = id & 31, grow = r * 32 + row, col = n0 + c * 8;
                // non-temporal: y is read again only by the combine, after the
                // launch, so it need not displace the h slots from L2
                if (grow < M && col < N)
                    __builtin_nontemporal_store(sv[row * 32 + (c ^ (((row >> 2) & 3) << 2))],
                                                reinterpret_cast<i32x4*>(y + (size_t)(row0 + grow) * N + col));
            }
        }
    } else {
        // fp32 y through LDS, one 32-row block at a time: each wave stages its 32 x 32
        // block in a private 4 KiB slice of the ring (free once every wave has
        // left the main loop), fp32, row r at r * 128 B with rows r and r ^ 1
        // exchanged when bit 2 of r is set -- the accumulator writes (rows r and
        // r + 4 in the two half-waves) and the 16-byte reads (8 lanes per row)
        // both touch 64 distinct banks -- then stores 4 columns per lane: 8
        // lanes cover a row's 32 columns.  LDS operations of one wave are
        // processed in order, so a block's reads finish before the next block's
        // writes land.
        float* st = reinterpret_cast<float*>(wave < 4 ? ring<0>() : ring<1>()) + (wave & 3) * 1024;
        const int cw = n0 + wg * 64 + wc * 32;  // first output column of this wave
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = c_row(i, lane);  // bit 2 of row is lane / 32
                st[(row ^ ((row >> 2) & 1)) * 32 + l32] = acc[r][i];
            }
            // the staged values are read by other lanes of this wave: keep the
            // compiler from moving the reads above the writes (no wait is needed)
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int q = it * 64 + lane;  // chunk q: row q / 8, columns 4 (q % 8) .. + 3
                const int row = q >> 3, c4 = (q & 7) * 4;
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + (row ^ ((row >> 2) & 1)) * 32 + c4);
                const int grow = r * 32 + row, col = cw + c4;
                if (grow < M && col < N)
                    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (size_t)(row0 + grow) * N + col) = v;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // reads before the next block's writes
        }
    }
}

// The tile body of this wave: whether it issues the extra A load of the
// tile's 16-row blocks (waves w < L % 8) is uniform per wave.
template <int MODE, int NRB, bool STREAM>
__device__ __forceinline__ void tile_of_wave(const GemmArgs& p, int mt, int g, int row0, int M, int n0, int K,
                                             int N, bool shared, int nt) {
    constexpr int extra_waves = kTileBlocks16<NRB> % NWAVES;
    if constexpr (extra_waves != 0) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (wave < extra_waves) {
            run_tile<MODE, NRB, true, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt);
            return;
        }
    }
    run_tile<MODE, NRB, false, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt);
}

template <int MODE, bool STREAM>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2)))
ffn_gemm_bf16(GemmArgs p) {
    // the launch's items: all, the routed groups' (the first n_tiles[1] M tiles)
    // or the shared group's (the rest)
    const int tot = p.n_tiles[0] * p.NT, nr = p.part == 0 ? tot : p.n_tiles[1] * p.NT;
    const int base = p.part == 2 ? nr : 0, cnt = p.part == 0 ? tot : (p.part == 1 ? nr : tot - nr);
    const int L0 = xcd_queue_tile(cnt, p.queue);
    if (L0 < 0) return;
    const int L = base + L0;
    if (p.wt.tab && wtab_layer(p.wt) < 0) return;
    const int2 wl = p.work[L];
    const int mt = wl.x, nt = wl.y;
    const int4 td = p.tiles[mt];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const bool shared = g == p.E;
    const int K = shared ? p.K_shared : p.K_routed;
    const int N = shared ? p.N_shared : p.N_routed;
    const int n0 = MODE == 0 ? nt * (BN / 2) : nt * BN;
    if (n0 >= N || M <= 0) return;
    switch ((M + 31) >> 5) {
    case 1: tile_of_wave<MODE, 1, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 2: tile_of_wave<MODE, 2, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 3: tile_of_wave<MODE, 3, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 4: tile_of_wave<MODE, 4, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 5: tile_of_wave<MODE, 5, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 6: tile_of_wave<MODE, 6, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 7: tile_of_wave<MODE, 7, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    case 8: tile_of_wave<MODE, 8, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    default: tile_of_wave<MODE, 9, STREAM>(p, mt, g, row0, M, n0, K, N, shared, nt); break;
    }
}

}  // namespace

// ------------------------------------------------------------- tile list
constexpr int kMBlock = 4;  // M tiles of one expert whose work items are interleaved
// Workgroups of 1024 threads; each computes the groups' tile prefix and
// writes its share of the tiles and work items.  Group g < E covers rows [offsets[g],
// offsets[g+1]); group E (the shared expert, when present) covers tokens
// [0, T).  A group of n rows gets nmt = ceil(n / bm) tiles of height
// ceil(ceil(n / nmt) / 32) * 32 (the last one shorter).  The work lists take a
// group's M tiles in blocks of four and, inside a block, N tile by N tile with
// the block's M tiles next to each other: the items that run side by side on
// one XCD share a few row panels and weight panels in its L2, so a panel
// streams from HBM about once per block instead of once per N tile.
__global__ void __launch_bounds__(1024)
ffn_build_tiles(const int32_t* __restrict__ offsets, int E, int has_shared, int T, int bm, int rows_cap,
                int4* __restrict__ tiles, int32_t* __restrict__ n_tiles, int2* __restrict__ work1, int nt1,
                int2* __restrict__ work2, int nt2) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t gend[1025];  // inclusive prefix of the groups' tile counts
    const int G = E + has_shared;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // Row ranges are clamped to [0, rows_cap] and never negative, so malformed
    // offsets cannot send a tile outside the caller's buffers.
    auto group_rows = [&](int g, int& b, int& e) {
        if (g < E) {
            b = min(max(offsets[g], 0), rows_cap);
            e = min(max(offsets[g + 1], b), rows_cap);
        } else {
            b = 0;
            e = T;
        }
    };
    // 1. tile counts and their prefix: thread tid owns group tid; thread 0
    //    also owns group 1024 (E == 1024 with a shared expert)
    int n0 = 0;
    if (tid < G) {
        int b, e;
        group_rows(tid, b, e);
        n0 = (e - b + bm - 1) / bm;
    }
    int incl = n0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    if (tid < G) gend[tid] = before + incl;
    if (tid == 0 && G > 1024) {
        int total = 0;
        for (int w = 0; w < 16; ++w) total += wsum[w];
        int b, e;
        group_rows(1024, b, e);
        gend[1024] = total + (e - b + bm - 1) / bm;
    }
    __syncthreads();
    const int total = G > 0 ? gend[G - 1] : 0;
    // the group holding tile ti: the first whose prefix end exceeds ti
    auto group_of = [&](int ti) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (gend[mid] > ti) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    };
    // Steps 2 and 3 are split over the launch's workgroups (each recomputed
    // the prefix above); item i goes to workgroup (i / 1024) % gridDim.x.
    const int first = blockIdx.x * 1024 + tid, stride = gridDim.x * 1024;
    // 2. tiles: a group of n rows gets nmt equal tiles of height rounded up to 32
    for (int ti = first; ti < total; ti += stride) {
        const int g = group_of(ti);
        const int st = g ? gend[g - 1] : 0, nmt = gend[g] - st;
        int b, e;
        group_rows(g, b, e);
        int hgt = (e - b + nmt - 1) / nmt;
        hgt = ((hgt + 31) / 32) * 32;
        const int rb = b + (ti - st) * hgt;
        tiles[ti] = int4{g, rb, min(e, rb + hgt), 0};
    }
    // 3. work lists: per group, blocks of kMBlock M tiles, N tile by N tile, the
    //    block's M tiles next to each other (32 consecutive items -- one XCD's
    //    CUs -- share kMBlock row panels and 32 / kMBlock weight panels)
    auto emit = [&](int2* __restrict__ work, int nt) {
        for (int i = first; i < total * nt; i += stride) {
            const int g = group_of(i / nt);
            const int st = g ? gend[g - 1] : 0, nmt = gend[g] - st;
            const int j = i - st * nt;
            const int mb = (j / (kMBlock * nt)) * kMBlock;
            const int r = j - mb * nt, mc = min(kMBlock, nmt - mb);
            work[i] = int2{st + mb + r % mc, r / mc};
        }
    };
    emit(work1, nt1);
    emit(work2, nt2);
    // the work queues of the launches that follow start empty
    if (blockIdx.x == 0 && tid >= 2 && tid < kFfnCtlWords) n_tiles[tid] = 0;
    if (blockIdx.x == 0 && tid == 0) {
        n_tiles[0] = total;
        n_tiles[1] = E > 0 ? gend[E - 1] : 0;  // the routed groups' M tiles come first
    }
}

hipError_t launch_build_tiles(const moe_cfg& c, const int32_t* offsets, int bm, int64_t rows_cap,
                              const FfnWork& wk, hipStream_t s) {
    // enough workgroups that each thread emits a few items of the longer list
    const int64_t items = (rows_cap / bm + c.E + 1) * (int64_t)(wk.nt1 > wk.nt2 ? wk.nt1 : wk.nt2);
    int64_t nbl = (items + 4095) / 4096;
    nbl = nbl < 1 ? 1 : (nbl > 32 ? 32 : nbl);
    const unsigned nb = (unsigned)nbl;
    hipLaunchKernelGGL(ffn_build_tiles, dim3(nb), dim3(1024), 0, s, offsets, c.E, c.has_shared ? 1 : 0, c.T,
                       bm, (int)rows_cap, reinterpret_cast<int4*>(wk.tiles), wk.n_tiles,
                       reinterpret_cast<int2*>(wk.work1), wk.nt1, reinterpret_cast<int2*>(wk.work2), wk.nt2);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const FfnOperands& op,
                            const int32_t* offsets, const moe_weights& w, const WTab& wt, const FfnWork& wk,
                            void* h_tiles, hipStream_t s) {
    const int has_sh = c.has_shared ? 1 : 0;
    hipError_t e0 = launch_build_tiles(c, offsets, BM, n_rows_cap, wk, s);
    if (e0 != hipSuccess) return e0;
    const bool tiled = w.layout == MOE_LAYOUT_TILED;
    const int imax = has_sh && c.I_shared > c.I ? c.I_shared : c.I;
    GemmArgs a{};
    a.tiles = reinterpret_cast<const int4*>(wk.tiles);
    a.n_tiles = wk.n_tiles;
    a.E = c.E;
    a.w_tiled = tiled;
    a.h_slot_ks = (imax + BK - 1) / BK;
    a.wt = wt;
    a.slot0 = 0;
    a.slot1 = 1;
    // GEMM1: gate/up + SwiGLU -> h tile slots
    a.work = reinterpret_cast<const int2*>(wk.work1);
    a.a_routed = static_cast<const uint16_t*>(op.x_rows);
    a.a_shared = static_cast<const uint16_t*>(op.x_tokens);
    a.a_tiled_routed = op.x_rows_tiled;
    a.a_tiled_shared = op.x_tokens_tiled;
    a.a_row_src = op.row_src;
    a.a_row_k = c.k;
    a.a_rows = c.T;
    a.w0_routed = static_cast<const uint16_t*>(w.w_gate);
    a.w1_routed = static_cast<const uint16_t*>(w.w_up);
    a.w0_shared = static_cast<const uint16_t*>(w.sh_gate);
    a.w1_shared = static_cast<const uint16_t*>(w.sh_up);
    a.out_routed = h_tiles;
    a.out_shared = h_tiles;
    a.K_routed = c.H;
    a.K_shared = c.H;
    a.N_routed = c.I;
    a.N_shared = has_sh ? c.I_shared : c.I;
    a.NT = wk.nt1;
    a.out_f32 = 0;
    // Streamed (non-temporal) gate/up weights when the routed rows average at
    // most one M tile per expert: each weight panel is then read about once,
    // and keeping it out of the caches leaves them to the row panels, which
    // every N tile of an M tile reads again.  With several M tiles per expert
    // the tiles of a block share each weight panel through L2, so the default
    // policy stays; GEMM2 keeps it always.
    const bool stream_w = n_rows_cap <= (int64_t)c.E * BM;
    a.queue = wk.n_tiles + 2;  // queue 0
    const dim3 g1((unsigned)xcd_queue_grid(max_tiles * a.NT));
    if (stream_w) hipLaunchKernelGGL((ffn_gemm_bf16<0, true>), g1, dim3(NTH), 0, s, a);
    else hipLaunchKernelGGL((ffn_gemm_bf16<0, false>), g1, dim3(NTH), 0, s, a);
    // GEMM2: down -> y
    a.work = reinterpret_cast<const int2*>(wk.work2);
    a.a_routed = static_cast<const uint16_t*>(h_tiles);
    a.a_shared = static_cast<const uint16_t*>(h_tiles);
    a.a_tiled_routed = 1;
    a.a_tiled_shared = 1;
    a.a_row_src = nullptr;
    a.w0_routed = static_cast<const uint16_t*>(w.w_down);
    a.w1_routed = nullptr;
    a.slot0 = 2;
    a.w0_shared = static_cast<const uint16_t*>(w.sh_down);
    a.w1_shared = nullptr;
    a.out_routed = op.y_rows;
    a.out_shared = op.y_shared;
    a.K_routed = c.I;
    a.K_shared = has_sh ? c.I_shared : c.I;
    a.N_routed = c.H;
    a.N_shared = c.H;
    a.NT = wk.nt2;
    a.out_f32 = c.y_dtype == MOE_F32;
    a.queue = wk.n_tiles + 2 + kQueueWords;  // queue 1
    const dim3 g2((unsigned)xcd_queue_grid(max_tiles * a.NT));
    if (!(op.comb_out && has_sh && c.y_dtype == MOE_BF16)) {
        hipLaunchKernelGGL((ffn_gemm_bf16<1, false>), g2, dim3(NTH), 0, s, a);
        return hipGetLastError();
    }
    // with the combine: the routed groups' GEMM2, then the shared group's with
    // the combine in its epilogue (its tiles own rows of out: tile row r is
    // token row0 + r)
    a.part = 1;
    hipLaunchKernelGGL((ffn_gemm_bf16<1, false>), g2, dim3(NTH), 0, s, a);
    a.part = 2;
    a.queue = wk.n_tiles + 2 + 2 * kQueueWords;  // queue 2
    a.out_shared = nullptr;
    a.y_routed = static_cast<const uint16_t*>(op.y_rows);
    a.tok_row = op.tok_row;
    a.topk_w = op.topk_w;
    a.comb_out = op.comb_out;
    a.comb_k = c.k;
    a.comb_out_f32 = c.out_dtype == MOE_F32;
    const int64_t sh_tiles = (c.T + BM - 1) / BM;  // the shared group's M tiles
    hipLaunchKernelGGL((ffn_gemm_bf16<2, false>), dim3((unsigned)xcd_queue_grid(sh_tiles * a.NT)), dim3(NTH), 0, s, a);
    return hipGetLastError();
}

// ------------------------------------------------------------- weight tiling
// Rewrites E row-major bf16 matrices [rows][K] into the fragment-order layout
// (see the operand layouts above), one thread per destination 16-byte chunk.
// With `pair` set, the 64 rows of group q are the 32 gate rows (src0) and then
// the 32 up rows (src1) of h columns 32 q .. 32 q + 31, the way a GEMM1 wave
// consumes them.  Rows and columns past the source are zero.
__global__ void __launch_bounds__(256)
tile_matrices(const uint16_t* __restrict__ src0, const uint16_t* __restrict__ src1, int E, int rows, int K,
              int pair, uint16_t* __restrict__ dst, int groups, int KS) {
    const size_t per = (size_t)groups * KS * 256;  // 16-byte chunks of one matrix
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= per * E) return;
    const int e = (int)(idx / per);
    const size_t rem = idx % per;
    const int lane = (int)(rem & 63), j = (int)((rem >> 6) & 3);
    const size_t qs = rem >> 8;
    const int ks = (int)(qs % KS), q = (int)(qs / KS);
    const int c = j >> 1, kk = j & 1;
    const int k0 = ks * BK + kk * 16 + (lane >> 5) * 8;
    const uint16_t* src = src0;
    int srow = q * 64 + c * 32 + (lane & 31);
    if (pair) {
        src = c ? src1 : src0;
        srow = q * 32 + (lane & 31);
    }
    i32x4 v = {0, 0, 0, 0};
    if (srow < rows && k0 < K) v = *reinterpret_cast<const i32x4*>(src + ((size_t)e * rows + srow) * K + k0);
    reinterpret_cast<i32x4*>(dst)[idx] = v;
}

// Groups of 64 rows of the fragment-order matrices: gate+up of I h columns
// (I padded to 128: whole GEMM1 N tiles), down of H rows.
static int groups13(int I) { return ((I + 127) / 128) * 4; }
static int groups2(int H) { return (H + 63) / 64; }

TiledSizes tiled_sizes(const moe_cfg& c) {
    TiledSizes t{};
    if (c.w_dtype == MOE_FP8_E4M3) {
        // tiled e4m3: the row-major sizes (H, I, I_shared are multiples of 128)
        t.w13 = (size_t)2 * c.I * c.H * c.E;
        t.w2 = (size_t)c.H * c.I * c.E;
        t.sh13 = c.has_shared ? (size_t)2 * c.I_shared * c.H : 0;
        t.sh2 = c.has_shared ? (size_t)c.H * c.I_shared : 0;
        return t;
    }
    const size_t ksh = (size_t)((c.H + BK - 1) / BK);
    auto w13 = [&](int I) { return (size_t)groups13(I) * ksh * 4096; };
    auto w2 = [&](int I) { return (size_t)groups2(c.H) * (size_t)((I + BK - 1) / BK) * 4096; };
    t.w13 = w13(c.I) * c.E;
    t.w2 = w2(c.I) * c.E;
    t.sh13 = c.has_shared ? w13(c.I_shared) : 0;
    t.sh2 = c.has_shared ? w2(c.I_shared) : 0;
    return t;
}

hipError_t launch_tile_weights(const moe_cfg& c, const moe_weights& src, void* w13, void* w2, void* sh13, void* sh2,
                               hipStream_t s) {
    if (c.w_dtype == MOE_FP8_E4M3) return launch_tile_weights_e4m3(c, src, w13, w2, sh13, sh2, s);
    auto go = [&](const void* a, const void* b, int E, int rows, int K, int pair, void* dst) {
        const int groups = pair ? groups13(rows) : groups2(rows), KS = (K + BK - 1) / BK;
        const size_t n = (size_t)E * groups * KS * 256;
        hipLaunchKernelGGL(tile_matrices, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), E, rows, K, pair,
                           static_cast<uint16_t*>(dst), groups, KS);
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
