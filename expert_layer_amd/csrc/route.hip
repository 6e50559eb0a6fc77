// route.hip -- router GEMM and top-k gating.
//
// The router is the "gated routing" half of the FFN side ("Memory-Compute
// Disaggregation ... AFD Architecture Analysis", section 3); its output, the
// expert IDs of every token, is what ASAP's dispatch buffers carry ("ASAP",
// Table 2, section 3.2.1).
//
// Kernel 1 (router_logits_bf16): logits[T][E] = x[T][H] . w_router[E][H]^T on
// bf16 MFMA with fp32 accumulation.  One workgroup (8 waves, two per SIMD) owns
// 128 tokens x 256 experts over one slice of K; each wave 64 tokens x 64
// experts (2 x 2 blocks of 32 x 32).  Operands move HBM -> LDS by buffer_load ... lds through
// a ring of four 32-wide stages (XOR-swizzled 16-byte chunks), so x streams
// from HBM once per 256 experts.  K is split so that T / 128 token blocks
// still fill the chip; the splits write fp32 partial logits that route_select
// adds in split order (a fixed order, so the result does not depend on
// scheduling).  The kernel is bound by the HBM read of x.  Its QUANT form also
// writes x's per-token e4m3 codes (1 x 128 blocks) from the x tiles it already
// holds in LDS, so that low-precision experts need no second pass over x.
// Kernel 2 (route_select_team; route_select for other shapes): a team of 8 or
// 16 lanes per token -- the partial logits summed, scores, group limit, top-k
// with ties to the lower index, renormalisation and scaling.
#include "common.hpp"

namespace moe {
namespace {

constexpr int RB_M = 128, RB_N = 256, RB_K = 32, RB_NST = 4, RB_THREADS = 512;
constexpr int LA = 1, LB = 2;  // A and B chunk loads per wave per stage
constexpr int kRA = RB_M * 4;                // 16-byte chunks of A (128 rows x 64 B) in one stage
constexpr int kRB = RB_N * 4;                // of B (256 expert rows x 64 B)
constexpr uint32_t kROOB = 0x40000000u;      // past every descriptor: the load returns zero

typedef __attribute__((address_space(3))) void* rlds_t;

// The four stage buffers [A | B], distinct objects (see gemm_bf16.hip).
__shared__ i32x4 rring0[kRA + kRB];
__shared__ i32x4 rring1[kRA + kRB];
__shared__ i32x4 rring2[kRA + kRB];
__shared__ i32x4 rring3[kRA + kRB];

template <int BUF>
__device__ __forceinline__ i32x4* rring() {
    if constexpr (BUF == 0) return rring0;
    else if constexpr (BUF == 1) return rring1;
    else if constexpr (BUF == 2) return rring2;
    else return rring3;
}

__device__ __forceinline__ void rbarrier() { asm volatile("s_barrier" ::: "memory"); }

struct RDma {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[LA], vb[LB];   // byte offset of this lane's chunk at k = k0 (kROOB: outside the tile)
    uint32_t lc[LA], lcb[LB];  // the chunk's column offset (elements) inside a stage
    int k0, k_end, nsteps;
};

// Loads of stage t into buffer BUF: 1 A and 2 B chunk loads per lane, zero
// past the tile's rows and past the split's K range.
template <int BUF>
__device__ __forceinline__ void rdma(const RDma& d, int t, int wave) {
    i32x4* buf = rring<BUF>();
    const int kst = d.k0 + t * RB_K;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const bool ok = d.va[i] != kROOB && kst + (int)d.lc[i] < d.k_end;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (rlds_t)(buf + (wave * LA + i) * 64), 16,
                                                 ok ? d.va[i] + (uint32_t)t * (RB_K * 2) : kROOB, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const bool ok = d.vb[i] != kROOB && kst + (int)d.lcb[i] < d.k_end;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (rlds_t)(buf + kRA + (wave * LB + i) * 64), 16,
                                                 ok ? d.vb[i] + (uint32_t)t * (RB_K * 2) : kROOB, 0, 0, 0);
    }
}

// One stage: two 16-wide k steps of the wave's 2 x 2 blocks of 32 x 32
// (tokens 64 (w / 4) + [0, 64), experts 64 (w % 4) + [0, 64)).
template <int BUF>
__device__ __forceinline__ void rstage(int wave, int lane, f32x16 (&acc)[2][2]) {
    const i32x4* buf = rring<BUF>();
    const int l32 = lane & 31;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = kk * 2 + (lane >> 5);
        i32x4 a[2], b[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = (wave >> 2) * 64 + r * 32 + l32;
            a[r] = buf[row * 4 + (chunk ^ tile_swz(row))];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = (wave & 3) * 64 + c * 32 + l32;  // provably inside the buffer
            b[c] = buf[kRA + row * 4 + (chunk ^ tile_swz(row))];
        }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                acc[r][c] = mfma32x32x16(__builtin_bit_cast(bf16x8, a[r]), __builtin_bit_cast(bf16x8, b[c]),
                                         acc[r][c]);
    }
}

// The per-token e4m3 quantisation of one 128-column block kb of a token block:
// thread (row, c) = (tid / 4, tid % 4) holds chunk c of each of the turn's four
// 32-column stages, i.e. x[t][128 kb + 32 j + 8 c + i], j < 4, i < 8.  The rule
// is moe_quantize_fp8's: s = max |x| / 448 over the block (1 for an all-zero
// block), code = e4m3_rne_sat(x / s) with the division in fp32.
__device__ __forceinline__ void rquant(const i32x4 (&qv)[4], int t, int T, int H, int kb, int c,
                                       uint8_t* __restrict__ xq, float* __restrict__ xs) {
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = (uint32_t)qv[j][i];
            v[8 * j + 2 * i] = bf16_to_f32((uint16_t)(word & 0xFFFFu));
            v[8 * j + 2 * i + 1] = bf16_to_f32((uint16_t)(word >> 16));
        }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1));  // the four threads of a row are adjacent lanes
    m = fmaxf(m, __shfl_xor(m, 2));
    const float sc = m > 0.0f ? m / 448.0f : 1.0f;
    if (t >= T) return;
    uint8_t* q = xq + (size_t)t * H + (size_t)kb * 128 + c * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float* u = v + 8 * j;
        const uint32_t lo = e4m3x4_rne_sat(u[0] / sc, u[1] / sc, u[2] / sc, u[3] / sc);
        const uint32_t hi = e4m3x4_rne_sat(u[4] / sc, u[5] / sc, u[6] / sc, u[7] / sc);
        *reinterpret_cast<uint2*>(q + j * 32) = make_uint2(lo, hi);
    }
    if (c == 0) xs[(size_t)t * (H / 128) + kb] = sc;
}

// partial[split][t][e] = sum over the split's K range of x[t][h] * w[e][h].
// Workgroup: 128 tokens x 256 experts x one K range, 8 waves (two per SIMD);
// wave w owns tokens 64 (w / 4) + [0, 64) and experts 64 (w % 4) + [0, 64).  Operands move HBM -> LDS by buffer_load ... lds through a
// ring of four stages (64-byte row segments, the chunks XOR-swizzled by row so
// that fragment reads are free of bank conflicts).  Splitting K lets T / 128
// token blocks fill the chip; the router weights are then read from L2 about
// T / 128 times instead of once per 32 tokens.
// QUANT: ksplit is a multiple of 128, so that each turn of four stages is one
// 128-column block of x; the workgroups of the first expert block quantise the
// blocks of their tokens (rquant) into xq [T][H] and xs [T][H / 128].
template <bool QUANT>
__global__ void __launch_bounds__(RB_THREADS)
router_logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ partial,
                   int T, int H, int E, int ksplit, uint8_t* __restrict__ xq, float* __restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = blockIdx.x * RB_M, e0 = blockIdx.y * RB_N, split = blockIdx.z;
    RDma d;
    d.k0 = split * ksplit;
    d.k_end = min(H, d.k0 + ksplit);
    d.nsteps = (d.k_end - d.k0 + RB_K - 1) / RB_K;
    const int mt = min(RB_M, T - t0), ne = min(RB_N, E - e0);
    d.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (size_t)t0 * H), (short)0,
                                              (int)((uint32_t)mt * (uint32_t)H * 2u), 0x00020000);
    d.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w + (size_t)e0 * H), (short)0,
                                              (int)((uint32_t)ne * (uint32_t)H * 2u), 0x00020000);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int row = (wave * LA + i) * 16 + (lane >> 2);
        const int logical = (lane & 3) ^ tile_swz(row);
        d.lc[i] = (uint32_t)(logical * 8);
        d.va[i] = row < mt ? ((uint32_t)row * (uint32_t)H + (uint32_t)(d.k0 + logical * 8)) * 2u : kROOB;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int row = (wave * LB + i) * 16 + (lane >> 2);
        const int logical = (lane & 3) ^ tile_swz(row);
        d.lcb[i] = (uint32_t)(logical * 8);
        d.vb[i] = row < ne ? ((uint32_t)row * (uint32_t)H + (uint32_t)(d.k0 + logical * 8)) * 2u : kROOB;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[r][c] = f32x16{};

    // Stages 0..2 in flight; at stage s (buffer s % 4): wait until its loads
    // have landed (the 6 loads of stages s+1, s+2 may still fly), one barrier
    // -- everyone's stage s has landed and everyone is done with stage s-1 --
    // refill stage s-1's buffer with stage s+3, then compute on stage s.
    // QUANT: this thread's chunk of x in each stage of the turn (row qrow, chunk qc)
    const bool quant = QUANT && blockIdx.y == 0;
    const int qrow = threadIdx.x >> 2, qc = threadIdx.x & 3;
    const int qphys = qrow * 4 + (qc ^ tile_swz(qrow));
    i32x4 qv[4];

    rdma<0>(d, 0, wave);
    rdma<1>(d, 1, wave);
    rdma<2>(d, 2, wave);
    const int nturns = (d.nsteps + RB_NST - 1) / RB_NST;
    for (int s = 0; s < nturns * RB_NST; s += RB_NST) {
#define ROUTER_STAGE(J)                                              \
        __builtin_amdgcn_s_waitcnt((6 & 15) | ((6 >> 4) << 14) | 0x0070);   \
        rbarrier();                                                  \
        __builtin_amdgcn_sched_barrier(0);                           \
        rdma<(J + 3) % RB_NST>(d, s + J + 3, wave);                  \
        __builtin_amdgcn_sched_barrier(0);                           \
        rstage<J>(wave, lane, acc);                                  \
        if (quant) qv[J] = rring<J>()[qphys];                        \
        __builtin_amdgcn_sched_barrier(0);
        ROUTER_STAGE(0)
        ROUTER_STAGE(1)
        ROUTER_STAGE(2)
        ROUTER_STAGE(3)
#undef ROUTER_STAGE
        if (quant) rquant(qv, t0 + qrow, T, H, (d.k0 + s * RB_K) / 128, qc, xq, xs);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no LDS DMA may outlive the workgroup
    float* out = partial + (size_t)split * T * E;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int e = e0 + (wave & 3) * 64 + c * 32 + (lane & 31);
        if (e < E) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = t0 + (wave >> 2) * 64 + r * 32 + c_row(i, lane);
                    if (t < T) out[(size_t)t * E + e] = acc[r][c][i];
                }
        }
    }
}

// fp32 operands: one thread per (token, expert) dot product.
__global__ void router_logits_f32(const float* __restrict__ x, const float* __restrict__ w,
                                  float* __restrict__ logits, int T, int H, int E) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)T * E) return;
    int t = (int)(idx / E), e = (int)(idx % E);
    const float* xr = x + (size_t)t * H;
    const float* wr = w + (size_t)e * H;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
    logits[idx] = acc;
}

// ---------------------------------------------------------------- selection


__device__ __forceinline__ bool beats(float ka, int ea, float kb, int eb) {
    return ka > kb || (ka == kb && ea < eb);
}

// Wave-wide argmax of (key, index) with ties to the lower index.
__device__ __forceinline__ void wave_argmax(float& key, int& idx) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float ok = __shfl_xor(key, off);
        int oi = __shfl_xor(idx, off);
        if (beats(ok, oi, key, idx)) {
            key = ok;
            idx = oi;
        }
    }
}

template <int PL>
__global__ void __launch_bounds__(256)
route_select(const float* __restrict__ logits, int nsplit, const float* __restrict__ bias,
             float* __restrict__ logits_copy, int32_t* __restrict__ ids, float* __restrict__ wout, int T, int E,
             int k, int score_fn, int n_groups, int topk_groups, int group_score, int renorm, float scale) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const float* l = logits + (size_t)t * E;
    float key[PL], raw[PL];
    bool ok[PL];
    // expert e = lane + 64 * i
    float zmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        int e = lane + 64 * i;
        ok[i] = e < E;
        // the logit is the sum of the K-split partials, in split order
        float v = 0.0f;
        if (ok[i]) {
            v = l[e];
            for (int p = 1; p < nsplit; ++p) v += l[(size_t)p * T * E + e];
        }
        if (logits_copy && ok[i]) logits_copy[(size_t)t * E + e] = v;
        float b = (bias && ok[i]) ? bias[e] : 0.0f;
        if (score_fn == MOE_SCORE_SOFTMAX) {
            key[i] = v + b;
            raw[i] = key[i];
            if (ok[i]) zmax = fmaxf(zmax, key[i]);
        } else {
            float s = 1.0f / (1.0f + __expf(-v));
            raw[i] = s;
            key[i] = s + b;
        }
    }
    if (score_fn == MOE_SCORE_SOFTMAX) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, off));
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            raw[i] = ok[i] ? __expf(raw[i] - zmax) : 0.0f;
            sum += raw[i];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if (!renorm) {
#pragma unroll
            for (int i = 0; i < PL; ++i) raw[i] = raw[i] / sum;
        }
    }
    // group limit
    bool allowed[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) allowed[i] = ok[i];
    if (n_groups > 1 && n_groups == 2 * PL && E == 64 * PL) {
        // Groups of 32 experts (the DeepSeek-V3 shape): group 2 i + h is
        // register i of lanes 32 h .. 32 h + 31, so one half-wave butterfly per
        // register gives two groups' top-2 keys at once.  The kept groups are
        // those ranked below topk_groups, ties to the lower group: the same
        // choice as taking the best group topk_groups times.
        float gsc[2 * PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            float b1 = key[i], b2 = -INFINITY;
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) {
                const float o1 = __shfl_xor(b1, off), o2 = __shfl_xor(b2, off);
                const float n1 = fmaxf(b1, o1);
                const float n2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
                b1 = n1;
                b2 = n2;
            }
            const float g = group_score == MOE_GROUP_MAX ? b1 : b1 + b2;
            gsc[2 * i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 0));
            gsc[2 * i + 1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 32));
        }
        uint32_t kept_mask = 0;
#pragma unroll
        for (int g = 0; g < 2 * PL; ++g) {
            int rank = 0;
#pragma unroll
            for (int h = 0; h < 2 * PL; ++h) rank += (gsc[h] > gsc[g] || (gsc[h] == gsc[g] && h < g)) ? 1 : 0;
            if (rank < topk_groups) kept_mask |= 1u << g;
        }
#pragma unroll
        for (int i = 0; i < PL; ++i) allowed[i] = (kept_mask >> (2 * i + (lane >> 5))) & 1u;
    } else if (n_groups > 1) {
        const int gs = E / n_groups;
        float gk = -INFINITY;  // lane g holds the score of group g
        for (int g = 0; g < n_groups; ++g) {
            float b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                int e = lane + 64 * i;
                if (ok[i] && e / gs == g) {
                    if (key[i] > b1) {
                        b2 = b1;
                        b1 = key[i];
                    } else if (key[i] > b2) {
                        b2 = key[i];
                    }
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                float o1 = __shfl_xor(b1, off), o2 = __shfl_xor(b2, off);
                float n1 = fmaxf(b1, o1);
                float n2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
                b1 = n1;
                b2 = n2;
            }
            if (lane == g) gk = (group_score == MOE_GROUP_MAX || gs == 1) ? b1 : b1 + b2;
        }
        bool kept = false, gtaken = lane >= n_groups;
        for (int r = 0; r < topk_groups; ++r) {
            float bk = gtaken ? -INFINITY : gk;
            int bi = gtaken ? 0x7FFFFFFF : lane;
            wave_argmax(bk, bi);
            if (lane == bi) {
                kept = true;
                gtaken = true;
            }
        }
        uint64_t kept_mask = __ballot(kept);
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            int e = lane + 64 * i;
            allowed[i] = ok[i] && ((kept_mask >> (e / gs)) & 1ull);
        }
    }
    // top-k, slot by slot
    float rsum = 0.0f, my_raw = 0.0f;  // lane j holds the raw score of slot j
    for (int j = 0; j < k; ++j) {
        float bk = -INFINITY;
        int bi = 0x7FFFFFFF;
        bool any = false;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            int e = lane + 64 * i;
            if (allowed[i] && (!any || key[i] > bk)) {  // ascending e: first wins ties
                bk = key[i];
                bi = e;
                any = true;
            }
        }
        wave_argmax(bk, bi);
        float rv = 0.0f;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            int e = lane + 64 * i;
            if (e == bi) {
                allowed[i] = false;
                rv = raw[i];
            }
        }
        // owner lane of expert bi is bi % 64
        rv = __shfl(rv, bi & 63);
        rsum += rv;
        if (lane == j) {
            ids[(size_t)t * k + j] = bi;
            my_raw = rv;
        }
    }
    if (lane < k) {
        float wgt = renorm ? my_raw / rsum : my_raw;
        wout[(size_t)t * k + lane] = wgt * scale;
    }
}

// TS lanes per token (a team of 8 or 16), lane j of a team holding experts
// j * M .. j * M + M - 1 of its token (E = TS * M) -- with 8 groups, group g
// is lanes g * TS / 8 .. of the team -- so a wave serves 64 / TS tokens and
// every reduction is a butterfly inside the team.  The same arithmetic and tie rules as
// route_select: the partial logits summed in split order, keys and raw scores,
// group scores (top-2 sum or max) ranked with ties to the lower group, then k
// rounds of (per-lane best allowed key, ties to the lower expert; team argmax,
// ties to the lower expert), the winner's raw score recorded by lane j % 8 of
// the team for slot j, the renormalising sum taken in slot order.
template <int TS, int M, bool SOFTMAX, bool BIAS>
__global__ void __launch_bounds__(256)
route_select_team(const float* __restrict__ logits, int nsplit, const float* __restrict__ bias,
                  float* __restrict__ logits_copy, int32_t* __restrict__ ids, float* __restrict__ wout, int T,
                  int k, int grouped, int topk_groups, int group_score, int renorm, float scale) {
    constexpr int E = TS * M, GL = TS / 8;  // GL: lanes of a group (8 groups)
    const int lane = threadIdx.x & 63, tl = lane & (TS - 1);
    const int t = (blockIdx.x * 256 + threadIdx.x) / TS;  // 256 / TS tokens per workgroup
    const bool live = t < T;
    const int tc = live ? t : T - 1;  // finished lanes shadow a live token and write nothing
    const int e0 = tl * M;
    // the logits: split 0, then each further split added in order (all loads
    // of a split in flight together)
    float key[M], raw[M];
    {
        const float* l = logits + (size_t)tc * E + e0;
#pragma unroll
        for (int i = 0; i < M; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(l + i);
            raw[i] = v[0];
            raw[i + 1] = v[1];
            raw[i + 2] = v[2];
            raw[i + 3] = v[3];
        }
        for (int p = 1; p < nsplit; ++p) {
            const float* lp = l + (size_t)p * T * E;
            f32x4 o[M / 4];
#pragma unroll
            for (int i = 0; i < M / 4; ++i) o[i] = *reinterpret_cast<const f32x4*>(lp + 4 * i);
#pragma unroll
            for (int i = 0; i < M / 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) raw[4 * i + j] += o[i][j];
        }
        if (logits_copy && live) {
#pragma unroll
            for (int i = 0; i < M; i += 4)
                *reinterpret_cast<f32x4*>(logits_copy + (size_t)tc * E + e0 + i) =
                    f32x4{raw[i], raw[i + 1], raw[i + 2], raw[i + 3]};
        }
    }
    float b[M];
#pragma unroll
    for (int i = 0; i < M; ++i) b[i] = BIAS ? bias[e0 + i] : 0.0f;
    float zmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if constexpr (SOFTMAX) {
            key[i] = raw[i] + b[i];
            raw[i] = key[i];
            zmax = fmaxf(zmax, key[i]);
        } else {
            const float sg = 1.0f / (1.0f + __expf(-raw[i]));
            raw[i] = sg;
            key[i] = sg + b[i];
        }
    }
    if constexpr (SOFTMAX) {
#pragma unroll
        for (int off = 1; off < TS; off <<= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, off, TS));
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            raw[i] = __expf(raw[i] - zmax);
            sum += raw[i];
        }
#pragma unroll
        for (int off = 1; off < TS; off <<= 1) sum += __shfl_xor(sum, off, TS);
        if (!renorm) {
#pragma unroll
            for (int i = 0; i < M; ++i) raw[i] = raw[i] / sum;
        }
    }
    // group limit: lane tl is in group tl / GL; kept when ranked below topk_groups
    bool kept = true;
    if (grouped) {
        float b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const float v = key[i];
            b2 = fmaxf(b2, fminf(b1, v));
            b1 = fmaxf(b1, v);
        }
#pragma unroll
        for (int off = 1; off < GL; off <<= 1) {  // the group's top two over its lanes
            const float o1 = __shfl_xor(b1, off, TS), o2 = __shfl_xor(b2, off, TS);
            const float n1 = fmaxf(b1, o1);
            b2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
            b1 = n1;
        }
        const float g = group_score == MOE_GROUP_MAX ? b1 : b1 + b2;
        const int mg = tl / GL;
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float o = __shfl(g, j * GL, TS);
            rank += (o > g || (o == g && j < mg)) ? 1 : 0;
        }
        kept = rank < topk_groups;
    }
    uint64_t taken = kept ? 0ull : ~0ull;  // bit i: expert e0 + i is no longer a candidate
    float rsum = 0.0f, my_raw[2] = {0.0f, 0.0f};
    int my_id[2] = {0, 0};
    for (int j = 0; j < k; ++j) {
        float bk = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            if (!((taken >> i) & 1ull) && (bi == 0x7FFFFFFF || key[i] > bk)) {  // ascending: first wins ties
                bk = key[i];
                bi = e0 + i;
            }
        }
#pragma unroll
        for (int off = 1; off < TS; off <<= 1) {
            const float ok = __shfl_xor(bk, off, TS);
            const int oi = __shfl_xor(bi, off, TS);
            if (beats(ok, oi, bk, bi)) {
                bk = ok;
                bi = oi;
            }
        }
        float rv = 0.0f;
        if (bi >= e0 && bi < e0 + M) {
            const int i = bi - e0;
#pragma unroll
            for (int q = 0; q < M; ++q)
                if (q == i) rv = raw[q];
            taken |= 1ull << i;
        }
        rv = __shfl(rv, bi / M, TS);  // from the owner lane of the team
        rsum += rv;
        if (j % TS == tl) {
            my_raw[j / TS] = rv;
            my_id[j / TS] = bi;
        }
    }
    if (!live) return;
#pragma unroll
    for (int h = 0; h < 16 / TS; ++h) {
        const int j = TS * h + tl;
        if (j < k) {
            ids[(size_t)t * k + j] = my_id[h];
            wout[(size_t)t * k + j] = (renorm ? my_raw[h] / rsum : my_raw[h]) * scale;
        }
    }
}

}  // namespace

int router_splits(const moe_cfg& c) {
    if (c.act_dtype != MOE_BF16) return 1;
    const int blocks = ((c.T + RB_M - 1) / RB_M) * ((c.E + RB_N - 1) / RB_N);
    if (blocks == 0) return 1;                      // T == 0
    int sp = (256 + blocks - 1) / blocks;          // about one workgroup per CU
    sp = sp < 1 ? 1 : (sp > 8 ? 8 : sp);
    const int kmax = (c.H + 255) / 256;             // at least 256 columns per split
    return sp < kmax ? sp : kmax;
}

hipError_t launch_router_logits(const moe_cfg& c, const void* x, const void* w_router, float* logits,
                                hipStream_t s, uint8_t* x_q, float* x_scale) {
    if (c.act_dtype == MOE_BF16) {
        const int sp = router_splits(c);
        const int kq = x_q ? 128 : RB_K;  // quantising: whole 128-column blocks per split
        const int ksplit = ((c.H + sp - 1) / sp + kq - 1) / kq * kq;
        dim3 grid((c.T + RB_M - 1) / RB_M, (c.E + RB_N - 1) / RB_N, sp);
        if (x_q)
            hipLaunchKernelGGL(router_logits_bf16<true>, grid, dim3(RB_THREADS), 0, s,
                               static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                               logits, c.T, c.H, c.E, ksplit, x_q, x_scale);
        else
            hipLaunchKernelGGL(router_logits_bf16<false>, grid, dim3(RB_THREADS), 0, s,
                               static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                               logits, c.T, c.H, c.E, ksplit, nullptr, nullptr);
    } else {
        int64_t n = (int64_t)c.T * c.E;
        hipLaunchKernelGGL(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(x), static_cast<const float*>(w_router), logits,
                           c.T, c.H, c.E);
    }
    return hipGetLastError();
}

hipError_t launch_route_select(const moe_cfg& c, const float* logits, int nsplit, const float* bias,
                               float* logits_copy, int32_t* ids, float* w, hipStream_t s) {
    // the team kernels: E = TS * M experts, M in {16, 32} (TS = 16 for E = 256
    // or 512, 8 for E = 128), no group limit or 8 groups, at most 16 slots
    const bool grouped = c.n_groups > 1;
    const int TS = (c.E == 256 || c.E == 512) ? 16 : 8;
    const int M = c.E / TS;
    if (c.E % TS == 0 && (M == 16 || M == 32) && (!grouped || c.n_groups == 8) && c.k <= 16) {
        const dim3 tg((unsigned)((c.T * TS + 255) / 256)), tb(256);
        const bool sm = c.score_fn == MOE_SCORE_SOFTMAX, bs = bias != nullptr;
#define TEAM(TT, MM, SM, BS)                                                                                   \
        hipLaunchKernelGGL((route_select_team<TT, MM, SM, BS>), tg, tb, 0, s, logits, nsplit, bias, logits_copy, \
                           ids, w, c.T, c.k, grouped ? 1 : 0, c.topk_groups, c.group_score, c.renormalize,     \
                           c.routed_scale)
#define TEAM_M(TT, MM)                              \
        if (sm && bs) TEAM(TT, MM, true, true);     \
        else if (sm) TEAM(TT, MM, true, false);     \
        else if (bs) TEAM(TT, MM, false, true);     \
        else TEAM(TT, MM, false, false);
        if (TS == 16 && M == 16) {
            TEAM_M(16, 16)
        } else if (TS == 16) {
            TEAM_M(16, 32)
        } else {
            TEAM_M(8, 16)
        }
#undef TEAM_M
#undef TEAM
        return hipGetLastError();
    }
    dim3 grid((c.T + 3) / 4), block(256);
    int pl = (c.E + 63) / 64;
#define SEL(P)                                                                                      \
    hipLaunchKernelGGL(route_select<P>, grid, block, 0, s, logits, nsplit, bias, logits_copy, ids, w, c.T, \
                       c.E, c.k, c.score_fn, c.n_groups, c.topk_groups, c.group_score,            \
                       c.renormalize, c.routed_scale)
    if (pl <= 1) SEL(1);
    else if (pl <= 2) SEL(2);
    else if (pl <= 4) SEL(4);
    else if (pl <= 8) SEL(8);
    else SEL(16);
#undef SEL
    return hipGetLastError();
}

}  // namespace moe
