// route.hip -- router GEMM and top-k gating.
//
// The router is the "gated routing" half of the FFN side ("Memory-Compute
// Disaggregation ... AFD Architecture Analysis", section 3); its output, the
// expert IDs of every token, is what ASAP's dispatch buffers carry ("ASAP",
// Table 2, section 3.2.1).
//
// Kernel 1 (router_logits_bf16): logits[T][E] = x[T][H] . w_router[E][H]^T on
// bf16 MFMA with fp32 accumulation.  One workgroup (4 waves) owns 128 tokens x
// 256 experts over one slice of K; each wave 128 tokens x 64 experts (4 x 2
// blocks of 32 x 32).  Operands move HBM -> LDS by buffer_load ... lds through
// a ring of four 32-wide stages (XOR-swizzled 16-byte chunks), so x streams
// from HBM once per 256 experts.  K is split so that T / 128 token blocks
// still fill the chip; the splits write fp32 partial logits that route_select
// adds in split order (a fixed order, so the result does not depend on
// scheduling).  The kernel is bound by the HBM read of x.
// Kernel 2 (route_select): one wave per token -- the partial logits summed,
// scores, group limit, top-k with ties to the lower index, renormalisation and
// scaling.
#include "common.hpp"

namespace moe {
namespace {

constexpr int RB_M = 128, RB_N = 256, RB_K = 32, RB_NST = 4, RB_THREADS = 256;
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
    uint32_t va[2], vb[4];   // byte offset of this lane's chunk at k = k0 (kROOB: outside the tile)
    uint32_t lc[2], lcb[4];  // the chunk's column offset (elements) inside a stage
    int k0, k_end, nsteps;
};

// Loads of stage t into buffer BUF: 2 A and 4 B chunk loads per lane, zero
// past the tile's rows and past the split's K range.
template <int BUF>
__device__ __forceinline__ void rdma(const RDma& d, int t, int wave) {
    i32x4* buf = rring<BUF>();
    const int kst = d.k0 + t * RB_K;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const bool ok = d.va[i] != kROOB && kst + (int)d.lc[i] < d.k_end;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (rlds_t)(buf + (wave * 2 + i) * 64), 16,
                                                 ok ? d.va[i] + (uint32_t)t * (RB_K * 2) : kROOB, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = d.vb[i] != kROOB && kst + (int)d.lcb[i] < d.k_end;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (rlds_t)(buf + kRA + (wave * 4 + i) * 64), 16,
                                                 ok ? d.vb[i] + (uint32_t)t * (RB_K * 2) : kROOB, 0, 0, 0);
    }
}

// One stage: two 16-wide k steps of the wave's 4 x 2 blocks of 32 x 32.
template <int BUF>
__device__ __forceinline__ void rstage(int wave, int lane, f32x16 (&acc)[4][2]) {
    const i32x4* buf = rring<BUF>();
    const int l32 = lane & 31;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = kk * 2 + (lane >> 5);
        i32x4 a[4], b[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r * 32 + l32;
            a[r] = buf[row * 4 + (chunk ^ tile_swz(row))];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = (wave & 3) * 64 + c * 32 + l32;  // provably inside the buffer
            b[c] = buf[kRA + row * 4 + (chunk ^ tile_swz(row))];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                acc[r][c] = mfma32x32x16(__builtin_bit_cast(bf16x8, a[r]), __builtin_bit_cast(bf16x8, b[c]),
                                         acc[r][c]);
    }
}

// partial[split][t][e] = sum over the split's K range of x[t][h] * w[e][h].
// Workgroup: 128 tokens x 256 experts x one K range; wave w owns experts
// 64 w + [0, 64).  Operands move HBM -> LDS by buffer_load ... lds through a
// ring of four stages (64-byte row segments, the chunks XOR-swizzled by row so
// that fragment reads are free of bank conflicts).  Splitting K lets T / 128
// token blocks fill the chip; the router weights are then read from L2 about
// T / 128 times instead of once per 32 tokens.
__global__ void __launch_bounds__(RB_THREADS)
router_logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ partial,
                   int T, int H, int E, int ksplit) {
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
    for (int i = 0; i < 2; ++i) {
        const int row = (wave * 2 + i) * 16 + (lane >> 2);
        const int logical = (lane & 3) ^ tile_swz(row);
        d.lc[i] = (uint32_t)(logical * 8);
        d.va[i] = row < mt ? ((uint32_t)row * (uint32_t)H + (uint32_t)(d.k0 + logical * 8)) * 2u : kROOB;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (wave * 4 + i) * 16 + (lane >> 2);
        const int logical = (lane & 3) ^ tile_swz(row);
        d.lcb[i] = (uint32_t)(logical * 8);
        d.vb[i] = row < ne ? ((uint32_t)row * (uint32_t)H + (uint32_t)(d.k0 + logical * 8)) * 2u : kROOB;
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[r][c] = f32x16{};

    // Stages 0..2 in flight; at stage s (buffer s % 4): wait until its loads
    // have landed (the 12 loads of stages s+1, s+2 may still fly), one barrier
    // -- everyone's stage s has landed and everyone is done with stage s-1 --
    // refill stage s-1's buffer with stage s+3, then compute on stage s.
    rdma<0>(d, 0, wave);
    rdma<1>(d, 1, wave);
    rdma<2>(d, 2, wave);
    const int nturns = (d.nsteps + RB_NST - 1) / RB_NST;
    for (int s = 0; s < nturns * RB_NST; s += RB_NST) {
#define ROUTER_STAGE(J)                                              \
        __builtin_amdgcn_s_waitcnt((12 & 15) | ((12 >> 4) << 14) | 0x0070); \
        rbarrier();                                                  \
        __builtin_amdgcn_sched_barrier(0);                           \
        rdma<(J + 3) % RB_NST>(d, s + J + 3, wave);                  \
        __builtin_amdgcn_sched_barrier(0);                           \
        rstage<J>(wave, lane, acc);                                  \
        __builtin_amdgcn_sched_barrier(0);
        ROUTER_STAGE(0)
        ROUTER_STAGE(1)
        ROUTER_STAGE(2)
        ROUTER_STAGE(3)
#undef ROUTER_STAGE
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no LDS DMA may outlive the workgroup
    float* out = partial + (size_t)split * T * E;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int e = e0 + wave * 64 + c * 32 + (lane & 31);
        if (e < E) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = t0 + r * 32 + c_row(i, lane);
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
                                hipStream_t s) {
    if (c.act_dtype == MOE_BF16) {
        const int sp = router_splits(c);
        const int ksplit = ((c.H + sp - 1) / sp + RB_K - 1) / RB_K * RB_K;
        dim3 grid((c.T + RB_M - 1) / RB_M, (c.E + RB_N - 1) / RB_N, sp);
        hipLaunchKernelGGL(router_logits_bf16, grid, dim3(RB_THREADS), 0, s,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                           logits, c.T, c.H, c.E, ksplit);
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
