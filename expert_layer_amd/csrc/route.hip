// route.hip -- router GEMM and top-k gating.
//
// The router is the "gated routing" half of the FFN side ("Memory-Compute
// Disaggregation ... AFD Architecture Analysis", section 3); its output, the
// expert IDs of every token, is what ASAP's dispatch buffers carry ("ASAP",
// Table 2, section 3.2.1).
//
// Kernel 1 (router_logits_bf16): logits[T][E] = x[T][H] . w_router[E][H]^T on
// bf16 MFMA with fp32 accumulation.  One workgroup (4 waves) owns 32 tokens x
// 128 experts; each wave one 32 x 32 block.  The K loop stages 64-wide slices
// of x and w_router through LDS (double-buffered, XOR-swizzled 16-byte
// chunks), so x streams from HBM once per expert slab and every global load is
// a coalesced 128-byte row segment.  The kernel is bound by the HBM read of x.
// Kernel 2 (route_select): one wave per token -- scores, group limit, top-k
// with ties to the lower index, renormalisation and scaling.
#include "common.hpp"

namespace moe {
namespace {

constexpr int RT_M = 32;    // tokens per workgroup
constexpr int RT_N = 128;   // experts per workgroup
constexpr int RT_K = 64;    // K slice per stage
constexpr int RT_THREADS = 256;

// LDS tile [rows][64 bf16]: 8 chunks of 16 B per row, chunk c stored at
// c ^ (row & 7) so that 8 consecutive rows reading the same logical chunk
// touch 8 different bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ void __launch_bounds__(RT_THREADS)
router_logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ logits,
                   int T, int H, int E) {
    __shared__ i32x4 sA[2][RT_M * 8];
    __shared__ i32x4 sB[2][RT_N * 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * RT_M, e0 = blockIdx.y * RT_N;
    const int nk = H / RT_K;  // H % 64 handled by the tail below

    // global -> register staging: A 256 chunks (1 per thread), B 1024 (4 per thread)
    auto load = [&](int ks, i32x4& ra, i32x4 (&rb)[4]) {
        {
            int r = tid >> 3, c = tid & 7;
            int t = t0 + r;
            int kcol = ks * RT_K + c * 8;
            if (t < T && kcol + 8 <= H) ra = *reinterpret_cast<const i32x4*>(x + (size_t)t * H + kcol);
            else ra = i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int q = tid + i * RT_THREADS;
            int r = q >> 3, c = q & 7;
            int e = e0 + r;
            int kcol = ks * RT_K + c * 8;
            if (e < E && kcol + 8 <= H) rb[i] = *reinterpret_cast<const i32x4*>(w + (size_t)e * H + kcol);
            else rb[i] = i32x4{0, 0, 0, 0};
        }
    };
    auto store = [&](int buf, const i32x4& ra, const i32x4 (&rb)[4]) {
        sA[buf][swz(tid >> 3, tid & 7)] = ra;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int q = tid + i * RT_THREADS;
            sB[buf][swz(q >> 3, q & 7)] = rb[i];
        }
    };

    f32x16 acc = {};
    i32x4 ra, rb[4];
    const int nsteps = (H + RT_K - 1) / RT_K;
    load(0, ra, rb);
    store(0, ra, rb);
    __syncthreads();
    for (int ks = 0; ks < nsteps; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nsteps) load(ks + 1, ra, rb);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            int chunk = kk * 2 + (lane >> 5);
            i32x4 a = sA[buf][swz(lane & 31, chunk)];
            i32x4 b = sB[buf][swz(wave * 32 + (lane & 31), chunk)];
            acc = mfma32x32x16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc);
        }
        if (ks + 1 < nsteps) store(buf ^ 1, ra, rb);
        __syncthreads();
    }
    (void)nk;
    // H not a multiple of 8 never reaches here (validated); a tail of H % 64
    // in multiples of 8 is covered by the zero-filled chunks above.
    const int e = e0 + wave * 32 + (lane & 31);
    if (e < E) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            int t = t0 + c_row(i, lane);
            if (t < T) logits[(size_t)t * E + e] = acc[i];
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
route_select(const float* __restrict__ logits, const float* __restrict__ bias, float* __restrict__ logits_copy,
             int32_t* __restrict__ ids, float* __restrict__ wout, int T, int E, int k, int score_fn,
             int n_groups, int topk_groups, int group_score, int renorm, float scale) {
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
        float v = ok[i] ? l[e] : 0.0f;
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
    if (n_groups > 1) {
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

hipError_t launch_router_logits(const moe_cfg& c, const void* x, const void* w_router, float* logits,
                                hipStream_t s) {
    if (c.act_dtype == MOE_BF16) {
        dim3 grid((c.T + RT_M - 1) / RT_M, (c.E + RT_N - 1) / RT_N);
        hipLaunchKernelGGL(router_logits_bf16, grid, dim3(RT_THREADS), 0, s,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                           logits, c.T, c.H, c.E);
    } else {
        int64_t n = (int64_t)c.T * c.E;
        hipLaunchKernelGGL(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(x), static_cast<const float*>(w_router), logits,
                           c.T, c.H, c.E);
    }
    return hipGetLastError();
}

hipError_t launch_route_select(const moe_cfg& c, const float* logits, const float* bias,
                               float* logits_copy, int32_t* ids, float* w, hipStream_t s) {
    dim3 grid((c.T + 3) / 4), block(256);
    int pl = (c.E + 63) / 64;
#define SEL(P)                                                                                      \
    hipLaunchKernelGGL(route_select<P>, grid, block, 0, s, logits, bias, logits_copy, ids, w, c.T, \
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
