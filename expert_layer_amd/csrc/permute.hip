// permute.hip -- dispatch of the (token, choice) pairs into expert-contiguous
// rows: token counts per expert, their prefix sums, and the token payload
// ("ASAP", section 3.2.1 and Table 2: token metadata = counts per expert;
// token payload = hidden states).
//
// A deterministic counting sort, no order-dependent atomics:
//  1. perm_hist    per block of 256 tokens, an LDS histogram of expert ids;
//  2. perm_scan    one workgroup: per expert, exclusive prefix over blocks, then
//                  the exclusive prefix of padded counts over experts;
//  3. perm_scatter per block, an LDS bitmask of the tokens that chose each
//                  expert; a pair's rank inside its expert is the population
//                  count of the mask below its token, so rows follow ascending
//                  token order whatever the scheduling;
//  4. perm_gather  token-major copy: each token row of x is read once from HBM
//                  and written to its k destination rows with 16-byte stores;
//  5. perm_zero    padding rows (m_tile > 1) are zero-filled.
#include "common.hpp"

namespace moe {
namespace {

constexpr int PB = 256;  // tokens per block

__global__ void __launch_bounds__(PB)
perm_hist(const int32_t* __restrict__ ids, int32_t* __restrict__ hist, int T, int k, int E) {
    extern __shared__ int32_t cnt[];
    for (int e = threadIdx.x; e < E; e += PB) cnt[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * PB + threadIdx.x;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicAdd(&cnt[ids[(size_t)t * k + j]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += PB) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads; thread e owns expert e (E <= 1024).
__global__ void __launch_bounds__(1024)
perm_scan(const int32_t* __restrict__ hist, int32_t* __restrict__ base, int32_t* __restrict__ counts,
          int32_t* __restrict__ offsets, int nblk, int E, int m_tile) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
    int total = 0;
    if (e < E)
        for (int b = 0; b < nblk; ++b) {
            int v = hist[(size_t)b * E + e];
            base[(size_t)b * E + e] = total;  // relative; made absolute below
            total += v;
        }
    int padded = e < E ? ((total + m_tile - 1) / m_tile) * m_tile : 0;
    // inclusive wave scan
    int incl = padded;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    int excl = before + incl - padded;
    if (e < E) {
        counts[e] = total;
        offsets[e] = excl;
        for (int b = 0; b < nblk; ++b) base[(size_t)b * E + e] += excl;
    }
    if (e == E - 1) offsets[E] = excl + padded;
}

__global__ void __launch_bounds__(256) fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void __launch_bounds__(PB)
perm_scatter(const int32_t* __restrict__ ids, const int32_t* __restrict__ base, int32_t* __restrict__ row_src,
             int32_t* __restrict__ tok_row, int T, int k, int E) {
    extern __shared__ uint32_t mask[];  // [E][PB / 32]
    constexpr int W = PB / 32;
    for (int i = threadIdx.x; i < E * W; i += PB) mask[i] = 0;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = blockIdx.x * PB + tl;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&mask[ids[(size_t)t * k + j] * W + (tl >> 5)], 1u << (tl & 31));
    __syncthreads();
    if (t >= T) return;
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const uint32_t* m = mask + e * W;
        int rank = __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
        for (int w = 0; w < (tl >> 5); ++w) rank += __popc(m[w]);
        const int row = base[(size_t)blockIdx.x * E + e] + rank;
        row_src[row] = t * k + j;
        tok_row[(size_t)t * k + j] = row;
    }
}

// One workgroup per token: x[t] is read once and stored to its k rows.
__global__ void __launch_bounds__(256)
perm_gather(const uint8_t* __restrict__ x, const float* __restrict__ x_scale, const int32_t* __restrict__ tok_row,
            uint8_t* __restrict__ x_perm, float* __restrict__ x_perm_scale, int k, int row_bytes,
            int n_scale) {
    const int t = blockIdx.x;
    __shared__ int32_t rows[32];
    if (threadIdx.x < k) rows[threadIdx.x] = tok_row[(size_t)t * k + threadIdx.x];
    __syncthreads();
    const int nchunk = row_bytes / 16;
    const i32x4* src = reinterpret_cast<const i32x4*>(x + (size_t)t * row_bytes);
    for (int c = threadIdx.x; c < nchunk; c += 256) {
        i32x4 v = __builtin_nontemporal_load(src + c);
        for (int j = 0; j < k; ++j)
            reinterpret_cast<i32x4*>(x_perm + (size_t)rows[j] * row_bytes)[c] = v;
    }
    if (x_scale)
        for (int c = threadIdx.x; c < n_scale; c += 256) {
            float v = x_scale[(size_t)t * n_scale + c];
            for (int j = 0; j < k; ++j) x_perm_scale[(size_t)rows[j] * n_scale + c] = v;
        }
}

// Tiled bf16 output: one workgroup per token; x[t] is read once and its
// 16-byte chunks are stored to the tiled blocks of its k rows (and of row
// shared_row0 + t when the shared expert needs the token too).
__global__ void __launch_bounds__(256)
perm_gather_tiled(const uint16_t* __restrict__ x, const int32_t* __restrict__ tok_row, uint16_t* __restrict__ x_perm,
                  int k, int H, int KS, int64_t shared_row0) {
    const int t = blockIdx.x;
    __shared__ int64_t rows[33];
    if (threadIdx.x < k) rows[threadIdx.x] = tok_row[(size_t)t * k + threadIdx.x];
    if (threadIdx.x == 32) rows[32] = shared_row0 >= 0 ? shared_row0 + t : -1;
    __syncthreads();
    // chunks past H up to the last 32-column block are K padding: zeros
    const int nchunk = H / 8, nchunk_pad = KS * 4;
    const i32x4* src = reinterpret_cast<const i32x4*>(x + (size_t)t * H);
    i32x4* dst = reinterpret_cast<i32x4*>(x_perm);
    const int64_t srow = rows[32];
    for (int c = threadIdx.x; c < nchunk_pad; c += 256) {
        const i32x4 v = c < nchunk ? __builtin_nontemporal_load(src + c) : i32x4{0, 0, 0, 0};
        for (int j = 0; j < k; ++j) dst[tiled_chunk(rows[j], c, KS)] = v;
        if (srow >= 0) dst[tiled_chunk(srow, c, KS)] = v;
    }
}

__global__ void __launch_bounds__(256)
perm_zero_tiled(const int32_t* __restrict__ row_src, uint16_t* __restrict__ x_perm, int64_t max_rows, int KS) {
    const int sub = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + sub;
    if (r >= max_rows || row_src[r] != -1) return;
    i32x4* dst = reinterpret_cast<i32x4*>(x_perm);
    for (int c = lane; c < KS * 4; c += 64) dst[tiled_chunk(r, c, KS)] = i32x4{0, 0, 0, 0};
}

// Zero the payload of padding rows (row_src == -1); 4 rows per workgroup.
__global__ void __launch_bounds__(256)
perm_zero(const int32_t* __restrict__ row_src, uint8_t* __restrict__ x_perm, float* __restrict__ x_perm_scale,
          int64_t max_rows, int row_bytes, int n_scale) {
    const int sub = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + sub;
    if (r >= max_rows || row_src[r] != -1) return;
    i32x4* dst = reinterpret_cast<i32x4*>(x_perm + (size_t)r * row_bytes);
    for (int c = lane; c < row_bytes / 16; c += 64) dst[c] = i32x4{0, 0, 0, 0};
    if (x_perm_scale)
        for (int c = lane; c < n_scale; c += 64) x_perm_scale[(size_t)r * n_scale + c] = 0.0f;
}

}  // namespace

int permute_blocks(int T) { return (T + PB - 1) / PB; }

static int dtype_bytes(int d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

hipError_t launch_permute(const moe_cfg& c, const void* x, const float* x_scale, const int32_t* ids,
                          int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t* tok_row,
                          void* x_perm, float* x_perm_scale, int64_t max_rows, PermuteWs ws,
                          PermuteLayout lay, hipStream_t s) {
    const int nblk = permute_blocks(c.T);
    const int m_tile = c.m_tile > 0 ? c.m_tile : 1;
    hipLaunchKernelGGL(perm_hist, dim3(nblk), dim3(PB), c.E * sizeof(int32_t), s, ids, ws.hist, c.T, c.k,
                       c.E);
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, ws.hist, ws.base, counts, offsets, nblk, c.E,
                       m_tile);
    if (m_tile > 1)
        hipLaunchKernelGGL(fill_i32, dim3((unsigned)((max_rows + 255) / 256)), dim3(256), 0, s, row_src,
                           max_rows, -1);
    hipLaunchKernelGGL(perm_scatter, dim3(nblk), dim3(PB), (size_t)c.E * (PB / 32) * sizeof(uint32_t), s,
                       ids, ws.base, row_src, tok_row, c.T, c.k, c.E);
    if (lay.tiled) {
        const int KS = (c.H + 31) / 32;
        hipLaunchKernelGGL(perm_gather_tiled, dim3(c.T), dim3(256), 0, s, static_cast<const uint16_t*>(x), tok_row,
                           static_cast<uint16_t*>(x_perm), c.k, c.H, KS, lay.shared_row0);
        if (m_tile > 1)
            hipLaunchKernelGGL(perm_zero_tiled, dim3((unsigned)((max_rows + 3) / 4)), dim3(256), 0, s, row_src,
                               static_cast<uint16_t*>(x_perm), max_rows, KS);
        return hipGetLastError();
    }
    const int row_bytes = c.H * dtype_bytes(c.act_dtype);
    const int n_scale = c.act_dtype == MOE_FP8_E4M3 ? c.H / 128 : 0;
    const float* xs = c.act_dtype == MOE_FP8_E4M3 ? x_scale : nullptr;
    float* xps = c.act_dtype == MOE_FP8_E4M3 ? x_perm_scale : nullptr;
    hipLaunchKernelGGL(perm_gather, dim3(c.T), dim3(256), 0, s, static_cast<const uint8_t*>(x), xs, tok_row,
                       static_cast<uint8_t*>(x_perm), xps, c.k, row_bytes, n_scale);
    if (m_tile > 1)
        hipLaunchKernelGGL(perm_zero, dim3((unsigned)((max_rows + 3) / 4)), dim3(256), 0, s, row_src,
                           static_cast<uint8_t*>(x_perm), xps, max_rows, row_bytes, n_scale);
    return hipGetLastError();
}

}  // namespace moe
