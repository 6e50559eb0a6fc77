// permute.hip -- dispatch of the (token, choice) pairs into expert-contiguous
// rows: token counts per expert, their prefix sums, and the token payload
// ("ASAP", section 3.2.1 and Table 2: token metadata = counts per expert;
// token payload = hidden states).
//
// A deterministic counting sort, no order-dependent atomics:
//  1. perm_hist    per block of 256 tokens, an LDS histogram of expert ids;
//  2. perm_scan    one workgroup: per expert, exclusive prefix over blocks, then
//                  the exclusive prefix of padded counts over experts, and -1 in
//                  row_src for the rows no pair fills;
//  3. perm_scatter per block, an LDS bitmask of the tokens that chose each
//                  expert; a pair's rank inside its expert is the population
//                  count of the mask below its token, so rows follow ascending
//                  token order whatever the scheduling;
//  4. perm_gather  token-major copy: each token row of x is read once from HBM
//                  and written to its k destination rows with 16-byte stores
//                  (row-major x_perm); perm_band_tiled instead writes the tiled
//                  x_perm band by band, gathering each row from its token;
//  5. perm_zero    padding rows (m_tile > 1) of the row-major x_perm are zeroed.
// With the indexed layout (moe_layer's) steps 4 and 5 do not run: only the
// maps are written, and the grouped FFN reads each dispatched row from x
// through row_src, so the payload crosses HBM once, inside GEMM1.
#include <mutex>

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

// One workgroup of 1024 threads; thread e owns expert e (E <= 1024).  The
// block counts are read in groups of 8 independent loads.  With row_src, the
// rows that no pair fills -- each segment's padding up to a multiple of m_tile
// and the rows from offsets[E] to max_rows -- get -1 here (perm_scatter
// writes the others).
__global__ void __launch_bounds__(1024)
perm_scan(const int32_t* __restrict__ hist, int32_t* __restrict__ base, int32_t* __restrict__ counts,
          int32_t* __restrict__ offsets, int nblk, int E, int m_tile, int32_t* __restrict__ row_src,
          int64_t max_rows) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
    int total = 0;
    if (e < E)
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = b0 + i < nblk ? hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) total += v[i];
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
    const int excl = before + incl - padded;
    if (e < E) {
        counts[e] = total;
        offsets[e] = excl;
        int run = excl;
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = b0 + i < nblk ? hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (b0 + i < nblk) base[(size_t)(b0 + i) * E + e] = run;
                run += v[i];
            }
        }
    }
    if (e == E - 1) offsets[E] = excl + padded;
    if (row_src) {
        if (e < E)
            for (int r = excl + total; r < excl + padded; ++r) row_src[r] = -1;
        int all = 0;  // offsets[E]: the padded counts of every wave
        for (int w = 0; w < 16; ++w) all += wsum[w];
        for (int64_t r = all + e; r < max_rows; r += 1024) row_src[r] = -1;
    }
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

// Tiled bf16 output, gathered by destination: one workgroup per band of 16
// rows writes the band's ceil(H / 32) blocks of 1 KiB as one contiguous run;
// each 16-byte chunk is read from the row's token in x (zeros for padding rows,
// for rows past max_rows and for the column padding).  Bands at and after
// rows_pad hold token rows_pad + t (the shared expert's copy of x).
__global__ void __launch_bounds__(256)
perm_band_tiled(const uint16_t* __restrict__ x, const int32_t* __restrict__ row_src, uint16_t* __restrict__ x_perm,
                int64_t max_rows, int64_t rows_pad, int T, int k, int H, int KS) {
    const int64_t band = blockIdx.x;
    __shared__ int32_t tok[16];  // token of each row of the band, -1 for a zero row
    if (threadIdx.x < 16) {
        const int64_t r = band * 16 + threadIdx.x;
        int32_t t = -1;
        if (r < rows_pad) {
            if (r < max_rows) {
                const int32_t v = row_src[r];
                t = v >= 0 ? v / k : -1;
            }
        } else if (r - rows_pad < T) {
            t = (int32_t)(r - rows_pad);
        }
        tok[threadIdx.x] = t;
    }
    __syncthreads();
    const int nq = KS * 64, nch = H / 8;
    i32x4* dst = reinterpret_cast<i32x4*>(x_perm) + band * (int64_t)nq;
    for (int q = threadIdx.x; q < nq; q += 256) {
        const int r = (q >> 2) & 15;
        const int c = (q >> 6) * 4 + ((q & 3) ^ tile_swz(r));
        const int32_t t = tok[r];
        i32x4 v = {0, 0, 0, 0};
        if (t >= 0 && c < nch) v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(x + (size_t)t * H) + c);
        dst[q] = v;
    }
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

// Per-token quantisation of bf16 activations to OCP e4m3 with one fp32 scale
// per 1 x 128 block: s = max|x| / 448 over the block (1 for an all-zero
// block), q = e4m3_rne_sat(x / s), both divisions in fp32 (the rule the fp8
// grouped GEMM applies to h, read for the activations of a layer whose experts
// are fp8).  16 lanes own a block, 8 values each (16-byte loads, 8-byte
// stores); a workgroup of 256 threads covers 16 blocks of the [T][H / 128]
// grid, in row order.
__global__ void __launch_bounds__(256)
quant_rows_e4m3(const uint16_t* __restrict__ x, int64_t n_blocks, int nb, int H, uint8_t* __restrict__ q,
                float* __restrict__ sc) {
    const int64_t b = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // block id: row b / nb, column block b % nb
    const int l = threadIdx.x & 15;
    if (b >= n_blocks) return;  // whole 16-lane groups leave together
    const int64_t row = b / nb;
    const int cb = (int)(b - row * nb);
    const size_t off = (size_t)row * H + (size_t)cb * 128 + (size_t)l * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(x + off);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 16));
    m = fmaxf(m, __shfl_xor(m, 2, 16));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    const float s = m > 0.0f ? m / 448.0f : 1.0f;
    const uint32_t lo = e4m3x4_rne_sat(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    const uint32_t hi = e4m3x4_rne_sat(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
    if (l == 0) sc[b] = s;
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
    // rows no pair fills (m_tile padding, the tail up to max_rows) are -1 in row_src
    const bool pad_rows = m_tile > 1 || lay.tiled || !lay.payload;
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, ws.hist, ws.base, counts, offsets, nblk, c.E,
                       m_tile, pad_rows ? row_src : nullptr, max_rows);
    hipLaunchKernelGGL(perm_scatter, dim3(nblk), dim3(PB), (size_t)c.E * (PB / 32) * sizeof(uint32_t), s,
                       ids, ws.base, row_src, tok_row, c.T, c.k, c.E);
    if (!lay.payload) return hipGetLastError();
    if (lay.tiled) {
        const int KS = (c.H + 31) / 32;
        const int64_t rows_pad = (max_rows + 15) / 16 * 16;
        const int64_t bands = rows_pad / 16 + (lay.shared_row0 >= 0 ? (c.T + 15) / 16 : 0);
        hipLaunchKernelGGL(perm_band_tiled, dim3((unsigned)bands), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                           row_src, static_cast<uint16_t*>(x_perm), max_rows, rows_pad, c.T, c.k, c.H, KS);
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

// ------------------------------------------------- allocation-free permute
// The scratch of moe_permute_noalloc: the per-block expert counts and row
// bases of the counting sort (2 * ceil(T / 256) * E int32), in a file-scope
// device array of a fixed size that every GPU the library runs on holds until
// the process ends.  In host code `scratch` only names the symbol: its device
// address, which differs per GPU, comes from hipGetSymbolAddress with that GPU
// current, once, and is the only address the kernels are given.
static __device__ __align__(256) int32_t scratch[kNoAllocPermuteInts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_permute_scratch(int32_t** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<int32_t*>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

hipError_t launch_offsets_one_group(int32_t* offsets, int n, hipStream_t s) {
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(256), 0, s, offsets, (int64_t)1, 0);
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(256), 0, s, offsets + 1, (int64_t)1, (int32_t)n);
    return hipGetLastError();
}

hipError_t launch_quant_rows_e4m3(const void* x, int T, int H, uint8_t* q, float* sc, hipStream_t s) {
    const int nb = H / 128;
    const int64_t n_blocks = (int64_t)T * nb;
    if (n_blocks == 0) return hipSuccess;
    const int64_t grid = (n_blocks + 15) / 16;
    hipLaunchKernelGGL(quant_rows_e4m3, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       n_blocks, nb, H, q, sc);
    return hipGetLastError();
}

}  // namespace moe
