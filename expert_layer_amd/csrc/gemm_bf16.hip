// gemm_bf16.hip -- the grouped SwiGLU FFN on bf16 MFMA ("ASAP", section
// 3.4.2: the MoE kernel is a grouped matrix multiplication, hidden states on
// the left, the layer's expert weights on the right).
//
// Work list.  ffn_build_tiles turns the expert offsets into a device-side list
// of M tiles {group, row_begin, row_end}: an expert with n rows gets
// ceil(n / 256) tiles of equal height (rounded up to 32 rows), so a skewed
// expert spreads over many workgroups and a cold one costs one short tile.  The
// shared expert is one more group over all T tokens.  Nothing returns to the
// host: the grid is sized from the host-known bound and blocks past the
// device-side count exit at once.
//
// Tile.  256 rows x 256 weight rows x 64-wide K slices, 4 waves.  Each wave
// owns all 256 rows and 64 weight rows (two 32-column MFMA blocks), so a short
// tile skips whole 32-row blocks and all four SIMDs stay equally busy.
//   GEMM1: the 64 weight rows of wave w are 32 gate rows and the 32 up rows of
//          the same h columns, so SwiGLU h = silu(g) * u is formed in
//          registers and stored once as bf16.
//   GEMM2: 256 output columns of y = h . w_down^T, fp32 or bf16.
// Operands stream through LDS in 16-byte chunks, double-buffered, with the
// chunk index XOR-swizzled by row; each global load instruction reads whole
// 128-byte row segments.  Tiles are ordered (M tile, N tile) with N fastest
// and remapped so that a contiguous run lives on one XCD: the 16 (or 28) N
// tiles of one M tile share the A panel in that XCD's L2.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTH = 256;
constexpr int kLdsBytes = 2 * (BM + BN) * BK * 2;  // 128 KiB

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

struct GemmArgs {
    const uint16_t* a_routed;  // GEMM1: x_rows [rows][H]; GEMM2: h [rows][I]
    const uint16_t* a_shared;  // GEMM1: x_tokens [T][H]; GEMM2: h_sh [T][I_sh]
    const uint16_t* w0_routed; // GEMM1: w_gate [E][I][H]; GEMM2: w_down [E][H][I]
    const uint16_t* w1_routed; // GEMM1: w_up
    const uint16_t* w0_shared;
    const uint16_t* w1_shared;
    void* out_routed;          // GEMM1: h; GEMM2: y_rows
    void* out_shared;          // GEMM1: h_sh; GEMM2: y_shared
    const int4* tiles;
    const int32_t* n_tiles;
    int E;
    int NT;                    // N tiles per M tile in the launch grid
    int K_routed, K_shared;    // reduction length
    int N_routed, N_shared;    // GEMM1: h columns (I, I_sh); GEMM2: H
    int out_f32;               // GEMM2 output dtype
};

template <int MODE>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
ffn_gemm_bf16(GemmArgs p) {
    extern __shared__ i32x4 lds[];
    i32x4* sA = lds;                   // [2][BM * 8]
    i32x4* sB = lds + 2 * BM * 8;      // [2][BN * 8]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31;
    const int n_valid = p.n_tiles[0] * p.NT;
    const int L = xcd_remap(blockIdx.x, n_valid);
    if (L < 0) return;
    const int mt = L / p.NT, nt = L % p.NT;
    const int4 td = p.tiles[mt];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const bool shared = g == p.E;
    const int K = shared ? p.K_shared : p.K_routed;
    const int N = shared ? p.N_shared : p.N_routed;
    const int n0 = MODE == 0 ? nt * (BN / 2) : nt * BN;
    if (n0 >= N) return;
    const int nrb = (M + 31) >> 5;

    const uint16_t* A = shared ? p.a_shared : p.a_routed;
    const size_t wmat = (size_t)K * (size_t)N;
    const uint16_t* W0 = shared ? p.w0_shared : p.w0_routed + (size_t)g * wmat;
    const uint16_t* W1 = MODE == 0 ? (shared ? p.w1_shared : p.w1_routed + (size_t)g * wmat) : nullptr;

    // Global source of the 8 A chunks and 8 B chunks this thread stages.
    const uint16_t* a_src[8];
    const uint16_t* b_src[8];
    bool a_ok[8], b_ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = tid + NTH * i, r = q >> 3, c = q & 7;
        a_ok[i] = r < M;
        a_src[i] = A + (size_t)(row0 + (a_ok[i] ? r : 0)) * K + c * 8;
        int col;
        const uint16_t* Wm;
        if (MODE == 0) {
            const int wj = r >> 6, jj = r & 63;
            col = n0 + wj * 32 + (jj & 31);
            Wm = jj < 32 ? W0 : W1;
        } else {
            col = n0 + r;
            Wm = W0;
        }
        b_ok[i] = col < N;
        b_src[i] = Wm + (size_t)(b_ok[i] ? col : 0) * K + c * 8;
    }
    const int ccol = (tid & 7) * 8;  // K offset of this thread's chunks inside a slice

    i32x4 ra[8], rb[8];
    auto load = [&](int ks) {
        const int kc = ks * BK;
        const bool kin = kc + ccol < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ra[i] = (a_ok[i] && kin) ? *reinterpret_cast<const i32x4*>(a_src[i] + kc) : i32x4{0, 0, 0, 0};
            rb[i] = (b_ok[i] && kin) ? *reinterpret_cast<const i32x4*>(b_src[i] + kc) : i32x4{0, 0, 0, 0};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + NTH * i, r = q >> 3, c = q & 7;
            sA[buf * BM * 8 + swz(r, c)] = ra[i];
            sB[buf * BN * 8 + swz(r, c)] = rb[i];
        }
    };

    f32x16 acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc0[i] = f32x16{};
        acc1[i] = f32x16{};
    }
    const int nsteps = (K + BK - 1) / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int ks = 0; ks < nsteps; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nsteps) load(ks + 1);
        const i32x4* A_l = sA + buf * BM * 8;
        const i32x4* B_l = sB + buf * BN * 8;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = kk * 2 + (lane >> 5);
            const bf16x8 b0 = __builtin_bit_cast(bf16x8, B_l[swz(wave * 64 + l32, chunk)]);
            const bf16x8 b1 = __builtin_bit_cast(bf16x8, B_l[swz(wave * 64 + 32 + l32, chunk)]);
#pragma unroll
            for (int rbk = 0; rbk < 8; ++rbk) {
                if (rbk < nrb) {
                    const bf16x8 a = __builtin_bit_cast(bf16x8, A_l[swz(rbk * 32 + l32, chunk)]);
                    acc0[rbk] = mfma32x32x16(a, b0, acc0[rbk]);
                    acc1[rbk] = mfma32x32x16(a, b1, acc1[rbk]);
                }
            }
        }
        if (ks + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }

    void* out = shared ? p.out_shared : p.out_routed;
    if (MODE == 0) {
        const int col = n0 + wave * 32 + l32;
        if (col < N) {
            uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
            for (int rbk = 0; rbk < 8; ++rbk) {
                if (rbk < nrb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = rbk * 32 + c_row(i, lane);
                        if (r < M) {
                            const float gv = acc0[rbk][i], uv = acc1[rbk][i];
                            h[(size_t)(row0 + r) * N + col] = f32_to_bf16(silu_f(gv) * uv);
                        }
                    }
                }
            }
        }
    } else {
        const int c0 = n0 + wave * 64 + l32, c1 = c0 + 32;
#pragma unroll
        for (int rbk = 0; rbk < 8; ++rbk) {
            if (rbk < nrb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rbk * 32 + c_row(i, lane);
                    if (r < M) {
                        const size_t o = (size_t)(row0 + r) * N;
                        if (p.out_f32) {
                            float* y = static_cast<float*>(out);
                            if (c0 < N) y[o + c0] = acc0[rbk][i];
                            if (c1 < N) y[o + c1] = acc1[rbk][i];
                        } else {
                            uint16_t* y = static_cast<uint16_t*>(out);
                            if (c0 < N) y[o + c0] = f32_to_bf16(acc0[rbk][i]);
                            if (c1 < N) y[o + c1] = f32_to_bf16(acc1[rbk][i]);
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

// ------------------------------------------------------------- tile list
// One workgroup of 1024 threads.  Group g < E covers rows [offsets[g],
// offsets[g+1]); group E (the shared expert, when present) covers tokens
// [0, T).  A group of n rows gets nmt = ceil(n / bm) tiles of height
// ceil(ceil(n / nmt) / 32) * 32 (the last one shorter).
__global__ void __launch_bounds__(1024)
ffn_build_tiles(const int32_t* __restrict__ offsets, int E, int has_shared, int T, int bm, int rows_cap,
                int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
    __shared__ int32_t wsum[16];
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
    // thread tid owns group tid; thread 0 also owns group 1024 (E == 1024 + shared)
    int b0 = 0, e0 = 0, n0 = 0;
    if (tid < G) {
        group_rows(tid, b0, e0);
        n0 = (e0 - b0 + bm - 1) / bm;
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
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    const int start = before + incl - n0;
    auto emit = [&](int g, int b, int e, int nmt, int st) {
        if (nmt == 0) return;
        const int n = e - b;
        int hgt = (n + nmt - 1) / nmt;
        hgt = ((hgt + 31) / 32) * 32;
        for (int m = 0; m < nmt; ++m) {
            const int rb = b + m * hgt;
            const int re = min(e, rb + hgt);
            tiles[st + m] = int4{g, rb, re, 0};
        }
    };
    if (tid < G) emit(tid, b0, e0, n0, start);
    if (tid == 0 && G > 1024) {
        int b, e;
        group_rows(1024, b, e);
        const int n = (e - b + bm - 1) / bm;
        emit(1024, b, e, n, total);
        total += n;
    }
    if (tid == 0) n_tiles[0] = total;
}

hipError_t launch_build_tiles(const moe_cfg& c, const int32_t* offsets, int bm, int64_t rows_cap,
                              int32_t* tiles, int32_t* n_tiles, hipStream_t s) {
    hipLaunchKernelGGL(ffn_build_tiles, dim3(1), dim3(1024), 0, s, offsets, c.E, c.has_shared ? 1 : 0, c.T,
                       bm, (int)rows_cap, reinterpret_cast<int4*>(tiles), n_tiles);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows, const int32_t* offsets,
                            const moe_weights& w, const void* x_tokens, void* y_rows, void* y_shared,
                            int32_t* tiles, int32_t* n_tiles, void* h, void* h_sh, hipStream_t s) {
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_bf16<0>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gemm_bf16<1>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e1 != hipSuccess) return e1;
        if (e2 != hipSuccess) return e2;
        attr_done = true;
    }
    const int has_sh = c.has_shared ? 1 : 0;
    hipError_t e0 = launch_build_tiles(c, offsets, BM, n_rows_cap, tiles, n_tiles, s);
    if (e0 != hipSuccess) return e0;
    GemmArgs a{};
    a.tiles = reinterpret_cast<const int4*>(tiles);
    a.n_tiles = n_tiles;
    a.E = c.E;
    // GEMM1: gate/up + SwiGLU -> h
    a.a_routed = static_cast<const uint16_t*>(x_rows);
    a.a_shared = static_cast<const uint16_t*>(x_tokens);
    a.w0_routed = static_cast<const uint16_t*>(w.w_gate);
    a.w1_routed = static_cast<const uint16_t*>(w.w_up);
    a.w0_shared = static_cast<const uint16_t*>(w.sh_gate);
    a.w1_shared = static_cast<const uint16_t*>(w.sh_up);
    a.out_routed = h;
    a.out_shared = h_sh;
    a.K_routed = c.H;
    a.K_shared = c.H;
    a.N_routed = c.I;
    a.N_shared = has_sh ? c.I_shared : c.I;
    const int nmax1 = has_sh ? (c.I > c.I_shared ? c.I : c.I_shared) : c.I;
    a.NT = (nmax1 + BN / 2 - 1) / (BN / 2);
    a.out_f32 = 0;
    hipLaunchKernelGGL(ffn_gemm_bf16<0>, dim3((unsigned)(max_tiles * a.NT)), dim3(NTH), kLdsBytes, s, a);
    // GEMM2: down -> y
    a.a_routed = static_cast<const uint16_t*>(h);
    a.a_shared = static_cast<const uint16_t*>(h_sh);
    a.w0_routed = static_cast<const uint16_t*>(w.w_down);
    a.w1_routed = nullptr;
    a.w0_shared = static_cast<const uint16_t*>(w.sh_down);
    a.w1_shared = nullptr;
    a.out_routed = y_rows;
    a.out_shared = y_shared;
    a.K_routed = c.I;
    a.K_shared = has_sh ? c.I_shared : c.I;
    a.N_routed = c.H;
    a.N_shared = c.H;
    a.NT = (c.H + BN - 1) / BN;
    a.out_f32 = c.y_dtype == MOE_F32;
    hipLaunchKernelGGL(ffn_gemm_bf16<1>, dim3((unsigned)(max_tiles * a.NT)), dim3(NTH), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace moe
