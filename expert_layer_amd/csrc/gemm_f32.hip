// gemm_f32.hip -- the grouped SwiGLU FFN for fp32 operands (no fp32 dense
// MFMA rate worth tiling for at the small shapes this path serves).  Same
// work list as the bf16 path, 64-row tiles; each workgroup computes a 64 x 64
// output tile with a 16-wide K slice staged in LDS and 4 x 4 outputs per
// thread (for GEMM1 both the gate and the up accumulator, so h = silu(g) * u
// is formed in registers).
#include "common.hpp"

namespace moe {
namespace {

constexpr int TB = 64, TK = 16;

struct F32Args {
    const float* a_routed;
    const float* a_shared;
    const float* w0_routed;
    const float* w1_routed;
    const float* w0_shared;
    const float* w1_shared;
    void* out_routed;
    void* out_shared;
    const int4* tiles;
    const int32_t* n_tiles;
    const int2* work;
    int E, NT, K_routed, K_shared, N_routed, N_shared, out_f32;
};

template <int MODE>
__global__ void __launch_bounds__(256) ffn_gemm_f32(F32Args p) {
    __shared__ float sA[TK][TB + 4];
    __shared__ float sB0[TK][TB + 4];
    __shared__ float sB1[TK][TB + 4];
    const int n_valid = p.n_tiles[0] * p.NT;
    const int L = blockIdx.x;
    if (L >= n_valid) return;
    const int2 wl = p.work[L];
    const int mt = wl.x, nt = wl.y;
    const int4 td = p.tiles[mt];
    const int g = td.x, row0 = td.y, M = td.z - td.y;
    const bool shared = g == p.E;
    const int K = shared ? p.K_shared : p.K_routed;
    const int N = shared ? p.N_shared : p.N_routed;
    const int n0 = nt * TB;
    if (n0 >= N) return;
    const float* A = shared ? p.a_shared : p.a_routed;
    const size_t wmat = (size_t)K * N;
    const float* W0 = shared ? p.w0_shared : p.w0_routed + (size_t)g * wmat;
    const float* W1 = MODE == 0 ? (shared ? p.w1_shared : p.w1_routed + (size_t)g * wmat) : nullptr;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc0[4][4] = {}, acc1[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        for (int i = 0; i < 4; ++i) {
            const int e = threadIdx.x + 256 * i, r = e / TK, kk = e % TK;
            const int kg = k0 + kk;
            sA[kk][r] = (r < M && kg < K) ? A[(size_t)(row0 + r) * K + kg] : 0.0f;
            const int col = n0 + r;
            sB0[kk][r] = (col < N && kg < K) ? W0[(size_t)col * K + kg] : 0.0f;
            if (MODE == 0) sB1[kk][r] = (col < N && kg < K) ? W1[(size_t)col * K + kg] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b0[4], b1[4];
            for (int i = 0; i < 4; ++i) {
                a[i] = sA[kk][ty * 4 + i];
                b0[i] = sB0[kk][tx * 4 + i];
                b1[i] = MODE == 0 ? sB1[kk][tx * 4 + i] : 0.0f;
            }
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j) {
                    acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
                    if (MODE == 0) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
                }
        }
        __syncthreads();
    }
    void* out = shared ? p.out_shared : p.out_routed;
    for (int i = 0; i < 4; ++i) {
        const int r = ty * 4 + i;
        if (r >= M) continue;
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx * 4 + j;
            if (col >= N) continue;
            const size_t o = (size_t)(row0 + r) * N + col;
            if (MODE == 0) {
                static_cast<float*>(out)[o] = silu_f(acc0[i][j]) * acc1[i][j];
            } else if (p.out_f32) {
                static_cast<float*>(out)[o] = acc0[i][j];
            } else {
                static_cast<uint16_t*>(out)[o] = f32_to_bf16(acc0[i][j]);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const moe_cfg& c, int64_t max_tiles, int64_t n_rows_cap, const void* x_rows,
                           const int32_t* offsets, const moe_weights& w, const void* x_tokens, void* y_rows,
                           void* y_shared, const FfnWork& wk, void* h, void* h_sh, hipStream_t s) {
    const int has_sh = c.has_shared ? 1 : 0;
    hipError_t e0 = launch_build_tiles(c, offsets, TB, n_rows_cap, wk, s);
    if (e0 != hipSuccess) return e0;
    F32Args a{};
    a.tiles = reinterpret_cast<const int4*>(wk.tiles);
    a.n_tiles = wk.n_tiles;
    a.work = reinterpret_cast<const int2*>(wk.work1);
    a.E = c.E;
    a.a_routed = static_cast<const float*>(x_rows);
    a.a_shared = static_cast<const float*>(x_tokens);
    a.w0_routed = static_cast<const float*>(w.w_gate);
    a.w1_routed = static_cast<const float*>(w.w_up);
    a.w0_shared = static_cast<const float*>(w.sh_gate);
    a.w1_shared = static_cast<const float*>(w.sh_up);
    a.out_routed = h;
    a.out_shared = h_sh;
    a.K_routed = c.H;
    a.K_shared = c.H;
    a.N_routed = c.I;
    a.N_shared = has_sh ? c.I_shared : c.I;
    a.NT = wk.nt1;
    a.out_f32 = 1;
    hipLaunchKernelGGL(ffn_gemm_f32<0>, dim3((unsigned)(max_tiles * a.NT)), dim3(256), 0, s, a);
    a.a_routed = static_cast<const float*>(h);
    a.a_shared = static_cast<const float*>(h_sh);
    a.w0_routed = static_cast<const float*>(w.w_down);
    a.w1_routed = nullptr;
    a.w0_shared = static_cast<const float*>(w.sh_down);
    a.w1_shared = nullptr;
    a.out_routed = y_rows;
    a.out_shared = y_shared;
    a.K_routed = c.I;
    a.K_shared = has_sh ? c.I_shared : c.I;
    a.N_routed = c.H;
    a.N_shared = c.H;
    a.NT = wk.nt2;
    a.work = reinterpret_cast<const int2*>(wk.work2);
    a.out_f32 = c.y_dtype == MOE_F32;
    hipLaunchKernelGGL(ffn_gemm_f32<1>, dim3((unsigned)(max_tiles * a.NT)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
