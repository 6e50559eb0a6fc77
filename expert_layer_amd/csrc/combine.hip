// combine.hip -- weighted gather-reduce of the expert results back to token
// order ("ASAP", section 3.2.2: the expert results of every token and choice
// return to the token's owner and are combined), plus the shared expert.
//
//   out[t][h] = sum_{j<k} w[t][j] * y_rows[tok_row[t][j]][h]  (+ y_shared[t][h])
//
// One workgroup per token; threads own 8-column chunks and read them from
// the k expert rows with 16-byte loads.  Pure HBM streaming: the expert rows
// are read once, the output written once.  The rows are gathered in expert
// order, so each read is a latency-bound random 16-byte access; the k reads of
// a chunk are issued together to keep enough of them in flight.
#include "common.hpp"

namespace moe {
namespace {

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    i32x4 a = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t u = (uint32_t)a[i];
        v[2 * i] = __uint_as_float(u << 16);
        v[2 * i + 1] = __uint_as_float(u & 0xFFFF0000u);
    }
}

template <typename OT>
__device__ __forceinline__ void store8(OT* o, const float (&acc)[8]) {
    if constexpr (sizeof(OT) == 4) {
        f32x4* p = reinterpret_cast<f32x4*>(o);
        p[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
        p[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
        i32x4 p;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = (int)((uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16));
        *reinterpret_cast<i32x4*>(o) = p;
    }
}

// Raw 16-byte loads of 8 values (fp32: two), unpacked after every load of a
// chunk has been issued.
template <typename YT>
struct Raw8;
template <>
struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    }
    __device__ __forceinline__ void fma_into(float wj, float (&acc)[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i] = fmaf(wj, a[i], acc[i]);
            acc[4 + i] = fmaf(wj, b[i], acc[4 + i]);
        }
    }
};
template <>
struct Raw8<uint16_t> {
    i32x4 a;
    __device__ __forceinline__ void load(const uint16_t* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
    }
    __device__ __forceinline__ void fma_into(float wj, float (&acc)[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = (uint32_t)a[i];
            acc[2 * i] = fmaf(wj, __uint_as_float(u << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wj, __uint_as_float(u & 0xFFFF0000u), acc[2 * i + 1]);
        }
    }
};

// One workgroup per token; thread i owns the 8-column chunks i and i + 256 of
// each pass of 512 chunks.  With KT = k known at compile time (the layer's
// common k = 8) the loads of all k rows of both chunks are issued before the
// first multiply-add, so 2 k loads a thread are in flight; otherwise rows are
// taken one at a time.  Either way the sum runs in slot order j = 0 .. k-1,
// then the shared term.
template <typename YT, typename OT, int KT>
__global__ void __launch_bounds__(256)
combine_kernel(const YT* __restrict__ y, const int32_t* __restrict__ tok_row, const float* __restrict__ tw,
               const YT* __restrict__ ysh, OT* __restrict__ out, int k, int H) {
    const int t = blockIdx.x;
    __shared__ int32_t rows[32];
    __shared__ float wts[32];
    if (threadIdx.x < k) {
        rows[threadIdx.x] = tok_row[(size_t)t * k + threadIdx.x];
        wts[threadIdx.x] = tw[(size_t)t * k + threadIdx.x];
    }
    __syncthreads();
    const int nchunk = H / 8;
    for (int c0 = threadIdx.x; c0 < nchunk; c0 += 512) {
        const int c1 = c0 + 256;
        const bool two = c1 < nchunk;
        float a0[8] = {0, 0, 0, 0, 0, 0, 0, 0}, a1[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (KT > 0) {
            Raw8<YT> r0[KT], r1[KT];
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const YT* row = y + (size_t)rows[j] * H;
                r0[j].load(row + c0 * 8);
                if (two) r1[j].load(row + c1 * 8);
            }
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                r0[j].fma_into(wts[j], a0);
                if (two) r1[j].fma_into(wts[j], a1);
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const YT* row = y + (size_t)rows[j] * H;
                Raw8<YT> v0, v1;
                v0.load(row + c0 * 8);
                if (two) v1.load(row + c1 * 8);
                v0.fma_into(wts[j], a0);
                if (two) v1.fma_into(wts[j], a1);
            }
        }
        if (ysh) {
            float v0[8], v1[8];
            load8<YT>(ysh + (size_t)t * H + c0 * 8, v0);
            if (two) load8<YT>(ysh + (size_t)t * H + c1 * 8, v1);
#pragma unroll
            for (int i = 0; i < 8; ++i) a0[i] += v0[i];
            if (two)
#pragma unroll
                for (int i = 0; i < 8; ++i) a1[i] += v1[i];
        }
        store8<OT>(out + (size_t)t * H + c0 * 8, a0);
        if (two) store8<OT>(out + (size_t)t * H + c1 * 8, a1);
    }
}

template <typename YT, typename OT>
void launch_combine_t(const moe_cfg& c, const YT* y, const int32_t* tok_row, const float* topk_w, const YT* ys,
                      OT* out, hipStream_t s) {
    const dim3 grid(c.T), block(256);
    if (c.k == 8)
        hipLaunchKernelGGL((combine_kernel<YT, OT, 8>), grid, block, 0, s, y, tok_row, topk_w, ys, out, c.k, c.H);
    else
        hipLaunchKernelGGL((combine_kernel<YT, OT, 0>), grid, block, 0, s, y, tok_row, topk_w, ys, out, c.k, c.H);
}

}  // namespace

hipError_t launch_combine(const moe_cfg& c, const void* y_rows, const int32_t* tok_row, const float* topk_w,
                          const void* y_shared, void* out, hipStream_t s) {
    if (c.y_dtype == MOE_F32) {
        auto y = static_cast<const float*>(y_rows);
        auto ys = static_cast<const float*>(y_shared);
        if (c.out_dtype == MOE_F32) launch_combine_t(c, y, tok_row, topk_w, ys, static_cast<float*>(out), s);
        else launch_combine_t(c, y, tok_row, topk_w, ys, static_cast<uint16_t*>(out), s);
    } else {
        auto y = static_cast<const uint16_t*>(y_rows);
        auto ys = static_cast<const uint16_t*>(y_shared);
        if (c.out_dtype == MOE_F32) launch_combine_t(c, y, tok_row, topk_w, ys, static_cast<float*>(out), s);
        else launch_combine_t(c, y, tok_row, topk_w, ys, static_cast<uint16_t*>(out), s);
    }
    return hipGetLastError();
}

}  // namespace moe
