// capi.cpp -- the C ABI of the MoE layer (include/moe.h): argument checks,
// workspace layout and the enqueue order of the kernels.  Host code only.
// Every entry point checks all arguments before the first launch, so an
// invalid call enqueues nothing; no entry point allocates, frees or
// synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "common.hpp"

// The layer can combine inside the shared expert's GEMM2 (bf16 y, from this
// many tokens on) when the environment sets MOE_FUSED_COMBINE=1.  With the
// grouped GEMMs' work queues the separate combine pass times 0.2-0.7% faster
// at 8192 tokens and the same at 16384, so it is the default; below 4096
// tokens the fused form costs 0.8% (512 tokens) and is never used.
#ifndef MOE_FUSED_COMBINE_MIN_T
#define MOE_FUSED_COMBINE_MIN_T 4096
#endif
constexpr int kFusedCombineMinT = MOE_FUSED_COMBINE_MIN_T;
bool fused_combine_requested() {
    const char* v = std::getenv("MOE_FUSED_COMBINE");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
}

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

int dtype_bytes(int d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

int m_tile_of(const moe_cfg& c) { return c.m_tile > 0 ? c.m_tile : 1; }

constexpr int64_t kMaxRows = INT32_MAX / 2;

int64_t max_rows_of(const moe_cfg& c) {
    return (int64_t)c.T * c.k + (int64_t)c.E * (m_tile_of(c) - 1);
}

moe_status check_cfg(const moe_cfg* cp) {
    if (!cp) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
    const moe_cfg& c = *cp;
    if (c.T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d must be >= 0", c.T);
    if (c.H <= 0 || c.H % 8) return fail(MOE_ERR_INVALID_ARG, "H=%d must be a positive multiple of 8", c.H);
    if (c.E < 1 || c.E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d must be in [1, 1024]", c.E);
    if (c.k < 1 || c.k > c.E || c.k > 32)
        return fail(MOE_ERR_INVALID_ARG, "k=%d must be in [1, min(E, 32)]", c.k);
    if (c.I <= 0 || c.I % 8) return fail(MOE_ERR_INVALID_ARG, "I=%d must be a positive multiple of 8", c.I);
    if (c.n_groups < 1 || c.n_groups > 64 || c.E % c.n_groups)
        return fail(MOE_ERR_INVALID_ARG, "n_groups=%d must divide E=%d and be in [1, 64]", c.n_groups, c.E);
    if (c.topk_groups < 1 || c.topk_groups > c.n_groups)
        return fail(MOE_ERR_INVALID_ARG, "topk_groups=%d must be in [1, n_groups]", c.topk_groups);
    if ((int64_t)c.k > (int64_t)c.topk_groups * (c.E / c.n_groups))
        return fail(MOE_ERR_INVALID_ARG, "k=%d exceeds the experts of the kept groups", c.k);
    if (c.score_fn != MOE_SCORE_SOFTMAX && c.score_fn != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARG, "score_fn=%d", c.score_fn);
    if (c.group_score != MOE_GROUP_TOP2_SUM && c.group_score != MOE_GROUP_MAX)
        return fail(MOE_ERR_INVALID_ARG, "group_score=%d", c.group_score);
    if (c.renormalize != 0 && c.renormalize != 1) return fail(MOE_ERR_INVALID_ARG, "renormalize=%d", c.renormalize);
    if (!std::isfinite(c.routed_scale)) return fail(MOE_ERR_INVALID_ARG, "routed_scale is not finite");
    if (c.has_shared != 0 && c.has_shared != 1) return fail(MOE_ERR_INVALID_ARG, "has_shared=%d", c.has_shared);
    if (c.has_shared && (c.I_shared <= 0 || c.I_shared % 8))
        return fail(MOE_ERR_INVALID_ARG, "I_shared=%d must be a positive multiple of 8", c.I_shared);
    if (c.act_dtype < MOE_F32 || c.act_dtype > MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "act_dtype=%d", c.act_dtype);
    if (c.w_dtype < MOE_F32 || c.w_dtype > MOE_FP4_E2M1) return fail(MOE_ERR_INVALID_ARG, "w_dtype=%d", c.w_dtype);
    // low-precision experts: e4m3 or MXFP4 weights; with bf16 activations the
    // layer quantises x per token to e4m3 (fp8x); the grouped FFN takes e4m3 rows
    const bool lowp = c.w_dtype == MOE_FP8_E4M3 || c.w_dtype == MOE_FP4_E2M1;
    const bool fp8x = c.act_dtype == MOE_BF16 && lowp;
    const bool fp4w = c.act_dtype == MOE_FP8_E4M3 && c.w_dtype == MOE_FP4_E2M1;
    if (c.w_dtype != c.act_dtype && !fp8x && !fp4w)
        return fail(MOE_ERR_UNSUPPORTED, "w_dtype=%d with act_dtype=%d", c.w_dtype, c.act_dtype);
    if (c.y_dtype != MOE_F32 && c.y_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "y_dtype=%d", c.y_dtype);
    if (c.out_dtype != MOE_F32 && c.out_dtype != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d", c.out_dtype);
    if (lowp) {
        if (c.H % 128 || c.I % 128)
            return fail(MOE_ERR_INVALID_ARG, "fp8 needs H and I multiples of 128 (H=%d, I=%d)", c.H, c.I);
        if (c.H > 16384 || c.I > 16384)
            return fail(MOE_ERR_UNSUPPORTED, "fp8 supports H and I up to 16384 (H=%d, I=%d)", c.H, c.I);
        if (c.has_shared && !fp8x) return fail(MOE_ERR_UNSUPPORTED, "fp8 activations with a shared expert");
        if (c.has_shared && (c.I_shared % 128 || c.I_shared > 16384))
            return fail(MOE_ERR_UNSUPPORTED, "fp8 needs I_shared a multiple of 128 up to 16384 (I_shared=%d)",
                        c.I_shared);
    }
    if (c.act_dtype == MOE_BF16 && !fp8x) {
        // the bf16 GEMMs address one expert's matrices (and, indexed, all of x)
        // through buffer descriptors below 2 GiB
        auto mat = [&](int I) { return (int64_t)((I + 127) / 128) * 128 * 2 * ((c.H + 31) / 32) * 32 * 2; };
        if (c.H > 65536 || c.I > 65536 || mat(c.I) >= ((int64_t)1 << 31) ||
            (c.has_shared && (c.I_shared > 65536 || mat(c.I_shared) >= ((int64_t)1 << 31))))
            return fail(MOE_ERR_UNSUPPORTED, "bf16 supports H, I <= 65536 and one expert's gate+up under 2 GiB");
    }
    if (c.m_tile < 0 || c.m_tile > 4096) return fail(MOE_ERR_INVALID_ARG, "m_tile=%d must be in [0, 4096]", c.m_tile);
    if (c.x_layout != MOE_LAYOUT_ROWMAJOR && c.x_layout != MOE_LAYOUT_TILED && c.x_layout != MOE_LAYOUT_INDEXED)
        return fail(MOE_ERR_INVALID_ARG, "x_layout=%d", c.x_layout);
    if (c.x_layout == MOE_LAYOUT_INDEXED) {
        if (c.act_dtype != MOE_BF16 && c.act_dtype != MOE_FP8_E4M3)
            return fail(MOE_ERR_UNSUPPORTED, "indexed x_perm is bf16 or e4m3 only");
        if ((int64_t)c.T * c.H * dtype_bytes(c.act_dtype) >= ((int64_t)1 << 31))
            return fail(MOE_ERR_UNSUPPORTED, "indexed x_perm needs x under 2 GiB");
    }
    if (c.x_layout == MOE_LAYOUT_TILED) {
        if (c.act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "tiled x_perm is bf16 only");
        if (c.m_tile % 16 || c.m_tile == 0)
            return fail(MOE_ERR_INVALID_ARG, "tiled x_perm needs m_tile a multiple of 16 (m_tile=%d)", c.m_tile);
    }
    if (max_rows_of(c) > kMaxRows) return fail(MOE_ERR_INVALID_ARG, "T*k + E*(m_tile-1) is too large");
    if ((int64_t)c.T * c.H > (int64_t)INT32_MAX * 8) return fail(MOE_ERR_INVALID_ARG, "T*H is too large");
    return MOE_OK;
}

// ---------------------------------------------------------------- workspace

struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t n) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off = align_up(off + n * sizeof(T));
        return p;
    }
};

int ffn_bm(const moe_cfg& c) {
    if (c.act_dtype == MOE_F32) return moe::kFfnBmF32;
    // fp8 launches run 224- or 128-row tiles: size the tile list for the shorter
    return c.act_dtype == MOE_FP8_E4M3 ? moe::kFfnBmFp8Small : moe::kFfnBmBf16;
}

int64_t ffn_max_tiles(const moe_cfg& c, int64_t n_rows_cap) {
    const int bm = ffn_bm(c);
    return (n_rows_cap + bm - 1) / bm + c.E + (c.has_shared ? (c.T + bm - 1) / bm : 0) + 1;
}

// K-split partial logits of the router
size_t route_ws(const moe_cfg& c) {
    return align_up((size_t)moe::router_splits(c) * c.T * c.E * sizeof(float));
}

struct PermuteCarve {
    moe::PermuteWs ws;
    size_t bytes;
};
PermuteCarve permute_carve(const moe_cfg& c, void* p) {
    Carve cv(p);
    const size_t n = (size_t)moe::permute_blocks(c.T) * c.E;
    moe::PermuteWs w;
    w.hist = cv.take<int32_t>(n);
    w.base = cv.take<int32_t>(n);
    return {w, cv.off};
}

struct FfnCarve {
    moe::FfnWork wk;
    void* h;         // bf16: the h tile slots (max_tiles x 256 rows, tiled); fp32: [n_rows_cap][I]
    float* h_scale;  // fp8: [n_rows_cap][I / 128]
    void* h_sh;      // fp32: [T][I_shared]
    int64_t max_tiles;
    size_t bytes;
};
FfnCarve ffn_carve(const moe_cfg& c, int64_t n_rows_cap, void* p) {
    Carve cv(p);
    FfnCarve f{};
    f.max_tiles = ffn_max_tiles(c, n_rows_cap);
    const bool f32 = c.act_dtype == MOE_F32;
    const int n1 = f32 ? moe::kFfnN1F32 : moe::kFfnN1Bf16, n2 = f32 ? moe::kFfnN2F32 : moe::kFfnN2Bf16;
    const int imax = c.has_shared && c.I_shared > c.I ? c.I_shared : c.I;
    f.wk.nt1 = (imax + n1 - 1) / n1;
    f.wk.nt2 = (c.H + n2 - 1) / n2;
    f.wk.tiles = cv.take<int32_t>((size_t)f.max_tiles * 4);
    f.wk.n_tiles = cv.take<int32_t>(moe::kFfnCtlWords);
    f.wk.work1 = cv.take<int32_t>((size_t)f.max_tiles * f.wk.nt1 * 2);
    f.wk.work2 = cv.take<int32_t>((size_t)f.max_tiles * f.wk.nt2 * 2);
    if (c.act_dtype == MOE_BF16) {
        f.h = cv.take<char>((size_t)f.max_tiles * moe::h_slot_bytes(c));
    } else {
        const int hb = f32 ? 4 : 1;
        f.h = cv.take<char>((size_t)n_rows_cap * c.I * hb);
        f.h_scale = c.act_dtype == MOE_FP8_E4M3 ? cv.take<float>((size_t)n_rows_cap * (c.I / 128)) : nullptr;
        f.h_sh = c.has_shared ? cv.take<char>((size_t)c.T * c.I_shared * hb) : nullptr;
    }
    f.bytes = cv.off;
    return f;
}

// x_perm geometry.  Tiled: the routed rows occupy R16 = roundup(max_rows, 16)
// rows and the shared expert's copy of the tokens follows them.
struct XPermGeom {
    bool tiled;
    int64_t rows_pad;       // first row of the shared-expert copy (tiled)
    size_t shared_off;      // its byte offset in x_perm (tiled)
    size_t bytes;
};
XPermGeom x_perm_geom(const moe_cfg& c) {
    XPermGeom g{};
    const int64_t rows = max_rows_of(c);
    g.tiled = c.x_layout == MOE_LAYOUT_TILED;
    if (c.x_layout == MOE_LAYOUT_INDEXED) {
        g.rows_pad = rows;
        g.bytes = 0;
    } else if (g.tiled) {
        const size_t blk = (size_t)((c.H + 31) / 32) * 1024;  // one 16-row band
        g.rows_pad = (rows + 15) / 16 * 16;
        g.shared_off = (size_t)(g.rows_pad / 16) * blk;
        g.bytes = g.shared_off + (c.has_shared ? (size_t)((c.T + 15) / 16) * blk : 0);
    } else {
        g.rows_pad = rows;
        g.bytes = (size_t)rows * c.H * dtype_bytes(c.act_dtype);
    }
    return g;
}

// The indexed layout addresses all of x through one buffer descriptor, whose
// 32-bit offsets reach 2 GiB.
bool x_indexable(const moe_cfg& c, int elem_bytes) { return (int64_t)c.T * c.H * elem_bytes < ((int64_t)1 << 31); }

// The configuration moe_layer runs its stages with: expert segments padded to
// 16 rows, and for bf16 no x_perm (GEMM1 reads x through row_src) while x is
// under 2 GiB; a larger x is dispatched into the tiled x_perm.
moe_cfg layer_stage_cfg(const moe_cfg& c) {
    moe_cfg s = c;
    s.m_tile = 16;
    if (c.act_dtype == MOE_BF16)
        s.x_layout = x_indexable(c, 2) ? MOE_LAYOUT_INDEXED : MOE_LAYOUT_TILED;
    else
        s.x_layout = MOE_LAYOUT_ROWMAJOR;
    return s;
}

// Fp8 experts (bf16 activations, e4m3 weights): the layer quantises x per
// token, then runs the stages on the fp8 cfg of the quantised rows -- the
// routed experts as one grouped FFN, the shared expert as a second one over
// the T quantised tokens (one group).
bool lowp_weights(const moe_cfg& c) { return c.w_dtype == MOE_FP8_E4M3 || c.w_dtype == MOE_FP4_E2M1; }
bool fp8_experts(const moe_cfg& c) { return c.act_dtype == MOE_BF16 && lowp_weights(c); }
moe_cfg fp8_routed_cfg(const moe_cfg& c) {
    moe_cfg q = c;
    q.act_dtype = MOE_FP8_E4M3;  // the weights keep their dtype (e4m3 or MXFP4)
    q.has_shared = 0;
    q.I_shared = 0;
    q.m_tile = 16;
    // GEMM1 reads the quantised tokens through row_src while they are under
    // 2 GiB; more are dispatched into a row-major x_perm with its scales
    q.x_layout = x_indexable(c, 1) ? MOE_LAYOUT_INDEXED : MOE_LAYOUT_ROWMAJOR;
    return q;
}
moe_cfg fp8_shared_cfg(const moe_cfg& c) {
    moe_cfg q = fp8_routed_cfg(c);
    q.E = q.k = q.n_groups = q.topk_groups = 1;
    q.I = c.I_shared;
    q.m_tile = 1;
    q.x_layout = MOE_LAYOUT_ROWMAJOR;  // all T quantised tokens, in order
    return q;
}

struct LayerCarve {
    int32_t *ids, *counts, *offsets, *row_src, *tok_row;
    float* topk_w;
    void *x_perm, *y_rows, *y_shared, *scratch;
    uint8_t* x_q;                // fp8 experts: x quantised [T][H]
    float *x_s, *x_perm_scale;   // ... its scales [T][H / 128]; x_perm_scale NULL (indexed rows)
    int32_t* offsets_sh;         // ... {0, T}
    size_t bytes;
};
LayerCarve layer_carve(const moe_cfg& c, void* p) {
    Carve cv(p);
    LayerCarve l{};
    const bool f8 = fp8_experts(c);
    const moe_cfg cs = f8 ? fp8_routed_cfg(c) : layer_stage_cfg(c);
    const int64_t rows = max_rows_of(cs);
    const size_t tk = (size_t)c.T * c.k;
    l.ids = cv.take<int32_t>(tk);
    l.topk_w = cv.take<float>(tk);
    l.counts = cv.take<int32_t>(c.E);
    l.offsets = cv.take<int32_t>(c.E + 1);
    l.row_src = cv.take<int32_t>((size_t)rows);
    l.tok_row = cv.take<int32_t>(tk);
    l.x_perm = cv.take<char>(x_perm_geom(cs).bytes);
    l.y_rows = cv.take<char>((size_t)rows * c.H * dtype_bytes(c.y_dtype));
    l.y_shared = c.has_shared ? cv.take<char>((size_t)c.T * c.H * dtype_bytes(c.y_dtype)) : nullptr;
    size_t scratch = route_ws(c);
    size_t pb = permute_carve(cs, nullptr).bytes;
    size_t fb = ffn_carve(cs, rows, nullptr).bytes;
    if (f8) {
        l.x_q = cv.take<uint8_t>((size_t)c.T * c.H);
        l.x_s = cv.take<float>((size_t)c.T * (c.H / 128));
        // indexed: no dispatched copy of the rows or their scales
        l.x_perm_scale = cs.x_layout == MOE_LAYOUT_INDEXED ? nullptr : cv.take<float>((size_t)rows * (c.H / 128));
        l.offsets_sh = cv.take<int32_t>(2);
        if (c.has_shared) {
            const size_t fs = ffn_carve(fp8_shared_cfg(c), c.T, nullptr).bytes;
            if (fs > fb) fb = fs;
        }
    }
    if (pb > scratch) scratch = pb;
    if (fb > scratch) scratch = fb;
    l.scratch = cv.take<char>(scratch);
    l.bytes = cv.off;
    return l;
}

moe_status check_ws(void* ws, size_t have, size_t need) {
    if (need == 0) return MOE_OK;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return MOE_OK;
}

#define REQUIRE(p, name) \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name)
#define REQUIRE_A16(p, name) \
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name)

// Weights moe_tile_weights can rewrite: bf16 experts on bf16 rows, e4m3 experts
// (on e4m3 rows, or on bf16 activations that the layer quantises).
bool tileable(const moe_cfg& c) {
    return (c.act_dtype == MOE_BF16 && c.w_dtype == MOE_BF16) || c.w_dtype == MOE_FP8_E4M3;
}

// Checks the weight pointers a call reads (before anything is enqueued).
moe_status check_weights(const moe_cfg& c, const moe_weights* w) {
    if (!w) return fail(MOE_ERR_INVALID_ARG, "w is NULL");
    if (w->layout != MOE_LAYOUT_ROWMAJOR && w->layout != MOE_LAYOUT_TILED)
        return fail(MOE_ERR_INVALID_ARG, "w->layout=%d", w->layout);
    const bool tiled = w->layout == MOE_LAYOUT_TILED;
    if (tiled && !tileable(c)) return fail(MOE_ERR_UNSUPPORTED, "tiled weights are bf16 or e4m3 only");
    if (w->table) {
        // the matrices are read on the device, through the table
        if (c.act_dtype == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "pointer-table weights on the fp32 path");
        REQUIRE(w->layer, "w->layer");
        if (w->n_layers < 1) return fail(MOE_ERR_INVALID_ARG, "w->n_layers=%d must be >= 1", w->n_layers);
        if (reinterpret_cast<uintptr_t>(w->table) % 8) return fail(MOE_ERR_INVALID_ARG, "w->table is not 8-byte aligned");
        if (reinterpret_cast<uintptr_t>(w->layer) % 4) return fail(MOE_ERR_INVALID_ARG, "w->layer is not 4-byte aligned");
        return MOE_OK;
    }
    REQUIRE(w->w_gate, "w->w_gate");
    if (!tiled) REQUIRE(w->w_up, "w->w_up");
    REQUIRE(w->w_down, "w->w_down");
    if (lowp_weights(c)) {
        REQUIRE(w->s_gate, "w->s_gate");
        REQUIRE(w->s_up, "w->s_up");
        REQUIRE(w->s_down, "w->s_down");
    }
    if (c.has_shared) {
        REQUIRE(w->sh_gate, "w->sh_gate");
        if (!tiled) REQUIRE(w->sh_up, "w->sh_up");
        REQUIRE(w->sh_down, "w->sh_down");
        if (lowp_weights(c)) {
            REQUIRE(w->sh_s_gate, "w->sh_s_gate");
            REQUIRE(w->sh_s_up, "w->sh_s_up");
            REQUIRE(w->sh_s_down, "w->sh_s_down");
        }
    }
    return MOE_OK;
}

// The weight table of a call (tab NULL for contiguous weights); `first` is the
// table entry of the launch's group 0.
moe::WTab wtab_of(const moe_cfg& c, const moe_weights& w, int first) {
    if (!w.table) return moe::WTab{nullptr, nullptr, 0, 0, 0};
    return moe::WTab{w.table, w.layer, w.n_layers, c.E + (c.has_shared ? 1 : 0), first};
}

// Enqueue halves of the stage entry points (arguments already checked); the
// layer calls the same functions, so its kernels are the stage kernels.
moe_status permute_enqueue(const moe_cfg& c, const void* x, const float* x_scale, const int32_t* ids,
                           int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t* tok_row, void* x_perm,
                           float* x_perm_scale, void* ws, hipStream_t s) {
    const PermuteCarve pc = permute_carve(c, ws);
    const XPermGeom g = x_perm_geom(c);
    const moe::PermuteLayout lay{g.tiled ? 1 : 0, (g.tiled && c.has_shared) ? g.rows_pad : -1,
                                 c.x_layout == MOE_LAYOUT_INDEXED ? 0 : 1};
    hipError_t e = moe::launch_permute(c, x, x_scale, ids, counts, offsets, row_src, tok_row, x_perm, x_perm_scale,
                                       max_rows_of(c), pc.ws, lay, s);
    if (e != hipSuccess) return hip_fail(e, "moe_permute");
    return MOE_OK;
}

// comb_out (with tok_row, topk_w): the bf16 path's shared expert also combines
// into comb_out (see FfnOperands); the caller then runs no combine.
moe_status ffn_enqueue(const moe_cfg& c, int64_t n_rows_cap, const void* x_rows, const float* x_scale,
                       const int32_t* offsets, const int32_t* row_src, const moe_weights& w, const moe::WTab& wt,
                       const void* x_tokens, void* y_rows, void* y_shared, void* ws, hipStream_t s,
                       void* comb_out = nullptr, const int32_t* tok_row = nullptr, const float* topk_w = nullptr) {
    moe::FfnOperands op{x_rows, x_tokens, 0, 0, y_rows, y_shared, nullptr, comb_out, tok_row, topk_w};
    const XPermGeom g = x_perm_geom(c);
    if (c.x_layout == MOE_LAYOUT_INDEXED) {
        op.row_src = row_src;
        op.x_tokens = x_rows;  // x itself: the shared expert's operand too
    } else if (g.tiled) {
        op.x_rows_tiled = 1;
        if (c.has_shared) {
            op.x_tokens = static_cast<const char*>(x_rows) + g.shared_off;
            op.x_tokens_tiled = 1;
        }
    }
    FfnCarve f = ffn_carve(c, n_rows_cap, ws);
    hipError_t e;
    if (c.act_dtype == MOE_BF16)
        e = moe::launch_gemm_bf16(c, f.max_tiles, n_rows_cap, op, offsets, w, wt, f.wk, f.h, s);
    else if (c.act_dtype == MOE_F32)
        e = moe::launch_gemm_f32(c, f.max_tiles, n_rows_cap, op.x_rows, offsets, w, op.x_tokens, op.y_rows,
                                 op.y_shared, f.wk, f.h, f.h_sh, s);
    else
        e = moe::launch_gemm_fp8(c, f.max_tiles, n_rows_cap, x_rows, x_scale, op.row_src, offsets, w, wt, y_rows,
                                 f.wk, f.h, f.h_scale, s);
    if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn");
    return MOE_OK;
}

// The rest of moe_layer for low-precision experts (routing done, x quantised
// by the router): the dispatch maps (GEMM1 reads the e4m3 token rows through
// row_src), the routed and the shared grouped FFN, combine.
moe_status layer_fp8_experts(const moe_cfg& c, const moe_weights& w, void* out, const LayerCarve& l,
                             hipStream_t s) {
    const moe_cfg cq = fp8_routed_cfg(c);
    hipError_t e;
    moe_status st = permute_enqueue(cq, l.x_q, l.x_s, l.ids, l.counts, l.offsets, l.row_src, l.tok_row, l.x_perm,
                                    l.x_perm_scale, l.scratch, s);
    if (st != MOE_OK) return st;
    const bool indexed = cq.x_layout == MOE_LAYOUT_INDEXED;
    st = ffn_enqueue(cq, max_rows_of(cq), indexed ? l.x_q : l.x_perm, indexed ? l.x_s : l.x_perm_scale, l.offsets,
                     l.row_src, w, wtab_of(c, w, 0), nullptr, l.y_rows, nullptr, l.scratch, s);
    if (st != MOE_OK) return st;
    if (c.has_shared) {
        const moe_cfg c1 = fp8_shared_cfg(c);
        // the shared expert as the one group of its own launch: table entry E
        const moe_weights ws1{w.sh_gate, w.sh_up,  w.sh_down, w.sh_s_gate, w.sh_s_up, w.sh_s_down,
                              nullptr,   nullptr,  nullptr,   w.layout, nullptr, nullptr,
                              nullptr,   nullptr,  nullptr,   0};
        e = moe::launch_offsets_one_group(l.offsets_sh, c.T, s);
        if (e != hipSuccess) return hip_fail(e, "moe_layer (shared offsets)");
        st = ffn_enqueue(c1, c.T, l.x_q, l.x_s, l.offsets_sh, nullptr, ws1, wtab_of(c, w, c.E), nullptr,
                         l.y_shared, nullptr, l.scratch, s);
        if (st != MOE_OK) return st;
    }
    e = moe::launch_combine(c, l.y_rows, l.tok_row, l.topk_w, l.y_shared, out, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer (combine)");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_validate(const moe_cfg* cfg) { return check_cfg(cfg); }

int64_t moe_max_rows(const moe_cfg* cfg) {
    if (check_cfg(cfg) != MOE_OK) return -1;
    return max_rows_of(*cfg);
}

size_t moe_workspace_bytes(const moe_cfg* cfg, int32_t stage) {
    if (check_cfg(cfg) != MOE_OK) return (size_t)-1;
    const moe_cfg& c = *cfg;
    switch (stage) {
    case MOE_STAGE_ROUTE: return route_ws(c);
    case MOE_STAGE_PERMUTE: return permute_carve(c, nullptr).bytes;
    case MOE_STAGE_FFN: return ffn_carve(c, max_rows_of(c), nullptr).bytes;
    case MOE_STAGE_LAYER: return layer_carve(c, nullptr).bytes;
    default: fail(MOE_ERR_INVALID_ARG, "stage=%d", stage); return (size_t)-1;
    }
}

size_t moe_ffn_workspace_bytes(const moe_cfg* cfg, int64_t n_rows_cap) {
    if (check_cfg(cfg) != MOE_OK) return (size_t)-1;
    if (n_rows_cap < 0 || n_rows_cap > kMaxRows) {
        fail(MOE_ERR_INVALID_ARG, "n_rows_cap=%lld must be in [0, 2^30)", (long long)n_rows_cap);
        return (size_t)-1;
    }
    return ffn_carve(*cfg, n_rows_cap, nullptr).bytes;
}

moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router, const float* bias,
                     const float* logits_in, float* logits_out, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (c.act_dtype == MOE_FP8_E4M3) return fail(MOE_ERR_UNSUPPORTED, "router on fp8 activations");
    if (!logits_in) {
        REQUIRE(x, "x");
        REQUIRE(w_router, "w_router");
        REQUIRE_A16(x, "x");
        REQUIRE_A16(w_router, "w_router");
    }
    REQUIRE(topk_ids, "topk_ids");
    REQUIRE(topk_w, "topk_w");
    const bool need_ws = !logits_in;
    if (need_ws && (st = check_ws(ws, ws_bytes, route_ws(c))) != MOE_OK) return st;
    if (c.T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float* l = logits_in;
    int nsplit = 1;
    if (!logits_in) {
        hipError_t e = moe::launch_router_logits(c, x, w_router, static_cast<float*>(ws), s);
        if (e != hipSuccess) return hip_fail(e, "moe_route (logits)");
        l = static_cast<const float*>(ws);
        nsplit = moe::router_splits(c);
    }
    hipError_t e = moe::launch_route_select(c, l, nsplit, bias, logits_out, topk_ids, topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "moe_route (select)");
    return MOE_OK;
}

moe_status moe_route_quantize(const moe_cfg* cfg, const void* x, const void* w_router, const float* bias,
                              float* logits_out, int32_t* topk_ids, float* topk_w, uint8_t* x_q, float* x_scale,
                              void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (c.act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_route_quantize takes bf16 x");
    if (c.H % 128) return fail(MOE_ERR_INVALID_ARG, "moe_route_quantize needs H a multiple of 128 (H=%d)", c.H);
    REQUIRE(x, "x");
    REQUIRE(w_router, "w_router");
    REQUIRE(topk_ids, "topk_ids");
    REQUIRE(topk_w, "topk_w");
    REQUIRE(x_q, "x_q");
    REQUIRE(x_scale, "x_scale");
    REQUIRE_A16(x, "x");
    REQUIRE_A16(w_router, "w_router");
    if (reinterpret_cast<uintptr_t>(x_q) % 8) return fail(MOE_ERR_INVALID_ARG, "x_q is not 8-byte aligned");
    if (reinterpret_cast<uintptr_t>(x_scale) % 4) return fail(MOE_ERR_INVALID_ARG, "x_scale is not 4-byte aligned");
    if ((st = check_ws(ws, ws_bytes, route_ws(c))) != MOE_OK) return st;
    if (c.T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = moe::launch_router_logits(c, x, w_router, static_cast<float*>(ws), s, x_q, x_scale);
    if (e != hipSuccess) return hip_fail(e, "moe_route_quantize (logits)");
    e = moe::launch_route_select(c, static_cast<const float*>(ws), moe::router_splits(c), bias, logits_out, topk_ids,
                                 topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "moe_route_quantize (select)");
    return MOE_OK;
}

moe_status moe_permute(const moe_cfg* cfg, const void* x, const float* x_scale, const int32_t* topk_ids,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_src, int32_t* tok_row,
                       void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    REQUIRE(x, "x");
    REQUIRE(topk_ids, "topk_ids");
    REQUIRE(expert_counts, "expert_counts");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(row_src, "row_src");
    REQUIRE(tok_row, "tok_row");
    if (c.x_layout != MOE_LAYOUT_INDEXED) REQUIRE(x_perm, "x_perm");
    REQUIRE_A16(x, "x");
    REQUIRE_A16(x_perm, "x_perm");
    if (c.act_dtype == MOE_FP8_E4M3 && c.x_layout != MOE_LAYOUT_INDEXED) {
        REQUIRE(x_scale, "x_scale");
        REQUIRE(x_perm_scale, "x_perm_scale");
    }
    PermuteCarve pc = permute_carve(c, ws);
    if ((st = check_ws(ws, ws_bytes, pc.bytes)) != MOE_OK) return st;
    if (c.T == 0) return MOE_OK;
    return permute_enqueue(c, x, x_scale, topk_ids, expert_counts, expert_offsets, row_src, tok_row, x_perm,
                           x_perm_scale, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_permute_noalloc(const moe_cfg* cfg, const void* x, const float* x_scale, const int32_t* topk_ids,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_src, int32_t* tok_row,
                               void* x_perm, float* x_perm_scale, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    REQUIRE(x, "x");
    REQUIRE(topk_ids, "topk_ids");
    REQUIRE(expert_counts, "expert_counts");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(row_src, "row_src");
    REQUIRE(tok_row, "tok_row");
    if (c.x_layout != MOE_LAYOUT_INDEXED) REQUIRE(x_perm, "x_perm");
    if (c.act_dtype == MOE_FP8_E4M3 && c.x_layout != MOE_LAYOUT_INDEXED) {
        REQUIRE(x_scale, "x_scale");
        REQUIRE(x_perm_scale, "x_perm_scale");
    }
    REQUIRE_A16(x, "x");
    REQUIRE_A16(x_perm, "x_perm");
    const int64_t need = 2 * (int64_t)moe::permute_blocks(c.T) * c.E;
    if (need > moe::kNoAllocPermuteInts)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_permute_noalloc holds 2 * ceil(T / 256) * E = %lld per-block counts at most %lld "
                    "(T=%d, E=%d); use moe_permute with a workspace",
                    (long long)need, (long long)moe::kNoAllocPermuteInts, c.T, c.E);
    if (c.T == 0) return MOE_OK;
    int32_t* scratch = nullptr;
    hipError_t e = moe::noalloc_permute_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc (scratch address)");
    const size_t n = (size_t)moe::permute_blocks(c.T) * c.E;
    const moe::PermuteWs ws{scratch, scratch + n};
    const XPermGeom g = x_perm_geom(c);
    const moe::PermuteLayout lay{g.tiled ? 1 : 0, (g.tiled && c.has_shared) ? g.rows_pad : -1,
                                 c.x_layout == MOE_LAYOUT_INDEXED ? 0 : 1};
    e = moe::launch_permute(c, x, x_scale, topk_ids, expert_counts, expert_offsets, row_src, tok_row, x_perm,
                            x_perm_scale, max_rows_of(c), ws, lay, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc");
    return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_cfg* cfg, int64_t n_rows_cap, const void* x_rows, const float* x_scale,
                           const int32_t* expert_offsets, const int32_t* row_src, const moe_weights* w,
                           const void* x_tokens, void* y_rows, void* y_shared, void* ws, size_t ws_bytes,
                           void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (n_rows_cap < 0 || n_rows_cap > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "n_rows_cap=%lld must be in [0, 2^30)", (long long)n_rows_cap);
    if (fp8_experts(c))
        return fail(MOE_ERR_UNSUPPORTED, "fp8 experts take fp8 rows: quantise with moe_quantize_fp8 and call "
                                         "moe_grouped_ffn with act_dtype = MOE_FP8_E4M3");
    REQUIRE(expert_offsets, "expert_offsets");
    if ((st = check_weights(c, w)) != MOE_OK) return st;
    if (n_rows_cap > 0) {
        REQUIRE(x_rows, "x_rows");
        REQUIRE(y_rows, "y_rows");
    }
    if (c.act_dtype == MOE_FP8_E4M3) REQUIRE(x_scale, "x_scale");
    const bool tiled = c.x_layout == MOE_LAYOUT_TILED, indexed = c.x_layout == MOE_LAYOUT_INDEXED;
    if (tiled) {
        if (n_rows_cap != max_rows_of(c))
            return fail(MOE_ERR_INVALID_ARG, "tiled x_rows: n_rows_cap=%lld must equal moe_max_rows (%lld)",
                        (long long)n_rows_cap, (long long)max_rows_of(c));
        if (c.has_shared) REQUIRE(x_rows, "x_rows");
    }
    if (indexed) {
        if (n_rows_cap > 0) REQUIRE(row_src, "row_src");
        if (c.has_shared) REQUIRE(x_rows, "x_rows");
    }
    if (c.has_shared) {
        if (!tiled && !indexed) REQUIRE(x_tokens, "x_tokens");
        REQUIRE(y_shared, "y_shared");
    }
    REQUIRE_A16(x_rows, "x_rows");
    REQUIRE_A16(x_tokens, "x_tokens");
    REQUIRE_A16(y_rows, "y_rows");
    REQUIRE_A16(y_shared, "y_shared");
    const size_t need = ffn_carve(c, n_rows_cap, nullptr).bytes;
    if ((st = check_ws(ws, ws_bytes, need)) != MOE_OK) return st;
    if (n_rows_cap == 0 && !(c.has_shared && c.T > 0)) return MOE_OK;
    return ffn_enqueue(c, n_rows_cap, x_rows, x_scale, expert_offsets, row_src, *w, wtab_of(c, *w, 0), x_tokens,
                       y_rows, y_shared, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_weight_table(const moe_cfg* cfg, const moe_weights* layers, int32_t n_layers, const void** table) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (c.act_dtype == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "pointer-table weights on the fp32 path");
    REQUIRE(layers, "layers");
    REQUIRE(table, "table");
    if (n_layers < 1) return fail(MOE_ERR_INVALID_ARG, "n_layers=%d must be >= 1", n_layers);
    const bool f8 = lowp_weights(c), f4 = c.w_dtype == MOE_FP4_E2M1;
    const int G = c.E + (c.has_shared ? 1 : 0);
    // bytes of one expert's matrices (tiled: the fragment-order gate+up and
    // down) and of its scales: fp8 one fp32 per 128 x 128 block, MXFP4 one
    // E8M0 byte per 32 elements of a row
    const moe::TiledSizes t = moe::tiled_sizes(c);
    const size_t mat = f4 ? (size_t)c.I * c.H / 2 : (size_t)c.I * c.H * dtype_bytes(c.w_dtype);
    const size_t nsc = f4 ? (size_t)c.I * (c.H / 32) : f8 ? (size_t)(c.I / 128) * (c.H / 128) * 4 : 0;
    for (int32_t L = 0; L < n_layers; ++L) {
        const moe_weights& w = layers[L];
        if (w.table) return fail(MOE_ERR_INVALID_ARG, "layers[%d].table must be NULL", L);
        if ((st = check_weights(c, &w)) != MOE_OK) return st;
        const bool tiled = w.layout == MOE_LAYOUT_TILED;
        const size_t m13 = tiled ? t.w13 / c.E : mat, m2 = tiled ? t.w2 / c.E : mat;
        const void** row = table + (size_t)L * G * 6;
        for (int e = 0; e < c.E; ++e) {
            const void** r = row + (size_t)e * 6;
            r[0] = static_cast<const char*>(w.w_gate) + e * m13;
            r[1] = tiled ? nullptr : static_cast<const char*>(w.w_up) + e * mat;
            r[2] = static_cast<const char*>(w.w_down) + e * m2;
            r[3] = f8 ? reinterpret_cast<const char*>(w.s_gate) + e * nsc : nullptr;
            r[4] = f8 ? reinterpret_cast<const char*>(w.s_up) + e * nsc : nullptr;
            r[5] = f8 ? reinterpret_cast<const char*>(w.s_down) + e * nsc : nullptr;
        }
        if (c.has_shared) {
            const void** r = row + (size_t)c.E * 6;
            r[0] = w.sh_gate;
            r[1] = tiled ? nullptr : w.sh_up;
            r[2] = w.sh_down;
            r[3] = f8 ? w.sh_s_gate : nullptr;
            r[4] = f8 ? w.sh_s_up : nullptr;
            r[5] = f8 ? w.sh_s_down : nullptr;
        }
    }
    return MOE_OK;
}

size_t moe_x_perm_bytes(const moe_cfg* cfg) {
    if (check_cfg(cfg) != MOE_OK) return (size_t)-1;
    return x_perm_geom(*cfg).bytes;
}

size_t moe_tiled_weights_bytes(const moe_cfg* cfg) {
    if (check_cfg(cfg) != MOE_OK) return (size_t)-1;
    if (!tileable(*cfg)) {
        fail(MOE_ERR_UNSUPPORTED, "tiled weights are bf16 or e4m3 only");
        return (size_t)-1;
    }
    const moe::TiledSizes t = moe::tiled_sizes(*cfg);
    return align_up(t.w13) + align_up(t.w2) + align_up(t.sh13) + align_up(t.sh2);
}

moe_status moe_tile_weights(const moe_cfg* cfg, const moe_weights* src, void* dst, size_t dst_bytes,
                            moe_weights* tiled, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (!tileable(c)) return fail(MOE_ERR_UNSUPPORTED, "tiled weights are bf16 or e4m3 only");
    if ((st = check_weights(c, src)) != MOE_OK) return st;
    if (src->layout != MOE_LAYOUT_ROWMAJOR) return fail(MOE_ERR_INVALID_ARG, "src must be row-major");
    if (src->table) return fail(MOE_ERR_INVALID_ARG, "src must be contiguous (table == NULL)");
    REQUIRE(tiled, "tiled");
    const moe::TiledSizes t = moe::tiled_sizes(c);
    const size_t need = align_up(t.w13) + align_up(t.w2) + align_up(t.sh13) + align_up(t.sh2);
    if ((st = check_ws(dst, dst_bytes, need)) != MOE_OK) return st;
    char* base = static_cast<char*>(dst);
    void* w13 = base;
    void* w2 = base + align_up(t.w13);
    void* sh13 = c.has_shared ? base + align_up(t.w13) + align_up(t.w2) : nullptr;
    void* sh2 = c.has_shared ? base + align_up(t.w13) + align_up(t.w2) + align_up(t.sh13) : nullptr;
    hipError_t e = moe::launch_tile_weights(c, *src, w13, w2, sh13, sh2, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "moe_tile_weights");
    moe_weights o{};
    o.w_gate = w13;
    o.w_down = w2;
    o.sh_gate = sh13;
    o.sh_down = sh2;
    o.layout = MOE_LAYOUT_TILED;
    if (c.w_dtype == MOE_FP8_E4M3) {  // the block scales are not rewritten: the caller's arrays
        o.s_gate = src->s_gate;
        o.s_up = src->s_up;
        o.s_down = src->s_down;
        o.sh_s_gate = src->sh_s_gate;
        o.sh_s_up = src->sh_s_up;
        o.sh_s_down = src->sh_s_down;
    }
    *tiled = o;
    return MOE_OK;
}

moe_status moe_combine(const moe_cfg* cfg, const void* y_rows, const int32_t* tok_row, const float* topk_w,
                       const void* y_shared, void* out, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    REQUIRE(y_rows, "y_rows");
    REQUIRE(tok_row, "tok_row");
    REQUIRE(topk_w, "topk_w");
    REQUIRE(out, "out");
    if (c.has_shared) REQUIRE(y_shared, "y_shared");
    REQUIRE_A16(y_rows, "y_rows");
    REQUIRE_A16(y_shared, "y_shared");
    REQUIRE_A16(out, "out");
    if (c.T == 0) return MOE_OK;
    hipError_t e = moe::launch_combine(c, y_rows, tok_row, topk_w, y_shared, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "moe_combine");
    return MOE_OK;
}

moe_status moe_quantize_fp8(const moe_cfg* cfg, const void* x, uint8_t* x_q, float* x_scale, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (c.act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_quantize_fp8 takes bf16 rows");
    if (c.H % 128) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_fp8 needs H a multiple of 128 (H=%d)", c.H);
    if (c.T == 0) return MOE_OK;
    REQUIRE(x, "x");
    REQUIRE(x_q, "x_q");
    REQUIRE(x_scale, "x_scale");
    REQUIRE_A16(x, "x");
    if (reinterpret_cast<uintptr_t>(x_q) % 8) return fail(MOE_ERR_INVALID_ARG, "x_q is not 8-byte aligned");
    if (reinterpret_cast<uintptr_t>(x_scale) % 4) return fail(MOE_ERR_INVALID_ARG, "x_scale is not 4-byte aligned");
    hipError_t e = moe::launch_quant_rows_e4m3(x, c.T, c.H, x_q, x_scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "moe_quantize_fp8");
    return MOE_OK;
}

moe_status moe_layer(const moe_cfg* cfg, const void* w_router, const float* bias, const moe_weights* w,
                     const void* x, void* out, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    const moe_cfg& c = *cfg;
    if (c.act_dtype == MOE_FP8_E4M3) return fail(MOE_ERR_UNSUPPORTED, "moe_layer on fp8 activations");
    REQUIRE(w_router, "w_router");
    if ((st = check_weights(c, w)) != MOE_OK) return st;
    REQUIRE(x, "x");
    REQUIRE(out, "out");
    REQUIRE_A16(x, "x");
    REQUIRE_A16(w_router, "w_router");
    REQUIRE_A16(out, "out");
    // the stage configuration the layer derives must be a valid one
    const moe_cfg derived = fp8_experts(c) ? fp8_routed_cfg(c) : layer_stage_cfg(c);
    if ((st = check_cfg(&derived)) != MOE_OK) return st;
    LayerCarve l = layer_carve(c, ws);
    if ((st = check_ws(ws, ws_bytes, l.bytes)) != MOE_OK) return st;
    if (c.T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // low-precision experts: the router also quantises x (moe_route_quantize)
    const bool f8 = fp8_experts(c);
    hipError_t e = moe::launch_router_logits(c, x, w_router, static_cast<float*>(l.scratch), s,
                                             f8 ? l.x_q : nullptr, f8 ? l.x_s : nullptr);
    if (e != hipSuccess) return hip_fail(e, "moe_layer (router)");
    e = moe::launch_route_select(c, static_cast<float*>(l.scratch), moe::router_splits(c), bias, nullptr, l.ids,
                                 l.topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer (select)");
    if (f8) return layer_fp8_experts(c, *w, out, l, s);
    const moe_cfg cs = layer_stage_cfg(c);
    st = permute_enqueue(cs, x, nullptr, l.ids, l.counts, l.offsets, l.row_src, l.tok_row, l.x_perm, nullptr,
                         l.scratch, s);
    if (st != MOE_OK) return st;
    const void* x_rows = cs.x_layout == MOE_LAYOUT_INDEXED ? x : l.x_perm;
    // bf16 y with a shared expert: the shared expert's tiles own rows of out,
    // so its GEMM2 can do the combine in its epilogue (no y_shared, no combine
    // pass; the same arithmetic as moe_combine)
    const bool fused = c.act_dtype == MOE_BF16 && c.has_shared && c.y_dtype == MOE_BF16 && c.T >= kFusedCombineMinT &&
                       fused_combine_requested();
    st = ffn_enqueue(cs, max_rows_of(cs), x_rows, nullptr, l.offsets, l.row_src, *w, wtab_of(c, *w, 0), x, l.y_rows,
                     l.y_shared, l.scratch, s, fused ? out : nullptr, l.tok_row, l.topk_w);
    if (st != MOE_OK) return st;
    if (fused) return MOE_OK;
    e = moe::launch_combine(c, l.y_rows, l.tok_row, l.topk_w, l.y_shared, out, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer (combine)");
    return MOE_OK;
}

const char* moe_status_string(moe_status status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
