"""GPU parity of pointer-table weights (the layer-oblivious grouped GEMM): the
expert matrices of several layers reached through a device array of
per-(layer, expert) pointers, the layer chosen by a device int32 read when the
kernels run.

The table only changes where a tile's weight rows are read from, so a call
through it must equal, bit for bit, the call on that layer's contiguous
weights; those contiguous calls are checked against the oracle in the other
GPU tests, and one scattered layer (each expert in its own allocation, as
weights prefetched into separate buffers are) is checked against the oracle
here too, to the bf16 bound (max|err| / rms(ref) <= 1e-2).  A graph captured
once with the table replays for any layer set between replays."""
import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._cases import dev, lib_cfg, rel_err, router_case
from tests._np import f64, to_np

pytestmark = pytest.mark.gpu

N_LAYERS = 3


def _bf16_layers(E, H, I, I_sh, d):
    """N_LAYERS sets of bf16 weights (seeded per layer): (wg, wu, wd, shg, shu, shd)."""
    out = []
    for L in range(N_LAYERS):
        s = synth.MoeShape("tab", T=1, H=H, E=E, k=1, I=I, dtype="bf16", seed=100 + L)
        wg = torch.empty((E, I, H), dtype=torch.bfloat16, device=d)
        wu, wd = torch.empty_like(wg), torch.empty((E, H, I), dtype=torch.bfloat16, device=d)
        for e in range(E):
            wg[e], wu[e], wd[e] = synth.expert_weights(s, e, d)
        ss = synth.MoeShape("tabsh", T=1, H=H, E=1, k=1, I=I_sh, dtype="bf16", seed=200 + L)
        out.append((wg, wu, wd) + tuple(synth.expert_weights(ss, 0, d)))
    return out


def _scattered(c, layer, d):
    """One layer with every expert matrix copied into its own allocation; the
    table row (E + 1 entries of 6 pointers) and the tensors that own them."""
    keep, row = [], []
    wg, wu, wd, shg, shu, shd = layer
    for e in range(c.E):
        mats = [wg[e].clone(), wu[e].clone(), wd[e].clone()]
        keep += mats
        row += [t.data_ptr() for t in mats] + [0, 0, 0]
    mats = [shg.clone(), shu.clone(), shd.clone()]
    keep += mats
    row += [t.data_ptr() for t in mats] + [0, 0, 0]
    return row, keep


def _ffn_case(H, I, counts, shared_T, I_sh, d):
    E = len(counts)
    n = int(sum(counts))
    x_rows = synth.normal(synth.stream_key(31, "rows"), (max(n, 1), H), 1.0, d, torch.bfloat16)
    x_tok = synth.normal(synth.stream_key(31, "tok"), (shared_T, H), 1.0, d, torch.bfloat16)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=d)
    c = moe.make_cfg(T=shared_T, H=H, E=E, k=1, I=I, has_shared=True, I_shared=I_sh, y_dtype=moe.MOE_F32)
    return c, n, x_rows, x_tok, offs


@pytest.mark.parametrize("tiled", [False, True])
def test_table_ffn_equals_contiguous_per_layer(tiled):
    d = dev()
    H, I, I_sh, counts, shared_T = 512, 384, 256, [37, 0, 5, 300, 64, 1], 70
    c, n, x_rows, x_tok, offs = _ffn_case(H, I, counts, shared_T, I_sh, d)
    layers = _bf16_layers(c.E, H, I, I_sh, d)
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=n)
    cont, keep = [], []
    for L in layers:
        w = moe.weights(L[0], L[1], L[2], sh_gate=L[3], sh_up=L[4], sh_down=L[5])
        if tiled:
            w, buf = moe.tile_weights(c, w, d)
            keep.append(buf)
        cont.append(w)

    def run(w):
        y = torch.full((n, H), -12345.0, device=d)
        y_sh = torch.full((shared_T, H), -12345.0, device=d)
        moe.moe_grouped_ffn(c, n, x_rows, None, offs, w, x_tok, y, y_sh, ws)
        torch.cuda.synchronize()
        return y, y_sh

    ref = [run(w) for w in cont]
    # layer 1 scattered (row-major only: a tiled copy keeps its own allocation)
    entries = moe.moe_weight_table(c, cont)
    G = c.E + 1
    if not tiled:
        row, sc = _scattered(c, layers[1], d)
        keep += sc
        entries[G * 6:2 * G * 6] = row
    table = torch.tensor(entries, dtype=torch.int64, device=d)
    lay = torch.zeros(1, dtype=torch.int32, device=d)
    wt = moe.weights(None, None, None, layout=moe.MOE_LAYOUT_TILED if tiled else moe.MOE_LAYOUT_ROWMAJOR,
                     table=table, layer=lay, n_layers=N_LAYERS)
    for L in (2, 0, 1, 2, 1):
        lay.fill_(L)
        y, y_sh = run(wt)
        assert torch.equal(y, ref[L][0]), L
        assert torch.equal(y_sh, ref[L][1]), L
    # the scattered layer against the oracle (bf16 h, as the layer stores it)
    wg, wu, wd, shg, shu, shd = layers[1]
    y, y_sh = ref[1]
    xh, yh = to_np(x_rows), f64(y)
    oc = np.concatenate([[0], np.cumsum(counts)])
    for e in range(c.E):
        if counts[e]:
            sl = slice(oc[e], oc[e + 1])
            r = oracle.expert_ffn(xh[sl], to_np(wg[e]), to_np(wu[e]), to_np(wd[e]), h_bf16=True)
            assert rel_err(yh[sl], r) <= 1e-2, e
    r = oracle.expert_ffn(to_np(x_tok), to_np(shg), to_np(shu), to_np(shd), h_bf16=True)
    assert rel_err(f64(y_sh), r) <= 1e-2
    # a layer id outside [0, n_layers): the kernels do nothing
    for bad in (N_LAYERS, -1):
        lay.fill_(bad)
        y, y_sh = run(wt)
        assert bool((y == -12345.0).all()) and bool((y_sh == -12345.0).all())


@pytest.mark.parametrize("mxfp4", [False, True])
def test_table_fp8_ffn_equals_contiguous_per_layer(mxfp4):
    """e4m3 rows with e4m3 weights (fp32 128 x 128 block scales) or MXFP4
    weights (E8M0 scales per 32): the table carries each expert's codes and
    scales."""
    d = dev()
    H, I, counts = 256, 384, [130, 0, 7, 290]
    E, n = len(counts), int(sum(counts))
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=d)
    c = moe.make_cfg(T=n, H=H, E=E, k=1, I=I, act_dtype=moe.MOE_FP8_E4M3, y_dtype=moe.MOE_BF16,
                     w_dtype=moe.MOE_FP4_E2M1 if mxfp4 else moe.MOE_FP8_E4M3)
    s = synth.MoeShape("tab8", T=n, H=H, E=E, k=1, I=I, dtype="fp8", seed=5)
    xq, xs = synth.fp8_rows(s, n, d)
    gen = synth.mxfp4_expert_weights if mxfp4 else synth.fp8_expert_weights
    cont, keep = [], []
    for L in range(N_LAYERS):
        sl = s.with_(seed=300 + L)
        wq = [gen(sl, e, d) for e in range(E)]
        wg, sg, wu, su, wd, sd = (torch.stack([w[i] for w in wq]) for i in range(6))
        keep.append((wg, sg, wu, su, wd, sd))
        cont.append(moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd))
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=n)

    def run(w):
        y = torch.full((n, H), -1.0, dtype=torch.bfloat16, device=d)
        moe.moe_grouped_ffn(c, n, xq, xs, offs, w, None, y, None, ws)
        torch.cuda.synchronize()
        return y

    ref = [run(w) for w in cont]
    entries = moe.moe_weight_table(c, cont)
    # the table holds each expert's own codes and block scales
    wg, sg = keep[2][0], keep[2][1]
    assert entries[(2 * E + 3) * 6 + 0] == wg[3].data_ptr()
    assert entries[(2 * E + 3) * 6 + 3] == sg[3].data_ptr()
    table = torch.tensor(entries, dtype=torch.int64, device=d)
    lay = torch.zeros(1, dtype=torch.int32, device=d)
    wt = moe.weights(None, None, None, table=table, layer=lay, n_layers=N_LAYERS)
    for L in (1, 2, 0, 1):
        lay.fill_(L)
        assert torch.equal(run(wt).view(torch.int16), ref[L].view(torch.int16)), L


def _layer_setup(fp8):
    d = dev()
    s = synth.config("c3_dsv3_bf16").with_(H=512, I=256, E=16, k=4, n_groups=4, topk_groups=2, I_shared=384)
    T = 77
    rc = router_case(s, T)
    c = lib_cfg(s, T=T, y_dtype=moe.MOE_F32, out_dtype=moe.MOE_F32)
    if fp8:
        c.w_dtype = moe.MOE_FP8_E4M3
    cont, keep = [], []
    for L in range(N_LAYERS):
        sl = s.with_(seed=400 + L)
        if fp8:
            wq = [synth.fp8_expert_weights(sl, e, d) for e in range(s.E)]
            wg, sg, wu, su, wd, sd = (torch.stack([w[i] for w in wq]) for i in range(6))
            sh = synth.fp8_expert_weights(sl.with_(I=s.I_shared), s.E, d)
            keep.append((wg, sg, wu, su, wd, sd) + tuple(sh))
            cont.append(moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd, sh_gate=sh[0], sh_up=sh[2],
                                    sh_down=sh[4], sh_s_gate=sh[1], sh_s_up=sh[3], sh_s_down=sh[5]))
        else:
            wg = torch.empty((s.E, s.I, s.H), dtype=torch.bfloat16, device=d)
            wu, wd = torch.empty_like(wg), torch.empty((s.E, s.H, s.I), dtype=torch.bfloat16, device=d)
            for e in range(s.E):
                wg[e], wu[e], wd[e] = synth.expert_weights(sl, e, d)
            sh = tuple(synth.shared_weights(sl, d))
            keep.append((wg, wu, wd) + sh)
            cont.append(moe.weights(wg, wu, wd, sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2]))
    return d, s, T, rc, c, cont, keep


@pytest.mark.parametrize("fp8", [False, True])
def test_layer_graph_with_table_replays_any_layer(fp8):
    """moe_layer through the table, captured once into a graph: each replay,
    with the layer id set by an eager fill kernel before it and a
    synchronisation after it, equals the eager layer on that layer's
    contiguous weights, bit for bit."""
    d, s, T, rc, c, cont, keep = _layer_setup(fp8)
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, d)

    def eager(w):
        out = torch.full((T, s.H), float("nan"), device=d)
        moe.moe_layer(c, rc["w_r"], rc["bias"], w, rc["x"], out, ws)
        torch.cuda.synchronize()
        return out

    ref = [eager(w) for w in cont]
    table = moe.weight_table(c, cont, d)
    lay = torch.zeros(1, dtype=torch.int32, device=d)
    wt = moe.weights(None, None, None, table=table, layer=lay, n_layers=N_LAYERS)
    assert torch.equal(eager(wt), ref[0])
    out = torch.full((T, s.H), float("nan"), device=d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer(c, rc["w_r"], rc["bias"], wt, rc["x"], out, ws)
    torch.cuda.synchronize()
    for L in (2, 0, 1, 1, 2, 0):
        lay.fill_(L)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[L]), L
        # eager work between replays
        assert torch.equal(eager(cont[(L + 1) % N_LAYERS]), ref[(L + 1) % N_LAYERS])
    del g
