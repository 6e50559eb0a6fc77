"""GPU parity of the router and the dispatch against the oracle.

Routing ids, counts, offsets and both row maps must match bit for bit;
routing weights within 1e-5 * routed_scale.  Inputs are seeded, drawn with the
workloads' shapes and distributions, and keep a decision margin of 1e-4 so
that fp32 accumulation order cannot flip a choice."""
import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._cases import dev, lib_cfg, route_kw, router_case
from tests._np import to_np

pytestmark = pytest.mark.gpu


def _route(c, x, w_r, bias, logits_in=None):
    T, E, k = c.T, c.E, c.k
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev())
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev())
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev())
    ws = None if logits_in is not None else moe.workspace(c, moe.MOE_STAGE_ROUTE, dev())
    moe.moe_route(c, x, w_r, bias, logits_in, lg, ids, w, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("name,T", [
    ("c1_tiny_fp32", None),
    ("c2_mixtral_bf16", 1000),
    ("c3_dsv3_bf16", 1000),
    ("c4_qwen3_skew_bf16", 1000),
    ("c3_dsv3_bf16", None),          # full size, T = 8192
    ("c4_qwen3_skew_bf16", None),    # full size, T = 16384
])
def test_route_matches_oracle(name, T):
    s = synth.config(name)
    rc = router_case(s, T)
    T = rc["x"].shape[0]
    c = lib_cfg(s, T=T)
    ids, w, lg = _route(c, rc["x"], rc["w_r"], rc["bias"])
    ref_ids, ref_w = oracle.route_select(rc["logits"], s.k, renormalize=s.renormalize,
                                         routed_scale=s.routed_scale, bias=rc["bh"], **route_kw(s))
    # logits: fp32 accumulation vs fp64 then rounded
    scale = np.sqrt(np.mean(rc["logits"].astype(np.float64) ** 2))
    assert np.max(np.abs(lg - rc["logits"])) <= 2e-5 * scale
    assert np.array_equal(ids, ref_ids)
    assert np.max(np.abs(w - ref_w)) <= 1e-5 * s.routed_scale
    # the same fp32 logits on both sides
    ids2, w2, lg2 = _route(c, None, None, rc["bias"], torch.from_numpy(rc["logits"]).to(dev()))
    assert np.array_equal(lg2, rc["logits"])
    assert np.array_equal(ids2, ref_ids)
    assert np.max(np.abs(w2 - ref_w)) <= 1e-5 * s.routed_scale


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
def test_route_ties_and_group_limit_edge_cases(score):
    rng = np.random.default_rng(20)
    T, E, k = 37, 24, 5
    cases = [
        np.zeros((T, E), np.float32),                                   # all tied
        (rng.integers(-2, 3, (T, E)) * 0.5).astype(np.float32),          # many exact ties
        rng.normal(0, 1, (T, E)).astype(np.float32),
    ]
    for G, KG, gsc in [(1, 1, 0), (4, 2, 0), (6, 3, 1), (24, 5, 0), (3, 3, 0)]:
        for renorm in (True, False):
            for lg in cases:
                c = moe.make_cfg(T=T, H=64, E=E, k=k, I=64, n_groups=G, topk_groups=KG, score_fn=score,
                                 group_score=gsc, renormalize=renorm, routed_scale=1.5)
                bias = rng.normal(0, 0.1, E).astype(np.float32) if G == 4 else None
                bt = None if bias is None else torch.from_numpy(bias).to(dev())
                ids, w, _ = _route(c, None, None, bt, torch.from_numpy(lg).to(dev()))
                rid, rw = oracle.route_select(lg, k, score, G, KG, gsc, renorm, 1.5, bias)
                assert np.array_equal(ids, rid), (G, KG, gsc, renorm)
                assert np.max(np.abs(w - rw)) <= 1.5e-5


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
def test_route_groups_of_32_ties_and_limits(score):
    """Groups of 32 experts with E = 64, 128, 256 (the kernel's half-wave
    group path, DeepSeek-V3's 8 groups at E = 256): exact ties between keys
    and between group scores, every topk_groups, both group scores."""
    rng = np.random.default_rng(23)
    T = 41
    for E in (64, 128, 256):
        G = E // 32
        cases = [
            np.zeros((T, E), np.float32),
            (rng.integers(-2, 3, (T, E)) * 0.5).astype(np.float32),
            rng.normal(0, 1, (T, E)).astype(np.float32),
        ]
        for KG in sorted({1, max(1, G // 2), G}):
            k = min(8, 32 * KG)
            for gsc in (0, 1):
                for lg in cases:
                    c = moe.make_cfg(T=T, H=64, E=E, k=k, I=64, n_groups=G, topk_groups=KG, score_fn=score,
                                     group_score=gsc, renormalize=True, routed_scale=2.5)
                    ids, w, _ = _route(c, None, None, None, torch.from_numpy(lg).to(dev()))
                    rid, rw = oracle.route_select(lg, k, score, G, KG, gsc, True, 2.5, None)
                    assert np.array_equal(ids, rid), (E, KG, gsc)
                    assert np.max(np.abs(w - rw)) <= 2.5e-5


def test_route_k_equals_e_and_single_expert():
    rng = np.random.default_rng(21)
    for E, k in [(1, 1), (8, 8), (32, 32), (64, 32), (65, 3), (1024, 8)]:
        T = 19
        lg = rng.normal(0, 1, (T, E)).astype(np.float32)
        c = moe.make_cfg(T=T, H=64, E=E, k=k, I=64)
        ids, w, _ = _route(c, None, None, None, torch.from_numpy(lg).to(dev()))
        rid, rw = oracle.route_select(lg, k)
        assert np.array_equal(ids, rid), (E, k)
        assert np.max(np.abs(w - rw)) <= 1e-5


# ------------------------------------------------------------------ permute

def _ids(rng, T, E, k, hot=None):
    if hot is not None:  # expert `hot` is in every token's choice
        rest = np.stack([rng.permutation([e for e in range(E) if e != hot])[:k - 1] for _ in range(T)])
        return np.concatenate([np.full((T, 1), hot), rest], 1).astype(np.int32) if k > 1 else \
            np.full((T, 1), hot, np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k,H,m_tile,dtype,hot", [
    (1000, 256, 8, 256, 1, "bf16", None),
    (1000, 256, 8, 7168, 16, "bf16", None),
    (333, 8, 2, 512, 1, "f32", None),
    (4099, 128, 8, 128, 64, "bf16", 3),
    (1, 1, 1, 64, 1, "bf16", None),
    (257, 4, 4, 64, 128, "bf16", None),
    (600, 1024, 8, 64, 1, "bf16", None),
    (513, 8, 1, 256, 1, "fp8", None),
    (300, 16, 3, 384, 32, "fp8", 5),
])
def test_permute_matches_oracle(T, E, k, H, m_tile, dtype, hot):
    rng = np.random.default_rng(T * 7 + E)
    ids = _ids(rng, T, E, k, hot)
    dt = {"bf16": moe.MOE_BF16, "f32": moe.MOE_F32, "fp8": moe.MOE_FP8_E4M3}[dtype]
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=128, act_dtype=dt, m_tile=m_tile,
                     y_dtype=moe.MOE_BF16 if dtype == "fp8" else moe.MOE_F32)
    rows = moe.moe_max_rows(c)
    d = dev()
    if dtype == "fp8":
        x = torch.from_numpy(rng.integers(0, 256, (T, H), dtype=np.uint8)).to(d)
        x[x == 0x7F] = 0
        xs = torch.from_numpy(rng.random((T, H // 128), dtype=np.float32)).to(d)
    else:
        x = torch.randn(T, H, device=d, generator=torch.Generator(d).manual_seed(T)).to(
            torch.bfloat16 if dtype == "bf16" else torch.float32)
        xs = None
    ids_t = torch.from_numpy(ids).to(d)
    counts = torch.full((E,), -1, dtype=torch.int32, device=d)
    offs = torch.full((E + 1,), -1, dtype=torch.int32, device=d)
    row_src = torch.full((rows,), -5, dtype=torch.int32, device=d)
    tok_row = torch.full((T, k), -5, dtype=torch.int32, device=d)
    x_perm = torch.full((rows, H), 77, dtype=torch.uint8, device=d).view(x.dtype) if dtype == "fp8" else \
        torch.full((rows, H), 7.0, dtype=x.dtype, device=d)
    xps = torch.full((rows, H // 128), 7.0, dtype=torch.float32, device=d) if dtype == "fp8" else None
    ws = moe.workspace(c, moe.MOE_STAGE_PERMUTE, d)
    moe.moe_permute(c, x, xs, ids_t, counts, offs, row_src, tok_row, x_perm, xps, ws)
    torch.cuda.synchronize()
    ref = oracle.dispatch(ids, E, m_tile, rows)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offs.cpu().numpy(), ref["padded_offsets"])
    assert np.array_equal(row_src.cpu().numpy(), ref["row_src"])
    assert np.array_equal(tok_row.cpu().numpy(), ref["tok_row"])
    rs = ref["row_src"]
    xh, xph = to_np(x), to_np(x_perm)
    valid = rs >= 0
    assert np.array_equal(xph[valid], xh[rs[valid] // k])
    assert np.all(xph[~valid] == 0)
    if dtype == "fp8":
        xsh, xpsh = xs.cpu().numpy(), xps.cpu().numpy()
        assert np.array_equal(xpsh[valid], xsh[rs[valid] // k])
        assert np.all(xpsh[~valid] == 0)


def test_permute_is_deterministic_across_runs_and_streams():
    rng = np.random.default_rng(5)
    T, E, k, H = 2048, 64, 6, 512
    ids = torch.from_numpy(_ids(rng, T, E, k)).to(dev())
    x = torch.randn(T, H, device=dev()).to(torch.bfloat16)
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=128)
    rows = moe.moe_max_rows(c)
    outs = []
    for rep in range(3):
        st = torch.cuda.Stream() if rep == 2 else torch.cuda.current_stream()
        with torch.cuda.stream(st):
            o = [torch.empty(E, dtype=torch.int32, device=dev()), torch.empty(E + 1, dtype=torch.int32, device=dev()),
                 torch.empty(rows, dtype=torch.int32, device=dev()), torch.empty(T, k, dtype=torch.int32, device=dev()),
                 torch.empty(rows, H, dtype=torch.bfloat16, device=dev())]
            ws = moe.workspace(c, moe.MOE_STAGE_PERMUTE, dev())
            moe.moe_permute(c, x, None, ids, o[0], o[1], o[2], o[3], o[4], None, ws, stream=st)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in o])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
