"""GPU check of moe_permute_noalloc, the allocation-free permute: through the
C ABI it must give, bit for bit, what moe_permute gives with a workspace, on
two calls in a row (the second with a smaller batch, so stale counts left in
the shared static scratch by the first would show)."""
import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
from tests._cases import dev

pytestmark = pytest.mark.gpu


def _case(T, E, k, H, seed, layout, m_tile):
    g = torch.Generator(device="cpu").manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32).to(dev())
    x = torch.randn((T, H), generator=g).to(torch.bfloat16).to(dev())
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=64, m_tile=m_tile, x_layout=layout)
    return c, ids, x


def _outputs(c, T, E, k, fill):
    rows = moe.moe_max_rows(c)
    i32 = dict(dtype=torch.int32, device=dev())
    o = dict(counts=torch.full((E,), fill, **i32), offs=torch.full((E + 1,), fill, **i32),
             row_src=torch.full((rows,), fill, **i32), tok_row=torch.full((T, k), fill, **i32),
             x_perm=moe.x_perm_buffer(c, dev()))
    o["x_perm"].fill_(0x5A)
    return o


@pytest.mark.parametrize("layout,m_tile", [(moe.MOE_LAYOUT_ROWMAJOR, 16), (moe.MOE_LAYOUT_TILED, 16),
                                           (moe.MOE_LAYOUT_INDEXED, 1)])
def test_permute_noalloc_equals_permute(layout, m_tile):
    E, k, H = 64, 6, 256
    for T, seed in ((3000, 1), (700, 2)):  # the second call is smaller
        c, ids, x = _case(T, E, k, H, seed, layout, m_tile)
        a = _outputs(c, T, E, k, -7)
        moe.moe_permute(c, x, None, ids, a["counts"], a["offs"], a["row_src"], a["tok_row"], a["x_perm"], None,
                        moe.workspace(c, moe.MOE_STAGE_PERMUTE, dev()))
        b = _outputs(c, T, E, k, -9)
        moe.moe_permute_noalloc(c, x, None, ids, b["counts"], b["offs"], b["row_src"], b["tok_row"], b["x_perm"],
                                None)
        torch.cuda.synchronize()
        for key in ("counts", "offs", "row_src", "tok_row"):
            assert torch.equal(a[key], b[key]), (T, key)
        if layout != moe.MOE_LAYOUT_INDEXED:
            assert torch.equal(a["x_perm"], b["x_perm"]), T
        # and both are the oracle's counting sort
        ref = oracle.dispatch(ids.cpu().numpy(), E, m_tile)
        assert np.array_equal(b["counts"].cpu().numpy(), ref["counts"])
        assert np.array_equal(b["tok_row"].cpu().numpy(), ref["tok_row"])
