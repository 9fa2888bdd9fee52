"""The allocation-free sparse-MLA entry point on the GPU (through the C ABI).

sparse_mla_decode_no_alloc keeps the split partials in the library's static device scratch
instead of a caller workspace; it runs the same kernels, so its outputs and lse must equal
sparse_mla_decode's bit for bit.  Two calls in a row, the second with a smaller input, check
that nothing left in the scratch by the first call leaks into the second.
"""
import numpy as np
import pytest
import torch

import dsa_testlib as tl
import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("kv_dt", ["fp8", "bf16"])
def test_no_alloc_entry_equals_workspace_entry(kv_dt):
    big = synth.make_case("no_alloc_big", 2, ctx=[9000, 3000, 4096, 2500, 7000, 2048, 3333, 5000],
                          kv_dt=kv_dt, sm_scale=1.0 / 16, device=DEV)
    small = synth.make_case("no_alloc_small", 2, ctx=[2100, 700, 5000], kv_dt=kv_dt, sm_scale=1.0 / 16,
                            device=DEV, seed=1)
    for case in (big, small):  # the second call is smaller: a different split geometry
        lay = dsa.Layout.of_case(case)
        scores = dsa.dsa_index_scores(lay, case.iq, case.iw, case.ik, k_scale=case.ik_scale)
        idx = dsa.dsa_topk(lay, scores, case.topk)
        L = case.layers[0]
        assert dsa.sparse_mla_workspace_size(lay, case.H, case.Dc, case.Dr, case.topk, 1) > 0  # key splits
        lse_ws = torch.empty((case.T, case.H), dtype=torch.float32, device=DEV)
        o_ws = dsa.sparse_mla_decode(lay, L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale, lse=lse_ws)
        o_na = torch.full_like(o_ws, 7.0)
        lse_na = torch.full_like(lse_ws, 7.0)
        dsa.sparse_mla_decode_no_alloc(lay, L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale, out=o_na,
                                       lse=lse_na)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), "%s: outputs differ from the workspace entry" % case.name
        assert torch.equal(lse_na, lse_ws), "%s: lse differs from the workspace entry" % case.name
        rows = [0, case.T - 1]
        o_or, _ = tl.oracle_mla_rows(case, rows, idx.cpu().numpy())
        g = tl.to_f64(o_na)
        for r, oo in zip(rows, o_or):
            tl.check_attention(g[r], oo, tl.ATTN_ATOL_LOWP, "%s row %d" % (case.name, r))
