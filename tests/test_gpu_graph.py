"""The path under HIP graph capture.

Every entry point only enqueues kernels (no allocation, no memset, no host synchronisation,
no other runtime call), so a whole step can be captured once and replayed.  Each test
captures a step (contiguous or paged caches) into a torch CUDA graph, replays it several
times with eager work and synchronisations between the replays, and checks every replay
bitwise against the eager step (the kernels are deterministic).  The top-k workspace of long rows must be left zero
by every call for the replays to stay correct; the second case exercises it.
"""
import pytest
import torch

import dsa_testlib as tl
import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


class Step:
    """Preallocated buffers and the three calls of one decode step."""

    def __init__(self, case, page=0):
        self.case = case
        self.layout = dsa.Layout.of_case(case)
        self.ik, self.ik_scale, self.kv = case.ik, case.ik_scale, case.layers[0].kv
        if page:  # paged caches: the same step through a block table
            self.layout, caches, _ = tl.paged(case, page, seed=1)
            self.ik, self.ik_scale, self.kv = caches["ik"], caches["ik_scale"], caches["kv"][0]
        c = case
        self.scores = torch.empty((c.T, c.max_ctx), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((c.T, c.topk), dtype=torch.int32, device=DEV)
        self.tk_ws = dsa.topk_workspace(self.layout, c.max_ctx, c.topk, DEV)
        self.ws = dsa.mla_workspace(self.layout, c.H, c.Dc, c.Dr, c.topk, 1, DEV)
        self.out = torch.empty((c.T, c.H, c.Dc), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((c.T, c.H), dtype=torch.float32, device=DEV)

    def run(self):
        c, L = self.case, self.case.layers[0]
        dsa.dsa_index_scores(self.layout, c.iq, c.iw, self.ik, k_scale=self.ik_scale, scores=self.scores)
        dsa.dsa_topk(self.layout, self.scores, c.topk, indices=self.idx, workspace=self.tk_ws)
        dsa.sparse_mla_decode(self.layout, L.q, self.kv, self.idx, c.sm_scale, c.Dc, L.kv_scale,
                              out=self.out, lse=self.lse, workspace=self.ws)

    def results(self):
        return self.idx.clone(), self.out.clone(), self.lse.clone()


@pytest.mark.parametrize("ctx,kv_dt,page", [([3000, 8192, 5000, 700], "bf16", 0), ([40000, 70000], "fp8", 0),
                                          ([3000, 8192, 5000, 700], "bf16", 16), ([40000, 70000], "fp8", 64)])
def test_decode_step_replays_equal_eager(ctx, kv_dt, page):
    case = synth.make_case("graph", 2, ctx=ctx, kv_dt=kv_dt, sm_scale=1.0 / 16, device=DEV)
    st = Step(case, page)
    st.run()
    torch.cuda.synchronize()
    ref = st.results()
    if st.tk_ws is not None:
        assert int(st.tk_ws.count_nonzero()) == 0  # left zero by the call

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm the binding on the capture stream
        st.run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()

    for rep in range(4):
        st.out.fill_(0)  # eager work between replays
        st.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = st.results()
        for a, b, what in zip(got, ref, ("indices", "out", "lse")):
            assert torch.equal(a, b), "replay %d: %s differs" % (rep, what)
        if st.tk_ws is not None:
            assert int(st.tk_ws.count_nonzero()) == 0


def test_writer_front_end_replays_equal_eager():
    T, H, rows = 600, 32, 700
    g0 = torch.Generator(device=DEV).manual_seed(3)
    q = torch.randn((T, H, 128), generator=g0, device=DEV).to(torch.bfloat16)
    k = torch.randn((T, 128), generator=g0, device=DEV).to(torch.bfloat16)
    pos = torch.arange(100, 100 + T, dtype=torch.int64, device=DEV)
    slots = torch.randperm(rows, device=DEV)[:T].to(torch.int64)
    tab = synth.rope_table(1024, device=DEV)
    cache = torch.zeros((rows, 128), dtype=torch.uint8, device=DEV)
    scale = torch.zeros(rows, dtype=torch.float32, device=DEV)
    q8 = torch.empty((T, H, 128), dtype=torch.uint8, device=DEV)
    qs = torch.empty((T, H), dtype=torch.float32, device=DEV)

    def run():
        dsa.dsa_index_front_end(q, k, slots, cache, scale, positions=pos, cos_sin=tab, q_fp8=q8, q_scale=qs)

    run()
    torch.cuda.synchronize()
    ref = (q8.clone(), qs.clone(), cache.clone(), scale.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in (q8, cache):
            t.fill_(0)
        qs.fill_(0)
        scale.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((q8, qs, cache, scale), ref):
            assert torch.equal(a, b), "replay %d differs" % rep
