"""The Cross-Decoder step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library enqueues kernels only (no allocation, no memset, no
synchronisation), so a captured step must give the eager step's results on every
replay.  Each replay is followed by unrelated eager work and a synchronisation,
and every replay is compared with the eager result (bit for bit: the step is
deterministic)."""
import numpy as np
import pytest
import torch

from kv_reuse_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_reuse_amd import hs2 as mod
    return mod


CASES = [
    ("decode_2k_b4", None),
    ("chunk_32_over_700", dict(batch=1, n_q_tokens=32, n_q_heads=16, n_kv_heads=2, ctx_len=700,
                               n_sparse_layers=2, top_k=64, window=16, n_needles=4,
                               config_id=51)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(hs2, name, kw):
    w = wl.WORKLOADS[name] if kw is None else wl.small(name=name, **kw)
    x = wl.generate(w)
    s = hs2.shape_of(w)
    B, T, Hq, Hkv, D, L = w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, \
        w.n_sparse_layers
    q, k, v, qs = gh.dev(x["q_full"]), gh.dev(x["k"]), gh.dev(x["v"]), gh.dev(x["q_sparse"])
    out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((L, B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, T, Hkv, s.cap), dtype=torch.int32, device="cuda")
    nsel = torch.empty((B, T, Hkv), dtype=torch.int32, device="cuda")
    ws = hs2.alloc_workspace(s, L)

    def step():
        hs2.cross_decoder_step(s, q, qs, k, v, out, outs, idx, nsel, ws=ws)

    gh.log(f"[graph] {name}: eager")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, outs, idx, nsel)]
    # capture on a side stream (torch's graph capture), after a warm-up there
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    gh.log(f"[graph] {name}: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        for t in (out, outs, idx, nsel):
            t.zero_()
        torch.cuda.synchronize()
        gh.log(f"[graph] {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, outs, idx, nsel), ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        scratch.normal_()                      # unrelated eager work between replays
        _ = float(scratch.sum())
    # and the graph's results are the oracle's
    res = {"out_full": gh.host_f64(out), "idx": idx.cpu().numpy(), "n_sel": nsel.cpu().numpy(),
           "out_sparse": gh.host_f64(outs)}
    gh.compare_step(w, x, res, check_scores=False)
