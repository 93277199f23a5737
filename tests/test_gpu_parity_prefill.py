"""GPU parity of the prefill-chunk path (T > 1 query tokens, causal full
attention, one selection per (token, KV head)) against the CPU oracle: small
chunks on every row, and the 4096-token chunk over a 128K context on sampled
rows in the launch configuration of the full step."""
import numpy as np
import pytest
import torch

import oracle.hs2_oracle as orc
from kv_reuse_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_reuse_amd import hs2 as mod
    return mod


SMALL = [
    ("chunk_40_over_300", dict(batch=1, n_q_tokens=40, n_q_heads=16, n_kv_heads=2, ctx_len=300,
                               n_sparse_layers=2, top_k=16, window=8, n_needles=6,
                               config_id=31)),
    ("chunk_is_context_33", dict(batch=2, n_q_tokens=33, n_q_heads=8, n_kv_heads=1, ctx_len=33,
                                 n_sparse_layers=1, top_k=8, window=4, config_id=32)),
    ("chunk_100_over_5000", dict(batch=1, n_q_tokens=100, n_q_heads=32, n_kv_heads=4,
                                 ctx_len=5000, n_sparse_layers=3, top_k=256, window=64,
                                 n_needles=20, heavy_frac=0.02, config_id=33)),
    ("chunk_64_over_2048_k1024", dict(batch=1, n_q_tokens=64, n_q_heads=16, n_kv_heads=2,
                                      ctx_len=2048, n_sparse_layers=2, top_k=1024, window=128,
                                      n_needles=12, config_id=34)),
    ("chunk_17_drift", dict(batch=2, n_q_tokens=17, n_q_heads=8, n_kv_heads=1, ctx_len=3001,
                            n_sparse_layers=1, top_k=64, window=16, drift_sd=0.05,
                            n_needles=5, config_id=35)),
    # rows of three and of five rounds of the selection's pass (16,384 older
    # keys a round): an odd count above one, whose last round runs beside one
    # past the row, and a ragged last round
    ("chunk_6_over_40000", dict(batch=1, n_q_tokens=6, n_q_heads=8, n_kv_heads=1, ctx_len=40000,
                                n_sparse_layers=1, top_k=512, window=64, n_needles=3,
                                config_id=61)),
    ("chunk_3_over_70000", dict(batch=1, n_q_tokens=3, n_q_heads=8, n_kv_heads=1, ctx_len=70000,
                                n_sparse_layers=1, top_k=2048, window=256, config_id=62)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_small(hs2, name, kw):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    gh.log(f"[prefill] {name} T={w.n_q_tokens} S={w.ctx_len} B={w.batch} Hkv={w.n_kv_heads}")
    res = gh.run_step(w, x)
    st = gh.compare_step(w, x, res)
    gh.log(f"  {st}")


@pytest.mark.parametrize("ctx,T", [(900, 24), (7000, 8), (9500, 6), (20000, 3)],
                         ids=["listed", "band_in_memory", "list_overflow_band_by_f16",
                              "two_rounds_list_overflow"])
def test_prefill_identical_keys(hs2, ctx, T):
    # every key the same: all importances of a row tie, the lowest indices win.
    # Past 2048 older keys the tied band leaves LDS for global memory; past 8192
    # it also overflows the selection's LDS list (a second read of the row) and
    # is ranked by its stored value.  At 20000 the pass takes two rounds, every
    # value of the second a candidate.
    w = wl.small(name="ties", batch=1, n_q_tokens=T, n_q_heads=8, n_kv_heads=1, ctx_len=ctx,
                 n_sparse_layers=1, top_k=50, window=10, config_id=36)
    gh.log(f"[prefill] identical keys S={ctx} T={T}")
    x = wl.generate(w)
    x["k"][:] = x["k"][:, :, :1, :]
    res = gh.run_step(w, x)
    gh.compare_step(w, x, res, check_lse2=False)
    for t in range(w.n_q_tokens):
        first = w.ctx_len - w.n_q_tokens + t - w.window + 1
        row = res["idx"][0, t, 0, : res["n_sel"][0, t, 0]]
        assert row[:50].tolist() == list(range(50)), f"token {t}"
        assert row[50:].tolist() == list(range(first, first + w.window))


def test_prefill_full_attn_scores_standalone(hs2):
    w = wl.small(name="scores", batch=1, n_q_tokens=20, n_q_heads=16, n_kv_heads=2, ctx_len=500,
                 n_sparse_layers=0, top_k=32, window=8, n_needles=3, config_id=37)
    x = wl.generate(w, with_sparse=False)
    s = hs2.shape_of(w)
    B, T, Hq, Hkv, D, S = w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_len
    q, k, v = gh.dev(x["q_full"]), gh.dev(x["k"]), gh.dev(x["v"])
    out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    sc = torch.empty((B, T, Hkv, S), dtype=torch.float32, device="cuda")
    ws = hs2.alloc_workspace(s, 0)
    hs2.full_attn_scores(s, q, k, v, out, lse=lse, scores=sc, ws=ws)
    torch.cuda.synchronize()
    ref = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale)
    o, l, scn = gh.host_f64(out), lse.cpu().numpy(), sc.cpu().numpy()
    G = w.group
    for (b, t, g), rr in ref.items():
        heads = slice(g * G, (g + 1) * G)
        gh.check_outputs(o[b, t, heads], rr["out_full"], f"out{(b, t, g)}")
        np.testing.assert_allclose(l[b, t, heads], rr["lse"], rtol=0, atol=2e-5)
        pos = rr["pos"]
        np.testing.assert_allclose(scn[b, t, g, : pos + 1], rr["score"],
                                   rtol=gh.SCORES_RTOL_PREFILL, atol=1e-30)
        assert np.all(scn[b, t, g, pos + 1:] == 0.0)


def test_prefill_4k_over_128k_sampled_rows(hs2):
    w = wl.WORKLOADS["prefill_4k_over_128k"]
    gh.log("[prefill] prefill_4k_over_128k: generating")
    x = wl.generate(w)
    gh.log("[prefill] prefill_4k_over_128k: GPU step")
    res = gh.run_step(w, x, with_scores=False)
    # every row: count, order, window and padding (structure only), and the
    # count the selection's pass listed
    gh.check_index_rows_all(res["idx"], res["n_sel"], w, refine=res["refine"])
    # against the oracle: every 16th query token (and the chunk's first and last
    # few) on all four KV heads, about 1,030 rows
    ts = sorted(set(range(0, w.n_q_tokens, 16)) | {1, 15, 2047, 4094, 4095})
    rows = [(0, t, g) for t in ts for g in range(w.n_kv_heads)]
    gh.log(f"[prefill] oracle on {len(rows)} rows")
    st = gh.compare_step(w, x, res, rows=rows)
    gh.log(f"  {st}")
    assert len(rows) >= 1024
