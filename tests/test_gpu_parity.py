"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at sizes
the oracle finishes in seconds: several tiles and ragged tails, the 2K decode
workload, and the method's degenerate cases."""
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
    # (name, workload kwargs)
    ("ragged_300_b2", dict(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=300, n_sparse_layers=3,
                           top_k=16, window=8, n_needles=4, config_id=11)),
    ("ragged_1000_b1_g4", dict(batch=1, n_q_heads=32, n_kv_heads=4, ctx_len=1000,
                               n_sparse_layers=2, top_k=100, window=32, n_needles=8,
                               config_id=12)),
    ("ragged_4099_k1024", dict(batch=1, n_q_heads=16, n_kv_heads=2, ctx_len=4099,
                               n_sparse_layers=4, top_k=1024, window=128, n_needles=16,
                               config_id=13)),
    ("drift_3000", dict(batch=2, n_q_heads=8, n_kv_heads=1, ctx_len=3000, n_sparse_layers=1,
                        top_k=64, window=16, n_needles=6, drift_sd=0.05, config_id=14)),
    ("heavy_5000_l8", dict(batch=1, n_q_heads=16, n_kv_heads=2, ctx_len=5000, n_sparse_layers=8,
                           top_k=200, window=40, n_needles=10, heavy_frac=0.02, config_id=15)),
    ("tiny_ctx_40", dict(batch=3, n_q_heads=8, n_kv_heads=1, ctx_len=40, n_sparse_layers=2,
                         top_k=16, window=8, config_id=16)),
    ("ctx_1", dict(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=1, n_sparse_layers=1,
                   top_k=4, window=2, config_id=17)),
    ("ten_layers", dict(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=700, n_sparse_layers=10,
                        top_k=50, window=20, config_id=18)),
    # three rounds of the dense path's per-row pass (16,384 older keys a round)
    ("mid_35000", dict(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=35000, n_sparse_layers=1,
                       top_k=256, window=32, config_id=63)),
]


# the two decode selections: from the full layer's subtile bounds (1), and
# from every key's importance with the per-row ranking of a prefill chunk (2)
PATHS = [1, 2]


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_step_small(hs2, name, kw, path):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    gh.log(f"[step] {name} S={w.ctx_len} B={w.batch} Hkv={w.n_kv_heads} L={w.n_sparse_layers} "
           f"selection path {path}")
    res = gh.run_step(w, x, decode_select=path)
    st = gh.compare_step(w, x, res)
    gh.log(f"  {st}")


CAPACITY = [
    # a cache allocated for more tokens than the context: the spare rows hold
    # NaN and must never be read (decode, and a prefill chunk)
    ("decode_1000_spare_77", dict(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=1000,
                                  n_sparse_layers=2, top_k=64, window=16, n_needles=4,
                                  config_id=19), 1077),
    ("chunk_24_over_500_spare_500", dict(batch=1, n_q_tokens=24, n_q_heads=16, n_kv_heads=2,
                                         ctx_len=500, n_sparse_layers=2, top_k=32, window=8,
                                         n_needles=4, config_id=20), 1000),
]


@pytest.mark.parametrize("name,kw,cap", CAPACITY, ids=[s[0] for s in CAPACITY])
def test_step_cache_with_spare_capacity(hs2, name, kw, cap):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    gh.log(f"[step] {name} S={w.ctx_len} T={w.n_q_tokens} capacity={cap}")
    res = gh.run_step(w, x, kv_capacity=cap)
    st = gh.compare_step(w, x, res)
    gh.log(f"  {st}")


def test_step_decode_2k_workload(hs2):
    w = wl.WORKLOADS["decode_2k_b4"]
    x = wl.generate(w)
    gh.log("[step] decode_2k_b4")
    res = gh.run_step(w, x)
    gh.log(f"  {gh.compare_step(w, x, res)}")


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
def test_k_covers_context_sparse_equals_dense(hs2, path):
    """k >= |C|: every key is selected, so a sparse layer fed the full layer's
    queries must reproduce the full layer's output."""
    w = wl.small(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=900, n_sparse_layers=2, top_k=1024,
                 window=128, config_id=21)
    x = wl.generate(w)
    x["q_sparse"][0] = x["q_full"]
    res = gh.run_step(w, x, decode_select=path)
    gh.compare_step(w, x, res)
    assert np.all(res["n_sel"] == 900)
    err = np.abs(res["out_sparse"][0] - res["out_full"])
    assert err.max() <= 2e-2 and err.mean() <= 5e-3


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
def test_k_zero_is_sliding_window(hs2, path):
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=500, n_sparse_layers=2, top_k=0,
                 window=32, config_id=22)
    x = wl.generate(w)
    res = gh.run_step(w, x, decode_select=path)
    gh.compare_step(w, x, res)
    assert res["n_sel"][0, 0, 0] == 32
    assert res["idx"][0, 0, 0, :32].tolist() == list(range(468, 500))


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
def test_identical_keys_take_lowest_indices(hs2, path):
    """All keys equal: every importance ties, so the lowest indices win.  The
    tie spans more keys than fit in LDS, which exercises the exact radix path."""
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=6000, n_sparse_layers=1, top_k=100,
                 window=16, config_id=23)
    x = wl.generate(w)
    x["k"][:] = x["k"][:, :, :1, :]
    res = gh.run_step(w, x, decode_select=path)
    gh.compare_step(w, x, res, check_lse2=False)
    assert res["idx"][0, 0, 0, :116].tolist() == list(range(100)) + list(range(5984, 6000))


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
def test_small_band_ties_take_lowest_indices(hs2, path):
    """40 identical keys scoring far above the rest, top_k 16: the bin of the
    k-th key holds just those 40 ties (a band small enough for the one-wave
    rank), so the 16 lowest of their positions win."""
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=2000, n_sparse_layers=1, top_k=16,
                 window=16, config_id=25)
    x = wl.generate(w)
    qf = wl.bf16_bits_to_f32(x["q_full"])
    vec = wl.f32_to_bf16_bits((4.0 * qf[0, 0, :, :].mean(axis=0)).astype(np.float32))
    pos = np.sort(np.random.default_rng(2025).choice(1984, 40, replace=False))
    x["k"][0, 0, pos, :] = vec[None, :]
    res = gh.run_step(w, x, decode_select=path)
    gh.compare_step(w, x, res)
    assert res["idx"][0, 0, 0, :32].tolist() == pos[:16].tolist() + list(range(1984, 2000))


@pytest.mark.parametrize("path", PATHS, ids=["subtile_path", "dense_path"])
def test_large_band_distinct_keys(hs2, path):
    """200 keys near one needle vector (distinct, within about one bin of each
    other) far above the rest, top_k 100: the bin of the k-th key holds more
    than 64 distinct entries, so the radix threshold (not the one-wave rank)
    decides, over digits that really differ."""
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=6000, n_sparse_layers=1, top_k=100,
                 window=16, config_id=26)
    x = wl.generate(w)
    qf = wl.bf16_bits_to_f32(x["q_full"])
    rng = np.random.default_rng(2026)
    base = 4.0 * qf[0, 0, :, :].mean(axis=0)
    pos = np.sort(rng.choice(5984, 200, replace=False))
    noise = rng.standard_normal((200, 128)).astype(np.float32) * 0.003
    x["k"][0, 0, pos, :] = wl.f32_to_bf16_bits((base[None, :] + noise).astype(np.float32))
    res = gh.run_step(w, x, decode_select=path)
    gh.compare_step(w, x, res)


def test_deterministic_across_runs(hs2):
    """Ten runs of one plan: every output bit for bit the same."""
    w = wl.small(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=3333, n_sparse_layers=3,
                 top_k=256, window=64, n_needles=8, config_id=24)
    x = wl.generate(w)
    a = gh.run_step(w, x)
    for _ in range(9):
        b = gh.run_step(w, x)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])


def test_results_do_not_depend_on_the_split_plan(hs2):
    """Decode with the library's plan and three caller split counts (1, 7 and
    33 context splits per row): the index lists are bit-identical (the
    selection ranks float64 importances of exact products), every output is
    within the parity tolerance of the oracle, and each plan repeats bit for
    bit.  The outputs themselves differ in their last bits between plans: the
    splits' partial sums are added in a different order."""
    w = wl.small(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=5000, n_sparse_layers=3,
                 top_k=256, window=64, n_needles=8, config_id=27)
    x = wl.generate(w)
    runs = {}
    for n in (0, 1, 7, 33):
        gh.log(f"[plan] decode_splits={n}")
        a = gh.run_step(w, x, decode_splits=n)
        b = gh.run_step(w, x, decode_splits=n)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])
        gh.compare_step(w, x, a)
        runs[n] = a
    for n in (1, 7, 33):
        np.testing.assert_array_equal(runs[n]["idx"], runs[0]["idx"])
        np.testing.assert_array_equal(runs[n]["n_sel"], runs[0]["n_sel"])


def test_topk_select_from_given_scores(hs2):
    """Standalone selection on float32 scores: bit-exact against the oracle's
    selection run on the same float32 values (no tolerance band)."""
    rng = np.random.default_rng(5)
    for (B, T, Hkv, S, k, w) in [(2, 1, 2, 3000, 100, 16), (1, 3, 1, 700, 50, 8),
                                 (1, 1, 4, 20000, 1024, 128), (2, 2, 1, 300, 400, 10)]:
        s = hs2.ShapeArgs(batch=B, n_q_tokens=T, n_q_heads=8 * Hkv, n_kv_heads=Hkv, head_dim=128,
                          ctx_len=S, top_k=k, window=w)
        sc = rng.random((B, T, Hkv, S)).astype(np.float32)
        sc[..., ::7] = sc[..., 3:4]          # plenty of exact ties
        idx = torch.empty((B, T, Hkv, k + w), dtype=torch.int32, device="cuda")
        ns = torch.empty((B, T, Hkv), dtype=torch.int32, device="cuda")
        hs2.topk_select(s, torch.from_numpy(sc).cuda(), idx, ns)
        torch.cuda.synchronize()
        gi, gn = idx.cpu().numpy(), ns.cpu().numpy()
        for b in range(B):
            for t in range(T):
                pos = S - T + t
                for g in range(Hkv):
                    ref, _, _ = orc.select_tokens(sc[b, t, g, : pos + 1].astype(np.float64), pos, k, w)
                    n = int(gn[b, t, g])
                    assert n == ref.size
                    assert gi[b, t, g, :n].tolist() == ref.tolist()
                    assert np.all(gi[b, t, g, n:] == -1)


def test_sparse_attn_standalone(hs2):
    w = wl.small(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=2500, n_sparse_layers=5, top_k=300,
                 window=50, config_id=25)
    x = wl.generate(w)
    ref = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale, keep_scores=False)
    s = hs2.shape_of(w)
    idx = np.full((w.batch, 1, w.n_kv_heads, s.cap), -1, dtype=np.int32)
    ns = np.zeros((w.batch, 1, w.n_kv_heads), dtype=np.int32)
    for (b, t, g), rr in ref.items():
        idx[b, t, g, : rr["idx"].size] = rr["idx"]
        ns[b, t, g] = rr["idx"].size
    ns[1, 0, 1] = 0                     # a row with nothing selected gets zeros
    ns[1, 0, 0] = s.cap + 500           # a count past the list's capacity reads only the list
    out = torch.empty((5, w.batch, 1, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    hs2.sparse_attn(s, gh.dev(x["q_sparse"]), gh.dev(x["k"]), gh.dev(x["v"]),
                    torch.from_numpy(idx).cuda(), torch.from_numpy(ns).cuda(), out)
    torch.cuda.synchronize()
    got = gh.host_f64(out)
    want = orc.sparse_step(x["q_sparse"], x["k"], x["v"], idx, np.minimum(ns, s.cap),
                           scale=w.scale)
    gh.check_outputs(got, want, "sparse standalone")
    assert np.all(got[:, 1, 0, 8:16] == 0.0)


def test_sparse_attn_index_check(hs2):
    """Malformed index lists: every entry outside [0, P_t] among the n_sel read
    is counted per row in the workspace (HS2_WS_INDEX_CHECK), the read stays in
    the cache (an entry below 0 reads row 0, one at or past S reads row S-1,
    one in (P_t, S) reads that row), and the outputs equal the oracle's on the
    clamped list.  Three query tokens, so that P_t < S - 1 for two of them."""
    w = wl.small(batch=2, n_q_tokens=3, n_q_heads=16, n_kv_heads=2, ctx_len=2500,
                 n_sparse_layers=3, top_k=300, window=50, config_id=27)
    x = wl.generate(w)
    ref = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale, keep_scores=False)
    s = hs2.shape_of(w)
    S, T = w.ctx_len, w.n_q_tokens
    idx = np.full((w.batch, T, w.n_kv_heads, s.cap), -1, dtype=np.int32)
    ns = np.zeros((w.batch, T, w.n_kv_heads), dtype=np.int32)
    for (b, t, g), rr in ref.items():
        idx[b, t, g, : rr["idx"].size] = rr["idx"]
        ns[b, t, g] = rr["idx"].size
    idx[0, 0, 0, [3, 40, 299]] = [-1, S + 7, S - 1]      # below 0, past S, past P_0 = S - 3
    idx[0, 2, 1, 10] = -(1 << 30)
    idx[1, 1, 0, 200] = S - 1                             # past P_1 = S - 2
    idx[1, 1, 1, 100] = 2_000_000_000
    idx[1, 0, 0, s.cap - 20:] = -1      # as if padding, and a count past the capacity reads it
    ns[1, 0, 0] = s.cap + 500
    rd = np.minimum(ns, s.cap)
    P = S - T + np.arange(T)[None, :, None]
    col = np.arange(s.cap)[None, None, None, :]
    want_bad = ((col < rd[..., None]) & ((idx < 0) | (idx > P[..., None]))).sum(axis=3)
    assert want_bad[1, 0, 0] == 20 and want_bad[0, 0, 0] == 3 and want_bad[1, 1, 0] == 1
    L = w.n_sparse_layers
    out = torch.empty((L, w.batch, T, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws = hs2.alloc_workspace(s, L)
    hs2.sparse_attn(s, gh.dev(x["q_sparse"]), gh.dev(x["k"]), gh.dev(x["v"]),
                    torch.from_numpy(idx).cuda(), torch.from_numpy(ns).cuda(), out, ws=ws)
    torch.cuda.synchronize()
    bad = hs2.workspace_index_check(s, L, ws).cpu().numpy().reshape(w.batch, T, w.n_kv_heads)
    gh.log(f"[index check] counted {bad.ravel().tolist()}")
    assert bad.tolist() == want_bad.tolist()
    got = gh.host_f64(out)
    want = orc.sparse_step(x["q_sparse"], x["k"], x["v"], np.clip(idx, 0, S - 1), rd,
                           scale=w.scale)
    gh.check_outputs(got, want, "sparse on a malformed list (clamped)")


def test_full_attn_scores_standalone(hs2):
    w = wl.small(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=1777, n_sparse_layers=0, top_k=64,
                 window=16, n_needles=5, config_id=26)
    x = wl.generate(w, with_sparse=False)
    s = hs2.shape_of(w)
    out = torch.empty((2, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 1, 16), dtype=torch.float32, device="cuda")
    sc = torch.empty((2, 1, 2, 1777), dtype=torch.float32, device="cuda")
    hs2.full_attn_scores(s, gh.dev(x["q_full"]), gh.dev(x["k"]), gh.dev(x["v"]), out, lse, sc)
    torch.cuda.synchronize()
    ref = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=64, window=16,
                                 scale=w.scale)
    for (b, t, g), rr in ref.items():
        gh.check_outputs(gh.host_f64(out)[b, t, 8 * g:8 * g + 8], rr["out_full"], "out")
        np.testing.assert_allclose(lse.cpu().numpy()[b, t, 8 * g:8 * g + 8], rr["lse"], atol=2e-5)
        np.testing.assert_allclose(sc.cpu().numpy()[b, t, g].astype(np.float64), rr["score"],
                                   rtol=gh.SCORES_RTOL_DECODE, atol=1e-30)
