"""The seeded input generator: determinism, bf16 rounding, planted structure."""
import numpy as np
import torch

from kv_reuse_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(10000).astype(np.float32) * 7,
                        np.array([1.0, -2.5, 3e-30, 1e30, 0.0, -0.0], dtype=np.float32)])
    # exact halfway cases: low 16 bits = 0x8000, both even and odd upper halves
    u = (np.arange(64, dtype=np.uint32) << 16) + 0x3F800000 + 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(wl.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(ref),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_determinism_and_seed_sensitivity():
    w = wl.small(batch=2, n_q_heads=8, n_kv_heads=2, ctx_len=300, n_sparse_layers=2, n_needles=3)
    a, b = wl.generate(w), wl.generate(w)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = wl.generate(w, seed=w.seed + 1)
    assert not np.array_equal(a["k"], c["k"])
    assert a["q_sparse"].shape == (2, 2, 1, 8, 128)
    assert a["k"].shape == (2, 2, 300, 128) and a["k"].dtype == np.uint16


def test_decode_needles_planted():
    w = wl.small(batch=2, n_q_heads=8, n_kv_heads=2, ctx_len=500, n_needles=7)
    x = wl.generate(w, with_sparse=False)
    q = wl.bf16_bits_to_f32(x["q_full"]).astype(np.float64)
    for b in range(2):
        for g in range(2):
            vec = wl.f32_to_bf16_bits((4.0 * q[b, 0, g * 4:(g + 1) * 4].mean(axis=0)).astype(np.float32))
            hits = np.all(x["k"][b, g] == vec[None, :], axis=1)
            assert hits.sum() == 7
            # the returned positions are exactly those rows
            pos = x["needles"][(x["needles"][:, 0] == b) & (x["needles"][:, 1] == g), 3]
            assert sorted(pos.tolist()) == np.flatnonzero(hits).tolist()


def test_needle_recall_diagnostic():
    """needle_recall counts the older-key needles kept by a selection: all of
    them for a list holding every older key, none for the window alone."""
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=300, n_needles=9, top_k=16,
                 window=8)
    x = wl.generate(w, with_sparse=False)
    older = x["needles"][x["needles"][:, 3] < 300 - 8 + 1]
    cap = 400
    every = np.full((1, 1, 1, cap), -1, dtype=np.int32)
    every[0, 0, 0, :300] = np.arange(300)
    r = wl.needle_recall(w, x["needles"], every, np.array([[[300]]]))
    assert r["needles"] == len(older) and r["found"] == len(older)
    window = np.full((1, 1, 1, cap), -1, dtype=np.int32)
    window[0, 0, 0, :8] = np.arange(292, 300)
    assert wl.needle_recall(w, x["needles"], window, np.array([[[8]]]))["found"] == 0


def test_prefill_needles_are_candidates_of_their_query():
    w = wl.small(batch=1, n_q_tokens=16, n_q_heads=8, n_kv_heads=2, ctx_len=400, window=8,
                 n_needles=5)
    x = wl.generate(w, with_sparse=False)
    q = wl.bf16_bits_to_f32(x["q_full"]).astype(np.float64)
    pos = w.positions()
    for g in range(2):
        found = 0
        for t in range(16):
            vec = wl.f32_to_bf16_bits((4.0 * q[0, t, g * 4:(g + 1) * 4].mean(axis=0)).astype(np.float32))
            hits = np.nonzero(np.all(x["k"][0, g] == vec[None, :], axis=1))[0]
            assert np.all(hits < pos[t] - w.window + 1)
            found += hits.size
        assert 1 <= found <= 5


def test_drift_and_heavy_tail():
    w = wl.small(ctx_len=4000, n_kv_heads=1, drift_sd=0.05)
    k = wl.bf16_bits_to_f32(wl.generate(w, with_sparse=False)["k"][0, 0]).astype(np.float64)
    # the drift makes neighbouring rows correlated; far rows much less
    near = np.mean(np.sum(k[1:] * k[:-1], axis=1))
    assert near > 0.5 * np.mean(np.sum(k * k, axis=1)) * 0.5
    w = wl.small(ctx_len=5000, n_kv_heads=1, heavy_frac=0.01)
    k = wl.bf16_bits_to_f32(wl.generate(w, with_sparse=False)["k"][0, 0]).astype(np.float64)
    norms = np.linalg.norm(k, axis=1)
    assert 40 <= np.sum(norms > 2 * np.sqrt(128)) <= 60      # 50 rows scaled by 3


def test_named_workloads_match_the_project_shapes():
    c = wl.WORKLOADS
    assert (c["decode_2k_b4"].batch, c["decode_2k_b4"].ctx_len, c["decode_2k_b4"].n_q_heads,
            c["decode_2k_b4"].n_kv_heads, c["decode_2k_b4"].n_sparse_layers) == (4, 2048, 16, 2, 3)
    assert c["decode_1m_b1_heavy"].ctx_len == 1 << 20 and c["decode_1m_b1_heavy"].n_sparse_layers == 8
    assert c["prefill_4k_over_128k"].n_q_tokens == 4096 and c["prefill_4k_over_128k"].ctx_len == 131072
    for w in c.values():
        assert (w.top_k, w.window, w.head_dim, w.group) == (1024, 128, 128, 8)
