"""GPU parity of the block-level selection variant (the previous generation's
whole-block picks, selected with select_block > 0) against the CPU oracle: the
fused decode step, the fused prefill chunk, and the standalone selection from
given scores."""
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


STEP = [
    # (name, workload kwargs, block size)
    ("ragged_4099_k1024_b128", dict(batch=1, n_q_heads=16, n_kv_heads=2, ctx_len=4099,
                                    n_sparse_layers=3, top_k=1024, window=128, n_needles=16,
                                    config_id=31), 128),
    ("ctx_3000_b2_k64_b16", dict(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=3000,
                                 n_sparse_layers=2, top_k=64, window=16, n_needles=6,
                                 config_id=32), 16),
    ("heavy_9000_k512_b64", dict(batch=1, n_q_heads=32, n_kv_heads=4, ctx_len=9000,
                                 n_sparse_layers=4, top_k=512, window=128, n_needles=12,
                                 heavy_frac=0.02, config_id=33), 64),
    ("drift_5000_k256_b256", dict(batch=2, n_q_heads=8, n_kv_heads=1, ctx_len=5000,
                                  n_sparse_layers=1, top_k=256, window=32, drift_sd=0.05,
                                  n_needles=4, config_id=34), 256),
    ("k_covers_context_b32", dict(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=600,
                                  n_sparse_layers=2, top_k=1024, window=64, config_id=35), 32),
    ("ctx_below_one_block", dict(batch=3, n_q_heads=8, n_kv_heads=1, ctx_len=40,
                                 n_sparse_layers=1, top_k=64, window=8, config_id=36), 64),
]


@pytest.mark.parametrize("path", [1, 2], ids=["subtile_path", "dense_path"])
@pytest.mark.parametrize("name,kw,bs", STEP, ids=[s[0] for s in STEP])
def test_block_step(hs2, name, kw, bs, path):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    gh.log(f"[block step] {name} S={w.ctx_len} k={w.top_k} block={bs} selection path {path}")
    res = gh.run_step(w, x, block=bs, decode_select=path)
    st = gh.compare_step(w, x, res, block=bs)
    gh.log(f"  {st}")


def test_block_identical_keys_take_lowest_blocks(hs2):
    w = wl.small(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=2000, n_sparse_layers=1, top_k=128,
                 window=16, config_id=37)
    x = wl.generate(w)
    x["k"][:] = x["k"][:, :, :1, :]
    res = gh.run_step(w, x, block=32)
    n = int(res["n_sel"][0, 0, 0])
    assert res["idx"][0, 0, 0, :n].tolist() == list(range(128)) + list(range(1984, 2000))


CHUNK = [
    # (name, workload kwargs, block size): prefill chunks, T > 1
    ("chunk_40_over_3000_b16", dict(batch=1, n_q_tokens=40, n_q_heads=16, n_kv_heads=2,
                                    ctx_len=3000, n_sparse_layers=2, top_k=64, window=16,
                                    n_needles=6, config_id=41), 16),
    ("chunk_64_over_2048_k1024_b128", dict(batch=1, n_q_tokens=64, n_q_heads=16, n_kv_heads=2,
                                           ctx_len=2048, n_sparse_layers=2, top_k=1024,
                                           window=128, n_needles=12, config_id=42), 128),
    ("chunk_100_over_5001_heavy_b64", dict(batch=1, n_q_tokens=100, n_q_heads=32, n_kv_heads=4,
                                           ctx_len=5001, n_sparse_layers=3, top_k=256,
                                           window=64, n_needles=20, heavy_frac=0.02,
                                           config_id=43), 64),
    ("chunk_17_drift_b256", dict(batch=2, n_q_tokens=17, n_q_heads=8, n_kv_heads=1, ctx_len=3001,
                                 n_sparse_layers=1, top_k=256, window=16, drift_sd=0.05,
                                 n_needles=5, config_id=44), 256),
    # the chunk is the whole context: the early rows keep every block, the
    # later ones choose, and most rows end in a partial block
    ("chunk_is_context_300_b32", dict(batch=2, n_q_tokens=300, n_q_heads=8, n_kv_heads=1,
                                      ctx_len=300, n_sparse_layers=1, top_k=64, window=8,
                                      config_id=45), 32),
]


@pytest.mark.parametrize("name,kw,bs", CHUNK, ids=[s[0] for s in CHUNK])
def test_block_prefill_chunk(hs2, name, kw, bs):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    gh.log(f"[block chunk] {name} T={w.n_q_tokens} S={w.ctx_len} k={w.top_k} block={bs}")
    res = gh.run_step(w, x, block=bs)
    st = gh.compare_step(w, x, res, block=bs)
    gh.log(f"  {st}")


@pytest.mark.parametrize("ctx,T,bs,k", [(2000, 8, 32, 128), (9000, 6, 16, 160),
                                        (20000, 4, 16, 160)],
                         ids=["band_by_one_wave", "band_by_threshold", "band_in_memory"])
def test_block_prefill_identical_keys(hs2, ctx, T, bs, k):
    # every key the same: every block ties, the lowest blocks win.  The band
    # holds every block: up to 64 are ranked by one wave, more by the key
    # threshold, and past 1024 blocks the band is kept in device memory.
    w = wl.small(name="ties", batch=1, n_q_tokens=T, n_q_heads=8, n_kv_heads=1, ctx_len=ctx,
                 n_sparse_layers=1, top_k=k, window=10, config_id=46)
    gh.log(f"[block chunk] identical keys S={ctx} T={T} block={bs}")
    x = wl.generate(w)
    x["k"][:] = x["k"][:, :, :1, :]
    res = gh.run_step(w, x, with_scores=False, block=bs)
    gh.compare_step(w, x, res, check_scores=False, block=bs, check_lse2=False)
    for t in range(w.n_q_tokens):
        first = w.ctx_len - w.n_q_tokens + t - w.window + 1
        row = res["idx"][0, t, 0, : res["n_sel"][0, t, 0]]
        assert row[:k].tolist() == list(range(k)), f"token {t}"
        assert row[k:].tolist() == list(range(first, first + w.window))


def test_block_prefill_4k_over_128k_sampled_rows(hs2):
    """The 4096-token chunk over a 128K context with blocks of 128, in the full
    step's launch configuration: every row's structure, and about 280 rows
    against the oracle."""
    w = wl.WORKLOADS["prefill_4k_over_128k"]
    x = wl.generate(w)
    gh.log("[block chunk] prefill_4k_over_128k block=128")
    res = gh.run_step(w, x, with_scores=False, block=128)
    # every row has more than top_k older keys: all its blocks are whole but
    # the last, which ends at the window and may be taken
    n = res["n_sel"]
    assert np.all(n <= w.top_k + w.window) and np.all(n > w.top_k + w.window - 128)
    ts = sorted(set(range(0, w.n_q_tokens, 64)) | {1, 63, 2047, 4094, 4095})
    rows = [(0, t, g) for t in ts for g in range(w.n_kv_heads)]
    gh.log(f"[block chunk] oracle on {len(rows)} rows")
    st = gh.compare_step(w, x, res, check_scores=False, rows=rows, block=128)
    gh.log(f"  {st}")


def test_block_select_from_given_scores(hs2):
    """Standalone block selection on float32 scores: bit-exact against the
    oracle run on the same values (block maxima compare exactly)."""
    rng = np.random.default_rng(8)
    for (B, T, Hkv, S, k, w, bs) in [(2, 1, 2, 3000, 128, 16, 16), (1, 3, 1, 700, 64, 8, 32),
                                     (1, 1, 4, 20000, 1024, 128, 128), (2, 2, 1, 300, 512, 10, 64),
                                     (1, 2, 2, 70000, 1024, 100, 256)]:
        s = hs2.ShapeArgs(batch=B, n_q_tokens=T, n_q_heads=8 * Hkv, n_kv_heads=Hkv, head_dim=128,
                          ctx_len=S, top_k=k, window=w, select_block=bs)
        sc = rng.random((B, T, Hkv, S)).astype(np.float32)
        sc[..., ::5] = sc[..., 3:4]          # many blocks share their maximum
        idx = torch.empty((B, T, Hkv, k + w), dtype=torch.int32, device="cuda")
        ns = torch.empty((B, T, Hkv), dtype=torch.int32, device="cuda")
        gh.log(f"[block scores] B={B} T={T} Hkv={Hkv} S={S} k={k} block={bs}")
        hs2.topk_select(s, torch.from_numpy(sc).cuda(), idx, ns)
        torch.cuda.synchronize()
        gi, gn = idx.cpu().numpy(), ns.cpu().numpy()
        for b in range(B):
            for t in range(T):
                pos = S - T + t
                for g in range(Hkv):
                    ref, _, _ = orc.select_blocks(sc[b, t, g, : pos + 1].astype(np.float64), pos,
                                                  k, w, bs)
                    n = int(gn[b, t, g])
                    assert n == ref.size
                    assert gi[b, t, g, :n].tolist() == ref.tolist()
                    assert np.all(gi[b, t, g, n:] == -1)


def test_block_step_full_size_1m(hs2):
    """Decode at 1M context with blocks of 128 (the block explainer page's
    choice): all 4 rows against the oracle."""
    w = wl.WORKLOADS["decode_1m_b1_heavy"]
    x = wl.generate(w)
    gh.log("[block step] decode_1m_b1_heavy block=128")
    res = gh.run_step(w, x, with_scores=False, block=128)
    st = gh.compare_step(w, x, res, check_scores=False, block=128)
    gh.log(f"  {st}")
