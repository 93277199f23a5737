"""GPU parity of the separate sliding-window branch variant of the sparse layers
(hs2_sparse_attn_swa: the previous generation's sparse layer, with the layer's
own local window cache) against the CPU oracle, on the oracle's own index lists."""
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


CASES = [
    # (name, workload kwargs)
    ("decode_3000_b2", dict(batch=2, n_q_heads=16, n_kv_heads=2, ctx_len=3000, n_sparse_layers=3,
                            top_k=64, window=16, n_needles=6, config_id=41)),
    ("decode_4099_k1024_w128_l8", dict(batch=1, n_q_heads=32, n_kv_heads=4, ctx_len=4099,
                                       n_sparse_layers=8, top_k=1024, window=128, n_needles=16,
                                       config_id=42)),
    ("chunk_24_over_500", dict(batch=1, n_q_tokens=24, n_q_heads=16, n_kv_heads=2, ctx_len=500,
                               n_sparse_layers=2, top_k=32, window=8, n_needles=4,
                               config_id=43)),
    ("no_window", dict(batch=1, n_q_heads=8, n_kv_heads=1, ctx_len=700, n_sparse_layers=2,
                       top_k=50, window=0, config_id=44)),
    ("k_covers_context", dict(batch=2, n_q_heads=8, n_kv_heads=1, ctx_len=100, n_sparse_layers=1,
                              top_k=200, window=30, config_id=45)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_swa_variant(hs2, name, kw):
    w = wl.small(name=name, **kw)
    x = wl.generate(w)
    s = hs2.shape_of(w)
    L, B, T, Hkv = w.n_sparse_layers, w.batch, w.n_q_tokens, w.n_kv_heads
    Lc = hs2.local_rows(s)
    k_loc, v_loc = wl.swa_local_cache(L, B, Hkv, Lc, seed=wl.BASE_SEED + 81 + len(name))
    gh.log(f"[swa] {name} S={w.ctx_len} T={T} k={w.top_k} w={w.window} L={L} Lc={Lc}")
    ref = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale, keep_scores=False)
    idx = np.full((B, T, Hkv, s.cap), -1, dtype=np.int32)
    ns = np.zeros((B, T, Hkv), dtype=np.int32)
    for (b, t, g), rr in ref.items():
        idx[b, t, g, : rr["idx"].size] = rr["idx"]
        ns[b, t, g] = rr["idx"].size
    if B > 1:
        ns[1, 0, 0] = 0            # nothing selected: only the window branch remains
    out = torch.empty((L, B, T, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    # with no local rows the caches are passed as NULL
    kl = gh.dev(k_loc) if Lc else None
    vl = gh.dev(v_loc) if Lc else None
    hs2.sparse_attn_swa(s, gh.dev(x["q_sparse"]), gh.dev(x["k"]), gh.dev(x["v"]),
                        torch.from_numpy(idx).cuda(), torch.from_numpy(ns).cuda(), kl, vl, out)
    torch.cuda.synchronize()
    want = orc.sparse_swa_step(x["q_sparse"], x["k"], x["v"], idx, ns, k_loc, v_loc,
                               scale=w.scale, window=w.window)
    e, m = gh.check_outputs(gh.host_f64(out), want, f"swa {name}")
    gh.log(f"  max {e:.3g} mean {m:.3g}")
