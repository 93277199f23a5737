"""The prefill early-exit harness's composition (kv_reuse_amd.prefill_pipeline)
against the CPU oracle, at a small size: the Self-Decoder full layer's output,
the cache rows the early exit builds by KV Bridging (the oracle's projection,
to the bridging tolerance derived in test_gpu_bridge), the rows before the chunk
left untouched, and every Cross-Decoder group's step over the caches so built
(the oracle's step on those same caches, to the parity rules of gpu_helpers)."""
import numpy as np
import pytest
import torch

import oracle.hs2_oracle as orc
from kv_reuse_amd import workloads as wl
from tests import gpu_helpers as gh
from tests.test_gpu_bridge import bits_of, check_rows

pytestmark = pytest.mark.gpu


def test_early_exit_pipeline_small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_reuse_amd import prefill_pipeline as pp
    T, S, Hq, Hkv, D, dm, G, N, k, w = 24, 400, 16, 2, 128, 256, 2, 2, 32, 8
    rng = np.random.default_rng(77)

    def bf(*shape, scale=1.0):
        return wl.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))

    arrays = {"q_self": bf(1, T, Hq, D), "k_self": bf(1, Hkv, S, D), "v_self": bf(1, Hkv, S, D),
              "hidden": bf(1, T, dm), "w_kv": [bf(2, Hkv, D, dm, scale=dm ** -0.5) for _ in range(G)],
              "k_grp": [bf(1, Hkv, S, D) for _ in range(G)],
              "v_grp": [bf(1, Hkv, S, D) for _ in range(G)],
              "q_full": [bf(1, T, Hq, D) for _ in range(G)],
              "q_sparse": [bf(N, 1, T, Hq, D) for _ in range(G)]}
    gh.log(f"[early exit] T={T} S={S} groups={G} sparse={N}")
    t = pp.from_host(arrays)
    p = pp.PrefillPipeline(t, top_k=k, window=w)
    p.full()
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    # the Self-Decoder's full-attention layer over the chunk
    ref = orc.cross_decoder_step(arrays["q_self"], arrays["k_self"], arrays["v_self"], None,
                                 top_k=k, window=w, scale=scale, keep_scores=False)
    out_self = gh.host_f64(p.out_self)
    for (b, tt, g), rr in ref.items():
        gh.check_outputs(out_self[b, tt, 8 * g:8 * g + 8], rr["out_full"], f"self{(b, tt, g)}")
    wk = wl.small(name="group", batch=1, n_q_tokens=T, n_q_heads=Hq, n_kv_heads=Hkv, ctx_len=S,
                  n_sparse_layers=N, top_k=k, window=w)
    for grp in range(G):
        kb, vb = bits_of(t.k_grp[grp]), bits_of(t.v_grp[grp])
        # the chunk's rows: KV Bridging of the hidden states; the older rows kept
        for kv, got in ((0, kb), (1, vb)):
            check_rows(got[:, :, S - T:], arrays["hidden"], arrays["w_kv"][grp], kv,
                       np.arange(T), f"group {grp} {'kv'[kv]}")
            before = (arrays["k_grp"] if kv == 0 else arrays["v_grp"])[grp][:, :, :S - T]
            assert np.array_equal(got[:, :, :S - T], before), f"group {grp}: older rows changed"
        # the group's step over the cache the early exit built
        x = {"q_full": arrays["q_full"][grp], "k": kb, "v": vb, "q_sparse": arrays["q_sparse"][grp]}
        res = {"out_full": gh.host_f64(p.out_full[grp]), "idx": p.idx[grp].cpu().numpy(),
               "n_sel": p.n_sel[grp].cpu().numpy(),
               "out_sparse": gh.host_f64(p.out_sparse[grp])}
        st = gh.compare_step(wk, x, res)
        gh.log(f"  group {grp}: {st}")
