"""hs2_cross_decoder_step_static (the step on the library-held device buffer,
for callers that cannot allocate) against hs2_cross_decoder_step with a
workspace: two calls in a row, the second on a smaller shape (so that it runs
on what the first left in the buffer), each compared bit for bit — the same
kernels on the same inputs give the same bits — with a prefill chunk last."""
import numpy as np
import pytest
import torch

from kv_reuse_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

CASES = [
    # (name, batch, T, Hq, Hkv, S, N, k, w): a larger decode, then a smaller one
    ("decode_s20000_b2", 2, 1, 16, 2, 20000, 2, 256, 64),
    ("decode_s3000_b1", 1, 1, 8, 1, 3000, 1, 64, 16),
    ("chunk_t12_s700", 1, 12, 16, 2, 700, 2, 32, 8),
]


def _run_pair(c, seed):
    from kv_reuse_amd import hs2
    name, B, T, Hq, Hkv, S, N, k, w = c
    wk = wl.small(name=name, batch=B, n_q_tokens=T, n_q_heads=Hq, n_kv_heads=Hkv, ctx_len=S,
                  n_sparse_layers=N, top_k=k, window=w)
    x = wl.generate(wk, seed=seed)
    s = hs2.shape_of(wk)
    assert hs2.workspace_bytes(s, N) <= hs2.HS2_STATIC_SCRATCH_BYTES
    q, kk, vv, qs = gh.dev(x["q_full"]), gh.dev(x["k"]), gh.dev(x["v"]), gh.dev(x["q_sparse"])

    def outputs():
        return {"out": torch.empty((B, T, Hq, 128), dtype=torch.bfloat16, device="cuda"),
                "outs": torch.empty((N, B, T, Hq, 128), dtype=torch.bfloat16, device="cuda"),
                "idx": torch.full((B, T, Hkv, s.cap), -7, dtype=torch.int32, device="cuda"),
                "nsel": torch.full((B, T, Hkv), -7, dtype=torch.int32, device="cuda"),
                "lse": torch.empty((B, T, Hq), dtype=torch.float32, device="cuda"),
                "scores": torch.empty((B, T, Hkv, S), dtype=torch.float32, device="cuda")}

    ref, got = outputs(), outputs()
    ws = hs2.alloc_workspace(s, N)
    hs2.cross_decoder_step(s, q, qs, kk, vv, ref["out"], ref["outs"], ref["idx"], ref["nsel"],
                           lse=ref["lse"], scores=ref["scores"], ws=ws)
    hs2.cross_decoder_step_static(s, q, qs, kk, vv, got["out"], got["outs"], got["idx"],
                                  got["nsel"], lse=got["lse"], scores=got["scores"])
    torch.cuda.synchronize()
    bits = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}
    for key in ref:
        a, b = ref[key].cpu(), got[key].cpu()
        assert torch.equal(a.view(bits[a.dtype]), b.view(bits[b.dtype])), \
            f"{name}: {key} differs from the workspace entry point"
    # the selection is a real one, not the fill values
    nsel = got["nsel"].cpu().numpy()
    assert np.all(nsel == min(S, k + w)) if T == 1 else np.all(nsel > 0)


def test_static_step_matches_the_workspace_step_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for i, c in enumerate(CASES):
        gh.log(f"[no-alloc] {c[0]}")
        _run_pair(c, seed=4100 + i)
