"""Prefill with early exit, as a composition of the library's calls (attention
layers only): the timing harness for the prefill saving the pages describe.

The news page "两天两连更：小米提前亮出V3底牌", section "两级KV共享：让模型少跑一半",
says that every KV cache the Cross-Decoder needs can be built from the
Self-Decoder's hidden states (KV Bridging for the group's full layer, KV Reuse
for its sparse layers), so a prefill can stop once the Self-Decoder has run;
section "Token级选择：精准定位大海里的那根针" adds that for the 49-layer model a
prefill node runs the first 25 layers, with a single full-attention layer
among them.  The video page "小米 MiMo-V3 HySparse2 架构：读长文省一半", section
"HySparse2 的解法：两派都用，还改了流程", says the same (the prefill may exit
early).

For one chunk of T tokens at the end of an S-token context the harness times
  early exit:  the Self-Decoder's full-attention layer over the chunk, then KV
               Bridging of the chunk's hidden states into the cache of every
               Cross-Decoder group (the prefill stops here);
  full:        the same, then every group's full layer, token selection and
               sparse layers over the chunk (a prefill that runs the
               Cross-Decoder too).
Readings (the pages give no such detail): the Cross-Decoder is n_groups groups
of one full and n_sparse sparse layers; the Self-Decoder's other layers
(sliding-window attention in the hybrid design the pages compare with) and
every MLP / MoE block are left out of both sides; all tensors are synthetic.
Nothing here computes: every step is a call of libhs2.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import hs2


@dataclass
class PipelineTensors:
    """Device tensors of one pipeline (bf16 unless stated)."""
    q_self: torch.Tensor          # [1][T][Hq][D]  the Self-Decoder full layer's queries
    k_self: torch.Tensor          # [1][Hkv][S][D] its cache
    v_self: torch.Tensor
    hidden: torch.Tensor          # [1][T][d_model] the chunk's Self-Decoder hidden states
    w_kv: List[torch.Tensor]      # per group [2][Hkv][D][d_model] KV Bridging weights
    k_grp: List[torch.Tensor]     # per group [1][Hkv][S][D] caches (rows S-T.. written by bridging)
    v_grp: List[torch.Tensor]
    q_full: List[torch.Tensor]    # per group [1][T][Hq][D]
    q_sparse: List[torch.Tensor]  # per group [N][1][T][Hq][D]


class PrefillPipeline:
    def __init__(self, t: PipelineTensors, *, top_k: int = 1024, window: int = 128):
        self.t = t
        _, T, Hq, D = t.q_self.shape
        _, Hkv, S, _ = t.k_self.shape
        self.T, self.S, self.Hq, self.Hkv, self.D = T, S, Hq, Hkv, D
        self.n_groups = len(t.w_kv)
        self.n_sparse = t.q_sparse[0].shape[0] if self.n_groups else 0
        self.shape = hs2.ShapeArgs(batch=1, n_q_tokens=T, n_q_heads=Hq, n_kv_heads=Hkv,
                                   head_dim=D, ctx_len=S, top_k=top_k, window=window)
        dev = t.q_self.device
        # one workspace serves every call (they run in order on one stream)
        self.ws = hs2.alloc_workspace(self.shape, self.n_sparse, device=dev)
        self.out_self = torch.empty((1, T, Hq, D), dtype=torch.bfloat16, device=dev)
        self.out_full = [torch.empty((1, T, Hq, D), dtype=torch.bfloat16, device=dev)
                         for _ in range(self.n_groups)]
        self.out_sparse = [torch.empty((self.n_sparse, 1, T, Hq, D), dtype=torch.bfloat16,
                                       device=dev) for _ in range(self.n_groups)]
        self.idx = [torch.empty((1, T, Hkv, self.shape.cap), dtype=torch.int32, device=dev)
                    for _ in range(self.n_groups)]
        self.n_sel = [torch.empty((1, T, Hkv), dtype=torch.int32, device=dev)
                      for _ in range(self.n_groups)]

    # ---- the steps
    def self_decoder(self):
        """The Self-Decoder's one full-attention layer over the chunk."""
        t = self.t
        hs2.full_attn_scores(self.shape, t.q_self, t.k_self, t.v_self, self.out_self, ws=self.ws)

    def bridge(self):
        """KV Bridging: every group's cache rows of the chunk from the hidden states."""
        t = self.t
        for g in range(self.n_groups):
            hs2.kv_bridge(t.hidden, t.w_kv[g], t.k_grp[g], t.v_grp[g], self.S - self.T)

    def cross_decoder(self):
        """Each group's full layer, selection and sparse layers over the chunk."""
        t = self.t
        for g in range(self.n_groups):
            hs2.cross_decoder_step(self.shape, t.q_full[g], t.q_sparse[g], t.k_grp[g], t.v_grp[g],
                                   self.out_full[g], self.out_sparse[g], self.idx[g],
                                   self.n_sel[g], ws=self.ws)

    def early_exit(self):
        self.self_decoder()
        self.bridge()

    def full(self):
        self.early_exit()
        self.cross_decoder()


def synthetic(*, chunk: int = 4096, ctx: int = 131072, n_q_heads: int = 32, n_kv_heads: int = 4,
              head_dim: int = 128, d_model: int = 4096, n_groups: int = 4, n_sparse: int = 5,
              seed: int = 20260970, device: str = "cuda") -> PipelineTensors:
    """Seeded synthetic tensors drawn on the device (torch's generator): queries,
    caches and hidden states N(0, 1), bridging weights N(0, 1/d_model), all
    float32 draws rounded to bf16; the group caches' chunk rows are left for
    the bridging to write."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def randn(*shape, scale: float = 1.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x *= scale
        return x.to(torch.bfloat16)

    T, S, Hq, Hkv, D = chunk, ctx, n_q_heads, n_kv_heads, head_dim
    k_grp, v_grp = [], []
    for _ in range(n_groups):
        k = randn(1, Hkv, S, D)
        v = randn(1, Hkv, S, D)
        k[:, :, S - T:] = 0      # written by the bridging
        v[:, :, S - T:] = 0
        k_grp.append(k)
        v_grp.append(v)
    return PipelineTensors(
        q_self=randn(1, T, Hq, D), k_self=randn(1, Hkv, S, D), v_self=randn(1, Hkv, S, D),
        hidden=randn(1, T, d_model),
        w_kv=[randn(2, Hkv, D, d_model, scale=d_model ** -0.5) for _ in range(n_groups)],
        k_grp=k_grp, v_grp=v_grp,
        q_full=[randn(1, T, Hq, D) for _ in range(n_groups)],
        q_sparse=[randn(n_sparse, 1, T, Hq, D) for _ in range(n_groups)])


def from_host(arrays: dict, device: str = "cuda") -> PipelineTensors:
    """PipelineTensors from host bf16 bit arrays (numpy uint16), e.g. for tests:
    keys q_self, k_self, v_self, hidden, w_kv, k_grp, v_grp, q_full, q_sparse
    (the per-group entries are lists)."""
    import numpy as np

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)

    def one(key: str):
        return dev(arrays[key])

    def many(key: str):
        return [dev(a) for a in arrays[key]]

    return PipelineTensors(q_self=one("q_self"), k_self=one("k_self"), v_self=one("v_self"),
                           hidden=one("hidden"), w_kv=many("w_kv"), k_grp=many("k_grp"),
                           v_grp=many("v_grp"), q_full=many("q_full"),
                           q_sparse=many("q_sparse"))
