"""Seeded synthetic inputs for the HySparse2 Cross-Decoder hot path.

This module only *builds inputs*: it draws seeded random tensors, plants
"needle" keys, adds the slow drift or the heavy tail that a workload asks for,
and rounds everything to bfloat16 bit patterns.  It computes nothing that the
method computes (no attention, no softmax, no selection), so that both the CPU
oracle and the HIP path can take their inputs from here without sharing any
of the method's arithmetic.

The five named workloads follow the five benchmark shapes of the project
(decode at 2K / 32K / 256K / 1M context and a 4096-token prefill chunk over a
128K context).  The needles stand in for the retrieval structure ("the needle
in the haystack") that the news page "两天两连更：小米提前亮出V3底牌"
describes in its section "Token级选择：精准定位大海里的那根针"; the long-context
benchmarks that page reports on are not available and are not reproduced.

Recipe (the same for every workload; sizes per workload below):

* one ``numpy.random.SeedSequence(seed)`` spawns independent child streams in
  this fixed order: q_full, k, v, needle positions, drift, heavy-tail
  positions, then one stream per sparse layer for q_sparse[n]; the k, v,
  drift and heavy-tail streams each spawn one grandchild per (batch, kv head)
  row, in row-major order, so that rows can be drawn in parallel threads;
* every tensor entry is a float32 standard normal, rounded to bfloat16 with
  round-to-nearest-even;
* drift (256K workload): per (batch, kv head, dim) a float32 random walk along
  the sequence with N(0, sd^2) steps, added to the N(0,1) draw before rounding;
* heavy tail (1M workload): round(frac * S) key rows per (batch, kv head),
  drawn without replacement, are multiplied by ``heavy_mult`` before rounding;
* needles (decode): ``n_needles`` positions per (batch, kv head) drawn
  uniformly without replacement from [0, S); each such key row is set to
  bf16(4 * mean over the group's query heads of q_full) (mean in float64 over
  the bf16 query values, rounded float64 -> float32 -> bf16).  Needles are
  written last and overwrite drift / heavy-tail rows;
* needles (prefill chunk): needle i draws a query token t_i uniformly in
  [0, T) and a position p_i uniformly in [0, P_{t_i} - w + 1) (an older token
  that query t_i may select), and sets K[b, g, p_i] = bf16(4 * mean of that
  token's group queries).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

BASE_SEED = 20260900


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_tokens: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    n_sparse_layers: int
    top_k: int = 1024
    window: int = 128
    n_needles: int = 0          # per (batch, kv head)
    drift_sd: float = 0.0       # random-walk step sd along the sequence
    heavy_frac: float = 0.0     # fraction of key rows scaled by heavy_mult
    heavy_mult: float = 3.0
    needle_scale: float = 4.0
    config_id: int = 0          # seed offset

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def seed(self) -> int:
        return BASE_SEED + self.config_id

    def positions(self) -> np.ndarray:
        """Position P_t of each query token: the chunk is the last T tokens."""
        return self.ctx_len - self.n_q_tokens + np.arange(self.n_q_tokens, dtype=np.int64)

    def rows(self) -> int:
        return self.batch * self.n_q_tokens * self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "decode_2k_b4": Workload(
        name="decode_2k_b4", batch=4, n_q_tokens=1, n_q_heads=16, n_kv_heads=2,
        head_dim=128, ctx_len=2048, n_sparse_layers=3, n_needles=16, config_id=1),
    "decode_32k_b16": Workload(
        name="decode_32k_b16", batch=16, n_q_tokens=1, n_q_heads=32, n_kv_heads=4,
        head_dim=128, ctx_len=32768, n_sparse_layers=4, n_needles=64, config_id=2),
    "decode_256k_b4_drift": Workload(
        name="decode_256k_b4_drift", batch=4, n_q_tokens=1, n_q_heads=32, n_kv_heads=4,
        head_dim=128, ctx_len=262144, n_sparse_layers=4, n_needles=256, drift_sd=0.01,
        config_id=3),
    "decode_1m_b1_heavy": Workload(
        name="decode_1m_b1_heavy", batch=1, n_q_tokens=1, n_q_heads=32, n_kv_heads=4,
        head_dim=128, ctx_len=1048576, n_sparse_layers=8, n_needles=1024, heavy_frac=0.01,
        config_id=4),
    "prefill_4k_over_128k": Workload(
        name="prefill_4k_over_128k", batch=1, n_q_tokens=4096, n_q_heads=32, n_kv_heads=4,
        head_dim=128, ctx_len=131072, n_sparse_layers=4, n_needles=512, config_id=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Finite inputs only (the sum below cannot overflow 32 bits for them)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (input construction only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def generate(w: Workload, seed: Optional[int] = None,
             with_sparse: bool = True) -> Dict[str, np.ndarray]:
    """Build the inputs of one workload as bf16 bit arrays (numpy uint16).

    Returns a dict with
      q_full   [B][T][Hq][D]
      k, v     [B][Hkv][S][D]
      q_sparse [N][B][T][Hq][D]   (if with_sparse)
    """
    seed = w.seed if seed is None else seed
    B, T, Hq, Hkv, D, S, G = (w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads,
                              w.head_dim, w.ctx_len, w.group)
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    children = np.random.SeedSequence(seed).spawn(6 + w.n_sparse_layers)
    rq = np.random.Generator(np.random.PCG64(children[0]))
    rneedle = np.random.Generator(np.random.PCG64(children[3]))

    q_full = f32_to_bf16_bits(_normal_f32(rq, (B, T, Hq, D)))
    k = np.empty((B, Hkv, S, D), dtype=np.uint16)
    v = np.empty((B, Hkv, S, D), dtype=np.uint16)
    n_rows = B * Hkv
    ks, vs, ds, hs = (c.spawn(n_rows) for c in (children[1], children[2], children[4],
                                                children[5]))

    def make_row(i: int) -> None:
        b, g = divmod(i, Hkv)
        z = _normal_f32(np.random.Generator(np.random.PCG64(ks[i])), (S, D))
        if w.drift_sd > 0.0:
            steps = _normal_f32(np.random.Generator(np.random.PCG64(ds[i])), (S, D))
            steps *= np.float32(w.drift_sd)
            np.cumsum(steps, axis=0, out=steps)        # float32 random walk along S
            z += steps
            del steps
        if w.heavy_frac > 0.0:
            n_heavy = int(round(w.heavy_frac * S))
            pos = np.random.Generator(np.random.PCG64(hs[i])).choice(S, size=n_heavy,
                                                                      replace=False)
            z[pos] *= np.float32(w.heavy_mult)
        k[b, g] = f32_to_bf16_bits(z)
        del z
        v[b, g] = f32_to_bf16_bits(_normal_f32(np.random.Generator(np.random.PCG64(vs[i])),
                                               (S, D)))

    workers = max(1, min(n_rows, os.cpu_count() or 1, 8))
    if workers == 1:
        for i in range(n_rows):
            make_row(i)
    else:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(make_row, range(n_rows)))

    needles = []   # (b, g, query token the needle is planted for, key position)
    if w.n_needles > 0:
        qf = bf16_bits_to_f32(q_full).astype(np.float64)
        pos_all = w.positions()
        for b in range(B):
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                if T == 1:
                    n = min(w.n_needles, S)
                    pos = rneedle.choice(S, size=n, replace=False)
                    vec = w.needle_scale * qf[b, 0, heads, :].mean(axis=0)
                    k[b, g, pos] = f32_to_bf16_bits(vec.astype(np.float32))[None, :]
                    needles.extend((b, g, 0, int(p)) for p in pos)
                else:
                    for _ in range(w.n_needles):
                        t = int(rneedle.integers(0, T))
                        hi = int(pos_all[t]) - w.window + 1
                        if hi <= 0:
                            continue
                        p = int(rneedle.integers(0, hi))
                        vec = w.needle_scale * qf[b, t, heads, :].mean(axis=0)
                        k[b, g, p] = f32_to_bf16_bits(vec.astype(np.float32))
                        needles.append((b, g, t, p))

    # a later needle at the same key overwrites an earlier one: keep the last
    last = {}
    for (b, g, t, p) in needles:
        last[(b, g, p)] = t
    out = {"q_full": q_full, "k": k, "v": v,
           "needles": np.array([(b, g, t, p) for (b, g, p), t in sorted(last.items())],
                               dtype=np.int64).reshape(-1, 4)}
    if with_sparse:
        qs = np.empty((w.n_sparse_layers, B, T, Hq, D), dtype=np.uint16)
        for n in range(w.n_sparse_layers):
            r = np.random.Generator(np.random.PCG64(children[6 + n]))
            qs[n] = f32_to_bf16_bits(_normal_f32(r, (B, T, Hq, D)))
        out["q_sparse"] = qs
    return out


def needle_recall(w: "Workload", needles: np.ndarray, idx: np.ndarray,
                  n_sel: np.ndarray) -> dict:
    """A diagnostic, not a pass criterion: of the planted needles that lie among
    their query row's older keys (below P_t - w + 1, so not forced in by the
    window), how many the selection kept.  idx [B][T][Hkv][cap], n_sel [B][T][Hkv]."""
    pos = w.positions()
    found = total = 0
    for b, g, t, p in needles:
        first = int(pos[t]) - w.window + 1
        if p >= first:
            continue
        total += 1
        row = idx[b, t, g, : int(n_sel[b, t, g])]
        found += int(np.any(row == p))
    return {"needles": total, "found": found,
            "recall": round(found / total, 4) if total else None, "kind": "diagnostic"}


def small(name: str = "small", *, batch=1, n_q_tokens=1, n_q_heads=8, n_kv_heads=1,
          head_dim=128, ctx_len=256, n_sparse_layers=2, top_k=16, window=8,
          n_needles=0, drift_sd=0.0, heavy_frac=0.0, config_id=100) -> Workload:
    """A small workload for tests (any shape the oracle finishes in seconds)."""
    return Workload(name=name, batch=batch, n_q_tokens=n_q_tokens, n_q_heads=n_q_heads,
                    n_kv_heads=n_kv_heads, head_dim=head_dim, ctx_len=ctx_len,
                    n_sparse_layers=n_sparse_layers, top_k=top_k, window=window,
                    n_needles=n_needles, drift_sd=drift_sd, heavy_frac=heavy_frac,
                    config_id=config_id)


# ---------------------------------------------------------------------------
# KV Bridging inputs: Self-Decoder hidden states and projection weights
# ---------------------------------------------------------------------------
# The pages give no hidden size and no weights.  The synthetic ones: hidden
# states N(0, 1); weights N(0, 1/d_model), so that every projected K/V entry is
# about N(0, 1) like the cache entries of the workloads above.  Both are float32
# draws rounded to bfloat16.  The bridge workloads use d_model = 4096.

BRIDGE_D_MODEL = 4096


def bridge_inputs(batch: int, n_tokens: int, d_model: int, n_kv_heads: int, head_dim: int = 128,
                  seed: int = BASE_SEED + 50):
    """(hidden [B][n][d_model], w_kv [2][Hkv][D][d_model]) as bf16 bit patterns
    (numpy); streams spawned in the order hidden, w_kv."""
    ss = np.random.SeedSequence(seed)
    rh, rw = (np.random.default_rng(c) for c in ss.spawn(2))
    hidden = f32_to_bf16_bits(_normal_f32(rh, (batch, n_tokens, d_model)))
    w = _normal_f32(rw, (2, n_kv_heads, head_dim, d_model)) * np.float32(1.0 / np.sqrt(d_model))
    return hidden, f32_to_bf16_bits(w.astype(np.float32))


def bridge_inputs_device(batch: int, n_tokens: int, d_model: int, n_kv_heads: int,
                         head_dim: int = 128, seed: int = BASE_SEED + 60):
    """The same distributions drawn on the GPU with torch's seeded generator, for
    sizes too large to draw on the host (a whole prompt's hidden states):
    (hidden, w_kv) as torch.bfloat16 device tensors."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hidden = torch.randn((batch, n_tokens, d_model), generator=g, device="cuda",
                         dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((2, n_kv_heads, head_dim, d_model), generator=g, device="cuda",
                    dtype=torch.float32) * (1.0 / float(np.sqrt(d_model)))
    return hidden, w.to(torch.bfloat16)


def swa_local_cache(n_layers: int, batch: int, n_kv_heads: int, rows: int, head_dim: int = 128,
                    seed: int = BASE_SEED + 80):
    """Each sparse layer's own local window cache for the separate-window
    variant, (k_loc, v_loc) [L][B][Hkv][rows][D] bf16 bits, N(0, 1) entries like
    the shared cache; streams spawned in the order k_loc, v_loc."""
    ss = np.random.SeedSequence(seed)
    rk, rv = (np.random.default_rng(c) for c in ss.spawn(2))
    shape = (n_layers, batch, n_kv_heads, rows, head_dim)
    return f32_to_bf16_bits(_normal_f32(rk, shape)), f32_to_bf16_bits(_normal_f32(rv, shape))
