"""CPU oracle for the HySparse2 Cross-Decoder hot path — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never imports, links or calls it.  It shares no code with the HIP path: the
only thing both sides take from elsewhere is the seeded input generator, which
holds none of the method's arithmetic.

What it computes (plain float64 numpy; inputs are bfloat16 bit patterns widened
exactly to float64):

For every batch b, query token t (at position P_t = S - T + t) and KV head g,
with query heads h in the GQA group {g*G, ..., g*G+G-1}:

  1. full attention over the shared KV cache, keys 0..P_t (the key/value rows
     are the cache that "KV Reuse" hands from the group's full-attention layer
     to its sparse layers: news page "两天两连更：小米提前亮出V3底牌",
     section "两级KV共享：让模型少跑一半", item "KV Reuse"):
         s_h[j] = scale * <q_h, k_j>,  p_h = softmax(s_h),  O_h = sum_j p_h[j] v_j
  2. importance of key j: the largest softmax probability that any query head
     of the group gives it, score[j] = max_h p_h[j].  The pages only say that
     the selection comes from the full layer's attention and needs no separately
     trained indexer (video page "小米 MiMo-V3 HySparse2 架构：读长文省一半",
     section "HySparse2 的解法：两派都用，还改了流程"); the max over the group is
     the reading fixed for this project.
  3. token-level selection (news page, section "Token级选择：精准定位大海里的
     那根针"): the most recent `window` tokens [P_t - w + 1, P_t] are always
     kept; from the older tokens [0, P_t - w + 1) the `top_k` with the largest
     score are kept, ties going to the lower index.  Reading: when fewer than
     top_k older tokens exist, all of them are kept.
     Variant (the previous generation's block-level selection, for the
     comparison the same section draws): the older tokens are cut into aligned
     blocks, a block's importance is the largest importance of its tokens, and
     top_k // block whole blocks are kept, ties to the lower block index.
  4'. variant (the previous generation's sparse layer, the one the news page's
     section "Token级选择" says was dropped together with its extra projections
     and local cache): a sliding-window branch with the layer's own local K/V
     for the w most recent positions, plus attention over the selected older
     tokens of the shared cache, each with its own softmax; reading: the two
     branch outputs are added (the pages give no gate).
  4. each sparse layer n attends with its own queries q^(n) to the selected
     rows of the same K/V only, with one softmax over selected + window
     (the same section: the separate sliding-window branch is dropped and local
     and global tokens share one KV cache):
         s'_h[i] = scale * <q^(n)_h, k_i>, i in idx;  O^(n)_h = softmax(s'_h) V[idx]

Upstream of the path (the step just before the full layer):

  0. KV Bridging (news page, section "两级KV共享：让模型少跑一半", item
     "KV Bridging"): the Cross-Decoder's full-attention layer builds its K and
     V from the Self-Decoder's hidden states.  Reading (the page gives no
     formula): a plain linear projection per KV head, no bias, no
     normalisation or position transform inside it,
         K[b, g, t] = W_K[g] h[b, t],   V[b, g, t] = W_V[g] h[b, t],
     written into the cache rows of the tokens' positions; one token at the
     end of the cache is the decode-time append.

Pins (tests/test_oracle_*.py, run with -m "not gpu"): agreement with
torch.nn.functional.scaled_dot_product_attention in float64 on CPU and with
scipy.special.logsumexp; closed forms (constant V, identical keys, one dominant
key); probability / score invariants; brute-force enumeration of every
size-k subset on tiny inputs for the selection; "k covers the context ⇒ sparse
equals dense"; "k = 0 ⇒ sliding-window attention" against SDPA with a band
mask; invariance to permutations of the index list; and planted-mistake
mutants of this module that the pins must reject.  No page prints a worked
example with numbers, so there is no golden value from the pages themselves.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# input widening
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# steps 1-2: full attention and per-key importance for one (b, t, g) row
# ---------------------------------------------------------------------------

def full_attention_row(q_g: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                       scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Dense softmax attention of the G query heads of one group.

    q_g    [G, D] float64 — the group's query heads for one token
    k_rows [n, D] float64 — keys 0..P_t
    v_rows [n, D] float64
    Returns (out [G, D], lse [G], probs [G, n]).
    """
    s = scale * (q_g @ k_rows.T)                      # [G, n]
    m = s.max(axis=1, keepdims=True)
    l = np.exp(s - m).sum(axis=1, keepdims=True)
    lse = m + np.log(l)                               # natural-log normaliser
    probs = np.exp(s - lse)
    out = probs @ v_rows
    return out, lse[:, 0], probs


def importance_scores(probs: np.ndarray) -> np.ndarray:
    """score[j] = max over the group's query heads of their probability for key j."""
    return probs.max(axis=0)


# ---------------------------------------------------------------------------
# step 3: forced recent window + token-level top-k
# ---------------------------------------------------------------------------

def window_and_candidates(pos: int, window: int) -> Tuple[np.ndarray, np.ndarray]:
    """Window W = [max(0, P-w+1), P] (the w most recent, P included); candidates C = [0, P-w+1)."""
    first = max(0, pos - window + 1)
    return np.arange(first, pos + 1, dtype=np.int64), np.arange(0, first, dtype=np.int64)


def select_tokens(score: np.ndarray, pos: int, top_k: int, window: int):
    """Token-level selection for one row.

    score : importance of keys 0..pos (length pos+1)
    Returns (idx ascending int64, tau, sigma) where tau is the score of the last
    key taken (the k-th threshold; nan if none taken) and sigma the largest
    candidate score not taken (nan if none left out).
    """
    win, cand = window_and_candidates(pos, window)
    n_take = min(top_k, cand.size)
    # stable full sort on (-score, index): largest score first, ties to the lower index
    order = np.lexsort((cand, -score[cand]))
    taken = cand[order[:n_take]]
    left = cand[order[n_take:]]
    idx = np.sort(np.concatenate([taken, win]))
    tau = float(score[taken].min()) if taken.size else float("nan")
    sigma = float(score[left].max()) if left.size else float("nan")
    return idx, tau, sigma


def select_blocks(score: np.ndarray, pos: int, top_k: int, window: int, block: int):
    """Block-level selection for one row: the previous generation's variant, in
    which every pick is a whole run of consecutive tokens (news page, section
    "Token级选择：精准定位大海里的那根针", which contrasts it with token-level
    picks; the block explainer page names blocks of 64 or 128 tokens).

    Readings (the pages give no formula): the window is forced as in the
    token-level selection; the older tokens [0, first) are cut into aligned
    blocks [c*block, (c+1)*block), the last one ending at `first`; a block's
    importance is the largest importance of its tokens; the top_k // block
    blocks with the largest importance are kept, ties to the lower block index
    (all blocks when there are fewer).  With block = 1 this is select_tokens.
    Returns (idx ascending int64, tau, sigma) with tau the importance of the
    last block taken and sigma the largest importance of a block left out.
    """
    win, cand = window_and_candidates(pos, window)
    first = cand.size
    n_blocks = (first + block - 1) // block
    bscore = np.array([score[c * block:min((c + 1) * block, first)].max()
                       for c in range(n_blocks)])
    blocks = np.arange(n_blocks, dtype=np.int64)
    n_take = min(top_k // block, n_blocks)
    order = np.lexsort((blocks, -bscore))
    taken = blocks[order[:n_take]]
    left = blocks[order[n_take:]]
    toks = [np.arange(c * block, min((c + 1) * block, first), dtype=np.int64) for c in taken]
    idx = np.sort(np.concatenate(toks + [win]))
    tau = float(bscore[taken].min()) if taken.size else float("nan")
    sigma = float(bscore[left].max()) if left.size else float("nan")
    return idx, tau, sigma


# ---------------------------------------------------------------------------
# step 4: one sparse layer for one row
# ---------------------------------------------------------------------------

def sparse_attention_row(q_g: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                         idx: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of the group's heads over the selected rows only."""
    ks = k_rows[idx]
    vs = v_rows[idx]
    s = scale * (q_g @ ks.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ vs


# ---------------------------------------------------------------------------
# the whole path over a batch
# ---------------------------------------------------------------------------

def cross_decoder_step(q_full: np.ndarray, k: np.ndarray, v: np.ndarray,
                       q_sparse: Optional[np.ndarray], *, top_k: int, window: int,
                       scale: float, rows: Optional[Iterable[Tuple[int, int, int]]] = None,
                       keep_scores: bool = True, block: int = 0) -> Dict[str, object]:
    """Run full attention -> importance -> selection -> N sparse layers.

    q_full   [B][T][Hq][D] bf16 bits
    k, v     [B][Hkv][S][D] bf16 bits
    q_sparse [N][B][T][Hq][D] bf16 bits, or None for no sparse layers
    rows     iterable of (b, t, g) to compute; None = all rows
    block    0: token-level selection; > 0: block-level selection of that size
    Returns a dict keyed by (b, t, g) -> per-row results:
      out_full [G, D], lse [G], score [P_t+1] (if keep_scores), idx, tau,
      sigma, out_sparse [N, G, D].
    """
    B, T, Hq, D = q_full.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    N = 0 if q_sparse is None else q_sparse.shape[0]
    if rows is None:
        rows = [(b, t, g) for b in range(B) for t in range(T) for g in range(Hkv)]
    rows = list(rows)
    results: Dict[Tuple[int, int, int], Dict[str, object]] = {}
    # widen one (b, g) cache at a time to bound memory
    by_bg: Dict[Tuple[int, int], list] = {}
    for (b, t, g) in rows:
        by_bg.setdefault((b, g), []).append(t)
    for (b, g), ts in by_bg.items():
        kk = widen_bf16(k[b, g])
        vv = widen_bf16(v[b, g])
        for t in ts:
            pos = S - T + t
            heads = slice(g * G, (g + 1) * G)
            qg = widen_bf16(q_full[b, t, heads])
            out, lse, probs = full_attention_row(qg, kk[: pos + 1], vv[: pos + 1], scale)
            score = importance_scores(probs)
            if block:
                idx, tau, sigma = select_blocks(score, pos, top_k, window, block)
            else:
                idx, tau, sigma = select_tokens(score, pos, top_k, window)
            outs = np.zeros((N, G, D))
            for n in range(N):
                qn = widen_bf16(q_sparse[n, b, t, heads])
                outs[n] = sparse_attention_row(qn, kk, vv, idx, scale)
            r = {"out_full": out, "lse": lse, "idx": idx, "tau": tau, "sigma": sigma,
                 "out_sparse": outs, "pos": pos}
            if keep_scores:
                r["score"] = score
            results[(b, t, g)] = r
        del kk, vv
    return results


def sparse_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                n_sel: np.ndarray, *, scale: float) -> np.ndarray:
    """Sparse attention alone, given index lists (as the sparse entry point takes them).

    q [L][B][T][Hq][D] bits, idx [B][T][Hkv][cap] int, n_sel [B][T][Hkv]
    Returns out [L][B][T][Hq][D] float64.
    """
    L, B, T, Hq, D = q.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((L, B, T, Hq, D))
    for b in range(B):
        for g in range(Hkv):
            kk = widen_bf16(k[b, g])
            vv = widen_bf16(v[b, g])
            for t in range(T):
                sel = np.asarray(idx[b, t, g, : int(n_sel[b, t, g])], dtype=np.int64)
                if sel.size == 0:
                    # reading: with nothing selected there is no softmax; the
                    # sparse entry point defines such a row's output as zeros
                    continue
                for n in range(L):
                    qn = widen_bf16(q[n, b, t, g * G:(g + 1) * G])
                    out[n, b, t, g * G:(g + 1) * G] = sparse_attention_row(qn, kk, vv, sel, scale)
    return out


# ---------------------------------------------------------------------------
# step 0: KV Bridging (the cache rows the path reads)
# ---------------------------------------------------------------------------

def kv_bridge(hidden: np.ndarray, w_kv: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Cross-Decoder K and V of new tokens from their Self-Decoder hidden states
    (news page, section "两级KV共享：让模型少跑一半", item "KV Bridging").

    hidden [B][n][d_model] bf16 bits; w_kv [2][Hkv][D][d_model] bf16 bits (row
    (0, g, d) is the weight vector of key feature d of KV head g, row (1, g, d)
    that of value feature d).  Returns K_new, V_new [B][Hkv][n][D] float64:
        K_new[b, g, t, d] = sum_m w_kv[0, g, d, m] * hidden[b, t, m]
    and likewise V_new with w_kv[1].
    """
    h = widen_bf16(hidden)
    wk = widen_bf16(w_kv[0])
    wv = widen_bf16(w_kv[1])
    k_new = np.einsum("gdm,btm->bgtd", wk, h)
    v_new = np.einsum("gdm,btm->bgtd", wv, h)
    return k_new, v_new


def cache_append(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
                 v_new: np.ndarray, pos0: int) -> Tuple[np.ndarray, np.ndarray]:
    """Write the new rows at positions pos0 .. pos0 + n - 1 of every KV head's
    cache [B][Hkv][capacity][D]; every other row keeps its value."""
    n = k_new.shape[2]
    k_out = np.array(k_cache, dtype=np.float64, copy=True)
    v_out = np.array(v_cache, dtype=np.float64, copy=True)
    k_out[:, :, pos0:pos0 + n] = k_new
    v_out[:, :, pos0:pos0 + n] = v_new
    return k_out, v_out


# ---------------------------------------------------------------------------
# step 4': the separate sliding-window branch variant of a sparse layer
# ---------------------------------------------------------------------------

def attention_or_zero(q_g: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                      scale: float) -> np.ndarray:
    """Softmax attention of the group's heads over the given rows; zeros when
    there are no rows (an empty branch contributes nothing)."""
    if k_rows.shape[0] == 0:
        return np.zeros((q_g.shape[0], v_rows.shape[1]))
    s = scale * (q_g @ k_rows.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v_rows


def sparse_swa_row(q_g: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, sel: np.ndarray,
                   kloc_rows: np.ndarray, vloc_rows: np.ndarray, scale: float) -> np.ndarray:
    """One sparse layer with a separate sliding-window branch: attention over the
    selected older rows of the shared cache plus attention over the layer's own
    local rows of the window, each normalised on its own, summed."""
    return (attention_or_zero(q_g, k_rows[sel], v_rows[sel], scale)
            + attention_or_zero(q_g, kloc_rows, vloc_rows, scale))


def sparse_swa_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                    n_sel: np.ndarray, k_loc: np.ndarray, v_loc: np.ndarray, *, scale: float,
                    window: int) -> np.ndarray:
    """The variant for every row and layer.

    q [L][B][T][Hq][D], k / v [B][Hkv][S][D] (the shared cache), idx / n_sel as
    the selection writes them (ascending, the window last: its entries are not
    used here), k_loc / v_loc [L][B][Hkv][Lc][D] each layer's own local cache of
    the last Lc = min(S, T + w - 1) positions (row i = position S - Lc + i).
    Returns out [L][B][T][Hq][D] float64.
    """
    L, B, T, Hq, D = q.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    Lc = k_loc.shape[3]
    out = np.zeros((L, B, T, Hq, D))
    for b in range(B):
        for g in range(Hkv):
            kk = widen_bf16(k[b, g])
            vv = widen_bf16(v[b, g])
            for t in range(T):
                pos = S - T + t
                first = max(0, pos - window + 1)
                lst = np.asarray(idx[b, t, g, : int(n_sel[b, t, g])], dtype=np.int64)
                sel = lst[lst < first]
                rows = np.arange(first, pos + 1) - (S - Lc)
                for n in range(L):
                    qn = widen_bf16(q[n, b, t, g * G:(g + 1) * G])
                    kl = widen_bf16(k_loc[n, b, g])[rows]
                    vl = widen_bf16(v_loc[n, b, g])[rows]
                    out[n, b, t, g * G:(g + 1) * G] = sparse_swa_row(qn, kk, vv, sel, kl, vl,
                                                                      scale)
    return out
