"""Pins that tie the CPU oracle to something other than itself.

Each pin takes the oracle module (so that the mutation test can hand in a copy
with a planted mistake) and raises AssertionError when the oracle disagrees
with a library routine, a closed form, a brute-force enumeration or an
invariant that the mathematics fixes.  None of them retypes the oracle's own
formula.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch
from scipy.special import logsumexp

from kv_reuse_amd import workloads as wl


def _rng(seed):
    return np.random.default_rng(seed)


def _bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA in float64 on CPU. q [H, Lq, D], k/v [H, Lk, D], mask [Lq, Lk] bool (True = keep)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, scale=scale).numpy()


# ---------------------------------------------------------------------------
# full attention
# ---------------------------------------------------------------------------

def pin_full_attention_vs_sdpa(orc, seed=1):
    """Whole step's full-attention output on a tiny GQA prefill chunk vs SDPA (float64)."""
    w = wl.small(batch=2, n_q_tokens=3, n_q_heads=4, n_kv_heads=2, head_dim=8,
                 ctx_len=11, n_sparse_layers=0, top_k=3, window=2, config_id=seed)
    x = wl.generate(w, with_sparse=False)
    res = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale)
    G = w.group
    pos = w.positions()
    for b in range(w.batch):
        kk = np.repeat(_f64(x["k"][b]), G, axis=0)          # [Hq, S, D]
        vv = np.repeat(_f64(x["v"][b]), G, axis=0)
        q = _f64(x["q_full"][b]).transpose(1, 0, 2)         # [Hq, T, D]
        mask = np.arange(w.ctx_len)[None, :] <= pos[:, None]
        ref = _sdpa(q, kk, vv, w.scale, mask)               # [Hq, T, D]
        for t in range(w.n_q_tokens):
            for g in range(w.n_kv_heads):
                got = res[(b, t, g)]["out_full"]
                np.testing.assert_allclose(got, ref[g * G:(g + 1) * G, t], rtol=1e-10, atol=1e-12)
                s = w.scale * (q[g * G:(g + 1) * G, t] @ kk[g * G, : pos[t] + 1].T)
                np.testing.assert_allclose(res[(b, t, g)]["lse"], logsumexp(s, axis=1),
                                           rtol=1e-12, atol=1e-12)


def pin_attention_closed_forms(orc, seed=2):
    r = _rng(seed)
    G, n, D = 3, 9, 8
    q = r.standard_normal((G, D))
    k = r.standard_normal((n, D))
    # constant V => output equals that constant for every head
    v = np.full((n, D), 0.625)
    out, _, p = orc.full_attention_row(q, k, v, 0.3)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # identical keys => uniform weights => output is the mean of V, lse = s + ln n
    kid = np.tile(k[:1], (n, 1))
    v = r.standard_normal((n, D))
    out, lse, p = orc.full_attention_row(q, kid, v, 0.3)
    np.testing.assert_allclose(p, 1.0 / n, rtol=1e-12)
    np.testing.assert_allclose(out, np.tile(v.mean(axis=0), (G, 1)), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, 0.3 * (q @ k[0]) + np.log(n), rtol=1e-12, atol=1e-12)
    # a hand-worked case: one head, logits 0, ln2, ln4 (scale 1, D = 1) => p = 1/7, 2/7, 4/7
    out, lse, p = orc.full_attention_row(np.array([[1.0]]), np.log(np.array([[1.0], [2.0], [4.0]])),
                                         np.array([[1.0], [0.0], [0.0]]), 1.0)
    np.testing.assert_allclose(p[0], [1 / 7, 2 / 7, 4 / 7], rtol=1e-14)
    np.testing.assert_allclose(lse, [np.log(7.0)], rtol=1e-14)
    np.testing.assert_allclose(out, [[1 / 7]], rtol=1e-14)
    # one dominant key: its value row comes out
    k2 = r.standard_normal((n, D))
    k2[4] = 100.0 * q[0] / np.linalg.norm(q[0])
    v = r.standard_normal((n, D))
    out, _, _ = orc.full_attention_row(q[:1], k2, v, 1.0)
    np.testing.assert_allclose(out[0], v[4], atol=1e-6)


# ---------------------------------------------------------------------------
# importance scores
# ---------------------------------------------------------------------------

def pin_score_invariants(orc, seed=3):
    w = wl.small(batch=1, n_q_tokens=2, n_q_heads=8, n_kv_heads=2, head_dim=16,
                 ctx_len=40, n_sparse_layers=0, top_k=5, window=4, n_needles=2,
                 config_id=seed)
    x = wl.generate(w, with_sparse=False)
    res = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=w.top_k,
                                 window=w.window, scale=w.scale)
    G = w.group
    for (b, t, g), rr in res.items():
        sc = rr["score"]
        pos = rr["pos"]
        assert sc.shape == (pos + 1,)
        assert np.all(sc > 0) and np.all(sc <= 1.0 + 1e-15)
        assert 1.0 - 1e-12 <= sc.sum() <= G + 1e-12
        q = _f64(x["q_full"][b, t, g * G:(g + 1) * G])
        kk = _f64(x["k"][b, g, : pos + 1])
        s = w.scale * (q @ kk.T)
        p = np.exp(s - logsumexp(s, axis=1, keepdims=True))
        assert np.all(sc >= p - 1e-15)                      # score dominates every head
        np.testing.assert_allclose(sc, p.max(axis=0), rtol=1e-12)
    # G = 1: the score is the head's own softmax probability
    q = _rng(seed).standard_normal((1, 8))
    k = _rng(seed + 1).standard_normal((12, 8))
    _, _, p = orc.full_attention_row(q, k, k, 0.5)
    np.testing.assert_allclose(orc.importance_scores(p), torch.softmax(
        torch.from_numpy(0.5 * (q @ k.T)), dim=-1).numpy()[0], rtol=1e-12)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _brute_force_select(score, pos, k, w):
    """Enumerate every size-m subset of the candidates and keep the one that
    beats every left-out candidate (larger score, or equal score and lower index)."""
    first = max(0, pos - w + 1)
    cand = list(range(first))
    m = min(k, len(cand))
    winners = []
    for sub in itertools.combinations(cand, m):
        s = set(sub)
        ok = all(score[i] > score[j] or (score[i] == score[j] and i < j)
                 for i in s for j in cand if j not in s)
        if ok:
            winners.append(s)
    assert len(winners) == 1, "the definition must single out one set"
    return sorted(winners[0] | set(range(first, pos + 1)))


def pin_selection_brute_force(orc, seed=4, trials=60):
    r = _rng(seed)
    for _ in range(trials):
        pos = int(r.integers(0, 14))
        w = int(r.integers(0, 5))
        k = int(r.integers(0, 8))
        # few distinct values so that ties are common
        score = r.integers(0, 4, size=pos + 1).astype(np.float64) / 8.0 + 1e-3
        idx, tau, sigma = orc.select_tokens(score, pos, k, w)
        assert list(idx) == _brute_force_select(score, pos, k, w)
        first = max(0, pos - w + 1)
        taken = [i for i in idx if i < first]
        if taken:
            assert tau == min(score[i] for i in taken)
        left = [j for j in range(first) if j not in set(idx)]
        if left:
            assert sigma == max(score[j] for j in left)


def pin_selection_invariants(orc, seed=5):
    r = _rng(seed)
    for pos, k, w in [(50, 10, 8), (7, 10, 8), (100, 0, 8), (30, 5, 0), (3, 2, 1), (0, 4, 4)]:
        score = r.random(pos + 1)
        idx, tau, sigma = orc.select_tokens(score, pos, k, w)
        first = max(0, pos - w + 1)
        win = set(range(first, pos + 1))
        assert win <= set(idx.tolist()), "forced window always present"
        assert len(win) == min(w, pos + 1)
        assert len(idx) == min(k, first) + len(win)
        assert np.all(np.diff(idx) > 0), "ascending, no duplicates"
        sel = [i for i in idx if i < first]
        rest = [j for j in range(first) if j not in set(sel)]
        if sel and rest:
            assert min(score[sel]) >= max(score[rest])
    # identical scores => the lowest indices win
    pos, k, w = 40, 7, 5
    idx, _, _ = orc.select_tokens(np.full(pos + 1, 0.25), pos, k, w)
    assert idx.tolist() == list(range(k)) + list(range(pos - w + 1, pos + 1))


def _brute_force_blocks(score, pos, k, w, bs):
    """Block selection by enumeration: block c = tokens [c*bs, min((c+1)*bs, first));
    its value is the largest score in it (explicit loop); keep the size-m set of
    blocks that beats every left-out block (larger value, or equal and lower index)."""
    first = max(0, pos - w + 1)
    nb = (first + bs - 1) // bs
    val = []
    for c in range(nb):
        best = -np.inf
        for j in range(c * bs, min((c + 1) * bs, first)):
            if score[j] > best:
                best = score[j]
        val.append(best)
    m = min(k // bs, nb)
    winners = []
    for sub in itertools.combinations(range(nb), m):
        s = set(sub)
        ok = all(val[i] > val[j] or (val[i] == val[j] and i < j)
                 for i in s for j in range(nb) if j not in s)
        if ok:
            winners.append(s)
    assert len(winners) == 1, "the definition must single out one set"
    toks = set()
    for c in winners[0]:
        toks |= set(range(c * bs, min((c + 1) * bs, first)))
    return sorted(toks | set(range(first, pos + 1))), val, winners[0]


def pin_block_selection_brute_force(orc, seed=15, trials=80):
    r = _rng(seed)
    for _ in range(trials):
        pos = int(r.integers(0, 30))
        w = int(r.integers(0, 6))
        bs = int(r.integers(2, 6))
        k = bs * int(r.integers(0, 5)) + int(r.integers(0, bs))   # not always a multiple
        score = r.integers(0, 4, size=pos + 1).astype(np.float64) / 8.0 + 1e-3
        idx, tau, sigma = orc.select_blocks(score, pos, k, w, bs)
        ref, val, won = _brute_force_blocks(score, pos, k, w, bs)
        assert list(idx) == ref
        if won:
            assert tau == min(val[c] for c in won)
        left = [c for c in range(len(val)) if c not in won]
        if left:
            assert sigma == max(val[c] for c in left)


def pin_block_selection_special_cases(orc, seed=16):
    """Blocks of one token are the token-level selection; equal scores keep the
    lowest blocks; the selected older tokens are whole blocks."""
    r = _rng(seed)
    for pos, k, w in [(50, 10, 8), (7, 10, 8), (100, 0, 8), (30, 5, 0), (0, 4, 4)]:
        score = r.random(pos + 1)
        a = orc.select_blocks(score, pos, k, w, 1)
        b = orc.select_tokens(score, pos, k, w)
        assert a[0].tolist() == b[0].tolist()
        np.testing.assert_equal(a[1:], b[1:])          # tau and sigma (nan when empty)
    pos, k, w, bs = 70, 16, 6, 8
    idx, _, _ = orc.select_blocks(np.full(pos + 1, 0.5), pos, k, w, bs)
    assert idx.tolist() == list(range(16)) + list(range(65, 71))
    score = r.random(pos + 1)
    idx, tau, sigma = orc.select_blocks(score, pos, k, w, bs)
    first = pos - w + 1
    older = [i for i in idx.tolist() if i < first]
    blocks = sorted(set(i // bs for i in older))
    assert len(blocks) == k // bs
    assert older == [j for c in blocks for j in range(c * bs, min((c + 1) * bs, first))]
    assert tau >= sigma


def pin_swa_branch_vs_sdpa(orc, seed=17):
    """The separate-window variant of a sparse layer is the sum of two softmax
    attentions: checked against torch SDPA (float64) run on each branch's rows."""
    r = _rng(seed)
    G, D, S = 4, 16, 60
    for n_sel, n_loc in [(10, 6), (0, 6), (10, 0), (1, 1)]:
        q = r.standard_normal((G, D))
        k = r.standard_normal((S, D))
        v = r.standard_normal((S, D))
        kl = r.standard_normal((n_loc, D))
        vl = r.standard_normal((n_loc, D))
        sel = np.sort(r.choice(S, size=n_sel, replace=False))
        got = orc.sparse_swa_row(q, k, v, sel, kl, vl, 0.3)
        ref = np.zeros((G, D))
        if n_sel:
            ref += _sdpa(q[:, None], np.broadcast_to(k[sel], (G, n_sel, D)).copy(),
                         np.broadcast_to(v[sel], (G, n_sel, D)).copy(), 0.3)[:, 0]
        if n_loc:
            ref += _sdpa(q[:, None], np.broadcast_to(kl, (G, n_loc, D)).copy(),
                         np.broadcast_to(vl, (G, n_loc, D)).copy(), 0.3)[:, 0]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        perm = r.permutation(n_sel)
        np.testing.assert_allclose(orc.sparse_swa_row(q, k, v, sel[perm], kl[::-1], vl[::-1], 0.3),
                                   got, rtol=1e-12, atol=1e-12)


def pin_swa_step_reads_the_window(orc, seed=18):
    """The step's window branch reads exactly the local rows of positions
    [P_t - w + 1, P_t], and the selected branch only the list's older entries:
    with equal local keys the branch is the mean of the local values, which are
    one-hot codes of their positions."""
    r = _rng(seed)
    L, B, T, Hkv, G, D, S, w = 2, 1, 3, 1, 8, 128, 50, 5
    Lc = min(S, T + w - 1)
    q = _bits(r.standard_normal((L, B, T, Hkv * G, D)))
    k = _bits(r.standard_normal((B, Hkv, S, D)))
    v = _bits(r.standard_normal((B, Hkv, S, D)))
    k_loc = _bits(np.ones((L, B, Hkv, Lc, D)))
    v_loc = np.zeros((L, B, Hkv, Lc, D), dtype=np.float32)
    for i in range(Lc):
        v_loc[:, :, :, i, (S - Lc + i) % D] = 1.0
    v_loc = _bits(v_loc)
    cap = 12
    idx = np.full((B, T, Hkv, cap), -1, dtype=np.int32)
    n_sel = np.zeros((B, T, Hkv), dtype=np.int32)
    for t in range(T):
        pos = S - T + t
        lst = list(range(3 + t, 9 + t)) + list(range(pos - w + 1, pos + 1))
        idx[0, t, 0, : len(lst)] = lst
        n_sel[0, t, 0] = len(lst)
    got = orc.sparse_swa_step(q, k, v, idx, n_sel, k_loc, v_loc, scale=0.1, window=w)
    kk, vv = _f64(k[0, 0]), _f64(v[0, 0])
    for t in range(T):
        pos = S - T + t
        sel = np.arange(3 + t, 9 + t)
        for n in range(L):
            qn = _f64(q[n, 0, t])
            loc = np.zeros(D)
            loc[[p % D for p in range(pos - w + 1, pos + 1)]] = 1.0 / w
            ref = _sdpa(qn[:, None], np.broadcast_to(kk[sel], (G, sel.size, D)).copy(),
                        np.broadcast_to(vv[sel], (G, sel.size, D)).copy(), 0.1)[:, 0] + loc
            np.testing.assert_allclose(got[n, 0, t], ref, rtol=1e-12, atol=1e-12)


def pin_identical_keys_select_prefix(orc, seed=6):
    """All keys equal => all scores tie => idx = [0, k) followed by the window."""
    w = wl.small(batch=1, n_q_tokens=1, n_q_heads=4, n_kv_heads=1, head_dim=8, ctx_len=30,
                 n_sparse_layers=0, top_k=6, window=5, config_id=seed)
    x = wl.generate(w, with_sparse=False)
    x["k"][:] = x["k"][:, :, :1, :]
    res = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], None, top_k=6, window=5,
                                 scale=w.scale)
    assert res[(0, 0, 0)]["idx"].tolist() == list(range(6)) + list(range(25, 30))


# ---------------------------------------------------------------------------
# sparse layers
# ---------------------------------------------------------------------------

def pin_sparse_dense_equivalence(orc, seed=7):
    """k >= |C| keeps every key, so a sparse layer with the full layer's
    queries reproduces the dense output exactly (up to rounding)."""
    w = wl.small(batch=1, n_q_tokens=2, n_q_heads=4, n_kv_heads=2, head_dim=8, ctx_len=25,
                 n_sparse_layers=1, top_k=100, window=3, config_id=seed)
    x = wl.generate(w)
    qs = x["q_full"][None].copy()
    res = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], qs, top_k=w.top_k,
                                 window=w.window, scale=w.scale)
    for key, rr in res.items():
        assert rr["idx"].size == rr["pos"] + 1
        np.testing.assert_allclose(rr["out_sparse"][0], rr["out_full"], rtol=1e-11, atol=1e-13)


def pin_sparse_sliding_window(orc, seed=8):
    """k = 0 leaves only the forced window: SDPA with a band mask."""
    w = wl.small(batch=1, n_q_tokens=3, n_q_heads=2, n_kv_heads=1, head_dim=8, ctx_len=20,
                 n_sparse_layers=2, top_k=0, window=4, config_id=seed)
    x = wl.generate(w)
    res = orc.cross_decoder_step(x["q_full"], x["k"], x["v"], x["q_sparse"], top_k=0,
                                 window=4, scale=w.scale)
    pos = w.positions()
    kk = _f64(x["k"][0])
    vv = _f64(x["v"][0])
    j = np.arange(w.ctx_len)
    mask = (j[None, :] <= pos[:, None]) & (j[None, :] > pos[:, None] - 4)
    for n in range(2):
        q = _f64(x["q_sparse"][n, 0]).transpose(1, 0, 2)     # [Hq, T, D]
        ref = _sdpa(q, np.repeat(kk, 2, axis=0), np.repeat(vv, 2, axis=0), w.scale, mask)
        for t in range(3):
            np.testing.assert_allclose(res[(0, t, 0)]["out_sparse"][n], ref[:, t],
                                       rtol=1e-11, atol=1e-13)


def pin_sparse_permutation_invariance(orc, seed=9):
    r = _rng(seed)
    q = r.standard_normal((3, 8))
    k = r.standard_normal((30, 8))
    v = r.standard_normal((30, 8))
    idx = np.array([0, 3, 4, 9, 17, 29])
    a = orc.sparse_attention_row(q, k, v, idx, 0.4)
    b = orc.sparse_attention_row(q, k, v, idx[r.permutation(idx.size)], 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    # and it equals SDPA restricted to those rows
    ref = _sdpa(q[:, None, :], np.repeat(k[idx][None], 3, 0), np.repeat(v[idx][None], 3, 0), 0.4)
    np.testing.assert_allclose(a, ref[:, 0], rtol=1e-12, atol=1e-13)


def pin_widening(orc, seed=10):
    r = _rng(seed)
    x = r.standard_normal(1000).astype(np.float32) * 10
    bits = _bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.widen_bf16(bits), ref)




def pin_sparse_step_empty_rows(orc, seed=11):
    """A row whose index list is empty gets zeros; the other rows are unaffected."""
    r = _rng(seed)
    bits = _bits(r.standard_normal((1, 1, 1, 8, 8)))
    kv = _bits(r.standard_normal((1, 1, 10, 8)))
    idx = np.array([[[[0, 3, 9, -1]]]])
    out = orc.sparse_step(bits, kv, kv, idx, np.array([[[0]]]), scale=0.3)
    assert np.all(out == 0.0)
    out = orc.sparse_step(bits, kv, kv, idx, np.array([[[3]]]), scale=0.3)
    ref = orc.sparse_attention_row(_f64(bits[0, 0, 0]), _f64(kv[0, 0]), _f64(kv[0, 0]),
                                   np.array([0, 3, 9]), 0.3)
    np.testing.assert_allclose(out[0, 0, 0], ref, rtol=1e-14)


def _bridge_inputs(rng, B, n, dm, Hkv, D):
    hidden = _bits(rng.standard_normal((B, n, dm)))
    w_kv = _bits(rng.standard_normal((2, Hkv, D, dm)) * 0.1)
    return hidden, w_kv


def pin_bridge_brute_force(orc, seed=12):
    """KV Bridging against explicit loops over every output element (tiny sizes)."""
    rng = _rng(seed)
    B, n, dm, Hkv, D = 2, 3, 5, 2, 4
    hidden, w_kv = _bridge_inputs(rng, B, n, dm, Hkv, D)
    h, w = _f64(hidden), _f64(w_kv)
    k_new, v_new = orc.kv_bridge(hidden, w_kv)
    assert k_new.shape == (B, Hkv, n, D) and v_new.shape == (B, Hkv, n, D)
    for b in range(B):
        for g in range(Hkv):
            for t in range(n):
                for d in range(D):
                    ek = sum(w[0, g, d, m] * h[b, t, m] for m in range(dm))
                    ev = sum(w[1, g, d, m] * h[b, t, m] for m in range(dm))
                    assert abs(k_new[b, g, t, d] - ek) <= 1e-12 * (1 + abs(ek))
                    assert abs(v_new[b, g, t, d] - ev) <= 1e-12 * (1 + abs(ev))


def pin_bridge_closed_forms(orc, seed=13):
    """Identity weights copy the hidden state's slice of each head; a one-hot
    hidden state picks one weight column; the projection is linear."""
    rng = _rng(seed)
    B, n, Hkv, D = 2, 3, 2, 8
    dm = Hkv * D
    hidden = _bits(rng.standard_normal((B, n, dm)))
    eye = np.zeros((2, Hkv, D, dm), dtype=np.float32)
    for g in range(Hkv):
        for d in range(D):
            eye[0, g, d, g * D + d] = 1.0
            eye[1, g, d, (g * D + d + 1) % dm] = 1.0     # V: shifted by one feature
    k_new, v_new = orc.kv_bridge(hidden, _bits(eye))
    h = _f64(hidden)
    for g in range(Hkv):
        assert np.array_equal(k_new[:, g], h[:, :, g * D:(g + 1) * D])
        assert np.array_equal(v_new[:, g], np.roll(h, -1, axis=2)[:, :, g * D:(g + 1) * D])
    # one-hot hidden state e_m: K[b, g, t, d] = W_K[g, d, m]
    w_kv = _bits(rng.standard_normal((2, Hkv, D, 6)))
    m = 4
    onehot = np.zeros((1, 1, 6), dtype=np.float32)
    onehot[0, 0, m] = 1.0
    k1, v1 = orc.kv_bridge(_bits(onehot), w_kv)
    assert np.array_equal(k1[0, :, 0], _f64(w_kv[0])[:, :, m])
    assert np.array_equal(v1[0, :, 0], _f64(w_kv[1])[:, :, m])
    # linearity in the hidden state (values exact in bf16: small integers)
    a = rng.integers(-3, 4, size=(2, 2, 6)).astype(np.float32)
    c = rng.integers(-3, 4, size=(2, 2, 6)).astype(np.float32)
    ka, va = orc.kv_bridge(_bits(a), w_kv)
    kc, vc = orc.kv_bridge(_bits(c), w_kv)
    ks, vs = orc.kv_bridge(_bits(2 * a + c), w_kv)
    np.testing.assert_allclose(ks, 2 * ka + kc, rtol=0, atol=1e-12)
    np.testing.assert_allclose(vs, 2 * va + vc, rtol=0, atol=1e-12)


def pin_cache_append(orc, seed=14):
    """Appending writes exactly the new rows; appending tokens one at a time
    equals projecting them together; the other rows are untouched."""
    rng = _rng(seed)
    B, n, dm, Hkv, D, cap, pos0 = 2, 4, 8, 2, 4, 12, 5
    hidden, w_kv = _bridge_inputs(rng, B, n, dm, Hkv, D)
    k0 = rng.standard_normal((B, Hkv, cap, D))
    v0 = rng.standard_normal((B, Hkv, cap, D))
    k_new, v_new = orc.kv_bridge(hidden, w_kv)
    k1, v1 = orc.cache_append(k0, v0, k_new, v_new, pos0)
    keep = np.ones(cap, dtype=bool)
    keep[pos0:pos0 + n] = False
    assert np.array_equal(k1[:, :, keep], k0[:, :, keep])
    assert np.array_equal(v1[:, :, keep], v0[:, :, keep])
    assert np.array_equal(k1[:, :, pos0:pos0 + n], k_new)
    assert np.array_equal(v1[:, :, pos0:pos0 + n], v_new)
    kk, vv = k0, v0
    for t in range(n):
        kt, vt = orc.kv_bridge(hidden[:, t:t + 1], w_kv)
        kk, vv = orc.cache_append(kk, vv, kt, vt, pos0 + t)
    np.testing.assert_allclose(kk, k1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(vv, v1, rtol=0, atol=1e-12)
    # the rows written hold the projection of their own token
    h = _f64(hidden)
    wk = _f64(w_kv[0])
    np.testing.assert_allclose(k1[1, 1, pos0 + 2], wk[1] @ h[1, 2], rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_full_attention_vs_sdpa,
    pin_attention_closed_forms,
    pin_score_invariants,
    pin_selection_brute_force,
    pin_selection_invariants,
    pin_identical_keys_select_prefix,
    pin_sparse_dense_equivalence,
    pin_sparse_sliding_window,
    pin_sparse_permutation_invariance,
    pin_widening,
    pin_sparse_step_empty_rows,
    pin_bridge_brute_force,
    pin_bridge_closed_forms,
    pin_cache_append,
    pin_block_selection_brute_force,
    pin_block_selection_special_cases,
    pin_swa_branch_vs_sdpa,
    pin_swa_step_reads_the_window,
]
