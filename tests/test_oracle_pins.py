"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: a closed
form, a library routine, an invariant the pages state, brute force over a tiny
input, or the worked 16-token example printed on the "DeepSeek-V4" page.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_16tok.txt")


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- bf16 storage
def test_bf16_rounding_matches_torch(orc):
    a = rng(1).standard_normal(20000).astype(np.float32) * 7
    ours = orc.round_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert orc.round_bf16(np.float32([1.0 + 2 ** -8]))[0] == 1.0
    assert orc.round_bf16(np.float32([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


# ----------------------------------------------------------------- RoPE
def test_rope_table_closed_forms(orc):
    theta = 160000.0
    cs = orc.rope_table(300, 64, theta)
    assert np.array_equal(cs[0, :, 0], np.ones(32, np.float32))
    assert np.array_equal(cs[0, :, 1], np.zeros(32, np.float32))
    p = np.arange(300)
    # pair 0 has frequency 1: the angle is the position itself
    np.testing.assert_allclose(cs[:, 0, 0], np.cos(p), atol=6e-8)
    np.testing.assert_allclose(cs[:, 0, 1], np.sin(p), atol=6e-8)
    # pair 16 of 32 has frequency theta^-1/2
    f16 = 1.0 / math.sqrt(theta)
    np.testing.assert_allclose(cs[:, 16, 0], np.cos(p * f16), atol=6e-8)
    np.testing.assert_allclose(cs[:, 16, 1], np.sin(p * f16), atol=6e-8)


def test_rope_is_complex_multiplication(orc):
    v = rng(2).standard_normal((50, 96)).astype(np.float32)
    pos = rng(3).integers(0, 131073, 50)
    ours = orc.rope_apply(v, 64, 160000.0, pos, +1)
    ref = brute.rope_complex(v, 64, 160000.0, pos, +1)
    np.testing.assert_allclose(ours, ref, atol=2e-5)
    assert np.array_equal(ours[:, :32], v[:, :32])        # leading channels untouched
    back = orc.rope_apply(ours, 64, 160000.0, pos, -1)
    np.testing.assert_allclose(back, v, atol=2e-5)


def test_rope_relative_position(orc):
    """<rot(q,a), rot(k,b)> depends only on a-b (what eq. 26 relies on)."""
    q = rng(4).standard_normal((1, 64)).astype(np.float32)
    k = rng(5).standard_normal((1, 64)).astype(np.float32)
    d1 = (orc.rope_apply(q, 64, 1e4, 1000, +1) @ orc.rope_apply(k, 64, 1e4, 990, +1).T).item()
    d2 = (orc.rope_apply(q, 64, 1e4, 10, +1) @ k.T).item()
    assert abs(d1 - d2) < 1e-3


# ----------------------------------------------------------------- YaRN
# DeepseekV4Config: compress_rope_theta is used with rope scaling for YaRN; the
# parameters below are the published YaRN defaults (beta_fast 32, beta_slow 1)
# at a 16x extension of a 65536-token context.
YARN = dict(rope_dim=64, theta=160000.0, factor=16.0, original_max_pos=65536)


def _plain_freqs(orc, rope_dim, theta):
    """Pair frequencies read back from the (already pinned) plain table: the
    angle at position 1 is the frequency itself (all are below pi)."""
    cs = orc.rope_table(2, rope_dim, theta).astype(np.float64)
    return np.arctan2(cs[1, :, 1], cs[1, :, 0])


def test_yarn_factor_one_is_plain_rope(orc):
    f = orc.yarn_freqs(64, 160000.0, 1.0, 65536)
    p = np.arange(0, 131073, 97)
    a = orc.rope_table(131073, 64, 160000.0, freqs=f)[p]
    b = orc.rope_table(131073, 64, 160000.0)[p]
    np.testing.assert_allclose(a, b, atol=1e-7)


def test_yarn_frequencies_by_turns(orc):
    """Pairs that turn many times over the original context (at least beta_fast
    times, with a pair of margin) keep their frequency; pairs that turn at most
    beta_slow times (with a pair of margin) are slowed down by the factor; the
    pairs between blend the two with a weight linear in the pair index."""
    d, theta, s, L = YARN["rope_dim"], YARN["theta"], YARN["factor"], YARN["original_max_pos"]
    f = _plain_freqs(orc, d, theta)
    fy = orc.yarn_freqs(d, theta, s, L, 32.0, 1.0)
    turns = L * f / (2 * np.pi)
    step = theta ** (2.0 / d)                 # turn ratio of neighbouring pairs
    fast = turns >= 32.0 * step
    slow = turns <= 1.0 / step
    assert fast.sum() >= 4 and slow.sum() >= 4 and (~fast & ~slow).sum() >= 4
    np.testing.assert_allclose(fy[fast], f[fast], rtol=1e-6)
    np.testing.assert_allclose(fy[slow], f[slow] / s, rtol=1e-6)
    ramp = (f - fy) / (f - f / s)
    assert np.all(ramp > -1e-6) and np.all(ramp < 1 + 1e-6)
    assert np.all(np.diff(ramp) > -1e-6)      # monotone: slower pairs interpolate more
    inner = np.nonzero((ramp > 1e-6) & (ramp < 1 - 1e-6))[0]
    assert len(inner) >= 4
    steps = np.diff(ramp[inner])
    np.testing.assert_allclose(steps, steps[0], rtol=1e-4)


def test_yarn_interpolated_pairs_stretch_positions(orc):
    """An interpolated (slow) pair at position factor * p has the angle the
    plain pair has at p: the original context, stretched by the factor."""
    d, theta, s, L = YARN["rope_dim"], YARN["theta"], YARN["factor"], YARN["original_max_pos"]
    fy = orc.yarn_freqs(d, theta, s, L)
    f = _plain_freqs(orc, d, theta)
    slow = np.nonzero(L * f / (2 * np.pi) <= 1.0 / theta ** (2.0 / d))[0]
    p = np.arange(0, 8000, 7)
    ty = orc.rope_table(int(s) * 8000, d, theta, freqs=fy)
    tp = orc.rope_table(8000, d, theta)
    np.testing.assert_allclose(ty[int(s) * p][:, slow], tp[p][:, slow], atol=1e-6)
    # and the fast pairs are untouched at every position
    fast = np.nonzero(L * f / (2 * np.pi) >= 32.0 * theta ** (2.0 / d))[0]
    np.testing.assert_array_equal(ty[:8000][:, fast], tp[:, fast])


# ----------------------------------------------------------------- compressor
def test_compress_null_gate_is_window_mean(orc):
    S, D, m = 37, 24, 4
    x = rng(6).standard_normal((S, D)).astype(np.float32)
    for ov in (0, 1):
        pool = orc.compress(x, None, None, m=m, overlap=ov)
        assert pool.shape == (S // m, D)
        for w in range(S // m):
            lo = max(0, (w - ov) * m)
            np.testing.assert_allclose(pool[w], x[lo:(w + 1) * m].mean(0), atol=1e-6)


def test_compress_constant_rows_and_dominant_slot(orc):
    S, D, m = 32, 16, 4
    row = rng(7).standard_normal(D).astype(np.float32)
    x = np.tile(row, (S, 1))
    gate = rng(8).standard_normal((S, D)).astype(np.float32)
    pool = orc.compress(x, gate, None, m=m, overlap=1)
    np.testing.assert_allclose(pool, np.tile(row, (S // m, 1)), atol=1e-6)
    # a slot bias that dominates slot 2 (the previous block's third token)
    x = rng(9).standard_normal((S, D)).astype(np.float32)
    bias = np.zeros((2 * m, D), np.float32)
    bias[2] = 80.0
    pool = orc.compress(x, None, bias, m=m, overlap=1)
    for w in range(1, S // m):
        np.testing.assert_allclose(pool[w], x[(w - 1) * m + 2], atol=1e-5)
    # entry 0 has no previous block: its slots 0..m-1 do not exist
    np.testing.assert_allclose(pool[0], x[0:m].mean(0), atol=1e-6)


def test_compress_softmax_gate_two_tokens(orc):
    """m=2, no overlap: weights are the two-way softmax of the gate logits."""
    x = rng(10).standard_normal((8, 6)).astype(np.float32)
    g = rng(11).standard_normal((8, 6)).astype(np.float32)
    pool = orc.compress(x, g, None, m=2, overlap=0)
    for w in range(4):
        a, b = g[2 * w].astype(np.float64), g[2 * w + 1].astype(np.float64)
        wa = 1.0 / (1.0 + np.exp(b - a))
        np.testing.assert_allclose(pool[w], wa * x[2 * w] + (1 - wa) * x[2 * w + 1], atol=1e-6)


def test_compress_token_level_is_rope_copy(orc):
    x = rng(12).standard_normal((40, 96)).astype(np.float32)
    pool = orc.compress(x, None, None, m=1, overlap=0, rope_dim=64, theta=1e4, pos0=7)
    ref = brute.rope_complex(x, 64, 1e4, np.arange(40) + 7, +1)
    np.testing.assert_allclose(pool, ref, atol=2e-5)
    pool0 = orc.compress(x, None, None, m=1, overlap=0)
    assert np.array_equal(pool0, x)


def test_compress_entry_rope_position_and_bf16(orc):
    x = rng(13).standard_normal((64, 32)).astype(np.float32)
    a = orc.compress(x, None, None, m=4, overlap=1, rope_dim=16, theta=160000.0, pos0=100)
    b = orc.compress(x, None, None, m=4, overlap=1)
    ref = brute.rope_complex(b, 16, 160000.0, 100 + 4 * np.arange(16), +1)
    np.testing.assert_allclose(a, ref, atol=2e-5)
    c = orc.compress(x, None, None, m=4, overlap=1, round_bf16=True)
    assert np.array_equal(c, orc.round_bf16(b))


# ----------------------------------------------------------------- readiness
def test_ready_count_rule(orc):
    for m in (1, 4, 8, 128):
        for T in (0, 3, 64):
            for t in range(-2, 600):
                assert orc.ready_count(t, m, T) == brute.ready(t, m, T)


# ----------------------------------------------------------------- index scores
def _idx_inputs(n=6, nI=4, cI=32, T=20, seed=20):
    r = rng(seed)
    q = r.standard_normal((n, nI, cI)).astype(np.float32)
    w = r.standard_normal((n, nI)).astype(np.float32)
    k = r.standard_normal((T, cI)).astype(np.float32)
    t = np.array([200, 79, 5, 3, 0, 150])[:n]
    return q, w, t, k


def test_index_score_single_head_is_positive_part_of_dot(orc):
    q, w, t, k = _idx_inputs(nI=1)
    s = orc.index_scores(q, np.ones_like(w), t, k, m=4)
    for r in range(len(t)):
        R = brute.ready(int(t[r]), 4, k.shape[0])
        dots = k.astype(np.float64) @ q[r, 0].astype(np.float64)
        np.testing.assert_allclose(s[r, :R], np.maximum(dots[:R], 0), rtol=1e-5, atol=1e-5)
        assert np.all(np.isneginf(s[r, R:]))
    # q = -k makes every dot product with that key negative -> exactly zero
    q2 = -k[None, None, 3].repeat(1, 0)
    s2 = orc.index_scores(q2, np.ones((1, 1), np.float32), np.array([100]), k, m=4)
    assert s2[0, 3] == 0.0 and not np.signbit(s2[0, 3])


def test_index_score_weights_linear_and_heads_additive(orc):
    q, w, t, k = _idx_inputs()
    s = orc.index_scores(q, w, t, k, m=4)
    s2 = orc.index_scores(q, 2 * w, t, k, m=4)
    fin = np.isfinite(s)
    np.testing.assert_allclose(s2[fin], 2 * s[fin], rtol=1e-6, atol=1e-6)
    sa = orc.index_scores(q[:, :2], w[:, :2], t, k, m=4)
    sb = orc.index_scores(q[:, 2:], w[:, 2:], t, k, m=4)
    np.testing.assert_allclose((sa + sb)[fin], s[fin], rtol=1e-5, atol=1e-5)
    perm = np.array([2, 0, 3, 1])
    sp = orc.index_scores(q[:, perm], w[:, perm], t, k, m=4)
    np.testing.assert_allclose(sp[fin], s[fin], rtol=1e-5, atol=1e-5)


def test_index_score_signed_weights_against_float64(orc):
    """Several heads with weights of both signs, against the score written out
    in float64 numpy: the head weight multiplies the ReLU'd dot product (a
    negative weight makes a head's positive match lower the score; the ReLU
    acts on the dot product alone, before the weight)."""
    r = rng(23)
    n, nI, cI, T = 9, 6, 32, 24
    q = r.standard_normal((n, nI, cI)).astype(np.float32)
    w = r.standard_normal((n, nI)).astype(np.float32)
    w[:, 0] = -np.abs(w[:, 0]) - 0.5            # at least one negative head per row
    w[:, 1] = np.abs(w[:, 1]) + 0.5             # and one positive
    k = r.standard_normal((T, cI)).astype(np.float32)
    t = np.array([95, 94, 40, 11, 7, 3, 60, 33, 200])
    s = orc.index_scores(q, w, t, k, m=4)
    dots = np.einsum("njc,wc->njw", q.astype(np.float64), k.astype(np.float64))
    ref = np.einsum("nj,njw->nw", w.astype(np.float64), np.maximum(dots, 0.0))
    for i in range(n):
        R = brute.ready(int(t[i]), 4, T)
        np.testing.assert_allclose(s[i, :R], ref[i, :R], rtol=1e-5, atol=1e-5)
    # the data really separates the two orderings: w * ReLU(dot) differs from
    # ReLU(w * dot) on many ready entries
    alt = np.maximum(w.astype(np.float64)[:, :, None] * dots, 0.0).sum(1)
    assert np.mean(np.abs(alt - ref) > 1e-2) > 0.5


@pytest.mark.parametrize("cI", [32, 128])
def test_index_score_hadamard_invariance(orc, cI):
    """An orthonormal transform applied to both q and k leaves the scores
    unchanged (the "DeepSeek-V3.2" page relies on Hq.Hk = q.k)."""
    q, w, t, k = _idx_inputs(cI=cI)
    Hm = scipy.linalg.hadamard(cI).astype(np.float64) / math.sqrt(cI)
    s = orc.index_scores(q, w, t, k, m=4)
    sh = orc.index_scores((q.astype(np.float64) @ Hm.T).astype(np.float32), w, t,
                          (k.astype(np.float64) @ Hm.T).astype(np.float32), m=4)
    fin = np.isfinite(s)
    np.testing.assert_allclose(sh[fin], s[fin], rtol=1e-4, atol=2e-4)


# ----------------------------------------------------------------- top-k
def _brute_topk(scores, t, k, m):
    n, T = scores.shape
    out = np.full((n, k), -1, np.int32)
    for r in range(n):
        R = brute.ready(int(t[r]), m, T)
        order = sorted(range(R), key=lambda w: (-float(scores[r, w]), w))[:k]
        sel = sorted(order)
        out[r, :len(sel)] = sel
    return out


def test_topk_matches_full_sort(orc):
    r = rng(30)
    n, T, k = 40, 90, 16
    scores = r.standard_normal((n, T)).astype(np.float32)
    scores[:, ::7] = 0.0                       # exact ties
    scores[:, 3::11] = -0.0                    # signed-zero ties
    scores[5, :] = 1.5                          # a row of all-equal scores
    t = r.integers(-1, 4 * T + 10, n)
    assert np.array_equal(orc.topk(scores, t, k=k, m=4), _brute_topk(scores, t, k, 4))


def test_index_topk_against_float64_selection(orc):
    """The fused indexer step picks the entries a float64 evaluation of the
    score ranks highest (inputs drawn so that no two ready scores of a row lie
    closer than the fp32 evaluation's error), ascending, -1 padded."""
    r = rng(41)
    n, nI, cI, T, k = 12, 8, 16, 40, 7
    q = r.standard_normal((n, nI, cI)).astype(np.float32)
    w = r.standard_normal((n, nI)).astype(np.float32)
    kk = r.standard_normal((T, cI)).astype(np.float32)
    t = np.array([3, 7, 11, 15, 27, 40, 80, 100, 159, 160, 30, 2])
    dots = np.einsum("njc,wc->njw", q.astype(np.float64), kk.astype(np.float64))
    s64 = np.einsum("nj,njw->nw", w.astype(np.float64), np.maximum(dots, 0.0))
    got = orc.index_topk(q, w, t, kk, k=k, m=4)
    for i in range(n):
        R = brute.ready(int(t[i]), 4, T)
        sv = np.sort(s64[i, :R])[::-1]
        if R > k:
            assert sv[k - 1] - sv[k] > 1e-3     # no near tie at the boundary: a unique set
        best = sorted(np.argsort(-s64[i, :R], kind="stable")[:min(k, R)].tolist())
        assert got[i, :len(best)].tolist() == best
        assert np.all(got[i, len(best):] == -1)


def test_topk_worked_example_and_padding(orc):
    """16 tokens, m=4, k=2: no entry before t=3, one at t=3..6, two from t=7."""
    T, k, m = 4, 2, 4
    scores = rng(31).standard_normal((16, T)).astype(np.float32)
    idx = orc.topk(scores, np.arange(16), k=k, m=m)
    golden = _read_golden()["csa_slots"]
    for t in range(16):
        assert int((idx[t] >= 0).sum()) == golden[t][0]
    assert np.all(idx[:3] == -1)
    assert list(idx[3]) == [0, -1]
    # k >= ready: every ready entry, ascending, then -1
    idx = orc.topk(scores, np.array([15]), k=6, m=m)
    assert list(idx[0]) == [0, 1, 2, 3, -1, -1]


# ----------------------------------------------------------------- attention
def _read_golden():
    d = {"sliding": {}, "hca": {}, "csa_slots": {}}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, vals = line.split(":")
        sec, tt = head.split()
        t = int(tt.split("=")[1])
        d[sec][t] = [] if vals.strip() == "-" else [int(v) for v in vals.split()]
    return d


def test_attention_worked_example_visibility(orc):
    """q = 0 gives uniform weights over the visible keys; one-hot keys then
    reveal exactly which window positions and pool entries a query sees."""
    golden = _read_golden()
    S, W = 16, 8
    D = 32
    kv = np.zeros((S, D), np.float32)
    kv[np.arange(S), np.arange(S)] = 1.0              # key s = e_s
    pool = np.zeros((2, D), np.float32)
    pool[0, 16] = pool[1, 17] = 1.0                   # entry w = e_{16+w}
    q = np.zeros((S, 1, D), np.float32)
    out = orc.attention(q, np.arange(S), kv_win=kv, win_pos0=0, window=W, pool=pool,
                        idx=None, m=8, sink=None, scale=1.0)[:, 0]
    for t in range(S):
        vis_win = [s for s in range(16) if out[t, s] > 0]
        vis_pool = [w for w in range(2) if out[t, 16 + w] > 0]
        assert vis_win == golden["sliding"][t]
        assert vis_pool == golden["hca"][t]
        n = len(vis_win) + len(vis_pool)
        np.testing.assert_allclose(out[t][out[t] > 0], 1.0 / n, rtol=1e-6)


def _attn_case(seed, n=12, H=3, D=32, rope=8, T=10, L=40, W=6, k=4, m=4, sink=True):
    r = rng(seed)
    q = r.standard_normal((n, H, D)).astype(np.float32)
    kv = r.standard_normal((L, D)).astype(np.float32)
    pool = r.standard_normal((T, D)).astype(np.float32)
    z = r.standard_normal(H).astype(np.float32) if sink else None
    t = r.integers(0, L, n)
    idx = np.full((n, k), -1, np.int32)
    for i in range(n):
        R = brute.ready(int(t[i]), m, T)
        ch = np.sort(r.choice(R, size=min(k, R), replace=False)) if R else []
        idx[i, :len(ch)] = ch
    return q, kv, pool, z, t, idx


@pytest.mark.parametrize("dense", [False, True])
@pytest.mark.parametrize("dv_mode", ["full", "latent"])
def test_attention_equals_dense_additive_mask(orc, dense, dv_mode):
    """P1/P9: gathered attention equals one dense softmax over all keys with an
    additive 0/-inf mask (window rule + selected or ready pool entries)."""
    q, kv, pool, z, t, idx = _attn_case(40 + dense)
    D, rope = q.shape[2], 8
    dv = D if dv_mode == "full" else D - rope
    kw = dict(kv_win=kv, win_pos0=0, window=6, pool=pool, m=4, sink=z, rope_dim=rope,
              theta=1e4, scale=0.3, dv=dv)
    out = orc.attention(q, t, idx=None if dense else idx, **kw)
    if dense:
        allowed = lambda tt, r: np.arange(pool.shape[0]) < brute.ready(tt, 4, pool.shape[0])
    else:
        allowed = lambda tt, r: np.isin(np.arange(pool.shape[0]), idx[r][idx[r] >= 0])
    ref = brute.dense_masked_attention(q, t, kv_win=kv, win_pos0=0, window=6, pool=pool,
                                       allowed_pool=allowed, sink=z, rope_dim=rope,
                                       theta=1e4, scale=0.3, dv=dv)
    np.testing.assert_allclose(out, ref, atol=1e-5, rtol=1e-5)


def test_attention_window_offset_rows(orc):
    """kv_win row r holds position win_pos0 + r; positions outside it are absent."""
    q, kv, pool, z, t, idx = _attn_case(50)
    t = t + 1000
    out = orc.attention(q, t, kv_win=kv, win_pos0=995, window=6, pool=pool, idx=idx, m=4,
                        sink=z, rope_dim=8, theta=1e4, scale=0.3)
    allowed = lambda tt, r: np.isin(np.arange(pool.shape[0]), idx[r][idx[r] >= 0])
    ref = brute.dense_masked_attention(q, t, kv_win=kv, win_pos0=995, window=6, pool=pool,
                                       allowed_pool=allowed, sink=z, rope_dim=8, theta=1e4,
                                       scale=0.3, dv=q.shape[2])
    np.testing.assert_allclose(out, ref, atol=1e-5, rtol=1e-5)


@pytest.mark.parametrize("delta", [1, 1000, 65536])
def test_attention_shift_invariance_eq26(orc, delta):
    """Shifting every position (queries, window rows, pool entries) by delta
    leaves the output unchanged: q rotated at +t, keys rotated at their
    positions, output rope slice rotated back at -t."""
    r = rng(60)
    S, D, H, rope, m = 48, 64, 2, 16, 4
    x = r.standard_normal((S, D)).astype(np.float32)
    g = r.standard_normal((S, D)).astype(np.float32)
    q = r.standard_normal((S, H, D)).astype(np.float32)
    z = r.standard_normal(H).astype(np.float32)
    outs = []
    for p0 in (0, delta):
        kv = orc.compress(x, None, None, m=1, overlap=0, rope_dim=rope, theta=160000.0, pos0=p0)
        pool = orc.compress(x, g, None, m=m, overlap=1, rope_dim=rope, theta=160000.0, pos0=p0)
        tpos = np.arange(S) + p0
        # readiness depends on the position within the sequence, so pass the
        # same idx (all entries ready at the in-sequence position) to both
        idx = np.full((S, 3), -1, np.int32)
        for i in range(S):
            R = brute.ready(i, m, pool.shape[0])
            sel = list(range(max(0, R - 3), R))
            idx[i, :len(sel)] = sel
        outs.append(orc.attention(q, tpos, kv_win=kv, win_pos0=p0, window=8, pool=pool,
                                  idx=idx, m=m, sink=z, rope_dim=rope, theta=160000.0,
                                  scale=0.125))
    np.testing.assert_allclose(outs[1], outs[0], atol=1e-4)


def test_attention_sink_limits(orc):
    """P3: no sink = textbook softmax attention (torch SDPA, fp64); a huge sink
    drives the output to zero; equal logits give p = 1/(n + e^(z - l))."""
    q, kv, pool, z, t, idx = _attn_case(70, rope=0)
    kw = dict(kv_win=kv, win_pos0=0, window=6, pool=pool, idx=idx, m=4, rope_dim=0,
              theta=1e4, scale=0.3)
    out = orc.attention(q, t, sink=None, **kw)
    keys = np.concatenate([kv, pool]).astype(np.float64)
    for r in range(len(t)):
        allow = np.zeros(len(keys), bool)
        lo = max(0, int(t[r]) - 6 + 1)
        allow[lo:int(t[r]) + 1] = True
        allow[kv.shape[0] + idx[r][idx[r] >= 0]] = True
        kt = torch.from_numpy(keys)[None, None]                      # [1, 1, L+T, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[r].astype(np.float64))[None, :, None, :],  # [1, H, 1, D]
            kt, kt, attn_mask=torch.from_numpy(allow)[None, None, None], scale=0.3)
        np.testing.assert_allclose(out[r], ref[0, :, 0].numpy(), atol=1e-5)
    big = orc.attention(q, t, sink=np.full(q.shape[1], 200.0, np.float32), **kw)
    assert np.abs(big).max() < 1e-30
    # equal logits: every key identical
    D = q.shape[2]
    key = rng(71).standard_normal(D).astype(np.float32)
    kvc = np.tile(key, (40, 1))
    qq = rng(72).standard_normal((1, 2, D)).astype(np.float32)
    zz = np.array([0.5, -1.0], np.float32)
    o = orc.attention(qq, np.array([20]), kv_win=kvc, win_pos0=0, window=6, sink=zz,
                      scale=0.3, rope_dim=0, m=4)
    for h in range(2):
        l = 0.3 * float(qq[0, h].astype(np.float64) @ key)
        p = 1.0 / (6 + math.exp(zz[h] - l))
        np.testing.assert_allclose(o[0, h], 6 * p * key, rtol=1e-5, atol=1e-6)


def test_attention_reduces_to_sliding_window_sdpa(orc):
    """P10: one head, no sink, no rope, no pool = causal sliding-window
    attention, as torch's scaled_dot_product_attention computes it."""
    r = rng(80)
    S, D, W = 30, 16, 5
    q = r.standard_normal((S, 1, D)).astype(np.float32)
    kv = r.standard_normal((S, D)).astype(np.float32)
    out = orc.attention(q, np.arange(S), kv_win=kv, win_pos0=0, window=W, scale=0.25)
    i = torch.arange(S)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    kvt = torch.from_numpy(kv.astype(np.float64))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, 0].astype(np.float64))[None, None], kvt, kvt,
        attn_mask=mask[None, None], scale=0.25)[0, 0].numpy()
    np.testing.assert_allclose(out[:, 0], ref, atol=1e-5)


def test_attention_sparse_all_ready_equals_hca(orc):
    """P8: a top-k that keeps every ready entry reproduces the dense HCA path."""
    q, kv, pool, z, t, _ = _attn_case(90)
    T = pool.shape[0]
    idx = np.full((len(t), T), -1, np.int32)
    for r in range(len(t)):
        R = brute.ready(int(t[r]), 4, T)
        idx[r, :R] = np.arange(R)
    kw = dict(kv_win=kv, win_pos0=0, window=6, pool=pool, m=4, sink=z, rope_dim=8,
              theta=1e4, scale=0.3)
    np.testing.assert_allclose(orc.attention(q, t, idx=idx, **kw),
                               orc.attention(q, t, idx=None, **kw), atol=1e-6)


def test_attention_empty_row_is_zero(orc):
    q = rng(95).standard_normal((2, 2, 16)).astype(np.float32)
    out = orc.attention(q, np.array([0, 5]), pool=np.zeros((3, 16), np.float32),
                        idx=np.full((2, 2), -1, np.int32), scale=0.25, m=4)
    assert np.all(out == 0)


def test_cache_state_is_causal_and_holds_the_last_tokens(orc):
    """The decode cache after `count` tokens ("DeepSeek-V4", section "Cache
    layers"): an entry, once its window has closed, never changes as tokens
    arrive (the compressor reads no token past its window); the buffer holds
    the raw rows of the last (1+overlap) m tokens; the window holds the last W
    tokens rotated at their positions (a rotation keeps each pair's length)."""
    r = np.random.default_rng(11)
    S, D, m, ov, R, W = 41, 16, 4, 1, 8, 6
    x = r.standard_normal((S, D)).astype(np.float32)
    g = r.standard_normal((S, D)).astype(np.float32)
    prev = None
    for count in range(S + 1):
        pool, rx, rg, win, rows, wrows = orc.cache_state(x, g, count=count, m=m, overlap=ov,
                                                         rope_dim=R, theta=1e4, W=W)
        assert pool.shape == (count // m, D)
        if prev is not None:
            assert np.array_equal(pool[:len(prev)], prev)
        prev = pool
        L = (1 + ov) * m
        assert rows == sorted(p % L for p in range(max(0, count - L), count))
        for p in range(max(0, count - L), count):
            assert np.array_equal(rx[p % L], x[p]) and np.array_equal(rg[p % L], g[p])
        for p in range(max(0, count - W), count):
            row = win[p % W]
            assert np.array_equal(row[:D - R], x[p, :D - R])
            # rotated at exactly its own position p (complex multiplication,
            # written independently of the oracle's rotation)
            np.testing.assert_allclose(row, brute.rope_complex(x[p], R, 1e4, p, +1),
                                       rtol=1e-5, atol=1e-5)
            pr = row[D - R:].reshape(-1, 2)
            px = x[p, D - R:].reshape(-1, 2)
            np.testing.assert_allclose(np.hypot(pr[:, 0], pr[:, 1]),
                                       np.hypot(px[:, 0], px[:, 1]), rtol=1e-6)
    # with no gate the entry is the window mean (as the compressor's own pin)
    pool = orc.cache_state(x, None, count=S, m=m, overlap=0, rope_dim=0, W=0)[0]
    np.testing.assert_allclose(pool, x[:S // m * m].reshape(-1, m, D).mean(1), rtol=1e-6,
                               atol=1e-6)
    # with no gate and RoPE, entry w is the mean of its (overlapping) window
    # rotated at w m: positions count from the sequence's first token
    pool = orc.cache_state(x, None, count=S, m=m, overlap=1, rope_dim=R, theta=1e4, W=0)[0]
    for w in range(S // m):
        lo = max(0, (w - 1) * m)
        ref = brute.rope_complex(x[lo:(w + 1) * m].astype(np.float64).mean(0), R, 1e4, w * m)
        np.testing.assert_allclose(pool[w], ref, rtol=1e-5, atol=1e-5)


# ----------------------------------------------------------------- output projection
def test_grouped_out_proj_is_block_diagonal_map(orc):
    """The grouped projection equals one dense map whose matrix holds the
    group maps on its diagonal blocks (zero elsewhere): group g reads only its
    own heads' columns and writes only its own rank slice."""
    r = rng(31)
    M, H, dv, G, rank, hidden = 7, 8, 6, 4, 5, 9
    Kg = H * dv // G
    o = r.standard_normal((M, H, dv))
    w_a = r.standard_normal((G, rank, Kg))
    w_b = r.standard_normal((hidden, G * rank))
    mid, out = orc.grouped_out_proj(o.reshape(M, H * dv), w_a, w_b)
    dense = scipy.linalg.block_diag(*[w_a[g] for g in range(G)])     # [G*rank, H*dv]
    np.testing.assert_allclose(mid, o.reshape(M, H * dv) @ dense.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, (o.reshape(M, H * dv) @ dense.T) @ w_b.T, rtol=1e-12,
                               atol=1e-12)
    # a head of group 1 changes only group 1's slice of mid
    o2 = o.copy()
    o2[:, H // G + 1, :] += 1.0
    mid2, _ = orc.grouped_out_proj(o2.reshape(M, H * dv), w_a, w_b)
    changed = np.any(np.abs(mid2 - mid) > 1e-9, axis=0).reshape(G, rank)
    assert changed[1].all() and not changed[[0, 2, 3]].any()


def test_grouped_out_proj_one_group_is_two_plain_products(orc):
    r = rng(32)
    o = r.standard_normal((5, 12))
    w_a = r.standard_normal((1, 4, 12))
    w_b = r.standard_normal((3, 4))
    mid, out = orc.grouped_out_proj(o, w_a, w_b)
    ref_mid = np.einsum("mc,jc->mj", o, w_a[0])
    np.testing.assert_allclose(mid, ref_mid, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, np.einsum("mj,nj->mn", ref_mid, w_b), rtol=1e-12, atol=1e-12)
    # bf16 storage of mid: the second product reads the rounded values
    mid_b, out_b = orc.grouped_out_proj(o, w_a, w_b, round_mid_bf16=True)
    assert np.array_equal(mid_b, orc.round_bf16(ref_mid.astype(np.float32)))
    np.testing.assert_allclose(out_b, mid_b @ w_b.T, rtol=1e-12, atol=1e-12)
    # the second product alone, from a given mid
    _, out_c = orc.grouped_out_proj(None, None, w_b, mid=mid_b)
    assert np.array_equal(out_c, out_b)
