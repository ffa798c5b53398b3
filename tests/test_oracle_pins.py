"""Pins of the fp64 oracle against things other than itself.

Each test ties an oracle function to a library routine, a closed form, brute
force on tiny inputs, an invariant, or a hand-worked case under
tests/golden/.  These run on the CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle import lighthouse as LH

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
with open(GOLD) as fh:
    HAND = json.load(fh)


def _num(v):
    if isinstance(v, str):
        assert v.startswith("ln")
        return math.log(float(v[2:]))
    return float(v)


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(v) for v in x]) if x and isinstance(x[0], list) else \
            np.array([_num(v) for v in x])
    return _num(x)


def sdpa64(q, K, V, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    q = torch.as_tensor(np.asarray(q), dtype=torch.float64)
    K = torch.as_tensor(np.asarray(K), dtype=torch.float64)
    V = torch.as_tensor(np.asarray(V), dtype=torch.float64)
    if q.dim() == 1:
        q = q[None]
    o = F.scaled_dot_product_attention(q[None, None], K[None, None], V[None, None],
                                       is_causal=causal)
    return o[0, 0].numpy()


# --------------------------------------------------------------- attention
@pytest.mark.parametrize("case", HAND["attention"])
def test_attend_hand_cases(case):
    o = oracle.attend(_arr(case["q"]), _arr(case["K"]), _arr(case["V"]), case["scale"])
    np.testing.assert_allclose(o, case["expect"], atol=1e-12)


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    for T, d in [(1, 8), (7, 16), (300, 64), (1000, 128)]:
        q = rng.standard_normal(d) * 2
        K = rng.standard_normal((T, d))
        V = rng.standard_normal((T, d))
        np.testing.assert_allclose(oracle.attend(q, K, V), sdpa64(q, K, V)[0],
                                   rtol=0, atol=1e-12)


def test_attend_weights_normalise():
    # constant values => output equals that constant: the weights sum to 1
    rng = np.random.default_rng(1)
    K = rng.standard_normal((500, 32)) * 3
    V = np.full((500, 32), 2.5)
    o = oracle.attend(rng.standard_normal(32) * 4, K, V)
    np.testing.assert_allclose(o, 2.5, atol=1e-12)


def test_attend_logsumexp_form():
    # second formula: o = sum_j exp(a_j - logsumexp(a)) v_j
    rng = np.random.default_rng(2)
    q, K, V = rng.standard_normal(16), rng.standard_normal((50, 16)), rng.standard_normal((50, 16))
    a = K @ q / 4.0
    lse = np.log(np.sum(np.exp(a - a.max()))) + a.max()
    np.testing.assert_allclose(oracle.attend(q, K, V), np.exp(a - lse) @ V, atol=1e-13)


def test_dense_causal_matches_sdpa():
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((40, 16)) for _ in range(3))
    o = oracle.dense_causal(Q, K, V)
    np.testing.assert_allclose(o, sdpa64(Q, K, V, causal=True), atol=1e-12)


# --------------------------------------------------------------- selectors
def test_topp_hand_cases():
    lg = _arr(HAND["topp"]["logits"])
    for c in HAND["topp"]["cases"]:
        s, m = oracle.select_topp(lg, c["p"], c["min_tokens"])
        assert s.tolist() == c["expect"], c


def test_topk_hand_cases():
    lg = _arr(HAND["topk"]["logits"])
    for c in HAND["topk"]["cases"]:
        s, _ = oracle.select_topk(lg, c["k"])
        assert s.tolist() == c["expect"], c


def _canon_mass(l, S):
    # sum over a canonical (sorted) order so equal multisets compare equal
    w = np.exp(np.asarray(l, np.float64) - np.max(l))
    return float(np.sum(np.sort(w[list(S)]))) / float(np.sum(np.sort(w)))


def _brute_topk(l, k):
    n = len(l)
    k = min(k, n)
    best = None
    for S in itertools.combinations(range(n), k):
        key = (sum(sorted(l[i] for i in S)), -sum(S))   # canonical order sum
        if best is None or key > best[0]:
            best = (key, S)
    return list(best[1])


def _brute_topp(l, p, m_min):
    n = len(l)
    if p >= 1:
        return list(range(n))
    for m in range(1, n + 1):
        cands = []
        for S in itertools.combinations(range(n), m):
            mass = _canon_mass(l, S)
            if mass >= p:
                cands.append((mass, -sum(S), S))
        if cands:
            break
    m = len(max(cands)[2])
    m = min(n, max(m, m_min))
    return _brute_topk(l, m)


def test_topk_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        l = rng.integers(-3, 4, n).astype(float)     # integer logits: many ties
        k = int(rng.integers(1, n + 2))
        s, _ = oracle.select_topk(l, k)
        assert s.tolist() == sorted(_brute_topk(l, k)), (l, k)


def test_topp_brute_force():
    rng = np.random.default_rng(5)
    checked = 0
    for trial in range(300):
        n = int(rng.integers(1, 10))
        l = rng.integers(-2, 3, n).astype(float) * 0.7
        p = float(rng.choice([0.3, 0.5, 0.62, 0.8, 0.9, 0.97, 1.0]))
        m_min = int(rng.integers(0, 3))
        if p < 1 and oracle.topp_margin(l, p) < 1e-9:
            continue                                      # exact-boundary draws
        s, _ = oracle.select_topp(l, p, m_min)
        assert s.tolist() == sorted(_brute_topp(l, p, m_min)), (l, p, m_min)
        checked += 1
    assert checked > 200


def test_topp_is_minimal_prefix():
    # the chosen prefix reaches p and one token fewer does not
    rng = np.random.default_rng(6)
    for _ in range(50):
        l = rng.standard_normal(400) * rng.uniform(0.2, 3)
        p = rng.uniform(0.2, 0.99)
        s, m = oracle.select_topp(l, p)
        w = np.exp(l - l.max())
        w /= w.sum()
        assert w[s].sum() >= p
        mass_sorted = np.sort(w)[::-1]
        assert mass_sorted[: m - 1].sum() < p


def test_topp_full_and_topk_full_select_everything():
    l = np.random.default_rng(7).standard_normal(64)
    assert oracle.select_topp(l, 1.0)[0].tolist() == list(range(64))
    assert oracle.select_topk(l, 64)[0].tolist() == list(range(64))
    assert oracle.select_topk(l, 1000)[0].tolist() == list(range(64))


# --------------------------------------------------------------- index
def test_index_identity_projector_is_plain_scaled_dot():
    # r = d and P = I: logits are q_pre . k_pre / sqrt(d)
    rng = np.random.default_rng(8)
    d, n = 16, 100
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((n, d))
    kk = oracle.index_keys(k, np.eye(d), "fp32")
    qq = oracle.index_query(q, np.eye(d))
    l = oracle.index_logits(qq, kk)
    # stored fp32 keys/queries: agreement to fp32 rounding
    np.testing.assert_allclose(l, (k @ q[0]) / 4.0, rtol=0, atol=2e-6)


def test_index_group_mean_is_mean_of_logits():
    rng = np.random.default_rng(9)
    qh = rng.standard_normal((4, 16))
    k = rng.standard_normal((50, 16))
    per_head = np.stack([k @ qh[h] / 4.0 for h in range(4)]).mean(axis=0)
    np.testing.assert_allclose(oracle.index_logits(qh, k), per_head, atol=1e-13)


def test_index_keys_rounding_is_bf16_rne():
    # stored index keys are exactly representable in bf16 and within half an ulp
    rng = np.random.default_rng(10)
    x = rng.standard_normal((200, 64))
    P = rng.standard_normal((16, 64)) / 8
    k = oracle.index_keys(x, P, "bf16")
    exact = x @ P.T
    as_bf16 = torch.tensor(k).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(k, as_bf16)
    assert np.all(np.abs(k - exact) <= 0.5 * oracle.bf16_ulp(exact) + 1e-300)


# --------------------------------------------------------------- local
def test_local_hand_cases():
    for c in HAND["local"]["cases"]:
        assert oracle.local_set(c["n"], c["sinks"], c["window"]).tolist() == c["expect"]


# --------------------------------------------------------------- RoPE
def test_rope_matches_complex_rotation_and_generator():
    rng = np.random.default_rng(11)
    d, base = 64, 1e4
    x = rng.standard_normal((10, d))
    pos = rng.integers(0, 100000, 10).astype(float)
    ours = oracle.rope_rotate(x, oracle.rope_angles(d, base, pos))
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    zr = z * np.exp(1j * pos[:, None] * theta)
    np.testing.assert_allclose(ours, np.concatenate([zr.real, zr.imag], 1), atol=1e-9)
    gen = workloads.apply_rope(torch.tensor(x), torch.tensor(pos), base).numpy()
    np.testing.assert_allclose(ours, gen, atol=1e-9)


def test_rope_invariants():
    rng = np.random.default_rng(12)
    d, base = 128, 5e5
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for t, j in [(0, 0), (5, 3), (70000, 123), (131071, 99999)]:
        rq = oracle.rope_rotate(q, oracle.rope_angles(d, base, t))
        rk = oracle.rope_rotate(k, oracle.rope_angles(d, base, j))
        rel = oracle.rope_rotate(k, oracle.rope_angles(d, base, j - t))
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-10
        np.testing.assert_allclose(rq @ rk, q @ rel, rtol=1e-9, atol=1e-9)


# --------------------------------------------------------------- summaries
def test_high_pair_counts():
    # cutoff theta_i*(span-1) > 1 at d=128, base 5e5: 21 pairs for 64-token
    # chunks, 14 for 16-token groups; at d=64, base 1e4: 15 and 10
    assert oracle.high_freq_pairs(128, 5e5, 64).sum() == 21
    assert oracle.high_freq_pairs(128, 5e5, 16).sum() == 14
    assert oracle.high_freq_pairs(64, 1e4, 64).sum() == 15
    assert oracle.high_freq_pairs(64, 1e4, 16).sum() == 10
    # high pairs are a prefix (frequencies fall with i)
    m = oracle.high_freq_pairs(128, 5e5, 64)
    assert not np.any(m[1:] & ~m[:-1])


def test_summary_constant_keys_dirichlet_closed_form():
    # all keys equal: high pairs give z e^{i theta m} D(theta) with the
    # Dirichlet kernel D = sin(S theta / 2) / (S sin(theta / 2)), low pairs
    # give z e^{i theta m}, m = start + (S-1)/2
    rng = np.random.default_rng(13)
    d, base, S, start = 64, 1e4, 64, 640
    k = rng.standard_normal(d)
    summ = oracle.chunk_summary(np.tile(k, (S, 1)), start, base)
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    m = start + (S - 1) / 2
    z = k[: d // 2] + 1j * k[d // 2:]
    D = np.sin(S * theta / 2) / (S * np.sin(theta / 2))
    high = theta * (S - 1) > 1
    expect = z * np.exp(1j * theta * m) * np.where(high, D, 1.0)
    np.testing.assert_allclose(summ, np.concatenate([expect.real, expect.imag]), atol=1e-9)


def test_summary_all_high_is_mean_rotated_key():
    # when every pair is high, q . S equals the mean over the chunk of
    # q . RoPE(k_j, j) (linearity), with RoPE from the input generator
    rng = np.random.default_rng(14)
    d, S, start, base = 32, 64, 128, 10.0
    assert oracle.high_freq_pairs(d, base, S).all()
    K = rng.standard_normal((S, d))
    q = rng.standard_normal(d)
    summ = oracle.chunk_summary(K, start, base)
    rot = workloads.apply_rope(torch.tensor(K), torch.arange(start, start + S), base).numpy()
    np.testing.assert_allclose(q @ summ, np.mean(rot @ q), atol=1e-10)


def test_summary_span_one_is_rotated_key():
    rng = np.random.default_rng(15)
    K = rng.standard_normal((1, 64))
    s = oracle.chunk_summary(K, 777, 1e4)
    rot = workloads.apply_rope(torch.tensor(K), torch.tensor([777.0]), 1e4).numpy()[0]
    np.testing.assert_allclose(s, rot, atol=1e-10)


def test_summary_shift_equivariance():
    # moving a chunk by D positions rotates its summary by D*theta
    rng = np.random.default_rng(16)
    d, base, S = 128, 5e5, 64
    K = rng.standard_normal((S, d))
    a = oracle.chunk_summary(K, 64 * 3, base)
    b = oracle.chunk_summary(K, 64 * 1000, base)
    np.testing.assert_allclose(oracle.rope_rotate(a, oracle.rope_angles(d, base, 64 * 997)), b,
                               atol=1e-9)


def test_summaries_cover_complete_spans():
    rng = np.random.default_rng(17)
    K = rng.standard_normal((64 * 5 + 10, 64))
    cs = oracle.chunk_summaries(K, 64, 1e4, None)
    gs = oracle.group_summaries(K, 16, 1e4, None)
    assert cs.shape == (5, 64) and gs.shape == (20, 64)
    np.testing.assert_allclose(cs[2], oracle.chunk_summary(K[128:192], 128, 1e4))
    np.testing.assert_allclose(gs[7], oracle.chunk_summary(K[112:128], 112, 1e4))


# --------------------------------------------------------------- routing
def test_route_hand_case():
    c = HAND["route"]
    d = c["d"]
    nc, ng = c["n"] // c["chunk"], c["n"] // c["group"]
    cs = np.zeros((nc, d))
    gs = np.zeros((ng, d))
    for k, v in c["chunk_dim0"].items():
        cs[int(k), 0] = v
    for k, v in c["group_dim0"].items():
        gs[int(k), 0] = v
    toks, info = oracle.route_token_list(np.array(c["q_heads"]), cs, gs, c["n"], c["chunk"],
                                         c["group"], c["top_chunks"], c["top_groups"],
                                         c["sink_chunks"], c["local_chunks"])
    assert toks.tolist() == c["expect"]


def test_route_everything_is_dense():
    # every candidate chunk and every group routed => all n tokens visible,
    # and the decode output is dense attention over the whole cache
    cfg = workloads.HGA_64K.with_(batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64,
                                  n_ctx=64 * 40 + 17, top_chunks=1000, top_groups=4)
    inp = {k: (v.numpy().astype(np.float64) if torch.is_tensor(v) else v)
           for k, v in workloads.decode_inputs(cfg, 3).items()}
    sets = oracle.decode_token_sets(cfg, inp)
    for T in sets.values():
        assert T.tolist() == list(range(cfg.n_ctx))
    out = oracle.decode_step(cfg, inp, sets=sets)
    for (b, h), o in out.items():
        g = h // cfg.gqa
        ref = sdpa64(inp["q"][b, h], inp["k_cache"][b, g], inp["v_cache"][b, g])[0]
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_route_short_context_has_no_candidates():
    cs = np.zeros((3, 4))
    toks, info = oracle.route_token_list(np.ones((1, 4)), cs, np.zeros((12, 4)), 64 * 3 + 5)
    assert toks.tolist() == list(range(64 * 3 + 5)) and info["chunks"].size == 0


# --------------------------------------------------------------- decode
def _np_inputs(cfg, seed, **kw):
    return {k: (v.numpy().astype(np.float64) if torch.is_tensor(v) else v)
            for k, v in workloads.decode_inputs(cfg, seed, **kw).items()}


@pytest.mark.parametrize("mode", ["p1", "kfull"])
def test_retrieval_full_selection_is_dense(mode):
    cfg = workloads.TINY.with_(n_ctx=700)
    cfg = cfg.with_(top_p=1.0) if mode == "p1" else cfg.with_(top_k=700)
    inp = _np_inputs(cfg, 1)
    out = oracle.decode_step(cfg, inp, groups=[(0, 0), (0, 1)])
    for (b, h), o in out.items():
        ref = sdpa64(inp["q"][b, h], inp["k_cache"][b, h], inp["v_cache"][b, h])[0]
        np.testing.assert_allclose(o, ref, atol=1e-12)


@pytest.mark.parametrize("sinks,window", [(4, 5000), (700, 0), (0, 700)])
def test_local_full_window_is_dense(sinks, window):
    cfg = workloads.TINY.with_(n_ctx=700, sinks=sinks, window=window)
    inp = _np_inputs(cfg, 2)
    out = oracle.decode_step(cfg, inp, groups=[(0, 2), (0, 3)])
    for (b, h), o in out.items():
        ref = sdpa64(inp["q"][b, h], inp["k_cache"][b, h], inp["v_cache"][b, h])[0]
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_local_window_equals_sdpa_on_slice():
    cfg = workloads.TINY.with_(n_ctx=900)
    inp = _np_inputs(cfg, 4)
    out = oracle.decode_step(cfg, inp, groups=[(0, 2)])
    T = np.r_[0:4, 900 - 128:900]
    ref = sdpa64(inp["q"][0, 2], inp["k_cache"][0, 2][T], inp["v_cache"][0, 2][T])[0]
    np.testing.assert_allclose(out[(0, 2)], ref, atol=1e-12)


def test_needles_are_retrieved_on_tiny():
    # sanity of the workload: the planted needles rank at the top of the index
    cfg = workloads.TINY
    inp = _np_inputs(cfg, 0)
    sets = oracle.decode_token_sets(cfg, inp, groups=[(0, 0), (0, 1)])
    for h in (0, 1):
        nd = inp["needles"][(0, h)].numpy()
        assert np.isin(nd, sets[(0, h)]).mean() >= 0.75


# --------------------------------------------------------------- pyramid
def test_pyramid_levels_are_span_means():
    rng = np.random.default_rng(18)
    X = rng.standard_normal((256, 8))
    lv = oracle.pyramid_levels(X, 3, 4, None)
    assert lv[0].shape == (64, 8) and lv[1].shape == (16, 8)
    for j in (0, 5, 15):
        np.testing.assert_allclose(lv[1][j], X[16 * j:16 * j + 16].mean(0), atol=1e-13)
    for j in (0, 33, 63):
        np.testing.assert_allclose(lv[0][j], X[4 * j:4 * j + 4].mean(0), atol=1e-13)


def test_pyramid_levels_exact_for_factor_three():
    """p = 3: an entry whose 9 rows sum to zero is exactly zero, though its
    three children (k/3 each) are not representable."""
    X = np.zeros((27, 2))
    X[:9, 0] = np.array([-7, -4, -7, 0, 8, 5, 4, 4, -3]) / 8   # children sums -18, 13, 5 (x 1/8)
    X[9:18, 1] = [0.125] * 9
    lv = oracle.pyramid_levels(X, 3, 3, None)
    assert lv[1][0, 0] == 0.0 and lv[1][1, 1] == 0.125
    assert lv[0][0, 0] == -0.75 and lv[0][1, 0] == 13 / 24


def test_pyramid_scores_inherit_span_max():
    rng = np.random.default_rng(19)
    Q, K = rng.standard_normal((256, 8)), rng.standard_normal((256, 8))
    sc = oracle.pyramid_scores(Q, K, 3, 4)
    s0 = np.array([Q[i] @ Q[i] + K[i] @ K[i] for i in range(256)])
    np.testing.assert_allclose(sc[0], s0, atol=1e-12)
    for lvl, span in ((1, 4), (2, 16)):
        brute = np.array([sc[0][j * span:(j + 1) * span].max() for j in range(256 // span)])
        np.testing.assert_array_equal(sc[lvl], brute)


def test_pyramid_select_hand_case():
    c = HAND["pyramid_select"]
    s0 = np.array(c["s0"], float)
    s1 = s0.reshape(-1, c["factor"]).max(1)
    for blk, exp in c["expect"].items():
        got = oracle.block_select([s0, s1], int(blk), c["N"], c["levels"], c["factor"],
                                  c["q_block"], c["top_k"])
        assert sorted(got.tolist()) == exp, blk


def test_pyramid_select_brute_force():
    rng = np.random.default_rng(20)
    N, L, p, qb = 64, 3, 2, 8
    for trial in range(20):
        s0 = rng.integers(0, 6, N).astype(float)
        sc = [s0, s0.reshape(-1, 2).max(1), s0.reshape(-1, 4).max(1)]
        K = int(rng.integers(1, 20))
        offs = LH.level_offsets(N, L, p)
        for blk in range(N // qb):
            vis = oracle.visible_entries(blk, N, L, p, qb)
            ranked = sorted(vis, key=lambda e: (-sc[e[0]][e[1]], e[0], e[1]))[:K]
            exp = sorted(offs[a] + b for a, b in ranked)
            got = oracle.block_select(sc, blk, N, L, p, qb, K)
            assert sorted(got.tolist()) == exp
            # visibility: every chosen span ends before the block
            for a, b in ranked:
                assert (b + 1) * p ** a <= qb * blk


def test_pyramid_one_level_full_budget_is_dense_causal():
    # L = 1 and K >= N: every block sees all earlier tokens plus its own
    # causal part, i.e. ordinary causal attention
    rng = np.random.default_rng(21)
    N, d = 96, 16
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    out, *_ = oracle.prefill(Q, K, V, levels=1, factor=4, q_block=16, top_k=N, store=None)
    np.testing.assert_allclose(out, sdpa64(Q, K, V, causal=True), atol=1e-12)


def test_prefill_block_matches_sdpa_on_gathered_rows():
    rng = np.random.default_rng(22)
    N, d = 128, 16
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    out, kc, vc, sels = oracle.prefill(Q, K, V, 3, 2, 16, 10, store=None, blocks=[5])
    sel = sels[5]
    Ks = LH.entry_rows(sel, K, kc, N, 3, 2)
    Vs = LH.entry_rows(sel, V, vc, N, 3, 2)
    for i in (80, 87, 95):
        Kt = np.concatenate([Ks, K[80:i + 1]])
        Vt = np.concatenate([Vs, V[80:i + 1]])
        np.testing.assert_allclose(out[i], sdpa64(Q[i], Kt, Vt)[0], atol=1e-12)


# ---------------------------------------------------------------- coarse queries (symmetric 2A/2C)
def _span_means(X, levels, factor):
    """Coarse levels 1 .. L-1 of X as plain reshaped means (no rounding)."""
    X = np.asarray(X, np.float64)
    return [X.reshape(-1, factor ** l, X.shape[1]).mean(axis=1) for l in range(1, levels)]


def test_coarse_queries_are_sdpa_on_gathered_rows():
    """Each coarse query of a block: torch SDPA over the block's selected rows
    followed by its own level's rows of the block up to itself."""
    rng = np.random.default_rng(31)
    N, d, L, p, qb = 128, 16, 3, 2, 16
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    qc, kc, vc = (_span_means(X, L, p) for X in (Q, K, V))
    sc = oracle.pyramid_scores(Q, K, L, p)
    for blk in (0, 3, 7):
        sel = oracle.block_select(sc, blk, N, L, p, qb, 12)
        Ks = LH.entry_rows(sel, K, kc, N, L, p)
        Vs = LH.entry_rows(sel, V, vc, N, L, p)
        outs = oracle.coarse_block(qc, kc, vc, K, V, sel, blk, qb, L, p)
        for lvl in (1, 2):
            lo = qb * blk // p ** lvl
            n = qb // p ** lvl
            assert outs[lvl - 1].shape == (n, d)
            for j in range(n):
                Kt = np.concatenate([Ks, kc[lvl - 1][lo:lo + j + 1]])
                Vt = np.concatenate([Vs, vc[lvl - 1][lo:lo + j + 1]])
                np.testing.assert_allclose(outs[lvl - 1][j], sdpa64(qc[lvl - 1][lo + j], Kt, Vt)[0],
                                           atol=1e-12)


def test_coarse_queries_of_first_block_are_causal_sdpa_per_level():
    """Block 0 sees nothing before it: each level's coarse queries are plain
    causal attention over that level's rows of the block; the first entry of
    each level sees only itself."""
    rng = np.random.default_rng(32)
    N, d, L, p, qb = 64, 8, 3, 4, 32
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    qc, kc, vc = (_span_means(X, L, p) for X in (Q, K, V))
    outs = oracle.coarse_block(qc, kc, vc, K, V, np.zeros(0, np.int64), 0, qb, L, p)
    for lvl in (1, 2):
        n = qb // p ** lvl
        ref = sdpa64(qc[lvl - 1][:n], kc[lvl - 1][:n], vc[lvl - 1][:n], causal=True)
        np.testing.assert_allclose(outs[lvl - 1], ref, atol=1e-12)
        np.testing.assert_allclose(outs[lvl - 1][0], vc[lvl - 1][0], atol=1e-14)


def test_coarse_queries_constant_values_and_list_order():
    """Equal value rows give that row for every coarse query; the order of
    the selected list does not matter (attention over a set)."""
    rng = np.random.default_rng(33)
    N, d, L, p, qb = 96, 8, 2, 4, 16
    Q, K = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    c = rng.standard_normal(d)
    V = np.tile(c, (N, 1))
    qc, kc, vc = (_span_means(X, L, p) for X in (Q, K, V))
    sc = oracle.pyramid_scores(Q, K, L, p)
    sel = oracle.block_select(sc, 4, N, L, p, qb, 9)
    outs = oracle.coarse_block(qc, kc, vc, K, V, sel, 4, qb, L, p)
    np.testing.assert_allclose(outs[0], np.tile(c, (qb // p, 1)), atol=1e-12)
    V = rng.standard_normal((N, d))
    vc = _span_means(V, L, p)
    a = oracle.coarse_block(qc, kc, vc, K, V, sel, 4, qb, L, p)[0]
    b = oracle.coarse_block(qc, kc, vc, K, V, sel[::-1].copy(), 4, qb, L, p)[0]
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_prefill_coarse_scatters_each_block_to_its_own_slots():
    """The pipeline writes a block's coarse outputs to the rows its entries
    occupy in each level and nothing else; with L = 1 there are none."""
    rng = np.random.default_rng(34)
    N, d, L, p, qb, K = 128, 8, 3, 2, 16, 10
    Q, K_, V = (rng.standard_normal((N, d)) for _ in range(3))
    outs = oracle.prefill_coarse(Q, K_, V, L, p, qb, K, store=None, blocks=[2, 5])
    qc, kc, vc = (_span_means(X, L, p) for X in (Q, K_, V))
    sc = oracle.pyramid_scores(Q, K_, L, p)
    for lvl in (1, 2):
        span = p ** lvl
        done = np.zeros(N // span, bool)
        for blk in (2, 5):
            sel = oracle.block_select(sc, blk, N, L, p, qb, K)
            ref = oracle.coarse_block(qc, kc, vc, K_, V, sel, blk, qb, L, p)[lvl - 1]
            lo = qb * blk // span
            np.testing.assert_allclose(outs[lvl - 1][lo:lo + qb // span], ref, atol=1e-12)
            done[lo:lo + qb // span] = True
        assert np.isnan(outs[lvl - 1][~done]).all() and not np.isnan(outs[lvl - 1][done]).any()
    assert oracle.prefill_coarse(Q, K_, V, 1, p, qb, K, store=None) == []


# ---------------------------------------------------------------- three-level pyramid, by hand
def _hand_value(v):
    """Numbers of the hand fixtures: plain, a fraction "a/b", or 2 sqrt(2) ln 2."""
    if isinstance(v, str):
        if v == "2sqrt2ln2":
            return 2.0 * np.sqrt(2.0) * np.log(2.0)
        a, b = v.split("/")
        return float(a) / float(b)
    return float(v)


def test_pyramid_three_levels_hand_fixture():
    """Lighthouse Attention summary, 2A-2C, on a 16-token three-level pyramid
    worked by hand (tests/golden/pyramid_three_levels_hand.json): the level
    scores with max inheritance, the joint top-K with the level tie-break,
    the rows of level-0, level-1 and level-2 entries, and the outputs (exact
    rationals) of queries in both blocks."""
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "pyramid_three_levels_hand.json")))
    N, d, L, p, qb = fx["N"], fx["d"], fx["levels"], fx["factor"], fx["q_block"]
    rows = {}
    for name in ("Q", "K", "V"):
        X = np.zeros((N, d))
        for i, r in fx.get(f"{name}_rows", {}).items():
            X[int(i)] = [_hand_value(v) for v in r]
        rows[name] = X
    Q, K, V = rows["Q"], rows["K"], rows["V"]
    sc = oracle.pyramid_scores(Q, K, L, p)
    for lvl, want in enumerate(("level0", "level1", "level2")):
        exp = fx["expect_scores_before_8"][want]
        np.testing.assert_allclose(sc[lvl][:len(exp)], exp, atol=1e-12)
    kc = oracle.pyramid_levels(K, L, p, None)
    vc = oracle.pyramid_levels(V, L, p, None)
    for case in fx["cases"]:
        sel = oracle.block_select(sc, 1, N, L, p, qb, case["top_k"])
        assert sel.tolist() == case["block1_ids"]
        np.testing.assert_allclose(LH.entry_rows(sel, K, kc, N, L, p), case["block1_K"], atol=1e-12)
        np.testing.assert_allclose(LH.entry_rows(sel, V, vc, N, L, p), case["block1_V"], atol=1e-12)
        out, _, _, _ = oracle.prefill(Q, K, V, L, p, qb, case["top_k"], store=None)
        for i, want in case["out"].items():
            np.testing.assert_allclose(out[int(i)], [_hand_value(v) for v in want], atol=1e-12)


# --------------------------------------------------------------- per-head selection
def _split_groups(cfg, inp):
    """The same step with every query head given a KV group of its own (the
    group's keys, values, pre-RoPE keys and projector repeated G times)."""
    G = cfg.gqa
    inp2 = dict(inp)
    for k in ("k_pre", "k_cache", "v_cache", "proj"):
        inp2[k] = np.repeat(inp[k], G, axis=1 if k != "proj" else 0)
    return cfg.with_(n_kv_heads=cfg.n_q_heads), inp2


@pytest.mark.parametrize("which", ["topp", "topk", "routed"])
def test_per_head_sets_equal_groups_of_one(which):
    # per-query-head mode under GQA (G = 4) against the group rule on a
    # layout where each query head owns a copy of its KV group: sets and
    # outputs must agree head by head
    base = workloads.TINY.with_(n_q_heads=8, n_kv_heads=2, n_ctx=1500, n_ret_q_heads=4,
                                needles_per_head=8)
    cfg = {"topp": base, "topk": base.with_(top_k=100),
           "routed": workloads.HGA_64K.with_(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                             n_ctx=64 * 30 + 9, top_chunks=5,
                                             needles_per_head=4)}[which]
    inp = _np_inputs(cfg, 11)
    cfg2, inp2 = _split_groups(cfg, inp)
    per_head = oracle.decode_token_sets_per_head(cfg, inp)
    groups = oracle.decode_token_sets(cfg2, inp2)
    assert per_head.keys() == groups.keys()
    differs = 0
    for key in per_head:
        assert per_head[key].tolist() == groups[key].tolist()
    G = cfg.gqa
    for h in range(cfg.n_q_heads):        # heads of one group pick different sets
        differs += per_head[(0, h)].tolist() != per_head[(0, (h // G) * G)].tolist()
    assert differs > 0
    o1 = oracle.decode_step(cfg, inp, per_head=True)
    o2 = oracle.decode_step(cfg2, inp2)
    for key in o1:
        np.testing.assert_allclose(o1[key], o2[key], atol=1e-12)


def test_per_head_equals_group_mode_without_gqa():
    cfg = workloads.TINY
    inp = _np_inputs(cfg, 12)
    a = oracle.decode_token_sets_per_head(cfg, inp)
    b = oracle.decode_token_sets(cfg, inp)
    assert {k: v.tolist() for k, v in a.items()} == {k: v.tolist() for k, v in b.items()}


def test_per_head_topk_brute_force():
    # each retrieval head's own top-k by brute force over its own logits
    cfg = workloads.TINY.with_(n_q_heads=4, n_kv_heads=1, n_ret_q_heads=4, n_ctx=300, top_k=7,
                               r=16)
    li = workloads.lattice_index_inputs(cfg, 5)
    inp = {"head_kind": li["head_kind"].numpy()}
    k_idx = li["k_idx"].numpy().astype(np.float64)
    q_idx = li["q_idx"].numpy().astype(np.float64)
    sets = oracle.decode_token_sets_per_head(cfg, inp, k_idx=k_idx, q_idx=q_idx)
    for h in range(4):
        lg = [float(np.dot(q_idx[0, h], k_idx[0, 0, j])) / 4.0 for j in range(300)]
        best = sorted(range(300), key=lambda j: (-lg[j], j))[:7]
        assert sets[(0, h)].tolist() == sorted(best)


# --------------------------------------------------------------- head-split prefill
def _qkv(seed, N=260, d=16):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((N, d)) for _ in range(3))


@pytest.mark.parametrize("kind,sinks,window", [(0, 4, 260), (0, 0, 1000), (0, 260, 0),
                                               (0, 300, 5), (1, 4, 16), (2, 0, 0)])
def test_head_prefill_reduces_to_dense_causal(kind, sinks, window):
    # window >= n (or sinks covering everything) on a local head, and every
    # retrieval or routed head: torch's causal attention
    Q, K, V = _qkv(20)
    o = oracle.head_prefill_rows(Q, K, V, kind, sinks, window, np.arange(260))
    np.testing.assert_allclose(o, sdpa64(Q, K, V, causal=True), atol=1e-12)


def test_head_prefill_window_one_is_own_value():
    Q, K, V = _qkv(21)
    o = oracle.head_prefill_rows(Q, K, V, 0, 0, 1, np.arange(260))
    np.testing.assert_allclose(o, V, atol=1e-15)


def test_head_prefill_one_sink_one_window_closed_form():
    # query i >= 1 sees keys 0 and i: a two-term softmax
    Q, K, V = _qkv(22)
    rows = np.arange(260)
    o = oracle.head_prefill_rows(Q, K, V, 0, 1, 1, rows)
    np.testing.assert_allclose(o[0], V[0], atol=1e-15)
    for i in rows[1:]:
        a0, ai = Q[i] @ K[0] / 4.0, Q[i] @ K[i] / 4.0
        w0 = 1.0 / (1.0 + math.exp(ai - a0))
        np.testing.assert_allclose(o[i], w0 * V[0] + (1 - w0) * V[i], atol=1e-13)


@pytest.mark.parametrize("window", [1, 7, 64])
def test_head_prefill_pure_window_is_sdpa_on_slice(window):
    Q, K, V = _qkv(23)
    o = oracle.head_prefill_rows(Q, K, V, 0, 0, window, np.arange(260))
    for i in range(260):
        lo = max(0, i - window + 1)
        np.testing.assert_allclose(o[i], sdpa64(Q[i], K[lo:i + 1], V[lo:i + 1])[0], atol=1e-12)


@pytest.mark.parametrize("sinks,window", [(4, 32), (3, 1), (40, 17)])
def test_head_prefill_sinks_and_window_masked_sdpa(sinks, window):
    # torch's attention with a boolean mask written from key distances
    Q, K, V = _qkv(24)
    N = 260
    mask = torch.zeros(N, N, dtype=torch.bool)
    for i in range(N):
        for j in range(i + 1):
            mask[i, j] = j < sinks or (i - j) < window
    qt, kt, vt = (torch.as_tensor(x)[None, None] for x in (Q, K, V))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None])[0, 0].numpy()
    o = oracle.head_prefill_rows(Q, K, V, 0, sinks, window, np.arange(N))
    np.testing.assert_allclose(o, ref, atol=1e-12)


@pytest.mark.parametrize("N,sinks,window", [(10, 2, 3), (300, 4, 64), (50, 60, 0), (77, 0, 5)])
def test_visible_pairs_closed_form(N, sinks, window):
    # |[0, min(s, i+1))| + |[max(0, i-w+1), i]| - their overlap, summed
    total = 0
    for i in range(N):
        a = min(sinks, i + 1)
        lo = max(0, i - window + 1)
        wcount = (i + 1 - lo) if window > 0 else 0
        over = max(0, a - lo) if window > 0 else 0
        total += a + wcount - over
    assert oracle.visible_pairs(N, 0, sinks, window) == total
    assert oracle.visible_pairs(N, 1, sinks, window) == N * (N + 1) // 2


# --------------------------------------------------------------- HGA chunked prefill
def _hga_prefill_case(seed, n=16 * 13 + 5, d=16, G=2, chunk=16, group=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, n, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    cs = rng.standard_normal((n // chunk, d))
    gs = rng.standard_normal((n // group, d))
    return q, K, V, cs, gs


def _hga_prefill_all(q, K, V, cs, gs, n, chunk, group, **kw):
    out = np.empty((q.shape[0], n, q.shape[2]))
    for blk in range((n + chunk - 1) // chunk):
        rows = np.arange(blk * chunk, min(n, (blk + 1) * chunk))
        lst, _ = oracle.route_prefill_block(q[:, rows].reshape(-1, q.shape[2]), cs, gs, blk, n,
                                            chunk, group, **kw)
        for h in range(q.shape[0]):
            out[h, rows] = oracle.route_prefill_rows(q[h], K, V, lst, blk, chunk, rows)
    return out


@pytest.mark.parametrize("kw", [
    dict(top_chunks=100, top_groups=4, sink_chunks=2, local_chunks=1),   # everything routed
    dict(top_chunks=1, top_groups=1, sink_chunks=0, local_chunks=100),   # everything local
    dict(top_chunks=1, top_groups=1, sink_chunks=100, local_chunks=0),   # everything a sink
])
def test_hga_prefill_keeping_everything_is_dense_causal(kw):
    n, chunk, group = 16 * 13 + 5, 16, 4
    q, K, V, cs, gs = _hga_prefill_case(30)
    out = _hga_prefill_all(q, K, V, cs, gs, n, chunk, group, **kw)
    for h in range(q.shape[0]):
        np.testing.assert_allclose(out[h], sdpa64(q[h], K, V, causal=True), atol=1e-12)


def test_hga_prefill_lists_brute_force():
    # the block's chunk-level query is the mean of its rows over the group's
    # heads; candidates are the complete chunks in [sinks, block - local);
    # top chunks, then top groups, by sorting (score desc, index asc)
    n, chunk, group = 16 * 13 + 5, 16, 4
    gpc = chunk // group
    q, K, V, cs, gs = _hga_prefill_case(31)
    kw = dict(top_chunks=3, top_groups=2, sink_chunks=1, local_chunks=2)
    for blk in range((n + chunk - 1) // chunk):
        rows = np.arange(blk * chunk, min(n, (blk + 1) * chunk))
        qr = q[:, rows].reshape(-1, q.shape[2])
        lst, _ = oracle.route_prefill_block(qr, cs, gs, blk, n, chunk, group, **kw)
        qbar = qr.sum(axis=0) / len(qr)
        cand = list(range(1, max(1, blk - 2)))
        top = sorted(cand, key=lambda c: (-float(qbar @ cs[c]), c))[:3]
        expect = set(range(0, min(1, blk) * chunk))
        expect |= set(range(max(1, blk - 2) * chunk, blk * chunk))
        for c in top:
            grp = sorted(range(c * gpc, (c + 1) * gpc), key=lambda gi: (-float(qbar @ gs[gi]), gi))[:2]
            for gi in grp:
                expect |= set(range(gi * group, (gi + 1) * group))
        assert lst.tolist() == sorted(expect), blk


def test_hga_prefill_rows_are_attention_over_list_and_causal_block():
    n, chunk, group = 16 * 13 + 5, 16, 4
    q, K, V, cs, gs = _hga_prefill_case(32)
    blk = 11
    rows = np.arange(blk * chunk, (blk + 1) * chunk)
    lst, _ = oracle.route_prefill_block(q[:, rows].reshape(-1, 16), cs, gs, blk, n, chunk, group,
                                        top_chunks=2, top_groups=1, sink_chunks=1, local_chunks=1)
    out = oracle.route_prefill_rows(q[0], K, V, lst, blk, chunk, rows)
    for r, i in enumerate(rows):
        T = np.r_[lst, blk * chunk:i + 1]
        np.testing.assert_allclose(out[r], sdpa64(q[0, i], K[T], V[T])[0], atol=1e-12)


# --------------------------------------------------------------- S2O early stop
def test_s2o_order_brute_force():
    rng = np.random.default_rng(40)
    lg = rng.integers(-3, 4, 50).astype(np.float64)       # many ties
    cand = rng.choice(50, 30, replace=False)
    got = oracle.s2o_order(lg, cand)
    assert got.tolist() == sorted(cand.tolist(), key=lambda j: (-lg[j], j))


def _s2o_case(seed, n=700, d=16):
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    init = np.r_[0:4, n - 32:n]
    order = rng.permutation(n - 36) + 4                     # every non-init token, shuffled
    return q, K, V, init, order


def test_s2o_tau_zero_keeps_everything():
    q, K, V, init, order = _s2o_case(41)
    o, nb = oracle.s2o_head(q, K, V, init, order, 0.0)
    assert nb == -(-len(order) // 64)
    ref = sdpa64(q, K, V)[0]                                 # init + all candidates = every token
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_s2o_huge_tau_keeps_one_block():
    q, K, V, init, order = _s2o_case(42)
    o, nb = oracle.s2o_head(q, K, V, init, order, 1e30)
    assert nb == 1
    T = np.r_[init, order[:64]]
    np.testing.assert_allclose(o, sdpa64(q, K[T], V[T])[0], atol=1e-12)


def test_s2o_stop_hand_case():
    # scale 1, q = e0, scores set on dim 0: the first pass is one token of
    # score 0 (mass 1); blocks of 64 equal scores x_i add 64 e^{x_i}:
    #   block 0: x = 0              -> gain 64 / 1          = 64   (go on, mass 65)
    #   block 1: x = ln(65/128)     -> gain 32.5 / 65       = 0.5  (go on, mass 97.5)
    #   block 2: x = ln(97.5/320)   -> gain 19.5 / 97.5     = 0.2  (< 0.3: stop, kept)
    #   block 3: never visited
    d = 4
    xs = [0.0, math.log(65 / 128), math.log(97.5 / 320), 5.0]
    K = np.zeros((1 + 64 * 4, d))
    V = np.zeros((1 + 64 * 4, d))
    for i, x in enumerate(xs):
        K[1 + 64 * i:1 + 64 * (i + 1), 0] = x
        V[1 + 64 * i:1 + 64 * (i + 1), 1] = i + 1
    q = np.eye(d)[0]
    order = np.arange(1, 1 + 64 * 4)
    o, nb = oracle.s2o_head(q, K, V, np.array([0]), order, 0.3, scale=1.0)
    assert nb == 3
    # weights: init 1, block masses 64, 32.5, 19.5 (total 117)
    expect = (64 * 1 + 32.5 * 2 + 19.5 * 3) / 117.0
    np.testing.assert_allclose(o, [0.0, expect, 0.0, 0.0], atol=1e-12)


def test_s2o_blocks_shrink_as_tau_grows():
    q, K, V, init, order = _s2o_case(43)
    nbs = [oracle.s2o_head(q, K, V, init, order, tau)[1] for tau in (0.0, 1e-4, 1e-3, 1e-2, 0.1, 1.0)]
    assert all(a >= b for a, b in zip(nbs, nbs[1:])) and nbs[0] > nbs[-1]


# ---------------------------------------------------------------- pyramid prefill backward
def _autograd_grads(Q, K, V, dO, sels, L, p, qb):
    """Gradients of sum(O * dO) by torch autograd (fp64, CPU) through a
    dense masked restatement of the forward: the coarse levels as means of
    level-0 rows, each block's gathered rows by index, a -inf mask, softmax."""
    N, d = Q.shape
    tQ, tK, tV = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))

    def flat(X):
        parts = [X]
        for lvl in range(1, L):
            span = p ** lvl
            m = N // span
            parts.append(X[: m * span].reshape(m, span, d).mean(dim=1))
        return torch.cat(parts)

    Kf, Vf = flat(tK), flat(tV)
    outs = []
    for b in range((N + qb - 1) // qb):
        lo, hi = qb * b, min(N, qb * b + qb)
        idx = torch.tensor(np.asarray(sels[b], np.int64), dtype=torch.long)
        Kt = torch.cat([Kf[idx], tK[lo:hi]])
        Vt = torch.cat([Vf[idx], tV[lo:hi]])
        a = (tQ[lo:hi] @ Kt.T) / math.sqrt(d)
        n = len(idx)
        mask = torch.zeros_like(a, dtype=torch.bool)
        mask[:, n:] = torch.triu(torch.ones(hi - lo, hi - lo, dtype=torch.bool), diagonal=1)
        a = a.masked_fill(mask, float("-inf"))
        outs.append(torch.softmax(a, dim=1) @ Vt)
    O = torch.cat(outs)
    (O * torch.tensor(dO)).sum().backward()
    return tQ.grad.numpy(), tK.grad.numpy(), tV.grad.numpy()


@pytest.mark.parametrize("shape", [(64, 8, 3, 2, 8, 5), (96, 16, 2, 4, 16, 9),
                                   (80, 8, 3, 2, 16, 40), (48, 4, 1, 4, 16, 48)])
def test_pyramid_backward_matches_autograd(shape):
    """Lighthouse Attention summary, 2B-2C: gradients flow through the
    gather, the attention and the scatter only.  The oracle's hand-written
    backward against torch autograd of the same forward (selection held
    fixed, coarse levels unrounded), ragged last block included."""
    N, d, L, p, qb, K_ = shape
    rng = np.random.default_rng(N + L)
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    _, _, _, sels = oracle.prefill(Q, K, V, L, p, qb, K_, store=None)
    got = oracle.prefill_grads(Q, K, V, dO, L, p, qb, K_, store=None, sels=sels)
    ref = _autograd_grads(Q, K, V, dO, sels, L, p, qb)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, atol=1e-11, rtol=1e-10)


def test_pyramid_backward_finite_differences():
    """Central differences of sum(O * dO) over single coordinates of Q, K
    and V (selection fixed, unrounded levels) against the oracle's
    gradients: brute force on a tiny pyramid."""
    N, d, L, p, qb, K_ = 16, 3, 3, 2, 4, 3
    rng = np.random.default_rng(5)
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    _, _, _, sels = oracle.prefill(Q, K, V, L, p, qb, K_, store=None)
    gQ, gK, gV = oracle.prefill_grads(Q, K, V, dO, L, p, qb, K_, store=None, sels=sels)

    def loss(Q_, K_, V_):
        kc = oracle.pyramid_levels(K_, L, p, None)
        vc = oracle.pyramid_levels(V_, L, p, None)
        tot = 0.0
        for b in range(N // qb):
            o = oracle.prefill_block(Q_, K_, V_, kc, vc, sels[b], b, qb, L, p)
            tot += float((o * dO[qb * b:qb * b + qb]).sum())
        return tot

    h = 1e-6
    for which, G in ((0, gQ), (1, gK), (2, gV)):
        for i in range(N):
            for c in range(d):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][i, c] += h
                up = loss(*args)
                args[which][i, c] -= 2 * h
                dn = loss(*args)
                assert abs((up - dn) / (2 * h) - G[i, c]) < 1e-7, (which, i, c)


def test_pyramid_backward_invariants():
    """Every query's softmax weights sum to one, so its score gradients sum
    to zero: the key gradients of a head sum to zero and its value
    gradients sum to the sum of dO (the coarse means pass both sums on
    unchanged)."""
    N, d, L, p, qb, K_ = 256, 16, 3, 4, 32, 24
    rng = np.random.default_rng(8)
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    _, gK, gV = oracle.prefill_grads(Q, K, V, dO, L, p, qb, K_, store="bf16")
    np.testing.assert_allclose(gK.sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(gV.sum(axis=0), dO.sum(axis=0), atol=1e-10)


def test_pyramid_backward_single_key_and_scatter():
    """One token: its only key is itself, so dV = dO and dQ = dK = 0.  And
    the scatter of a coarse gradient by hand: an entry at level 2 of a
    factor-2 pyramid spreads its gradient over 4 rows as quarters."""
    rng = np.random.default_rng(3)
    Q, K, V, dO = (rng.standard_normal((1, 4)) for _ in range(4))
    gQ, gK, gV = oracle.prefill_grads(Q, K, V, dO, 1, 2, 1, 0, store=None)
    np.testing.assert_allclose(gV, dO, atol=1e-15)
    np.testing.assert_allclose(gQ, 0.0, atol=1e-15)
    np.testing.assert_allclose(gK, 0.0, atol=1e-15)
    # flat ids for N = 8, L = 3, p = 2: level 0 -> 0..7, level 1 -> 8..11, level 2 -> 12..13
    g = np.zeros((14, 1))
    g[13] = 8.0           # level-2 entry 1: rows 4..7
    g[9] = 2.0            # level-1 entry 1: rows 2..3
    g[0] = 1.0
    np.testing.assert_allclose(oracle.pyramid_backward(g, 8, 3, 2)[:, 0],
                               [1, 0, 1, 1, 2, 2, 2, 2])


# ---------------------------------------------------------------- tiered K/V (HGA memory architecture)
def test_warm_cache_one_group_per_step_is_plain_lru():
    """With one group per step the warm tier is an ordinary LRU cache:
    against an OrderedDict LRU on a random access sequence, the same hits
    and misses and the same resident groups after every step."""
    from collections import OrderedDict
    rng = np.random.default_rng(1)
    cache = oracle.WarmCache(5)
    ref = OrderedDict()
    for step, g in enumerate(rng.integers(0, 12, 400).tolist(), start=1):
        hits, misses, place = cache.step([g], step)
        if g in ref:
            ref.move_to_end(g)
            want = (1, 0)
        else:
            if len(ref) == 5:
                ref.popitem(last=False)
            ref[g] = True
            want = (0, 1)
        assert (hits, misses) == want, step
        assert sorted(x for x in cache.group if x >= 0) == sorted(ref), step


def test_warm_cache_hand_case():
    """Two slots.  Step 1 needs {5}: slot 0.  Step 2 needs {7}: the empty
    slot 1.  Step 3 needs {5, 9}: 5 hits in slot 0; 9 evicts 7 (slot 1, the
    only slot step 3 does not need).  Step 4 needs {7, 9}: 9 hits; 7 takes
    the least recently used other slot, slot 0 (last used at step 3, same as
    slot 1, which step 4 needs)."""
    c = oracle.WarmCache(2)
    assert c.step([5], 1) == (0, 1, {5: 0})
    assert c.step([7], 2) == (0, 1, {7: 1})
    assert c.step([5, 9], 3) == (1, 1, {5: 0, 9: 1})
    assert c.step([7, 9], 4) == (1, 1, {9: 1, 7: 0})
    assert c.group == [7, 9] and c.stamp == [4, 4]
    with pytest.raises(ValueError):
        c.step([1, 2, 3], 5)


def test_tier_rows_round_trip():
    """Brute force on a small routed list: build the device tier the way the
    rows say (sink rows, the ring of the last chunks, warm slots filled from
    the cold store) and read every listed position back from its row."""
    n, C, grp, sc, lc = 64 * 20 + 17, 64, 16, 2, 3
    rng = np.random.default_rng(2)
    K = rng.standard_normal((n, 4))
    kappa = (n - 1) // C
    routed = sorted(rng.choice(np.arange(sc * C // grp, (kappa - lc) * C // grp), 6, replace=False))
    pos = np.concatenate([np.arange(sc * C)] + [np.arange(g * grp, (g + 1) * grp) for g in routed]
                         + [np.arange((kappa - lc) * C, n)])
    hot, rt = oracle.split_positions(pos, n, C, grp, sc, lc)
    assert hot.sum() == sc * C + n - (kappa - lc) * C and rt.sum() == 6 * grp
    need = oracle.needed_groups(pos, n, C, grp, sc, lc)
    assert need == [int(g) for g in routed]
    cache = oracle.WarmCache(8)
    _, _, place = cache.step(need, 1)
    rows = oracle.tier_rows(pos, n, C, grp, sc, lc, place)
    assert len(set(rows.tolist())) == len(rows)               # one row per position
    ring = (lc + 1) * C
    tier = np.full((sc * C + ring + 8 * grp, 4), np.nan)
    tier[:sc * C] = K[:sc * C]
    for p in range((kappa - lc) * C, n):
        tier[sc * C + p % ring] = K[p]
    for g, s in place.items():
        tier[sc * C + ring + s * grp: sc * C + ring + (s + 1) * grp] = K[g * grp:(g + 1) * grp]
    np.testing.assert_array_equal(tier[rows], K[pos])
