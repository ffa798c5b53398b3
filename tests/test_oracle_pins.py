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
