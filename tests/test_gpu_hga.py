"""GPU parity of hierarchical chunk/group routing (summaries -> two-level
routing -> decode) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DecodeRun, DEV, log, max_err, np64, np_inputs, to_dev

pytestmark = pytest.mark.gpu

SMALL = workloads.HGA_64K.with_(batch=2, n_q_heads=8, n_kv_heads=2, n_ctx=64 * 40 + 37)


def _oracle_summaries(cfg, kp, store):
    cs = oracle.chunk_summaries(kp[:cfg.n_ctx], cfg.chunk, cfg.rope_base, store)
    gs = oracle.group_summaries(kp[:cfg.n_ctx], cfg.group, cfg.rope_base, store)
    return cs, gs


@pytest.mark.parametrize("cfg", [
    SMALL,
    SMALL.with_(dtype="fp32", head_dim=64, rope_base=1e4, n_ctx=64 * 9 + 5),
    SMALL.with_(chunk=32, group=8, n_ctx=32 * 50),
])
def test_summaries_match_oracle(cfg):
    log("summaries", cfg.dtype, cfg.head_dim, cfg.n_ctx, cfg.chunk)
    inp = workloads.decode_inputs(cfg, 3)
    run = DecodeRun(cfg, inp)
    run.summaries()
    torch.cuda.synchronize()
    ni = np_inputs(inp)
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            cs, gs = _oracle_summaries(cfg, ni["k_pre"][b, g], cfg.dtype)
            got_c = np64(run.t["chunk_sum"][b, g, :len(cs)])
            got_g = np64(run.t["group_sum"][b, g, :len(gs)])
            if cfg.dtype == "bf16":
                csx, gsx = _oracle_summaries(cfg, ni["k_pre"][b, g], None)
                for got, ref, ex in ((got_c, cs, csx), (got_g, gs, gsx)):
                    ulp = np.maximum(oracle.bf16_ulp(ex), oracle.bf16_ulp(ref))
                    assert np.all(np.abs(got - ref) <= ulp * 1.0001 + 1e-12)
                    assert np.mean(got == ref) > 0.999
            else:
                np.testing.assert_allclose(got_c, cs, rtol=1e-6, atol=1e-7)
                np.testing.assert_allclose(got_g, gs, rtol=1e-6, atol=1e-7)


def test_summary_incremental_build_equals_full():
    cfg = SMALL
    inp = workloads.decode_inputs(cfg, 4)
    full = DecodeRun(cfg, inp)
    full.summaries()
    inc = DecodeRun(cfg, inp)
    inc.summaries(0, 700)
    for t in range(700, cfg.n_ctx, 333):
        inc.summaries(t, min(cfg.n_ctx, t + 333))
    torch.cuda.synchronize()
    assert torch.equal(full.t["chunk_sum"], inc.t["chunk_sum"])
    assert torch.equal(full.t["group_sum"], inc.t["group_sum"])


def _route_oracle(cfg, q, cs, gs, b, g):
    G = cfg.gqa
    return oracle.route_token_list(q[b, g * G:(g + 1) * G], cs[b, g], gs[b, g], cfg.n_ctx,
                                   cfg.chunk, cfg.group, cfg.top_chunks, cfg.top_groups,
                                   cfg.sink_chunks, cfg.local_chunks)


def _run_route_lattice(cfg, lat):
    run = DecodeRun(cfg, {})
    nc, ng = lat["chunk_sum"].shape[2], lat["group_sum"].shape[2]
    run.t["chunk_sum"][:, :, :nc] = to_dev(lat["chunk_sum"], cfg.dtype)
    run.t["group_sum"][:, :, :ng] = to_dev(lat["group_sum"], cfg.dtype)
    run.t["q"] = to_dev(lat["q"], cfg.dtype)
    run.select()
    torch.cuda.synchronize()
    return run.sets()


ROUTE_CASES = [
    SMALL,                                               # 28 candidates, top 16
    SMALL.with_(n_ctx=64 * 12 + 1),                      # no candidate chunk
    SMALL.with_(n_ctx=64 * 20),                          # fewer candidates than top_chunks
    SMALL.with_(n_ctx=64 * 7 + 63, sink_chunks=4, local_chunks=8),   # locals overlap sinks
    SMALL.with_(n_ctx=1),
    SMALL.with_(n_ctx=64 * 300 + 17, top_chunks=40, top_groups=3),
    SMALL.with_(head_dim=64, dtype="fp32", n_ctx=64 * 100),
]


@pytest.mark.parametrize("cfg", ROUTE_CASES, ids=lambda c: f"n{c.n_ctx}-d{c.head_dim}-{c.dtype}")
@pytest.mark.parametrize("amp", [2, 16])
def test_route_lattice_exact(cfg, amp):
    """Lattice summaries and queries make every routing score exact on both
    sides; small amplitudes force exact ties, decided by the lower index."""
    lat = workloads.lattice_summary_inputs(cfg, 40 + amp, amp=amp, q_amp=4)
    idx, cnt = _run_route_lattice(cfg, lat)
    q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            ref, _ = _route_oracle(cfg, q, cs, gs, b, g)
            assert cnt[b, g] == len(ref), (b, g, cnt[b, g], len(ref))
            assert np.array_equal(idx[b, g, :len(ref)], ref), (b, g)


def _random_route_configs(count, seed):
    """Seeded routing shapes with every knob varied: chunk and group sizes,
    top chunks and groups, sink and local chunks, GQA group, head dim,
    dtype and ragged contexts (including none or fewer candidates than the
    top count)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        chunk = int(rng.choice([16, 32, 64, 128]))
        group = chunk // int(rng.choice([g for g in (1, 2, 4, 8) if chunk // g >= 2]))
        gpc = chunk // group
        hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        out.append(SMALL.with_(
            batch=int(rng.integers(1, 3)), n_q_heads=hkv * G, n_kv_heads=hkv,
            head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "fp32"])),
            n_ctx=int(rng.integers(1, 20000)), chunk=chunk, group=group,
            top_chunks=int(rng.integers(1, 65)), top_groups=int(rng.integers(1, gpc + 1)),
            sink_chunks=int(rng.integers(0, 7)), local_chunks=int(rng.integers(0, 11))))
    return out


@pytest.mark.parametrize("cfg", _random_route_configs(20, 7),
                         ids=lambda c: f"c{c.chunk}g{c.group}t{c.top_chunks}x{c.top_groups}-n{c.n_ctx}")
def test_route_random_shapes_exact(cfg):
    """Exact lists on lattice inputs for seeded random routing shapes."""
    amp = 2 if cfg.n_ctx % 2 else 16
    log("route random", cfg.n_ctx, cfg.chunk, cfg.group, cfg.top_chunks, cfg.top_groups,
        cfg.sink_chunks, cfg.local_chunks, cfg.gqa, cfg.head_dim, cfg.dtype, amp)
    lat = workloads.lattice_summary_inputs(cfg, 77, amp=amp, q_amp=4)
    idx, cnt = _run_route_lattice(cfg, lat)
    q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            ref, _ = _route_oracle(cfg, q, cs, gs, b, g)
            assert cnt[b, g] == len(ref), (b, g, cnt[b, g], len(ref))
            assert np.array_equal(idx[b, g, :len(ref)], ref), (b, g)


def test_route_strict_gap_variant():
    """Lattice inputs redrawn until every chunk and group cut falls between
    scores at least 1e-3 apart (no tie decides the set)."""
    cfg = SMALL.with_(n_ctx=64 * 200)
    for s in range(200):
        lat = workloads.lattice_summary_inputs(cfg, 900 + s, amp=16, q_amp=4)
        q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
        ok = True
        for b in range(cfg.batch):
            for g in range(cfg.n_kv_heads):
                _, info = _route_oracle(cfg, q, cs, gs, b, g)
                if info["chunk_gap"] < 1e-3 or min(info["group_gaps"]) < 1e-3:
                    ok = False
        if ok:
            break
    else:
        pytest.fail("no strict-gap draw")
    log("strict gap draw", s)
    idx, cnt = _run_route_lattice(cfg, lat)
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            ref, _ = _route_oracle(cfg, q, cs, gs, b, g)
            assert cnt[b, g] == len(ref) and np.array_equal(idx[b, g, :len(ref)], ref)


def _robust_hga_seed(cfg, start, tries=60, gap=1e-3):
    """First seed whose oracle routing (on the oracle's own summaries) has
    every chunk and group cut at least ``gap`` apart in every group."""
    for s in range(start, start + tries):
        ni = np_inputs(workloads.decode_inputs(cfg, s))
        ok = True
        for b in range(cfg.batch):
            for g in range(cfg.n_kv_heads):
                cs, gs = _oracle_summaries(cfg, ni["k_pre"][b, g], cfg.dtype)
                G = cfg.gqa
                _, info = oracle.route_token_list(
                    ni["q"][b, g * G:(g + 1) * G], cs, gs, cfg.n_ctx, cfg.chunk, cfg.group,
                    cfg.top_chunks, cfg.top_groups, cfg.sink_chunks, cfg.local_chunks)
                if info["chunk_gap"] < gap or (info["group_gaps"] and min(info["group_gaps"]) < gap):
                    ok = False
        if ok:
            return s
    raise AssertionError("no robust seed")


def test_hga_end_to_end_small():
    cfg = SMALL.with_(n_ctx=64 * 60 + 9)
    seed = _robust_hga_seed(cfg, 0)
    log("hga seed", seed)
    inp = workloads.decode_inputs(cfg, seed)
    run = DecodeRun(cfg, inp)
    run.summaries()
    run.select()
    run.decode()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    out = np64(run.t["out"])
    ni = np_inputs(inp)
    sets = oracle.decode_token_sets(cfg, ni)
    for (b, g), T in sets.items():
        assert cnt[b, g] == len(T) and np.array_equal(idx[b, g, :len(T)], T), (b, g)
    ref = oracle.decode_step(cfg, ni, sets=sets)
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    log("hga small max err", err)
    assert err <= 2e-3


def test_hga_full_size_sampled():
    """The 64K routed workload at full size (16 x 8 groups), inputs drawn on
    the GPU.  Eight sampled groups are checked exactly, stage by stage: the
    oracle routes over the GPU's own bf16 summaries, and a sampled group whose
    17 routing cuts (top chunks, then the groups of each) are not all at
    least 1e-3 apart has the non-needle dims of its queries re-drawn until
    they are; its set must then equal the oracle's, and its outputs the
    oracle's attention over that set."""
    cfg = workloads.HGA_64K
    seed = 5
    inp = workloads.decode_inputs(cfg, seed, device=DEV)
    run = DecodeRun(cfg, inp)
    run.summaries()
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    pairs = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]
    groups = [pairs[i] for i in sorted(rng.choice(len(pairs), 8, replace=False))]
    G = cfg.gqa
    q_pre = inp["q_pre"].to(DEV)
    q = run.t["q"].float()
    expect = {}
    redraws = 0
    for b, g in groups:
        cs = np64(run.t["chunk_sum"][b, g])
        gs = np64(run.t["group_sum"][b, g])
        for rnd in range(1, 40):
            qg = np64(q[b, g * G:(g + 1) * G])
            T, info = oracle.route_token_list(qg, cs, gs, cfg.n_ctx, cfg.chunk, cfg.group,
                                              cfg.top_chunks, cfg.top_groups, cfg.sink_chunks,
                                              cfg.local_chunks)
            if info["chunk_gap"] >= 1e-3 and min(info["group_gaps"]) >= 1e-3:
                break
            q_pre, q = workloads.redraw_query_dims(cfg, q_pre, seed, [(b, h) for h in
                                                   range(g * G, (g + 1) * G)], rnd)
            redraws += 1
        else:
            raise AssertionError(f"no robust redraw for group {(b, g)}")
        expect[(b, g)] = (T, qg)
    log("full-size routed groups redrawn", redraws, "times over", len(groups), "groups")
    run.t["q"].copy_(q.to(run.t["q"].dtype))
    run.select()
    run.decode()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    out = np64(run.t["out"])
    for (b, g), (T, qg) in expect.items():
        got = idx[b, g, :cnt[b, g]]
        assert cnt[b, g] == len(T) and np.array_equal(got, T), (b, g)
        K = np64(run.t["k_cache"][b, g])[T]
        V = np64(run.t["v_cache"][b, g])[T]
        for hh in range(G):
            o = oracle.attend(qg[hh], K, V)
            assert max_err(out[b, g * G + hh], o) <= 2e-3
