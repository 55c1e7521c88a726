"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against a published value, a closed form, an
invariant, a library routine, or a brute-force evaluation written as per-element
loops, chosen so that a dropped term, a sign or index slip or a transposed
operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import dg_inputs as di
from oracle import numerics as nm
from oracle import philox, sampler as smp
from oracle.model import OracleModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ Philox
def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_philox_known_answers():
    for r in _kat():
        out = philox.philox4x32_10(np.array(r[:4], np.uint32), np.array(r[4:6], np.uint32))
        assert [int(v) for v in out] == r[6:]


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(3)
    ctr = rng.integers(0, 2**32, size=(50, 4), dtype=np.uint64).astype(np.uint32)
    key = np.array([0x12345678, 0x9abcdef0], np.uint32)
    out = philox.philox4x32_10(ctr, key)
    for i in range(50):
        assert np.array_equal(out[i], philox.philox4x32_10(ctr[i], key))


def test_stream_layout_words():
    # word j of a call sits at counter word 0 = j >> 2, output lane j & 3
    seed = (7 << 32) | 5
    w = philox.words(seed, philox.TAG_GUMBEL, 3, 9, np.full(8, 11), np.arange(8))
    ctr0 = np.array([0, 11, 9, (philox.TAG_GUMBEL << 24) | 3], np.uint32)
    ctr1 = np.array([1, 11, 9, (philox.TAG_GUMBEL << 24) | 3], np.uint32)
    key = np.array([5, 7], np.uint32)
    ref = np.concatenate([philox.philox4x32_10(ctr0, key), philox.philox4x32_10(ctr1, key)])
    assert np.array_equal(w, ref)


def test_gumbel_stream_layout():
    # hand-listed (vocabulary id -> counter word 0, output word) of the GUMBEL stream
    cases = {0: (0, 0), 5: (5, 0), 16: (0, 1), 33: (1, 2), 63: (15, 3), 64: (16, 0), 80: (16, 1),
             127: (31, 3), 200: (56, 0), 4095: (1023, 3)}
    seed, canvas, step, pos = (7 << 32) | 5, 3, 9, 11
    key = np.array([5, 7], np.uint32)
    g = smp.gumbel_block(seed, canvas, step, np.array([pos]), 4096)[0]
    for v, (c0, word) in cases.items():
        ctr = np.array([c0, pos, step, (philox.TAG_GUMBEL << 24) | canvas], np.uint32)
        assert g[v] == philox.gumbel(philox.philox4x32_10(ctr, key)[word:word + 1])[0], v
    # every id of a 4096-id range draws its own word: (call, word) pairs are all distinct
    call, word = smp.gumbel_call_of(np.arange(4096))
    assert len(set(zip(call.tolist(), word.tolist()))) == 4096
    assert call.max() == 1023


def test_uniform01_range_and_exactness():
    x = np.array([0, 1, 511, 512, 2**32 - 1], np.uint64).astype(np.uint32)
    u = philox.uniform01(x)
    assert u.dtype == np.float32
    assert u[0] == np.float32(2.0 ** -24) and u[1] == u[0] and u[2] == u[0]
    assert u[3] == np.float32(3 * 2.0 ** -24)
    assert u[4] == np.float32(1 - 2.0 ** -24) and u[4] < 1
    k = np.arange(0, 2**23, 4099, dtype=np.uint64)
    uu = philox.uniform01((k << np.uint64(9)).astype(np.uint32)).astype(np.float64)
    assert np.array_equal(uu, (2 * k + 1) * 2.0 ** -24)


def _chi2_uniform(counts):
    e = counts.sum() / counts.size
    return float(((counts - e) ** 2 / e).sum())


def test_uniform_token_chi2():
    V = 64
    w = philox.words(99, philox.TAG_RENOISE, 0, 0, np.arange(200_000), 0)
    tok = philox.uniform_token(w, V)
    assert tok.min() >= 0 and tok.max() < V
    c = np.bincount(tok, minlength=V).astype(np.float64)
    # df = 63: mean 63, sd ~11.2; 140 is beyond the 1e-9 tail
    assert _chi2_uniform(c) < 140
    # exact for powers of two: the token is the top log2(V) bits
    assert np.array_equal(tok, (w >> np.uint32(26)).astype(np.int32))


def test_gumbel_moments():
    w = philox.words(5, philox.TAG_GUMBEL, 0, 0, np.zeros(400_000, np.int64), np.arange(400_000))
    g = philox.gumbel(w).astype(np.float64)
    assert abs(g.mean() - 0.5772156649) < 0.01           # Euler-Mascheroni constant
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03


# ------------------------------------------------------------------ numerics
def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        np.float32([0, 1, -1, 1.00390625, 1.01171875, 3e-5, -7.5e3])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(nm.bf16_round(x.astype(np.float64)), ref)
    # ties go to even: 1 + 2**-8 sits halfway between 1 and 1 + 2**-7
    assert nm.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert nm.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2 * 2.0 ** -7


def test_bf16_round_matches_input_generator_bits():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000).astype(np.float32)
    bits = di.f32_to_bf16_bits(x)
    assert np.array_equal(nm.upcast(bits), nm.bf16_round(x.astype(np.float64)))


def test_rmsnorm_unit_rms_and_gain():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 64)) * 5
    y = nm.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt((y ** 2).mean(-1)), 1.0, atol=1e-12)
    g = rng.standard_normal(64)
    assert np.allclose(nm.rmsnorm(x, g, 1e-6), nm.rmsnorm(x, np.ones(64), 1e-6) * g)
    # eps enters under the root: a zero row stays zero, a tiny row is not blown up
    assert np.all(nm.rmsnorm(np.zeros((1, 4)), np.ones(4), 1e-6) == 0)
    assert np.allclose(nm.rmsnorm(np.full((1, 4), 1e-3), np.ones(4), 1e-6),
                       1e-3 / math.sqrt(1e-6 + 1e-6))


def test_rope_hand_value_and_sign():
    # hd = 2: one pair, frequency theta**0 = 1; position p rotates (1, 0) to (cos p, sin p)
    x = np.array([[[1.0, 0.0]]])
    y = nm.rope(x, np.array([1]), 10000.0)
    assert np.allclose(y[0, 0], [math.cos(1), math.sin(1)])
    # hd = 4: second pair (indices 1 and 3) uses theta**(-2/4)
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y = nm.rope(x, np.array([3]), 100.0)
    a = 3 * 100.0 ** -0.5
    assert np.allclose(y[0, 0], [0, math.cos(a), 0, math.sin(a)])


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    for p in (0, 5, 1000):
        assert np.isclose(np.linalg.norm(nm.rope(q, np.array([p]), 1e4)), np.linalg.norm(q))
    assert np.allclose(nm.rope(q, np.array([0]), 1e4), q)
    d1 = (nm.rope(q, np.array([17]), 1e4) * nm.rope(k, np.array([10]), 1e4)).sum()
    d2 = (nm.rope(q, np.array([107]), 1e4) * nm.rope(k, np.array([100]), 1e4)).sum()
    assert np.isclose(d1, d2, rtol=1e-9)


def _attention_loops(q, k, v, qp, kp, causal):
    nq, Hq, hd = q.shape
    Hkv = k.shape[1]
    out = np.zeros_like(q)
    for i in range(nq):
        for h in range(Hq):
            g = h * Hkv // Hq
            sc, idx = [], []
            for j in range(k.shape[0]):
                if causal and kp[j] > qp[i]:
                    continue
                sc.append(sum(q[i, h, c] * k[j, g, c] for c in range(hd)) / math.sqrt(hd))
                idx.append(j)
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            tot = sum(ex)
            for c in range(hd):
                out[i, h, c] = sum(e * v[j, g, c] for e, j in zip(ex, idx)) / tot
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_attention_brute_force(causal):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 4, 8))
    k = rng.standard_normal((7, 2, 8))
    v = rng.standard_normal((7, 2, 8))
    qp = np.array([3, 4, 5, 6])
    kp = np.arange(7)
    assert np.allclose(nm.attention(q, k, v, qp, kp, causal), _attention_loops(q, k, v, qp, kp, causal))


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 2, 4))
    v = rng.standard_normal((5, 1, 4))
    # identical keys -> plain mean of the values
    k = np.repeat(rng.standard_normal((1, 1, 4)), 5, axis=0)
    o = nm.attention(q, k, v, np.arange(3), np.arange(5), False)
    assert np.allclose(o, v.mean(0)[None].repeat(3, 0).repeat(2, 1))
    # causal: the query at position 0 sees only key 0
    o = nm.attention(q, rng.standard_normal((5, 1, 4)), v, np.array([0, 1, 2]), np.arange(5), True)
    assert np.allclose(o[0], v[0])


def test_entropy_uniform_and_peaked():
    V = 4096
    st = smp.head_stats(np.zeros((2, V), np.float32), np.float32(1.25), 1, 0, 0, np.arange(2))
    assert np.all(st["H"] == np.float32(math.log(V)))             # closed form: log V
    lg = np.zeros((1, V), np.float32)
    lg[0, 17] = 200.0
    st = smp.head_stats(lg, np.float32(1.0), 1, 0, 0, np.arange(1))
    assert 0 <= st["H"][0] < 1e-60 or st["H"][0] == 0
    assert st["am"][0] == 17 and st["y"][0] == 17
    rng = np.random.default_rng(7)
    lg = (rng.standard_normal((8, 64)) * 4).astype(np.float32)
    st = smp.head_stats(lg, np.float32(1 / 0.8), 1, 0, 0, np.arange(8), want_probs=True)
    assert np.all(st["H"] >= 0) and np.all(st["H"] <= np.float32(math.log(64)))
    # the tempered distribution: explicit formula -sum p log p with p = softmax(l / T)
    z = lg.astype(np.float64) * np.float64(np.float32(1 / 0.8))
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(st["H"], -(p * np.log(p)).sum(1), rtol=1e-6)
    assert np.allclose(st["p"], p)


def test_gumbel_max_frequencies():
    # textbook: argmax(z + Gumbel) is distributed as softmax(z)
    z = np.log(np.array([0.05, 0.1, 0.2, 0.3, 0.15, 0.1, 0.06, 0.04]))
    n = 20000
    lg = np.tile(z.astype(np.float32), (n, 1))
    st = smp.head_stats(lg, np.float32(1.0), 11, 0, 0, np.arange(n), chunk=4096)
    c = np.bincount(st["y"], minlength=8).astype(np.float64)
    e = n * np.exp(z) / np.exp(z).sum()
    chi2 = ((c - e) ** 2 / e).sum()
    assert chi2 < 40                                              # df = 7
    assert np.all(st["margin"] >= 0)


def _gumbel_by_hand(seed, canvas, step, pos, ids):
    """Gumbel draws of ids < 16 from hand-written counters: id v is word 0 of the
    call with counter (v, pos, step, GUMBEL << 24 | canvas) under key (seed lo, seed hi)."""
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    out = []
    for v in ids:
        ctr = np.array([v, pos, step, (3 << 24) | canvas], np.uint32)
        out.append(philox.gumbel(philox.philox4x32_10(ctr, key)[0:1])[0])
    return np.array(out, np.float32)


def test_margin_is_top2_gap_of_perturbed_tempered_scores():
    # 4-id vocabulary: the top two of z + g (ids 0 and 1 here) differ from the
    # top two of z alone (ids 0 and 2), so a margin over z, over unperturbed
    # logits, or without the 1/T factor gives another value
    seed, canvas, step, pos = (3 << 32) | 1, 0, 2, 5
    g = _gumbel_by_hand(seed, canvas, step, pos, range(4))
    lg = np.array([[2.0, 0.9, 1.9, 0.0]], np.float32)
    inv_t = np.float32(1.25)
    st = smp.head_stats(lg, inv_t, seed, canvas, step, np.array([pos]))
    score = lg[0] * inv_t + g                                  # fp32, as the scores are defined
    srt = np.sort(score)
    assert st["y"][0] == int(np.argmax(score)) == 0
    assert st["margin"][0] == np.float32(srt[-1] - srt[-2])
    # the hand-computed draws: g = (1.00097, 2.13609, 0.45004, 0.14130) to 5 digits,
    # z = (2.5, 1.125, 2.375, 0), scores (3.50097, 3.26109, 2.82504, 0.14130):
    # margin = 3.50097 - 3.26109; over z alone it would be 0.125, and without
    # the 1/T factor id 1 would win
    assert abs(float(st["margin"][0]) - (3.50097 - 3.26109)) < 2e-5
    assert int(np.argmax(lg[0] + g)) == 1


def test_margin_zero_on_exact_tie():
    # logits -g make the scores of ids 1 and 3 exactly 0 (x + (-x) is exact);
    # the others sit far below: y is the lower tied id and the margin is 0
    seed, canvas, step, pos = (9 << 32) | 4, 1, 0, 17
    g = _gumbel_by_hand(seed, canvas, step, pos, range(4))
    lg = np.array([[-g[0] - 10, -g[1], -g[2] - 10, -g[3]]], np.float32)
    st = smp.head_stats(lg, np.float32(1.0), seed, canvas, step, np.array([pos]))
    assert st["y"][0] == 1
    assert st["margin"][0] == 0.0


def test_ties_take_lowest_id():
    lg = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    st = smp.head_stats(lg, np.float32(1.0), 1, 0, 0, np.arange(1))
    assert st["am"][0] == 1


def test_temperature_schedule():
    S = 48
    Ts = [smp.temperature(t, S) for t in range(S)]
    assert Ts[0] == np.float32(0.8) and Ts[-1] == np.float32(0.4)
    d2 = np.diff(np.array(Ts, np.float64), 2)
    assert np.abs(d2).max() < 1e-7
    assert smp.temperature(0, 1) == np.float32(0.8)
    assert smp.temperature(11, 12) == np.float32(0.4)
    assert np.isclose(float(smp.temperature(6, 13)), 0.6, atol=1e-7)


def _commit_cases():
    out = []
    with open(os.path.join(GOLDEN, "commit_cases.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                b, h, e = [s.strip() for s in line.split("|")]
                exp = [] if e == "-" else [int(t) for t in e.split()]
                out.append((float(b), np.array([float(t) for t in h.split()], np.float32), exp))
    return out


@pytest.mark.parametrize("case", _commit_cases())
def test_commit_hand_cases(case):
    bound, H, expected = case
    n = H.size
    y = np.arange(100, 100 + n, dtype=np.int32)
    new, mask, ncom, done = smp.commit(H, y, y, None, np.zeros(n, np.int32), 0, 10, bound,
                                       smp.STOP_NONE, 0.0, 3, 0, 1 << 20)
    assert sorted(np.nonzero(mask)[0].tolist()) == expected
    assert ncom == len(expected) and not done
    assert np.all(new[mask == 1] == y[mask == 1])


def test_commit_bound_and_prefix_random():
    rng = np.random.default_rng(8)
    for trial in range(200):
        H = (rng.exponential(0.05, 256) * (rng.random(256) < 0.5)).astype(np.float32)
        bound = float(rng.uniform(0, 2))
        y = rng.integers(0, 1000, 256).astype(np.int32)
        new, mask, ncom, _ = smp.commit(H, y, y, None, y, 3, 48, bound, 0, 0.0, trial, 0, 1000)
        sel = mask == 1
        assert H[sel].astype(np.float64).sum() <= float(np.float32(bound)) + 1e-12
        # maximal: the cheapest uncommitted position would break the bound
        if (~sel).any():
            assert H[sel].astype(np.float64).sum() + H[~sel].min() > float(np.float32(bound))
            assert H[~sel].min() >= H[sel].max() if sel.any() else True
        assert np.all(new[sel] == y[sel])


def test_renoise_uniform_and_committed_keep_y():
    V = 32
    H = np.full(256, 5.0, np.float32)                              # nothing commits
    counts = np.zeros(V)
    for s in range(400):
        y = np.zeros(256, np.int32)
        new, mask, ncom, _ = smp.commit(H, y, y, None, y, 1, 48, 0.1, 0, 0.0, s, 0, V)
        assert ncom == 0
        counts += np.bincount(new, minlength=V)
    assert _chi2_uniform(counts) < 90                              # df = 31


def test_stop_rules_and_final_step():
    n = 256
    y = np.arange(n, dtype=np.int32)
    am = y.copy()
    low = np.full(n, 0.001, np.float32)
    high = np.full(n, 1.0, np.float32)
    # mode 1: mean < tau stops and writes y everywhere
    new, mask, ncom, done = smp.commit(low, y, am, None, y * 0, 2, 48, 0.1, 1, 0.05, 1, 0, 512)
    assert done and ncom == n and np.array_equal(new, y)
    new, mask, ncom, done = smp.commit(high, y, am, None, y * 0, 2, 48, 0.1, 1, 0.05, 1, 0, 512)
    assert not done
    # mode 2 needs the argmax to be unchanged from the previous step
    _, _, _, done = smp.commit(low, y, am, am.copy(), y, 2, 48, 0.1, 2, 0.005, 1, 0, 512)
    assert done
    prev = am.copy()
    prev[7] += 1
    _, _, _, done = smp.commit(low, y, am, prev, y, 2, 48, 0.1, 2, 0.005, 1, 0, 512)
    assert not done
    _, _, _, done = smp.commit(low, y, am, None, y, 0, 48, 0.1, 2, 0.005, 1, 0, 512)
    assert not done
    # last step of the budget: every position takes y
    new, _, ncom, done = smp.commit(high, y, am, None, y * 0, 47, 48, 0.1, 0, 0.0, 1, 0, 512)
    assert done and ncom == n and np.array_equal(new, y)


def test_self_cond_special_cases():
    rng = np.random.default_rng(9)
    E = rng.standard_normal((16, 8))
    V = 16
    st = smp.head_stats(np.zeros((1, V), np.float32), np.float32(1.0), 1, 0, 0, np.arange(1),
                        want_probs=True)
    assert np.allclose(st["p"][0] @ E, E.mean(0))                  # uniform p -> column mean
    lg = np.full((1, V), -1e4, np.float32)
    lg[0, 5] = 0
    st = smp.head_stats(lg, np.float32(1.0), 1, 0, 0, np.arange(1), want_probs=True)
    assert np.allclose(st["p"][0] @ E, E[5])                      # one-hot p -> a row of E


# ------------------------------------------------------------------ MoE and model
def _micro_cfg(dtype="f32", E=4, k=2, L=2, sc=False):
    return di.ModelConfig(n_layers=L, d_model=8, n_q_heads=2, n_kv_heads=1, head_dim=4,
                          n_experts=E, ffn_hidden=6, top_k=k, vocab=16, dtype=dtype,
                          self_cond=sc, canvas_len=5)


def test_moe_weights_sum_to_one_and_ties():
    cfg = _micro_cfg(E=6, k=3)
    W = di.make_weights(cfg, 3, gain_std=0.3)
    m = OracleModel(cfg, W, 1, 16)
    rng = np.random.default_rng(10)
    tr = {}
    m._moe(0, rng.standard_normal((9, 8)), tr)
    assert np.allclose(tr["route_w"][0].sum(1), 1.0)
    r = tr["router_logits"][0]
    idx = tr["route_idx"][0]
    for i in range(9):
        assert set(idx[i]) == set(np.argsort(-r[i], kind="stable")[:3])
        assert np.all(np.diff(r[i][idx[i]]) <= 0)
    # tied router logits: a zero input gives all-zero logits -> lowest ids 0, 1, 2
    tr = {}
    m._moe(0, np.zeros((1, 8)), tr)
    assert list(tr["route_idx"][0][0]) == [0, 1, 2]


def test_moe_dense_when_all_experts_selected():
    cfg = _micro_cfg(E=3, k=3)
    W = di.make_weights(cfg, 4)
    m = OracleModel(cfg, W, 1, 16)
    x = np.random.default_rng(11).standard_normal((5, 8))
    y = m._moe(0, x, None)
    r = x @ m.W("l0.w_router").T
    w = np.exp(r - r.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    dense = np.zeros_like(y)
    for e in range(3):
        g, u = x @ m.W("l0.w_gate")[e].T, x @ m.W("l0.w_up")[e].T
        dense += w[:, e:e + 1] * ((g / (1 + np.exp(-g)) * u) @ m.W("l0.w_down")[e].T)
    assert np.allclose(y, dense, rtol=1e-6, atol=1e-12)
    # k = 1 gives weight exactly 1 to the chosen expert
    cfg1 = _micro_cfg(E=3, k=1)
    m1 = OracleModel(cfg1, di.make_weights(cfg1, 4), 1, 16)
    tr = {}
    m1._moe(0, x, tr)
    assert np.all(tr["route_w"][0] == 1.0)


def _bf(x, on):
    if not on:
        return x
    if x == 0:
        return 0.0
    mnt, e = math.frexp(x)
    return math.ldexp(round(mnt * 256) / 256, e)   # Python round: half to even


def _forward_loops(cfg, W, ids, pos, ctx_k, ctx_v, causal, extra=None):
    """Per-element loop version of the stack for tiny shapes (independent of numpy matmul)."""
    bf = cfg.dtype == "bf16"
    d, Hq, Hkv, hd, E, F, K = (cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                               cfg.n_experts, cfg.ffn_hidden, cfg.top_k)
    g = {n: nm.upcast(W.get(n)) for n in W.names()}

    def mv(M, x):                     # [out, in] matrix times vector
        return [sum(M[o][i] * x[i] for i in range(len(x))) for o in range(len(M))]

    def norm(x, gain):
        r = math.sqrt(sum(v * v for v in x) / len(x) + cfg.rms_eps)
        return [_bf(x[i] / r * gain[i], bf) for i in range(len(x))]

    def rot(vec, p):
        out = list(vec)
        half = hd // 2
        for j in range(half):
            a = p * cfg.rope_theta ** (-2 * j / hd)
            out[j] = vec[j] * math.cos(a) - vec[j + half] * math.sin(a)
            out[j + half] = vec[j + half] * math.cos(a) + vec[j] * math.sin(a)
        return out

    n = len(ids)
    h = [list(g["emb"][t]) for t in ids]
    if extra is not None:
        h = [[h[i][c] + extra[i][c] for c in range(d)] for i in range(n)]
    new_k, new_v = [], []
    for l in range(cfg.n_layers):
        xs = [norm(h[i], g[f"l{l}.attn_norm"]) for i in range(n)]
        qs, ks, vs = [], [], []
        for i in range(n):
            q = mv(g[f"l{l}.wq"], xs[i])
            k = mv(g[f"l{l}.wk"], xs[i])
            v = mv(g[f"l{l}.wv"], xs[i])
            qs.append([[_bf(t, bf) for t in rot(q[hh * hd:(hh + 1) * hd], pos[i])] for hh in range(Hq)])
            ks.append([[_bf(t, bf) for t in rot(k[hh * hd:(hh + 1) * hd], pos[i])] for hh in range(Hkv)])
            vs.append([[_bf(t, bf) for t in v[hh * hd:(hh + 1) * hd]] for hh in range(Hkv)])
        Kall = [list(map(list, ctx_k[l][j])) for j in range(len(ctx_k[l]))] + ks
        Vall = [list(map(list, ctx_v[l][j])) for j in range(len(ctx_v[l]))] + vs
        kpos = list(range(len(ctx_k[l]))) + list(pos)
        new_k.append(ks)
        new_v.append(vs)
        for i in range(n):
            o = []
            for hh in range(Hq):
                gg = hh * Hkv // Hq
                sc = [(j, sum(qs[i][hh][c] * Kall[j][gg][c] for c in range(hd)) / math.sqrt(hd))
                      for j in range(len(Kall)) if not (causal and kpos[j] > pos[i])]
                mx = max(s for _, s in sc)
                tot = sum(math.exp(s - mx) for _, s in sc)
                o += [_bf(sum(math.exp(s - mx) * Vall[j][gg][c] for j, s in sc) / tot, bf)
                      for c in range(hd)]
            att = mv(g[f"l{l}.wo"], o)
            h[i] = [h[i][c] + att[c] for c in range(d)]
        for i in range(n):
            x = norm(h[i], g[f"l{l}.ffn_norm"])
            r = [float(np.float32(v)) for v in mv(g[f"l{l}.w_router"], x)]
            sel = sorted(range(E), key=lambda e: (-r[e], e))[:K]
            mx = max(r[e] for e in sel)
            wsum = sum(math.exp(r[e] - mx) for e in sel)
            y = [0.0] * d
            for e in sel:
                gt = mv(g[f"l{l}.w_gate"][e], x)
                up = mv(g[f"l{l}.w_up"][e], x)
                a = [_bf(gt[f] / (1 + math.exp(-gt[f])) * up[f], bf) for f in range(F)]
                dn = mv(g[f"l{l}.w_down"][e], a)
                wt = math.exp(r[e] - mx) / wsum
                y = [y[c] + wt * dn[c] for c in range(d)]
            h[i] = [h[i][c] + y[c] for c in range(d)]
    xf = [norm(h[i], g["final_norm"]) for i in range(n)]
    logits = [mv(g["emb"], xf[i]) for i in range(n)]
    return np.array(logits), new_k, new_v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_model_matches_loop_forward(dtype):
    cfg = _micro_cfg(dtype=dtype, E=4, k=2, L=2)
    W = di.make_weights(cfg, 12, gain_std=0.2)
    m = OracleModel(cfg, W, 1, 32)
    prompt = np.array([[3, 9, 1, 15]])
    m.encode_prompt(prompt)
    # loop reference for the prompt (causal) gives the cache the canvas step sees
    _, pk, pv = _forward_loops(cfg, W, list(prompt[0]), list(range(4)), [[]] * 2, [[]] * 2, True)
    for l in range(2):
        kk = np.array(pk[l])                                  # [4, Hkv, hd]
        assert np.allclose(m.k_cache[l][0, :, :4].transpose(1, 0, 2), kk, rtol=1e-9, atol=1e-12)
    canvas = np.array([[2, 2, 7, 0, 11]])
    sp = di.SamplerConfig(max_steps=4, entropy_bound=0.1)
    out = m.denoise_step(canvas, 0, sp, np.array([5], np.uint64), want_logits=True)
    ref, _, _ = _forward_loops(cfg, W, list(canvas[0]), list(range(4, 9)),
                               [np.array(pk[l]) for l in range(2)],
                               [np.array(pv[l]) for l in range(2)], False)
    assert np.allclose(out["logits"][0], ref, rtol=1e-5, atol=1e-7)


def test_encode_then_commit_equals_joint_encode():
    cfg = _micro_cfg(dtype="bf16", E=4, k=2, L=2)
    W = di.make_weights(cfg, 13)
    a = OracleModel(cfg, W, 1, 32)
    b = OracleModel(cfg, W, 1, 32)
    p = np.array([[1, 2, 3, 4, 5, 6]])
    c = np.array([[7, 8, 9, 10, 11]])
    a.encode_prompt(p)
    a.commit_canvas_to_kv(c)
    b.encode_prompt(np.concatenate([p, c], 1))
    for l in range(2):
        assert np.array_equal(a.k_cache[l], b.k_cache[l])
        assert np.array_equal(a.v_cache[l], b.v_cache[l])
    assert a.ctx == b.ctx == 11 and a.canvas_index == 1


def test_self_conditioning_enters_next_step():
    cfg = _micro_cfg(dtype="f32", E=4, k=2, L=1, sc=True)
    W = di.make_weights(cfg, 14)
    m = OracleModel(cfg, W, 1, 32)
    m.encode_prompt(np.array([[1, 2, 3]]))
    sp = di.SamplerConfig(max_steps=4, entropy_bound=0.1)
    c = np.array([[4, 5, 6, 7, 8]])
    seeds = np.array([1], np.uint64)
    o0 = m.denoise_step(c, 0, sp, seeds, want_logits=True, trace_requests=[0])
    s1 = m.s[0].copy()
    # s equals softmax(l / T) E with the step-0 temperature
    z = o0["logits"][0].astype(np.float64) * float(o0["inv_t"])
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(s1, p @ nm.upcast(W.get("emb")))
    o1 = m.denoise_step(c, 1, sp, seeds, trace_requests=[0])
    h0 = o1["traces"][0]["h0"]
    assert np.allclose(h0, nm.upcast(W.get("emb"))[c[0]] + s1 @ nm.upcast(W.get("w_sc")).T)


def test_random_weights_never_commit_or_stop():
    wl = di.workload("tiny")
    W = di.make_weights(wl.model, wl.seed)
    m = OracleModel(wl.model, W, 1, 64 + 256)
    seeds = di.request_seeds(wl.seed, 1)
    m.encode_prompt(di.make_prompts(wl.model.vocab, 1, wl.prompt_len, wl.seed))
    from oracle.loop import run_canvas
    sp = di.SamplerConfig(max_steps=3, entropy_bound=0.5, stop_mode=1, stop_tau=0.05)
    res = run_canvas(m, sp, seeds)
    assert [int(s["n_committed"][0]) for s in res["steps"]] == [0, 0, 256]


# ------------------------------------------------------------------ FP8 (OCP E4M3)
def test_e4m3_hand_listed_codes():
    from oracle import fp8
    # (value, code) pairs written out from the format: bias 7, 3 mantissa bits
    cases = [(0.0, 0x00), (1.0, 0x38), (-1.0, 0xB8), (0.5, 0x30), (1.125, 0x39), (1.75, 0x3E), (2.0, 0x40),
             (448.0, 0x7E), (-448.0, 0xFE), (256.0, 0x78), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
             (7 * 2.0 ** -9, 0x07), (1.75 * 2.0 ** -6, 0x0E), (1.875 * 2.0 ** -6, 0x0F), (240.0, 0x77)]
    for v, c in cases:
        assert int(fp8.encode(np.array([v]))[0]) == c, (v, hex(c))
        assert fp8.decode(np.array([c], np.uint8))[0] == v, (v, hex(c))
    # NaN codes; -0
    assert np.isnan(fp8.decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert int(fp8.encode(np.array([-0.0]))[0]) == 0x80


def test_e4m3_round_to_nearest_even_and_saturation():
    from oracle import fp8
    cases = [(1.0625, 0x38),          # halfway 1.0 / 1.125 -> even mantissa 0
             (1.1875, 0x3A),          # halfway 1.125 / 1.25 -> even mantissa 2
             (1.06, 0x38), (1.07, 0x39), (1.1, 0x39),
             (2.0 ** -10, 0x00),      # halfway 0 / 2^-9 -> 0
             (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8 -> even mantissa 2
             (15.5 * 2.0 ** -10, 0x08),  # halfway 7 * 2^-9 / 2^-6 -> even: the smallest normal
             (464.0, 0x7E), (500.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE),   # saturate, never NaN
             (0.9999999, 0x38), (447.9, 0x7E), (432.0, 0x7E), (431.0, 0x7D)]
    for v, c in cases:
        assert int(fp8.encode(np.array([v]))[0]) == c, (v, hex(int(fp8.encode(np.array([v]))[0])), hex(c))


def test_e4m3_round_trip_and_nearest():
    from oracle import fp8
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = fp8.decode(codes)
    # every finite code survives decode -> encode (the zero pair aside, -0 keeps its sign bit)
    assert np.array_equal(fp8.encode(vals), codes)
    # brute force: random values map to the nearest representable value (ties to even code)
    rng = np.random.default_rng(12)
    x = rng.standard_normal(20000) * 50
    pos = np.sort(np.unique(np.abs(vals)))
    got = np.abs(fp8.decode(fp8.encode(x)))
    a = np.minimum(np.abs(x), 448.0)
    best = pos[np.argmin(np.abs(pos[None, :] - a[:, None]), axis=1)]
    assert np.array_equal(got, best)


def test_e4m3_row_quantisation():
    from oracle import fp8
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((6, 40)) * 0.02).astype(np.float32)
    w[3] = 0.0
    q, s = fp8.quantize_rows(w)
    # the largest magnitude of a row maps to 448 (or just below it by the fp32 division)
    assert s[3] == 1.0 and (q[3] == 0).all()
    for r in (0, 1, 2, 4, 5):
        assert s[r] == np.float32(np.abs(w[r]).max() / 448.0)
        assert np.abs(fp8.decode(q[r])).max() == 448.0
    deq = fp8.dequantize_rows(q, s)
    # relative error of a quantised weight: at most half an ulp of 3 mantissa bits (1/16) above the subnormals
    big = np.abs(w) >= 2.0 ** -6 * s[:, None]
    assert (np.abs(deq - w)[big] <= np.abs(w)[big] / 16 + 1e-12).all()


class _Replaced:
    """A weight set with some tensors replaced (the rest from the base set)."""

    def __init__(self, base, **tensors):
        self.base, self.tensors = base, tensors

    def get(self, name):
        return self.tensors[name] if name in self.tensors else self.base.get(name)


def test_fp8_head_rounds_only_off_grid_entries():
    """The FP8 LM head reads each row of E as its E4M3 codes times the row's scale.

    Rows of E here are exact E4M3 values times 2^-8 with a 448 * 2^-8 entry, so
    each row's scale is exactly 2^-8 and the codes hold those rows exactly,
    except two hand-placed entries off the E4M3 grid in column 5: 1.0625 in row
    3 (a tie between 1.0 and 1.125: to the even mantissa, 1.0) and 1.1875 in
    row 7 (a tie between 1.125 and 1.25: to 1.25), both times 2^-8.  The FP8
    head's logits then equal the stored-E head's on every other row, and on rows
    3 and 7 differ by x[5] * (-1/16) * 2^-8 and x[5] * (+1/16) * 2^-8: equal
    and opposite.  The embedding lookup keeps the stored E."""
    import dataclasses
    from oracle import fp8
    cfg = _micro_cfg(sc=True)
    cfg8 = dataclasses.replace(cfg, head_dtype="fp8")
    V, d = cfg.vocab, cfg.d_model
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 0x7F, size=(V, d)).astype(np.uint8) | (rng.integers(0, 2, size=(V, d)) << 7).astype(np.uint8)
    codes[:, 0] = np.where(rng.integers(0, 2, size=V) == 1, 0xFE, 0x7E)      # -448 or +448
    E = (fp8.decode(codes) * 2.0 ** -8).astype(np.float32)
    E[3, 5] = 1.0625 * 2.0 ** -8
    E[7, 5] = 1.1875 * 2.0 ** -8
    W = _Replaced(di.make_weights(cfg, 5, gain_std=0.3), emb=E)
    sp = di.SamplerConfig(4, 0.1)
    seeds = di.request_seeds(5, 1)
    canvas = rng.integers(0, V, size=(1, cfg.canvas_len)).astype(np.int32)
    prompt = rng.integers(0, V, size=(1, 3))
    res = []
    for c in (cfg, cfg8):
        m = OracleModel(c, W, 1, 16)
        m.encode_prompt(prompt)
        res.append(m.denoise_step(canvas, 0, sp, seeds, want_logits=True, trace_requests=[0]))
    a, b = res[0]["logits"][0].astype(np.float64), res[1]["logits"][0].astype(np.float64)
    others = [v for v in range(V) if v not in (3, 7)]
    assert np.array_equal(a[:, others], b[:, others])
    d3, d7 = b[:, 3] - a[:, 3], b[:, 7] - a[:, 7]
    assert np.abs(d3).min() > 0
    scale = np.abs(a).max()
    assert np.allclose(d3, -d7, rtol=0, atol=4 * 2.0 ** -24 * scale)
    assert np.array_equal(res[0]["traces"][0]["h0"], res[1]["traces"][0]["h0"])


# ------------------------------------------------------------------ training-side corruption and loss
def test_corruption_rates_and_uniform_replacement():
    from oracle import training as tr
    V, n = 64, 256
    clean = np.arange(n, dtype=np.int32) % V
    # rate 0: nothing changes; rate 1: every position redrawn (a redraw may hit the clean token)
    x0, r0 = tr.corrupt(clean, 0.0, 5, 0, V)
    assert np.array_equal(x0, clean) and not r0.any()
    x1, r1 = tr.corrupt(clean, 1.0, 5, 0, V)
    assert r1.all()
    # the replaced fraction follows the rate (binomial, 5 sigma over 200 canvases)
    hits, toks = 0, []
    for s in range(200):
        x, r = tr.corrupt(clean, 0.3, s, 0, V)
        hits += int(r.sum())
        toks.append(x[r])
        assert np.array_equal(x[~r], clean[~r])
    N = 200 * n
    assert abs(hits - 0.3 * N) < 5 * np.sqrt(N * 0.3 * 0.7)
    c = np.bincount(np.concatenate(toks), minlength=V).astype(np.float64)
    e = c.sum() / V
    assert ((c - e) ** 2 / e).sum() < 140                     # df = 63
    # the draws are the counter layout's: word 0 of the call decides, word 1 is the token
    w = philox.philox4x32_10(np.array([0, 7, 0, (tr.TAG_CORRUPT << 24) | 3], np.uint32),
                             philox.seed_key(11))
    x, r = tr.corrupt(np.zeros(8, np.int32), 0.5, 11, 3, V)
    assert r[7] == (philox.uniform01(w[0:1])[0] < np.float32(0.5))
    assert x[7] == (philox.uniform_token(w[1:2], V)[0] if r[7] else 0)


def test_denoising_cross_entropy_closed_forms():
    from oracle import training as tr
    V = 512
    # uniform logits: CE = log V for any target
    assert np.allclose(tr.logsumexp(np.zeros((3, V))) - 0.0, math.log(V), rtol=0, atol=1e-12)
    # a dominant logit at the target: CE -> 0; at another id: CE ~ the gap
    lg = np.zeros(V)
    lg[7] = 50.0
    assert tr.logsumexp(lg) - lg[7] < 1e-19
    assert abs((tr.logsumexp(lg) - lg[8]) - 50.0) < 1e-12
    # the explicit formula -log softmax(l)[t] by a per-element loop on a small vocabulary
    rng = np.random.default_rng(14)
    l = rng.standard_normal(9) * 3
    for t in range(9):
        p = math.exp(l[t]) / sum(math.exp(v) for v in l)
        assert abs((tr.logsumexp(l) - l[t]) - (-math.log(p))) < 1e-12


def test_forward_loss_scores_the_clean_tokens():
    from oracle import training as tr
    cfg = _micro_cfg(dtype="f32", E=4, k=2, L=1)
    W = di.make_weights(cfg, 15)
    m = OracleModel(cfg, W, 2, 32)
    m.encode_prompt(np.array([[1, 2, 3], [4, 5, 6]]))
    clean = np.array([[3, 9, 1, 15, 0], [2, 2, 7, 0, 11]], np.int32)
    out = tr.forward_loss(m, clean, [0.0, 1.0], np.array([3, 4], np.uint64), want_logits=True)
    assert np.array_equal(out["corrupted"][0], clean[0])            # rate 0 keeps the canvas
    assert out["replaced"][1].all()
    for b in range(2):
        lg = out["logits"][b]
        for i in range(5):
            ce = -math.log(math.exp(lg[i, clean[b, i]]) / sum(math.exp(v) for v in lg[i]))
            assert abs(out["ce"][b, i] - ce) < 1e-12
        assert abs(out["loss"][b] - out["ce"][b].mean()) < 1e-15
    # the rate-0 request's logits are the denoising round's on the same canvas
    sp = di.SamplerConfig(max_steps=4, entropy_bound=0.1)
    ref = m.denoise_step(clean, 0, sp, np.array([3, 4], np.uint64), want_logits=True)
    assert np.allclose(out["logits"][0], ref["logits"][0], rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ top-k truncated sampler
def test_topk_truncation_special_cases():
    V = 4096
    rng = np.random.default_rng(16)
    lg = (rng.standard_normal((6, V)) * 2).astype(np.float32)
    full = smp.head_stats(lg, np.float32(1.25), 3, 1, 2, np.arange(6))
    # k = V: the truncated distribution is the full one (same draws, same statistics)
    allk = smp.head_stats_topk(lg, np.float32(1.25), V, 3, 1, 2, np.arange(6))
    assert np.array_equal(allk["y"], full["y"]) and np.array_equal(allk["am"], full["am"])
    assert np.allclose(allk["H"], full["H"], rtol=1e-6)
    assert np.allclose(allk["margin"], full["margin"], atol=1e-6)
    # k = 1: the argmax with probability 1, entropy 0
    one = smp.head_stats_topk(lg, np.float32(1.25), 1, 3, 1, 2, np.arange(6))
    assert np.array_equal(one["y"], full["am"]) and np.all(one["H"] == 0)
    # k = 8: entropy at most log 8, the sample among the 8 largest logits, ids in descending order
    k8 = smp.head_stats_topk(lg, np.float32(1.25), 8, 3, 1, 2, np.arange(6), want_probs=True)
    for r in range(6):
        top = np.argsort(-lg[r], kind="stable")[:8]
        assert list(k8["ids"][r]) == list(top)
        assert k8["y"][r] in top and 0 <= k8["H"][r] <= math.log(8) + 1e-6
        z = lg[r, top].astype(np.float64) * np.float64(np.float32(1.25))
        p = np.exp(z - z.max()); p /= p.sum()
        assert np.allclose(k8["p"][r], p) and abs(k8["H"][r] + (p * np.log(p)).sum()) < 1e-5
    # uniform logits: the lowest k ids, entropy exactly log k
    u = smp.head_stats_topk(np.zeros((1, V), np.float32), np.float32(1.0), 8, 3, 1, 2, np.arange(1))
    assert list(u["ids"][0]) == list(range(8)) and u["H"][0] == np.float32(math.log(8))


def test_topk_gumbel_max_frequencies():
    # over many positions the truncated sample follows the renormalised top-k softmax (chi-square)
    z = np.log(np.array([0.3, 0.25, 0.2, 0.1, 0.05, 0.04, 0.03, 0.03]))
    n = 20000
    lg = np.tile(z.astype(np.float32), (n, 1))
    st = smp.head_stats_topk(lg, np.float32(1.0), 4, 11, 0, 0, np.arange(n))
    c = np.bincount(st["y"], minlength=8).astype(np.float64)
    assert c[4:].sum() == 0
    p = np.exp(z[:4]) / np.exp(z[:4]).sum()
    chi2 = ((c[:4] - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 25                                             # df = 3


def test_topk_forced_selection():
    # a forced id set equal to the row's own selection changes nothing; another set is
    # reordered by logit and the statistics are those of its renormalised softmax
    V = 512
    rng = np.random.default_rng(17)
    lg = (rng.standard_normal((3, V)) * 2).astype(np.float32)
    own = smp.head_stats_topk(lg, np.float32(1.0), 4, 5, 0, 1, np.arange(3), want_probs=True)
    same = smp.head_stats_topk(lg, np.float32(1.0), 4, 5, 0, 1, np.arange(3), want_probs=True,
                               forced_ids=[own["ids"][0][::-1].copy(), None, None])
    for key in ("H", "y", "am", "margin", "ids", "p"):
        assert np.array_equal(own[key], same[key])
    alt = np.argsort(-lg[1], kind="stable")[[0, 1, 2, 4]]          # the 4th largest swapped for the 5th
    f = smp.head_stats_topk(lg, np.float32(1.0), 4, 5, 0, 1, np.arange(3), want_probs=True,
                            forced_ids=[None, alt[::-1].copy(), None])
    assert list(f["ids"][1]) == list(alt)
    z = lg[1, alt].astype(np.float64)
    p = np.exp(z - z.max()); p /= p.sum()
    assert np.allclose(f["p"][1], p) and abs(f["H"][1] + (p * np.log(p)).sum()) < 1e-5
    assert f["y"][1] in alt
    for key in ("H", "y", "am", "margin"):
        assert f[key][0] == own[key][0] and f[key][2] == own[key][2]
