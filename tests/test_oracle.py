"""Pins of the CPU fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: the golden
mask of the Guide's demo layer, mpmath at 40 digits, a library attention routine
(torch's scaled_dot_product_attention in float64 with the cap switched off),
closed forms and invariants.  Chosen so that a dropped scale, a wrong tanh sign,
a wrong head index, a transposed operand, an off-by-one window, a mask applied
before the cap or a wrong causal alignment fails at least one test.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from attention_g2attn_prefill_amd import synth

mpmath.mp.dps = 40


def rand(shape, seed, mul=1.0):
    return synth.draw(shape, seed, 0, dtype="f32", mul=mul).numpy()


def page_mask(T, S, window, is_local):
    """Visibility built with torch.triu / torch.tril the way the Guide's demo
    layer builds it (-inf above the diagonal; on sliding layers also at and below
    offset -window), shifted so query row t sits at key column t + S - T."""
    off = S - T
    causal = torch.triu(torch.full((T, S), float("-inf"), dtype=torch.float64),
                        diagonal=1 + off)
    m = causal
    if is_local:
        m = m + torch.tril(torch.full((T, S), float("-inf"), dtype=torch.float64),
                           diagonal=off - window)
    return (m == 0).numpy()


# --------------------------------------------------------------- mask and cap

def test_mask_matches_guide_demo_golden(golden_dir):
    rows = [ln.strip() for ln in open(f"{golden_dir}/mask_seq16_window4.txt")
            if ln.strip() and not ln.startswith("#")]
    gold = np.array([[c == "1" for c in r] for r in rows])
    assert gold.shape == (16, 16)
    got = np.array([[oracle.allowed(p, j, 4, True) for j in range(16)]
                    for p in range(16)])
    assert np.array_equal(got, gold)
    # the oracle's logits put -inf exactly where the golden grid says masked
    q = rand((1, 16, 1, 4), 11)
    k = rand((1, 16, 1, 4), 12)
    for t in range(16):
        s = oracle.row_logits(q, k, 0, t, 0, query_scale=0.5, softcap=50.0,
                              window=4, is_local=True)
        assert np.array_equal(np.isfinite(s), gold[t])


def test_global_mask_is_causal():
    got = np.array([[oracle.allowed(p, j, 4, False) for j in range(16)]
                    for p in range(16)])
    assert np.array_equal(got, np.tril(np.ones((16, 16), bool)))


@pytest.mark.parametrize("x", [0.0, 1e-8, -3.5, 12.25, 49.0, -50.0, 77.7,
                               -300.0, 899.0, 2000.0, -1e6])
def test_softcap_matches_mpmath(x):
    cap = 50.0
    ref = mpmath.mpf(cap) * mpmath.tanh(mpmath.mpf(x) / cap)
    got = oracle.softcap(x, cap)
    assert abs(mpmath.mpf(got) - ref) <= 4e-16 * max(1.0, abs(float(ref)))
    assert abs(got) <= cap
    if abs(x) < 900:
        assert abs(got) < cap


@pytest.mark.parametrize("cap", [0.0, -1.0, math.inf])
def test_softcap_disabled_is_identity(cap):
    for x in (-123.5, 0.0, 7.25, 1e5):
        assert oracle.softcap(x, cap) == x


def test_softcap_taylor_limit():
    # cap*tanh(x/cap) = x - x^3/(3 cap^2) + ...: within |x|^3/(3cap^2) of x
    cap = 1e4
    for x in np.linspace(-20, 20, 41):
        s = oracle.softcap(float(x), cap)
        assert abs(s - x) <= abs(x) ** 3 / (3 * cap * cap) + 1e-15


# ------------------------------------------------------- logits and weights

def _mp_logits(q, k, b, t, h, qs, cap, window, is_local, G):
    T, S = q.shape[1], k.shape[1]
    p = t + S - T
    g = h // G
    out = []
    for j in range(S):
        if j > p or (is_local and not j > p - window):
            out.append(None)
            continue
        x = mpmath.fsum(mpmath.mpf(float(q[b, t, h, e])) * qs *
                        mpmath.mpf(float(k[b, j, g, e])) for e in range(q.shape[3]))
        out.append(cap * mpmath.tanh(x / cap) if cap > 0 else x)
    return out


@pytest.mark.parametrize("is_local", [False, True])
def test_row_logits_and_weights_match_mpmath(is_local):
    B, T, S, H, KVH, d = 2, 9, 13, 4, 2, 8
    q = rand((B, T, H, d), 21, mul=6.0)
    k = rand((B, S, KVH, d), 22, mul=3.0)
    qs, cap, W = 0.35, 50.0, 5
    for (b, t, h) in [(0, 0, 0), (1, 8, 3), (0, 4, 1), (1, 2, 2)]:
        ref = _mp_logits(q, k, b, t, h, mpmath.mpf(qs), mpmath.mpf(cap), W,
                         is_local, H // KVH)
        s = oracle.row_logits(q, k, b, t, h, query_scale=qs, softcap=cap,
                              window=W, is_local=is_local)
        w = oracle.row_weights(q, k, b, t, h, query_scale=qs, softcap=cap,
                               window=W, is_local=is_local)
        live = [r for r in ref if r is not None]
        m = max(live)
        z = mpmath.fsum(mpmath.exp(r - m) for r in live)
        for j, r in enumerate(ref):
            if r is None:
                assert s[j] == -math.inf and w[j] == 0.0
            else:
                assert abs(s[j] - float(r)) <= 1e-13 * max(1.0, abs(float(r)))
                assert abs(w[j] - float(mpmath.exp(r - m) / z)) <= 1e-14
        assert abs(w.sum() - 1.0) <= 1e-14


def test_capped_logits_are_bounded():
    q = rand((1, 64, 2, 16), 31, mul=40.0)
    k = rand((1, 64, 1, 16), 32, mul=40.0)
    xs = []
    for t in range(0, 64, 7):
        s = oracle.row_logits(q, k, 0, t, 1, query_scale=0.25, softcap=50.0,
                              window=64, is_local=False)
        f = s[np.isfinite(s)]
        assert np.all(np.abs(f) <= 50.0)
        raw = oracle.row_logits(q, k, 0, t, 1, query_scale=0.25, softcap=0.0,
                                window=64, is_local=False)
        xs.append(np.abs(raw[np.isfinite(raw)]).max())
    assert max(xs) > 100.0  # the check saw logits far beyond the cap


# ------------------------------------------------ library routine (cap off)

def _sdpa(q, k, v, qs, window, is_local):
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    G = H // KVH
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3)
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    mask = torch.from_numpy(page_mask(T, S, window, is_local))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                         scale=qs)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("T,S", [(37, 37), (7, 37), (1, 20)])
@pytest.mark.parametrize("is_local,window", [(False, 1), (True, 5), (True, 1),
                                             (True, 40)])
@pytest.mark.parametrize("H,KVH", [(4, 2), (6, 6), (4, 1)])
def test_cap_off_matches_library_attention(T, S, is_local, window, H, KVH):
    B, d = 2, 16
    q = rand((B, T, H, d), 41)
    k = rand((B, S, KVH, d), 42)
    v = rand((B, S, KVH, d), 43)
    qs = 0.3
    for cap in (0.0, math.inf):
        got = oracle.prefill(q, k, v, query_scale=qs, softcap=cap, window=window,
                             is_local=is_local)
        ref = _sdpa(q, k, v, qs, window, is_local)
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_large_cap_approaches_plain_attention():
    B, T, H, KVH, d = 1, 24, 2, 1, 8
    q = rand((B, T, H, d), 51)
    k = rand((B, T, KVH, d), 52)
    v = rand((B, T, KVH, d), 53)
    qs, cap = 0.5, 1e4
    capped = oracle.prefill(q, k, v, query_scale=qs, softcap=cap, window=4, is_local=True)
    plain = _sdpa(q, k, v, qs, 4, True)
    xmax = max(np.abs(oracle.row_logits(q, k, 0, t, h, query_scale=qs, softcap=0.0,
                                        window=4, is_local=True)[np.isfinite(
        oracle.row_logits(q, k, 0, t, h, query_scale=qs, softcap=0.0, window=4,
                          is_local=True))]).max() for t in range(T) for h in range(H))
    dlogit = xmax ** 3 / (3 * cap * cap)
    # each weight moves by at most a factor exp(+-2 dlogit)
    bound = 4 * dlogit * np.abs(v).max() + 1e-12
    assert np.max(np.abs(capped - plain)) <= bound
    assert np.max(np.abs(capped - plain)) > 0.0


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("is_local,window", [(False, 1), (True, 1), (True, 3),
                                             (True, 16), (True, 30)])
def test_zero_query_gives_window_mean(is_local, window):
    B, T, H, KVH, d = 2, 20, 4, 2, 6
    q = np.zeros((B, T, H, d), np.float32)
    k = rand((B, T, KVH, d), 61)
    v = rand((B, T, KVH, d), 62)
    out = oracle.prefill(q, k, v, query_scale=0.7, softcap=50.0, window=window,
                         is_local=is_local)
    v64 = v.astype(np.float64)
    for b in range(B):
        for t in range(T):
            lo = max(0, t - window + 1) if is_local else 0
            for h in range(H):
                ref = v64[b, lo:t + 1, h // 2].mean(axis=0)
                assert np.max(np.abs(out[b, t, h] - ref)) <= 1e-14


def test_window_one_returns_own_value():
    q = rand((2, 11, 4, 8), 71, mul=5.0)
    k = rand((2, 11, 2, 8), 72)
    v = rand((2, 11, 2, 8), 73)
    out = oracle.prefill(q, k, v, query_scale=0.3, softcap=50.0, window=1, is_local=True)
    for h in range(4):
        assert np.array_equal(out[:, :, h], v[:, :, h // 2].astype(np.float64))


@pytest.mark.parametrize("is_local", [False, True])
def test_first_row_returns_first_value(is_local):
    q = rand((3, 9, 2, 8), 81, mul=9.0)
    k = rand((3, 9, 1, 8), 82)
    v = rand((3, 9, 1, 8), 83)
    out = oracle.prefill(q, k, v, query_scale=1.0, softcap=50.0, window=3,
                         is_local=is_local)
    for h in range(2):
        assert np.array_equal(out[:, 0, h], v[:, 0, 0].astype(np.float64))


def test_window_at_least_T_equals_global():
    q = rand((1, 33, 4, 8), 91, mul=4.0)
    k = rand((1, 33, 2, 8), 92)
    v = rand((1, 33, 2, 8), 93)
    g = oracle.prefill(q, k, v, query_scale=0.4, softcap=50.0, window=1, is_local=False)
    for W in (33, 34, 1000):
        loc = oracle.prefill(q, k, v, query_scale=0.4, softcap=50.0, window=W,
                             is_local=True)
        assert np.array_equal(loc, g)
    loc = oracle.prefill(q, k, v, query_scale=0.4, softcap=50.0, window=32, is_local=True)
    assert not np.array_equal(loc, g)


def test_gqa_equals_repeated_heads():
    q = rand((2, 15, 8, 8), 101, mul=3.0)
    k = rand((2, 15, 4, 8), 102)
    v = rand((2, 15, 4, 8), 103)
    for is_local in (False, True):
        a = oracle.prefill(q, k, v, query_scale=0.5, softcap=50.0, window=4,
                           is_local=is_local)
        kr = np.repeat(k, 2, axis=2)
        vr = np.repeat(v, 2, axis=2)
        m = oracle.prefill(q, kr, vr, query_scale=0.5, softcap=50.0, window=4,
                           is_local=is_local)
        assert np.array_equal(a, m)


def test_constant_values_pass_through():
    q = rand((1, 12, 2, 8), 111, mul=10.0)
    k = rand((1, 12, 1, 8), 112)
    c = np.linspace(-2, 3, 8).astype(np.float32)
    v = np.broadcast_to(c, (1, 12, 1, 8)).copy()
    out = oracle.prefill(q, k, v, query_scale=0.9, softcap=50.0, window=5, is_local=True)
    assert np.max(np.abs(out - c.astype(np.float64))) <= 1e-14


def test_two_key_row_is_logistic_mix():
    q = rand((1, 2, 1, 4), 121, mul=8.0)
    k = rand((1, 2, 1, 4), 122, mul=8.0)
    v = rand((1, 2, 1, 4), 123)
    qs, cap = 0.5, 50.0
    out = oracle.prefill(q, k, v, query_scale=qs, softcap=cap, window=2, is_local=False)
    s = [cap * mpmath.tanh(mpmath.fsum(mpmath.mpf(float(q[0, 1, 0, e])) * qs *
                                       mpmath.mpf(float(k[0, j, 0, e]))
                                       for e in range(4)) / cap) for j in range(2)]
    w1 = 1 / (1 + mpmath.exp(s[0] - s[1]))
    w0 = 1 / (1 + mpmath.exp(s[1] - s[0]))
    ref = [float(w1 * float(v[0, 1, 0, e]) + w0 * float(v[0, 0, 0, e])) for e in range(4)]
    assert np.max(np.abs(out[0, 1, 0] - np.array(ref))) <= 1e-15


def test_saturated_logits_closed_form():
    # key 0 at x = +2000, the other n-1 keys at x = -2000: s = +-50 exactly
    n, d = 10, 2
    q = np.zeros((1, n, 1, d), np.float32)
    q[0, n - 1, 0, 0] = 40.0
    k = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = -50.0
    k[0, 0, 0, 0] = 50.0
    v = rand((1, n, 1, d), 131)
    out = oracle.prefill(q, k, v, query_scale=1.0, softcap=50.0, window=n, is_local=False)
    s = oracle.row_logits(q, k, 0, n - 1, 0, query_scale=1.0, softcap=50.0, window=n,
                          is_local=False)
    assert s[0] == 50.0 and np.all(s[1:] == -50.0)
    e = math.exp(-100.0)
    vm = v[0, 1:, 0].astype(np.float64).mean(axis=0)
    ref = (v[0, 0, 0].astype(np.float64) + (n - 1) * e * vm) / (1 + (n - 1) * e)
    assert np.max(np.abs(out[0, n - 1, 0] - ref)) <= 1e-15


def test_cap_is_applied_before_the_mask():
    # Every visible key has x = -2000 (s = -50).  Masked keys have x = +2000.
    # Capping first and then masking gives them weight 0, so the output is the
    # plain mean of the visible values; masking first and capping -inf to -50
    # would give masked keys the same weight as visible ones.
    T, d, W = 12, 2, 3
    q = np.zeros((1, T, 1, d), np.float32)
    q[0, :, 0, 0] = 40.0
    k = np.zeros((1, T, 1, d), np.float32)
    k[0, :, 0, 0] = -50.0
    k[0, 0:T:2, 0, 0] = 50.0  # even positions: large positive logits
    v = rand((1, T, 1, d), 141)
    out = oracle.prefill(q, k, v, query_scale=1.0, softcap=50.0, window=W, is_local=True)
    for t in range(T):
        lo = max(0, t - W + 1)
        vis = list(range(lo, t + 1))
        s = np.array([50.0 if j % 2 == 0 else -50.0 for j in vis])
        w = np.exp(s - s.max())
        w /= w.sum()
        ref = (w[:, None] * v[0, vis, 0].astype(np.float64)).sum(axis=0)
        assert np.max(np.abs(out[0, t, 0] - ref)) <= 1e-14


def test_linearity_in_values():
    q = rand((1, 17, 2, 8), 151, mul=4.0)
    k = rand((1, 17, 1, 8), 152)
    v1 = rand((1, 17, 1, 8), 153)
    v2 = rand((1, 17, 1, 8), 154)
    a, b = 0.75, -1.5
    kw = dict(query_scale=0.5, softcap=50.0, window=6, is_local=True)
    o1 = oracle.prefill(q, k, v1, **kw)
    o2 = oracle.prefill(q, k, v2, **kw)
    # round the combination to float32 and use the exact float32 value as input
    vc = (np.float32(a) * v1 + np.float32(b) * v2)
    dv = vc.astype(np.float64) - (a * v1.astype(np.float64) + b * v2.astype(np.float64))
    o = oracle.prefill(q, k, vc, **kw)
    bound = 1e-13 + np.abs(dv).max()
    assert np.max(np.abs(o - (a * o1 + b * o2))) <= bound


# ------------------------------------------------------------------- decode

@pytest.mark.parametrize("is_local", [False, True])
def test_decode_equals_last_prefill_row(is_local):
    B, S, H, KVH, d, W = 3, 40, 4, 2, 8, 7
    q = rand((B, 1, H, d), 161, mul=3.0)
    kc = rand((B, S, KVH, d), 162)
    vc = rand((B, S, KVH, d), 163)
    lens = np.array([1, 17, 40], np.int32)
    got = oracle.decode(q, kc, vc, lens, query_scale=0.4, softcap=50.0, window=W,
                        is_local=is_local)
    for b in range(B):
        L = int(lens[b])
        ref = oracle.prefill(q[b:b + 1], kc[b:b + 1, :L], vc[b:b + 1, :L],
                             query_scale=0.4, softcap=50.0, window=W, is_local=is_local)
        assert np.array_equal(got[b, 0], ref[0, 0])


@pytest.mark.parametrize("lens", [[13, 50, 64, 200], [1, 3, 8, 9]])
def test_decode_ring_equals_linear_cache(lens):
    B, S, H, KVH, d, W = 4, 200, 4, 2, 8, 8
    q = torch.from_numpy(rand((B, 1, H, d), 171, mul=3.0))
    kc = torch.from_numpy(rand((B, S, KVH, d), 172))
    vc = torch.from_numpy(rand((B, S, KVH, d), 173))
    lens = np.array(lens, np.int32)
    kr = synth.ring_from_linear(kc, lens, W)
    vr = synth.ring_from_linear(vc, lens, W)
    lin = oracle.decode(q.numpy(), kc.numpy(), vc.numpy(), lens, query_scale=0.4,
                        softcap=50.0, window=W, is_local=True)
    ring = oracle.decode(q.numpy(), kr.numpy(), vr.numpy(), lens, query_scale=0.4,
                         softcap=50.0, window=W, is_local=True)
    assert np.all(np.isfinite(ring))  # NaN-filled unused slots never read
    assert np.max(np.abs(ring - lin)) <= 1e-14


def test_decode_partial_ring_equals_global_prefix():
    B, H, KVH, d, W = 2, 2, 1, 8, 16
    q = torch.from_numpy(rand((B, 1, H, d), 181, mul=2.0))
    kc = torch.from_numpy(rand((B, 40, KVH, d), 182))
    vc = torch.from_numpy(rand((B, 40, KVH, d), 183))
    lens = np.array([5, 16], np.int32)
    kr = synth.ring_from_linear(kc, lens, W)
    vr = synth.ring_from_linear(vc, lens, W)
    loc = oracle.decode(q.numpy(), kr.numpy(), vr.numpy(), lens, query_scale=0.5,
                        softcap=50.0, window=W, is_local=True)
    glob = oracle.decode(q.numpy(), kc.numpy(), vc.numpy(), lens, query_scale=0.5,
                         softcap=50.0, window=W, is_local=False)
    assert np.max(np.abs(loc - glob)) <= 1e-14


def test_decode_rejects_unreachable_positions():
    q = rand((1, 1, 2, 4), 191)
    kc = rand((1, 8, 1, 4), 192)
    with pytest.raises(oracle.OracleError):
        oracle.decode(q, kc, kc, np.array([9], np.int32), query_scale=1.0, softcap=50.0,
                      window=8, is_local=False)
    with pytest.raises(oracle.OracleError):
        oracle.decode(q, kc, kc, np.array([0], np.int32), query_scale=1.0, softcap=50.0,
                      window=8, is_local=False)
    # a local layer with window <= S may hold any number of tokens (ring)
    oracle.decode(q, kc, kc, np.array([100], np.int32), query_scale=1.0, softcap=50.0,
                  window=8, is_local=True)


def test_rows_subset_matches_full():
    q = rand((2, 10, 4, 8), 201, mul=2.0)
    k = rand((2, 10, 2, 8), 202)
    v = rand((2, 10, 2, 8), 203)
    full = oracle.prefill(q, k, v, query_scale=0.4, softcap=50.0, window=3, is_local=True)
    rows = [0, 5, 79, 33]
    part = oracle.prefill(q, k, v, query_scale=0.4, softcap=50.0, window=3, is_local=True,
                          rows=rows)
    assert np.array_equal(part, full.reshape(-1, 8)[rows])


# ---------------------------------------------------------------- brute force

def test_brute_force_mpmath_tiny():
    """Every output element of a tiny layer recomputed at 40 digits with the
    mask taken from the Guide-style triu/tril construction."""
    B, T, S, H, KVH, d, W = 1, 6, 6, 2, 1, 3, 2
    q = rand((B, T, H, d), 211, mul=20.0)
    k = rand((B, S, KVH, d), 212, mul=3.0)
    v = rand((B, S, KVH, d), 213)
    qs, cap = 0.75, 50.0
    for is_local in (False, True):
        mask = page_mask(T, S, W, is_local)
        out = oracle.prefill(q, k, v, query_scale=qs, softcap=cap, window=W,
                             is_local=is_local)
        for t in range(T):
            for h in range(H):
                qv = [mpmath.mpf(float(x)) * mpmath.mpf(qs) for x in q[0, t, h]]
                s = {}
                for j in range(S):
                    if mask[t, j]:
                        x = mpmath.fsum(qv[e] * mpmath.mpf(float(k[0, j, 0, e]))
                                        for e in range(d))
                        s[j] = cap * mpmath.tanh(x / cap)
                m = max(s.values())
                z = mpmath.fsum(mpmath.exp(x - m) for x in s.values())
                for e in range(d):
                    ref = mpmath.fsum(mpmath.exp(s[j] - m) / z * mpmath.mpf(float(v[0, j, 0, e]))
                                      for j in s)
                    # logits near the cap carry ~ulp(50) = 7e-15 absolute error in fp64
                    assert abs(out[0, t, h, e] - float(ref)) <= 2e-14


# ---- paged-KV decode (Guide "Deep Dive" item 2: KV memory managed in blocks;
# local layers drop blocks older than the window)

def _paged_case(seed, B=3, S=48, H=4, KVH=2, d=8, lens=(1, 21, 48)):
    q = torch.from_numpy(rand((B, 1, H, d), seed, mul=3.0))
    kc = torch.from_numpy(rand((B, S, KVH, d), seed + 1))
    vc = torch.from_numpy(rand((B, S, KVH, d), seed + 2))
    return q, kc, vc, np.array(lens, np.int32)


@pytest.mark.parametrize("block_size", [1, 4, 16, 64])
@pytest.mark.parametrize("is_local,window", [(False, 4096), (True, 7), (True, 1), (True, 48)])
def test_decode_paged_equals_linear_cache(block_size, is_local, window):
    """Where a position's block sits in the pool does not change the result:
    any block placement gives exactly the (pinned) linear-cache decode, and
    dropped or unwritten blocks (NaN) are never read."""
    q, kc, vc, lens = _paged_case(201)
    kp, tab = synth.paged_from_linear(kc, lens, block_size, seed=3,
                                      keep_last=window if is_local else 0, spare_blocks=2)
    vp, tab2 = synth.paged_from_linear(vc, lens, block_size, seed=3,
                                       keep_last=window if is_local else 0, spare_blocks=2)
    assert np.array_equal(tab, tab2)
    kw = dict(query_scale=0.4, softcap=50.0, window=window, is_local=is_local)
    lin = oracle.decode(q.numpy(), kc.numpy(), vc.numpy(), lens, **kw)
    got = oracle.decode_paged(q.numpy(), kp.numpy(), vp.numpy(), tab, lens, **kw)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, lin)


def test_decode_paged_brute_force():
    """Independent numpy evaluation of the definition on a scattered pool."""
    B, H, KVH, d, bs, W = 2, 4, 2, 6, 3, 5
    rng = np.random.default_rng(211)
    nb = 9
    kp = rng.standard_normal((nb, bs, KVH, d)).astype(np.float32)
    vp = rng.standard_normal((nb, bs, KVH, d)).astype(np.float32)
    q = (3.0 * rng.standard_normal((B, 1, H, d))).astype(np.float32)
    tab = np.array([[4, 0, 7, -1], [2, 8, 1, 5]], np.int32)
    lens = np.array([8, 11], np.int32)
    qs, cap = 0.6, 5.0
    for is_local in (False, True):
        got = oracle.decode_paged(q, kp, vp, tab, lens, query_scale=qs, softcap=cap,
                                  window=W, is_local=is_local)
        for b in range(B):
            L = int(lens[b])
            js = np.arange(max(0, L - W) if is_local else 0, L)
            for h in range(H):
                g = h // (H // KVH)
                K = np.stack([kp[tab[b, j // bs], j % bs, g] for j in js]).astype(np.float64)
                V = np.stack([vp[tab[b, j // bs], j % bs, g] for j in js]).astype(np.float64)
                x = (q[b, 0, h].astype(np.float64) * qs) @ K.T
                s = cap * np.tanh(x / cap)
                w = np.exp(s - s.max())
                w /= w.sum()
                assert np.max(np.abs(got[b, 0, h] - w @ V)) <= 1e-13


def test_decode_paged_bad_block_gives_nan_row():
    q, kc, vc, lens = _paged_case(221)
    kp, tab = synth.paged_from_linear(kc, lens, 4, seed=5)
    vp, _ = synth.paged_from_linear(vc, lens, 4, seed=5)
    kw = dict(query_scale=0.4, softcap=50.0, window=4096, is_local=False)
    good = oracle.decode_paged(q.numpy(), kp.numpy(), vp.numpy(), tab, lens, **kw)
    bad_tab = tab.copy()
    bad_tab[1, 2] = kp.shape[0]          # a block the query needs, outside the pool
    bad = oracle.decode_paged(q.numpy(), kp.numpy(), vp.numpy(), bad_tab, lens, **kw)
    assert np.all(np.isnan(bad[1]))
    assert np.array_equal(bad[0], good[0]) and np.array_equal(bad[2], good[2])
    # an entry of a block the query cannot see is never looked up
    loc = dict(kw, window=5, is_local=True)
    ref = oracle.decode_paged(q.numpy(), kp.numpy(), vp.numpy(), tab, lens, **loc)
    far = tab.copy()
    far[2, 0] = 10 ** 6                   # positions 0..3, outside the window of L = 48
    assert np.array_equal(oracle.decode_paged(q.numpy(), kp.numpy(), vp.numpy(), far, lens, **loc), ref)


def test_decode_paged_rejects_bad_lengths():
    q, kc, vc, lens = _paged_case(231)
    kp, tab = synth.paged_from_linear(kc, lens, 8, seed=1)
    for bad in ([0, 21, 48], [1, 21, 49]):
        with pytest.raises(oracle.OracleError):
            oracle.decode_paged(q.numpy(), kp.numpy(), kp.numpy(), tab, np.array(bad, np.int32),
                                query_scale=1.0, softcap=50.0, window=4, is_local=True)


# ---- log-sum-exp of prefill rows (what a backward pass saves from the forward)

@pytest.mark.parametrize("is_local", [False, True])
def test_prefill_lse_matches_mpmath(is_local):
    B, T, S, H, KVH, d, W = 1, 9, 12, 4, 2, 6, 4
    q, k = rand((B, T, H, d), 241, mul=4.0), rand((B, S, KVH, d), 242)
    qs = mpmath.mpf(0.7)
    got = oracle.prefill_lse(q, k, query_scale=0.7, softcap=5.0, window=W, is_local=is_local)
    for t in range(T):
        for h in range(H):
            s = [x for x in _mp_logits(q, k, 0, t, h, qs, mpmath.mpf(5), W, is_local, 2)
                 if x is not None]
            ref = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
            assert abs(got[0, t, h] - float(ref)) <= 1e-13


def test_prefill_lse_closed_forms():
    B, T, S, H, KVH, d = 1, 30, 30, 2, 1, 8
    k = rand((B, S, KVH, d), 251)
    q0 = np.zeros((B, T, H, d), np.float32)
    # zero query: every visible logit is 0, lse = log(number of visible keys)
    glob = oracle.prefill_lse(q0, k, query_scale=1.0, softcap=50.0, window=7, is_local=False)
    loc = oracle.prefill_lse(q0, k, query_scale=1.0, softcap=50.0, window=7, is_local=True)
    t = np.arange(T)[None, :, None]
    assert np.max(np.abs(glob - np.log(t + 1.0))) <= 1e-14
    assert np.max(np.abs(loc - np.log(np.minimum(t + 1.0, 7.0)))) <= 1e-14
    # window 1: the row sees only itself, lse = its own capped logit
    q = rand((B, T, H, d), 252, mul=3.0)
    one = oracle.prefill_lse(q, k, query_scale=0.5, softcap=4.0, window=1, is_local=True)
    for tt in range(T):
        x = float(np.dot(q[0, tt, 0].astype(np.float64) * 0.5, k[0, tt, 0].astype(np.float64)))
        assert abs(one[0, tt, 0] - 4.0 * math.tanh(x / 4.0)) <= 1e-13


def test_prefill_lse_normalises_the_weights():
    """exp(s_j - lse) are the attention weights the (pinned) row routine gives."""
    B, T, S, H, KVH, d = 1, 20, 20, 2, 1, 8
    q, k = rand((B, T, H, d), 261, mul=3.0), rand((B, S, KVH, d), 262)
    kw = dict(query_scale=0.5, softcap=50.0, window=6, is_local=True)
    lse = oracle.prefill_lse(q, k, **kw)
    for t in (0, 5, 19):
        s = oracle.row_logits(q, k, 0, t, 1, **kw)
        w = oracle.row_weights(q, k, 0, t, 1, **kw)
        assert np.max(np.abs(np.exp(s - lse[0, t, 1]) - w)) <= 1e-14


# ---- adjacent steps: rotary embedding and the final-logit cap

def _rope_case(seed, B=2, T=9, NH=3, d=16, pmax=9000):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, NH, d)).astype(np.float32)
    pos = rng.integers(0, pmax, size=(B, T)).astype(np.int32)
    return x, pos


def test_rope_position_zero_is_identity():
    x, _ = _rope_case(271)
    assert np.array_equal(oracle.rope(x, np.zeros(x.shape[:2], np.int32)), x.astype(np.float64))


def test_rope_preserves_pair_norms():
    x, pos = _rope_case(272)
    y = oracle.rope(x, pos, base=10000.0)
    h = x.shape[-1] // 2
    nx = x[..., :h].astype(np.float64) ** 2 + x[..., h:].astype(np.float64) ** 2
    ny = y[..., :h] ** 2 + y[..., h:] ** 2
    assert np.max(np.abs(nx - ny)) <= 1e-12


def test_rope_scores_depend_only_on_relative_position():
    """<R(m) q, R(n) k> is unchanged when both positions shift by the same s."""
    x, pos = _rope_case(273, B=1, T=2, NH=1, d=64, pmax=4000)
    shifted = pos + 3171
    a = oracle.rope(x, pos)
    b = oracle.rope(x, shifted)
    assert abs(float(a[0, 0, 0] @ a[0, 1, 0]) - float(b[0, 0, 0] @ b[0, 1, 0])) <= 1e-10
    # and it does change with the distance
    c = oracle.rope(x, np.array([[pos[0, 0], pos[0, 1] + 1]], np.int32))
    assert abs(float(a[0, 0, 0] @ a[0, 1, 0]) - float(c[0, 0, 0] @ c[0, 1, 0])) > 1e-6


def test_rope_frequency_schedule():
    """A unit vector in pair i turns by pos * base**(-2i/d): pair 0 by pos
    radians, pair d/4 by pos / sqrt(base) (measured as an angle)."""
    d, base, p = 16, 10000.0, 5
    x = np.zeros((1, 1, 1, d), np.float32)
    x[..., 0] = 1.0
    x[..., d // 4] = 1.0
    y = oracle.rope(x, np.array([[p]], np.int32), base=base)[0, 0, 0]
    ang0 = math.atan2(y[d // 2], y[0])
    ang4 = math.atan2(y[d // 4 + d // 2], y[d // 4])
    assert abs(math.remainder(ang0 - p, 2 * math.pi)) <= 1e-12
    assert abs(ang4 - p / math.sqrt(base)) <= 1e-12


def test_softcap_array_matches_scalar_routine():
    x = np.array([-1e4, -75.0, -30.0, -1.5, 0.0, 1e-6, 2.0, 29.0, 300.0], np.float32)
    got = oracle.softcap_array(x, 30.0)
    for xi, gi in zip(x, got):
        assert gi == oracle.softcap(float(xi), 30.0)
    assert np.all(np.abs(got) < 30.0 + 1e-12)


# ---- backward pass (Guide "Deep Dive" item 1: d/dx cap*tanh(x/cap) = 1 - tanh^2)

def _grid_case(seed, B, T, S, H, KVH, d, span=3.0):
    """Inputs on a 2^-6 grid inside [-span, span], so x +- 2^-12 is exact in float32."""
    rng = np.random.default_rng(seed)
    f = lambda shape: (np.round(rng.uniform(-span, span, size=shape) * 64) / 64).astype(np.float32)
    return f((B, T, H, d)), f((B, S, KVH, d)), f((B, S, KVH, d)), f((B, T, H, d))


@pytest.mark.parametrize("is_local,window,cap", [(False, 4096, 5.0), (True, 3, 5.0),
                                                  (True, 4, 0.0), (False, 1, 2.0)])
def test_backward_matches_central_differences(is_local, window, cap):
    """Every gradient entry of L = sum(out * R) against central differences of
    the (pinned) forward oracle, step 2^-12."""
    B, T, S, H, KVH, d = 1, 6, 7, 4, 2, 4
    q, k, v, R = _grid_case(281, B, T, S, H, KVH, d)
    kw = dict(query_scale=0.5, softcap=cap, window=window, is_local=is_local)
    dq, dk, dv = oracle.prefill_backward(q, k, v, R, **kw)
    h = 2.0 ** -12
    R64 = R.astype(np.float64)

    def loss(qq, kk, vv):
        return float(np.sum(oracle.prefill(qq, kk, vv, **kw) * R64))

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += np.float32(h)
            minus[idx] -= np.float32(h)
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [plus if a is arr else a for a in args]
            am = [minus if a is arr else a for a in args]
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1.0 + abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("T,S", [(9, 9), (5, 11)])
@pytest.mark.parametrize("is_local,window", [(False, 1), (True, 3)])
def test_backward_cap_off_matches_library_autograd(T, S, is_local, window):
    """With the cap disabled the gradients are those of plain attention: torch
    autograd through scaled_dot_product_attention in float64, K/V repeated per
    query head (their gradients summed back over the group)."""
    B, H, KVH, d = 2, 4, 2, 8
    q, k, v = rand((B, T, H, d), 291, mul=2.0), rand((B, S, KVH, d), 292), rand((B, S, KVH, d), 293)
    R = rand((B, T, H, d), 294)
    dq, dk, dv = oracle.prefill_backward(q, k, v, R, query_scale=0.4, softcap=0.0, window=window,
                                         is_local=is_local)
    G = H // KVH
    qt = torch.tensor(q.astype(np.float64), requires_grad=True)
    kt = torch.tensor(k.astype(np.float64), requires_grad=True)
    vt = torch.tensor(v.astype(np.float64), requires_grad=True)
    mask = torch.from_numpy(page_mask(T, S, window, is_local))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(0, 2, 1, 3), kt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1),
        vt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1), attn_mask=mask, scale=0.4)
    (o.permute(0, 2, 1, 3) * torch.from_numpy(R.astype(np.float64))).sum().backward()
    assert np.max(np.abs(dq - qt.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dk - kt.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dv - vt.grad.numpy())) <= 1e-12


def test_backward_window_one_closed_form():
    """A row that sees only itself has weight 1: dv of a key is the sum of its
    group's upstream gradients at that position, and dq = dk = 0."""
    B, T, H, KVH, d = 1, 6, 4, 2, 8
    q, k, v = rand((B, T, H, d), 301, mul=3.0), rand((B, T, KVH, d), 302), rand((B, T, KVH, d), 303)
    R = rand((B, T, H, d), 304)
    dq, dk, dv = oracle.prefill_backward(q, k, v, R, query_scale=0.5, softcap=50.0, window=1,
                                         is_local=True)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    want = R.astype(np.float64).reshape(B, T, KVH, H // KVH, d).sum(axis=3)
    assert np.max(np.abs(dv - want)) <= 1e-14


# ---- gradients at sampled rows and keys (used where the full backward is too slow)

@pytest.mark.parametrize("B,T,S,H,KVH,d,window,is_local,cap", [
    (2, 40, 55, 4, 2, 16, 12, True, 50.0),    # T < S, local
    (1, 33, 33, 2, 1, 8, 33, False, 0.0),     # cap disabled
    (1, 30, 30, 4, 2, 8, 5, True, 1e6),       # accurate cap range
    (1, 20, 20, 4, 4, 8, 1, True, 5.0),       # window 1, one query head per K/V head
])
def test_backward_at_equals_full_backward(B, T, S, H, KVH, d, window, is_local, cap):
    """At every row and key, the sampled routine equals the full backward."""
    q, k, v, R = (rand((B, T, H, d), 311, mul=3.0), rand((B, S, KVH, d), 312, mul=3.0),
                  rand((B, S, KVH, d), 313), rand((B, T, H, d), 314))
    kw = dict(query_scale=0.3, softcap=cap, window=window, is_local=is_local)
    dq, dk, dv = oracle.prefill_backward(q, k, v, R, **kw)
    out, lse = oracle.prefill(q, k, v, **kw), oracle.prefill_lse(q, k, **kw)
    rows = [(b, t, h) for b in range(B) for t in range(T) for h in range(H)]
    keys = [(b, j, g) for b in range(B) for j in range(S) for g in range(KVH)]
    sq, sk, sv = oracle.prefill_backward_at(q, k, v, R, out, lse, rows=rows, keys=keys, **kw)
    for got, ref in ((sq, dq), (sk, dk), (sv, dv)):
        ref = ref.reshape(got.shape)
        assert np.max(np.abs(got - ref)) <= 1e-12 * (1.0 + np.max(np.abs(ref)))


def test_backward_at_matches_central_differences():
    """Sampled gradient entries against central differences of the forward
    oracle, step 2^-12 on grid inputs (independent of the full backward)."""
    B, T, S, H, KVH, d = 1, 7, 9, 4, 2, 4
    q, k, v, R = _grid_case(321, B, T, S, H, KVH, d)
    kw = dict(query_scale=0.5, softcap=5.0, window=4, is_local=True)
    out, lse = oracle.prefill(q, k, v, **kw), oracle.prefill_lse(q, k, **kw)
    rows, keys = [(0, 6, 1), (0, 3, 2)], [(0, 2, 0), (0, 8, 1)]
    sq, sk, sv = oracle.prefill_backward_at(q, k, v, R, out, lse, rows=rows, keys=keys, **kw)
    h = 2.0 ** -12
    R64 = R.astype(np.float64)

    def fd(arr, idx, which):
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += np.float32(h)
        minus[idx] -= np.float32(h)
        args = lambda a: tuple(a if n == which else x for n, x in (("q", q), ("k", k), ("v", v)))
        lp = np.sum(oracle.prefill(*args(plus), **kw) * R64)
        lm = np.sum(oracle.prefill(*args(minus), **kw) * R64)
        return (lp - lm) / (2 * h)

    for n, (b, t, hh) in enumerate(rows):
        for e in range(d):
            want = fd(q, (b, t, hh, e), "q")
            assert abs(want - sq[n, e]) <= 1e-6 * (1.0 + abs(want))
    for n, (b, j, g) in enumerate(keys):
        for e in range(d):
            want_k, want_v = fd(k, (b, j, g, e), "k"), fd(v, (b, j, g, e), "v")
            assert abs(want_k - sk[n, e]) <= 1e-6 * (1.0 + abs(want_k))
            assert abs(want_v - sv[n, e]) <= 1e-6 * (1.0 + abs(want_v))


def test_backward_dv_sums_to_upstream_gradient():
    """Each row's weights sum to 1, so summed over every key of a group, dv
    equals the sum of that group's upstream gradients over rows and heads."""
    B, T, S, H, KVH, d = 2, 30, 36, 4, 2, 8
    q, k, v, R = (rand((B, T, H, d), 331, mul=3.0), rand((B, S, KVH, d), 332),
                  rand((B, S, KVH, d), 333), rand((B, T, H, d), 334))
    for is_local, window in ((True, 5), (False, 36)):
        _, _, dv = oracle.prefill_backward(q, k, v, R, query_scale=0.4, softcap=50.0,
                                           window=window, is_local=is_local)
        want = R.astype(np.float64).reshape(B, T, KVH, H // KVH, d).sum(axis=(1, 3))
        assert np.max(np.abs(dv.sum(axis=1) - want)) <= 1e-12
