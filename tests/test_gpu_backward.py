"""GPU parity of the prefill backward pass (through the C ABI) against the
fp64 oracle, which recomputes the gradients from q, k, v and dO alone (the GPU
forward's out and lse are not trusted by the reference).

Tolerances, relative to the size of each reference gradient: max |diff| <=
2e-2 * max |ref| and mean |diff| <= 1e-2 * mean |ref|.  They follow from the
arithmetic: P and dS are rounded to bf16 (2^-9 relative) before the MFMAs that
build dV, dK and dQ, and the gradients are stored in bf16 (about 3e-3 of
relative error together); D = <dO, out> is formed from the bf16 output, an
error of about 2^-9 |D| that enters every dS_j = P_j (<dO, v_j> - D) of a row.
Where a row's attention is nearly one-hot (saturated logits, or a row that sees
few keys) the exact dS is far below that floor, so such rows' dq carries O(1)
relative error at a tiny absolute size; it raises the mean ratio to ~7e-3 on
the saturating case, hence the 1e-2 bound on the mean.  Gradients that are
exactly zero by definition (a row that sees only itself: dq = dk = 0) keep the
fp32 residue of <dO, v> - <dO, out> summed in two orders, so both bounds also
allow 1e-4 absolute.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_g2attn_prefill_amd import synth

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN, ABS_FLOOR = 2e-2, 1e-2, 1e-4


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def g2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_g2attn_prefill_amd as mod
    return mod


def check_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - ref)
    scale_max, scale_mean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    if got.ndim == 4:  # where the error sits: per position, relative to that position's size
        pe = err.mean(axis=(0, 2, 3)) / np.maximum(np.abs(ref).mean(axis=(0, 2, 3)), 1e-30)
        worst = np.argsort(pe)[-5:][::-1]
        say(f"{what}: worst positions {[(int(t), round(float(pe[t]), 4)) for t in worst]}")
    say(f"{what}: max|d|/max|ref|={err.max() / max(scale_max, 1e-30):.3e} "
        f"mean|d|/mean|ref|={err.mean() / max(scale_mean, 1e-30):.3e}")
    assert err.max() <= REL_MAX * scale_max + ABS_FLOOR, what
    assert err.mean() <= REL_MEAN * scale_mean + ABS_FLOOR, what


def run_backward(g2, q, k, v, dout, kw):
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), dout.cuda()
    out, lse = g2.prefill_lse(qd, kd, vd, **kw)
    dq, dk, dv = g2.prefill_backward(qd, kd, vd, out, gd, lse, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


BWD_CASES = [
    # B, T, S, H, KVH, d, window, is_local, q_mul, softcap
    (1, 200, 200, 4, 2, 256, 64, True, 3.0, 50.0),
    (1, 200, 200, 4, 2, 256, 64, False, 3.0, 50.0),
    (1, 300, 300, 4, 2, 128, 100, True, 3.0, 50.0),
    (2, 150, 150, 2, 2, 64, 150, False, 2.0, 50.0),        # one query head per K/V head
    (1, 100, 260, 4, 2, 256, 70, True, 3.0, 50.0),         # T < S
    (1, 130, 130, 4, 2, 128, 40, True, 5.5, 50.0),         # saturating logits
    (1, 120, 120, 4, 2, 256, 32, False, 2.0, 0.0),         # cap disabled
    (1, 120, 120, 4, 2, 64, 32, True, 2.0, 1e6),           # accurate cap form
    (1, 1, 1, 2, 1, 128, 1, True, 1.0, 50.0),              # one token
    (1, 77, 77, 2, 1, 256, 1, True, 3.0, 50.0),            # window 1
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"bwd{i}" for i in range(len(BWD_CASES))])
def test_backward_small(g2, case):
    B, T, S, H, KVH, d, W, is_local, qm, cap = case
    say(f"backward {case}")
    seed = 800 + d + T
    q = synth.draw((B, T, H, d), seed, 0, mul=qm)
    k = synth.draw((B, S, KVH, d), seed, 1, mul=qm if qm > 4 else 1.0)
    v = synth.draw((B, S, KVH, d), seed, 2)
    dout = synth.draw((B, T, H, d), seed, 3)
    kw = dict(query_scale=1 / np.sqrt(d), softcap=cap, window=W, is_local=is_local)
    dq, dk, dv = run_backward(g2, q, k, v, dout, kw)
    rq, rk, rv = oracle.prefill_backward(*(synth.to_f32_numpy(x) for x in (q, k, v, dout)), **kw)
    check_grad(synth.to_f32_numpy(dq), rq, f"dq {case}")
    check_grad(synth.to_f32_numpy(dk), rk, f"dk {case}")
    check_grad(synth.to_f32_numpy(dv), rv, f"dv {case}")


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_backward_9b_heads_1k(g2, is_local):
    """The 9B head layout (H=16, KVH=8, d=256) at 1024 positions, window 256."""
    B, T, H, KVH, d, W = 1, 1024, 16, 8, 256, 256
    say(f"backward 9b heads T={T} {'local' if is_local else 'global'}")
    q = synth.draw((B, T, H, d), 901, 0, mul=3.0)
    k = synth.draw((B, T, KVH, d), 901, 1, mul=3.0)
    v = synth.draw((B, T, KVH, d), 901, 2)
    dout = synth.draw((B, T, H, d), 901, 3)
    kw = dict(query_scale=1 / 16, softcap=50.0, window=W, is_local=is_local)
    dq, dk, dv = run_backward(g2, q, k, v, dout, kw)
    rq, rk, rv = oracle.prefill_backward(*(synth.to_f32_numpy(x) for x in (q, k, v, dout)), **kw)
    check_grad(synth.to_f32_numpy(dq), rq, "dq 9b-heads")
    check_grad(synth.to_f32_numpy(dk), rk, "dk 9b-heads")
    check_grad(synth.to_f32_numpy(dv), rv, "dv 9b-heads")


def test_backward_deterministic(g2):
    say("backward determinism")
    q = synth.draw((1, 300, 4, 256), 911, 0, mul=3.0)
    k = synth.draw((1, 300, 2, 256), 911, 1)
    v = synth.draw((1, 300, 2, 256), 911, 2)
    dout = synth.draw((1, 300, 4, 256), 911, 3)
    kw = dict(query_scale=1 / 16, softcap=50.0, window=100, is_local=True)
    a = run_backward(g2, q, k, v, dout, kw)
    b = run_backward(g2, q, k, v, dout, kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_backward_9b_8k_sampled(g2, is_local):
    """The 9B layer at full size, in the launch configuration the benchmark
    times (B=2, T=S=8192, H=16, KVH=8, d=256, window 4096).  Two (batch, K/V
    head) groups, one at each end of the grid, are checked at sampled query
    rows (dq) and keys (dk, dv) against the oracle, whose forward out and lse
    come from the oracle itself on that group's slice (groups are independent).
    Over every key, dv summed per group must equal the group's upstream
    gradient summed over rows and heads (each row's weights sum to 1)."""
    cfg = synth.WORKLOADS["9b-8k"]
    q, k, v = synth.prefill_inputs(cfg)
    dout = synth.draw(tuple(q.shape), 17, 3)
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    G, W = H // KVH, cfg["window"]
    kw = dict(query_scale=cfg["query_scale"], softcap=cfg["softcap"], window=W, is_local=is_local)
    say(f"backward full 9b-8k {'local' if is_local else 'global'}")
    dq, dk, dv = run_backward(g2, q, k, v, dout, kw)
    dqn, dkn, dvn = (synth.to_f32_numpy(x).astype(np.float64) for x in (dq, dk, dv))
    assert np.all(np.isfinite(dqn)) and np.all(np.isfinite(dkn)) and np.all(np.isfinite(dvn))

    # every key: sum of dv over keys == sum of dO over the group's rows and heads.
    # The weights enter dv rounded to bf16; a peaky row's top weight sits just
    # below 1, where the bf16 step is 2^-8, so each row's weights sum to 1 only
    # within about 2^-9.  Against the row's dO that gives an error of standard
    # deviation <= 2^-9 * sqrt(sum over the group's rows of dO^2) per element
    # (~0.25 here, |sum| ~ 100); the bound is five of those.
    g64 = synth.to_f32_numpy(dout).astype(np.float64).reshape(B, T, KVH, G, d)
    want = g64.sum(axis=(1, 3))
    bound = 5 * 2.0 ** -9 * np.sqrt((g64 ** 2).sum(axis=(1, 3)))
    got = dvn.sum(axis=1)
    err = np.abs(got - want)
    say(f"sum dv over keys: max|d|={err.max():.3e}, max |d|/bound={np.max(err / bound):.3f}")
    assert np.all(err <= bound)

    rng = np.random.default_rng(41)
    ts = sorted({0, 1, 31, 32, 63, W - 1, W, W + 1, T - 33, T - 1, *rng.integers(0, T, 6).tolist()})
    js = sorted({0, 1, 15, 16, 63, 64, W - 1, W, T - 65, T - 64, T - 2, T - 1,
                 *rng.integers(0, S, 6).tolist()})
    for b, g in ((0, 0), (B - 1, KVH - 1)):
        hs = slice(g * G, g * G + G)
        qn = synth.to_f32_numpy(q[b:b + 1, :, hs])
        kn = synth.to_f32_numpy(k[b:b + 1, :, g:g + 1])
        vn = synth.to_f32_numpy(v[b:b + 1, :, g:g + 1])
        gn = synth.to_f32_numpy(dout[b:b + 1, :, hs])
        out = oracle.prefill(qn, kn, vn, **kw)
        lse = oracle.prefill_lse(qn, kn, **kw)
        rows = [(0, t, hh) for t in ts for hh in range(G)]
        keys = [(0, j, 0) for j in js]
        rq, rk, rv = oracle.prefill_backward_at(qn, kn, vn, gn, out, lse, rows=rows, keys=keys,
                                                **kw)
        got_q = np.stack([dqn[b, t, g * G + hh] for (_, t, hh) in rows])
        check_grad(got_q, rq, f"dq rows of group ({b},{g})")
        check_grad(dkn[b, js, g], rk, f"dk keys of group ({b},{g})")
        check_grad(dvn[b, js, g], rv, f"dv keys of group ({b},{g})")


def test_backward_lse_at_a_4_byte_offset(g2):
    """lse need only be 4-byte aligned: a buffer starting one float into an
    allocation gives the same gradients, bit for bit, as an aligned one."""
    say("backward with lse at a 4-byte offset")
    B, T, H, KVH, d = 1, 96, 4, 2, 256
    q = synth.draw((B, T, H, d), 921, 0, mul=3.0).cuda()
    k = synth.draw((B, T, KVH, d), 921, 1).cuda()
    v = synth.draw((B, T, KVH, d), 921, 2).cuda()
    dout = synth.draw((B, T, H, d), 921, 3).cuda()
    kw = dict(query_scale=1 / 16, softcap=50.0, window=40, is_local=True)
    out_a, lse_a = g2.prefill_lse(q, k, v, **kw)
    base = torch.empty(B * H * T + 1, dtype=torch.float32, device="cuda")
    lse_b = base[1:].view(B, H, T)
    assert lse_b.data_ptr() % 16 == 4
    out_b = torch.empty_like(out_a)
    g2.prefill_lse(q, k, v, out=out_b, lse=lse_b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    ga = g2.prefill_backward(q, k, v, out_a, dout, lse_a, **kw)
    gb = g2.prefill_backward(q, k, v, out_b, dout, lse_b, **kw)
    torch.cuda.synchronize()
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)
