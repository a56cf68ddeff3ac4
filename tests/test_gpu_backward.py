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
the saturating case, hence the 1e-2 bound on the mean.

Rows that see only their own key (window 1, or a single token) have dq = dk = 0
exactly: the weight is 1, out = v, and dS = <dO, v> - <dO, out> = 0.  The GPU
forms the two dot products in fp32 in different orders, so it returns their
rounding residue instead; test_backward_rows_that_see_only_themselves bounds it
element by element from the summation error bound (see there).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_g2attn_prefill_amd import synth
from _report import report

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 1e-2


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
    report(f"{what}: max|d|/max|ref|={err.max() / max(scale_max, 1e-30):.3e} "
        f"mean|d|/mean|ref|={err.mean() / max(scale_mean, 1e-30):.3e}")
    assert scale_max > 0, f"{what}: all-zero reference (use the self-only test)"
    assert err.max() <= REL_MAX * scale_max, what
    assert err.mean() <= REL_MEAN * scale_mean, what


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
    (1, 100, 260, 4, 2, 256, 60, True, 3.0, 50.0),         # T < S: the oldest key blocks no row sees
    (1, 200, 330, 4, 2, 128, 20, True, 3.0, 50.0),
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


SELF_CASES = [
    # B, T, H, KVH, d, q_mul, softcap
    (1, 1, 2, 1, 128, 1.0, 50.0),       # one token
    (1, 77, 2, 1, 256, 3.0, 50.0),      # window 1
    (2, 64, 4, 2, 64, 3.0, 0.0),        # window 1, cap disabled
    (1, 50, 4, 4, 128, 3.0, 1e6),       # window 1, accurate cap form
]


@pytest.mark.parametrize("case", SELF_CASES, ids=[f"self{i}" for i in range(len(SELF_CASES))])
def test_backward_rows_that_see_only_themselves(g2, case):
    """Window 1 (or one token): every row sees only its own key with weight 1,
    so out = v, dv_j = the group's dO summed over its heads, and dq = dk = 0.

    The GPU's dq and dk are the rounding residue of dS = p (dP - D) with
    dP = <dO, v> (MFMA) and D = <dO, out> (the prep kernel): both sum the same
    d exact fp32 products of bf16 values, in different orders, so
    |dP - D| <= 2 gamma_d sum_e |dO_e v_e| with gamma_d = d u / (1 - d u),
    u = 2^-24 (the worst-case bound of recursive fp32 summation, any order).
    The cap's derivative is at most 1, and the recomputed weight
    p = exp(s - lse) is 1 up to the fp32 rounding of lse (p < 1.001), so
      |dq[t,h,e]| <= qs |k[t,e]| R[t,h],   |dk[t,e]| <= qs sum_h |q[t,h,e]| R[t,h],
    R = 1.001 * 2 gamma_d sum_e |dO v|, times (1 + 2^-7) for the two bf16
    roundings on the way (dS before its MFMA, and the stored gradient).
    dv is compared with the oracle like every other gradient."""
    B, T, H, KVH, d, qm, cap = case
    say(f"backward self-only rows {case}")
    seed = 700 + d + T
    q = synth.draw((B, T, H, d), seed, 0, mul=qm)
    k = synth.draw((B, T, KVH, d), seed, 1)
    v = synth.draw((B, T, KVH, d), seed, 2)
    dout = synth.draw((B, T, H, d), seed, 3)
    qs = 1 / np.sqrt(d)
    kw = dict(query_scale=qs, softcap=cap, window=1, is_local=True)
    dq, dk, dv = run_backward(g2, q, k, v, dout, kw)
    rq, rk, rv = oracle.prefill_backward(*(synth.to_f32_numpy(x) for x in (q, k, v, dout)), **kw)
    assert np.all(rq == 0.0) and np.all(rk == 0.0)          # the definition's exact zeros
    check_grad(synth.to_f32_numpy(dv), rv, f"dv {case}")
    G = H // KVH
    qn, kn, vn, gn = (synth.to_f32_numpy(x).astype(np.float64) for x in (q, k, v, dout))
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    vh = np.repeat(vn, G, axis=2)                            # (B, T, H, d): head h reads K/V head h // G
    R = 1.001 * 2 * gamma * np.abs(gn * vh).sum(axis=-1)          # (B, T, H)
    bq = (1 + 2.0 ** -7) * qs * np.abs(np.repeat(kn, G, axis=2)) * R[..., None]
    bk = (1 + 2.0 ** -7) * qs * (np.abs(qn) * R[..., None]).reshape(B, T, KVH, G, d).sum(axis=3)
    gq, gk = synth.to_f32_numpy(dq).astype(np.float64), synth.to_f32_numpy(dk).astype(np.float64)
    report(f"self-only {case}: max|dq|={np.abs(gq).max():.3e} (bound {bq.max():.3e}), "
        f"max|dk|={np.abs(gk).max():.3e} (bound {bk.max():.3e}), "
        f"max ratio dq {np.max(np.abs(gq) / bq):.3f} dk {np.max(np.abs(gk) / bk):.3f}")
    assert np.all(np.abs(gq) <= bq) and np.all(np.abs(gk) <= bk)


@pytest.mark.parametrize("chunk", [False, True], ids=["T=S", "T<S"])
def test_backward_window_int_max_equals_global(g2, chunk):
    """A local layer whose window is INT_MAX sees what a global layer sees, so
    its gradients equal the global layer's bit for bit (the window bound of the
    key-stationary kernel is formed in 64 bits); also for a chunk (T < S)."""
    say("backward window INT_MAX == global")
    B, T, S, H, KVH, d = 1, 100, 260 if chunk else 100, 4, 2, 256
    q = synth.draw((B, T, H, d), 931, 0, mul=3.0)
    k = synth.draw((B, S, KVH, d), 931, 1)
    v = synth.draw((B, S, KVH, d), 931, 2)
    dout = synth.draw((B, T, H, d), 931, 3)
    kw = dict(query_scale=1 / 16, softcap=50.0)
    glob = run_backward(g2, q, k, v, dout, dict(kw, window=1, is_local=False))
    loc = run_backward(g2, q, k, v, dout, dict(kw, window=2 ** 31 - 1, is_local=True))
    for x, y in zip(glob, loc):
        assert torch.equal(x, y)


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_backward_by_query_chunks(g2, is_local):
    """A backward with bounded workspace: rows [t0, t1) of a T = S layer are
    passed as a chunk (q, out, dO and lse sliced to those rows) against the
    first t1 keys (S = t1), where bottom-right alignment puts them at their own
    positions.  Each chunk gives its rows' dq and its rows' share of dk and dv;
    the shares summed over the chunks are the layer's gradients (oracle), and
    each chunk's workspace is that of its own (T, S) only."""
    B, T, H, KVH, d, W = 1, 1000, 4, 2, 128, 300
    say(f"backward by query chunks {'local' if is_local else 'global'}")
    q = synth.draw((B, T, H, d), 951, 0, mul=3.0)
    k = synth.draw((B, T, KVH, d), 951, 1, mul=3.0)
    v = synth.draw((B, T, KVH, d), 951, 2)
    dout = synth.draw((B, T, H, d), 951, 3)
    kw = dict(query_scale=d ** -0.5, softcap=50.0, window=W, is_local=is_local)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), dout.cuda()
    out, lse = g2.prefill_lse(qd, kd, vd, **kw)
    dq = torch.empty_like(qd)
    dk = torch.zeros(kd.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    bounds = [0, 352, 700, T]
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        rows = slice(t0, t1)
        cq, ck, cv = qd[:, rows].contiguous(), kd[:, :t1].contiguous(), vd[:, :t1].contiguous()
        ws = torch.empty(g2.backward_workspace_bytes(B, t1 - t0, t1, H), dtype=torch.uint8, device="cuda")
        gq, gk, gv = g2.prefill_backward(cq, ck, cv, out[:, rows].contiguous(), gd[:, rows].contiguous(),
                                         lse[:, :, rows].contiguous(), workspace=ws, **kw)
        dq[:, rows] = gq
        dk[:, :t1] += gk.float()
        dv[:, :t1] += gv.float()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prefill_backward(*(synth.to_f32_numpy(x) for x in (q, k, v, dout)), **kw)
    check_grad(synth.to_f32_numpy(dq), rq, f"dq by chunks {'local' if is_local else 'global'}")
    check_grad(dk.cpu().numpy(), rk, f"dk by chunks {'local' if is_local else 'global'}")
    check_grad(dv.cpu().numpy(), rv, f"dv by chunks {'local' if is_local else 'global'}")


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
def test_backward_9b_8k_whole_output(g2, is_local):
    """The 9B layer at full size, in the launch configuration the benchmark
    times (B=2, T=S=8192, H=16, KVH=8, d=256, window 4096): every element of
    dq, dk and dv against the oracle's full fp64 backward, which runs its 16
    (batch, K/V head) groups on parallel threads.  Over every key, dv summed
    per group must also equal the group's upstream gradient summed over rows
    and heads (each row's weights sum to 1)."""
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
    report(f"sum dv over keys: max|d|={err.max():.3e}, max |d|/bound={np.max(err / bound):.3f}")
    assert np.all(err <= bound)
    del g64

    rq, rk, rv = oracle.prefill_backward(*(synth.to_f32_numpy(x) for x in (q, k, v, dout)), **kw)
    check_grad(dqn, rq, f"dq, whole 9b-8k {'local' if is_local else 'global'}")
    check_grad(dkn, rk, f"dk, whole 9b-8k {'local' if is_local else 'global'}")
    check_grad(dvn, rv, f"dv, whole 9b-8k {'local' if is_local else 'global'}")


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
