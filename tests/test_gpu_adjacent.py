"""GPU parity of the steps adjacent to the attention call against the fp64
oracle: the rotary embedding of Q and K and the final-logit soft-cap.

Tolerances: fp32 storage, max |diff| <= 2e-5 (rope; angles reduced in fp64,
sin/cos in fp32) and 2e-5 (cap 30); bf16 storage, every element within one
bf16 unit in the last place of the exact value, and at least 99% of them
equal to its round-to-nearest-even value.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_g2attn_prefill_amd import synth
from _report import report

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def g2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_g2attn_prefill_amd as mod
    return mod


def bf16_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_storage(got, ref, dtype, what, f32_tol=2e-5, arith=None):
    """arith: optional per-element bound on the fp32 arithmetic error before
    the result is stored (e.g. the cancellation in a rotation)."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    report(f"{what}: max|d|={err.max():.3e}")
    if dtype == "f32":
        assert err.max() <= f32_tol, what
    else:
        extra = 0.0 if arith is None else arith
        bad = err > bf16_ulp(ref) + extra + 1e-30
        assert not np.any(bad), f"{what}: {int(bad.sum())} elements, e.g. got {got[bad][:3]} ref {ref[bad][:3]}"
        rne = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        assert np.mean(got == rne) >= 0.99, what


ROPE_CASES = [
    # B, T, NH, d, dtype, base, max position
    (2, 300, 16, 256, "bf16", 10000.0, 8192),
    (2, 300, 8, 256, "f32", 10000.0, 8192),
    (1, 77, 4, 128, "bf16", 10000.0, 70000),
    (1, 77, 4, 128, "f32", 500000.0, 70000),
    (3, 5, 2, 64, "f32", 10000.0, 16),
    (1, 1, 1, 64, "bf16", 10000.0, 1),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=[f"rope{i}" for i in range(len(ROPE_CASES))])
def test_rope(g2, case):
    B, T, NH, d, dt, base, pmax = case
    say(f"rope {case}")
    x = synth.draw((B, T, NH, d), 700 + d + T, 0, dtype=dt, mul=2.0)
    pos = np.random.default_rng(T).integers(0, pmax, size=(B, T)).astype(np.int32)
    pos[0, 0] = 0
    ref = oracle.rope(synth.to_f32_numpy(x), pos, base=base)
    xd = x.cuda()
    g2.rope_(xd, torch.from_numpy(pos).cuda(), base=base)
    torch.cuda.synchronize()
    got = synth.to_f32_numpy(xd)
    xn = synth.to_f32_numpy(x).astype(np.float64)
    assert np.array_equal(got[0, 0], xn[0, 0])   # position 0 untouched
    # fp32 rotation of a pair (a, b): error below a few units of 2^-24 (|a| + |b|)
    h = d // 2
    pair = np.abs(xn[..., :h]) + np.abs(xn[..., h:])
    arith = 4.0 * 2.0 ** -24 * np.concatenate([pair, pair], axis=-1)
    check_storage(got, ref, dt, f"rope {case}", arith=arith)


def test_rope_then_attention_scores_are_relative(g2):
    """Rotating Q and K at positions p and p + s gives the same prefill output
    for every s (scores depend only on the distance), up to bf16 rounding."""
    B, T, H, KVH, d = 1, 200, 4, 2, 128
    q = synth.draw((B, T, H, d), 711, 0, mul=2.0)
    k = synth.draw((B, T, KVH, d), 711, 1)
    v = synth.draw((B, T, KVH, d), 711, 2)
    outs = []
    for shift in (0, 3000):
        pos = torch.arange(shift, shift + T, dtype=torch.int32).view(1, T).cuda()
        qd, kd = q.cuda(), k.cuda()
        g2.rope_(qd, pos)
        g2.rope_(kd, pos)
        outs.append(g2.prefill(qd, kd, v.cuda(), query_scale=1 / np.sqrt(d), softcap=50.0,
                               window=64, is_local=True).float())
    torch.cuda.synchronize()
    assert float((outs[0] - outs[1]).abs().max()) <= 3e-2


SOFTCAP_CASES = [
    # n, dtype, spread
    (2 * 8192 * 1000 + 5, "bf16", 40.0),
    (64 * 256000, "bf16", 15.0),
    (1_000_003, "f32", 60.0),
    (7, "bf16", 100.0),
    (1, "f32", 10.0),
]


@pytest.mark.parametrize("case", SOFTCAP_CASES, ids=[f"cap{i}" for i in range(len(SOFTCAP_CASES))])
def test_final_softcap(g2, case):
    n, dt, spread = case
    say(f"final soft-cap {case}")
    x = synth.draw((n,), 720 + n % 97, 0, dtype=dt, mul=spread)
    x[: min(n, 4)] = torch.tensor([0.0, -1e-3, 1e4, -1e4][: min(n, 4)], dtype=x.dtype)
    ref = oracle.softcap_array(synth.to_f32_numpy(x), 30.0)
    xd = x.cuda()
    g2.softcap_(xd, 30.0)
    torch.cuda.synchronize()
    got = synth.to_f32_numpy(xd)
    assert np.all(np.abs(got) <= 30.0)
    check_storage(got, ref, dt, f"soft-cap {case}")


def test_final_softcap_disabled_leaves_data(g2):
    x = synth.draw((1000,), 731, 0, mul=50.0).cuda()
    y = x.clone()
    for cap in (0.0, -1.0, float("inf")):
        g2.softcap_(y, cap)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


# ---------------------------------------------- the sizes the benchmark times

def test_rope_9b_full_size_whole_output(g2):
    """Q (16 heads) and K (8 heads) of the 9B layer (B=2, T=8192, d=256) at
    positions 0..T-1, in place as the benchmark runs it; every element against
    the oracle, one batch entry at a time."""
    cfg = synth.WORKLOADS["9b-8k"]
    B, T, d = cfg["B"], cfg["T"], cfg["d"]
    q, k, _ = synth.prefill_inputs(cfg)
    pos = torch.arange(T, dtype=torch.int32).repeat(B, 1).contiguous()
    for name, x in (("q", q), ("k", k)):
        say(f"rope full 9b {name}")
        xd = x.cuda()
        g2.rope_(xd, pos.cuda())
        torch.cuda.synchronize()
        for b in range(B):
            xs = synth.to_f32_numpy(x[b:b + 1])                       # (1, T, NH, d)
            ref = oracle.rope(xs, pos[b:b + 1].numpy())
            got = synth.to_f32_numpy(xd[b:b + 1].cpu())
            xn = xs.astype(np.float64)
            h = d // 2
            pair = np.abs(xn[..., :h]) + np.abs(xn[..., h:])
            arith = 4.0 * 2.0 ** -24 * np.concatenate([pair, pair], axis=-1)
            check_storage(got, ref, "bf16", f"rope full 9b {name} batch {b}", arith=arith)


def test_final_softcap_full_size_sampled(g2):
    """The final cap (30) over the 9B batch's logits, 16384 x 256000 bf16
    (4.19e9 elements, so offsets pass 2^31), in place.  Inputs come from a
    seeded generator on the device; sampled elements, among them the first
    and last ones and both sides of 2^31, are read before and after the call
    and checked against the oracle; every element must lie within the cap."""
    rows, vocab = 16384, 256000
    n = rows * vocab
    say("final soft-cap full 16384 x 256000")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(61)
    x = torch.randn((rows, vocab), generator=gen, device="cuda", dtype=torch.float32).mul_(15.0)
    x = x.to(torch.bfloat16)
    flat = x.view(-1)
    rng = np.random.default_rng(62)
    idx = np.unique(np.concatenate([
        np.array([0, 1, 7, 8, 2 ** 31 - 9, 2 ** 31 - 1, 2 ** 31, 2 ** 31 + 8, n - 9, n - 1]),
        rng.integers(0, n, 20000)])).astype(np.int64)
    it = torch.from_numpy(idx).cuda()
    before = synth.to_f32_numpy(flat.index_select(0, it).cpu())
    g2.softcap_(x, 30.0)
    torch.cuda.synchronize()
    assert float(flat.abs().max()) <= 30.0
    got = synth.to_f32_numpy(flat.index_select(0, it).cpu())
    ref = oracle.softcap_array(before, 30.0)
    check_storage(got, ref, "bf16", f"soft-cap full ({idx.size} sampled elements)")
    del x, flat
