"""GPU parity: the HIP kernels (through the C ABI) against the CPU fp64 oracle.

Tolerances (stated for the layer's inputs): bf16 storage with fp32
accumulation, max |diff| <= 2e-2 and mean |diff| <= 2e-3 over the compared
elements; fp32 storage, max |diff| <= 1e-4.  The oracle consumes exactly the
values the GPU reads (bf16 values are exact in float32) and returns float64.

Small shapes and the four full-size bf16 workloads (2B, 9B, 9B-sat, 27B, local
and global layer each) are compared element by element over the whole output;
decode over all 64 sequences of the 9B workload.  The log-sum-exp and the
chunked prefill at full size are compared on sampled rows (first rows, tile
and window boundaries, the last rows and a seeded random set), with every
output also checked to be finite.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_g2attn_prefill_amd import synth
from _report import report

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def g2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_g2attn_prefill_amd as mod
    return mod


def check(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    report(f"{what}: max|d|={mx:.3e} mean|d|={mean:.3e}")
    if dtype == "f32":
        assert mx <= F32_MAX, f"{what}: max {mx}"
    else:
        assert mx <= BF16_MAX, f"{what}: max {mx}"
        assert mean <= BF16_MEAN, f"{what}: mean {mean}"


def layer_kw(cfg, is_local):
    return dict(query_scale=cfg["query_scale"], softcap=cfg["softcap"], window=cfg["window"],
                is_local=is_local)


# ------------------------------------------------------------ small shapes

SMALL = [
    # B, T, S, H, KVH, d, window, is_local, dtype, q_mul
    (1, 256, 256, 4, 2, 64, 64, True, "f32", 4.0),
    (1, 256, 256, 4, 2, 64, 64, False, "f32", 4.0),
    (1, 256, 256, 4, 2, 64, 64, True, "f32", 32.0),
    (2, 300, 300, 4, 2, 256, 64, True, "bf16", 3.0),
    (2, 300, 300, 4, 2, 256, 64, False, "bf16", 3.0),
    (1, 300, 300, 4, 2, 128, 37, True, "bf16", 3.0),
    (1, 300, 300, 4, 2, 64, 100, True, "bf16", 3.0),
    (2, 300, 300, 4, 4, 128, 50, True, "bf16", 2.0),      # one query head per K/V head
    (1, 333, 333, 2, 2, 256, 333, False, "bf16", 2.0),
    (1, 1, 1, 2, 1, 256, 1, True, "bf16", 1.0),            # a single token
    (1, 17, 17, 2, 1, 128, 4, True, "bf16", 1.0),
    (1, 200, 200, 2, 1, 256, 1, True, "bf16", 5.0),        # window 1: own value
    (2, 100, 330, 4, 2, 256, 70, True, "bf16", 3.0),       # T < S: rows at t + S - T
    (2, 100, 330, 4, 2, 64, 70, False, "bf16", 3.0),
    (1, 129, 257, 2, 2, 128, 128, False, "f32", 2.0),
    (1, 250, 250, 4, 2, 256, 64, False, "bf16", 5.5),      # saturating logits
    (1, 190, 190, 2, 1, 256, 64, True, "f32", 3.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[
    f"B{c[0]}T{c[1]}S{c[2]}H{c[3]}K{c[4]}d{c[5]}W{c[6]}{'L' if c[7] else 'G'}-{c[8]}-x{c[9]}"
    for c in SMALL])
def test_prefill_small_full(g2, case):
    B, T, S, H, KVH, d, W, is_local, dt, qm = case
    say(f"prefill small {case}")
    seed = 1000 + SMALL.index(case)
    q = synth.draw((B, T, H, d), seed, 0, dtype=dt, mul=qm)
    k = synth.draw((B, S, KVH, d), seed, 1, dtype=dt, mul=1.5)
    v = synth.draw((B, S, KVH, d), seed, 2, dtype=dt)
    qs = 1.0 / np.sqrt(d)
    out = g2.prefill(q.cuda(), k.cuda(), v.cuda(), query_scale=qs, softcap=50.0, window=W,
                     is_local=is_local)
    torch.cuda.synchronize()
    ref = oracle.prefill(synth.to_f32_numpy(q), synth.to_f32_numpy(k), synth.to_f32_numpy(v),
                         query_scale=qs, softcap=50.0, window=W, is_local=is_local)
    check(synth.to_f32_numpy(out), ref, dt, f"small {case}")


def test_prefill_uncapped_and_large_cap(g2):
    say("prefill cap disabled / huge cap")
    B, T, H, KVH, d = 1, 160, 4, 2, 128
    q = synth.draw((B, T, H, d), 7, 0, mul=2.0)
    k = synth.draw((B, T, KVH, d), 7, 1)
    v = synth.draw((B, T, KVH, d), 7, 2)
    qn, kn, vn = (synth.to_f32_numpy(x) for x in (q, k, v))
    # 30, 50, 55: the constant-offset softmax; 56, 200: the fast cap with a
    # running max; 1e6: the accurate cap form; 0 and inf: no cap
    for cap in (0.0, float("inf"), 1e6, 30.0, 50.0, 55.0, 56.0, 200.0):
        out = g2.prefill(q.cuda(), k.cuda(), v.cuda(), query_scale=0.1, softcap=cap, window=40,
                         is_local=True)
        torch.cuda.synchronize()
        ref = oracle.prefill(qn, kn, vn, query_scale=0.1, softcap=cap, window=40, is_local=True)
        check(synth.to_f32_numpy(out), ref, "bf16", f"cap={cap}")


@pytest.mark.parametrize("cap", [50.0, 55.0, 56.0])
@pytest.mark.parametrize("sign", [-1.0, 1.0], ids=["low", "high"])
def test_prefill_rows_saturated_at_the_cap(g2, cap, sign):
    """Every key equal to sign * (a large multiple of) the one query direction:
    all logits saturate at +-cap, every visible key has the same weight, and
    each output row is the mean of the value rows it sees (the smallest and the
    largest weights the constant softmax offset must represent)."""
    say(f"prefill saturated rows cap={cap} sign={sign}")
    B, T, H, KVH, d, W = 1, 150, 2, 1, 128, 40
    u = np.zeros(d, np.float32)
    u[::3] = 1.0
    q = torch.from_numpy(np.broadcast_to(u * 4.0, (B, T, H, d)).copy()).to(torch.bfloat16)
    k = torch.from_numpy(np.broadcast_to(u * (sign * 4.0), (B, T, KVH, d)).copy()).to(torch.bfloat16)
    v = synth.draw((B, T, KVH, d), 41, 2)
    vn = synth.to_f32_numpy(v).astype(np.float64)
    for is_local in (True, False):
        out = g2.prefill(q.cuda(), k.cuda(), v.cuda(), query_scale=1.0, softcap=cap, window=W,
                         is_local=is_local)
        torch.cuda.synchronize()
        lo = lambda t: max(0, t - W + 1) if is_local else 0
        want = np.stack([vn[0, lo(t):t + 1, 0].mean(axis=0) for t in range(T)])
        want = np.broadcast_to(want[None, :, None, :], (B, T, H, d))
        check(synth.to_f32_numpy(out), want, "bf16", f"saturated cap={cap} sign={sign}")


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_prefill_long_context(g2, is_local):
    """65536 positions (16x the 9B span), 9B head size and logit scale: sampled
    rows of the whole prefill and of a 1000-query chunk against the full cache."""
    B, T, H, KVH, d, W = 1, 65536, 4, 2, 256, 4096
    say(f"prefill long context T={T} {'local' if is_local else 'global'}")
    q = synth.draw((B, T, H, d), 51, 0, mul=3.0)
    k = synth.draw((B, T, KVH, d), 51, 1, mul=3.0)
    v = synth.draw((B, T, KVH, d), 51, 2)
    kw = dict(query_scale=1 / 16, softcap=50.0, window=W, is_local=is_local)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = g2.prefill(qd, kd, vd, **kw)
    CT = 1000
    chunk = g2.prefill(qd[:, T - CT:].contiguous(), kd, vd, **kw)
    torch.cuda.synchronize()
    qn, kn, vn = (synth.to_f32_numpy(x) for x in (q, k, v))
    rng = np.random.default_rng(52)
    ts = sorted({0, 1, 4095, 4096, 32767, 32768, T - 2, T - 1, *rng.integers(0, T, 24).tolist()})
    rows = np.asarray([(t * H + h) for t in ts for h in range(H)], np.int64)
    ref = oracle.prefill(qn, kn, vn, rows=rows, **kw)
    check(synth.to_f32_numpy(out).reshape(-1, d)[rows], ref, "bf16", f"long context ({rows.size} rows)")
    crow = np.asarray([(t * H + h) for t in (0, 1, 499, CT - 1) for h in range(H)], np.int64)
    cref = oracle.prefill(qn[:, T - CT:], kn, vn, rows=crow, **kw)
    check(synth.to_f32_numpy(chunk).reshape(-1, d)[crow], cref, "bf16", "long-context chunk")


# ------------------------------------------------------- full-size prefill

def sample_rows(B, T, H, W, seed, n_random=160):
    ts = {0, 1, 2, 15, 16, 31, 32, 63, 64, 65, 127, 128, 255, 256, W - 2, W - 1, W, W + 1,
          W + 63, W + 64, T // 2, T - 65, T - 64, T - 2, T - 1}
    ts = sorted(t for t in ts if 0 <= t < T)
    rows = [((b * T + t) * H + h) for b in range(B) for t in ts for h in range(H)]
    rng = np.random.default_rng(seed)
    rows += list(rng.integers(0, B * T * H, size=n_random))
    return np.unique(np.asarray(rows, np.int64))


@pytest.fixture(scope="module")
def prefill_inputs_cache():
    return {}


def _workload_on_gpu(cache, name):
    """Seeded inputs of a workload on the host (float32 copies for the oracle)
    and on the GPU; one workload is kept at a time."""
    if name not in cache:
        cache.clear()
        q, k, v = synth.prefill_inputs(synth.WORKLOADS[name])
        cache[name] = (q, k, v, q.cuda(), k.cuda(), v.cuda(),
                       synth.to_f32_numpy(k), synth.to_f32_numpy(v))
    return cache[name]


# Whole-output parity of the four full-size bf16 workloads, both layers of
# each pair: the GPU output is computed once per layer and every element is
# compared with the oracle, which runs on the host in FULL_CHUNKS contiguous
# row ranges (flat rows (b*T + t)*H + h) so that each test stays well under a
# minute on 16 threads.  Each chunk must meet both bounds, so the whole output
# meets them; the per-layer summary test reports max and mean over all of it.
FULL_CHUNKS = 4
FULL_CASES = [(name, is_local, c) for name in ("2b-8k", "9b-8k", "9b-8k-sat", "27b-8k")
              for is_local in (True, False) for c in range(FULL_CHUNKS)]


@pytest.fixture(scope="module")
def full_outputs():
    return {"out": {}, "stats": {}}


@pytest.mark.parametrize("case", FULL_CASES, ids=[
    f"{n}-{'local' if l else 'global'}-part{c}" for n, l, c in FULL_CASES])
def test_prefill_full_size_whole_output(g2, case, prefill_inputs_cache, full_outputs):
    name, is_local, chunk = case
    cfg = synth.WORKLOADS[name]
    layer = "local" if is_local else "global"
    say(f"prefill full {name} {layer} rows part {chunk + 1}/{FULL_CHUNKS}")
    q, k, v, qd, kd, vd, kn, vn = _workload_on_gpu(prefill_inputs_cache, name)
    kw = layer_kw(cfg, is_local)
    key = (name, is_local)
    if key not in full_outputs["out"]:
        full_outputs["out"].clear()
        out = g2.prefill(qd, kd, vd, **kw)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        full_outputs["out"][key] = synth.to_f32_numpy(out)
    got_all = full_outputs["out"][key]
    B, T, H, d = q.shape
    n = B * T * H
    lo, hi = chunk * n // FULL_CHUNKS, (chunk + 1) * n // FULL_CHUNKS
    rows = np.arange(lo, hi, dtype=np.int64)
    ref = oracle.prefill(synth.to_f32_numpy(q), kn, vn, rows=rows, **kw)
    got = got_all.reshape(-1, d)[lo:hi].astype(np.float64)
    err = np.abs(got - ref)
    st = full_outputs["stats"].setdefault(key, {"sum": 0.0, "n": 0, "max": 0.0, "parts": 0})
    st["sum"] += float(err.sum())
    st["n"] += err.size
    st["max"] = max(st["max"], float(err.max()))
    st["parts"] += 1
    check(got, ref, cfg["dtype"], f"{name} {layer} rows [{lo}, {hi})")


@pytest.mark.parametrize("name", ["2b-8k", "9b-8k", "9b-8k-sat", "27b-8k"])
@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_prefill_full_size_summary(g2, name, is_local, full_outputs):
    """Max and mean |diff| over every element of the layer's output (all row
    chunks above), against the stated bounds."""
    st = full_outputs["stats"].get((name, is_local))
    if st is None or st["parts"] != FULL_CHUNKS:
        pytest.skip("run together with test_prefill_full_size_whole_output")
    mean = st["sum"] / st["n"]
    report(f"whole output {name} {'local' if is_local else 'global'}: {st['n']} elements, "
        f"max|d|={st['max']:.3e} mean|d|={mean:.3e}")
    assert st["max"] <= BF16_MAX and mean <= BF16_MEAN


@pytest.mark.parametrize("name", ["tiny", "tiny-sat"])
@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_tiny_workloads_as_specified(g2, name, is_local):
    """The fp32 correctness workload exactly as specified (B=1, T=S=256, H=4,
    KVH=2, d=64, query_scale 1/8, cap 50, window 64, seed 0, q x4; the -sat
    variant q x32), both layers, every element within 1e-4 of the oracle."""
    cfg = synth.WORKLOADS[name]
    say(f"{name} {'local' if is_local else 'global'}")
    q, k, v = synth.prefill_inputs(cfg)
    assert q.dtype == torch.float32
    kw = layer_kw(cfg, is_local)
    out = g2.prefill(q.cuda(), k.cuda(), v.cuda(), **kw)
    torch.cuda.synchronize()
    ref = oracle.prefill(synth.to_f32_numpy(q), synth.to_f32_numpy(k), synth.to_f32_numpy(v), **kw)
    check(synth.to_f32_numpy(out), ref, "f32", f"{name} {'local' if is_local else 'global'}")


# --------------------------------------------------- log-sum-exp of each row

LSE_BF16_MAX, LSE_F32_MAX = 2e-3, 1e-4

LSE_CASES = [
    # B, T, S, H, KVH, d, window, is_local, dtype, q_mul
    (2, 300, 300, 4, 2, 256, 64, True, "bf16", 3.0),
    (2, 300, 300, 4, 2, 256, 64, False, "bf16", 3.0),
    (1, 100, 330, 4, 2, 128, 70, True, "bf16", 5.5),       # T < S, saturating logits
    (1, 200, 200, 2, 2, 64, 33, False, "bf16", 2.0),
    (1, 256, 256, 4, 2, 64, 64, True, "f32", 4.0),
    (1, 129, 257, 2, 1, 256, 100, False, "f32", 2.0),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[f"lse{i}" for i in range(len(LSE_CASES))])
def test_prefill_lse(g2, case):
    B, T, S, H, KVH, d, W, is_local, dt, qm = case
    say(f"prefill lse {case}")
    seed = 600 + d + T
    q = synth.draw((B, T, H, d), seed, 0, dtype=dt, mul=qm)
    k = synth.draw((B, S, KVH, d), seed, 1, dtype=dt, mul=qm if qm > 4 else 1.0)
    v = synth.draw((B, S, KVH, d), seed, 2, dtype=dt)
    kw = dict(query_scale=1 / np.sqrt(d), softcap=50.0, window=W, is_local=is_local)
    out, lse = g2.prefill_lse(q.cuda(), k.cuda(), v.cuda(), **kw)
    plain = g2.prefill(q.cuda(), k.cuda(), v.cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)          # the extra output changes nothing else
    qn, kn = synth.to_f32_numpy(q), synth.to_f32_numpy(k)
    ref = oracle.prefill_lse(qn, kn, **kw).transpose(0, 2, 1)     # (B, H, T)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref)
    report(f"lse {case}: max|d|={err.max():.3e}")
    assert np.all(np.isfinite(err)) and err.max() <= (LSE_F32_MAX if dt == "f32" else LSE_BF16_MAX)


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_prefill_lse_full_size_sampled(g2, is_local, prefill_inputs_cache):
    name = "9b-8k"
    cfg = synth.WORKLOADS[name]
    say(f"prefill lse full {name} {'local' if is_local else 'global'}")
    q, k, v, qd, kd, vd, kn, vn = _workload_on_gpu(prefill_inputs_cache, name)
    kw = layer_kw(cfg, is_local)
    _, lse = g2.prefill_lse(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    B, T, H, d = q.shape
    rows = sample_rows(B, T, H, cfg["window"], seed=cfg["seed"] + 1, n_random=60)
    ref = oracle.prefill_lse(synth.to_f32_numpy(q), kn, rows=rows, **kw)
    b, t, h = rows // (T * H), (rows // H) % T, rows % H
    got = lse.cpu().numpy()[b, h, t].astype(np.float64)
    err = np.abs(got - ref)
    report(f"lse full: max|d|={err.max():.3e} over {rows.size} rows")
    assert np.all(np.isfinite(got)) and err.max() <= LSE_BF16_MAX


# ---------------------------------------------- chunked prefill (T < S)

@pytest.mark.parametrize("T", [2048, 1000])
@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_chunked_prefill_9b(g2, T, is_local, prefill_inputs_cache):
    """The last T queries against the whole 8192-token cache: rows sit at
    positions t + S - T.  They equal the last T rows of the full prefill
    (bit for bit when the chunk starts on a 64-row boundary) and the oracle
    on sampled rows."""
    name = "9b-8k"
    cfg = synth.WORKLOADS[name]
    say(f"chunked prefill T={T} {'local' if is_local else 'global'}")
    q, k, v, qd, kd, vd, kn, vn = _workload_on_gpu(prefill_inputs_cache, name)
    kw = layer_kw(cfg, is_local)
    S = k.shape[1]
    full = g2.prefill(qd, kd, vd, **kw)
    chunk = g2.prefill(qd[:, S - T:].contiguous(), kd, vd, **kw)
    torch.cuda.synchronize()
    tail = full[:, S - T:]
    if (S - T) % 64 == 0:
        assert torch.equal(chunk, tail)
    else:
        assert float((chunk.float() - tail.float()).abs().max()) <= 1e-2
    B, _, H, d = q.shape
    rows = sample_rows(B, T, H, cfg["window"], seed=T, n_random=60)
    ref = oracle.prefill(synth.to_f32_numpy(q[:, S - T:]), kn, vn, rows=rows, **kw)
    got = synth.to_f32_numpy(chunk).reshape(-1, d)[rows]
    check(got, ref, "bf16", f"chunk T={T} {'local' if is_local else 'global'} ({rows.size} rows)")


# -------------------------------------------------------------- invariants

def test_window_at_least_T_equals_global_bitwise(g2):
    say("window >= T: local == global")
    q = synth.draw((2, 257, 4, 256), 11, 0, mul=3.0).cuda()
    k = synth.draw((2, 257, 2, 256), 11, 1, mul=3.0).cuda()
    v = synth.draw((2, 257, 2, 256), 11, 2).cuda()
    g = g2.prefill(q, k, v, query_scale=1 / 16, softcap=50.0, window=1, is_local=False)
    for W in (257, 4096):
        loc = g2.prefill(q, k, v, query_scale=1 / 16, softcap=50.0, window=W, is_local=True)
        torch.cuda.synchronize()
        assert torch.equal(loc, g)


def test_gqa_equals_repeated_heads(g2):
    say("GQA == repeated K/V heads (G=1 kernel)")
    q = synth.draw((1, 300, 4, 128), 12, 0, mul=3.0).cuda()
    k = synth.draw((1, 300, 2, 128), 12, 1).cuda()
    v = synth.draw((1, 300, 2, 128), 12, 2).cuda()
    a = g2.prefill(q, k, v, query_scale=0.09, softcap=50.0, window=64, is_local=True)
    kr = k.repeat_interleave(2, dim=2).contiguous()
    vr = v.repeat_interleave(2, dim=2).contiguous()
    m = g2.prefill(q, kr, vr, query_scale=0.09, softcap=50.0, window=64, is_local=True)
    torch.cuda.synchronize()
    d = (a.float() - m.float()).abs()
    assert float(d.max()) <= 2e-2 and float(d.mean()) <= 2e-3


def test_prefill_deterministic_and_canaries(g2):
    say("determinism + out-of-bounds canaries")
    B, T, H, KVH, d = 2, 300, 4, 2, 256
    q = synth.draw((B, T, H, d), 13, 0, mul=3.0).cuda()
    k = synth.draw((B, T, KVH, d), 13, 1).cuda()
    v = synth.draw((B, T, KVH, d), 13, 2).cuda()
    n = B * T * H * d
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[:n].view(B, T, H, d)
    g2.prefill(q, k, v, query_scale=1 / 16, softcap=50.0, window=64, is_local=True, out=out)
    first = out.clone()
    g2.prefill(q, k, v, query_scale=1 / 16, softcap=50.0, window=64, is_local=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool(torch.isnan(buf[n:]).all())


# ------------------------------------------------------------------ decode

def decode_check(g2, q, kc, vc, lens, cfg_kw, dtype, what, rows=None):
    out = g2.decode(q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(lens).cuda(), **cfg_kw)
    torch.cuda.synchronize()
    ref = oracle.decode(synth.to_f32_numpy(q), synth.to_f32_numpy(kc), synth.to_f32_numpy(vc),
                        lens, **cfg_kw)
    check(synth.to_f32_numpy(out), ref, dtype, what)


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_decode_full_size(g2, is_local):
    cfg = synth.WORKLOADS["9b-decode"]
    say(f"decode full 9b {'local' if is_local else 'global'}")
    q, k_g, v_g, lens, k_l, v_l = synth.decode_inputs(cfg, poison=True)
    kc, vc = (k_l, v_l) if is_local else (k_g, v_g)
    kw = layer_kw(cfg, is_local)
    out = g2.decode(q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(lens).cuda(), **kw)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    # every sequence, in slices of 8 so the float32 host copies of the caches stay small
    got = synth.to_f32_numpy(out)
    refs = []
    for s0 in range(0, q.shape[0], 8):
        bs = slice(s0, s0 + 8)
        refs.append(oracle.decode(synth.to_f32_numpy(q[bs]), synth.to_f32_numpy(kc[bs]),
                                  synth.to_f32_numpy(vc[bs]), lens[bs], **kw))
    check(got, np.concatenate(refs), "bf16",
          f"decode {'local' if is_local else 'global'}, all {q.shape[0]} sequences")


DECODE_EDGE = [
    # B, S, H, KVH, d, window, is_local, dtype, lens
    (5, 4096, 4, 2, 256, 4096, True, "bf16", [1, 100, 4095, 4096, 4097]),
    (5, 4096, 4, 2, 256, 4096, False, "bf16", [1, 100, 4095, 4096, 2]),
    (4, 300, 4, 2, 128, 64, True, "bf16", [1, 63, 64, 1000]),
    (3, 257, 2, 1, 64, 257, True, "bf16", [1, 256, 700]),
    (3, 600, 4, 4, 128, 50, False, "bf16", [600, 1, 333]),
    (3, 300, 4, 2, 256, 64, True, "f32", [5, 300, 999]),
    (2, 300, 4, 2, 64, 64, False, "f32", [300, 7]),
    # long contexts: a 65536-token linear cache, and a 4096-slot ring that has
    # wrapped 16 times
    (2, 65536, 4, 2, 256, 4096, False, "bf16", [65536, 40001]),
    (2, 4096, 4, 2, 256, 4096, True, "bf16", [65536, 33333]),
]


@pytest.mark.parametrize("case", DECODE_EDGE, ids=[f"edge{i}" for i in range(len(DECODE_EDGE))])
def test_decode_edges(g2, case):
    B, S, H, KVH, d, W, is_local, dt, lens = case
    say(f"decode edge {case}")
    lens = np.asarray(lens, np.int32)
    seed = 300 + len(lens) + d
    q = synth.draw((B, 1, H, d), seed, 0, dtype=dt, mul=3.0)
    maxlen = int(lens.max())
    lin_k = synth.draw((B, max(maxlen, S), KVH, d), seed, 1, dtype=dt)
    lin_v = synth.draw((B, max(maxlen, S), KVH, d), seed, 2, dtype=dt)
    if is_local:
        kc = synth.ring_from_linear(lin_k, lens, S)
        vc = synth.ring_from_linear(lin_v, lens, S)
    else:
        kc, vc = lin_k[:, :S].clone(), lin_v[:, :S].clone()
        synth.poison_beyond(kc, lens)
        synth.poison_beyond(vc, lens)
    kw = dict(query_scale=1 / np.sqrt(d), softcap=50.0, window=W, is_local=is_local)
    decode_check(g2, q, kc, vc, lens, kw, dt, f"decode edge {case}")


def test_decode_invalid_length_gives_nan_only_there(g2):
    say("decode: a sequence longer than a global cache")
    q = synth.draw((3, 1, 4, 128), 21, 0)
    kc = synth.draw((3, 64, 2, 128), 21, 1)
    vc = synth.draw((3, 64, 2, 128), 21, 2)
    lens = np.array([64, 65, 10], np.int32)
    out = g2.decode(q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(lens).cuda(),
                    query_scale=0.1, softcap=50.0, window=64, is_local=False)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert bool(torch.isnan(o[1]).all())
    assert bool(torch.isfinite(o[0]).all()) and bool(torch.isfinite(o[2]).all())


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_decode_equals_last_prefill_row(g2, is_local):
    say("decode == last prefill row")
    L, H, KVH, d, W = 777, 4, 2, 256, 100
    q = synth.draw((1, L, H, d), 31, 0, mul=3.0).cuda()
    k = synth.draw((1, L, KVH, d), 31, 1).cuda()
    v = synth.draw((1, L, KVH, d), 31, 2).cuda()
    pre = g2.prefill(q, k, v, query_scale=1 / 16, softcap=50.0, window=W, is_local=is_local)
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    dec = g2.decode(q[:, L - 1:L].contiguous(), k, v, lens, query_scale=1 / 16, softcap=50.0,
                    window=W, is_local=is_local)
    torch.cuda.synchronize()
    diff = (pre[:, L - 1].float() - dec[:, 0].float()).abs()
    assert float(diff.max()) <= 2e-2
