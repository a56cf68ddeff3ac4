"""GPU parity of the paged-KV decode (through the C ABI) against the fp64 oracle.

K/V live in a pool of fixed-size blocks addressed through a per-sequence block
table (Gemma 2 Guide, "Deep Dive" item 2).  Inputs are laid out from seeded
linear caches by synth.paged_from_linear: blocks sit at seeded random pool
positions, slots past a sequence's length and spare pool blocks are NaN, and
on local layers the blocks older than the window are dropped (table entry -1).
Tolerances are those of the other parity tests: bf16 max |diff| <= 2e-2 and
mean |diff| <= 2e-3, fp32 max |diff| <= 1e-4.
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


def make_paged(B, S, H, KVH, d, bs, W, is_local, dt, lens, seed, spare=3):
    lens = np.asarray(lens, np.int32)
    q = synth.draw((B, 1, H, d), seed, 0, dtype=dt, mul=3.0)
    kc = synth.draw((B, S, KVH, d), seed, 1, dtype=dt)
    vc = synth.draw((B, S, KVH, d), seed, 2, dtype=dt)
    keep = W if is_local else 0
    kp, tab = synth.paged_from_linear(kc, lens, bs, seed=seed, keep_last=keep, spare_blocks=spare)
    vp, tab_v = synth.paged_from_linear(vc, lens, bs, seed=seed, keep_last=keep, spare_blocks=spare)
    assert np.array_equal(tab, tab_v)
    return q, kp, vp, tab, lens


def run_paged(g2, q, kp, vp, tab, lens, kw):
    out = g2.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(tab).cuda(),
                          torch.from_numpy(lens).cuda(), **kw)
    torch.cuda.synchronize()
    return out


PAGED_SMALL = [
    # B, S, H, KVH, d, block_size, window, is_local, dtype, lens
    (3, 300, 4, 2, 256, 16, 64, True, "bf16", [1, 150, 300]),
    (3, 300, 4, 2, 256, 16, 64, False, "bf16", [1, 150, 300]),
    (4, 1100, 4, 2, 128, 1, 100, True, "bf16", [1, 2, 513, 1100]),
    (4, 1100, 4, 2, 128, 64, 1024, False, "bf16", [1, 64, 65, 1100]),
    (4, 1100, 4, 2, 128, 64, 1024, True, "bf16", [1, 64, 1025, 1100]),
    (2, 700, 2, 1, 64, 256, 4096, True, "bf16", [700, 256]),      # window longer than L
    (3, 600, 4, 4, 128, 32, 50, True, "f32", [600, 33, 32]),
    (2, 520, 4, 2, 256, 8, 520, False, "f32", [520, 9]),
    (2, 2048, 4, 2, 256, 2048, 4096, False, "bf16", [2048, 1999]),  # one block per sequence
]


@pytest.mark.parametrize("case", PAGED_SMALL, ids=[f"paged{i}" for i in range(len(PAGED_SMALL))])
def test_paged_decode_small(g2, case):
    B, S, H, KVH, d, bs, W, is_local, dt, lens = case
    say(f"paged decode {case}")
    q, kp, vp, tab, lens = make_paged(B, S, H, KVH, d, bs, W, is_local, dt, lens,
                                      seed=400 + bs + d)
    kw = dict(query_scale=1 / np.sqrt(d), softcap=50.0, window=W, is_local=is_local)
    out = run_paged(g2, q, kp, vp, tab, lens, kw)
    ref = oracle.decode_paged(synth.to_f32_numpy(q), synth.to_f32_numpy(kp),
                              synth.to_f32_numpy(vp), tab, lens, **kw)
    check(synth.to_f32_numpy(out), ref, dt, f"paged decode {case}")


def _subpool(pool, tab, seqs):
    """Blocks used by the chosen sequences, compacted into a small pool."""
    sub = tab[seqs]
    used = np.unique(sub[sub >= 0])
    remap = np.full(pool.shape[0], -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    new_tab = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
    return pool[torch.from_numpy(used.astype(np.int64))], new_tab


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_paged_decode_full_size(g2, is_local):
    """The 9B decode workload (B=64, 8192-position caches, 16-token blocks):
    every sequence against the oracle, every output finite."""
    cfg = synth.WORKLOADS["9b-decode"]
    say(f"paged decode full 9b {'local' if is_local else 'global'}")
    q, k_g, v_g, lens, _, _ = synth.decode_inputs(cfg)
    keep = cfg["window"] if is_local else 0
    kp, tab = synth.paged_from_linear(k_g, lens, 16, seed=9, keep_last=keep, spare_blocks=5)
    del k_g
    vp, _ = synth.paged_from_linear(v_g, lens, 16, seed=9, keep_last=keep, spare_blocks=5)
    del v_g
    kw = dict(query_scale=cfg["query_scale"], softcap=cfg["softcap"], window=cfg["window"],
              is_local=is_local)
    out = run_paged(g2, q, kp, vp, tab, lens, kw)
    assert bool(torch.isfinite(out).all())
    # every sequence, in slices of 8 (each slice's blocks copied out of the pool)
    refs = []
    for s0 in range(0, q.shape[0], 8):
        seqs = list(range(s0, min(s0 + 8, q.shape[0])))
        skp, stab = _subpool(kp, tab, seqs)
        svp, _ = _subpool(vp, tab, seqs)
        refs.append(oracle.decode_paged(synth.to_f32_numpy(q[seqs]), synth.to_f32_numpy(skp),
                                        synth.to_f32_numpy(svp), stab, lens[seqs], **kw))
    check(synth.to_f32_numpy(out), np.concatenate(refs), "bf16",
          f"paged decode {'local' if is_local else 'global'}, all {q.shape[0]} sequences")


@pytest.mark.parametrize("is_local", [True, False], ids=["local", "global"])
def test_paged_matches_ring_and_linear_kernel_bitwise(g2, is_local):
    """Same positions per split in the same order: the paged kernel reproduces
    the ring / linear-cache kernel bit for bit."""
    B, S, H, KVH, d, W = 6, 2048, 4, 2, 256, 1024
    lens = np.array([1, 511, 512, 1024, 1500, 2048], np.int32)
    seed = 77
    q = synth.draw((B, 1, H, d), seed, 0, mul=3.0)
    kc = synth.draw((B, S, KVH, d), seed, 1)
    vc = synth.draw((B, S, KVH, d), seed, 2)
    kw = dict(query_scale=1 / 16, softcap=50.0, window=W, is_local=is_local)
    say(f"paged vs {'ring' if is_local else 'linear'} kernel")
    if is_local:
        kr, vr = synth.ring_from_linear(kc, lens, W), synth.ring_from_linear(vc, lens, W)
        ref = g2.decode(q.cuda(), kr.cuda(), vr.cuda(), torch.from_numpy(lens).cuda(), **kw)
        kp, tab = synth.paged_from_linear(kc, lens, 64, seed=1, keep_last=W)
        vp, _ = synth.paged_from_linear(vc, lens, 64, seed=1, keep_last=W)
    else:
        ref = g2.decode(q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(lens).cuda(), **kw)
        kp, tab = synth.paged_from_linear(kc, lens, 64, seed=1)
        vp, _ = synth.paged_from_linear(vc, lens, 64, seed=1)
    out = run_paged(g2, q, kp, vp, tab, lens, kw)
    assert torch.equal(out.cpu(), ref.cpu())


def test_paged_bad_block_or_length_gives_nan_only_there(g2):
    say("paged decode: bad table entry and out-of-range length")
    B, S, H, KVH, d, bs = 4, 256, 4, 2, 128, 16
    q, kp, vp, tab, lens = make_paged(B, S, H, KVH, d, bs, 64, False, "bf16",
                                      [256, 100, 200, 50], seed=501)
    kw = dict(query_scale=0.1, softcap=50.0, window=64, is_local=False)
    good = run_paged(g2, q, kp, vp, tab, lens, kw).float().cpu()
    bad_tab = tab.copy()
    bad_tab[1, 3] = kp.shape[0]             # needed by sequence 1, outside the pool
    bad_lens = lens.copy()
    bad_lens[2] = tab.shape[1] * bs + 1     # longer than the table can address
    out = run_paged(g2, q, kp, vp, bad_tab, bad_lens, kw).float().cpu()
    assert bool(torch.isnan(out[1]).all()) and bool(torch.isnan(out[2]).all())
    assert torch.equal(out[0], good[0]) and torch.equal(out[3], good[3])
    # a dropped block the query cannot see is never read (local layer, W = 64)
    loc = dict(kw, is_local=True)
    ref = run_paged(g2, q, kp, vp, tab, lens, loc).float().cpu()
    far = tab.copy()
    far[0, 0] = -5                           # positions 0..15, outside L = 256's window
    assert torch.equal(run_paged(g2, q, kp, vp, far, lens, loc).float().cpu(), ref)
