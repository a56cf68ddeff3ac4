"""The allocation-free decode entry point (g2attn_decode_noalloc) against the
decode entry point with a caller-owned workspace (g2attn_decode): both run the
same kernels, so the outputs must be equal bit for bit.  Two calls in a row
share the library's scratch array, the second with a smaller input; a size
beyond the scratch is rejected on the host before any launch."""
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


def _inputs(B, S, H, KVH, d, lens, seed, is_local, W):
    q = synth.draw((B, 1, H, d), seed, 0, mul=3.0)
    maxlen = int(max(lens))
    lin_k = synth.draw((B, max(maxlen, S), KVH, d), seed, 1)
    lin_v = synth.draw((B, max(maxlen, S), KVH, d), seed, 2)
    if is_local:
        kc, vc = synth.ring_from_linear(lin_k, lens, S), synth.ring_from_linear(lin_v, lens, S)
    else:
        kc, vc = lin_k[:, :S].clone(), lin_v[:, :S].clone()
        synth.poison_beyond(kc, lens)
        synth.poison_beyond(vc, lens)
    return q, kc, vc


def test_noalloc_decode_equals_decode_on_two_calls(g2):
    cases = [
        # B, S, H, KVH, d, window, is_local, lens: a 9B-shaped global layer, then a smaller local ring
        (24, 8192, 16, 8, 256, 4096, False, None),
        (5, 2048, 4, 2, 128, 2048, True, [1, 100, 2047, 2048, 9000]),
    ]
    for i, (B, S, H, KVH, d, W, is_local, lens) in enumerate(cases):
        say(f"noalloc decode call {i + 1}: B={B} S={S} H={H} KVH={KVH} d={d} "
            f"{'local' if is_local else 'global'}")
        if lens is None:
            lens = np.random.default_rng(5).integers(4096, S + 1, size=B)
        lens = np.asarray(lens, np.int32)
        need = g2.decode_workspace_bytes(B, H, d, S)
        assert 0 < need <= g2.NOALLOC_SCRATCH_BYTES
        q, kc, vc = _inputs(B, S, H, KVH, d, lens, 960 + i, is_local, W)
        kw = dict(query_scale=1 / np.sqrt(d), softcap=50.0, window=W, is_local=is_local)
        qd, kd, vd, ld = q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(lens).cuda()
        ref = g2.decode(qd, kd, vd, ld, **kw)
        out = torch.full_like(qd, float("nan"))
        g2.decode_noalloc(qd, kd, vd, ld, out=out, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i + 1}: differs from g2attn_decode"
        # and both against the oracle, on the first sequences
        nb = min(B, 4)
        want = oracle.decode(synth.to_f32_numpy(q[:nb]), synth.to_f32_numpy(kc[:nb]),
                             synth.to_f32_numpy(vc[:nb]), lens[:nb], **kw)
        err = np.abs(synth.to_f32_numpy(out[:nb]).astype(np.float64) - want)
        report(f"call {i + 1}: equal to g2attn_decode; vs oracle max|d|={err.max():.3e} "
            f"mean|d|={err.mean():.3e}")
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_noalloc_decode_rejects_sizes_beyond_its_scratch(g2):
    B, S, H, KVH, d = 128, 8192, 16, 8, 256    # 33.8 MB of split-K scratch > 32 MiB
    assert g2.decode_workspace_bytes(B, H, d, S) > g2.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 1, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, S, KVH, d), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(g2.G2attnError) as ei:
        g2.decode_noalloc(q, kc, kc, lens, query_scale=1 / 16, softcap=50.0, window=4096,
                          is_local=False, out=out)
    assert ei.value.status == -4                # G2_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 0).all())               # nothing was launched
