"""The C-ABI library loads, exports every function include/g2attn.h declares, and
rejects bad arguments on the host (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import attention_g2attn_prefill_amd as g2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g2attn.h")

OK, ARG, UNSUP, ALIGN, WS, LAUNCH = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(g2attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("g2attn_prefill", "g2attn_prefill_lse", "g2attn_decode", "g2attn_decode_workspace_bytes",
              "g2attn_check_args", "g2attn_status_string", "g2attn_decode_paged",
              "g2attn_decode_paged_workspace_bytes", "g2attn_check_paged_args",
              "g2attn_rope", "g2attn_softcap", "g2attn_prefill_backward",
              "g2attn_prefill_backward_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g2.library_path)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (OK, ARG, UNSUP, ALIGN, WS, LAUNCH):
        assert g2.status_string(code) and g2.status_string(code) != "unknown status"
    assert g2.status_string(12345) == "unknown status"


@pytest.mark.parametrize("args,expect", [
    # B, T, S, H, KVH, d, window, is_local, dtype, decode
    ((2, 8192, 8192, 16, 8, 256, 4096, 1, 0, 0), OK),
    ((1, 256, 256, 4, 2, 64, 64, 0, 1, 0), OK),
    ((1, 8192, 8192, 32, 16, 128, 4096, 1, 0, 0), OK),
    ((64, 1, 8192, 16, 8, 256, 4096, 0, 0, 1), OK),
    ((0, 16, 16, 4, 2, 64, 4, 0, 0, 0), ARG),
    ((1, 17, 16, 4, 2, 64, 4, 0, 0, 0), ARG),      # T > S
    ((1, 16, 16, 4, 3, 64, 4, 0, 0, 0), ARG),      # H % KVH
    ((1, 16, 16, 4, 2, 64, 0, 1, 0, 0), ARG),      # local with window 0
    ((1, 16, 16, 4, 2, 64, 0, 0, 0, 0), OK),       # window ignored on global
    ((1, 2, 16, 4, 2, 64, 4, 0, 0, 1), ARG),       # decode with T != 1
    ((1, 16, 16, 4, 2, 64, 4, 0, 7, 0), ARG),      # unknown dtype
    ((1, 16, 16, 4, 2, 64, 4, 2, 0, 0), ARG),      # is_local not 0/1
    ((1, 16, 16, 4, 2, 96, 4, 0, 0, 0), UNSUP),    # d
    ((1, 16, 16, 8, 2, 64, 4, 0, 0, 0), UNSUP),    # four heads per K/V head
    ((1, 0, 16, 4, 2, 64, 4, 0, 0, 0), ARG),       # empty query block
    ((1, 16, 0, 4, 2, 64, 4, 0, 0, 0), ARG),       # empty cache
    ((1, 16, 16, 0, 2, 64, 4, 0, 0, 0), ARG),      # no heads
    ((1, 16, 16, 4, 2, 0, 4, 0, 0, 0), ARG),       # d = 0
    ((1, -5, 16, 4, 2, 64, 4, 0, 0, 0), ARG),      # negative size
    # element counts per sequence must stay below 2^31 (32-bit in-sequence offsets)
    ((1, 524287, 524287, 16, 8, 256, 4096, 1, 0, 0), OK),      # T*H*d = 2^31 - 4096
    ((1, 524288, 524288, 16, 8, 256, 4096, 1, 0, 0), UNSUP),   # T*H*d = 2^31
    ((1, 1, 1 << 20, 16, 8, 256, 4096, 0, 0, 1), UNSUP),       # S*KVH*d = 2^31 (decode)
    ((64, 1, (1 << 20) - 1, 16, 8, 256, 4096, 0, 0, 1), OK),   # the longest 9B cache
])
def test_check_args(args, expect):
    assert g2.check_args(*args[:8], dtype=args[8], decode=args[9]) == expect


def test_backward_workspace_bytes():
    # row statistics (rounded up to 256 bytes), then 1 KiB per (b, h, 32-row tile, 16-key block)
    assert g2.backward_workspace_bytes(2, 8192, 8192, 16) == 2 * 16 * 8192 * 4 + 2 * 16 * 256 * 512 * 1024
    assert g2.backward_workspace_bytes(1, 1, 1, 1) == 256 + 1024
    assert g2.backward_workspace_bytes(1, 33, 40, 3) == 512 + 3 * 2 * 3 * 1024
    for bad in ((0, 4, 4, 1), (1, 5, 4, 1), (1, 4, 4, 0)):
        with pytest.raises(ValueError):
            g2.backward_workspace_bytes(*bad)


def test_workspace_bytes():
    # splits of 512 positions; per (sequence, head, split): max, sum, d floats
    assert g2.decode_workspace_bytes(64, 16, 256, 8192) == 64 * 16 * 16 * (2 + 256) * 4
    assert g2.decode_workspace_bytes(1, 1, 64, 1) == 1 * 1 * 1 * 66 * 4
    assert g2.decode_workspace_bytes(0, 16, 256, 8192) == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_entry_points_reject_before_launching():
    lib = g2.lib
    a = _fake(0x10000)
    null = ctypes.c_void_p(0)
    # invalid scalars: rejected before any pointer is looked at
    assert lib.g2attn_prefill(a, a, a, a, 1, 17, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0, null) == ARG
    # null pointer
    assert lib.g2attn_prefill(null, a, a, a, 1, 16, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0, null) == ARG
    # misaligned pointer
    assert lib.g2attn_prefill(a, _fake(0x10008), a, a, 1, 16, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0,
                              null) == ALIGN
    # decode: missing or short workspace
    assert lib.g2attn_decode(a, a, a, a, a, 2, 1, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0, null, 0,
                             null) == WS
    need = g2.decode_workspace_bytes(2, 4, 64, 16)
    assert lib.g2attn_decode(a, a, a, a, a, 2, 1, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0, a, need - 1,
                             null) == WS
    assert lib.g2attn_decode(a, a, a, a, null, 2, 1, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0, a, need,
                             null) == ARG
    assert lib.g2attn_decode(a, a, a, a, a, 2, 1, 16, 4, 2, 64, 1.0, 50.0, 4, 0, 0,
                             _fake(0x10004), need, null) == ALIGN


def test_backward_entry_point_rejects_before_launching():
    """The backward's workspace (row statistics and dS blocks) is checked for
    size and 16-byte alignment on the host, before anything is launched."""
    lib = g2.lib
    a, lse = _fake(0x10000), _fake(0x20000)
    null = ctypes.c_void_p(0)
    B, T, S, H, KVH, d = 1, 40, 70, 4, 2, 64
    need = g2.backward_workspace_bytes(B, T, S, H)

    def call(ws, nbytes, lse_ptr=lse, bf16=0):
        return lib.g2attn_prefill_backward(a, a, a, a, a, lse_ptr, a, a, a, B, T, S, H, KVH, d,
                                           0.125, 50.0, 16, 1, bf16, ws, nbytes, null)

    assert call(null, need) == WS
    assert call(a, need - 1) == WS
    assert call(_fake(0x10008), need) == ALIGN          # 8-byte aligned workspace
    assert call(a, need, lse_ptr=_fake(0x20002)) == ALIGN
    assert call(a, need, bf16=1) == UNSUP                # the backward is bf16 only
    assert lib.g2attn_prefill_backward_workspace_bytes(B, T, T - 1, H) == 0   # S < T


def test_binding_requires_gpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        g2.prefill(q, k, k, query_scale=0.125, is_local=False)


@pytest.mark.parametrize("bad", ["dq", "dk", "dv"])
def test_backward_rejects_wrong_output_buffers_before_launching(bad):
    """dq, dk and dv handed in by the caller are checked for shape and dtype
    before anything reaches the library (the C ABI cannot see their sizes)."""
    import torch
    B, T, H, KVH, d = 1, 8, 4, 2, 64
    q = torch.zeros(B, T, H, d, dtype=torch.bfloat16)
    k = torch.zeros(B, T, KVH, d, dtype=torch.bfloat16)
    lse = torch.zeros(B, H, T, dtype=torch.float32)
    outs = {"dq": torch.zeros_like(q), "dk": torch.zeros_like(k), "dv": torch.zeros_like(k)}
    short = dict(outs)
    short[bad] = torch.zeros(outs[bad].numel() - d, dtype=torch.bfloat16).view(-1, d)
    with pytest.raises(ValueError, match=bad):
        g2.prefill_backward(q, k, k, q, q, lse, query_scale=0.125, window=4, is_local=True,
                            **short)
    wrong_dtype = dict(outs)
    wrong_dtype[bad] = outs[bad].float()
    with pytest.raises(ValueError, match=bad):
        g2.prefill_backward(q, k, k, q, q, lse, query_scale=0.125, window=4, is_local=True,
                            **wrong_dtype)


def test_workspaces_are_checked_before_launching():
    import torch
    q = torch.zeros(2, 1, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(2, 16, 2, 64, dtype=torch.bfloat16)
    lens = torch.ones(2, dtype=torch.int32)
    need = g2.decode_workspace_bytes(2, 4, 64, 16)
    with pytest.raises(ValueError, match="workspace"):
        g2.decode(q, kc, kc, lens, query_scale=0.125, is_local=False,
                  workspace=torch.zeros(need - 1, dtype=torch.uint8))
    qb = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    kb = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="workspace"):
        g2.prefill_backward(qb, kb, kb, qb, qb, torch.zeros(1, 4, 8), query_scale=0.125,
                            window=4, is_local=True, workspace=torch.zeros(3, dtype=torch.uint8))


@pytest.mark.parametrize("args,expect", [
    # B, H, KVH, d, block_size, max_blocks, num_blocks, window, is_local, dtype
    ((64, 16, 8, 256, 16, 512, 32768, 4096, 1, 0), OK),
    ((2, 4, 2, 64, 1, 100, 7, 5, 0, 1), OK),
    ((2, 4, 2, 64, 65536, 2, 7, 5, 0, 0), OK),
    ((2, 4, 2, 64, 24, 10, 7, 5, 0, 0), ARG),          # block size not a power of two
    ((2, 4, 2, 64, 0, 10, 7, 5, 0, 0), ARG),
    ((2, 4, 2, 64, 131072, 10, 7, 5, 0, 0), ARG),     # block size above 65536
    ((2, 4, 2, 64, 16, 0, 7, 5, 0, 0), ARG),
    ((2, 4, 2, 64, 16, 10, 0, 5, 0, 0), ARG),
    ((2, 4, 2, 64, 65536, 1 << 15, 7, 5, 0, 0), ARG),  # capacity beyond 2^31 positions
    ((2, 4, 2, 64, 16, 10, 7, 0, 1, 0), ARG),          # local with window 0
    ((2, 4, 3, 64, 16, 10, 7, 5, 0, 0), ARG),          # H % KVH
    ((2, 4, 2, 96, 16, 10, 7, 5, 0, 0), UNSUP),
    ((2, 8, 2, 64, 16, 10, 7, 5, 0, 0), UNSUP),
])
def test_check_paged_args(args, expect):
    assert g2.check_paged_args(*args) == expect


def test_paged_workspace_bytes():
    # splits of 512 positions over the table's capacity max_blocks * block_size
    assert g2.decode_paged_workspace_bytes(64, 16, 256, 512, 16) == 64 * 16 * 16 * 258 * 4
    assert g2.decode_paged_workspace_bytes(1, 1, 64, 3, 1) == 66 * 4
    assert g2.decode_paged_workspace_bytes(1, 1, 64, 0, 16) == 0


def test_paged_entry_point_rejects_before_launching():
    lib = g2.lib
    a = _fake(0x10000)
    null = ctypes.c_void_p(0)
    need = g2.decode_paged_workspace_bytes(2, 4, 64, 8, 16)
    args = lambda q=a, kp=a, vp=a, out=a, tab=a, lens=a, ws=a, nbytes=need, bs=16: (
        q, kp, vp, out, tab, 8, lens, 2, 4, 2, 64, bs, 10, 1.0, 50.0, 64, 1, 0, ws, nbytes, null)
    assert lib.g2attn_decode_paged(*args(bs=12)) == ARG
    assert lib.g2attn_decode_paged(*args(tab=null)) == ARG
    assert lib.g2attn_decode_paged(*args(lens=null)) == ARG
    assert lib.g2attn_decode_paged(*args(kp=_fake(0x10004))) == ALIGN
    assert lib.g2attn_decode_paged(*args(ws=null)) == WS
    # a local layer needs only the splits of its window: 64 positions here
    small = g2.decode_paged_workspace_bytes(2, 4, 64, 1, 64)
    assert lib.g2attn_decode_paged(*args(nbytes=small - 1)) == WS


def test_adjacent_steps_reject_before_launching():
    lib = g2.lib
    a = _fake(0x10000)
    null = ctypes.c_void_p(0)
    assert lib.g2attn_rope(a, a, 2, 3, 4, 96, 10000.0, 0, null) == UNSUP
    assert lib.g2attn_rope(a, a, 2, 3, 4, 128, 1.0, 0, null) == ARG      # base must exceed 1
    assert lib.g2attn_rope(a, a, 0, 3, 4, 128, 10000.0, 0, null) == ARG
    assert lib.g2attn_rope(null, a, 2, 3, 4, 128, 10000.0, 0, null) == ARG
    assert lib.g2attn_rope(_fake(0x10008), a, 2, 3, 4, 128, 10000.0, 0, null) == ALIGN
    assert lib.g2attn_rope(a, _fake(0x10002), 2, 3, 4, 128, 10000.0, 0, null) == ALIGN
    assert lib.g2attn_softcap(a, 10, 30.0, 5, null) == ARG
    assert lib.g2attn_softcap(_fake(0x10004), 10, 30.0, 0, null) == ALIGN
    # nothing to do: no pointer is looked at, nothing is launched
    assert lib.g2attn_softcap(null, 0, 30.0, 0, null) == OK
    assert lib.g2attn_softcap(null, 10, 0.0, 0, null) == OK


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: a copy of the package without libg2attn.so raises on first
    use of an entry point instead of computing anything elsewhere."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "attention_g2attn_prefill_amd")
    dst = tmp_path / "attention_g2attn_prefill_amd"
    dst.mkdir()
    for name in ("__init__.py", "_binding.py", "synth.py"):
        shutil.copy(os.path.join(pkg, name), dst / name)
    code = ("import attention_g2attn_prefill_amd as g\n"
            "try:\n    g.prefill\nexcept ImportError as e:\n    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=str(tmp_path), timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "libg2attn.so is not built" in r.stdout
