"""ctypes binding of libg2attn.so: argument marshalling only.

Every step of prefill and decode runs in the library's HIP kernels; torch
provides device memory and the current HIP stream.  There is no fallback: if
the library is missing, importing this module raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libg2attn.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is not built; run `python -m attention_g2attn_prefill_amd.build` "
        "(or __graft_entry__.build()) first")

lib = ctypes.CDLL(library_path)

_vp = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

lib.g2attn_prefill.argtypes = [_vp, _vp, _vp, _vp, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I,
                               _I, _vp]
lib.g2attn_prefill.restype = _I
lib.g2attn_prefill_lse.argtypes = [_vp, _vp, _vp, _vp, _vp, _I, _I, _I, _I, _I, _I, _F, _F,
                                   _I, _I, _I, _vp]
lib.g2attn_prefill_lse.restype = _I
lib.g2attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _I, _I, _I, _I, _I, _I, _F, _F, _I,
                              _I, _I, _vp, ctypes.c_size_t, _vp]
lib.g2attn_decode.restype = _I
lib.g2attn_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _I, _I, _I, _I, _I, _I, _F, _F,
                                      _I, _I, _I, _vp]
lib.g2attn_decode_noalloc.restype = _I
lib.g2attn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
lib.g2attn_decode_workspace_bytes.restype = ctypes.c_size_t
lib.g2attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _I, _vp, _I, _I, _I, _I, _I, _I,
                                    _F, _F, _I, _I, _I, _vp, ctypes.c_size_t, _vp]
lib.g2attn_decode_paged.restype = _I
lib.g2attn_decode_paged_workspace_bytes.argtypes = [_I] * 5
lib.g2attn_decode_paged_workspace_bytes.restype = ctypes.c_size_t
lib.g2attn_check_paged_args.argtypes = [_I] * 10
lib.g2attn_check_paged_args.restype = _I
lib.g2attn_prefill_backward.argtypes = [_vp] * 9 + [_I] * 6 + [_F, _F, _I, _I, _I, _vp,
                                                                ctypes.c_size_t, _vp]
lib.g2attn_prefill_backward.restype = _I
lib.g2attn_prefill_backward_workspace_bytes.argtypes = [_I, _I, _I, _I]
lib.g2attn_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
lib.g2attn_rope.argtypes = [_vp, _vp, _I, _I, _I, _I, _F, _I, _vp]
lib.g2attn_rope.restype = _I
lib.g2attn_softcap.argtypes = [_vp, ctypes.c_size_t, _F, _I, _vp]
lib.g2attn_softcap.restype = _I
lib.g2attn_check_args.argtypes = [_I] * 10
lib.g2attn_check_args.restype = _I
lib.g2attn_status_string.argtypes = [_I]
lib.g2attn_status_string.restype = ctypes.c_char_p
lib.g2attn_build_id.argtypes = []
lib.g2attn_build_id.restype = ctypes.c_char_p

G2_BF16, G2_F32 = 0, 1
_DTYPES = {torch.bfloat16: G2_BF16, torch.float32: G2_F32}


class G2attnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return lib.g2attn_status_string(int(status)).decode()


def build_id() -> str:
    """sha256 of the sources the loaded library was built from."""
    return lib.g2attn_build_id().decode()


def check_args(B, T, S, H, KVH, d, window, is_local, dtype=G2_BF16, decode=False) -> int:
    """Host-only validation; returns the status the call would return."""
    return lib.g2attn_check_args(B, T, S, H, KVH, d, window, int(is_local), dtype,
                                 int(bool(decode)))


def decode_workspace_bytes(B, H, d, S) -> int:
    return int(lib.g2attn_decode_workspace_bytes(B, H, d, S))


def decode_paged_workspace_bytes(B, H, d, max_blocks, block_size) -> int:
    return int(lib.g2attn_decode_paged_workspace_bytes(B, H, d, max_blocks, block_size))


def check_paged_args(B, H, KVH, d, block_size, max_blocks, num_blocks, window, is_local,
                     dtype=G2_BF16) -> int:
    """Host-only validation of paged-decode scalars; the status the call would return."""
    return lib.g2attn_check_paged_args(B, H, KVH, d, block_size, max_blocks, num_blocks,
                                       window, int(is_local), dtype)


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_workspace(ws, need: int) -> None:
    """A caller-supplied workspace: a tensor of at least `need` bytes (the
    library checks the size too; this names the problem before any call)."""
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a GPU tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def prefill(q, k, v, *, query_scale, softcap=50.0, window=4096, is_local, out=None,
            stream=None):
    """Soft-capped GQA attention for a prefill: q (B,T,H,d), k/v (B,S,KVH,d).

    Returns out (B,T,H,d) in q's dtype.  Enqueued on `stream` (default: the
    current stream); the call does not synchronise.
    """
    B, T, H, d = q.shape
    Bk, S, KVH, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype bfloat16 or float32")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    st = lib.g2attn_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                            B, T, S, H, KVH, d, float(query_scale), float(softcap),
                            int(window), int(bool(is_local)), _DTYPES[q.dtype],
                            _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_prefill")
    return out


def prefill_lse(q, k, v, *, query_scale, softcap=50.0, window=4096, is_local, out=None,
                lse=None, stream=None):
    """prefill() that also returns the (B, H, T) float32 natural-log log-sum-exp
    of each row's capped, masked logits.  Returns (out, lse)."""
    B, T, H, d = q.shape
    Bk, S, KVH, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype bfloat16 or float32")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != (B, H, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 of shape (B, H, T)")
    st = lib.g2attn_prefill_lse(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                _dev(lse, "lse"), B, T, S, H, KVH, d, float(query_scale),
                                float(softcap), int(window), int(bool(is_local)),
                                _DTYPES[q.dtype], _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_prefill_lse")
    return out, lse


def decode(q, k_cache, v_cache, kv_lens, *, query_scale, softcap=50.0, window=4096,
           is_local, out=None, workspace=None, stream=None):
    """One query token per sequence against a KV cache.

    q (B,1,H,d); k_cache/v_cache (B,S,KVH,d) with position j in slot j mod S;
    kv_lens int32 (B,) on the GPU.  workspace: a uint8 GPU tensor of at least
    decode_workspace_bytes(B,H,d,S) bytes (allocated here if None).
    """
    B, T, H, d = q.shape
    Bk, S, KVH, dk = k_cache.shape
    if (Bk, dk) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and the caches")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share dtype bfloat16 or float32")
    if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
        raise TypeError("kv_lens must be int32 of shape (B,)")
    need = decode_workspace_bytes(B, H, d, S)
    _check_workspace(workspace, need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    st = lib.g2attn_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(out, "out"), _dev(kv_lens, "kv_lens"), B, T, S, H, KVH, d,
                           float(query_scale), float(softcap), int(window),
                           int(bool(is_local)), _DTYPES[q.dtype], _dev(workspace, "workspace"),
                           workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_decode")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # G2ATTN_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q, k_cache, v_cache, kv_lens, *, query_scale, softcap=50.0, window=4096,
                   is_local, out, stream=None):
    """decode() through the allocation-free entry point: the split-K scratch is
    the library's own per-GPU array (at most NOALLOC_SCRATCH_BYTES of
    workspace), so nothing is allocated; `out` must be given."""
    B, T, H, d = q.shape
    Bk, S, KVH, dk = k_cache.shape
    if (Bk, dk) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and the caches")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share dtype bfloat16 or float32")
    if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
        raise TypeError("kv_lens must be int32 of shape (B,)")
    if out is None or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be given and match q's shape and dtype")
    st = lib.g2attn_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                   _dev(v_cache, "v_cache"), _dev(out, "out"),
                                   _dev(kv_lens, "kv_lens"), B, T, S, H, KVH, d,
                                   float(query_scale), float(softcap), int(window),
                                   int(bool(is_local)), _DTYPES[q.dtype], _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_decode_noalloc")
    return out


def decode_paged(q, k_pool, v_pool, block_table, kv_lens, *, query_scale, softcap=50.0,
                 window=4096, is_local, out=None, workspace=None, stream=None):
    """One query token per sequence against a paged KV cache.

    q (B,1,H,d); k_pool/v_pool (num_blocks, block_size, KVH, d); block_table
    int32 (B, max_blocks) on the GPU, entry [b][i] = pool block of positions
    i*block_size .. (i+1)*block_size - 1 (entries of blocks the query cannot
    see are never read); kv_lens int32 (B,) on the GPU.  workspace: a uint8
    GPU tensor of at least decode_paged_workspace_bytes(B,H,d,max_blocks,
    block_size) bytes (allocated here if None).
    """
    B, T, H, d = q.shape
    NB, BS, KVH, dk = k_pool.shape
    if T != 1 or dk != d or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("shape mismatch between q and the pools")
    if q.dtype not in _DTYPES or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q and pools must share dtype bfloat16 or float32")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise TypeError("block_table must be int32 of shape (B, max_blocks)")
    if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
        raise TypeError("kv_lens must be int32 of shape (B,)")
    max_blocks = block_table.shape[1]
    if workspace is None:
        need = decode_paged_workspace_bytes(B, H, d, max_blocks, BS)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a GPU tensor")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    st = lib.g2attn_decode_paged(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                 _dev(out, "out"), _dev(block_table, "block_table"), max_blocks,
                                 _dev(kv_lens, "kv_lens"), B, H, KVH, d, BS, NB,
                                 float(query_scale), float(softcap), int(window),
                                 int(bool(is_local)), _DTYPES[q.dtype],
                                 _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_decode_paged")
    return out


def rope_(x, positions, *, base=10000.0, stream=None):
    """Rotary embedding of x (B, T, NH, d) in place at positions int32 (B, T)
    on the GPU; pair i is (x[..., i], x[..., i + d/2]) turned by
    pos * base**(-2i/d).  Returns x."""
    B, T, NH, d = x.shape
    if x.dtype not in _DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    if positions.dtype != torch.int32 or tuple(positions.shape) != (B, T):
        raise TypeError("positions must be int32 of shape (B, T)")
    st = lib.g2attn_rope(_dev(x, "x"), _dev(positions, "positions"), B, T, NH, d, float(base),
                         _DTYPES[x.dtype], _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_rope")
    return x


def softcap_(x, cap=30.0, stream=None):
    """Final-logit soft-cap in place: x = cap * tanh(x / cap).  Returns x."""
    if x.dtype not in _DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    st = lib.g2attn_softcap(_dev(x, "x"), x.numel(), float(cap), _DTYPES[x.dtype],
                            _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_softcap")
    return x


def backward_workspace_bytes(B, T, S, H):
    """Bytes of workspace prefill_backward needs (row statistics and the bf16
    dS blocks, about 2*B*T*S*H bytes)."""
    n = int(lib.g2attn_prefill_backward_workspace_bytes(int(B), int(T), int(S), int(H)))
    if n == 0:
        raise ValueError(f"invalid backward sizes B={B} T={T} S={S} H={H}")
    return n


def prefill_backward(q, k, v, out, dout, lse, *, query_scale, softcap=50.0, window=4096,
                     is_local, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the prefill for an upstream gradient dout of
    its output; out and lse come from prefill_lse() with the same arguments.
    bfloat16 only."""
    B, T, H, d = q.shape
    Bk, S, KVH, dk_ = k.shape
    if (Bk, dk_) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q and k/v")
    for t, name in ((out, "out"), (dout, "dout")):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("the backward pass takes bfloat16 tensors")
    if tuple(lse.shape) != (B, H, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 of shape (B, H, T)")
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is not None and (tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype):
            raise ValueError(f"{name} must have shape {tuple(ref.shape)} and dtype {ref.dtype}")
    need = backward_workspace_bytes(B, T, S, H)
    _check_workspace(workspace, need)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.g2attn_prefill_backward(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(dout, "dout"),
        _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), B, T, S, H, KVH, d,
        float(query_scale), float(softcap), int(window), int(bool(is_local)), G2_BF16,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream_handle(stream))
    if st != 0:
        raise G2attnError(st, "g2attn_prefill_backward")
    return dq, dk, dv
