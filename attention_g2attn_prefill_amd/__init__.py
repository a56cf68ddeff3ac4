"""Gemma 2 attention layer for MI355X (gfx950): prefill, decode and paged decode,
plus the steps on either side of it (rotary embedding, final-logit soft-cap).

The compute path is the C-ABI library libg2attn.so (hand-written HIP kernels);
this package is a thin ctypes binding over it plus a seeded input generator
(`synth`).  The binding is loaded on first use of any entry point and raises
if the library has not been built: there is no CPU fallback.
"""
_BINDING_NAMES = (
    "prefill", "prefill_lse", "prefill_backward", "backward_workspace_bytes", "decode", "decode_workspace_bytes", "check_args", "status_string",
    "decode_paged", "decode_paged_workspace_bytes", "check_paged_args", "rope_", "softcap_",
    "library_path", "G2attnError", "lib", "build_id", "decode_noalloc",
    "NOALLOC_SCRATCH_BYTES",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
