"""CPU fp64 oracle for the Gemma 2 attention layer (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It is the slow, plain definition the GPU kernels are checked
against and shares no code with them (see g2_oracle.c for the definition and
the passages it follows).

Inputs are numpy arrays (or anything np.asarray accepts) that are converted to
float32 without change of value (bf16 and fp32 inputs are exact in float32);
results are float64.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libg2oracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_I = ctypes.c_int
_D = ctypes.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.g2o_softcap.argtypes = [_D, _D]
    lib.g2o_softcap.restype = _D
    lib.g2o_allowed.argtypes = [ctypes.c_int64, ctypes.c_int64, _I, _I]
    lib.g2o_allowed.restype = _I
    row_args = [_f32p, _f32p, _I, _I, _I, _I, _I, _I, _D, _D, _I, _I, _I, _I,
                _I, _f64p]
    lib.g2o_prefill_row_logits.argtypes = row_args
    lib.g2o_prefill_row_logits.restype = _I
    lib.g2o_prefill_row_weights.argtypes = row_args
    lib.g2o_prefill_row_weights.restype = _I
    lib.g2o_prefill.argtypes = [_f32p, _f32p, _f32p, _f64p, _I, _I, _I, _I, _I,
                                _I, _D, _D, _I, _I, _i64p, ctypes.c_int64]
    lib.g2o_prefill.restype = _I
    lib.g2o_decode.argtypes = [_f32p, _f32p, _f32p, _i32p, _f64p, _I, _I, _I,
                               _I, _I, _D, _D, _I, _I, _i64p, ctypes.c_int64]
    lib.g2o_decode.restype = _I
    lib.g2o_decode_paged.argtypes = [_f32p, _f32p, _f32p, _i32p, _I, _i32p, _f64p, _I,
                                     _I, _I, _I, _I, _I, _D, _D, _I, _I, _i64p,
                                     ctypes.c_int64]
    lib.g2o_decode_paged.restype = _I
    lib.g2o_prefill_lse.argtypes = [_f32p, _f32p, _f64p, _I, _I, _I, _I, _I, _I, _D, _D,
                                    _I, _I, _i64p, ctypes.c_int64]
    lib.g2o_prefill_lse.restype = _I
    lib.g2o_rope.argtypes = [_f32p, _i32p, _f64p, _I, _I, _I, _I, _D]
    lib.g2o_rope.restype = _I
    lib.g2o_softcap_array.argtypes = [_f32p, _f64p, ctypes.c_int64, _D]
    lib.g2o_softcap_array.restype = None
    lib.g2o_prefill_backward.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _f64p, _f64p, _I,
                                         _I, _I, _I, _I, _I, _D, _D, _I, _I]
    lib.g2o_prefill_backward.restype = _I
    lib.g2o_threads.argtypes = []
    lib.g2o_threads.restype = _I
    _lib = lib
    return lib


def _f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        a32 = a.astype(np.float32)
        if not np.array_equal(a32.astype(a.dtype), a, equal_nan=True):
            raise ValueError("oracle inputs must be exactly representable in float32")
        a = a32
    return np.ascontiguousarray(a)


def _ptr(a, t):
    return a.ctypes.data_as(t)


class OracleError(ValueError):
    pass


def softcap(x, cap):
    """cap * tanh(x / cap) in double; identity when cap <= 0 or cap = inf."""
    lib = _load()
    return lib.g2o_softcap(float(x), float(cap))


def threads():
    """Threads the oracle's parallel loops use."""
    return int(_load().g2o_threads())


def allowed(p, j, window, is_local):
    """Mask predicate: can query position p see key position j."""
    return bool(_load().g2o_allowed(int(p), int(j), int(window), int(bool(is_local))))


def _shape_prefill(q, k, v):
    B, T, H, d = q.shape
    B2, S, KVH, d2 = k.shape
    if (B2, d2) != (B, d) or v.shape != k.shape:
        raise OracleError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, T, S, H, KVH, d


def row_logits(q, k, b, t, h, *, query_scale, softcap, window, is_local):
    """Capped, masked logits of prefill row (b, t, h): float64 array of S."""
    q, k = _f32(q), _f32(k)
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    out = np.empty(S, np.float64)
    st = _load().g2o_prefill_row_logits(_ptr(q, _f32p), _ptr(k, _f32p), B, T, S, H,
                                        KVH, d, query_scale, softcap, window,
                                        int(bool(is_local)), b, t, h, _ptr(out, _f64p))
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def row_weights(q, k, b, t, h, *, query_scale, softcap, window, is_local):
    """Attention weights of prefill row (b, t, h): float64 array of S."""
    q, k = _f32(q), _f32(k)
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    out = np.empty(S, np.float64)
    st = _load().g2o_prefill_row_weights(_ptr(q, _f32p), _ptr(k, _f32p), B, T, S, H,
                                         KVH, d, query_scale, softcap, window,
                                         int(bool(is_local)), b, t, h, _ptr(out, _f64p))
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def prefill(q, k, v, *, query_scale, softcap, window, is_local, rows=None):
    """Attention output in float64.

    q: (B,T,H,d); k, v: (B,S,KVH,d).  rows=None returns (B,T,H,d); otherwise
    rows is a sequence of flat ids (b*T + t)*H + h and the result is (n, d).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, T, S, H, KVH, d = _shape_prefill(q, k, v)
    if rows is None:
        out = np.empty((B, T, H, d), np.float64)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rows.size, d), np.float64)
        rp, n = _ptr(rows, _i64p), rows.size
    st = _load().g2o_prefill(_ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
                             _ptr(out, _f64p), B, T, S, H, KVH, d, query_scale,
                             softcap, window, int(bool(is_local)), rp, n)
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def decode(q, k_cache, v_cache, kv_lens, *, query_scale, softcap, window, is_local,
           rows=None):
    """Decode output in float64.

    q: (B,1,H,d); caches: (B,S,KVH,d); kv_lens: (B,) ints >= 1.  Position j of
    sequence b is read from slot j mod S.  rows=None returns (B,1,H,d);
    otherwise rows are flat ids b*H + h and the result is (n, d).
    """
    q, kc, vc = _f32(q), _f32(k_cache), _f32(v_cache)
    B, T, H, d = q.shape
    if T != 1:
        raise OracleError("decode takes one query token per sequence")
    S, KVH = kc.shape[1], kc.shape[2]
    if kc.shape[0] != B or kc.shape[3] != d or vc.shape != kc.shape:
        raise OracleError("cache shape mismatch")
    lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    if lens.shape != (B,):
        raise OracleError("kv_lens must have B entries")
    if rows is None:
        out = np.empty((B, 1, H, d), np.float64)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rows.size, d), np.float64)
        rp, n = _ptr(rows, _i64p), rows.size
    st = _load().g2o_decode(_ptr(q, _f32p), _ptr(kc, _f32p), _ptr(vc, _f32p),
                            _ptr(lens, _i32p), _ptr(out, _f64p), B, S, H, KVH, d,
                            query_scale, softcap, window, int(bool(is_local)), rp, n)
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def decode_paged(q, k_pool, v_pool, block_table, kv_lens, *, query_scale, softcap,
                 window, is_local, rows=None):
    """Decode output in float64 against a paged KV cache.

    q: (B,1,H,d); pools: (num_blocks, block_size, KVH, d); block_table:
    (B, max_blocks) ints, entry [b][i] = physical block of positions
    i*block_size .. (i+1)*block_size - 1; kv_lens: (B,) ints in
    [1, max_blocks*block_size].  Only entries of blocks holding a position the
    query sees are read; a needed entry outside the pool gives a NaN row.
    rows=None returns (B,1,H,d); otherwise rows are flat ids b*H + h and the
    result is (n, d).
    """
    q, kp, vp = _f32(q), _f32(k_pool), _f32(v_pool)
    B, T, H, d = q.shape
    if T != 1:
        raise OracleError("decode takes one query token per sequence")
    NB, BS, KVH = kp.shape[0], kp.shape[1], kp.shape[2]
    if kp.shape[3] != d or vp.shape != kp.shape:
        raise OracleError("pool shape mismatch")
    table = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    if table.ndim != 2 or table.shape[0] != B:
        raise OracleError("block_table must be (B, max_blocks)")
    lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    if lens.shape != (B,):
        raise OracleError("kv_lens must have B entries")
    if rows is None:
        out = np.empty((B, 1, H, d), np.float64)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rows.size, d), np.float64)
        rp, n = _ptr(rows, _i64p), rows.size
    st = _load().g2o_decode_paged(_ptr(q, _f32p), _ptr(kp, _f32p), _ptr(vp, _f32p),
                                  _ptr(table, _i32p), table.shape[1], _ptr(lens, _i32p),
                                  _ptr(out, _f64p), B, H, KVH, d, BS, NB, query_scale,
                                  softcap, window, int(bool(is_local)), rp, n)
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def prefill_lse(q, k, *, query_scale, softcap, window, is_local, rows=None):
    """Natural-log log-sum-exp of each prefill row's capped, masked logits.

    q: (B,T,H,d); k: (B,S,KVH,d).  rows=None returns (B,T,H); otherwise rows
    are flat ids (b*T + t)*H + h and the result has one entry per row.
    """
    q, k = _f32(q), _f32(k)
    B, T, H, d = q.shape
    S, KVH = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise OracleError("shape mismatch")
    if rows is None:
        out = np.empty((B, T, H), np.float64)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty(rows.size, np.float64)
        rp, n = _ptr(rows, _i64p), rows.size
    st = _load().g2o_prefill_lse(_ptr(q, _f32p), _ptr(k, _f32p), _ptr(out, _f64p), B, T, S, H,
                                 KVH, d, query_scale, softcap, window, int(bool(is_local)),
                                 rp, n)
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def rope(x, positions, *, base=10000.0):
    """Rotary embedding of x (B, T, NH, d) at positions (B, T), in float64.
    Pair i is (x[..., i], x[..., i + d/2]), rotated by pos * base**(-2i/d)."""
    x = _f32(x)
    B, T, NH, d = x.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    if pos.shape != (B, T):
        raise OracleError("positions must be (B, T)")
    out = np.empty(x.shape, np.float64)
    st = _load().g2o_rope(_ptr(x, _f32p), _ptr(pos, _i32p), _ptr(out, _f64p), B, T, NH, d,
                          float(base))
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return out


def softcap_array(x, cap):
    """cap * tanh(x / cap) of every element, float64 (identity if cap <= 0 or inf)."""
    x = _f32(x)
    out = np.empty(x.shape, np.float64)
    _load().g2o_softcap_array(_ptr(x, _f32p), _ptr(out, _f64p), x.size, float(cap))
    return out


def prefill_backward(q, k, v, dout, *, query_scale, softcap, window, is_local):
    """Gradients (dq, dk, dv) in float64 of the prefill for an upstream
    gradient dout (B,T,H,d) of its output."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, T, S, H, KVH, d = _shape_prefill(q, k, v)
    if g.shape != q.shape:
        raise OracleError("dout must match q")
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(v.shape, np.float64)
    st = _load().g2o_prefill_backward(_ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
                                      _ptr(g, _f32p), _ptr(dq, _f64p), _ptr(dk, _f64p),
                                      _ptr(dv, _f64p), B, T, S, H, KVH, d, query_scale, softcap,
                                      window, int(bool(is_local)))
    if st != 0:
        raise OracleError(f"oracle rejected arguments (status {st})")
    return dq, dk, dv


def prefill_backward_at(q, k, v, dout, out, lse, *, rows=(), keys=(), query_scale, softcap,
                        window, is_local):
    """Gradients of the prefill at chosen rows and keys, in float64.

    Same definition as `prefill_backward` (Gemma 2 Guide, "Deep Dive" item 1,
    the cap's derivative 1 - tanh^2; the model card's one-layer pseudocode for
    the layer), evaluated only where asked, so that layers too large for the
    full backward can be checked at sampled places.  Each row's weights come
    from its capped logits and its log-sum-exp: w_j = exp(s_j - lse).

    q, dout: (B,T,H,d); k, v: (B,S,KVH,d); out (B,T,H,d) and lse (B,T,H) are
    the layer's output and natural-log log-sum-exp from this oracle's own
    `prefill` and `prefill_lse` on the same inputs.  rows: (b, t, h) triples;
    keys: (b, j, g) triples (g is the K/V head).  Returns (dq (len(rows), d),
    dk (len(keys), d), dv (len(keys), d)).
    """
    q = _f32(q).astype(np.float64)
    k = _f32(k).astype(np.float64)
    v = _f32(v).astype(np.float64)
    g = _f32(dout).astype(np.float64)
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    B, T, S, H, KVH, d = _shape_prefill(q, k, v)
    if g.shape != q.shape or out.shape != q.shape or lse.shape != (B, T, H):
        raise OracleError("dout/out must match q and lse must be (B, T, H)")
    G = H // KVH
    use_cap = softcap > 0 and np.isfinite(softcap)
    off = S - T
    dsum = np.einsum("bthe,bthe->bth", g, out)  # D = <dO, out> of every row

    def sees(p, j):  # the mask of `allowed`, elementwise over arrays
        ok = j <= p
        if is_local:
            ok &= j > p - window
        return ok

    def capped(x):  # capped logit s and the factor 1 - tanh^2 of dx = ds * factor
        if not use_cap:
            return x, np.ones_like(x)
        th = np.tanh(x / softcap)
        return softcap * th, 1.0 - th * th

    dq = np.zeros((len(rows), d))
    for n, (b, t, h) in enumerate(rows):
        kg, vg = k[b, :, h // G], v[b, :, h // G]                    # (S, d)
        x = query_scale * (kg @ q[b, t, h])
        s, fac = capped(x)
        js = np.arange(S)
        w = np.where(sees(t + off, js), np.exp(s - lse[b, t, h]), 0.0)
        ds = w * (vg @ g[b, t, h] - dsum[b, t, h])
        dq[n] = query_scale * ((ds * fac) @ kg)

    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    ts = np.arange(T)
    for n, (b, j, gh) in enumerate(keys):
        vis = sees(ts + off, j)
        for h in range(gh * G, gh * G + G):
            qh, gr = q[b, :, h], g[b, :, h]                            # (T, d)
            x = query_scale * (qh @ k[b, j, gh])
            s, fac = capped(x)
            w = np.where(vis, np.exp(s - lse[b, :, h]), 0.0)
            ds = w * (gr @ v[b, j, gh] - dsum[b, :, h])
            dk[n] += query_scale * ((ds * fac) @ qh)
            dv[n] += w @ gr
    return dq, dk, dv
