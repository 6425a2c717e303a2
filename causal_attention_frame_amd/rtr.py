"""Thin Python binding over librtr_attn.so (ctypes).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.  The
functions carry the C names; see include/rtr_attn.h for the full contract
(layouts, ownership, error behaviour).

There is no fallback: if the library is missing, loading it raises.
"""

import ctypes
import os

from .build import LIB_PATH

RTR_OK, RTR_EINVAL, RTR_EUNSUPPORTED, RTR_EHIP, RTR_ESTATE = 0, -1, -2, -3, -4
RTR_BF16, RTR_F32 = 0, 1
RTR_REF_KEEP, RTR_REF_REPLACE, RTR_REF_CLEAR = 0, 1, 2
RTR_MAX_WINDOW, RTR_MAX_REF, RTR_MAX_CHUNK = 64, 4, 16

_c_i32, _c_i64, _c_f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class rtr_kv_state(ctypes.Structure):
    _fields_ = [
        ("window_frames", _c_i32),
        ("count", _c_i32),
        ("head", _c_i32),
        ("ref_frames", _c_i32),
        ("ref_generation", _c_i64),
        ("next_frame_id", _c_i64),
        ("slot", _c_i32 * RTR_MAX_WINDOW),
        ("frame_id", _c_i64 * RTR_MAX_WINDOW),
        ("ring_slots", _c_i32),
    ]

    def as_dict(self):
        n = self.count
        return dict(window_frames=self.window_frames, ring_slots=self.ring_slots, count=n, head=self.head,
                    ref_frames=self.ref_frames, ref_generation=self.ref_generation,
                    next_frame_id=self.next_frame_id, slot=list(self.slot[:n]),
                    frame_id=list(self.frame_id[:n]))


# name -> (restype, argtypes); mirrors include/rtr_attn.h
_SIGNATURES = {
    "rtr_attn_block_causal": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32,
                                             _c_i64, ctypes.c_int, ctypes.c_int, _c_f32, _vp,
                                             ctypes.c_size_t, _vp]),
    "rtr_attn_workspace_size": (ctypes.c_int, [_c_i32, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "rtr_attn_block_causal_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64,
                                                 _c_i32, _c_i32, _c_i64, ctypes.c_int, _c_f32, _vp,
                                                 ctypes.c_size_t, _vp]),
    "rtr_attn_bwd_workspace_size": (ctypes.c_int, [_c_i64, _c_i32, _c_i32, ctypes.POINTER(ctypes.c_size_t)]),
    "rtr_kv_create": (ctypes.c_int, [ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                     _c_i64, _c_i32, _c_i32, ctypes.c_int]),
    "rtr_kv_create_slots": (ctypes.c_int, [ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                           _c_i32, _c_i64, _c_i32, _c_i32, ctypes.c_int]),
    "rtr_kv_destroy": (ctypes.c_int, [_vp]),
    "rtr_kv_append_evict": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _vp]),
    "rtr_kv_next_slots": (ctypes.c_int, [_vp, _c_i32, ctypes.POINTER(_c_i32)]),
    "rtr_kv_commit_inplace": (ctypes.c_int, [_vp, _c_i32]),
    "rtr_attn_stream_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, ctypes.c_int,
                                            _c_f32, _vp, ctypes.c_size_t, _vp]),
    "rtr_attn_stream_step_blocked": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                                    ctypes.c_int, _c_f32, _vp, ctypes.c_size_t, _vp]),
    "rtr_attn_stream_step_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                                _vp, _vp, _vp, _vp, _vp, _c_f32, _vp, ctypes.c_size_t,
                                                _vp]),
    "rtr_kv_set_ref_rope": (ctypes.c_int, [_vp, _vp, _c_i32, _c_f32, _c_i64]),
    "rtr_kv_reset_ref": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _c_i32, _c_i32, _vp]),
    "rtr_kv_get_state": (ctypes.c_int, [_vp, ctypes.POINTER(rtr_kv_state)]),
    "rtr_kv_set_state": (ctypes.c_int, [_vp, ctypes.POINTER(rtr_kv_state)]),
    "rtr_text_cache_create": (ctypes.c_int, [ctypes.POINTER(_vp), _vp, _vp, _c_i32, _c_i32, _c_i32,
                                             ctypes.c_int]),
    "rtr_text_cache_destroy": (ctypes.c_int, [_vp]),
    "rtr_text_cache_reset": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _vp]),
    "rtr_text_cache_state": (ctypes.c_int, [_vp, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i64)]),
    "rtr_attn_cross": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i64, ctypes.c_int, _c_f32, _vp,
                                      ctypes.c_size_t, _vp]),
    "rtr_attn_cross_bwd_workspace_size": (ctypes.c_int, [_c_i64, _c_i32, _c_i32, _c_i32,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
    "rtr_attn_cross_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _vp, _vp, _c_f32, _vp,
                                          ctypes.c_size_t, _vp]),
    "rtr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rtr_last_error": (ctypes.c_char_p, []),
    "rtr_version": (ctypes.c_int, []),
    "rtr_clock_sample": (ctypes.c_int, [_vp, _c_i64, _vp]),
    "rtr_attn_stream_step_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                                    ctypes.c_int, _c_f32, _vp]),
}

_lib = None


def lib():
    """Load librtr_attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class RtrError(RuntimeError):
    def __init__(self, code, fn):
        L = lib()
        msg = L.rtr_last_error().decode()
        super().__init__(f"{fn}: {L.rtr_status_string(code).decode()} ({code}): {msg}")
        self.code = code


def _check(code, fn):
    if code != RTR_OK:
        raise RtrError(code, fn)


# ---------------------------------------------------------------- marshalling
def _ptr(x):
    """Device address of a tensor (must be contiguous), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensors passed to librtr_attn must be contiguous")
    return x.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RTR_BF16
    if t.dtype == torch.float32:
        return RTR_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _workspace(ws):
    """(pointer, bytes) of an optional split-K workspace tensor."""
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def rtr_attn_workspace_size(d, dtype=RTR_BF16):
    """Bytes of split-K workspace the current device needs (0: never splits)."""
    n = ctypes.c_size_t(0)
    _check(lib().rtr_attn_workspace_size(int(d), int(dtype), ctypes.byref(n)), "rtr_attn_workspace_size")
    return n.value


def new_workspace(d, dtype=RTR_BF16, device="cuda"):
    """A device byte tensor sized for rtr_attn_workspace_size, or None when
    the configuration never splits."""
    import torch
    n = rtr_attn_workspace_size(d, dtype)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


# ---------------------------------------------------------------- full form
def rtr_attn_block_causal(q, k, v, tokens_per_frame, o=None, lse=None, scale=0.0,
                          out_dtype=None, want_lse=False, workspace=None, stream=None):
    """Frame-block-causal attention over one [T, H, d] sequence.
    Returns (o, lse or None)."""
    import torch
    T, H, d = q.shape
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((T, H, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_block_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), T, H, d,
                                       int(tokens_per_frame), _dtype_code(q), _dtype_code(o),
                                       float(scale), ws, ws_bytes, _stream(stream, q.device)),
           "rtr_attn_block_causal")
    return o, lse


def rtr_attn_bwd_workspace_size(T, H, d=128):
    """Bytes of device workspace rtr_attn_block_causal_bwd needs."""
    n = ctypes.c_size_t(0)
    _check(lib().rtr_attn_bwd_workspace_size(int(T), int(H), int(d), ctypes.byref(n)),
           "rtr_attn_bwd_workspace_size")
    return n.value


def rtr_attn_block_causal_bwd(q, k, v, o, lse, d_o, tokens_per_frame, dq=None, dk=None, dv=None,
                              scale=0.0, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of rtr_attn_block_causal for the upstream
    gradient d_o, from the forward's o and lse.  The workspace (a device byte
    tensor of rtr_attn_bwd_workspace_size bytes) is allocated when not given."""
    import torch
    T, H, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(1, rtr_attn_bwd_workspace_size(T, H, d)), dtype=torch.uint8,
                                device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_block_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o),
                                           _ptr(dq), _ptr(dk), _ptr(dv), T, H, d,
                                           int(tokens_per_frame), _dtype_code(q), float(scale), ws,
                                           ws_bytes, _stream(stream, q.device)),
           "rtr_attn_block_causal_bwd")
    return dq, dk, dv


# ---------------------------------------------------------------- the cache
def rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, d_o, chunk_frames, block_frames=1, dq=None, dk=None,
                             dv=None, dk_cache=None, dv_cache=None, want_cache_grads=False, scale=0.0,
                             workspace=None, stream=None):
    """Gradients of a streaming step from its forward o and lse (the cache in
    the state it had then).  Returns (dq, dk, dv, dk_cache, dv_cache); the
    cache gradients ([P, H, d], reference then window frames oldest first) are
    None unless given or want_cache_grads."""
    import torch
    Tq, H, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if want_cache_grads and dk_cache is None:
        st = rtr_kv_get_state(kv)
        P = (st.ref_frames + st.count) * kv.kpf
        dk_cache = torch.empty((P, H, d), dtype=q.dtype, device=q.device)
        dv_cache = torch.empty((P, H, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, rtr_attn_bwd_workspace_size(Tq, H, d)), dtype=torch.uint8,
                                device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_stream_step_bwd(kv.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                          _ptr(d_o), int(chunk_frames), int(block_frames), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(dk_cache), _ptr(dv_cache),
                                          float(scale), ws, ws_bytes, _stream(stream, q.device)),
           "rtr_attn_stream_step_bwd")
    return dq, dk, dv, dk_cache, dv_cache


class KVCache:
    """One layer's reference-anchored rolling KV cache (handle + buffers).

    k_ring, v_ring: [N, k, H, d] with N = ring_slots (W when None);
    k_ref, v_ref: [R_cap, k, H, d] (or None).  Tensors are kept referenced for
    the handle's lifetime.  Integer device addresses are accepted too
    (metadata-only use)."""

    def __init__(self, k_ring, v_ring, k_ref, v_ref, window_frames, ref_capacity_frames,
                 tokens_per_frame, H, d, dtype, ring_slots=None):
        self._bufs = (k_ring, v_ring, k_ref, v_ref)
        self.W, self.R_cap, self.kpf, self.H, self.d = (window_frames, ref_capacity_frames,
                                                        tokens_per_frame, H, d)
        self.N = window_frames if ring_slots is None else ring_slots
        self.dtype = dtype
        h = _vp()
        if ring_slots is None:
            _check(lib().rtr_kv_create(ctypes.byref(h), _ptr(k_ring), _ptr(v_ring), _ptr(k_ref),
                                       _ptr(v_ref), window_frames, ref_capacity_frames,
                                       tokens_per_frame, H, d, dtype), "rtr_kv_create")
        else:
            _check(lib().rtr_kv_create_slots(ctypes.byref(h), _ptr(k_ring), _ptr(v_ring), _ptr(k_ref),
                                             _ptr(v_ref), window_frames, ring_slots, ref_capacity_frames,
                                             tokens_per_frame, H, d, dtype), "rtr_kv_create_slots")
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            lib().rtr_kv_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rtr_kv_create(k_ring, v_ring, k_ref, v_ref, window_frames, ref_capacity_frames,
                  tokens_per_frame, H, d, dtype=RTR_BF16):
    return KVCache(k_ring, v_ring, k_ref, v_ref, window_frames, ref_capacity_frames,
                   tokens_per_frame, H, d, dtype)


def rtr_kv_create_slots(k_ring, v_ring, k_ref, v_ref, window_frames, ring_slots, ref_capacity_frames,
                        tokens_per_frame, H, d, dtype=RTR_BF16):
    return KVCache(k_ring, v_ring, k_ref, v_ref, window_frames, ref_capacity_frames,
                   tokens_per_frame, H, d, dtype, ring_slots=ring_slots)


def rtr_kv_destroy(kv):
    kv.close()


def rtr_kv_append_evict(kv, k_new, v_new, n_frames, stream=None):
    dev = k_new.device if hasattr(k_new, "device") else None
    _check(lib().rtr_kv_append_evict(kv.handle, _ptr(k_new), _ptr(v_new), int(n_frames),
                                     _stream(stream, dev) if dev is not None else stream),
           "rtr_kv_append_evict")


def rtr_kv_next_slots(kv, n_frames):
    arr = (_c_i32 * max(1, n_frames))()
    _check(lib().rtr_kv_next_slots(kv.handle, int(n_frames), arr), "rtr_kv_next_slots")
    return list(arr[:n_frames])


def rtr_kv_commit_inplace(kv, n_frames):
    _check(lib().rtr_kv_commit_inplace(kv.handle, int(n_frames)), "rtr_kv_commit_inplace")


def rtr_attn_stream_step(kv, q, k, v, chunk_frames, o=None, lse=None, scale=0.0, out_dtype=None,
                         want_lse=False, workspace=None, stream=None):
    """One streaming step for a chunk of `chunk_frames` frames.  Returns (o, lse or None)."""
    import torch
    Tq, H, d = q.shape
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((Tq, H, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_stream_step(kv.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      int(chunk_frames), _dtype_code(o), float(scale), ws, ws_bytes,
                                      _stream(stream, q.device)),
           "rtr_attn_stream_step")
    return o, lse


def rtr_attn_stream_step_noalloc(kv, q, k, v, chunk_frames, o, lse=None, block_frames=1, scale=0.0,
                                 stream=None):
    """The streaming step with the library's static split-K scratch: o (and
    lse) are caller-provided, nothing is allocated.  Returns (o, lse)."""
    _check(lib().rtr_attn_stream_step_noalloc(kv.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              int(chunk_frames), int(block_frames), _dtype_code(o),
                                              float(scale), _stream(stream, q.device)),
           "rtr_attn_stream_step_noalloc")
    return o, lse


def rtr_attn_stream_step_blocked(kv, q, k, v, chunk_frames, block_frames, o=None, lse=None, scale=0.0,
                                 out_dtype=None, want_lse=False, workspace=None, stream=None):
    """A streaming step whose in-chunk mask works in blocks of `block_frames`
    frames (chunk-level causality).  Returns (o, lse or None)."""
    import torch
    Tq, H, d = q.shape
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((Tq, H, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_stream_step_blocked(kv.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              int(chunk_frames), int(block_frames), _dtype_code(o),
                                              float(scale), ws, ws_bytes, _stream(stream, q.device)),
           "rtr_attn_stream_step_blocked")
    return o, lse


def rtr_kv_set_ref_rope(kv, k_ref_view, rope_pairs=22, rope_base=10000.0, position_offset=1):
    """Keep the anchored reference in front of the oldest visible frame (rotary
    position re-encoding into k_ref_view); k_ref_view None switches it off."""
    if k_ref_view is not None:
        kv._view = k_ref_view  # keep the buffer alive with the handle
    _check(lib().rtr_kv_set_ref_rope(kv.handle, _ptr(k_ref_view), int(rope_pairs), float(rope_base),
                                     int(position_offset)), "rtr_kv_set_ref_rope")


def rtr_kv_reset_ref(kv, mode, k_ref=None, v_ref=None, ref_frames=1, keep_recent=1, stream=None):
    dev = k_ref.device if hasattr(k_ref, "device") else None
    s = _stream(stream, dev) if dev is not None else stream
    _check(lib().rtr_kv_reset_ref(kv.handle, int(mode), _ptr(k_ref), _ptr(v_ref), int(ref_frames),
                                  int(keep_recent), s), "rtr_kv_reset_ref")


def rtr_kv_get_state(kv):
    st = rtr_kv_state()
    _check(lib().rtr_kv_get_state(kv.handle, ctypes.byref(st)), "rtr_kv_get_state")
    return st


def rtr_kv_set_state(kv, st):
    _check(lib().rtr_kv_set_state(kv.handle, ctypes.byref(st)), "rtr_kv_set_state")


# ---------------------------------------------------------------- text cross-attention
class TextCache:
    """One layer's text cross-attention cache (handle + buffers [capacity, H, d])."""

    def __init__(self, k_buf, v_buf, capacity_tokens, H, d, dtype):
        self._bufs = (k_buf, v_buf)
        self.capacity, self.H, self.d, self.dtype = capacity_tokens, H, d, dtype
        h = _vp()
        _check(lib().rtr_text_cache_create(ctypes.byref(h), _ptr(k_buf), _ptr(v_buf), capacity_tokens,
                                           H, d, dtype), "rtr_text_cache_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            lib().rtr_text_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rtr_text_cache_create(k_buf, v_buf, capacity_tokens, H, d, dtype=RTR_BF16):
    return TextCache(k_buf, v_buf, capacity_tokens, H, d, dtype)


def rtr_text_cache_reset(tc, k_text, v_text, n_tokens, stream=None):
    dev = k_text.device if k_text is not None else tc._bufs[0].device
    _check(lib().rtr_text_cache_reset(tc.handle, _ptr(k_text), _ptr(v_text), int(n_tokens),
                                      _stream(stream, dev)), "rtr_text_cache_reset")


def rtr_text_cache_state(tc):
    n, g = _c_i32(0), _c_i64(0)
    _check(lib().rtr_text_cache_state(tc.handle, ctypes.byref(n), ctypes.byref(g)), "rtr_text_cache_state")
    return n.value, g.value


def rtr_attn_cross(tc, q, o=None, lse=None, scale=0.0, out_dtype=None, want_lse=False, workspace=None,
                   stream=None):
    """Cross-attention of q [Tq, H, d] to the cache's text tokens.  Returns (o, lse or None)."""
    import torch
    Tq, H, d = q.shape
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((Tq, H, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_cross(tc.handle, _ptr(q), _ptr(o), _ptr(lse), Tq, _dtype_code(o), float(scale), ws,
                                ws_bytes, _stream(stream, q.device)), "rtr_attn_cross")
    return o, lse


def rtr_version():
    return lib().rtr_version()


def rtr_attn_cross_bwd_workspace_size(Tq, n_text, H, d=128):
    """Bytes of device workspace rtr_attn_cross_bwd needs with text gradients."""
    n = ctypes.c_size_t(0)
    _check(lib().rtr_attn_cross_bwd_workspace_size(int(Tq), int(n_text), int(H), int(d), ctypes.byref(n)),
           "rtr_attn_cross_bwd_workspace_size")
    return n.value


def rtr_attn_cross_bwd(tc, q, o, lse, d_o, dq=None, dk_text=None, dv_text=None, want_text_grads=False,
                       scale=0.0, workspace=None, stream=None):
    """Gradients of rtr_attn_cross from its o and lse.  Returns (dq, dk_text,
    dv_text); the text gradients ([n, H, d]) are None unless given or
    want_text_grads."""
    import torch
    Tq, H, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    if want_text_grads and dk_text is None:
        n, _ = rtr_text_cache_state(tc)
        dk_text = torch.empty((n, H, d), dtype=q.dtype, device=q.device)
        dv_text = torch.empty((n, H, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        if dk_text is not None:
            nbytes = rtr_attn_cross_bwd_workspace_size(Tq, dk_text.shape[0], H, d)
        else:
            nbytes = rtr_attn_bwd_workspace_size(Tq, H, d)
        workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=q.device)
    ws, ws_bytes = _workspace(workspace)
    _check(lib().rtr_attn_cross_bwd(tc.handle, _ptr(q), _ptr(o), _ptr(lse), _ptr(d_o), Tq, _ptr(dq),
                                    _ptr(dk_text), _ptr(dv_text), float(scale), ws, ws_bytes,
                                    _stream(stream, q.device)),
           "rtr_attn_cross_bwd")
    return dq, dk_text, dv_text


def rtr_clock_sample(device, span_ticks=5000, stream=None):
    """Shader clock in MHz over ~span_ticks / 100 MHz (default 50 us), measured
    by the library's clock probe on `device`'s current stream; synchronizes."""
    import torch
    buf = torch.zeros(2, dtype=torch.int64, device=device)
    _check(lib().rtr_clock_sample(_ptr(buf), int(span_ticks), _stream(stream, buf.device)),
           "rtr_clock_sample")
    t = buf.cpu().tolist()
    return 100.0 * t[0] / t[1] if t[1] > 0 else float("nan")

