"""Python binding of libkvc: one function per C entry point, argument marshalling only.

Every step of the path runs in the library's HIP kernels; torch supplies device memory
(tensors) and streams.  Tensors must be CUDA (HIP) tensors, contiguous, in the layouts of
include/kvc.h: bf16 data as torch.bfloat16, float outputs as torch.float32, widths as
torch.uint8.  Calls enqueue on the given stream (default: torch's current stream) and
return immediately.  A non-OK status raises KvcError.
"""

import ctypes
import struct

import numpy as np
import torch

from . import _lib as C


class KvcError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.name = C.STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


def _check(st):
    if st != C.KVC_OK:
        lib = C.load()
        raise KvcError(st, lib.kvc_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, got {type(t)}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def make_desc(n_q_heads, n_kv_heads, head_dim, n_keys, n_queries, causal=True, softmax_scale=0.0):
    return C.LayerDesc(int(n_q_heads), int(n_kv_heads), int(head_dim), 1 if causal else 0,
                       int(n_keys), int(n_queries), float(softmax_scale), 0)


def kvc_workspace_size(op, desc, mode=0):
    return int(C.load().kvc_workspace_size(int(op), ctypes.byref(desc), int(mode)))


def workspace(op, desc, mode=0, device="cuda"):
    """A device workspace of the size the library asks for (at least 256 bytes)."""
    n = max(256, kvc_workspace_size(op, desc, mode))
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def kvc_row_lse(desc, q, k, lse, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(C.load().kvc_row_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), wp, wn,
                                _stream(stream)))


def kvc_score_tokens(desc, mode, q, k, lse, scores, ws, hidden=None, w_o=None, v=None,
                     hidden_dim=0, stream=None):
    zp = None
    if mode == C.SCORE_MAX:
        if hidden_dim == 0 and hidden is not None:
            hidden_dim = hidden.shape[-1]
        zip_args = C.KvzipArgs(_ptr(hidden), _ptr(w_o), _ptr(v), int(hidden_dim), 0)
        zp = ctypes.byref(zip_args)
    wp, wn = _ws(ws)
    _check(C.load().kvc_score_tokens(ctypes.byref(desc), int(mode), _ptr(q), _ptr(k), _ptr(lse),
                                     zp, _ptr(scores), wp, wn, _stream(stream)))


def kvc_channel_weights(desc, q, k, w_c, ws, stream=None):
    wp, wn = _ws(ws)
    _check(C.load().kvc_channel_weights(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(w_c), wp, wn,
                                        _stream(stream)))


def kvc_allocate_bits(desc, stage, weight, bits_out, ws, sigma=None, bits_v=None, avg_bits=0.0,
                      keep_fraction=0.0, keep_bits=16, result=None, stream=None):
    wp, wn = _ws(ws)
    _check(C.load().kvc_allocate_bits(ctypes.byref(desc), int(stage), _ptr(weight), _ptr(sigma),
                                      _ptr(bits_v), float(avg_bits), float(keep_fraction),
                                      int(keep_bits), _ptr(bits_out), _ptr(result), wp, wn,
                                      _stream(stream)))


def kvc_keep_threshold(desc, scores, threshold, bits_out, window=128, keep_bits=16, kept=None,
                       stream=None):
    _check(C.load().kvc_keep_threshold(ctypes.byref(desc), _ptr(scores), float(threshold), int(window),
                                       int(keep_bits), _ptr(bits_out), _ptr(kept), _stream(stream)))


def alloc_result_buffer(device="cuda"):
    return torch.zeros(32, dtype=torch.uint8, device=device)


def decode_alloc_result(buf):
    raw = bytes(buf.cpu().numpy().tobytes())
    lam, budget, used, dist = struct.unpack("<dqqd", raw)
    return {"lam": lam, "budget": budget, "used": used, "distortion": dist}


def kvc_packed_capacity(desc, group_size=32):
    arr = (ctypes.c_size_t * C.PK_NBUF)()
    _check(C.load().kvc_packed_capacity(ctypes.byref(desc), int(group_size), arr))
    return [int(x) for x in arr]


class PackedCache:
    """Device buffers of one packed cache, sized by kvc_packed_capacity."""

    def __init__(self, desc, device="cuda", group_size=32):
        self.caps = kvc_packed_capacity(desc, group_size)
        self.buffers = {name: torch.empty(max(256, cap), dtype=torch.uint8, device=device)
                        for name, cap in zip(C.PK_NAMES, self.caps)}
        self.n_kv_heads = desc.n_kv_heads
        self.head_dim = desc.head_dim

    def c_struct(self):
        return C.PackedCacheC(*[self.buffers[n].data_ptr() for n in C.PK_NAMES])

    def header(self):
        n = C.HDR_GLOBAL + self.n_kv_heads * C.HDR_PER_HEAD
        return self.buffers["header"][: 8 * n].cpu().numpy().view(np.int64).copy()

    def to_numpy(self):
        """Copy every buffer back, trimmed to the lengths the header records."""
        H = self.header()
        out = {"header": H}
        spec = (("v_idx", np.int32, H[4], 1), ("v_words", np.uint32, H[5], 1),
                ("v_par", np.float32, H[6], 2), ("k_keep", np.int32, H[7], 1),
                ("k_vloc", np.int32, H[7], 1), ("k_words", np.uint32, H[8], 1),
                ("k_par", np.float32, H[9], 2))
        for name, dt, n, w in spec:
            nbytes = int(n) * w * np.dtype(dt).itemsize
            a = self.buffers[name][:nbytes].cpu().numpy().view(dt)
            out[name] = a.reshape(-1, 2) if w == 2 else a.copy()
        kw = self.buffers["k_width"][: self.n_kv_heads * self.head_dim].cpu().numpy()
        out["k_width"] = kw.reshape(self.n_kv_heads, self.head_dim).copy()
        return out


def kvc_quantize_pack(desc, k, v, bits_v, bits_k, cache, ws, group_size=32, stream=None):
    cs = cache.c_struct()
    wp, wn = _ws(ws)
    _check(C.load().kvc_quantize_pack(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(bits_v),
                                      _ptr(bits_k), int(group_size), ctypes.byref(cs), wp, wn,
                                      _stream(stream)))


def kvc_compressed_attend(desc, q, cache, out, lse, ws, stream=None):
    cs = cache.c_struct()
    wp, wn = _ws(ws)
    _check(C.load().kvc_compressed_attend(ctypes.byref(desc), _ptr(q), ctypes.byref(cs),
                                          _ptr(out), _ptr(lse), wp, wn, _stream(stream)))


def kvc_compressed_attend_append(desc, q, cache, k_new, v_new, out, lse, ws, stream=None):
    """k_new, v_new: bf16 tensors [H_kv][n_new][d] of the tokens generated after compression."""
    cs = cache.c_struct()
    wp, wn = _ws(ws)
    n_new = 0 if k_new is None else int(k_new.shape[-2])
    _check(C.load().kvc_compressed_attend_append(ctypes.byref(desc), _ptr(q), ctypes.byref(cs), _ptr(k_new),
                                                 _ptr(v_new), n_new, _ptr(out), _ptr(lse), wp, wn,
                                                 _stream(stream)))


def kvc_fidelity_terms(desc, y_hat, lse_hat, y, lse, terms, stream=None):
    """terms: float64 tensor [H_q][2] on the device (output)."""
    _check(C.load().kvc_fidelity_terms(ctypes.byref(desc), _ptr(y_hat), _ptr(lse_hat), _ptr(y), _ptr(lse),
                                       _ptr(terms), _stream(stream)))


def kvc_pilot_budgets(mse, total, floor_each=0):
    """Host call: mse is a sequence of per-head pilot MSE values; returns int64 numpy budgets."""
    m = np.ascontiguousarray(np.asarray(mse, dtype=np.float64).ravel())
    out = np.zeros(m.size, dtype=np.int64)
    _check(C.load().kvc_pilot_budgets(m.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(m.size), int(total),
                                      int(floor_each), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out


def kvc_ridge_value_fit(desc, n_compressed, q, k, v_r, y, lam, v_c, ws, stream=None):
    """k: bf16 [H_kv][n_c + m][d] (compressed keys first); v_r: bf16 [H_kv][m][d] or None when
    m = 0; y: float32 [H_q][Nq][d]; v_c: float32 [H_kv][n_c][d] (output)."""
    wp, wn = _ws(ws)
    _check(C.load().kvc_ridge_value_fit(ctypes.byref(desc), int(n_compressed), _ptr(q), _ptr(k), _ptr(v_r), _ptr(y),
                                        float(lam), _ptr(v_c), wp, wn, _stream(stream)))


def kvc_get_device_status(ws, stream=None):
    code = ctypes.c_int32(0)
    _check(C.load().kvc_get_device_status(_ptr(ws), ctypes.byref(code), _stream(stream)))
    return int(code.value)


def kvc_version():
    return C.load().kvc_version().decode()


def bf16_tensor(bits, device="cuda"):
    """numpy uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device` (exact)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
