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


BF16, F32, F64, U8, I64 = torch.bfloat16, torch.float32, torch.float64, torch.uint8, torch.int64


def _arg(t, name, dtype, numel, optional=False):
    """Check what the C ABI cannot see of one tensor argument: its dtype, the element count the
    descriptor implies, and contiguity.  Returns (name, tensor), or None for an absent optional
    argument.  The device is checked by _addresses() once every argument has passed this."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    return (name, t)


def _addresses(*args):
    """Device addresses of checked arguments (None stays None), after checking that every tensor
    lives on the current GPU.  A wrong tensor raises here, before anything is enqueued: on the
    device it would be read or written out of bounds."""
    for a in args:
        if a is not None and a[1].device.type != "cuda":
            raise ValueError(f"{a[0]}: tensor on {a[1].device}, expected a GPU tensor")
    if any(a is not None for a in args):
        cur = torch.cuda.current_device()
        for a in args:
            if a is not None and a[1].device.index != cur:
                raise ValueError(f"{a[0]}: tensor on {a[1].device}, but the current device is cuda:{cur}")
    out = tuple(None if a is None else a[1].data_ptr() for a in args)
    return out if len(out) != 1 else out[0]


def _dims(desc):
    return (int(desc.n_q_heads), int(desc.n_kv_heads), int(desc.head_dim), int(desc.n_keys),
            int(desc.n_queries))


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
    """A workspace is a uint8 GPU tensor of any size (the library checks that it is large enough)."""
    return _arg(ws, "ws", U8, None, optional=True)


def _nbytes(ws):
    return 0 if ws is None else ws.numel()


def kvc_row_lse(desc, q, k, lse, ws=None, stream=None):
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k, "k", BF16, hkv * n * d), _arg(lse, "lse", F32, hq * nq), _ws(ws))
    qp, kp, lp, wp = _addresses(*a)
    _check(C.load().kvc_row_lse(ctypes.byref(desc), qp, kp, lp, wp, _nbytes(ws), _stream(stream)))


def kvc_row_lse_noalloc(desc, q, k, lse, stream=None):
    """kvc_row_lse with the library's static scratch instead of a workspace (allocates nothing)."""
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k, "k", BF16, hkv * n * d), _arg(lse, "lse", F32, hq * nq))
    qp, kp, lp = _addresses(*a)
    _check(C.load().kvc_row_lse_noalloc(ctypes.byref(desc), qp, kp, lp, _stream(stream)))


def kvc_score_tokens(desc, mode, q, k, lse, scores, ws, hidden=None, w_o=None, v=None,
                     hidden_dim=0, stream=None):
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k, "k", BF16, hkv * n * d), _arg(lse, "lse", F32, hq * nq),
         _arg(scores, "scores", F32, hkv * n), _ws(ws))
    zp = None
    if mode == C.SCORE_MAX:
        if hidden_dim == 0 and hidden is not None:
            hidden_dim = hidden.shape[-1]
        dh = int(hidden_dim)
        z = (_arg(hidden, "hidden", BF16, nq * dh), _arg(w_o, "w_o", BF16, dh * hq * d),
             _arg(v, "v", BF16, hkv * n * d))
        hp, op, vp = _addresses(*z)
        zip_args = C.KvzipArgs(hp, op, vp, dh, 0)
        zp = ctypes.byref(zip_args)
    qp, kp, lp, sp, wp = _addresses(*a)
    _check(C.load().kvc_score_tokens(ctypes.byref(desc), int(mode), qp, kp, lp, zp, sp, wp, _nbytes(ws),
                                     _stream(stream)))


def kvc_channel_weights(desc, q, k, w_c, ws, stream=None):
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k, "k", BF16, hkv * n * d), _arg(w_c, "w_c", F32, hkv * d), _ws(ws))
    qp, kp, cp, wp = _addresses(*a)
    _check(C.load().kvc_channel_weights(ctypes.byref(desc), qp, kp, cp, wp, _nbytes(ws), _stream(stream)))


def kvc_allocate_bits(desc, stage, weight, bits_out, ws, sigma=None, bits_v=None, avg_bits=0.0,
                      keep_fraction=0.0, keep_bits=16, result=None, stream=None):
    """weight, sigma: float32 [H_kv][N] (V tokens, top-k) or [H_kv][d] (K channels); bits_v: uint8
    [H_kv][N] (K channels only); bits_out: uint8, the shape of weight; result: the 32-byte device
    buffer of alloc_result_buffer(), or None."""
    hq, hkv, d, n, nq = _dims(desc)
    units = hkv * d if stage == C.ALLOC_K_CHANNELS else hkv * n
    a = (_arg(weight, "weight", F32, units), _arg(sigma, "sigma", F32, units, optional=True),
         _arg(bits_v, "bits_v", U8, hkv * n, optional=(stage != C.ALLOC_K_CHANNELS)),
         _arg(bits_out, "bits_out", U8, units), _arg(result, "result", U8, 32, optional=True), _ws(ws))
    tp, sp, vp, bp, rp, wp = _addresses(*a)
    _check(C.load().kvc_allocate_bits(ctypes.byref(desc), int(stage), tp, sp, vp, float(avg_bits),
                                      float(keep_fraction), int(keep_bits), bp, rp, wp, _nbytes(ws),
                                      _stream(stream)))


def kvc_keep_threshold(desc, scores, threshold, bits_out, window=128, keep_bits=16, kept=None,
                       stream=None):
    """scores: float32 [H_kv][N]; bits_out: uint8 [H_kv][N]; kept: int64 [H_kv] or None."""
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(scores, "scores", F32, hkv * n), _arg(bits_out, "bits_out", U8, hkv * n),
         _arg(kept, "kept", I64, hkv, optional=True))
    sp, bp, kp = _addresses(*a)
    _check(C.load().kvc_keep_threshold(ctypes.byref(desc), sp, float(threshold), int(window), int(keep_bits),
                                       bp, kp, _stream(stream)))


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

    def c_struct_for(self, desc, group_size=32):
        """The C struct, after checking that every buffer holds what `desc` may need and lives on
        the current GPU (the kernels index the buffers by the descriptor's sizes)."""
        need = kvc_packed_capacity(desc, group_size)
        bufs = []
        for name, cap in zip(C.PK_NAMES, need):
            b = self.buffers[name]
            if b.numel() < cap:
                raise ValueError(f"packed cache buffer {name}: {b.numel()} bytes, {cap} needed for this layer")
            bufs.append(_arg(b, f"packed cache buffer {name}", U8, None))
        return C.PackedCacheC(*_addresses(*bufs))

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
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(k, "k", BF16, hkv * n * d), _arg(v, "v", BF16, hkv * n * d), _arg(bits_v, "bits_v", U8, hkv * n),
         _arg(bits_k, "bits_k", U8, hkv * d), _ws(ws))
    kp, vp, bvp, bkp, wp = _addresses(*a)
    cs = cache.c_struct_for(desc, group_size)
    _check(C.load().kvc_quantize_pack(ctypes.byref(desc), kp, vp, bvp, bkp, int(group_size), ctypes.byref(cs), wp,
                                      _nbytes(ws), _stream(stream)))


def kvc_compressed_attend(desc, q, cache, out, lse, ws, stream=None):
    """q: bf16 [H_q][Nq][d] (the last Nq rows of the sequence); out: float32 [H_q][Nq][d]; lse:
    float32 [H_q][Nq]."""
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(out, "out", F32, hq * nq * d), _arg(lse, "lse", F32, hq * nq),
         _ws(ws))
    qp, op, lp, wp = _addresses(*a)
    cs = cache.c_struct_for(desc)
    _check(C.load().kvc_compressed_attend(ctypes.byref(desc), qp, ctypes.byref(cs), op, lp, wp, _nbytes(ws),
                                          _stream(stream)))


def kvc_compressed_attend_append(desc, q, cache, k_new, v_new, out, lse, ws, stream=None):
    """k_new, v_new: bf16 tensors [H_kv][n_new][d] of the tokens generated after compression (both
    or neither)."""
    hq, hkv, d, n, nq = _dims(desc)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new: give both or neither")
    n_new = 0 if k_new is None else int(k_new.shape[-2])
    if k_new is not None and (tuple(k_new.shape) != (hkv, n_new, d) or tuple(v_new.shape) != (hkv, n_new, d)):
        raise ValueError(f"k_new {tuple(k_new.shape)}, v_new {tuple(v_new.shape)}: expected [{hkv}][n_new][{d}] both")
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k_new, "k_new", BF16, hkv * n_new * d, optional=True),
         _arg(v_new, "v_new", BF16, hkv * n_new * d, optional=True), _arg(out, "out", F32, hq * nq * d),
         _arg(lse, "lse", F32, hq * nq), _ws(ws))
    qp, knp, vnp, op, lp, wp = _addresses(*a)
    cs = cache.c_struct_for(desc)
    _check(C.load().kvc_compressed_attend_append(ctypes.byref(desc), qp, ctypes.byref(cs), knp, vnp, n_new, op, lp,
                                                 wp, _nbytes(ws), _stream(stream)))


def kvc_fidelity_terms(desc, y_hat, lse_hat, y, lse, terms, stream=None):
    """y_hat, y: float32 [H_q][Nq][d]; lse_hat, lse: float32 [H_q][Nq]; terms: float64 [H_q][2] (output)."""
    hq, hkv, d, n, nq = _dims(desc)
    a = (_arg(y_hat, "y_hat", F32, hq * nq * d), _arg(lse_hat, "lse_hat", F32, hq * nq),
         _arg(y, "y", F32, hq * nq * d), _arg(lse, "lse", F32, hq * nq), _arg(terms, "terms", F64, hq * 2))
    _check(C.load().kvc_fidelity_terms(ctypes.byref(desc), *_addresses(*a), _stream(stream)))


def kvc_pilot_budgets(mse, total, floor_each=0):
    """Host call: mse is a sequence of per-head pilot MSE values; returns int64 numpy budgets."""
    m = np.ascontiguousarray(np.asarray(mse, dtype=np.float64).ravel())
    out = np.zeros(m.size, dtype=np.int64)
    _check(C.load().kvc_pilot_budgets(m.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(m.size), int(total),
                                      int(floor_each), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out


def kvc_ridge_value_fit(desc, n_compressed, q, k, v_r, y, lam, v_c, ws, stream=None):
    """k: bf16 [H_kv][n_c + m][d] (compressed keys first; desc.n_keys = n_c + m); v_r: bf16
    [H_kv][m][d] or None when m = 0; y: float32 [H_q][Nq][d]; v_c: float32 [H_kv][n_c][d] (output)."""
    hq, hkv, d, n, nq = _dims(desc)
    nc = int(n_compressed)
    m = n - nc
    a = (_arg(q, "q", BF16, hq * nq * d), _arg(k, "k", BF16, hkv * n * d),
         _arg(v_r, "v_r", BF16, hkv * m * d, optional=(m == 0)), _arg(y, "y", F32, hq * nq * d),
         _arg(v_c, "v_c", F32, hkv * nc * d), _ws(ws))
    qp, kp, vp, yp, cp, wp = _addresses(*a)
    _check(C.load().kvc_ridge_value_fit(ctypes.byref(desc), nc, qp, kp, vp, yp, float(lam), cp, wp, _nbytes(ws),
                                        _stream(stream)))


def kvc_get_device_status(ws, stream=None):
    code = ctypes.c_int32(0)
    _check(C.load().kvc_get_device_status(_addresses(_ws(ws)), ctypes.byref(code), _stream(stream)))
    return int(code.value)


def kvc_version():
    return C.load().kvc_version().decode()


def bf16_tensor(bits, device="cuda"):
    """numpy uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device` (exact)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
