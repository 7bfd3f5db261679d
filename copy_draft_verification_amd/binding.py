"""Python binding of libswitchsd.so (argument marshalling only).

Every function here forwards device pointers and sizes to the C ABI declared
in include/switchsd.h; every step of the copy path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
import ctypes
import os

import torch  # loaded first so the library binds to the same HIP runtime as torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libswitchsd.so")

SSD_F32, SSD_BF16, SSD_BF16_ROWS = 0, 1, 2
_lib = None

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGS = {
    "ssd_abi_version": (ctypes.c_int, []),
    "ssd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssd_probe_score": (ctypes.c_int, [_c_p, ctypes.c_int, _c_p, _i32, _i32, ctypes.c_float, _c_p,
                                       _c_p, _c_p]),
    "ssd_kgram_retrieve": (ctypes.c_int, [_c_p, _c_p, _i32, _i32, _i32, _i32, _c_p, _c_p, _c_p,
                                          _c_p, _c_p, _c_p, _c_p]),
    "ssd_probe_kgram_retrieve": (ctypes.c_int, [_c_p, ctypes.c_int, _c_p, _i32, ctypes.c_float, _c_p,
                                                _c_p, _c_p, _c_p, _i32, _i32, _i32, _i32, _c_p, _c_p,
                                                _c_p, _c_p, _c_p, _c_p]),
    "ssd_pack_weight_bytes": (ctypes.c_size_t, [_i32, _i32]),
    "ssd_pack_weight": (ctypes.c_int, [_c_p, _i32, _i32, _c_p, ctypes.c_size_t, _c_p]),
    "ssd_pack_gate_up_bytes": (ctypes.c_size_t, [_i32, _i32]),
    "ssd_pack_gate_up": (ctypes.c_int, [_c_p, _c_p, _i32, _i32, _c_p, ctypes.c_size_t, _c_p]),
    "ssd_verify_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _i32, ctypes.c_int]),
    "ssd_blocktri_verify": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _c_p, _c_p,
                                           _c_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                           ctypes.c_int, ctypes.c_float, _c_p, _c_p, _c_p, _c_p,
                                           ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "ssd_blocktri_verify_accept": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _c_p,
                                                  _c_p, _c_p, _c_p, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, ctypes.c_int, ctypes.c_float, _c_p,
                                                  _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                  ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "ssd_blocktri_verify_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _c_p,
                                                   _c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                                   _i32, ctypes.c_int, ctypes.c_float, _c_p, _c_p,
                                                   _c_p, _c_p]),
    "ssd_accept_longest": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i32, _i32, _i32, _c_p, _c_p,
                                          _c_p, _c_p, _c_p]),
    "ssd_commit_accepted": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i32, _i32, _i32,
                                           _i32, _i32, ctypes.c_int, _c_p, _c_p, ctypes.c_int64,
                                           _c_p, _c_p, _c_p, _c_p]),
    "ssd_blocktri_verify_sample": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _c_p,
                                                  _c_p, _c_p, _c_p, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, ctypes.c_int, ctypes.c_float,
                                                  ctypes.c_float, ctypes.c_uint64, _c_p, _c_p, _c_p,
                                                  _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t,
                                                  _c_p, _c_p, _c_p]),
    "ssd_accept_sample": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i32, _i32, _i32,
                                         ctypes.c_uint64, _c_p, _c_p, _c_p, _c_p]),
    "ssd_verify_forward_workspace_bytes": (ctypes.c_size_t, [_i32] * 9),
    "ssd_verify_forward": (ctypes.c_int, [_c_p, _c_p, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _i32,
                                          _c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _i32, ctypes.c_float, ctypes.c_float, _c_p, _c_p, _c_p,
                                          ctypes.c_size_t, _c_p, _c_p, _c_p]),
    "ssd_copy_labels_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64]),
    "ssd_copy_labels": (ctypes.c_int, [_c_p, _c_p, _i32, ctypes.c_int64, _i32, _c_p, _c_p,
                                       ctypes.c_size_t, _c_p]),
    "ssd_probe_logits": (ctypes.c_int, [_c_p, ctypes.c_int, _c_p, _i32, ctypes.c_int64, _i32, _c_p,
                                        _c_p]),
    "ssd_calibrate_workspace_bytes": (ctypes.c_size_t, [_i32, ctypes.c_int64]),
    "ssd_calibrate": (ctypes.c_int, [_c_p, _c_p, _i32, ctypes.c_int64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                     _c_p, _c_p, ctypes.c_size_t, _c_p]),
}


class SwitchSDError(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load the C-ABI library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m copy_draft_verification_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        msg = load().ssd_status_string(status).decode()
        raise SwitchSDError(f"{what} failed: status {status} ({msg})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SwitchSDError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise SwitchSDError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise SwitchSDError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise SwitchSDError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    return t


def _out(t, name, dtype, shape, device):
    """A caller-supplied output: a contiguous tensor of exactly this dtype and shape on
    the device of the inputs (the kernels write every element of it)."""
    _dev(t, name, (dtype,))
    _shape(t, name, shape)
    if t.device != device:
        raise SwitchSDError(f"{name} is on {t.device}, the inputs on {device}")
    return t


def _same_device(device, *named):
    for t, n in named:
        if t is not None and t.device != device:
            raise SwitchSDError(f"{n} is on {t.device}, expected {device}")


def _torch_stream(stream, device):
    return stream if stream is not None else torch.cuda.current_stream(device)


def _torch_stream_handle(ts):
    return ctypes.c_void_p(ts.cuda_stream)


def _alloc(stream, shape, dtype, device):
    """torch.empty on the stream the library's kernels will use: the caching allocator
    then ties the block to that stream, so it is not handed to other work before the
    kernels queued there are done with it."""
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(workspace, need, stream, device):
    if workspace is None:
        return _alloc(stream, (max(need, 1),), torch.uint8, device)
    _dev(workspace, "workspace", (torch.uint8,))
    if workspace.device != device:
        raise SwitchSDError(f"workspace is on {workspace.device}, expected {device}")
    if workspace.numel() < need:
        raise SwitchSDError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    return workspace


def _dt(t):
    return SSD_BF16 if t.dtype == torch.bfloat16 else SSD_F32


def abi_version():
    return load().ssd_abi_version()


def probe_score(h, w, tau, z_out=None, fire_out=None, stream=None):
    """Probe decision per sequence.  h [B, hid] (fp32 | bf16), w [hid] fp32."""
    _dev(h, "h", (torch.float32, torch.bfloat16))
    _dev(w, "w", (torch.float32,))
    if h.dim() != 2:
        raise SwitchSDError("h must be [B, hid]")
    B, hid = h.shape
    _shape(w, "w", (hid,))
    dev = h.device
    _same_device(dev, (w, "w"))
    ts = _torch_stream(stream, dev)
    if z_out is None:
        z_out = _alloc(ts, (B,), torch.float32, dev)
    if fire_out is None:
        fire_out = _alloc(ts, (B,), torch.uint8, dev)
    _out(z_out, "z_out", torch.float32, (B,), dev)
    _out(fire_out, "fire_out", torch.uint8, (B,), dev)
    _check(load().ssd_probe_score(_ptr(h), _dt(h), _ptr(w), B, hid, float(tau), _ptr(z_out),
                                  _ptr(fire_out), _torch_stream_handle(ts)), "probe_score")
    return z_out, fire_out


def kgram_retrieve(ids, cu_len, kappa, W, D, fire=None, out=None, stream=None):
    """kappa-gram evidence + candidates.  Returns dict of match_end, n_match, cand,
    cand_len, copy_gate (device tensors)."""
    _dev(ids, "ids", (torch.int32,))
    _dev(cu_len, "cu_len", (torch.int32,))
    B = cu_len.numel() - 1
    dev = ids.device
    _same_device(dev, (cu_len, "cu_len"), (fire, "fire"))
    if fire is not None:
        _dev(fire, "fire", (torch.uint8,))
        _shape(fire, "fire", (B,))
    ts = _torch_stream(stream, dev)
    shapes = {"match_end": ((B, W), torch.int32), "n_match": ((B,), torch.int32),
              "cand": ((B, W, D), torch.int32), "cand_len": ((B, W), torch.int32),
              "copy_gate": ((B,), torch.uint8)}
    if out is None:
        out = {k: _alloc(ts, sh, dt, dev) for k, (sh, dt) in shapes.items()}
    for k, (sh, dt) in shapes.items():
        _out(out[k], f"out[{k!r}]", dt, sh, dev)
    _check(load().ssd_kgram_retrieve(_ptr(ids), _ptr(cu_len), B, kappa, W, D, _ptr(fire),
                                     _ptr(out["match_end"]), _ptr(out["n_match"]), _ptr(out["cand"]),
                                     _ptr(out["cand_len"]), _ptr(out["copy_gate"]),
                                     _torch_stream_handle(ts)),
           "kgram_retrieve")
    return out


def probe_kgram_retrieve(h, w, tau, ids, cu_len, kappa, W, D, z_out=None, fire_out=None, out=None,
                         stream=None):
    """probe_score then kgram_retrieve gated by its decision, in one launch.  Returns
    (z_out, fire_out, out) with out as from kgram_retrieve."""
    _dev(h, "h", (torch.float32, torch.bfloat16))
    _dev(w, "w", (torch.float32,))
    _dev(ids, "ids", (torch.int32,))
    _dev(cu_len, "cu_len", (torch.int32,))
    if h.dim() != 2:
        raise SwitchSDError("h must be [B, hid]")
    B, hid = h.shape
    if cu_len.numel() != B + 1:
        raise SwitchSDError(f"cu_len has {cu_len.numel()} entries, expected B + 1 = {B + 1}")
    _shape(w, "w", (hid,))
    dev = h.device
    _same_device(dev, (w, "w"), (ids, "ids"), (cu_len, "cu_len"))
    ts = _torch_stream(stream, dev)
    if z_out is None:
        z_out = _alloc(ts, (B,), torch.float32, dev)
    if fire_out is None:
        fire_out = _alloc(ts, (B,), torch.uint8, dev)
    _out(z_out, "z_out", torch.float32, (B,), dev)
    _out(fire_out, "fire_out", torch.uint8, (B,), dev)
    shapes = {"match_end": ((B, W), torch.int32), "n_match": ((B,), torch.int32),
              "cand": ((B, W, D), torch.int32), "cand_len": ((B, W), torch.int32),
              "copy_gate": ((B,), torch.uint8)}
    if out is None:
        out = {k: _alloc(ts, sh, dt, dev) for k, (sh, dt) in shapes.items()}
    for k, (sh, dt) in shapes.items():
        _out(out[k], f"out[{k!r}]", dt, sh, dev)
    _check(load().ssd_probe_kgram_retrieve(_ptr(h), _dt(h), _ptr(w), hid, float(tau), _ptr(z_out),
                                           _ptr(fire_out), _ptr(ids), _ptr(cu_len), B, kappa, W, D,
                                           _ptr(out["match_end"]), _ptr(out["n_match"]),
                                           _ptr(out["cand"]), _ptr(out["cand_len"]),
                                           _ptr(out["copy_gate"]), _torch_stream_handle(ts)),
           "probe_kgram_retrieve")
    return z_out, fire_out, out


class PackedWeight:
    """A bf16 weight matrix [rows, K] rearranged by pack_weight, or a gate / up pair
    [rows, K] each rearranged by pack_gate_up (pair=True); device bytes in `data`."""

    def __init__(self, data, rows, K, pair=False):
        self.data, self.rows, self.K, self.pair = data, int(rows), int(K), bool(pair)


def pack_weight_bytes(rows, K):
    return int(load().ssd_pack_weight_bytes(int(rows), int(K)))


def pack_gate_up_bytes(inter, K):
    return int(load().ssd_pack_gate_up_bytes(int(inter), int(K)))


def pack_weight(w, out=None, stream=None):
    """Rearrange a bf16 weight matrix [rows, K] (an LM head or a projection) into the
    packed layout the bf16 calls read.  Returns a PackedWeight."""
    _dev(w, "w", (torch.bfloat16,))
    if w.dim() != 2:
        raise SwitchSDError("w must be [rows, K]")
    rows, K = w.shape
    need = pack_weight_bytes(rows, K)
    ts = _torch_stream(stream, w.device)
    if out is None:
        out = _alloc(ts, (max(need, 1),), torch.uint8, w.device)
    _dev(out, "out", (torch.uint8,))
    _same_device(w.device, (out, "out"))
    _check(load().ssd_pack_weight(_ptr(w), rows, K, _ptr(out), out.numel() * out.element_size(),
                                  _torch_stream_handle(ts)), "pack_weight")
    return PackedWeight(out, rows, K)


def pack_gate_up(w_gate, w_up, out=None, stream=None):
    """Pack an MLP's gate and up projections ([inter, K] bf16 each) into one buffer.
    Returns a PackedWeight with pair=True."""
    _dev(w_gate, "w_gate", (torch.bfloat16,))
    _dev(w_up, "w_up", (torch.bfloat16,))
    if w_gate.shape != w_up.shape:
        raise SwitchSDError("w_gate and w_up must have the same shape")
    if w_gate.dim() != 2:
        raise SwitchSDError("w_gate must be [inter, K]")
    inter, K = w_gate.shape
    need = pack_gate_up_bytes(inter, K)
    dev = w_gate.device
    _same_device(dev, (w_up, "w_up"))
    ts = _torch_stream(stream, dev)
    if out is None:
        out = _alloc(ts, (max(need, 1),), torch.uint8, dev)
    _dev(out, "out", (torch.uint8,))
    _same_device(dev, (out, "out"))
    _check(load().ssd_pack_gate_up(_ptr(w_gate), _ptr(w_up), inter, K, _ptr(out),
                                   out.numel() * out.element_size(), _torch_stream_handle(ts)),
           "pack_gate_up")
    return PackedWeight(out, inter, K, pair=True)


def _packed(w, name, rows, K, pair=False):
    """Device tensor of a PackedWeight argument, checked against the expected shape."""
    if not isinstance(w, PackedWeight) or w.pair != pair:
        how = "pack_gate_up" if pair else "pack_weight"
        raise SwitchSDError(f"{name} must be packed with {how} first")
    if (rows is not None and w.rows != rows) or w.K != K:
        raise SwitchSDError(f"{name} is packed as [{w.rows}, {w.K}], expected [{rows}, {K}]")
    return w.data


def _lm_arg(lm_head, dtype, K, rows_ok=False):
    """(tensor, V, dtype code) of the LM-head argument: for bf16 a PackedWeight, or, where
    the call takes it (rows_ok), the plain [V, K] bf16 matrix (SSD_BF16_ROWS); a plain
    [V, K] fp32 matrix otherwise."""
    if dtype == torch.bfloat16:
        if rows_ok and isinstance(lm_head, torch.Tensor):
            _dev(lm_head, "lm_head", (torch.bfloat16,))
            if lm_head.dim() != 2 or lm_head.shape[1] != K:
                raise SwitchSDError(f"lm_head must be [V, {K}], got {tuple(lm_head.shape)}")
            return lm_head, lm_head.shape[0], SSD_BF16_ROWS
        return _packed(lm_head, "lm_head", None, K), lm_head.rows, SSD_BF16
    _dev(lm_head, "lm_head", (torch.float32,))
    if lm_head.dim() != 2 or lm_head.shape[1] != K:
        raise SwitchSDError(f"lm_head has K = {lm_head.shape[-1]}, the rows have {K}")
    return lm_head, lm_head.shape[0], SSD_F32


def verify_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, V, dtype):
    code = SSD_BF16 if dtype == torch.bfloat16 else SSD_F32
    return int(load().ssd_verify_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, V, code))


def _verify_inputs(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len, copy_gate, W, D, dtypes):
    """Checks shared by the verification calls; returns (B, R, Hq, Hkv, d)."""
    for t, n in ((q, "q"), (k_pre, "k_pre"), (v_pre, "v_pre"), (k_cand, "k_cand"),
                 (v_cand, "v_cand")):
        _dev(t, n, dtypes)
        if t.dtype != q.dtype:
            raise SwitchSDError(f"{n} dtype {t.dtype} differs from q dtype {q.dtype}")
    _dev(cu_len, "cu_len", (torch.int32,))
    _dev(cand_len, "cand_len", (torch.int32,))
    _dev(copy_gate, "copy_gate", (torch.uint8,))
    if q.dim() != 4 or k_pre.dim() != 3:
        raise SwitchSDError("q must be [B, R, Hq, d] and k_pre [N, Hkv, d]")
    B, R, Hq, d = q.shape
    Hkv = k_pre.shape[1]
    if R != 1 + W * D:
        raise SwitchSDError(f"q has {R} rows per sequence, 1 + W*D = {1 + W * D}")
    _shape(k_pre, "k_pre", (k_pre.shape[0], Hkv, d))
    _shape(v_pre, "v_pre", k_pre.shape)
    _shape(k_cand, "k_cand", (B, W * D, Hkv, d))
    _shape(v_cand, "v_cand", (B, W * D, Hkv, d))
    _shape(cand_len, "cand_len", (B, W))
    _shape(cu_len, "cu_len", (B + 1,))
    _shape(copy_gate, "copy_gate", (B,))
    _same_device(q.device, (k_pre, "k_pre"), (v_pre, "v_pre"), (k_cand, "k_cand"),
                 (v_cand, "v_cand"), (cu_len, "cu_len"), (cand_len, "cand_len"),
                 (copy_gate, "copy_gate"))
    return B, R, Hq, Hkv, d


def blocktri_verify(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand_len, copy_gate, lm_head,
                    W, D, scale, attn_out=None, argmax_out=None, logits_out=None, workspace=None,
                    events=None, stream=None):
    """One verification pass.  q [B, R, Hq, d]; k_pre/v_pre [N, Hkv, d]; k_cand/v_cand
    [B, W*D, Hkv, d]; cand_len [B, W]; cu_len [B+1]; copy_gate [B]; lm_head [V, Hq*d]
    (fp32), or for bf16 a PackedWeight (the fast layout) or the plain [V, Hq*d] matrix.
    Outputs, when given: attn_out [B, R, Hq*d] of
    q's dtype, argmax_out [B, R] int32, logits_out [B, R, V] float32; workspace uint8
    of at least verify_workspace_bytes.  cu_len[B] <= N is the caller's to keep (it
    lives on the device).  Returns (attn_out, argmax_out)."""
    B, R, Hq, Hkv, d = _verify_inputs(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len,
                                      copy_gate, W, D, (torch.float32, torch.bfloat16))
    lm, V, code = _lm_arg(lm_head, q.dtype, Hq * d, rows_ok=True)
    dev = q.device
    ts = _torch_stream(stream, dev)
    if attn_out is None:
        attn_out = _alloc(ts, (B, R, Hq * d), q.dtype, dev)
    _out(attn_out, "attn_out", q.dtype, (B, R, Hq * d), dev)
    if argmax_out is None:
        argmax_out = _alloc(ts, (B, R), torch.int32, dev)
    _out(argmax_out, "argmax_out", torch.int32, (B, R), dev)
    if logits_out is not None:
        _out(logits_out, "logits_out", torch.float32, (B, R, V), dev)
    need = verify_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, V, q.dtype)
    workspace = _workspace(workspace, need, ts, dev)
    ev0, ev1 = _events(events)
    _check(load().ssd_blocktri_verify(
        _ptr(q), _ptr(k_pre), _ptr(v_pre), _ptr(cu_len), int(max_n), _ptr(k_cand), _ptr(v_cand),
        _ptr(cand_len), _ptr(copy_gate), _ptr(lm), B, W, D, Hq, Hkv, d, V, code,
        float(scale), _ptr(attn_out), _ptr(argmax_out), _ptr(logits_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ev0, ev1, _torch_stream_handle(ts)),
        "blocktri_verify")
    return attn_out, argmax_out


def blocktri_verify_noalloc(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand_len, copy_gate,
                            lm_head, W, D, scale, attn_out, argmax_out, logits_out=None, stream=None):
    """blocktri_verify with no workspace: the library's own device scratch (64 MiB per
    GPU) holds the partials, so nothing is allocated.  The outputs must be given
    (attn_out [B, R, Hq*d] of q's dtype, argmax_out [B, R] int32, logits_out [B, R, V]
    float32 or None).  Calls that overlap on one GPU race on the shared scratch."""
    B, R, Hq, Hkv, d = _verify_inputs(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len,
                                      copy_gate, W, D, (torch.float32, torch.bfloat16))
    lm, V, code = _lm_arg(lm_head, q.dtype, Hq * d, rows_ok=True)
    dev = q.device
    ts = _torch_stream(stream, dev)
    _out(attn_out, "attn_out", q.dtype, (B, R, Hq * d), dev)
    _out(argmax_out, "argmax_out", torch.int32, (B, R), dev)
    if logits_out is not None:
        _out(logits_out, "logits_out", torch.float32, (B, R, V), dev)
    _check(load().ssd_blocktri_verify_noalloc(
        _ptr(q), _ptr(k_pre), _ptr(v_pre), _ptr(cu_len), int(max_n), _ptr(k_cand), _ptr(v_cand),
        _ptr(cand_len), _ptr(copy_gate), _ptr(lm), B, W, D, Hq, Hkv, d, V, code, float(scale),
        _ptr(attn_out), _ptr(argmax_out), _ptr(logits_out), _torch_stream_handle(ts)),
        "blocktri_verify_noalloc")
    return attn_out, argmax_out


def blocktri_verify_accept(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand, cand_len, copy_gate,
                           lm_head, W, D, scale, attn_out=None, argmax_out=None, out=None,
                           workspace=None, events=None, stream=None):
    """blocktri_verify then accept_longest on its argmax, in the verification's
    launches (bf16: the accept runs in the LM-head launch).  cand [B, W, D] int32;
    other arguments as blocktri_verify; out as accept_longest's.  Returns
    (attn_out, argmax_out, out)."""
    B, R, Hq, Hkv, d = _verify_inputs(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len,
                                      copy_gate, W, D, (torch.float32, torch.bfloat16))
    _dev(cand, "cand", (torch.int32,))
    _shape(cand, "cand", (B, W, D))
    lm, V, code = _lm_arg(lm_head, q.dtype, Hq * d, rows_ok=True)
    dev = q.device
    _same_device(dev, (cand, "cand"))
    ts = _torch_stream(stream, dev)
    if attn_out is None:
        attn_out = _alloc(ts, (B, R, Hq * d), q.dtype, dev)
    _out(attn_out, "attn_out", q.dtype, (B, R, Hq * d), dev)
    if argmax_out is None:
        argmax_out = _alloc(ts, (B, R), torch.int32, dev)
    _out(argmax_out, "argmax_out", torch.int32, (B, R), dev)
    shapes = {"accept_len": (B, W), "best_w": (B,), "best_len": (B,), "next_token": (B,)}
    if out is None:
        out = {k: _alloc(ts, sh, torch.int32, dev) for k, sh in shapes.items()}
    for k, sh in shapes.items():
        _out(out[k], f"out[{k!r}]", torch.int32, sh, dev)
    need = verify_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, V, q.dtype)
    workspace = _workspace(workspace, need, ts, dev)
    ev0, ev1 = _events(events)
    _check(load().ssd_blocktri_verify_accept(
        _ptr(q), _ptr(k_pre), _ptr(v_pre), _ptr(cu_len), int(max_n), _ptr(k_cand), _ptr(v_cand),
        _ptr(cand), _ptr(cand_len), _ptr(copy_gate), _ptr(lm), B, W, D, Hq, Hkv, d, V, code,
        float(scale), _ptr(attn_out), _ptr(argmax_out), _ptr(out["accept_len"]), _ptr(out["best_w"]),
        _ptr(out["best_len"]), _ptr(out["next_token"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ev0, ev1, _torch_stream_handle(ts)),
        "blocktri_verify_accept")
    return attn_out, argmax_out, out


def _events(events):
    if events is None:
        return None, None
    if not events[0].cuda_event or not events[1].cuda_event:
        raise SwitchSDError("events must be created (recorded once) before they are passed")
    return ctypes.c_void_p(events[0].cuda_event), ctypes.c_void_p(events[1].cuda_event)


def blocktri_verify_sample(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand, cand_len,
                           copy_gate, lm_head, W, D, scale, temperature, seed, attn_out=None,
                           rows=None, workspace=None, events=None, stream=None):
    """Verification pass at temperature > 0 (bf16; lm_head a PackedWeight).  Shapes as
    blocktri_verify; cand
    [B, W, D] int32.  Returns (attn_out, rows) with rows a dict of n_children [B, R],
    children / child_w [B, R, W], child_logit [B, R, W], lse [B, R], resample [B, R]."""
    B, R, Hq, Hkv, d = _verify_inputs(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len,
                                      copy_gate, W, D, (torch.bfloat16,))
    _dev(cand, "cand", (torch.int32,))
    _shape(cand, "cand", (B, W, D))
    lm, V, code = _lm_arg(lm_head, q.dtype, Hq * d)
    dev = q.device
    ts = _torch_stream(stream, dev)
    if attn_out is None:
        attn_out = _alloc(ts, (B, R, Hq * d), q.dtype, dev)
    _out(attn_out, "attn_out", q.dtype, (B, R, Hq * d), dev)
    shapes = {"n_children": ((B, R), torch.int32), "children": ((B, R, W), torch.int32),
              "child_w": ((B, R, W), torch.int32), "child_logit": ((B, R, W), torch.float32),
              "lse": ((B, R), torch.float32), "resample": ((B, R), torch.int32)}
    if rows is None:
        rows = {k: _alloc(ts, sh, dt, dev) for k, (sh, dt) in shapes.items()}
    for k, (sh, dt) in shapes.items():
        _out(rows[k], f"rows[{k!r}]", dt, sh, dev)
    need = verify_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, V, q.dtype)
    workspace = _workspace(workspace, need, ts, dev)
    ev0, ev1 = _events(events)
    _check(load().ssd_blocktri_verify_sample(
        _ptr(q), _ptr(k_pre), _ptr(v_pre), _ptr(cu_len), int(max_n), _ptr(k_cand), _ptr(v_cand),
        _ptr(cand), _ptr(cand_len), _ptr(copy_gate), _ptr(lm), B, W, D, Hq, Hkv, d, V,
        code, float(scale), float(temperature), int(seed) & ((1 << 64) - 1), _ptr(attn_out),
        _ptr(rows["n_children"]), _ptr(rows["children"]), _ptr(rows["child_w"]),
        _ptr(rows["child_logit"]), _ptr(rows["lse"]), _ptr(rows["resample"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ev0, ev1, _torch_stream_handle(ts)),
        "blocktri_verify_sample")
    return attn_out, rows


def accept_sample(rows, copy_gate, W, D, seed, out=None, stream=None):
    """Acceptance walk at temperature > 0 over the rows written by
    blocktri_verify_sample.  Returns dict best_w, best_len, next_token [B]."""
    _dev(copy_gate, "copy_gate", (torch.uint8,))
    B = copy_gate.numel()
    dev = copy_gate.device
    R = 1 + W * D
    shapes = {"n_children": ((B, R), torch.int32), "child_w": ((B, R, W), torch.int32),
              "child_logit": ((B, R, W), torch.float32), "lse": ((B, R), torch.float32),
              "resample": ((B, R), torch.int32)}
    for k, (sh, dt) in shapes.items():
        _out(rows[k], f"rows[{k!r}]", dt, sh, dev)
    ts = _torch_stream(stream, dev)
    if out is None:
        out = {k: _alloc(ts, (B,), torch.int32, dev) for k in ("best_w", "best_len", "next_token")}
    for k in ("best_w", "best_len", "next_token"):
        _out(out[k], f"out[{k!r}]", torch.int32, (B,), dev)
    _check(load().ssd_accept_sample(
        _ptr(rows["n_children"]), _ptr(rows["child_w"]), _ptr(rows["child_logit"]),
        _ptr(rows["lse"]), _ptr(rows["resample"]), _ptr(copy_gate), B, W, D,
        int(seed) & ((1 << 64) - 1), _ptr(out["best_w"]), _ptr(out["best_len"]),
        _ptr(out["next_token"]), _torch_stream_handle(ts)), "accept_sample")
    return out


def accept_longest(cand, cand_len, copy_gate, argmax, W, D, out=None, stream=None):
    """Longest accepted continuation.  Returns dict accept_len, best_w, best_len, next_token."""
    for t, n in ((cand, "cand"), (cand_len, "cand_len"), (argmax, "argmax")):
        _dev(t, n, (torch.int32,))
    _dev(copy_gate, "copy_gate", (torch.uint8,))
    B = copy_gate.numel()
    dev = cand.device
    _shape(cand, "cand", (B, W, D))
    _shape(cand_len, "cand_len", (B, W))
    _shape(argmax, "argmax", (B, 1 + W * D))
    _same_device(dev, (cand_len, "cand_len"), (argmax, "argmax"), (copy_gate, "copy_gate"))
    ts = _torch_stream(stream, dev)
    shapes = {"accept_len": (B, W), "best_w": (B,), "best_len": (B,), "next_token": (B,)}
    if out is None:
        out = {k: _alloc(ts, sh, torch.int32, dev) for k, sh in shapes.items()}
    for k, sh in shapes.items():
        _out(out[k], f"out[{k!r}]", torch.int32, sh, dev)
    _check(load().ssd_accept_longest(_ptr(cand), _ptr(cand_len), _ptr(copy_gate), _ptr(argmax), B, W,
                                     D, _ptr(out["accept_len"]), _ptr(out["best_w"]),
                                     _ptr(out["best_len"]), _ptr(out["next_token"]),
                                     _torch_stream_handle(ts)),
           "accept_longest")
    return out


def commit_accepted(k_cand, v_cand, cand, best_w, best_len, next_token, W, D, k_cache, v_cache,
                    cache_off, out=None, stream=None):
    """Copy the accepted candidate rows' K/V into the cache and list the tokens that
    extend the context.  k_cand/v_cand [B, W*D, Hkv, d]; k_cache/v_cache [rows, Hkv, d]
    (same dtype); cache_off [B] int64.  Returns dict tokens [B, D+1], n_tokens [B]."""
    dts = (torch.float32, torch.bfloat16)
    for t, n in ((k_cand, "k_cand"), (v_cand, "v_cand"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n, dts)
        if t.dtype != k_cand.dtype:
            raise SwitchSDError(f"{n} dtype {t.dtype} differs from k_cand dtype {k_cand.dtype}")
    for t, n in ((cand, "cand"), (best_w, "best_w"), (best_len, "best_len"),
                 (next_token, "next_token")):
        _dev(t, n, (torch.int32,))
    _dev(cache_off, "cache_off", (torch.int64,))
    if k_cand.dim() != 4:
        raise SwitchSDError("k_cand must be [B, W*D, Hkv, d]")
    B, _, Hkv, d = k_cand.shape
    _shape(k_cand, "k_cand", (B, W * D, Hkv, d))
    _shape(v_cand, "v_cand", k_cand.shape)
    _shape(cand, "cand", (B, W, D))
    for t, n in ((best_w, "best_w"), (best_len, "best_len"), (next_token, "next_token"),
                 (cache_off, "cache_off")):
        _shape(t, n, (B,))
    if k_cache.shape[1:] != k_cand.shape[2:] or v_cache.shape != k_cache.shape:
        raise SwitchSDError("k_cache / v_cache must be [rows, Hkv, d] matching k_cand")
    dev = k_cand.device
    _same_device(dev, (v_cand, "v_cand"), (cand, "cand"), (best_w, "best_w"),
                 (best_len, "best_len"), (next_token, "next_token"), (k_cache, "k_cache"),
                 (v_cache, "v_cache"), (cache_off, "cache_off"))
    ts = _torch_stream(stream, dev)
    if out is None:
        out = {"tokens": _alloc(ts, (B, D + 1), torch.int32, dev),
               "n_tokens": _alloc(ts, (B,), torch.int32, dev)}
    _out(out["tokens"], "out['tokens']", torch.int32, (B, D + 1), dev)
    _out(out["n_tokens"], "out['n_tokens']", torch.int32, (B,), dev)
    _check(load().ssd_commit_accepted(
        _ptr(k_cand), _ptr(v_cand), _ptr(cand), _ptr(best_w), _ptr(best_len), _ptr(next_token),
        B, W, D, Hkv, d, _dt(k_cand), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        _ptr(cache_off), _ptr(out["tokens"]), _ptr(out["n_tokens"]), _torch_stream_handle(ts)),
        "commit_accepted")
    return out


def copy_labels_workspace_bytes(total_n):
    return load().ssd_copy_labels_workspace_bytes(int(total_n))


def copy_labels(ids, cu_len, n_train=5, labels=None, workspace=None, stream=None):
    """Copy-mode label (uint8) of every position of the concatenated contexts.
    ids [total_n] int32, cu_len [B+1] int32 (cu_len[B] == total_n)."""
    _dev(ids, "ids", (torch.int32,))
    _dev(cu_len, "cu_len", (torch.int32,))
    n, B = ids.numel(), cu_len.numel() - 1
    dev = ids.device
    _same_device(dev, (cu_len, "cu_len"))
    ts = _torch_stream(stream, dev)
    if labels is None:
        labels = _alloc(ts, (n,), torch.uint8, dev)
    _out(labels, "labels", torch.uint8, (n,), dev)
    workspace = _workspace(workspace, copy_labels_workspace_bytes(n), ts, dev)
    _check(load().ssd_copy_labels(_ptr(ids), _ptr(cu_len), B, n, n_train, _ptr(labels),
                                  _ptr(workspace), workspace.numel(), _torch_stream_handle(ts)),
           "copy_labels")
    return labels


def probe_logits(h, w, z_out=None, stream=None):
    """z[l][i] = w[l] . h[l][i].  h [L, N, hid] (fp32 | bf16), w [L, hid] fp32 -> z [L, N] fp32."""
    _dev(h, "h", (torch.float32, torch.bfloat16))
    _dev(w, "w", (torch.float32,))
    if h.dim() != 3:
        raise SwitchSDError("h must be [L, N, hid]")
    L, N, hid = h.shape
    if tuple(w.shape) != (L, hid):
        raise SwitchSDError(f"w must be [{L}, {hid}], got {tuple(w.shape)}")
    dev = h.device
    _same_device(dev, (w, "w"))
    ts = _torch_stream(stream, dev)
    if z_out is None:
        z_out = _alloc(ts, (L, N), torch.float32, dev)
    _out(z_out, "z_out", torch.float32, (L, N), dev)
    _check(load().ssd_probe_logits(_ptr(h), _dt(h), _ptr(w), L, N, hid, _ptr(z_out),
                                   _torch_stream_handle(ts)), "probe_logits")
    return z_out


def calibrate_workspace_bytes(L, N):
    return load().ssd_calibrate_workspace_bytes(int(L), int(N))


def calibrate(z, labels, out=None, workspace=None, stream=None):
    """Per-layer F1-optimal threshold and ROC AUC, then the layer and tau.  z [L, N] fp32,
    labels [N] uint8.  Returns dict thr [L], counts [L, 4] (TP, FP, FN, P), u2 [L] int64,
    auc [L], best_layer [1] int32, tau [1] fp32 (device tensors)."""
    _dev(z, "z", (torch.float32,))
    _dev(labels, "labels", (torch.uint8,))
    L, N = z.shape
    if labels.numel() != N:
        raise SwitchSDError(f"labels must hold {N} entries, got {labels.numel()}")
    dev = z.device
    _same_device(dev, (labels, "labels"))
    ts = _torch_stream(stream, dev)
    shapes = {"thr": ((L,), torch.float32), "counts": ((L, 4), torch.int32),
              "u2": ((L,), torch.int64), "auc": ((L,), torch.float32),
              "best_layer": ((1,), torch.int32), "tau": ((1,), torch.float32)}
    if out is None:
        out = {k: _alloc(ts, sh, dt, dev) for k, (sh, dt) in shapes.items()}
    for k, (sh, dt) in shapes.items():
        _out(out[k], f"out[{k!r}]", dt, sh, dev)
    workspace = _workspace(workspace, calibrate_workspace_bytes(L, N), ts, dev)
    _check(load().ssd_calibrate(_ptr(z), _ptr(labels), L, N, _ptr(out["thr"]), _ptr(out["counts"]),
                                _ptr(out["u2"]), _ptr(out["auc"]), _ptr(out["best_layer"]),
                                _ptr(out["tau"]), _ptr(workspace), workspace.numel(),
                                _torch_stream_handle(ts)), "calibrate")
    return out


LAYER_FIELDS = ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate_up", "w_down", "k_cache", "v_cache")


def pack_layer(layer):
    """A layer dict with plain bf16 projections (wqkv, wo, w_gate, w_up, w_down) ->
    the dict verify_forward takes, its projections packed."""
    out = {k: layer[k] for k in ("attn_norm", "mlp_norm", "k_cache", "v_cache")}
    out["wqkv"], out["wo"] = pack_weight(layer["wqkv"]), pack_weight(layer["wo"])
    out["w_gate_up"] = pack_gate_up(layer["w_gate"], layer["w_up"])
    out["w_down"] = pack_weight(layer["w_down"])
    return out


class _Layer(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in LAYER_FIELDS]


def verify_forward_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, inter, V):
    return load().ssd_verify_forward_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, inter, V)


def verify_forward(ids, cu_len, max_n, cand, cand_len, copy_gate, embed, layers, final_norm,
                   lm_head, W, D, Hq, Hkv, d, inter, rope_base=500000.0, eps=1e-5,
                   argmax_out=None, x_out=None, workspace=None, events=None, stream=None):
    """The verification pass as a full target forward (bf16 weights; lm_head a
    PackedWeight).  layers: list of dicts with the LAYER_FIELDS entries, the
    projections packed (pack_layer).  Returns (argmax [B, R] int32, x_out or None)."""
    for t, n in ((ids, "ids"), (cu_len, "cu_len"), (cand, "cand"), (cand_len, "cand_len")):
        _dev(t, n, (torch.int32,))
    _dev(copy_gate, "copy_gate", (torch.uint8,))
    for t, n in ((embed, "embed"), (final_norm, "final_norm")):
        _dev(t, n, (torch.bfloat16,))
    lm, V, _ = _lm_arg(lm_head, torch.bfloat16, Hq * d)
    hid = Hq * d
    shapes = {"wqkv": ((Hq + 2 * Hkv) * d, hid, False), "wo": (hid, hid, False),
              "w_gate_up": (inter, hid, True), "w_down": (hid, inter, False)}
    arr = (_Layer * max(len(layers), 1))()
    for i, L in enumerate(layers):
        for f in LAYER_FIELDS:
            t = _packed(L[f], f, *shapes[f]) if f in shapes else _dev(L[f], f, (torch.bfloat16,))
            setattr(arr[i], f, t.data_ptr())
    B = cu_len.numel() - 1
    R = 1 + W * D
    dev = cand.device
    _shape(cand, "cand", (B, W, D))
    _shape(cand_len, "cand_len", (B, W))
    _shape(copy_gate, "copy_gate", (B,))
    _shape(final_norm, "final_norm", (hid,))
    if embed.dim() != 2 or embed.shape[1] != hid:
        raise SwitchSDError(f"embed must be [vocab, {hid}], got {list(embed.shape)}")
    for i, L in enumerate(layers):
        for f in ("attn_norm", "mlp_norm"):
            _shape(L[f], f"layers[{i}][{f!r}]", (hid,))
        for f in ("k_cache", "v_cache"):
            if L[f].dim() != 3 or tuple(L[f].shape[1:]) != (Hkv, d):
                raise SwitchSDError(f"layers[{i}][{f!r}] must be [N, {Hkv}, {d}]")
    _same_device(dev, (ids, "ids"), (cu_len, "cu_len"), (cand_len, "cand_len"),
                 (copy_gate, "copy_gate"), (embed, "embed"), (final_norm, "final_norm"))
    ts = _torch_stream(stream, dev)
    if argmax_out is None:
        argmax_out = _alloc(ts, (B, R), torch.int32, dev)
    _out(argmax_out, "argmax_out", torch.int32, (B, R), dev)
    if x_out is not None:
        _out(x_out, "x_out", torch.float32, (B, R, hid), dev)
    need = verify_forward_workspace_bytes(B, max_n, W, D, Hq, Hkv, d, inter, V)
    workspace = _workspace(workspace, need, ts, dev)
    ev0, ev1 = _events(events)
    _check(load().ssd_verify_forward(
        _ptr(ids), _ptr(cu_len), int(max_n), _ptr(cand), _ptr(cand_len), _ptr(copy_gate),
        _ptr(embed), ctypes.cast(arr, ctypes.c_void_p), len(layers), _ptr(final_norm),
        _ptr(lm), B, W, D, Hq, Hkv, d, inter, V, float(rope_base), float(eps),
        _ptr(argmax_out), _ptr(x_out), _ptr(workspace), workspace.numel(), ev0, ev1,
        _torch_stream_handle(ts)), "verify_forward")
    return argmax_out, x_out
