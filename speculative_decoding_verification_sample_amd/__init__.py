"""Speculative-decoding verify-and-resample on MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libspecverify.so`` (declared in
``include/spec_verify.h``).  Every step of the verification runs in the HIP
kernels; this module only checks tensor shapes / dtypes / devices, allocates
outputs and workspace with PyTorch, and passes device pointers and the
current HIP stream.  If the library has not been built the calls raise: there
is no fallback implementation.

Entry points (same names as the C ABI, minus the ``spec_`` prefix):
``verify_greedy``, ``verify_sample``, ``verify_sample_noalloc``, ``verify_mixed``,
``verify_tree``, ``tree_merge``,
``kv_commit``,
``verify_workspace_bytes``, ``status_string``, ``profile_begin``,
``profile_end``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_OP_GREEDY, SPEC_OP_SAMPLE, SPEC_OP_TREE = 0, 1, 2
SPEC_OK = 0
SPEC_SCRATCH_BYTES = 32 << 20  # the library-held workspace of spec_verify_sample_noalloc
ERRORS = {-1: "SPEC_ERR_NULL", -2: "SPEC_ERR_SHAPE", -3: "SPEC_ERR_PARAM",
          -4: "SPEC_ERR_WORKSPACE", -5: "SPEC_ERR_ALIGN", -6: "SPEC_ERR_HIP"}

EXPORTS = ("spec_verify_workspace_bytes", "spec_verify_greedy", "spec_verify_sample",
           "spec_verify_sample_noalloc", "spec_verify_mixed", "spec_verify_tree", "spec_tree_merge",
           "spec_lmhead_greedy", "spec_lmhead_workspace_bytes", "spec_kv_commit", "spec_status_string", "spec_profile_begin",
           "spec_profile_end")

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({status_string(code)})")


def load() -> ctypes.CDLL:
    """Load libspecverify.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.spec_verify_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.spec_verify_workspace_bytes.restype = Z
    L.spec_verify_greedy.argtypes = [P, I, P, I, I, I, P, P, P, Z, P]
    L.spec_verify_greedy.restype = I
    L.spec_verify_sample.argtypes = [P, P, I, P, P, P, F, F, I, I, I, P, P, P, P, P, P, Z, P]
    L.spec_verify_sample.restype = I
    L.spec_verify_sample_noalloc.argtypes = [P, P, I, P, P, P, F, F, I, I, I, P, P, P, P, P, P]
    L.spec_verify_sample_noalloc.restype = I
    L.spec_verify_mixed.argtypes = [P, P, I, P, P, P, P, P, I, I, I, P, P, P, P, P, P, Z, P]
    L.spec_verify_mixed.restype = I
    L.spec_verify_tree.argtypes = [P, I, P, P, P, I, I, I, P, P, P, P, Z, P]
    L.spec_verify_tree.restype = I
    L.spec_lmhead_workspace_bytes.argtypes = [I, I, I, I]
    L.spec_lmhead_workspace_bytes.restype = ctypes.c_size_t
    L.spec_lmhead_greedy.argtypes = [P, P, P, I, I, I, I, P, P, P, P, ctypes.c_size_t, P]
    L.spec_lmhead_greedy.restype = I
    L.spec_tree_merge.argtypes = [P, P, P, I, P, P, P, I, I, P, P, P, P, P, P]
    L.spec_tree_merge.restype = I
    L.spec_kv_commit.argtypes = [P, P, I, I, I, I, I, I, P, P, P, I, P, P]
    L.spec_kv_commit.restype = I
    L.spec_status_string.argtypes = [I]
    L.spec_status_string.restype = ctypes.c_char_p
    L.spec_profile_begin.argtypes = [I]
    L.spec_profile_begin.restype = I
    L.spec_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    L.spec_profile_end.restype = I
    _lib = L
    return L


def status_string(code: int) -> str:
    return load().spec_status_string(int(code)).decode()


def verify_workspace_bytes(op: int, B: int, K_or_N: int, V: int, dtype: int,
                           use_top_p: bool = False) -> int:
    return int(load().spec_verify_workspace_bytes(op, B, K_or_N, V, dtype, int(bool(use_top_p))))


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _logit_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SPEC_BF16  # raw bf16 bit patterns are accepted as int16 / uint16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    # +256 so the pointer can be rounded up to 256 B
    return torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws) -> int:
    p = ws.data_ptr()
    return (p + 255) // 256 * 256


def _ws_avail(ws) -> int:
    return ws.numel() * ws.element_size() - (_ws_ptr(ws) - ws.data_ptr())


def verify_greedy(target, draft_tokens, *, workspace=None, stream=None,
                  out=None) -> Dict[str, object]:
    """Greedy verify.  target [B, K+1, V] fp32/bf16 (cuda), draft_tokens [B, K] int32.
    Returns dict(accepted [B], tokens [B, K+1]) of int32 device tensors."""
    torch = _torch()
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", (B, K1, V), device=dev)
    _check(draft_tokens, "draft_tokens", (B, K), torch.int32, dev)
    dt = _logit_dtype(target)
    ws = _workspace(verify_workspace_bytes(SPEC_OP_GREEDY, B, K, V, dt), dev, workspace)
    out = out if out is not None else dict(
        accepted=torch.empty(B, dtype=torch.int32, device=dev),
        tokens=torch.empty((B, K1), dtype=torch.int32, device=dev))
    _check(out["accepted"], "out accepted", (B,), torch.int32, dev)
    _check(out["tokens"], "out tokens", (B, K1), torch.int32, dev)
    rc = load().spec_verify_greedy(_ptr(target), dt, _ptr(draft_tokens), B, K, V,
                                   _ptr(out["accepted"]), _ptr(out["tokens"]),
                                   _ws_ptr(ws), _ws_avail(ws), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_verify_greedy")
    return out


def verify_sample(target, draft, draft_tokens, u_accept, u_sample, temperature: float,
                  top_p: float = 1.0, *, diagnostics: bool = True, workspace=None,
                  stream=None, out=None) -> Dict[str, object]:
    """Sampling verify.  target [B, K+1, V], draft [B, K, V] (same dtype),
    draft_tokens [B, K] int32, u_accept [B, K] and u_sample [B] float32.
    Returns dict(accepted, tokens[, p, q, residual_mass])."""
    torch = _torch()
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", (B, K1, V), device=dev)
    _check(draft, "draft", (B, K, V), target.dtype, dev)
    _check(draft_tokens, "draft_tokens", (B, K), torch.int32, dev)
    _check(u_accept, "u_accept", (B, K), torch.float32, dev)
    _check(u_sample, "u_sample", (B,), torch.float32, dev)
    dt = _logit_dtype(target)
    ws = _workspace(verify_workspace_bytes(SPEC_OP_SAMPLE, B, K, V, dt, top_p < 1.0), dev,
                    workspace)
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   tokens=torch.empty((B, K1), dtype=torch.int32, device=dev))
        if diagnostics:
            out["p"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            out["q"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            out["residual_mass"] = torch.empty(B, dtype=torch.float32, device=dev)
    _check(out["accepted"], "out accepted", (B,), torch.int32, dev)
    _check(out["tokens"], "out tokens", (B, K1), torch.int32, dev)
    for name, shape in (("p", (B, K)), ("q", (B, K)), ("residual_mass", (B,))):
        if out.get(name) is not None:
            _check(out[name], f"out {name}", shape, torch.float32, dev)
    rc = load().spec_verify_sample(
        _ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample),
        float(temperature), float(top_p), B, K, V, _ptr(out["accepted"]), _ptr(out["tokens"]),
        _ptr(out.get("p")), _ptr(out.get("q")), _ptr(out.get("residual_mass")),
        _ws_ptr(ws), _ws_avail(ws), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_verify_sample")
    return out


def verify_sample_noalloc(target, draft, draft_tokens, u_accept, u_sample, temperature: float,
                          top_p: float = 1.0, *, out, stream=None) -> Dict[str, object]:
    """verify_sample on the library's own workspace (spec_verify_sample_noalloc):
    nothing is allocated, by the library or here; `out` holds the caller's
    output tensors (accepted, tokens and optionally p, q, residual_mass)."""
    torch = _torch()
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", (B, K1, V), device=dev)
    _check(draft, "draft", (B, K, V), target.dtype, dev)
    _check(draft_tokens, "draft_tokens", (B, K), torch.int32, dev)
    _check(u_accept, "u_accept", (B, K), torch.float32, dev)
    _check(u_sample, "u_sample", (B,), torch.float32, dev)
    _check(out["accepted"], "out accepted", (B,), torch.int32, dev)
    _check(out["tokens"], "out tokens", (B, K1), torch.int32, dev)
    for name, shape in (("p", (B, K)), ("q", (B, K)), ("residual_mass", (B,))):
        if out.get(name) is not None:
            _check(out[name], f"out {name}", shape, torch.float32, dev)
    rc = load().spec_verify_sample_noalloc(
        _ptr(target), _ptr(draft), _logit_dtype(target), _ptr(draft_tokens), _ptr(u_accept),
        _ptr(u_sample), float(temperature), float(top_p), B, K, V, _ptr(out["accepted"]),
        _ptr(out["tokens"]), _ptr(out.get("p")), _ptr(out.get("q")),
        _ptr(out.get("residual_mass")), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_verify_sample_noalloc")
    return out


def verify_mixed(target, draft, draft_tokens, u_accept, u_sample, temperature, top_p=None, *,
                 diagnostics: bool = True, workspace=None, stream=None,
                 out=None) -> Dict[str, object]:
    """Per-request temperature [B] (0 = greedy) and top_p [B] (or None),
    float32 device tensors; otherwise as verify_sample."""
    torch = _torch()
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", (B, K1, V), device=dev)
    _check(draft, "draft", (B, K, V), target.dtype, dev)
    _check(draft_tokens, "draft_tokens", (B, K), torch.int32, dev)
    _check(u_accept, "u_accept", (B, K), torch.float32, dev)
    _check(u_sample, "u_sample", (B,), torch.float32, dev)
    _check(temperature, "temperature", (B,), torch.float32, dev)
    if top_p is not None:
        _check(top_p, "top_p", (B,), torch.float32, dev)
    dt = _logit_dtype(target)
    ws = _workspace(verify_workspace_bytes(SPEC_OP_SAMPLE, B, K, V, dt, top_p is not None), dev,
                    workspace)
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   tokens=torch.empty((B, K1), dtype=torch.int32, device=dev))
        if diagnostics:
            out["p"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            out["q"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            out["residual_mass"] = torch.empty(B, dtype=torch.float32, device=dev)
    _check(out["accepted"], "out accepted", (B,), torch.int32, dev)
    _check(out["tokens"], "out tokens", (B, K1), torch.int32, dev)
    rc = load().spec_verify_mixed(
        _ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample),
        _ptr(temperature), _ptr(top_p), B, K, V, _ptr(out["accepted"]), _ptr(out["tokens"]),
        _ptr(out.get("p")), _ptr(out.get("q")), _ptr(out.get("residual_mass")),
        _ws_ptr(ws), _ws_avail(ws), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_verify_mixed")
    return out


def verify_tree(target, parents, node_tokens, anc_mask, *, workspace=None,
                stream=None, out=None) -> Dict[str, object]:
    """Greedy merged-tree verify.  target [B, N, V], parents / node_tokens
    [B, N] int32, anc_mask [B, N, N] uint8.
    Returns dict(path_len [B], path_nodes [B, N], tokens [B, N])."""
    torch = _torch()
    B, N, V = target.shape
    dev = target.device
    _check(target, "target", (B, N, V), device=dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    _check(node_tokens, "node_tokens", (B, N), torch.int32, dev)
    _check(anc_mask, "anc_mask", (B, N, N), torch.uint8, dev)
    dt = _logit_dtype(target)
    ws = _workspace(verify_workspace_bytes(SPEC_OP_TREE, B, N, V, dt), dev, workspace)
    out = out if out is not None else dict(
        path_len=torch.empty(B, dtype=torch.int32, device=dev),
        path_nodes=torch.empty((B, N), dtype=torch.int32, device=dev),
        tokens=torch.empty((B, N), dtype=torch.int32, device=dev))
    _check(out["path_len"], "out path_len", (B,), torch.int32, dev)
    _check(out["path_nodes"], "out path_nodes", (B, N), torch.int32, dev)
    _check(out["tokens"], "out tokens", (B, N), torch.int32, dev)
    rc = load().spec_verify_tree(_ptr(target), dt, _ptr(parents), _ptr(node_tokens),
                                 _ptr(anc_mask), B, N, V, _ptr(out["path_len"]),
                                 _ptr(out["path_nodes"]), _ptr(out["tokens"]),
                                 _ws_ptr(ws), _ws_avail(ws), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_verify_tree")
    return out


def lmhead_greedy(hidden, weight, tokens, *, argmax: bool = False, workspace=None,
                  stream=None, out=None) -> Dict[str, object]:
    """Greedy verification with the target's LM head fused in front: hidden
    [B, K+1, d] and weight [V, d] bf16 (torch.bfloat16 or int16 bit
    patterns), tokens [B, K] int32.  Returns dict(accepted [B], tokens
    [B, K+1], argmax [B, K+1] if asked)."""
    torch = _torch()
    B, K1, d = hidden.shape
    K = K1 - 1
    V = weight.shape[0]
    dev = hidden.device
    for t, name, shape in ((hidden, "hidden", (B, K1, d)), (weight, "weight", (V, d))):
        if tuple(t.shape) != shape or t.dtype not in (torch.bfloat16, torch.int16) or t.device != dev:
            raise ValueError(f"{name}: expected bf16 {shape} on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
    _check(tokens, "tokens", (B, K), torch.int32, dev)
    L = load()
    need = L.spec_lmhead_workspace_bytes(B, K, d, V)
    if need == 0:
        raise SpecVerifyError(-2, "spec_lmhead_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr()
    ws_off = (-ws_ptr) % 256
    out = out if out is not None else dict(
        accepted=torch.empty(B, dtype=torch.int32, device=dev),
        tokens=torch.empty((B, K1), dtype=torch.int32, device=dev))
    if argmax and "argmax" not in out:
        out["argmax"] = torch.empty((B, K1), dtype=torch.int32, device=dev)
    rc = L.spec_lmhead_greedy(_ptr(hidden), _ptr(weight), _ptr(tokens), B, K, d, V,
                              _ptr(out["accepted"]), _ptr(out["tokens"]), _ptr(out.get("argmax")),
                              ctypes.c_void_p(ws_ptr + ws_off), workspace.numel() - ws_off,
                              _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_lmhead_greedy")
    return out


def tree_merge(parents1, tokens1, conf1, parents2, tokens2, conf2, *, stream=None,
               out=None) -> Dict[str, object]:
    """Merge two trees per request ([B, n_t + 1] int32 parents / tokens,
    float32 conf) under one root.  Returns dict(parents [B, N], tokens
    [B, N], mask [B, N, N] uint8, conf [B, 2], route [B])."""
    torch = _torch()
    B, n1p = parents1.shape
    n2p = parents2.shape[1]
    dev = parents1.device
    for t, name, shape, dt in ((parents1, "parents1", (B, n1p), torch.int32),
                               (tokens1, "tokens1", (B, n1p), torch.int32),
                               (conf1, "conf1", (B, n1p), torch.float32),
                               (parents2, "parents2", (B, n2p), torch.int32),
                               (tokens2, "tokens2", (B, n2p), torch.int32),
                               (conf2, "conf2", (B, n2p), torch.float32)):
        _check(t, name, shape, dt, dev)
    N = n1p + n2p - 1
    out = out if out is not None else dict(
        parents=torch.empty((B, N), dtype=torch.int32, device=dev),
        tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
        mask=torch.empty((B, N, N), dtype=torch.uint8, device=dev),
        conf=torch.empty((B, 2), dtype=torch.float32, device=dev),
        route=torch.empty(B, dtype=torch.int32, device=dev))
    rc = load().spec_tree_merge(_ptr(parents1), _ptr(tokens1), _ptr(conf1), n1p - 1,
                                _ptr(parents2), _ptr(tokens2), _ptr(conf2), n2p - 1, B,
                                _ptr(out["parents"]), _ptr(out["tokens"]), _ptr(out["mask"]),
                                _ptr(out.get("conf")), _ptr(out.get("route")),
                                _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_tree_merge")
    return out


def kv_commit(kv, cache_len, path_len, path_nodes=None, *, N: Optional[int] = None,
              mirror=None, stream=None, out=None):
    """KV-cache commit after a cycle.  kv [L, 2, B, H, S, D] (any dtype; only
    bytes move), cache_len / path_len [B] int32, path_nodes [B, N] int32 or
    None (linear draft: give N).  Updates kv (and mirror) in place on the
    stream; returns new_len [B] int32."""
    torch = _torch()
    if kv.dim() != 6 or kv.shape[1] != 2:
        raise ValueError(f"kv must be [L, 2, B, H, S, D], got {tuple(kv.shape)}")
    L, _, B, H, S, D = kv.shape
    dev = kv.device
    _check(kv, "kv", kv.shape, device=dev)
    _check(cache_len, "cache_len", (B,), torch.int32, dev)
    _check(path_len, "path_len", (B,), torch.int32, dev)
    if path_nodes is not None:
        N = path_nodes.shape[1]
        _check(path_nodes, "path_nodes", (B, N), torch.int32, dev)
    if N is None:
        raise ValueError("N is required for a linear draft (path_nodes=None)")
    if mirror is not None:
        _check(mirror, "mirror", kv.shape, kv.dtype, dev)
    new_len = out if out is not None else torch.empty(B, dtype=torch.int32, device=dev)
    _check(new_len, "out new_len", (B,), torch.int32, dev)
    rc = load().spec_kv_commit(_ptr(kv), _ptr(mirror), kv.element_size(), L, B, H, S, D,
                               _ptr(cache_len), _ptr(path_len), _ptr(path_nodes), int(N),
                               _ptr(new_len), _stream(dev, stream))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_kv_commit")
    return new_len


def profile_begin(max_launches: int) -> None:
    rc = load().spec_profile_begin(int(max_launches))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_profile_begin")


def profile_end():
    """Returns (total milliseconds, launches) of the streaming kernel."""
    ms = ctypes.c_double()
    n = ctypes.c_int()
    rc = load().spec_profile_end(ctypes.byref(ms), ctypes.byref(n))
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, "spec_profile_end")
    return ms.value, n.value
