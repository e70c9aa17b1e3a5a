"""ctypes wrapper around the fp64 CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The GPU library never imports or links it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
FLAG_ACCEPT_NEAR, FLAG_CDF_NEAR, FLAG_TOPP_NEAR, FLAG_FALLBACK, FLAG_TOKEN_RANGE = 1, 2, 4, 8, 16
FLAG_TOPP_EDGE, FLAG_S_NEAR = 32, 64
FLAG_AMBIGUOUS = FLAG_ACCEPT_NEAR | FLAG_CDF_NEAR | FLAG_TOPP_NEAR | FLAG_S_NEAR
S_RESOLUTION = 2.0 ** -20  # residual mass taken as empty (draw from p')

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with plain gcc: -O2, no fast-math, no OpenMP."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-fPIC",
                               "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L.oracle_verify_sample.argtypes = [P, P, I, P, P, P, D, D, I, I, I, P, P, P, P, P, P, P,
                                           P, P, P, P, P]
        L.oracle_verify_sample.restype = I
        L.oracle_verify_greedy.argtypes = [P, I, P, I, I, I, P, P, P]
        L.oracle_verify_greedy.restype = I
        L.oracle_verify_tree.argtypes = [P, I, P, P, P, I, I, I, P, P, P, P, P]
        L.oracle_verify_tree.restype = I
        L.oracle_row_distribution.argtypes = [P, I, I, D, D, P, P]
        L.oracle_row_distribution.restype = I
        L.oracle_tree_is_valid.argtypes = [P, P, I]
        L.oracle_tree_is_valid.restype = I
        L.oracle_kv_commit.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, I, P]
        L.oracle_kv_commit.restype = I
        L.oracle_tree_merge.argtypes = [P, P, P, I, P, P, P, I, I, P, P, P, P, P]
        L.oracle_tree_merge.restype = I
        L.oracle_lmhead_logits.argtypes = [P, P, I, I, I, P, P]
        L.oracle_lmhead_logits.restype = I
        L.oracle_lmhead_greedy.argtypes = [P, P, P, I, I, I, I, P, P, P]
        L.oracle_lmhead_greedy.restype = I
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {arr.dtype}")


def row_distribution(logits: np.ndarray, temperature: float, top_p: float = 1.0):
    """One row's tempered (and nucleus-filtered) distribution, fp64.
    Returns (prob[V], info dict)."""
    logits = np.ascontiguousarray(logits)
    V = logits.shape[-1]
    prob = np.empty(V, np.float64)
    info = np.empty(7, np.float64)
    rc = lib().oracle_row_distribution(_p(logits), _dtype_code(logits), V,
                                       float(temperature), float(top_p), _p(prob), _p(info))
    if rc != 0:
        raise ValueError(f"oracle_row_distribution: {rc}")
    return prob, dict(max=info[0], Z=info[1], kept=info[2], tau=info[3],
                      before=info[4], after=info[5], cut_group=int(info[6]))


def verify_sample(target, draft, tokens, u_accept, u_sample, temperature, top_p=1.0,
                  row_info=False):
    """Sampling verify (oracle.c, oracle_verify_sample).  Besides the
    outputs it returns, per request, the variants with one row's nucleus cut
    moved by one tie group where that row's cumulative mass before or after
    its cut group lies within 1e-6 of top_p: `alt_n`, `alt_token`, `alt_S`
    [B, 2K+1, 2] (alt_n -1: no variant) and `alt_p`, `alt_q` [B, 2K+1, 2, K];
    alternative [row, 0] moves the cut one group earlier, [row, 1] later."""
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    if draft.dtype != target.dtype:
        raise TypeError("target and draft dtypes differ")
    B, K1, V = target.shape
    K = K1 - 1
    assert draft.shape == (B, K, V)
    tokens = np.ascontiguousarray(tokens, np.int32)
    ua = np.ascontiguousarray(u_accept, np.float32)
    us = np.ascontiguousarray(u_sample, np.float32)
    assert tokens.shape == (B, K) and ua.shape == (B, K) and us.shape == (B,)
    out = dict(accepted=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               p=np.empty((B, K), np.float64), q=np.empty((B, K), np.float64),
               S=np.empty(B, np.float64), flags=np.empty(B, np.int32),
               alt_n=np.empty((B, 2 * K + 1, 2), np.int32),
               alt_token=np.empty((B, 2 * K + 1, 2), np.int32),
               alt_S=np.empty((B, 2 * K + 1, 2), np.float64),
               alt_p=np.zeros((B, 2 * K + 1, 2, K), np.float64),
               alt_q=np.zeros((B, 2 * K + 1, 2, K), np.float64))
    info = np.empty((B, 2 * K + 1, 7), np.float64) if row_info else None
    rc = lib().oracle_verify_sample(
        _p(target), _p(draft), _dtype_code(target), _p(tokens), _p(ua), _p(us),
        float(temperature), float(top_p), B, K, V, _p(out["accepted"]), _p(out["tokens"]),
        _p(out["p"]), _p(out["q"]), _p(out["S"]), _p(out["flags"]), _p(info),
        _p(out["alt_n"]), _p(out["alt_token"]), _p(out["alt_S"]), _p(out["alt_p"]),
        _p(out["alt_q"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_sample: {rc}")
    if row_info:
        out["row_info"] = info
    return out


def verify_greedy(target, tokens):
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = np.ascontiguousarray(tokens, np.int32)
    assert tokens.shape == (B, K)
    out = dict(accepted=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               argmax=np.empty((B, K + 1), np.int32))
    rc = lib().oracle_verify_greedy(_p(target), _dtype_code(target), _p(tokens), B, K, V,
                                    _p(out["accepted"]), _p(out["tokens"]), _p(out["argmax"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy: {rc}")
    return out


def lmhead_logits(hidden, weight, absdot=False):
    """Logits of hidden-state rows against the vocabulary matrix (oracle.c,
    oracle_lmhead_logits): hidden [R, d], weight [V, d] as bf16 bit patterns
    (uint16).  Returns fp64 logits [R, V] (and sum |h w| [R, V] if asked)."""
    h = np.ascontiguousarray(hidden, np.uint16)
    w = np.ascontiguousarray(weight, np.uint16)
    R, d = h.shape
    V, d2 = w.shape
    assert d == d2
    logits = np.empty((R, V), np.float64)
    ad = np.empty((R, V), np.float64) if absdot else None
    rc = lib().oracle_lmhead_logits(_p(h), _p(w), R, d, V, _p(logits), _p(ad))
    if rc != 0:
        raise ValueError(f"oracle_lmhead_logits: {rc}")
    return (logits, ad) if absdot else logits


def lmhead_greedy(hidden, weight, tokens):
    """Greedy verification on logits computed from hidden states (oracle.c,
    oracle_lmhead_greedy): hidden [B, K+1, d], weight [V, d] bf16 bits."""
    h = np.ascontiguousarray(hidden, np.uint16)
    w = np.ascontiguousarray(weight, np.uint16)
    B, K1, d = h.shape
    K = K1 - 1
    V = w.shape[0]
    tokens = np.ascontiguousarray(tokens, np.int32)
    assert tokens.shape == (B, K) and w.shape == (V, d)
    out = dict(accepted=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               argmax=np.empty((B, K + 1), np.int32))
    rc = lib().oracle_lmhead_greedy(_p(h), _p(w), _p(tokens), B, K, d, V, _p(out["accepted"]),
                                    _p(out["tokens"]), _p(out["argmax"]))
    if rc != 0:
        raise ValueError(f"oracle_lmhead_greedy: {rc}")
    return out


def verify_tree(target, parents, node_tokens, anc_mask):
    target = np.ascontiguousarray(target)
    B, N, V = target.shape
    parents = np.ascontiguousarray(parents, np.int32)
    node_tokens = np.ascontiguousarray(node_tokens, np.int32)
    anc_mask = np.ascontiguousarray(anc_mask, np.uint8)
    assert parents.shape == (B, N) and node_tokens.shape == (B, N)
    assert anc_mask.shape == (B, N, N)
    out = dict(path_len=np.empty(B, np.int32), path_nodes=np.empty((B, N), np.int32),
               tokens=np.empty((B, N), np.int32), valid=np.empty(B, np.int32),
               argmax=np.empty((B, N), np.int32))
    rc = lib().oracle_verify_tree(_p(target), _dtype_code(target), _p(parents),
                                  _p(node_tokens), _p(anc_mask), B, N, V,
                                  _p(out["path_len"]), _p(out["path_nodes"]),
                                  _p(out["tokens"]), _p(out["valid"]), _p(out["argmax"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree: {rc}")
    return out


def tree_is_valid(parents, anc_mask) -> bool:
    parents = np.ascontiguousarray(parents, np.int32)
    anc_mask = np.ascontiguousarray(anc_mask, np.uint8)
    N = parents.shape[0]
    rc = lib().oracle_tree_is_valid(_p(parents), _p(anc_mask), N)
    if rc < 0:
        raise ValueError("oracle_tree_is_valid: bad arguments")
    return bool(rc)


def verify_mixed(target, draft, tokens, u_accept, u_sample, temperature, top_p=None):
    """Per-request parameters: each request is verified on its own with its
    own temperature (0: the greedy rule on its target rows) and top_p (the
    requests are independent).  A request with a temperature not finite or
    < 0, or a top_p outside (0, 1], is marked accepted = -3, tokens -1.
    Returns the verify_sample fields; p, q, S are 0 for greedy requests."""
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    temperature = np.asarray(temperature, np.float32)
    top_p = np.ones(B, np.float32) if top_p is None else np.asarray(top_p, np.float32)
    out = dict(accepted=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               p=np.zeros((B, K)), q=np.zeros((B, K)), S=np.zeros(B),
               flags=np.zeros(B, np.int32),
               alt_n=np.full((B, 2 * K + 1, 2), -1, np.int32),
               alt_token=np.full((B, 2 * K + 1, 2), -1, np.int32),
               alt_S=np.zeros((B, 2 * K + 1, 2)), alt_p=np.zeros((B, 2 * K + 1, 2, K)),
               alt_q=np.zeros((B, 2 * K + 1, 2, K)))
    for b in range(B):
        T, P = float(temperature[b]), float(top_p[b])
        if not (np.isfinite(T) and T >= 0.0) or not (0.0 < P <= 1.0):
            out["accepted"][b] = -3
            out["tokens"][b] = -1
            continue
        if T == 0.0:
            r = verify_greedy(target[b:b + 1], tokens[b:b + 1])
        else:
            r = verify_sample(target[b:b + 1], draft[b:b + 1], tokens[b:b + 1],
                              u_accept[b:b + 1], u_sample[b:b + 1], T, P)
            for key in ("p", "q", "S", "flags", "alt_n", "alt_token", "alt_S", "alt_p",
                        "alt_q"):
                out[key][b] = r[key][0]
        out["accepted"][b] = r["accepted"][0]
        out["tokens"][b] = r["tokens"][0]
    return out


def tree_merge(parents1, tokens1, conf1, parents2, tokens2, conf2):
    """Merge two trees per request under one root and route by mean
    confidence (oracle.c, oracle_tree_merge).  Inputs [B, n_t + 1]."""
    p1 = np.ascontiguousarray(parents1, np.int32)
    p2 = np.ascontiguousarray(parents2, np.int32)
    B, n1p = p1.shape
    n2p = p2.shape[1]
    t1 = np.ascontiguousarray(tokens1, np.int32)
    t2 = np.ascontiguousarray(tokens2, np.int32)
    c1 = np.ascontiguousarray(conf1, np.float32)
    c2 = np.ascontiguousarray(conf2, np.float32)
    N = n1p + n2p - 1
    out = dict(parents=np.empty((B, N), np.int32), tokens=np.empty((B, N), np.int32),
               mask=np.empty((B, N, N), np.uint8), conf=np.empty((B, 2), np.float64),
               route=np.empty(B, np.int32))
    rc = lib().oracle_tree_merge(_p(p1), _p(t1), _p(c1), n1p - 1, _p(p2), _p(t2), _p(c2),
                                 n2p - 1, B, _p(out["parents"]), _p(out["tokens"]),
                                 _p(out["mask"]), _p(out["conf"]), _p(out["route"]))
    if rc != 0:
        raise ValueError(f"oracle_tree_merge: {rc}")
    return out


def kv_commit(kv, cache_len, path_len, path_nodes=None, N=None, mirror=None):
    """KV-cache commit (oracle.c, oracle_kv_commit).  kv [L, 2, B, H, S, D]
    (any dtype: bytes are copied); path_nodes [B, N] int32 or None (linear:
    positions 1..d).  Returns (kv after, mirror after or None, new_len)."""
    kv = np.ascontiguousarray(kv)
    L, two, B, H, S, D = kv.shape
    assert two == 2
    cache_len = np.ascontiguousarray(cache_len, np.int32)
    path_len = np.ascontiguousarray(path_len, np.int32)
    if path_nodes is not None:
        path_nodes = np.ascontiguousarray(path_nodes, np.int32)
        N = path_nodes.shape[1]
        assert path_nodes.shape == (B, N)
    assert N is not None and cache_len.shape == (B,) and path_len.shape == (B,)
    out = kv.copy()
    mout = None
    if mirror is not None:
        mout = np.ascontiguousarray(mirror).copy()
        assert mout.shape == kv.shape and mout.dtype == kv.dtype
    new_len = np.empty(B, np.int32)
    rc = lib().oracle_kv_commit(_p(kv), _p(out), _p(mout), kv.dtype.itemsize, L, B, H, S, D,
                                _p(cache_len), _p(path_len), _p(path_nodes), int(N), _p(new_len))
    if rc != 0:
        raise ValueError(f"oracle_kv_commit: {rc}")
    return out, mout, new_len


def verify_workload(w):
    """Run the oracle on a workloads.Workload."""
    if w.kind == "sample":
        return verify_sample(w.target, w.draft, w.tokens, w.u_accept, w.u_sample,
                             w.temperature, w.top_p)
    if w.kind == "greedy":
        return verify_greedy(w.target, w.tokens)
    return verify_tree(w.target, w.parents, w.tokens, w.anc_mask)
