"""CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may load it; the product path never does.
It shares no code with the GPU library (``rejection_sampling_verify_amd``) and
neither imports the other.

``sv_oracle.c`` holds the fp64 plain-loop implementation (compiled with gcc,
loaded with ctypes); ``brute.py`` holds an exact-rational enumeration used to
pin it; ``trees.py`` holds the tree-structure helpers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsv_oracle.so")
SRC_PATH = os.path.join(HERE, "sv_oracle.c")

DTYPE_F32 = 0
DTYPE_BF16 = 1
SEQ_BAD_TOKEN = -1
SEQ_BAD_TEMPERATURE = -2
SEQ_BAD_TREE = -3
SEQ_BAD_LOGITS = -5
FLAG_KNIFE_EDGE = 1
FLAG_FALLBACK = 2
KNIFE_EDGE = 1e-5

_lib = None


def build(force: bool = True) -> str:
    """Compile sv_oracle.c into libsv_oracle.so with gcc (-O2, OpenMP, IEEE math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True, cwd=HERE)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        L.or_philox4x32_10.argtypes = [P, P, P]
        L.or_philox4x32_10.restype = None
        L.or_accept_uniform.argtypes = [u64, u64, i32, i32]
        L.or_accept_uniform.restype = ctypes.c_double
        L.or_gumbel.argtypes = [u64, u64, i32, i32, i32]
        L.or_gumbel.restype = ctypes.c_double
        L.or_verify_sample.argtypes = [P, i64, P, i64, ctypes.c_int, P, P, i32, i32, i32, u64, u64,
                                       P, P, P, P, ctypes.c_int]
        L.or_verify_sample.restype = ctypes.c_int
        L.or_verify_greedy.argtypes = [P, i64, ctypes.c_int, P, i32, i32, i32, P, P, ctypes.c_int]
        L.or_verify_greedy.restype = ctypes.c_int
        L.or_tree_is_valid.argtypes = [P, P, i32, i32]
        L.or_tree_is_valid.restype = ctypes.c_int
        L.or_verify_tree.argtypes = [P, i64, ctypes.c_int, P, P, P, i32, i32, i32, i32, P, P, P, P,
                                     ctypes.c_int]
        L.or_verify_tree.restype = ctypes.c_int
        L.or_verify_tree_sample.argtypes = [P, i64, P, i64, ctypes.c_int, P, P, P, P, i32, i32, i32, i32,
                                            u64, u64, i32, P, P, P, P, P, P, P, ctypes.c_int]
        L.or_verify_tree_sample.restype = ctypes.c_int
        L.or_tree_depths.argtypes = [P, i32, P]
        L.or_tree_depths.restype = ctypes.c_int
        _lib = L
    return _lib


class _Diag(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("accept_prob", "uniforms", "logz_target", "logz_draft", "residual_mass",
                 "top_gap", "top_score", "flags")]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits_dtype(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bit patterns), got %s" % a.dtype)


def _rows(a: np.ndarray, rows_per_seq: int, V: int | None):
    """Check a [B, rows, Vs] C-contiguous logits array; return (V, row stride)."""
    if a.ndim != 3 or a.shape[1] != rows_per_seq or not a.flags.c_contiguous:
        raise ValueError("logits must be C-contiguous [B, %d, V_stride], got %s" % (rows_per_seq, a.shape))
    stride = a.shape[2]
    V = stride if V is None else V
    if V > stride:
        raise ValueError("V larger than the row stride")
    return V, stride


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def accept_uniform(seed: int, offset: int, b: int, i: int) -> float:
    return lib().or_accept_uniform(seed, offset, b, i)


def gumbel(seed: int, offset: int, b: int, pos: int, v: int) -> float:
    return lib().or_gumbel(seed, offset, b, pos, v)


def verify_sample(target, draft, draft_ids, temperature, seed=0, offset=0, V=None,
                  u_override=None, nthreads=None) -> dict:
    """Sampled (T>0) / greedy (T=0) chain verification of every sequence.

    target: [B, gamma+1, Vs] float32 or uint16 (bf16 bits); draft: [B, gamma, Vs]
    of the same dtype or None (one-hot draft); draft_ids: [B, gamma] int32;
    temperature: [B] float32. Returns tokens [B, gamma+1], n [B] and fp64
    diagnostics.
    """
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32)
    B, gamma = ids.shape
    V, tstride = _rows(target, gamma + 1, V)
    dt = _logits_dtype(target)
    dstride = 0
    if draft is not None:
        Vd, dstride = _rows(draft, gamma, V)
        if draft.dtype != target.dtype or draft.shape[0] != B:
            raise ValueError("draft must match target in dtype and batch")
    temp = np.ascontiguousarray(temperature, dtype=np.float32)
    assert temp.shape == (B,)
    u = None if u_override is None else np.ascontiguousarray(u_override, dtype=np.float64)
    out = {
        "tokens": np.zeros((B, gamma + 1), np.int32),
        "n": np.zeros(B, np.int32),
        "accept_prob": np.zeros((B, gamma)),
        "uniforms": np.zeros((B, gamma)),
        "logz_target": np.zeros((B, gamma)),
        "logz_draft": np.zeros((B, gamma)),
        "residual_mass": np.zeros(B),
        "top_gap": np.zeros(B),
        "top_score": np.zeros(B),
        "flags": np.zeros(B, np.int32),
    }
    d = _Diag(*[out[k].ctypes.data for k in ("accept_prob", "uniforms", "logz_target", "logz_draft",
                                            "residual_mass", "top_gap", "top_score", "flags")])
    nt = nthreads or os.cpu_count() or 1
    rc = lib().or_verify_sample(_ptr(target), tstride, _ptr(draft), dstride, dt, _ptr(ids),
                                _ptr(temp), B, gamma, V, seed, offset, _ptr(u),
                                _ptr(out["tokens"]), _ptr(out["n"]), ctypes.byref(d), nt)
    if rc != 0:
        raise ValueError("or_verify_sample rejected its arguments (code %d)" % rc)
    return out


def verify_greedy(target, draft_ids, V=None, nthreads=None) -> dict:
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32)
    B, gamma = ids.shape
    V, tstride = _rows(target, gamma + 1, V)
    out = {"tokens": np.zeros((B, gamma + 1), np.int32), "n": np.zeros(B, np.int32)}
    nt = nthreads or os.cpu_count() or 1
    rc = lib().or_verify_greedy(_ptr(target), tstride, _logits_dtype(target), _ptr(ids), B, gamma, V,
                                _ptr(out["tokens"]), _ptr(out["n"]), nt)
    if rc != 0:
        raise ValueError("or_verify_greedy rejected its arguments (code %d)" % rc)
    return out


def verify_tree(target, parents, depth, node_tokens, max_depth, V=None, nthreads=None) -> dict:
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32)
    B, N = tok.shape
    V, tstride = _rows(target, N, V)
    par = np.ascontiguousarray(parents, dtype=np.int32)
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    assert par.shape == (N,) and dep.shape == (N,)
    out = {"path": np.zeros((B, max_depth + 1), np.int32), "path_len": np.zeros(B, np.int32),
           "bonus": np.zeros(B, np.int32), "first_match_node": np.zeros(B, np.int32)}
    nt = nthreads or os.cpu_count() or 1
    rc = lib().or_verify_tree(_ptr(target), tstride, _logits_dtype(target), _ptr(par), _ptr(dep),
                              _ptr(tok), B, N, V, max_depth, _ptr(out["path"]), _ptr(out["path_len"]),
                              _ptr(out["bonus"]), _ptr(out["first_match_node"]), nt)
    if rc != 0:
        raise ValueError("or_verify_tree rejected its arguments (code %d)" % rc)
    return out


def verify_tree_sample(target, draft, parents, depth, node_tokens, temperature, max_depth, seed=0, offset=0,
                       V=None, nthreads=None, without_replacement=False) -> dict:
    """Sampled tree verification by multi-round rejection sampling ([SB] "Tree
    Attention"). target and draft are [B, N, Vs] (draft row v: q at node v,
    from which v's children were drawn). Returns path [B, max_depth + 1],
    path_len [B] (nodes on the path, or a negative code), token [B] (the bonus
    or replacement token after the path), top_gap, flags, rejections and
    margin (the smallest |u - a| over the siblings tested) [B].
    without_replacement: siblings were drawn without replacement, so each
    round's q is q over the tokens not drawn yet, renormalized (the page's
    variant); siblings must then carry distinct tokens (else code -1)."""
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32)
    B, N = tok.shape
    V, tstride = _rows(target, N, V)
    _, dstride = _rows(draft, N, V)
    if _logits_dtype(draft) != _logits_dtype(target):
        raise TypeError("target and draft logits must have the same dtype")
    par = np.ascontiguousarray(parents, dtype=np.int32)
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    temp = np.ascontiguousarray(temperature, dtype=np.float32)
    assert par.shape == (N,) and dep.shape == (N,) and temp.shape == (B,)
    out = {"path": np.zeros((B, max_depth + 1), np.int32), "path_len": np.zeros(B, np.int32),
           "token": np.zeros(B, np.int32), "top_gap": np.zeros(B, np.float64),
           "flags": np.zeros(B, np.int32), "rejections": np.zeros(B, np.int32),
           "margin": np.zeros(B, np.float64)}
    nt = nthreads or os.cpu_count() or 1
    rc = lib().or_verify_tree_sample(_ptr(target), tstride, _ptr(draft), dstride, _logits_dtype(target),
                                     _ptr(par), _ptr(dep), _ptr(tok), _ptr(temp), B, N, V, max_depth,
                                     seed, offset, int(bool(without_replacement)), _ptr(out["path"]),
                                     _ptr(out["path_len"]), _ptr(out["token"]),
                                     _ptr(out["top_gap"]), _ptr(out["flags"]), _ptr(out["rejections"]),
                                     _ptr(out["margin"]), nt)
    if rc != 0:
        raise ValueError("or_verify_tree_sample rejected its arguments (code %d)" % rc)
    return out


def tree_is_valid(parents, depth, max_depth) -> bool:
    par = np.ascontiguousarray(parents, dtype=np.int32)
    dep = np.ascontiguousarray(depth, dtype=np.int32)
    return bool(lib().or_tree_is_valid(_ptr(par), _ptr(dep), len(par), max_depth))


def tree_depths(parents) -> np.ndarray:
    par = np.ascontiguousarray(parents, dtype=np.int32)
    out = np.zeros(len(par), np.int32)
    if not lib().or_tree_depths(_ptr(par), len(par), _ptr(out)):
        raise ValueError("malformed parent array")
    return out
