"""ctypes binding of librsv_hip.so (argument marshalling only).

Tensors are torch tensors on the GPU; their ``data_ptr()`` is handed to the C
ABI together with ``torch.cuda.current_stream().cuda_stream`` (the hipStream_t
of ROCm builds of torch). Every step of the verify path runs in the library's
kernels.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SV_LIB_PATH selects another build of the same library (for A/B timing).
LIB_PATH = os.environ.get("SV_LIB_PATH") or os.path.join(HERE, "librsv_hip.so")

SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_SEQ_BAD_TOKEN = -1
SV_SEQ_BAD_TEMPERATURE = -2
SV_SEQ_BAD_TREE = -3
SV_SEQ_INTERNAL = -4
SV_SEQ_BAD_LOGITS = -5
SV_ERR_SCRATCH_LIMIT = 7
SV_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ["sv_workspace_bytes", "sv_workspace_init", "sv_status_string", "spec_verify_sample",
           "spec_verify_greedy", "spec_verify_tree", "spec_verify_tree_sample", "sv_kv_rollback",
           "sv_kv_rollback_layers", "sv_ngram_draft", "sv_tree_mask", "sv_debug_philox", "sv_debug_noise",
           "sv_debug_wave_max", "sv_debug_read_stream", "sv_debug_sample_tiled", "spec_verify_sample_noalloc"]

_lib = None


class SVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, sv_status_string(status), status))


class _Diag(ctypes.Structure):
    _fields_ = [("accept_prob", ctypes.c_void_p), ("logz_target", ctypes.c_void_p),
                ("logz_draft", ctypes.c_void_p), ("residual_mass", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """Load librsv_hip.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librsv_hip.so is not built; run rejection_sampling_verify_amd.build.build() "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
        L.sv_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_workspace_bytes.restype = sz
        L.sv_workspace_init.argtypes = [P, sz, P]
        L.sv_workspace_init.restype = ctypes.c_int
        L.sv_status_string.argtypes = [ctypes.c_int]
        L.sv_status_string.restype = ctypes.c_char_p
        u32 = ctypes.c_uint32
        L.spec_verify_sample.argtypes = [P, i64, P, i64, ctypes.c_int, P, P, i32, i32, i32, u64, u64, u32, P, P,
                                         ctypes.POINTER(_Diag), P, sz, P]
        L.spec_verify_sample.restype = ctypes.c_int
        L.sv_debug_sample_tiled.argtypes = L.spec_verify_sample.argtypes + [i32, i32]
        L.sv_debug_sample_tiled.restype = ctypes.c_int
        L.spec_verify_sample_noalloc.argtypes = [P, i64, P, i64, ctypes.c_int, P, P, i32, i32, i32, u64, u64, u32,
                                                 P, P, ctypes.POINTER(_Diag), P]
        L.spec_verify_sample_noalloc.restype = ctypes.c_int
        L.spec_verify_greedy.argtypes = [P, i64, ctypes.c_int, P, i32, i32, i32, P, P, P, sz, P]
        L.spec_verify_greedy.restype = ctypes.c_int
        L.spec_verify_tree.argtypes = [P, i64, ctypes.c_int, P, P, P, i32, i32, i32, i32, P, P, P, P, sz, P]
        L.spec_verify_tree.restype = ctypes.c_int
        L.spec_verify_tree_sample.argtypes = [P, i64, P, i64, ctypes.c_int, P, P, P, P, i32, i32, i32, i32, u64, u64,
                                              u32, i32, P, P, P, P, sz, P]
        L.spec_verify_tree_sample.restype = ctypes.c_int
        L.sv_kv_rollback.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, P, i32, P, P, P]
        L.sv_kv_rollback.restype = ctypes.c_int
        L.sv_kv_rollback_layers.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, P, i32, P, P, P]
        L.sv_kv_rollback_layers.restype = ctypes.c_int
        L.sv_ngram_draft.argtypes = [P, i64, P, i32, i32, i32, i32, P, P, P, P]
        L.sv_ngram_draft.restype = ctypes.c_int
        L.sv_tree_mask.argtypes = [P, i64, i32, i32, P, P, P, P, P]
        L.sv_tree_mask.restype = ctypes.c_int
        L.sv_debug_philox.argtypes = [P, P, P, i32, P]
        L.sv_debug_philox.restype = ctypes.c_int
        L.sv_debug_noise.argtypes = [P, P, P, i32, P]
        L.sv_debug_noise.restype = ctypes.c_int
        L.sv_debug_wave_max.argtypes = [P, P, i32, P]
        L.sv_debug_wave_max.restype = ctypes.c_int
        L.sv_debug_read_stream.argtypes = [P, sz, P, i32, P]
        L.sv_debug_read_stream.restype = ctypes.c_int
        _lib = L
    return _lib


def exported_symbols() -> list[str]:
    L = lib()
    return [name for name in EXPORTS if hasattr(L, name)]


def sv_status_string(status: int) -> str:
    return lib().sv_status_string(int(status)).decode()


def sv_workspace_bytes(B: int, rows: int, V: int) -> int:
    return int(lib().sv_workspace_bytes(B, rows, V))


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocations made inside belong to `stream` (the caller's side stream, if
    any): torch fills them on it, and its caching allocator reuses their
    memory only after the work queued there, which includes the kernels that
    use them."""
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def sv_workspace_init(ws, stream=None) -> None:
    st = lib().sv_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if st != 0:
        raise SVError(st, "sv_workspace_init")


class Workspace:
    """Zeroed device workspace that grows to the largest call it has served."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, B: int, rows: int, V: int):
        import torch
        need = sv_workspace_bytes(B, rows, V)
        if need == 0:
            raise ValueError("shape out of range for the library")
        if self.buf is None or self.buf.numel() < need:
            # torch's caching allocator aligns blocks to at least 512 bytes.
            self.buf = torch.zeros(need, dtype=torch.uint8, device=self.device)
        return self.buf


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    raise TypeError("logits must be torch.bfloat16 or torch.float32, got %s" % t.dtype)


def _row_stride(t, rows: int, V: int) -> int:
    """Elements between consecutive rows of a [B, rows, >=V] view whose rows are
    evenly spaced (contiguous innermost dimension)."""
    if t.dim() != 3 or t.shape[1] != rows or t.stride(2) != 1:
        raise ValueError("logits must be [B, %d, V] with a contiguous last dimension" % rows)
    if t.shape[0] > 1 and t.stride(0) != rows * t.stride(1):
        raise ValueError("rows of consecutive sequences must be evenly spaced")
    return int(t.stride(1)) if rows > 1 or t.shape[0] == 1 else int(t.stride(0))


def _check_i32(t, shape, name):
    import torch
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("%s must be a contiguous int32 CUDA tensor of shape %s" % (name, tuple(shape)))


def spec_verify_sample(target_logits, draft_logits, draft_ids, temperature, seed: int = 0, offset: int = 0,
                       out_tokens=None, out_num_accepted=None, diag: dict | None = None, workspace=None,
                       V: int | None = None, stream=None, seq_base: int = 0, tiling: tuple | None = None):
    """Sampled (temperature > 0) / greedy (temperature == 0) verification.

    target_logits [B, gamma+1, V'] and draft_logits [B, gamma, V'] (or None for a
    one-hot draft) of bf16 or fp32 with V' >= V; draft_ids [B, gamma] int32;
    temperature [B] float32. Returns (out_tokens [B, gamma+1], out_num_accepted [B]).
    diag: optional dict of preallocated float32 tensors with keys accept_prob,
    logz_target, logz_draft ([B, gamma]) and residual_mass ([B]).
    seq_base: global index of the first sequence (Philox counter word 2).
    tiling: (p1_vectors, p2_chunks) to fix the tiling through the debug entry
    point sv_debug_sample_tiled (results must not depend on it).
    """
    import torch
    B, gamma = draft_ids.shape
    V = int(target_logits.shape[2]) if V is None else int(V)
    _check_i32(draft_ids, (B, gamma), "draft_ids")
    if temperature.dtype != torch.float32 or tuple(temperature.shape) != (B,) or not temperature.is_contiguous():
        raise ValueError("temperature must be a contiguous float32 tensor of shape [B]")
    ts = _row_stride(target_logits, gamma + 1, V)
    ds = 0
    if draft_logits is not None:
        if draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft and target logits must share a dtype")
        ds = _row_stride(draft_logits, gamma, V)
    with _on(stream):
        if out_tokens is None:
            out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=target_logits.device)
        if out_num_accepted is None:
            out_num_accepted = torch.empty((B,), dtype=torch.int32, device=target_logits.device)
        if workspace is None:
            workspace = Workspace(target_logits.device).get(B, gamma + 1, V)
    d = None
    if diag:
        d = _Diag(*[diag[k].data_ptr() if diag.get(k) is not None else None
                    for k in ("accept_prob", "logz_target", "logz_draft", "residual_mass")])
    args = (_ptr(target_logits), ts, _ptr(draft_logits), ds, _dtype_code(target_logits),
            _ptr(draft_ids), _ptr(temperature), B, gamma, V, seed, offset, seq_base,
            _ptr(out_tokens), _ptr(out_num_accepted), ctypes.byref(d) if d is not None else None,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if tiling is None:
        st = lib().spec_verify_sample(*args)
    else:
        st = lib().sv_debug_sample_tiled(*args, int(tiling[0]), int(tiling[1]))
    if st != 0:
        raise SVError(st, "spec_verify_sample")
    return out_tokens, out_num_accepted


def spec_verify_sample_noalloc(target_logits, draft_logits, draft_ids, temperature, out_tokens, out_num_accepted,
                               seed: int = 0, offset: int = 0, seq_base: int = 0, diag: dict | None = None,
                               V: int | None = None, stream=None):
    """spec_verify_sample through the allocation-free entry point: no workspace
    (the library's static scratch on this GPU), and outputs preallocated by
    the caller, so that the call allocates nothing."""
    B, gamma = draft_ids.shape
    V = int(target_logits.shape[2]) if V is None else int(V)
    _check_i32(draft_ids, (B, gamma), "draft_ids")
    _check_i32(out_tokens, (B, gamma + 1), "out_tokens")
    _check_i32(out_num_accepted, (B,), "out_num_accepted")
    ts = _row_stride(target_logits, gamma + 1, V)
    ds = 0 if draft_logits is None else _row_stride(draft_logits, gamma, V)
    d = None
    if diag:
        d = _Diag(*[diag[k].data_ptr() if diag.get(k) is not None else None
                    for k in ("accept_prob", "logz_target", "logz_draft", "residual_mass")])
    st = lib().spec_verify_sample_noalloc(_ptr(target_logits), ts, _ptr(draft_logits), ds,
                                          _dtype_code(target_logits), _ptr(draft_ids), _ptr(temperature), B, gamma,
                                          V, seed, offset, seq_base, _ptr(out_tokens), _ptr(out_num_accepted),
                                          ctypes.byref(d) if d is not None else None, _stream(stream))
    if st != 0:
        raise SVError(st, "spec_verify_sample_noalloc")
    return out_tokens, out_num_accepted


def spec_verify_greedy(target_logits, draft_ids, out_tokens=None, out_num_accepted=None, workspace=None,
                       V: int | None = None, stream=None):
    """Argmax-match verification; same outputs as spec_verify_sample."""
    import torch
    B, gamma = draft_ids.shape
    V = int(target_logits.shape[2]) if V is None else int(V)
    _check_i32(draft_ids, (B, gamma), "draft_ids")
    ts = _row_stride(target_logits, gamma + 1, V)
    with _on(stream):
        if out_tokens is None:
            out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=target_logits.device)
        if out_num_accepted is None:
            out_num_accepted = torch.empty((B,), dtype=torch.int32, device=target_logits.device)
        if workspace is None:
            workspace = Workspace(target_logits.device).get(B, gamma + 1, V)
    st = lib().spec_verify_greedy(_ptr(target_logits), ts, _dtype_code(target_logits), _ptr(draft_ids), B, gamma,
                                  V, _ptr(out_tokens), _ptr(out_num_accepted), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise SVError(st, "spec_verify_greedy")
    return out_tokens, out_num_accepted


def spec_verify_tree(target_logits, parents, depth, node_tokens, max_depth: int, out_path=None,
                     out_path_len=None, out_bonus=None, workspace=None, V: int | None = None, stream=None):
    """Greedy tree verification. Returns (out_path [B, max_depth+1], out_path_len [B], out_bonus [B])."""
    import torch
    B, N = node_tokens.shape
    V = int(target_logits.shape[2]) if V is None else int(V)
    _check_i32(node_tokens, (B, N), "node_tokens")
    _check_i32(parents, (N,), "parents")
    _check_i32(depth, (N,), "depth")
    ts = _row_stride(target_logits, N, V)
    dev = target_logits.device
    with _on(stream):
        if out_path is None:
            out_path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
        if out_path_len is None:
            out_path_len = torch.empty((B,), dtype=torch.int32, device=dev)
        if out_bonus is None:
            out_bonus = torch.empty((B,), dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = Workspace(dev).get(B, N, V)
    st = lib().spec_verify_tree(_ptr(target_logits), ts, _dtype_code(target_logits), _ptr(parents), _ptr(depth),
                                _ptr(node_tokens), B, N, V, max_depth, _ptr(out_path), _ptr(out_path_len),
                                _ptr(out_bonus), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    if st != 0:
        raise SVError(st, "spec_verify_tree")
    return out_path, out_path_len, out_bonus


def spec_verify_tree_sample(target_logits, draft_logits, parents, depth, node_tokens, temperature, max_depth: int,
                            seed: int = 0, offset: int = 0, out_path=None, out_path_len=None, out_token=None,
                            workspace=None, V: int | None = None, stream=None, without_replacement: bool = False,
                            seq_base: int = 0):
    """Sampled tree verification (multi-round rejection sampling). target and
    draft logits [B, N, V] (draft row v: q at node v), temperature [B] > 0.
    Returns (out_path [B, max_depth+1], out_path_len [B], out_token [B])."""
    import torch
    B, N = node_tokens.shape
    V = int(target_logits.shape[2]) if V is None else int(V)
    _check_i32(node_tokens, (B, N), "node_tokens")
    _check_i32(parents, (N,), "parents")
    _check_i32(depth, (N,), "depth")
    if temperature.dtype != torch.float32 or tuple(temperature.shape) != (B,) or not temperature.is_contiguous():
        raise ValueError("temperature must be a contiguous float32 tensor of shape [B]")
    if draft_logits.dtype != target_logits.dtype:
        raise ValueError("target and draft logits must have the same dtype")
    ts = _row_stride(target_logits, N, V)
    ds = _row_stride(draft_logits, N, V)
    dev = target_logits.device
    with _on(stream):
        if out_path is None:
            out_path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
        if out_path_len is None:
            out_path_len = torch.empty((B,), dtype=torch.int32, device=dev)
        if out_token is None:
            out_token = torch.empty((B,), dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = Workspace(dev).get(B, N, V)
    st = lib().spec_verify_tree_sample(_ptr(target_logits), ts, _ptr(draft_logits), ds, _dtype_code(target_logits),
                                       _ptr(parents), _ptr(depth), _ptr(node_tokens), _ptr(temperature), B, N, V,
                                       max_depth, seed, offset, seq_base, int(bool(without_replacement)), _ptr(out_path),
                                       _ptr(out_path_len), _ptr(out_token),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise SVError(st, "spec_verify_tree_sample")
    return out_path, out_path_len, out_token


def sv_kv_rollback(k_cache, v_cache, root_pos, path, path_len, cache_len=None, stream=None):
    """In-place KV-cache rollback to the accepted path. k_cache / v_cache:
    contiguous device tensors [L, B, H, S, D] (v_cache may be None); root_pos
    [B], path [B, P], path_len [B] int32. Returns cache_len [B] int32."""
    import torch
    if k_cache.dim() != 5 or not k_cache.is_contiguous() or not k_cache.is_cuda:
        raise ValueError("k_cache must be a contiguous [L, B, H, S, D] CUDA tensor")
    L, B, H, S, D = k_cache.shape
    if v_cache is not None and (tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype
                                or not v_cache.is_contiguous() or not v_cache.is_cuda):
        raise ValueError("v_cache must match k_cache")
    _check_i32(root_pos, (B,), "root_pos")
    _check_i32(path_len, (B,), "path_len")
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError("path must be [B, P]")
    _check_i32(path, tuple(path.shape), "path")
    if cache_len is None:
        with _on(stream):
            cache_len = torch.empty((B,), dtype=torch.int32, device=k_cache.device)
    st = lib().sv_kv_rollback(_ptr(k_cache), _ptr(v_cache) if v_cache is not None else None, k_cache.element_size(),
                              L, B, H, S, D, _ptr(root_pos), _ptr(path), int(path.shape[1]), _ptr(path_len),
                              _ptr(cache_len), _stream(stream))
    if st != 0:
        raise SVError(st, "sv_kv_rollback")
    return cache_len


def sv_kv_rollback_layers(k_layers, v_layers, root_pos, path, path_len, cache_len=None, stream=None):
    """sv_kv_rollback for caches kept as one tensor per layer: k_layers (and
    v_layers, or None) are lists of contiguous device tensors [B, H, S, D],
    all of one shape and dtype, 16-byte aligned. Returns cache_len [B]."""
    import torch
    if not k_layers:
        raise ValueError("k_layers must hold at least one layer")
    ref = k_layers[0]
    layers = list(k_layers) + (list(v_layers) if v_layers is not None else [])
    if v_layers is not None and len(v_layers) != len(k_layers):
        raise ValueError("v_layers must have as many layers as k_layers")
    for t in layers:
        if (t.dim() != 4 or tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or not t.is_contiguous()
                or not t.is_cuda or t.data_ptr() % 16 != 0):
            raise ValueError("every layer must be a contiguous, 16-byte aligned CUDA tensor of one shape and dtype")
    B, H, S, D = ref.shape
    _check_i32(root_pos, (B,), "root_pos")
    _check_i32(path_len, (B,), "path_len")
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError("path must be [B, P]")
    _check_i32(path, tuple(path.shape), "path")
    dev = ref.device
    with _on(stream):
        kp = torch.tensor([t.data_ptr() for t in k_layers], dtype=torch.int64, device=dev)
        vp = (torch.tensor([t.data_ptr() for t in v_layers], dtype=torch.int64, device=dev)
              if v_layers is not None else None)
        if cache_len is None:
            cache_len = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib().sv_kv_rollback_layers(_ptr(kp), _ptr(vp), ref.element_size(), len(k_layers), B, H, S, D,
                                     _ptr(root_pos), _ptr(path), int(path.shape[1]), _ptr(path_len), _ptr(cache_len),
                                     _stream(stream))
    if st != 0:
        raise SVError(st, "sv_kv_rollback_layers")
    return cache_len


def sv_ngram_draft(tokens, lengths, ngram, gamma, pad_with_last=True, out_draft=None, out_count=None,
                   out_match=None, stream=None):
    """Prompt-lookup drafting. tokens: device int32 [B, stride] (rows may be a
    strided view with unit element stride); lengths: int32 [B]. Returns
    (draft [B, gamma], count [B], match [B])."""
    import torch
    if tokens.dim() != 2 or tokens.dtype != torch.int32 or tokens.stride(1) != 1 or not tokens.is_cuda:
        raise ValueError("tokens must be an int32 [B, stride] CUDA tensor with contiguous rows")
    B = tokens.shape[0]
    _check_i32(lengths, (B,), "lengths")
    dev = tokens.device
    with _on(stream):
        if out_draft is None:
            out_draft = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        if out_count is None:
            out_count = torch.empty((B,), dtype=torch.int32, device=dev)
        if out_match is None:
            out_match = torch.empty((B,), dtype=torch.int32, device=dev)
    _check_i32(out_draft, (B, gamma), "out_draft")
    _check_i32(out_count, (B,), "out_count")
    _check_i32(out_match, (B,), "out_match")
    stride = tokens.stride(0) if B > 1 else tokens.shape[1]
    if stride < tokens.shape[1]:
        raise ValueError("rows of tokens overlap")
    st = lib().sv_ngram_draft(_ptr(tokens), stride, _ptr(lengths), B, int(ngram), int(gamma), int(bool(pad_with_last)),
                              _ptr(out_draft), _ptr(out_count), _ptr(out_match), _stream(stream))
    if st != 0:
        raise SVError(st, "sv_ngram_draft")
    return out_draft, out_count, out_match


def sv_tree_mask(parents, position_offset=None, B=None, mask=True, packed=False, position_ids=True,
                 out_mask=None, out_position_ids=None, stream=None):
    """Tree attention mask and position ids. parents: device int32 [B, N] (one
    tree per sequence; an expanded view shares one) or [N] (one tree, B from
    position_offset or the B argument). Returns (mask, position_ids): mask is
    bool [B, N, N], or with packed=True int32 words [B, N, ceil(N / 32)]
    holding the bits; either is None when not asked for."""
    import torch
    if parents.dtype != torch.int32 or not parents.is_cuda or parents.dim() not in (1, 2) or parents.stride(-1) != 1:
        raise ValueError("parents must be an int32 CUDA tensor [B, N] or [N] with contiguous rows")
    N = parents.shape[-1]
    if parents.dim() == 2:
        B = parents.shape[0]
        stride = parents.stride(0) if B > 1 else N
    else:
        B = B if B is not None else (position_offset.shape[0] if position_offset is not None else 1)
        stride = 0
    if position_offset is not None:
        _check_i32(position_offset, (B,), "position_offset")
    dev = parents.device
    with _on(stream):
        if mask and out_mask is None:
            out_mask = (torch.empty((B, N, (N + 31) // 32), dtype=torch.int32, device=dev) if packed
                        else torch.empty((B, N, N), dtype=torch.bool, device=dev))
        if position_ids and out_position_ids is None:
            out_position_ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_position_ids is not None:
        _check_i32(out_position_ids, (B, N), "out_position_ids")
    if out_mask is not None:
        want = (B, N, (N + 31) // 32) if packed else (B, N, N)
        if tuple(out_mask.shape) != want or not out_mask.is_contiguous() or not out_mask.is_cuda or \
                out_mask.element_size() != (4 if packed else 1):
            raise ValueError("out_mask must be a contiguous CUDA tensor of shape %s" % (want,))
    st = lib().sv_tree_mask(_ptr(parents), stride, B, N, _ptr(position_offset),
                            None if packed else _ptr(out_mask), _ptr(out_mask) if packed else None,
                            _ptr(out_position_ids), _stream(stream))
    if st != 0:
        raise SVError(st, "sv_tree_mask")
    return out_mask, out_position_ids


def sv_debug_philox(ctr, key, out=None, stream=None):
    """Philox4x32-10 blocks on the device: ctr [n, 4] and key [n, 2] int32
    tensors (bit patterns of uint32) -> out [n, 4]."""
    import torch
    n = ctr.shape[0]
    if out is None:
        out = torch.empty((n, 4), dtype=torch.int32, device=ctr.device)
    st = lib().sv_debug_philox(_ptr(ctr), _ptr(key), _ptr(out), n, _stream(stream))
    if st != 0:
        raise SVError(st, "sv_debug_philox")
    return out


def sv_debug_noise(words, stream=None):
    """Accept uniforms and Gumbel noise of 32-bit words (int32 tensor [n])."""
    import torch
    n = words.shape[0]
    g = torch.empty(n, dtype=torch.float32, device=words.device)
    u = torch.empty(n, dtype=torch.float32, device=words.device)
    st = lib().sv_debug_noise(_ptr(words), _ptr(g), _ptr(u), n, _stream(stream))
    if st != 0:
        raise SVError(st, "sv_debug_noise")
    return g, u


def sv_debug_read_stream(buf, nblocks: int, out=None, stream=None):
    """One plain streaming read of a device buffer (the read-bandwidth
    yardstick); returns the [4 * nblocks] int32 tensor of per-wave XOR folds."""
    import torch
    if out is None:
        out = torch.empty(4 * nblocks, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = lib().sv_debug_read_stream(_ptr(buf), nbytes, _ptr(out), nblocks, _stream(stream))
    if st != 0:
        raise SVError(st, "sv_debug_read_stream")
    return out


def sv_debug_wave_max(x, stream=None):
    """Wave-wide maximum of each group of 64 consecutive fp32 values (device
    tensor [64 * n]); returns [64 * n], every lane's result."""
    import torch
    if x.numel() % 64:
        raise ValueError("need a multiple of 64 values")
    out = torch.empty_like(x)
    st = lib().sv_debug_wave_max(_ptr(x), _ptr(out), x.numel() // 64, _stream(stream))
    if st != 0:
        raise SVError(st, "sv_debug_wave_max")
    return out
