"""Seeded synthetic inputs of the verify step (host numpy arrays).

This module only PRODUCES inputs: logits, drafted ids, temperatures and tree
descriptions. It holds none of the verify arithmetic and is shared by the
tests, the benchmark and the smoke check, which hand the same arrays to the GPU
library and to the CPU oracle.

The drafter is emulated: drafted ids are drawn from softmax(draft / T) of the
stored (rounded) draft logits with numpy's own Gumbel-max draw, i.e. x ~ q as
the drafting loop of "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE &
Lookahead" ("A From-Scratch Implementation", step 1) produces them; at T = 0
the drafter proposes its argmax. bf16 logits are generated in fp32 and rounded
to nearest-even; they are handed over as uint16 bit patterns.

The five named workloads (``CONFIGS``) are:
  chain_f32_small  B=1,   gamma=4, V=1000,   fp32, T=1.0
  chain_bf16_peaked B=64, gamma=5, V=32000,  bf16, T=0.8, 5 boosted ids per row
  chain_bf16_llama B=256, gamma=8, V=128256, bf16, T in {0, 0.7, 1.0}, Zipf boost
  onehot_bf16_qwen B=512, gamma=6, V=152064, bf16, one-hot draft, T=1.0
  tree_bf16_llama  B=32,  N=65 nodes (root + 4 + 16 + 44), V=128256, bf16, greedy
and, for sampled tree verification (multi-round rejection sampling):
  tree_sample_bf16_llama  the same tree, B=32, V=128256, bf16, T in {0.7, 1.0}:
      target as chain_bf16_llama's, draft row of each inner node = target +
      N(0, sigma_b^2), sigma_b ~ U[0.2, 2]; children drawn i.i.d. from q at
      their parent.
  tree_sample_wor_bf16_llama  the same, with each node's children drawn
      without replacement (the top-k of the Gumbel-perturbed draft scores).
and, for the KV-cache rollback after a verify step:
  kv_rollback_bf16_llama  K and V caches [L=32, B=32, H=8, S=4096, D=128] bf16
      (the KV layout of a 32-layer model with 8 KV heads of dimension 128),
      root positions U[512, 3008), accepted paths drawn as walks in the same
      65-node tree (a uniformly random child at each level, 1 to 4 nodes).
and, for prompt-lookup drafting:
  ngram_draft_qwen  B=512 token histories of T ~ U[2048, 16384] tokens over
      V=152064 (row stride 16384), ngram=3, gamma=6, padded to gamma with the
      last token (the one-hot drafts of onehot_bf16_qwen); text is Zipf(1.1)
      with copies of earlier spans, and half the sequences end inside a copy.
and, for the tree attention mask and position ids:
  tree_mask_b256  B=256 sequences, each with its own 65-node tree (breadth-first,
      1 to 4 children per node, as dynamic trees are), position offsets
      U[512, 4096) (the root's place in the sequence), bool mask.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CONFIGS = ["chain_f32_small", "chain_bf16_peaked", "chain_bf16_llama", "onehot_bf16_qwen",
           "tree_bf16_llama"]
CONFIG_INDEX = {name: k for k, name in enumerate(CONFIGS)}
EXTRA = ["tree_sample_bf16_llama", "kv_rollback_bf16_llama", "ngram_draft_qwen", "tree_mask_b256",
         "tree_sample_wor_bf16_llama"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_values(a: np.ndarray) -> np.ndarray:
    """The fp32 values of a stored logits array (float32 or bf16 bits)."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else a


@dataclass
class ChainInputs:
    name: str
    target: np.ndarray             # [B, gamma+1, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray | None       # [B, gamma, V] same dtype, or None (one-hot draft)
    draft_ids: np.ndarray          # [B, gamma] int32
    temperature: np.ndarray        # [B] float32
    seed: int = 0
    offset: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.draft_ids.shape[0]

    @property
    def gamma(self):
        return self.draft_ids.shape[1]

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def is_bf16(self):
        return self.target.dtype == np.uint16

    def algorithmic_bytes(self) -> int:
        """Every target row once, plus every draft row the verifier needs
        (dense draft and T > 0)."""
        es = self.target.itemsize
        n = self.B * (self.gamma + 1) * self.V * es
        if self.draft is not None:
            n += int(np.count_nonzero(self.temperature > 0)) * self.gamma * self.V * es
        return n


@dataclass
class TreeInputs:
    name: str
    target: np.ndarray        # [B, N, V]
    parents: np.ndarray       # [N] int32
    depth: np.ndarray         # [N] int32
    node_tokens: np.ndarray   # [B, N] int32
    max_depth: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.node_tokens.shape[0]

    @property
    def N(self):
        return self.node_tokens.shape[1]

    @property
    def V(self):
        return self.target.shape[2]

    def algorithmic_bytes(self) -> int:
        return self.B * self.N * self.V * self.target.itemsize


@dataclass
class TreeSampleInputs:
    name: str
    target: np.ndarray        # [B, N, V]
    draft: np.ndarray         # [B, N, V]; row v: q at node v (zeros at leaves: never read)
    parents: np.ndarray       # [N] int32
    depth: np.ndarray         # [N] int32
    node_tokens: np.ndarray   # [B, N] int32
    temperature: np.ndarray   # [B] float32
    max_depth: int
    seed: int = 0
    offset: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.node_tokens.shape[0]

    @property
    def N(self):
        return self.node_tokens.shape[1]

    @property
    def V(self):
        return self.target.shape[2]

    def inner_nodes(self) -> int:
        return int(len(set(int(p) for p in self.parents[1:])))

    paths: tuple | None = None  # (path [B, max_depth + 1], path_len [B]) of a verified step

    def algorithmic_bytes(self) -> int:
        """Rows a step must read at least once: the target and draft row of
        every inner node on each sequence's accepted path, plus the leaf row
        when the path ends at a leaf (its bonus draw). Needs self.paths; without
        it, the bound for the deepest possible path of every sequence."""
        inner = set(int(p) for p in self.parents[1:])
        row = self.V * self.target.itemsize
        if self.paths is None:
            return self.B * (2 * (self.max_depth + 1)) * row
        path, plen = self.paths
        rows = 0
        for b in range(self.B):
            nodes = [int(v) for v in path[b, :max(int(plen[b]), 0)]]
            rows += sum(2 for v in nodes if v in inner)
            if nodes and nodes[-1] not in inner:
                rows += 1
        return rows * row


def _seq_rng(seed: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))


def _parallel(fn, n, workers=None):
    workers = workers or min(16, os.cpu_count() or 1)
    if n <= 1 or workers <= 1:
        for b in range(n):
            fn(b)
        return
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, range(n)))


def _draw_from_logits(rng, logits_f32: np.ndarray, T: float) -> int:
    """Emulated drafter: one draw from softmax(logits / T) (argmax at T = 0)."""
    y = logits_f32.astype(np.float64)
    if T == 0.0:
        return int(np.argmax(y))
    g = rng.gumbel(size=y.shape[0])
    return int(np.argmax(y / T + g))


def make_chain(name: str, B: int, gamma: int, V: int, *, bf16: bool, seed: int,
               target_sigma: float, boost: str | None = None, n_boost: int = 0,
               boost_value: float = 0.0, draft_scale: float = 1.0,
               draft_sigma: float | tuple = 0.5, temperatures=(1.0,), one_hot: bool = False,
               onehot_hit: float = 0.7, row_stride: int | None = None, workers=None) -> ChainInputs:
    """Generic chain workload.

    target = N(0, target_sigma^2) [+ boost]; draft = draft_scale * target[:, :gamma]
    + N(0, sigma_b^2) with sigma_b fixed or drawn per sequence from a (lo, hi)
    range; temperatures drawn per sequence uniformly from ``temperatures``;
    one_hot: no draft logits, drafted id = target argmax w.p. onehot_hit else
    uniform. ``row_stride`` > V pads every row (the padding holds large values
    that must never be read).
    """
    S = row_stride or V
    dt = np.uint16 if bf16 else np.float32
    target = np.empty((B, gamma + 1, S), dt)
    draft = None if one_hot else np.empty((B, gamma, S), dt)
    ids = np.empty((B, gamma), np.int32)
    temp = np.empty(B, np.float32)
    sigmas = np.empty(B, np.float64)
    logtab = np.log(np.arange(1, V + 1, dtype=np.float64)) if boost == "zipf" else None

    def one(b):
        rng = _seq_rng(seed, b)
        T = float(temperatures[rng.integers(len(temperatures))]) if len(temperatures) > 1 else float(temperatures[0])
        temp[b] = T
        t = rng.standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(target_sigma)
        if boost == "zipf":
            for r in range(gamma + 1):
                rank0 = rng.permutation(V)  # rank - 1 of every vocab entry
                t[r] -= (1.1 * logtab[rank0]).astype(np.float32)
        elif boost == "peaks":
            for r in range(gamma + 1):
                hot = rng.choice(V, size=n_boost, replace=False)
                t[r, hot] += np.float32(boost_value)
        if S > V:
            pad = np.full((gamma + 1, S - V), 1.0e4, np.float32)
            t_store = np.concatenate([t, pad], axis=1)
        else:
            t_store = t
        target[b] = round_bf16(t_store) if bf16 else t_store
        t_vals = stored_values(target[b])[:, :V]
        if one_hot:
            for i in range(gamma):
                if rng.random() < onehot_hit:
                    ids[b, i] = int(np.argmax(t_vals[i]))
                else:
                    ids[b, i] = int(rng.integers(V))
            sigmas[b] = np.nan
            return
        sig = float(rng.uniform(*draft_sigma)) if isinstance(draft_sigma, tuple) else float(draft_sigma)
        sigmas[b] = sig
        d = np.float32(draft_scale) * t[:gamma] + rng.standard_normal((gamma, V), dtype=np.float32) * np.float32(sig)
        if S > V:
            d = np.concatenate([d, np.full((gamma, S - V), 1.0e4, np.float32)], axis=1)
        draft[b] = round_bf16(d) if bf16 else d
        d_vals = stored_values(draft[b])[:, :V]
        for i in range(gamma):
            ids[b, i] = _draw_from_logits(rng, d_vals[i], T)

    _parallel(one, B, workers)
    inp = ChainInputs(name, target, draft, ids, temp, seed=0, offset=0,
                      meta={"V": V, "row_stride": S, "draft_sigma": sigmas})
    if S > V:
        inp.meta["padded"] = True
    return inp


def _c5_tree():
    """Root, 4 children, 16 grandchildren, then the first 44 great-grandchildren
    in breadth-first order (branching 4, last level truncated)."""
    parents = [-1] + [0] * 4 + [1 + (k - 5) // 4 for k in range(5, 21)] + [5 + (k - 21) // 4 for k in range(21, 65)]
    depth = [0] + [1] * 4 + [2] * 16 + [3] * 44
    return np.array(parents, np.int32), np.array(depth, np.int32)


def make_tree(name: str, B: int, V: int, parents: np.ndarray, depth: np.ndarray, *, bf16: bool,
              seed: int, target_sigma: float = 3.0, hit: float = 0.5, workers=None) -> TreeInputs:
    N = len(parents)
    dt = np.uint16 if bf16 else np.float32
    target = np.empty((B, N, V), dt)
    tokens = np.empty((B, N), np.int32)

    def one(b):
        rng = _seq_rng(seed, b)
        t = rng.standard_normal((N, V), dtype=np.float32) * np.float32(target_sigma)
        target[b] = round_bf16(t) if bf16 else t
        vals = stored_values(target[b])
        tokens[b, 0] = int(rng.integers(V))
        for c in range(1, N):
            if rng.random() < hit:
                tokens[b, c] = int(np.argmax(vals[parents[c]]))
            else:
                tokens[b, c] = int(rng.integers(V))

    _parallel(one, B, workers)
    return TreeInputs(name, target, np.asarray(parents, np.int32), np.asarray(depth, np.int32),
                      tokens, int(np.max(depth)))


def make_tree_sample(name: str, B: int, V: int, parents: np.ndarray, depth: np.ndarray, *, bf16: bool,
                     seed: int, temperatures=(0.7, 1.0), target_sigma: float = 3.0, zipf: float = 1.1,
                     draft_sigma=(0.2, 2.0), workers=None, without_replacement: bool = False) -> TreeSampleInputs:
    """Sampled-tree inputs: children are i.i.d. draws from q at their parent,
    or (without_replacement) a draw without replacement in index order: the
    top-k of the Gumbel-perturbed draft scores, in order of perturbed score."""
    N = len(parents)
    dt = np.uint16 if bf16 else np.float32
    target = np.empty((B, N, V), dt)
    draft = np.zeros((B, N, V), dt)
    tokens = np.empty((B, N), np.int32)
    temp = np.empty(B, np.float32)
    inner = sorted(set(int(p) for p in parents[1:]))

    def one(b):
        rng = _seq_rng(seed, b)
        T = float(temperatures[b % len(temperatures)])
        temp[b] = T
        sig = rng.uniform(*draft_sigma) if isinstance(draft_sigma, tuple) else float(draft_sigma)
        for v in range(N):
            t = rng.standard_normal(V, dtype=np.float32) * np.float32(target_sigma)
            if zipf:
                rank = rng.permutation(V).astype(np.float32) + 1.0
                t = t - np.float32(zipf) * np.log(rank)
            target[b, v] = round_bf16(t) if bf16 else t
            if v in inner:
                d = t + rng.standard_normal(V, dtype=np.float32) * np.float32(sig)
                draft[b, v] = round_bf16(d) if bf16 else d
        tokens[b, 0] = int(rng.integers(V))
        q_vals = stored_values(draft[b])
        if without_replacement:
            for v in inner:
                kids = [c for c in range(1, N) if parents[c] == v]
                y = q_vals[v].astype(np.float64) / T + rng.gumbel(size=V)
                order = np.argsort(-y, kind="stable")[:len(kids)]
                for c, x in zip(kids, order):
                    tokens[b, c] = int(x)
            return
        for c in range(1, N):
            tokens[b, c] = _draw_from_logits(rng, q_vals[parents[c]], T)

    _parallel(one, B, workers)
    return TreeSampleInputs(name, target, draft, np.asarray(parents, np.int32), np.asarray(depth, np.int32),
                            tokens, temp, int(np.max(depth)), meta={"V": V, "without_replacement": without_replacement})


def make(name: str, workers=None):
    """One of the five named workloads at full size (generator seed 1000 + k)."""
    k = CONFIG_INDEX[name]
    seed = 1000 + k
    if name == "chain_f32_small":
        return make_chain(name, 1, 4, 1000, bf16=False, seed=seed, target_sigma=2.0,
                          draft_sigma=0.5, temperatures=(1.0,), workers=workers)
    if name == "chain_bf16_peaked":
        return make_chain(name, 64, 5, 32000, bf16=True, seed=seed, target_sigma=3.0, boost="peaks",
                          n_boost=5, boost_value=8.0, draft_scale=0.8, draft_sigma=1.0,
                          temperatures=(0.8,), workers=workers)
    if name == "chain_bf16_llama":
        return make_chain(name, 256, 8, 128256, bf16=True, seed=seed, target_sigma=3.0, boost="zipf",
                          draft_sigma=(0.2, 2.0), temperatures=(0.0, 0.7, 1.0), workers=workers)
    if name == "onehot_bf16_qwen":
        return make_chain(name, 512, 6, 152064, bf16=True, seed=seed, target_sigma=3.0,
                          temperatures=(1.0,), one_hot=True, onehot_hit=0.7, workers=workers)
    if name == "tree_bf16_llama":
        parents, depth = _c5_tree()
        return make_tree(name, 32, 128256, parents, depth, bf16=True, seed=seed, workers=workers)
    raise KeyError(name)


@dataclass
class KvRollbackInputs:
    """A KV-cache rollback: caches of shape [L, B, H, S, D] with elements of
    elem_bytes bytes (generated on demand: cache_host for small shapes,
    fill_kv_device for resident ones), and per sequence the root position and
    the accepted path (root first, node i at position root + i)."""
    name: str
    shape: tuple              # (L, B, H, S, D)
    elem_bytes: int
    root: np.ndarray          # [B] int32
    path: np.ndarray          # [B, P] int32, -1 past path_len
    path_len: np.ndarray      # [B] int32
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.shape[1]

    def int_dtype(self):
        return {1: np.uint8, 2: np.int16, 4: np.int32}[self.elem_bytes]

    def cache_host(self, which: int) -> np.ndarray:
        """Random bit patterns (which = 0 for K, 1 for V)."""
        rng = np.random.default_rng([self.seed, 77, which])
        dt = self.int_dtype()
        info = np.iinfo(dt)
        return rng.integers(info.min, info.max, size=self.shape, dtype=dt, endpoint=True)

    def moved_rows(self) -> np.ndarray:
        """Per sequence, the path nodes whose row changes place (node k taken
        from a node other than k)."""
        return np.array([int(np.count_nonzero(self.path[b, :self.path_len[b]] != np.arange(self.path_len[b])))
                         for b in range(self.B)], np.int64)

    def algorithmic_bytes(self, with_v: bool = True) -> int:
        """Each moved row read once and written once in every layer and head,
        for K (and V), plus the root, path and length reads and the length
        writes."""
        L, B, H, S, D = self.shape
        row = D * self.elem_bytes
        moved = int(self.moved_rows().sum()) * L * H * row * 2 * (2 if with_v else 1)
        return moved + self.path.nbytes + 3 * B * 4


def fill_kv_device(torch, t, seed: int, which: int):
    """Seeded random bits into a resident cache tensor (integer dtype)."""
    g = torch.Generator(device=t.device)
    g.manual_seed(seed * 16 + which)
    t.random_(generator=g)
    return t


def _children(parents: np.ndarray):
    ch = [[] for _ in range(len(parents))]
    for v in range(1, len(parents)):
        ch[int(parents[v])].append(v)
    return ch


def make_kv_rollback(name: str, L: int, B: int, H: int, S: int, D: int, *, elem_bytes: int, seed: int,
                     kind: str = "tree", parents: np.ndarray | None = None, P: int | None = None,
                     root_lo: int = 0, root_hi: int | None = None) -> KvRollbackInputs:
    """kind 'tree': walks from the root of `parents`, a uniformly random child
    at each level and 1 .. depth + 1 nodes; 'chain': the identity path 0 .. n
    of a chain step, n uniform in [0, P); 'sparse': 0 followed by n - 1
    increasing node indices below S - root (long paths), n uniform in [1, P].
    Roots are uniform in [root_lo, root_hi) with root_hi defaulting to the
    largest root that keeps every node of the path inside the cache."""
    if kind == "tree":
        ch = _children(parents)
        depth = [0] * len(parents)
        for v in range(1, len(parents)):
            depth[v] = depth[int(parents[v])] + 1
        P = max(depth) + 1
        span = len(parents)
    elif kind == "chain":
        span = P
    elif kind == "sparse":
        span = S - root_lo if root_hi is None else S - root_hi + 1
    else:
        raise ValueError(kind)
    hi = S - span + 1 if root_hi is None else root_hi
    path = np.full((B, P), -1, np.int32)
    plen = np.empty(B, np.int32)
    root = np.empty(B, np.int32)
    for b in range(B):
        rng = _seq_rng(seed, b)
        root[b] = int(rng.integers(root_lo, hi))
        if kind == "tree":
            nodes = [0]
            n = int(rng.integers(1, P + 1))
            while len(nodes) < n and ch[nodes[-1]]:
                c = ch[nodes[-1]]
                nodes.append(c[int(rng.integers(len(c)))])
        elif kind == "chain":
            nodes = list(range(int(rng.integers(0, P)) + 1))
        else:
            n = int(rng.integers(1, P + 1))
            room = S - int(root[b])
            n = min(n, room)
            nodes = [0] + sorted(int(x) for x in rng.choice(np.arange(1, room), size=n - 1, replace=False))
        path[b, :len(nodes)] = nodes
        plen[b] = len(nodes)
    return KvRollbackInputs(name, (L, B, H, S, D), elem_bytes, root, path, plen, seed=seed, meta={"kind": kind})


@dataclass
class NgramInputs:
    """Token histories for n-gram drafting: tokens [B, stride] int32 (row b
    holds lengths[b] tokens, the rest -1), and the drafter's settings."""
    name: str
    tokens: np.ndarray
    lengths: np.ndarray
    ngram: int
    gamma: int
    pad: bool
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.tokens.shape[0]

    def algorithmic_bytes(self, match: np.ndarray) -> int:
        """Per sequence, the tokens from the match's start to the end (all of
        them without a match: a right-to-left scan has to read that far), the
        length, and the outputs (gamma + 2 words)."""
        n = 0
        for b in range(self.B):
            T = int(self.lengths[b])
            n += 4 * (T - int(match[b]) if match[b] >= 0 else T) + 4 * (self.gamma + 3)
        return n


def _zipf_sampler(V: int, s: float):
    w = np.arange(1, V + 1, dtype=np.float64) ** -s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    return lambda rng, size: np.minimum(np.searchsorted(cdf, rng.random(size)), V - 1).astype(np.int32)


def make_ngram(name: str, B: int, V: int, T_range, *, ngram: int, gamma: int, pad: bool, seed: int,
               stride: int | None = None, zipf: float = 1.1, copy_prob: float = 0.15, tail_copy: float = 0.5):
    """Zipf(zipf) text over V with copies: pieces of 16-256 fresh tokens, or
    (probability copy_prob, once 64 tokens exist) a copy of 8-128 earlier
    tokens from a uniform earlier start; with probability tail_copy the last
    c ~ U[ngram, 48] tokens are replaced by a copy of an earlier span, so the
    tail n-gram has an earlier occurrence. A per-sequence shift of the ids
    makes the frequent ids differ between sequences."""
    draw = _zipf_sampler(V, zipf)
    lo, hi = T_range
    stride = stride or hi
    tokens = np.full((B, stride), -1, np.int32)
    lengths = np.empty(B, np.int32)
    for b in range(B):
        rng = _seq_rng(seed, b)
        T = int(rng.integers(lo, hi + 1))
        seq = np.empty(T + 256, np.int32)
        n = 0
        while n < T:
            if n >= 64 and rng.random() < copy_prob:
                c = int(rng.integers(8, 129))
                src = int(rng.integers(0, n - 8))
                c = min(c, n - src)
                seq[n:n + c] = seq[src:src + c]
            else:
                c = int(rng.integers(16, 257))
                seq[n:n + c] = draw(rng, c)
            n += c
        seq = seq[:T]
        if T > 2 * 48 and rng.random() < tail_copy:
            c = int(rng.integers(ngram, 49))
            src = int(rng.integers(0, T - 2 * c))
            seq[T - c:] = seq[src:src + c].copy()
        shift = int(rng.integers(V))
        tokens[b, :T] = (seq.astype(np.int64) + shift) % V
        lengths[b] = T
    return NgramInputs(name, tokens, lengths, ngram, gamma, pad, meta={"V": V, "seed": seed})


def random_tree(rng, N: int, branching=(1, 4)) -> np.ndarray:
    """A breadth-first tree of N nodes (parents before children): each node of
    a level gets branching[0] .. branching[1] children until N nodes exist."""
    parents = [-1]
    frontier = [0]
    while len(parents) < N:
        nxt = []
        for p in frontier:
            for _ in range(int(rng.integers(branching[0], branching[1] + 1))):
                if len(parents) < N:
                    parents.append(p)
                    nxt.append(len(parents) - 1)
        frontier = nxt or [len(parents) - 1]
    return np.array(parents, np.int32)


@dataclass
class TreeMaskInputs:
    name: str
    parents: np.ndarray   # [B, N] int32
    offsets: np.ndarray   # [B] int32
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.parents.shape[0]

    @property
    def N(self):
        return self.parents.shape[1]

    def algorithmic_bytes(self, packed: bool = False) -> int:
        """Parents and offsets read; mask (bytes, or packed words) and
        position ids written."""
        B, N = self.parents.shape
        mask = B * N * ((N + 31) // 32) * 4 if packed else B * N * N
        return B * N * 4 + B * 4 + mask + B * N * 4


def make_tree_mask(name: str, B: int, N: int, *, seed: int, branching=(1, 4), offset_range=(512, 4096),
                   chain: bool = False) -> TreeMaskInputs:
    parents = np.empty((B, N), np.int32)
    offsets = np.empty(B, np.int32)
    for b in range(B):
        rng = _seq_rng(seed, b)
        parents[b] = np.arange(-1, N - 1, dtype=np.int32) if chain else random_tree(rng, N, branching)
        offsets[b] = int(rng.integers(offset_range[0], offset_range[1]))
    return TreeMaskInputs(name, parents, offsets)


def make_extra(name: str, workers=None):
    """Workloads of the rows beyond the five configurations (seed 2000 + k)."""
    seed = 2000 + EXTRA.index(name)
    if name == "tree_sample_bf16_llama":
        parents, depth = _c5_tree()
        return make_tree_sample(name, 32, 128256, parents, depth, bf16=True, seed=seed, workers=workers)
    if name == "kv_rollback_bf16_llama":
        parents, _ = _c5_tree()
        return make_kv_rollback(name, 32, 32, 8, 4096, 128, elem_bytes=2, seed=seed, kind="tree", parents=parents,
                                root_lo=512, root_hi=3008)
    if name == "ngram_draft_qwen":
        return make_ngram(name, 512, 152064, (2048, 16384), ngram=3, gamma=6, pad=True, seed=seed)
    if name == "tree_mask_b256":
        return make_tree_mask(name, 256, 65, seed=seed)
    if name == "tree_sample_wor_bf16_llama":
        parents, depth = _c5_tree()
        return make_tree_sample(name, 32, 128256, parents, depth, bf16=True, seed=seed, workers=workers,
                                without_replacement=True)
    raise KeyError(name)


def tree_c5_structure():
    return _c5_tree()
