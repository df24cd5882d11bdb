"""The C-ABI library on the host (no GPU): it loads, exports every entry point
include/spec_verify.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

rsv = pytest.importorskip("rejection_sampling_verify_amd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:sv_status_t|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rsv.LIB_PATH):
        pytest.skip("library not built")
    return rsv.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) >= {"spec_verify_sample", "spec_verify_greedy", "spec_verify_tree", "spec_verify_tree_sample",
                          "sv_kv_rollback", "sv_ngram_draft", "sv_tree_mask",
                          "sv_workspace_bytes",
                          "sv_workspace_init", "sv_status_string", "sv_debug_philox", "sv_debug_noise",
                          "sv_debug_wave_max", "sv_debug_read_stream", "sv_debug_sample_tiled"}
    out = subprocess.run(["nm", "-D", "--defined-only", rsv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(rsv.binding.EXPORTS) == names


def test_status_strings(L):
    for code in range(8):
        assert rsv.sv_status_string(code)
    assert rsv.sv_status_string(99) == "unknown status"


def test_workspace_bytes(L):
    a = rsv.sv_workspace_bytes(256, 9, 128256)
    assert a > 0 and a % 256 == 0
    assert rsv.sv_workspace_bytes(512, 9, 128256) > a
    assert rsv.sv_workspace_bytes(0, 9, 1000) > 0
    for bad in ((-1, 9, 1000), (1, 0, 1000), (1, 9, 0), (1, 2000, 10)):
        assert rsv.sv_workspace_bytes(*bad) == 0


class _Fake:
    """Host memory standing in for device pointers: validation never reads them."""

    def __init__(self, nbytes=1 << 16):
        self.buf = ctypes.create_string_buffer(nbytes + 256)
        addr = ctypes.addressof(self.buf)
        self.ptr = ctypes.c_void_p((addr + 255) // 256 * 256)
        self.nbytes = nbytes


def _sample(L, **kw):
    f = _Fake(1 << 20)
    args = dict(target=f.ptr, ts=1000, draft=f.ptr, ds=1000, dtype=1, ids=f.ptr, temp=f.ptr, B=4, gamma=3,
                V=1000, seed=0, offset=0, base=0, tok=f.ptr, n=f.ptr, diag=None, ws=f.ptr, wsb=f.nbytes,
                stream=None, tiling=None)
    args.update(kw)
    common = (args["target"], args["ts"], args["draft"], args["ds"], args["dtype"], args["ids"], args["temp"],
              args["B"], args["gamma"], args["V"], args["seed"], args["offset"], args["base"], args["tok"],
              args["n"], args["diag"], args["ws"], args["wsb"], args["stream"])
    if args["tiling"] is not None:
        return L.sv_debug_sample_tiled(*common, *args["tiling"])
    return L.spec_verify_sample(*common)


def test_sample_argument_validation(L):
    assert _sample(L, target=None) == 1
    assert _sample(L, ids=None) == 1
    assert _sample(L, temp=None) == 1
    assert _sample(L, gamma=0) == 2 and _sample(L, gamma=17) == 2
    assert _sample(L, V=0) == 2 and _sample(L, B=-1) == 2
    assert _sample(L, dtype=7) == 3
    assert _sample(L, ts=999) == 4 and _sample(L, ds=10) == 4
    assert _sample(L, offset=1 << 31) == 4
    assert _sample(L, base=(1 << 32) - 3) == 4 and _sample(L, base=(1 << 32) - 4, B=0) == 0
    assert _sample(L, tiling=(3, 0)) == 4 and _sample(L, tiling=(16, 0)) == 4 and _sample(L, tiling=(0, -1)) == 4
    assert _sample(L, tiling=(2, 5), B=0) == 0
    assert _sample(L, ws=None) == 5 and _sample(L, wsb=100) == 5
    f = _Fake(1 << 20)
    assert _sample(L, ws=ctypes.c_void_p(f.ptr.value + 16)) == 4  # misaligned workspace
    assert _sample(L, B=0) == 0  # nothing to do, nothing launched


def test_greedy_and_tree_argument_validation(L):
    f = _Fake(1 << 20)
    P = f.ptr
    assert L.spec_verify_greedy(None, 100, 1, P, 2, 2, 100, P, P, P, f.nbytes, None) == 1
    assert L.spec_verify_greedy(P, 100, 1, P, 2, 0, 100, P, P, P, f.nbytes, None) == 2
    assert L.spec_verify_greedy(P, 50, 1, P, 2, 2, 100, P, P, P, f.nbytes, None) == 4
    assert L.spec_verify_greedy(P, 100, 1, P, 0, 2, 100, P, P, P, f.nbytes, None) == 0
    tree = lambda **k: L.spec_verify_tree(k.get("t", P), k.get("ts", 100), k.get("dt", 1), k.get("par", P), P, P,
                                          k.get("B", 2), k.get("N", 5), k.get("V", 100), k.get("md", 3), P, P, P,
                                          k.get("ws", P), k.get("wsb", f.nbytes), None)
    assert tree(par=None) == 1
    assert tree(N=0) == 2 and tree(N=1025) == 2 and tree(md=5) == 2 and tree(md=-1) == 2
    assert tree(dt=2) == 3
    assert tree(ts=99) == 4
    assert tree(wsb=10) == 5
    assert tree(B=0) == 0
    assert L.sv_debug_philox(None, P, P, 1, None) == 1
    assert L.sv_debug_noise(P, None, None, -1, None) == 2
    assert L.sv_debug_wave_max(None, P, 1, None) == 1 and L.sv_debug_wave_max(P, P, -1, None) == 2
    # the read yardstick: validation happens before any launch
    A16, A17 = ctypes.c_void_p(4096), ctypes.c_void_p(4097)
    assert L.sv_debug_read_stream(None, 16, P, 1, None) == 1 and L.sv_debug_read_stream(A16, 16, None, 1, None) == 1
    assert L.sv_debug_read_stream(A16, 16, P, 0, None) == 2 and L.sv_debug_read_stream(A16, 15, P, 1, None) == 2
    assert L.sv_debug_read_stream(A17, 16, P, 1, None) == 4
    assert L.sv_workspace_init(None, 1024, None) == 1


def test_tree_sample_argument_validation(L):
    f = _Fake(1 << 20)
    P = f.ptr
    ts = lambda **k: L.spec_verify_tree_sample(k.get("t", P), k.get("ts", 100), k.get("d", P), k.get("ds", 100),
                                               k.get("dt", 1), k.get("par", P), P, P, k.get("temp", P),
                                               k.get("B", 2), k.get("N", 5), k.get("V", 100), k.get("md", 3),
                                               0, k.get("off", 0), k.get("base", 0), k.get("wor", 0), P, P, P,
                                               k.get("ws", P),
                                               k.get("wsb", f.nbytes), None)
    assert ts(d=None) == 1 and ts(temp=None) == 1 and ts(par=None) == 1
    assert ts(N=0) == 2 and ts(N=1025) == 2 and ts(md=5) == 2 and ts(md=-1) == 2 and ts(B=-1) == 2
    assert ts(dt=2) == 3
    assert ts(ts=99) == 4 and ts(ds=99) == 4 and ts(off=1 << 31) == 4 and ts(wor=2) == 4
    assert ts(base=(1 << 32) - 1) == 4
    assert ts(wsb=10) == 5
    assert ts(B=0) == 0


def test_kv_rollback_argument_validation(L):
    f = _Fake(1 << 16)
    P = f.ptr
    kv = lambda **k: L.sv_kv_rollback(k.get("k", P), k.get("v", P), k.get("es", 2), k.get("L", 2), k.get("B", 2),
                                      k.get("H", 2), k.get("S", 8), k.get("D", 64), k.get("root", P), P,
                                      k.get("P", 4), P, k.get("out", P), None)
    assert kv(k=None) == 1 and kv(root=None) == 1 and kv(out=None) == 1
    assert kv(S=0) == 2 and kv(D=0) == 2 and kv(P=0) == 2 and kv(P=1025) == 2 and kv(L=-1) == 2
    assert kv(D=7) == 2 and kv(D=8193) == 2 and kv(D=16384) == 2  # rows of 14 B; rows above 16 KiB
    assert kv(es=3) == 3
    assert kv(k=ctypes.c_void_p(P.value + 8)) == 4
    assert kv(L=0) == 0 and kv(H=0) == 0
    kl = lambda **k: L.sv_kv_rollback_layers(k.get("k", P), None, 2, 2, 2, 2, 8, k.get("D", 64), k.get("root", P), P, 4,
                                             P, P, None)
    assert kl(k=None) == 1 and kl(root=None) == 1 and kl(D=7) == 2


def test_ngram_argument_validation(L):
    f = _Fake(1 << 12)
    P = f.ptr
    ng = lambda **k: L.sv_ngram_draft(k.get("tok", P), k.get("stride", 64), k.get("len", P), k.get("B", 2),
                                      k.get("n", 3), k.get("g", 4), k.get("pad", 1), k.get("d", P), k.get("c", P),
                                      None, None)
    assert ng(tok=None) == 1 and ng(len=None) == 1 and ng(d=None) == 1 and ng(c=None) == 1
    assert ng(B=-1) == 2 and ng(stride=0) == 2 and ng(stride=1 << 31) == 2
    assert ng(n=0) == 2 and ng(n=17) == 2 and ng(g=0) == 2
    assert ng(pad=2) == 4
    assert ng(B=0) == 0


def test_tree_mask_argument_validation(L):
    f = _Fake(1 << 12)
    P = f.ptr
    tm = lambda **k: L.sv_tree_mask(k.get("par", P), k.get("stride", 8), k.get("B", 2), k.get("N", 8), None,
                                    k.get("m", P), k.get("bits", None), k.get("pos", None), None)
    assert tm(par=None) == 1 and tm(m=None) == 1
    assert tm(B=-1) == 2 and tm(N=0) == 2 and tm(N=1025) == 2 and tm(stride=-1) == 2 and tm(stride=7) == 2
    assert tm(B=0) == 0 and tm(B=0, stride=0) == 0


def test_library_reads_no_environment(L):
    """Tuning is fixed in the library or passed explicitly (sv_debug_sample_tiled):
    the library imports no environment lookup."""
    out = subprocess.run(["nm", "-D", "--undefined-only", rsv.LIB_PATH], capture_output=True, text=True).stdout
    imported = set(line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip())
    assert not imported & {"getenv", "secure_getenv", "__secure_getenv"}


def test_noalloc_argument_validation(L):
    """The allocation-free entry point refuses, before any HIP call, a call
    whose scratch need exceeds its static array, and validates like
    spec_verify_sample otherwise."""
    f = _Fake(1 << 16)
    P = f.ptr
    na = lambda **k: L.spec_verify_sample_noalloc(k.get("t", P), k.get("ts", 1000), None, 0, k.get("dt", 1), P,
                                                  k.get("temp", P), k.get("B", 4), k.get("G", 3), k.get("V", 1000),
                                                  0, k.get("off", 0), 0, P, P, None, None)
    assert na(B=4096, G=16, V=152064, ts=152064) == rsv.SV_ERR_SCRATCH_LIMIT
    assert na(temp=None) == 1 and na(t=None) == 1
    assert na(G=0) == 2 and na(dt=5) == 3 and na(ts=10) == 4 and na(off=1 << 31) == 4
    assert na(B=0) == 0
    assert "scratch" in rsv.sv_status_string(rsv.SV_ERR_SCRATCH_LIMIT)
