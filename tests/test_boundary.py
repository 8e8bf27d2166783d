"""The C ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before launching anything.

Only calls that fail validation (or are pure host functions) are made here;
fake device addresses are never dereferenced because validation returns first.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.environ.get("VP_LMHEAD_LIB") or os.path.join(ROOT, "vocab_lm_head_amd", "libvplmhead.so")

OK, NULL, SHAPE, RANGE, ALIGN, WORKSPACE, HIP = 0, -1, -2, -3, -4, -5, -6


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(vp_\w+)\s*\(", src, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python vocab_lm_head_amd/build.py)")
    from vocab_lm_head_amd import _lib
    return _lib.lib


def test_header_declares_the_four_entry_points():
    d = _declared()
    for name in ("vp_embed_fwd", "vp_lmhead_ce_fwd", "vp_ce_combine", "vp_lmhead_ce_bwd"):
        assert name in d


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (vp_\w+)$", out, flags=re.M))
    declared = _declared()
    assert declared, "no declarations parsed from include/*.h"
    assert declared <= exported, f"missing exports: {declared - exported}"
    from vocab_lm_head_amd import _lib
    assert set(_lib.SIGNATURES) == declared, "binding signatures must cover exactly the header"


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, RANGE, ALIGN, WORKSPACE, HIP):
        assert lib.vp_status_string(code)
    assert b"unknown" in lib.vp_status_string(12345)


def test_shard_range(lib):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.vp_shard_range(128256, 8, 3, ctypes.byref(a), ctypes.byref(b)) == OK
    assert (a.value, b.value) == (3 * 16032, 4 * 16032)
    assert lib.vp_shard_range(152064, 8, 7, ctypes.byref(a), ctypes.byref(b)) == OK
    assert (a.value, b.value) == (7 * 19008, 152064)
    assert lib.vp_shard_range(10, 4, 0, ctypes.byref(a), ctypes.byref(b)) == SHAPE   # V % T
    assert lib.vp_shard_range(8, 0, 0, ctypes.byref(a), ctypes.byref(b)) == SHAPE
    assert lib.vp_shard_range(8, 2, 2, ctypes.byref(a), ctypes.byref(b)) == RANGE
    assert lib.vp_shard_range(8, 2, -1, ctypes.byref(a), ctypes.byref(b)) == RANGE
    assert lib.vp_shard_range(8, 2, 0, None, ctypes.byref(b)) == NULL


def test_padded_vocab_matches_the_oracle(lib):
    """Host-only helper: the pages' 50257 -> 51200 (T = 8) and random sizes, against the
    oracle's definition; bad arguments are rejected."""
    import numpy as np

    import oracle
    out = ctypes.c_int64()
    assert lib.vp_padded_vocab(50257, 8, 128, ctypes.byref(out)) == OK and out.value == 51200
    rng = np.random.default_rng(3)
    for _ in range(300):
        V, T, m = int(rng.integers(1, 10**9)), int(rng.integers(1, 65)), int(rng.choice([1, 8, 128, 256]))
        assert lib.vp_padded_vocab(V, T, m, ctypes.byref(out)) == OK
        assert out.value == oracle.padded_vocab(V, T, m), (V, T, m)
    assert lib.vp_padded_vocab(0, 8, 128, ctypes.byref(out)) == SHAPE
    assert lib.vp_padded_vocab(100, 0, 128, ctypes.byref(out)) == SHAPE
    assert lib.vp_padded_vocab(100, 8, 0, ctypes.byref(out)) == SHAPE
    assert lib.vp_padded_vocab(2**62, 8, 2**60, ctypes.byref(out)) == SHAPE
    assert lib.vp_padded_vocab(100, 8, 128, None) == NULL


FAKE = 0x10000          # 256-byte aligned, never dereferenced (validation fails first)
FAKE_ODD = 0x10002


def test_embed_validation(lib):
    f = lib.vp_embed_fwd
    assert f(FAKE, -1, FAKE, 0, 8, 16, FAKE, None) == SHAPE
    assert f(FAKE, 4, FAKE, 0, 8, 0, FAKE, None) == SHAPE
    assert f(FAKE, 4, FAKE, 8, 8, 16, FAKE, None) == RANGE
    assert f(FAKE, 4, FAKE, -1, 8, 16, FAKE, None) == RANGE
    assert f(FAKE, 4, FAKE, 0, 8, 12, FAKE, None) == ALIGN
    assert f(None, 4, FAKE, 0, 8, 16, FAKE, None) == NULL
    assert f(FAKE, 4, None, 0, 8, 16, FAKE, None) == NULL
    assert f(FAKE, 4, FAKE, 0, 8, 16, None, None) == NULL
    assert f(FAKE, 4, FAKE_ODD, 0, 8, 16, FAKE, None) == ALIGN
    assert f(FAKE + 4, 4, FAKE, 0, 8, 16, FAKE, None) == ALIGN
    assert f(None, 0, None, 0, 8, 16, None, None) == OK      # n == 0: nothing to do


def test_fwd_validation_and_workspace(lib):
    ws = lib.vp_lmhead_ce_fwd_workspace
    assert ws(0, 4096, 0, 16032) == 0
    need = ws(8192, 4096, 0, 16032)
    slices = -(-16032 // 128)
    assert need == -(-(3 * slices * 8192 * 4) // 256) * 256
    assert ws(8192, 12, 0, 16032) == 0          # invalid h -> 0
    # few tokens over many slices: the merge splits the 2000 slices 8 ways, whose results
    # ([3, 8, n] fp32) follow the per-slice partials
    r256 = lambda b: -(-b // 256) * 256
    assert ws(4096, 4096, 0, 256000) == r256(3 * 2000 * 4096 * 4) + r256(3 * 8 * 4096 * 4)
    f = lib.vp_lmhead_ce_fwd
    args = lambda **k: [k.get("x", FAKE), k.get("w", FAKE), k.get("t", FAKE), k.get("n", 8192),
                        k.get("h", 4096), k.get("lo", 0), k.get("hi", 16032), FAKE, FAKE, FAKE,
                        k.get("ws", FAKE), k.get("wsb", need), None]
    assert f(*args(ws=None)) == WORKSPACE
    assert f(*args(wsb=need - 1)) == WORKSPACE
    assert f(*args(ws=FAKE + 16)) == WORKSPACE                # not 256-byte aligned
    assert f(*args(x=None)) == NULL
    assert f(*args(t=FAKE + 4)) == ALIGN
    assert f(*args(w=FAKE_ODD)) == ALIGN
    assert f(*args(h=4100)) == ALIGN
    assert f(*args(n=-5)) == SHAPE
    assert f(*args(hi=0)) == RANGE
    assert f(*args(n=0, x=None, w=None, t=None, ws=None, wsb=0)) == OK


def test_embed_bwd_validation_and_workspace(lib):
    ws = lib.vp_embed_bwd_workspace
    n, h, vs = 65536, 4096, 64000
    r256 = lambda b: -(-b // 256) * 256
    nblk, nseg = -(-n // 1024), -(-n // 64)     # radix-sort tiles, segment-sum blocks
    need = ws(n, h, 0, vs)
    assert need == 4 * r256(4 * n) + r256(256 * nblk * 4) + 2 * r256(nseg * h * 4)
    assert ws(0, h, 0, vs) == 0 and ws(n, 12, 0, vs) == 0 and ws(n, h, 5, 5) == 0
    f = lib.vp_embed_bwd
    base = dict(ids=FAKE, n=n, dout=FAKE, lo=0, hi=vs, h=h, dw=FAKE, ws=FAKE, wsb=need)
    call = lambda **k: f(*[{**base, **k}[a] for a in ("ids", "n", "dout", "lo", "hi", "h", "dw",
                                                      "ws", "wsb")], None)
    assert call(ids=None) == NULL and call(dout=None) == NULL and call(dw=None) == NULL
    assert call(n=-1) == SHAPE and call(n=(1 << 24) + 1) == SHAPE and call(h=0) == SHAPE
    assert call(hi=0) == RANGE and call(lo=-1) == RANGE
    assert call(h=12) == ALIGN and call(ids=FAKE + 4) == ALIGN and call(dout=FAKE + 8) == ALIGN
    assert call(dw=FAKE + 4) == ALIGN
    assert call(ws=None) == WORKSPACE and call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 128) == WORKSPACE
    assert call(n=0, ids=None, dout=None, dw=None, ws=None, wsb=0) == OK


def test_comparator_validation(lib):
    n, h, vs = 8192, 4096, 16032
    f = lib.vp_lmhead_logits
    assert f(FAKE, FAKE, n, h, 0, vs, FAKE, vs - 4, None) == SHAPE      # ld < Vs
    assert f(FAKE, FAKE, n, h, 0, vs, FAKE, vs + 2, None) == ALIGN      # ld % 4
    assert f(FAKE, FAKE, n, h, 0, vs, FAKE, (1 << 21), None) == SHAPE   # ld too large
    assert f(None, FAKE, n, h, 0, vs, FAKE, vs, None) == NULL
    assert f(FAKE, FAKE, n, h, 0, vs, FAKE + 4, vs, None) == ALIGN
    assert f(None, None, 0, h, 0, vs, None, vs, None) == OK
    g = lib.vp_logits_ce_stats
    assert g(FAKE, vs, FAKE, n, 0, vs, None, FAKE, FAKE, None, None) == NULL
    assert g(FAKE, vs, FAKE, n, 10, 10, None, FAKE, FAKE, FAKE, None) == RANGE
    assert g(FAKE, vs - 4, FAKE, n, 0, vs, None, FAKE, FAKE, FAKE, None) == SHAPE
    assert g(FAKE, vs, FAKE + 4, n, 0, vs, None, FAKE, FAKE, FAKE, None) == ALIGN
    assert g(FAKE, vs, FAKE, n, 0, vs, FAKE + 2, FAKE, FAKE, FAKE, None) == ALIGN
    m = lib.vp_ce_max
    assert m(FAKE, n, 0, FAKE, None) == SHAPE and m(None, n, 8, FAKE, None) == NULL
    assert m(None, 0, 8, None, None) == OK
    b = lib.vp_logits_ce_bwd
    ws = lib.vp_lmhead_ce_bwd_workspace(n, h, 0, vs)
    args = [FAKE, vs, FAKE, FAKE, FAKE, FAKE, n, h, 0, vs, -100, 1.0, FAKE, FAKE, FAKE, ws, None]
    call = lambda i, v: b(*(args[:i] + [v] + args[i + 1:]))
    assert call(0, None) == NULL and call(1, vs - 4) == SHAPE and call(1, vs + 1) == ALIGN
    assert call(15, ws - 1) == WORKSPACE and call(14, None) == WORKSPACE
    assert call(13, FAKE + 4) == ALIGN


def test_combine_validation(lib):
    f = lib.vp_ce_combine
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 0, -100, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 2, -100, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 2, -100, FAKE, FAKE, None, None) == NULL
    assert f(None, FAKE, FAKE, FAKE, 16, 2, -100, FAKE, FAKE, FAKE, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE + 4, 16, 2, -100, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, (1 << 31) + 1, 2, -100, FAKE, FAKE, FAKE, None) == SHAPE


def test_bwd_validation_and_workspace(lib):
    ws = lib.vp_lmhead_ce_bwd_workspace
    n, h, vs = 8192, 4096, 16032
    need = ws(n, h, 0, vs)
    r256 = lambda b: -(-b // 256) * 256
    r64 = lambda e: -(-e // 64) * 64      # rows padded to 64 elements
    n64, vs64 = r64(n), r64(vs)
    assert need == r256(h * n64 * 2) + r256(h * vs64 * 2) + r256(n * vs64 * 2) + r256(vs * n64 * 2)
    assert ws(6, 32, 0, 4) == r256(32 * 64 * 2) * 2 + r256(6 * 64 * 2) + r256(4 * 64 * 2)
    def bufs(n_, h_, vs_):   # the four bf16 buffers
        return (r256(h_ * r64(n_) * 2) + r256(h_ * r64(vs_) * 2) + r256(n_ * r64(vs_) * 2)
                + r256(vs_ * r64(n_) * 2))
    # small LM (n 4096, h 512, Vs 3200): as 128 x 128 tiles dX has 4 x 32 and dW 4 x 25, one
    # round of 228 workgroups, with K loops of 50 and 64 steps: one launch, no fp32 partials
    assert ws(4096, 512, 0, 3200) == bufs(4096, 512, 3200)
    assert ws(64, 520, 0, 1000) == bufs(64, 520, 1000)
    # n 2048, h 512, Vs 9000: 348 small tiles, so 256 x 256 tiles (dX 2 x 8, dW 2 x 36), both
    # split over K in one grouped launch sized for one round: 21 K steps per workgroup,
    # 7 + 2 splits, both GEMMs' fp32 partials side by side
    assert ws(2048, 512, 0, 9000) == (bufs(2048, 512, 9000) + r256(7 * 2048 * 512 * 4)
                                      + r256(2 * 9000 * 512 * 4))
    # only dX split (n 256, h 512, Vs 16000: dX K 250 steps over 2 tiles; dW's K is 4 steps):
    # 16 splits in a single partials region
    assert ws(256, 512, 0, 16000) == bufs(256, 512, 16000) + r256(16 * 256 * 512 * 4)
    # only dW split (n 12000, h 64, Vs 900: dW's K is 188 steps over 4 tiles; dX's 15)
    assert ws(12000, 64, 0, 900) == bufs(12000, 64, 900) + r256(16 * 900 * 64 * 4)
    f = lib.vp_lmhead_ce_bwd
    base = dict(x=FAKE, w=FAKE, t=FAKE, lse=FAKE, n=n, h=h, lo=0, hi=vs, ign=-100, g=1.0,
                dx=FAKE, dw=FAKE, ws=FAKE, wsb=need)
    call = lambda **k: f(*[{**base, **k}[a] for a in ("x", "w", "t", "lse", "n", "h", "lo", "hi",
                                                      "ign", "g", "dx", "dw", "ws", "wsb")], None)
    assert call(dw=None) == NULL
    assert call(lse=None) == NULL
    assert call(wsb=need - 256) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(dx=FAKE + 8) == ALIGN
    assert call(h=8, hi=0) == RANGE
    assert call(n=-1) == SHAPE
    assert call(h=(1 << 20) + 8) == SHAPE      # rows above 2^20 elements
    assert call(hi=(1 << 20) + 1) == SHAPE
    assert call(n=(1 << 20) + 1) == SHAPE


def test_product_package_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding must raise (not fall back) when the shared library is absent."""
    import importlib.util
    monkeypatch.delenv("VP_LMHEAD_LIB", raising=False)   # no other build of it either
    src = os.path.join(ROOT, "vocab_lm_head_amd", "_lib.py")
    dst = tmp_path / "_lib.py"
    dst.write_text(open(src).read())   # a copy with no libvplmhead.so beside it
    spec = importlib.util.spec_from_file_location("vp_lib_copy", dst)
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="no CPU fallback"):
        spec.loader.exec_module(mod)


def test_product_does_not_reference_oracle():
    """Nothing under the package imports or names the oracle."""
    pkg = os.path.join(ROOT, "vocab_lm_head_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
            txt = open(path).read()
            assert not re.search(r"\boracle\b", txt), path


def test_binding_refuses_host_and_mismatched_tensors():
    """Without a GPU: the binding refuses host tensors (their pointers would reach the
    kernels), wrong dtypes, a host workspace, tensors spread over two devices and
    mis-shaped buffers, each before the library is called."""
    import torch
    import vocab_lm_head_amd as vp
    from vocab_lm_head_amd import _lib
    n, h, vs = 16, 8, 24
    x = torch.zeros((n, h), dtype=torch.bfloat16)
    w = torch.zeros((vs, h), dtype=torch.bfloat16)
    y = torch.zeros(n, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU tensor"):
        vp.vp_lmhead_ce_fwd(x, w, y, 0, vs)
    with pytest.raises(ValueError, match="GPU tensor"):
        vp.vp_embed_fwd(y, w, 0, vs)
    with pytest.raises(TypeError):
        vp.vp_lmhead_ce_fwd(x.float(), w, y, 0, vs)
    with pytest.raises(TypeError):
        vp.vp_embed_fwd(y.int(), w, 0, vs)
    with pytest.raises(ValueError, match="workspace"):
        _lib._workspace(torch.zeros(64, dtype=torch.uint8), 64, "cpu")
    with pytest.raises(ValueError, match="one GPU"):
        _lib._same_device(x, torch.zeros(1, device="meta"))
    with pytest.raises(ValueError):
        _lib._shape(torch.zeros((n - 1, h)), (n, h), "dx")
