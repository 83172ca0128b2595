"""Host-side tests of the C ABI (no GPU): the library loads, exports every function the
header declares, and rejects bad arguments with the documented codes before touching a
device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

torch = pytest.importorskip("torch")
sv = pytest.importorskip("speculative_sampling_verify_03_amd")

if not os.path.exists(sv.LIB_PATH):
    pytest.skip("library not built", allow_module_level=True)


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"SV_API\s+[\w\s\*]+?\b(spec_\w+)\s*\(", text)


def header_codes():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"(SV_E_\w+|SV_OK)\s*=\s*(-?\d+)", text)}


def test_exports_match_header():
    lib = sv.library()
    fns = header_functions()
    assert set(fns) == set(sv.EXPORTS)
    for fn in fns:
        assert hasattr(lib, fn), fn


def test_error_codes_match_binding():
    codes = header_codes()
    for name, val in codes.items():
        assert sv._lib.ERRORS[val] == name
    for val in codes.values():
        assert sv.spec_verify_strerror(val)


def test_single_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch already loaded (same soname)."""
    sv.library()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_workspace_bytes():
    f = sv.spec_verify_workspace_bytes
    assert f(sv.SV_KIND_LINEAR, 64, 5, 32000) >= 64 * 4 + 64 * 6 * 8
    assert f(sv.SV_KIND_TREE, 16, 61, 128256) >= 16 * 4 + 16 * 61 * 8
    assert f(sv.SV_KIND_GREEDY, 256, 8, 128256) >= 256 * 4 + 256 * 9 * 8
    assert f(sv.SV_KIND_LINEAR, 1, 64, 100) == 0      # k + 1 > 64
    assert f(sv.SV_KIND_TREE, 1, 65, 100) == 0        # N > 64
    assert f(sv.SV_KIND_LINEAR, -1, 4, 100) == 0
    assert f(99, 1, 4, 100) == 0
    assert f(sv.SV_KIND_LINEAR, 0, 4, 100) > 0        # empty call still has a valid layout


C = ctypes.c_void_p
FAKE = C(0x1000)    # never dereferenced: validation fails first
FAKE_WS = C(0x2000)


def linear(**kw):
    a = dict(logits=FAKE, lt=1, probs=FAKE, qt=1, tokens=FAKE, B=2, k=3, V=100, T=1.0, seed=0, off=0,
             out=FAKE, alen=FAKE, tp=None, ap=None, ws=FAKE_WS, wsb=1 << 20, stream=None)
    a.update(kw)
    return sv.library().spec_verify_linear(*a.values())


def test_linear_validation_codes():
    assert linear(logits=None) == -1
    assert linear(out=None) == -1
    assert linear(alen=None) == -1
    assert linear(probs=None) == -1
    assert linear(k=0, probs=None, tokens=None, B=0) == 0       # empty call
    assert linear(B=-1) == -2
    assert linear(k=-1) == -2
    assert linear(k=64) == -2
    assert linear(V=0) == -2
    assert linear(lt=7) == -3
    assert linear(qt=-1) == -3
    assert linear(T=0.0) == -4
    assert linear(T=-1.0) == -4
    assert linear(T=float("nan")) == -4
    assert linear(T=float("inf")) == -4
    assert linear(ws=None) == -6
    assert linear(wsb=16) == -6
    assert linear(logits=C(0x1001)) == -9
    assert linear(lt=0, logits=C(0x1002)) == -9
    assert linear(B=0) == 0


def greedy(**kw):
    a = dict(logits=FAKE, lt=1, tokens=FAKE, B=2, k=3, V=100, out=FAKE, alen=FAKE, ws=FAKE_WS,
             wsb=1 << 20, stream=None)
    a.update(kw)
    return sv.library().spec_verify_greedy(*a.values())


def test_greedy_validation_codes():
    assert greedy(logits=None) == -1
    assert greedy(tokens=None) == -1
    assert greedy(k=0, tokens=None, B=0) == 0
    assert greedy(k=70) == -2
    assert greedy(lt=3) == -3
    assert greedy(wsb=8) == -6
    assert greedy(B=0) == 0


def tree(parents, **kw):
    par = (ctypes.c_int32 * len(parents))(*parents) if parents is not None else None
    a = dict(logits=FAKE, lt=1, probs=FAKE, qt=1, toks=FAKE, par=ctypes.cast(par, C) if par else None,
             B=2, N=len(parents) if parents else 3, V=100, T=1.0, seed=0, off=0, out=FAKE, alen=FAKE,
             path=None, ws=FAKE_WS, wsb=1 << 20, stream=None)
    a.update(kw)
    return sv.library().spec_verify_tree(*a.values())


def test_tree_validation_codes():
    assert tree([-1, 0, 0, 1], B=0) == 0
    assert tree(None, N=3) == -1
    assert tree([0, 0, 0]) == -5          # root must have parent -1
    assert tree([-1, 1, 0]) == -5         # parent must precede the child
    assert tree([-1, 0, 1, 0]) == -5      # parents must be non-decreasing (BFS order)
    assert tree([-1, -1]) == -5
    assert tree([-1] + [0] * 64) == -2    # N > 64
    assert tree([-1, 0], T=0.0) == -4
    assert tree([-1, 0], wsb=4) == -6


def tree_lossless(parents, **kw):
    par = (ctypes.c_int32 * len(parents))(*parents) if parents is not None else None
    a = dict(logits=FAKE, lt=1, toks=FAKE, par=ctypes.cast(par, C) if par else None,
             B=2, N=len(parents) if parents else 3, V=100, T=1.0, seed=0, off=0, out=FAKE, alen=FAKE,
             path=None, ws=FAKE_WS, wsb=1 << 20, stream=None)
    a.update(kw)
    return sv.library().spec_verify_tree_lossless(*a.values())


def test_tree_lossless_validation_codes():
    assert tree_lossless([-1, 0, 0, 1], B=0) == 0
    assert tree_lossless(None, N=3) == -1
    assert tree_lossless([-1, 0, 0], toks=None) == -1
    assert tree_lossless([-1], toks=None, wsb=1 << 20) != -1   # a root-only tree reads no tokens
    assert tree_lossless([-1, 1, 0]) == -5
    assert tree_lossless([-1, 0, 1, 0]) == -5
    assert tree_lossless([-1] + [0] * 64) == -2
    assert tree_lossless([-1, 0], lt=7) == -3
    assert tree_lossless([-1, 0], T=float("nan")) == -4
    assert tree_lossless([-1, 0], wsb=4) == -6
    assert tree_lossless([-1, 0], logits=C(0x1001)) == -9


def lmhead(**kw):
    a = dict(h=C(0x1000), w=FAKE, probs=FAKE, qt=1, toks=FAKE, B=2, k=3, H=128, V=100, T=1.0, seed=0,
             off=0, logits=FAKE, out=FAKE, alen=FAKE, tp=None, ap=None, ws=FAKE_WS, wsb=1 << 20, stream=None)
    a.update(kw)
    return sv.library().spec_lmhead_verify(*a.values())


def test_lmhead_validation_codes():
    assert lmhead(logits=None) == -1
    assert lmhead(h=None) == -1
    assert lmhead(H=100) == -2            # H must be a multiple of 64
    assert lmhead(H=0) == -2
    assert lmhead(h=C(0x1008)) == -9      # hidden must be 16-byte aligned
    assert lmhead(qt=5) == -3
    assert lmhead(T=0.0) == -4
    assert lmhead(B=0) == 0


def lmhead_logits(**kw):
    a = dict(h=C(0x1000), w=FAKE, M=12, H=128, V=100, logits=FAKE, stream=None)
    a.update(kw)
    return sv.library().spec_lmhead_logits(*a.values())


def test_lmhead_logits_validation_codes():
    assert lmhead_logits(M=0) == 0
    assert lmhead_logits(logits=None) == -1
    assert lmhead_logits(w=None) == -1
    assert lmhead_logits(H=96) == -2        # H must be a multiple of 64
    assert lmhead_logits(M=-1) == -2
    assert lmhead_logits(V=0) == -2
    assert lmhead_logits(h=C(0x1008)) == -9  # hidden must be 16-byte aligned
    assert lmhead_logits(logits=C(0x1002)) == -9


def plug(**kw):
    a = dict(toks=FAKE, alen=FAKE, B=2, W=6, seq=FAKE, hist=FAKE, cap=100, nxt=None, status=None, stream=None)
    a.update(kw)
    return sv.library().spec_plug_tokens(*a.values())


def test_plug_validation_codes():
    assert plug(B=0) == 0
    assert plug(toks=None) == -1
    assert plug(hist=None) == -1
    assert plug(seq=None) == -1
    assert plug(W=0) == -2
    assert plug(W=65) == -2
    assert plug(cap=0) == -2
    assert plug(B=-1) == -2
    assert plug(nxt=C(0x1002)) == -9      # int32 outputs must be 4-byte aligned


def lookup(**kw):
    a = dict(hist=FAKE, lens=FAKE, B=2, cap=100, mn=1, mx=3, k=5, drafts=FAKE, count=FAKE, stream=None)
    a.update(kw)
    return sv.library().spec_lookup_drafts(*a.values())


def test_lookup_validation_codes():
    assert lookup(B=0) == 0
    assert lookup(hist=None) == -1
    assert lookup(count=None) == -1
    assert lookup(mn=0) == -2
    assert lookup(mn=3, mx=2) == -2
    assert lookup(mx=17) == -2
    assert lookup(k=0) == -2
    assert lookup(k=65) == -2
    assert lookup(cap=0) == -2
    assert lookup(drafts=C(0x1001)) == -9


@pytest.mark.parametrize("fn", ["spec_verify_tree", "spec_verify_tree_lossless"])
@pytest.mark.parametrize("width", [1, 3, 5, 7])
def test_tree_binding_rejects_wrong_output_width(fn, width):
    """The tree kernels write B * (D + 1) entries with stride D + 1, D the tree's depth
    (3 here).  The binding derives D + 1 from the parent array and refuses buffers of any
    other width before anything reaches the library (CPU tensors never get that far)."""
    B, N, V = 2, 5, 16
    parents = [-1, 0, 0, 1, 3]  # depths 0, 1, 1, 2, 3
    lg = torch.zeros((B, N, V))
    toks = torch.zeros((B, N), dtype=torch.int32)
    out = torch.zeros((B, width), dtype=torch.int32)
    alen = torch.zeros((B,), dtype=torch.int32)
    args = (lg, lg, toks, parents) if fn == "spec_verify_tree" else (lg, toks, parents)
    with pytest.raises(ValueError, match="out_tokens must have shape"):
        getattr(sv, fn)(*args, 1.0, 0, 0, out, alen)
    good = torch.zeros((B, 4), dtype=torch.int32)
    bad_path = torch.zeros((B, width), dtype=torch.int32)
    with pytest.raises(ValueError, match="out_path must have shape"):
        getattr(sv, fn)(*args, 1.0, 0, 0, good, alen, bad_path)


def test_tree_binding_rejects_parent_count():
    lg = torch.zeros((1, 3, 8))
    with pytest.raises(ValueError, match="parents must have"):
        sv.spec_verify_tree_lossless(lg, torch.zeros((1, 3), dtype=torch.int32), [-1, 0], 1.0, 0, 0,
                                     torch.zeros((1, 2), dtype=torch.int32), torch.zeros(1, dtype=torch.int32))


def linear_noalloc(**kw):
    a = dict(logits=FAKE, lt=1, probs=FAKE, qt=1, tokens=FAKE, B=2, k=3, V=100, T=1.0, seed=0, off=0,
             out=FAKE, alen=FAKE, tp=None, ap=None, stream=None)
    a.update(kw)
    return sv.library().spec_verify_linear_noalloc(*a.values())


def test_linear_noalloc_validation_codes():
    """The allocation-free call refuses sizes beyond its 4 MiB static scratch before any
    device call, and otherwise validates like spec_verify_linear."""
    ws = sv.spec_verify_workspace_bytes
    assert ws(sv.SV_KIND_LINEAR, 100000, 5, 100) > (4 << 20)
    assert ws(sv.SV_KIND_LINEAR, 30000, 5, 100) < (4 << 20)
    assert linear_noalloc(B=100000, k=5) == -10
    assert linear_noalloc(B=8192, k=63, V=8) == -10
    assert linear_noalloc(B=0) == 0
    assert linear_noalloc(logits=None) == -1
    assert linear_noalloc(k=64) == -2
    assert linear_noalloc(lt=4) == -3
    assert linear_noalloc(T=0.0) == -4
    assert linear_noalloc(logits=C(0x1001)) == -9
    assert "scratch" in sv.spec_verify_strerror(-10)
