"""ctypes binding of libspecverify.so (the C ABI in include/spec_verify.h).

Argument marshalling only: every function takes torch tensors that already live on the
current HIP device, checks that their shapes and dtypes agree with one another, and
passes raw device pointers, sizes and the current stream to the library.  All the
arithmetic happens in the library's kernels.  A non-zero return code raises
SpecVerifyError.  The library must have been built (``__graft_entry__.build()`` or
``python -m speculative_sampling_verify_03_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_KIND_LINEAR, SV_KIND_GREEDY, SV_KIND_TREE, SV_KIND_LMHEAD = 0, 1, 2, 3
ERRORS = {
    0: "SV_OK", -1: "SV_E_NULL", -2: "SV_E_SHAPE", -3: "SV_E_DTYPE", -4: "SV_E_TEMP",
    -5: "SV_E_TREE", -6: "SV_E_WORKSPACE", -7: "SV_E_DEVICE", -8: "SV_E_LAUNCH", -9: "SV_E_ALIGN",
    -10: "SV_E_SCRATCH",
}
EXPORTS = ("spec_verify_linear", "spec_verify_linear_noalloc", "spec_verify_greedy", "spec_verify_tree", "spec_verify_tree_lossless",
           "spec_lmhead_verify", "spec_lmhead_logits",
           "spec_plug_tokens", "spec_lookup_drafts", "spec_verify_workspace_bytes", "spec_verify_strerror")


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib().spec_verify_strerror(code).decode()
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({msg})")


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        lib.spec_verify_linear.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int, _P, _I32, _I32, _I32, _F32,
                                           _U64, _U64, _P, _P, _P, _P, _P, _SZ, _P]
        lib.spec_verify_linear_noalloc.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int, _P, _I32, _I32, _I32,
                                                   _F32, _U64, _U64, _P, _P, _P, _P, _P]
        lib.spec_verify_greedy.argtypes = [_P, ctypes.c_int, _P, _I32, _I32, _I32, _P, _P, _P, _SZ, _P]
        lib.spec_verify_tree.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int, _P, _P, _I32, _I32, _I32, _F32,
                                         _U64, _U64, _P, _P, _P, _P, _SZ, _P]
        lib.spec_verify_tree_lossless.argtypes = [_P, ctypes.c_int, _P, _P, _I32, _I32, _I32, _F32,
                                                  _U64, _U64, _P, _P, _P, _P, _SZ, _P]
        lib.spec_lmhead_verify.argtypes = [_P, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _I32, _F32,
                                           _U64, _U64, _P, _P, _P, _P, _P, _P, _SZ, _P]
        lib.spec_lmhead_logits.argtypes = [_P, _P, _I32, _I32, _I32, _P, _P]
        lib.spec_plug_tokens.argtypes = [_P, _P, _I32, _I32, _P, _P, _I32, _P, _P, _P]
        lib.spec_lookup_drafts.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]
        for fn in ("spec_verify_linear", "spec_verify_linear_noalloc", "spec_verify_greedy", "spec_verify_tree", "spec_verify_tree_lossless",
                   "spec_lmhead_verify", "spec_lmhead_logits",
                   "spec_plug_tokens", "spec_lookup_drafts"):
            getattr(lib, fn).restype = ctypes.c_int
        lib.spec_verify_workspace_bytes.argtypes = [ctypes.c_int, _I32, _I32, _I32, _I32]
        lib.spec_verify_workspace_bytes.restype = _SZ
        lib.spec_verify_strerror.argtypes = [ctypes.c_int]
        lib.spec_verify_strerror.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _i32(t, shape, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be int32 with shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return _ptr(t)


def _f32(t, shape, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be float32 with shape {tuple(shape)}")
    return _ptr(t)


def _tree_width(parents, B, out_tokens, out_path):
    """D + 1 for a parent array (D = depth of its deepest node), checked against the
    output buffers: the kernels write exactly B * (D + 1) entries with that row stride."""
    depth = [0] * len(parents)
    for c in range(1, len(parents)):
        p = int(parents[c])
        if not 0 <= p < c:
            raise ValueError("parents must satisfy 0 <= parents[c] < c for c >= 1")
        depth[c] = depth[p] + 1
    W = max(depth) + 1 if depth else 1
    for name, t in (("out_tokens", out_tokens), ("out_path", out_path)):
        if t is not None and tuple(t.shape) != (B, W):
            raise ValueError(f"{name} must have shape {(B, W)} for this tree, got {tuple(t.shape)}")
    return W


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, where):
    if rc != 0:
        raise SpecVerifyError(rc, where)


def spec_verify_workspace_bytes(kind: int, B: int, k_or_N: int, V: int, H: int = 0) -> int:
    return int(_lib().spec_verify_workspace_bytes(kind, B, k_or_N, V, H))


def spec_verify_strerror(code: int) -> str:
    return _lib().spec_verify_strerror(code).decode()


def new_workspace(kind: int, B: int, k_or_N: int, V: int, H: int = 0, device=None) -> torch.Tensor:
    """Zero-filled workspace of the size the library asks for (reusable across calls on
    one stream)."""
    n = spec_verify_workspace_bytes(kind, B, k_or_N, V, H)
    if n == 0:
        raise ValueError("invalid sizes for a workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def spec_verify_linear(target_logits, draft_probs, draft_tokens, temperature, seed, offset,
                       out_tokens, out_accept_len, out_target_prob=None, out_accept_prob=None,
                       workspace=None, stream=None):
    """target_logits [B, k+1, V], draft_probs [B, k, V] (f32/bf16), draft_tokens int32 [B, k];
    outputs int32 [B, k+1] and [B], optional float32 [B, k] probabilities."""
    B, R, V = target_logits.shape
    k = R - 1
    if tuple(draft_probs.shape) != (B, k, V):
        raise ValueError("draft_probs must have shape [B, k, V]")
    rc = _lib().spec_verify_linear(
        _ptr(target_logits), _dt(target_logits), _ptr(draft_probs), _dt(draft_probs),
        _i32(draft_tokens, (B, k), "draft_tokens"), B, k, V, float(temperature), int(seed), int(offset),
        _i32(out_tokens, (B, R), "out_tokens"), _i32(out_accept_len, (B,), "out_accept_len"),
        _f32(out_target_prob, (B, k), "out_target_prob"), _f32(out_accept_prob, (B, k), "out_accept_prob"),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "spec_verify_linear")


def spec_verify_linear_noalloc(target_logits, draft_probs, draft_tokens, temperature, seed, offset,
                               out_tokens, out_accept_len, out_target_prob=None, out_accept_prob=None,
                               stream=None):
    """spec_verify_linear without a workspace (the library's static per-device scratch;
    calls that overlap on one device race)."""
    B, R, V = target_logits.shape
    k = R - 1
    if tuple(draft_probs.shape) != (B, k, V):
        raise ValueError("draft_probs must have shape [B, k, V]")
    rc = _lib().spec_verify_linear_noalloc(
        _ptr(target_logits), _dt(target_logits), _ptr(draft_probs), _dt(draft_probs),
        _i32(draft_tokens, (B, k), "draft_tokens"), B, k, V, float(temperature), int(seed), int(offset),
        _i32(out_tokens, (B, R), "out_tokens"), _i32(out_accept_len, (B,), "out_accept_len"),
        _f32(out_target_prob, (B, k), "out_target_prob"), _f32(out_accept_prob, (B, k), "out_accept_prob"),
        _stream(stream))
    _check(rc, "spec_verify_linear_noalloc")


def spec_verify_greedy(target_logits, draft_tokens, out_tokens, out_accept_len, workspace=None, stream=None):
    B, R, V = target_logits.shape
    k = R - 1
    rc = _lib().spec_verify_greedy(
        _ptr(target_logits), _dt(target_logits), _i32(draft_tokens, (B, k), "draft_tokens"), B, k, V,
        _i32(out_tokens, (B, R), "out_tokens"), _i32(out_accept_len, (B,), "out_accept_len"),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "spec_verify_greedy")


def spec_plug_tokens(out_tokens, out_accept_len, seq_len, history, next_token=None, status=None, stream=None):
    """out_tokens int32 [B, W], out_accept_len [B] (a verify call's outputs); seq_len int32
    [B] and history int32 [B, cap] are updated in place; next_token / status int32 [B]."""
    B, W = out_tokens.shape
    cap = history.shape[1] if history.dim() == 2 else 0
    rc = _lib().spec_plug_tokens(
        _i32(out_tokens, (B, W), "out_tokens"), _i32(out_accept_len, (B,), "out_accept_len"), B, W,
        _i32(seq_len, (B,), "seq_len"), _i32(history, (B, cap), "history"), cap,
        _i32(next_token, (B,), "next_token"), _i32(status, (B,), "status"), _stream(stream))
    _check(rc, "spec_plug_tokens")


def spec_lookup_drafts(history, seq_len, min_ngram, max_ngram, out_drafts, out_count, stream=None):
    """history int32 [B, cap], seq_len int32 [B]; out_drafts int32 [B, k], out_count [B]."""
    B, cap = history.shape
    k = out_drafts.shape[1]
    rc = _lib().spec_lookup_drafts(
        _i32(history, (B, cap), "history"), _i32(seq_len, (B,), "seq_len"), B, cap, int(min_ngram),
        int(max_ngram), k, _i32(out_drafts, (B, k), "out_drafts"), _i32(out_count, (B,), "out_count"),
        _stream(stream))
    _check(rc, "spec_lookup_drafts")


def spec_verify_tree(target_logits, draft_probs, node_tokens, parents, temperature, seed, offset,
                     out_tokens, out_accept_len, out_path=None, workspace=None, stream=None):
    """target_logits / draft_probs [B, N, V]; node_tokens int32 [B, N]; parents: host
    sequence of N ints (BFS order, parents[0] = -1); outputs [B, D+1], [B], [B, D+1]."""
    B, N, V = target_logits.shape
    if len(parents) != N:
        raise ValueError(f"parents must have N = {N} entries")
    par = (ctypes.c_int32 * N)(*[int(x) for x in parents])
    W = _tree_width(parents, B, out_tokens, out_path)
    rc = _lib().spec_verify_tree(
        _ptr(target_logits), _dt(target_logits), _ptr(draft_probs), _dt(draft_probs),
        _i32(node_tokens, (B, N), "node_tokens"), ctypes.cast(par, ctypes.c_void_p), B, N, V,
        float(temperature), int(seed), int(offset), _i32(out_tokens, (B, W), "out_tokens"),
        _i32(out_accept_len, (B,), "out_accept_len"), _i32(out_path, (B, W), "out_path"),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "spec_verify_tree")


def spec_verify_tree_lossless(target_logits, node_tokens, parents, temperature, seed, offset,
                              out_tokens, out_accept_len, out_path=None, workspace=None, stream=None):
    """target_logits [B, N, V]; node_tokens int32 [B, N]; parents: host sequence of N ints
    (BFS order, parents[0] = -1); outputs [B, D+1], [B], [B, D+1].  No draft
    probabilities: each node's token is a fixed top-K candidate."""
    B, N, V = target_logits.shape
    if len(parents) != N:
        raise ValueError(f"parents must have N = {N} entries")
    par = (ctypes.c_int32 * N)(*[int(x) for x in parents])
    W = _tree_width(parents, B, out_tokens, out_path)
    rc = _lib().spec_verify_tree_lossless(
        _ptr(target_logits), _dt(target_logits), _i32(node_tokens, (B, N), "node_tokens"),
        ctypes.cast(par, ctypes.c_void_p), B, N, V, float(temperature), int(seed), int(offset),
        _i32(out_tokens, (B, W), "out_tokens"), _i32(out_accept_len, (B,), "out_accept_len"),
        _i32(out_path, (B, W), "out_path"),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "spec_verify_tree_lossless")


def spec_lmhead_verify(hidden, lm_head, draft_probs, draft_tokens, temperature, seed, offset, logits_out,
                       out_tokens, out_accept_len, out_target_prob=None, out_accept_prob=None,
                       workspace=None, stream=None):
    """hidden bf16 [B, k+1, H]; lm_head bf16 [H, V]; logits_out float32 [B, k+1, V]."""
    B, R, H = hidden.shape
    k = R - 1
    V = lm_head.shape[1]
    if hidden.dtype != torch.bfloat16 or lm_head.dtype != torch.bfloat16 or lm_head.shape[0] != H:
        raise ValueError("hidden [B, k+1, H] and lm_head [H, V] must be bfloat16")
    rc = _lib().spec_lmhead_verify(
        _ptr(hidden), _ptr(lm_head), _ptr(draft_probs), _dt(draft_probs),
        _i32(draft_tokens, (B, k), "draft_tokens"), B, k, H, V, float(temperature), int(seed), int(offset),
        _f32(logits_out, (B, R, V), "logits_out"), _i32(out_tokens, (B, R), "out_tokens"),
        _i32(out_accept_len, (B,), "out_accept_len"), _f32(out_target_prob, (B, k), "out_target_prob"),
        _f32(out_accept_prob, (B, k), "out_accept_prob"),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "spec_lmhead_verify")


def spec_lmhead_logits(hidden, lm_head, logits_out, stream=None):
    """hidden bf16 [..., H] (M rows); lm_head bf16 [H, V]; logits_out float32 [..., V] with the
    same leading shape: logits_out = hidden @ lm_head (the first stage of spec_lmhead_verify)."""
    H = hidden.shape[-1]
    V = lm_head.shape[1]
    M = hidden.numel() // H if H else 0
    if hidden.dtype != torch.bfloat16 or lm_head.dtype != torch.bfloat16 or lm_head.shape[0] != H:
        raise ValueError("hidden [..., H] and lm_head [H, V] must be bfloat16")
    if not hidden.is_contiguous() or not lm_head.is_contiguous():
        raise ValueError("hidden and lm_head must be contiguous")
    rc = _lib().spec_lmhead_logits(_ptr(hidden), _ptr(lm_head), M, H, V,
                                   _f32(logits_out, tuple(hidden.shape[:-1]) + (V,), "logits_out"), _stream(stream))
    _check(rc, "spec_lmhead_logits")
