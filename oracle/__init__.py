"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports this package.

Inputs are host numpy arrays: bf16 tensors as uint16 bit patterns (see
``top_chunk_sparse_amd.synth.bf16_bits``), page tables / indices as int32, S as float32.
Outputs are float64 (and int32 for indices).
"""
import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TCS_ORACLE_LIB: another build of oracle.c (the sanitizer test runs the pins against one)
_SO = os.environ.get("TCS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math: IEEE double arithmetic)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", "-Wall",
                               "-o", tmp, os.path.join(_HERE, "oracle.c"), "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _DecodeShape(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("B", "Hq", "Hkv", "d", "N", "C", "g", "k", "gate",
                                       "gists_in_softmax", "levels", "J", "k2", "max_chunks",
                                       "num_pages", "gist_cap")] + [("scale", C.c_double),
                                                                    ("top_p", C.c_double),
                                                                    ("head_select", C.c_int),
                                                                    ("adaptive_k", C.c_int)]


_P = C.c_void_p


class _DecodeIO(C.Structure):
    _fields_ = [("q", _P), ("k_pages", _P), ("v_pages", _P), ("page_table", _P),
                ("gist_k", _P), ("gist_v", _P), ("gist2_k", _P), ("gist2_v", _P),
                ("forced_sel", _P), ("forced_groups", _P), ("units", _P), ("n_units", C.c_int),
                ("out", _P), ("lse", _P), ("sel", _P), ("sel_groups", _P),
                ("chunk_scores", _P), ("group_scores", _P), ("weights", _P),
                ("weights_cap", C.c_int), ("n_tokens", _P)]


class _PrefillShape(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("B", "Hq", "Hkv", "d", "T", "blk", "k", "gate")] + \
               [("scale", C.c_double)]


class _GistPrefillShape(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("B", "Hq", "Hkv", "d", "M", "L", "g")] + \
               [("scale", C.c_double)]


class _GistPrefillIO(C.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("rows", _P), ("n_rows", C.c_int),
                ("out", _P), ("lse", _P)]


class _PrefillBwdIO(C.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("S", _P), ("dout", _P), ("dlse", _P),
                ("forced_sel", _P), ("dq", _P), ("dk", _P), ("dv", _P), ("dS", _P),
                ("n_blocks", C.c_int)]


class _PrefillIO(C.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("S", _P), ("forced_sel", _P),
                ("blocks", _P), ("n_blocks", C.c_int), ("out", _P), ("lse", _P), ("sel", _P)]


_lib = None


def _open(path):
    h = C.CDLL(path)
    h.or_decode.argtypes = [C.POINTER(_DecodeShape), C.POINTER(_DecodeIO)]
    h.or_prefill.argtypes = [C.POINTER(_PrefillShape), C.POINTER(_PrefillIO)]
    h.or_prefill_backward.argtypes = [C.POINTER(_PrefillShape), C.POINTER(_PrefillBwdIO)]
    h.or_gist_prefill.argtypes = [C.POINTER(_GistPrefillShape), C.POINTER(_GistPrefillIO)]
    h.or_decode_token_count.argtypes = [C.POINTER(_DecodeShape), C.c_int, C.c_int, C.c_int]
    h.or_adaptive_k.argtypes = [C.POINTER(_DecodeShape)]
    return h


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _open(_SO)
    return _lib


def swap_library(path):
    """Route every later call to the oracle built at ``path`` (None: the default build).
    Returns the previous handle.  Used by the mutation test to run the pins against
    deliberately broken copies of oracle.c."""
    global _lib
    prev = _lib
    _lib = None if path is None else _open(path)
    return prev


def threads() -> int:
    return int(lib().or_threads())


def _ptr(a: Optional[np.ndarray], dtype=None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a.ctypes.data


@dataclass
class DecodeResult:
    out: np.ndarray            # float64 [B][Hq][d]
    lse: np.ndarray            # float64 [B][Hq]
    sel: np.ndarray            # int32 [B][Hkv][k]
    sel_groups: Optional[np.ndarray]
    chunk_scores: np.ndarray   # float64 [B][Hkv][M-1]
    group_scores: Optional[np.ndarray]
    weights: Optional[np.ndarray]
    n_tokens: np.ndarray       # int32 [B][Hq]


def _gist_mode(x) -> int:
    """True/"all": every scored gist; False/"none": raw tokens only; "selected": the gists of the
    selected chunks only and, at two levels, the meta-gists of the selected groups
    ("Simplified Sparse Attention via Gist Tokens", sections 3.3 and B.2)."""
    if isinstance(x, str):
        return {"none": 0, "all": 1, "selected": 2}[x]
    return int(bool(x))


def decode(*, B, Hq, Hkv, d, N, C_, g, k, q, k_pages, v_pages, page_table, gist_k, gist_v,
           gate=0, levels=1, J=0, k2=0, gist2_k=None, gist2_v=None, scale=0.0,
           gists_in_softmax=True, gist_cap=0, forced_sel=None, forced_groups=None,
           units=None, weights_cap=0, top_p=0.0, head_select=0, adaptive_k=0) -> DecodeResult:
    """Decode attention for every (b, kv) (or the flat ids in ``units``).  head_select = 1:
    per-head selection with the union unfolded; sel then holds G * k entries per unit and
    chunk_scores one row per query head.  adaptive_k = 1: each level selects
    min(cap, adaptive_k_budget(...)) with caps k (chunks) and k2 (groups)."""
    M = -(-N // C_)
    H = M - 1
    nG = -(-H // J) if levels == 2 else 0
    u16 = np.uint16
    sh = _DecodeShape(B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, C=C_, g=g, k=k, gate=gate,
                      gists_in_softmax=_gist_mode(gists_in_softmax), levels=levels, J=J, k2=k2,
                      max_chunks=page_table.shape[-1], num_pages=k_pages.shape[0],
                      gist_cap=gist_cap, scale=scale, top_p=top_p, head_select=head_select,
                      adaptive_k=adaptive_k)
    G = Hq // Hkv
    sk = G * k if head_select else k
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    sel = np.full((B, Hkv, max(sk, 1)), -7, np.int32)
    selg = np.full((B, Hkv, max(k2, 1)), -7, np.int32) if levels == 2 else None
    cs = np.full((B, Hq if head_select else Hkv, max(H, 1)), np.nan)
    gs = np.full((B, Hkv, max(nG, 1)), np.nan) if levels == 2 else None
    w = np.zeros((B, Hq, weights_cap)) if weights_cap else None
    nt = np.zeros((B, Hq), np.int32)
    u = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    io = _DecodeIO(q=_ptr(q, u16), k_pages=_ptr(k_pages, u16), v_pages=_ptr(v_pages, u16),
                   page_table=_ptr(page_table, np.int32), gist_k=_ptr(gist_k, u16),
                   gist_v=_ptr(gist_v, u16), gist2_k=_ptr(gist2_k, u16), gist2_v=_ptr(gist2_v, u16),
                   forced_sel=_ptr(forced_sel, np.int32), forced_groups=_ptr(forced_groups, np.int32),
                   units=_ptr(u), n_units=0 if u is None else len(u),
                   out=_ptr(out), lse=_ptr(lse), sel=_ptr(sel), sel_groups=_ptr(selg),
                   chunk_scores=_ptr(cs), group_scores=_ptr(gs), weights=_ptr(w),
                   weights_cap=weights_cap, n_tokens=_ptr(nt))
    rc = lib().or_decode(C.byref(sh), C.byref(io))
    if rc:
        raise ValueError(f"oracle decode rejected the arguments (code {rc})")
    return DecodeResult(out, lse, sel[..., :sk], None if selg is None else selg[..., :k2],
                        cs[..., :H], gs, w, nt)


def adaptive_k_budget(*, N, C_, Hq, Hkv, levels=1, J=0) -> int:
    """Per-level selection budget of adaptive top-k (SSA appendix A; the reading is stated
    in oracle.c at or_adaptive_k)."""
    sh = _DecodeShape(N=N, C=C_, Hq=Hq, Hkv=Hkv, levels=levels, J=J)
    return int(lib().or_adaptive_k(C.byref(sh)))


def token_count(*, N, C_, g, k_eff, levels=1, J=0, n_cand=0, k2_eff=0, gists_in_softmax=True) -> int:
    sh = _DecodeShape(N=N, C=C_, g=g, levels=levels, J=J, gists_in_softmax=_gist_mode(gists_in_softmax))
    return int(lib().or_decode_token_count(C.byref(sh), k_eff, n_cand, k2_eff))


@dataclass
class PrefillResult:
    out: np.ndarray   # float64 [B][Hq][T][d] (NaN where not computed)
    lse: np.ndarray   # float64 [B][Hq][T]
    sel: np.ndarray   # int32 [B][Hkv][nb][k]


def prefill(*, B, Hq, Hkv, d, T, blk, k, gate, q, k_, v, S, scale=0.0, forced_sel=None,
            blocks=None) -> PrefillResult:
    nb = T // blk
    u16 = np.uint16
    sh = _PrefillShape(B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, blk=blk, k=k, gate=gate, scale=scale)
    out = np.full((B, Hq, T, d), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    sel = np.full((B, Hkv, nb, max(k, 1)), -7, np.int32)
    bl = None if blocks is None else np.ascontiguousarray(blocks, dtype=np.int32)
    io = _PrefillIO(q=_ptr(q, u16), k=_ptr(k_, u16), v=_ptr(v, u16), S=_ptr(S, np.float32),
                    forced_sel=_ptr(forced_sel, np.int32), blocks=_ptr(bl),
                    n_blocks=0 if bl is None else len(bl), out=_ptr(out), lse=_ptr(lse),
                    sel=_ptr(sel))
    rc = lib().or_prefill(C.byref(sh), C.byref(io))
    if rc:
        raise ValueError(f"oracle prefill rejected the arguments (code {rc})")
    return PrefillResult(out, lse, sel[..., :k])


@dataclass
class PrefillGrads:
    dq: np.ndarray    # float64 [B][Hq][T][d]
    dk: np.ndarray    # float64 [B][Hkv][T][d]
    dv: np.ndarray    # float64 [B][Hkv][T][d]
    dS: np.ndarray    # float64 [B][Hkv][nb][nb]


def prefill_backward(*, B, Hq, Hkv, d, T, blk, k, gate, q, k_, v, S, dout, dlse=None, scale=0.0,
                     forced_sel=None, n_blocks=0) -> PrefillGrads:
    """Gradients of L = sum dout . out + sum dlse . lse of the block-sparse causal prefill with
    respect to q, k, v and the selector scores S (bf16 inputs as uint16 bit patterns).
    n_blocks > 0 limits the work to query blocks i < n_blocks of each unit (timing samples)."""
    nb = T // blk
    u16 = np.uint16
    sh = _PrefillShape(B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, blk=blk, k=k, gate=gate, scale=scale)
    dq = np.full((B, Hq, T, d), np.nan)
    dk = np.full((B, Hkv, T, d), np.nan)
    dv = np.full((B, Hkv, T, d), np.nan)
    dS = np.full((B, Hkv, nb, nb), np.nan)
    io = _PrefillBwdIO(q=_ptr(q, u16), k=_ptr(k_, u16), v=_ptr(v, u16), S=_ptr(S, np.float32),
                       dout=_ptr(dout, u16), dlse=_ptr(dlse, np.float32),
                       forced_sel=_ptr(forced_sel, np.int32), dq=_ptr(dq), dk=_ptr(dk),
                       dv=_ptr(dv), dS=_ptr(dS), n_blocks=n_blocks)
    rc = lib().or_prefill_backward(C.byref(sh), C.byref(io))
    if rc:
        raise ValueError(f"oracle prefill backward rejected the arguments (code {rc})")
    return PrefillGrads(dq, dk, dv, dS)


def gist_prefill(*, B, Hq, Hkv, d, M, L, g, q, k_, v, scale=0.0, rows=None):
    """SSA gist-masked prefill over the interleaved sequence (M chunks of L raw tokens, each
    followed by its g gist tokens).  Returns (out [B][Hq][T'][d], lse [B][Hq][T']) in float64,
    NaN where a row was not computed (``rows``: flat ids (b * Hq + h) * T' + p)."""
    Tp = M * (L + g)
    u16 = np.uint16
    sh = _GistPrefillShape(B=B, Hq=Hq, Hkv=Hkv, d=d, M=M, L=L, g=g, scale=scale)
    out = np.full((B, Hq, Tp, d), np.nan)
    lse = np.full((B, Hq, Tp), np.nan)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    io = _GistPrefillIO(q=_ptr(q, u16), k=_ptr(k_, u16), v=_ptr(v, u16), rows=_ptr(r),
                        n_rows=0 if r is None else len(r), out=_ptr(out), lse=_ptr(lse))
    rc = lib().or_gist_prefill(C.byref(sh), C.byref(io))
    if rc:
        raise ValueError(f"oracle gist prefill rejected the arguments (code {rc})")
    return out, lse
