"""Python binding of libtcsparse.so (ctypes).  Argument marshalling only: torch supplies
device memory (``data_ptr``) and the stream; every step of the computation runs in the HIP
kernels behind the C ABI (include/tcsparse.h).  If the library is missing or fails to load,
every call raises: there is no fallback implementation.
"""
import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TCS_LIB_PATH") or os.path.join(_HERE, "libtcsparse.so")

(TCS_OK, TCS_ERR_NULL, TCS_ERR_SHAPE, TCS_ERR_UNSUPPORTED, TCS_ERR_WORKSPACE, TCS_ERR_HIP,
 TCS_ERR_TOO_LARGE) = range(7)
NOALLOC_SCRATCH_BYTES = 16 << 20   # TCS_NOALLOC_SCRATCH_BYTES
GATE_NONE, GATE_SAS = 0, 1


class TcsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"tcsparse error {code}: {msg}")
        self.code = code


class DecodeParams(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("struct_size", "B", "Hq", "Hkv", "d", "N", "C", "g",
                                         "k", "gate_mode", "gist_mode", "levels", "J", "k2",
                                         "max_chunks",
                                         "num_pages", "gist_cap")] + [("scale", C.c_float),
                                                                      ("top_p", C.c_float),
                                                                      ("select_mode", C.c_int32),
                                                                      ("k_mode", C.c_int32)]


class GistPrefillParams(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("struct_size", "B", "Hq", "Hkv", "d", "M", "L",
                                         "g")] + [("scale", C.c_float)]


class PrefillParams(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("struct_size", "B", "Hq", "Hkv", "d", "T", "blk", "k",
                                         "gate_mode")] + [("scale", C.c_float)]


_V = C.c_void_p
_lib = None

EXPORTS = ("tcs_abi_version", "tcs_status_str", "tcs_decode_workspace_size", "sparse_attn_decode",
           "sparse_attn_decode_timed", "tcs_decode_stage_count", "tcs_workspace_init",
           "tcs_prefill_workspace_size", "sparse_attn_prefill", "sparse_attn_prefill_timed",
           "tcs_prefill_backward_workspace_size", "sparse_attn_prefill_backward",
           "sparse_attn_prefill_backward_timed", "tcs_gist_prefill_workspace_size",
           "sparse_attn_gist_prefill", "sparse_attn_gist_prefill_timed", "tcs_stream_read",
           "sparse_attn_decode_noalloc")


def lib():
    """Load libtcsparse.so (after torch, so it binds to the HIP runtime torch loaded)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m top_chunk_sparse_amd.build`")
        h = C.CDLL(LIB_PATH)
        h.tcs_abi_version.restype = C.c_int
        h.tcs_status_str.restype = C.c_char_p
        h.tcs_status_str.argtypes = [C.c_int]
        h.tcs_decode_workspace_size.argtypes = [C.POINTER(DecodeParams), C.POINTER(C.c_size_t)]
        h.sparse_attn_decode.argtypes = [C.POINTER(DecodeParams)] + [_V] * 14 + [C.c_size_t, _V]
        h.tcs_prefill_workspace_size.argtypes = [C.POINTER(PrefillParams), C.POINTER(C.c_size_t)]
        h.sparse_attn_prefill.argtypes = [C.POINTER(PrefillParams)] + [_V] * 8 + [C.c_size_t, _V]
        h.sparse_attn_decode_timed.argtypes = h.sparse_attn_decode.argtypes + [_V, C.c_int]
        h.sparse_attn_prefill_timed.argtypes = h.sparse_attn_prefill.argtypes + [_V, C.c_int]
        h.tcs_gist_prefill_workspace_size.argtypes = [C.POINTER(GistPrefillParams),
                                                      C.POINTER(C.c_size_t)]
        h.sparse_attn_gist_prefill.argtypes = ([C.POINTER(GistPrefillParams)] + [_V] * 6 +
                                               [C.c_size_t, _V])
        h.sparse_attn_gist_prefill_timed.argtypes = (h.sparse_attn_gist_prefill.argtypes +
                                                     [_V, C.c_int])
        h.tcs_prefill_backward_workspace_size.argtypes = [C.POINTER(PrefillParams),
                                                          C.POINTER(C.c_size_t)]
        h.sparse_attn_prefill_backward.argtypes = ([C.POINTER(PrefillParams)] + [_V] * 13 +
                                                   [C.c_size_t, _V])
        h.sparse_attn_prefill_backward_timed.argtypes = (h.sparse_attn_prefill_backward.argtypes +
                                                         [_V, C.c_int])
        h.tcs_decode_stage_count.argtypes = [C.POINTER(DecodeParams)]
        h.tcs_workspace_init.argtypes = [_V, C.c_size_t, _V]
        h.tcs_stream_read.argtypes = [_V, C.c_size_t, _V, _V]
        h.sparse_attn_decode_noalloc.argtypes = [C.POINTER(DecodeParams)] + [_V] * 14
        _lib = h
    return _lib


STREAM_READ_BLOCKS = 4096   # TCS_STREAM_READ_BLOCKS


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue a plain streaming read of ``src`` (the HBM read ceiling; measurement only)."""
    assert sink.numel() * sink.element_size() >= 4 * STREAM_READ_BLOCKS
    _check(lib().tcs_stream_read(_p(src), src.numel() * src.element_size(), _p(sink),
                                 _stream_handle(stream, src)))


def status_str(code: int) -> str:
    return lib().tcs_status_str(code).decode()


def _check(code):
    if code != TCS_OK:
        raise TcsError(code, status_str(code))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream_handle(stream, like: torch.Tensor) -> int:
    """The raw hipStream_t of ``stream``, or of torch's current stream on ``like``'s device (read
    without building a Stream object: this lookup is most of a call's host time otherwise)."""
    if stream is not None:
        return stream.cuda_stream
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is None:
        return torch.cuda.current_stream(like.device).cuda_stream
    idx = like.device.index
    return get(idx if idx is not None else torch.cuda.current_device())


GISTS_ALL, GISTS_SELECTED = 0, 1   # TCS_GISTS_*
SELECT_KV_HEAD, SELECT_PER_HEAD = 0, 1   # TCS_SELECT_*
K_FIXED, K_ADAPTIVE = 0, 1   # TCS_K_*


def decode_params(*, B, Hq, Hkv, d, N, C_, g, k, gate=0, levels=1, J=0, k2=0, max_chunks=None,
                  num_pages, gist_cap=0, scale=0.0, gist_mode=GISTS_ALL,
                  top_p=0.0, select_mode=SELECT_KV_HEAD, k_mode=K_FIXED) -> DecodeParams:
    M = -(-N // C_) if C_ > 0 else 1
    return DecodeParams(struct_size=C.sizeof(DecodeParams), B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, C=C_,
                        g=g, k=k, gate_mode=gate, gist_mode=gist_mode, levels=levels, J=J, k2=k2,
                        max_chunks=M if max_chunks is None else max_chunks,
                        num_pages=num_pages, gist_cap=gist_cap, scale=scale, top_p=top_p,
                        select_mode=select_mode, k_mode=k_mode)


def decode_workspace_size(p: DecodeParams) -> int:
    n = C.c_size_t(0)
    _check(lib().tcs_decode_workspace_size(C.byref(p), C.byref(n)))
    return n.value


def sparse_attn_decode(p: DecodeParams, q, k_pages, v_pages, page_table, gist_k, gist_v,
                       gist2_k=None, gist2_v=None, *, out, lse=None, sel=None, sel_groups=None,
                       chunk_scores=None, workspace, stream=None, events=None) -> None:
    """Enqueue one decode call on ``stream`` (default: torch's current stream).  ``events``:
    optional ctypes array of raw hipEvent_t handles for the per-kernel timing variant."""
    args = (C.byref(p), _p(q), _p(k_pages), _p(v_pages), _p(page_table), _p(gist_k), _p(gist_v),
            _p(gist2_k), _p(gist2_v), _p(out), _p(lse), _p(sel), _p(sel_groups), _p(chunk_scores),
            _p(workspace),
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            _stream_handle(stream, out))
    if events is None:
        code = lib().sparse_attn_decode(*args)
    else:
        code = lib().sparse_attn_decode_timed(*args, C.cast(events, _V), len(events))
    _check(code)


def sparse_attn_decode_noalloc(p: DecodeParams, q, k_pages, v_pages, page_table, gist_k,
                               gist_v, gist2_k=None, gist2_v=None, *, out, lse=None, sel=None,
                               sel_groups=None, chunk_scores=None, stream=None) -> None:
    """sparse_attn_decode without a workspace: the library's static per-GPU scratch serves
    instead (for callers that cannot allocate)."""
    _check(lib().sparse_attn_decode_noalloc(
        C.byref(p), _p(q), _p(k_pages), _p(v_pages), _p(page_table), _p(gist_k), _p(gist_v),
        _p(gist2_k), _p(gist2_v), _p(out), _p(lse), _p(sel), _p(sel_groups), _p(chunk_scores),
        _stream_handle(stream, out)))


def decode_stage_count(p: DecodeParams) -> int:
    return int(lib().tcs_decode_stage_count(C.byref(p)))


def prefill_params(*, B, Hq, Hkv, d, T, blk, k, gate=1, scale=0.0) -> PrefillParams:
    return PrefillParams(struct_size=C.sizeof(PrefillParams), B=B, Hq=Hq, Hkv=Hkv, d=d, T=T,
                         blk=blk, k=k, gate_mode=gate, scale=scale)


def prefill_workspace_size(p: PrefillParams) -> int:
    n = C.c_size_t(0)
    _check(lib().tcs_prefill_workspace_size(C.byref(p), C.byref(n)))
    return n.value


def sparse_attn_prefill(p: PrefillParams, q, k, v, S, *, out, lse=None, sel=None, workspace,
                        stream=None, events=None) -> None:
    args = (C.byref(p), _p(q), _p(k), _p(v), _p(S), _p(out), _p(lse), _p(sel), _p(workspace),
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            _stream_handle(stream, out))
    if events is None:
        code = lib().sparse_attn_prefill(*args)
    else:
        code = lib().sparse_attn_prefill_timed(*args, C.cast(events, _V), len(events))
    _check(code)


def prefill_backward_workspace_size(p: PrefillParams) -> int:
    n = C.c_size_t(0)
    _check(lib().tcs_prefill_backward_workspace_size(C.byref(p), C.byref(n)))
    return n.value


def sparse_attn_prefill_backward(p: PrefillParams, q, k, v, S, out, lse, dout, dlse=None, *,
                                 dq, dk, dv, dS=None, workspace, stream=None,
                                 events=None) -> None:
    """Enqueue the prefill gradients on ``stream`` (default: torch's current stream)."""
    args = (C.byref(p), _p(q), _p(k), _p(v), _p(S), _p(out), _p(lse), _p(dout), _p(dlse),
            _p(dq), _p(dk), _p(dv), _p(dS), _p(workspace),
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            _stream_handle(stream, dq))
    if events is None:
        code = lib().sparse_attn_prefill_backward(*args)
    else:
        code = lib().sparse_attn_prefill_backward_timed(*args, C.cast(events, _V), len(events))
    _check(code)


def gist_prefill_params(*, B, Hq, Hkv, d, M, L, g, scale=0.0) -> GistPrefillParams:
    return GistPrefillParams(struct_size=C.sizeof(GistPrefillParams), B=B, Hq=Hq, Hkv=Hkv, d=d,
                             M=M, L=L, g=g, scale=scale)


def gist_prefill_workspace_size(p: GistPrefillParams) -> int:
    n = C.c_size_t(0)
    _check(lib().tcs_gist_prefill_workspace_size(C.byref(p), C.byref(n)))
    return n.value


def sparse_attn_gist_prefill(p: GistPrefillParams, q, k, v, *, out, lse=None, workspace,
                             stream=None, events=None) -> None:
    args = (C.byref(p), _p(q), _p(k), _p(v), _p(out), _p(lse), _p(workspace),
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            _stream_handle(stream, out))
    if events is None:
        code = lib().sparse_attn_gist_prefill(*args)
    else:
        code = lib().sparse_attn_gist_prefill_timed(*args, C.cast(events, _V), len(events))
    _check(code)


def workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """A caller-owned workspace (256-byte aligned by the torch allocator), zero-filled by the
    library's init kernel as a new decode workspace must be."""
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _check(lib().tcs_workspace_init(ws.data_ptr(), ws.numel(), _stream_handle(stream, ws)))
    return ws


# ---- convenience wrappers over the generator's input bundles ----------------------------
class DecodeCall:
    """Outputs and workspace for repeated decode calls on one input bundle."""

    def __init__(self, inp, with_scores=True, k=None, scale=0.0, gist_mode=GISTS_ALL,
                 top_p=0.0, head_select=0, adaptive_k=0):
        c = inp.cfg
        dev = inp.q.device
        self.inp = inp
        self.gist_mode = gist_mode
        self.head_select = head_select
        self.adaptive_k = adaptive_k
        self.p = decode_params(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, N=c.N, C_=c.C, g=c.g,
                               k=c.k if k is None else k, gate=c.gate, levels=c.levels, J=c.J,
                               k2=c.k2, max_chunks=inp.page_table.shape[1],
                               num_pages=inp.num_pages, gist_cap=inp.gist_k.shape[2],
                               scale=scale, gist_mode=gist_mode, top_p=top_p,
                               select_mode=SELECT_PER_HEAD if head_select else SELECT_KV_HEAD,
                               k_mode=K_ADAPTIVE if adaptive_k else K_FIXED)
        kk = self.p.k * (c.G if head_select else 1)   # sel entries per (b, kv)
        self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)
        self.sel = torch.empty((c.B, c.Hkv, max(kk, 1)), dtype=torch.int32, device=dev)[..., :kk]
        self.sel_groups = (torch.empty((c.B, c.Hkv, max(c.k2, 1)), dtype=torch.int32,
                                       device=dev)[..., :c.k2] if c.levels == 2 else None)
        self.chunk_scores = (torch.empty((c.B, c.Hq if head_select else c.Hkv, max(c.H, 1)),
                                         dtype=torch.float32, device=dev)
                             if with_scores else None)
        self.ws = workspace(decode_workspace_size(self.p), dev)

    def noalloc(self, stream=None):
        """The same call through the allocation-free entry point (no workspace)."""
        i = self.inp
        sparse_attn_decode_noalloc(self.p, i.q, i.k_pages, i.v_pages, i.page_table, i.gist_k,
                                   i.gist_v, i.gist2_k, i.gist2_v, out=self.out, lse=self.lse,
                                   sel=self.sel if self.p.k > 0 else None,
                                   sel_groups=self.sel_groups, chunk_scores=self.chunk_scores,
                                   stream=stream)
        return self

    def __call__(self, stream=None, events=None):
        i = self.inp
        sparse_attn_decode(self.p, i.q, i.k_pages, i.v_pages, i.page_table, i.gist_k, i.gist_v,
                           i.gist2_k, i.gist2_v, out=self.out, lse=self.lse,
                           sel=self.sel if self.p.k > 0 else None,
                           sel_groups=self.sel_groups, chunk_scores=self.chunk_scores,
                           workspace=self.ws, stream=stream, events=events)
        return self


class PrefillCall:
    def __init__(self, inp, k=None, scale=0.0):
        c = inp.cfg
        dev = inp.q.device
        self.inp = inp
        self.p = prefill_params(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk,
                                k=c.k if k is None else k, gate=c.gate, scale=scale)
        kk = self.p.k
        self.out = torch.empty((c.B, c.Hq, c.T, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq, c.T), dtype=torch.float32, device=dev)
        self.sel = torch.empty((c.B, c.Hkv, c.nb, max(kk, 1)), dtype=torch.int32,
                               device=dev)[..., :kk]
        self.ws = workspace(prefill_workspace_size(self.p), dev)

    def __call__(self, stream=None, events=None):
        i = self.inp
        sparse_attn_prefill(self.p, i.q, i.k, i.v, i.S, out=self.out, lse=self.lse,
                            sel=self.sel if self.p.k > 0 else None,
                            workspace=self.ws, stream=stream, events=events)
        return self


class PrefillBwdCall:
    """Gradient buffers and workspace for repeated backward calls on one input bundle; the
    forward's out and lse come from a finished PrefillCall on the same inputs."""

    def __init__(self, inp, fwd, dout, dlse=None, k=None, scale=0.0, with_dS=True):
        c = inp.cfg
        dev = inp.q.device
        self.inp, self.fwd, self.dout, self.dlse = inp, fwd, dout, dlse
        self.p = prefill_params(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk,
                                k=c.k if k is None else k, gate=c.gate, scale=scale)
        self.dq = torch.empty((c.B, c.Hq, c.T, c.d), dtype=torch.float32, device=dev)
        self.dk = torch.empty((c.B, c.Hkv, c.T, c.d), dtype=torch.float32, device=dev)
        self.dv = torch.empty((c.B, c.Hkv, c.T, c.d), dtype=torch.float32, device=dev)
        self.dS = (torch.empty((c.B, c.Hkv, c.nb, c.nb), dtype=torch.float32, device=dev)
                   if with_dS else None)
        self.ws = torch.empty(max(prefill_backward_workspace_size(self.p), 1), dtype=torch.uint8,
                              device=dev)

    def __call__(self, stream=None, events=None):
        i = self.inp
        sparse_attn_prefill_backward(self.p, i.q, i.k, i.v, i.S, self.fwd.out, self.fwd.lse,
                                     self.dout, self.dlse, dq=self.dq, dk=self.dk, dv=self.dv,
                                     dS=self.dS, workspace=self.ws, stream=stream, events=events)
        return self


class GistPrefillCall:
    """Outputs and workspace for repeated SSA gist-masked prefill calls on one input bundle."""

    def __init__(self, inp, scale=0.0):
        c = inp.cfg
        dev = inp.q.device
        self.inp = inp
        self.p = gist_prefill_params(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, M=c.M, L=c.L, g=c.g,
                                     scale=scale)
        self.out = torch.empty((c.B, c.Hq, c.Tp, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq, c.Tp), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(gist_prefill_workspace_size(self.p), 1), dtype=torch.uint8,
                              device=dev)

    def __call__(self, stream=None, events=None):
        i = self.inp
        sparse_attn_gist_prefill(self.p, i.q, i.k, i.v, out=self.out, lse=self.lse,
                                 workspace=self.ws, stream=stream, events=events)
        return self
