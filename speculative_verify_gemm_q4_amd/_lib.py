"""ctypes binding of ``libq4verify.so`` (see include/q4verify.h)."""
from __future__ import annotations

import ctypes
import functools
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq4verify.so")

GROUP = 64
MAX_ROWS = 16
MAX_ROWS_TILED = 32
LAYOUT_PLANAR = 0
LAYOUT_TILED16 = 1
KERNEL_PLANAR = 0
KERNEL_TILED_STREAM = 1
KERNEL_TILED_RESIDENT = 2
KERNEL_TILED_KSLICE = 3

OK, EINVAL, EALIGN, EOVERFLOW, EDEVICE, ELAUNCH, ESCRATCH = \
    0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 8 << 20


class Q4Error(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {q4_status_string(status)} ({status})")


class _Layout(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32),
                ("layout_id", ctypes.c_uint32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("group", ctypes.c_int64),
                ("total_bytes", ctypes.c_uint64),
                ("code_off", ctypes.c_uint64), ("code_bytes", ctypes.c_uint64),
                ("scale_off", ctypes.c_uint64),
                ("scale_bytes", ctypes.c_uint64),
                ("bias_off", ctypes.c_uint64), ("bias_bytes", ctypes.c_uint64),
                ("tile_rows", ctypes.c_uint32),
                ("record_groups", ctypes.c_uint32),
                ("record_bytes", ctypes.c_uint64)]


class _SampleParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("top_k", ctypes.c_int32), ("draft_k", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_uint32), ("block", ctypes.c_uint32),
                ("row_tiles", ctypes.c_uint32),
                ("tiles_per_wave", ctypes.c_uint32),
                ("k_splits", ctypes.c_uint32), ("lookahead", ctypes.c_uint32),
                ("kernel", ctypes.c_uint32), ("lds_bytes", ctypes.c_uint32),
                ("k_parts", ctypes.c_uint32), ("m_tiles", ctypes.c_uint32),
                ("workspace_bytes", ctypes.c_uint64),
                ("k_seq_parts", ctypes.c_uint32),
                ("layout_id", ctypes.c_uint32)]


_lib = None

_SIGNATURES = {
    "q4_pack_layout": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32,
                        ctypes.POINTER(_Layout)], ctypes.c_int),
    "q4_gemm_verify": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                        ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                        ctypes.c_void_p], ctypes.c_int),
    "q4_gemm_verify_tiled": ([ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_void_p], ctypes.c_int),
    "q4_gemm_verify_tiled_dot": ([ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p], ctypes.c_int),
    "q4_repack": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int64, ctypes.c_void_p], ctypes.c_int),
    "q4_dequant": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                    ctypes.c_int64, ctypes.c_void_p], ctypes.c_int),
    "q4_stream_read": ([ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                        ctypes.c_void_p], ctypes.c_int),
    "q4_stream_copy": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                        ctypes.c_void_p], ctypes.c_int),
    "q4_gemm_verify_plan": ([ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_uint32, ctypes.POINTER(_Plan)],
                            ctypes.c_int),
    "q4_gemm_verify_tiled_ws": ([ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_uint64, ctypes.c_void_p],
                                ctypes.c_int),
    "q4_gemm_verify_tiled_noalloc": ([ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p], ctypes.c_int),
    "q4_gemm_verify_tiled_ws_plan": ([ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.POINTER(_Plan)],
                                     ctypes.c_int),
    "q4_verify_sample_workspace": ([ctypes.c_int, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_uint64)],
                                   ctypes.c_int),
    "q4_verify_sample": ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                          ctypes.POINTER(_SampleParams)] +
                         [ctypes.c_void_p] * 12 +
                         [ctypes.c_uint64, ctypes.c_void_p], ctypes.c_int),
    "q4_gemm_verify_sample_workspace": ([ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64,
                                         ctypes.POINTER(ctypes.c_uint64)],
                                        ctypes.c_int),
    "q4_gemm_verify_sample": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_int64, ctypes.c_int64,
                               ctypes.POINTER(_SampleParams)] +
                              [ctypes.c_void_p] * 12 +
                              [ctypes.c_uint64, ctypes.c_void_p], ctypes.c_int),
    "q4_gdn_commit_lds_bytes": ([ctypes.c_int, ctypes.POINTER(ctypes.c_int)],
                                ctypes.c_int),
    "q4_gdn_commit": ([ctypes.c_void_p] + [ctypes.c_int] * 6 +
                      [ctypes.c_void_p] * 8, ctypes.c_int),
    "q4_gdn_tree_out": ([ctypes.c_void_p] + [ctypes.c_int] * 5 +
                        [ctypes.c_void_p] * 9, ctypes.c_int),
    "q4_tree_attn_plan": ([ctypes.c_int] * 4 + [ctypes.c_int64, ctypes.c_int,
                           ctypes.POINTER(ctypes.c_int),
                           ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "q4_tree_attn": ([ctypes.c_void_p] + [ctypes.c_int] * 4 +
                     [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_float,
                                              ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_uint64,
                                              ctypes.c_void_p, ctypes.c_void_p],
                     ctypes.c_int),
    "q4_status_string": ([ctypes.c_int], ctypes.c_char_p),
}


def lib_exports():
    """Names of the C entry points this binding uses."""
    return sorted(_SIGNATURES)


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def q4_status_string(status: int) -> str:
    return load().q4_status_string(int(status)).decode()


def q4_pack_layout(N: int, K: int, layout_id: int = LAYOUT_PLANAR) -> dict:
    out = _Layout()
    st = load().q4_pack_layout(int(N), int(K), int(layout_id),
                               ctypes.byref(out))
    if st != OK:
        raise Q4Error(st, f"q4_pack_layout({N}, {K}, {layout_id})")
    return {name: getattr(out, name) for name, _ in _Layout._fields_}


@functools.lru_cache(maxsize=256)
def _total_bytes(N: int, K: int, layout_id: int) -> int:
    return q4_pack_layout(N, K, layout_id)["total_bytes"]


def q4_gemm_verify_plan(M: int, N: int, K: int,
                        layout_id: int = LAYOUT_PLANAR) -> dict:
    """The launch plan q4_gemm_verify (layout 0) or q4_gemm_verify_tiled
    (layout 1) uses for this shape (host only)."""
    out = _Plan()
    st = load().q4_gemm_verify_plan(int(M), int(N), int(K), int(layout_id),
                                    ctypes.byref(out))
    if st != OK:
        raise Q4Error(st, f"q4_gemm_verify_plan({M}, {N}, {K}, {layout_id})")
    return {name: getattr(out, name) for name, _ in _Plan._fields_}


def q4_gemm_verify_tiled_ws_plan(M: int, N: int, K: int) -> dict:
    """The plan q4_gemm_verify_tiled_ws uses for this shape on the current
    device, with its ``workspace_bytes``."""
    out = _Plan()
    st = load().q4_gemm_verify_tiled_ws_plan(int(M), int(N), int(K),
                                             ctypes.byref(out))
    if st != OK:
        raise Q4Error(st, f"q4_gemm_verify_tiled_ws_plan({M}, {N}, {K})")
    return {name: getattr(out, name) for name, _ in _Plan._fields_}


def workspace_for(M: int, N: int, K: int, device):
    """A uint8 device tensor of the size q4_gemm_verify_tiled_ws needs for
    (M, N, K), or None when it needs none."""
    import torch
    n = q4_gemm_verify_tiled_ws_plan(M, N, K)["workspace_bytes"]
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t, name, dtype=None, numel=None, shape=None):
    """Device pointer of a contiguous CUDA tensor after checking it."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    return t.data_ptr()


def q4_gemm_verify(x, W, y, M: int, N: int, K: int, stream=None) -> None:
    """y[M, N] = x[M, K] @ W^T.  x bf16 [M, K], W packed uint8, y fp32
    [M, N]; all on the same GPU.  Enqueued on ``stream`` (default: torch's
    current stream)."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_PLANAR)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(W, "W", torch.uint8, numel=total)
    py = _ptr(y, "y", torch.float32, shape=(M, N))
    if not (x.device == W.device == y.device):
        raise ValueError("x, W and y must be on one device")
    st = load().q4_gemm_verify(px, pw, py, int(M), int(N), int(K),
                               _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify")


def q4_gemm_verify_tiled(x, Wt, y, M: int, N: int, K: int,
                         stream=None) -> None:
    """y[M, N] = x[M, K] @ W^T with W repacked by q4_repack."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(Wt, "Wt", torch.uint8, numel=total)
    py = _ptr(y, "y", torch.float32, shape=(M, N))
    if not (x.device == Wt.device == y.device):
        raise ValueError("x, Wt and y must be on one device")
    st = load().q4_gemm_verify_tiled(px, pw, py, int(M), int(N), int(K),
                                     _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify_tiled")


def q4_gemm_verify_tiled_dot(x, Wt, y, M: int, N: int, K: int,
                             stream=None) -> None:
    """q4_gemm_verify_tiled for M <= 4 with the dot products on the vector
    ALU (v_dot2_f32_bf16) instead of MFMA."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(Wt, "Wt", torch.uint8, numel=total)
    py = _ptr(y, "y", torch.float32, shape=(M, N))
    if not (x.device == Wt.device == y.device):
        raise ValueError("x, Wt and y must be on one device")
    st = load().q4_gemm_verify_tiled_dot(px, pw, py, int(M), int(N), int(K),
                                         _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify_tiled_dot")


def q4_gemm_verify_tiled_ws(x, Wt, y, M: int, N: int, K: int, ws=None,
                            stream=None) -> None:
    """q4_gemm_verify_tiled with a device workspace ``ws`` (uint8 tensor
    of at least the plan's workspace_bytes, or None when that is 0), which
    lets K > 5120 be split across workgroups."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(Wt, "Wt", torch.uint8, numel=total)
    py = _ptr(y, "y", torch.float32, shape=(M, N))
    if not (x.device == Wt.device == y.device):
        raise ValueError("x, Wt and y must be on one device")
    pws, nws = None, 0
    if ws is not None:
        pws = _ptr(ws, "ws", torch.uint8)
        nws = ws.numel()
        if ws.device != y.device:
            raise ValueError("ws must be on the device of y")
    st = load().q4_gemm_verify_tiled_ws(px, pw, py, int(M), int(N), int(K),
                                        pws, nws, _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify_tiled_ws")


def q4_gemm_verify_tiled_noalloc(x, Wt, y, M: int, N: int, K: int,
                                 stream=None) -> None:
    """q4_gemm_verify_tiled_ws with the library's static device scratch in
    place of a workspace: the call allocates nothing.  Calls that overlap on
    one GPU race (they share its scratch)."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(Wt, "Wt", torch.uint8, numel=total)
    py = _ptr(y, "y", torch.float32, shape=(M, N))
    if not (x.device == Wt.device == y.device):
        raise ValueError("x, Wt and y must be on one device")
    st = load().q4_gemm_verify_tiled_noalloc(px, pw, py, int(M), int(N),
                                             int(K), _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify_tiled_noalloc")


def q4_verify_sample_workspace(M: int, V: int) -> int:
    """Workspace bytes q4_verify_sample needs for M rows of V logits."""
    out = ctypes.c_uint64(0)
    st = load().q4_verify_sample_workspace(int(M), int(V), ctypes.byref(out))
    if st != OK:
        raise Q4Error(st, f"q4_verify_sample_workspace({M}, {V})")
    return out.value


def q4_verify_sample(logits, temperature: float, top_p: float, top_k: int,
                     draft_tok, draft_idx, draft_q, u, v, top_idx, top_val,
                     top_prob, greedy, accept, token, ws,
                     stream=None) -> None:
    """The verify sampling epilogue over logits [M, V] (fp32): top-k
    candidates, target probabilities, accept test and residual draw (see
    include/q4verify.h).  draft_idx / draft_q are [M, draft_k] (int32 /
    fp32) or None; u, v [M] fp32; outputs top_idx / top_val / top_prob
    [M, top_k], greedy / accept / token [M]; ws a uint8 device tensor of at
    least q4_verify_sample_workspace(M, V) bytes."""
    import torch
    M, V = logits.shape
    k = int(top_k)
    kd = 0 if draft_idx is None else int(draft_idx.shape[1])
    pl = _ptr(logits, "logits", torch.float32)
    pdt = _ptr(draft_tok, "draft_tok", torch.int32, numel=M)
    pdi = pdq = None
    if kd:
        pdi = _ptr(draft_idx, "draft_idx", torch.int32, shape=(M, kd))
        pdq = _ptr(draft_q, "draft_q", torch.float32, shape=(M, kd))
    pu = _ptr(u, "u", torch.float32, numel=M)
    pv = _ptr(v, "v", torch.float32, numel=M)
    pti = _ptr(top_idx, "top_idx", torch.int32, shape=(M, k))
    ptv = _ptr(top_val, "top_val", torch.float32, shape=(M, k))
    ptp = _ptr(top_prob, "top_prob", torch.float32, shape=(M, k))
    pg = _ptr(greedy, "greedy", torch.int32, numel=M)
    pa = _ptr(accept, "accept", torch.int32, numel=M)
    pt = _ptr(token, "token", torch.int32, numel=M)
    pws = _ptr(ws, "ws", torch.uint8)
    prm = _SampleParams(float(temperature), float(top_p), k, kd)
    st = load().q4_verify_sample(pl, int(M), int(V), ctypes.byref(prm), pdt,
                                 pdi, pdq, pu, pv, pti, ptv, ptp, pg, pa, pt,
                                 pws, ws.numel(), _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_verify_sample")


def verify_sample(logits, temperature: float, top_p: float, top_k: int,
                  draft_tok, draft_idx, draft_q, u, v, stream=None) -> dict:
    """q4_verify_sample with its outputs and workspace allocated here
    (torch tensors on the logits' device); returns the outputs by name."""
    import torch
    M, V = logits.shape
    dev = logits.device
    out = {"top_idx": torch.empty((M, top_k), dtype=torch.int32, device=dev),
           "top_val": torch.empty((M, top_k), dtype=torch.float32, device=dev),
           "top_prob": torch.empty((M, top_k), dtype=torch.float32,
                                   device=dev),
           "greedy": torch.empty(M, dtype=torch.int32, device=dev),
           "accept": torch.empty(M, dtype=torch.int32, device=dev),
           "token": torch.empty(M, dtype=torch.int32, device=dev)}
    ws = torch.empty(q4_verify_sample_workspace(M, V), dtype=torch.uint8,
                     device=dev)
    q4_verify_sample(logits, temperature, top_p, top_k, draft_tok, draft_idx,
                     draft_q, u, v, out["top_idx"], out["top_val"],
                     out["top_prob"], out["greedy"], out["accept"],
                     out["token"], ws, stream)
    return out


def q4_gemm_verify_sample_workspace(M: int, N: int, K: int) -> int:
    """Workspace bytes q4_gemm_verify_sample needs (current device)."""
    out = ctypes.c_uint64(0)
    st = load().q4_gemm_verify_sample_workspace(int(M), int(N), int(K),
                                                ctypes.byref(out))
    if st != OK:
        raise Q4Error(st, f"q4_gemm_verify_sample_workspace({M}, {N}, {K})")
    return out.value


def q4_gemm_verify_sample(x, Wt, M: int, N: int, K: int, temperature: float,
                          top_p: float, top_k: int, draft_tok, draft_idx,
                          draft_q, u, v, top_idx, top_val, top_prob, greedy,
                          accept, token, ws, stream=None) -> None:
    """The LM-head product x[M, K] @ W^T (W repacked by q4_repack, N the
    vocabulary) with the sampling epilogue fused in: the outputs of
    q4_verify_sample without writing the logits.  Same argument meanings as
    q4_verify_sample; ws a uint8 device tensor of at least
    q4_gemm_verify_sample_workspace(M, N, K) bytes."""
    import torch
    k = int(top_k)
    kd = 0 if draft_idx is None else int(draft_idx.shape[1])
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    px = _ptr(x, "x", torch.bfloat16, shape=(M, K))
    pw = _ptr(Wt, "Wt", torch.uint8, numel=total)
    pdt = _ptr(draft_tok, "draft_tok", torch.int32, numel=M)
    pdi = pdq = None
    if kd:
        pdi = _ptr(draft_idx, "draft_idx", torch.int32, shape=(M, kd))
        pdq = _ptr(draft_q, "draft_q", torch.float32, shape=(M, kd))
    pu = _ptr(u, "u", torch.float32, numel=M)
    pv = _ptr(v, "v", torch.float32, numel=M)
    pti = _ptr(top_idx, "top_idx", torch.int32, shape=(M, k))
    ptv = _ptr(top_val, "top_val", torch.float32, shape=(M, k))
    ptp = _ptr(top_prob, "top_prob", torch.float32, shape=(M, k))
    pg = _ptr(greedy, "greedy", torch.int32, numel=M)
    pa = _ptr(accept, "accept", torch.int32, numel=M)
    pt = _ptr(token, "token", torch.int32, numel=M)
    pws = _ptr(ws, "ws", torch.uint8)
    if not (x.device == Wt.device == ws.device):
        raise ValueError("x, Wt and ws must be on one device")
    prm = _SampleParams(float(temperature), float(top_p), k, kd)
    st = load().q4_gemm_verify_sample(px, pw, int(M), int(N), int(K),
                                      ctypes.byref(prm), pdt, pdi, pdq, pu, pv,
                                      pti, ptv, ptp, pg, pa, pt, pws,
                                      ws.numel(), _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gemm_verify_sample")


def gemm_verify_sample(x, Wt, N: int, K: int, temperature: float,
                       top_p: float, top_k: int, draft_tok, draft_idx,
                       draft_q, u, v, stream=None) -> dict:
    """q4_gemm_verify_sample with its outputs and workspace allocated here
    (torch tensors on x's device); returns the outputs by name."""
    import torch
    M = x.shape[0]
    dev = x.device
    out = {"top_idx": torch.empty((M, top_k), dtype=torch.int32, device=dev),
           "top_val": torch.empty((M, top_k), dtype=torch.float32, device=dev),
           "top_prob": torch.empty((M, top_k), dtype=torch.float32,
                                   device=dev),
           "greedy": torch.empty(M, dtype=torch.int32, device=dev),
           "accept": torch.empty(M, dtype=torch.int32, device=dev),
           "token": torch.empty(M, dtype=torch.int32, device=dev)}
    ws = torch.empty(q4_gemm_verify_sample_workspace(M, N, K),
                     dtype=torch.uint8, device=dev)
    q4_gemm_verify_sample(x, Wt, M, N, K, temperature, top_p, top_k,
                          draft_tok, draft_idx, draft_q, u, v, out["top_idx"],
                          out["top_val"], out["top_prob"], out["greedy"],
                          out["accept"], out["token"], ws, stream)
    return out


GDN_DK = 128
GDN_MAX_NODES = 32


def q4_gdn_commit(S, k, v, alpha, beta, path, n_accept, status=None,
                  stream=None) -> None:
    """Write the accepted tree nodes into the Gated DeltaNet states, in
    place (see include/q4verify.h).  S [L, H, dv, dk] fp32; k [L, M, Hk, dk],
    v [L, M, H, dv], alpha / beta [L, M, H] fp32; path [M] int32 (the
    accepted nodes, root first); n_accept [1] int32 (their count); status
    None or [1] int32 (receives 0, or -1 for an out-of-range count or path
    entry, in which case S is left as it was).  All on the same GPU."""
    import torch
    if S.dim() != 4 or k.dim() != 4:
        raise ValueError("S must be [L, H, dv, dk] and k [L, M, Hk, dk]")
    L, H, dv, dk = S.shape
    M, Hk = int(k.shape[1]), int(k.shape[2])
    pS = _ptr(S, "S", torch.float32)
    pk = _ptr(k, "k", torch.float32, shape=(L, M, Hk, dk))
    pv = _ptr(v, "v", torch.float32, shape=(L, M, H, dv))
    pa = _ptr(alpha, "alpha", torch.float32, shape=(L, M, H))
    pb = _ptr(beta, "beta", torch.float32, shape=(L, M, H))
    pp = _ptr(path, "path", torch.int32, numel=M)
    pn = _ptr(n_accept, "n_accept", torch.int32, numel=1)
    ps = None if status is None else _ptr(status, "status", torch.int32,
                                          numel=1)
    st = load().q4_gdn_commit(pS, int(L), int(H), Hk, int(dv), int(dk), M,
                              pk, pv, pa, pb, pp, pn, ps,
                              _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gdn_commit")


def q4_gdn_tree_out(S, q, k, v, alpha, beta, parent, out=None, status=None,
                    stream=None):
    """Every tree node's output of one recurrent layer from the shared state
    (see include/q4verify.h): S [H, dv, dk] fp32 (read only); q, k
    [M, Hk, dk], v [M, H, dv], alpha / beta [M, H] fp32; parent [M] int32 on
    the device (-1: child of the context; parents precede children); out
    None or [M, H, dv] fp32; status None or [1] int32 (receives 0, or -1 for
    an out-of-range parent, in which case out is not written).  Returns
    out."""
    import torch
    if S.dim() != 3 or k.dim() != 3:
        raise ValueError("S must be [H, dv, dk] and k [M, Hk, dk]")
    H, dv, dk = S.shape
    M, Hk = int(k.shape[0]), int(k.shape[1])
    if out is None:
        out = torch.empty((M, H, dv), dtype=torch.float32, device=S.device)
    pS = _ptr(S, "S", torch.float32)
    pq = _ptr(q, "q", torch.float32, shape=(M, Hk, dk))
    pk = _ptr(k, "k", torch.float32, shape=(M, Hk, dk))
    pv = _ptr(v, "v", torch.float32, shape=(M, H, dv))
    pa = _ptr(alpha, "alpha", torch.float32, shape=(M, H))
    pb = _ptr(beta, "beta", torch.float32, shape=(M, H))
    pp = _ptr(parent, "parent", torch.int32, numel=M)
    po = _ptr(out, "out", torch.float32, shape=(M, H, dv))
    ps = None if status is None else _ptr(status, "status", torch.int32,
                                          numel=1)
    st = load().q4_gdn_tree_out(pS, int(H), Hk, int(dv), int(dk), M, pq, pk,
                                pv, pa, pb, pp, po, ps,
                                _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_gdn_tree_out")
    return out


ATTN_HEAD_DIM = 256
ATTN_PAGE = 32
ATTN_MAX_NODES = 16


def q4_tree_attn_plan(M: int, Hq: int, Hkv: int, ctx_len: int,
                      splits: int = 0, D: int = ATTN_HEAD_DIM):
    """(runs of pages, workspace bytes) of a q4_tree_attn call."""
    s = ctypes.c_int(0)
    ws = ctypes.c_uint64(0)
    st = load().q4_tree_attn_plan(int(M), int(Hq), int(Hkv), int(D),
                                  int(ctx_len), int(splits), ctypes.byref(s),
                                  ctypes.byref(ws))
    if st != OK:
        raise Q4Error(st, f"q4_tree_attn_plan({M}, {Hq}, {Hkv}, {ctx_len})")
    return s.value, ws.value


def q4_tree_attn(q, k_pages, v_pages, k_scale, v_scale, page_table,
                 ctx_len: int, anc, scale: float, out, splits: int = 0,
                 ws=None, status=None, stream=None) -> None:
    """Tree-verify attention of one layer (see include/q4verify.h).
    q [M, Hq, D] bf16; k_pages [pool, Hkv, 32, D] int8; v_pages
    [pool, Hkv, D, 32] int8; k_scale / v_scale [pool, Hkv, 32] fp32;
    page_table int32 (logical -> physical page); anc [M] int32 holding the
    uint32 ancestor-or-self sets; out [M, Hq, D] fp32; ws a uint8 tensor of
    q4_tree_attn_plan's bytes when that is not 0; status None or [1] int32."""
    import torch
    M, Hq, D = q.shape
    pool, Hkv = int(k_pages.shape[0]), int(k_pages.shape[1])
    pages = (int(ctx_len) + M + ATTN_PAGE - 1) // ATTN_PAGE
    pq = _ptr(q, "q", torch.bfloat16)
    pk = _ptr(k_pages, "k_pages", torch.int8, shape=(pool, Hkv, ATTN_PAGE, D))
    pv = _ptr(v_pages, "v_pages", torch.int8, shape=(pool, Hkv, D, ATTN_PAGE))
    pks = _ptr(k_scale, "k_scale", torch.float32, shape=(pool, Hkv, ATTN_PAGE))
    pvs = _ptr(v_scale, "v_scale", torch.float32, shape=(pool, Hkv, ATTN_PAGE))
    if page_table.numel() < pages:
        raise ValueError(f"page_table must hold {pages} entries")
    ppt = _ptr(page_table, "page_table", torch.int32)
    pa = _ptr(anc, "anc", torch.int32, numel=M)
    po = _ptr(out, "out", torch.float32, shape=(M, Hq, D))
    pws, nws = None, 0
    if ws is not None:
        pws, nws = _ptr(ws, "ws", torch.uint8), ws.numel()
    ps = None if status is None else _ptr(status, "status", torch.int32,
                                          numel=1)
    st = load().q4_tree_attn(pq, int(M), int(Hq), Hkv, int(D), pk, pv, pks,
                             pvs, ppt, pool, int(ctx_len), pa, float(scale),
                             po, int(splits), pws, nws, ps,
                             _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_tree_attn")


def tree_attn(q, k_pages, v_pages, k_scale, v_scale, page_table,
              ctx_len: int, anc, scale: float, splits: int = 0, status=None,
              stream=None):
    """q4_tree_attn with its output and workspace allocated here."""
    import torch
    M, Hq, D = q.shape
    Hkv = int(k_pages.shape[1])
    _, nws = q4_tree_attn_plan(M, Hq, Hkv, ctx_len, splits, D)
    out = torch.empty((M, Hq, D), dtype=torch.float32, device=q.device)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    q4_tree_attn(q, k_pages, v_pages, k_scale, v_scale, page_table, ctx_len,
                 anc, scale, out, splits, ws, status, stream)
    return out


def q4_repack(W, Wt, N: int, K: int, stream=None) -> None:
    """Reorder planar W into the tiled layout Wt (same byte count)."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_TILED16)
    pw = _ptr(W, "W", torch.uint8, numel=total)
    pt = _ptr(Wt, "Wt", torch.uint8, numel=total)
    if W.device != Wt.device:
        raise ValueError("W and Wt must be on one device")
    st = load().q4_repack(pw, pt, int(N), int(K), _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_repack")


def q4_dequant(W, W_out, N: int, K: int, stream=None) -> None:
    """W_out[N, K] fp32 = dequantised packed W."""
    import torch
    total = _total_bytes(int(N), int(K), LAYOUT_PLANAR)
    pw = _ptr(W, "W", torch.uint8, numel=total)
    po = _ptr(W_out, "W_out", torch.float32, shape=(N, K))
    if W.device != W_out.device:
        raise ValueError("W and W_out must be on one device")
    st = load().q4_dequant(pw, po, int(N), int(K), _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_dequant")


def q4_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    """Read ``nbytes`` of ``buf`` once; ``sink`` is an int32 GPU tensor with
    at least one element."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    pb = _ptr(buf, "buf")
    ps = _ptr(sink, "sink")
    st = load().q4_stream_read(pb, int(nbytes), ps, _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_stream_read")


def q4_stream_copy(src, dst, nbytes: int, stream=None) -> None:
    """Copy ``nbytes`` from src to dst."""
    if nbytes > src.numel() * src.element_size() or \
            nbytes > dst.numel() * dst.element_size():
        raise ValueError("nbytes exceeds a buffer")
    st = load().q4_stream_copy(_ptr(src, "src"), _ptr(dst, "dst"), int(nbytes),
                               _stream_handle(stream))
    if st != OK:
        raise Q4Error(st, "q4_stream_copy")
