"""ctypes binding over libchunk_attn.so (the C ABI in include/chunk_attn.h).

Argument marshalling only: tensors are torch tensors on the GPU, passed by
data pointer together with torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels. If the library is missing the
import fails; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

# torch first: its HIP runtime (torch/lib/libamdhip64.so, soname
# libamdhip64.so.7) must be the one the library's libamdhip64.so.7 dependency
# binds to. Loading the library first would map the system runtime, and torch,
# which asks for the file name rather than the soname, would then map a second
# one; two HIP runtimes in one process do not share devices or memory.
import torch  # noqa: F401  (imported for its side effect on library loading)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libchunk_attn.so")

CA_F32, CA_BF16 = 0, 1
CA_OP_FWD, CA_OP_BWD, CA_OP_SPARSE_BWD, CA_OP_BWD_MIN, CA_OP_BWD_DS = 0, 1, 2, 3, 4
KERNELS = {"fwd": 0, "delta": 1, "dkdv": 2, "dq": 3, "accumulate": 4, "zero": 5, "proj": 6, "proj_prep": 7,
           "residual": 8, "head": 9, "head_aux": 10, "bwd": 11}
ERRORS = {0: "CA_OK", -1: "CA_ERR_NULL", -2: "CA_ERR_SHAPE", -3: "CA_ERR_DTYPE", -4: "CA_ERR_ALIGN",
          -5: "CA_ERR_WORKSPACE", -6: "CA_ERR_UNSUPPORTED", -7: "CA_ERR_HIP"}


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("q_capacity", ctypes.c_int32),
        ("q_row_offset", ctypes.c_int32),
        ("chunk_start", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class SpacoLayer(ctypes.Structure):
    """One layer of the stack for spaco_stack_* (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wq", "wk", "wv", "k_cache", "v_cache", "dk_acc", "dv_acc", "dwq", "dwk", "dwv")]


class HeadDesc(ctypes.Structure):
    """lm_head_desc of include/chunk_attn.h."""
    _fields_ = [("batch", ctypes.c_int32), ("seq_capacity", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class ChunkAttnError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__(f"{ERRORS.get(code, code)}: {detail}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python sequence_chunked_exact_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(Desc)
    sig = {
        "chunk_attn_workspace_size": (SZ, [D, I32]),
        "chunk_attn_fwd": (ctypes.c_int, [D, P, P, P, P, P, P, SZ, P]),
        "chunk_attn_bwd": (ctypes.c_int, [D, P, P, P, P, P, P, F, P, P, P, P, SZ, P]),
        "chunk_attn_bwd_noalloc": (ctypes.c_int, [D, P, P, P, P, P, P, F, P, P, P, P]),
        "chunked_fwd_sweep": (ctypes.c_int, [D, I32, P, P, P, P, P, P]),
        "chunked_bwd_sweep": (ctypes.c_int, [D, I32, P, P, P, P, P, P, F, P, P, P, P, SZ, P]),
        "prefix_grad_accumulate": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, I32, F, P]),
        "chunk_select": (ctypes.c_int, [I32, I32, U64, ctypes.POINTER(I32)]),
        "sparse_chunk_bwd": (ctypes.c_int, [D, I32, I32, U64, P, P, P, P, P, P, P, P, P,
                                            ctypes.POINTER(I32), P, SZ, P]),
        "qkv_proj_bwd_workspace_size": (SZ, [D, I32]),
        "qkv_proj_fwd": (ctypes.c_int, [D, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "qkv_proj_bwd": (ctypes.c_int, [D, I32, I32, I32, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "qkv_proj_weights_t_bytes": (SZ, [D, I32]),
        "qkv_proj_weights_t": (ctypes.c_int, [D, I32, P, P, P, P, P]),
        "qkv_proj_bwd_wt": (ctypes.c_int, [D, I32, I32, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "spaco_stack_workspace_size": (SZ, [D, I32]),
        "spaco_stack_forward": (ctypes.c_int, [D, I32, I32, ctypes.POINTER(SpacoLayer), P, I32, P, SZ, P]),
        "spaco_stack_backward": (ctypes.c_int, [D, I32, I32, ctypes.POINTER(SpacoLayer), P, P, P, I32,
                                                ctypes.POINTER(I32), I32, F, P, SZ, P]),
        "lm_head_transpose": (ctypes.c_int, [ctypes.POINTER(HeadDesc), P, P, P]),
        "lm_head_sft_workspace_size": (SZ, [ctypes.POINTER(HeadDesc), I32]),
        "lm_head_sft_partition": (ctypes.c_int, [ctypes.POINTER(HeadDesc), I32, I32, P, P, P, P, P, F, P, P, P, P,
                                                 SZ, P]),
        "lm_head_dpo_finish": (ctypes.c_int, [ctypes.POINTER(HeadDesc), I32, P, F, F, F, P, P,
                                              ctypes.POINTER(F), ctypes.POINTER(F), P]),
        "lm_head_sft_sweep_workspace_size": (SZ, [ctypes.POINTER(HeadDesc), I32, I32]),
        "lm_head_sft_sweep": (ctypes.c_int, [ctypes.POINTER(HeadDesc), I32, I32, I32, P, P, P, P, P, F, P, P, P,
                                             P, SZ, P]),
        "chunk_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "chunk_attn_last_error": (ctypes.c_char_p, []),
        "chunk_attn_profile_start": (ctypes.c_int, []),
        "chunk_attn_profile_stop": (ctypes.c_int, []),
        "chunk_attn_profile_select": (ctypes.c_int, [ctypes.c_uint32]),
        "chunk_attn_profile_read": (ctypes.c_int, [I32, ctypes.POINTER(ctypes.c_int64),
                                                   ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _check(rc: int):
    if rc != 0:
        raise ChunkAttnError(rc, lib.chunk_attn_last_error().decode())


def _ptr(t) -> int:
    return t.data_ptr()


def _stream(t) -> Optional[int]:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CA_BF16
    if t.dtype == torch.float32:
        return CA_F32
    raise TypeError(f"q/k/v/o/dout must be float32 or bfloat16, got {t.dtype}")


def make_desc(q, k, *, chunk_start: int, chunk_len: int, q_row_offset: int = 0,
              softmax_scale: float = 1.0) -> Desc:
    """Descriptor from [B, Hq, q_capacity, d] queries and [B, Hkv, kv_capacity, d] keys."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [batch, heads, rows, head_dim]")
    B, Hq, Tq, d = q.shape
    _, Hkv, Tk, _ = k.shape
    return Desc(B, Hq, Hkv, d, Tk, Tq, q_row_offset, chunk_start, chunk_len, float(softmax_scale),
                _dtype_code(q))


def _contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def chunk_attn_workspace_size(desc: Desc, op: int) -> int:
    return int(lib.chunk_attn_workspace_size(ctypes.byref(desc), op))


def _workspace(desc: Desc, op: int, like, ws):
    import torch
    need = chunk_attn_workspace_size(desc, op)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=like.device)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def chunk_attn_fwd(q, k, v, o, lse, *, chunk_start: int, chunk_len: int, q_row_offset: int = 0,
                   softmax_scale: float = 1.0):
    """Forward of one chunk; writes o and lse rows [q_row_offset, +chunk_len)."""
    _contig(q, k, v, o, lse)
    desc = make_desc(q, k, chunk_start=chunk_start, chunk_len=chunk_len, q_row_offset=q_row_offset,
                     softmax_scale=softmax_scale)
    _check(lib.chunk_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              None, 0, _stream(q)))


def chunk_attn_bwd(q, k, v, o, lse, dout, dq, dk_acc, dv_acc, *, chunk_start: int, chunk_len: int,
                   q_row_offset: int = 0, softmax_scale: float = 1.0, grad_scale: float = 1.0,
                   workspace=None, ds_handover: bool = False):
    """Backward of one chunk: dq rows overwritten, dk_acc/dv_acc prefix rows incremented.
    Without a workspace one is allocated: CA_OP_BWD (bounded, dQ recomputes dS), or
    CA_OP_BWD_DS when ds_handover (dS handed to the dQ pass; memory grows with the prefix)."""
    _contig(q, k, v, o, lse, dout, dq, dk_acc, dv_acc)
    desc = make_desc(q, k, chunk_start=chunk_start, chunk_len=chunk_len, q_row_offset=q_row_offset,
                     softmax_scale=softmax_scale)
    ws, nbytes = _workspace(desc, CA_OP_BWD_DS if ds_handover else CA_OP_BWD, q, workspace)
    _check(lib.chunk_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _ptr(dout), float(grad_scale), _ptr(dq), _ptr(dk_acc), _ptr(dv_acc),
                              None if ws is None else _ptr(ws), nbytes, _stream(q)))


def chunk_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk_acc, dv_acc, *, chunk_start: int, chunk_len: int,
                           q_row_offset: int = 0, softmax_scale: float = 1.0, grad_scale: float = 1.0):
    """chunk_attn_bwd with the library's static scratch instead of a workspace (allocates nothing)."""
    _contig(q, k, v, o, lse, dout, dq, dk_acc, dv_acc)
    desc = make_desc(q, k, chunk_start=chunk_start, chunk_len=chunk_len, q_row_offset=q_row_offset,
                     softmax_scale=softmax_scale)
    _check(lib.chunk_attn_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(dout), float(grad_scale), _ptr(dq), _ptr(dk_acc), _ptr(dv_acc),
                                      _stream(q)))


def prefix_grad_accumulate(acc, src, prefix_len: int, scale: float = 1.0):
    """acc[:, :, :prefix_len] += scale * src[:, :, :prefix_len] (float32, [B, H, rows, d])."""
    _contig(acc, src)
    B, H, Ta, d = acc.shape
    Ts = src.shape[2]
    _check(lib.prefix_grad_accumulate(_ptr(acc), _ptr(src), B, H, Ta, Ts, d, int(prefix_len),
                                      float(scale), _stream(acc)))


def qkv_proj_bwd_workspace_size(desc: Desc, d_model: int) -> int:
    return int(lib.qkv_proj_bwd_workspace_size(ctypes.byref(desc), int(d_model)))


def qkv_proj_fwd(h, wq, wk, wv, q, k, v, *, chunk_start: int, chunk_len: int, q_row_offset: int = 0,
                 h_row_offset: Optional[int] = None):
    """Q/K/V of one chunk from the layer input h [B, T_h, d_model] and weights [d_model, H*d]:
    q rows [q_row_offset, +chunk_len), k and v rows [chunk_start, +chunk_len)."""
    _contig(h, wq, wk, wv, q, k, v)
    desc = make_desc(q, k, chunk_start=chunk_start, chunk_len=chunk_len, q_row_offset=q_row_offset)
    B, Th, dm = h.shape
    hoff = chunk_start if h_row_offset is None else h_row_offset
    _check(lib.qkv_proj_fwd(ctypes.byref(desc), dm, Th, int(hoff), _ptr(h), _ptr(wq), _ptr(wk), _ptr(wv),
                            _ptr(q), _ptr(k), _ptr(v), _stream(q)))


def qkv_proj_weights_t_bytes(desc: Desc, d_model: int) -> int:
    return int(lib.qkv_proj_weights_t_bytes(ctypes.byref(desc), int(d_model)))


def qkv_proj_weights_t(wq, wk, wv, q, k, out=None):
    """W_cat^T = [wq | wk | wv]^T (bf16, [(Hq + 2 Hkv) d, d_model]) for qkv_proj_bwd(..., w_cat_t=)
    over a backward sweep with these weights. q and k only give the descriptor's shapes."""
    _contig(wq, wk, wv)
    desc = make_desc(q, k, chunk_start=0, chunk_len=1)
    dm = wq.shape[0]
    if out is None:
        import torch
        out = torch.empty(wq.shape[1] + wk.shape[1] + wv.shape[1], dm, dtype=wq.dtype, device=wq.device)
    _contig(out)
    _check(lib.qkv_proj_weights_t(ctypes.byref(desc), dm, _ptr(wq), _ptr(wk), _ptr(wv), _ptr(out), _stream(wq)))
    return out


def qkv_proj_bwd(h, wq, wk, wv, q, k, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh, *, chunk_start: int,
                 chunk_len: int, q_row_offset: int = 0, h_row_offset: Optional[int] = None, workspace=None,
                 w_cat_t=None):
    """Projection gradients of one chunk: dW += H_in^T (dQ, dK, dV rows of the chunk), dh rows of
    the chunk = dQ Wq^T + dK Wk^T + dV Wv^T. q and k only give the descriptor's shapes. w_cat_t:
    the weights' transpose from qkv_proj_weights_t (bf16 layers), written once per sweep instead
    of by every call."""
    _contig(h, wq, wk, wv, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh)
    desc = make_desc(q, k, chunk_start=chunk_start, chunk_len=chunk_len, q_row_offset=q_row_offset)
    B, Th, dm = h.shape
    hoff = chunk_start if h_row_offset is None else h_row_offset
    need = qkv_proj_bwd_workspace_size(desc, dm)
    if w_cat_t is not None:
        need -= qkv_proj_weights_t_bytes(desc, dm)
    if workspace is None and need > 0:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    ws, nbytes = workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())
    wsp = None if ws is None else _ptr(ws)
    if w_cat_t is None:
        _check(lib.qkv_proj_bwd(ctypes.byref(desc), dm, Th, int(hoff), _ptr(h), _ptr(wq), _ptr(wk), _ptr(wv),
                                _ptr(dq), _ptr(dk_acc), _ptr(dv_acc), _ptr(dwq), _ptr(dwk), _ptr(dwv), _ptr(dh),
                                wsp, nbytes, _stream(h)))
    else:
        _contig(w_cat_t)
        _check(lib.qkv_proj_bwd_wt(ctypes.byref(desc), dm, Th, int(hoff), _ptr(h), _ptr(wq), _ptr(wk), _ptr(wv),
                                   _ptr(w_cat_t), _ptr(dq), _ptr(dk_acc), _ptr(dv_acc), _ptr(dwq), _ptr(dwk),
                                   _ptr(dwv), _ptr(dh), wsp, nbytes, _stream(h)))


def chunk_select(k: int, t: int, seed: int) -> list:
    out = (ctypes.c_int32 * max(t, 1))()
    _check(lib.chunk_select(int(k), int(t), ctypes.c_uint64(seed & (2**64 - 1)), out))
    return list(out[:t])


def sparse_chunk_bwd(q, k, v, o, lse, dout, dq, dk, dv, *, seq_len: int, chunk: int, t: int, seed: int,
                     softmax_scale: float = 1.0, workspace=None, ds_handover: bool = False) -> list:
    """SpaCO backward over t of the k chunks (scaled by k/t); returns the selected chunks."""
    _contig(q, k, v, o, lse, dout, dq, dk, dv)
    desc = make_desc(q, k, chunk_start=0, chunk_len=chunk, softmax_scale=softmax_scale)
    ws, nbytes = _workspace(desc, CA_OP_BWD_DS if ds_handover else CA_OP_SPARSE_BWD, q, workspace)
    sel = (ctypes.c_int32 * t)()
    _check(lib.sparse_chunk_bwd(ctypes.byref(desc), int(seq_len), int(t),
                                ctypes.c_uint64(seed & (2**64 - 1)), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), sel,
                                None if ws is None else _ptr(ws), nbytes, _stream(q)))
    return list(sel)


def chunked_forward(q, k, v, o, lse, *, chunk: int, seq_len: Optional[int] = None,
                    softmax_scale: float = 1.0, chunks: Optional[Sequence[int]] = None):
    """SeCO's inference-mode pass: every chunk's forward in ascending order
    (chunked_fwd_sweep), or only the chunks listed in ``chunks``."""
    T = q.shape[2] if seq_len is None else seq_len
    if chunks is not None:
        for i in chunks:
            s = i * chunk
            chunk_attn_fwd(q, k, v, o, lse, chunk_start=s, chunk_len=min(chunk, T - s), q_row_offset=s,
                           softmax_scale=softmax_scale)
        return
    _contig(q, k, v, o, lse)
    desc = make_desc(q, k, chunk_start=0, chunk_len=chunk, softmax_scale=softmax_scale)
    _check(lib.chunked_fwd_sweep(ctypes.byref(desc), int(T), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 _stream(q)))


def chunked_backward(q, k, v, o, lse, dout, dq, dk_acc, dv_acc, *, chunk: int,
                     seq_len: Optional[int] = None, softmax_scale: float = 1.0, grad_scale: float = 1.0,
                     workspace=None, ds_handover: bool = False):
    """Exact chunked backward (SeCO, chunked_bwd_sweep): every chunk, descending; dk_acc/dv_acc
    are incremented (zero them first), dq rows overwritten."""
    _contig(q, k, v, o, lse, dout, dq, dk_acc, dv_acc)
    T = q.shape[2] if seq_len is None else seq_len
    desc = make_desc(q, k, chunk_start=0, chunk_len=chunk, softmax_scale=softmax_scale)
    ws, nbytes = _workspace(desc, CA_OP_BWD_DS if ds_handover else CA_OP_SPARSE_BWD, q, workspace)
    _check(lib.chunked_bwd_sweep(ctypes.byref(desc), int(T), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 _ptr(dout), float(grad_scale), _ptr(dq), _ptr(dk_acc), _ptr(dv_acc),
                                 None if ws is None else _ptr(ws), nbytes, _stream(q)))


def _stack_layers(layers):
    arr = (SpacoLayer * len(layers))()
    for i, lay in enumerate(layers):
        for name, _ in SpacoLayer._fields_:
            t = lay.get(name)
            setattr(arr[i], name, None if t is None else _ptr(t))
    return arr


def stack_desc(h0, layers, *, chunk: int, softmax_scale: float = 1.0) -> Desc:
    """Whole-sequence descriptor of a layer stack: h0 [B, T_h, Hq*d], caches [B, Hkv, T_cap, d]."""
    B, Th, dm = h0.shape
    _, Hkv, Tcap, d = layers[0]["k_cache"].shape
    return Desc(B, dm // d, Hkv, d, Tcap, chunk, 0, 0, chunk, float(softmax_scale), _dtype_code(h0))


def spaco_stack_workspace(desc: Desc, n_layers: int, like):
    import torch
    need = int(lib.spaco_stack_workspace_size(ctypes.byref(desc), int(n_layers)))
    return torch.empty(max(need, 256), dtype=torch.uint8, device=like.device)


def spaco_stack_forward(h0, layers, *, chunk: int, seq_len: Optional[int] = None, softmax_scale: float = 1.0,
                        workspace=None):
    """Inference-mode pass of the stack: fills every layer's k_cache / v_cache.
    layers: list of dicts of tensors (wq, wk, wv, k_cache, v_cache[, dk_acc, dv_acc, dwq, dwk, dwv])."""
    desc = stack_desc(h0, layers, chunk=chunk, softmax_scale=softmax_scale)
    T = h0.shape[1] if seq_len is None else seq_len
    ws = spaco_stack_workspace(desc, len(layers), h0) if workspace is None else workspace
    _check(lib.spaco_stack_forward(ctypes.byref(desc), int(T), len(layers), _stack_layers(layers), _ptr(h0),
                                   h0.shape[1], _ptr(ws), ws.numel(), _stream(h0)))


def spaco_stack_backward(h0, dy, dh0, layers, *, chunk: int, chunks: Sequence[int], relay_factor: float,
                         seq_len: Optional[int] = None, softmax_scale: float = 1.0, workspace=None):
    """SpaCO's relayed backward over the drawn chunks (after spaco_stack_forward)."""
    _contig(h0, dy, dh0)
    desc = stack_desc(h0, layers, chunk=chunk, softmax_scale=softmax_scale)
    T = h0.shape[1] if seq_len is None else seq_len
    ws = spaco_stack_workspace(desc, len(layers), h0) if workspace is None else workspace
    sel = (ctypes.c_int32 * len(chunks))(*[int(c) for c in chunks])
    _check(lib.spaco_stack_backward(ctypes.byref(desc), int(T), len(layers), _stack_layers(layers), _ptr(h0),
                                    _ptr(dy), _ptr(dh0), h0.shape[1], sel, len(chunks), float(relay_factor),
                                    _ptr(ws), ws.numel(), _stream(h0)))


def head_desc(h, w) -> HeadDesc:
    """Descriptor from h [B, T, d_model] and w [vocab, d_model]."""
    B, T, dm = h.shape
    return HeadDesc(B, T, dm, w.shape[0], _dtype_code(h))


def lm_head_transpose(w, wt):
    """wt [d_model, vocab] = w^T (bf16)."""
    _contig(w, wt)
    d = HeadDesc(1, 1, w.shape[1], w.shape[0], _dtype_code(w))
    _check(lib.lm_head_transpose(ctypes.byref(d), _ptr(w), _ptr(wt), _stream(w)))


def lm_head_sft_workspace(h, w, rows: int):
    import torch
    d = head_desc(h, w)
    need = int(lib.lm_head_sft_workspace_size(ctypes.byref(d), int(rows)))
    return torch.empty(max(need, 256), dtype=torch.uint8, device=h.device)


def lm_head_sft_partition(h, w, wt, labels, row_loss, dh, dw, *, row_start: int, rows: int, loss_scale: float,
                          row_weight=None, workspace=None):
    """One partition of the streamed SFT head (see lm_head_sft_partition in chunk_attn.h)."""
    _contig(h, w, wt, labels, row_loss, dh, dw)
    d = head_desc(h, w)
    ws = lm_head_sft_workspace(h, w, rows) if workspace is None else workspace
    _check(lib.lm_head_sft_partition(ctypes.byref(d), int(row_start), int(rows), _ptr(h), _ptr(w), _ptr(wt),
                                     _ptr(labels), None if row_weight is None else _ptr(row_weight),
                                     float(loss_scale), _ptr(row_loss), _ptr(dh), _ptr(dw), _ptr(ws), ws.numel(),
                                     _stream(h)))


def lm_head_sweep_workspace(h, w, ps: int, dw_group: int):
    import torch
    d = head_desc(h, w)
    need = int(lib.lm_head_sft_sweep_workspace_size(ctypes.byref(d), int(ps), int(dw_group)))
    return torch.empty(max(need, 256), dtype=torch.uint8, device=h.device)


def lm_head_sft(h, w, wt, labels, row_loss, dh, dw, *, loss_scale: float, ps: int = 100, dw_group: int = 1,
                seq_len: Optional[int] = None, row_weight=None, workspace=None):
    """StreamBP's streamed SFT head over every partition of ps positions (lm_head_sft_sweep)."""
    _contig(h, w, wt, labels, row_loss, dh, dw)
    d = head_desc(h, w)
    T = h.shape[1] if seq_len is None else seq_len
    ws = lm_head_sweep_workspace(h, w, ps, dw_group) if workspace is None else workspace
    _check(lib.lm_head_sft_sweep(ctypes.byref(d), int(T), int(ps), int(dw_group), _ptr(h), _ptr(w), _ptr(wt),
                                 _ptr(labels), None if row_weight is None else _ptr(row_weight),
                                 float(loss_scale), _ptr(row_loss), _ptr(dh), _ptr(dw), _ptr(ws), ws.numel(),
                                 _stream(h)))


def lm_head_dpo_finish(row_loss, dh, dw, w, *, ref_logp, beta: float, seq_len: Optional[int] = None):
    """DPO's final scalar on one preference pair (see lm_head_dpo_finish); returns (loss, c)."""
    _contig(row_loss, dh, dw)
    B, T = row_loss.shape
    d = HeadDesc(B, T, dh.shape[2], w.shape[0], _dtype_code(w))
    loss, c = ctypes.c_float(), ctypes.c_float()
    _check(lib.lm_head_dpo_finish(ctypes.byref(d), int(T if seq_len is None else seq_len), _ptr(row_loss),
                                  float(ref_logp[0]), float(ref_logp[1]), float(beta), _ptr(dh), _ptr(dw),
                                  ctypes.byref(loss), ctypes.byref(c), _stream(dh)))
    return float(loss.value), float(c.value)


def profile_start():
    """Bracket every later kernel launch with HIP events (see chunk_attn.h)."""
    _check(lib.chunk_attn_profile_start())


def profile_select(kernels=None):
    """Record events only for the named kernels (None: all) from the next profile_start()."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNELS[k] for k in kernels)
    _check(lib.chunk_attn_profile_select(mask))


def profile_stop():
    _check(lib.chunk_attn_profile_stop())


def profile_read() -> dict:
    """{kernel name: (launches, total GPU ms)} for the launches since profile_start()."""
    out = {}
    for name, kid in KERNELS.items():
        n, ms = ctypes.c_int64(), ctypes.c_double()
        _check(lib.chunk_attn_profile_read(kid, ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (int(n.value), float(ms.value))
    return out
