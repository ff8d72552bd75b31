"""MI355X-native fused attention + Ulysses post-attention all-to-all (FlashAttention-A2A).

Thin Python binding over ``libxstage.so`` (C ABI in ``include/xstage.h``): argument
marshalling only.  Tensors are torch CUDA (HIP) tensors used as plain device buffers; every
step of the computation runs in the library's HIP kernels.  Functions carry the C names.

Layouts: q, k, v, out are [B, S, H_local, D] bf16; ``out_slabs`` is either a list of P
tensors [B, S/P, H_local, D] or one tensor [P, B, S/P, H_local, D] whose leading index
selects the destination.
"""

from __future__ import annotations

import ctypes
import math

from ._lib import (  # noqa: F401
    LIB_PATH,
    WS_FULL,
    XSTAGE_ERR_HIP,
    XSTAGE_ERR_INVALID,
    XSTAGE_ERR_UNSUPPORTED,
    XSTAGE_MAX_P,
    XSTAGE_OK,
    BGParams,
    MoeParams,
    LibraryMissing,
    XStageError,
    lib,
    ptr_array,
    status_name,
)

__all__ = [
    "xstage_attn_a2a_fwd",
    "xstage_attn_split_ws_size",
    "split_workspace",
    "xstage_attn_a2a_fwd_noalloc",
    "xstage_attn_fwd",
    "xstage_a2a_scatter",
    "xstage_attn_a2a_unfused",
    "xstage_attn_a2a_fwd_strided",
    "xstage_ulysses_attn_fwd",
    "xstage_ulysses_gather",
    "xstage_a2a_scatter_strided",
    "xstage_ulysses_attn_unfused",
    "xstage_ulysses_attn_fwd_kv_staged",
    "xstage_attn_a2a_plan",
    "xstage_attn_a2a_wg_rows",
    "xstage_attn_a2a_schedule",
    "xstage_attn_a2a_fwd_traced",
    "xstage_attn_a2a_fwd_paced",
    "xstage_attn_a2a_paced_plan",
    "xstage_attn_a2a_fwd_nsplit",
    "xstage_attn_nsplit_ws_size",
    "xstage_moe_waves_run",
    "xstage_moe_waves_plan",
    "xstage_burst_gap_run",
    "xstage_wallclock_hz",
    "xstage_bg_t_iss",
    "xstage_bg_pacing_chunks",
    "xstage_status_str",
    "bind",
    "LibraryMissing",
    "XStageError",
]


def _check(status: int, where: str) -> None:
    if status != XSTAGE_OK:
        raise XStageError(status, where)


def _dev_tensor(t, name: str, device=None, min_bytes=None, bf16=True):
    """Checks that ``t`` is a contiguous device tensor (bf16 storage unless bf16=False), on
    ``device`` if given, holding at least ``min_bytes`` bytes if given.  The C ABI sees only
    pointers, so the sizes and devices of the buffers it writes are checked here."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if bf16 and (t.element_size() != 2 or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16)):
        raise ValueError(f"{name} must hold bf16 values (bfloat16 or 16-bit integer storage)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the call writes {min_bytes}")
    return t


def _stream_of(t, stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _split_ws(split_ws, device):
    """(pointer, bytes) of an optional split workspace (any dtype, contiguous, on ``device``)."""
    if split_ws is None:
        return None, 0
    _dev_tensor(split_ws, "split_ws", device=device, bf16=False)
    return split_ws.data_ptr(), split_ws.numel() * split_ws.element_size()


def _slab_ptrs(out_slabs, device=None, slab_bytes=None):
    """Device pointers of P destination buffers, given as a list of tensors or one tensor whose
    leading index selects the destination; each must hold ``slab_bytes(P)`` bytes."""
    import torch

    if isinstance(out_slabs, torch.Tensor):
        _dev_tensor(out_slabs, "out_slabs", device=device)
        P = int(out_slabs.shape[0])
        need = slab_bytes(P) if slab_bytes else None
        if need is not None:
            _dev_tensor(out_slabs, "out_slabs", min_bytes=need * P)
        return [out_slabs[p].data_ptr() for p in range(P)], P
    slabs = list(out_slabs)
    P = len(slabs)
    need = slab_bytes(P) if (slab_bytes and P) else None
    for i, t in enumerate(slabs):
        _dev_tensor(t, f"out_slabs[{i}]", device=device, min_bytes=need)
    return [t.data_ptr() for t in slabs], P


def _shards(x, name, device=None):
    """Device pointers and the common [B, S/P, H, D] shape of P shards, given as a list of
    tensors or one [P, B, S/P, H, D] tensor."""
    import torch

    if isinstance(x, torch.Tensor):
        _dev_tensor(x, name, device=device)
        if x.dim() != 5:
            raise ValueError(f"{name} must be [P, B, S/P, H, D]")
        return [x[p].data_ptr() for p in range(x.shape[0])], tuple(int(d) for d in x.shape[1:])
    xs_ = list(x)
    if not xs_:
        raise ValueError(f"{name} is empty")
    for i, t in enumerate(xs_):
        _dev_tensor(t, f"{name}[{i}]", device=device)
        if t.dim() != 4 or t.shape != xs_[0].shape:
            raise ValueError(f"{name} must be P tensors of one [B, S/P, H, D] shape")
    return [t.data_ptr() for t in xs_], tuple(int(d) for d in xs_[0].shape)


def _qkv(q, k, v):
    _dev_tensor(q, "q")
    _dev_tensor(k, "k", device=q.device)
    _dev_tensor(v, "v", device=q.device)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, S, H_local, D] shape")
    return tuple(int(x) for x in q.shape)


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _slab_need(B, S, H, D):
    """Bytes of one of P slabs [B, S/P, H, D] (None when S % P != 0: the library rejects it)."""
    return lambda P: (B * (S // P) * H * D * 2) if P > 0 and S % P == 0 else None


# ---- marshalling: one function per entry point, shared by the calls and by bind() -------
# Each returns (C arguments, objects to keep alive during the call, device).

def _m_attn_a2a_fwd(q, k, v, out_slabs, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    ws, wsb = _split_ws(split_ws, q.device)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, _scale(scale, D), ws, wsb,
            _stream_of(q, stream))
    return call, (q, k, v, out_slabs, keep, split_ws), q.device


def _m_attn_fwd(q, k, v, out, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    _dev_tensor(out, "out", device=q.device, min_bytes=B * S * H * D * 2)
    ws, wsb = _split_ws(split_ws, q.device)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, H, D, _scale(scale, D), ws, wsb,
            _stream_of(q, stream))
    return call, (q, k, v, out, split_ws), q.device


def _m_a2a_scatter(inp, out_slabs, stream=None):
    _dev_tensor(inp, "in")
    B, S, H, D = (int(x) for x in inp.shape)
    ptrs, P = _slab_ptrs(out_slabs, inp.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    return (inp.data_ptr(), arr, B, S, H, D, P, _stream_of(inp, stream)), (inp, out_slabs, keep), inp.device


def _m_attn_a2a_unfused(q, k, v, workspace, out_slabs, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    _dev_tensor(workspace, "workspace", device=q.device, min_bytes=B * S * H * D * 2)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    ws, wsb = _split_ws(split_ws, q.device)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), workspace.data_ptr(), arr, B, S, H, D, P, _scale(scale, D),
            ws, wsb, _stream_of(q, stream))
    return call, (q, k, v, workspace, out_slabs, keep, split_ws), q.device


def _m_attn_a2a_fwd_traced(q, k, v, out_slabs, mode, stamps, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    ws, wsb = _split_ws(split_ws, q.device)
    nwg, _ = xstage_attn_a2a_plan(B, S, H, D, wsb)
    waves = xstage_attn_a2a_wg_rows(B, S, H, D, wsb) // 32
    _dev_tensor(stamps, "stamps", device=q.device, min_bytes=nwg * waves * 4 * 8, bf16=False)
    if stamps.element_size() != 8:
        raise ValueError("stamps must be a 64-bit tensor")
    arr, keep = ptr_array(ptrs)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, _scale(scale, D), int(mode),
            stamps.data_ptr(), ws, wsb, _stream_of(q, stream))
    return call, (q, k, v, out_slabs, stamps, keep, split_ws), q.device


def _m_attn_a2a_fwd_strided(q, k, v, out_dst, h_dst0, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, shp = _shards(out_dst, "out_dst", device=q.device)
    P = len(ptrs)
    if shp[0] != B or shp[1] * P != S or shp[3] != D:
        raise ValueError("out_dst must be P buffers of [B, S/P, H_dst, D]")
    arr, keep = ptr_array(ptrs)
    ws, wsb = _split_ws(split_ws, q.device)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, shp[2], int(h_dst0), _scale(scale, D),
            ws, wsb, _stream_of(q, stream))
    return call, (q, k, v, out_dst, keep, split_ws), q.device


def _ulysses_common(q_src, k_src, v_src, out_dst):
    qp, shp = _shards(q_src, "q_src")
    t0 = q_src if not isinstance(q_src, (list, tuple)) else q_src[0]
    dev = t0.device
    kp, kshp = _shards(k_src, "k_src", device=dev)
    vp, vshp = _shards(v_src, "v_src", device=dev)
    op, oshp = _shards(out_dst, "out_dst", device=dev)
    P = len(qp)
    if not (len(kp) == len(vp) == len(op) == P and kshp == vshp == oshp == shp):
        raise ValueError("q_src, k_src, v_src, out_dst must be P shards of one [B, S/P, H, D] shape")
    arrs = [ptr_array(x) for x in (qp, kp, vp, op)]
    return arrs, shp, P, t0, dev


def _m_ulysses_attn_fwd(q_src, k_src, v_src, out_dst, H_local, h0, scale=None, split_ws=None, stream=None):
    arrs, (B, sp, H, D), P, t0, dev = _ulysses_common(q_src, k_src, v_src, out_dst)
    ws, wsb = _split_ws(split_ws, dev)
    call = (arrs[0][0], arrs[1][0], arrs[2][0], arrs[3][0], B, sp * P, H, int(H_local), int(h0), D, P,
            _scale(scale, D), ws, wsb, _stream_of(t0, stream))
    return call, (q_src, k_src, v_src, out_dst, [a[1] for a in arrs], split_ws), dev


def _ulysses_ws_call(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale, split_ws, stream, n_tensors):
    arrs, (B, sp, H, D), P, t0, dev = _ulysses_common(q_src, k_src, v_src, out_dst)
    _dev_tensor(workspace, "workspace", device=dev, min_bytes=n_tensors * B * sp * P * int(H_local) * D * 2)
    ws, wsb = _split_ws(split_ws, dev)
    call = (arrs[0][0], arrs[1][0], arrs[2][0], workspace.data_ptr(), arrs[3][0], B, sp * P, H, int(H_local),
            int(h0), D, P, _scale(scale, D), ws, wsb, _stream_of(t0, stream))
    return call, (q_src, k_src, v_src, workspace, out_dst, [a[1] for a in arrs], split_ws), dev


def _m_ulysses_attn_unfused(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=None, split_ws=None,
                            stream=None):
    return _ulysses_ws_call(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale, split_ws, stream, 4)


def _m_ulysses_attn_fwd_kv_staged(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=None,
                                  split_ws=None, stream=None):
    return _ulysses_ws_call(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale, split_ws, stream, 2)


def _m_attn_a2a_fwd_nsplit(q, k, v, out_slabs, n_split, scale=None, split_ws=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    need = xstage_attn_nsplit_ws_size(B, S, H, D, n_split)
    if need and split_ws is None:
        raise ValueError(f"n_split={n_split} needs a split workspace of {need} bytes (xstage_attn_nsplit_ws_size)")
    ws, wsb = (None, 0) if split_ws is None else (_dev_tensor(split_ws, "split_ws", device=q.device, min_bytes=need,
                                                              bf16=False).data_ptr(), split_ws.numel() * split_ws.element_size())
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, _scale(scale, D), int(n_split), ws, wsb,
            _stream_of(q, stream))
    return call, (q, k, v, out_slabs, keep, split_ws), q.device


def _m_attn_a2a_fwd_paced(q, k, v, out_slabs, chunks, scale=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, _scale(scale, D), int(chunks),
            _stream_of(q, stream))
    return call, (q, k, v, out_slabs, keep), q.device


def _m_attn_a2a_fwd_noalloc(q, k, v, out_slabs, scale=None, stream=None):
    B, S, H, D = _qkv(q, k, v)
    ptrs, P = _slab_ptrs(out_slabs, q.device, _slab_need(B, S, H, D))
    arr, keep = ptr_array(ptrs)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), arr, B, S, H, D, P, _scale(scale, D), _stream_of(q, stream))
    return call, (q, k, v, out_slabs, keep), q.device


_MARSHAL = {
    "xstage_attn_a2a_fwd_noalloc": _m_attn_a2a_fwd_noalloc,
    "xstage_attn_a2a_fwd": _m_attn_a2a_fwd,
    "xstage_attn_fwd": _m_attn_fwd,
    "xstage_a2a_scatter": _m_a2a_scatter,
    "xstage_attn_a2a_unfused": _m_attn_a2a_unfused,
    "xstage_attn_a2a_fwd_traced": _m_attn_a2a_fwd_traced,
    "xstage_attn_a2a_fwd_paced": _m_attn_a2a_fwd_paced,
    "xstage_attn_a2a_fwd_nsplit": _m_attn_a2a_fwd_nsplit,
    "xstage_attn_a2a_fwd_strided": _m_attn_a2a_fwd_strided,
    "xstage_ulysses_attn_fwd": _m_ulysses_attn_fwd,
    "xstage_ulysses_attn_unfused": _m_ulysses_attn_unfused,
    "xstage_ulysses_attn_fwd_kv_staged": _m_ulysses_attn_fwd_kv_staged,
}


def _invoke(name, *args, **kwargs) -> None:
    import torch

    call, keep, dev = _MARSHAL[name](*args, **kwargs)
    with torch.cuda.device(dev):
        st = getattr(lib(), name)(*call)
    del keep
    _check(st, name)


def xstage_attn_a2a_fwd(q, k, v, out_slabs, scale=None, split_ws=None, stream=None) -> None:
    """Fused attention + all-to-all scatter into the P slabs (a list of P tensors
    [B, S/P, H_local, D] or one [P, B, S/P, H_local, D] tensor); ``split_ws``: optional
    caller-owned split workspace (``split_workspace``); see include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd", q, k, v, out_slabs, scale=scale, split_ws=split_ws, stream=stream)


def xstage_attn_a2a_fwd_noalloc(q, k, v, out_slabs, scale=None, stream=None) -> None:
    """xstage_attn_a2a_fwd with the split workspace in the library's static device array (no
    allocation by anyone); see include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd_noalloc", q, k, v, out_slabs, scale=scale, stream=stream)


def xstage_attn_fwd(q, k, v, out, scale=None, split_ws=None, stream=None) -> None:
    """Attention into a contiguous [B, S, H_local, D] output (first half of the serial path)."""
    _invoke("xstage_attn_fwd", q, k, v, out, scale=scale, split_ws=split_ws, stream=stream)


def xstage_a2a_scatter(inp, out_slabs, stream=None) -> None:
    """Separate all-to-all send step: contiguous [B, S, H_local, D] -> P slabs."""
    _invoke("xstage_a2a_scatter", inp, out_slabs, stream=stream)


def xstage_attn_a2a_unfused(q, k, v, workspace, out_slabs, scale=None, split_ws=None, stream=None) -> None:
    """Serial baseline: attention into ``workspace`` ([B, S, H_local, D] bf16) then the separate
    scatter."""
    _invoke("xstage_attn_a2a_unfused", q, k, v, workspace, out_slabs, scale=scale, split_ws=split_ws, stream=stream)


def xstage_attn_a2a_fwd_traced(q, k, v, out_slabs, mode, stamps, scale=None, split_ws=None, stream=None) -> None:
    """Instrumented fused call (store-span study); ``stamps`` is an int64 device tensor of
    n_workgroups * waves * 4 entries, [workgroup][wave][4] (xstage_attn_a2a_plan and
    xstage_attn_a2a_wg_rows with the same workspace: waves = rows // 32); modes as in
    include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd_traced", q, k, v, out_slabs, mode, stamps, scale=scale, split_ws=split_ws,
            stream=stream)


def xstage_attn_a2a_fwd_paced(q, k, v, out_slabs, chunks, scale=None, stream=None) -> None:
    """Paced persistent fused call: each finished tile's rows are issued in ``chunks`` chunks
    over the next tile's first key-loop iterations; slabs as xstage_attn_a2a_fwd's without
    split workspace, bit for bit; see include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd_paced", q, k, v, out_slabs, chunks, scale=scale, stream=stream)


def xstage_attn_a2a_fwd_nsplit(q, k, v, out_slabs, n_split, scale=None, split_ws=None, stream=None) -> None:
    """Fused call with exactly ``n_split`` key splits per tile; ``split_ws`` holds at least
    xstage_attn_nsplit_ws_size bytes (zero-filled; None for n_split = 1); see include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd_nsplit", q, k, v, out_slabs, n_split, scale=scale, split_ws=split_ws, stream=stream)


def xstage_attn_nsplit_ws_size(B: int, S: int, H_local: int, D: int, n_split: int) -> int:
    """Split workspace bytes of xstage_attn_a2a_fwd_nsplit for this shape and split count."""
    b = ctypes.c_ulonglong(0)
    _check(lib().xstage_attn_nsplit_ws_size(int(B), int(S), int(H_local), int(D), int(n_split), ctypes.byref(b)),
           "xstage_attn_nsplit_ws_size")
    return b.value


def xstage_attn_a2a_paced_plan(B: int, S: int, H_local: int, D: int):
    """(n_workgroups, n_tiles) of the paced launch for this shape on the current device."""
    nwg, nt = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().xstage_attn_a2a_paced_plan(int(B), int(S), int(H_local), int(D), ctypes.byref(nwg),
                                            ctypes.byref(nt)), "xstage_attn_a2a_paced_plan")
    return nwg.value, nt.value


def xstage_attn_a2a_fwd_strided(q, k, v, out_dst, h_dst0, scale=None, split_ws=None, stream=None) -> None:
    """Fused call writing head columns [h_dst0, h_dst0 + H_local) of full-head receive
    buffers out_dst (P x [B, S/P, H_dst, D]); see include/xstage.h."""
    _invoke("xstage_attn_a2a_fwd_strided", q, k, v, out_dst, h_dst0, scale=scale, split_ws=split_ws, stream=stream)


def xstage_ulysses_attn_fwd(q_src, k_src, v_src, out_dst, H_local, h0, scale=None, split_ws=None,
                            stream=None) -> None:
    """One rank's Ulysses attention layer: heads [h0, h0 + H_local) read from the P sequence
    shards (P x [B, S/P, H, D] each) and written into the P receive buffers; see
    include/xstage.h."""
    _invoke("xstage_ulysses_attn_fwd", q_src, k_src, v_src, out_dst, H_local, h0, scale=scale, split_ws=split_ws,
            stream=stream)


def xstage_ulysses_attn_unfused(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=None, split_ws=None,
                                stream=None) -> None:
    """Serial Ulysses layer: separate gather, attention, separate strided scatter;
    ``workspace`` holds 4 x [B, S, H_local, D] bf16."""
    _invoke("xstage_ulysses_attn_unfused", q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=scale,
            split_ws=split_ws, stream=stream)


def xstage_ulysses_attn_fwd_kv_staged(q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=None,
                                      split_ws=None, stream=None) -> None:
    """Ulysses layer with K and V gathered into ``workspace`` (2 x [B, S, H_local, D] bf16)
    and Q read from the shards in place; same output as xstage_ulysses_attn_fwd."""
    _invoke("xstage_ulysses_attn_fwd_kv_staged", q_src, k_src, v_src, workspace, out_dst, H_local, h0, scale=scale,
            split_ws=split_ws, stream=stream)


def xstage_ulysses_gather(src_shards, out, H_local, h0, stream=None) -> None:
    """Pre-attention all-to-all as a separate copy: heads [h0, h0 + H_local) of the P sequence
    shards into the contiguous out [B, S, H_local, D]; see include/xstage.h."""
    import torch

    ptrs, (B, sp, H, D) = _shards(src_shards, "src_shards")
    P = len(ptrs)
    _dev_tensor(out, "out", min_bytes=B * sp * P * int(H_local) * D * 2)
    arr, keep = ptr_array(ptrs)
    with torch.cuda.device(out.device):
        st = lib().xstage_ulysses_gather(arr, out.data_ptr(), B, sp * P, H, int(H_local), int(h0), D, P,
                                         _stream_of(out, stream))
    del keep
    _check(st, "xstage_ulysses_gather")


def xstage_a2a_scatter_strided(inp, out_dst, h_dst0, stream=None) -> None:
    """Post-attention all-to-all as a separate copy into full-head receive buffers."""
    import torch

    _dev_tensor(inp, "in")
    B, S, H, D = (int(x) for x in inp.shape)
    ptrs, shp = _shards(out_dst, "out_dst", device=inp.device)
    P = len(ptrs)
    if shp[0] != B or shp[1] * P != S or shp[3] != D:
        raise ValueError("out_dst must be P buffers of [B, S/P, H_dst, D]")
    arr, keep = ptr_array(ptrs)
    with torch.cuda.device(inp.device):
        st = lib().xstage_a2a_scatter_strided(inp.data_ptr(), arr, B, S, H, D, P, shp[2], int(h_dst0),
                                              _stream_of(inp, stream))
    del keep
    _check(st, "xstage_a2a_scatter_strided")


def xstage_attn_split_ws_size(B: int, S: int, H_local: int, D: int) -> int:
    """Bytes of split workspace the attention entry points use for this shape at full speed
    (0 when the shape is not split)."""
    n = ctypes.c_ulonglong(0)
    _check(lib().xstage_attn_split_ws_size(int(B), int(S), int(H_local), int(D), ctypes.byref(n)),
           "xstage_attn_split_ws_size")
    return n.value


def split_workspace(B: int, S: int, H_local: int, D: int, device=None):
    """A zero-filled split workspace for this shape (torch uint8 device tensor), or None when
    the shape is not split.  Allocation is the caller's (torch's), never the library's."""
    import torch

    n = xstage_attn_split_ws_size(B, S, H_local, D)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def xstage_attn_a2a_plan(B: int, S: int, H_local: int, D: int, split_ws_bytes=None):
    """(n_workgroups, n_split) of the attention launch for this shape on the current device
    given ``split_ws_bytes`` of split workspace (None: as much as the fastest plan uses)."""
    nwg, nsp = ctypes.c_int(0), ctypes.c_int(0)
    wsb = WS_FULL if split_ws_bytes is None else int(split_ws_bytes)
    _check(lib().xstage_attn_a2a_plan(int(B), int(S), int(H_local), int(D), wsb, ctypes.byref(nwg),
                                      ctypes.byref(nsp)), "xstage_attn_a2a_plan")
    return nwg.value, nsp.value


def xstage_attn_a2a_wg_rows(B: int, S: int, H_local: int, D: int, split_ws_bytes=None) -> int:
    """Query rows per workgroup (128: 4 waves, or 256: 8 waves) of the attention launch for
    this shape on the current device given ``split_ws_bytes`` of split workspace (None: as
    much as the fastest plan uses)."""
    rows = ctypes.c_int(0)
    wsb = WS_FULL if split_ws_bytes is None else int(split_ws_bytes)
    _check(lib().xstage_attn_a2a_wg_rows(int(B), int(S), int(H_local), int(D), wsb, ctypes.byref(rows)),
           "xstage_attn_a2a_wg_rows")
    return rows.value


def xstage_attn_a2a_schedule(B: int, S: int, H_local: int, D: int, split_ws_bytes=None):
    """Per-workgroup (tile, split, j0, j1) of the attention launch for this shape on the
    current device, as four lists (tiles of xstage_attn_a2a_wg_rows query rows; key blocks
    of 64 in [j0, j1))."""
    nwg, _ = xstage_attn_a2a_plan(B, S, H_local, D, split_ws_bytes)
    wsb = WS_FULL if split_ws_bytes is None else int(split_ws_bytes)
    arrs = [(ctypes.c_int * max(nwg, 1))() for _ in range(4)]
    n = ctypes.c_int(0)
    _check(lib().xstage_attn_a2a_schedule(int(B), int(S), int(H_local), int(D), wsb, nwg, *arrs, ctypes.byref(n)),
           "xstage_attn_a2a_schedule")
    return tuple(list(a)[: n.value] for a in arrs)


def _int_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int * max(1, len(vals)))(*vals)


def xstage_moe_waves_plan(expert_offsets, d_model, d_ff, experts_per_wave, schedule):
    """(l1_launch, l2_launch, n_launches, n_tiles) of a schedule; see include/xstage.h."""
    offs = _int_array(expert_offsets)
    E = len(expert_offsets) - 1
    l1, l2 = (ctypes.c_int * max(1, E))(), (ctypes.c_int * max(1, E))()
    nl, nt = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().xstage_moe_waves_plan(E, offs, int(d_model), int(d_ff), int(experts_per_wave), int(schedule), l1, l2,
                                       ctypes.byref(nl), ctypes.byref(nt)), "xstage_moe_waves_plan")
    return list(l1)[:E], list(l2)[:E], nl.value, nt.value


def _moe_call(x, w1, w2, h, expert_offsets, dst_slab, dst_row, outs, experts_per_wave, schedule, stamps, stream):
    import torch

    for t, name in ((x, "x"), (w1, "w1"), (w2, "w2"), (h, "h")):
        _dev_tensor(t, name)
    for t, name in ((dst_slab, "dst_slab"), (dst_row, "dst_row")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if x.dim() != 2 or w1.dim() != 3 or w2.dim() != 3 or h.dim() != 2:
        raise ValueError("x [T, d_model], w1 [E, d_ff, d_model], w2 [E, d_model, d_ff], h [T, d_ff]")
    E, d_ff, d_model = (int(d) for d in w1.shape)
    outs = list(outs)
    for i, o in enumerate(outs):
        _dev_tensor(o, f"outs[{i}]")
    offs = _int_array(expert_offsets)
    if len(expert_offsets) != E + 1:
        raise ValueError("expert_offsets must have E + 1 entries")
    out_arr, keep = ptr_array([o.data_ptr() for o in outs])
    rows = _int_array([o.shape[0] if o.dim() == 2 else 0 for o in outs])
    prm = MoeParams(E, d_model, d_ff, int(experts_per_wave), int(schedule), offs, x.data_ptr(), w1.data_ptr(),
                    w2.data_ptr(), h.data_ptr(), dst_slab.data_ptr(), dst_row.data_ptr(), len(outs), out_arr, rows,
                    stamps.data_ptr() if stamps is not None else None)
    return prm, (offs, keep, rows, x, w1, w2, h, dst_slab, dst_row, outs, stamps), _stream_of(x, stream)


def xstage_moe_waves_run(x, w1, w2, h, expert_offsets, dst_slab, dst_row, outs, experts_per_wave, schedule,
                         stamps=None, stream=None) -> None:
    """Expert-wave grouped GEMM with the combine all-to-all in the Linear-2 epilogue; see
    include/xstage.h (outs: P device tensors [rows_p, d_model])."""
    import torch

    prm, keep, st_ = _moe_call(x, w1, w2, h, expert_offsets, dst_slab, dst_row, outs, experts_per_wave, schedule,
                               stamps, stream)
    with torch.cuda.device(x.device):
        st = lib().xstage_moe_waves_run(ctypes.byref(prm), st_)
    del keep
    _check(st, "xstage_moe_waves_run")


def xstage_burst_gap_run(K, V_bytes, gap_fma_iters, rounds, dst, stamps, n_dst_sets=1, nontemporal=False,
                         sync=None, sync_timeout_ticks=0, stream=None) -> None:
    """Burst-Gap store microbenchmark; ``stamps`` is an int64 device tensor of K*rounds*3
    entries; ``sync`` (optional) a zero-filled int32 device tensor of ``rounds`` entries that
    turns on the per-round start barrier across producers (bounded by sync_timeout_ticks)."""
    import torch

    _dev_tensor(stamps, "stamps", min_bytes=K * rounds * 3 * 8, bf16=False)
    if stamps.element_size() != 8:
        raise ValueError("stamps must be a 64-bit tensor")
    if V_bytes:
        if dst is None:
            raise ValueError("dst must hold n_dst_sets * V_bytes bytes")
        _dev_tensor(dst, "dst", device=stamps.device, min_bytes=n_dst_sets * V_bytes, bf16=False)
    if sync is not None:
        _dev_tensor(sync, "sync", device=stamps.device, min_bytes=rounds * 4, bf16=False)
    p = BGParams(int(K), int(rounds), int(n_dst_sets), int(bool(nontemporal)), int(V_bytes), int(gap_fma_iters),
                 dst.data_ptr() if dst is not None else None, stamps.data_ptr(),
                 sync.data_ptr() if sync is not None else None, int(sync_timeout_ticks))
    with torch.cuda.device(stamps.device):
        st = lib().xstage_burst_gap_run(ctypes.byref(p), _stream_of(stamps, stream))
    _check(st, "xstage_burst_gap_run")


def xstage_wallclock_hz() -> float:
    hz = ctypes.c_double(0.0)
    _check(lib().xstage_wallclock_hz(ctypes.byref(hz)), "xstage_wallclock_hz")
    return hz.value


def xstage_bg_t_iss(G_s: float, T0_s: float, V_bytes: float, R_bytes_per_s: float) -> float:
    return lib().xstage_bg_t_iss(float(G_s), float(T0_s), float(V_bytes), float(R_bytes_per_s))


def xstage_bg_pacing_chunks(V_bytes, G_s, a_s, f1_Bps, R_Bps, Q_bytes, c_max=64):
    """(c, issuer-visible seconds) of the Burst-Gap pacing choice; see include/xstage.h."""
    t = ctypes.c_double(0.0)
    c = lib().xstage_bg_pacing_chunks(float(V_bytes), float(G_s), float(a_s), float(f1_Bps), float(R_Bps),
                                      float(Q_bytes), int(c_max), ctypes.byref(t))
    if c < 1:
        raise ValueError("xstage_bg_pacing_chunks: invalid parameters")
    return c, t.value


def xstage_status_str(status: int) -> str:
    return lib().xstage_status_str(int(status)).decode()


class _Bound:
    """A prepared launch: one C call with arguments marshalled once (see ``bind``)."""

    __slots__ = ("_fn", "_args", "_name", "_refs")

    def __init__(self, fn, args, name, refs):
        self._fn, self._args, self._name, self._refs = fn, args, name, refs

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != XSTAGE_OK:
            raise XStageError(st, self._name)


def bind(name: str, *args, **kwargs) -> _Bound:
    """Validates and marshals the arguments of entry point ``name`` once and returns a
    zero-argument callable that issues that call.

    Meant for launch loops (benchmarks, serving steps), where the per-call Python checks
    would otherwise cost about as much host time as a short kernel takes on the GPU.  The
    bound buffers are kept alive by the callable; the stream is fixed at bind time (the
    current stream of the tensors' device unless ``stream`` is given), and the calls must be
    made with that device current.  Supported: the attention entry points
    (xstage_attn_a2a_fwd, xstage_attn_fwd, xstage_a2a_scatter, xstage_attn_a2a_unfused,
    xstage_attn_a2a_fwd_traced, xstage_attn_a2a_fwd_paced, xstage_attn_a2a_fwd_nsplit,
    xstage_attn_a2a_fwd_strided, xstage_ulysses_attn_fwd, xstage_ulysses_attn_unfused,
    xstage_ulysses_attn_fwd_kv_staged, xstage_attn_a2a_fwd_noalloc) and
    xstage_moe_waves_run, with the same arguments as the functions.
    """
    import torch

    L = lib()
    if name in _MARSHAL:
        call, refs, dev = _MARSHAL[name](*args, **kwargs)
    elif name == "xstage_moe_waves_run":
        x, w1, w2, h, expert_offsets, dst_slab, dst_row, outs, epw, schedule = args[:10]
        stamps, stream = kwargs.get("stamps", args[10] if len(args) > 10 else None), kwargs.get("stream")
        prm, keep, st_ = _moe_call(x, w1, w2, h, expert_offsets, dst_slab, dst_row, outs, epw, schedule, stamps,
                                   stream)
        call = (ctypes.byref(prm), st_)
        refs, dev = (prm, keep), x.device
    else:
        raise ValueError(f"bind: unsupported entry point {name!r}")
    if torch.cuda.current_device() != dev.index:
        raise ValueError(f"bind: make {dev} the current device first")
    return _Bound(getattr(L, name), call, name, refs)
