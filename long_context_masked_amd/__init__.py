"""MI355X-native masked attention (forward and backward) for long contexts.

Python face of libattn.so (include/attn.h).  PyTorch supplies device memory
and the current stream; every step of the computation (mask compilation,
forward, backward) runs in the library.  There is no fallback path: if the
library is not built, every call raises.

    plan = Plan(B, S, Hq, Hkv, d, mask_spec)        # compile + upload the mask
    o, lse = fwd(plan, q, k, v)                      # q [B,S,Hq,d] bf16, k/v [B,S,Hkv,d]
    dq, dk, dv = bwd(plan, q, k, v, o, lse, do)
"""
from __future__ import annotations

import collections
import ctypes as C

import numpy as np

from . import _lib as L
from .masks import MaskDescriptor, column_bounds  # noqa: F401

__all__ = ["Plan", "fwd", "bwd", "attention", "MaskDescriptor", "column_bounds",
           "AttnError", "library_path", "fwd_partial", "merge", "fwd_desc", "bwd_desc",
           "desc_cache_clear"]

AttnError = L.AttnError
library_path = L.LIB_PATH


class Plan:
    """A compiled mask for one shape: work lists, bounds and bitmap.

    Creation runs on the host only; ``bind()`` (called lazily by fwd/bwd)
    uploads the metadata into a torch-allocated device buffer.
    """

    def __init__(self, B, S, Hq, Hkv, d, mask, scale=0.0):
        self.shape = (int(B), int(S), int(Hq), int(Hkv), int(d))
        self.desc = mask if isinstance(mask, MaskDescriptor) else MaskDescriptor(mask)
        if self.desc.S != int(S):
            raise ValueError(f"mask is for S={self.desc.S}, shape has S={S}")
        sh = L.Shape(int(B), int(S), int(Hq), int(Hkv), int(d), float(scale))
        h = C.c_void_p()
        L.check(L.lib().attn_plan_create(C.byref(sh), C.byref(self.desc.c), C.byref(h)))
        self._h = h
        st = L.Stats()
        L.check(L.lib().attn_plan_stats(h, C.byref(st)))
        self.stats = {name: getattr(st, name) for name, _ in L.Stats._fields_}
        self._dev = None
        self._dev_index = None
        self._dev_off = 0
        # bumped by set_bitmap: a backward must see the mask its forward saw
        self.bitmap_generation = 0

    @property
    def handle(self):
        return self._h

    def device_bytes(self):
        return int(L.lib().attn_plan_device_bytes(self._h))

    def workspace_bytes(self):
        return int(L.lib().attn_bwd_workspace_bytes(self._h))

    def atomic_workspace_bytes(self):
        return int(L.lib().attn_bwd_atomic_workspace_bytes(self._h))

    def bind(self, device=None):
        import torch
        dev = torch.device("cuda" if device is None else device)
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        if self._dev is not None and self._dev_index == idx:
            return self
        n = self.device_bytes()
        buf = torch.empty(max(n, 256) + 256, dtype=torch.uint8, device=dev)
        ptr = buf.data_ptr()
        off = (-ptr) % 256
        stream = torch.cuda.current_stream(dev).cuda_stream
        L.check(L.lib().attn_plan_bind(self._h, C.c_void_p(ptr + off), C.c_size_t(n),
                                       C.c_void_p(stream)))
        self._dev, self._dev_index, self._dev_off = buf, idx, off
        return self

    def set_bitmap(self, bits):
        """Replace the block bitmap of a dynamic plan (created with
        ``"dynamic": True`` in its mask spec) by ``bits``, a uint8 or bool GPU
        tensor [bitmap_heads, n_qblk, n_kblk], and rebuild the work lists on
        the GPU, on the current stream."""
        import torch
        d = self.desc.c
        shape = (int(d.bitmap_heads), int(d.n_qblk), int(d.n_kblk))
        if bits.dtype not in (torch.uint8, torch.bool) or not bits.is_cuda:
            raise TypeError("bits must be a uint8 or bool GPU tensor")
        if tuple(bits.shape) != shape or not bits.is_contiguous():
            raise ValueError(f"bits must be contiguous with shape {shape}")
        self.bind(bits.device)
        stream = torch.cuda.current_stream(bits.device).cuda_stream
        L.check(L.lib().attn_plan_set_bitmap(self._h, C.c_void_p(bits.data_ptr()),
                                             C.c_void_p(stream)))
        self.bitmap_generation += 1
        return self

    def layout(self):
        """Host copy of the blob's sections as numpy arrays (as created)."""
        lay = L.Layout()
        L.check(L.lib().attn_plan_get_layout(self._h, C.byref(lay)))
        raw = np.ctypeslib.as_array((C.c_uint8 * lay.blob_bytes).from_address(lay.blob)).copy()
        return self._sections(lay, raw)

    def device_layout(self):
        """The same sections read back from the bound device buffer (after
        set_bitmap they hold the rebuilt lists)."""
        import torch
        if self._dev is None:
            raise RuntimeError("plan is not bound")
        lay = L.Layout()
        L.check(L.lib().attn_plan_get_layout(self._h, C.byref(lay)))
        torch.cuda.current_stream(self._dev.device).synchronize()
        raw = self._dev[self._dev_off:self._dev_off + lay.blob_bytes].cpu().numpy()
        return self._sections(lay, raw)

    def _sections(self, lay, raw):
        S = self.shape[1]

        def i32(off, n):
            return raw[off:off + 4 * n].view(np.int32)

        out = {
            "rowb": i32(lay.off_rowb, 4 * S).reshape(S, 4),
            "colb": i32(lay.off_colb, 4 * S).reshape(S, 4),
            "fwd_items": i32(lay.off_fwd_items, 4 * lay.n_fwd_items).reshape(-1, 4),
            "fwd_list": raw[lay.off_fwd_list:lay.off_fwd_list + 4 * lay.n_fwd_list].view(np.uint32),
            "bwd_items": i32(lay.off_bwd_items, 4 * lay.n_bwd_items).reshape(-1, 4),
            "bwd_list": raw[lay.off_bwd_list:lay.off_bwd_list + 4 * lay.n_bwd_list].view(np.uint32),
            "bwd_slot": i32(lay.off_bwd_slot, lay.n_bwd_items),
            "bwd_reduce": i32(lay.off_bwd_reduce, 4 * lay.n_bwd_reduce).reshape(-1, 4),
            "n_slots": int(lay.n_slots),
        }
        if lay.off_kwords >= 0:
            # bitmap words: [heads][n_qblk][nM] allowed keys, [heads][n_kblk][nM] allowed rows
            c, nM = self.desc.c, (S + 63) // 64
            nk, nr = c.bitmap_heads * c.n_qblk * nM, c.bitmap_heads * c.n_kblk * nM
            out["kwords"] = raw[lay.off_kwords:lay.off_kwords + 8 * nk].view(np.uint64).reshape(
                c.bitmap_heads, c.n_qblk, nM)
            out["rwords"] = raw[lay.off_rwords:lay.off_rwords + 8 * nr].view(np.uint64).reshape(
                c.bitmap_heads, c.n_kblk, nM)
        return out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                L.lib().attn_plan_destroy(h)
            except Exception:
                pass
            self._h = None


def _check_tensor(t, name, shape, torch):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def fwd(plan, q, k, v=None, out=None, lse=None):
    """O [B,S,Hq,d] bf16 and LSE [B,Hq,S] fp32 (natural log).

    ``fwd(plan, q, k, v)`` runs on a compiled Plan; ``fwd(q, k, v, mask)``
    takes the mask spec (or MaskDescriptor) and uses the library's plan
    cache (fwd_desc)."""
    if not isinstance(plan, Plan):
        return fwd_desc(plan, q, k, v, out=out, lse=lse)
    import torch
    B, S, Hq, Hkv, d = plan.shape
    _check_tensor(q, "q", (B, S, Hq, d), torch)
    _check_tensor(k, "k", (B, S, Hkv, d), torch)
    _check_tensor(v, "v", (B, S, Hkv, d), torch)
    plan.bind(q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    L.check(L.lib().attn_fwd(plan.handle, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                             C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()),
                             C.c_void_p(lse.data_ptr()), C.c_void_p(stream)))
    return o, lse


def bwd(plan, q, k, v, o, lse, do, workspace=None, grads=None, atomic_dq=False):
    """dQ, dK, dV (bf16) from the forward's O and LSE and the output gradient dO.

    ``bwd(plan, q, k, v, o, lse, do)`` runs on a compiled Plan;
    ``bwd(q, k, v, o, lse, do, mask)`` takes the mask and uses the plan cache
    (bwd_desc).  ``atomic_dq=True`` accumulates dQ inside the dK/dV pass with
    fp32 atomics (attn_bwd_atomic_dq) instead of the separate dQ pass."""
    if not isinstance(plan, Plan):
        if grads is not None or atomic_dq:
            raise ValueError("grads= and atomic_dq= are only for the Plan form")
        return bwd_desc(plan, q, k, v, o, lse, do, workspace=workspace)
    import torch
    B, S, Hq, Hkv, d = plan.shape
    for t, n, s in ((q, "q", (B, S, Hq, d)), (k, "k", (B, S, Hkv, d)), (v, "v", (B, S, Hkv, d)),
                    (o, "o", (B, S, Hq, d)), (do, "do", (B, S, Hq, d))):
        _check_tensor(t, n, s, torch)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, S]")
    plan.bind(q.device)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
    nws = plan.atomic_workspace_bytes() if atomic_dq else plan.workspace_bytes()
    ws = torch.empty(nws + 256, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    wptr = ws.data_ptr()
    wptr += (-wptr) % 256
    stream = torch.cuda.current_stream(q.device).cuda_stream
    P = C.c_void_p
    fn = L.lib().attn_bwd_atomic_dq if atomic_dq else L.lib().attn_bwd
    L.check(fn(plan.handle, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
               P(o.data_ptr()), P(lse.data_ptr()), P(do.data_ptr()),
               P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), P(wptr),
               C.c_size_t(nws), P(stream)))
    return dq, dk, dv


def fwd_partial(plan: Plan, q, k, v, out=None, lse=None):
    """The forward over the keys the plan's mask keeps, with O in fp32
    [B,S,Hq,d] (to be merged with other chunks) and LSE [B,Hq,S]."""
    import torch
    B, S, Hq, Hkv, d = plan.shape
    _check_tensor(q, "q", (B, S, Hq, d), torch)
    _check_tensor(k, "k", (B, S, Hkv, d), torch)
    _check_tensor(v, "v", (B, S, Hkv, d), torch)
    plan.bind(q.device)
    o = torch.empty((B, S, Hq, d), dtype=torch.float32, device=q.device) if out is None else out
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    P = C.c_void_p
    L.check(L.lib().attn_fwd_partial(plan.handle, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                                     P(o.data_ptr()), P(lse.data_ptr()), P(stream)))
    return o, lse


def merge(o1, lse1, o2, lse2, bf16_out=False, out=None, lse_out=None):
    """O and LSE over the union of two disjoint key sets from the results
    over each set (fp32 O [B,S,Hq,d], LSE [B,Hq,S]); the merged O is fp32,
    or bf16 with bf16_out (the final result, as attn_fwd returns it)."""
    import torch
    B, S, Hq, d = o1.shape
    for t, n in ((o1, "o1"), (o2, "o2")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, S, Hq, d) or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous float32 [B, S, Hq, d]")
    for t, n in ((lse1, "lse1"), (lse2, "lse2")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, Hq, S) or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous float32 [B, Hq, S]")
    dt = torch.bfloat16 if bf16_out else torch.float32
    o = torch.empty((B, S, Hq, d), dtype=dt, device=o1.device) if out is None else out
    lse = torch.empty_like(lse1) if lse_out is None else lse_out
    stream = torch.cuda.current_stream(o1.device).cuda_stream
    P = C.c_void_p
    L.check(L.lib().attn_merge(P(o1.data_ptr()), P(lse1.data_ptr()), P(o2.data_ptr()),
                               P(lse2.data_ptr()), P(o.data_ptr()), int(bool(bf16_out)),
                               P(lse.data_ptr()), B, S, Hq, d, P(stream)))
    return o, lse


# Plan buffers of the descriptor calls: one torch buffer per (device, mask
# content hash, size), least recently used dropped first; the library is
# told before a buffer is dropped.
_DESC_BUFS = collections.OrderedDict()
_DESC_BUF_LIMIT = 32


def _aligned(buf):
    ptr = buf.data_ptr()
    return ptr + (-ptr) % 256


def _desc_setup(q, k, mask, scale):
    """(shape struct, descriptor, plan buffer pointer, plan bytes, workspace bytes)."""
    import torch
    B, S, Hq, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[2])
    desc = mask if isinstance(mask, MaskDescriptor) else MaskDescriptor(mask)
    sh = L.Shape(B, S, Hq, Hkv, d, float(scale))
    pb, wb, kh = C.c_size_t(), C.c_size_t(), C.c_uint64()
    L.check(L.lib().attn_desc_plan_bytes(C.byref(sh), C.byref(desc.c), C.byref(pb), C.byref(wb),
                                         C.byref(kh)))
    idx = q.device.index if q.device.index is not None else torch.cuda.current_device()
    key = (idx, kh.value, pb.value)
    buf = _DESC_BUFS.get(key)
    if buf is None:
        buf = torch.empty(max(pb.value, 256) + 256, dtype=torch.uint8, device=q.device)
        _DESC_BUFS[key] = buf
        while len(_DESC_BUFS) > _DESC_BUF_LIMIT:
            _, old = _DESC_BUFS.popitem(last=False)
            L.lib().attn_desc_release(C.c_void_p(_aligned(old)))
    else:
        _DESC_BUFS.move_to_end(key)
    return sh, desc, _aligned(buf), pb.value, wb.value


def fwd_desc(q, k, v, mask, scale=0.0, out=None, lse=None):
    """fwd() from the mask spec (or MaskDescriptor) directly: the library
    compiles each distinct mask once and caches it (attn_fwd_desc)."""
    import torch
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    _check_tensor(q, "q", (B, S, Hq, d), torch)
    _check_tensor(k, "k", (B, S, Hkv, d), torch)
    _check_tensor(v, "v", (B, S, Hkv, d), torch)
    sh, desc, pbuf, pbytes, _ = _desc_setup(q, k, mask, scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    P = C.c_void_p
    L.check(L.lib().attn_fwd_desc(C.byref(sh), C.byref(desc.c), P(q.data_ptr()), P(k.data_ptr()),
                                  P(v.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()), P(pbuf),
                                  C.c_size_t(pbytes), P(stream)))
    return o, lse


def bwd_desc(q, k, v, o, lse, do, mask, scale=0.0, workspace=None):
    """bwd() from the mask spec (or MaskDescriptor) directly (attn_bwd_desc)."""
    import torch
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    for t, n, s in ((q, "q", (B, S, Hq, d)), (k, "k", (B, S, Hkv, d)), (v, "v", (B, S, Hkv, d)),
                    (o, "o", (B, S, Hq, d)), (do, "do", (B, S, Hq, d))):
        _check_tensor(t, n, s, torch)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, S]")
    sh, desc, pbuf, pbytes, nws = _desc_setup(q, k, mask, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(nws + 256, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    P = C.c_void_p
    L.check(L.lib().attn_bwd_desc(C.byref(sh), C.byref(desc.c), P(q.data_ptr()), P(k.data_ptr()),
                                  P(v.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()),
                                  P(do.data_ptr()), P(dq.data_ptr()), P(dk.data_ptr()),
                                  P(dv.data_ptr()), P(_aligned(ws)), C.c_size_t(nws), P(pbuf),
                                  C.c_size_t(pbytes), P(stream)))
    return dq, dk, dv


def desc_cache_clear():
    """Drop every cached plan and plan buffer of the descriptor calls."""
    for buf in _DESC_BUFS.values():
        L.lib().attn_desc_release(C.c_void_p(_aligned(buf)))
    _DESC_BUFS.clear()
    L.lib().attn_desc_cache_clear()


def attention(q, k, v, plan):
    """Differentiable masked attention through torch.autograd; ``plan`` is a
    Plan or a mask spec / MaskDescriptor (then the plan cache is used).  A
    dynamic plan whose bitmap is replaced between the forward and the
    backward raises in the backward instead of differentiating another
    mask."""
    import torch

    class _Attn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_):
            if isinstance(plan, Plan):
                ctx.generation = plan.bitmap_generation
                o, lse = fwd(plan, q_, k_, v_)
            else:
                o, lse = fwd_desc(q_, k_, v_, plan)
            ctx.save_for_backward(q_, k_, v_, o, lse)
            return o

        @staticmethod
        def backward(ctx, do):
            q_, k_, v_, o, lse = ctx.saved_tensors
            if isinstance(plan, Plan):
                if plan.bitmap_generation != ctx.generation:
                    raise RuntimeError("the plan's bitmap was replaced (set_bitmap) after the forward; "
                                       "the backward would differentiate another mask")
                return bwd(plan, q_, k_, v_, o, lse, do.contiguous())
            return bwd_desc(q_, k_, v_, o, lse, do.contiguous(), plan)

    return _Attn.apply(q, k, v)
