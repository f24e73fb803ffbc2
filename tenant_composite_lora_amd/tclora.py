"""Python binding of libtclora (ctypes).

Argument marshalling only: every step of the apply runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream (the current torch
stream of the tensors' device).  The library must be built
(``python -m tenant_composite_lora_amd.build``); nothing here computes a
result on the host, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtclora.so")

OK, EINVAL, EALIGN, ENOSPC, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
MAX_RANK = 64
MAX_PAIRS_PER_GROUP = 64

_NAMES = {OK: "OK", EINVAL: "EINVAL", EALIGN: "EALIGN", ENOSPC: "ENOSPC",
          EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP"}

EXPORTS = ["tcl_last_error", "tcl_version", "tcl_plan_bytes", "tcl_plan_map", "tcl_plan_remap",
           "tcl_plan_status", "tcl_plan_copy_out", "tcl_plan_free", "tcl_module_load_ranks",
           "tcl_workspace_bytes", "tcl_shrink", "tcl_expand", "tcl_fused_apply",
           "tcl_fused_shrink", "tcl_fused_expand", "tcl_remap_apply", "tcl_remap_shrink",
           "tcl_gate_topk", "tcl_factor_workspace_bytes",
           "tcl_factor_balanced", "tcl_rank_uniform", "tcl_rank_spectral",
           "tcl_bam_create", "tcl_bam_free", "tcl_bam_acquire", "tcl_bam_slots", "tcl_lag_select",
           "tcl_module_init", "tcl_composites_validate", "tcl_plan_map_host",
           "tcl_plan_remap_host", "tcl_plan_info", "tcl_plan_status_async",
           "tcl_module_pack_bytes", "tcl_module_pack", "tcl_fused_apply_noalloc",
           "tcl_bam_pool_init", "tcl_bam_load"]

# bytes of the static device workspace of tcl_fused_apply_noalloc
SCRATCH_BYTES = 32 << 20


class TclError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class Composites(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("n_pairs", ctypes.c_int32), ("n_adapters", ctypes.c_int32),
                ("max_tuples", ctypes.c_int32),
                ("group_tok_ptr", ctypes.c_void_p), ("group_pair_ptr", ctypes.c_void_p),
                ("pair_adapter", ctypes.c_void_p), ("pair_alpha", ctypes.c_void_p)]


class ModuleDesc(ctypes.Structure):
    _fields_ = [("n_adapters", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32), ("r_max", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("A_t", ctypes.c_void_p),
                ("B_t", ctypes.c_void_p), ("k_dev", ctypes.c_void_p),
                ("B_k", ctypes.c_void_p)]


_lib = None


def lib(path: Optional[str] = None):
    """Load libtclora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m tenant_composite_lora_amd.build`")
    L = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.tcl_last_error.restype = ctypes.c_char_p
    L.tcl_version.restype = ctypes.c_char_p
    L.tcl_plan_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.tcl_plan_map.argtypes = [ctypes.POINTER(Composites), vp, sz, vp, ctypes.POINTER(vp)]
    L.tcl_plan_remap.argtypes = [vp, ctypes.POINTER(Composites), vp]
    L.tcl_plan_status.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.tcl_plan_copy_out.argtypes = [vp] * 9 + [vp]
    L.tcl_plan_free.argtypes = [vp]
    L.tcl_plan_free.restype = None
    L.tcl_module_load_ranks.argtypes = [ctypes.POINTER(ModuleDesc), vp, vp, vp]
    L.tcl_module_init.argtypes = [ctypes.POINTER(ModuleDesc), vp, vp, vp]
    L.tcl_composites_validate.argtypes = [ctypes.POINTER(Composites), ctypes.POINTER(i32),
                                          ctypes.POINTER(i32)]
    L.tcl_plan_map_host.argtypes = [ctypes.POINTER(Composites), vp, sz, vp, ctypes.POINTER(vp)]
    L.tcl_plan_remap_host.argtypes = [vp, ctypes.POINTER(Composites), vp]
    L.tcl_plan_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.tcl_plan_status_async.argtypes = [vp, vp, vp]
    L.tcl_module_pack_bytes.argtypes = [ctypes.POINTER(ModuleDesc), ctypes.POINTER(sz)]
    L.tcl_module_pack.argtypes = [ctypes.POINTER(ModuleDesc), vp, sz, vp]
    L.tcl_workspace_bytes.argtypes = [vp, ctypes.POINTER(ModuleDesc), i32, ctypes.POINTER(sz)]
    L.tcl_shrink.argtypes = [vp, ctypes.POINTER(ModuleDesc), vp, i64, i32, vp, vp]
    L.tcl_expand.argtypes = [vp, ctypes.POINTER(ModuleDesc), vp, vp, i64, i32, vp]
    L.tcl_fused_apply.argtypes = [vp, ctypes.POINTER(ModuleDesc), i32, ctypes.POINTER(vp),
                                  ctypes.POINTER(i64), i32, ctypes.POINTER(vp),
                                  ctypes.POINTER(i64), i32, vp, sz, vp]
    L.tcl_fused_apply_noalloc.argtypes = [vp, ctypes.POINTER(ModuleDesc), i32,
                                          ctypes.POINTER(vp), ctypes.POINTER(i64), i32,
                                          ctypes.POINTER(vp), ctypes.POINTER(i64), i32, vp]
    L.tcl_fused_shrink.argtypes = [vp, ctypes.POINTER(ModuleDesc), i32, ctypes.POINTER(vp),
                                   ctypes.POINTER(i64), i32, vp, sz, vp]
    L.tcl_fused_expand.argtypes = [vp, ctypes.POINTER(ModuleDesc), i32, vp, sz,
                                   ctypes.POINTER(vp), ctypes.POINTER(i64), i32, vp]
    L.tcl_remap_apply.argtypes = [vp, ctypes.POINTER(Composites), ctypes.POINTER(ModuleDesc),
                                  i32, ctypes.POINTER(vp), ctypes.POINTER(i64), i32,
                                  ctypes.POINTER(vp), ctypes.POINTER(i64), i32, vp, sz, vp]
    L.tcl_remap_shrink.argtypes = [vp, ctypes.POINTER(Composites), ctypes.POINTER(ModuleDesc),
                                   i32, ctypes.POINTER(vp), ctypes.POINTER(i64), i32, vp, sz, vp]
    L.tcl_gate_topk.argtypes = [vp, i64, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp]
    L.tcl_factor_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.tcl_factor_balanced.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.tcl_rank_uniform.argtypes = [vp, vp, i32, i32, vp, ctypes.POINTER(i64)]
    L.tcl_rank_spectral.argtypes = [vp, i64, vp, vp, vp, i32, i64, vp]
    L.tcl_bam_create.argtypes = [i32, ctypes.POINTER(vp)]
    L.tcl_bam_free.argtypes = [vp]
    L.tcl_bam_free.restype = None
    L.tcl_bam_acquire.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
    L.tcl_bam_slots.argtypes = [vp, vp]
    L.tcl_bam_pool_init.argtypes = [ctypes.POINTER(ModuleDesc), vp, vp, sz, vp]
    L.tcl_bam_load.argtypes = [ctypes.POINTER(ModuleDesc), vp, vp, vp, i32, i32, vp, vp, vp]
    L.tcl_lag_select.argtypes = [vp, vp, vp, i32, vp, i32, ctypes.c_double, ctypes.c_double,
                                 i32, i32, vp, vp]
    if path is None:
        _lib = L
    return L


def check(rc: int) -> None:
    if rc != OK:
        raise TclError(rc, lib().tcl_last_error().decode(errors="replace"))


def _stream(dev: torch.device, stream=None) -> int:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    return int(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def plan_bytes(n_tokens: int, n_groups: int, n_pairs: int, n_adapters: int,
               max_tuples: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib().tcl_plan_bytes(n_tokens, n_groups, n_pairs, n_adapters, max_tuples,
                               ctypes.byref(out)))
    return out.value


def _host_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha):
    import numpy as np
    return (np.ascontiguousarray(group_tok_ptr, dtype=np.int32),
            np.ascontiguousarray(group_pair_ptr, dtype=np.int32),
            np.ascontiguousarray(pair_adapter, dtype=np.int32),
            np.ascontiguousarray(pair_alpha, dtype=np.float32))


def _host_composites(arrs, n_tokens: int, n_adapters: int, max_tuples: int) -> Composites:
    gtp, gpp, pa, pw = arrs
    ptr = lambda a: a.ctypes.data if a.size else None  # noqa: E731
    return Composites(int(n_tokens), gtp.shape[0] - 1, pa.shape[0], int(n_adapters),
                      int(max_tuples), ptr(gtp), ptr(gpp), ptr(pa), ptr(pw))


def validate_composites(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                        n_adapters: int, n_tokens: Optional[int] = None,
                        max_tuples: Optional[int] = None):
    """Host-side check of a HOST-resident table (tcl_composites_validate, no
    GPU): returns (status code, tuples, segments)."""
    arrs = _host_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
    T = int(arrs[0][-1]) if n_tokens is None and arrs[0].size else int(n_tokens or 0)
    cap = (1 << 31) - 1 if max_tuples is None else int(max_tuples)
    c = _host_composites(arrs, T, n_adapters, cap)
    P, U = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib().tcl_composites_validate(ctypes.byref(c), ctypes.byref(P), ctypes.byref(U))
    return rc, P.value, U.value


class Plan:
    """A mapped batch: tuples reordered by adapter id plus the token index.

    ``group_tok_ptr``, ``group_pair_ptr``, ``pair_adapter`` (int32) and
    ``pair_alpha`` (float32) are device tensors.  ``max_tuples`` bounds the
    tuple count; if omitted it is taken as n_tokens * max pairs per group
    computed from ``group_pair_ptr`` on the device (a small reduction)."""

    def __init__(self, group_tok_ptr: torch.Tensor, group_pair_ptr: torch.Tensor,
                 pair_adapter: torch.Tensor, pair_alpha: torch.Tensor, n_adapters: int,
                 n_tokens: Optional[int] = None, max_tuples: Optional[int] = None,
                 buf: Optional[torch.Tensor] = None, stream=None):
        dev = group_tok_ptr.device
        self.device = dev
        G = int(group_tok_ptr.shape[0]) - 1
        NP = int(pair_adapter.shape[0])
        if n_tokens is None:
            # the token count is the last CSR entry (a 4-byte read-back)
            n_tokens = int(group_tok_ptr[-1].item()) if group_tok_ptr.numel() else 0
        if max_tuples is None:
            if G > 0:
                tl = (group_tok_ptr[1:] - group_tok_ptr[:-1]).to(torch.int64)
                pl = (group_pair_ptr[1:] - group_pair_ptr[:-1]).to(torch.int64)
                max_tuples = int((tl * pl).sum().item())
            else:
                max_tuples = 0
        T = int(n_tokens)
        self.n_tokens, self.n_groups, self.n_pairs = T, G, NP
        self.n_adapters, self.max_tuples = int(n_adapters), int(max_tuples)
        nbytes = plan_bytes(T, G, NP, n_adapters, self.max_tuples)
        if buf is None:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.buf = buf
        # keep the inputs alive until the mapping kernel has run
        self._inputs = (group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
        self._c = Composites(T, G, NP, int(n_adapters), self.max_tuples,
                             _ptr(group_tok_ptr), _ptr(group_pair_ptr), _ptr(pair_adapter),
                             _ptr(pair_alpha))
        h = ctypes.c_void_p(0)
        check(lib().tcl_plan_map(ctypes.byref(self._c), buf.data_ptr(), buf.numel(),
                                 _stream(dev, stream), ctypes.byref(h)))
        self.handle = h

    def remap(self, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha, n_tokens: int,
              stream=None) -> None:
        G = int(group_tok_ptr.shape[0]) - 1
        NP = int(pair_adapter.shape[0])
        self._inputs = (group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
        self._c = Composites(int(n_tokens), G, NP, self.n_adapters, self.max_tuples,
                             _ptr(group_tok_ptr), _ptr(group_pair_ptr), _ptr(pair_adapter),
                             _ptr(pair_alpha))
        check(lib().tcl_plan_remap(self.handle, ctypes.byref(self._c), _stream(self.device, stream)))
        self.n_tokens, self.n_groups, self.n_pairs = int(n_tokens), G, NP

    @classmethod
    def from_host(cls, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                  n_adapters: int, device, n_tokens: Optional[int] = None,
                  max_tuples: Optional[int] = None, buf: Optional[torch.Tensor] = None,
                  stream=None) -> "Plan":
        """A plan from a HOST-resident table (numpy arrays): validated on the
        host (tcl_plan_map_host), then copied and mapped on the device."""
        import numpy as np
        arrs = _host_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
        gtp, gpp, pa, pw = arrs
        G, NP = gtp.shape[0] - 1, pa.shape[0]
        T = int(gtp[-1]) if n_tokens is None else int(n_tokens)
        if max_tuples is None:
            max_tuples = int((np.diff(gtp.astype(np.int64)) * np.diff(gpp.astype(np.int64))).sum())
        self = cls.__new__(cls)
        self.device = torch.device(device)
        self.n_tokens, self.n_groups, self.n_pairs = T, G, NP
        self.n_adapters, self.max_tuples = int(n_adapters), int(max_tuples)
        nbytes = plan_bytes(T, G, NP, self.n_adapters, self.max_tuples)
        if buf is None:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.buf = buf
        self._inputs = None
        self._c = _host_composites(arrs, T, self.n_adapters, self.max_tuples)
        h = ctypes.c_void_p(0)
        check(lib().tcl_plan_map_host(ctypes.byref(self._c), buf.data_ptr(), buf.numel(),
                                      _stream(self.device, stream), ctypes.byref(h)))
        self.handle = h
        return self

    def remap_host(self, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                   n_tokens: Optional[int] = None, stream=None) -> None:
        """Re-map with a HOST-resident table (tcl_plan_remap_host)."""
        arrs = _host_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
        T = int(arrs[0][-1]) if n_tokens is None else int(n_tokens)
        c = _host_composites(arrs, T, self.n_adapters, self.max_tuples)
        check(lib().tcl_plan_remap_host(self.handle, ctypes.byref(c),
                                        _stream(self.device, stream)))
        self._inputs = None
        self.n_tokens, self.n_groups, self.n_pairs = T, arrs[0].shape[0] - 1, arrs[2].shape[0]

    def info(self):
        """(rc, tuples, segments) known on the host (tcl_plan_info)."""
        P, U = ctypes.c_int32(0), ctypes.c_int32(0)
        rc = lib().tcl_plan_info(self.handle, ctypes.byref(P), ctypes.byref(U))
        return rc, P.value, U.value

    def status_async(self, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Queues a copy of {code, tuples, segments, items} into a device int32
        tensor of 4 entries (tcl_plan_status_async); no synchronisation."""
        if out is None:
            out = torch.empty(4, dtype=torch.int32, device=self.device)
        check(lib().tcl_plan_status_async(self.handle, out.data_ptr(),
                                          _stream(self.device, stream)))
        return out

    def status(self, stream=None):
        P, U = ctypes.c_int32(0), ctypes.c_int32(0)
        rc = lib().tcl_plan_status(self.handle, _stream(self.device, stream), ctypes.byref(P),
                                   ctypes.byref(U))
        return rc, P.value, U.value

    def copy_out(self, stream=None) -> dict:
        """Host copy of the plan arrays (synchronises)."""
        import numpy as np
        rc, P, U = self.status(stream)
        check(rc)
        cap, N, T = self.max_tuples, self.n_adapters, self.n_tokens
        arrs = {
            "tup_token": np.zeros(cap, np.int32), "tup_adapter": np.zeros(cap, np.int32),
            "tup_alpha": np.zeros(cap, np.float32), "tup_slot": np.zeros(cap, np.int32),
            "seg_adapter": np.zeros(N, np.int32), "seg_begin": np.zeros(N + 1, np.int32),
            "tok_ptr": np.zeros(T + 1, np.int32), "tok_tuple": np.zeros(cap, np.int32),
        }
        order = ["tup_token", "tup_adapter", "tup_alpha", "tup_slot", "seg_adapter",
                 "seg_begin", "tok_ptr", "tok_tuple"]
        ptrs = [arrs[k].ctypes.data_as(ctypes.c_void_p) if arrs[k].size else None for k in order]
        check(lib().tcl_plan_copy_out(self.handle, *ptrs, _stream(self.device, stream)))
        return {
            "tup_token": arrs["tup_token"][:P], "tup_adapter": arrs["tup_adapter"][:P],
            "tup_alpha": arrs["tup_alpha"][:P], "tup_slot": arrs["tup_slot"][:P],
            "seg_adapter": arrs["seg_adapter"][:U], "seg_begin": arrs["seg_begin"][:U + 1],
            "tok_ptr": arrs["tok_ptr"], "tok_tuple": arrs["tok_tuple"][:P],
        }

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                lib().tcl_plan_free(h)
            except Exception:  # noqa: BLE001 - interpreter shutdown
                pass
            self.handle = None


class Module:
    """One projection's adapter pool: A_t [N, r_max, d_in], B_t [N, r_max,
    d_out] (rank-major, bf16 or fp32, on the GPU) and optional effective
    ranks k (host ints, loaded to the device once).  bf16 pools also get the
    rank-contiguous copy of B the prefill expand reads (tcl_module_pack)
    unless ``pack`` is False."""

    def __init__(self, A_t: torch.Tensor, B_t: torch.Tensor, k=None, stream=None,
                 pack: bool = True):
        if A_t.dim() != 3 or B_t.dim() != 3 or A_t.shape[:2] != B_t.shape[:2]:
            raise ValueError("A_t and B_t must be [N, r_max, d] with equal N and r_max")
        if A_t.dtype != B_t.dtype:
            raise ValueError("A_t and B_t must share a dtype")
        self.A_t = A_t.contiguous()
        self.B_t = B_t.contiguous()
        N, r, d_in = self.A_t.shape
        d_out = self.B_t.shape[2]
        self.desc = ModuleDesc(N, d_in, d_out, r, _dtype_code(A_t.dtype), self.A_t.data_ptr(),
                               self.B_t.data_ptr(), None)
        self.k_dev = None
        if k is not None:
            import numpy as np
            kh = np.ascontiguousarray(np.asarray(k, dtype=np.int32))
            if kh.shape != (N,):
                raise ValueError("k must have one entry per adapter")
            self.k_dev = torch.empty(N, dtype=torch.int32, device=A_t.device)
            check(lib().tcl_module_init(ctypes.byref(self.desc),
                                        kh.ctypes.data_as(ctypes.c_void_p),
                                        self.k_dev.data_ptr(), _stream(A_t.device, stream)))
        else:
            check(lib().tcl_module_init(ctypes.byref(self.desc), None, None,
                                        _stream(A_t.device, stream)))
        self.B_k = None
        if pack and self.desc.wdtype == BF16:
            nb = ctypes.c_size_t(0)
            check(lib().tcl_module_pack_bytes(ctypes.byref(self.desc), ctypes.byref(nb)))
            self.B_k = torch.empty(max(nb.value // 2, 8), dtype=torch.bfloat16,
                                   device=A_t.device)
            check(lib().tcl_module_pack(ctypes.byref(self.desc), self.B_k.data_ptr(), nb.value,
                                        _stream(A_t.device, stream)))

    @property
    def n_adapters(self):
        return self.desc.n_adapters

    @property
    def d_in(self):
        return self.desc.d_in

    @property
    def d_out(self):
        return self.desc.d_out

    @property
    def r_max(self):
        return self.desc.r_max


def shrink(plan: Plan, m: Module, x: torch.Tensor, z: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """z [max_tuples, r_max] fp32 in the plan's sorted-tuple order."""
    if z is None:
        z = torch.empty((max(plan.max_tuples, 1), m.r_max), dtype=torch.float32, device=x.device)
    check(lib().tcl_shrink(plan.handle, ctypes.byref(m.desc), x.data_ptr(), x.stride(0),
                           _dtype_code(x.dtype), z.data_ptr(), _stream(x.device, stream)))
    return z


def expand(plan: Plan, m: Module, z: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y += aggregated alpha * B z, in place."""
    check(lib().tcl_expand(plan.handle, ctypes.byref(m.desc), z.data_ptr(), y.data_ptr(),
                           y.stride(0), _dtype_code(y.dtype), _stream(y.device, stream)))
    return y


def workspace_bytes(plan: Plan, mods: Sequence[Module]) -> int:
    arr = (ModuleDesc * len(mods))(*[m.desc for m in mods])
    out = ctypes.c_size_t(0)
    check(lib().tcl_workspace_bytes(plan.handle, arr, len(mods), ctypes.byref(out)))
    return out.value


class FusedCall:
    """Pre-marshalled arguments of tcl_fused_apply for repeated calls."""

    def __init__(self, plan: Plan, mods: Sequence[Module], xs: Sequence[torch.Tensor],
                 ys: Sequence[torch.Tensor], ws: Optional[torch.Tensor] = None):
        n = len(mods)
        assert len(xs) == n and len(ys) == n
        self.plan, self.mods, self.xs, self.ys = plan, list(mods), list(xs), list(ys)
        self.descs = (ModuleDesc * n)(*[m.desc for m in mods])
        self.xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
        self.yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
        self.ldx = (ctypes.c_int64 * n)(*[x.stride(0) for x in xs])
        self.ldy = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
        self.xd = _dtype_code(xs[0].dtype)
        self.yd = _dtype_code(ys[0].dtype)
        need = workspace_bytes(plan, mods)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device=xs[0].device)
        self.ws = ws
        self.n = n

    def __call__(self, stream=None):
        check(lib().tcl_fused_apply(self.plan.handle, self.descs, self.n, self.xp, self.ldx,
                                    self.xd, self.yp, self.ldy, self.yd, self.ws.data_ptr(),
                                    self.ws.numel(), _stream(self.xs[0].device, stream)))

    def noalloc(self, stream=None):
        """The same apply through tcl_fused_apply_noalloc: the library's static
        device workspace instead of self.ws."""
        check(lib().tcl_fused_apply_noalloc(self.plan.handle, self.descs, self.n, self.xp,
                                            self.ldx, self.xd, self.yp, self.ldy, self.yd,
                                            _stream(self.xs[0].device, stream)))

    def shrink(self, stream=None):
        """First half only: z of every module into the workspace."""
        check(lib().tcl_fused_shrink(self.plan.handle, self.descs, self.n, self.xp, self.ldx,
                                     self.xd, self.ws.data_ptr(), self.ws.numel(),
                                     _stream(self.xs[0].device, stream)))

    def expand(self, stream=None):
        """Second half only: y += aggregated alpha * B z from the workspace."""
        check(lib().tcl_fused_expand(self.plan.handle, self.descs, self.n, self.ws.data_ptr(),
                                     self.ws.numel(), self.yp, self.ldy, self.yd,
                                     _stream(self.xs[0].device, stream)))

    def _remap_table(self, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha, n_tokens):
        plan = self.plan
        G = int(group_tok_ptr.shape[0]) - 1
        NP = int(pair_adapter.shape[0])
        plan._inputs = (group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha)
        plan._c = Composites(int(n_tokens), G, NP, plan.n_adapters, plan.max_tuples,
                             _ptr(group_tok_ptr), _ptr(group_pair_ptr), _ptr(pair_adapter),
                             _ptr(pair_alpha))
        return G, NP

    def remap_apply(self, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                    n_tokens: int, stream=None):
        """One step (tcl_remap_apply): re-map the plan with this composite
        table, then shrink and expand every module."""
        plan = self.plan
        G, NP = self._remap_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                                  n_tokens)
        check(lib().tcl_remap_apply(plan.handle, ctypes.byref(plan._c), self.descs, self.n,
                                    self.xp, self.ldx, self.xd, self.yp, self.ldy, self.yd,
                                    self.ws.data_ptr(), self.ws.numel(),
                                    _stream(self.xs[0].device, stream)))
        plan.n_tokens, plan.n_groups, plan.n_pairs = int(n_tokens), G, NP

    def remap_shrink(self, group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                     n_tokens: int, stream=None):
        """First half of a step (tcl_remap_shrink); expand() completes it."""
        plan = self.plan
        G, NP = self._remap_table(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
                                  n_tokens)
        check(lib().tcl_remap_shrink(plan.handle, ctypes.byref(plan._c), self.descs, self.n,
                                     self.xp, self.ldx, self.xd, self.ws.data_ptr(),
                                     self.ws.numel(), _stream(self.xs[0].device, stream)))
        plan.n_tokens, plan.n_groups, plan.n_pairs = int(n_tokens), G, NP


def fused_apply(plan: Plan, mods: Sequence[Module], xs: Sequence[torch.Tensor],
                ys: Sequence[torch.Tensor], ws: Optional[torch.Tensor] = None,
                stream=None) -> List[torch.Tensor]:
    FusedCall(plan, mods, xs, ys, ws)(stream)
    return list(ys)


def gate_topk(logits: torch.Tensor, candidates: torch.Tensor, k: int, stream=None):
    """tcl_gate_topk: the composite table of a token-level gate on the GPU.
    logits: fp32 [T, C]; candidates: int32 [T, C] adapter ids (< 0 = padding).
    Returns (group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha), device
    tensors ready for Plan / Plan.remap / FusedCall.remap_apply."""
    if logits.dim() != 2 or candidates.shape != logits.shape:
        raise ValueError("logits and candidates must both be [T, C]")
    if logits.dtype != torch.float32 or candidates.dtype != torch.int32:
        raise ValueError("logits must be float32 and candidates int32")
    T, C = logits.shape
    if T > 0 and (logits.stride(1) != 1 or candidates.stride(1) != 1):
        raise ValueError("logits and candidates must have contiguous rows")
    ldl, ldc = (logits.stride(0), candidates.stride(0)) if T > 0 else (C, C)
    dev = logits.device
    gtp = torch.empty(T + 1, dtype=torch.int32, device=dev)
    gpp = torch.empty(T + 1, dtype=torch.int32, device=dev)
    pa = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    pw = torch.empty(max(T * k, 1), dtype=torch.float32, device=dev)
    check(lib().tcl_gate_topk(logits.data_ptr(), ldl, candidates.data_ptr(),
                              ldc, T, C, k, gtp.data_ptr(), gpp.data_ptr(),
                              pa.data_ptr(), pw.data_ptr(), _stream(dev, stream)))
    return gtp, gpp, pa[:T * k], pw[:T * k]


def factor_balanced(B_t: torch.Tensor, A_t: torch.Tensor, stream=None):
    """tcl_factor_balanced: balanced factors of a batch of modules of one
    shape (LoRAForge, approach (3)).  B_t: bf16 [M, r, d_out] and A_t: bf16
    [M, r, d_in], contiguous, on one device.  Returns (F_t, T, sigma): the
    new B_t and A_t rows (bf16, same shapes), directions largest first, and
    the singular values (fp32 [M, r])."""
    if B_t.dtype != torch.bfloat16 or A_t.dtype != torch.bfloat16:
        raise TypeError("factor_balanced: B_t and A_t must be bfloat16")
    if B_t.dim() != 3 or A_t.dim() != 3 or B_t.shape[:2] != A_t.shape[:2]:
        raise ValueError("factor_balanced: B_t [M, r, d_out] and A_t [M, r, d_in] expected")
    if not (B_t.is_contiguous() and A_t.is_contiguous()):
        raise ValueError("factor_balanced: contiguous tensors expected")
    M, r, d_out = B_t.shape
    d_in = A_t.shape[2]
    L = lib()
    nb = ctypes.c_size_t()
    check(L.tcl_factor_workspace_bytes(M, d_out, d_in, r, ctypes.byref(nb)))
    dev = B_t.device
    F_t = torch.empty_like(B_t)
    T = torch.empty_like(A_t)
    sigma = torch.empty(M, r, dtype=torch.float32, device=dev)
    ws = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    check(L.tcl_factor_balanced(B_t.data_ptr(), A_t.data_ptr(), M, d_out, d_in, r,
                                F_t.data_ptr(), T.data_ptr(), sigma.data_ptr(), ws.data_ptr(),
                                nb.value, int(st.cuda_stream)))
    return F_t, T, sigma


def rank_uniform(ranks, costs, denominator: int):
    """tcl_rank_uniform (host): LoRAForge-U's kept ranks and budget P_U."""
    import numpy as np
    rk = np.ascontiguousarray(ranks, dtype=np.int32)
    cs = np.ascontiguousarray(costs, dtype=np.int64)
    u = np.empty(len(rk), dtype=np.int32)
    b = ctypes.c_int64()
    check(lib().tcl_rank_uniform(rk.ctypes.data, cs.ctypes.data, len(rk), int(denominator),
                                 u.ctypes.data, ctypes.byref(b)))
    return u, int(b.value)


def rank_spectral(sigma, ranks, costs, floors, budget: int):
    """tcl_rank_spectral (host): LoRAForge-S's kept ranks.  sigma: float64
    [M, ld] (row m's first ranks[m] entries are module m's spectrum)."""
    import numpy as np
    sg = np.ascontiguousarray(sigma, dtype=np.float64)
    rk = np.ascontiguousarray(ranks, dtype=np.int32)
    cs = np.ascontiguousarray(costs, dtype=np.int64)
    fl = np.ascontiguousarray(floors, dtype=np.int32)
    k = np.empty(len(rk), dtype=np.int32)
    ld = sg.shape[1] if sg.ndim == 2 else 0
    check(lib().tcl_rank_spectral(sg.ctypes.data, ld, rk.ctypes.data, cs.ctypes.data,
                                  fl.ctypes.data, len(rk), int(budget), k.ctypes.data))
    return k


class Bam:
    """tcl_bam_*: the adapter slot pool (host bookkeeping; the caller copies
    each loaded adapter into its slot)."""

    def __init__(self, n_slots: int):
        self.n_slots = int(n_slots)
        h = ctypes.c_void_p()
        check(lib().tcl_bam_create(self.n_slots, ctypes.byref(h)))
        self._h = h

    def acquire(self, adapters):
        """Returns (slot of each entry, [(slot, loaded adapter, evicted or -1)])."""
        import numpy as np
        a = np.ascontiguousarray(adapters, dtype=np.int32)
        n = len(a)
        so, ls, la, le = (np.empty(max(n, 1), np.int32) for _ in range(4))
        nl = ctypes.c_int32()
        check(lib().tcl_bam_acquire(self._h, a.ctypes.data, n, so.ctypes.data, ls.ctypes.data,
                                    la.ctypes.data, le.ctypes.data, ctypes.byref(nl)))
        k = nl.value
        return so[:n].copy(), list(zip(ls[:k].tolist(), la[:k].tolist(), le[:k].tolist()))

    def slots(self):
        import numpy as np
        out = np.empty(self.n_slots, np.int32)
        check(lib().tcl_bam_slots(self._h, out.ctypes.data))
        return out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.tcl_bam_free(h)
            self._h = None


class SlotPool:
    """BAM on the GPU: n_slots device slots per module, filled from host pools.

    ``host_pools``: one (A_t, B_t, k) per module, A_t [N, r_max, d_in] and
    B_t [N, r_max, d_out] CPU tensors (bf16 or fp32; copied once into pinned
    memory here) over the N logical adapters, k their retained ranks (ints,
    or None for r_max).  ``modules`` are the device slot pools (tcl_module
    descriptors whose adapter ids are slots); load() makes a batch's adapters
    resident (tcl_bam_acquire, then tcl_bam_load for every module) and
    returns the slot of each adapter."""

    def __init__(self, n_slots: int, host_pools, device, stream=None):
        import numpy as np
        self.bam = Bam(n_slots)
        self.device = torch.device(device)
        self.n_logical = int(host_pools[0][0].shape[0])
        self.modules, self._host, self.h2d_bytes = [], [], 0
        for A_h, B_h, k in host_pools:
            if A_h.shape[0] != self.n_logical or B_h.shape[0] != self.n_logical:
                raise ValueError("every host pool holds the same logical adapters")
            A_p, B_p = A_h.contiguous().pin_memory(), B_h.contiguous().pin_memory()
            kh = None if k is None else np.ascontiguousarray(np.asarray(k, dtype=np.int32))
            _, r, d_in = A_p.shape
            d_out = B_p.shape[2]
            A_t = torch.zeros(n_slots, r, d_in, dtype=A_p.dtype, device=self.device)
            B_t = torch.zeros(n_slots, r, d_out, dtype=B_p.dtype, device=self.device)
            mod = Module(A_t, B_t, pack=False)
            mod.k_dev = torch.empty(n_slots, dtype=torch.int32, device=self.device)
            if mod.desc.wdtype == BF16:
                nb = ctypes.c_size_t(0)
                check(lib().tcl_module_pack_bytes(ctypes.byref(mod.desc), ctypes.byref(nb)))
                mod.B_k = torch.empty(max(nb.value // 2, 8), dtype=torch.bfloat16,
                                      device=self.device)
                bk, nbytes = mod.B_k.data_ptr(), nb.value
            else:
                bk, nbytes = None, 0
            check(lib().tcl_bam_pool_init(ctypes.byref(mod.desc), mod.k_dev.data_ptr(), bk,
                                          nbytes, _stream(self.device, stream)))
            self.modules.append(mod)
            self._host.append((A_p, B_p, kh))

    def load(self, adapters, stream=None):
        """Slots for the adapters of one batch (in the order given); the loads
        are queued on the stream.  Returns (slot of each entry, loads)."""
        import numpy as np
        slot_of, loads = self.bam.acquire(adapters)
        if loads:
            ls = np.ascontiguousarray([l[0] for l in loads], dtype=np.int32)
            la = np.ascontiguousarray([l[1] for l in loads], dtype=np.int32)
            for mod, (A_p, B_p, kh) in zip(self.modules, self._host):
                check(lib().tcl_bam_load(ctypes.byref(mod.desc), A_p.data_ptr(), B_p.data_ptr(),
                                         None if kh is None else kh.ctypes.data,
                                         self.n_logical, len(loads), ls.ctypes.data,
                                         la.ctypes.data, _stream(self.device, stream)))
                es = A_p.element_size()
                ks = [mod.r_max if kh is None else int(kh[a]) for a in la.tolist()]
                self.h2d_bytes += sum(ks) * (mod.d_in + mod.d_out) * es
        return slot_of, loads


def lag_select(now: float, theta: float, arrival, adapters, resident, max_batch: int,
               n_slots: int):
    """tcl_lag_select (host): the chosen request indices, in order."""
    import numpy as np
    arr = np.ascontiguousarray(arrival, dtype=np.float64)
    n = len(arr)
    ptr = np.zeros(n + 1, np.int32)
    ptr[1:] = np.cumsum([len(a) for a in adapters]) if n else []
    flat = np.ascontiguousarray(np.concatenate([np.asarray(a, np.int32) for a in adapters])
                                if n and ptr[-1] else np.zeros(1, np.int32), dtype=np.int32)
    res = np.ascontiguousarray(resident, dtype=np.int32) if len(resident) else np.zeros(1, np.int32)
    out = np.empty(max(1, min(int(max_batch), n)), np.int32)
    nc = ctypes.c_int32()
    check(lib().tcl_lag_select(arr.ctypes.data if n else None, ptr.ctypes.data, flat.ctypes.data,
                               n, res.ctypes.data, len(resident), float(now), float(theta),
                               int(max_batch), int(n_slots), out.ctypes.data, ctypes.byref(nc)))
    return out[:nc.value].tolist()
