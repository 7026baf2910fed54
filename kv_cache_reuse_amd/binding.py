"""ctypes binding of libmac (include/mac.h), argument marshalling only.

Every function here has the name of the C entry point it calls and takes
plain integers (device addresses) and sizes.  ``MacSession`` adds the
plumbing a caller needs on top: it allocates the caller-owned device buffers
with PyTorch (ring, workspace, KV caches, lengths) and passes their addresses
through; every step of the decode path runs in libmac's HIP kernels.

If the shared library has not been built the import of this module fails
loudly: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmac.so")

MAC_OK = 0
MAC_ERR_INVALID_ARG = 1
MAC_ERR_UNSUPPORTED = 2
MAC_ERR_CAPACITY = 3
MAC_ERR_DEVICE = 4
MAC_ERR_STATE = 5

MAC_DTYPE_F32 = 0
MAC_DTYPE_BF16 = 1

MAC_KV_TILES = 0
MAC_KV_ROWS = 1

EXPORTED = (
    "mac_kv_cache_bytes", "mac_ring_bytes", "mac_workspace_bytes", "mac_init",
    "mac_resume", "mac_append_kv", "mac_prefill_kv", "mac_read_kv", "mac_decode_step",
    "mac_decode_step_append", "mac_decode_step_append_noalloc", "mac_seed_ring", "mac_query_cache_push", "mac_profile_enable",
    "mac_profile_read",
    "mac_destroy", "mac_last_error",
)


class MacError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmac status {status}: {message}")
        self.status = status


class MacConfig(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
        ("head_dim", c_int32), ("dtype", c_int32), ("max_context", c_int32),
        ("page_size", c_int32), ("max_pages_per_seq", c_int32), ("n_pages", c_int32),
        ("window", c_int32), ("band", c_int32), ("tau", c_float),
        ("rope_theta", c_double), ("max_slices", c_int32), ("kv_layout", c_int32),
    ]


def _load():
    # torch ships its own HIP runtime; libmac has to bind to the one torch
    # uses (same device memory, same streams), so torch is loaded first
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmac is not built ({LIB_PATH} missing); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "mac_kv_cache_bytes": (c_size_t, [POINTER(MacConfig)]),
        "mac_ring_bytes": (c_size_t, [POINTER(MacConfig)]),
        "mac_workspace_bytes": (c_size_t, [POINTER(MacConfig)]),
        "mac_init": (c_int, [POINTER(MacConfig), P, P, P, P, P, POINTER(c_void_p)]),
        "mac_resume": (c_int, [POINTER(MacConfig), P, P, P, P, P, POINTER(c_void_p)]),
        "mac_append_kv": (c_int, [P, P, P, P, P, P, P]),
        "mac_prefill_kv": (c_int, [P, P, P, P, c_int32, P, P, c_int32, P]),
        "mac_read_kv": (c_int, [P, P, P, P, c_int32, c_int32, c_int32, P, P, P]),
        "mac_decode_step": (c_int, [P, P, P, P, P, P, P, P, P]),
        "mac_decode_step_append": (c_int, [P, P, P, P, P, P, P, P, P, P, P]),
        "mac_decode_step_append_noalloc": (c_int, [P, P, P, P, P, P, P, P, P, P, P]),
        "mac_seed_ring": (c_int, [P, P, c_int32, P, P, P, P]),
        "mac_query_cache_push": (c_int, [P, P, P, P, P, P, P, P, P]),
        "mac_profile_enable": (c_int, [P, c_int]),
        "mac_profile_read": (c_int, [P, POINTER(c_double), POINTER(c_int64)]),
        "mac_destroy": (c_int, [P]),
        "mac_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != MAC_OK:
        raise MacError(status, _lib.mac_last_error().decode())


def library():
    return _lib


# --------------------------------------------------------------------------
# the C entry points, same names
# --------------------------------------------------------------------------

def mac_kv_cache_bytes(cfg: MacConfig) -> int:
    return _lib.mac_kv_cache_bytes(ctypes.byref(cfg))


def mac_ring_bytes(cfg: MacConfig) -> int:
    return _lib.mac_ring_bytes(ctypes.byref(cfg))


def mac_workspace_bytes(cfg: MacConfig) -> int:
    return _lib.mac_workspace_bytes(ctypes.byref(cfg))


def mac_init(cfg: MacConfig, ring: int, workspace: int, seq_lens_dev: int,
             seq_lens_host, stream: int) -> int:
    """Returns the context handle (an opaque integer)."""
    n = cfg.batch
    host = (c_int32 * n)(*[int(x) for x in seq_lens_host])
    out = c_void_p()
    _check(_lib.mac_init(ctypes.byref(cfg), ring, workspace, seq_lens_dev,
                         ctypes.cast(host, c_void_p), stream, ctypes.byref(out)))
    return out.value


def mac_resume(cfg: MacConfig, ring: int, workspace: int, seq_lens_dev: int,
               seq_lens_host, stream: int) -> int:
    """Like mac_init, but the ring's entries are kept (continuing from a
    checkpoint).  Returns the context handle."""
    n = cfg.batch
    host = (c_int32 * n)(*[int(x) for x in seq_lens_host])
    out = c_void_p()
    _check(_lib.mac_resume(ctypes.byref(cfg), ring, workspace, seq_lens_dev,
                           ctypes.cast(host, c_void_p), stream, ctypes.byref(out)))
    return out.value


def mac_append_kv(ctx, k_cache, v_cache, page_table, k_new, v_new, stream):
    _check(_lib.mac_append_kv(ctx, k_cache, v_cache, page_table or None, k_new, v_new, stream))


def mac_prefill_kv(ctx, k_cache, v_cache, page_table, seq, k_src, v_src, count, stream):
    _check(_lib.mac_prefill_kv(ctx, k_cache, v_cache, page_table or None, seq, k_src,
                               v_src, count, stream))


def mac_read_kv(ctx, k_cache, v_cache, page_table, seq, start, count, k_dst, v_dst, stream):
    _check(_lib.mac_read_kv(ctx, k_cache, v_cache, page_table or None, seq, start, count,
                            k_dst, v_dst, stream))


def mac_decode_step(ctx, q_pre, k_cache, v_cache, page_table, out, match_ctx_out,
                    dist_out, stream):
    _check(_lib.mac_decode_step(ctx, q_pre, k_cache, v_cache, page_table or None, out,
                                match_ctx_out or None, dist_out or None, stream))


def mac_decode_step_append(ctx, q_pre, k_new, v_new, k_cache, v_cache, page_table, out,
                           match_ctx_out, dist_out, stream):
    _check(_lib.mac_decode_step_append(ctx, q_pre, k_new, v_new, k_cache, v_cache,
                                       page_table or None, out, match_ctx_out or None,
                                       dist_out or None, stream))


def mac_decode_step_append_noalloc(ctx, q_pre, k_new, v_new, k_cache, v_cache, page_table,
                                   out, match_ctx_out, dist_out, stream):
    _check(_lib.mac_decode_step_append_noalloc(ctx, q_pre, k_new, v_new, k_cache, v_cache,
                                               page_table or None, out, match_ctx_out or None,
                                               dist_out or None, stream))


def mac_seed_ring(ctx, q_hist, n_hist, k_cache, v_cache, page_table, stream):
    _check(_lib.mac_seed_ring(ctx, q_hist, n_hist, k_cache, v_cache, page_table or None, stream))


def mac_query_cache_push(ctx, q_pre, o, m, l, prefix_end, ctx_len, mask, stream):
    _check(_lib.mac_query_cache_push(ctx, q_pre, o, m, l, prefix_end, ctx_len,
                                     mask or None, stream))


def mac_profile_enable(ctx, enable: bool):
    _check(_lib.mac_profile_enable(ctx, 1 if enable else 0))


def mac_profile_read(ctx):
    ms = c_double()
    n = c_int64()
    _check(_lib.mac_profile_read(ctx, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def mac_destroy(ctx):
    _check(_lib.mac_destroy(ctx))


def mac_last_error() -> str:
    return _lib.mac_last_error().decode()


# --------------------------------------------------------------------------
# PyTorch plumbing: caller-owned buffers for one attention layer
# --------------------------------------------------------------------------

def config_from_workload(w, max_context: Optional[int] = None, n_pages: int = 0,
                         max_pages_per_seq: int = 0, max_slices: int = 0,
                         kv_layout: int = MAC_KV_TILES) -> MacConfig:
    c = MacConfig()
    c.batch, c.n_q_heads, c.n_kv_heads = w.batch, w.n_q_heads, w.n_kv_heads
    c.head_dim = w.head_dim
    c.dtype = MAC_DTYPE_F32 if w.dtype == "f32" else MAC_DTYPE_BF16
    c.max_context = max_context or 0
    c.page_size = w.page_size
    c.max_pages_per_seq = max_pages_per_seq
    c.n_pages = n_pages
    c.window, c.band, c.tau = w.window, w.band, float(w.tau)
    c.rope_theta = float(w.rope_theta)
    c.max_slices = max_slices
    c.kv_layout = kv_layout
    return c


class MacSession:
    """One attention layer's libmac state on a CUDA (HIP) device.

    Allocates with torch: the K and V caches (library tile layout), the ring,
    the workspace, the device length array and, when paged, the page table.
    """

    def __init__(self, cfg: MacConfig, device="cuda", page_table=None, stream=None,
                 workspace=None, resume_from=None, no_workspace=False):
        """`workspace`: a uint8 device tensor of mac_workspace_bytes(cfg) to
        use instead of a new one (contexts of identical configs whose calls
        never overlap may share one).  `no_workspace`: bind none (the context
        can then step only through mac_decode_step_append_noalloc).
        `resume_from`: a checkpoint made by `checkpoint()`; its buffers are
        adopted and bound with mac_resume."""
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.dtype = torch.float32 if cfg.dtype == MAC_DTYPE_F32 else torch.bfloat16
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        kvb = mac_kv_cache_bytes(cfg)
        if kvb == 0:
            _lib.mac_kv_cache_bytes(ctypes.byref(cfg))
            raise MacError(MAC_ERR_INVALID_ARG, mac_last_error())
        es = 4 if cfg.dtype == MAC_DTYPE_F32 else 2
        if workspace is None and not no_workspace:
            workspace = torch.empty(mac_workspace_bytes(cfg), dtype=torch.uint8,
                                    device=self.device)
        self.workspace = workspace
        if resume_from is not None:
            ck = resume_from
            self.k_cache, self.v_cache = ck["k_cache"], ck["v_cache"]
            self.ring, self.seq_lens = ck["ring"], ck["seq_lens"]
            host = [int(x) for x in ck["seq_lens_host"]]
            page_table = ck.get("page_table", page_table)
        else:
            self.k_cache = torch.empty(kvb // es, dtype=self.dtype, device=self.device)
            self.v_cache = torch.empty(kvb // es, dtype=self.dtype, device=self.device)
            self.ring = torch.empty(mac_ring_bytes(cfg), dtype=torch.uint8, device=self.device)
            self.seq_lens = torch.zeros(cfg.batch, dtype=torch.int32, device=self.device)
            host = [0] * cfg.batch
        self.page_table = None
        if cfg.page_size:
            if page_table is None:
                raise ValueError("a paged config needs a page table")
            self.page_table = torch.as_tensor(page_table, dtype=torch.int32).to(self.device).contiguous()
        bind = mac_resume if resume_from is not None else mac_init
        self.ctx = bind(cfg, self.ring.data_ptr(),
                        self.workspace.data_ptr() if self.workspace is not None else 0,
                        self.seq_lens.data_ptr(), host, self._s())
        hq, d = cfg.n_q_heads, cfg.head_dim
        self.out = torch.empty((cfg.batch, hq, d), dtype=torch.float32, device=self.device)
        self.match_ctx = torch.empty((cfg.batch, hq), dtype=torch.int32, device=self.device)
        self.dist = torch.empty((cfg.batch, hq), dtype=torch.float32, device=self.device)

    def _s(self) -> int:
        return self.stream.cuda_stream

    def _pt(self) -> int:
        return self.page_table.data_ptr() if self.page_table is not None else 0

    def prefill(self, seq: int, k_src, v_src) -> None:
        """k_src, v_src: device tensors [Hkv, count, d] in the config dtype."""
        k_src = k_src.contiguous()
        v_src = v_src.contiguous()
        mac_prefill_kv(self.ctx, self.k_cache.data_ptr(), self.v_cache.data_ptr(), self._pt(),
                       seq, k_src.data_ptr(), v_src.data_ptr(), k_src.shape[1], self._s())
        self._keep = (k_src, v_src)

    def append(self, k_new, v_new) -> None:
        """k_new, v_new: device tensors [batch, Hkv, d]."""
        mac_append_kv(self.ctx, self.k_cache.data_ptr(), self.v_cache.data_ptr(), self._pt(),
                      k_new.data_ptr(), v_new.data_ptr(), self._s())

    def decode(self, q_pre, out=None, match_ctx=True, dist=True):
        """q_pre: device tensor [batch, Hq, d].  Returns (out, match_ctx, dist)."""
        out = self.out if out is None else out
        mc = self.match_ctx if match_ctx else None
        ds = self.dist if dist else None
        mac_decode_step(self.ctx, q_pre.data_ptr(), self.k_cache.data_ptr(),
                        self.v_cache.data_ptr(), self._pt(), out.data_ptr(),
                        mc.data_ptr() if mc is not None else 0,
                        ds.data_ptr() if ds is not None else 0, self._s())
        return out, mc, ds

    def decode_append(self, q_pre, k_new, v_new, out=None, match_ctx=True, dist=True):
        """Append k_new/v_new [batch, Hkv, d] and decode q_pre in one call."""
        out = self.out if out is None else out
        mc = self.match_ctx if match_ctx else None
        ds = self.dist if dist else None
        mac_decode_step_append(self.ctx, q_pre.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                               self.k_cache.data_ptr(), self.v_cache.data_ptr(), self._pt(),
                               out.data_ptr(), mc.data_ptr() if mc is not None else 0,
                               ds.data_ptr() if ds is not None else 0, self._s())
        return out, mc, ds

    def decode_append_noalloc(self, q_pre, k_new, v_new, out=None, match_ctx=True, dist=True):
        """decode_append through mac_decode_step_append_noalloc (the step's
        scratch is the library's static device array)."""
        out = self.out if out is None else out
        mc = self.match_ctx if match_ctx else None
        ds = self.dist if dist else None
        mac_decode_step_append_noalloc(self.ctx, q_pre.data_ptr(), k_new.data_ptr(),
                                       v_new.data_ptr(), self.k_cache.data_ptr(),
                                       self.v_cache.data_ptr(), self._pt(), out.data_ptr(),
                                       mc.data_ptr() if mc is not None else 0,
                                       ds.data_ptr() if ds is not None else 0, self._s())
        return out, mc, ds

    def read_kv(self, seq: int, start: int, count: int):
        t = self.torch
        k = t.empty((self.cfg.n_kv_heads, count, self.cfg.head_dim), dtype=self.dtype,
                    device=self.device)
        v = t.empty_like(k)
        mac_read_kv(self.ctx, self.k_cache.data_ptr(), self.v_cache.data_ptr(), self._pt(),
                    seq, start, count, k.data_ptr(), v.data_ptr(), self._s())
        return k, v

    def seed(self, q_hist):
        """q_hist: [n_hist, batch, Hq, d] pre-RoPE queries of the last n_hist
        positions of every sequence (contiguous, config dtype, on device)."""
        assert q_hist.is_contiguous() and q_hist.dtype == self.dtype
        mac_seed_ring(self.ctx, q_hist.data_ptr(), int(q_hist.shape[0]), self.k_cache.data_ptr(),
                      self.v_cache.data_ptr(), self._pt(), self._s())

    def push(self, q_pre, o, m, l, prefix_end, ctx_len, mask=None):
        mac_query_cache_push(self.ctx, q_pre.data_ptr(), o.data_ptr(), m.data_ptr(),
                             l.data_ptr(), prefix_end.data_ptr(), ctx_len.data_ptr(),
                             mask.data_ptr() if mask is not None else 0, self._s())

    def checkpoint(self):
        """Byte copies of everything a context carries between steps (ring,
        caches, page table, lengths on device and host).  Synchronizes."""
        t = self.torch
        t.cuda.synchronize(self.device)
        ck = {"ring": self.ring.clone(), "k_cache": self.k_cache.clone(),
              "v_cache": self.v_cache.clone(), "seq_lens": self.seq_lens.clone()}
        if self.page_table is not None:
            ck["page_table"] = self.page_table.clone()
        t.cuda.synchronize(self.device)
        ck["seq_lens_host"] = ck["seq_lens"].cpu().tolist()
        return ck

    def close(self) -> None:
        if getattr(self, "ctx", None):
            mac_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
