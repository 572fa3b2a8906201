"""ctypes binding of libhisparse.so (the C ABI in include/hisparse.h).

Argument marshalling only: every step of the decode path runs in the HIP library.
PyTorch is used for device memory and streams.  The library must be built
(``python -m sparse_mla_attention_score_amd.build``); importing this module
without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhisparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_OUT_OF_MEMORY, HS_ERR_HIP, HS_ERR_STATE = \
    0, -1, -2, -3, -4, -5
HS_BF16, HS_FP8_E4M3 = 0, 1
HS_DEVERR_NO_HOST_COPY = 0x1
HS_DEVERR_BAD_BLOCK = 0x2
HS_DEVERR_BAD_ROW = 0x4
HS_DEVERR_SHORT_CONTEXT = 0x8
HS_DEVERR_TOPK_COUNT = 0x10
HS_DEVERR_HOT_FULL = 0x20
HS_DEVERR_TAIL_PAGE = 0x40
HS_DEVERR_POOL_EMPTY = 0x80
HS_DEVERR_POOL_FULL = 0x100
HS_DEVERR_BAD_REQUEST = 0x200

# hs_kernel_id
KERNEL_NAMES = ["index_score", "topk_select", "resolve", "miss_copy", "decode", "decode_merge",
                "hot_reset", "materialize", "release", "lease", "hot_release", "pool_give",
                "index_rescore", "topk_rescored"]
HS_KERNEL_COUNT = len(KERNEL_NAMES)

EXPORTED = ["hs_create", "hs_destroy", "hs_workspace_bytes", "hs_host_pool_bytes",
            "hs_host_pool_alloc", "hs_bind", "hs_hot_reset", "hisparse_index_topk",
            "hisparse_resolve", "sparse_mla_decode", "hs_read_device_error", "hs_decode_splits",
            "hs_hot_state", "hs_kernel_timing", "hs_kernel_times", "hs_select_paths",
            "hisparse_materialize_pages", "hisparse_release_pages", "hisparse_resolve_plan",
            "hs_hot_release", "hs_hot_pool_give", "hs_hot_pool_read",
            "hisparse_prefill_index_topk", "sparse_mla_prefill", "hs_measure_read_gbps",
            "sparse_mla_decode_noalloc",
            "hs_status_string", "hs_last_error"]


class hs_config(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("idx_dtype", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_queries", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("hot_rows_per_req", ctypes.c_int32), ("topk_lds_candidates", ctypes.c_int32),
                ("hot_leasing", ctypes.c_int32), ("num_gpu_blocks", ctypes.c_int64),
                ("num_idx_blocks", ctypes.c_int64), ("num_host_blocks", ctypes.c_int64)]


class hs_buffers(ctypes.Structure):
    _fields_ = [("kv_pool", ctypes.c_void_p), ("idx_pool", ctypes.c_void_p),
                ("idx_block_table", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("host_block_table", ctypes.c_void_p), ("hot_blocks", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p)]


class hs_hot_state_ptrs(ctypes.Structure):
    _fields_ = [("slot_token", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("tok2slot", ctypes.c_void_p), ("req_step", ctypes.c_void_p),
                ("hot_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tokens_per_req", ctypes.c_int64)]


class HiSparseError(RuntimeError):
    def __init__(self, what: str, status: int):
        self.status = status
        super().__init__(f"{what}: {hs_status_string(status)}: {hs_last_error()}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mla_attention_score_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        sig = {
            "hs_create": [ctypes.POINTER(hs_config), ctypes.POINTER(P)],
            "hs_destroy": [P],
            "hs_workspace_bytes": [ctypes.POINTER(hs_config), ctypes.POINTER(ctypes.c_size_t)],
            "hs_host_pool_bytes": [ctypes.POINTER(hs_config), ctypes.POINTER(ctypes.c_size_t)],
            "hs_host_pool_alloc": [P, ctypes.POINTER(P)],
            "hs_bind": [P, ctypes.POINTER(hs_buffers)],
            "hs_hot_reset": [P, P],
            "hisparse_index_topk": [P, P, P, P, i32, i32, P, P],
            "hisparse_resolve": [P, P, P, i32, i32, P, P, P],
            "hisparse_resolve_plan": [P, P, P, i32, i32, P, P, P, P],
            "hs_hot_release": [P, P, i32, P],
            "hs_hot_pool_give": [P, P, i32, P],
            "hs_hot_pool_read": [P, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)],
            "hisparse_prefill_index_topk": [P, i32, P, P, i32, i32, P, P],
            "sparse_mla_prefill": [P, i32, i32, P, P, i32, i32, f32, P, P, P],
            "hs_measure_read_gbps": [P, ctypes.c_size_t, P, i32, ctypes.POINTER(ctypes.c_double)],
            "sparse_mla_decode": [P, i32, P, P, P, i32, i32, f32, P, P, P],
            "sparse_mla_decode_noalloc": [P, i32, P, P, P, i32, i32, f32, P, P, P],
            "hs_read_device_error": [P, ctypes.POINTER(i32)],
            "hs_decode_splits": [P, i32, i32, ctypes.POINTER(i32)],
            "hs_select_paths": [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)],
            "hisparse_materialize_pages": [P, P, i32, P],
            "hisparse_release_pages": [P, P, i32, P, P, P],
            "hs_hot_state": [P, ctypes.POINTER(hs_hot_state_ptrs)],
            "hs_kernel_timing": [P, i32],
            "hs_kernel_times": [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                i32],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.hs_status_string.argtypes = [ctypes.c_int]
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_last_error.argtypes = []
        L.hs_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def hs_status_string(status: int) -> str:
    return lib().hs_status_string(status).decode()


def hs_last_error() -> str:
    return lib().hs_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != HS_OK:
        raise HiSparseError(what, status)


# ---------------------------------------------------------------- thin wrappers (same names)

def hs_workspace_bytes(cfg: hs_config) -> int:
    n = ctypes.c_size_t()
    _check(lib().hs_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)), "hs_workspace_bytes")
    return n.value


def hs_host_pool_bytes(cfg: hs_config) -> int:
    n = ctypes.c_size_t()
    _check(lib().hs_host_pool_bytes(ctypes.byref(cfg), ctypes.byref(n)), "hs_host_pool_bytes")
    return n.value


def hs_create(cfg: hs_config) -> int:
    ctx = ctypes.c_void_p()
    _check(lib().hs_create(ctypes.byref(cfg), ctypes.byref(ctx)), "hs_create")
    return ctx.value


def hs_destroy(ctx: int) -> None:
    _check(lib().hs_destroy(ctx), "hs_destroy")


def hs_host_pool_alloc(ctx: int) -> int:
    p = ctypes.c_void_p()
    _check(lib().hs_host_pool_alloc(ctx, ctypes.byref(p)), "hs_host_pool_alloc")
    return p.value or 0


def hs_bind(ctx: int, bufs: hs_buffers) -> None:
    _check(lib().hs_bind(ctx, ctypes.byref(bufs)), "hs_bind")


def hs_hot_reset(ctx: int, stream: int) -> None:
    _check(lib().hs_hot_reset(ctx, stream), "hs_hot_reset")


def hisparse_index_topk(ctx: int, q_idx: int, w: int, ctx_lens: int, B: int, S: int, topk_out: int,
                        stream: int) -> None:
    _check(lib().hisparse_index_topk(ctx, q_idx, w, ctx_lens, B, S, topk_out, stream),
           "hisparse_index_topk")


def hisparse_resolve(ctx: int, topk: int, ctx_lens: int, B: int, S: int, row_ids_out: int,
                     stats_out: int, stream: int) -> None:
    _check(lib().hisparse_resolve(ctx, topk, ctx_lens, B, S, row_ids_out, stats_out or None, stream),
           "hisparse_resolve")


def hisparse_resolve_plan(ctx: int, topk: int, ctx_lens: int, B: int, S: int, begin_window: int,
                          row_ids_out: int, stats_out: int, stream: int) -> None:
    _check(lib().hisparse_resolve_plan(ctx, topk, ctx_lens, B, S, begin_window or None, row_ids_out,
                                       stats_out or None, stream), "hisparse_resolve_plan")


def hs_hot_release(ctx: int, reqs: int, n: int, stream: int) -> None:
    _check(lib().hs_hot_release(ctx, reqs, n, stream), "hs_hot_release")


def hs_hot_pool_give(ctx: int, blocks: int, n: int, stream: int) -> None:
    _check(lib().hs_hot_pool_give(ctx, blocks, n, stream), "hs_hot_pool_give")


def hs_hot_pool_read(ctx: int, cap: int) -> list:
    """The free-block pool, front first (synchronises)."""
    buf = (ctypes.c_int32 * max(cap, 1))()
    n = ctypes.c_int32()
    _check(lib().hs_hot_pool_read(ctx, buf, cap, ctypes.byref(n)), "hs_hot_pool_read")
    return [buf[i] for i in range(min(n.value, cap))]


def hisparse_prefill_index_topk(ctx: int, b: int, q_idx: int, w: int, L: int, P: int, topk_out: int,
                                stream: int) -> None:
    _check(lib().hisparse_prefill_index_topk(ctx, b, q_idx, w, L, P, topk_out, stream),
           "hisparse_prefill_index_topk")


def sparse_mla_prefill(ctx: int, layer: int, b: int, q: int, topk: int, L: int, P: int,
                       sm_scale: float, out: int, lse: int, stream: int) -> None:
    _check(lib().sparse_mla_prefill(ctx, layer, b, q, topk or None, L, P, sm_scale, out, lse or None,
                                    stream), "sparse_mla_prefill")


def hs_measure_read_gbps(buf: int, nbytes: int, sink: int, reps: int = 5) -> float:
    g = ctypes.c_double()
    _check(lib().hs_measure_read_gbps(buf, nbytes, sink, reps, ctypes.byref(g)), "hs_measure_read_gbps")
    return g.value


def sparse_mla_decode(ctx: int, layer: int, q: int, row_ids: int, ctx_lens: int, B: int, S: int,
                      sm_scale: float, out: int, lse: int, stream: int) -> None:
    _check(lib().sparse_mla_decode(ctx, layer, q, row_ids, ctx_lens, B, S, sm_scale, out,
                                   lse or None, stream), "sparse_mla_decode")


def sparse_mla_decode_noalloc(ctx: int, layer: int, q: int, row_ids: int, ctx_lens: int, B: int,
                              S: int, sm_scale: float, out: int, lse: int, stream: int) -> None:
    _check(lib().sparse_mla_decode_noalloc(ctx, layer, q, row_ids, ctx_lens, B, S, sm_scale, out,
                                           lse or None, stream), "sparse_mla_decode_noalloc")


def hs_read_device_error(ctx: int) -> int:
    code = ctypes.c_int32()
    _check(lib().hs_read_device_error(ctx, ctypes.byref(code)), "hs_read_device_error")
    return code.value


def hs_decode_splits(ctx: int, B: int, S: int) -> int:
    n = ctypes.c_int32()
    _check(lib().hs_decode_splits(ctx, B, S, ctypes.byref(n)), "hs_decode_splits")
    return n.value


def hisparse_materialize_pages(ctx: int, pages: int, n: int, stream: int) -> None:
    _check(lib().hisparse_materialize_pages(ctx, pages, n, stream), "hisparse_materialize_pages")


def hisparse_release_pages(ctx: int, pages: int, n: int, ctx_lens: int, freed_out: int, stream: int) -> None:
    _check(lib().hisparse_release_pages(ctx, pages, n, ctx_lens, freed_out, stream), "hisparse_release_pages")


def hs_select_paths(ctx: int) -> tuple:
    """(selections made from the sweep's candidate list, selections made from all scores)."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().hs_select_paths(ctx, ctypes.byref(a), ctypes.byref(b)), "hs_select_paths")
    return a.value, b.value


def hs_hot_state(ctx: int) -> hs_hot_state_ptrs:
    out = hs_hot_state_ptrs()
    _check(lib().hs_hot_state(ctx, ctypes.byref(out)), "hs_hot_state")
    return out


def hs_kernel_timing(ctx: int, enable: bool) -> None:
    _check(lib().hs_kernel_timing(ctx, 1 if enable else 0), "hs_kernel_timing")


def hs_kernel_times(ctx: int) -> dict:
    """{kernel name: (summed ms, launches)} since timing was enabled or last read."""
    ms = (ctypes.c_double * HS_KERNEL_COUNT)()
    n = (ctypes.c_int64 * HS_KERNEL_COUNT)()
    _check(lib().hs_kernel_times(ctx, ms, n, HS_KERNEL_COUNT), "hs_kernel_times")
    return {name: (ms[i], n[i]) for i, name in enumerate(KERNEL_NAMES)}


def make_config(*, topk: int = 2048, kv_dtype: int = HS_FP8_E4M3, idx_dtype: int = HS_FP8_E4M3,
                n_layers: int = 1, max_batch: int, max_queries: int, max_pages_per_req: int,
                hot_rows_per_req: int = 0, num_gpu_blocks: int, num_idx_blocks: int,
                num_host_blocks: int, topk_lds_candidates: int = 0, hot_leasing: int = 0) -> hs_config:
    return hs_config(64, topk, 32, 128, 64, 576, 512, kv_dtype, idx_dtype, n_layers, max_batch,
                     max_queries, max_pages_per_req, hot_rows_per_req, topk_lds_candidates,
                     hot_leasing, num_gpu_blocks, num_idx_blocks, num_host_blocks)


# ---------------------------------------------------------------- torch plumbing

class Context:
    """A bound context whose device buffers are torch tensors on `device`.

    Pools and tables are allocated here; the caller fills them (e.g. from the
    synthetic generator) through the tensors / the host-pool numpy view.
    """

    def __init__(self, cfg: hs_config, device="cuda:0"):
        import numpy as np
        import torch

        self.cfg = cfg
        self.device = torch.device(device)
        torch.cuda.set_device(self.device)
        rb = 656 if cfg.kv_dtype == HS_FP8_E4M3 else 1152
        ib = 8448 if cfg.idx_dtype == HS_FP8_E4M3 else 16384
        self.row_bytes = rb
        self.idx_block_bytes = ib
        self.hot_rows = cfg.hot_rows_per_req or -(-((cfg.max_queries + 1) * cfg.topk) // 64) * 64
        u8 = dict(dtype=torch.uint8, device=self.device)
        i32 = dict(dtype=torch.int32, device=self.device)
        self.kv_pool = torch.empty(cfg.n_layers * cfg.num_gpu_blocks * 64 * rb, **u8)
        self.idx_pool = torch.empty(cfg.num_idx_blocks * ib, **u8)
        P = cfg.max_pages_per_req
        self.idx_block_table = torch.full((cfg.max_batch, P), -1, **i32)
        self.block_table = torch.full((cfg.max_batch, P), -1, **i32)
        self.host_block_table = torch.full((cfg.max_batch, P), -1, **i32)
        self.hot_blocks = torch.zeros((cfg.max_batch, max(1, self.hot_rows // 64)), **i32)
        ws = hs_workspace_bytes(cfg)
        self.workspace = torch.empty(ws + 256, **u8)
        ws_ptr = (self.workspace.data_ptr() + 255) // 256 * 256
        self.ctx = hs_create(cfg)
        self.host_base = hs_host_pool_alloc(self.ctx)
        nh = hs_host_pool_bytes(cfg)
        self.host_pool = None
        if self.host_base and nh:
            buf = (ctypes.c_uint8 * nh).from_address(self.host_base)
            self.host_pool = np.frombuffer(buf, dtype=np.uint8)
        bufs = hs_buffers(self.kv_pool.data_ptr(), self.idx_pool.data_ptr(),
                          self.idx_block_table.data_ptr(), self.block_table.data_ptr(),
                          self.host_block_table.data_ptr(), self.hot_blocks.data_ptr(), ws_ptr)
        hs_bind(self.ctx, bufs)
        self.reset()

    @staticmethod
    def stream() -> int:
        import torch
        return torch.cuda.current_stream().cuda_stream

    def reset(self) -> None:
        hs_hot_reset(self.ctx, self.stream())

    def index_topk(self, q_idx, w, ctx_lens, topk_out) -> None:
        B, S = q_idx.shape[0], q_idx.shape[1]
        hisparse_index_topk(self.ctx, q_idx.data_ptr(), w.data_ptr(), ctx_lens.data_ptr(), B, S,
                            topk_out.data_ptr(), self.stream())

    def resolve(self, topk, ctx_lens, row_ids_out, stats_out=None, begin_window=None) -> None:
        """begin_window: None (every call begins a plan window) or a device int32 [B]."""
        B, S = topk.shape[0], topk.shape[1]
        st = stats_out.data_ptr() if stats_out is not None else 0
        if begin_window is None:
            hisparse_resolve(self.ctx, topk.data_ptr(), ctx_lens.data_ptr(), B, S,
                             row_ids_out.data_ptr(), st, self.stream())
        else:
            hisparse_resolve_plan(self.ctx, topk.data_ptr(), ctx_lens.data_ptr(), B, S,
                                  begin_window.data_ptr(), row_ids_out.data_ptr(), st, self.stream())

    def hot_release(self, reqs) -> None:
        """reqs: device int32 [n] of request slots whose hot buffers become cold."""
        hs_hot_release(self.ctx, reqs.data_ptr(), reqs.shape[0], self.stream())

    def pool_give(self, blocks) -> None:
        """blocks: device int32 [n] appended to the free-block pool (entries < 0 skipped)."""
        hs_hot_pool_give(self.ctx, blocks.data_ptr(), blocks.shape[0], self.stream())

    def pool_free(self) -> list:
        return hs_hot_pool_read(self.ctx, int(self.cfg.num_gpu_blocks))

    def decode(self, layer, q, row_ids, ctx_lens, sm_scale, out, lse=None) -> None:
        B, S = q.shape[0], q.shape[1]
        sparse_mla_decode(self.ctx, layer, q.data_ptr(), row_ids.data_ptr(), ctx_lens.data_ptr(),
                          B, S, sm_scale, out.data_ptr(), lse.data_ptr() if lse is not None else 0,
                          self.stream())

    def prefill_index_topk(self, b, q_idx, w, L, topk_out) -> None:
        """q_idx [P][32][128] bf16, w [P][32] fp32, topk_out [P][K] int32 (device)."""
        hisparse_prefill_index_topk(self.ctx, b, q_idx.data_ptr(), w.data_ptr(), L, q_idx.shape[0],
                                    topk_out.data_ptr(), self.stream())

    def prefill(self, layer, b, q, topk, L, sm_scale, out, lse=None) -> None:
        """q [P][64][576] bf16; topk [P][K] int32 or None (every visible row, L <= K)."""
        sparse_mla_prefill(self.ctx, layer, b, q.data_ptr(), topk.data_ptr() if topk is not None else 0,
                           L, q.shape[0], sm_scale, out.data_ptr(),
                           lse.data_ptr() if lse is not None else 0, self.stream())

    def decode_noalloc(self, layer, q, row_ids, ctx_lens, sm_scale, out, lse=None) -> None:
        B, S = q.shape[0], q.shape[1]
        sparse_mla_decode_noalloc(self.ctx, layer, q.data_ptr(), row_ids.data_ptr(), ctx_lens.data_ptr(),
                                  B, S, sm_scale, out.data_ptr(), lse.data_ptr() if lse is not None else 0,
                                  self.stream())

    def device_error(self) -> int:
        return hs_read_device_error(self.ctx)

    def select_paths(self) -> tuple:
        return hs_select_paths(self.ctx)

    def materialize_pages(self, pages) -> None:
        """pages: device int32 [n][2] of (request, page)."""
        hisparse_materialize_pages(self.ctx, pages.data_ptr(), pages.shape[0], self.stream())

    def release_pages(self, pages, ctx_lens, freed_out) -> None:
        hisparse_release_pages(self.ctx, pages.data_ptr(), pages.shape[0], ctx_lens.data_ptr(),
                               freed_out.data_ptr(), self.stream())

    def kernel_timing(self, enable: bool) -> None:
        hs_kernel_timing(self.ctx, enable)

    def kernel_times(self) -> dict:
        return hs_kernel_times(self.ctx)

    def hot_state(self, requests=None):
        """Copies of (slot_token [B][H], slot_stamp [B][H], tok2slot [B][L], req_step [B]) as
        int32 numpy arrays, read from the workspace the library bound; with `requests`, only
        those requests' rows (in that order)."""
        import torch
        p = hs_hot_state(self.ctx)
        ws0 = (self.workspace.data_ptr() + 255) // 256 * 256
        base = self.workspace.data_ptr()
        B, H, L = self.cfg.max_batch, p.hot_rows, p.tokens_per_req
        pick = None if requests is None else torch.as_tensor(list(requests), device=self.device)

        def view(addr, rows, cols):
            off = addr - base
            n = rows * cols
            assert off >= ws0 - base and off + 4 * n <= self.workspace.numel()
            t = self.workspace[off:off + 4 * n].view(torch.int32).view(rows, cols)
            if pick is not None:
                t = t.index_select(0, pick)
            return t.cpu().numpy()

        torch.cuda.synchronize()
        return (view(p.slot_token, B, H), view(p.slot_stamp, B, H), view(p.tok2slot, B, L),
                view(p.req_step, B, 1).reshape(-1).copy())

    def close(self) -> None:
        if getattr(self, "ctx", None):
            hs_destroy(self.ctx)
            self.ctx = None
            self.host_pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
