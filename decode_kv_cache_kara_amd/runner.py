"""Device-side buffers for running the compression step on a synthetic
workload through the C ABI (used by the tests and the benchmark).  Allocation
and argument marshalling only."""

from __future__ import annotations

import torch

from . import kara


def shape_of(wl):
    return kara.kara_shape(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size,
                           kara.dtype_code(wl.dtype))


def params_of(wl, flags=0):
    return kara.kara_params(wl.window, wl.protect, wl.top_k, wl.budget, flags)


class Session:
    """Buffers for repeated kara_compress calls on one GPU-resident workload.

    Compaction is out of place and each call starts from a pool rebuilt from
    the workload's free list, so repeated calls do identical work.
    """

    def __init__(self, wl, outputs=True, flags=0):
        if wl.pool.device.type != "cuda":
            raise ValueError("workload must be on the GPU")
        self.wl = wl
        self.shape = shape_of(wl)
        self.params = params_of(wl, flags)
        dev = wl.pool.device
        self.table_h = wl.table.to("cpu", torch.int32).contiguous()
        self.table_d = wl.table.to(torch.int32).contiguous()
        self.lens_h = wl.lens.to("cpu", torch.int32).contiguous()
        self.lens_d = wl.lens.to(torch.int32).contiguous()
        self.new_table_h = torch.empty_like(self.table_h)
        self.new_table_d = torch.empty_like(self.table_d)
        self.new_lens_h = torch.empty_like(self.lens_h)
        self.free_ids = torch.tensor(wl.free_ids, dtype=torch.int32)
        nbytes = kara.kara_workspace_bytes(self.shape, self.params, wl.n_seqs)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        U, C = wl.n_units, wl.region
        self.scores = torch.empty((U, C), dtype=torch.float32, device=dev) if outputs else None
        self.cand = torch.empty((U, wl.top_k), dtype=torch.int32, device=dev) if outputs else None
        self.retained = torch.empty((U, wl.budget), dtype=torch.int32, device=dev) if outputs else None
        self.pool = None

    def new_pool(self):
        return kara.Pool(self.wl.n_blocks, self.free_ids)

    def compress(self, stream=None, pool=None, stage_events=None):
        self.pool = pool if pool is not None else self.new_pool()
        kara.kara_compress(self.shape, self.params, self.wl.q_window, self.wl.pool, self.table_h,
                           self.table_d, self.lens_h, self.lens_d, self.pool, self.new_table_h,
                           self.new_table_d, self.new_lens_h, self.workspace, stream=stream,
                           scores_out=self.scores, cand_out=self.cand, retained_out=self.retained,
                           stage_events=stage_events)
        return self.pool

    def score(self, scores_out, stream=None):
        kara.kara_score(self.shape, self.params, self.wl.q_window, self.wl.pool, self.table_h,
                        self.table_d, self.lens_h, self.lens_d, scores_out, self.workspace,
                        stream=stream)
