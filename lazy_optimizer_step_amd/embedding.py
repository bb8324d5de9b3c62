"""An embedding table trained by the sparse / lazy optimizer step.

The steps either side of the optimizer, as the DiskSparseAdam README's training
loop uses them (read_rows for the forward pass, then step with the lookup
indices and the gradient rows): ``forward(ids)`` gathers the current rows with
``read_rows``; autograd hands the backward the per-lookup gradient rows, in
lookup order, which is the value layout ``csr_from_lookups`` sorts and sums
directly (no re-layout); ``step()`` canonicalises them, assembles the CSR
gradient over every table row and applies the optimizer to the touched rows
only, all in one call (``sparse_step_from_lookups``).  Every step of the path
runs in the library's kernels; this module only keeps the buffers and the order
of the calls.
"""
from __future__ import annotations

import torch

from . import SparseAdam, SparseSgd, read_rows, sparse_opt_workspace_size


class _Lookup(torch.autograd.Function):
    @staticmethod
    def forward(ctx, anchor, ids, table):
        ctx.table = table
        ctx.ids = ids
        return read_rows(table.weight, ids)

    @staticmethod
    def backward(ctx, grad_rows):
        ctx.table._pending.append((ctx.ids, grad_rows.contiguous()))
        return torch.zeros_like(ctx.table._anchor), None, None


class SparseEmbedding(torch.nn.Module):
    """``num_rows x dim`` float32 table on the GPU.

    optimizer: "adam" (keyword arguments of SparseAdam: lr, beta1, beta2, eps,
    mode, weight_decay, weight_decay_mode, last_step_per_row) or "sgd"
    (SparseSgd: lr, momentum, weight_decay).  weight: an initial table (copied),
    else N(0, init_std)."""

    def __init__(self, num_rows: int, dim: int, *, optimizer: str = "adam", weight=None,
                 init_std: float = 0.01, device="cuda", **opt_kw):
        super().__init__()
        if weight is None:
            w = torch.empty((num_rows, dim), dtype=torch.float32, device=device)
            w.normal_(0.0, init_std)
        else:
            w = torch.as_tensor(weight, dtype=torch.float32).to(device).clone()
        self.weight = w                       # updated in place by step(), not by autograd
        self._anchor = torch.zeros((), device=device, requires_grad=True)
        if optimizer == "adam":
            self.opt = SparseAdam(self.weight, **opt_kw)
        elif optimizer == "sgd":
            self.opt = SparseSgd(self.weight, **opt_kw)
        else:
            raise ValueError(f"optimizer {optimizer!r}: 'adam' or 'sgd'")
        self._pending: list[tuple[torch.Tensor, torch.Tensor]] = []
        self._bufs: dict[int, dict] = {}

    @property
    def num_rows(self) -> int:
        return self.weight.shape[0]

    @property
    def dim(self) -> int:
        return self.weight.shape[1]

    def forward(self, ids: torch.Tensor) -> torch.Tensor:
        """Rows of the current table for int64 ids (any shape); duplicates allowed."""
        flat = ids.reshape(-1).to(device=self.weight.device, dtype=torch.int64).contiguous()
        rows = _Lookup.apply(self._anchor, flat, self)
        return rows.view(*ids.shape, self.dim)

    def _buffers_for(self, n: int) -> dict:
        b = self._bufs.get(n)
        if b is None:
            dev = self.weight.device
            R, C = self.num_rows, self.dim
            b = {"keys": torch.empty(n, dtype=torch.int64, device=dev),
                 "sums": torch.empty((n, C), dtype=torch.float32, device=dev),
                 "counts": torch.empty(n, dtype=torch.int32, device=dev),
                 "U": torch.empty(1, dtype=torch.int64, device=dev),
                 "ws": torch.empty(max(sparse_opt_workspace_size(n, C, R), 1), dtype=torch.uint8,
                                   device=dev),
                 "row_offsets": torch.empty(R + 1, dtype=torch.int32, device=dev)}
            self._bufs = {n: b}                 # keep the buffers of the latest size only
        return b

    def step(self, *, stream=None) -> int:
        """Apply the optimizer to the gradient rows gathered since the last step
        (all lookups of the step together, duplicates summed).  Returns the
        number of lookups consumed; with none pending nothing happens."""
        if not self._pending:
            return 0
        if len(self._pending) == 1:
            ids, grads = self._pending[0]
        else:
            ids = torch.cat([i for i, _ in self._pending])
            grads = torch.cat([g for _, g in self._pending])
        self._pending.clear()
        n = ids.numel()
        b = self._buffers_for(n)
        self.opt.step_lookups(ids, grads, out_keys=b["keys"], out_vals=b["sums"],
                              out_counts=b["counts"], d_nunique=b["U"],
                              row_offsets=b["row_offsets"], want_col_indices=False,
                              workspace=b["ws"], stream=stream)
        return n
