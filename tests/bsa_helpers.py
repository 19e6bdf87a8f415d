"""Glue between the seeded workloads and the library binding (tests/bench)."""
import numpy as np

import block_sparse_attention_fwd_amd as bsa
import workloads as wl


def plan_workload(w, device=0, force_regime=-1, bits=False, lut_path=None, dtype=bsa.DTYPE_BF16, task_order=-1):
    kw = dict(T=w.T, Hg=w.Hg, Wg=w.Wg, head_layout=w.head_layout, force_regime=force_regime, device=device,
              lut_path=lut_path, dtype=dtype, task_order=task_order)
    if w.kind == wl.BLOCK:
        if bits:
            return bsa.plan(bsa.MASK_BLOCK_BITS, w.B, w.H, w.L, w.d, w.bq, w.bk, data=w.block_bits(), **kw)
        return bsa.plan(bsa.MASK_BLOCK_U8, w.B, w.H, w.L, w.d, w.bq, w.bk, data=w.block, **kw)
    if w.kind == wl.SLICE:
        return bsa.plan(bsa.MASK_SLICE_CSR, w.B, w.H, w.L, w.d, w.bq, 1, row_ptr=w.row_ptr, col_idx=w.col_idx, **kw)
    if w.kind == wl.VIDEO:
        return bsa.plan(bsa.MASK_VIDEO, w.B, w.H, w.L, w.d, 1, 1, head_pattern=w.head_pattern,
                        anchor_frame=w.anchor, radius=w.radius, **kw)
    raise ValueError(w.kind)


def to_device_bf16(x_u16: np.ndarray, device: str = "cuda:0"):
    """bf16 bit patterns (uint16 numpy) -> a bfloat16 torch tensor on ``device``."""
    import torch
    return torch.from_numpy(x_u16.view(np.int16)).view(torch.bfloat16).to(device)


def tok_of_logical(T, HW):
    return np.arange(T * HW).reshape(T, HW).T.reshape(-1)


def plan_workload_device(w, device=0, force_regime=-1, bits=False, lut_path=None, dtype=bsa.DTYPE_BF16,
                         task_order=-1, stream=None, mask=None):
    """bsa_plan_device on a BLOCK workload: the mask is first copied to the
    device (or taken from ``mask``, a device tensor of the kind's layout)."""
    import torch
    assert w.kind == wl.BLOCK
    kind = bsa.MASK_BLOCK_BITS if bits else bsa.MASK_BLOCK_U8
    if mask is None:
        host = w.block_bits().view(np.int64) if bits else np.ascontiguousarray(w.block, dtype=np.uint8)
        mask = torch.from_numpy(host).to(f"cuda:{device}")
    return bsa.plan_device(kind, w.B, w.H, w.L, w.d, w.bq, w.bk, mask, stream=stream, dtype=dtype, T=w.T, Hg=w.Hg,
                           Wg=w.Wg, head_layout=w.head_layout, force_regime=force_regime, lut_path=lut_path,
                           device=device, task_order=task_order)
