"""Device-memory plumbing for the C-ABI: uploads seeded workloads into torch device tensors,
allocates workspaces and downloads results. No arithmetic of the method happens here."""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np
import torch

from . import _native as N
from .inputs import BlockParams, Workload, bf16_to_f32


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> device torch.bfloat16 tensor (same bits)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).to(device).view(torch.bfloat16)


def to_dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> host uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values_of(t: torch.Tensor) -> np.ndarray:
    return bf16_to_f32(bf16_bits_of(t))


@dataclass
class DeviceBlock:
    tensors: dict
    weights: N.DitBlockWeights


def upload_block(bp: BlockParams, device="cuda") -> DeviceBlock:
    t = dict(w_qkv=to_dev_bf16(bp.w_qkv, device), w_o=to_dev_bf16(bp.w_o, device),
             w_gate_up=to_dev_bf16(bp.w_gate_up, device), w_down=to_dev_bf16(bp.w_down, device),
             norm1_g=to_dev_f32(bp.norm1_g, device), norm2_g=to_dev_f32(bp.norm2_g, device),
             q_g=to_dev_f32(bp.q_g, device), k_g=to_dev_f32(bp.k_g, device),
             ada=to_dev_f32(bp.ada, device))
    return DeviceBlock(t, N.make_block_weights(t))


def dims_of(wl: Workload) -> N.DitDims:
    return N.make_dims(wl.hidden, wl.heads, wl.head_dim, wl.ffn, wl.norm_eps, wl.qk_eps,
                       wl.rope_base)


def layout_of(wl: Workload, positions=None) -> N.DitLayout:
    return N.make_layout(wl.n_video, wl.n_audio, wl.seq_pad, positions)


def workspace(dims: N.DitDims, layout: N.DitLayout, n_blocks: int = 0, device="cuda"):
    """Returns (uint8 device tensor of the needed size, DitWorkspaceMap)."""
    n, m = N.dit_workspace_size(dims, layout, n_blocks)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    assert ws.data_ptr() % 256 == 0
    return ws, m


def ws_view_bf16(ws: torch.Tensor, offset: int, rows: int, cols: int) -> torch.Tensor:
    """bf16 [rows, cols] view of a workspace region."""
    return ws[offset:offset + rows * cols * 2].view(torch.bfloat16).view(rows, cols)


def upload_blocks(blocks: List[BlockParams], device="cuda") -> List[DeviceBlock]:
    return [upload_block(b, device) for b in blocks]
