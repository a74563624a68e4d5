"""Storage layouts the library expects (host-side marshalling, no arithmetic).

Prompt KV of one layer: requests packed back to back, each request's block padded to a
multiple of 64 prompt rows; keys as [Hkv][Pp][D], values transposed as [Hkv][D][Pp] so
the shared stage's PV contraction streams V^T tiles straight into LDS.
"""
from __future__ import annotations

import numpy as np
import torch

PAD_P = 64


def _torch_view(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "f32":
        return t.to(torch.float32)
    if dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16) if t.dtype != torch.int16 else t.view(torch.bfloat16)
    if dtype == "fp8":
        return t.to(torch.uint8)
    raise ValueError(dtype)


def stored_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """A stored array (float32 values, uint16 bf16 bits, uint8 e4m3 bits) as a device tensor."""
    if dtype == "bf16":
        a = np.asarray(a, np.uint16).view(np.int16)
    return _torch_view(a, dtype).to(device)


def pack_shared_kv(k_list, v_list, dtype: str, device="cuda", pad=0):
    """Pack per-request prompt KV arrays ([Hkv][P_r][D] each, stored format) into the
    library's per-layer buffers (k: [Hkv][Pp][D] blocks, v: [Hkv][D][Pp] blocks).  ``pad`` is
    the stored value (element bits for bf16 and fp8) written to the padding rows, which the
    library ignores whatever they hold."""
    kb, vb = [], []
    for k, v in zip(k_list, v_list):
        Hkv, P, D = k.shape
        Pp = (P + PAD_P - 1) // PAD_P * PAD_P
        kp = np.full((Hkv, Pp, D), pad, dtype=k.dtype)
        kp[:, :P] = k
        vp = np.full((Hkv, D, Pp), pad, dtype=v.dtype)
        vp[:, :, :P] = np.transpose(v, (0, 2, 1))
        kb.append(kp.reshape(-1))
        vb.append(vp.reshape(-1))
    return (stored_tensor(np.concatenate(kb), dtype, device),
            stored_tensor(np.concatenate(vb), dtype, device))
