"""Helpers for the GPU tests: seeded NumPy inputs to device tensors and back."""
import numpy as np
import torch

import gated_deltanet_decode_amd as gdn

DEV = "cuda"


def dims_of(shape, batch=1):
    return gdn.dims(batch, shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim,
                    shape.conv_width, shape.act)


def act_to_dev(arr):
    """bf16 bit patterns (uint16) -> torch.bfloat16 on the device; float32 stays float32."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(arr).to(DEV)


def f32_to_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def i32_to_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(DEV)


def act_to_host(t):
    """Device activation tensor -> uint16 bits (bf16) or float32 array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host(t):
    return t.detach().cpu().numpy()


def bits(t):
    """Exact bit patterns of a float32 device tensor."""
    return t.detach().cpu().contiguous().view(torch.int32).numpy()
