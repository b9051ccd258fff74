"""Upload generated workloads to the GPU as the library's input tensors.

Pure marshalling (numpy bytes -> torch device tensors); no step of the
method happens here.
"""
import numpy as np
import torch

import compressed_sparse_long_compress_amd as csa


def bf16(a, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def t(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def kv_cache(ent, cap, device="cuda"):
    nope, rope, scale = ent
    return csa.KvCache(t(nope, device), bf16(rope, device), t(scale, device), cap)


def index_keys(keys, cap, device="cuda"):
    return csa.IndexKeys(t(keys[0], device), t(keys[1], device), cap)


def host_entries(cache):
    """KvCache on device -> (nope uint8, rope uint16 bits, scale float32) numpy."""
    return (cache.nope.cpu().numpy(), cache.rope.view(torch.int16).cpu().numpy().view(np.uint16),
            cache.scale.cpu().numpy())
