"""Helpers of the GPU tests: move seeded inputs and oracle-built indexes to the device."""
import numpy as np
import torch

import retrieval_sparse_attention_amd as rsa

DEV = torch.device("cuda:0")


def to_dev_bf16(a):
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def upload_index(idx):
    """An oracle.Index as a device WaveIndex (same arrays, same layout)."""
    arrays = {
        "k_sorted": to_dev_bf16(idx.k_sorted),
        "v_sorted": to_dev_bf16(idx.v_sorted),
        "perm": torch.from_numpy(idx.perm).to(DEV),
        "inv_perm": torch.from_numpy(idx.inv_perm).to(DEV),
        "assign": torch.from_numpy(idx.assign).to(DEV),
        "offsets": torch.from_numpy(idx.offsets).to(DEV),
        "sizes": torch.from_numpy(idx.sizes).to(DEV),
        "centroids": torch.from_numpy(idx.centroids).to(DEV),
        "centroids_bf16": to_dev_bf16(idx.centroids_bf16),
        "vsum": torch.from_numpy(idx.vsum).to(DEV),
    }
    return rsa.WaveIndex(idx.G, idx.ctx.tolist(), idx.seg_len, idx.K_s, arrays)


def index_to_host(ix):
    """Every array of a device WaveIndex as numpy (bf16 arrays as uint16 bits)."""
    out = {}
    for k, v in ix.arrays.items():
        out[k] = to_host_u16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()
    return out


def say(msg):
    print(msg, flush=True)
