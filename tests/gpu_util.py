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


def upload_index(idx, value_sums="f32"):
    """An oracle.Index as a device WaveIndex (same arrays, same layout). value_sums "bf16" or
    "both" also uploads the oracle's bf16 value sums (the estimation zone then reads those)."""
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
    }
    if value_sums in ("f32", "both"):
        arrays["vsum"] = torch.from_numpy(idx.vsum).to(DEV)
    if value_sums in ("bf16", "both"):
        import oracle
        arrays["vsum_bf16"] = to_dev_bf16(oracle.value_sums_bf16(idx))
    return rsa.WaveIndex(idx.G, idx.ctx.tolist(), idx.seg_len, idx.K_s, arrays)


def index_to_host(ix):
    """Every array of a device WaveIndex as numpy (bf16 arrays as uint16 bits)."""
    out = {}
    for k, v in ix.arrays.items():
        out[k] = to_host_u16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()
    return out


def say(msg):
    print(msg, flush=True)


def dense_from_capacity(h, G, ctx, seg_len, K_s, cap):
    """Host arrays of a capacity index (every (b, g) block with room for `cap` segments) in
    the dense ragged layout of the oracle: each block's filled rows, clusters and offsets."""
    from oracle import Index, num_clusters
    R, Cs = cap * seg_len, cap * K_s
    rows, clus, offs = [], [], []
    for b, N in enumerate(ctx):
        N = int(N)
        C = num_clusters(N, seg_len, K_s)
        for g in range(G):
            blk = b * G + g
            rows.append((blk * R, blk * R + N))
            clus.append((blk * Cs, blk * Cs + C))
            offs.append((blk * (Cs + 1), blk * (Cs + 1) + C + 1))
    out = {}
    for f in Index.FIELDS:
        a = h[f]
        sel = rows if f in ("k_sorted", "v_sorted", "perm", "inv_perm", "assign") else (
            offs if f == "offsets" else clus)
        out[f] = np.concatenate([a[i:j] for i, j in sel])
    return out
