"""The Python binding rejects mismatched tensors before any library call (CPU, no GPU needed).

Every check below fires on the host before the C library is entered: a reused index must
have been planned for the same shape, K/V/q and the outputs must have the dtype, shape and
contiguity the C ABI's layout describes, and every tensor must live in GPU memory (the
library reads and writes device memory only). CPU tensors therefore reach the device check
last, which lets these tests exercise every earlier check without a GPU.
"""
import pytest
import torch

import retrieval_sparse_attention_amd as rsa

G, CTX, SEG, KS = 2, [3000, 1700], 1024, 64


@pytest.fixture(scope="module")
def cpu_index():
    ix, z = rsa.WaveIndex.allocate(G, CTX, SEG, KS, device="cpu")
    return ix, z


def _kv(z, dtype=torch.bfloat16):
    return torch.zeros((z["rows"], 128), dtype=dtype), torch.zeros((z["rows"], 128), dtype=dtype)


def test_build_rejects_host_tensors(cpu_index):
    _, z = cpu_index
    K, V = _kv(z)
    with pytest.raises(ValueError, match="must be on the GPU"):
        rsa.wave_index_build(K, V, G, CTX, SEG, KS, 2, 1)


def test_build_rejects_wrong_dtype_and_shape(cpu_index):
    _, z = cpu_index
    K, V = _kv(z, torch.float16)
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        rsa.wave_index_build(K, V, G, CTX, SEG, KS, 2, 1)
    K = torch.zeros((z["rows"] - 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must have shape"):
        rsa.wave_index_build(K, K, G, CTX, SEG, KS, 2, 1)
    K = torch.zeros((128, z["rows"]), dtype=torch.bfloat16).t()
    with pytest.raises(ValueError, match="contiguous"):
        rsa.wave_index_build(K, K, G, CTX, SEG, KS, 2, 1)


@pytest.mark.parametrize("change", ["seg_len", "clusters_per_seg", "ctx", "n_kv_heads"])
def test_build_rejects_reuse_of_another_shape(cpu_index, change):
    ix, z = cpu_index
    args = dict(n_kv_heads=G, ctx=CTX, seg_len=SEG, clusters_per_seg=KS)
    args[change] = {"seg_len": 512, "clusters_per_seg": 128, "ctx": [3000, 1600], "n_kv_heads": 1}[change]
    zz = rsa.wave_index_plan(args["n_kv_heads"], args["ctx"], args["seg_len"], args["clusters_per_seg"])
    K, V = _kv(zz)
    with pytest.raises(ValueError, match="index was allocated for"):
        rsa.wave_index_build(K, V, args["n_kv_heads"], args["ctx"], args["seg_len"], args["clusters_per_seg"], 2, 1,
                             index=ix)
    with pytest.raises(ValueError, match="index was allocated for"):
        rsa.wave_index_build_blocks(K, V, args["n_kv_heads"], args["ctx"], args["seg_len"], args["clusters_per_seg"],
                                    index=ix)


def test_build_rejects_small_workspace(cpu_index):
    ix, z = cpu_index
    K, V = _kv(z)
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace has 16 bytes"):
        rsa.wave_index_build(K, V, G, CTX, SEG, KS, 2, 1, index=ix, ws=ws)


def _q(B=2, H=8, dtype=torch.bfloat16):
    return torch.zeros((B, H, 128), dtype=dtype)


def test_decode_rejects_wrong_batch_and_dtype(cpu_index):
    ix, _ = cpu_index
    with pytest.raises(ValueError, match="q holds 1 sequences, the index 2"):
        rsa.wave_attn_decode(ix, _q(B=1), 4, 64, 0.05)
    with pytest.raises(ValueError, match="q must be torch.bfloat16"):
        rsa.wave_attn_decode(ix, _q(dtype=torch.float32), 4, 64, 0.05)
    with pytest.raises(ValueError, match=r"q must be a \[B, H, 128\]"):
        rsa.wave_attn_decode(ix, torch.zeros((2, 8, 128, 1), dtype=torch.bfloat16), 4, 64, 0.05)


def test_decode_rejects_mis_sized_outputs(cpu_index):
    ix, _ = cpu_index
    k_max, wsb = rsa.wave_attn_decode_plan(ix, 8, 4, 64, 0.05)
    assert k_max > 1
    with pytest.raises(ValueError, match="sel_ids must have shape"):
        rsa.wave_attn_decode(ix, _q(), 4, 64, 0.05, sel_ids=torch.zeros((2, 8, k_max + 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="out must be torch.float32"):
        rsa.wave_attn_decode(ix, _q(), 4, 64, 0.05, out=torch.zeros((2, 8, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must have shape"):
        rsa.wave_attn_decode(ix, _q(), 4, 64, 0.05, lse=torch.zeros((2, 7), dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace has"):
        rsa.wave_attn_decode(ix, _q(), 4, 64, 0.05, ws=torch.empty(wsb - 1, dtype=torch.uint8))


def test_decode_rejects_host_tensors(cpu_index):
    ix, _ = cpu_index
    with pytest.raises(ValueError, match="must be on the GPU"):
        rsa.wave_attn_decode(ix, _q(), 4, 64, 0.05)


def test_tail_decode_rejects_mis_shaped_tail(cpu_index):
    ix, _ = cpu_index
    kt = torch.zeros((2, G, 64, 128), dtype=torch.bfloat16)
    tl = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="v_tail must have shape"):
        rsa.wave_attn_decode_tail(ix, _q(), 4, 64, 0.05, kt, kt[:, :, :32].contiguous(), tl)
    with pytest.raises(ValueError, match="tail_len must be torch.int32"):
        rsa.wave_attn_decode_tail(ix, _q(), 4, 64, 0.05, kt, kt, tl.to(torch.int64))
    with pytest.raises(ValueError, match="must be on the GPU"):
        rsa.wave_attn_decode_tail(ix, _q(), 4, 64, 0.05, kt, kt, tl)
