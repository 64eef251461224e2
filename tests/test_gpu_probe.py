"""The HBM read-ceiling probe reads exactly the listed K and V blocks: the XOR
of its sink words equals the XOR of every 32-bit word of those blocks,
computed on the host (each block listed once, in any order, with lists
shorter and longer than the number of waves)."""
import numpy as np
import pytest
import torch

from speculative_decoding_verification_attn_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_list", [1, 7, 1000, 5003])
def test_probe_xor_of_listed_blocks(d, n_list):
    rng = np.random.default_rng(n_list + d)
    pages, hkv = 700, 8
    k = rng.integers(0, 2**16, size=(pages, hkv, 16, d), dtype=np.uint16)
    v = rng.integers(0, 2**16, size=(pages, hkv, d, 16), dtype=np.uint16)  # V pages are stored transposed
    chunks = rng.choice(pages * hkv, size=n_list, replace=False).astype(np.int32)
    dev = "cuda:0"
    kd = torch.from_numpy(k.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
    sink = ops.spec_hbm_read_probe(kd, vd, torch.from_numpy(chunks).to(dev))
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    kb = k.reshape(pages * hkv, -1).view(np.uint32)[chunks]
    vb = v.reshape(pages * hkv, -1).view(np.uint32)[chunks]
    want = np.bitwise_xor.reduce(np.concatenate([kb.ravel(), vb.ravel()]))
    assert got == want
