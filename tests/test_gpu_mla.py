"""GPU parity of the fp8 MLA cache writer against the CPU oracle (bit-exact
bytes, untouched entries left alone)."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, bf16_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((n, 512)).astype(np.float32)
    kv *= np.exp(rng.standard_normal((n, 4, 1)) * 4).astype(np.float32).repeat(128, axis=1).reshape(n, 512)
    kv[0, 128:256] = 0.0                          # all-zero tile -> FLT_MIN scale
    kv[1, :128] = -0.0
    kv[2, 256:384] = 3.0                          # constant tile
    kv[3, 384:] *= 1e-30                          # tiny tile (subnormal codes)
    kv[4, 0] = 2.0 ** -133                        # bf16 subnormal next to zeros
    kv[4, 1:128] = 0.0
    kpe = rng.standard_normal((n, 64)).astype(np.float32) * 10
    return synth.f32_to_bf16_bits(kv), synth.f32_to_bf16_bits(kpe)


@pytest.mark.parametrize("block_size,num_blocks", [(64, 6), (16, 20)])
def test_mla_cache_write_bit_exact(block_size, num_blocks):
    _say(f"mla_cache_write: block_size {block_size}, {num_blocks} blocks")
    n = 300
    kv_bits, kpe_bits = _inputs(n, 11 + block_size)
    rng = np.random.default_rng(7)
    nslots = num_blocks * block_size
    slots = rng.permutation(nslots)[:n].astype(np.int64)
    slots[::17] = -1                               # skipped
    slots[5::23] = nslots + np.arange(len(slots[5::23]))   # past the cache: skipped
    cache_np = np.full((num_blocks, block_size, 656), 0xA5, np.uint8)
    ref = O.mla.mla_cache_write(synth.bf16_bits_to_f32(kv_bits), synth.bf16_bits_to_f32(kpe_bits),
                                slots, cache_np.copy())
    cache = torch.from_numpy(cache_np).to(DEV)
    # row strides wider than the used width (kv [n, 576], kpe [n, 80])
    kv_wide = torch.zeros((n, 576), dtype=torch.bfloat16, device=DEV)
    kv_wide[:, :512] = bf16_tensor(kv_bits)
    kpe_wide = torch.zeros((n, 80), dtype=torch.bfloat16, device=DEV)
    kpe_wide[:, :64] = bf16_tensor(kpe_bits)
    sai.mla_cache_write(kv_wide[:, :512], kpe_wide[:, :64], torch.from_numpy(slots).to(DEV), cache)
    got = cache.cpu().numpy()
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{len(diff)} bytes differ, first at {diff[:5].tolist()}")
