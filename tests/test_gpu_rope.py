"""Rotary position embedding on the GPU against the oracle (reading R10):
both storage dtypes, the rope part at the end of the head (beside a non-rope
part) and over the whole head, positions from 0 to past a million, inactive
rows, a row count that leaves a ragged last workgroup."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,rows,heads,d,off,rd,base", [
    (binding.DTYPE_BF16, 2 * 300, 4, 96, 32, 64, 10000.0),     # rope part after a 32-channel non-rope part
    (binding.DTYPE_BF16, 257, 1, 128, 0, 128, 10000.0),
    (binding.DTYPE_F32, 2 * 300, 4, 96, 32, 64, 10000.0),
    (binding.DTYPE_F32, 129, 3, 64, 16, 32, 500.0),
])
def test_rope_matches_oracle(dtype, rows, heads, d, off, rd, base):
    lib()
    inp = synth.make_rope(rows=rows, heads=heads, d=d, dtype=dtype, seed=rows + d)
    x = dev(inp["x"])
    binding.rope_apply(x, dev(inp["pos"]), rope_off=off, rope_dim=rd, base=base)
    got = host(x)
    want = O.rope(inp["x"], inp["pos"], rope_off=off, rope_dim=rd, dtype=dtype, base=base)
    assert_close(got, want, f"rope {dtype} rows={rows} heads={heads} d={d} [{off}, {off + rd})")
    keep = [c for c in range(d) if not off <= c < off + rd]
    assert np.array_equal(got[:, :, keep], inp["x"][:, :, keep])        # other channels bitwise untouched
    assert np.array_equal(got[1], inp["x"][1])                          # inactive row untouched
    assert np.array_equal(got[0], inp["x"][0])                          # position 0: identity


def test_rope_on_query_tensor_shape_and_empty():
    # a [B, T, H, d] query tensor with [B, T] positions; an empty tensor is a no-op
    lib()
    inp = synth.make_rope(rows=3 * 50, heads=8, d=128, seed=5)
    q = dev(inp["x"]).view(3, 50, 8, 128)
    binding.rope_apply(q, dev(inp["pos"]).view(3, 50), rope_off=64, rope_dim=64)
    want = O.rope(inp["x"], inp["pos"], rope_off=64, rope_dim=64, dtype=binding.DTYPE_BF16)
    assert_close(host(q).reshape(150, 8, 128), want, "rope on [B, T, H, d]")
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=q.device)
    binding.rope_apply(e, torch.empty((0,), dtype=torch.int64, device=q.device), rope_off=0, rope_dim=128)
