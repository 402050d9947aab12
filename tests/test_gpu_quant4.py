"""4-bit cache storage on the GPU against the oracle (reading R11): codes and
(min, step) bit-exact, decoded values within the float tolerance; both
dtypes, an odd element count, a one-element and a constant tensor, a tensor
of the HCA decode-cache shape."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,n,constant", [
    (binding.DTYPE_BF16, 16 * 8192 * 128, None),     # an HCA cache of the 1M decode shape (16 x 8192 x 128)
    (binding.DTYPE_BF16, 2 * 300 * 128 + 1, None),
    (binding.DTYPE_F32, 1001, None),
    (binding.DTYPE_F32, 1, None),
    (binding.DTYPE_BF16, 77, 1.5),
])
def test_quant4_matches_oracle(dtype, n, constant):
    lib()
    x = synth.make_quant(n=n, dtype=dtype, constant=constant, seed=n % 1000)
    xd = dev(x)
    codes, params = binding.cache_quant4(xd)
    want_codes, mn, st = O.quant4(x, dtype)
    got_params = host(params)
    assert got_params[0] == mn and got_params[1] == st, (got_params, mn, st)
    got_codes = host(codes)
    bad = np.nonzero(got_codes != want_codes)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[0]}"
    out = torch.empty_like(xd)
    binding.cache_dequant4(codes, params, out)
    assert_close(host(out), O.dequant4(want_codes, mn, st, n, dtype), f"dequant4 dtype={dtype} n={n}")


def test_quant4_repeat_reuses_params():
    # the params buffer is also the reduction scratch: a second call on it must start afresh
    lib()
    a = dev(synth.make_quant(n=5000, seed=1))
    b = dev(synth.make_quant(n=4000, seed=2)) * 0.25
    codes_a, params = binding.cache_quant4(a)
    codes_b = torch.empty((4000 + 1) // 2, dtype=torch.uint8, device=a.device)
    binding.cache_quant4(b, codes=codes_b, params=params)
    want_codes, mn, st = O.quant4(host(b), binding.DTYPE_BF16)
    assert tuple(host(params)) == (mn, st)
    assert np.array_equal(host(codes_b), want_codes)
