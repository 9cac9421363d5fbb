"""subspec_reject_noalloc (the rejection round with static scratch, for
callers that cannot allocate) against subspec_reject on the same inputs: two
calls in a row, the second with a smaller input, so the second runs on the
array the first left behind."""
import numpy as np
import pytest
import torch

from oracle.sampling import sample as osample
from self_speculative_decoding_w4a16_amd import _lib
from synth import logits_pair, uniform_codes
from tests.gpu_util import codes_i32, log, ws
from tests.helpers import host

pytestmark = pytest.mark.gpu


def _outs(cuda, gamma):
    return (torch.full((1,), -7, dtype=torch.int32, device=cuda),
            torch.full((gamma + 1,), -7, dtype=torch.int32, device=cuda),
            torch.full((1,), -7, dtype=torch.int32, device=cuda),
            torch.zeros((max(gamma, 1), 2), dtype=torch.float32, device=cuda))


def _case(cuda, gamma, V, T, Td, seed):
    zt, zd = logits_pair(gamma, V, seed, device=cuda)
    zdh = host(zd).astype(np.float32)
    Ud, _ = uniform_codes(gamma, seed + 1)
    R, _ = uniform_codes(gamma, seed + 2)
    toks = [osample(zdh[i], Td, int(Ud[i])) for i in range(gamma)]
    if gamma > 2:
        toks[gamma // 2] = (toks[gamma // 2] + 1) % V  # a rejection somewhere
    return zt, zd, codes_i32(toks, cuda), codes_i32(R, cuda), codes_i32([int(seed) * 7919 % (1 << 24)], cuda)


@pytest.mark.parametrize("first,second", [((48, 152064, 0.6, 0.6), (4, 1000, 1.0, 1.0)),
                                          ((16, 152064, 0.0, 0.0), (3, 5000, 1.0, 0.2))])
def test_reject_noalloc_matches_workspace_reject(cuda, first, second):
    buf = ws(1 << 22, cuda)
    for k, (gamma, V, T, Td) in enumerate((first, second)):
        log(f"reject_noalloc call {k}: gamma={gamma} V={V} T={T} Td={Td}")
        zt, zd, toks, rr, uf = _case(cuda, gamma, V, T, Td, 300 + 10 * k + gamma)
        a = _outs(cuda, gamma)
        b = _outs(cuda, gamma)
        _lib.reject(gamma, V, T, Td, zt, zd, toks, rr, uf, *a, buf)
        _lib.reject_noalloc(gamma, V, T, Td, zt, zd, toks, rr, uf, *b)
        torch.cuda.synchronize()
        n = int(a[0].item())
        assert 0 <= n <= gamma
        assert int(b[0].item()) == n
        assert torch.equal(a[1][:n + 1], b[1][:n + 1])
        assert int(a[2].item()) == int(b[2].item())
        assert torch.equal(a[3], b[3])


def test_reject_noalloc_rejects_oversized_calls(cuda):
    log("reject_noalloc size limit")
    out = _outs(cuda, 64)
    z = torch.zeros(1, dtype=torch.bfloat16, device=cuda)
    t = torch.zeros(64, dtype=torch.int32, device=cuda)
    with pytest.raises(_lib.SubspecError) as e:
        _lib.reject_noalloc(64, 1 << 24, 1.0, 1.0, z, z, t, t, t, *out)
    assert e.value.code == _lib.ECAPACITY
    assert int(out[0].item()) == -7  # nothing was enqueued
