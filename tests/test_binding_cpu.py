"""The Python binding on the CPU: it marshals only GPU tensors, so host tensors are
refused with a clear error before the library is called (the library sees raw
addresses and could not tell a host pointer from a device one)."""
import pytest
import torch

import decode_mhc_pre_amd as M

C = 5120


def test_host_tensors_are_refused_before_any_call():
    x = torch.zeros((8, 4, C), dtype=torch.bfloat16)
    pin = torch.zeros((8, 4), dtype=torch.float32)
    w = M.Weights(torch.zeros(M.mhc_fn_packed_bytes(4 * C), dtype=torch.uint8), torch.zeros(24), torch.ones(3), 4 * C)
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_pre(x, w)
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_pre_delayed(x, pin, w)
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_post(torch.zeros((8, C), dtype=torch.bfloat16), x, pin, torch.zeros((8, 4, 4)))
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_collapse(x, pin)
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_broadcast_entry(torch.zeros((8, C), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="must be on"):
        M.mhc_pack_fn(torch.zeros((4 * C, 24)))


def test_malformed_residuals_are_refused():
    with pytest.raises(ValueError, match="streams"):
        M.mhc_pre(torch.zeros((8, 3, C), dtype=torch.bfloat16), None)
    with pytest.raises(ValueError, match=r"\[T, 4, C\]"):
        M.mhc_pre_delayed(torch.zeros((8, 4 * C), dtype=torch.bfloat16), None, None)
