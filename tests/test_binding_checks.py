"""The Python binding's argument checks, without a GPU: tensors that are not on a GPU, of the
wrong dtype, shape or layout are refused with ValueError before the library is called."""
import pytest
import torch

from paged_kv_decode_write_amd import _binding as pk


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="GPU device"):
        pk.paged_kv_write(bf16(2, 8, 128), bf16(2, 8, 128), torch.zeros(2, dtype=torch.int64),
                          bf16(4, 16, 8, 128), bf16(4, 16, 8, 128))
    with pytest.raises(ValueError, match="GPU device"):
        pk.paged_decode_attention(bf16(2, 32, 128), bf16(4, 16, 8, 128), bf16(4, 16, 8, 128),
                                  torch.zeros(2, 4, dtype=torch.int32),
                                  torch.ones(2, dtype=torch.int32), 0.1,
                                  torch.zeros(2, 32, 128))


def test_wrong_dtypes_are_refused_before_devices_are_looked_at():
    with pytest.raises(ValueError, match="must be"):
        pk.paged_decode_attention(bf16(2, 32, 128), torch.zeros(4, 16, 8, 128),
                                  bf16(4, 16, 8, 128), torch.zeros(2, 4, dtype=torch.int32),
                                  torch.ones(2, dtype=torch.int32), 0.1,
                                  torch.zeros(2, 32, 128))
    with pytest.raises(ValueError, match="must have 4 dimensions"):
        pk.paged_kv_write(bf16(2, 8, 128), bf16(2, 8, 128), torch.zeros(2, dtype=torch.int64),
                          bf16(4, 16, 1024), bf16(4, 16, 8, 128))


def test_non_tensors_are_refused():
    with pytest.raises(TypeError):  # the pools are checked first
        pk.paged_kv_write(bf16(2, 8, 128), bf16(2, 8, 128), torch.zeros(2, dtype=torch.int64),
                          [0], bf16(4, 16, 8, 128))


def test_prepared_step_checks_at_preparation():
    """A prepared decode step runs the same checks as paged_decode_step when it is built."""
    with pytest.raises(ValueError, match="GPU device"):
        pk.prepare_decode_step(bf16(2, 32, 128), bf16(2, 8, 128), bf16(2, 8, 128),
                               torch.zeros(2, dtype=torch.int64), bf16(4, 16, 8, 128),
                               bf16(4, 16, 8, 128), torch.zeros(2, 4, dtype=torch.int32),
                               torch.ones(2, dtype=torch.int32), 0.1, torch.zeros(2, 32, 128))
    with pytest.raises(ValueError, match="must be"):
        pk.prepare_decode_step(bf16(2, 32, 128), bf16(2, 8, 128), bf16(2, 8, 128),
                               torch.zeros(2, dtype=torch.int32), bf16(4, 16, 8, 128),
                               bf16(4, 16, 8, 128), torch.zeros(2, 4, dtype=torch.int32),
                               torch.ones(2, dtype=torch.int32), 0.1, torch.zeros(2, 32, 128))
