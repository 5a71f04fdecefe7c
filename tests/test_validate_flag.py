"""MEDUSA_VALIDATE: with the flag set, every device entry point of the binding waits for its
work and raises if the round's status word holds an error; host-detected errors raise as
always.  Runs on the CPU (status words held in host tensors; the host checks of a device
entry point return before any launch)."""
import pytest
import torch

import medusa_tree_attention_amd as M
from medusa_tree_attention_amd import _binding as B


def test_flag_off_by_default(monkeypatch):
    monkeypatch.delenv(B.VALIDATE_ENV, raising=False)
    assert not B.validating()
    B._validate("medusa_kv_compact", torch.tensor([-3], dtype=torch.int32))  # ignored


@pytest.mark.parametrize("value,on", [("1", True), ("yes", True), ("0", False), ("", False)])
def test_flag_values(monkeypatch, value, on):
    monkeypatch.setenv(B.VALIDATE_ENV, value)
    assert B.validating() is on


@pytest.mark.parametrize("code,name", [(-1, "MEDUSA_EINVAL"), (-3, "MEDUSA_ECAPACITY"),
                                       (-4, "MEDUSA_EUNSUPPORTED")])
def test_nonzero_status_word_raises(monkeypatch, code, name):
    monkeypatch.setenv(B.VALIDATE_ENV, "1")
    with pytest.raises(M.MedusaError) as e:
        B._validate("medusa_tree_attn", torch.tensor([code], dtype=torch.int32))
    assert e.value.name == name and e.value.code == code
    B._validate("medusa_tree_attn", torch.tensor([0], dtype=torch.int32))  # a clean round passes


def test_host_errors_still_raise_in_validation_mode(monkeypatch):
    """A head size the library does not support is refused on the host, before any launch
    and before the status word is looked at."""
    monkeypatch.setenv(B.VALIDATE_ENV, "1")
    q = torch.zeros((1, 7, 1, 96))
    kv = torch.zeros((1, 7, 1, 96))
    cache = torch.zeros((1, 1, 135, 96))
    depth = torch.zeros(7, dtype=torch.int32)
    mask = torch.zeros((7, 1), dtype=torch.int64)
    prefix = torch.tensor([128], dtype=torch.int32)
    status = torch.tensor([-1], dtype=torch.int32)  # would raise EINVAL if it were read
    with pytest.raises(M.MedusaError) as e:
        M.medusa_tree_attn(q, kv, kv, cache, cache, depth, mask, prefix, 1e4, q, None, status, stream=0)
    assert e.value.name == "MEDUSA_EUNSUPPORTED"
