"""The Python binding rejects arguments the library would read or write through
a device pointer when they are host tensors, of the wrong type, too short or
strided: it raises before any call into the library (a host address handed to
a kernel would fault the GPU).  Host only: every case fails in the binding's
own checks, so no GPU is needed."""
import ctypes

import pytest
import torch

import silent_corruption_detection_amd as sdc

CUDA0 = torch.device("cuda", 0)


def fake_plan(n_tensors=3):
    info = sdc._PlanInfo()
    info.n_tensors = n_tensors
    return sdc.Plan(torch.empty(1, dtype=torch.uint8), info, [], CUDA0)


def host(*shape, dtype=torch.int64):
    return torch.zeros(shape, dtype=dtype)


def test_arg_helper_rules(monkeypatch):
    t = host(8)
    with pytest.raises(ValueError, match="must be on"):
        sdc._arg(t, "x", torch.int64, 1, CUDA0)
    with pytest.raises(TypeError):
        sdc._arg([0, 1], "x", torch.int64, 1, CUDA0)
    assert not sdc._on_device(t, CUDA0)
    assert not sdc._on_device(t, torch.device("cuda"))
    # a tensor on GPU 1: matches "cuda" and cuda:1, not cuda:0
    monkeypatch.setattr(torch.Tensor, "get_device", lambda self: 1)
    assert sdc._on_device(t, torch.device("cuda"))
    assert sdc._on_device(t, torch.device("cuda", 1))
    assert not sdc._on_device(t, CUDA0)


def test_plan_scans_reject_host_outputs():
    plan = fake_plan()
    with pytest.raises(ValueError, match="out must be on"):
        sdc.sdc_fingerprint_plan(plan, out=host(3, 4))
    with pytest.raises(ValueError, match="counts must be on"):
        sdc.sdc_nonfinite(plan, counts=host(3), total=host(1))
    with pytest.raises(ValueError, match="sq must be on"):
        sdc.sdc_sqnorm(plan, sq=host(3, dtype=torch.float64), total=host(1, dtype=torch.float64),
                       flag=host(1, dtype=torch.int32))


def test_compares_reject_host_tables():
    with pytest.raises(ValueError, match="table must be on"):
        sdc.sdc_majority_compare(host(3, 4), 3, 1)
    with pytest.raises(ValueError, match="a must be on"):
        sdc.sdc_fingerprint_diff(host(5, 4), host(5, 4))
    with pytest.raises(ValueError, match="table must be on"):
        sdc.sdc_ring_compare(host(4, 2, 3), 4, 1)
    with pytest.raises(ValueError, match="must be on"):
        sdc.sdc_confirm_verdict(host(6), host(6), host(6), host(6))


def test_read_sum_and_tensor_scan_reject_host_tensors():
    with pytest.raises(ValueError):
        sdc.sdc_read_sum(host(64, dtype=torch.int32))
    with pytest.raises(ValueError, match="not on a GPU"):
        sdc.sdc_fingerprint_tensor(host(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="not on a GPU"):
        sdc.sdc_plan_build([host(64, dtype=torch.float32)])


def test_shapes_and_types_are_checked(monkeypatch):
    # pretend the host tensors are on cuda:0 so that the later checks are reached
    monkeypatch.setattr(sdc, "_on_device", lambda t, device: True)
    plan = fake_plan(3)
    with pytest.raises(ValueError, match="at least 12"):
        sdc.sdc_fingerprint_plan(plan, out=host(2, 4))
    with pytest.raises(ValueError, match="must be torch.int64"):
        sdc.sdc_fingerprint_plan(plan, out=host(3, 4, dtype=torch.int32))
    with pytest.raises(ValueError, match="contiguous"):
        sdc.sdc_fingerprint_plan(plan, out=host(4, 3).t())
    with pytest.raises(ValueError, match="counts needs at least 3"):
        sdc.sdc_nonfinite(plan, counts=host(2), total=host(1))
    with pytest.raises(ValueError, match="flag must be torch.int32"):
        sdc.sdc_sqnorm(plan, sq=host(3, dtype=torch.float64), total=host(1, dtype=torch.float64),
                       flag=host(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="tensor_status"):
        sdc.sdc_majority_compare(host(3, 4), 3, 1, tensor_status=host(1, dtype=torch.int8))
