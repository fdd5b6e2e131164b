"""GPU: the binding refuses tensors a kernel must never see -- host tensors,
non-contiguous views, mixed dtypes, windows off the device -- before any
pointer reaches the C ABI."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


def test_host_tensor_is_refused(dt):
    xs = [torch.ones(64, device="cuda"), torch.ones(64)]
    with pytest.raises(ValueError):
        dt.dt_allreduce(xs, [torch.empty(64, device="cuda") for _ in range(2)])
    with pytest.raises(ValueError):
        dt.dt_all_gather([torch.ones(8, device="cuda")] * 2, [torch.empty(16), torch.empty(16, device="cuda")])
    with pytest.raises(ValueError):
        dt.dt_bucket_allreduce([[torch.ones(8, device="cuda")]] * 2, bucket_bytes=64, bucket_ws=[torch.empty(64)] * 2)


def test_non_contiguous_and_mixed_dtypes_are_refused(dt):
    base = torch.ones(8, 8, device="cuda")
    with pytest.raises(ValueError):
        dt.dt_allreduce([base.t(), base.t().clone()])  # a transposed view is not contiguous
    with pytest.raises(TypeError):
        dt.dt_allreduce([torch.ones(8, device="cuda"), torch.ones(8, device="cuda", dtype=torch.int32)])


def test_barrier_windows_on_the_host_are_refused(dt):
    windows = [torch.zeros(2, dtype=torch.int32, device="cuda"), torch.zeros(2, dtype=torch.int32)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dt.dt_barrier(windows, status, 1)
    with pytest.raises(ValueError):
        dt.dt_barrier([w.cuda() for w in windows], torch.zeros(1, dtype=torch.int32), 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
