"""The Python binding's checks on tensor arguments, without a GPU: the C ABI
sees only pointers and n, so a tensor of the wrong element width, a
non-contiguous one, one shorter than n, one off the GPU, or a strided view
reaching outside its source's storage is refused before the library is
called."""
import pytest
import torch

import memory_bound_elementwise_amd as ew


def test_element_width_is_checked():
    h = torch.zeros(8, dtype=torch.float16)
    f = torch.zeros(8)
    with pytest.raises(TypeError, match="2-byte elements, the operation takes 4"):
        ew.ew_add_f32(h, f, f)
    with pytest.raises(TypeError, match="4-byte elements, the operation takes 2"):
        ew.ew_relu_bf16(f, h)
    with pytest.raises(TypeError):
        ew.ew_sqrt_f16(f, h)


def test_non_contiguous_tensors_are_refused():
    x = torch.zeros(16)[::2]
    with pytest.raises(ValueError, match="not contiguous"):
        ew.ew_relu_f32(x, torch.zeros(8))


def test_a_tensor_shorter_than_n_is_refused():
    a, c = torch.zeros(4), torch.zeros(8)
    with pytest.raises(ValueError, match="4 elements, the call covers 8"):
        ew.ew_add_f32(a, c, c)
    with pytest.raises(ValueError, match="call covers 9"):
        ew.ew_scale_f32(2.0, c, c, n=9)
    with pytest.raises(ValueError, match="bias: 3 elements, the call covers 4"):
        ew.ew_bias_relu_f32(1 << 40, torch.zeros(3), torch.zeros(12), 3, 4)


def test_tensors_off_the_gpu_are_refused():
    x = torch.zeros(8)
    with pytest.raises(ValueError, match="not on a GPU"):
        ew.ew_copy_f32(x, torch.zeros(8))
    with pytest.raises(ValueError, match="not on a GPU"):
        ew.ew_gather_f32(x, torch.zeros(8), 3)


def test_strided_view_must_stay_inside_its_source():
    base = torch.zeros(100)
    with pytest.raises(ValueError, match="view reaches elements 0..100 of a storage of 100"):
        ew.ew_copy2d_f32(base, 10, 1, torch.zeros(110), 10, 11)     # row 9 ends at 100
    with pytest.raises(ValueError, match="view reaches"):
        ew.ew_copy2d_f32(base[5:], -1, 1, torch.zeros(14), 7, 2)     # reaches element -1
    with pytest.raises(ValueError, match="not on a GPU"):             # inside: device check
        ew.ew_copy2d_f32(base, 10, 1, torch.zeros(27), 9, 3)
