"""The Python binding's argument checks that run before any library call
(host only): tensors off the GPU, wrong dtypes and layouts are refused with
TypeError / ValueError, so nothing reaches the C ABI with pointers that do not
describe the sizes passed."""
import pytest
import torch

import elementwise_symmetry_range_amd as pa


def test_elementwise_refuses_host_tensors_and_bad_dtypes():
    x = torch.zeros(16, dtype=torch.float16)
    with pytest.raises(TypeError):
        pa.poly_act_fwd(x, "sigmoid")
    with pytest.raises(TypeError):
        pa.poly_act_bwd(x, x, "tanh")
    with pytest.raises(TypeError):
        pa.native_act_fwd(torch.zeros(16, dtype=torch.float32), "gelu")
    with pytest.raises(TypeError):
        pa.stream_copy(x)


def test_swiglu_refuses_host_tensors():
    g = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        pa.poly_swiglu_fwd(g, g)
    with pytest.raises(TypeError):
        pa.poly_swiglu_bwd(g, g, g)


def test_attention_refuses_host_tensors_and_bad_ranks():
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        pa.poly_softcap_attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        pa.poly_sigmoid_attn_fwd(q[0], q[0], q[0])


def test_unknown_names():
    with pytest.raises(KeyError):
        pa.program_info("relu", 0)
