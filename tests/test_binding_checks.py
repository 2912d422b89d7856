"""The Python binding rejects buffers the kernels would read or write out of
bounds (wrong device, dtype, shape, layout or element count) with ValueError,
before the library is called. Runs on the CPU: no GPU and no built library
are needed, because every check precedes the library call."""
import pytest
import torch

import temporally_biased_flashattention_amd as tara


def _args(B=1, H=2, N=64, D=64, dtype=torch.bfloat16):
    q, k, v, o = (torch.zeros(B, H, N, D, dtype=dtype) for _ in range(4))
    return dict(q=q, k=k, v=v, o=o, lse=torch.zeros(B, H, N), seg_type=torch.zeros(B, N, dtype=torch.uint8),
                token_time=torch.zeros(B, N), picture_id=None, mask_weight=None, params=tara.TaraParams(),
                workspace=torch.zeros(256, dtype=torch.uint8))


def _raises(match, **over):
    a = _args()
    a.update(over)
    with pytest.raises(ValueError, match=match):
        tara.tara_attn_fwd(**a)


def test_well_formed_cpu_buffers_are_refused_for_their_device():
    _raises("HIP device")


@pytest.mark.parametrize("name", ["k", "v", "o"])
def test_shape_and_dtype_must_match_q(name):
    _raises(f"{name} has shape", **{name: torch.zeros(1, 2, 63, 64, dtype=torch.bfloat16)})
    _raises(f"{name} is torch.float32", **{name: torch.zeros(1, 2, 64, 64)})


def test_q_must_be_4d():
    _raises("4-D", q=torch.zeros(2, 64, 64, dtype=torch.bfloat16))


def test_lse_layout():
    _raises("lse must be", lse=torch.zeros(1, 2, 63))
    _raises("lse must be", lse=torch.zeros(1, 2, 64, dtype=torch.float64))
    _raises("lse must be", lse=torch.zeros(1, 64, 2).transpose(1, 2))


def test_metadata_layout():
    _raises("seg_type must be", seg_type=torch.zeros(1, 64, dtype=torch.int32))
    _raises("seg_type must be", seg_type=torch.zeros(1, 63, dtype=torch.uint8))
    _raises("token_time must be", token_time=torch.zeros(1, 64, dtype=torch.float16))
    _raises("token_time must be", token_time=torch.zeros(1, 128)[:, ::2])
    _raises("picture_id must be", picture_id=torch.zeros(1, 64, dtype=torch.int32))
    _raises("picture_id must be", picture_id=torch.zeros(1, 32, dtype=torch.int16))


def test_mask_planes_follow_the_binding_count():
    p = tara.TaraParams()
    p.binding_enabled, p.num_pictures, p.num_bindings = 1, 2, 2
    # two chained bindings read two mask planes: one [B, N] plane is too small
    _raises("mask_weight must hold \\[2, 1, 64\\]", params=p, mask_weight=torch.zeros(1, 64))
    _raises("mask_weight must hold", params=p, mask_weight=torch.zeros(2, 64))
    _raises("mask_weight must be a contiguous float32", params=p, mask_weight=torch.zeros(2, 1, 64,
                                                                                           dtype=torch.float64))
    # the right plane count passes the mask check and fails only for the device
    _raises("HIP device", params=p, mask_weight=torch.zeros(2, 1, 64))
    # more planes than bindings: the library reads the first ones
    p.num_bindings = 1
    _raises("HIP device", params=p, mask_weight=torch.zeros(2, 1, 64))


def test_mask_is_not_sized_when_binding_is_off():
    # the library never reads the mask without binding
    _raises("HIP device", mask_weight=torch.zeros(3, 1, 64))


def test_workspace_must_be_contiguous():
    _raises("workspace must be", workspace=torch.zeros(64, 4, dtype=torch.uint8).t())
