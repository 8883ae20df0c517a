"""The binding checks every tensor argument before it calls the library, which reads
raw pointers: a wrong dtype, shape, layout or device must raise ValueError, never
reach a kernel.  These run on the CPU (the device requirement is relaxed, every other
check is the one chunk_fwd, chunk_inverse and gate_scan apply); nothing is launched."""
import pytest
import torch

from gated_deltanet_chunked_fwd_amd.binding import (check_forward_args, check_gate_args,
                                                    check_inverse_args)

B, T, H, DK, DV = 2, 70, 3, 64, 128


def valid(dtype=torch.bfloat16):
    return dict(q=torch.zeros(B, T, H, DK, dtype=dtype), k=torch.zeros(B, T, H, DK, dtype=dtype),
                v=torch.zeros(B, T, H, DV, dtype=dtype), g=torch.zeros(B, T, H),
                beta=torch.zeros(B, T, H, dtype=dtype))


def check(**kw):
    return check_forward_args(require_cuda=False, **kw)


def test_valid_arguments_pass():
    for dt in (torch.bfloat16, torch.float32):
        a = valid(dt)
        assert check(**a) is None
        check(**a, initial_state=torch.zeros(B, H, DK, DV), out=torch.zeros(B, T, H, DV, dtype=dt),
              final_state_out=torch.zeros(B, H, DK, DV), workspace=torch.zeros(16, dtype=torch.uint8))
    a = valid()
    a["beta"] = a["beta"].float()   # fp32 beta with bf16 q/k/v is a supported combination
    check(**a)


@pytest.mark.parametrize("name,bad", [
    ("q", torch.zeros(B, T, H, DK, dtype=torch.float16)),
    ("k", torch.zeros(B, T, H, DK)),                            # fp32 k with bf16 q
    ("k", torch.zeros(B, T, H, DK + 64, dtype=torch.bfloat16)),
    ("v", torch.zeros(B, T, H, DV)),                            # fp32 v with bf16 q
    ("v", torch.zeros(B, T + 1, H, DV, dtype=torch.bfloat16)),
    ("g", torch.zeros(B, T, H, dtype=torch.bfloat16)),          # g must be fp32
    ("g", torch.zeros(B, T, H + 1)),
    ("beta", torch.zeros(B, T, H, dtype=torch.float16)),
    ("beta", torch.zeros(B, T)),
    ("q", torch.zeros(B, T, DK, H, dtype=torch.bfloat16).transpose(2, 3)),   # not contiguous
    ("v", torch.zeros(B, T, DV, H, dtype=torch.bfloat16).transpose(2, 3)),
])
def test_bad_input_raises(name, bad):
    a = valid()
    a[name] = bad
    with pytest.raises(ValueError):
        check(**a)


@pytest.mark.parametrize("name,bad", [
    ("initial_state", torch.zeros(B, H, DK, DV, dtype=torch.bfloat16)),
    ("initial_state", torch.zeros(B, H, DV, DK + 1)),
    ("initial_state", torch.zeros(B + 1, H, DK, DV)),
    ("out", torch.zeros(B, T, H, DV)),                                  # fp32 out for bf16 v
    ("out", torch.zeros(B, T, H, DK, dtype=torch.bfloat16)),
    ("final_state_out", torch.zeros(B, H, DK, DV, dtype=torch.bfloat16)),
    ("final_state_out", torch.zeros(B, H, DV, DK + 1)),
    ("workspace", torch.zeros(16, dtype=torch.int32)),
    ("workspace", torch.zeros(4, 4, dtype=torch.uint8)),
])
def test_bad_optional_raises(name, bad):
    a = valid()
    a[name] = bad
    with pytest.raises(ValueError):
        check(**a)


def packed():
    lens = [30, 0, 64, 11]
    tot = sum(lens)
    a = dict(q=torch.zeros(1, tot, H, DK, dtype=torch.bfloat16), k=torch.zeros(1, tot, H, DK, dtype=torch.bfloat16),
             v=torch.zeros(1, tot, H, DV, dtype=torch.bfloat16), g=torch.zeros(1, tot, H),
             beta=torch.zeros(1, tot, H, dtype=torch.bfloat16))
    cu = torch.tensor([0, 30, 30, 94, 105], dtype=torch.int32)
    return a, cu


def test_packed_offsets():
    a, cu = packed()
    assert check(**a, cu_seqlens=cu).dtype == torch.int32
    # FLA passes int64 offsets: accepted and handed to the library as int32
    out = check(**a, cu_seqlens=cu.long(), cu_seqlens_host=cu.long())
    assert out.dtype == torch.int32 and out.tolist() == cu.tolist()
    check(**a, cu_seqlens=cu, initial_state=torch.zeros(4, H, DK, DV))
    with pytest.raises(ValueError):   # N follows cu_seqlens: 4 sequences, not B = 1
        check(**a, cu_seqlens=cu, initial_state=torch.zeros(1, H, DK, DV))
    with pytest.raises(ValueError):
        check(**a, cu_seqlens=cu.float())
    with pytest.raises(ValueError):
        check(**a, cu_seqlens=cu.reshape(1, -1))
    with pytest.raises(ValueError):   # host copy that does not end at T
        check(**a, cu_seqlens=cu, cu_seqlens_host=torch.tensor([0, 30, 30, 94, 104], dtype=torch.int32))
    with pytest.raises(ValueError):   # host copy without the device array
        check(**a, cu_seqlens_host=cu)
    b = valid()
    with pytest.raises(ValueError):   # packing needs B == 1
        check(**b, cu_seqlens=torch.tensor([0, T], dtype=torch.int32))


def test_gate_and_inverse_checks():
    g = torch.zeros(1, 100, 4)
    assert check_gate_args(g, require_cuda=False) is None
    assert check_gate_args(g, torch.tensor([0, 40, 100]), require_cuda=False).dtype == torch.int32
    with pytest.raises(ValueError):
        check_gate_args(g.to(torch.bfloat16), require_cuda=False)
    with pytest.raises(ValueError):
        check_gate_args(torch.zeros(2, 100, 4), torch.tensor([0, 40, 100], dtype=torch.int32),
                        require_cuda=False)
    k = torch.zeros(1, 100, 4, 64, dtype=torch.bfloat16)
    check_inverse_args(k, g, torch.zeros(1, 100, 4), require_cuda=False)
    with pytest.raises(ValueError):
        check_inverse_args(k, g, torch.zeros(1, 100, 3), require_cuda=False)
    with pytest.raises(ValueError):
        check_inverse_args(k, g.double(), torch.zeros(1, 100, 4), require_cuda=False)
    with pytest.raises(ValueError):
        check_inverse_args(k.to(torch.float16), g, torch.zeros(1, 100, 4), require_cuda=False)


def test_device_required_by_default():
    with pytest.raises(ValueError):
        check_forward_args(**valid())
