"""The Python binding checks the shapes and dtypes of the buffers it hands
to the library (which trusts its sizes) before anything touches a device,
so these run on CPU tensors without a GPU."""
import pytest
import torch

import quantization_dit_linear_amd as q


def test_linear_rejects_mismatched_buffers():
    K = 256
    a = torch.zeros((4, K // 2), dtype=torch.uint8)
    w = torch.zeros((3, K // 2), dtype=torch.uint8)
    an = torch.zeros((4,), dtype=torch.float32)
    wn = torch.zeros((3,), dtype=torch.float32)
    with pytest.raises(ValueError, match="a_codes"):
        q.linear(a, an, 8, w, wn, 4, K)                      # 4-bit bytes read as 8-bit
    with pytest.raises(ValueError, match="w_norms"):
        q.linear(a, an, 4, w, wn[:2], 4, K)
    with pytest.raises(ValueError, match="out"):
        q.linear(a, an, 4, w, wn, 4, K, out=torch.zeros((4, 4), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        q.linear(a, an, 4, w, wn, 4, K, out=torch.zeros((4, 3), dtype=torch.float32))
    # consistent shapes get as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        q.linear(a, an, 4, w, wn, 4, K, out=torch.zeros((4, 3), dtype=torch.bfloat16))


def test_rotate_and_prepare_reject_mismatched_outputs():
    x = torch.zeros((5, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        q.rotate_quantize(x, 1, 4, out=torch.zeros((5, 64), dtype=torch.uint8))
    with pytest.raises(ValueError, match="norms"):
        q.rotate_quantize(x, 1, 4, norms=torch.zeros((4,), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        q.fake_quantize(x, 1, 4, out=torch.zeros((5, 256), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        q.prepare_weights(x, 1, 8, out=torch.zeros((5, 128), dtype=torch.uint8))


def test_rtn4_and_permute_reject_mismatched_buffers():
    W = torch.zeros((6, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="scales"):
        q.rtn4_prepare_weights(W, scales=torch.zeros((5,), dtype=torch.float32))
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    q4 = torch.zeros((6, 32), dtype=torch.uint8)
    with pytest.raises(ValueError, match="q4"):
        q.rtn4_linear(x, q4[:, :16], torch.zeros((6,), dtype=torch.float32))
    src = torch.zeros((256, 3), dtype=torch.float32)
    with pytest.raises(ValueError, match="out"):
        q.permute_rows(src, 1, out=torch.zeros((256, 3), dtype=torch.float16))
