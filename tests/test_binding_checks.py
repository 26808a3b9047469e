"""Host-side buffer checks of the Python binding (CPU only).

The C ABI takes raw device pointers, so the binding checks dtype, size,
contiguity and device of every tensor it hands over; each mismatch must
raise ValueError before any launch. Run here with CPU tensors and
device_type="cpu" (the dtype/size/contiguity checks), plus the rejection of
a host tensor where a device tensor is required."""
import pytest
import torch

from moe_expert_ffn_persistent_amd import check_combine_inputs, check_layout_inputs, make_shape

S, T, E, K, L, H, I = 2, 5, 8, 3, 4, 256, 128
N = S * T


def shape():
    return make_shape(S, T, E, K, 0, L, H, I, "bf16")


def f32(*sz):
    return torch.zeros(*sz, dtype=torch.float32)


def i32(*sz):
    return torch.zeros(*sz, dtype=torch.int32)


def test_layout_inputs_accept_the_right_buffers():
    check_layout_inputs(shape(), logits=f32(N, E), bias=f32(E), device_type="cpu")
    check_layout_inputs(shape(), logits=f32(N, E), device_type="cpu")
    check_layout_inputs(shape(), topk_idx=i32(N, K), topk_w=f32(N, K), device_type="cpu")


@pytest.mark.parametrize("case", ["logits_dtype", "logits_short", "logits_noncontig", "bias_short",
                                  "bias_dtype", "idx_dtype", "idx_short", "w_dtype", "w_missing",
                                  "bias_without_logits"])
def test_layout_inputs_reject_mismatches(case):
    kw = dict(logits=f32(N, E), bias=f32(E))
    if case == "logits_dtype":
        kw["logits"] = torch.zeros(N, E, dtype=torch.float16)
    elif case == "logits_short":
        kw["logits"] = f32(N, E - 1)
    elif case == "logits_noncontig":
        kw["logits"] = f32(E, N).t()
    elif case == "bias_short":
        kw["bias"] = f32(E - 1)
    elif case == "bias_dtype":
        kw["bias"] = torch.zeros(E, dtype=torch.float64)
    elif case == "idx_dtype":
        kw = dict(topk_idx=torch.zeros(N, K, dtype=torch.int64), topk_w=f32(N, K))
    elif case == "idx_short":
        kw = dict(topk_idx=i32(N, K - 1), topk_w=f32(N, K))
    elif case == "w_dtype":
        kw = dict(topk_idx=i32(N, K), topk_w=torch.zeros(N, K, dtype=torch.bfloat16))
    elif case == "w_missing":
        kw = dict(topk_idx=i32(N, K))
    elif case == "bias_without_logits":
        kw = dict(topk_idx=i32(N, K), topk_w=f32(N, K), bias=f32(E))
    with pytest.raises(ValueError):
        check_layout_inputs(shape(), device_type="cpu", **kw)


def test_host_tensor_rejected_where_device_memory_is_needed():
    with pytest.raises(ValueError):
        check_layout_inputs(shape(), logits=f32(N, E))          # device_type defaults to cuda
    with pytest.raises(ValueError):
        check_combine_inputs(shape(), [torch.zeros(T, K, H, dtype=torch.int16)] * S)


def comb():
    return [torch.zeros(T, K, H, dtype=torch.int16) for _ in range(S)]


def test_combine_inputs_accept_the_right_buffers():
    check_combine_inputs(shape(), comb(), f32(N, H), i32(4), device_type="cpu")
    check_combine_inputs(shape(), [torch.zeros(T, K, H, dtype=torch.bfloat16) for _ in range(S)],
                         device_type="cpu")
    check_combine_inputs(shape(), comb(), torch.zeros(N, H, dtype=torch.bfloat16), device_type="cpu")


@pytest.mark.parametrize("case", ["slices_count", "slice_dtype", "slice_short", "slice_noncontig",
                                  "y_dtype", "y_half", "y_short", "y_bf16_short", "report_short",
                                  "report_dtype"])
def test_combine_inputs_reject_mismatches(case):
    c, y, rep = comb(), f32(N, H), i32(4)
    if case == "slices_count":
        c = c[:-1]
    elif case == "slice_dtype":
        c[0] = torch.zeros(T, K, H, dtype=torch.float32)
    elif case == "slice_short":
        c[1] = torch.zeros(T, K, H - 1, dtype=torch.int16)
    elif case == "slice_noncontig":
        c[0] = torch.zeros(H, K, T, dtype=torch.int16).permute(2, 1, 0)
    elif case == "y_dtype":
        y = torch.zeros(N, H, dtype=torch.float64)[:, : H // 2]
    elif case == "y_half":
        y = torch.zeros(N, H, dtype=torch.float16)
    elif case == "y_short":
        y = f32(N, H - 1)
    elif case == "y_bf16_short":
        y = torch.zeros(N, H - 1, dtype=torch.bfloat16)
    elif case == "report_short":
        rep = i32(3)
    elif case == "report_dtype":
        rep = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        check_combine_inputs(shape(), c, y, rep, device_type="cpu")
