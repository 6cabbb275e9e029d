"""The torch binding rejects tensors the C library cannot check for itself (dtype,
shape, device) before any pointer reaches it.  CPU only: every call here raises
ValueError before the library is touched."""
import pytest
import torch

from tiled_exact_attention_bf16_amd import attention as FA

B, S, H, D = 2, 64, 3, 128


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def qkv():
    return bf(B, S, H, D), bf(B, S, H, D), bf(B, S, H, D)


def test_forward_rejects_wrong_input_dtypes_and_shapes():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="q must be torch.bfloat16"):
        FA.fwd(q.float(), k, v)
    with pytest.raises(ValueError, match="v must be torch.bfloat16"):
        FA.fwd(q, k, v.half())
    with pytest.raises(ValueError, match=r"\[B, S, H, D\]"):
        FA.fwd(q[0], k, v)
    with pytest.raises(ValueError, match="v must have the shape of k"):
        FA.fwd(q, k, bf(B, S + 1, H, D))
    with pytest.raises(ValueError, match="head dimension"):
        FA.fwd(bf(B, S, H, 64), k, v)
    with pytest.raises(ValueError, match="number of heads"):
        FA.fwd(bf(B, S, H + 1, D), k, v)
    with pytest.raises(ValueError, match="same batch"):
        FA.fwd(bf(B + 1, S, H, D), k, v)


def test_forward_rejects_wrong_outputs():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out must be torch.bfloat16"):
        FA.fwd(q, k, v, out=torch.zeros(q.shape, dtype=torch.float16))
    with pytest.raises(ValueError, match="out must have shape"):
        FA.fwd(q, k, v, out=bf(B, S, H, 64))
    with pytest.raises(ValueError, match="lse must be torch.float32"):
        FA.fwd(q, k, v, lse=torch.zeros((B, H, S), dtype=torch.float16))
    with pytest.raises(ValueError, match="lse must have shape"):
        FA.fwd(q, k, v, lse=torch.zeros((B, S, H), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must be contiguous"):
        FA.fwd(q, k, v, lse=torch.zeros((B, S, H), dtype=torch.float32).transpose(1, 2))
    with pytest.raises(ValueError, match="workspace"):
        FA.fwd(q, k, v, workspace=torch.zeros(16, dtype=torch.float32))


def test_forward_rejects_host_tensors():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        FA.fwd(q, k, v)


def test_varlen_lengths_are_checked():
    q = bf(100, H, D)
    with pytest.raises(ValueError, match="int32"):
        FA.fwd(q, q, q, cu_seqlens_q=torch.tensor([0, 50, 100], dtype=torch.int64))
    with pytest.raises(ValueError, match=r"\[T, H, D\]"):
        FA.fwd(bf(1, 100, H, D), q, q, cu_seqlens_q=torch.tensor([0, 100], dtype=torch.int32))
    with pytest.raises(ValueError, match="as many entries"):
        FA.fwd(q, q, q, cu_seqlens_q=torch.tensor([0, 50, 100], dtype=torch.int32),
               cu_seqlens_k=torch.tensor([0, 100], dtype=torch.int32))
    with pytest.raises(ValueError, match="cu_seqlens_k without cu_seqlens_q"):
        FA.fwd(*qkv(), cu_seqlens_k=torch.tensor([0, 100], dtype=torch.int32))
    with pytest.raises(ValueError, match="cu_seqlens_q must be a GPU tensor|q must be a GPU tensor"):
        FA.fwd(q, q, q, cu_seqlens_q=torch.tensor([0, 100], dtype=torch.int32))


def grads_args():
    q, k, v = qkv()
    return dict(dout=bf(B, S, H, D), q=q, k=k, v=v, o=bf(B, S, H, D),
                lse=torch.zeros((B, H, S), dtype=torch.float32))


@pytest.mark.parametrize("field,value,msg", [
    ("o", torch.zeros((B, S, H, D), dtype=torch.float32), "o must be torch.bfloat16"),
    ("dout", bf(B, S, H, 64), "dout must have shape"),
    ("lse", torch.zeros((B, H, S), dtype=torch.float16), "lse must be torch.float32"),
    ("lse", torch.zeros((B, S, H), dtype=torch.float32), "lse must have shape"),
])
def test_backward_rejects_wrong_inputs(field, value, msg):
    kw = grads_args()
    kw[field] = value
    with pytest.raises(ValueError, match=msg):
        FA.bwd(**kw)


def test_backward_gradient_buffers_must_match_grad_dtype():
    # a bf16 buffer given for fp32 gradients would receive 4-byte writes at 2-byte strides
    kw = grads_args()
    with pytest.raises(ValueError, match="dq must be torch.float32"):
        FA.bwd(**kw, dq=torch.zeros((B, S, H, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dk must be torch.bfloat16"):
        FA.bwd(**kw, grad_dtype=torch.bfloat16, dk=torch.zeros((B, S, H, D), dtype=torch.float32))
    with pytest.raises(ValueError, match="dv must have shape"):
        FA.bwd(**kw, dv=torch.zeros((B, S, H, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="grad_dtype"):
        FA.bwd(**kw, grad_dtype=torch.float16)


def test_backward_rejects_host_tensors():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        FA.bwd(**grads_args())


def test_exp2_probe_rejects_host_and_wrong_dtype():
    with pytest.raises(ValueError):
        FA.exp2_probe(torch.zeros(8, dtype=torch.float32))
    with pytest.raises(ValueError):
        FA.exp2_probe(torch.zeros(8, dtype=torch.float64))
