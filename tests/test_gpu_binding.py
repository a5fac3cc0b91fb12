"""The Python binding rejects tensors whose shapes disagree with the sizes it
passes to the C-ABI (the kernels trust those sizes), before any launch."""

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def t():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp
    mmsp.lib()
    sq, sk, hq, hkv, d = 96, 64, 4, 2, 64
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    x = dict(q=torch.zeros(sq, hq, d, **bf), k=torch.zeros(sk, hkv, d, **bf),
             v=torch.zeros(sk, hkv, d, **bf), dout=torch.zeros(sq, hq, d, **bf),
             o=torch.zeros(sq, hq, d, **f32), lse=torch.zeros(hq, sq, **f32),
             delta=torch.zeros(hq, sq, **f32), dq=torch.zeros(sq, hq, d, **f32),
             qp=torch.arange(sq, **i32), kp=torch.arange(sk, **i32))
    return mmsp, torch, x


def _bad(torch, like, **kw):
    shape = list(like.shape)
    shape[0] += 1
    return torch.zeros(shape, dtype=like.dtype, device=like.device)


def test_forward_rejects_mismatched_shapes(t):
    mmsp, torch, x = t
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(x["q"], x["k"], _bad(torch, x["v"]), x["qp"], x["kp"])
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(x["q"], x["k"], x["v"], x["qp"], x["kp"], o=_bad(torch, x["o"]))
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(x["q"], x["k"], x["v"], x["qp"], x["kp"], lse=_bad(torch, x["lse"]))
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(x["q"], x["k"], x["v"], x["qp"][:-1], x["kp"])


def test_merge_and_preprocess_reject_mismatched_shapes(t):
    mmsp, torch, x = t
    with pytest.raises(ValueError):
        mmsp.lse_merge(x["o"], x["lse"], _bad(torch, x["o"]), x["lse"])
    with pytest.raises(ValueError):
        mmsp.lse_merge(x["o"], _bad(torch, x["lse"]))
    with pytest.raises(ValueError):
        mmsp.lse_merge(x["o"], x["lse"], x["o"], None)
    with pytest.raises(ValueError):
        mmsp.attn_bwd_preprocess(x["q"], _bad(torch, x["dout"]))
    with pytest.raises(ValueError):
        mmsp.attn_bwd_preprocess(x["q"], x["dout"], _bad(torch, x["delta"]))


@pytest.mark.parametrize("which", ["v", "dout", "lse", "delta", "dq", "dk", "dv", "kp"])
def test_backward_rejects_mismatched_shapes(t, which):
    mmsp, torch, x = t
    args = dict(q=x["q"], k=x["k"], v=x["v"], dout=x["dout"], lse=x["lse"], delta=x["delta"],
                q_pos=x["qp"], k_pos=x["kp"], dq_acc=x["dq"])
    key = {"dq": "dq_acc", "kp": "k_pos"}.get(which, which)
    if which in ("dk", "dv"):
        args[which] = torch.zeros(x["k"].shape[0] + 1, x["k"].shape[1], x["k"].shape[2],
                                  dtype=torch.float32, device="cuda")
    elif which == "kp":
        args[key] = x["kp"][:-1]
    else:
        args[key] = _bad(torch, args[key])
    with pytest.raises(ValueError):
        mmsp.attn_bwd_chunk(**args)


def test_rope_rejects_mismatched_output(t):
    mmsp, torch, x = t
    with pytest.raises(ValueError):
        mmsp.rope(x["q"], x["qp"], out=_bad(torch, x["q"]))
    with pytest.raises(ValueError):
        mmsp.rope(x["q"], x["qp"][:-1])
