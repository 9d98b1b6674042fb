"""Host-side checks of the Python binding (no GPU): every tensor argument is checked against q
and k (shape, dtype, device, layout) before any pointer reaches the C interface, which cannot
see tensor sizes.  Each call below fails one check with ValueError; CPU tensors suffice because
shape and dtype are checked before the device."""

import pytest
import torch

import mask_aware_flashattention_amd as fm

B, H, NQ, NK, D = 1, 2, 40, 48, 128
BF = torch.bfloat16


def t(*shape, dtype=BF):
    return torch.zeros(*shape, dtype=dtype)


def vecs(n=NK):
    return [torch.zeros(n, dtype=torch.int32) for _ in range(4)]


def base():
    return dict(q=t(B, H, NQ, D), k=t(B, H, NK, D), v=t(B, H, NK, D))


@pytest.mark.parametrize("bad,msg", [
    (dict(v=t(B, H, NK - 1, D)), "v must have shape"),          # short v
    (dict(v=t(B, H, NK, D, dtype=torch.float32)), "v must be"),  # v dtype
    (dict(k=t(B, H, NK, D, dtype=torch.float32)), "k must be"),  # k dtype
    (dict(k=t(B, H + 1, NK, D)), "disagree"),
])
def test_fwd_rejects_mismatched_inputs(bad, msg):
    a = base()
    a.update(bad)
    with pytest.raises(ValueError, match=msg):
        fm.fwd(a["q"], a["k"], a["v"], *vecs())


@pytest.mark.parametrize("kw,msg", [
    (dict(out=t(B, H, NQ - 1, D)), "out must have shape"),
    (dict(out=t(B, H, NQ, D, dtype=torch.float32)), "out must be"),
    (dict(lse=t(B, H, NQ, dtype=torch.float32)[..., :-1]), "lse must have shape"),
    (dict(lse=t(B, H, NQ, dtype=BF)), "lse must be"),
])
def test_fwd_rejects_bad_outputs(kw, msg):
    a = base()
    with pytest.raises(ValueError, match=msg):
        fm.fwd(a["q"], a["k"], a["v"], *vecs(), **kw)


def test_fwd_valid_cpu_tensors_stop_at_the_device_check():
    a = base()
    with pytest.raises(ValueError, match="device"):
        fm.fwd(a["q"], a["k"], a["v"], *vecs(), out=t(B, H, NQ, D),
               lse=t(B, H, NQ, dtype=torch.float32))


def bwd_args():
    a = base()
    a.update(o=t(B, H, NQ, D), do=t(B, H, NQ, D), lse=t(B, H, NQ, dtype=torch.float32))
    return a


@pytest.mark.parametrize("bad,msg", [
    (dict(o=t(B, H, NQ, D - 8)), "o must have shape"),
    (dict(do=t(B, H, NQ - 3, D)), "do must have shape"),
    (dict(do=t(B, H, NQ, D, dtype=torch.float32)), "do must be"),
    (dict(lse=t(B, H, NQ + 1, dtype=torch.float32)), "lse must have shape"),
    (dict(lse=t(B, H, NQ, dtype=BF)), "lse must be"),
    (dict(v=t(B, H, NK + 5, D)), "v must have shape"),
])
def test_bwd_rejects_mismatched_inputs(bad, msg):
    a = bwd_args()
    a.update(bad)
    with pytest.raises(ValueError, match=msg):
        fm.bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], *vecs())


@pytest.mark.parametrize("which,shape,dtype,msg", [
    (0, (B, H, NQ, D - 8), BF, "dq must have shape"),
    (1, (B, H, NK, D), torch.float32, "dk must be"),
    (2, (B, H, NK - 1, D), BF, "dv must have shape"),
])
def test_bwd_rejects_bad_grads(which, shape, dtype, msg):
    a = bwd_args()
    grads = [t(B, H, NQ, D), t(B, H, NK, D), t(B, H, NK, D)]
    grads[which] = t(*shape, dtype=dtype)
    with pytest.raises(ValueError, match=msg):
        fm.bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], *vecs(), grads=tuple(grads))


def test_ex_rejects_expanded_and_interleaved_views():
    q = t(1, H, NQ, D).expand(3, H, NQ, D)          # batch stride 0
    k = t(3, H, NK, D)
    with pytest.raises(ValueError, match="overlap"):
        fm.fwd_ex(q, k, k.clone(), *vecs())
    q = t(3, H, NQ, D)
    k = t(3, 1, NK, D).expand(3, H, NK, D)          # head stride 0 with two key/value heads
    with pytest.raises(ValueError, match="overlap"):
        fm.fwd_ex(q, k, k, *vecs())
    with pytest.raises(ValueError, match="overlap"):
        fm.bwd_ex(q, k, k, q, q, t(3, H, NQ, dtype=torch.float32), *vecs())
    # a packed [B, n, 3, H, d] projection is a valid (non-overlapping) strided view: it passes
    # the layout checks and stops at the device check
    qkv = t(2, NQ, 3, H, D)
    qv, kv, vv = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    with pytest.raises(ValueError, match="device"):
        fm.fwd_ex(qv, kv, vv, *vecs(NQ))


def test_ex_valid_cpu_tensors_stop_at_the_device_check():
    a = base()
    with pytest.raises(ValueError, match="device"):   # valid everything, CPU tensors
        fm.fwd_ex(a["q"], a["k"], a["v"], *vecs())
