"""Each forward kernel of the bf16 path against a plain PyTorch fp32 reference
of the same op, fed with the kernel's own (bf16) inputs read back from the
workspace; this localises a fault to one kernel.  Shapes span several tiles
and a ragged tail (T = 200 is not a multiple of the 64/128 tiles); 17 x 1,000
tokens is a launch large enough for the persistent GEMM grid (several tiles
per workgroup) with a partial last tile row, and partial last tile columns
in the lm_head product."""

import numpy as np
import pytest

from gpt2_inputs import init_params
from tests.gpu_helpers import batches_for, gpu_step, say, shape, to_dev

pytestmark = pytest.mark.gpu


def _max_rel(got, want):
    d = (got - want).abs().max().item()
    return d / max(want.abs().max().item(), 1e-30)


@pytest.mark.parametrize("C,NH,T,B", [(768, 12, 200, 2), (1600, 25, 128, 1), (768, 12, 1000, 17)])
def test_bf16_forward_stages_against_torch_fp32(C, NH, T, B):
    import torch
    import torch.nn.functional as F
    s = shape("stage", 2, NH, C, 1024, 50257, 50304)
    say(f"stages C={C} NH={NH} T={T} B={B}")
    p = init_params(s, 1)
    rng = np.random.default_rng(2)
    for n in p:  # non-trivial biases and LN parameters
        if n.endswith("_b") or n.startswith("ln"):
            p[n] = (p[n] + 0.1 * rng.standard_normal(p[n].shape)).astype(np.float32)
    (x, y), = batches_for(s, B, T, 1, kind="zipf", seed=4)
    st = gpu_step(s, "bf16", B, p)
    xd, yd = to_dev([(x, y)])
    st.forward_loss(xd[0], yd[0], 1.0)
    torch.cuda.synchronize()
    M = B * T
    W = {n: torch.tensor(a, device="cuda") for n, a in p.items()}
    Wb = {n: a.to(torch.bfloat16).float() for n, a in W.items()}  # the bf16 copy the kernels read

    def act(name, l, cols):
        return st.activation(name, l).float().reshape(M, cols)

    x0 = st.activation("resid", 0).reshape(M, C)
    want = W["wte"][torch.tensor(x.ravel(), device="cuda").long()] + W["wpe"][:T].repeat(B, 1)
    assert torch.equal(x0, want), "embedding"
    for l in range(2):
        xin = st.activation("resid", 2 * l).reshape(M, C)
        ln1 = act("ln1", l, C)
        ref = F.layer_norm(xin, (C,), W["ln1_w"][l], W["ln1_b"][l], eps=1e-5)
        assert _max_rel(ln1, ref) < 1e-2, ("ln1", l, _max_rel(ln1, ref))
        qkv = act("qkv", l, 3 * C)
        ref = ln1 @ Wb["qkv_w"][l].T + W["qkv_b"][l]
        assert _max_rel(qkv, ref) < 1e-2, ("qkv gemm", l, _max_rel(qkv, ref))
        q, k, v = qkv.split(C, dim=1)
        hd = C // NH
        q, k, v = (t.reshape(B, T, NH, hd).transpose(1, 2).contiguous() for t in (q, k, v))
        sc = (q @ k.transpose(-1, -2).contiguous()) / hd ** 0.5
        mask = torch.triu(torch.ones(T, T, dtype=torch.bool, device="cuda"), 1)
        sc = sc.masked_fill(mask, float("-inf"))
        lse_ref = torch.logsumexp(sc, -1)
        ref = (torch.softmax(sc, -1) @ v).transpose(1, 2).reshape(M, C)
        atty = act("atty", l, C)
        assert _max_rel(atty, ref) < 2e-2, ("attention", l, _max_rel(atty, ref))
        lse = st.activation("lse", l).reshape(B, NH, T)
        assert (lse - lse_ref).abs().max().item() < 1e-2, ("lse", l)
        xmid = st.activation("resid", 2 * l + 1).reshape(M, C)
        ref = xin + atty @ Wb["proj_w"][l].T + W["proj_b"][l]
        assert _max_rel(xmid, ref) < 1e-3, ("proj gemm + residual", l, _max_rel(xmid, ref))
        ln2 = act("ln2", l, C)
        ref = F.layer_norm(xmid, (C,), W["ln2_w"][l], W["ln2_b"][l], eps=1e-5)
        assert _max_rel(ln2, ref) < 1e-2, ("ln2", l)
        # the fc GEMM keeps gelu(u) and gelu'(u) of u = LN2 Wfc^T + bfc
        u = (ln2 @ Wb["fc_w"][l].T + W["fc_b"][l]).requires_grad_(True)
        gref = F.gelu(u, approximate="tanh")
        (dref,) = torch.autograd.grad(gref.sum(), u)
        g = act("fcg", l, 4 * C)
        assert _max_rel(g, gref.detach()) < 1e-2, ("fc gemm + gelu", l, _max_rel(g, gref.detach()))
        d = act("fcgd", l, 4 * C)
        assert _max_rel(d, dref) < 1e-2, ("fc gemm + gelu'", l, _max_rel(d, dref))
        xout = st.activation("resid", 2 * l + 2).reshape(M, C)
        ref = xmid + g @ Wb["fcproj_w"][l].T + W["fcproj_b"][l]
        assert _max_rel(xout, ref) < 1e-3, ("fcproj gemm + residual", l, _max_rel(xout, ref))
    lnf = st.activation("lnf").float().reshape(M, C)
    ref = F.layer_norm(st.activation("resid", 4).reshape(M, C), (C,), W["lnf_w"], W["lnf_b"], eps=1e-5)
    assert _max_rel(lnf, ref) < 1e-2, "lnf"
    # after the forward the logits buffer holds (softmax - onehot) / M
    z = lnf @ Wb["wte"].T
    yt = torch.tensor(y.ravel(), device="cuda").long()
    rows = st.activation("row_loss")
    ref_rows = torch.logsumexp(z, -1) - z.gather(1, yt[:, None])[:, 0]
    assert (rows - ref_rows).abs().max().item() < 5e-2, ("cross-entropy rows", (rows - ref_rows).abs().max().item())
    dz = st.activation("logits").float().reshape(M, -1)
    ref = torch.softmax(z, -1)
    ref[torch.arange(M, device="cuda"), yt] -= 1
    ref /= M
    assert _max_rel(dz, ref) < 2e-2, ("dlogits", _max_rel(dz, ref))
    st.close()
