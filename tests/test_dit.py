"""The synthetic Pixel-DiT-S step (LLSA inside the network it was made for).

CPU: the network's own Morton permutation equals the oracle's.  GPU: the network with the
reorder hoisted to its entry (LLSA in Morton layout) matches the same network with the
reorder folded into the op (raster layout), outputs and parameter gradients; the dense
baseline's attention module matches float32 softmax attention; a training step runs."""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import dit
from oracle import llsa_oracle as orc


@pytest.mark.parametrize("h,w", [(4, 4), (2, 4), (8, 2), (16, 64), (64, 64)])
def test_morton_permutation_matches_oracle(h, w):
    assert np.array_equal(dit.morton_permutation(h, w).numpy(), orc.morton_perm(h, w))


def _pair(h, w, depth, **kw):
    torch.manual_seed(0)
    a = dit.PixelDiT(h, w, depth=depth, hoist_reorder=True, **kw).cuda()
    b = dit.PixelDiT(h, w, depth=depth, hoist_reorder=False, **kw).cuda()
    b.load_state_dict(a.state_dict())
    return a, b


@pytest.mark.gpu
def test_hoisted_reorder_matches_folded_reorder():
    h = w = 64
    a, b = _pair(h, w, depth=2, levels=2)
    batch = dit.synthetic_batch(2, h, w, "cuda", seed=3)
    outs = []
    for m in (a, b):
        xt, noise, t, y = batch
        with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
            pred = m(xt, t, y)
        loss = torch.nn.functional.mse_loss(pred.float(), noise)
        loss.backward()
        outs.append((pred.float(), {n: p.grad.float() for n, p in m.named_parameters()}))
    (pa, ga), (pb, gb) = outs
    assert torch.allclose(pa, pb, rtol=1e-2, atol=1e-2), (pa - pb).abs().max()
    for n in ga:
        ref = gb[n]
        err = (ga[n] - ref).abs().max().item()
        assert err <= 2e-2 * max(1.0, ref.abs().max().item()), (n, err)


@pytest.mark.gpu
def test_dense_attention_module_matches_float32_softmax():
    torch.manual_seed(1)
    n, c = 4096, 384
    att = dit.Attention(c, 6, 64, 64, mode="dense").cuda()
    x = torch.randn(2, n, c, device="cuda")
    with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
        got = att(x).float()
    qkv = (x.to(torch.bfloat16).float() @ att.qkv.weight.to(torch.bfloat16).float().T
           + att.qkv.bias.to(torch.bfloat16).float())
    q, k, v = qkv.view(2, n, 3, 6, 64).permute(2, 0, 3, 1, 4)
    q, k, v = (t.to(torch.bfloat16).float() for t in (q, k, v))
    s = (q @ k.transpose(-1, -2)) / 8.0
    o = torch.softmax(s, dim=-1) @ v
    o = o.transpose(1, 2).reshape(2, n, c).to(torch.bfloat16).float()
    want = o @ att.proj.weight.to(torch.bfloat16).float().T + att.proj.bias.float()
    err = (got - want).abs().max().item()
    assert err <= 2e-2 * max(1.0, want.abs().max().item()), err


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["llsa", "dense"])
def test_training_step_runs(mode):
    h = w = 64
    torch.manual_seed(2)
    m = dit.PixelDiT(h, w, depth=2, levels=2, mode=mode).cuda()
    opt = torch.optim.AdamW(m.parameters(), lr=1e-4)
    before = [p.detach().clone() for p in m.parameters()]
    loss = dit.train_step(m, opt, dit.synthetic_batch(2, h, w, "cuda", seed=4))
    torch.cuda.synchronize()
    assert torch.isfinite(loss)
    moved = sum(int(not torch.equal(p0, p.detach())) for p0, p in zip(before, m.parameters()))
    assert moved == len(before)
