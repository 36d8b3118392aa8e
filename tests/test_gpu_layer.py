"""GPU test of one chunk-recurrent attention layer (paged_chunk_attention_amd.layer):
the layer's output and every gradient (input and the four projection weights), from the
chunk-by-chunk forward and the reverse, recomputing backward with in-place paged key/value
gradients (gist.science explainer of OOMB, 2.A-2.B), against the same layer written as one
full-sequence computation in float64 with PyTorch autograd on the CPU (the oracle's rotary
embedding, an explicit attention mask: causal; for top-k layers the pages each chunk
selected plus its own; for local layers the window).
"""
import math

import pytest
import torch

import oracle as orc
from paged_chunk_attention_amd.layer import ChunkRecurrentAttention
from tests.gpu_harness import DEV, TOL, compare, log

pytestmark = pytest.mark.gpu


def _reference(x, layer: ChunkRecurrentAttention, dy):
    """float64 CPU reference of the layer over the whole sequence; returns y and the
    gradients of sum(dy * y) with respect to x, Wq, Wk, Wv, Wo."""
    f64 = torch.float64
    xs = x.detach().cpu().to(f64).requires_grad_()
    ws = [w.detach().cpu().to(f64).requires_grad_() for w in (layer.wq, layer.wk, layer.wv, layer.wo)]
    wq, wk, wv, wo = ws
    T = xs.shape[0]
    hq, hkv, d, P, C = layer.hq, layer.hkv, layer.d, layer.page, layer.chunk
    G = hq // hkv
    q = orc.rope((xs @ wq).view(T, hq, d).transpose(0, 1), 0, layer.theta)
    k = orc.rope((xs @ wk).view(T, hkv, d).transpose(0, 1), 0, layer.theta)
    v = (xs @ wv).view(T, hkv, d).transpose(0, 1)
    pos = torch.arange(T)
    mask = torch.zeros(hq, T, T, dtype=torch.bool)
    for h in range(hq):
        g = h // G
        allowed = pos[None, :] <= pos[:, None]
        if layer.window:
            allowed &= pos[None, :] > pos[:, None] - layer.window
        if layer.top_k is not None:
            page_ok = torch.zeros(T, T, dtype=torch.bool)
            for ci, (sel, count) in enumerate(layer.sels):
                t0 = ci * C
                chosen = set(sel[g, :int(count[g])].tolist())
                rows = slice(t0, t0 + C)
                for t in range(T):
                    if t // P in chosen or t // P >= t0 // P:
                        page_ok[rows, t] = True
            allowed &= page_ok
        mask[h] = allowed
    kk = k.repeat_interleave(G, dim=0)
    vv = v.repeat_interleave(G, dim=0)
    s = (q @ kk.transpose(1, 2)) * layer.scale
    s = s.masked_fill(~mask, -math.inf)
    o = torch.softmax(s, dim=-1) @ vv
    y = o.transpose(0, 1).reshape(T, hq * d) @ wo
    (y * dy.cpu().to(f64)).sum().backward()
    return y.detach(), xs.grad, [w.grad for w in ws]


@pytest.mark.parametrize("kw", [
    dict(name="layer_dense_bf16", T=512, chunk=128, page=32),
    dict(name="layer_topk_bf16", T=1024, chunk=256, page=32, top_k=3),
    dict(name="layer_window_bf16", T=512, chunk=128, page=32, window=100),
    dict(name="layer_dense_f32_d64", T=384, chunk=128, page=16, d=64, dtype=torch.float32),
])
def test_chunk_recurrent_layer_matches_full_sequence(kw):
    kw = dict(kw)
    name, T = kw.pop("name"), kw.pop("T")
    d, dtype = kw.pop("d", 128), kw.pop("dtype", torch.bfloat16)
    hidden, hq, hkv = 256, 4, 2
    log(f"[case {name}] T={T} hidden={hidden} hq={hq} hkv={hkv} d={d} {kw} {dtype}")
    layer = ChunkRecurrentAttention(hidden, hq, hkv, d, max_tokens=T, dtype=dtype, device=DEV,
                                    seed=3, **kw)
    g = torch.Generator().manual_seed(11)
    x = torch.randn(T, hidden, generator=g).to(device=DEV, dtype=dtype).requires_grad_()
    dy = torch.randn(T, hidden, generator=g).to(device=DEV, dtype=dtype)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    log("    gpu done")
    y_ref, dx_ref, dw_ref = _reference(x, layer, dy)
    compare("y", y, y_ref, dtype)
    compare("dx", x.grad, dx_ref, dtype)
    for nm, w, ref in zip(("dWq", "dWk", "dWv", "dWo"), (layer.wq, layer.wk, layer.wv, layer.wo),
                          dw_ref):
        # weight gradients sum over every token: compare relative to their size
        atol = TOL[dtype][0] * max(1.0, ref.abs().max().item())
        got = w.grad.detach().cpu().double()
        err = (got - ref).abs().max().item()
        rel = (got - ref).norm().item() / ref.norm().item()
        log(f"    {nm:6s} max_abs={err:.3e} (scaled bar {atol:.3e}) rel_l2={rel:.3e}")
        assert rel <= TOL[dtype][1] and err <= atol, nm


@pytest.mark.parametrize("dtype,pos0", [(torch.bfloat16, 0), (torch.bfloat16, 4_190_000),
                                        (torch.float32, 1_048_576)])
def test_rope_kernel_matches_oracle(dtype, pos0):
    """The rotary-embedding kernel against the oracle's float64 rotation, forward and
    inverse, on a strided view, out of place and in place, at positions up to 4M
    (where the kernel's fp64 angles matter)."""
    import paged_chunk_attention_amd as pca
    log(f"[case rope {dtype} pos0={pos0}]")
    g = torch.Generator().manual_seed(7)
    base = torch.randn(300, 6, 128, generator=g).to(dtype)   # [tokens, heads, D]
    x = base.to(DEV).transpose(0, 1)                           # [heads, tokens, D] view
    y = pca.oomb_rope(x, pos0, theta=1.0e6)
    ref = orc.rope(base.transpose(0, 1), pos0, theta=1.0e6)
    compare("rope", y, ref, dtype)
    back = pca.oomb_rope(y, pos0, theta=1.0e6, inverse=True)
    compare("inverse", back, orc.rope(y.cpu(), pos0, theta=1.0e6, inverse=True), dtype)
    z = x.contiguous()
    pca.oomb_rope(z, pos0, theta=1.0e6, out=z)                 # in place
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), y.cpu())
