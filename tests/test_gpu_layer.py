"""GPU test of one chunk-recurrent attention layer (paged_chunk_attention_amd.layer):
the layer's output and every gradient (input and the four projection weights), from the
chunk-by-chunk forward and the reverse, recomputing backward with in-place paged key/value
gradients (gist.science explainer of OOMB, 2.A-2.B), against the oracle's layer reference:
the same layer as one full-sequence float64 computation with autograd, which makes its own
page selections (top-k layers) from its own queries and keys.

Bars: y and dx at the bf16 (fp32) bars of the attention outputs. The weight gradients sum
over every token, reach tens in magnitude and are returned in the parameter dtype, whose
spacing there (0.125 for bf16 at 16..32) exceeds the absolute bar; they are compared
divided by their largest reference magnitude, at the same max-abs and relative-L2 bars.
"""
import pytest
import torch

import oracle as orc
from paged_chunk_attention_amd.layer import ChunkRecurrentAttention
from tests.gpu_harness import DEV, compare, log

pytestmark = pytest.mark.gpu


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
    y_ref, dx_ref, dw_ref, sels_ref = orc.layer_reference(
        x, layer.wq, layer.wk, layer.wv, layer.wo, hq, hkv, d, layer.page, layer.chunk,
        layer.scale, layer.theta, dy, top_k=layer.top_k, window=layer.window, sel_dtype=dtype)
    if layer.top_k is not None:
        got = [[sel[g, :int(count[g])].tolist() for g in range(hkv)] for sel, count in layer.sels]
        assert got == sels_ref, (got, sels_ref)
        log(f"    selections equal the oracle's: {sels_ref}")
    compare("y", y, y_ref, dtype)
    compare("dx", x.grad, dx_ref, dtype)
    for nm, w, ref in zip(("dWq", "dWk", "dWv", "dWo"), (layer.wq, layer.wk, layer.wv, layer.wo),
                          dw_ref):
        s_ = ref.abs().max().item()
        compare(nm + "/max", w.grad.detach().double().cpu() / s_, ref / s_, dtype)


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
