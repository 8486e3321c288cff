"""moe_forward_noalloc (the forward on the library's own scratch array)
through the C ABI against moe_forward with a caller workspace: bit-equal
outputs, indices, weights and offsets (the same kernels), on calls in a row
of different sizes, the second smaller than the first; and a batch whose
workspace exceeds the scratch array rejected with WORKSPACE, nothing run."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_top_amd import inputs as I
from mixture_experts_ffn_top_amd import moe
from oracle import moe_oracle as O
from parity_helpers import assert_close, dev, host

pytestmark = pytest.mark.gpu


def _case(seed, T, k, E, H, I_):
    g = np.random.default_rng(seed)
    x = O.round_to(g.standard_normal((T, H)), "bf16")
    z = I.gapped_logits(seed, T, E, k)
    z[min(3, T - 1), 0] = np.nan  # a NaN row: NaN weights and output row
    w = [O.round_to(g.standard_normal(s) / np.sqrt(s[-1]), "bf16") for s in ((E, I_, H), (E, I_, H), (E, H, I_))]
    return x, z, w


def _run(fn, x, z, k, w, **kw):
    T, E = z.shape
    outs = dict(out=torch.full((T, x.shape[1]), 7.0, dtype=torch.bfloat16, device="cuda"),
                indices_out=torch.full((T, k), -5, dtype=torch.int32, device="cuda"),
                weights_out=torch.full((T, k), 3.0, dtype=torch.float32, device="cuda"),
                offsets_out=torch.full((E + 1,), -9, dtype=torch.int32, device="cuda"))
    fn(dev(x, "bf16"), dev(z, "f32"), k, True, *[dev(a, "bf16") for a in w], **outs, **kw)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in outs.items()}


# (T, top_k, E, H, I): a 256-row-tile batch, then a smaller decode-sized one
# (the weight-streaming path), then one in between (128-row tiles)
SHAPES = [(300, 2, 8, 512, 768), (16, 8, 64, 256, 128), (96, 8, 64, 264, 392)]


def test_forward_noalloc_matches_forward_on_successive_calls():
    for i, (T, k, E, H, I_) in enumerate(SHAPES):
        print("noalloc case", i, (T, k, E, H, I_), flush=True)
        assert moe.moe_forward_workspace_size(T, H, I_, E, k, torch.bfloat16, torch.float32) \
            <= moe.NOALLOC_SCRATCH_BYTES
        x, z, w = _case(80 + i, T, k, E, H, I_)
        ref = _run(moe.moe_forward, x, z, k, w)
        got = _run(moe.moe_forward_noalloc, x, z, k, w)
        for n in ref:
            assert torch.equal(ref[n].view(torch.uint8) if ref[n].dtype != torch.int32 else ref[n],
                               got[n].view(torch.uint8) if got[n].dtype != torch.int32 else got[n]), (i, n)
        # and the values themselves against the oracle
        _, _, _, _, out_r = O.forward(x, z, "f32", k, True, lambda e: (w[0][e], w[1][e], w[2][e]), E, "bf16")
        assert_close(host(got["out"]), out_r, "bf16", f"noalloc forward case {i}")


def test_forward_noalloc_rejects_a_batch_beyond_its_scratch():
    T, k, E, H, I_ = 4096, 2, 8, 4096, 14336  # needs about 300 MB of workspace
    assert moe.moe_forward_workspace_size(T, H, I_, E, k, torch.bfloat16, torch.float32) \
        > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    wg = torch.zeros((E, I_, H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, H), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="MOE_ERROR_WORKSPACE"):
        moe.moe_forward_noalloc(x, z, k, True, wg, wg, wg.view(E, H, I_), out=out)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())  # nothing ran
