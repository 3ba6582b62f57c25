"""The allocation-free decode call (mla_decode_attn_noalloc), through the C
ABI, against the allocating one (mla_decode_attn) on the same inputs, and
against the fp64 oracle: two calls in a row, the second with a smaller input
(the library's scratch array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

from test_gpu_parity import SCALE, _assert_close, _f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


CALLS = [
    # the larger call first: 8 sequences of up to 1500 rows, fp32 latent output
    (W.Workload("na_big", B=8, H=128, s_q=1, causal=False, T_range=(700, 1500), seed=91), torch.float32),
    # then a smaller one: fewer sequences, rows, heads; causal, bf16 output
    (W.Workload("na_small", B=3, H=64, s_q=2, causal=True, T=300, T_stride=320, seed=92), torch.bfloat16),
]


def test_noalloc_matches_decode_attn_twice(mla):
    for w, o_dtype in CALLS:
        print(f"[noalloc] {w} o_lat {o_dtype}", flush=True)
        inp = W.generate(w)
        q, w_uk, w_uv, cache = W.to_torch(inp)
        B, s_q, H = w.B, w.s_q, w.H
        q_lat = mla.absorb_q(q.view(B * s_q, H, -1), w_uk).view(B, s_q, H, -1)
        o_ref, lse_ref = mla.decode_attn(q_lat, cache, SCALE, w.causal, o_dtype=o_dtype)
        o_got = torch.full((B, s_q, H, 512), float("nan"), dtype=o_dtype, device=q.device)
        lse_got = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device=q.device)
        mla.decode_attn_noalloc(q_lat, cache, SCALE, w.causal, o_lat=o_got, lse=lse_got)
        torch.cuda.synchronize()
        # the same kernels on the same plan: the same bits as the allocating call
        np.testing.assert_array_equal(_f64(o_got), _f64(o_ref))
        np.testing.assert_array_equal(lse_got.cpu().numpy(), lse_ref.cpu().numpy())
        # and the oracle's bar on the GPU's own latent queries
        o_oracle, lse_oracle = O.latent_attention(inp, _f64(q_lat), SCALE)
        m = _assert_close(_f64(o_got), o_oracle, what=f"noalloc {w.name}", out_bf16=o_dtype == torch.bfloat16)
        np.testing.assert_allclose(lse_got.cpu().numpy(), lse_oracle, rtol=0, atol=2e-3)
        print(f"[noalloc] {w.name}: {m}", flush=True)


def test_noalloc_rejects_oversized_call(mla):
    """An argument set whose workspace exceeds the scratch array is refused
    before anything is enqueued (B = 64, H = 128, 4096 rows, fp32 output)."""
    cap = int(mla._lib.mla_decode_noalloc_max_bytes())
    assert mla.decode_workspace_bytes(64, 1, 128, 4096) > cap
    dev = torch.device("cuda")
    rows = torch.zeros((64, 4096, 576), dtype=torch.bfloat16, device=dev)
    cache = mla.LatentCache(rows=rows, seqlens=torch.full((64,), 4096, dtype=torch.int32, device=dev),
                            max_seqlen=4096)
    q_lat = torch.zeros((64, 1, 128, 576), dtype=torch.bfloat16, device=dev)
    o = torch.full((64, 1, 128, 512), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(mla.MLAError, match="WORKSPACE"):
        mla.decode_attn_noalloc(q_lat, cache, SCALE, False, o_lat=o)
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0))      # nothing ran
