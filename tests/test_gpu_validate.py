"""mla_validate_kv on device-resident lengths and block tables (it copies
them to the host and checks them there; no kernel reads the bad values):
a valid ragged paged cache and a valid contiguous cache pass, and each kind
of broken precondition -- a length above max_seqlen, a length below s_q, a
block id outside the pool, a negative block id in use -- is refused."""
import dataclasses

import pytest
import torch

from head_latent_attention_mla_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


def _cache(kind):
    if kind == "paged":
        w = W.Workload("val_paged", B=3, H=8, s_q=1, causal=False, T_range=(70, 300), paged=True, seed=91)
    else:
        w = W.Workload("val_contig", B=3, H=8, s_q=2, causal=True, T=200, T_stride=256, seed=92)
    return W.to_torch(W.generate(w))[3]


@pytest.mark.parametrize("kind", ["paged", "contiguous"])
def test_valid_cache_passes(mla, kind):
    cache = _cache(kind)
    cache.validate(1)
    torch.cuda.synchronize()


def test_length_above_max_seqlen_is_refused(mla):
    cache = _cache("contiguous")
    bad = dataclasses.replace(cache, seqlens=cache.seqlens.clone())
    bad.seqlens[1] = cache.max_seqlen + 1
    with pytest.raises(mla.MLAError, match="ARG"):
        bad.validate(1)


def test_length_below_s_q_is_refused(mla):
    cache = _cache("contiguous")
    bad = dataclasses.replace(cache, seqlens=cache.seqlens.clone())
    bad.seqlens[0] = 1
    with pytest.raises(mla.MLAError, match="ARG"):
        bad.validate(2)
    bad.validate(1)


def test_block_outside_the_pool_is_refused(mla):
    cache = _cache("paged")
    n_pool = int(cache.rows.shape[0])
    bad = dataclasses.replace(cache, block_table=cache.block_table.clone())
    bad.block_table[2, 0] = n_pool
    with pytest.raises(mla.MLAError, match="ARG"):
        bad.validate(1)
    bad.block_table[2, 0] = -3
    with pytest.raises(mla.MLAError, match="ARG"):
        bad.validate(1)
    # entries past a sequence's last block are never read
    good = dataclasses.replace(cache, block_table=cache.block_table.clone())
    T2 = int(cache.seqlens[2])
    used = (T2 + 63) // 64
    if used < good.block_table.shape[1]:
        good.block_table[2, used:] = -7
        good.validate(1)
