"""The analytic cost model reproduces every number the pages print (CPU)."""
import json
import os

import pytest

from oracle import costmodel as cm

HERE = os.path.dirname(__file__)
PINS = {p["name"]: p for p in json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))["pins"]}


def _computed():
    c = {}
    by, fl, ai = cm.gqa_decode_cached_token(8, 1, 128, 8192, 2)
    c["gqa_llama70b_bytes_per_kv_head"], c["gqa_llama70b_flops_per_kv_head"], c["gqa_llama70b_intensity"] = by, fl, ai
    c["gqa_fp8_intensity"] = cm.gqa_decode_cached_token(8, 1, 128, 8192, 1)[2]
    by, fl, ai = cm.mla_absorbed_cached_token(128, 512, 64, 2)
    c["dsv3_bytes_per_cached_token"], c["dsv3_flops_per_cached_token"], c["dsv3_intensity_bf16"] = by, fl, ai
    c["dsv3_intensity_fp8"] = cm.mla_absorbed_cached_token(128, 512, 64, 1)[2]
    c["dsv3_vs_gqa_ratio"] = ai / cm.gqa_decode_cached_token(8, 1, 128, 8192, 2)[2]
    c["dsv3_tp8_intensity"] = cm.mla_tp_intensity(128, 512, 64, 2, 8)
    c["dsv3_verify_s4_intensity"] = cm.mla_absorbed_cached_token(128, 512, 64, 2, s_q=4)[2]
    c["gqa_verify_s4_intensity"] = 4 * cm.gqa_decode_cached_token(8, 1, 128, 8192, 2)[2]
    c["naive_decompress_flops_per_cached_token"] = cm.naive_expand_flops_per_cached_token(128, 512, 128, 128)
    c["naive_over_absorbed"] = c["naive_decompress_flops_per_cached_token"] / fl
    c["dsv3_decompressed_kv_mb_per_token_61_layers"] = 61 * 128 * (128 + 64 + 128) * 2
    c["h100_ridge"] = cm.ridge(989.5e12, 3.35e12)
    c["h200_ridge"] = cm.ridge(989.5e12, 4.8e12)
    c["b200_ridge"] = cm.ridge(2.25e15, 8e12)
    fixed = cm.mla_fixed_flops(7168, 128, 512, 128, 128)
    per_l = cm.mla_per_length_flops(128, 512)
    c["dsv3_fixed_flops"], c["dsv3_per_length_flops"] = fixed, per_l
    c["dsv3_fixed_share_8k"] = fixed / (per_l * 8192)
    c["dsv3_fixed_share_32k"] = fixed / (per_l * 32768)
    c["mla_ai_2h_dsv3_norope"] = cm.mla_absorbed_cached_token(128, 512, 0, 2)[2]
    c["mla_ai_2h_k3_norope"] = cm.mla_absorbed_cached_token(96, 512, 0, 2)[2]
    gib = 2 ** 30
    c["k3_cache_mha_gb"] = cm.cache_bytes(256 * 96, 32768, 93) / gib
    c["k3_cache_gqa8_gb"] = cm.cache_bytes(256 * 8, 32768, 93) / gib
    c["k3_cache_mqa_gb"] = cm.cache_bytes(256, 32768, 93) / gib
    c["k3_cache_mla_gb"] = cm.cache_bytes(512, 32768, 93) / gib
    proj = 512 * (128 + 128)
    ab, ex = cm.per_pair_macs(512, 128, 128)
    c["one_to_one_expand_total"], c["one_to_one_absorb_total"] = proj + ex, proj + ab
    for L in (2048, 8192, 32768):
        (fm, bm), (fh, bh) = cm.decode_algorithms(96, 512, 128, 128, L)
        c[f"k3_decode_mla_{L}"] = [fm, bm, fm / bm]
        c[f"k3_decode_mha_{L}"] = [fh, bh, fh / bh]
    (fm, _), (fh, _) = cm.decode_algorithms(96, 512, 128, 128, 32768, S=1)
    c["decode_flop_ratio_s1_L32768"] = fm / fh
    c["crossover_S_L512"] = cm.crossover_S(512, 128, 128, 512)
    c["crossover_S_L128k"] = cm.crossover_S(512, 128, 128, 131072)
    c["crossover_S_limit"] = 512 * 256 / (2 * 512 - 256)
    c["per_pair_absorb_norope"], c["per_pair_expand_norope"] = cm.per_pair_macs(512, 128, 128)
    c["per_pair_absorb_rope"], c["per_pair_expand_rope"] = cm.per_pair_macs(512, 128, 128, 64)
    c["per_pair_ratio_rope"] = c["per_pair_absorb_rope"] / c["per_pair_expand_rope"]
    sp = cm.sparse_mla_flops(128, 512, 128, 128, 2048)
    c["sparse_mla_flops_k2048"] = sp
    dense = [cm.decode_algorithms(128, 512, 128, 128, L)[1][0] for L in (2048, 8192, 32768, 131072)]
    c["dense_mha_alg_h128"] = dense
    c["sparse_gap"] = [d / sp for d in dense]
    c["mha_kv_dims_per_token"] = 128 * (128 + 128)
    kv = 80 * 32 * 8192 * 2 * (8 // 4) * 128 * 2
    c["llama70b_tp4_kv_per_gpu"] = kv
    c["llama70b_tp4_hbm_ms"] = kv / 3.35e12 * 1e3
    return c


COMPUTED = _computed()


@pytest.mark.parametrize("name", sorted(PINS))
def test_page_number(name):
    pin = PINS[name]
    assert name in COMPUTED, f"no computation for pin {name}"
    got, want = COMPUTED[name], pin["value"]
    got = got if isinstance(got, list) else [got]
    want = want if isinstance(want, list) else [want]
    assert len(got) == len(want)
    for g, w in zip(got, want):
        # printed values are rounded: accept the printed precision (rtol) plus half a unit
        assert g == pytest.approx(w, rel=max(pin["rtol"], 1e-12), abs=0.5 if pin["rtol"] == 0 and w > 100 else 1e-9), (name, g, w, pin["cite"])


def test_every_computation_has_a_pin():
    assert set(COMPUTED) == set(PINS)
