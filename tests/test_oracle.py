"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: pure-Python scalar loops on tiny inputs;
* library reduction: torch CPU float64 scaled_dot_product_attention;
* associativity: the naive (expand) and absorbed forms agree;
* closed forms and invariants: one row, zero query, equal rows, a dominant
  row, a two-row sigmoid, causal masking, permutation, paging, independence;
* negative control: a score-blind (uniform-weight) output fails the parity
  tolerance on the unit-activation inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W

SCALE = 1.0 / math.sqrt(192.0)


def tiny(B=2, H=4, T=7, s_q=1, causal=False, paged=False, fp8=False, seed=0, scaling="unit", T_stride=None):
    w = W.Workload("t", B=B, H=H, s_q=s_q, causal=causal, T=None if paged else T,
                   T_range=(T, T + 70) if paged else None, paged=paged,
                   cache_dtype="fp8" if fp8 else "bf16", scaling=scaling, seed=seed,
                   T_stride=T_stride)
    return W.generate(w)


# ----------------------------------------------------------------------------
# brute force: scalar loops, written straight from the definition
# ----------------------------------------------------------------------------
def _brute(inp, scale, causal):
    q = O.bf16_to_f64(inp["q"]).tolist()
    wuk = O.bf16_to_f64(inp["w_uk"]).tolist()
    wuv = O.bf16_to_f64(inp["w_uv"]).tolist()
    B, s_q, H = len(q), len(q[0]), len(q[0][0])
    out = [[[None] * H for _ in range(s_q)] for _ in range(B)]
    for b in range(B):
        C = O.sequence_rows(inp, b).tolist()
        T = len(C)
        for j in range(s_q):
            n = T - s_q + j + 1 if causal else T
            for h in range(H):
                scores = []
                for t in range(n):
                    acc = 0.0
                    for k in range(128):                 # content: q_nope . (W_UK[h] c_t)
                        kk = 0.0
                        for c in range(512):
                            kk += wuk[h][k][c] * C[t][c]
                        acc += q[b][j][h][k] * kk
                    for r in range(64):                  # rope: q_rope . k_rope
                        acc += q[b][j][h][128 + r] * C[t][512 + r]
                    scores.append(acc * scale)
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                z = sum(e)
                o = [0.0] * 128
                for t in range(n):
                    for v in range(128):
                        vv = 0.0
                        for c in range(512):
                            vv += C[t][c] * wuv[h][c][v]
                        o[v] += e[t] / z * vv
                out[b][j][h] = o
    return np.array(out)


@pytest.mark.parametrize("causal,s_q,T", [(False, 1, 3), (True, 2, 3)])
def test_naive_matches_scalar_brute_force(causal, s_q, T):
    inp = tiny(B=1, H=2, T=T, s_q=s_q, causal=causal, seed=11)
    ref = _brute(inp, SCALE, causal)
    got = O.naive_decode(inp, SCALE)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# associativity: absorbed == naive
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 7, 64])
@pytest.mark.parametrize("causal,s_q", [(False, 1), (True, 1), (True, 3), (False, 3)])
def test_absorbed_equals_naive(T, causal, s_q):
    if s_q > T:
        pytest.skip("s_q > T has no visible rows under the causal reading")
    inp = tiny(B=2, H=4, T=T, s_q=s_q, causal=causal, seed=T * 10 + s_q)
    a = O.absorbed_decode(inp, SCALE)
    n = O.naive_decode(inp, SCALE)
    assert np.max(np.abs(a - n)) <= 1e-12 * max(1.0, np.max(np.abs(n)))


# ----------------------------------------------------------------------------
# library reduction: latent attention == torch fp64 SDPA with one KV head
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal,s_q,T", [(False, 1, 37), (True, 4, 37), (True, 2, 5)])
def test_latent_attention_vs_torch_sdpa(causal, s_q, T):
    inp = tiny(B=2, H=8, T=T, s_q=s_q, causal=causal, seed=5)
    rng = np.random.default_rng(3)
    B, H = 2, 8
    q_lat = rng.standard_normal((B, s_q, H, 576))
    o, lse = O.latent_attention(inp, q_lat, SCALE)
    for b in range(B):
        C = torch.from_numpy(O.sequence_rows(inp, b))
        Tb = C.shape[0]
        q = torch.from_numpy(q_lat[b]).reshape(s_q * H, 576)[None, None]        # [1,1,sH,576]
        k = C[None, None]                                                          # [1,1,T,576]
        v = C[None, None, :, :512].contiguous()
        mask = torch.ones(s_q * H, Tb, dtype=torch.bool)
        if causal:
            for j in range(s_q):
                mask[j * H:(j + 1) * H, Tb - s_q + j + 1:] = False
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=SCALE)
        ref = ref[0, 0].reshape(s_q, H, 512).numpy()
        np.testing.assert_allclose(o[b], ref, rtol=1e-10, atol=1e-12)
        s = (q[0, 0] @ k[0, 0].T) * SCALE
        s = s.masked_fill(~mask, float("-inf"))
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).reshape(s_q, H).numpy(), rtol=1e-12)


def test_naive_vs_torch_einsum_expand_then_sdpa():
    """The up-project-then-attend form written with torch einsum + SDPA."""
    inp = tiny(B=2, H=4, T=29, s_q=2, causal=True, seed=8)
    q = torch.from_numpy(O.bf16_to_f64(inp["q"]))                      # [B,s,H,192]
    wuk = torch.from_numpy(O.bf16_to_f64(inp["w_uk"]))                 # [H,128,512]
    wuv = torch.from_numpy(O.bf16_to_f64(inp["w_uv"]))                 # [H,512,128]
    got = O.naive_decode(inp, SCALE)
    for b in range(2):
        C = torch.from_numpy(O.sequence_rows(inp, b))
        T = C.shape[0]
        K = torch.cat([torch.einsum("tc,hkc->htk", C[:, :512], wuk),
                       C[None, :, 512:].expand(4, T, 64)], dim=-1)       # [H,T,192]
        V = torch.einsum("tc,hcv->htv", C[:, :512], wuv)                 # [H,T,128]
        qq = q[b].permute(1, 0, 2)                                        # [H,s,192]
        mask = torch.ones(2, T, dtype=torch.bool)
        mask[0, T - 1:] = False
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, attn_mask=mask, scale=SCALE)
        np.testing.assert_allclose(got[b], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_absorb_steps_vs_einsum():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 3, 192))
    wuk = rng.standard_normal((3, 128, 512))
    ql = O.absorb_q(q, wuk)
    ref = np.einsum("nhk,hkc->nhc", q[..., :128], wuk)
    np.testing.assert_allclose(ql[..., :512], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(ql[..., 512:], q[..., 128:])
    ol = rng.standard_normal((5, 3, 512))
    wuv = rng.standard_normal((3, 512, 128))
    np.testing.assert_allclose(O.absorb_out(ol, wuv), np.einsum("nhc,hcv->nhv", ol, wuv), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def _values(inp, b, h):
    C = O.sequence_rows(inp, b)
    return C[:, :512] @ O.bf16_to_f64(inp["w_uv"])[h]


def test_single_row_returns_its_value():
    inp = tiny(B=2, H=4, T=1, seed=21)
    out = O.naive_decode(inp, SCALE)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, 0, h], _values(inp, b, h)[0], rtol=1e-13, atol=1e-14)


def test_zero_query_gives_uniform_average():
    inp = tiny(B=2, H=3, T=17, s_q=2, causal=True, seed=22)
    inp["q"][:] = 0
    out = O.naive_decode(inp, SCALE)
    for b in range(2):
        for h in range(3):
            V = _values(inp, b, h)
            np.testing.assert_allclose(out[b, 0, h], V[:16].mean(0), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(out[b, 1, h], V[:17].mean(0), rtol=1e-12, atol=1e-13)


def test_equal_rows_give_that_row():
    inp = tiny(B=1, H=3, T=9, seed=23)
    inp["rows"][0, 1:9] = inp["rows"][0, 0]
    out = O.naive_decode(inp, SCALE)
    for h in range(3):
        np.testing.assert_allclose(out[0, 0, h], _values(inp, 0, h)[0], rtol=1e-12, atol=1e-13)


def test_two_rows_rope_only_sigmoid():
    """q_nope = 0: the score is the rope term alone; two rows -> logistic weight."""
    inp = tiny(B=1, H=2, T=2, seed=24)
    inp["q"][..., :128] = 0
    q = O.bf16_to_f64(inp["q"])[0, 0]
    C = O.sequence_rows(inp, 0)
    out = O.naive_decode(inp, SCALE)
    for h in range(2):
        s0 = SCALE * sum(q[h, 128 + r] * C[0, 512 + r] for r in range(64))
        s1 = SCALE * sum(q[h, 128 + r] * C[1, 512 + r] for r in range(64))
        p1 = 1.0 / (1.0 + math.exp(s0 - s1))
        V = _values(inp, 0, h)
        np.testing.assert_allclose(out[0, 0, h], (1 - p1) * V[0] + p1 * V[1], rtol=1e-12, atol=1e-13)


def test_dominant_row_wins():
    """A row whose rope key aligns with a large rope query takes all the weight."""
    inp = tiny(B=1, H=2, T=12, seed=25)
    inp["q"][...] = 0
    inp["q"][0, 0, :, 128] = W.to_bf16_bits(np.array([64.0], np.float32))[0]
    inp["rows"][0, :, 512:] = 0
    inp["rows"][0, 5, 512] = W.to_bf16_bits(np.array([64.0], np.float32))[0]   # s_5 = 4096/sqrt(192) ~ 296
    out = O.naive_decode(inp, SCALE)
    for h in range(2):
        np.testing.assert_allclose(out[0, 0, h], _values(inp, 0, h)[5], rtol=1e-12, atol=1e-13)


def test_causal_all_new_rows():
    """T = s_q: query j sees rows 0..j only, so query 0 returns row 0's value."""
    inp = tiny(B=1, H=2, T=3, s_q=3, causal=True, seed=26)
    out = O.naive_decode(inp, SCALE)
    for h in range(2):
        np.testing.assert_allclose(out[0, 0, h], _values(inp, 0, h)[0], rtol=1e-13, atol=1e-14)
    full = O.naive_decode(inp, SCALE, causal=False)
    assert not np.allclose(full[0, 0], out[0, 0])
    np.testing.assert_allclose(full[0, 2], out[0, 2], rtol=1e-13)  # the last query sees every row


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_masked_rows_do_not_matter():
    inp = tiny(B=2, H=3, T=20, s_q=3, causal=True, seed=27, T_stride=32)
    a = O.naive_decode(inp, SCALE)
    assert np.all(np.isfinite(a))                       # NaN pad rows beyond T never read
    inp["rows"][:, 18:20] = W.to_bf16_bits(np.full((2, 2, 576), 7.0, np.float32))  # rows only the last queries see
    b = O.naive_decode(inp, SCALE)
    np.testing.assert_array_equal(a[:, 0], b[:, 0])
    assert not np.allclose(a[:, 2], b[:, 2])


def test_row_permutation_noncausal():
    inp = tiny(B=1, H=3, T=33, seed=28)
    a = O.naive_decode(inp, SCALE)
    perm = np.random.default_rng(0).permutation(33)
    inp["rows"][0, :33] = inp["rows"][0, perm]
    np.testing.assert_allclose(O.naive_decode(inp, SCALE), a, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fp8", [False, True])
def test_paged_equals_contiguous(fp8):
    inp = tiny(B=3, H=2, T=70, paged=True, fp8=fp8, seed=29)
    assert np.any(inp["block_table"] < 0)       # tail entries are don't-care (-1)
    a = O.naive_decode(inp, SCALE)
    c = W.as_contiguous(inp)
    np.testing.assert_array_equal(O.naive_decode(c, SCALE), a)


def test_sequences_are_independent():
    inp = tiny(B=3, H=2, T=40, seed=30)
    a = O.naive_decode(inp, SCALE)
    inp["rows"][1] = inp["rows"][2]
    b = O.naive_decode(inp, SCALE)
    np.testing.assert_array_equal(a[[0, 2]], b[[0, 2]])


def test_fp8_rows_are_code_times_scale():
    inp = tiny(B=1, H=2, T=5, fp8=True, seed=31)
    C = O.sequence_rows(inp, 0)
    for t in range(5):
        for i in (0, 100, 511, 512, 575):
            code = int(inp["rows"][0, t, i])
            s, e, m = code >> 7, (code >> 3) & 15, code & 7
            v = (m / 8) * 2 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            assert C[t, i] == (-v if s else v) * float(inp["row_scale"][0, t])


# ----------------------------------------------------------------------------
# negative control
# ----------------------------------------------------------------------------
def test_uniform_weights_fail_tolerance_on_unit_inputs():
    """A kernel that ignored the scores would return the uniform average; on
    unit-activation inputs that is far outside the parity tolerance."""
    inp = tiny(B=2, H=8, T=256, seed=32)
    ref = O.naive_decode(inp, SCALE)
    inp0 = dict(inp)
    inp0["q"] = np.zeros_like(inp["q"])
    blind = O.naive_decode(inp0, SCALE)
    m = oracle.compare(blind, ref)
    assert m["rel_l2"] > 0.3 and m["max_abs"] > 2e-2
