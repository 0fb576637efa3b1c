"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes the oracle to something independent: a library conversion
routine, a brute-force pure-Python computation, a closed form, an invariant
of the definition, or a number printed on the pages.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import get_config, make_case
from synth.make import repermute

TINY_SHAPES = [
    # (q heads, kv heads, head_dim, q dtype, kv dtype, page size, lengths)
    (4, 2, 64, "f16", "f16", 16, (37, 100)),
    (2, 2, 64, "bf16", "bf16", 64, (1, 65)),
    (8, 2, 64, "bf16", "bf16", 16, (15, 16, 17)),
    (4, 1, 64, "f16", "i8", 16, (33, 5)),
    (2, 2, 128, "bf16", "i8", 64, (64, 130)),
    (4, 2, 64, "f16", "fp8", 16, (37, 20)),
    (2, 1, 128, "bf16", "fp8", 64, (1, 70)),
]


def tiny_case(Hq, Hkv, D, qd, kvd, PS, lens, seed=11, num_pages=None, **kw):
    maxlen = max(lens)
    pages = sum(-(-n // PS) for n in lens)
    cfg = get_config("tiny", batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv,
                     head_dim=D, q_dtype=qd, kv_dtype=kvd, page_size=PS,
                     num_pages=num_pages or max(2 * pages, 8), lens_kind="fixed",
                     lens_args=tuple(lens))
    assert cfg.max_context_len == maxlen
    return make_case(cfg, seed=seed, keep_logical=True, **kw)


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Library conversion of stored bits to float64 (numpy / torch)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    import torch

    if dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def logical_floats(case, b, which):
    enc, sc = (case.logical_k if which == "k" else case.logical_v)[b]
    if case.cfg.kv_dtype == "i8":
        return enc.astype(np.float64) * sc.astype(np.float64)[..., None]
    if case.cfg.kv_dtype == "fp8":
        return decode_bits(enc, "fp8") * sc.astype(np.float64)[..., None]
    return decode_bits(enc, case.cfg.kv_dtype)


# --------------------------------------------------------------------------
# Element decoding: every f16 / bf16 bit pattern against library routines.

def test_f16_decode_matches_numpy_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.oracle_f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bf16_decode_matches_torch_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = decode_bits(bits, "bf16")
    got = np.array([oracle_lib.oracle_bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


def test_fp8_e4m3_decode_matches_torch_all_patterns(oracle_lib):
    bits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ref = decode_bits(bits, "fp8")
    got = np.array([oracle_lib.oracle_fp8e4m3_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert nan.sum() == 2                      # S.1111.111, both signs
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


def test_fp8_e4m3_closed_forms(oracle_lib):
    """Values the OCP E4M3 definition fixes: 1.0, the largest finite value
    (1.75 * 2^8), the smallest subnormal (2^-9), the largest subnormal, the
    smallest normal (2^-6), negative zero; no infinities."""
    f = oracle_lib.oracle_fp8e4m3_to_f64
    assert f(0x38) == 1.0
    assert f(0x7E) == 448.0 and f(0xFE) == -448.0
    assert f(0x01) == 2.0 ** -9 and f(0x07) == 7 * 2.0 ** -9
    assert f(0x08) == 2.0 ** -6
    assert f(0x80) == 0.0 and math.copysign(1.0, f(0x80)) == -1.0
    assert math.isnan(f(0x7F)) and math.isnan(f(0xFF))
    assert all(math.isfinite(f(b)) for b in range(256) if b & 0x7F != 0x7F)


# --------------------------------------------------------------------------
# Brute force: contiguous pure-Python attention, no pages.

@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_oracle_matches_pure_python_brute_force(shape):
    case = tiny_case(*shape)
    cfg = case.cfg
    got = oracle.paged_decode(case)
    q = decode_bits(case.q_bits, cfg.q_dtype)
    keys = [logical_floats(case, b, "k").tolist() for b in range(cfg.batch)]
    vals = [logical_floats(case, b, "v").tolist() for b in range(cfg.batch)]
    ref = np.array(brute.decode_batch(q.tolist(), keys, vals, case.scale, cfg.group))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_oracle_matches_brute_force_with_poisoned_tails():
    """NaN in every unused slot and unused page never reaches the output."""
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), poison=True)
    got = oracle.paged_decode(case)
    assert np.isfinite(got).all()
    clean = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), poison=False)
    assert (oracle.paged_decode(clean) == got).all()


# --------------------------------------------------------------------------
# Invariants of the definition.

@pytest.mark.parametrize("shape", TINY_SHAPES[:3])
def test_physical_page_permutation_invariance_bitwise(shape):
    case = tiny_case(*shape)
    base = oracle.paged_decode(case)
    for s in (1, 2, 3):
        moved = repermute(case, seed=s)
        assert not (moved.block_tables == case.block_tables).all()
        assert (oracle.paged_decode(moved) == base).all()


def test_gqa_equals_mha_with_repeated_kv_heads_bitwise():
    case = tiny_case(8, 2, 64, "bf16", "bf16", 16, (37, 3), seed=5)
    G = case.cfg.group
    mha = make_case(case.cfg, seed=5, keep_logical=True)
    fields = {k: v for k, v in case.cfg.__dict__.items() if k != "name"}
    fields["num_kv_heads"] = 8
    mha.cfg = get_config("tiny", **fields)
    mha.k_pages = np.repeat(case.k_pages, G, axis=1)
    mha.v_pages = np.repeat(case.v_pages, G, axis=1)
    assert (oracle.paged_decode(mha) == oracle.paged_decode(case)).all()


def test_int8_with_unit_scales_equals_f16_of_same_integers():
    """Dequantisation is exact: int8 codes with scale 1 give the same fp64
    inputs as f16 storage of the same integers (all exact in f16)."""
    c8 = tiny_case(4, 2, 64, "f16", "i8", 16, (37, 100), seed=7)
    c8.k_scale[:] = 1.0
    c8.v_scale[:] = 1.0
    c16 = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=7)
    c16.k_pages = c8.k_pages.astype(np.float16).view(np.uint16)
    c16.v_pages = c8.v_pages.astype(np.float16).view(np.uint16)
    c16.q_bits = c8.q_bits
    assert (oracle.paged_decode(c8) == oracle.paged_decode(c16)).all()


def test_fp8_with_unit_scales_equals_f16_of_same_values():
    """Every finite E4M3 value is exact in f16: fp8 codes with scale 1 give
    the same fp64 inputs as f16 storage of the decoded values."""
    c8 = tiny_case(4, 2, 64, "f16", "fp8", 16, (37, 100), seed=8)
    c8.k_scale[:] = 1.0
    c8.v_scale[:] = 1.0
    c16 = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=8)
    c16.k_pages = decode_bits(c8.k_pages, "fp8").astype(np.float16).view(np.uint16)
    c16.v_pages = decode_bits(c8.v_pages, "fp8").astype(np.float16).view(np.uint16)
    c16.q_bits = c8.q_bits
    assert (oracle.paged_decode(c8) == oracle.paged_decode(c16)).all()


@pytest.mark.parametrize("T", [16, 32, 64, 96])
def test_split_merge_matches_unsplit(T):
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100, 1, 64), seed=3)
    full = oracle.paged_decode(case)
    out, m, l, o = oracle.paged_decode_split(case, T, with_stats=True)
    np.testing.assert_allclose(out, full, rtol=0, atol=1e-12)
    # per-partition stats against the brute-force definition on that range
    cfg = case.cfg
    q = decode_bits(case.q_bits, cfg.q_dtype)
    for b in range(cfg.batch):
        keys, vals = logical_floats(case, b, "k"), logical_floats(case, b, "v")
        n = int(case.context_lens[b])
        for h in range(cfg.num_q_heads):
            g = h // cfg.group
            for k in range(m.shape[2]):
                t0, t1 = k * T, min(n, (k + 1) * T)
                if t0 >= n:
                    assert m[b, h, k] == -np.inf and l[b, h, k] == 0
                    continue
                s = [case.scale * math.fsum(q[b, h] * keys[t, g]) for t in range(t0, t1)]
                mk = max(s)
                assert m[b, h, k] == pytest.approx(mk, abs=1e-12)
                w = [math.exp(x - mk) for x in s]
                assert l[b, h, k] == pytest.approx(math.fsum(w), rel=1e-12)
                ov = [math.fsum(w[i] * vals[t0 + i, g, d] for i in range(t1 - t0))
                      for d in range(cfg.head_dim)]
                np.testing.assert_allclose(o[b, h, k], ov, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms.

def test_single_token_returns_its_value_exactly():
    case = tiny_case(4, 2, 64, "bf16", "bf16", 16, (1, 1), seed=9)
    out = oracle.paged_decode(case)
    for b in range(2):
        v0 = logical_floats(case, b, "v")[0]
        for h in range(4):
            assert (out[b, h] == v0[h // 2]).all()


def test_zero_query_gives_mean_of_values():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=4)
    case.q_bits = np.zeros_like(case.q_bits)
    out = oracle.paged_decode(case)
    for b in range(2):
        v = logical_floats(case, b, "v")
        for h in range(4):
            ref = [math.fsum(v[:, h // 2, d]) / v.shape[0] for d in range(64)]
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-14)


def test_zero_scale_gives_mean_of_values():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=4)
    case.scale = 0.0
    out = oracle.paged_decode(case)
    for b in range(2):
        v = logical_floats(case, b, "v")
        ref = v.mean(axis=0)
        np.testing.assert_allclose(out[b, 0], ref[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[b, 3], ref[1], rtol=0, atol=1e-14)


def test_constant_values_give_that_constant():
    case = tiny_case(4, 2, 64, "bf16", "bf16", 16, (37, 100), seed=6)
    case.v_pages[:] = np.uint16(0x3FC0)          # 1.5 in bf16
    out = oracle.paged_decode(case)
    np.testing.assert_allclose(out, 1.5, rtol=1e-15, atol=0)


def test_identical_keys_give_mean_of_values():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=8)
    case.k_pages[:] = case.k_pages[0, 0, 0]
    out = oracle.paged_decode(case)
    for b in range(2):
        v = logical_floats(case, b, "v")
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    case = tiny_case(2, 1, 64, "f16", "f16", 16, (50,), seed=12)
    q = np.zeros((1, 2, 64), dtype=np.float16)
    q[0, :, 0] = 1.0
    case.q_bits = q.view(np.uint16)
    j = 23
    row, slot = 1, j % 16          # token 23 lives in the sequence's 2nd page
    k = case.k_pages.view(np.float16)
    k[:] = np.float16(0)
    k[row, 0, slot, 0] = np.float16(1000.0)  # score 1000/8 = 125 vs 0 elsewhere
    out = oracle.paged_decode(case)
    vj = logical_floats(case, 0, "v")[j, 0]
    np.testing.assert_allclose(out[0, 0], vj, rtol=0, atol=1e-40)


def test_large_common_score_shift_is_harmless():
    """Adding the same (huge) amount to every score leaves the softmax alone:
    exp would overflow without the max subtraction."""
    base = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=13)
    shifted = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=13)
    q = shifted.q_bits.view(np.float16)
    k = shifted.k_pages.view(np.float16)
    q[..., 63] = np.float16(100.0)
    k[..., 63] = np.float16(100.0)            # + 100*100/8 = 1250 on every score
    qb = base.q_bits.view(np.float16)
    kb = base.k_pages.view(np.float16)
    qb[..., 63] = 0
    kb[..., 63] = 0
    a, b = oracle.paged_decode(base), oracle.paged_decode(shifted)
    assert np.isfinite(b).all()
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-11)


def test_empty_sequence_gives_zeros():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (0, 5), seed=2)
    out = oracle.paged_decode(case)
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()


def test_block_table_entry_outside_pool_is_an_error():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (37, 100), seed=2)
    case.block_tables[1, 3] = case.cfg.num_pages
    with pytest.raises(oracle.OracleError):
        oracle.paged_decode(case)


def test_scatter_rows_matches_numpy_indexing():
    rng = np.random.default_rng(0)
    pool = rng.integers(0, 65535, size=(8, 2, 16, 64), dtype=np.uint16)
    ref = pool.copy()
    slots = np.array([5, 17, 127, 64], dtype=np.int64)
    src = rng.integers(0, 65535, size=(4, 2, 64), dtype=np.uint16)
    oracle.scatter_rows(pool, slots, src)
    ref[slots // 16, :, slots % 16, :] = src
    assert (pool == ref).all()
