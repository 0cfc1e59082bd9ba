"""Pins for the oracle's FP8 KV cache (OCP FP8 E4M3 storage with per-tensor scales).

* ``fp8e4m3_bits_to_f64`` against PyTorch's ``float8_e4m3fn`` widening for all
  256 codes, and hand-checked codes from the format's definition;
* attention over an FP8 pool with scales equals attention over a float32 pool
  holding the dequantized values (widened and scaled by PyTorch): both are
  the same float64 inputs, so the results agree bit for bit;
* the same against PyTorch's float64 SDPA on the dequantized dense cache;
* the generator's FP8 pool is N(0,1) rounded to E4M3 by PyTorch.

``test_planted_fp8_mistakes_are_caught`` plants the FNUZ exponent bias (8), a
dropped subnormal branch and swapped K/V scales, and checks that a pin fails.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.paged_kv as oa
import pkv_inputs as gen
from tests.oracle_bridge import oracle_attention
from tests.test_oracle import dense_reference_torch


def check_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN codes differ"
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]), "finite codes differ from torch"


def check_hand_codes():
    v = oracle.fp8e4m3_bits_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0x80, 0x00, 0xB8, 0x3C, 0x07], dtype=np.uint8))
    want = [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -0.0, 0.0, -1.0, 1.5, 7 * 2.0 ** -9]
    assert list(v) == want
    assert np.signbit(v[4]) and not np.signbit(v[5])
    assert np.isnan(oracle.fp8e4m3_bits_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def _fp8_case(seed, layout="interleaved"):
    g = torch.Generator().manual_seed(seed)
    batch, hq, hk, d, bs, sk = 3, 8, 2, 16, 8, 40
    nb = gen.pool_num_blocks(sk, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, "fp8", layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    seqlens = [max(x, 5) for x in gen.uniform_int(1, sk, batch, generator=g)]
    cu = gen.cu_from_lengths([1, 5, 2])
    q = gen.randn((int(cu[-1]), hq, d), "bf16", generator=g)
    return q, pool, bt, seqlens, cu


def _dequantized(pool, k_scale, v_scale):
    """A float32 pool with K = stored * k_scale, V = stored * v_scale, computed by torch."""
    k = pool.k.to(torch.float32) * k_scale
    v = pool.v.to(torch.float32) * v_scale
    out = gen.PagedKV(k.contiguous(), v.contiguous(), "contiguous", [])
    out.storage = [out.k, out.v]
    return out


def check_equals_dequantized_pool():
    for seed, layout in ((201, "interleaved"), (202, "contiguous")):
        q, pool, bt, seqlens, cu = _fp8_case(seed, layout)
        for ks, vs in ((1.0, 1.0), (0.5, 1.25), (3.0, 0.0625)):
            a = oracle_attention(q, pool, bt, seqlens, cu, True, 0.3, ks, vs)
            deq = _dequantized(pool, ks, vs)
            b = oracle_attention(q.to(torch.float32), deq, bt, seqlens, cu, True, 0.3)
            for x, y in zip(a, b):
                assert np.array_equal(x, y), f"fp8 pool != dequantized pool (scales {ks}, {vs})"


def check_equals_torch_sdpa():
    q, pool, bt, seqlens, cu = _fp8_case(203)
    for causal in (False, True):
        a = oracle_attention(q, pool, bt, seqlens, cu, causal, 0.25, 0.5, 1.25)
        r = dense_reference_torch(q, _dequantized(pool, 0.5, 1.25), bt, seqlens, cu, causal, 0.25)
        for x, y in zip(a, r):
            assert np.max(np.abs(x - y)) <= 1e-12


PINS = [check_all_codes_match_torch, check_hand_codes, check_equals_dequantized_pool, check_equals_torch_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_fp8_oracle_pin(pin):
    pin()


def test_fp8_generator_rounds_with_torch():
    g1 = torch.Generator().manual_seed(5)
    g2 = torch.Generator().manual_seed(5)
    pool = gen.new_pool(4, 8, 2, 16, "fp8", "contiguous", generator=g1)
    ref = torch.randn((2, 4, 8, 2, 16), generator=g2).to(torch.float8_e4m3fn)
    assert torch.equal(pool.k.view(torch.uint8), ref[0].view(torch.uint8))
    assert torch.equal(pool.v.view(torch.uint8), ref[1].view(torch.uint8))


def _fnuz_bias(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    return np.where(e == 0, sign * m * 2.0 ** -10, sign * (1 + m / 8) * np.exp2(e - 8.0))


def _no_subnormals(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    out = sign * (1 + m / 8) * np.exp2(e - 7.0)
    return np.where((e == 15) & (m == 7), np.nan, out)


def _swapped_scales(k_flat, v_flat, layout, row, n):
    args = (row, n, layout.block_size, layout.num_heads_k, layout.head_dim)
    K = oa.gather_sequence(k_flat, layout.stored_dtype, layout.k_offset, layout.k_strides, *args)
    V = oa.gather_sequence(v_flat, layout.stored_dtype, layout.v_offset, layout.v_strides, *args)
    return K * layout.v_scale, V * layout.k_scale


MISTAKES = {
    "fnuz_bias": ("fp8e4m3_bits_to_f64", _fnuz_bias),
    "no_subnormals": ("fp8e4m3_bits_to_f64", _no_subnormals),
    "swapped_scales": ("gather_kv", _swapped_scales),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_fp8_mistakes_are_caught(name, monkeypatch):
    attr, fn = MISTAKES[name]
    monkeypatch.setattr(oa, attr, fn)
    if attr == "fp8e4m3_bits_to_f64":
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
