"""CPU tests: the oracle against its pins, and planted mistakes that the pins catch."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle_pins as P  # noqa: E402  (tests/ is on sys.path under pytest)
from oracle import qmm_oracle as O


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)


def _fresh_oracle_copy():
    path = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "qmm_oracle.py")
    spec = importlib.util.spec_from_file_location("qmm_oracle_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _msb_first_unpack(W, bits, K, block):
    W = np.asarray(W, dtype=np.uint8)
    k = np.arange(K)
    b, j = k // block, k % block
    byte_index = (j * bits) // 8
    shift = (8 - bits - (j * bits) % 8).astype(np.uint8)
    return (W[..., b, byte_index] >> shift) & np.uint8((1 << bits) - 1)


def _mutants():
    """Plausible mistakes, each planted in a fresh copy of the oracle."""
    muts = {}

    m = _fresh_oracle_copy()
    m.unpack_codes = _msb_first_unpack
    muts["msb_first_codes"] = m

    m = _fresh_oracle_copy()
    orig = m.zero_points_f64
    m.zero_points_f64 = lambda *a, **kw: -orig(*a, **kw)  # zp added instead of subtracted
    muts["zero_point_sign"] = m

    m = _fresh_oracle_copy()
    orig_dq = m.dequant_nbits

    def dq_wrong_block(W, bits, K, block, scales_f16, zp=None, zp_kind="none", uniform_zp=0.0):
        s = np.asarray(scales_f16)
        return orig_dq(W, bits, K, block, s[..., ::-1].copy(), zp, zp_kind, uniform_zp)
    m.dequant_nbits = dq_wrong_block  # scale of the wrong block
    muts["scale_block_index"] = m

    m = _fresh_oracle_copy()
    m.swiglu = lambda gu, I: gu[..., I:2 * I] * m.sigmoid(gu[..., I:2 * I]) * gu[..., :I]
    muts["swiglu_g_u_swapped"] = m

    m = _fresh_oracle_copy()
    m.matmul_f64 = lambda a, w, b=None: a @ w.T  # bias dropped
    muts["bias_dropped"] = m

    m = _fresh_oracle_copy()
    orig_q = m.quantize_int8_groups

    def q_floor(v64, group=32):
        v = np.asarray(v64, dtype=np.float64)
        q, s = orig_q(v, group)
        safe = np.repeat(np.where(s == 0, 1.0, s.astype(np.float64)), group, axis=-1).reshape(v.shape)
        return np.clip(np.floor(v / safe), -127, 127).astype(np.int8), s
    m.quantize_int8_groups = q_floor  # truncation instead of round-to-nearest
    muts["int8_floor"] = m

    m = _fresh_oracle_copy()
    orig_cb = m.dequant_codebook4

    def cb_off_by_one(W, K, block, absmax, codebook):
        cb = np.roll(np.asarray(codebook, dtype=np.float32), 1)
        return orig_cb(W, K, block, absmax, cb)
    m.dequant_codebook4 = cb_off_by_one  # codebook index off by one
    muts["codebook_index"] = m

    m = _fresh_oracle_copy()
    orig_fq = m.fake_quantize
    m.fake_quantize = lambda x, s, zp, bits: orig_fq(x, s, zp + 1, bits)  # wrong zp in fused Q->DQ
    muts["fake_quant_zp"] = m

    m = _fresh_oracle_copy()
    m.to_f16 = lambda x: np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16)
    muts["f16_double_rounding"] = m

    m = _fresh_oracle_copy()
    m.f32_to_bf16_bits = lambda x: (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    muts["bf16_truncation"] = m

    m = _fresh_oracle_copy()
    orig_ro = m._round_operand
    m._round_operand = lambda x, mode: orig_ro(x, "bf16" if mode in ("f16", "f16_rows") else mode)
    muts["bf16_for_f16_operands"] = m

    m = _fresh_oracle_copy()
    orig_ro2 = m._round_operand
    m._round_operand = lambda x, mode: orig_ro2(x, "f16" if mode == "f16_rows" else mode)
    muts["no_row_prescale"] = m

    m = _fresh_oracle_copy()
    orig_ro3 = m._round_operand
    m._round_operand = lambda x, mode: x if mode == "f16" else orig_ro3(x, mode)
    muts["weight_operand_not_rounded"] = m

    m = _fresh_oracle_copy()
    orig_l2 = m.rel_l2
    m.rel_l2 = lambda y, ref: orig_l2(y, ref) ** 2  # squared norm ratio
    muts["rel_l2_squared"] = m

    m = _fresh_oracle_copy()
    m.rel_l2 = lambda y, ref: float(np.max(np.abs(np.asarray(y) - np.asarray(ref))) /
                                    max(np.max(np.abs(np.asarray(ref))), 1e-300))
    muts["rel_l2_max_norm"] = m

    m = _fresh_oracle_copy()
    m.qsigmoid = lambda q, si, zi, so, zo, bits: m.quantize_linear(
        m.dequantize_linear(q, si, zi) * 0.25 + 0.5, so, zo, bits)   # linearised sigmoid
    muts["qsigmoid_linearised"] = m

    m = _fresh_oracle_copy()
    orig_sw = m.qswiglu

    def sw_no_requant(gate, up, qp, bits):   # the chain without the sigmoid's requantize
        (sg, zg), (st, zt), (sm, zm), (su, zu), (sh, zh) = qp
        g = m.quantize_linear(gate, sg, zg, bits)
        gd = m.dequantize_linear(g, sg, zg)
        mm = m.quantize_linear(m.to_f32(gd.astype(np.float64) * m.sigmoid_f32(gd)), sm, zm, bits)
        u = m.quantize_linear(up, su, zu, bits)
        return m.dequantize_linear(m.qmul(mm, sm, zm, u, su, zu, sh, zh, bits), sh, zh)
    m.qswiglu = sw_no_requant
    muts["qswiglu_sigmoid_not_requantized"] = m

    m = _fresh_oracle_copy()
    m.div_f32 = lambda x, s: m.to_f32(np.asarray(x, dtype=np.float32).astype(np.float64) *
                                      m.to_f32(1.0 / np.asarray(s, dtype=np.float32).astype(np.float64)))
    muts["quotient_by_reciprocal"] = m
    return muts


@pytest.mark.parametrize("name", sorted(_mutants().keys()))
def test_planted_mistake_is_caught(name):
    mutant = _mutants()[name]
    failures = 0
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failures += 1
        except Exception:  # a crash also counts as caught
            failures += 1
    assert failures >= 1, f"no pin catches the planted mistake {name}"
