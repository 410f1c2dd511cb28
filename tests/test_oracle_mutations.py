"""Mutation check of the oracle's pins (CPU only).

The FP4 backward page validates its tests by planting an error in the code
under test and counting the tests that fail.  Here each plausible mistake is
planted in the oracle (never in the GPU path) and at least one pin must
fail; a mutation that no pin catches means the pins are vacuous for it.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

import oracle_pins  # noqa: E402
from oracle import formats as F  # noqa: E402
from oracle import gemm as O  # noqa: E402
from oracle import pertensor as PT  # noqa: E402


def _swap_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0x0F
    return out


def _truncating_bf16(f, nan_sign=None):
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


_orig_round = F.round_to_grid


def _ties_up(t, elem):
    # nudge every value up by a hair so that ties round away from zero
    return _orig_round(np.asarray(t) * (1 + 2.0 ** -40), elem)


_orig_nv = F.dequant_nvfp4


def _nv_without_tensor_scale(codes, scales, tensor_scale):
    return _orig_nv(codes, scales, np.float32(1.0))


_orig_expand = F.expand_scales


def _expand_block64(scales, rows, cols, br, bc):
    if br == 128:
        s = _orig_expand(scales, rows, cols, 64, 64)
        pad = [(0, 0)] * (s.ndim - 2) + [(0, rows - s.shape[-2]), (0, cols - s.shape[-1])]
        return np.pad(s, pad, mode="edge")
    return _orig_expand(scales, rows, cols, br, bc)


def _expand_rows_off_by_one_block(scales, rows, cols, br, bc):
    if (br, bc) == (F.MX_BLOCK, 1):
        return _orig_expand(np.roll(scales, 1, axis=-2), rows, cols, br, bc)
    return _orig_expand(scales, rows, cols, br, bc)


def _dw_wrong_operand(grad_bits, x_bits):
    return O._f64(grad_bits).T @ O._f64(x_bits)[::-1]


_orig_bounds = O.group_bounds


def _bounds_shifted(offsets):
    b = _orig_bounds(offsets)
    return [(s, e) for (s, e) in b[1:]] + [b[0]]


def _no_f32_step(x):
    return np.asarray(x, dtype=np.float64)


_orig_pt_quant = PT.quantize


def _pt_quant_multiplies(bits, elem, scale):
    return _orig_pt_quant(bits, elem, np.float32(1.0) / np.float32(scale))


_orig_pt_round = PT.round_to_fp8


def _pt_no_saturation(t, elem):
    t = np.asarray(t, dtype=np.float64)
    return np.where(np.abs(t) > PT.FP8_MAX[elem], np.uint8(0x7F) | (np.signbit(t) * 0x80).astype(np.uint8),
                    _orig_pt_round(t, elem)).astype(np.uint8)


_orig_pt_scale = PT.scale_from_history


def _pt_scale_no_margin(hist, elem, margin=0):
    return _orig_pt_scale(hist, elem, 0)


def _pt_scale_latest(hist, elem, margin=0):
    return _orig_pt_scale(np.asarray(hist)[-1:], elem, margin)


_orig_pt_dx = PT.linear_dx


def _pt_dx_one_scale(g_codes, g_elem, g_scale, w_codes, w_elem, w_scale):
    return _orig_pt_dx(g_codes, g_elem, g_scale, w_codes, w_elem, 1.0)


def _fwd_no_transpose(x_bits, w_bits):
    return O._f64(x_bits) @ O._f64(w_bits).reshape(O._f64(w_bits).shape[::-1])


_orig_rows_dx = O.rows_dx
_orig_rows_dw = O.rows_dw


def _rows_dx_next_row(grad_bits, w_bits, rows):
    r = np.minimum(np.asarray(rows) + 1, np.asarray(grad_bits).shape[0] - 1)
    return _orig_rows_dx(grad_bits, w_bits, r)


def _rows_dw_next_n(grad_bits, x_bits, n_rows):
    n = np.minimum(np.asarray(n_rows) + 1, np.asarray(grad_bits).shape[1] - 1)
    return _orig_rows_dw(grad_bits, x_bits, n)


def _scale_rows_lag(r0, r1, srow):
    return slice(max(r0 - 1, 0) // srow, -(-r1 // srow))


def _chunks_drop_last_block(n, size):
    size = max(1, size)
    return [(i, min(n, i + size) - (1 if min(n, i + size) - i > 1 else 0)) for i in range(0, n, size)]


_orig_nv_fwd = O.nvfp4_fwd
_orig_fp8_fwd = O.fp8_block_fwd
_orig_grouped_fwd = O.grouped_fwd


def _nv_fwd_without_w_tensor_scale(x_codes, x_scales, x_ts, w_codes, w_scales, w_ts, offsets=None):
    return _orig_nv_fwd(x_codes, x_scales, x_ts, w_codes, w_scales, 1.0, offsets)


def _fp8_fwd_unit_scales(x_bits, w_codes, w_scale_inv, offsets=None):
    return _orig_fp8_fwd(x_bits, w_codes, np.ones_like(w_scale_inv), offsets)


def _grouped_fwd_next_weight(x_bits, w_bits, offsets):
    return _orig_grouped_fwd(x_bits, np.roll(np.asarray(w_bits), -1, axis=0), offsets)


MUTATIONS = {
    "sampled dX takes the next row": (O, "rows_dx", _rows_dx_next_row),
    "sampled dW takes the next n": (O, "rows_dw", _rows_dw_next_n),
    "dequant row slab lags one scale row": (F, "_scale_rows", _scale_rows_lag),
    "MX quant chunks skip their last block": (F, "_block_chunks", _chunks_drop_last_block),
    "forward multiplies W untransposed": (O, "linear_fwd", _fwd_no_transpose),
    "NVFP4 forward drops the weight tensor scale": (O, "nvfp4_fwd", _nv_fwd_without_w_tensor_scale),
    "block-FP8 forward ignores the block scales": (O, "fp8_block_fwd", _fp8_fwd_unit_scales),
    "grouped forward takes the next group's weight": (O, "grouped_fwd", _grouped_fwd_next_weight),
    "per-tensor quantization multiplies by the scale": (PT, "quantize", _pt_quant_multiplies),
    "per-tensor quantization without saturation": (PT, "round_to_fp8", _pt_no_saturation),
    "scale ignores the margin": (PT, "scale_from_history", _pt_scale_no_margin),
    "delayed scale from the latest amax only": (PT, "scale_from_history", _pt_scale_latest),
    "E5M2 bias 16": (PT, "TABLES", {"e4m3": F.E4M3_TABLE, "e5m2": PT.E5M2_TABLE / 2}),
    "per-tensor dX drops the weight scale": (PT, "linear_dx", _pt_dx_one_scale),
    "nibble order swapped": (F, "unpack_e2m1", _swap_nibbles),
    "bf16 truncation instead of RNE": (F, "f32_to_bf16_bits", _truncating_bf16),
    "ties away from zero": (F, "round_to_grid", _ties_up),
    "NVFP4 tensor scale dropped": (F, "dequant_nvfp4", _nv_without_tensor_scale),
    "FP8 block 64 instead of 128": (F, "expand_scales", _expand_block64),
    "MX axis -2 scale rows off by one block": (F, "expand_scales", _expand_rows_off_by_one_block),
    "E4M3 MX emax 7": (F, "ELEM_EMAX", {"e4m3": 7, "e2m1": 2}),
    "E2M1 MX emax 3": (F, "ELEM_EMAX", {"e4m3": 8, "e2m1": 3}),
    "E4M3 bias 8": (F, "E4M3_TABLE", F.E4M3_TABLE / 2),
    "E2M1 subnormal 0.25": (F, "E2M1_TABLE", np.where(np.abs(F.E2M1_TABLE) == 0.5, F.E2M1_TABLE / 2, F.E2M1_TABLE)),
    "E8M0 bias 128": (F, "E8M0_TABLE", F.E8M0_TABLE / 2),
    "dW operand rows reversed": (O, "linear_dw", _dw_wrong_operand),
    "group bounds shifted": (O, "group_bounds", _bounds_shifted),
}


def _failing_pins():
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    module, attr, value = MUTATIONS[name]
    monkeypatch.setattr(module, attr, value)
    failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []
