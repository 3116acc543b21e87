"""Planted mistakes in the oracle (CPU only): every one must fail some pin.

Each mutant is a copy of ``oracle/gdn_oracle.c`` with one textual change (a dropped term,
a flipped sign, a wrong index or operand), compiled to a temporary library and swapped in
for the real one while the pins of test_oracle_pins.py run against it.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "decay_sign": ("const double a = exp(gi);", "const double a = exp(-gi);"),
    "decay_dropped": ("S[(int64_t)i * dv + j] *= a;", "(void)a;"),
    "delta_sign": ("e[j] = acc - vt[j];", "e[j] = acc + vt[j];"),
    "update_sign": ("-= bt * e[j] * kn[i];", "+= bt * e[j] * kn[i];"),
    "beta_dropped": ("-= bt * e[j] * kn[i];", "-= e[j] * kn[i];"),
    "output_uses_key": ("acc += S[(int64_t)i * dv + j] * qn[i];",
                        "acc += S[(int64_t)i * dv + j] * kn[i];"),
    "eps_dropped": ("1.0 / sqrt(ss + eps);", "1.0 / sqrt(ss);"),
    "scale_dropped": ("dst[i] = src[i] * inv * scale;", "dst[i] = src[i] * inv;"),
    "l2_q_skipped": ("l2_scale(qn, qt, dk, eps, scale);",
                     "memcpy(qn, qt, sizeof(double) * dk);"),
    "conv_taps_reversed": ("z += w[(int64_t)c * K + j] * xe[t + j];",
                           "z += w[(int64_t)c * K + (K - 1 - j)] * xe[t + j];"),
    "conv_state_shift": ("st_out[(int64_t)c * W + j] = xe[T + j];",
                         "st_out[(int64_t)c * W + j] = xe[T + j - 1];"),
    "silu_sign": ("y[t * C + c] = z / (1.0 + exp(-z));",
                  "y[t * C + c] = z / (1.0 + exp(z));"),
    "kda_channel_index": ("g[(t * H + hd) * dk + i]", "g[(t * H + hd) * dk]"),
    "norm_sum_not_mean": ("sqrt(ss / dv + eps)", "sqrt(ss + eps)"),
    "norm_eps_outside": ("sqrt(ss / dv + eps)", "(sqrt(ss / dv) + eps)"),
    "gate_silu_sign": ("(zj / (1.0 + exp(-zj)))", "(zj / (1.0 + exp(zj)))"),
    "gate_weight_index": ("* w[j] *", "* w[0] *"),
    "gate_before_norm": ("ss += orow[j] * orow[j];",
                         "ss += orow[j] * orow[j] * zrow[j] * zrow[j];"),
    "output_before_update": ("/* o = S q */", "/* o = S q */ for (int32_t i2 = 0; "
                             "i2 < dk; ++i2) for (int32_t j2 = 0; j2 < dv; ++j2) "
                             "S[(int64_t)i2 * dv + j2] += bt * e[j2] * kn[i2];"),
}


def _pin_calls():
    """Every pin, with representative parameters."""
    return [
        lambda: pins.test_hand_worked_recurrence("gdn_scalar_gate"),
        lambda: pins.test_hand_worked_recurrence("kda_channel_gate"),
        pins.test_hand_worked_conv,
        lambda: pins.test_dense_unrolling(False, 5, 4, 3),
        lambda: pins.test_dense_unrolling(True, 7, 3, 5),
        lambda: pins.test_chunk_size_invariance(True, 16),
        pins.test_beta_zero_is_pure_decay,
        pins.test_beta_zero_gate_zero_is_a_matmul,
        pins.test_full_forgetting,
        pins.test_orthonormal_keys_give_causal_linear_attention,
        pins.test_retrieval_identity_with_in_call_l2,
        pins.test_l2_properties,
        lambda: pins.test_conv_matches_torch_conv1d(37),
        lambda: pins.test_conv_matches_torch_conv1d(2),
        pins.test_gated_rmsnorm_hand_worked,
        pins.test_gated_rmsnorm_matches_torch,
        pins.test_gated_rmsnorm_invariants,
    ]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique: %s" % name
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(mpath), "-o",
                    str(so), "-lm"], check=True)
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fn in ("gdn_oracle_conv_silu", "gdn_oracle_recurrence", "gdn_oracle_gated_rmsnorm",
               "gdn_oracle_num_threads"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    oracle._lib = lib
    caught = []
    try:
        for i, call in enumerate(_pin_calls()):
            try:
                call()
            except AssertionError:
                caught.append(i)
    finally:
        oracle._lib = real
    assert caught, "planted mistake %r passed every pin" % name


def test_unmutated_oracle_passes_every_pin():
    for call in _pin_calls():
        call()
