"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is a one-line slip one could make when writing the oracle -- a dropped
term, a flipped comparison, a swapped index or operand.  The test builds a temporary copy of
the oracle with that slip, points the oracle package at it, and runs the pin tests: at
least one pin must fail for every mutant.  The mistakes are planted in a private copy on
the CPU; the committed oracle is never modified.
"""
import json
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pi_oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "pi_oracle.h")

MUTANTS = {
    "predictor hidden ReLU dropped": ("z[j] = acc > 0.0 ? acc : 0.0;", "z[j] = acc;"),
    "offset c dropped": ("l[i] = acc + g_half[c[i]];", "l[i] = acc;"),
    "threshold not strict": ("uint8_t m = l[i] > 0.0;", "uint8_t m = l[i] >= 0.0;"),
    "batch union lost": ("mask[i] = (uint8_t)(mask[i] | m);", "mask[i] = m;"),
    "placement ignored": ("if (slot_of == NULL || slot_of[i] >= 0) idx[n++]", "if (1) idx[n++]"),
    "Q4_0 nibbles swapped": ("(t & 1) ? (byte >> 4) : (byte & 0x0F)", "(t & 1) ? (byte & 0x0F) : (byte >> 4)"),
    "Q4_0 zero point dropped": ("(double)(code - 8)", "(double)(code)"),
    "up bias dropped": ("if (b_up) u += g_half[b_up[slot[k]]];", ";"),
    "gate and up swapped": ("hv = (g > 0.0 ? g : 0.0) * u;", "hv = (u > 0.0 ? u : 0.0) * g;"),
    "up row read from gate row": ("pio_dot_row(row + rb, wtype, d, xb);", "pio_dot_row(row, wtype, d, xb);"),
    "down bias dropped": ("y[b * d + j] = b_down ? g_half[b_down[j]] : 0.0;", "y[b * d + j] = 0.0;"),
    "down row by neuron id, not slot": ("const uint8_t *row = wdn + slot[k] * rb;",
                                       "const uint8_t *row = wdn + (int64_t)idx[k] * rb;"),
    "binary16 exponent off by one": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "P1 transposed": ("g_half[p1[j * d + k]]", "g_half[p1[k * r + j]]"),
    "P2 transposed": ("g_half[p2[i * r + j]]", "g_half[p2[j * f + i]]"),
    "output ReLU dropped": ("hv = u > 0.0 ? u : 0.0;", "hv = u;"),
    "squared ReLU not squared": ("if (gated == PIO_SQUARED_RELU) hv = hv * hv;", ";"),
    "squared ReLU squares before the ReLU": ("hv = u > 0.0 ? u : 0.0;\n                if (gated == PIO_SQUARED_RELU) hv = hv * hv;",
                                             "hv = u > 0.0 ? u : 0.0;\n                if (gated == PIO_SQUARED_RELU) hv = u * u;"),
}


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "tiny_layers.json")) as fh:
        return json.load(fh)


def _pin_suite(golden):
    return [
        lambda: pins.test_half_exhaustive_matches_ieee_binary16(),
        lambda: pins.test_q4_0_decode_golden(golden),
        lambda: pins.test_q4_0_code_eight_is_zero_and_scale_per_block(),
        lambda: pins.test_predictor_golden_rank1(golden),
        lambda: pins.test_predictor_golden_relu_layer(golden),
        lambda: pins.test_predictor_zero_p2_gives_offsets(),
        lambda: pins.test_predictor_matches_library_matmul_and_union(),
        lambda: pins.test_compact_brute_force(1000, 0.5),
        lambda: pins.test_relu_golden(golden),
        lambda: pins.test_reglu_golden(golden),
        lambda: pins.test_q4_0_ffn_golden(golden),
        lambda: pins.test_q4_0_zero_codes_give_relu_bias(),
        lambda: pins.test_brute_force_all_masks_tiny(False),
        lambda: pins.test_brute_force_all_masks_tiny(True),
        lambda: pins.test_dense_equals_sparse_invariants(pins.LAYER_CASES[0]),
        lambda: pins.test_dense_equals_sparse_invariants(pins.LAYER_CASES[2]),
        lambda: pins.test_dense_equals_sparse_invariants(pins.LAYER_CASES[3]),
        lambda: pins.test_squared_relu_by_hand(),
        lambda: pins.test_placement_slots_are_an_indirection(),
        lambda: pins.test_empty_active_set_gives_down_bias(),
    ]


def _count_failures(golden):
    fails = 0
    for fn in _pin_suite(golden):
        try:
            fn()
        except Exception:          # an assertion, a ValueError from a bad code path, ...
            fails += 1
    return fails


@pytest.fixture
def swap_lib():
    saved = (oracle._lib, oracle._LIB_PATH)
    tmp = tempfile.mkdtemp(prefix="pio_mut_")
    yield tmp
    oracle._lib, oracle._LIB_PATH = saved
    shutil.rmtree(tmp, ignore_errors=True)


def test_unmutated_oracle_passes_the_suite(golden):
    assert _count_failures(golden) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, golden, swap_lib):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
    path_c = os.path.join(swap_lib, "pi_oracle.c")
    with open(path_c, "w") as fh:
        fh.write(src.replace(old, new))
    shutil.copy(HDR, swap_lib)
    so = os.path.join(swap_lib, "libmut.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", so, path_c, "-lm"], check=True)
    oracle._lib, oracle._LIB_PATH = None, so
    assert _count_failures(golden) > 0, f"no pin catches the mutant {name!r}"
