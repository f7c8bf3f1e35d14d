"""Mutation checks of the oracle's pins (CPU only).

Each mutant is a copy of oracle/mx_oracle.cpp with one plausible mistake planted by a text
replacement, built with g++ into a temporary directory next to a copy of the oracle's Python binding.
The pin named for it (tests/test_oracle_worked_examples.py, tests/test_oracle_producer_bwd.py) must fail on the mutant, and the test
first checks that the replacement really changed the source (exactly one match), so a mutant can
never silently be the unchanged oracle. The unmutated oracle passes every pin (the worked-example
tests themselves).
"""
import concurrent.futures
import importlib.util
import os
import shutil
import subprocess

import numpy as np
import pytest

import test_oracle_producer_bwd as producer
import test_oracle_worked_examples as worked

PINS = {**worked.PINS, **producer.PINS}

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# name: (list of (original text, replacement), pin that must fail)
MUTANTS = {
    # the forward quantizes P at scale 1 (code 127) instead of 2^-8 (code 119)
    "fwd_p_scale_1": ([("int code = 119;", "int code = 127;")], "static_p_forward"),
    # the backward's recomputed P quantized at scale 1
    "bwd_p_scale_1": ([("e4m3_decode(e4m3_encode(p * 256.0)) * e8m0_value(119)",
                        "e4m3_decode(e4m3_encode(p * 1.0)) * e8m0_value(127)")], "static_p_backward"),
    # dV from the unquantized P
    "dv_from_fp32_p": ([("acc += Pq[i * TILE + j] * a.dO_mm", "acc += P[i * TILE + j] * a.dO_mm")],
                       "static_p_backward"),
    # binary16 rounding that truncates
    "fp16_truncates": ([("double y = std::nearbyint(a / quantum) * quantum;",
                         "double y = std::trunc(a / quantum) * quantum;")], "fp16_round"),
    # Delta from the quantized dO
    "delta_from_quantized_do": ([("od.data(), dobf.data(), lse", "od.data(), dod.data(), lse")],
                                "delta_from_bf16_do"),
    # dS quantized in 32 x 128 blocks (one scale across the tile's keys)
    "ds_blocks_32x128": ([("for (int64_t bj = 0; bj < nk; bj += 32) {", "for (int64_t bj = 0; bj < nk; bj += 128) {"),
                          ("ej = std::min<int64_t>(nk, bj + 32);", "ej = std::min<int64_t>(nk, bj + 128);")],
                         "ds_square_blocks"),
    # dK from the unquantized dS
    "dk_from_fp32_ds": ([("acc += dSq[i * TILE + j] * a.q[", "acc += dS[i * TILE + j] * a.q[")], "ds_square_blocks"),
    # the FP16 accumulator never rounded after an addition
    "fp16_acc_not_rounded": ([("cell = fp16_round(cell + fp16_round(a.sigma * acc));",
                               "cell = cell + fp16_round(a.sigma * acc);")], "dq_accumulators"),
    # the static dQ scale ignored
    "sigma_ignored": ([("cell = fp16_round(cell + fp16_round(a.sigma * acc));",
                        "cell = fp16_round(cell + fp16_round(acc));"),
                       ("double sig = (dq_mode == 1) ? (double)dq_sigma : 1.0;", "double sig = 1.0;")],
                      "dq_accumulators"),
    # the weight gradient reads the scale grid untransposed ([NB][C/32] instead of [C/32][NB])
    "wgrad_grid_untransposed": ([("e8m0_value(scale_t[(int64_t)(c / 32) * nb + br])",
                                  "e8m0_value(scale_t[br * (C / 32) + c / 32])")], "linear_bwd_weight_scaled_blocks"),
    # the data gradient multiplies by W^T's transpose (W read as [C_out, C_in])
    "dgrad_w_untransposed": ([("acc += dyd[(size_t)t * C_out + o] * wtd[(size_t)i * C_out + o];",
                               "acc += dyd[(size_t)t * C_out + o] * wtd[(size_t)o * C_in + i];")],
                             "linear_bwd_data_exact"),
    # the weight gradient sums over the first sequence only
    "wgrad_first_sequence": ([("for (int64_t t = 0; t < T; ++t) acc += dyd",
                               "for (int64_t t = 0; t < cu[1]; ++t) acc += dyd")], "linear_bwd_adjoint"),
    # the accumulated data gradient drops the earlier one
    "dgrad_accumulate_ignored": ([("if (dx_in) f = (float)((double)f + bf16_value(dx_in[(size_t)t * C_in + i]));",
                                   "if (dx_in) f = (float)((double)f);")], "linear_bwd_data_accumulate"),
    # RMSNorm backward with r^2 in place of r^3
    "rms_bwd_r_squared": ([("xk * r * r * r * S", "xk * r * r * S")], "rmsnorm_bwd_finite_differences"),
    # RMSNorm backward without gamma on the direct term
    "rms_bwd_gamma_missing": ([("r * (double)gamma[k] * dyk", "r * dyk")], "rmsnorm_bwd_finite_differences"),
    # dgamma without the row's r
    "dgamma_without_r": ([("dg[k] += dyk * xk * r;", "dg[k] += dyk * xk;")], "rmsnorm_bwd_finite_differences"),
    # the projection term of the RMSNorm backward with the wrong sign
    "rms_bwd_sign": ([("r * (double)gamma[k] * dyk - xk", "r * (double)gamma[k] * dyk + xk")],
                     "rmsnorm_bwd_scale_invariance"),
}


@pytest.fixture(scope="module")
def mutant_modules(tmp_path_factory):
    """Build every mutant in parallel; returns {name: imported oracle module}."""
    root = tmp_path_factory.mktemp("oracle_mutants")
    src = open(os.path.join(ORACLE_DIR, "mx_oracle.cpp")).read()
    dirs = {}
    for name, (edits, _) in MUTANTS.items():
        text = src
        for old, new in edits:
            assert text.count(old) == 1, f"{name}: pattern {old!r} must occur exactly once in the oracle source"
            text = text.replace(old, new)
        d = root / name
        d.mkdir()
        shutil.copy(os.path.join(ORACLE_DIR, "__init__.py"), d / "__init__.py")
        (d / "mx_oracle.cpp").write_text(text)
        dirs[name] = d

    def build(d):
        subprocess.run(["g++", "-O1", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                        str(d / "mx_oracle.cpp"), "-o", str(d / "libmxoracle.so")], check=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(build, dirs.values()))
    mods = {}
    for name, d in dirs.items():
        spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", d / "__init__.py",
                                                      submodule_search_locations=[str(d)])
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mods[name] = mod
    return mods


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pin_catches_mutant(name, mutant_modules):
    pin = PINS[MUTANTS[name][1]]
    with pytest.raises(AssertionError):
        pin(mutant_modules[name])


# ---------------------------------------------------------------------------------------------
# The GPU structure cases can fail: each planted mistake moves some (32-token block, head) of a
# gradient by more than ten times the stated tolerance on the inputs test_gpu_structure.py uses.
# ---------------------------------------------------------------------------------------------

SENSITIVITY = [
    # (structured case, mutant, gradient that must move)
    ("delta_sensitive", "delta_from_quantized_do", "dk"),
    ("delta_sensitive", "delta_from_quantized_do", "dq"),
    ("ds_block_range", "ds_blocks_32x128", "dk"),
    ("p_subnormal_band", "bwd_p_scale_1", "dv"),
]


@pytest.mark.parametrize("case_name,mutant,grad", SENSITIVITY)
def test_structured_case_separates_mutant(case_name, mutant, grad, mutant_modules):
    import oracle
    from mx_cases import GRAD_REL_FRO, AttnCase, block_rel_errors
    from synth import structured
    case = getattr(structured, case_name)()
    lens, H = case["lens"], case["inputs"]["q"].shape[1] // 128
    c = AttnCase(0, lens, None, H=H, softmax_scale=case["softmax_scale"], inputs=case["inputs"])
    c.run_oracle_fwd()
    good = c.run_oracle_bwd(1, 1.0)
    bad = c.run_oracle_bwd(1, 1.0, orc=mutant_modules[mutant])
    errs = block_rel_errors(bad[grad + "_f"], good[grad + "_f"], lens, H)
    assert errs.max() >= 10 * GRAD_REL_FRO, (case_name, mutant, grad, errs.max())


def test_fp16_rounding_case_separates_truncation(mutant_modules):
    from mx_cases import AttnCase
    from synth import structured
    case = structured.dq_fp16_rounding()
    vals = {}
    import oracle
    for name, orc in (("good", oracle), ("bad", mutant_modules["fp16_truncates"])):
        c = AttnCase(0, case["lens_q"], case["lens_k"], H=1, softmax_scale=case["softmax_scale"], inputs=case["inputs"])
        c.run_oracle_fwd(orc=orc)
        r = c.run_oracle_bwd(1, 2.0 ** -23, orc=orc, o16=np.zeros((1, 128), np.uint16), lse=np.zeros((1, 1), np.float32))
        vals[name] = float(r["dq_f"][0, 1])
    assert vals == {"good": 1.5, "bad": 1.0}
