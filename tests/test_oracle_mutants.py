"""Planted mistakes in a copy of the oracle source must fail at least one pin.

Each mutant is compiled from ``oracle/modal_oracle.c`` with one plausible
mistake (a sign, an ordering, a dropped term, a wrong index), on the CPU.  The
pins of ``test_oracle.py`` are then run against the mutant; at least one must
fail.  This shows the pins constrain every part of the oracle's arithmetic.
The projected layer (``oracle.stack_layer``, Python) gets the same treatment:
its source is copied with one mistake planted and executed in the oracle
module's namespace, and the stack pins must reject it.
"""

import inspect
import os
import subprocess
import textwrap

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "modal_oracle.c")

MUTANTS = {
    "readout-conjugates-residue": ("z += creal(R[n] * x[n]);", "z += creal(conj(R[n]) * x[n]);"),
    "update-before-read": (
        "                double z = Dg * u;\n                for (int64_t n = 0; n < d; ++n)\n"
        "                    z += creal(R[n] * x[n]);",
        "                for (int64_t n = 0; n < d; ++n)\n                    x[n] = lam[n] * x[n] + u;\n"
        "                double z = Dg * u;\n                for (int64_t n = 0; n < d; ++n)\n"
        "                    z += creal(R[n] * x[n]);"),
    "dropped-skip": ("double z = Dg * u;", "double z = 0.0 * Dg * u;"),
    "conjugated-pole": ("x[n] = lam[n] * x[n] + u;", "x[n] = conj(lam[n]) * x[n] + u;"),
    "head-map-modulo": ("const int64_t g = c / P;", "const int64_t g = c % H;"),
    "filter-exponent-off-by-one": ("cplx p = 1.0; /* lambda^(t-1) at t = 1 */", "cplx p = lam;"),
    "state-re-im-swapped": ("st[2 * n] = creal(x[n]);", "st[2 * n] = cimag(x[n]);"),
    "gate-uses-k": ("y[(b * T + t) * n_sel + i] = act_load(q, dtype, a) * z;",
                    "y[(b * T + t) * n_sel + i] = act_load(k, dtype, a) * z;"),
}

PIN_TESTS = [
    lambda o: [pins.test_hand_worked_examples(o, ex) for ex in pins._read_golden()],
    lambda o: [pins.test_recurrence_equals_direct_convolution(o, d) for d in (1, 3, 8)],
    pins.test_one_mode_geometric_series,
    pins.test_final_state_is_horner_polynomial,
    pins.test_impulse_response_is_filter,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(so), str(mpath), "-lm"], check=True)
    mutant = oracle.Bound(str(so))
    failures = 0
    for pin in PIN_TESTS:
        try:
            pin(mutant)
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(so), SRC, "-lm"], check=True)
    copy = oracle.Bound(str(so))
    for pin in PIN_TESTS:
        pin(copy)


# Mistakes planted in the Python source of oracle.stack_layer (generated-step leg
# and its hand-off from the prompt).
STACK_MUTANTS = {
    "steps-start-from-zero-state": ("state=st_prompt, batch_axis=1", "state=None, batch_axis=1"),
    "steps-output-reshaped-not-transposed": ("ys.transpose(1, 0, 2)",
                                             "ys.reshape(ys.shape[1], ys.shape[0], ys.shape[2])"),
    "steps-scanned-as-batch-major": ("batch_axis=1, time_axis=0", "batch_axis=0, time_axis=1"),
    "final-state-is-prompt-state": ("return out_prompt, out_steps, st_prompt, st",
                                    "return out_prompt, out_steps, st_prompt, st_prompt"),
    "normalisation-dropped": ("dense(x, w_in) * rms_inv(x, eps)[..., None]", "dense(x, w_in)"),
    "q-and-k-thirds-swapped": ("return (np.ascontiguousarray(qkv[..., :D]), np.ascontiguousarray(qkv[..., D:2 * D]),",
                               "return (np.ascontiguousarray(qkv[..., D:2 * D]), np.ascontiguousarray(qkv[..., :D]),"),
}

STACK_PINS = [pins.test_stack_layer_matches_unrolled_definition,
              pins.test_stack_layer_generated_steps_match_unrolled_definition]


class _StackMutant:
    """The oracle with its stack_layer replaced by a mutated copy."""

    def __init__(self, old, new):
        src = textwrap.dedent(inspect.getsource(oracle.stack_layer))
        assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
        ns = dict(vars(oracle))
        exec(compile(src.replace(old, new), "<stack_layer mutant>", "exec"), ns)
        self.stack_layer = ns["stack_layer"]
        self.modal_scan = oracle.modal_scan
        self.filter_taps = oracle.filter_taps


@pytest.mark.parametrize("name", sorted(STACK_MUTANTS))
def test_stack_mutant_fails_a_pin(name):
    mutant = _StackMutant(*STACK_MUTANTS[name])
    failures = 0
    for pin in STACK_PINS:
        try:
            pin(mutant)
        except Exception:  # an assertion, or a shape the mistake made inconsistent
            failures += 1
    assert failures >= 1, f"no pin caught stack mutant {name}"


def test_unmutated_stack_copy_passes_every_pin():
    copy = _StackMutant("eps: float = 1e-6", "eps: float = 1e-6")
    for pin in STACK_PINS:
        pin(copy)
    bound = oracle.Bound(oracle.build(force=False))
    for pin in STACK_PINS:
        pin(bound)
