"""Planted mistakes in the oracle must each fail at least one of its pins.

Each case copies the oracle package into a scratch directory, changes one
expression in it (a plausible slip: a dropped term, a wrong sign, index or
operand, an off-by-one mask, a missing normalisation) and runs the pin tests
of that part in a fresh interpreter whose ``import oracle`` resolves to the
copy, which builds its own liboracle.so from the changed source.  The pins
must fail (pytest exit status 1).  The unchanged copy must pass, and must be
the module the pins import, or the other cases would prove nothing.

Every mistake is in bounds: a changed index stays inside its array, so a case
fails by wrong values, never by a crash.  All of this runs on the CPU.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

# (case id, file in oracle/, text to change (must occur exactly once), replacement, pin file)
MUTANTS = [
    # pointwise chain ("C-05", section 3)
    ("chain-relu-odd-stages", "oracle.c", "if (relu_even && (s % 2) == 0 && v < 0.0)\n",
     "if (relu_even && (s % 2) == 1 && v < 0.0)\n", "test_oracle_chain.py"),
    ("chain-a-times-y-plus-b", "oracle.c", "v = (double)a[s] * v + (double)b[s];",
     "v = (double)a[s] * (v + (double)b[s]);", "test_oracle_chain.py"),
    ("chain-bias-sign", "oracle.c", "v = (double)a[s] * v + (double)b[s];",
     "v = (double)a[s] * v - (double)b[s];", "test_oracle_chain.py"),
    ("chain-f32-two-roundings", "oracle.c", "v = fmaf(a[s], v, b[s]);", "v = a[s] * v + b[s];",
     "test_oracle_chain.py"),
    ("chain-f32-relu-odd-stages", "oracle.c", "(s % 2) == 0 && v < 0.0f", "(s % 2) == 1 && v < 0.0f",
     "test_oracle_chain.py"),
    # fat-probe sink ("C-05", section 3, fat row)
    ("fat-sink-no-halving", "oracle.c", "t = 0.5 * t + y;", "t = t + y;", "test_oracle_chain.py"),
    ("fat-sink-stage-modulo", "oracle.c", "for (; j < T && ((int64_t)j * K) / T == s; ++j) {\n                    t = 0.5",
     "for (; j < T && (j % K) == s; ++j) {\n                    t = 0.5", "test_oracle_chain.py"),
    ("fat-sink-lane-stride", "oracle.c", "q += lanes) {\n            double y", "q += 1) {\n            double y",
     "test_oracle_chain.py"),
    ("fat-sink-f32-forward-sum", "oracle.c",
     "float r = t[T - 1];\n                        for (int jj = T - 2; jj >= 0; --jj)\n                            r = t[jj] + r;",
     "float r = t[0];\n                        for (int jj = 1; jj < T; ++jj)\n                            r = r + t[jj];",
     "test_oracle_chain.py"),
    ("fat-sink-f32-two-roundings", "oracle.c", "y = fmaf(a[s], y, b[s]);\n                        if (relu_even",
     "y = a[s] * y + b[s];\n                        if (relu_even", "test_oracle_chain.py"),
    # GEMM + bias + GELU + residual ("K4", section 1)
    ("gemm-b-transposed", "oracle.c", "half_bits_to_double(B[k * N + j])", "half_bits_to_double(B[j * K + k])",
     "test_oracle_gemm.py"),
    ("gemm-last-k-dropped", "oracle.c", "for (int64_t k = 0; k < K; ++k)\n        acc +=",
     "for (int64_t k = 0; k < K - 1; ++k)\n        acc +=", "test_oracle_gemm.py"),
    ("gemm-bias-dropped", "oracle.c", "double c1 = c + half_bits_to_double(bias[j]);", "double c1 = c;",
     "test_oracle_gemm.py"),
    ("gemm-bias-reversed", "oracle.c", "double c1 = c + half_bits_to_double(bias[j]);",
     "double c1 = c + half_bits_to_double(bias[N - 1 - j]);", "test_oracle_gemm.py"),
    ("gelu-without-sqrt2", "oracle.c", "erf(z / sqrt(2.0))", "erf(z)", "test_oracle_gemm.py"),
    ("gelu-erf-sign", "oracle.c", "(1.0 + erf(", "(1.0 - erf(", "test_oracle_gemm.py"),
    ("gemm-residual-dropped", "oracle.c", "return c2 + half_bits_to_double(R[i * N + j]);", "return c2;",
     "test_oracle_gemm.py"),
    ("gemm-residual-columns-reversed", "oracle.c", "return c2 + half_bits_to_double(R[i * N + j]);",
     "return c2 + half_bits_to_double(R[i * N + (N - 1 - j)]);", "test_oracle_gemm.py"),
    ("fp16-exponent-off-by-one", "oracle.c", "ldexp((double)(1024 + m), e - 25)",
     "ldexp((double)(1024 + m), e - 24)", "test_oracle_gemm.py"),
    ("fp16-subnormal-scale", "oracle.c", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);",
     "test_oracle_gemm.py"),
    # causal softmax ("AIGC", section 3.5 and the attention-tail section)
    ("softmax-strict-mask", "oracle.c", "orow[j] = (j <= i) ?", "orow[j] = (j < i) ?",
     "test_oracle_softmax.py"),
    ("softmax-max-without-diagonal", "oracle.c", "for (int64_t j = 0; j <= i; ++j) {\n        double z = scale",
     "for (int64_t j = 0; j < i; ++j) {\n        double z = scale", "test_oracle_softmax.py"),
    ("softmax-unscaled-sum", "oracle.c", "l += exp(scale * bf16_bits_to_double(srow[j]) - m);",
     "l += exp(bf16_bits_to_double(srow[j]) - m);", "test_oracle_softmax.py"),
    ("softmax-sum-over-masked-keys", "oracle.c", "for (int64_t j = 0; j <= i; ++j)\n        l += exp(",
     "for (int64_t j = 0; j < S; ++j)\n        l += exp(", "test_oracle_softmax.py"),
    ("softmax-exponent-sign", "oracle.c", "? exp(scale * bf16_bits_to_double(srow[j]) - m) / l",
     "? exp(m - scale * bf16_bits_to_double(srow[j])) / l", "test_oracle_softmax.py"),
    ("bf16-decode-shift", "oracle.c", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;",
     "test_oracle_softmax.py"),
    # causal attention
    ("attention-strict-mask-in-pv", "oracle.c", "for (int64_t j = 0; j <= i; ++j) {\n        const uint16_t *v = V",
     "for (int64_t j = 0; j < i; ++j) {\n        const uint16_t *v = V", "test_oracle_attention.py"),
    ("attention-no-normalisation", "oracle.c", "orow[d] /= l;", "orow[d] /= 1.0;", "test_oracle_attention.py"),
    ("attention-k-from-q", "oracle.c", "const uint16_t *k = K + (bh * S + j) * D;",
     "const uint16_t *k = Q + (bh * S + j) * D;", "test_oracle_attention.py"),
    ("attention-q-from-k", "oracle.c", "const uint16_t *q = Q + (bh * S + i) * D;",
     "const uint16_t *q = K + (bh * S + i) * D;", "test_oracle_attention.py"),
    ("attention-v-of-query-row", "oracle.c", "const uint16_t *v = V + (bh * S + j) * D;",
     "const uint16_t *v = V + (bh * S + i) * D;", "test_oracle_attention.py"),
    ("attention-scale-twice", "oracle.c", "z[j] = scale * dot;", "z[j] = scale * scale * dot;",
     "test_oracle_attention.py"),
    ("attention-exponent-sign", "oracle.c", "z[j] = exp(z[j] - m);", "z[j] = exp(m - z[j]);",
     "test_oracle_attention.py"),
    ("attention-last-d-dropped", "oracle.c", "for (int64_t d = 0; d < D; ++d)\n            dot +=",
     "for (int64_t d = 0; d < D - 1; ++d)\n            dot +=", "test_oracle_attention.py"),
    # RMSNorm
    ("rmsnorm-sum-not-mean", "oracle.c", "sqrt(ss / (double)d + eps)", "sqrt(ss + eps)",
     "test_oracle_rmsnorm.py"),
    ("rmsnorm-eps-outside-root", "oracle.c", "sqrt(ss / (double)d + eps)", "sqrt(ss / (double)d) + eps",
     "test_oracle_rmsnorm.py"),
    ("rmsnorm-no-root", "oracle.c", "sqrt(ss / (double)d + eps)", "(ss / (double)d + eps)",
     "test_oracle_rmsnorm.py"),
    ("rmsnorm-gain-reversed", "oracle.c", "/ r * (double)g[j];", "/ r * (double)g[d - 1 - j];",
     "test_oracle_rmsnorm.py"),
    ("rmsnorm-sum-not-squares", "oracle.c", "ss += (double)xr[j] * (double)xr[j];", "ss += (double)xr[j];",
     "test_oracle_rmsnorm.py"),
    # byte and launch ledgers
    ("ledger-cut-not-reread", "ledger.py", "elems += seg[0].chain_reads", "elems += 0 * seg[0].chain_reads",
     "test_oracle_ledger.py"),
    ("ledger-external-reads-first-op-only", "ledger.py", "for st in seg:\n            elems += st.external_reads",
     "for st in seg[:1]:\n            elems += st.external_reads", "test_oracle_ledger.py"),
    ("ledger-bias-reads-mn", "ledger.py", 'Stage("bias", MN, N, MN)', 'Stage("bias", MN, MN, MN)',
     "test_oracle_ledger.py"),
    ("ledger-chain-x-not-read", "ledger.py", "Stage(f\"s{s}\", n, n if s == 0 else 0, 0 if s == 0 else n)",
     "Stage(f\"s{s}\", n, 0, 0 if s == 0 else n)", "test_oracle_ledger.py"),
    ("ledger-softmax-exp-step-no-write", "ledger.py", '("exp_mask", 1, 1)', '("exp_mask", 1, 0)',
     "test_oracle_ledger.py"),
    ("ledger-softmax-mask-not-read", "ledger.py", "mask_reads = 1", "mask_reads = 0", "test_oracle_ledger.py"),
    ("ledger-block-fraction-strict", "ledger.py", "if kb <= q)", "if kb < q)", "test_oracle_ledger.py"),
    ("ledger-softmax-one-tile-too-many", "ledger.py", "min(S, (i // tile + 1) * tile)",
     "min(S, (i // tile + 2) * tile)", "test_oracle_ledger.py"),
    ("ledger-rmsnorm-write-missing", "ledger.py", "passes * 2 * n * elem_bytes", "passes * n * elem_bytes",
     "test_oracle_rmsnorm.py"),
    ("ledger-rmsnorm-three-passes", "ledger.py", "passes = 1 if fused else len(RMSNORM_PASSES)",
     "passes = 1 if fused else len(RMSNORM_PASSES) - 1", "test_oracle_rmsnorm.py"),
    ("ledger-compositions-last-run-dropped", "ledger.py", "        plan.append(run)\n        out.append(plan)",
     "        out.append(plan)", "test_oracle_ledger.py"),
]

UNCHANGED_PINS = sorted({m[4] for m in MUTANTS})


def _copy_oracle(dst_root, fname=None, old=None, new=None):
    dst = os.path.join(dst_root, "oracle")
    os.makedirs(dst)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, f))
    if fname is not None:
        path = os.path.join(dst, fname)
        with open(path) as fh:
            text = fh.read()
        assert text.count(old) == 1, f"{fname}: the text to change occurs {text.count(old)} times"
        with open(path, "w") as fh:
            fh.write(text.replace(old, new))


def _env():
    env = dict(os.environ)
    # ROOT on the path (for synth) behind the working directory, which holds the copy
    env["PYTHONPATH"] = ROOT
    env["OMP_NUM_THREADS"] = "2"
    return env


def _run_pins(workdir, pin_files):
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-c", os.path.join(ROOT, "pytest.ini"), "--rootdir", ROOT] + [os.path.join(TESTS, p) for p in pin_files]
    r = subprocess.run(cmd, cwd=workdir, env=_env(), stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    return r.returncode, r.stdout


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Exit status and tail of output of the pins for every planted mistake
    (run four at a time), plus the unchanged copy under the key None."""
    jobs = {}
    base = str(tmp_path_factory.mktemp("oracle_unchanged"))
    _copy_oracle(base)
    jobs[None] = (base, UNCHANGED_PINS)
    for mid, fname, old, new, pins in MUTANTS:
        d = str(tmp_path_factory.mktemp(mid))
        _copy_oracle(d, fname, old, new)
        jobs[mid] = (d, [pins])
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {k: ex.submit(_run_pins, d, p) for k, (d, p) in jobs.items()}
        return {k: (f.result()[0], f.result()[1][-2000:], jobs[k][0]) for k, f in futs.items()}


def test_unchanged_copy_passes_and_is_the_one_imported(outcomes):
    rc, out, workdir = outcomes[None]
    assert rc == 0, out
    r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"], cwd=workdir,
                       env=_env(), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert os.path.realpath(r.stdout.strip()).startswith(os.path.realpath(workdir)), r.stdout
    # the copy built its own library from its own source
    assert os.path.exists(os.path.join(workdir, "oracle", "liboracle.so"))


@pytest.mark.parametrize("mid", [m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(outcomes, mid):
    rc, out, _ = outcomes[mid]
    assert rc == 1, f"{mid}: pins exited with {rc} (1 = a pin failed)\n{out}"
