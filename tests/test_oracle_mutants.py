"""The oracle's pins catch plausible mistakes in the oracle itself.

Each mutant below is a copy of oracle/ssm_oracle.c with one planted mistake
of the kinds the pins are meant to catch: a dropped term, a wrong sign, an
index off by one, a wrong operand, two steps in the wrong order.  Every
mutant is compiled on its own (the real library is not touched) and the four
pin suites are run against it in a subprocess; at least one pin must fail.
The mistakes are planted on the CPU only; no device code is involved.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(REPO, "oracle", "ssm_oracle.c")
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py", "tests/test_oracle_conv_pins.py",
              "tests/test_oracle_ssd_pins.py"]

# name -> (original text, mutated text); the original must occur exactly once.
MUTANTS = {
    # scan (the decode update is the scan body run for one step)
    "scan: decay sign": ("      double abar = exp(dt * a);\n      double bbar;",
                         "      double abar = exp(-dt * a);\n      double bbar;"),
    "scan: input term without delta": ("        bbar = dt * Bt[n];\n", "        bbar = Bt[n];\n"),
    "scan: readout before the update": (
        "      state[n] = abar * state[n] + bbar * xv;\n      acc += Ct[n] * state[n];",
        "      acc += Ct[n] * state[n];\n      state[n] = abar * state[n] + bbar * xv;"),
    "scan: D term dropped": ("double yv = acc + Dval * xv;", "double yv = acc;"),
    "scan: gate is sigmoid, not SiLU": (
        "      double zv = z[t * io_stride];\n      yv = yv * (zv / (1.0 + exp(-zv)));",
        "      double zv = z[t * io_stride];\n      yv = yv / (1.0 + exp(-zv));"),
    "scan: h0 ignored": ("state[n] = h0 ? h0[(b * d_inner + d) * d_state + n] : 0.0;", "state[n] = 0.0;"),
    "scan: B of the previous step": ("const double* Bt = B + t * bc_stride;",
                                     "const double* Bt = B + (t > 0 ? t - 1 : 0) * bc_stride;"),
    "scan: A row of the next channel": ("oracle_scan_channel(x + off, delta + off, A + d * d_state,",
                                        "oracle_scan_channel(x + off, delta + off, A + ((d + 1) % d_inner) * d_state,"),
    "scan: h_last from state 0": ("h_last[(b * d_inner + d) * d_state + n] = state[n];",
                                  "h_last[(b * d_inner + d) * d_state + n] = state[0];"),
    "softplus: exp instead": ("  return log1p(exp(v));", "  return exp(v);"),
    "scan: dt_bias not added": ("if (delta_mode == 1) dt = oracle_softplus(dt + dt_bias);",
                                "if (delta_mode == 1) dt = oracle_softplus(dt);"),
    "scan: exact ZOH without 1/a": ("bbar = (a != 0.0) ? (expm1(dt * a) / a) * Bt[n] : dt * Bt[n];",
                                    "bbar = (a != 0.0) ? (expm1(dt * a)) * Bt[n] : dt * Bt[n];"),
    # conv
    "conv: taps reversed": ("acc += w[d * K + k] * xe[t + k];", "acc += w[d * K + (K - 1 - k)] * xe[t + k];"),
    "conv: bias dropped": ("        double acc = bias ? bias[d] : 0.0;", "        double acc = 0.0;"),
    "conv: carried state ignored": ("xe[j] = state_in ? state_in[(b * d_inner + d) * S + j] : 0.0;", "xe[j] = 0.0;"),
    "conv: state out from the start": ("state_out[(b * d_inner + d) * S + j] = xe[seqlen + j];",
                                       "state_out[(b * d_inner + d) * S + j] = xe[j];"),
    "conv: sigmoid instead of SiLU": ("if (apply_silu) acc = acc / (1.0 + exp(-acc));",
                                      "if (apply_silu) acc = 1.0 / (1.0 + exp(-acc));"),
    # backward
    "bwd: ddelta without the decay term": ("ddt += lam[n] * (a * abar * hp[n] + dcoef_ddt * Bt[n] * xv);",
                                           "ddt += lam[n] * (dcoef_ddt * Bt[n] * xv);"),
    "bwd: dA without abar": ("dA[d * N + n] += lam[n] * (dt * abar * hp[n] + dcoef_da * Bt[n] * xv);",
                             "dA[d * N + n] += lam[n] * (dt * hp[n] + dcoef_da * Bt[n] * xv);"),
    "bwd: adjoint not decayed": ("          lam[n] *= abar;\n", "\n"),
    "bwd: dz without silu' term": ("dz[io] = dy[io] * ypre * sg * (1.0 + zv * (1.0 - sg));",
                                   "dz[io] = dy[io] * ypre * sg;"),
    "bwd: dB without coefficient": ("dB[(b * seqlen + t) * N + n] += lam[n] * coef * xv;",
                                    "dB[(b * seqlen + t) * N + n] += lam[n] * xv;"),
    "bwd: dx without coefficient": ("dxv += lam[n] * coef * Bt[n];", "dxv += lam[n] * Bt[n];"),
    "bwd: dC from the previous state": ("dC[(b * seqlen + t) * N + n] += g * ht[n];",
                                        "dC[(b * seqlen + t) * N + n] += g * hp[n];"),
    "bwd: exact-ZOH d/ddelta = 1": ("dcoef_ddt = abar;", "dcoef_ddt = 1.0;"),
    "bwd: exact-ZOH d/da dropped": ("dcoef_da = oracle_dcoef_da(dt, a);", "dcoef_da = 0.0;"),
    "bwd: d/da series without k": ("term = (double)k * ypow / fact;", "term = ypow / fact;"),
    "bwd: softplus chain rule dropped": ("ddelta[io] = ddt * sg;", "ddelta[io] = ddt;"),
    "bwd: dD ignores the gate": ("if (dD) dD[d] += g * xv;", "if (dD) dD[d] += dy[io] * xv;"),
    "bwd: recomputed state without coefficient": (
        "hs[(t + 1) * N + n] = exp(dt * a) * hs[t * N + n] + coef * Bt[n] * xv;",
        "hs[(t + 1) * N + n] = exp(dt * a) * hs[t * N + n] + Bt[n] * xv;"),
    "bwd: dh0 is zero": ("dh0[(b * d_inner + d) * N + n] = lam[n];", "dh0[(b * d_inner + d) * N + n] = 0.0;"),
    # SSD form
    "ssd: decay without dt": ("const double a = exp(d * A[h]);", "const double a = exp(A[h]);"),
    "ssd: heads mapped to groups round-robin": ("const int64_t g = h / (nheads / ngroups);",
                                                "const int64_t g = h % ngroups;"),
    "ssd: readout before the update": (
        "            state[n] = a * state[n] + d * Bt[n] * xv;\n            acc += Ct[n] * state[n];",
        "            acc += Ct[n] * state[n];\n            state[n] = a * state[n] + d * Bt[n] * xv;"),
    "ssd: D term dropped": ("double yv = acc + (D ? D[h] : 0.0) * xv;", "double yv = acc;"),
    "ssd: dt_bias not added": ("if (delta_mode == 1) d = oracle_softplus(d + dt_bias[h]);",
                               "if (delta_mode == 1) d = oracle_softplus(d);"),
    "ssd: h0 ignored": ("state[n] = h0 ? h0[((b * nheads + h) * P + p) * N + n] : 0.0;", "state[n] = 0.0;"),
    "ssd: gate is sigmoid": ("            const double zv = z[io];\n            yv = yv * (zv / (1.0 + exp(-zv)));",
                             "            const double zv = z[io];\n            yv = yv / (1.0 + exp(-zv));"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique or missing: %s" % name
    idx = list(MUTANTS).index(name)
    c_path = os.path.join(tmp, "m%02d.c" % idx)
    so_path = os.path.join(tmp, "m%02d.so" % idx)
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99", "-shared", "-fPIC", "-o",
                    so_path, c_path, "-lm"], check=True)
    env = dict(os.environ, SSM_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-rf", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + PIN_SUITES, cwd=REPO, env=env, capture_output=True, text=True, timeout=600)
    failed = [ln.split()[1] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
    return name, r.returncode, failed[0] if failed else r.stdout[-400:]


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            results = list(ex.map(lambda n: _run_mutant(n, tmp), MUTANTS))
    for n, rc, out in results:
        print("%-44s %s" % (n, ("caught by " + out) if rc == 1 else "rc %d: %s" % (rc, out)))
    # Exit status 1: pins failed (not a crash, a collection error or no tests).
    bad = [(n, rc, out) for n, rc, out in results if rc != 1]
    assert not bad, bad


def test_unmutated_copy_passes_the_pins():
    """The harness itself is sound: an unmodified copy built the same way passes."""
    with tempfile.TemporaryDirectory() as tmp:
        so_path = os.path.join(tmp, "orig.so")
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99", "-shared", "-fPIC", "-o",
                        so_path, SRC, "-lm"], check=True)
        env = dict(os.environ, SSM_ORACLE_LIB=so_path)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                           + PIN_SUITES, cwd=REPO, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:]
