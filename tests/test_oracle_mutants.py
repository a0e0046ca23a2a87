"""Mutation test of the oracle's pins (CPU only).

Each mutant is a copy of oracle/zs_oracle.c with one plausible mistake
planted (a wrong ring index, a dropped term, a swapped operand, a wrong
rounding or scaler rule). Every mutant is compiled and the oracle's pin
suites (tests/test_oracle_pins.py, tests/test_oracle_casts.py, which check
the oracle against the pages, closed forms and library routines, never
against the GPU path) are run against it: each mutant must make them fail.
A mutant that survives is a gap in the pins. The unmutated copy must pass.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "zs_oracle.c")
INC = os.path.join(ROOT, "oracle")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_casts.py")]

# (name, original text, mutated text): the original must occur in the source
MUTANTS = [
    ("partition rounds down", "uint64_t p = phi / world + (phi % world != 0);",
     "uint64_t p = phi / world;"),
    ("fp16 widening: subnormal scale", "mag = ldexpf((float)f, -24);", "mag = ldexpf((float)f, -25);"),
    ("bf16 widening: wrong shift", "return float_of((uint32_t)h << 16);",
     "return float_of((uint32_t)h << 15);"),
    ("bf16 narrowing truncates", "uint32_t q = rne_shift(mag, 16);", "uint32_t q = mag >> 16;"),
    ("narrowing ties away from zero", "if (rem > half || (rem == half && (q & 1u))) q += 1u;",
     "if (rem >= half) q += 1u;"),
    ("fp16 overflow saturates", "if (b >= 0x7c00u) b = 0x7c00u;", "if (b >= 0x7c00u) b = 0x7bffu;"),
    ("fp16 narrowing flushes subnormals", "int e_eff = e < -14 ? -14 : e;",
     "if (e < -14) return (uint16_t)(sign << 15);\n  int e_eff = e;"),
    ("bf16 NaN becomes inf", "return (uint16_t)((sign << 15) | 0x7fc0u);",
     "return (uint16_t)((sign << 15) | 0x7f80u);"),
    ("scatter-reduce sends the wrong chunk", "uint32_t c = mod_w((int64_t)k - s + sigma, world);",
     "uint32_t c = mod_w((int64_t)k + s + sigma, world);"),
    ("all-gather forwards the wrong chunk", "uint32_t c = mod_w((int64_t)k + sigma - s + 1, world);",
     "uint32_t c = mod_w((int64_t)k + sigma - s, world);"),
    ("chunk trace starts at the owner",
     "float acc = zso_half_to_float(part[(rank + 1) % world][i], dtype);\n"
     "    for (uint32_t s = 2; s <= world; ++s)",
     "float acc = zso_half_to_float(part[rank % world][i], dtype);\n"
     "    for (uint32_t s = 1; s < world; ++s)"),
    ("step's ring starts at the owner",
     "float acc = on_wire(zso_half_to_float(part[(rank + 1) % world][i], dtype), wire);\n"
     "  for (uint32_t s = 2; s <= world; ++s)",
     "float acc = on_wire(zso_half_to_float(part[rank % world][i], dtype), wire);\n"
     "  for (uint32_t s = 1; s < world; ++s)"),
    ("average by reciprocal", "float a = ring_elem(world, rank, part, dtype, wire, i) / wf;",
     "float a = ring_elem(world, rank, part, dtype, wire, i) * (1.0f / wf);"),
    ("step's average by reciprocal", "float avg = s / wf;", "float avg = s * (1.0f / wf);"),
    ("accumulation dropped", "if (accumulate) a = out[i] + a;", "if (accumulate) a = a + 0.0f;"),
    ("step's accumulation dropped", "if (a->acc_in) avg = a->acc_in[i] + avg;",
     "if (a->acc_in) avg = avg + 0.0f;"),
    ("reduce flag before the unscale", "float g = a / loss_scale;\n    if (!isfinite(g)) flag = 1;",
     "float g = a / loss_scale;\n    if (!isfinite(a)) flag = 1;"),
    ("check before the unscale", "if (!isfinite(a[i] / loss_scale)) return 1;",
     "if (!isfinite(a[i])) return 1;"),
    ("step flag before the unscale", "if (!isfinite(g)) flag = 1;\n    float m = a->m_in[i]",
     "if (!isfinite(avg)) flag = 1;\n    float m = a->m_in[i]"),
    ("beta^t one short", "for (uint32_t k = 0; k < t; ++k) {", "for (uint32_t k = 1; k < t; ++k) {"),
    ("no first bias correction", "out->alpha = (float)(l / (1.0 - b1t));", "out->alpha = (float)l;"),
    ("no second bias correction", "out->b2 = (float)sqrt(1.0 - b2t);", "out->b2 = 1.0f;"),
    ("decay factor without lr", "out->delta = (float)(1.0 - l * wd);", "out->delta = (float)(1.0 - wd);"),
    ("decay applied after the update", "float theta1 = decayed - k->alpha * (m1 / d);",
     "float theta1 = (theta - k->alpha * (m1 / d)) * k->delta;"),
    ("eps inside the square root", "float d = sqrtf(v1) / k->b2 + k->eps;",
     "float d = sqrtf(v1 + k->eps) / k->b2;"),
    ("second moment of g, not g^2", "k->c2 * (g * g)", "k->c2 * g"),
    ("first-moment coefficients swapped", "float m1 = k->beta1 * *m + k->c1 * g;",
     "float m1 = k->c1 * *m + k->beta1 * g;"),
    ("adamw without the unscale", "float g = a[i] / loss_scale;", "float g = a[i];"),
    ("step without the unscale", "float g = avg / a->loss_scale;", "float g = avg;"),
    ("step casts the old master", "a->param_out[i] = zso_float_to_half(theta, a->param_dtype);",
     "a->param_out[i] = zso_float_to_half(a->master_in[i], a->param_dtype);"),
    ("step drops a range end", "jobs[t].hi = a->n * (uint64_t)(t + 1) / (uint64_t)threads;",
     "jobs[t].hi = a->n * (uint64_t)(t + 1) / (uint64_t)threads - (t + 1 < threads ? 1 : 0);"),
    ("scaler keeps the clean count on overflow", "s->clean = 0;\n    s->skipped += 1;",
     "s->skipped += 1;"),
    ("scaler grows one step late", "if (s->clean >= s->interval) {", "if (s->clean > s->interval) {"),
    ("scaler counts a skipped step", "s->skipped += 1;\n    return;",
     "s->skipped += 1;\n    s->t += 1;\n    return;"),
    ("stage 2 accounted as stage 1", "case 2: return 2.0 * psi + (2.0 + k) * psi / n_gpus;",
     "case 2: return (2.0 + 2.0) * psi + k * psi / n_gpus;"),
    ("ring time without the factor 2", "2.0 * msg_bytes * (world - 1.0) / (world * beta)",
     "msg_bytes * (world - 1.0) / (world * beta)"),
    ("bf16 wire does not round",
     "if (wire == ZSO_WIRE_BF16) return zso_half_to_float(zso_float_to_half(x, ZSO_BF16), ZSO_BF16);",
     "if (wire == ZSO_WIRE_BF16) return x;"),
    ("wire leaves the first term unrounded",
     "float acc = on_wire(zso_half_to_float(part[(rank + 1) % world][i], dtype), wire);",
     "float acc = zso_half_to_float(part[(rank + 1) % world][i], dtype);"),
]


def _build_and_run(tmp, idx, name, old, new):
    src = open(SRC).read()
    if old is not None:
        assert old in src, f"mutant {name!r}: original text not found in zs_oracle.c"
        src = src.replace(old, new)
    c = os.path.join(tmp, f"mut{idx}.c")
    lib = os.path.join(tmp, f"libmut{idx}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-pthread", "-I", INC, c, "-o", lib, "-lm"], check=True,
                   capture_output=True)
    env = dict(os.environ, ZSO_ORACLE_LIB=lib, ZS_EXHAUSTIVE_CASTS="0")
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=os.path.join(ROOT, "tests"), env=env,
                       capture_output=True, text=True, timeout=900)
    return name, r.returncode, r.stdout[-600:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    tmp = str(tmp_path)
    jobs = [(i, name, old, new) for i, (name, old, new) in enumerate(MUTANTS)]
    jobs.append((len(MUTANTS), "unmutated control", None, None))
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _build_and_run(tmp, *j), jobs))
    control = results[-1]
    assert control[1] == 0, f"the unmutated oracle fails its pins:\n{control[2]}"
    survivors = [(name, out) for name, rc, out in results[:-1] if rc == 0]
    errors = [(name, rc, out) for name, rc, out in results[:-1] if rc not in (0, 1)]
    assert not errors, f"mutants that broke the run rather than a pin: {errors}"
    assert not survivors, "mutants no pin catches: " + ", ".join(n for n, _ in survivors)
