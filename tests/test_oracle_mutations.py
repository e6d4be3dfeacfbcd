"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The copy of oracle/ref.c is edited textually, compiled with gcc into a
temporary directory and run through the same pins as the real oracle
(tests/pins.py).  The real oracle is never modified.
"""
import functools
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ref.c")

# (name, original text, planted text)
MUTATIONS = [
    ("dropped_scale", "s[j] = J->scale * acc;", "s[j] = acc;"),
    ("wrong_gqa_index", "const int hk = h / g;", "const int hk = h % J->Hkv;"),
    ("causal_off_by_one", "nvis = last < 0 ? 0 : (last + 1 < J->Nk ? (int)(last + 1) : J->Nk);",
     "nvis = last < 0 ? 0 : (last < J->Nk ? (int)(last > 0 ? last : 1) : J->Nk);"),
    ("causal_top_left", "const int64_t last = (int64_t)i + (J->Nk - J->Nq);", "const int64_t last = (int64_t)i;"),
    ("empty_row_not_zero", "for (int x = 0; x < d; ++x) o_out[x] = 0.0;\n        *lse_out = -INFINITY;",
     "for (int x = 0; x < d; ++x) o_out[x] = 1.0;\n        *lse_out = 0.0;"),
    ("lse_dropped_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("exp_sign", "l += exp(s[j] - m);", "l += exp(m - s[j]);"),
    ("v_for_k", "const float *kj = J->k + (((int64_t)b * J->Nk + j)", "const float *kj = J->v + (((int64_t)b * J->Nk + j)"),
    ("v_reversed_coord", "o_out[x] += a * (double)vj[x];", "o_out[x] += a * (double)vj[d - 1 - x];"),
    ("q_from_key_row", "const float *qi = J->q + (((int64_t)b * J->Nq + i)", "const float *qi = J->q + (((int64_t)b * J->Nq + 0)"),
    ("no_normalise", "const double a = exp(s[j] - m) / l;", "const double a = exp(s[j] - m);"),
    ("max_not_subtracted_in_weights", "const double a = exp(s[j] - m) / l;", "const double a = exp(s[j]) / l;"),
    ("mask_ignored", "if (!J->mask) return 1;", "return 1;"),
    ("mask_blocks_swapped", "return J->mask[((int64_t)h * nqb + i / J->bq) * nkb + j / J->bk] != 0;",
     "return J->mask[((int64_t)h * nqb + i / J->bk) * nkb + j / J->bq] != 0;"),
    ("mask_kv_head", "return J->mask[((int64_t)h * nqb", "return J->mask[((int64_t)(h / (J->Hq / J->Hkv)) * nqb"),
    # backward
    ("bwd_no_softmax_jacobian", "const double ds = p[j] * (dp[j] - pdp);", "const double ds = p[j] * dp[j];"),
    ("bwd_dk_sign", "dkj[x] += J->scale * ds * (double)qi[x];", "dkj[x] -= J->scale * ds * (double)qi[x];"),
    ("bwd_dq_no_scale", "dqi[x] += J->scale * ds * (double)kj[x];", "dqi[x] += ds * (double)kj[x];"),
    ("bwd_dv_unnormalised", "p[j] /= l;", "p[j] /= 1.0;"),
    ("bwd_interleaved_groups", "const int h = J->hk * g + hh;", "const int h = J->hk + hh * J->Hkv;"),
    ("bwd_causal_top_left", "const int64_t last = (int64_t)i + (Nk - Nq);", "const int64_t last = (int64_t)i;"),
    ("bwd_dp_uses_k", "t += (double)doi[x] * (double)vj[x];", "t += (double)doi[x] * (double)kj[x];"),
    ("bwd_last_thread_sum_dropped", "for (int t = 0; t < nthreads; ++t) {\n                sk +=",
     "for (int t = 1; t < nthreads; ++t) {\n                sk +="),
]


@functools.lru_cache(maxsize=None)
def _build(name, tmpdir):
    src = open(SRC).read()
    orig, new = next((o, n) for nm, o, n in MUTATIONS if nm == name)
    assert src.count(orig) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(tmpdir, f"ref_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(orig, new))
    so = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", so, path, "-lm", "-lpthread"], check=True)
    return so


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, tmp_path_factory):
    so = _build(name, str(tmp_path_factory.mktemp("mut")))
    lib = oracle._open(so)
    att = functools.partial(oracle.attention, _lib_override=lib)
    bwd = functools.partial(oracle.attention_bwd, _lib_override=lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(att)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    if name.startswith("bwd_"):
        for pin in pins.BWD_PINS:
            try:
                pin(att, bwd)
            except (AssertionError, RuntimeError, FloatingPointError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
