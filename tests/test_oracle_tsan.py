"""The C oracle's row threading (oracle/ref.c: a mutex-guarded row counter
in the forward, per-thread dK/dV partials in the backward) under
ThreadSanitizer.  A small C driver, compiled with ref.c and
-fsanitize=thread, runs the forward (with and without a block mask) and the
backward on seeded inputs with 1 and 7 threads and checks that the results
agree; the run must end without a report.  The same driver on a copy of
ref.c whose row counter is read and advanced without its lock must stop
with a data-race report."""
import os
import subprocess

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "ref.c")

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention_masked(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int Nq,
                            int Nk, int d, double scale, int causal, const uint8_t *mask, int bq, int bk,
                            const int32_t *rows, int64_t nrows, double *o, double *lse, int nthreads);
int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout, int B, int Hq,
                         int Hkv, int Nq, int Nk, int d, double scale, int causal, const int32_t *groups,
                         int64_t ngroups, double *dq, double *dk, double *dv, int nthreads);

static uint64_t st = 88172645463325252ull;
static float rnd(void)   /* xorshift64, uniform in [-1, 1) */
{
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (float)((double)(st >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

int main(void)
{
    enum { B = 2, Hq = 4, Hkv = 2, Nq = 70, Nk = 90, d = 32, G = 4 };
    const int g = Hq / Hkv, nq = (Nq + 15) / 16, nk = (Nk + 15) / 16;
    float *q = malloc(sizeof(float) * B * Nq * Hq * d), *dout = malloc(sizeof(float) * B * Nq * Hq * d);
    float *k = malloc(sizeof(float) * B * Nk * Hkv * d), *v = malloc(sizeof(float) * B * Nk * Hkv * d);
    for (int i = 0; i < B * Nq * Hq * d; ++i) { q[i] = rnd(); dout[i] = rnd(); }
    for (int i = 0; i < B * Nk * Hkv * d; ++i) { k[i] = rnd(); v[i] = rnd(); }
    uint8_t *mask = malloc((size_t)Hq * nq * nk);
    for (int i = 0; i < Hq * nq * nk; ++i) mask[i] = rnd() > -0.4f;
    const int64_t R = (int64_t)B * Hq * Nq;
    int32_t *rows = malloc(sizeof(int32_t) * 3 * R);
    for (int64_t r = 0; r < R; ++r) {
        rows[3 * r] = (int32_t)(r / (Hq * Nq)); rows[3 * r + 1] = (int32_t)(r / Nq % Hq); rows[3 * r + 2] = (int32_t)(r % Nq);
    }
    int32_t groups[2 * G] = {0, 0, 0, 1, 1, 0, 1, 1};
    double *o1 = malloc(sizeof(double) * R * d), *o7 = malloc(sizeof(double) * R * d);
    double *l1 = malloc(sizeof(double) * R), *l7 = malloc(sizeof(double) * R);
    for (int m = 0; m < 2; ++m) {
        const uint8_t *mk = m ? mask : NULL;
        if (oracle_attention_masked(q, k, v, B, Hq, Hkv, Nq, Nk, d, 0.2, 1, mk, 16, 16, rows, R, o1, l1, 1) ||
            oracle_attention_masked(q, k, v, B, Hq, Hkv, Nq, Nk, d, 0.2, 1, mk, 16, 16, rows, R, o7, l7, 7)) {
            puts("forward failed"); return 1;
        }
        for (int64_t i = 0; i < R * d; ++i) if (o1[i] != o7[i]) { puts("forward: thread counts differ"); return 1; }
        for (int64_t i = 0; i < R; ++i) if (l1[i] != l7[i] && !(isinf(l1[i]) && isinf(l7[i]))) { puts("lse differs"); return 1; }
    }
    const size_t nqd = (size_t)G * g * Nq * d, nkd = (size_t)G * Nk * d;
    double *dq1 = malloc(sizeof(double) * nqd), *dk1 = malloc(sizeof(double) * nkd), *dv1 = malloc(sizeof(double) * nkd);
    double *dq7 = malloc(sizeof(double) * nqd), *dk7 = malloc(sizeof(double) * nkd), *dv7 = malloc(sizeof(double) * nkd);
    if (oracle_attention_bwd(q, k, v, dout, B, Hq, Hkv, Nq, Nk, d, 0.2, 1, groups, G, dq1, dk1, dv1, 1) ||
        oracle_attention_bwd(q, k, v, dout, B, Hq, Hkv, Nq, Nk, d, 0.2, 1, groups, G, dq7, dk7, dv7, 7)) {
        puts("backward failed"); return 1;
    }
    for (size_t i = 0; i < nqd; ++i) if (dq1[i] != dq7[i]) { puts("dq: thread counts differ"); return 1; }
    for (size_t i = 0; i < nkd; ++i)
        if (fabs(dk1[i] - dk7[i]) > 1e-12 || fabs(dv1[i] - dv7[i]) > 1e-12) { puts("dk/dv differ"); return 1; }
    puts("TSAN-DRIVER-OK");
    return 0;
}
"""

LOCKED = """        pthread_mutex_lock(&J->lock);
        r = J->next;
        J->next += 16;
        pthread_mutex_unlock(&J->lock);"""


def _build_and_run(tmp_path, src_path):
    if subprocess.run(["gcc", "-print-file-name=libtsan.so"], capture_output=True, text=True).stdout.strip() \
            == "libtsan.so":
        pytest.skip("gcc's ThreadSanitizer runtime is not installed")
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = str(tmp_path / "driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=thread", "-fno-omit-frame-pointer", "-o", exe,
                    str(drv), src_path, "-lm", "-lpthread"], check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.mark.timeout(400)
def test_oracle_threads_under_tsan(tmp_path):
    r = _build_and_run(tmp_path, SRC)
    out = r.stdout + r.stderr
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "TSAN-DRIVER-OK" in r.stdout, out[-4000:]


@pytest.mark.timeout(400)
def test_a_planted_race_is_caught(tmp_path):
    src = open(SRC).read()
    assert src.count(LOCKED) == 1
    bad = tmp_path / "ref_unlocked.c"
    bad.write_text(src.replace(LOCKED, "        r = J->next;\n        J->next += 16;"))
    r = _build_and_run(tmp_path, str(bad))
    assert r.returncode != 0 and "ThreadSanitizer: data race" in r.stderr, (r.stdout + r.stderr)[-3000:]
