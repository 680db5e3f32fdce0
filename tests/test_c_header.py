"""The C ABI used from C: include/pps.h compiles as strict C99, and a C
program linked against libpps.so drives a bookkeeping-only stage through a
whole schedule.  No device is touched (bookkeeping-only handles allocate
nothing and launch nothing), so this runs without a GPU."""

import os
import shutil
import subprocess

import pytest

from oracle import schedule as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "pipeline_schedules_amd")

C_SRC = r"""
#include <stdio.h>
#include <stdlib.h>
#include "pps.h"

int main(int argc, char** argv) {
    if (argc != 5) return 1;
    const int P = atoi(argv[1]), M = atoi(argv[2]), k = atoi(argv[3]), kind = atoi(argv[4]);
    int n = 0;
    if (pps_make_schedule(P, M, k, 1, kind, NULL, 0, &n) != PPS_EFULL || n <= 0) return 2;
    pps_op* ops = (pps_op*)malloc(sizeof(pps_op) * (size_t)n);
    if (pps_make_schedule(P, M, k, 1, kind, ops, n, &n) != PPS_OK) return 3;

    pps_stage_desc d = {0};
    d.P = P; d.M = M; d.k = k; d.v = 1; d.kind = kind;
    d.block_type = PPS_BLOCK_SWIGLU; d.dtype = PPS_DTYPE_BF16; d.L = 2;
    d.d = 64; d.ffn = 128; d.T = 16; d.eps = 1e-6f;
    d.flags = PPS_FLAG_BOOKKEEPING_ONLY;
    pps_stage* st = NULL;
    if (pps_stage_create(&d, &st) != PPS_OK || !st) return 4;
    for (int i = 0; i < n; ++i) {
        int rc;
        if (ops[i].op == PPS_OP_F) rc = pps_stage_forward(st, ops[i].mb, 0, NULL, NULL);
        else if (ops[i].op == PPS_OP_B) rc = pps_stage_backward(st, ops[i].mb, 0, NULL, NULL);
        else rc = pps_stage_backward_weight(st, ops[i].mb, 0);
        if (rc != PPS_OK) { fprintf(stderr, "op %d: %s\n", i, pps_strerror(rc)); return 5; }
    }
    pps_op* log = (pps_op*)malloc(sizeof(pps_op) * (size_t)n);
    int nl = 0;
    if (pps_stage_get_oplog(st, log, n, &nl) != PPS_OK || nl != n) return 6;
    pps_stats s;
    if (pps_stage_get_stats(st, &s) != PPS_OK) return 7;
    for (int i = 0; i < n; ++i)
        printf("%d %d %d %d %d %d\n", log[i].op, log[i].mb, log[i].chunk, log[i].slot, log[i].inflight_after,
               log[i].t_start);
    printf("peak %lld slots %lld\n", (long long)s.peak_live_entries, (long long)s.n_slots);
    pps_stage_destroy(st);
    free(ops);
    free(log);
    return 0;
}
"""


@pytest.fixture(scope="module")
def c_prog(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(PKG, "libpps.so")):
        pytest.skip("libpps.so not built")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "drive.c"
    src.write_text(C_SRC)
    exe = d / "drive"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC, str(src), "-o", str(exe),
           "-L", PKG, "-lpps", "-Wl,-rpath," + PKG]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(exe)


@pytest.mark.parametrize("P,M,k,kind", [(4, 6, 0, S.ONE_F_ONE_B), (4, 8, 1, S.ONE_F_ONE_B), (2, 4, 0, S.GPIPE),
                                        (4, 8, 0, S.ZB1P), (4, 8, 0, S.ZB2P)])
def test_c_program_drives_a_stage(c_prog, P, M, k, kind):
    r = subprocess.run([c_prog, str(P), str(M), str(k), str(kind)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    lines = r.stdout.strip().splitlines()
    got = [tuple(int(x) for x in ln.split()) for ln in lines[:-1]]
    want = [tuple(o) for o in S.stage_ops(P, M, k, 1, kind)]
    assert got == want
    peak = max(o[4] for o in want)
    assert lines[-1] == f"peak {peak} slots {peak}"
