"""The quotient form of QSGD's dequantization, fl(fl(nu * level) / s), in the kernels.

For a level count s in [1, 127] (and the min-max level counts 15 and 255) and t = 0 or
t >= 2^-100, the kernels compute fl(t / s)
as q0 = fl(t * fl(1/s)) followed by one correction with the exact remainder
fma(-q0, s, t), and divide for t below 2^-100.  tests/pins/level_count_division.c
compares that form with the IEEE binary32 division bit for bit: here over every t of the
domain for the level counts of the configurations (15, 127, 255), and over whole binades of t
for every s in [1, 127] (the form scales with t's exponent inside the normal range).  The
last case shows why the domain stops at 2^-100: for even s that are not powers of two a
subnormal quotient can be an exact midpoint that the correction rounds the wrong way.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LO = 0x0D800000      # bit pattern of 2^-100
INF = 0x7F800000


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("divcheck") / "level_count_division")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "pins", "level_count_division.c"),
                    "-lm"], check=True, capture_output=True)

    def run(jobs):
        def one(j):
            out = subprocess.run([exe] + [str(a) for a in j], capture_output=True, text=True, check=True)
            return int(out.stdout.strip()), out.stderr
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            return list(ex.map(one, jobs))
    return run


def test_domain_exact(checker):
    # 15 and 127: the QSGD level counts of the configurations; 15 and 255 also divide the
    # min-max range into its scale (int4, int8)
    jobs = [(15, 15, LO, INF), (127, 127, LO, INF), (255, 255, LO, INF), (1, 255, 0, 1),   # t = 0
            (1, 127, LO, LO + (1 << 23)),                                      # [2^-100, 2^-99)
            (1, 127, 127 << 23, 128 << 23),                                    # [1, 2)
            (1, 127, 254 << 23, INF)]                                          # [2^127, max]
    for job, (bad, err) in zip(jobs, checker(jobs)):
        assert bad == 0, f"{job}: {bad} mismatches\n{err}"


def test_subnormal_quotients_need_the_division(checker):
    # s = 6: some subnormal quotients are exact midpoints; the checker must see them
    (bad, _), = checker([(6, 6, 1, 0x00800000)])
    assert bad > 0
