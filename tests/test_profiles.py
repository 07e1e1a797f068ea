"""Every derived rate a committed profile summary states follows from the
numbers beside it. A statement of the form

    <amount> <unit> / <time> <time unit> = <rate> <rate unit> [= <pct>% of [the] <peak> <rate unit>]

written on one line (GB, MB, B, GFLOP or TFLOP over ns, us/µs or ms, giving
GB/s, TB/s or TFLOP/s) is recomputed here; its rounded figures must agree
with the recomputation to the precision they are printed with. CPU only."""

import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NUM = r"(\d[\d,]*(?:\.\d+)?)"
AMOUNT = {"B": 1.0, "KB": 1e3, "MB": 1e6, "GB": 1e9, "GFLOP": 1e9, "TFLOP": 1e12}
TIME = {"ns": 1e-9, "us": 1e-6, "µs": 1e-6, "ms": 1e-3, "s": 1.0}
RATE = {"GB/s": 1e9, "TB/s": 1e12, "TFLOP/s": 1e12}
PATTERN = re.compile(
    NUM + r" (B|KB|MB|GB|GFLOP|TFLOP) / " + NUM + r" (ns|us|µs|ms|s) = " + NUM + r" (GB/s|TB/s|TFLOP/s)"
    r"(?: \(?= ?" + NUM + r"% of (?:the )?" + NUM + r" (GB/s|TB/s|TFLOP/s))?")


def num(s):
    return float(s.replace(",", ""))


def printed_precision(s):
    """Half a unit in the last printed digit of s."""
    s = s.replace(",", "")
    return 0.5 * 10.0 ** (-(len(s.split(".")[1]) if "." in s else 0))


def statements():
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for i, line in enumerate(open(path, encoding="utf-8"), 1):
            for m in PATTERN.finditer(line):
                yield f"{os.path.basename(path)}:{i}", m


def check_statement(m):
    amount = num(m.group(1)) * AMOUNT[m.group(2)]
    t = num(m.group(3)) * TIME[m.group(4)]
    rate = amount / t
    stated = num(m.group(5)) * RATE[m.group(6)]
    # the amount and the time are themselves rounded: allow their relative error too
    rel = printed_precision(m.group(1)) / num(m.group(1)) + printed_precision(m.group(3)) / num(m.group(3))
    tol = printed_precision(m.group(5)) * RATE[m.group(6)] + rel * rate
    assert abs(rate - stated) <= tol * 1.01, f"{m.group(0)}: recomputed {rate / RATE[m.group(6)]:.4g}"
    if m.group(7):
        peak = num(m.group(8)) * RATE[m.group(9)]
        pct = 100.0 * rate / peak
        tol_pct = printed_precision(m.group(7)) + 100.0 * rel * rate / peak
        assert abs(pct - num(m.group(7))) <= tol_pct * 1.01, f"{m.group(0)}: recomputed {pct:.3f}%"


def test_profile_rate_statements_follow_from_their_numbers():
    found = list(statements())
    assert found, "no rate statements found in profiles/"
    bad = []
    for where, m in found:
        try:
            check_statement(m)
        except AssertionError as e:
            bad.append(f"{where}: {e}")
    assert not bad, "\n".join(bad)


@pytest.mark.parametrize("text,ok", [
    ("835.3 GFLOP / 1.497 ms = 558 TFLOP/s = 22.3% of the 2,500 TFLOP/s", True),
    ("835.3 GFLOP / 1.497 ms = 1 TFLOP/s = 0.0% of the 2,500 TFLOP/s", False),
    ("1,303,255,804 B / 205.4 us = 6,345 GB/s (= 79.3% of 8,000 GB/s)", True),
    ("1,303,255,804 B / 205.4 us = 6,344 GB/s (= 75.3% of 8,000 GB/s)", False),
])
def test_the_checker_catches_a_wrong_ratio(text, ok):
    m = PATTERN.search(text)
    assert m is not None
    if ok:
        check_statement(m)
    else:
        with pytest.raises(AssertionError):
            check_statement(m)
