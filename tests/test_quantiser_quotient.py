"""The GPU quantiser replaces the division x / s by a reciprocal, a multiply and two fused
multiply-adds (Markstein's correction).  This CPU test proves, by enumerating every block scale
the quantiser can produce and every bf16 value a block can hold, that the replacement yields the
same E4M3 code as the correctly rounded quotient (bit-identical wherever |x/s| >= 2^-11)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_three_op_quotient_equals_division_exhaustively(tmp_path):
    exe = tmp_path / "quotient_exhaustive"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-o", str(exe),
                           os.path.join(HERE, "quotient_exhaustive.c"), "-lm"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    scales, pairs = int(r.stdout.split()[1]), int(r.stdout.split()[3])
    assert scales == 18095 and pairs > 8.5e8, r.stdout
