"""The quantize kernel's bucket-table encode equals the threshold count for every input.

The gfx950 quantize kernel finds the NF4 code of a normalised value x (|x| <= 1) by one
read of a bucket table (bucket floor(32 x) + 32: the count of thresholds below the bucket
and the bucket's own threshold; one extra entry for a NaN quotient) and one strict
comparison, instead of comparing x with all fifteen thresholds.  This test compiles a C program that builds the
table from the library's own levels and compares the two for every fp32 value in [-1, 1];
it also checks the premise that no bucket holds two thresholds.
"""
import os
import shutil
import subprocess

import pytest

import bit_nf4_quantized_09_amd as nf4

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bucket_encode_matches_threshold_count_exhaustively(tmp_path):
    levels = nf4.nf4_codebook()
    exe = tmp_path / "bucket_encode"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "c", "bucket_encode_exhaustive.c"), "-o", str(exe), "-lm"],
                   check=True)
    out = subprocess.run([str(exe)] + [float(v).hex() for v in levels], check=True,
                         capture_output=True, text=True).stdout.split()
    n, bad, most = int(out[0]), int(out[1]), int(out[2])
    assert n == 2 * (0x3F800000 + 1) + 1    # every fp32 in [0, 1], with both signs, and NaN
    assert most == 1
    assert bad == 0
