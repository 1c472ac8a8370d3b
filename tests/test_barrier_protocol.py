"""The grid barrier's arrival and wait protocol, run on the host with one
thread per block (CPU only; the GPU is never made to give up): every block
present -> every barrier passes and the workspace is left at rest; a block
missing -> the others give up and count themselves, and every later launch on
that workspace is refused without touching it until the caller zeroes it; a
block arriving after a give-up stops at once."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_group_limited_amd", "csrc")


def test_barrier_protocol_on_host(tmp_path):
    exe = str(tmp_path / "barrier_host")
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-pthread", "-I", CSRC,
                           os.path.join(ROOT, "tests", "helpers", "barrier_host.cpp"), "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120).stdout
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert set(lines) == {"all_present", "give_up_then_refused", "late_block_stops"}, out
    assert all(v == "ok" for v in lines.values()), out
