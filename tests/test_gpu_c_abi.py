"""The C ABI from C: tests/c_abi/dart_c_smoke.c, a plain C program built by
the package's build step against include/dart.h, libdart.so and the HIP
runtime (no Python, no torch in the process), run on the GPU.

The program checks properties fixed by the definitions on both kernel
families [DART §3 Eq. 5, 8-11; §4 "Inference Cache"]: gate 0 leaves Y_ssm
unchanged bit for bit, gate 1 gives bf16(Y_ssm + R) bit for bit, tokens of
chunk 0 see no chunk (R = 0, lse = -inf), repeated launches agree bit for
bit, decode of the last token reproduces the forward's row, the backward
with gate 0 gives exactly zero gradients and dgate = dout * R [App. C
Eq. 33-35], the chunk-state backward of a zero d_dH is exactly zero, the two
kernel families' backward agree at the bf16 bar, and a NULL input is refused
with DART_ERR_NULL."""
import os
import subprocess

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "dart_c_smoke.bin")


def test_c_program_uses_the_library():
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing: build the package first (state_memory_attention_amd.build)")
    say("C program", BIN)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c abi smoke ok" in r.stdout
