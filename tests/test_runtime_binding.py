"""The library must share the HIP runtime that torch loads, whatever the import order."""
import subprocess
import sys

from tests.harness import ROOT


def test_single_hip_runtime_after_load():
    # A fresh interpreter that loads the library before anything imports torch must still
    # end up with exactly one libamdhip64 mapped (torch's).
    code = (
        "from bit_trainable_attention_amd import _lib; _lib.load(); import torch\n"
        "maps = [l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l]\n"
        "print(len(set(maps)))\n"
    )
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout
