"""libecho must share torch's HIP runtime: importing the binding before
torch must not load a second libamdhip64 into the process (CPU check of the
loaded objects; the GPU suite depends on it)."""
import subprocess
import sys
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_loads_a_single_hip_runtime():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from error_feedback_quant_amd import echo\n"
        "import torch; torch.zeros(1)\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "libs = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
        "print(len(libs)); print('\\n'.join(libs))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout.split()
    assert out[0] == "1", out
