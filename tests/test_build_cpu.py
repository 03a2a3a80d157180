"""Build checks that need no GPU: every split/combine kernel of the head_dim 128
units (and of the shared-tile multi-query units) compiles without scratch (no
register spills or stack arrays) and within two waves per SIMD, the occupancy
the kernels are tuned for."""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "int8_quantized_kv_amd"))


def _resource_usage(tmp_path, defines):
    import build
    obj = str(tmp_path / ("k" + "_".join(d.split("=")[1] for d in defines) + ".o"))
    cmd = build.compile_command("kernels.hip", obj, defines) + ["-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "hipcc")) is None, reason="hipcc not available")
def test_kernels_use_no_scratch(tmp_path):
    units = [["-DDATTN_D=128", "-DDATTN_CAP=0"], ["-DDATTN_D=128", "-DDATTN_CAP=1"],
             ["-DDATTN_D=128", "-DDATTN_CAP=1", "-DDATTN_SHARED=1"], ["-DDATTN_D=64", "-DDATTN_CAP=0", "-DDATTN_SHARED=1"]]
    with ThreadPoolExecutor(4) as ex:
        reports = list(ex.map(lambda d: _resource_usage(tmp_path, d), units))
    bad, n = [], 0
    for rep in reports:
        for blk in rep.split("Function Name: ")[1:]:
            name = blk.split()[0]
            n += 1
            scratch = int(re.search(r"ScratchSize \[bytes/lane\]: (\d+)", blk).group(1))
            occ = int(re.search(r"Occupancy \[waves/SIMD\]: (\d+)", blk).group(1))
            if scratch or occ < 2:
                bad.append((name, scratch, occ))
    assert n > 50 and not bad, bad
