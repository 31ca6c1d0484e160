"""The LDS-tiled kernel's build options still compile for gfx950 (device code
only, no GPU needed): 32-key tiles through four LDS buffers with the fp16
residual-weight product on heavy tiles, and the default 64-key tiles with
that product on every tile.  Each is an A/B switch that the default build
does not instantiate, so only this test keeps it from rotting."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from paged_gqa_kv_decode_amd import build as B

OPTIONS = [["-DVK_TILE_KEYS=32", "-DVK_TILE_SPLIT_WEIGHTS=1"],
           ["-DVK_TILE_KEYS=64", "-DVK_TILE_SPLIT_WEIGHTS=2"]]


def _compile(defs, out_dir):
    src = os.path.join(B.CSRC, "decode_varlen_tile.hip")
    obj = os.path.join(out_dir, "_".join(d.lstrip("-D").replace("=", "") for d in defs) + ".o")
    cmd = [B.HIPCC, *B.COMMON, *B.EXTRA["decode_varlen_tile.hip"], *defs, "--cuda-device-only",
           "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stderr[-2000:]


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not installed")
def test_tiled_kernel_build_options_compile():
    with tempfile.TemporaryDirectory(dir=B.ROOT, prefix="_build_opts_") as d:
        with ThreadPoolExecutor(len(OPTIONS)) as ex:
            results = list(ex.map(lambda o: _compile(o, d), OPTIONS))
    for defs, (rc, err) in zip(OPTIONS, results):
        assert rc == 0, f"{' '.join(defs)}: hipcc failed\n{err}"
