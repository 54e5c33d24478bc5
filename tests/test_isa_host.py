"""The kernels' direct global->LDS loads are written as inline assembly
whose buffer resource operand must be scalar registers.  Should the
compiler ever hand such an operand a vector register tuple (it does when it
cannot prove the value uniform), the instruction would be malformed.  Each
kernel source is compiled to gfx950 assembly here (no GPU needed) and every
direct load is checked to name an SGPR resource."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from transformer_head_scaled_fwd_amd import build as b

LOADS = re.compile(r"buffer_load_dword\w*\s+v\d+,\s*(\S+),\s*\S+\s+offen\s+lds")


def _asm(src, tmp):
    out = os.path.join(tmp, src.replace(".hip", ".s"))
    cmd = ([b.hipcc()] + [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
           + ["-I", b.INCLUDE, "-I", b.CSRC, "-c", os.path.join(b.CSRC, src),
              "--offload-device-only", "-S", "-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("isa"))
    kernels = [s for s in b.SOURCES if s != "mha_abi.hip"]
    with ThreadPoolExecutor(max_workers=len(kernels)) as ex:
        texts = list(ex.map(lambda s: _asm(s, tmp), kernels))
    return dict(zip(kernels, texts))


def test_direct_loads_use_scalar_resources(assembly):
    total = 0
    for src, text in assembly.items():
        for m in LOADS.finditer(text):
            total += 1
            assert re.fullmatch(r"s\[\d+:\d+\]", m.group(1)), \
                "%s: direct load with a non-scalar resource: %s" % (src, m.group(0))
    assert total > 0
