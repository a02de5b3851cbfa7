"""Every kernel of the library fits its register budget (CPU): each HIP source
is compiled for gfx950 with the compiler's resource remarks, and no kernel may
spill VGPRs or use per-lane scratch (a spill turns register traffic into
memory traffic on every loop trip, and the parity tests would not notice)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from paged_kv_cache_432_amd import _build

HIP_SOURCES = [s for s in _build.SOURCES if s.endswith(".hip")]


def _remarks(src):
    cmd = [_build.hipcc(), *[f for f in _build.DEVICE_FLAGS if f != "-fPIC"], f"-I{_build.INCLUDE}",
           f"-I{_build.CSRC}", "--cuda-device-only", "-c", os.path.join(_build.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stderr


@pytest.fixture(scope="module")
def remarks():
    with ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        return dict(zip(HIP_SOURCES, ex.map(_remarks, HIP_SOURCES)))


def _kernels(text):
    """(kernel name, {field: value}) for each function the remarks report."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = (m.group(1), {})
            out.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+(?:\[[^\]]*\])?): (\d+)", line)
        if m and cur is not None:
            cur[1][m.group(1).strip()] = int(m.group(2))
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_spills(remarks, src):
    ks = _kernels(remarks[src])
    if not ks:                                      # a source with device data but no kernel
        assert "__global__" not in open(os.path.join(_build.CSRC, src)).read(), f"{src}: no kernels reported"
        return
    bad = [(n, f) for n, f in ks if f.get("VGPRs Spill", 0) or f.get("ScratchSize [bytes/lane]", 0)]
    assert not bad, "\n".join(f"{n}: {f}" for n, f in bad)
