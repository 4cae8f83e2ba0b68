"""Every gfx950 kernel compiles without register spills (no per-lane scratch), and no
kernel writes through the scalar data cache. The device code of each source is compiled
to assembly with the library's own flags and its kernel metadata read back."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from decoder_only_transformer_bf16_amd import _build

pytestmark = pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc not installed")

HIP_SOURCES = [s for s in _build.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module")
def assembly():
    tmp = tempfile.mkdtemp(prefix="fwd_asm_")

    def compile_one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [_build.HIPCC, *_build.FLAGS, "--cuda-device-only", "-S", "-x", "hip",
               os.path.join(_build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
        assert r.returncode == 0, r.stdout.decode(errors="replace")[-2000:]
        return src, open(out).read()

    try:
        with ThreadPoolExecutor(len(HIP_SOURCES)) as ex:
            yield dict(ex.map(compile_one, HIP_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _kernels(text):
    """(name, scratch bytes) for every kernel in the code object metadata."""
    out = []
    for blk in re.findall(r"- \.agpr_count:.*?\.vgpr_spill_count:\s+\d+", text, re.S):
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk).group(1))
        out.append((name, scratch))
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_kernel_spills(assembly, src):
    ks = _kernels(assembly[src])
    assert ks, f"no kernel metadata found for {src}"
    spilled = [(n, b) for n, b in ks if b]
    assert not spilled, f"{src}: kernels with scratch: {spilled}"


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scalar_memory_writes(assembly, src):
    bad = re.findall(r"^\s*(s_store_\w+|s_atomic_\w+|s_buffer_store\w*|s_buffer_atomic\w*|s_dcache_wb\w*)",
                     assembly[src], re.M)
    assert not bad, f"{src}: {sorted(set(bad))}"
