"""The kernels' gfx950 assembly, on the host (hipcc cross-compiles; no GPU).

Two workgroup barriers with nothing but waits between them mean the compiler
moved all the code between two __syncthreads() below the second one.  That
happened once: the LDS reads of the one-frame step's state fragments were sunk
below the barrier after which other waves overwrite those bytes (the reads are
now pinned with hold()).  The source has no back-to-back barriers, so any pair
in the assembly is such a move.
"""
import os
import re
import shutil
import subprocess

import pytest

from gated_deltanet_scan_amd import build

CSRC = os.path.join(build.PKG, "csrc", "gdn_api.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gdn_api.s"
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only", "-S", CSRC,
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def test_every_kernel_is_in_the_assembly(asm):
    names = {m.group(1) for l in asm for m in [re.match(r"^(_ZN3gdn\w+):", l)] if m}
    for k in ("frame_gram_kernel", "state_scan_kernel", "frame_output_kernel", "frame_step_kernel",
              "frame_dkv_kernel", "state_copy_kernel"):
        assert any(k in n for n in names), k


def test_no_back_to_back_barriers(asm):
    fn, bad = None, []
    for i, line in enumerate(asm):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1)
        if line.strip() != "s_barrier":
            continue
        j = i + 1
        while j < len(asm) and (not asm[j].strip() or asm[j].strip().startswith((";", "s_waitcnt"))):
            j += 1
        if j < len(asm) and asm[j].strip() == "s_barrier":
            bad.append((fn, i + 1))
    assert not bad, "code sunk below a barrier in: %s" % bad


def _vgprs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]$", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def test_buffer_store_data_is_not_rewritten_at_once(asm):
    """A buffer store of 8 or 16 bytes keeps its data registers unchanged for
    at least three wait states after it issues.  A write to them right after
    the store once corrupted single stored values of the state planes (the
    compiler pads this only for buffer stores without a scalar offset
    register); every such store now goes through store_b64 / store_b128,
    which hold the data through an s_nop pad.  Counted: instructions after
    the store (an s_nop n counts n + 1) up to the first one that writes one
    of the data registers."""
    bad = []
    fn = None
    for i, line in enumerate(asm):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1)
        t = line.strip()
        m = re.match(r"buffer_store_dwordx(2|4)\s+(v\[\d+:\d+\]),", t)
        if not m:
            continue
        data = _vgprs(m.group(2))
        waits = 0
        for nxt in asm[i + 1:i + 12]:
            u = nxt.strip()
            if not u or u.startswith((";", ".")) or u.endswith(":"):
                continue
            if u.startswith("s_nop"):
                waits += int(re.findall(r"\d+", u)[0]) + 1
                continue
            dst = u.split(None, 1)[1].split(",")[0].strip() if " " in u else ""
            writes = u.startswith(("v_", "ds_read", "buffer_load", "global_load")) and _vgprs(dst) & data
            if writes and waits < 3:
                bad.append((fn, i + 1, t))
                break
            waits += 1
            if waits >= 3:
                break
    assert not bad, "store data rewritten within three wait states: %s" % bad[:5]
