"""Register, scratch and LDS budgets of the kernels for gfx950, read from the compiler's
resource-usage remarks (a device-only compile of each source; no GPU needed).

- No kernel keeps anything in scratch memory or spills vector registers.
- The kernels that stream the logits keep 8 waves per SIMD: the argmax sweep, its
  streaming-read probe, the shared router + sweep launch, the early-exit chain sweep and
  the entropy pass.  The shared launch's lean router tile must also stay small in LDS,
  so that LDS never holds the sweep's workgroups below that occupancy."""

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from drafter_routing_verification_amd import build

SOURCES = ["sweep.hip", "round.hip", "router.hip", "early_exit.hip", "entropy.hip",
           "finalize.hip", "catchup.hip"]
STREAMING = ("argmax_sweep_kernel", "stream_read_kernel", "router_mfma_sweep_kernel",
             "early_exit_sweep_kernel", "entropy_partial_kernel")
SHARED_LDS_MAX = 20 * 1024  # bytes: 8 workgroups of 4 waves in 160 KiB with room to spare


def _hipcc_available() -> bool:
    try:
        build.hipcc()
        return True
    except RuntimeError:
        return False


def _remarks(src: str, out: str) -> dict:
    cmd = build.command(out)
    base = cmd[:cmd.index("-o")]
    base = [a for a in base if a not in ("-shared", "-fPIC")]
    cmd = base + ["-c", os.path.join(build.CSRC, src), "--offload-device-only",
                  "-Rpass-analysis=kernel-resource-usage", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\S+) \[", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = m.group(2)
    return kernels


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if not _hipcc_available():
        pytest.skip("hipcc is not available")
    d = tmp_path_factory.mktemp("res")
    with ThreadPoolExecutor(max_workers=4) as pool:
        futures = {src: pool.submit(_remarks, src, str(d / (src + ".o"))) for src in SOURCES}
        return {src: f.result() for src, f in futures.items()}


def test_every_source_has_kernels(resources):
    for src, kernels in resources.items():
        assert kernels, f"no kernel remarks for {src}"


def test_no_scratch_and_no_vector_spills(resources):
    for src, kernels in resources.items():
        for name, r in kernels.items():
            assert r["ScratchSize [bytes/lane]"] == "0", f"{name} uses scratch"
            assert r["VGPRs Spill"] == "0", f"{name} spills vector registers"


def test_streaming_kernels_keep_full_occupancy(resources):
    seen = set()
    for kernels in resources.values():
        for name, r in kernels.items():
            for stem in STREAMING:
                if stem in name:
                    seen.add(stem)
                    assert r["Occupancy [waves/SIMD]"] == "8", f"{name}: {r}"
    assert seen == set(STREAMING)


def test_shared_router_launch_lds(resources):
    shared = {n: r for n, r in resources["round.hip"].items() if "router_mfma_sweep_kernel" in n}
    assert shared
    for name, r in shared.items():
        assert int(r["LDS Size [bytes/block]"]) <= SHARED_LDS_MAX, f"{name}: {r}"
