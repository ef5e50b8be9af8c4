"""Every kernel keeps its values in registers: no scratch memory and no spilled
vector registers; the matrix-core kernels also keep the occupancy they are tiled
for (two wavefronts per SIMD).  Checked on the compiler's resource report, so it
runs on the CPU; a spill turns into scratch traffic (and, before a reload, a
wait for every load in flight) in the kernels' loops.
"""

import pytest

from exact_blockwise_attention_attn_amd import build

# Kernel name fragments of the bf16 MFMA kernels (each instantiated for head_dim 64 and 128).
MFMA_KERNELS = [
    "fwd_bf16_kernel", "fwd_chunks_kernel", "fwd_varlen_kernel", "tree_fwd_kernel",
    "dkdv_bf16_kernel", "dkdv_chunks_kernel", "dkdv_varlen_kernel",
    "dq_bf16_kernel", "dq_chunks_kernel", "dq_varlen_kernel",
    "decode_split_kernel", "decode_streamk_kernel",
]


@pytest.fixture(scope="module")
def usage():
    return build.resource_usage()


def _find(usage, frag, d):
    hits = [(k, v) for k, v in usage.items() if frag in k and f"ILi{d}E" in k]
    assert len(hits) == 1, f"{frag}<{d}>: {len(hits)} matches"
    return hits[0][1]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("frag", MFMA_KERNELS)
def test_no_scratch_no_spill(usage, frag, d):
    r = _find(usage, frag, d)
    assert r["ScratchSize"] == 0, f"{frag}<{d}> uses {r['ScratchSize']} B/lane of scratch"
    assert r["VGPRs Spill"] == 0, f"{frag}<{d}> spills {r['VGPRs Spill']} VGPRs"
    assert r["Occupancy"] >= 2, f"{frag}<{d}> occupancy {r['Occupancy']} waves/SIMD"


def test_every_kernel_keeps_its_values_in_registers(usage):
    """No kernel of the library (the fp32, statistics, merge, decode-tree, decode-merge and
    non-finite-scan kernels as well) uses scratch memory or spills vector registers."""
    kernels = {k: v for k, v in usage.items() if "_kernel" in k}
    assert len(kernels) >= 42, sorted(kernels)
    bad = {k: (v["ScratchSize"], v["VGPRs Spill"]) for k, v in kernels.items()
           if v["ScratchSize"] != 0 or v["VGPRs Spill"] != 0}
    assert not bad, bad
