"""The build refuses kernels that spill registers to scratch memory (a spilling kernel runs
many times slower while every result stays right, so no parity test would notice)."""

import pytest

from bit_nf4_quantized_dq_amd import build as Bd

REMARKS = """\
x.hip:10:1: remark: Function Name: _ZN5qlora12_GLOBAL__N_19k_gemm_ntILb1ELb1EEEvPKtlS3_llS3_llS3_iPtPfj [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 5868 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: _ZN5qlora12_GLOBAL__N_111k_gemv_rowsILi8EEEvNS0_8RowsArgsENS_3LutE [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs: 157 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_remarks_are_parsed():
    res = Bd._kernel_resources(REMARKS)
    assert [(Bd._short(n), v, s) for n, v, s in res] == [("k_gemm_nt", 256, 5868), ("k_gemv_rows", 157, 0)]


@pytest.mark.parametrize("mangled,name", [
    ("_ZN5qlora12_GLOBAL__N_19k_gemm_dxEPKjPKhPKfS6_llPKtlS8_S8_iPtNS_9Nf4TablesE", "k_gemm_dx"),
    ("_ZN5qlora12_GLOBAL__N_111k_sum_partsEPKfillPt", "k_sum_parts"),
    ("_ZN5qlora12_GLOBAL__N_113k_quant_pass1ILb0EEEvPKvPjPfPyPilNS_9Nf4TablesE", "k_quant_pass1"),
])
def test_kernel_names_from_mangled_symbols(mangled, name):
    assert Bd._short(mangled) == name


def test_every_built_kernel_is_within_its_scratch_allowance():
    """The resource reports the last build wrote: no kernel beyond its allowance."""
    import glob
    import os

    reports = glob.glob(os.path.join(Bd.BUILD_DIR, "*.resources.txt"))
    if not reports:
        pytest.skip("no build in this tree")
    for path in reports:
        for line in open(path):
            name, _, scratch = line.split()
            assert int(scratch.split("=")[1]) <= Bd.SCRATCH_ALLOWANCE.get(Bd._short(name), 0), (path, line)
