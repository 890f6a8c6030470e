"""The build's occupancy guard: the compiler's per-kernel resource report is parsed and a hot kernel
that loses a wave per SIMD (or spills where it should not) fails the build."""
from selective_state_space_41_amd.build import check_resources, kernel_resources


def _report(name, vgprs, occ, scratch=0):
    loc = "vmscan.hip:1:1: remark: "
    return "\n".join([f"{loc}Function Name: {name} [-Rpass-analysis=kernel-resource-usage]",
                      f"{loc}    TotalSGPRs: 106 [-Rpass-analysis=kernel-resource-usage]",
                      f"{loc}    VGPRs: {vgprs} [-Rpass-analysis=kernel-resource-usage]",
                      f"{loc}    AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]",
                      f"{loc}    ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]",
                      f"{loc}    Occupancy [waves/SIMD]: {occ} [-Rpass-analysis=kernel-resource-usage]"])


WALK16 = "_ZN12_GLOBAL__N_115bwd_scan_kernelItLi0ELi1ELb0EEEvNS_7BwdArgsES1_"
WALK32 = "_ZN12_GLOBAL__N_115bwd_scan_kernelIfLi0ELi1ELb0EEEvNS_7BwdArgsES1_"
SCAN16 = "_ZN12_GLOBAL__N_116scan_pair_kernelItLi0ELi2EEEvNS_8ScanArgsE"


def test_parse():
    res = kernel_resources(_report(WALK16, 255, 2) + "\n" + _report(SCAN16, 124, 4))
    assert res[WALK16] == {"VGPRs": 255, "AGPRs": 0, "ScratchSize": 0, "Occupancy": 2}
    assert res[SCAN16]["Occupancy"] == 4


def test_floors():
    ok = kernel_resources(_report(WALK16, 255, 2) + "\n" + _report(WALK32, 256, 2, 28) + "\n" + _report(SCAN16, 124, 4))
    assert check_resources(ok) == []
    # the bf16 walk at 260 registers: one wave per SIMD, which the build must refuse
    lost = kernel_resources(_report(WALK16, 260, 1))
    assert len(check_resources(lost)) == 1 and "needs 2" in check_resources(lost)[0]
    assert check_resources(kernel_resources(_report(SCAN16, 172, 2)))
    # scratch: a few bytes only in the float32 walk
    assert check_resources(kernel_resources(_report(WALK16, 250, 2, 16)))
    assert check_resources(kernel_resources(_report(WALK32, 256, 2, 96)))
    # kernels off the hot path are not checked
    assert check_resources(kernel_resources(_report("_ZN12_GLOBAL__N_115transpose_kernelIfEEv", 200, 1, 8))) == []
