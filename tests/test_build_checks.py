"""Host-side checks of the build script: the scan of the compiler's
resource-usage remarks that fails the build when a kernel gets a scratch
frame or spills vector registers (a lambda left un-inlined once turned a
decode kernel's loads into calls with a stack frame, 9x slower)."""

from efficient_transformer_attention_amd import build as B

REMARKS = """\
x.hip:100:1: remark: Function Name: _ZN3cca7kernelAEv [-Rpass-analysis=kernel-resource-usage]
x.hip:100:1: remark:     VGPRs: 112 [-Rpass-analysis=kernel-resource-usage]
x.hip:100:1: remark:     ScratchSize [bytes/lane]: 560 [-Rpass-analysis=kernel-resource-usage]
x.hip:100:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:100:1: remark:     SGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:200:1: remark: Function Name: _ZN3cca7kernelBEv [-Rpass-analysis=kernel-resource-usage]
x.hip:200:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:200:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:200:1: remark:     SGPRs Spill: 49 [-Rpass-analysis=kernel-resource-usage]
x.hip:300:1: remark: Function Name: _ZN3cca15attn_fwd_kernelIDF16bDF16bLi128EEEvv [-Rpass-analysis=kernel-resource-usage]
x.hip:300:1: remark:     ScratchSize [bytes/lane]: 108 [-Rpass-analysis=kernel-resource-usage]
x.hip:300:1: remark:     VGPRs Spill: 26 [-Rpass-analysis=kernel-resource-usage]
x.hip:400:1: remark: Function Name: _ZN3cca15attn_fwd_kernelIDF16bDF16bLi64EEEvv [-Rpass-analysis=kernel-resource-usage]
x.hip:400:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:400:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_scan_flags_frames_and_vector_spills_only():
    bad = B._scratch_users(REMARKS)
    assert bad == ["_ZN3cca7kernelAEv: ScratchSize [bytes/lane] 560",
                   "_ZN3cca15attn_fwd_kernelIDF16bDF16bLi64EEEvv: VGPRs Spill 3"]


def test_scratch_scan_clean_input():
    assert B._scratch_users("") == []
    assert B._scratch_users(REMARKS.split("x.hip:300")[0].replace("560", "0")) == []
