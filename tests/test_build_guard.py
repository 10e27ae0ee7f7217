"""The build's guard against spill code inside the attention kernel's MFMA
blocks (host-side text check of the compiler's assembly)."""
import pytest

from mla_latent_kv_15_amd import build

KERNEL = build.HOT_KERNELS["k_attn_v2.hip"]


def _asm(body):
    return "\n".join([f"_Z{KERNEL}v:                 ; @_Z{KERNEL}v", *body, ".Lfunc_end0:"])


CLEAN = [
    "\tscratch_store_dword off, v5, off offset:12 ; 4-byte Folded Spill",
    ".LBB0_1:                    ;   in Loop: Header=BB0_1 Depth=1",
    "\tds_read_b128 v[190:193], v148",
    "\tv_mfma_f32_32x32x16_bf16 v[2:17], v[190:193], v[18:21], 0",
    "\ts_cbranch_scc1 .LBB0_1",
    ".LBB0_2:",
    "\tscratch_load_dword v6, off, off offset:12 ; 4-byte Folded Reload",
    "\ts_endpgm",
]


def test_spills_outside_mfma_blocks_pass():
    build._check_hot_blocks("k_attn_v2.hip", _asm(CLEAN))


def test_direct_to_lds_loads_are_not_spills():
    body = list(CLEAN)
    body.insert(3, "\tbuffer_load_dwordx4 v184, s[20:23], s61 offen lds")
    build._check_hot_blocks("k_attn_v2.hip", _asm(body))


@pytest.mark.parametrize("spill", [
    "\tscratch_load_dword v6, off, off offset:12 ; 4-byte Folded Reload",
    "\tbuffer_store_dword v6, off, s[0:3], 0 offset:12 ; 4-byte Folded Spill",
    "\tv_accvgpr_read_b32 v2, a240",
    "\tv_accvgpr_write_b32 a3, v7",
])
def test_spill_inside_an_mfma_block_fails(spill):
    body = list(CLEAN)
    body.insert(3, spill)
    with pytest.raises(RuntimeError, match="spill code in MFMA blocks"):
        build._check_hot_blocks("k_attn_v2.hip", _asm(body))


def test_scratch_cap():
    remarks = (f"remark: x.hip:1:0: Function Name: _Z{KERNEL}v\n"
               f"remark: x.hip:1:0:     ScratchSize [bytes/lane]: {build.MAX_SCRATCH + 4}\n")
    with pytest.raises(RuntimeError, match="scratch"):
        build._check_scratch("k_attn_v2.hip", remarks)
    build._check_scratch("k_attn_v2.hip", remarks.replace(str(build.MAX_SCRATCH + 4), "24"))


def test_no_scratch_kernels_reject_any_spill():
    from mla_latent_kv_15_amd import build
    ok = ("remark: Function Name: _ZN3mla12_GLOBAL__N_117combine_v2_kernelEv\n"
          "remark:     ScratchSize [bytes/lane]: 0\n")
    build._check_scratch("/x/k_attn_v2.hip", ok)
    bad = ok.replace("ScratchSize [bytes/lane]: 0", "ScratchSize [bytes/lane]: 16")
    with pytest.raises(RuntimeError):
        build._check_scratch("/x/k_attn_v2.hip", bad)
    # the attention kernel keeps its own cap
    hot = ("remark: Function Name: _ZN3mla12_GLOBAL__N_114attn_v2_kernelEv\n"
           "remark:     ScratchSize [bytes/lane]: 64\n")
    build._check_scratch("/x/k_attn_v2.hip", hot)
    with pytest.raises(RuntimeError):
        build._check_scratch("/x/k_attn_v2.hip", hot.replace(": 64", ": 4096"))


def _span_asm(body, name="_ZN3mla12_GLOBAL__N_112wgemm_kernelILi5ELi32ELi4ELb1ELb1EEEv"):
    return "\n".join([f"{name}:", *body, "\ts_endpgm", ".Lfunc_end1:"])


SPAN_CLEAN = [
    "\tv_accvgpr_write_b32 a0, 0",
    "\tv_accvgpr_mov_b32 a1, a0",
    "\tglobal_load_dwordx4 v[8:11], v[2:3], off",
    "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
    "\tglobal_load_dwordx4 v[8:11], v[2:3], off offset:1024",
    "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
    "\ts_nop 7",
    "\tv_accvgpr_read_b32 v12, a0",
]


def test_mfma_span_allows_copies_outside_the_chain():
    build._check_mfma_spans("k_gemm_v2.hip", _span_asm(SPAN_CLEAN))


@pytest.mark.parametrize("copy", [
    "\tv_accvgpr_read_b32 v152, a214",      # a VGPR restored from a spill AGPR
    "\tv_accvgpr_write_b32 a187, v103",     # a VGPR spilled into an AGPR
    "\tv_accvgpr_mov_b32 a40, a0",
    "\tscratch_load_dword v6, off, off offset:12",
])
def test_mfma_span_rejects_copies_inside_the_chain(copy):
    body = list(SPAN_CLEAN)
    body.insert(4, copy)
    with pytest.raises(RuntimeError, match="register copies between inline-asm MFMAs"):
        build._check_mfma_spans("k_gemm_v2.hip", _span_asm(body))


def test_mfma_span_needs_the_kernel():
    with pytest.raises(RuntimeError, match="found in the assembly"):
        build._check_mfma_spans("k_gemm_v2.hip", _span_asm(SPAN_CLEAN, name="_Z5otherv"))
