"""The build's assembly check for global->LDS loads whose scalar base address
was written by a vector instruction without the required wait states (CPU)."""
from causal_video_diffusion_amd.build import check_dma_base_hazards


def test_vector_written_base_is_flagged():
    asm = """
\tv_readfirstlane_b32 s1, v15
\tv_readfirstlane_b32 s0, v14
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v225, s[0:1]
\t;;#ASMEND
"""
    found = check_dma_base_hazards(asm)
    assert len(found) == 1 and "v_readfirstlane_b32 s0, v14" in found[0]


def test_scalar_written_base_and_enough_wait_states_pass():
    salu = """
\ts_add_u32 s4, s50, s4
\ts_mov_b32 m0, s6
\ts_addc_u32 s5, s51, s5
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v238, s[4:5]
\t;;#ASMEND
"""
    nops = """
\tv_readfirstlane_b32 s0, v14
\ts_nop 4
\tglobal_load_lds_dwordx4 v225, s[0:1]
"""
    far = "\tv_readlane_b32 s9, v253, 3\n" + "\ts_add_i32 s20, s20, 1\n" * 5 + \
          "\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    other = "\tv_readfirstlane_b32 s2, v4\n\tglobal_load_lds_dwordx4 v1, s[0:1]\n"
    for asm in (salu, nops, far, other):
        assert check_dma_base_hazards(asm) == []


def test_too_few_wait_states_and_block_boundaries_are_flagged():
    short = "\tv_readlane_b32 s9, v253, 3\n\ts_nop 2\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    assert len(check_dma_base_hazards(short)) == 1
    # another predecessor of the block could hold the write
    label = "\ts_mov_b32 s4, 0\n.LBB0_7:\n\tglobal_load_lds_dwordx4 v1, s[4:5]\n"
    assert len(check_dma_base_hazards(label)) == 1
