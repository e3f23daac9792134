"""CPU float64 oracle for the windowed chunk-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the benchmark's GPU leg) may import, call or link anything in
this package; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path: the only common module is the
seeded input generator, which holds none of the method's arithmetic.

Citations name the UnStep paper (arXiv 2609.32518, "UnStep: Training-Free
Acceleration of Causal Video Diffusion with Fewer Steps Than Distillation"):
its abstract, figure captions and tables as the paper's web pages give them.

Parity status of each function (every one is pinned by a test that does not
restate its formula; see tests/test_oracle_pins.py):
  rope_table, rope_apply      pinned (norm, relative-position, identity,
                              closed-form angles, 2x2-matrix brute force)
  slot_of_frame, window_*     pinned (ring simulation, printed window counts)
  kv_append                   pinned (brute force, untouched slots)
  window_attn                 pinned (row sums, V=1, K=0 closed form, SDPA,
                              block-masked full causal attention, brute force)
  lowrank_proj                pinned (full rank = dense, Eckart-Young on the
                              factors, associativity, brute force)
  clip_schedule               pinned (forward counts printed in Table 3)
  shifted_sigma, dit_label    pinned (levels and labels printed in Table 4)
  flow_step, sample_chunk     pinned (forward counts printed in Table 3, the
                              level endpoints of Table 4, recovery of the
                              clean latent from exact velocities, scalar
                              brute force by another algebraic route)
  conv3d_causal               pinned (scalar brute force, delta kernels that
                              copy and shift the input in time and space,
                              causality, torch conv3d in fp64 on explicitly
                              padded input)
"""
from .ust_oracle import *  # noqa: F401,F403
