"""MI355X-native (gfx950) windowed chunk attention for causal video diffusion.

The per-chunk DiT self-attention path of UnStep (arXiv 2609.32518): 3-D RoPE
from a precomputed cos/sin table, KV append into a frame-slot ring, chunk-causal
attention over a limited temporal window, and truncated-SVD value/output
projections, as the C-ABI library libust.so (include/ust.h) over hand-written
HIP kernels.  `_binding` exposes the C entry points under the same names;
`path` holds the device drivers; `workload` the seeded synthetic inputs.
"""
from ._binding import (UstError, Geom, Kv, geom, kv, load, ust_v_row_len,  # noqa: F401
                       ust_rope_table_build, ust_kv_append, ust_window_attn,
                       ust_lowrank_proj, ust_slot_of_frame, ust_window_plan,
                       ust_window_attn_split, ust_window_attn_work_bytes,
                       ust_qkv_append, ust_flow_step, ust_sigma_schedule)
