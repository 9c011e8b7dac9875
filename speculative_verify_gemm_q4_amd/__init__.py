"""Skinny-M Q4 verify GEMM for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/q4verify.h``: argument
marshalling and shape/dtype/device checks only.  Every step of the
computation runs in the HIP kernels of ``libq4verify.so``; if that library
has not been built, importing the functions raises instead of falling back
to anything else.

Functions (same names as the C entry points):

* :func:`q4_pack_layout` -- byte layout of a packed N x K matrix (host only).
* :func:`q4_gemm_verify` -- y[M, N] = x[M, K] @ W^T for Q4 W, fp32 out.
* :func:`q4_repack` -- one-time reorder into the tiled layout.
* :func:`q4_gemm_verify_tiled` -- the same product on tiled weights.
* :func:`q4_gemm_verify_tiled_dot` -- the tiled product for M <= 4 on the
  vector ALU (v_dot2) instead of MFMA.
* :func:`q4_gemm_verify_tiled_ws` -- the tiled product with a workspace
  (K split across workgroups for K > 5120); :func:`workspace_for` sizes it.
* :func:`q4_gemm_verify_tiled_noalloc` -- the workspace product with the
  library's static device scratch instead: allocates nothing.
* :func:`q4_gemm_verify_plan`, :func:`q4_gemm_verify_tiled_ws_plan` -- launch
  plans of a shape.
* :func:`q4_verify_sample` (:func:`verify_sample` allocates its outputs) --
  the verify sampling epilogue over the LM head's logits: top-k candidates,
  target probabilities, the accept test and the residual draw.
* :func:`q4_gemm_verify_sample` (:func:`gemm_verify_sample` allocates its
  outputs) -- the LM-head product with that epilogue fused in: the logits
  never leave the chip.
* :func:`q4_gdn_commit` -- writes a verify pass's accepted tree nodes into
  the Gated DeltaNet recurrent states of every layer (gated delta rule).
* :func:`q4_gdn_tree_out` -- every tree node's output of one recurrent layer
  from the shared state plus the updates along its path.
* :func:`q4_tree_attn`, :func:`tree_attn` -- tree-verify attention of one
  layer over the paged int8 KV cache with the ancestor mask.
* :func:`q4_dequant` -- fp32 weights of a packed matrix (test hook).
* :func:`q4_stream_read`, :func:`q4_stream_copy` -- bandwidth probes.
* :func:`q4_status_string` -- name of a status code.
"""
from ._lib import (ESCRATCH, ATTN_HEAD_DIM, ATTN_MAX_NODES, ATTN_PAGE, GDN_DK, GDN_MAX_NODES, GROUP, KERNEL_PLANAR, KERNEL_TILED_KSLICE,
                   KERNEL_TILED_RESIDENT,
                   KERNEL_TILED_STREAM, LAYOUT_PLANAR, LAYOUT_TILED16, MAX_ROWS,
                   MAX_ROWS_TILED, Q4Error,
                   LIB_PATH, lib_exports, load, q4_dequant, q4_gemm_verify,
                   q4_gemm_verify_plan, q4_gemm_verify_tiled,
                   q4_gemm_verify_tiled_dot,
                   q4_gemm_verify_tiled_ws, q4_gemm_verify_tiled_ws_plan,
                   q4_gemm_verify_tiled_noalloc, NOALLOC_SCRATCH_BYTES,
                   q4_gdn_commit, q4_gdn_tree_out, q4_pack_layout, q4_verify_sample,
                   q4_gemm_verify_sample, q4_gemm_verify_sample_workspace,
                   gemm_verify_sample,
                   q4_verify_sample_workspace, verify_sample,
                   workspace_for,
                   q4_repack, q4_status_string, q4_stream_copy,
                   q4_stream_read, q4_tree_attn, q4_tree_attn_plan,
                   tree_attn)

__all__ = ["ESCRATCH", "ATTN_HEAD_DIM", "ATTN_MAX_NODES", "ATTN_PAGE", "GDN_DK", "GDN_MAX_NODES", "GROUP", "KERNEL_PLANAR", "KERNEL_TILED_KSLICE",
           "KERNEL_TILED_RESIDENT",
           "KERNEL_TILED_STREAM", "LAYOUT_PLANAR", "LAYOUT_TILED16", "MAX_ROWS",
           "MAX_ROWS_TILED", "Q4Error",
           "LIB_PATH", "lib_exports", "load", "q4_dequant", "q4_gemm_verify",
           "q4_gemm_verify_plan", "q4_gemm_verify_tiled",
           "q4_gemm_verify_tiled_ws", "q4_gemm_verify_tiled_ws_plan",
           "q4_gemm_verify_tiled_noalloc", "NOALLOC_SCRATCH_BYTES",
           "q4_gdn_commit", "q4_gdn_tree_out", "q4_pack_layout", "q4_verify_sample",
           "q4_gemm_verify_sample", "q4_gemm_verify_sample_workspace",
           "gemm_verify_sample",
           "q4_verify_sample_workspace", "verify_sample", "workspace_for",
           "q4_repack", "q4_status_string", "q4_stream_copy",
           "q4_stream_read", "q4_tree_attn", "q4_tree_attn_plan", "tree_attn"]
