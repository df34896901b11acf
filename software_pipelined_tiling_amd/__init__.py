"""software_pipelined_tiling_amd -- software-pipelined tiled GEMM for MI355X (gfx950)."""
