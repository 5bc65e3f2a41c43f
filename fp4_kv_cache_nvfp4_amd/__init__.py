"""NVFP4 / MXFP4 KV-cache page quantization and paged FP4 decode attention
for AMD MI355X (gfx950)."""
