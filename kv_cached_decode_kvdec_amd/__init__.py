"""kvdec: single-token KV-cached decode attention for AMD Instinct MI355X (gfx950)."""
