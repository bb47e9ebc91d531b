"""MI355X (gfx950) chunkwise-parallel gated delta rule forward pass."""
