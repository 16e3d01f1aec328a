"""MI355X (gfx950) dense matrix product C = A·B behind a small C ABI."""
