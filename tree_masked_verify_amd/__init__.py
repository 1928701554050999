"""Tree-masked speculative verify on MI355X (gfx950)."""
