"""MI355X-native tiled scaled-dot-product attention forward (gfx950)."""
