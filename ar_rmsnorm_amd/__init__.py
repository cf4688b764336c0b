"""MI355X-native per-GPU reduction of a custom all-reduce (gfx950, HIP)."""
