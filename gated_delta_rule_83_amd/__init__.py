"""libgdn2: Gated DeltaNet-2 forward sequence mixing on MI355X (gfx950)."""
