"""MI355X (gfx950) fused causal-conv1d + KDA multi-token verify-decode step."""
