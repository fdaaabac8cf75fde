"""MI355X (gfx950) DSA lightning indexer -> top-k -> sparse MLA with cross-layer IndexShare."""
