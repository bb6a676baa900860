"""MI355X (gfx950) grouped MLA latent-KV insert, context epilogue and chunked-context pack."""
