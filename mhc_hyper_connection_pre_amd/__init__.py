"""mHC (multi-stream hyper-connection) pre/post mixing for MI355X (gfx950)."""
