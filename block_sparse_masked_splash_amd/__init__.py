"""Block-sparse masked ("Splash") attention forward for AMD MI355X (gfx950)."""
