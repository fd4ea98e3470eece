"""Stream-Factorized Attention (Hidden Decoding) on AMD Instinct MI355X (gfx950)."""
