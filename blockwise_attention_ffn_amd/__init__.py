"""MI355X (gfx950) BPT layer forward: Python binding over the C-ABI library."""
