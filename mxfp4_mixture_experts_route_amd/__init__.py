"""MI355X (gfx950) routed MXFP4 mixture-of-experts chain: HIP kernels behind a C ABI."""
