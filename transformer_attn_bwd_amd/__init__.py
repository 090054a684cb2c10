"""MI355X (gfx950) attention backward: HIP kernels behind a C ABI."""
