"""MI355X (gfx950) W8A8 ConvRot expert-choice MoE: HIP kernels behind a C ABI (include/convrot.h) and a thin
ctypes binding (``binding``).  ``synth`` holds the seeded synthetic input generators; ``build`` compiles the
library in-tree with hipcc."""
