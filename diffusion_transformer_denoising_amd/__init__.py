"""MI355X (gfx950) DiT denoise step: hand-written HIP kernels behind a C ABI
(include/dit.h, libdit.so), a ctypes binding with the same names
(``binding``) and a torch-backed holder of device buffers (``model``).

Importing the package loads nothing; ``binding.lib()`` loads libdit.so and
raises if it is missing.
"""
