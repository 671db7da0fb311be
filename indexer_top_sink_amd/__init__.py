"""MI355X (gfx950) hot path of DeepSeek-V4.1 compressed sparse attention.

libv41.so (HIP kernels behind a C ABI, include/v41.h) does all the work;
`v41` is the ctypes binding with the same entry-point names and `layer`
chains the five calls into a decode step or a prefill chunk.
"""
