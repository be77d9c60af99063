"""TurboQuant hot path for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libtq.so (see include/tq.h); this
package holds its thin ctypes binding (`tq`) and seeded synthetic workloads
(`workloads`).
"""
