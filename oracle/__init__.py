"""Oracle package: plain fp64 CPU definitions used to check the HIP library.

Test infrastructure only: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the library itself.
"""
