"""CPU oracle for the Pingala-8 (format P8F v1) hot path.

Test infrastructure: imported only by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark, never by the product library."""
from . import p8f  # noqa: F401
