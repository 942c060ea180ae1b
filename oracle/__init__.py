"""Float64 CPU oracle for the ZeroS forward pass. Test infrastructure only: the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; the library never does."""
from . import zeros_ref  # noqa: F401
