"""fp64 CPU oracle for the DART hot path -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
package; the HIP library never imports or calls it."""
from .dart_oracle import *  # noqa: F401,F403
from .dart_oracle import __all__  # noqa: F401
