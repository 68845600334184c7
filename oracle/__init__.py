"""CPU oracle of the folded verify layer -- test infrastructure only.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg import this
package.  The HIP library neither imports nor links anything from it."""
from .specfold_oracle import *  # noqa: F401,F403
