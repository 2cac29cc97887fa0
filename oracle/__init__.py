"""CPU oracle of the CSA forward hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's cpu_baseline leg import this
package; the product path (the HIP library and its binding) never does.
"""
from .csa_oracle import *  # noqa: F401,F403
from .csa_oracle import _logsumexp  # noqa: F401
from .compressed_only import compressed_only_teacher  # noqa: F401
