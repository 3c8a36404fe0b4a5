"""CPU oracle for the ViT encoder forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  The GPU library never calls it and shares no code with it.
"""

from . import head_oracle, quant_oracle, vit_oracle  # noqa: F401
