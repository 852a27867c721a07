"""CPU float64 oracle for the attention-KL path: test infrastructure only.

Imported by the tests, the smoke check and the bench's CPU-baseline leg; never by the
product path, and it shares no code with it.
"""
from .streamkl_oracle import (allowed_mask, backward, backward_head, forward,  # noqa: F401
                              forward_head, js_backward, js_backward_head, js_forward, js_forward_head)
