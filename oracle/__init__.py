"""The float64 CPU oracle: test infrastructure, never part of the product path.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.
"""
from .attention import attention_ref, attention_rows_ref, materialised_rows_ref  # noqa: F401
from .backward import (attention_backward_ref, backward_key_rows_ref,  # noqa: F401
                       backward_query_rows_ref, row_terms_ref)
