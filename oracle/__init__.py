"""fp64 CPU oracle for exact attention forward.  Test infrastructure only: the product path
never imports it (see oracle/attention.py for what it computes and where that is defined)."""

from .attention import (attention_dense, attention_head, attention_rows_dense,  # noqa: F401
                        attention_rows_varlen, attention_varlen, flops_dense, visibility,
                        visible_pairs)
