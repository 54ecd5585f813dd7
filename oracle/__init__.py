"""fp64 CPU oracle for exact attention, forward and backward.  Test infrastructure only: the
product path never imports it (see oracle/attention.py and oracle/attention_bwd.py for what
they compute and where that is defined)."""

from .attention import (attention_dense, attention_head, attention_rows_dense,  # noqa: F401
                        attention_rows_varlen, attention_varlen, flops_dense, visibility,
                        visible_pairs)
from .attention_bwd import (attention_backward_dense, attention_backward_varlen,  # noqa: F401
                            attention_head_backward, flops_backward_dense)
