"""FP64 CPU oracle for streaming (online-softmax) attention (forward and
backward) and row softmax.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
load anything from this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
constants or helpers with the HIP library under
``online_softmax_streaming_amd/``, and it imports nothing from there.

Sources (three web pages on one subject):
  * "Intermediate and advanced kernel workshops" (the workshops page):
    section "Scope and contracts" -- the streaming_attention and
    split_softmax contracts; the I2 softmax-backward workshop.
  * "Compare reasoning after your own attempt" (the answer-key page):
    the I2 / A1 / A2 / A3 rows of its table, "Worked answers worth memorizing
    by derivation" (I2 VJP, A1 merge, A2 scratch size, A3 six/seven) and the
    closing note that the attention oracle materialises FP64 scores.
  * "Kernel Notes & Checklist": section 4, "The gotchas ledger" (-inf padding
    before a max, 0 before a sum, ghost rows pinned so they cannot give NaN).

Every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_softmax_oracle_pins.py`` and ``tests/test_backward_oracle_pins.py``
against values the pages print, closed forms, invariants, library routines,
finite differences and 50-digit brute force.
"""

from .attention import (  # noqa: F401
    EMPTY_STATE,
    attention,
    attention_rows,
    merge_state_of,
    online_merge,
    streaming_model,
    visible_mask,
)
from .softmax import (  # noqa: F401
    num_chunks,
    scratch_bytes,
    softmax_rows,
    split_softmax_model,
)
from .paged import attention_paged, gather_pages  # noqa: F401
from .varlen import attention_varlen  # noqa: F401
from .dropout import attention_dropout, keep_mask, philox4x64, threshold  # noqa: F401
from .attention_backward import (  # noqa: F401
    attention_backward,
    attention_backward_head,
    probabilities,
    softmax_vjp,
)
