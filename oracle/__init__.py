"""CPU oracle of the BitLinear (W1.58A8) forward: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""

from .bitlinear_ref import (  # noqa: F401
    EPS_A,
    EPS_W,
    QB,
    absmean_gamma,
    contract,
    forward,
    pack_ternary,
    pack_weights,
    quant_act,
    rescale,
    ternarize,
    widen_bf16,
)
from .subln_ref import (  # noqa: F401
    EPS_N,
    normalise,
    rms_factor,
    subln_plain,
    subln_quant_act,
    sum_squares,
)
from .ffn_ref import (  # noqa: F401
    a3_f32,
    bf16_rne,
    gated_relu2,
    gated_relu2_plain,
)
from .binary_ref import (  # noqa: F401
    binarize,
    forward_binary,
    pack_binary,
    pack_weights_binary,
)
