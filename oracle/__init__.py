"""CPU oracle for multi-stream hyper-connection (mHC) pre/post mixing.

This package is TEST INFRASTRUCTURE. It is a plain, slow, float64 statement of
what the mHC boundary computes, used only to check the HIP implementation:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (the C-ABI library and its Python
binding) never imports, links or calls anything here, and nothing here imports
the product path.

Modules
-------
``mhc_oracle``  numpy float64, vectorised over tokens (the definition).
``brute``       the same definition as pure-Python scalar loops over ``math``,
                for tiny shapes only; it pins the vectorised oracle.

Parity status of every function is stated in its docstring. The conventions
the pages leave open (fn row/column order, gate function, Sinkhorn positivity
map and step counting, combine weights, rounding points) are readings, marked
"Reading:" where they are applied; the pages cannot pin them, so the tests pin
only their self-consistency and the mathematics around them.
"""

from .mhc_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    f64_to_f32,
    decode,
    pre_logits,
    gates,
    sinkhorn,
    stream_reduce,
    post_mix,
    mhc_pre,
    mhc_post,
    mhc_post_combine_norm,
    rms_norm,
)
