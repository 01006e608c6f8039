"""CPU oracle for the SVDQuant W4A4 linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the layer computes,
written from the Diffusers "Nunchaku Lite" documentation ("Supported quantization
types" table, "NunchakuLiteQuantizationConfig" section) and the plain readings
recorded beside each function.  Floating point that decides an integer is done in
the precision the definition states; everything else is float64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library shares no code with it.

Modules
    formats  bf16 / E4M3 / E2M1 encodings and nibble packing
    quant    activation quantizers (int4 group 64, NVFP4 group 16) and the
             low-rank down projection
    linear   the W4A4 linear (int4, NVFP4), the AWQ W4A16 linear, brute force
    prep     offline weight preparation (smoothing, low-rank split, residual
             quantization, AWQ weights) -- the step before the layer runs

Parity status: every function is pinned by ``tests/test_oracle_*.py`` except
``quant``/``linear`` *method quality* (how much error SVDQuant removes), for which
the pages give no number: that sanity check is marked "parity unpinned".
"""

from . import formats, quant, linear, prep  # noqa: F401
