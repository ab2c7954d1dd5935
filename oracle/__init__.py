"""CPU oracle for the BitDelta fused multi-tenant linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct CPU
statement of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product library (``tenant_linear_layers_amd``) never imports,
calls or links it, and this package imports nothing from the product.

Source of the method: the page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli
sunmak" (hanzo.blog, 2026-02-28) and its Spanish translation "BitDelta: cómo
servir 14 modelos Zen desde un solo cluster de GPU" (hanzo-blog.hanzo.app).
Citations name the section of that page ("Matematiksel temel" = mathematical
foundation, "Sunum mimarisi" = serving architecture, "Altyapı ayrıntıları" =
infrastructure details) and the equation or figure in it.

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (the arithmetic) or ``tests/test_cache_policy.py``
(the delta-cache policy of ``cache_policy``) against something other than
itself (closed forms, textbook routines, brute force, hand-built cases).  No
function is "parity unpinned".
"""

from .bitdelta_oracle import (  # noqa: F401
    ABS_LIMIT,
    F32_NAN_BITS,
    Q_FRACTION_BITS,
    alpha_from_delta,
    bf16_bits_to_f32,
    compress,
    delta_f32,
    f32_to_bf16_bits,
    fixed_point_scope_sums,
    linear,
    linear_by_element,
    linear_multi,
    pack_sign_bits,
    reconstruct,
    rne_ratio_to_f32_bits,
    sign_bits,
    unpack_sign_bits,
)
