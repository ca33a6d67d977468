"""Plain, slow CPU oracle for the E8 projection / core-escape encoding path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``bit_e8_lattice_amd`` and its HIP kernels) never imports, links or calls it,
and the oracle shares no code, table or constant generator with the product.

Citation keys used throughout the oracle:

* **E8-QAT** -- the web page "E8-QAT: Efficient 2-Bit Quantization-Aware Training
  with Implicit Lattice Codebooks" (abstract, captions of Figures 1, 2 and 6,
  appendix Tables 3, 4, 9 and 10).
* **SPLAG** -- Conway & Sloane, *Sphere Packings, Lattices and Groups*, ch. 4
  sec. 8.1 (E8 = D8 u (D8 + 1/2)), ch. 20 (nearest-point decoders for D_n and E8).
* **CS82** -- Conway & Sloane, "Fast quantizing and decoding algorithms for
  lattice quantizers and codes", IEEE Trans. Inf. Theory 28 (1982).

Every function says which passage it follows.  Where the pages leave a step
open, the reading taken is stated next to the code (tie rules, scale, core,
record layout).

Parity status: every function here is pinned by an independent check in
``tests/test_oracle_*.py`` (brute force, closed forms, textbook counts, values
printed in the E8-QAT tables), except the items listed as "parity unpinned" in
the module docstrings: the tie-break choices, the core ordering and the escape
record field layout are conventions with no printed example to pin them to.
"""

from .lattice import (  # noqa: F401
    nearest_e8_two_z,
    is_e8_two_z,
)
from .hadamard import kappa, fwht_blocks, sylvester_matrix  # noqa: F401
from .core import (  # noqa: F401
    core_points,
    core_size,
    core_rank,
    core_unrank,
    ESCAPE_SLOT,
)
from .pipeline import (  # noqa: F401
    STATUS_NONFINITE,
    STATUS_BAD_SCALE,
    STATUS_INT8_RANGE,
    STATUS_ESC_OVERFLOW,
    STATUS_X_RANGE,
    STATUS_BAD_INDEX,
    STATUS_ESC_MISSING,
    X_LIMIT,
    ESCAPE_RECORD_DTYPE,
    bf16_to_f32,
    f32_to_bf16,
    row_coefficients,
    normalized_groups,
    project,
    encode_core_escape,
    decode_core_escape,
    dequantize,
    ste_backward,
    sgd_update,
    escape_fraction,
    payload_bits,
    rms_scale,
)
from .restore import (  # noqa: F401
    restore_coefficients,
    restore_original,
    project_restore,
    rotate_grad,
    ste_backward_hadamard,
)
from .decode import decode_outputs  # noqa: F401
from .gemv import exact_restored, gemv_reference, rotated_bound, rotated_magnitude  # noqa: F401
from .roots import (  # noqa: F401
    e8_roots,
    pack_escapes,
    unpack_escapes,
    PACKED_RECORD_DTYPE,
    ROOT_NONE,
)
from .ptq import core_search_two_z, core_project_two_z, exact_row_errors, ptq_init  # noqa: F401
from .brute import brute_nearest_e8  # noqa: F401
