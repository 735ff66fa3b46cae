"""MI355X (gfx950) modal-SSM Hyena operator: prefill, decode step and filter
materialisation as hand-written HIP kernels behind a C ABI
(``include/hyena_modal.h``), with a ctypes binding.

Importing the package loads nothing; the library is loaded on first use and a
missing build raises :class:`binding.LibraryMissing`.
"""

from . import binding  # noqa: F401
from .binding import (HMError, LibraryMissing, ModalHyena, hm_desc, hyena_filter_materialize,  # noqa: F401
                      hyena_modal_decode_step, hyena_modal_prefill, hyena_modal_prefill_workspace,
                      make_desc)
