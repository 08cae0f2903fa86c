"""MI355X decode megakernel: host lowering to 64-byte task descriptors + a persistent
HIP interpreter kernel, behind the C ABI of include/mk.h (libmk.so)."""
from .binding import (EXPORTS, Graph, Lowered, MkError, lib, make_cfg, mk_abi_version,  # noqa: F401
                      mk_build_graph, mk_last_error, mk_lower, mk_plan)
