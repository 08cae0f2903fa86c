"""MI355X decode megakernel: host lowering to 64-byte task descriptors + a persistent
HIP interpreter kernel, behind the C ABI of include/mk.h (libmk.so)."""
from .binding import (EXPORTS, MK_SCHED_DYNAMIC, MK_SCHED_LEVELS, MK_SCHED_STATIC, Graph, Lowered, MkError, lib,  # noqa: F401
                      make_cfg, mk_abi_version, mk_build_graph, mk_last_error, mk_lower, mk_pack_matrix, mk_plan,
                      packed_matrix_indices)
