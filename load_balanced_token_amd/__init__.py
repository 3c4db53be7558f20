"""MI355X-native load-balanced MoE token path: router top-K, load histogram,
online S*K balancing plan (or a quota plan with a searched threshold), block-aligned sort, zero-copy dispatch, combine.

The compute lives in liblbt.so (HIP, gfx950) behind include/lbt.h; this
package only marshals arguments.  Importing it does not load the library;
the first call does, and fails loudly if it has not been built.
"""
from .binding import (Shape, Path, query_sizes, plan_fields, lib, LbtError,  # noqa: F401
                      SOFTMAX, SIGMOID, Y_F32, Y_BF16, ST_BADCOUNT, ST_CAPACITY, ST_BADID,
                      ST_DUPID, EXPORTS, LIB_PATH)
