"""MI355X-native decode attention over a KIVI-style asymmetric low-bit KV cache.

The compute path is the HIP library libkvq.so (C ABI in include/kvq.h); this
package only binds it.
"""
from ._lib import (Fp16Decode, KVCache, KVQConfig, KVQError, cache_bytes, group_bytes, load,  # noqa: F401
                   make_config, stream_read)
from ._lib import (KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_CAPACITY, KVQ_ERR_OOM, KVQ_ERR_HIP,  # noqa: F401
                   KVQ_ERR_NO_DEVICE, KVQ_ERR_EMPTY)
