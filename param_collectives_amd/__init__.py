"""Layout-aware FSDP2 collective local stages on MI355X (gfx950).

  Plan                   host shard-layout plan (dimension-0 shards, padding)
  reduce_scatter_local   W ranks' bf16 (or fp32) gradients -> W packed fp32
                         shards (with Equation 5's alpha and accumulate)
  reduce_scatter_local_noalloc
                         the same from bf16 gradients, allocating nothing
                         (tables in a fixed device scratch array)
  allgather_copyout      rank-major bf16 buffer -> per-parameter tensors
  allgather_copyin       every rank's fp32/bf16 shards -> rank-major bf16 buffer
  stock_chunk_cat        stock FSDP2's gradient pack of one rank (the baseline)
  probe, victim_axpb, Stream
                         interference instruments: hardware-ID probe,
                         elementwise victim, CU-masked streams

The *_call variants check and marshal the tensors once and return a callable
that launches with one library call (for buffers reused every step).

The work runs in the HIP library libtide.so (include/tide.h); importing this
package fails if that library has not been built.
"""
from .tide import (  # noqa: F401
    FLAG_CACHED_LOADS,
    FLAG_CACHED_STORES,
    FLAG_NO_LDS,
    MAX_WORLD,
    Plan,
    DTYPE_BF16,
    DTYPE_F32,
    TideError,
    allgather_copyin,
    allgather_copyin_call,
    allgather_copyout,
    allgather_copyout_call,
    reduce_scatter_call,
    reduce_scatter_local,
    reduce_scatter_local_noalloc,
    stock_chunk_cat,
    stock_chunk_cat_call,
    Stream,
    decode_probe,
    device_info,
    probe,
    victim_axpb,
)
