"""CPU oracle for paged decode attention, the cache scatter, the block copy and
the block manager.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports, links or calls it, and it shares no code with the library: it is a
plain, slow, obviously correct restatement of what the pages define, in fp64
for floating point.

What it follows (page, section):
* "What is PagedAttention" (tecyfy), "How it works": per-request fixed-size
  blocks, handed out as the sequence grows, located through a table, and an
  attention that reads keys and values from those scattered blocks.
* "PagedAttention" (lastdictionary): blocks of e.g. 16 tokens; a per-sequence
  block table translates token positions to physical blocks; the attention
  kernel reads keys and values through it; blocks are shared copy-on-write.
* systemdesign.academy glossary "Paged Attention": the kernel reads the same
  numbers through the table, so the model computes the same thing.
* chipfoundryservices glossary "pagedattention vllm", "Attention Computation"
  (Block-Wise Attention, Address Translation), "Copy-on-Write Sharing"
  (Reference Counting, Divergence Handling), "Memory Management" (Block
  Allocation), "Implementation Details" (Metadata Overhead: 4-byte table
  entries), "Advanced Features" (Sliding Window) and "Comparison with
  Alternatives" (vs Compression: an 8-bit E4M3 cache with per-tensor scales).

Every function here is pinned by tests that do not re-type its formula:
torch's scaled-dot-product attention on independently laid-out data, closed
forms, exact invariances under block placement, block size, batch order and
copy-on-write, exhaustive format decoding, and the pages' worked numbers.
No function is "parity unpinned".
"""
from .formats import E4M3_MAX, decode, decode_e4m3, quantize_e4m3
from .attention import gather_sequence, paged_attention_decode
from .cache_ops import copy_blocks, reshape_and_cache, reshape_and_cache_fp8, swap_blocks
from .block_manager import BlockManager, NoFreeBlocks, BlockManagerError

__all__ = [
    "E4M3_MAX", "decode", "decode_e4m3", "quantize_e4m3", "reshape_and_cache_fp8", "swap_blocks",
    "decode", "gather_sequence", "paged_attention_decode", "copy_blocks", "reshape_and_cache",
    "BlockManager", "NoFreeBlocks", "BlockManagerError",
]
