"""Paged KV pool addressing and the plain ``kv_write`` scatter (oracle; test
infrastructure).

What the pages fix:
  * "nano-vLLM learning note", ``ModelRunner.prepare_decode`` block: the slot
    of the token being decoded is ``block_table[-1] * block_size +
    last_block_num_tokens - 1`` -- a slot is ``page * page_size + offset``.
  * same page, ``store_kvcache_kernel`` block: one program per new token
    loads its key/value row (``num_kv_heads * head_dim`` elements at
    ``idx * stride``) and stores it at the slot; a slot of -1 means "do not
    store".
  * same page, ``Sequence`` block (``num_blocks``): a request of L tokens
    occupies ceil(L / block_size) pages.

Pool layout (the library header states the same layout in prose; this module
restates it independently): K and V live in two separate pools, each indexed
``[page][kv_head][offset][dim]``, i.e. element (slot s, head g, dim d) sits at
flat index ``((s // P * Hkv + g) * P + s % P) * D + d``.

The write is a copy, so the oracle moves raw element bits (uint16 for bf16,
uint32 for fp32) and is bit-exact by construction.
"""

import numpy as np


def pool_view(pool, num_pages, num_kv_heads, page_size, head_dim):
    """Reshape a flat raw-bits pool into [page][kv_head][offset][dim]."""
    return np.asarray(pool).reshape(num_pages, num_kv_heads, page_size, head_dim)


def slot_to_page_offset(slot, page_size):
    """A slot names (physical page, offset within the page)."""
    return slot // page_size, slot % page_size


def logical_slot(block_table_row, j, page_size):
    """Slot of logical token j of a request: its page from the block table,
    then the offset inside the page."""
    return int(block_table_row[j // page_size]) * page_size + j % page_size


def kv_write(k_pool, v_pool, k_rows, v_rows, slot_mapping, page_size):
    """Scatter new K/V rows into the pools (in place).

    k_pool, v_pool : raw bits, shape [num_pages][Hkv][P][D]
    k_rows, v_rows : raw bits, shape [T][Hkv][D] (token t's row)
    slot_mapping   : [T] int; -1 = skip this token
    """
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        page, off = slot_to_page_offset(slot, page_size)
        k_pool[page, :, off, :] = k_rows[t]
        v_pool[page, :, off, :] = v_rows[t]


def gather_request(pool, block_table_row, length, page_size):
    """Logical rows 0..length-1 of one request, read through its block
    table: returns raw bits [length][Hkv][D]."""
    rows = []
    for j in range(length):
        page = int(block_table_row[j // page_size])
        rows.append(pool[page, :, j % page_size, :])
    if not rows:
        return np.zeros((0,) + pool.shape[1:2] + pool.shape[3:], dtype=pool.dtype)
    return np.stack(rows, axis=0)
