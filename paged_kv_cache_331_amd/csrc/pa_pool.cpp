// Host block pool of the KV cache: reference counts, a free queue and
// copy-on-write, the bookkeeping that produces the block tables the kernels
// read.
//  * "PagedAttention 机制" §5.3.4 (BlockAllocator): allocate takes a free
//    block and sets its count to 1, or fails when none is free; free drops
//    one reference and returns the block at 0; incr_ref shares a block.
//  * "01. PagedAttention 详解" 自检 Q3: the free list is a queue -- blocks are
//    taken from its head and a block whose count reaches 0 joins its tail, so
//    the least recently freed block is reused first. The pool starts with
//    every block free, in id order.
//  * The same book's §6: a block shared by several tables is copied before a
//    writer changes it; the writer gets a fresh block and the shared one
//    loses that reference. The (src, dst) pairs go to pa_copy_blocks.
// The queue is a ring buffer over num_blocks entries: a block is in it at
// most once, so it never holds more.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "pa.h"

struct pa_pool {
  std::vector<int32_t> ref;     // reference count per block
  std::vector<int32_t> ring;    // free queue
  int64_t head = 0;             // index of the queue's head in ring
  int64_t size = 0;             // blocks in the queue

  explicit pa_pool(int32_t n) : ref(n, 0), ring(n) {
    for (int32_t i = 0; i < n; ++i) ring[i] = i;
    size = n;
  }
  int32_t num_blocks() const { return (int32_t)ref.size(); }
  int32_t pop() {
    const int32_t b = ring[head];
    head = (head + 1) % (int64_t)ring.size();
    --size;
    return b;
  }
  void push(int32_t b) {
    ring[(head + size) % (int64_t)ring.size()] = b;
    ++size;
  }
  bool allocated(int32_t b) const { return b >= 0 && b < num_blocks() && ref[b] > 0; }
};

extern "C" {

pa_pool* pa_pool_create(int32_t num_blocks) {
  if (num_blocks < 1) return nullptr;
  return new (std::nothrow) pa_pool(num_blocks);
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_pool* pool) { return pool ? (int32_t)pool->size : -1; }

int32_t pa_pool_ref_count(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks()) return -1;
  return pool->ref[block];
}

int pa_pool_allocate(pa_pool* pool, int32_t n, int32_t* blocks) {
  if (!pool || (n > 0 && !blocks)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > pool->size) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pool->pop();
    pool->ref[b] = 1;
    blocks[i] = b;
  }
  return PA_OK;
}

int pa_pool_free(pa_pool* pool, const int32_t* blocks, int32_t n) {
  if (!pool || (n > 0 && !blocks)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  // Check every block first: each must hold at least as many references as
  // it appears in the list, so that nothing changes when the call fails.
  std::vector<int32_t> sorted(blocks, blocks + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 0; i < n;) {
    const int32_t b = sorted[i];
    int32_t k = i;
    while (k < n && sorted[k] == b) ++k;
    if (!pool->allocated(b) || k - i > pool->ref[b]) return PA_ERR_STATE;
    i = k;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (--pool->ref[b] == 0) pool->push(b);
  }
  return PA_OK;
}

int pa_pool_share(pa_pool* pool, const int32_t* blocks, int32_t n) {
  if (!pool || (n > 0 && !blocks)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!pool->allocated(blocks[i])) return PA_ERR_STATE;
  for (int32_t i = 0; i < n; ++i) ++pool->ref[blocks[i]];
  return PA_OK;
}

int pa_pool_copy_on_write(pa_pool* pool, int32_t* block, int32_t* src, int32_t* dst) {
  if (!pool || !block || !src || !dst) return PA_ERR_NULL;
  const int32_t b = *block;
  if (!pool->allocated(b)) return PA_ERR_STATE;
  if (pool->ref[b] == 1) return 0;                 // sole owner: write in place
  if (pool->size == 0) return PA_ERR_NO_BLOCKS;
  const int32_t fresh = pool->pop();
  pool->ref[fresh] = 1;
  --pool->ref[b];
  *src = b;
  *dst = fresh;
  *block = fresh;
  return 1;
}

}  // extern "C"
