// Host-side block allocator for a paged KV pool: a free set and one reference
// count per physical block.  Blocks are granted on demand and returned when
// their last owner lets go; a block shared by several sequences (a common
// prompt prefix) has one count per sequence.  (Survey page on FlashAttention
// and PagedAttention, section 3, "core principle": on-demand allocation,
// reclaiming a finished request's blocks, reference counts for sharing.)
#include <cstdint>
#include <new>
#include <set>
#include <vector>

#include "pa.h"

struct pa_allocator {
  std::vector<int32_t> refcount;
  std::set<int32_t> free_ids;  // ordered: lowest id first, deterministic grants
};

extern "C" {

pa_allocator* pa_allocator_create(int32_t num_blocks) {
  if (num_blocks < 1) return nullptr;
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return nullptr;
  try {
    a->refcount.assign(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) a->free_ids.insert(a->free_ids.end(), i);
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_block(pa_allocator* a) {
  if (!a || a->free_ids.empty()) return -1;
  int32_t id = *a->free_ids.begin();
  a->free_ids.erase(a->free_ids.begin());
  a->refcount[static_cast<size_t>(id)] = 1;
  return id;
}

static bool valid(const pa_allocator* a, int32_t id) {
  return a && id >= 0 && static_cast<size_t>(id) < a->refcount.size();
}

pa_status pa_block_incref(pa_allocator* a, int32_t id) {
  if (!valid(a, id) || a->refcount[static_cast<size_t>(id)] == 0) return PA_ERR_INVALID_ARG;
  if (a->refcount[static_cast<size_t>(id)] == INT32_MAX) return PA_ERR_INVALID_ARG;
  ++a->refcount[static_cast<size_t>(id)];
  return PA_OK;
}

pa_status pa_block_decref(pa_allocator* a, int32_t id) {
  if (!valid(a, id) || a->refcount[static_cast<size_t>(id)] == 0) return PA_ERR_INVALID_ARG;
  if (--a->refcount[static_cast<size_t>(id)] == 0) {
    try {
      a->free_ids.insert(id);
    } catch (...) {
      ++a->refcount[static_cast<size_t>(id)];
      return PA_ERR_OOM;
    }
  }
  return PA_OK;
}

int32_t pa_block_refcount(const pa_allocator* a, int32_t id) {
  if (!valid(a, id)) return -1;
  return a->refcount[static_cast<size_t>(id)];
}

int32_t pa_num_free_blocks(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->free_ids.size()) : 0;
}

}  // extern "C"
