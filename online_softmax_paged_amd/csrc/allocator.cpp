// Host-side block allocator for a paged KV pool: a free set and one reference
// count per physical block.  Blocks are granted on demand and returned when
// their last owner lets go; a block shared by several sequences (a common
// prompt prefix) has one count per sequence.  (Survey page on FlashAttention
// and PagedAttention, section 3, "core principle": on-demand allocation,
// reclaiming a finished request's blocks, reference counts for sharing.)
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
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

// Appending num_new[b] tokens to each sequence b.  A token at position p goes
// to page p / 16, offset p % 16 of its sequence.  A position that starts a
// page takes a fresh block (on-demand allocation).  The partly filled last
// page of a sequence is written in place when the sequence is its only owner;
// when it is shared, the sequence first gets a private copy (copy on write):
// a fresh block, a (source, destination) pair for the device copy, one
// reference fewer on the shared block.  Everything is checked and counted
// before anything changes, so a failed call leaves the allocator and the
// tables as they were.
pa_status pa_plan_append(pa_allocator* a, int32_t* block_table, int32_t bt_stride,
                         int32_t* ctx_lens, const int32_t* num_new, int32_t num_seqs,
                         int32_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                         int32_t max_copies, int32_t* num_copies) {
  if (!a || num_seqs < 0 || bt_stride < 1 || max_copies < 0 || !num_copies)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_table || !ctx_lens || !num_new)) return PA_ERR_INVALID_ARG;
  const int64_t P = PA_BLOCK_SIZE;
  auto pages = [&](int64_t tokens) { return (tokens + P - 1) / P; };
  // pass 1: validate and count (reference drops of copied pages simulated)
  int64_t total = 0, fresh = 0, copies = 0;
  try {
    std::unordered_map<int32_t, int32_t> rc;  // refcounts as they will be
    for (int32_t b = 0; b < num_seqs; ++b) {
      const int64_t c = ctx_lens[b], n = num_new[b];
      if (c < 0 || n < 0 || c + n > static_cast<int64_t>(bt_stride) * P) return PA_ERR_INVALID_ARG;
      if (n == 0) continue;
      if (c % P) {
        const int32_t phys = block_table[static_cast<int64_t>(b) * bt_stride + c / P];
        if (!valid(a, phys) || a->refcount[static_cast<size_t>(phys)] == 0)
          return PA_ERR_INVALID_ARG;
        auto it = rc.find(phys);
        if (it == rc.end()) it = rc.emplace(phys, a->refcount[static_cast<size_t>(phys)]).first;
        if (it->second > 1) {
          --it->second;
          ++copies;
        }
      }
      fresh += pages(c + n) - pages(c);
      total += n;
    }
  } catch (...) {
    return PA_ERR_OOM;
  }
  if (total > 0 && !slot_mapping) return PA_ERR_INVALID_ARG;
  if (copies > max_copies || (copies > 0 && (!copy_src || !copy_dst))) return PA_ERR_INVALID_ARG;
  if (fresh + copies > static_cast<int64_t>(a->free_ids.size())) return PA_ERR_OOM;
  // pass 2: apply
  int64_t k = 0;
  int32_t nc = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t c = ctx_lens[b], n = num_new[b];
    if (n == 0) continue;
    int32_t* row = block_table + static_cast<int64_t>(b) * bt_stride;
    if (c % P) {
      const int32_t phys = row[c / P];
      if (a->refcount[static_cast<size_t>(phys)] > 1) {
        const int32_t id = pa_alloc_block(a);
        copy_src[nc] = phys;
        copy_dst[nc] = id;
        ++nc;
        --a->refcount[static_cast<size_t>(phys)];  // stays >= 1: the block is not freed
        row[c / P] = id;
      }
    }
    for (int64_t p = c; p < c + n; ++p) {
      if (p % P == 0) row[p / P] = pa_alloc_block(a);
      slot_mapping[k++] = static_cast<int32_t>(row[p / P] * P + p % P);
    }
    ctx_lens[b] = static_cast<int32_t>(c + n);
  }
  *num_copies = nc;
  return PA_OK;
}

}  // extern "C"
