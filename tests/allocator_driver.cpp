// Randomised exercise of the host block allocator through its C ABI, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_allocator_sanitizers.py.  Every sequence's table entry below its
// page count holds one reference; sequences end and release their pages, and
// an empty one may take over another's pages as a shared prefix (one reference
// per sharer); appends go through pa_plan_append, copies of shared partial
// pages are applied to the model, and a failed plan must change nothing.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pa.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

static int pages(int32_t tokens) { return (tokens + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE; }

int main() {
  std::mt19937 rng(20261203u);
  int plans_ok = 0, plans_refused = 0, copies_seen = 0;
  for (int trial = 0; trial < 300; ++trial) {
    const int32_t nb = 1 + static_cast<int32_t>(rng() % 96);
    const int32_t B = 1 + static_cast<int32_t>(rng() % 6);
    const int32_t stride = 1 + static_cast<int32_t>(rng() % 6);
    pa_allocator* a = pa_allocator_create(nb);
    CHECK(a != nullptr);
    CHECK(pa_num_free_blocks(a) == nb);
    std::vector<int32_t> bt(static_cast<size_t>(B) * stride, -1), ctx(B, 0);
    for (int round = 0; round < 12; ++round) {
      // now and then a sequence ends and releases its pages
      if (rng() % 3 == 0) {
        const int32_t s = static_cast<int32_t>(rng() % B);
        for (int j = 0; j < pages(ctx[s]); ++j) {
          int32_t& id = bt[static_cast<size_t>(s) * stride + j];
          CHECK(pa_block_decref(a, id) == PA_OK);
          id = -1;
        }
        ctx[s] = 0;
      }
      // and an empty sequence takes over another's pages (a shared prefix)
      if (rng() % 2 == 0 && B > 1) {
        const int32_t s = static_cast<int32_t>(rng() % B), t = static_cast<int32_t>(rng() % B);
        if (s != t && ctx[s] == 0 && ctx[t] > 0) {
          for (int j = 0; j < pages(ctx[t]); ++j) {
            const int32_t id = bt[static_cast<size_t>(t) * stride + j];
            CHECK(pa_block_incref(a, id) == PA_OK);
            bt[static_cast<size_t>(s) * stride + j] = id;
          }
          ctx[s] = ctx[t];
        }
      }
      std::vector<int32_t> nn(B);
      int64_t total = 0;
      for (int32_t b = 0; b < B; ++b) {
        nn[b] = static_cast<int32_t>(rng() % 12);
        total += nn[b];
      }
      std::vector<int32_t> slots(static_cast<size_t>(total) + 1, -7), src(B, -7), dst(B, -7);
      const std::vector<int32_t> bt0 = bt, ctx0 = ctx;
      const int32_t free0 = pa_num_free_blocks(a);
      std::vector<int32_t> rc0(nb);
      for (int32_t i = 0; i < nb; ++i) rc0[i] = pa_block_refcount(a, i);
      int32_t ncopies = -1;
      const int32_t max_copies = static_cast<int32_t>(rng() % (B + 1));
      const pa_status st = pa_plan_append(a, bt.data(), stride, ctx.data(), nn.data(), B,
                                          slots.data(), src.data(), dst.data(), max_copies,
                                          &ncopies);
      if (st != PA_OK) {
        ++plans_refused;
        CHECK(st == PA_ERR_OOM || st == PA_ERR_INVALID_ARG);
        CHECK(bt == bt0 && ctx == ctx0 && pa_num_free_blocks(a) == free0);
        for (int32_t i = 0; i < nb; ++i) CHECK(pa_block_refcount(a, i) == rc0[i]);
        continue;
      }
      ++plans_ok;
      CHECK(ncopies >= 0 && ncopies <= max_copies);
      copies_seen += ncopies;
      for (int32_t c = 0; c < ncopies; ++c) {
        CHECK(pa_block_refcount(a, src[c]) >= 1);
        CHECK(pa_block_refcount(a, dst[c]) == 1);
      }
      // every new slot lies in a page the sequence now owns, and no slot repeats
      std::vector<char> used(static_cast<size_t>(nb) * PA_BLOCK_SIZE, 0);
      int64_t k = 0;
      for (int32_t b = 0; b < B; ++b) {
        CHECK(ctx[b] == ctx0[b] + nn[b]);
        for (int32_t p = ctx0[b]; p < ctx[b]; ++p, ++k) {
          const int32_t id = bt[static_cast<size_t>(b) * stride + p / PA_BLOCK_SIZE];
          CHECK(id >= 0 && id < nb && pa_block_refcount(a, id) == 1);
          CHECK(slots[k] == id * PA_BLOCK_SIZE + p % PA_BLOCK_SIZE);
          CHECK(!used[slots[k]]);
          used[slots[k]] = 1;
        }
      }
      CHECK(slots[total] == -7);
    }
    // reference counts equal the number of table entries that name each block
    std::vector<int32_t> refs(nb, 0);
    for (int32_t b = 0; b < B; ++b)
      for (int j = 0; j < pages(ctx[b]); ++j) ++refs[bt[static_cast<size_t>(b) * stride + j]];
    int32_t in_use = 0;
    for (int32_t i = 0; i < nb; ++i) {
      CHECK(pa_block_refcount(a, i) == refs[i]);
      in_use += refs[i] > 0;
    }
    CHECK(pa_num_free_blocks(a) == nb - in_use);
    // error paths leave the state alone
    CHECK(pa_block_incref(a, -1) == PA_ERR_INVALID_ARG);
    CHECK(pa_block_incref(a, nb) == PA_ERR_INVALID_ARG);
    CHECK(pa_block_refcount(a, nb) == -1);
    // release every reference; the pool is whole again and a second release fails
    for (int32_t b = 0; b < B; ++b)
      for (int j = 0; j < pages(ctx[b]); ++j)
        CHECK(pa_block_decref(a, bt[static_cast<size_t>(b) * stride + j]) == PA_OK);
    CHECK(pa_num_free_blocks(a) == nb);
    if (nb > 0) CHECK(pa_block_decref(a, 0) == PA_ERR_INVALID_ARG);
    pa_allocator_destroy(a);
  }
  CHECK(pa_allocator_create(0) == nullptr);
  pa_allocator_destroy(nullptr);
  std::printf("ok plans=%d refused=%d copies=%d\n", plans_ok, plans_refused, copies_seen);
  return 0;
}
