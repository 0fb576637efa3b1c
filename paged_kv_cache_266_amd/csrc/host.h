// Host-only declarations shared by the translation units of libpagedkv that
// need no HIP: the error reporting behind pkv_last_error() and the pool
// geometry the scheduler reads.  The page pool and the scheduler build from
// this header alone, so they also build as a plain C++ library (the
// sanitizer build of the host code).
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/pagedkv.h"

namespace pkv {

// Thread-local error message behind pkv_last_error().
void clear_error();
pkv_status fail(pkv_status code, const char *msg);

// Pool geometry, for the scheduler.
int32_t pool_page_size(const pkv_pool *pool);
int32_t pool_num_pages(const pkv_pool *pool);

// The scheduler's pool and batch limit, for the serving step.
pkv_pool *sched_pool(const pkv_sched *sched);
int32_t sched_max_batch(const pkv_sched *sched);

}  // namespace pkv
