// pi_host.h -- the host-core side of the hybrid FFN (pi_host.cpp): the sparse
// FFN over a row list of a partition held in host memory, and the cold list
// read from a predicted mask.  Arguments are validated by the callers in
// pi_api.hip; nothing here touches the GPU.
#pragma once
#include <cstdint>

#include "pi.h"

namespace pi {
namespace host {

// y [B][d] fp32 (host), overwritten: the sparse FFN of partition p (host
// pointers) for x [B][d] (host, PI_F32 or PI_F16) over idx[0 .. count) (ids
// outside the partition add nothing), on min(nthreads, pool size, count)
// threads (nthreads <= 0: the pool size).  Calls are serialised.
void sparse_ffn(const pi_ffn_part& p, const void* x, int B, int xdtype, const int32_t* idx, int count, float* y,
                int nthreads);

// Worker threads the pool holds (the CPUs this process may run on, at most 64).
int threads_available();

// The set bits i in [n_hot, n) of mask (host), ascending, as i - n_hot into
// out; returns how many.
int cold_list(const uint64_t* mask, int n_hot, int n, int32_t* out);

}  // namespace host
}  // namespace pi
