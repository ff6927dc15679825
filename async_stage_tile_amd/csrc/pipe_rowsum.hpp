// Row-sum completion inside the stream kernels: the segments of a row strip
// meet through one arrival counter per strip instead of a second launch.
//
// The row sum of a strip is cut into p.split column segments (each a work
// item, possibly on different workgroups and XCDs). Every wave that summed
// rows of a segment writes its fp32 partials to p.out[seg][row] and then
// counts one arrival on the strip's ticket. The wave whose arrival is the
// strip's last (ARRIVALS waves per segment, p.split segments) adds the
// strip's partials in segment order 0, 1, ..., split - 1 -- a fixed order, so
// the sums do not depend on which workgroup arrives last -- and writes
// p.final_out for the strip's rows. The tickets hold zero at launch: the
// entry point zeroes them with a fill kernel on the same stream before the
// stream kernel.
//
// Visibility across workgroups (and XCDs, whose L2 caches are not coherent
// with one another) comes from the accesses themselves, not from cache-wide
// maintenance: partials are written with agent-scope atomic stores and read
// back with agent-scope atomic loads, which go to the device's coherence
// point; a wave counts its arrival only after `s_waitcnt vmcnt(0)` has seen
// every one of its partial stores complete, and the last arriver reads the
// partials only after its ticket atomic has returned. An agent-scope release
// or acquire fence would write back or invalidate the whole L2 of the XCD,
// once per wave; measured on MI355X, that cost the 8192 x 65536 row sum 16 %.
#pragma once

#include "pipe_device.hpp"
#include "pipe_kernels.hpp"

namespace pipe {

// A segment partial, stored coherently at agent scope (see above).
__device__ __forceinline__ void store_partial(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int R, int ARRIVALS>
__device__ __forceinline__ void rowsum_strip_arrive(const StreamParams& p, int strip) {
  // Every partial store of this wave has completed before the arrival counts.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t before = 0;
  if (lane_id() == 0)
    before = __hip_atomic_fetch_add(&p.tickets[strip], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  before = uniform(before);
  if (before != (uint32_t)(ARRIVALS * p.split) - 1u) return;
  const int64_t r0 = (int64_t)strip * R;
  const int64_t left = p.M - r0;
  const int rows = left < R ? (int)left : R;
  for (int r = lane_id(); r < rows; r += kWave) {
    float s = __hip_atomic_load(&p.out[r0 + r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int k = 1; k < p.split; ++k)
      s += __hip_atomic_load(&p.out[(int64_t)k * p.M + r0 + r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    p.final_out[r0 + r] = s;
  }
}

}  // namespace pipe
