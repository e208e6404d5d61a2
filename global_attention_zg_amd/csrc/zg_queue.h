// Work queues of the persistent grid of the global causal forward.
//
// A persistent grid launches a fixed number of workgroups (a whole number
// per CU) that take jobs until every queue is empty.  Job j sits in queue
// j % nq at place j / nq, and queue[y] counts the places of queue y handed
// out so far.  Workgroup b drains queue b % nq first.  Workgroups are dealt
// to the XCDs in turn, so with nq = 8 the workgroups of one XCD share one
// queue; the kernels number their jobs with the (batch, KV head) index
// fastest, so that queue's jobs share a KV head and the XCD's L2 serves that
// head's tiles.  An empty queue sends the workgroup to the others in turn,
// which evens out XCDs that run at different speeds.  Every place is handed
// out at most once and every job has a place, so each job runs exactly once.
// The counters must be zero at launch.
//
// A claim is split in two so that its latency can hide under other work:
// claim_own takes a ticket from the workgroup's own queue, and next_job turns
// the ticket into a job, taking from the other queues if the ticket is past
// the end; -1 when all queues are empty.  Every lane of one wave calls both
// with the same arguments and only the atomics themselves sit under a lane-0
// branch (a larger divergent region made the compiler treat kernel arguments
// loaded on both of its sides as per-lane values).  claim_own returns lane
// 0's raw result (read it with readfirstlane once it is needed; -1 once the
// own queue is known to be empty); next_job returns a wave-uniform job.
// Files that claim before other work build with the atomic optimizer off,
// whose wave-wide form of the atomic reads its result at once.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace zg {

__device__ __forceinline__ int claim_own(int* queue, int own, bool own_done) {
  int t = -1;
  if (!own_done && (threadIdx.x & 63) == 0) t = atomicAdd(queue + own, 1);
  return t;
}

__device__ __forceinline__ int next_job(int* queue, int own, int nq, int n_jobs, bool& own_done,
                                        int ticket) {
  if (!own_done) {
    const int j = own + nq * ticket;
    if (j < n_jobs) return j;
    own_done = true;
  }
  for (int d = 1; d < nq; ++d) {
    const int y = own + d < nq ? own + d : own + d - nq;
    const int seen = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(queue + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (y + nq * seen >= n_jobs) continue;  // already empty
    int t = 0;
    if ((threadIdx.x & 63) == 0) t = atomicAdd(queue + y, 1);
    const int j = y + nq * __builtin_amdgcn_readfirstlane(t);
    if (j < n_jobs) return j;
  }
  return -1;
}

// Compute units of the current device (looked up once per device).
inline int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess || n < 1)
    n = 256;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace zg
